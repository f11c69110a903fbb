// Rank-r ("skinny") contractions on MFMA, and the fixed-order reductions of
// their split partial sums.
//
//   rowproj : out[m, j] = scale * sum_k P[m, k] * Q[j, k]       (U = X.A^T, V = dY.B,
//             P = W0.A^T, G = A.A^T); P, Q bf16 with k contiguous, both read
//             straight from global memory into MFMA fragments.
//   colproj : part[split][c, j] = sum_{m in split} X[m, c] * S[m, j]   (dB = dY^T.U,
//             dA^T = X^T.V and the DoRA norm terms); X bf16 is staged through
//             LDS with an 8x8 register transpose so that each lane holds eight
//             consecutive m; S fp32 is split into bf16 hi + lo parts, so the
//             product keeps ~16 bits of S.  Optionally also the column sums
//             sum_m X[m, c] * Z[m, c] (DoRA dg) or sum_m X[m, c] (bias gradient).
//
// These are the "skinny MFMA contractions" for the factor gradients: each is
// one pass over the [M, *] operand and bound by HBM bandwidth.
#include "internal.hpp"

namespace ldl {

// ============================================================================ rowproj
// 16 output rows per 512-thread block; the eight waves split the reduction
// (wave w takes the 32-element steps w, w+8, ...), each keeping up to eight
// 1 KiB row fragments of P in flight, then reduce through LDS.
constexpr int RP_WAVES = 8;

template <int RP>
__global__ __launch_bounds__(512) void rowproj_kernel(const RowProjParams p) {
  constexpr int NB = RP / 16;
  __shared__ f32x4 red[RP_WAVES][NB][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int m0 = blockIdx.x * 16;
  const int m = m0 + lr;
  const bool mval = m < p.M;
  const uint16_t* prow = p.P + (size_t)(mval ? m : 0) * p.ldp + lq * 8;

  const uint16_t* qrow[NB];
  bool qval[NB];
#pragma unroll
  for (int jb = 0; jb < NB; ++jb) {
    const int j = jb * 16 + lr;
    qval[jb] = j < p.R;
    const uint16_t* base = (j < p.R0) ? (p.q0 + (size_t)j * p.ldq) : (p.q1 + (size_t)(j - p.R0) * p.ldq);
    qrow[jb] = (qval[jb] ? base : p.q0) + lq * 8;
  }

  f32x4 acc[NB];
#pragma unroll
  for (int jb = 0; jb < NB; ++jb) acc[jb] = f32x4{0, 0, 0, 0};

  const int nsteps = p.K / 32;
  const u32x4 zero = {0, 0, 0, 0};
  constexpr int U = 8;
  int ks = wave;
  for (; ks + (U - 1) * RP_WAVES < nsteps; ks += U * RP_WAVES) {
    u32x4 pf[U];
#pragma unroll
    for (int u = 0; u < U; ++u) pf[u] = mval ? ld16(prow + (ks + u * RP_WAVES) * 32) : zero;
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int jb = 0; jb < NB; ++jb) {
        const u32x4 qf = qval[jb] ? ld16(qrow[jb] + (ks + u * RP_WAVES) * 32) : zero;
        acc[jb] = mfma_bf16(qf, pf[u], acc[jb]);
      }
    }
  }
  for (; ks < nsteps; ks += RP_WAVES) {
    const u32x4 pf = mval ? ld16(prow + ks * 32) : zero;
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) {
      const u32x4 qf = qval[jb] ? ld16(qrow[jb] + ks * 32) : zero;
      acc[jb] = mfma_bf16(qf, pf, acc[jb]);
    }
  }

#pragma unroll
  for (int jb = 0; jb < NB; ++jb) red[wave][jb][lane] = acc[jb];
  __syncthreads();
  // lane holds out[m][jb*16 + 4*lq + i]; waves 0..NB-1 finish one jb each
  for (int jb = wave; jb < NB; jb += RP_WAVES) {
    f32x4 v = red[0][jb][lane];
#pragma unroll
    for (int w = 1; w < RP_WAVES; ++w) v += red[w][jb][lane];
    if (mval) {
      const int j0 = jb * 16 + 4 * lq;
      float* dst = p.out + (size_t)m * p.ldo;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (j0 + i < p.R) dst[j0 + i] = v[i] * p.scale;
    }
  }
}

// ============================================================================ colproj
// Block = 64 columns of X and one split of rows, walked in sub-tiles of MS rows.
// Per sub-tile: X^T (64 x MS bf16) and S^T as bf16 hi/lo parts (R x MS each) are
// staged in LDS; each of the four waves owns 16 columns.
__device__ __forceinline__ int xt_off(int c, int chunk, int rowbytes) {
  return c * rowbytes + ((chunk ^ swz(c)) << 4);
}

template <int RP>
struct ColProjTile {
  static constexpr int MS = RP <= 64 ? 256 : 128;        // rows per sub-tile
  static constexpr int XBYTES = 64 * MS * 2;
  static constexpr int SBYTES = RP * MS * 2;             // one of hi / lo
};

template <int RP>
__global__ __launch_bounds__(256) void colproj_kernel(const ColProjParams p) {
  using T = ColProjTile<RP>;
  constexpr int NB = RP / 16;
  constexpr int MS = T::MS;
  constexpr int ROWB = MS * 2;          // bytes per transposed row
  __shared__ __attribute__((aligned(16))) uint8_t xt[T::XBYTES];
  __shared__ __attribute__((aligned(16))) uint16_t shi[RP * MS];
  __shared__ __attribute__((aligned(16))) uint16_t slo[RP * MS];
  __shared__ float csred[32][64 + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int c0 = blockIdx.x * 64;
  const int split = blockIdx.y;
  const int mbeg = split * p.msplit;
  const int mend = min(p.M, mbeg + p.msplit);

  // X loader role: 8 consecutive columns x 8 consecutive rows; the MS/8 row
  // groups x 8 column groups of a sub-tile are spread over the 256 threads
  const int cb = tid & 7, mb = tid >> 3;       // mb in [0, 32)
  const int cl = c0 + cb * 8;
  const bool cval = cl < p.C;                   // C is a multiple of 8

  f32x4 acc[NB];
#pragma unroll
  for (int jb = 0; jb < NB; ++jb) acc[jb] = f32x4{0, 0, 0, 0};
  float cs[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) cs[e] = 0.f;

  for (int sub = mbeg; sub < mend; sub += MS) {
    __syncthreads();   // previous sub-tile fully consumed
    // ---- X[sub .. sub+MS, c0 .. c0+63] -> LDS, transposed (8x8 register transposes)
#pragma unroll
    for (int h = 0; h < (MS + 255) / 256; ++h) {
      const int mg = mb + 32 * h;             // row group of 8
      if (mg >= MS / 8) break;
      u32x4 rows[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int m = sub + mg * 8 + e;
        rows[e] = u32x4{0, 0, 0, 0};
        if (cval && m < mend) {
          rows[e] = ld16(p.X + (size_t)m * p.ldx + cl);
          if (p.colsum_mode == 1) {
            const u32x4 z = ld16(p.Z + (size_t)m * p.ldz + cl);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              cs[2 * t] += bf16_lo(rows[e][t]) * bf16_lo(z[t]);
              cs[2 * t + 1] += bf16_hi(rows[e][t]) * bf16_hi(z[t]);
            }
          } else if (p.colsum_mode == 2) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              cs[2 * t] += bf16_lo(rows[e][t]);
              cs[2 * t + 1] += bf16_hi(rows[e][t]);
            }
          }
        }
      }
      u32x4 cols[8];
      transpose8x8_b16(rows, cols);
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) *reinterpret_cast<u32x4*>(xt + xt_off(cb * 8 + cc, mg, ROWB)) = cols[cc];
    }
    // ---- S[sub .. sub+MS, 0 .. R) -> LDS as bf16 hi / lo, transposed [j][m]
    for (int idx = tid; idx < MS * RP; idx += 256) {
      const int j = idx / MS, mm = idx % MS;   // consecutive threads: consecutive rows m
      const int m = sub + mm;
      float v = 0.f;
      if (j < p.R && m < mend) v = p.S[(size_t)m * p.lds + j] * p.s_in;
      const uint32_t h = f32_to_bf16_bits(v);
      const int off = (xt_off(j, mm >> 3, ROWB) >> 1) + (mm & 7);   // same swizzle as the X tile
      shi[off] = (uint16_t)h;
      slo[off] = (uint16_t)f32_to_bf16_bits(v - __uint_as_float(h << 16));
    }
    __syncthreads();

    // ---- MS/32 reduction steps of 32 rows
    const int c_frag = wave * 16 + lr;
#pragma unroll 2
    for (int s = 0; s < MS / 32; ++s) {
      const u32x4 xf = *reinterpret_cast<const u32x4*>(xt + xt_off(c_frag, s * 4 + lq, ROWB));
#pragma unroll
      for (int jb = 0; jb < NB; ++jb) {
        const int j = jb * 16 + lr;
        const int so = xt_off(j, s * 4 + lq, ROWB);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(shi) + so);
        const u32x4 lo = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(slo) + so);
        acc[jb] = mfma_bf16(hi, xf, acc[jb]);
        acc[jb] = mfma_bf16(lo, xf, acc[jb]);
      }
    }
  }

  // ---- partial product: lane holds (j = jb*16 + 4*lq + i, c = c0 + 16*wave + lr)
  const int c = c0 + wave * 16 + lr;
  if (c < p.C) {
    float* dst = p.part + ((size_t)split * p.C + c) * RP;
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) *reinterpret_cast<f32x4*>(dst + jb * 16 + 4 * lq) = acc[jb];
  }

  // ---- column sums: reduce the row groups of each column
  if (p.colsum_mode != 0) {
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; ++e) csred[mb][cb * 8 + e] = cs[e];
    __syncthreads();
    if (tid < 64 && c0 + tid < p.C) {
      float t = 0.f;
      for (int g = 0; g < 32; ++g) t += csred[g][tid];
      p.cspart[(size_t)split * p.C + c0 + tid] = t;
    }
  }
}

// ============================================================================ reductions
// out[row, col] = alpha * sum_s part[s][...] (+ row scale) (+ alpha2 * sum_l Qm[row, l] * Am[l, col]).
// Threads walk the partial buffer in its own order ([C][rp], j fastest) so the
// split reads are coalesced; `trans` selects whether the partial's column index
// (j) is the output row (dA = part^T) or the output column (dB).
__global__ void reduce_parts_kernel(const ReduceParams p) {
  const int C = p.trans ? p.cols : p.rows;          // partial rows
  const int R = p.trans ? p.rows : p.cols;          // valid partial columns
  const size_t total = (size_t)C * p.rp;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += (size_t)gridDim.x * blockDim.x) {
    const int c = (int)(idx / p.rp), j = (int)(idx % p.rp);
    if (j >= R) continue;
    float acc = 0.f;
    for (int s = 0; s < p.nsplit; ++s) acc += p.part[(size_t)s * p.pstride + idx];
    const int row = p.trans ? j : c, col = p.trans ? c : j;
    float v = acc * p.alpha;
    if (p.rowscale != nullptr) v *= p.rowscale[row];
    if (p.Qm != nullptr) {
      float t = 0.f;
      for (int l = 0; l < p.rq; ++l) t += p.Qm[(size_t)row * p.ldq + l] * bf16_to_f32(p.Am[(size_t)l * p.lda + col]);
      v += p.alpha2 * t;
    }
    p.out[(size_t)row * p.ldo + col] = v;
  }
}

__global__ void reduce_colsum_kernel(const float* cspart, int nsplit, int C, float* out) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= C) return;
  float acc = 0.f;
  for (int s = 0; s < nsplit; ++s) acc += cspart[(size_t)s * C + c];
  out[c] = acc;
}

// Bt[j, n] = bf16(B[n, j] * (scale ? scale[n] : 1)), B [N, r] bf16 -> Bt [r, N] bf16.
__global__ void transpose_scale_kernel(const uint16_t* B, const float* scale, int N, int r, uint16_t* Bt) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  const float sc = scale ? scale[n] : 1.f;
  for (int j = 0; j < r; ++j) {
    const float v = bf16_to_f32(B[(size_t)n * r + j]);
    Bt[(size_t)j * N + n] = scale ? (uint16_t)f32_to_bf16_bits(v * sc) : B[(size_t)n * r + j];
  }
}

__global__ void fill_zero_kernel(float* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0.f;
}

// ============================================================================ launchers
hipError_t launch_rowproj(const RowProjParams& p, hipStream_t st) {
  if (p.M <= 0) return hipSuccess;
  const dim3 grid((p.M + 15) / 16), block(64 * RP_WAVES);
  const int rp = p.R <= 16 ? 16 : p.R <= 32 ? 32 : p.R <= 64 ? 64 : 128;
  switch (rp) {
    case 16: hipLaunchKernelGGL(rowproj_kernel<16>, grid, block, 0, st, p); break;
    case 32: hipLaunchKernelGGL(rowproj_kernel<32>, grid, block, 0, st, p); break;
    case 64: hipLaunchKernelGGL(rowproj_kernel<64>, grid, block, 0, st, p); break;
    default: hipLaunchKernelGGL(rowproj_kernel<128>, grid, block, 0, st, p); break;
  }
  return hipGetLastError();
}

int colproj_rp(int R) { return R <= 16 ? 16 : R <= 32 ? 32 : R <= 64 ? 64 : 128; }

void colproj_plan(int M, int C, int* nsplit, int* msplit) {
  if (M <= 0) {
    *nsplit = 1;
    *msplit = 256;
    return;
  }
  // splits are whole multiples of 256 rows (a multiple of every sub-tile height);
  // aim for ~1024 blocks, at most 32 splits
  const int ctiles = (C + 63) / 64;
  const int mchunks = (M + 255) / 256;
  int want = (1024 + ctiles - 1) / ctiles;
  if (want < 1) want = 1;
  if (want > 32) want = 32;
  int ns = mchunks < want ? mchunks : want;
  if (ns < 1) ns = 1;
  const int per = (mchunks + ns - 1) / ns;      // 256-row chunks per split
  *msplit = per * 256;
  *nsplit = (M + *msplit - 1) / *msplit;
  if (*nsplit < 1) *nsplit = 1;
}

hipError_t launch_colproj(const ColProjParams& p, int nsplit, hipStream_t st) {
  const dim3 grid((p.C + 63) / 64, nsplit), block(256);
  switch (colproj_rp(p.R)) {
    case 16: hipLaunchKernelGGL(colproj_kernel<16>, grid, block, 0, st, p); break;
    case 32: hipLaunchKernelGGL(colproj_kernel<32>, grid, block, 0, st, p); break;
    case 64: hipLaunchKernelGGL(colproj_kernel<64>, grid, block, 0, st, p); break;
    default: hipLaunchKernelGGL(colproj_kernel<128>, grid, block, 0, st, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_reduce(const ReduceParams& p, hipStream_t st) {
  const size_t total = (size_t)(p.trans ? p.cols : p.rows) * p.rp;
  if (total == 0) return hipSuccess;
  size_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(reduce_parts_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_reduce_colsum(const float* cspart, int nsplit, int C, float* out, hipStream_t st) {
  hipLaunchKernelGGL(reduce_colsum_kernel, dim3((C + 255) / 256), dim3(256), 0, st, cspart, nsplit, C, out);
  return hipGetLastError();
}

hipError_t launch_transpose_scale(const uint16_t* B, const float* scale, int N, int r, uint16_t* Bt, hipStream_t st) {
  hipLaunchKernelGGL(transpose_scale_kernel, dim3((N + 255) / 256), dim3(256), 0, st, B, scale, N, r, Bt);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

}  // namespace ldl
