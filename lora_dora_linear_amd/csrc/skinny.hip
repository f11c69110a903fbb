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
template <int RP>
__global__ __launch_bounds__(256) void rowproj_kernel(const RowProjParams p) {
  constexpr int NB = RP / 16;
  __shared__ f32x4 red[4][NB][64];
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
  int ks = wave;
  for (; ks + 12 < nsteps; ks += 16) {
    u32x4 pf[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) pf[u] = mval ? ld16(prow + (ks + 4 * u) * 32) : zero;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int jb = 0; jb < NB; ++jb) {
        const u32x4 qf = qval[jb] ? ld16(qrow[jb] + (ks + 4 * u) * 32) : zero;
        acc[jb] = mfma_bf16(qf, pf[u], acc[jb]);
      }
    }
  }
  for (; ks < nsteps; ks += 4) {
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
  if (wave == 0 && mval) {
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) {
      const f32x4 v = red[0][jb][lane] + red[1][jb][lane] + red[2][jb][lane] + red[3][jb][lane];
      const int j0 = jb * 16 + 4 * lq;
      float* dst = p.out + (size_t)m * p.ldo;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (j0 + i < p.R) dst[j0 + i] = v[i] * p.scale;
    }
  }
}

// ============================================================================ colproj
// LDS tile of X^T: 64 columns x 256 rows of m (512 bytes per column row,
// 16-byte chunk index XOR-swizzled with swz(c)).
__device__ __forceinline__ int xt_off(int c, int chunk) { return c * 512 + ((chunk ^ swz(c)) << 4); }

template <int RP>
__global__ __launch_bounds__(256) void colproj_kernel(const ColProjParams p) {
  constexpr int NB = RP / 16;
  __shared__ __attribute__((aligned(16))) uint8_t xt[64 * 512];
  __shared__ float csred[32][64 + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int c0 = blockIdx.x * 64;
  const int split = blockIdx.y;
  const int mbeg = split * p.msplit;
  const int mend = min(p.M, mbeg + p.msplit);

  // loader role: 8 consecutive columns x 8 consecutive rows
  const int cb = tid & 7, mb = tid >> 3;
  const int cl = c0 + cb * 8;
  const bool cval = cl < p.C;   // C is a multiple of 8

  f32x4 acc[NB];
#pragma unroll
  for (int jb = 0; jb < NB; ++jb) acc[jb] = f32x4{0, 0, 0, 0};
  float cs[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) cs[e] = 0.f;

  for (int sub = mbeg; sub < mend; sub += 256) {
    // ---- stage X[sub .. sub+255, c0 .. c0+63] transposed into LDS
    u32x4 rows[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int m = sub + mb * 8 + e;
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
    __syncthreads();   // previous sub-tile fully consumed
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) *reinterpret_cast<u32x4*>(xt + xt_off(cb * 8 + cc, mb)) = cols[cc];
    __syncthreads();

    // ---- 8 reduction steps of 32 rows each
    const int c_frag = wave * 16 + lr;
#pragma unroll 2
    for (int s = 0; s < 8; ++s) {
      const int mrow0 = sub + s * 32 + lq * 8;   // rows past mend were staged as zeros
      const u32x4 xf = *reinterpret_cast<const u32x4*>(xt + xt_off(c_frag, s * 4 + lq));
#pragma unroll
      for (int jb = 0; jb < NB; ++jb) {
        const int j = jb * 16 + lr;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int m = mrow0 + e;
          v[e] = (j < p.R && m < mend) ? p.S[(size_t)m * p.lds + j] * p.s_in : 0.f;
        }
        u32x4 hi, lo;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t h0 = f32_to_bf16_bits(v[2 * t]), h1 = f32_to_bf16_bits(v[2 * t + 1]);
          hi[t] = h0 | (h1 << 16);
          lo[t] = pack_bf16x2(v[2 * t] - __uint_as_float(h0 << 16), v[2 * t + 1] - __uint_as_float(h1 << 16));
        }
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

  // ---- column sums: reduce the 32 row-groups of each column
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
// out[row, col] = alpha * sum_s part[s][...] (+ row scale) (+ alpha2 * sum_l Qm[row, l] * Am[l, col])
__global__ void reduce_parts_kernel(const ReduceParams p) {
  const size_t total = (size_t)p.rows * p.cols;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += (size_t)gridDim.x * blockDim.x) {
    const int row = (int)(idx / p.cols), col = (int)(idx % p.cols);
    const size_t off = p.trans ? ((size_t)col * p.rp + row) : ((size_t)row * p.rp + col);
    float acc = 0.f;
    for (int s = 0; s < p.nsplit; ++s) acc += p.part[(size_t)s * p.pstride + off];
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
  const dim3 grid((p.M + 15) / 16), block(256);
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
  const int ctiles = (C + 63) / 64;
  const int mchunks = (M + 255) / 256;
  int want = (1024 + ctiles - 1) / ctiles;
  if (want < 1) want = 1;
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
  const size_t total = (size_t)p.rows * p.cols;
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
