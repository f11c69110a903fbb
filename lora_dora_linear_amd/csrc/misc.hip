// Small per-row kernels: the DoRA norm terms, the int8 quantiser, and the
// fp32 path (a plain tiled SIMT GEMM, used for fp32 layers, which are small).
#include "internal.hpp"

namespace ldl {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// ============================================================================ DoRA
// w0_sumsq[n] = sum_k W0[n,k]^2 : one wave per row.  The squared row norm of the frozen base
// weight is kept from call to call; only the two rank-sized terms of the norm change per step
// ("LoRA/DoRA fast forward: no weight materialization", commit message).
template <bool BF16>
__global__ __launch_bounds__(256) void rowsumsq_kernel(const void* W0, int N, int K, int ldw, float* out) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  float acc = 0.f;
  if (BF16) {
    const uint16_t* row = static_cast<const uint16_t*>(W0) + (size_t)n * ldw;
    for (int k = lane * 8; k < K; k += 512) {
      const u32x4 v = ld16(row + k);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float a = bf16_lo(v[t]), b = bf16_hi(v[t]);
        acc += a * a + b * b;
      }
    }
  } else {
    const float* row = static_cast<const float*>(W0) + (size_t)n * ldw;
    for (int k = lane; k < K; k += 64) acc += row[k] * row[k];
  }
  acc = wave_sum(acc);
  if (lane == 0) out[n] = acc;
}

// Broadcast of lane l's value (l wave-uniform).
__device__ __forceinline__ float lane_bcast(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Closed-form row norm: nu^2 = c + 2s <B_n, P_n> + s^2 B_n G B_n^T, clamped at 0;
// g = m / max(nu, eps).  One wave per output row, lane j holding ranks j and j + 64
// (r <= 128); G staged in LDS transposed so that lane j reads G[j][l] at consecutive
// addresses; B_n[l] broadcast from the lane that holds it.
// the r x r Gram matrix into LDS, 16 bytes per thread and load (G 16-byte aligned, r a
// multiple of 8), then a block barrier
__device__ __forceinline__ void stage_g(float* sG, const float* G, int r) {
  const int nq = r * r / 4;
  for (int i = threadIdx.x; i < nq; i += blockDim.x)
    reinterpret_cast<f32x4*>(sG)[i] = reinterpret_cast<const f32x4*>(G)[i];
  __syncthreads();
}

__global__ __launch_bounds__(256) void dora_norm_kernel(int N, int r, float s, float eps, const float* c,
                                                        const float* P, const float* G, const uint16_t* B,
                                                        const float* m, float* norm, float* g) {
  extern __shared__ float sG[];                  // G = A.A^T as stored (symmetric: row l = column l)
  const int lane = threadIdx.x & 63;
  const int n = min(blockIdx.x * 4 + (threadIdx.x >> 6), N - 1);   // rows past N redo row N-1, unstored
  // the row's operands first, so their latency overlaps the staging of G
  const uint16_t* bn = B + (size_t)n * r;
  const float* pn = P + (size_t)n * r;
  const bool h0 = lane < r, h1 = lane + 64 < r;
  const float b0 = h0 ? bf16_to_f32(bn[lane]) : 0.f, b1 = h1 ? bf16_to_f32(bn[lane + 64]) : 0.f;
  const float p0 = h0 ? pn[lane] : 0.f, p1 = h1 ? pn[lane + 64] : 0.f;
  const float cn = c[n], mn = m[n];
  stage_g(sG, G, r);
  float t1 = b0 * p0 + b1 * p1;
  float bg0 = 0.f, bg1 = 0.f;                    // (B_n G)[j] = (G B_n^T)[j] for the lane's ranks
  for (int l = 0; l < r; ++l) {
    const float bl = l < 64 ? lane_bcast(b0, l) : lane_bcast(b1, l - 64);
    if (h0) bg0 += bl * sG[l * r + lane];
    if (h1) bg1 += bl * sG[l * r + lane + 64];
  }
  float t2 = b0 * bg0 + b1 * bg1;
  t1 = wave_sum(t1);
  t2 = wave_sum(t2);
  if (lane == 0 && blockIdx.x * 4 + (threadIdx.x >> 6) < N) {
    const float nu2 = cn + 2.f * s * t1 + s * s * t2;
    const float nu = sqrtf(fmaxf(nu2, 0.f));
    norm[n] = nu;
    g[n] = mn / fmaxf(nu, eps);
  }
}

// Backward per output row, with the norm kept in the graph:
//   T = sum_splits partT (= dY^T.U row n);  dg = sum_splits cspart (= sum_m dY*Z)
//   dm = dg / max(nu, eps);  w = -dg m / (2 nu^3) if nu > eps else 0
//   dB[n,:] = s g_n T + w (2s P_n + 2s^2 (B G)_n);  wB[n,:] = 2s w B_n
// One wave per output row, lane j computing ranks j and j + 64 (r <= 128); every sum
// runs in a fixed order (splits in order, l = 0 .. r-1).
__global__ __launch_bounds__(256) void dora_finalize_kernel(int N, int r, float s, float eps, const float* partT,
                                                            const float* cspart, int nsplit, int rpT,
                                                            const float* norm, const float* g, const float* m,
                                                            const float* P, const float* G, const uint16_t* B,
                                                            float* dB, float* dm, float* wB, uint16_t* wB_pk,
                                                            int pk_rp) {
  extern __shared__ float sG[];
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int n = min(row, N - 1);                 // rows past N redo row N-1, unstored
  const bool live = row < N;
  const bool h0 = lane < r, h1 = lane + 64 < r;
  // loads first (their latency overlaps the staging of G): the row's own operands, then the
  // split partials of dg and of T for the lane's ranks, eight splits in flight, each sum in
  // split order
  const uint16_t* bn = B + (size_t)n * r;
  const float b0 = h0 ? bf16_to_f32(bn[lane]) : 0.f, b1 = h1 ? bf16_to_f32(bn[lane + 64]) : 0.f;
  const float p0 = h0 ? P[(size_t)n * r + lane] : 0.f, p1 = h1 ? P[(size_t)n * r + lane + 64] : 0.f;
  const float nu = norm[n], gn = g[n], mn = m[n];
  float dg = 0.f, t0 = 0.f, t1 = 0.f;
  {
    const float* cp = cspart + n;
    const float* tp = partT + (size_t)n * rpT + lane;
    const size_t ts = (size_t)N * rpT;
    int sp = 0;
    for (; sp + 16 <= nsplit; sp += 16) {        // sixteen splits in flight
      float c8[16], a8[16], b8[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        c8[q] = cp[(size_t)(sp + q) * N];
        a8[q] = h0 ? tp[(sp + q) * ts] : 0.f;
        b8[q] = h1 ? tp[(sp + q) * ts + 64] : 0.f;
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) { dg += c8[q]; t0 += a8[q]; t1 += b8[q]; }
    }
    for (; sp + 8 <= nsplit; sp += 8) {
      float c8[8], a8[8], b8[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        c8[q] = cp[(size_t)(sp + q) * N];
        a8[q] = h0 ? tp[(sp + q) * ts] : 0.f;
        b8[q] = h1 ? tp[(sp + q) * ts + 64] : 0.f;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) { dg += c8[q]; t0 += a8[q]; t1 += b8[q]; }
    }
    for (; sp < nsplit; ++sp) {
      dg += cp[(size_t)sp * N];
      if (h0) t0 += tp[sp * ts];
      if (h1) t1 += tp[sp * ts + 64];
    }
  }
  stage_g(sG, G, r);
  const float den = fmaxf(nu, eps);
  if (lane == 0 && live) dm[n] = dg / den;
  const float w = (nu > eps) ? (-dg * mn / (2.f * nu * nu * nu)) : 0.f;
  float bg0 = 0.f, bg1 = 0.f;                    // (B_n G)[j] for the lane's ranks
  for (int l = 0; l < r; ++l) {
    const float bl = l < 64 ? lane_bcast(b0, l) : lane_bcast(b1, l - 64);
    if (h0) bg0 += bl * sG[l * r + lane];
    if (h1) bg1 += bl * sG[l * r + lane + 64];
  }
  if (!live) return;
  if (h0) {
    dB[(size_t)n * r + lane] = s * gn * t0 + w * (2.f * s * p0 + 2.f * s * s * bg0);
    wB[(size_t)n * r + lane] = 2.f * s * w * b0;
  }
  if (h1) {
    dB[(size_t)n * r + lane + 64] = s * gn * t1 + w * (2.f * s * p1 + 2.f * s * s * bg1);
    wB[(size_t)n * r + lane + 64] = 2.f * s * w * b1;
  }
  if (wB_pk != nullptr && lane < pk_rp) {
    // wB also in the packed bf16 hi / lo layout of the column projections that read it
    // (rank padding pk_rp <= 64, zero past r): row n is half (n & 1) of word
    // 4 lane + ((n & 7) >> 1) of its 8-row group (hi) and of word 4 (pk_rp + lane) + .. (lo)
    const float x = h0 ? 2.f * s * w * b0 : 0.f;
    const uint32_t hi = f32_to_bf16_bits(x);
    uint16_t* grp = wB_pk + (size_t)(n >> 3) * (16 * pk_rp) + (n & 1);
    const int e = (n & 7) >> 1;
    grp[2 * (4 * lane + e)] = (uint16_t)hi;
    grp[2 * (4 * (pk_rp + lane) + e)] = (uint16_t)f32_to_bf16_bits(x - __uint_as_float(hi << 16));
  }
}

// out[m, n] = bf16(in[m, n] * g[n]) (round to nearest even): the DoRA backward's dY.diag(g),
// written once so the input-gradient product runs as a plain bf16 GEMM (the same values
// a fragment-wise scaling would feed the MFMAs).  8 columns per thread, rows of ld elements.
__global__ __launch_bounds__(256) void scale_cols_kernel(const uint16_t* in, int M, int N, int ld, const float* g,
                                                         uint16_t* out, int ldo) {
  const int per_row = N / 8;
  const size_t total = (size_t)M * per_row;
  for (size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (size_t)gridDim.x * blockDim.x) {
    const int m = (int)(t / per_row), c = (int)(t % per_row) * 8;
    const u32x4 v = ld16(in + (size_t)m * ld + c);
    const f32x4 s0 = *reinterpret_cast<const f32x4*>(g + c), s1 = *reinterpret_cast<const f32x4*>(g + c + 4);
    st16(out + (size_t)m * ldo + c, scale_bf16x8(v, s0, s1));
  }
}

// Two row-scaled copies in one launch: out[n, :] = bf16(in[n, :] * g[n]) for in = W0 [N, K]
// (row stride ld) and in2 = B [N, r] (dense), each into a dense bf16 array; 8 columns per
// thread, 16-byte aligned rows.
__global__ __launch_bounds__(256) void scale_rows_kernel(const uint16_t* in, int N, int K, int ld, const uint16_t* in2,
                                                         int r, const float* g, uint16_t* out, uint16_t* out2) {
  const int pr1 = K / 8, pr2 = r / 8;
  const size_t t1 = (size_t)N * pr1, total = t1 + (size_t)N * pr2;
  for (size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (size_t)gridDim.x * blockDim.x) {
    const bool first = t < t1;
    const size_t u = first ? t : t - t1;
    const int per = first ? pr1 : pr2;
    const int n = (int)(u / per), c = (int)(u % per) * 8;
    const float gn = g[n];
    const f32x4 s4 = f32x4{gn, gn, gn, gn};
    const uint16_t* src = first ? in + (size_t)n * ld + c : in2 + (size_t)n * r + c;
    uint16_t* dst = first ? out + (size_t)n * K + c : out2 + (size_t)n * r + c;
    st16(dst, scale_bf16x8(ld16(src), s4, s4));
  }
}

hipError_t launch_scale_rows(const void* in, int N, int K, int ld, const void* in2, int r, const float* g, void* out,
                             void* out2, hipStream_t st) {
  const size_t total = (size_t)N * (K / 8 + r / 8);
  if (total == 0) return hipSuccess;
  size_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(scale_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, st, static_cast<const uint16_t*>(in), N,
                     K, ld, static_cast<const uint16_t*>(in2), r, g, static_cast<uint16_t*>(out),
                     static_cast<uint16_t*>(out2));
  return hipGetLastError();
}

hipError_t launch_scale_cols(const void* in, int M, int N, int ld, const float* g, void* out, int ldo,
                             hipStream_t st) {
  if (M <= 0) return hipSuccess;
  const size_t total = (size_t)M * (N / 8);
  size_t blocks = (total + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(scale_cols_kernel, dim3((unsigned)blocks), dim3(256), 0, st, static_cast<const uint16_t*>(in), M,
                     N, ld, g, static_cast<uint16_t*>(out), ldo);
  return hipGetLastError();
}

// Gated-MLP backward from the stored bf16 dh, e and u (8 columns per thread):
// de = dh u act'(e) overwrites dh in place, du = dh act(e) (SiLU: act' = sigma (1 + e (1 - sigma))).
// Each thread reads its own dh chunk before writing de there.
template <int ACT>
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(uint16_t* dE, int ld_de, const uint16_t* E, int ld_e,
                                                         const uint16_t* U, int ld_u, uint16_t* dU, int ld_du, int M,
                                                         int N) {
  constexpr int act = ACT;
  const unsigned per_row = (unsigned)N / 8u;
  const size_t total = (size_t)M * per_row;
  for (size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (size_t)gridDim.x * blockDim.x) {
    const size_t m = t / per_row, c = (t % per_row) * 8;
    const u32x4 d = ld16(dE + m * (size_t)ld_de + c), e = ld16(E + m * (size_t)ld_e + c),
                u = ld16(U + m * (size_t)ld_u + c);
    u32x4 de, du;
    for (int i = 0; i < 4; ++i) {
      const float e0 = bf16_lo(e[i]), e1 = bf16_hi(e[i]), d0 = bf16_lo(d[i]), d1 = bf16_hi(d[i]);
      de[i] = pack_bf16x2(d0 * bf16_lo(u[i]) * glu_act_grad(e0, act), d1 * bf16_hi(u[i]) * glu_act_grad(e1, act));
      du[i] = pack_bf16x2(d0 * glu_act(e0, act), d1 * glu_act(e1, act));
    }
    st16(dE + m * (size_t)ld_de + c, de);
    st16(dU + m * (size_t)ld_du + c, du);
  }
}

hipError_t launch_swiglu_bwd(void* dE, int ld_de, const void* E, int ld_e, const void* U, int ld_u, void* dU,
                             int ld_du, int M, int N, int act, hipStream_t st) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (N % 8 || ld_de % 8 || ld_e % 8 || ld_u % 8 || ld_du % 8 || ld_de < N || ld_e < N || ld_u < N || ld_du < N)
    return hipErrorInvalidValue;
  const size_t total = (size_t)M * (N / 8);
  size_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;   // ~7 grid-stride steps a thread at 8192 x 14336 (2048 blocks: 222 -> 213 us)
  auto k = act == ACT_GELU ? swiglu_bwd_kernel<ACT_GELU>
                            : (act == ACT_GELU_TANH ? swiglu_bwd_kernel<ACT_GELU_TANH> : swiglu_bwd_kernel<ACT_SILU>);
  hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(256), 0, st, static_cast<uint16_t*>(dE), ld_de,
                     static_cast<const uint16_t*>(E), ld_e, static_cast<const uint16_t*>(U), ld_u,
                     static_cast<uint16_t*>(dU), ld_du, M, N);
  return hipGetLastError();
}

hipError_t launch_rowsumsq(const void* W0, int dtype_bf16, int N, int K, int ldw, float* out, hipStream_t st) {
  const dim3 grid((N + 3) / 4), block(256);
  if (dtype_bf16) hipLaunchKernelGGL(rowsumsq_kernel<true>, grid, block, 0, st, W0, N, K, ldw, out);
  else hipLaunchKernelGGL(rowsumsq_kernel<false>, grid, block, 0, st, W0, N, K, ldw, out);
  return hipGetLastError();
}

hipError_t launch_dora_norm(int N, int r, float s, float eps, const float* w0_sumsq, const float* P,
                            const float* G, const uint16_t* B, const float* m, float* norm, float* g, hipStream_t st) {
  hipLaunchKernelGGL(dora_norm_kernel, dim3((N + 3) / 4), dim3(256), r * r * sizeof(float), st,
                     N, r, s, eps, w0_sumsq, P, G, B, m, norm, g);
  return hipGetLastError();
}

hipError_t launch_dora_finalize(int N, int r, float s, float eps, const float* partT, const float* cspart,
                                int nsplit, int rpT, const float* norm, const float* g, const float* m,
                                const float* P, const float* G, const uint16_t* B,
                                float* dB, float* dm, float* wB, uint16_t* wB_pk, int pk_rp, hipStream_t st) {
  if (wB_pk != nullptr && (pk_rp < r || pk_rp > 64 || N % 8)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dora_finalize_kernel, dim3((N + 3) / 4), dim3(256), r * r * sizeof(float), st,
                     N, r, s, eps, partT, cspart, nsplit, rpT, norm, g, m, P, G, B, dB, dm, wB, wB_pk, pk_rp);
  return hipGetLastError();
}

// ============================================================================ weight-space dropout
// out[j, k] = keep[k] ? A[j, k] : 0 over an [r, K] factor (element size esz bytes), and the
// same masking in place on an fp32 gradient.  Exact (elements are copied or zeroed).
template <class T>
__global__ void mask_cols_kernel(const T* in, const uint8_t* keep, size_t rows, int K, T* out) {
  const size_t n = rows * (size_t)K;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    out[i] = keep[i % K] ? in[i] : T(0);
}

hipError_t launch_mask_cols(const void* in, const uint8_t* keep, int rows, int K, int esz, void* out, hipStream_t st) {
  const size_t n = (size_t)rows * K;
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  if (esz == 2)
    hipLaunchKernelGGL(mask_cols_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, st,
                       static_cast<const uint16_t*>(in), keep, (size_t)rows, K, static_cast<uint16_t*>(out));
  else
    hipLaunchKernelGGL(mask_cols_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, st, static_cast<const float*>(in),
                       keep, (size_t)rows, K, static_cast<float*>(out));
  return hipGetLastError();
}

// ============================================================================ 8-bit weight, dequantised
// out[n, k] = bf16(value(q[n, k]) * scale[n]) for int8 or e4m3 codes: the value times the
// scale rounded once to fp32, then to bf16 (the rounding the widening in the input-gradient
// tile applies).  16 codes per thread and step; K a multiple of 16, 16-byte aligned rows.
__global__ __launch_bounds__(256) void dequant8_kernel(const uint8_t* q, int N, int K, int ldq, const float* scale,
                                                       int fp8, uint16_t* out) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  const int per_row = K / 16;
  const size_t total = (size_t)N * per_row;
  for (size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (size_t)gridDim.x * blockDim.x) {
    const int n = (int)(t / per_row), c = (int)(t % per_row) * 16;
    const u32x4 v = ld16(q + (size_t)n * ldq + c);
    const float sc = scale[n];
    uint32_t o[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      f2 lo, hi;
      if (fp8) {
        lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[w], false) * sc;
        hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[w], true) * sc;
      } else {
        lo = f2{(float)(int8_t)(v[w] & 0xffu) * sc, (float)(int8_t)((v[w] >> 8) & 0xffu) * sc};
        hi = f2{(float)(int8_t)((v[w] >> 16) & 0xffu) * sc, (float)(int8_t)(v[w] >> 24) * sc};
      }
      o[2 * w] = pack_bf16x2(lo[0], lo[1]);
      o[2 * w + 1] = pack_bf16x2(hi[0], hi[1]);
    }
    uint16_t* dst = out + (size_t)n * K + c;
    st16(dst, u32x4{o[0], o[1], o[2], o[3]});
    st16(dst + 8, u32x4{o[4], o[5], o[6], o[7]});
  }
}

hipError_t launch_dequant8(const void* q, int N, int K, int ldq, const float* scale, int fp8, void* out,
                           hipStream_t st) {
  const size_t total = (size_t)N * (K / 16);
  if (total == 0) return hipSuccess;
  size_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(dequant8_kernel, dim3((unsigned)blocks), dim3(256), 0, st, static_cast<const uint8_t*>(q), N, K,
                     ldq, scale, fp8, static_cast<uint16_t*>(out));
  return hipGetLastError();
}

// ============================================================================ 8-bit quantisers
// Symmetric per-row codes with the quotient x / scale in fp32; scale 0 -> code 0.  One wave
// per row.  int8: scale = absmax / 127, code = clamp(rint(x / scale), +-127) (ties to even).
// e4m3 (FP8): scale = absmax / 448, code = the e4m3 rounding (nearest, ties to even) of the
// quotient clamped to +-448, by the hardware conversion.
template <bool FP8>
__device__ __forceinline__ uint32_t q8_code(float x, float sc) {
  if (!(sc > 0.f)) return 0u;
  if constexpr (FP8) {
    const float t = fminf(fmaxf(x / sc, -448.f), 448.f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(t, 0.f, 0, false) & 0xffu;
  } else {
    float t = rintf(x / sc);
    t = fminf(fmaxf(t, -127.f), 127.f);
    return (uint32_t)((int)t & 0xff);
  }
}

template <bool F32IN, bool FP8>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const void* X, int M, int K, int ldx, int8_t* q,
                                                            float* scale) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  float amax = 0.f;
  if (F32IN) {
    const float* x = static_cast<const float*>(X) + (size_t)row * ldx;
    for (int k = lane; k < K; k += 64) amax = fmaxf(amax, fabsf(x[k]));
  } else {
    const uint16_t* x = static_cast<const uint16_t*>(X) + (size_t)row * ldx;
    for (int k = lane * 8; k < K; k += 512) {
      const u32x4 v = ld16(x + k);
#pragma unroll
      for (int t = 0; t < 4; ++t) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(v[t])), fabsf(bf16_hi(v[t]))));
    }
  }
  amax = wave_max(amax);
  const float sc = amax / (FP8 ? 448.0f : 127.0f);
  if (lane == 0) scale[row] = sc;
  int8_t* qrow = q + (size_t)row * K;
  auto code = [&](float x) -> uint32_t { return q8_code<FP8>(x, sc); };
  if (F32IN) {
    const float* x = static_cast<const float*>(X) + (size_t)row * ldx;
    for (int k = lane; k < K; k += 64) qrow[k] = (int8_t)(uint8_t)code(x[k]);
  } else {
    const uint16_t* x = static_cast<const uint16_t*>(X) + (size_t)row * ldx;
    for (int k = lane * 8; k < K; k += 512) {
      const u32x4 v = ld16(x + k);
      u32x2 o;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t b0 = code(bf16_lo(v[2 * h]));
        const uint32_t b1 = code(bf16_hi(v[2 * h]));
        const uint32_t b2 = code(bf16_lo(v[2 * h + 1]));
        const uint32_t b3 = code(bf16_hi(v[2 * h + 1]));
        o[h] = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
      }
      *reinterpret_cast<u32x2*>(qrow + k) = o;
    }
  }
}

// bf16 rows of K <= 512 QV elements (K a multiple of 512): the same codes from one read of
// the row, kept in registers (QV 16-byte pieces per lane) between the absmax and the codes.
constexpr int kQuantRegPieces = 16;
template <bool FP8>
__global__ __launch_bounds__(256) void quantize_rows_reg_kernel(const uint16_t* X, int M, int K, int ldx, int8_t* q,
                                                                float* scale) {
  constexpr int QV = kQuantRegPieces;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const int nv = K / 512;
  const uint16_t* x = X + (size_t)row * ldx + lane * 8;
  u32x4 v[QV];
#pragma unroll
  for (int i = 0; i < QV; ++i) v[i] = i < nv ? ld16(x + i * 512) : u32x4{0u, 0u, 0u, 0u};
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < QV; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(v[i][t])), fabsf(bf16_hi(v[i][t]))));
  amax = wave_max(amax);
  const float sc = amax / (FP8 ? 448.0f : 127.0f);
  if (lane == 0) scale[row] = sc;
  auto code = [&](float xv) -> uint32_t { return q8_code<FP8>(xv, sc); };
  int8_t* qrow = q + (size_t)row * K + lane * 8;
#pragma unroll
  for (int i = 0; i < QV; ++i) {
    if (i < nv) {
      u32x2 o;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        o[h] = code(bf16_lo(v[i][2 * h])) | (code(bf16_hi(v[i][2 * h])) << 8) |
               (code(bf16_lo(v[i][2 * h + 1])) << 16) | (code(bf16_hi(v[i][2 * h + 1])) << 24);
      *reinterpret_cast<u32x2*>(qrow + i * 512) = o;
    }
  }
}

// X rows of leading dimension ldx (16-byte aligned rows for bf16), codes written as dense [M, K].
template <bool FP8>
static void quantize_rows_launch(const void* X, int in_f32, int M, int K, int ldx, int8_t* q, float* scale,
                                 hipStream_t st) {
  const dim3 grid((M + 3) / 4), block(256);
  if (in_f32) hipLaunchKernelGGL((quantize_rows_kernel<true, FP8>), grid, block, 0, st, X, M, K, ldx, q, scale);
  else if (K % 512 == 0 && K <= 512 * kQuantRegPieces &&
           (reinterpret_cast<uintptr_t>(X) & 15) == 0 && (reinterpret_cast<uintptr_t>(q) & 7) == 0)
    hipLaunchKernelGGL(quantize_rows_reg_kernel<FP8>, grid, block, 0, st, static_cast<const uint16_t*>(X), M, K, ldx,
                       q, scale);
  else hipLaunchKernelGGL((quantize_rows_kernel<false, FP8>), grid, block, 0, st, X, M, K, ldx, q, scale);
}

hipError_t launch_quantize_rows(const void* X, int in_f32, int M, int K, int ldx, int8_t* q, float* scale,
                                hipStream_t st, int fp8) {
  if (M <= 0) return hipSuccess;
  if (fp8) quantize_rows_launch<true>(X, in_f32, M, K, ldx, q, scale, st);
  else quantize_rows_launch<false>(X, in_f32, M, K, ldx, q, scale, st);
  return hipGetLastError();
}

// ============================================================================ fp32 path
// C[m,n] = alpha * sum_k A(m,k) B(k,n) + beta * C[m,n] (+ bias[n]); element strides are
// arbitrary, so the same kernel serves every product of the fp32 layer.  On
// v_mfma_f32_16x16x4_f32 (fp32 products and accumulation): one wave per 16 x 16 output tile,
// four waves per block (32 x 32).  The reduction index of MFMA c of a chunk is
// k0 + 4 c + (lane >> 4) on both operands; each lane loads its row of A and its column of B
// for the 16 MFMAs of the next chunk (64 k) while the current chunk is multiplied, so a
// small product waits for memory about once per chunk rather than once per load.  Rows,
// columns and k past the ends load as zero.
constexpr int kF32Chunk = 16;
__global__ __launch_bounds__(256) void f32_gemm_kernel(const F32GemmParams p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m0 = blockIdx.y * 32 + (wave >> 1) * 16, n0 = blockIdx.x * 32 + (wave & 1) * 16;
  const int lr = lane & 15, q = lane >> 4;
  const bool va = m0 + lr < p.M, vb = n0 + lr < p.N;
  const float* a = p.A + (long)(va ? m0 + lr : 0) * p.sam;
  const float* b = p.B + (long)(vb ? n0 + lr : 0) * p.sbn;
  float fa[kF32Chunk], fb[kF32Chunk], na[kF32Chunk], nb[kF32Chunk];
  auto load = [&](int k0, float* xa, float* xb) {
#pragma unroll
    for (int c = 0; c < kF32Chunk; ++c) {
      const int k = k0 + 4 * c + q;
      const bool kv = k < p.K;
      xa[c] = (va && kv) ? a[(long)k * p.sak] : 0.f;
      xb[c] = (vb && kv) ? b[(long)k * p.sbk] : 0.f;
    }
  };
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  load(0, fa, fb);
  for (int k0 = 0; k0 < p.K; k0 += 4 * kF32Chunk) {
    const bool more = k0 + 4 * kF32Chunk < p.K;
    if (more) load(k0 + 4 * kF32Chunk, na, nb);
#pragma unroll
    for (int c = 0; c < kF32Chunk; ++c) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[c], fb[c], acc, 0, 0, 0);
    if (more) {
#pragma unroll
      for (int c = 0; c < kF32Chunk; ++c) { fa[c] = na[c]; fb[c] = nb[c]; }
    }
  }
  // lane holds D[4 q + i][lr] of the 16 x 16 tile
  const int n = n0 + lr;
  if (n >= p.N) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + 4 * q + i;
    if (m >= p.M) continue;
    float v = p.alpha * acc[i];
    if (p.beta != 0.f) v += p.beta * p.C[(size_t)m * p.ldc + n];
    if (p.bias != nullptr) v += p.bias[n];
    p.C[(size_t)m * p.ldc + n] = v;
  }
}

__global__ void f32_colsum_kernel(const float* X, int M, int N, int ld, float* out) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  float acc = 0.f;
  for (int m = 0; m < M; ++m) acc += X[(size_t)m * ld + n];
  out[n] = acc;
}

hipError_t launch_f32_gemm(const F32GemmParams& p, hipStream_t st) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  const dim3 grid((p.N + 31) / 32, (p.M + 31) / 32), block(256);
  hipLaunchKernelGGL(f32_gemm_kernel, grid, block, 0, st, p);
  return hipGetLastError();
}

hipError_t launch_f32_colsum(const float* X, int M, int N, int ld, float* out, hipStream_t st) {
  hipLaunchKernelGGL(f32_colsum_kernel, dim3((N + 255) / 256), dim3(256), 0, st, X, M, N, ld, out);
  return hipGetLastError();
}

}  // namespace ldl
