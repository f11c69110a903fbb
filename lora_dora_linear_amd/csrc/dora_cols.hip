// Column-scaled DoRA ("dora-cols"): the norm of each input column k of the adapted weight
// W' = W0 + s.B.A, from the closed form
//   nu_k^2 = colsum(W0^2)_k + 2s <A[:,k], Pc[:,k]> + s^2 A[:,k]^T Gc A[:,k],
//   Pc = B^T.W0 [r,K],  Gc = B^T.B [r,r],
// so no [N,K] tensor beyond W0 itself is read ("LoRA/DoRA fast forward: no weight
// materialization", sections "What" and "Fidelity": the same closed-form expansion as the
// row form, norm in the graph, eps clamp).  The magnitude over the norm then scales the
// layer input per feature.  These kernels are the rank-sized pieces around the LoRA
// products: the cached column sums of W0^2, the norm, and the backward's norm terms.
#include "internal.hpp"

namespace ldl {

namespace {

// colsq[k] = sum_n W0[n,k]^2: 64 columns per block, four row phases per column summed in a
// fixed order (once per frozen W0)
template <class T>
__global__ __launch_bounds__(256) void col_sumsq_kernel(const T* W0, int N, int K, int ldw, float* colsq) {
  __shared__ float part[4][64];
  const int c = blockIdx.x * 64 + (threadIdx.x & 63), ph = threadIdx.x >> 6;
  float acc = 0.f;
  if (c < K)
    for (int n = ph; n < N; n += 4) {
      float v;
      if constexpr (sizeof(T) == 2) v = bf16_to_f32(W0[(size_t)n * ldw + c]);
      else v = W0[(size_t)n * ldw + c];
      acc = fmaf(v, v, acc);
    }
  part[ph][threadIdx.x & 63] = acc;
  __syncthreads();
  if (ph == 0 && c < K) colsq[c] = ((part[0][threadIdx.x] + part[1][threadIdx.x]) + part[2][threadIdx.x]) +
                                   part[3][threadIdx.x];
}

// One thread per column k (64 per block): the block's A columns are staged in LDS as fp32
// [r][64]; q_j = sum_i Gc[j,i] A[i,k] reads Gc with one address per wave.
constexpr int kColBlk = 64;

__device__ __forceinline__ void stage_a_cols(const uint16_t* A, int K, int r, int k0, float (*sa)[kColBlk]) {
  for (int e = threadIdx.x; e < r * kColBlk; e += kColBlk) {
    const int j = e / kColBlk, c = e % kColBlk;
    sa[j][c] = (k0 + c < K) ? bf16_to_f32(A[(size_t)j * K + k0 + c]) : 0.f;
  }
}

// nu_k, g_k = m_k / max(nu_k, eps)
__global__ __launch_bounds__(kColBlk) void dora_cols_norm_kernel(int K, int r, float s, float eps, const float* colsq,
                                                                 const float* m, const uint16_t* A, const float* Pc,
                                                                 const float* Gc, float* norm, float* g) {
  __shared__ float sa[128][kColBlk];
  const int k0 = blockIdx.x * kColBlk, t = threadIdx.x, k = k0 + t;
  stage_a_cols(A, K, r, k0, sa);
  __syncthreads();
  if (k >= K) return;
  float lin = 0.f, quad = 0.f;
  for (int j = 0; j < r; ++j) {
    float q = 0.f;
    for (int i = 0; i < r; ++i) q = fmaf(Gc[j * r + i], sa[i][t], q);
    lin = fmaf(sa[j][t], Pc[(size_t)j * K + k], lin);
    quad = fmaf(sa[j][t], q, quad);
  }
  const float c2 = colsq[k] + 2.f * s * lin + s * s * quad;
  const float nu = sqrtf(fmaxf(c2, 0.f));
  norm[k] = nu;
  g[k] = m[k] / fmaxf(nu, eps);
}

// Backward norm terms per column k, from dg_k = sum_m dXs[m,k] X[m,k]:
//   dm_k = dg_k / max(nu_k, eps);  w_k = -dg_k m_k / (2 nu_k^3) (0 where nu_k <= eps);
//   dA[:,k] += 2s w_k (Pc[:,k] + s Gc A[:,k]);
//   Aw = A.diag(w) as bf16 hi ([0, r) rows) and lo ([r, 2r) rows) for the dB products.
__global__ __launch_bounds__(kColBlk) void dora_cols_bwd_kernel(int K, int r, float s, float eps, const float* dg,
                                                                const float* norm, const float* m, const uint16_t* A,
                                                                const float* Pc, const float* Gc, float* dm,
                                                                float* dA, uint16_t* Aw) {
  __shared__ float sa[128][kColBlk];
  const int k0 = blockIdx.x * kColBlk, t = threadIdx.x, k = k0 + t;
  stage_a_cols(A, K, r, k0, sa);
  __syncthreads();
  if (k >= K) return;
  const float nu = norm[k], d = dg[k];
  dm[k] = d / fmaxf(nu, eps);
  const float w = nu > eps ? -d * m[k] / (2.f * nu * nu * nu) : 0.f;
  for (int j = 0; j < r; ++j) {
    float q = 0.f;
    for (int i = 0; i < r; ++i) q = fmaf(Gc[j * r + i], sa[i][t], q);
    const size_t o = (size_t)j * K + k;
    dA[o] += 2.f * s * w * (Pc[o] + s * q);
    const float v = sa[j][t] * w;
    const uint32_t hi = f32_to_bf16_bits(v);
    Aw[o] = (uint16_t)hi;
    Aw[(size_t)(r + j) * K + k] = (uint16_t)f32_to_bf16_bits(v - __uint_as_float(hi << 16));
  }
}

// dB[n,j] += 2s (T[n,j] + T[n,r+j]) + 2s^2 sum_i B[n,i] (H[i,j] + H[i,r+j]) with
// T = W0.Aw^T [N, 2r] (hi | lo halves) and H = A.Aw^T = A.diag(w).A^T in rows N .. N+r-1.
__global__ __launch_bounds__(256) void dora_cols_db_kernel(int N, int r, float s, const uint16_t* B, const float* T,
                                                           float* dB) {
  const size_t total = (size_t)N * r;
  const float* H = T + (size_t)N * 2 * r;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (size_t)gridDim.x * blockDim.x) {
    const int n = (int)(e / r), j = (int)(e % r);
    float q = 0.f;
    for (int i = 0; i < r; ++i)
      q = fmaf(bf16_to_f32(B[(size_t)n * r + i]), H[(size_t)i * 2 * r + j] + H[(size_t)i * 2 * r + r + j], q);
    const float* tr = T + (size_t)n * 2 * r;
    dB[e] += 2.f * s * (tr[j] + tr[r + j]) + 2.f * s * s * q;
  }
}

}  // namespace

hipError_t launch_col_sumsq(const void* W0, int bf16, int N, int K, int ldw, float* colsq, hipStream_t st) {
  if (K <= 0) return hipSuccess;
  const dim3 grid((K + 63) / 64), block(256);
  if (bf16)
    hipLaunchKernelGGL(col_sumsq_kernel<uint16_t>, grid, block, 0, st, static_cast<const uint16_t*>(W0), N, K, ldw,
                       colsq);
  else
    hipLaunchKernelGGL(col_sumsq_kernel<float>, grid, block, 0, st, static_cast<const float*>(W0), N, K, ldw, colsq);
  return hipGetLastError();
}

hipError_t launch_dora_cols_norm(int K, int r, float s, float eps, const float* colsq, const float* m,
                                 const void* A, const float* Pc, const float* Gc, float* norm, float* g,
                                 hipStream_t st) {
  if (r > 128) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dora_cols_norm_kernel, dim3((K + kColBlk - 1) / kColBlk), dim3(kColBlk), 0, st, K, r, s, eps,
                     colsq, m, static_cast<const uint16_t*>(A), Pc, Gc, norm, g);
  return hipGetLastError();
}

hipError_t launch_dora_cols_bwd(int K, int r, float s, float eps, const float* dg, const float* norm, const float* m,
                                const void* A, const float* Pc, const float* Gc, float* dm, float* dA, void* Aw,
                                hipStream_t st) {
  if (r > 128) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dora_cols_bwd_kernel, dim3((K + kColBlk - 1) / kColBlk), dim3(kColBlk), 0, st, K, r, s, eps, dg,
                     norm, m, static_cast<const uint16_t*>(A), Pc, Gc, dm, dA, static_cast<uint16_t*>(Aw));
  return hipGetLastError();
}

hipError_t launch_dora_cols_db(int N, int r, float s, const void* B, const float* T, float* dB, hipStream_t st) {
  const size_t total = (size_t)N * r;
  if (total == 0) return hipSuccess;
  size_t blocks = (total + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(dora_cols_db_kernel, dim3((unsigned)blocks), dim3(256), 0, st, N, r, s,
                     static_cast<const uint16_t*>(B), T, dB);
  return hipGetLastError();
}

}  // namespace ldl
