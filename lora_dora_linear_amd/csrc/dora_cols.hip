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

// colsq[k] = sum_n W0[n,k]^2 (once per frozen W0): 32 columns per 1024-thread block, 8
// columns per thread (16-byte loads of bf16 rows) and 256 row phases, whose partial sums are
// combined in LDS by a fixed-order tree.
template <class T>
__global__ __launch_bounds__(1024) void col_sumsq_kernel(const T* W0, int N, int K, int ldw, float* colsq) {
  __shared__ float part[256][33];
  const int tid = threadIdx.x, cg = tid & 3, ph = tid >> 2;      // 4 groups of 8 columns, 256 phases
  const int c0 = blockIdx.x * 32 + cg * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (c0 < K)
    for (int n = ph; n < N; n += 256) {
      if constexpr (sizeof(T) == 2) {
        const u32x4 v = ld16(W0 + (size_t)n * ldw + c0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = bf16_lo(v[i]), b = bf16_hi(v[i]);
          acc[2 * i] = fmaf(a, a, acc[2 * i]);
          acc[2 * i + 1] = fmaf(b, b, acc[2 * i + 1]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float a = (c0 + i < K) ? W0[(size_t)n * ldw + c0 + i] : 0.f;
          acc[i] = fmaf(a, a, acc[i]);
        }
      }
    }
#pragma unroll
  for (int i = 0; i < 8; ++i) part[ph][cg * 8 + i] = acc[i];
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {                // phases ph and ph + h, then half as many
    for (int e = tid; e < h * 32; e += 1024) {
      const int q = e >> 5, c = e & 31;
      part[q][c] += part[q + h][c];
    }
    __syncthreads();
  }
  if (tid < 32 && blockIdx.x * 32 + tid < K) colsq[blockIdx.x * 32 + tid] = part[0][tid];
}

// Per input column k, the block's 16 columns by 16 rank groups: group q takes ranks j = q,
// q + 16, ..; A's columns (fp32) and Gc sit in LDS.  T_j = (Gc A)[j,k].
constexpr int kColBlk = 16, kRankGroups = 16;

__device__ __forceinline__ void stage_cols(const uint16_t* A, const float* Gc, int K, int r, int k0,
                                           float (*sa)[kColBlk], float* sg) {
  for (int e = threadIdx.x; e < r * kColBlk; e += 256) {
    const int j = e / kColBlk, c = e % kColBlk;
    sa[j][c] = (k0 + c < K) ? bf16_to_f32(A[(size_t)j * K + k0 + c]) : 0.f;
  }
  for (int e = threadIdx.x; e < r * r; e += 256) sg[e] = Gc[e];
}

// nu_k, g_k = m_k / max(nu_k, eps): per column, lin = <A_k, Pc_k> and quad = A_k^T Gc A_k from
// the rank groups' partial sums, combined in group order
__global__ __launch_bounds__(256) void dora_cols_norm_kernel(int K, int r, float s, float eps, const float* colsq,
                                                             const float* m, const uint16_t* A, const float* Pc,
                                                             const float* Gc, float* norm, float* g) {
  __shared__ float sa[64][kColBlk];
  __shared__ float sg[64 * 64];
  __shared__ float pl[kRankGroups][kColBlk], pq[kRankGroups][kColBlk];
  const int k0 = blockIdx.x * kColBlk, c = threadIdx.x % kColBlk, q = threadIdx.x / kColBlk, k = k0 + c;
  stage_cols(A, Gc, K, r, k0, sa, sg);
  __syncthreads();
  float lin = 0.f, quad = 0.f;
  if (k < K)
    for (int j = q; j < r; j += kRankGroups) {
      float t = 0.f;
      for (int i = 0; i < r; ++i) t = fmaf(sg[j * r + i], sa[i][c], t);
      lin = fmaf(sa[j][c], Pc[(size_t)j * K + k], lin);
      quad = fmaf(sa[j][c], t, quad);
    }
  pl[q][c] = lin;
  pq[q][c] = quad;
  __syncthreads();
  if (q == 0 && k < K) {
    for (int u = 1; u < kRankGroups; ++u) { lin += pl[u][c]; quad += pq[u][c]; }
    const float c2 = colsq[k] + 2.f * s * lin + s * s * quad;
    const float nu = sqrtf(fmaxf(c2, 0.f));
    norm[k] = nu;
    g[k] = m[k] / fmaxf(nu, eps);
  }
}

// Backward norm terms per column k, from dg_k = sum_m dXs[m,k] X[m,k]:
//   dm_k = dg_k / max(nu_k, eps);  w_k = -dg_k m_k / (2 nu_k^3) (0 where nu_k <= eps);
//   dA[:,k] += 2s w_k (Pc[:,k] + s Gc A[:,k]);
//   Aw = A.diag(w) as bf16 hi ([0, r) rows) and lo ([r, 2r) rows) for the dB products.
__global__ __launch_bounds__(256) void dora_cols_bwd_kernel(int K, int r, float s, float eps, const float* dg_part,
                                                            int dg_nsplit, const float* norm, const float* m,
                                                            const uint16_t* A,
                                                            const float* Pc, const float* Gc, float* dm, float* dA,
                                                            uint16_t* Aw) {
  __shared__ float sa[64][kColBlk];
  __shared__ float sg[64 * 64];
  const int k0 = blockIdx.x * kColBlk, c = threadIdx.x % kColBlk, q = threadIdx.x / kColBlk, k = k0 + c;
  // dg_k: the split partial sums in split order, eight loads in flight, issued before the
  // staging so that their latency overlaps it
  float d = 0.f;
  if (k < K) {
    int sp = 0;
    for (; sp + 8 <= dg_nsplit; sp += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = dg_part[(size_t)(sp + u) * K + k];
#pragma unroll
      for (int u = 0; u < 8; ++u) d += v[u];
    }
    for (; sp < dg_nsplit; ++sp) d += dg_part[(size_t)sp * K + k];
  }
  stage_cols(A, Gc, K, r, k0, sa, sg);
  __syncthreads();
  if (k >= K) return;
  const float nu = norm[k];
  if (q == 0) dm[k] = d / fmaxf(nu, eps);
  const float w = nu > eps ? -d * m[k] / (2.f * nu * nu * nu) : 0.f;
  for (int j = q; j < r; j += kRankGroups) {
    float t = 0.f;
    for (int i = 0; i < r; ++i) t = fmaf(sg[j * r + i], sa[i][c], t);
    const size_t o = (size_t)j * K + k;
    dA[o] += 2.f * s * w * (Pc[o] + s * t);
    const float v = sa[j][c] * w;
    const uint32_t hi = f32_to_bf16_bits(v);
    Aw[o] = (uint16_t)hi;
    Aw[(size_t)(r + j) * K + k] = (uint16_t)f32_to_bf16_bits(v - __uint_as_float(hi << 16));
  }
}

// dB[n,j] += 2s (T[n,j] + T[n,r+j]) + 2s^2 sum_i B[n,i] (H[i,j] + H[i,r+j]) with
// T = W0.Aw^T [N, 2r] (hi | lo halves) and H = A.Aw^T = A.diag(w).A^T in rows N .. N+r-1;
// H (hi + lo) staged in LDS, one thread per (n, j).
__global__ __launch_bounds__(256) void dora_cols_db_kernel(int N, int r, float s, const uint16_t* B, const float* T,
                                                           float* dB) {
  __shared__ float sh[64 * 64];
  const float* H = T + (size_t)N * 2 * r;
  for (int e = threadIdx.x; e < r * r; e += 256) {
    const int i = e / r, j = e % r;
    sh[e] = H[(size_t)i * 2 * r + j] + H[(size_t)i * 2 * r + r + j];
  }
  __syncthreads();
  const size_t total = (size_t)N * r;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (size_t)gridDim.x * blockDim.x) {
    const int n = (int)(e / r), j = (int)(e % r);
    float q = 0.f;
    for (int i = 0; i < r; ++i) q = fmaf(bf16_to_f32(B[(size_t)n * r + i]), sh[i * r + j], q);
    const float* tr = T + (size_t)n * 2 * r;
    dB[e] += 2.f * s * (tr[j] + tr[r + j]) + 2.f * s * s * q;
  }
}

}  // namespace

hipError_t launch_col_sumsq(const void* W0, int bf16, int N, int K, int ldw, float* colsq, hipStream_t st) {
  if (K <= 0) return hipSuccess;
  const dim3 grid((K + 31) / 32), block(1024);
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
  if (r > 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dora_cols_norm_kernel, dim3((K + kColBlk - 1) / kColBlk), dim3(256), 0, st, K, r, s, eps,
                     colsq, m, static_cast<const uint16_t*>(A), Pc, Gc, norm, g);
  return hipGetLastError();
}

hipError_t launch_dora_cols_bwd(int K, int r, float s, float eps, const float* dg_part, int dg_nsplit,
                                const float* norm, const float* m, const void* A, const float* Pc, const float* Gc,
                                float* dm, float* dA, void* Aw, hipStream_t st) {
  if (r > 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dora_cols_bwd_kernel, dim3((K + kColBlk - 1) / kColBlk), dim3(256), 0, st, K, r, s, eps,
                     dg_part, dg_nsplit, norm, m, static_cast<const uint16_t*>(A), Pc, Gc, dm, dA, static_cast<uint16_t*>(Aw));
  return hipGetLastError();
}

hipError_t launch_dora_cols_db(int N, int r, float s, const void* B, const float* T, float* dB, hipStream_t st) {
  if (r > 64) return hipErrorInvalidValue;
  const size_t total = (size_t)N * r;
  if (total == 0) return hipSuccess;
  size_t blocks = (total + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(dora_cols_db_kernel, dim3((unsigned)blocks), dim3(256), 0, st, N, r, s,
                     static_cast<const uint16_t*>(B), T, dB);
  return hipGetLastError();
}

}  // namespace ldl
