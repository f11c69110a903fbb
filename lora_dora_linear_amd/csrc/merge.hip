// LoRA merge: the adapted weight formed explicitly, W_out = W0 + s.B.A (or the delta s.B.A
// alone), for export or for merging an adapter into its base weight ("Fused Kernels
// (experimental)", section "What is fused": the merge kernels of the lora family).  The
// rank-r product is generated tile by tile in registers and written once; HBM-bound
// (read W0, write W_out).
#include "internal.hpp"

namespace ldl {

namespace {

// Block tile 64 rows x 128 columns, 256 threads; thread t computes rows 4 (t / 16) .. +3 and
// columns 8 (t % 16) .. +7.  The block's slice of A ([r][128], as fp32) and of B ([r][64] in
// rank-major order, so a thread reads its four rows' values of one rank as one 16-byte
// vector) are staged in LDS in chunks of up to 32 ranks.
template <class T>
__device__ __forceinline__ void load8(const T* p, float* v);
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float* v) {
  const u32x4 w = ld16(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[2 * i] = bf16_lo(w[i]); v[2 * i + 1] = bf16_hi(w[i]); }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* v) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
}
template <class T>
__device__ __forceinline__ void store8(T* p, const float* v);
template <>
__device__ __forceinline__ void store8<uint16_t>(uint16_t* p, const float* v) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
  st16(p, w);
}
template <>
__device__ __forceinline__ void store8<float>(float* p, const float* v) {
  *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}
template <class T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t v) { return bf16_to_f32(v); }
template <>
__device__ __forceinline__ float to_f32<float>(float v) { return v; }

constexpr int kMergeRC = 32;   // ranks per LDS chunk

template <class T>
__global__ __launch_bounds__(256) void merge_kernel(int N, int K, int r, float s, const T* W0, int ldw, const T* A,
                                                    const T* B, T* W, int ldo) {
  __shared__ float sa[kMergeRC][128];
  __shared__ float sb[kMergeRC][64];
  const int tid = threadIdx.x;
  const int n0 = blockIdx.y * 64, k0 = blockIdx.x * 128;
  const int rt = 4 * (tid >> 4), ct = 8 * (tid & 15);
  float acc[4][8] = {};
  for (int j0 = 0; j0 < r; j0 += kMergeRC) {
    const int rc = min(kMergeRC, r - j0);
    __syncthreads();
    // A[j0 .. j0 + rc)[k0 .. k0 + 128): 16 threads per rank row, 8 columns each
    for (int e = tid; e < rc * 16; e += 256) {
      const int j = e >> 4, c = 8 * (e & 15);
      float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (k0 + c < K) load8<T>(A + (size_t)(j0 + j) * K + k0 + c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) sa[j][c + i] = v[i];
    }
    // B[n0 .. n0 + 64)[j0 .. j0 + rc) transposed to rank-major
    for (int e = tid; e < rc * 64; e += 256) {
      const int row = e / rc, j = e % rc;
      sb[j][row] = (n0 + row < N) ? to_f32<T>(B[(size_t)(n0 + row) * r + j0 + j]) : 0.f;
    }
    __syncthreads();
    for (int j = 0; j < rc; ++j) {
      const f32x4 b4 = *reinterpret_cast<const f32x4*>(&sb[j][rt]);
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(&sa[j][ct]);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(&sa[j][ct + 4]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          acc[i][c] = fmaf(b4[i], a0[c], acc[i][c]);
          acc[i][4 + c] = fmaf(b4[i], a1[c], acc[i][4 + c]);
        }
    }
  }
  if (k0 + ct >= K) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = n0 + rt + i;
    if (n >= N) break;
    float v[8];
    if (W0 != nullptr) load8<T>(W0 + (size_t)n * ldw + k0 + ct, v);
    else {
#pragma unroll
      for (int c = 0; c < 8; ++c) v[c] = 0.f;
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] += s * acc[i][c];
    store8<T>(W + (size_t)n * ldo + k0 + ct, v);
  }
}

__global__ void bf16_to_f32_kernel(const uint16_t* in, size_t n, float* out) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    out[i] = bf16_to_f32(in[i]);
}

}  // namespace

hipError_t launch_merge(int N, int K, int r, float s, int bf16, const void* W0, int ldw, const void* A, const void* B,
                        void* W, int ldo, hipStream_t st) {
  if (N <= 0 || K <= 0) return hipSuccess;
  const dim3 grid((K + 127) / 128, (N + 63) / 64), block(256);
  if (bf16)
    hipLaunchKernelGGL(merge_kernel<uint16_t>, grid, block, 0, st, N, K, r, s, static_cast<const uint16_t*>(W0), ldw,
                       static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B), static_cast<uint16_t*>(W),
                       ldo);
  else
    hipLaunchKernelGGL(merge_kernel<float>, grid, block, 0, st, N, K, r, s, static_cast<const float*>(W0), ldw,
                       static_cast<const float*>(A), static_cast<const float*>(B), static_cast<float*>(W), ldo);
  return hipGetLastError();
}

hipError_t launch_bf16_to_f32(const void* in, size_t n, float* out, hipStream_t st) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(bf16_to_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, st, static_cast<const uint16_t*>(in), n,
                     out);
  return hipGetLastError();
}

}  // namespace ldl
