// The fp32 LoRA layer at small sizes (the launch-bound tiny configuration): the forward in
// one launch and the backward in one launch, on v_mfma_f32_16x16x4_f32 (fp32 products and
// accumulation), instead of one GEMM launch per product.  At these sizes a launch is bound by
// load latency, so every block issues all the loads of its reduction at once and the four
// waves of a block split the reduction, their partial sums added in wave order through LDS.
//
// Forward (LoRA bypass form: the adapter's down-projection, then its up-projection added to
// the frozen product): one block per 16 x 16 tile of Y; its K loop multiplies the X rows against
// the W0 rows and against the rank rows of A at once, so U = X.A^T for its 16 rows comes with
// Y = X.W0^T; s.U is then turned into the MFMA row operand through LDS and multiplied with B^T
// (r <= 16: one rank block).  The blocks of the first column of tiles store U.
// Backward: every block takes one job: a 16 x 16 tile of dX = dY.W0 + s.V.A (V = dY.B for its
// 16 rows computed alongside, as U in the forward), a 16-column tile of dA = s.V^T.X (the
// waves take the row blocks in turn, V of each first), or a 16-row tile of dB = s.dY^T.U (U
// read, or recomputed exactly as the forward computes it) with the column sums of dY (dbias).
//
// MFMA operand convention (16x16x4, fp32): lane l = 16 q + lr carries row lr of the A operand
// and column lr of the B operand; in a group of four steps lane q holds reduction indices
// 16 g + 4 q .. + 3 (one 16-byte load where the operand is contiguous along the reduction).
// The result lane holds D[4 q + i][lr].  Reductions run in a fixed order, so a quantity that
// two jobs compute (U in the forward and in dB) has the same bits.
#include "internal.hpp"

namespace ldl {

namespace {

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// acc1 += A.B1 (and acc2 += A.B2 if TWO) over reduction indices [lo, hi), lo and hi multiples
// of 4: la(k) / lb1(k) / lb2(k) give this lane's four operand values at k .. k + 3.  Chunks of
// 256 indices; a chunk's loads are all issued before its first MFMA.
template <bool TWO, class LA, class LB1, class LB2>
__device__ __forceinline__ void reduce_q(int lo, int hi, int q, LA la, LB1 lb1, LB2 lb2, f32x4& acc1, f32x4& acc2) {
  for (int k0 = lo; k0 < hi; k0 += 256) {
    f32x4 va[16], v1[16], v2[16];
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      const int k = k0 + 16 * g + 4 * q;
      const bool kv = k < hi;
      va[g] = kv ? la(k) : f32x4{0.f, 0.f, 0.f, 0.f};
      v1[g] = kv ? lb1(k) : f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (TWO) v2[g] = kv ? lb2(k) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int g = 0; g < 16; ++g)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        acc1 = mfma4(va[g][u], v1[g][u], acc1);
        if constexpr (TWO) acc2 = mfma4(va[g][u], v2[g][u], acc2);
      }
  }
}

__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 ld4s(const float* p, size_t stride) {
  return f32x4{p[0], p[stride], p[2 * stride], p[3 * stride]};
}
constexpr f32x4 kZero4 = {0.f, 0.f, 0.f, 0.f};

// A result tile (lane holds D[4 q + i][lr]) times scale into an LDS tile t[row][col]
__device__ __forceinline__ void to_lds(float (*t)[17], f32x4 v, float scale, int q, int lr) {
#pragma unroll
  for (int i = 0; i < 4; ++i) t[4 * q + i][lr] = v[i] * scale;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // (the wave reads other lanes' values next)
}

// sum over the four waves' partials part[w][lane], in wave order
__device__ __forceinline__ f32x4 wave_sum4(const f32x4 (*part)[64], int lane) {
  return ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
}

struct F32SmallFwd {
  int M, N, K, r;
  float s;
  const float* X; int ldx;
  const float* W0; int ldw;
  const float* A;              // [r, K] dense
  const float* B;              // [N, r] dense
  const float* bias;
  float* Y; int ldy;
  float* U; int ldu;           // optional
};

// U tile partial of wave w: X rows m0.. against the rank rows of A over K quarter w
__device__ __forceinline__ void u_partial(const float* X, int ldx, const float* A, int M, int K, int r, int m0, int w,
                                          int q, int lr, f32x4& acc) {
  const bool vm = m0 + lr < M, vj = lr < r;
  const float* xr = X + (size_t)(vm ? m0 + lr : 0) * ldx;
  const float* ar = A + (size_t)(vj ? lr : 0) * K;
  f32x4 unused = kZero4;
  const int part = K / 4;
  reduce_q<false>(w * part, (w + 1) * part, q, [&](int k) { return vm ? ld4(xr + k) : kZero4; },
                  [&](int k) { return vj ? ld4(ar + k) : kZero4; }, [&](int) { return kZero4; }, acc, unused);
}

__global__ __launch_bounds__(256) void f32_small_fwd_kernel(const F32SmallFwd p) {
  __shared__ f32x4 part[2][4][64];
  __shared__ float su[16][17];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, q = lane >> 4;
  const int m0 = blockIdx.y * 16, n0 = blockIdx.x * 16;
  const bool vm = m0 + lr < p.M, vn = n0 + lr < p.N, vj = lr < p.r;
  const float* xr = p.X + (size_t)(vm ? m0 + lr : 0) * p.ldx;
  const float* wr = p.W0 + (size_t)(vn ? n0 + lr : 0) * p.ldw;
  const float* ar = p.A + (size_t)(vj ? lr : 0) * p.K;
  // the rank slab of B and the bias, loaded before the reduction so that their latency
  // overlaps it (r <= 16: four rank groups of four)
  float bv[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int j = 4 * c + q;
    bv[c] = (vn && j < p.r) ? p.B[(size_t)(n0 + lr) * p.r + j] : 0.f;
  }
  const float bn = (p.bias != nullptr && vn) ? p.bias[n0 + lr] : 0.f;
  f32x4 accY = kZero4, accU = kZero4;
  const int kq = p.K / 4;
  reduce_q<true>(wave * kq, (wave + 1) * kq, q, [&](int k) { return vm ? ld4(xr + k) : kZero4; },
                 [&](int k) { return vn ? ld4(wr + k) : kZero4; }, [&](int k) { return vj ? ld4(ar + k) : kZero4; },
                 accY, accU);
  part[0][wave][lane] = accY;
  part[1][wave][lane] = accU;
  __syncthreads();
  if (wave != 0) return;
  accY = wave_sum4(part[0], lane);
  accU = wave_sum4(part[1], lane);
  // U (unscaled) from the first column of tiles
  if (p.U != nullptr && n0 == 0 && lr < p.r) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (m0 + 4 * q + i < p.M) p.U[(size_t)(m0 + 4 * q + i) * p.ldu + lr] = accU[i];
  }
  // + (s.U).B^T: s.U as the row operand (rank = reduction index) through LDS
  to_lds(su, accU, p.s, q, lr);
#pragma unroll
  for (int c = 0; c < 4; ++c)
    if (4 * c < p.r) accY = mfma4(su[lr][4 * c + q], bv[c], accY);
  if (!vn) return;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (m0 + 4 * q + i < p.M) p.Y[(size_t)(m0 + 4 * q + i) * p.ldy + n0 + lr] = accY[i] + bn;
}

struct F32SmallBwd {
  int M, N, K, r;
  float s;
  const float* dY; int lddy;
  const float* X; int ldx;
  const float* W0; int ldw;
  const float* A;              // [r, K]
  const float* B;              // [N, r]
  const float* U; int ldu;     // optional: recomputed from X and A when null
  float* dX; int lddx;         // optional
  float* dA;                   // [r, K]
  float* dB;                   // [N, r]
  float* dbias;                // optional
  int ndx, nda, ndb;           // jobs of each kind (dX tiles, dA column tiles, dB row tiles)
};

__global__ __launch_bounds__(256) void f32_small_bwd_kernel(const F32SmallBwd p) {
  __shared__ f32x4 part[3][4][64];
  __shared__ float st[4][16][17];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, q = lane >> 4;
  float (*t)[17] = st[wave];
  const bool vj = lr < p.r;
  int job = blockIdx.x;
  if (job < p.ndx) {
    // dX tile (m0, c0): the waves take quarters of N: dY rows against the W0 columns c0.. and
    // the rank columns of B (V); then wave 0 adds (s.V).A
    const int tk = (p.K + 15) / 16;
    const int m0 = (job / tk) * 16, c0 = (job % tk) * 16;
    const bool vm = m0 + lr < p.M, vc = c0 + lr < p.K;
    const float* dyr = p.dY + (size_t)(vm ? m0 + lr : 0) * p.lddy;
    const float* wc = p.W0 + c0 + (vc ? lr : 0);
    const float* bc = p.B + (vj ? lr : 0);
    float av[4];                               // A's rank rows at the tile's columns, prefetched
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = 4 * c + q;
      av[c] = (vc && j < p.r) ? p.A[(size_t)j * p.K + c0 + lr] : 0.f;
    }
    f32x4 accX = kZero4, accV = kZero4;
    const int nq = p.N / 4;
    reduce_q<true>(wave * nq, (wave + 1) * nq, q, [&](int n) { return vm ? ld4(dyr + n) : kZero4; },
                   [&](int n) { return vc ? ld4s(wc + (size_t)n * p.ldw, p.ldw) : kZero4; },
                   [&](int n) { return vj ? ld4s(bc + (size_t)n * p.r, p.r) : kZero4; }, accX, accV);
    part[0][wave][lane] = accX;
    part[1][wave][lane] = accV;
    __syncthreads();
    if (wave != 0) return;
    accX = wave_sum4(part[0], lane);
    accV = wave_sum4(part[1], lane);
    to_lds(t, accV, p.s, q, lr);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (4 * c < p.r) accX = mfma4(t[lr][4 * c + q], av[c], accX);
    if (!vc) return;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (m0 + 4 * q + i < p.M) p.dX[(size_t)(m0 + 4 * q + i) * p.lddx + c0 + lr] = accX[i];
    return;
  }
  job -= p.ndx;
  if (job < p.nda) {
    // dA columns c0..c0+15: wave w takes the row blocks w, w + 4, ..: V of the block (dY rows
    // against the rank columns of B over all of N), then (s.V)^T.X of the block
    const int c0 = job * 16;
    const bool vc = c0 + lr < p.K;
    const float* bc = p.B + (vj ? lr : 0);
    f32x4 accA = kZero4;
    for (int m0 = wave * 16; m0 < p.M; m0 += 64) {
      const bool vm = m0 + lr < p.M;
      const float* dyr = p.dY + (size_t)(vm ? m0 + lr : 0) * p.lddy;
      float xv[4];                             // X[m][c0 + lr] of the block's rows, prefetched
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int mm = 4 * c + q;
        xv[c] = (vc && m0 + mm < p.M) ? p.X[(size_t)(m0 + mm) * p.ldx + c0 + lr] : 0.f;
      }
      f32x4 accV = kZero4, unused = kZero4;
      reduce_q<false>(0, p.N, q, [&](int n) { return vm ? ld4(dyr + n) : kZero4; },
                      [&](int n) { return vj ? ld4s(bc + (size_t)n * p.r, p.r) : kZero4; },
                      [&](int) { return kZero4; }, accV, unused);
      to_lds(t, accV, p.s, q, lr);
      // row operand: (s.V)^T (rank lr, reduction index = row 4 c + q of the block); column
      // operand: X[m][c0 + lr]
#pragma unroll
      for (int c = 0; c < 4; ++c) accA = mfma4(t[4 * c + q][lr], xv[c], accA);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // (the tile is rewritten next)
    }
    part[0][wave][lane] = accA;
    __syncthreads();
    if (wave != 0 || !vc) return;
    accA = wave_sum4(part[0], lane);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * q + i < p.r) p.dA[(size_t)(4 * q + i) * p.K + c0 + lr] = accA[i];
    return;
  }
  job -= p.nda;
  if (job < p.ndb) {
    // dB rows n0..n0+15: wave w takes the row blocks w, w + 4, ..: s.dY^T.U of the block (U
    // read, or recomputed as the forward computes it: four K quarters added in order) and the
    // column sums of dY
    const int n0 = job * 16;
    const bool vn = n0 + lr < p.N;
    f32x4 accB = kZero4;
    float csum = 0.f;
    for (int m0 = wave * 16; m0 < p.M; m0 += 64) {
      if (p.U == nullptr) {
        f32x4 pu[4] = {kZero4, kZero4, kZero4, kZero4};
#pragma unroll
        for (int w = 0; w < 4; ++w) u_partial(p.X, p.ldx, p.A, p.M, p.K, p.r, m0, w, q, lr, pu[w]);
        to_lds(t, ((pu[0] + pu[1]) + pu[2]) + pu[3], 1.f, q, lr);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int m = m0 + 4 * c + q;
        const float a = (vn && m < p.M) ? p.dY[(size_t)m * p.lddy + n0 + lr] : 0.f;
        float b = 0.f;
        if (m < p.M && vj) b = p.U != nullptr ? p.U[(size_t)m * p.ldu + lr] : t[4 * c + q][lr];
        accB = mfma4(a, b, accB);
        csum += a;
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    part[0][wave][lane] = accB;
    part[1][wave][lane] = f32x4{csum, 0.f, 0.f, 0.f};
    __syncthreads();
    if (wave != 0) return;
    accB = wave_sum4(part[0], lane);
    if (p.dbias != nullptr) {
      // each column's partial sums: four row phases (q) of four waves, waves first
      t[q][lr] = wave_sum4(part[1], lane)[0];
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (q == 0 && vn) p.dbias[n0 + lr] = ((t[0][lr] + t[1][lr]) + t[2][lr]) + t[3][lr];
    }
    if (!vn) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + 4 * q + i;
      if (n < p.N && lr < p.r) p.dB[(size_t)n * p.r + lr] = p.s * accB[i];
    }
  }
}

}  // namespace

// Sizes where one block's loads stay within a few chunks of 256 (the reductions are split in
// four quarters of whole 4-index steps: K and N multiples of 16) and the dA / dB jobs walk few
// row blocks.  The caller also keeps the rows that take 16-byte loads 16-byte aligned.
bool f32_small_ok(int M, int N, int K, int r) {
  return M > 0 && M <= 256 && r > 0 && r <= 16 && N % 16 == 0 && K % 16 == 0 && N <= 1024 && K <= 1024;
}

hipError_t launch_f32_small_fwd(int M, int N, int K, int r, float s, const float* X, int ldx, const float* W0,
                                int ldw, const float* A, const float* B, const float* bias, float* Y, int ldy,
                                float* U, int ldu, hipStream_t st) {
  F32SmallFwd p{M, N, K, r, s, X, ldx, W0, ldw, A, B, bias, Y, ldy, U, ldu};
  hipLaunchKernelGGL(f32_small_fwd_kernel, dim3(N / 16, (M + 15) / 16), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_f32_small_bwd(int M, int N, int K, int r, float s, const float* dY, int lddy, const float* X,
                                int ldx, const float* W0, int ldw, const float* A, const float* B, const float* U,
                                int ldu, float* dX, int lddx, float* dA, float* dB, float* dbias, hipStream_t st) {
  F32SmallBwd p{M, N, K, r, s, dY, lddy, X, ldx, W0, ldw, A, B, U, ldu, dX, lddx, dA, dB, dbias, 0, 0, 0};
  p.ndx = dX != nullptr ? ((M + 15) / 16) * (K / 16) : 0;
  p.nda = K / 16;
  p.ndb = N / 16;
  hipLaunchKernelGGL(f32_small_bwd_kernel, dim3(p.ndx + p.nda + p.ndb), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace ldl
