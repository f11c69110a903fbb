// Four-wave 256x256 GEMM tile on v_mfma_f32_16x16x32_bf16 for the plain NT
// product with a low-rank term (LoRA forward: Y = X.W0^T + s.U.B^T (+ bias)).
//
// Same data path as gemm_kernel (two 64 KB LDS stages filled by direct
// buffer->LDS copies, the output staged through LDS), with one wave per SIMD and
// a 128x128 wave tile: half the LDS fragment traffic per MFMA of the eight-wave
// 128x64 tiling.  With one wave per SIMD nothing hides a stalled wave, so the
// k-loop is scheduled by hand: each k-tile is two 32-element MFMA steps (64
// MFMAs each); the fragment reads of the next step are spread over the first half
// of the current step's MFMAs, and the stage copies (16 per wave) over the whole
// hand-over step.  The two stage buffers are separate arrays and the loop is
// unrolled by two, so the compiler sees which buffer a copy writes and which a
// read reads and inserts no waits between them.  The low-rank term enters as
// extra k-steps before the loop: s.S (rounded to bf16, as the eight-wave seed
// does) and E are written into the second stage buffer in the tile layout and
// multiplied with the loop's own step code.
#pragma once

#include "gemm_tile.hpp"

namespace ldl {

// LDS tile layout: 128-byte rows (64 k); 16-byte chunk c of row r sits at
// physical chunk c ^ swz(r & 15).  The pattern repeats every 16 rows, so the
// fragments one wave reads differ by constant offsets, and the 16 rows of one
// fragment read cover all banks.
__device__ __forceinline__ int g16_off(int row, int chunk) { return row * 128 + ((chunk ^ swz(row & 15)) << 4); }

// NN Q tile ([64 k][256 n] as stored): k-row k at k * 512 + (k / 8) * 128, 16-byte
// chunk c at physical chunk c ^ 2 (k & 3).  A transposing read takes 4 k-rows x 32
// bytes per 16 lanes: the XOR spreads the 4 rows over distinct banks and the 128-byte
// pad every 8 rows moves the next 16 lanes' rows (k + 8) onto the other half of the banks.
constexpr int kG16NNRow = 512, kG16NNPad = 128;
__host__ __device__ constexpr int g16_nn_row(int k) { return k * kG16NNRow + (k >> 3) * kG16NNPad; }

// NN: Q is [K, N] (else [N, K]); SS: 32-rank MFMA steps of the low-rank term (r_epi <= 32 SS)
template <bool NN, int SS>
__global__ __launch_bounds__(256, 1) void gemm16_kernel(const GemmParams p) {
  constexpr int BM = 256, BN = 256, NW = 4;
  constexpr int QB = NN ? g16_nn_row(64) : BN * 128;
  constexpr int SB = BM * 128 + QB;                 // one stage: P tile then Q tile
  __shared__ __attribute__((aligned(16))) uint8_t smem0[SB];
  __shared__ __attribute__((aligned(16))) uint8_t smem1[SB];

  const int M = p.M, N = p.N, K = p.K;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = N / BN;
  // XCD-contiguous tile ranges, walked in groups of 4 row-tiles (as gemm_kernel)
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  constexpr int GM = 4;
  const int group = bid / (GM * tiles_n);
  const int first_m = group * GM;
  const int gm = min(GM, tiles_m - first_m);
  const int in_g = bid - group * GM * tiles_n;
  const int m0 = (first_m + in_g % gm) * BM, n0 = (in_g / gm) * BN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l16 = lane & 15, lq = lane >> 4;
  const uint32_t lda_b = (uint32_t)p.lda * 2u, ldb_b = (uint32_t)p.ldb * 2u;

  const __amdgpu_buffer_rsrc_t rs_a = make_rsrc(p.a, (uint32_t)M * lda_b);
  const __amdgpu_buffer_rsrc_t rs_b = make_rsrc(p.b0, (uint32_t)(NN ? K : N) * ldb_b);
  const __amdgpu_buffer_rsrc_t rs_none = make_rsrc(p.a, 0u);    // copies that read nothing

  // per-lane copy offsets: 8 instructions for each tile (1 KB each); rows past M read as zero
  const int lrow = lane >> 3, lphys = lane & 7;
  uint32_t a_off[8], b_off[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = (i * NW + wave) * 8 + lrow;
    a_off[i] = (uint32_t)(m0 + row) * lda_b + ((lphys ^ swz(row & 15)) << 4);
    if constexpr (NN) {           // k-rows 2q, 2q+1 of the stage, 32 chunks each
      const int k = 2 * (i * NW + wave) + (lane >> 5), chunk = (lane & 31) ^ (2 * (k & 3));
      b_off[i] = (uint32_t)k * ldb_b + (uint32_t)(n0 + 8 * chunk) * 2u;
    } else {
      b_off[i] = (uint32_t)(n0 + row) * ldb_b + ((lphys ^ swz(row & 15)) << 4);
    }
  }
  auto q_dst = [&](int i) { const int q = i * NW + wave; return BM * 128 + q * 1024 + (NN ? (q >> 2) * kG16NNPad : 0); };
  auto copy = [](__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint8_t* lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
  };
  // copies of stage kt into sb; stages past the last read nothing and land as zeros
  auto copy_stage = [&](int kt, uint8_t* sb) {
    const bool valid = kt < K / 64;
    const __amdgpu_buffer_rsrc_t ra = valid ? rs_a : rs_none, rb = valid ? rs_b : rs_none;
#pragma unroll
    for (int i = 0; i < 8; ++i) copy(ra, a_off[i], (uint32_t)kt * 128u, sb + (i * NW + wave) * 1024);
#pragma unroll
    for (int i = 0; i < 8; ++i) copy(rb, b_off[i], NN ? (uint32_t)kt * 64u * ldb_b : (uint32_t)kt * 128u, sb + q_dst(i));
  };

  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

  // fragments of 32-element step ks (P rows wm*128 + 16 i + l16, Q rows or columns
  // wn*128 + 16 j + l16, k = 32 ks + 8 lq ..), read in order of first use: fa[0], fb[0..7], fa[1..7]
  const int a_base0 = g16_off(wm * 128 + l16, lq), a_base1 = g16_off(wm * 128 + l16, 4 + lq);
  const int b_base0 = BM * 128 + g16_off(wn * 128 + l16, lq), b_base1 = BM * 128 + g16_off(wn * 128 + l16, 4 + lq);
  auto ldf_rows = [&](const uint8_t* s, int ks, u32x4* fa, u32x4* fb) {   // both tiles k-contiguous rows
    const int a = ks ? a_base1 : a_base0, b = ks ? b_base1 : b_base0;
    fa[0] = lds_ld16(s, a);
#pragma unroll
    for (int j = 0; j < 8; ++j) fb[j] = lds_ld16(s, b + j * 2048);
#pragma unroll
    for (int i = 1; i < 8; ++i) fa[i] = lds_ld16(s, a + i * 2048);
  };
  // NN: lane l16 of 16-lane group lq reads k-row 32 ks + 8 lq + (l16 >> 2) (+4 for the upper
  // half), columns 4 (l16 & 3) .. +3 of column block j; the transposing read hands lane l16
  // column l16 of the block at 4 consecutive k.  Physical chunk of column block j: 2 (j ^ a)
  // with a = l16 >> 2 = k & 3, so four per-lane bases (j & 3) and constant offsets cover all j.
  int bq[4];
  {
    const int a = l16 >> 2;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      bq[t] = BM * 128 + g16_nn_row(8 * lq + a) + wn * 256 + 8 * (l16 & 3) + 32 * (t ^ a);
  }
  auto ldf = [&](const uint8_t* s, int ks, u32x4* fa, u32x4* fb) {
    if constexpr (NN) {
      const int a = ks ? a_base1 : a_base0;
      const int kso = ks * (g16_nn_row(32) - g16_nn_row(0));
      fa[0] = lds_ld16(s, a);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int o = bq[j & 3] + kso + 128 * (j >> 2);
        const u32x2 lo = lds_tr16(s, o), hi = lds_tr16(s, o + 4 * kG16NNRow);
        fb[j] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
#pragma unroll
      for (int i = 1; i < 8; ++i) fa[i] = lds_ld16(s, a + i * 2048);
    } else {
      ldf_rows(s, ks, fa, fb);
    }
  };
  // D[n][m]: lane l of acc[i][j] holds n = 16 j + 4 (l >> 4) + v, m = 16 i + (l & 15) of the wave tile
  auto mm = [&](const u32x4* fa, const u32x4* fb) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = mfma_bf16(fb[j], fa[i], acc[i][j]);
  };

  constexpr int NRQ = NN ? 2 : 1;       // LDS read instructions per Q fragment
  const int KT = K / 64;
  u32x4 fa0[8], fb0[8], fa1[8], fb1[8];
  copy_stage(0, smem0);

  // Low-rank term through the second stage buffer while stage 0 lands: thread t writes
  // row t of each tile (s.S[m0 + t][..] as bf16, E[n0 + t][..]) in the k-contiguous row
  // layout, zero past r_epi.
  if constexpr (SS > 0) {
    const int m = m0 + tid;
    const float* srow = p.S + (size_t)min(m, M - 1) * p.ld_s;
#pragma unroll
    for (int c = 0; c < 4 * SS; ++c) {
      const int k = 8 * c;
      u32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = (m < M && k + 2 * e < p.r_epi) ? srow[k + 2 * e] * p.s_epi : 0.f;
        const float hi = (m < M && k + 2 * e + 1 < p.r_epi) ? srow[k + 2 * e + 1] * p.s_epi : 0.f;
        v[e] = pack_bf16x2(lo, hi);
      }
      lds_st16(smem1, g16_off(tid, c), v);
      lds_st16(smem1, BM * 128 + g16_off(tid, c), e_frag(p, n0 + tid, k));
    }
    __syncthreads();
    ldf_rows(smem1, 0, fa0, fb0);
    mm(fa0, fb0);
    if constexpr (SS > 1) {
      ldf_rows(smem1, 1, fa1, fb1);
      mm(fa1, fb1);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  copy_stage(1, smem1);
  ldf(smem0, 0, fa0, fb0);
  __builtin_amdgcn_s_waitcnt(0xc07f);     // settle the prologue's LDS / scalar reads

  auto tile = [&](auto par_c, int kt) {
    constexpr int PAR = decltype(par_c)::value;
    uint8_t* cur = PAR ? smem1 : smem0;
    uint8_t* nxt = PAR ? smem0 : smem1;
    // The accumulators enter every tile in AGPRs (an empty asm with an AGPR operand):
    // without this the register allocator moves some of them between register files
    // inside the loop and runs out of registers for the fragments.
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) asm volatile("" : "+a"(acc[i][j]));
    // step 0 of this stage, with the reads of step 1 over its first half
    __builtin_amdgcn_sched_barrier(0);
    ldf(cur, 1, fa1, fb1);
    mm(fa0, fb0);
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, NRQ, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 32, 0);
    __builtin_amdgcn_sched_barrier(0);
    // hand-over: the next stage has landed and every wave is done with this one
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // step 1, with the reads of the next stage's step 0 and this buffer's copies of stage kt+2
    copy_stage(kt + 2, cur);
    ldf(nxt, 0, fa0, fb0);
    mm(fa1, fb1);
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, NRQ, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // One loop body for every k-tile, so the accumulators keep their registers to the end:
  // an odd count runs one more tile, whose stage the empty copies filled with zeros.
  for (int kt = 0; kt < KT; kt += 2) {
    tile(std::integral_constant<int, 0>{}, kt);
    tile(std::integral_constant<int, 1>{}, kt + 1);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the last (empty) copies
  __syncthreads();

  static_assert(128 * 512 <= SB, "half of the output tile fits in a stage buffer");
  // ---- epilogue: bias, bf16, staged through LDS (rows < 128 in smem0, the rest in smem1),
  // written out as whole 16-byte row segments
  auto st_ptr = [&](int r, int col) -> uint8_t* {
    uint8_t* base = r < 128 ? smem0 : smem1;
    const int rr = r & 127;
    return base + rr * 512 + ((((col >> 3) ^ (rr & 31))) << 4) + ((col & 4) << 1);
  };
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = wm * 128 + i * 16 + l16;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int cl = wn * 128 + j * 16 + 4 * lq;
      float b4[4] = {0.f, 0.f, 0.f, 0.f};
      if (p.bias != nullptr) {
        const u32x2 bb = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p.bias) + n0 + cl);
        b4[0] = bf16_lo(bb[0]); b4[1] = bf16_hi(bb[0]); b4[2] = bf16_lo(bb[1]); b4[3] = bf16_hi(bb[1]);
      }
      const f32x4 v = acc[i][j];
      u32x2 w;
      w[0] = pack_bf16x2(v[0] + b4[0], v[1] + b4[1]);
      w[1] = pack_bf16x2(v[2] + b4[2], v[3] + b4[3]);
      *reinterpret_cast<u32x2*>(st_ptr(r, cl)) = w;
    }
  }
  __syncthreads();
  uint16_t* out = static_cast<uint16_t*>(p.out);
  for (int idx = tid; idx < BM * 32; idx += 256) {
    const int r = idx >> 5, c = idx & 31;
    if (m0 + r < M) {
      const uint8_t* base = r < 128 ? smem0 : smem1;
      const int rr = r & 127;
      st16(out + (size_t)(m0 + r) * p.ldo + n0 + c * 8, lds_ld16(base, rr * 512 + ((c ^ (rr & 31)) << 4)));
    }
  }
}

}  // namespace ldl
