// Four-wave 256x256 GEMM tile on v_mfma_f32_16x16x32_bf16 for the plain products
// with a low-rank term: NT (LoRA forward Y = X.W0^T + s.U.B^T (+ bias)) and NN (input
// gradient dX = dY.W0 + s.V.A, W0 read as stored).
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
// read reads and inserts no waits between them.  The low-rank term enters as one or
// two more k-tiles at the front: s.S (as a bf16 pair hi + lo where the rank slots allow)
// and E are written into the stage buffers in the stage layout and multiplied by the
// loop itself.  Every MFMA sits in the one loop body: MFMAs before the loop made the
// register allocator shuffle accumulators through VGPRs inside it.
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

// NN: Q is [K, N] (else [N, K]); LR: number of low-rank k-tiles in front of the loop (0: no
// low-rank term; 1: rank r_epi <= 64 of one segment; 2: the dual tile's gate and up terms);
// DORA (NT: DoRA's row scale; NN: a per-feature scale of an input gradient): two outputs, out2 = z (the unscaled sum) and out = z * col_scale[n] + bias[n];
// SWB (NN only): the gated-MLP backward of the product dh with e = aux0, u = aux1:
// out = dh u act'(e) (de) and out2 = dh act(e) (du), act = p.act (SiLU: act' = sigma (1 + e (1 - sigma)))
// BN_: tile width, 256, or 192 for NT (3072 columns at 4096 rows then make 256 tiles, one full
// round of the 256 CUs, where 256-column tiles leave a quarter of the chip idle)
// SWF (NT only, the SwiGLU forward): each tile covers 128 hidden units; its Q rows are the 128
// gate rows (b0) then the 128 up rows (b1) of those units, so the waves with wn = 0 hold
// e and the waves with wn = 1 hold u of the same (token, unit) in the same lanes.  Outputs:
// out = e, out2 = u, out3 = h = act(e) u (act = p.act: SiLU or GELU), all from the fp32
// accumulators (e is handed to the u waves through LDS).
// I8 (NT only, the W8A8 forward): P and Q are int8 with 128 k per k-tile (the same 128-byte
// LDS rows and 16-byte fragments), v_mfma_i32_16x16x64_i8 into exact int32 accumulators,
// dequantised after the loop to acc . row_scale[m] . col_scale[n] in fp32; the low-rank term
// is then one bf16 k-tile on those fp32 accumulators (LR = 0 in the loop).
// LEAF (NT, LR = 1): several adapters over the concatenated output (p.nleaf leaves of rank
// p.leaf_r): the k-tile's E slot of rank j holds the up row of output column n only where n's
// leaf owns rank j, and the S side carries each leaf's own scale.
template <bool NN, int LR, bool DORA = false, bool SWB = false, int BN_ = 256, bool SWF = false, bool I8 = false,
          bool LEAF = false, int ACT = ACT_SILU, bool SPLITK = false>
__global__ __launch_bounds__(256, 1) void gemm16_kernel(const GemmParams p) {
  static_assert(!SPLITK || (!DORA && !SWB && !SWF && !LEAF && BN_ == 256), "split reduction: the plain 256-wide tiles");
  static_assert(!LEAF || (!NN && LR == 1 && !DORA && !I8), "leaves: the plain NT tile with one low-rank k-tile");
  static_assert(BN_ == 256 || (!NN && BN_ == 192), "tile widths: 256, or 192 for NT");
  static_assert(!SWB || (NN && !DORA), "the SwiGLU backward epilogue is an NN epilogue");
  static_assert(!SWF || (!NN && !DORA && !SWB && BN_ == 256 && LR != 1), "the dual tile is a plain 256-wide NT tile");
  // NN2: the NN tile over two stacked Q segments (rows k < kseg from b0, the rest from b1)
  // with a two-segment low-rank term (two seed k-tiles)
  constexpr bool NN2 = NN && LR == 2;
  static_assert(LR >= 0 && LR <= 2 && (LR != 2 || SWF || (NN && !DORA && !SWB && !I8 && !LEAF && BN_ == 256)),
                "two low-rank k-tiles: the dual tile's two segments, or the NN tile over two stacked weights");
  static_assert(!I8 || (!NN && !DORA && !SWB && !SWF && LR == 0 && BN_ == 256), "int8: the plain 256-wide NT tile");
  constexpr int KB = I8 ? 128 : 64;                 // reduction elements per k-tile (128 bytes per row)
  constexpr int BM = 256, BN = BN_, NW = 4;
  constexpr int TNO = SWF ? 128 : BN;               // output columns (hidden units) per tile
  constexpr int FN = BN / 32;                       // 16-column fragments per wave (wave tile BN / 2)
  constexpr int QB = NN ? g16_nn_row(64) : BN * 128;
  constexpr int SB = BM * 128 + QB;                 // one stage: P tile then Q tile
  __shared__ __attribute__((aligned(16))) uint8_t smem0[SB];
  __shared__ __attribute__((aligned(16))) uint8_t smem1[SB];

  const int M = p.M, N = p.N;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = N / TNO;
  // XCD-contiguous tile ranges, walked in groups of 4 row-tiles (as gemm_kernel).
  // SPLITK (the split reduction of the tiles past the last full round of the chip, a launch
  // of its own after the full rounds): block t S + q computes k-tiles [q KT / S, (q + 1) KT / S)
  // of tile split_first + t (S = split_s) into an fp32 partial that the fixup pass sums; the
  // operands are addressed from the first k-tile of the range on, and only q = 0 carries the
  // low-rank term.
  int bid = blockIdx.x;
  [[maybe_unused]] int split = 0, kb = 0;
  int KTl = p.K / KB;
  if constexpr (SPLITK) {
    split = bid % p.split_s;
    bid = p.split_first + bid / p.split_s;
    kb = split * KTl / p.split_s;
    KTl = (split + 1) * KTl / p.split_s - kb;
  } else {
    const int nblk = gridDim.x;
    if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  }
  const int K = KTl * KB;                           // this block's reduction length
  constexpr int GM = 4;
  const int group = bid / (GM * tiles_n);
  const int first_m = group * GM;
  const int gm = min(GM, tiles_m - first_m);
  const int in_g = bid - group * GM * tiles_n;
  const int m0 = (first_m + in_g % gm) * BM, n0 = (in_g / gm) * TNO;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l16 = lane & 15, lq = lane >> 4;
  const uint32_t lda_b = (uint32_t)p.lda * (I8 ? 1u : 2u), ldb_b = (uint32_t)p.ldb * (I8 ? 1u : 2u);

  // (SPLITK: P and the NT Q from k-tile kb on, 128 bytes a row per k-tile; the NN Q from its
  // row kb KB on; the bounds shrink by the same offset)
  const uint32_t koff_a = SPLITK ? (uint32_t)kb * 128u : 0u;
  const uint32_t koff_b = SPLITK ? (NN ? (uint32_t)kb * KB * ldb_b : (uint32_t)kb * 128u) : 0u;
  const __amdgpu_buffer_rsrc_t rs_a =
      make_rsrc(static_cast<const uint8_t*>(p.a) + koff_a, (uint32_t)M * lda_b - koff_a);
  const __amdgpu_buffer_rsrc_t rs_b =
      make_rsrc(static_cast<const uint8_t*>(p.b0) + koff_b, (uint32_t)(NN ? (NN2 ? p.kseg : p.K) : N) * ldb_b - koff_b);
  // dual: up rows; NN2: the second segment's k-rows
  const __amdgpu_buffer_rsrc_t rs_b1 =
      SWF ? make_rsrc(p.b1, (uint32_t)N * ldb_b) : (NN2 ? make_rsrc(p.b1, (uint32_t)(p.K - p.kseg) * ldb_b) : rs_b);
  const __amdgpu_buffer_rsrc_t rs_none = make_rsrc(p.a, 0u);    // copies that read nothing

  // Copies: 8 instructions per tile per wave, 1 KB each; rows past M read as zero.  Copy i
  // reads rows 32 i further down (NN: k-rows 8 i) than copy 0 with the same swizzle.  NT
  // keeps one per-lane offset per operand and adds the wave-uniform step in the scalar
  // offset; NN keeps all eight per-lane offsets (the register allocator assigns the NN
  // loop's accumulators with fewer moves that way).
  const int lrow = lane >> 3, lphys = lane & 7;
  constexpr int NOFF = NN ? 8 : 1;
  uint32_t a_off[NOFF], b_off[NOFF];
#pragma unroll
  for (int i = 0; i < NOFF; ++i) {
    const int row = (i * NW + wave) * 8 + lrow;
    a_off[i] = (uint32_t)(m0 + row) * lda_b + ((lphys ^ swz(row & 15)) << 4);
    if constexpr (NN) {           // k-rows 2q, 2q+1 of the stage (q = i NW + wave), 32 chunks each
      const int k = 2 * (i * NW + wave) + (lane >> 5), chunk = (lane & 31) ^ (2 * (k & 3));
      b_off[i] = (uint32_t)k * ldb_b + (uint32_t)(n0 + 8 * chunk) * 2u;
    } else {
      b_off[i] = (uint32_t)(n0 + row) * ldb_b + ((lphys ^ swz(row & 15)) << 4);
    }
  }
  const uint32_t a_step = NN ? 0u : 32u * lda_b, b_step = NN ? 0u : 32u * ldb_b;
  auto q_dst = [&](int i) { const int q = i * NW + wave; return BM * 128 + q * 1024 + (NN ? (q >> 2) * kG16NNPad : 0); };
  auto copy = [](__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint8_t* lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
  };
  // copies of stage kt into sb; stages past the last read nothing and land as zeros
  auto copy_stage = [&](int kt, uint8_t* sb) {
    const bool valid = kt < K / KB;
    const __amdgpu_buffer_rsrc_t ra = valid ? rs_a : rs_none, rb = valid ? rs_b : rs_none;
    const __amdgpu_buffer_rsrc_t rb1 = valid ? rs_b1 : rs_none;
    const uint32_t ka = (uint32_t)kt * 128u, kb = NN ? (uint32_t)kt * 64u * ldb_b : (uint32_t)kt * 128u;
#pragma unroll
    for (int i = 0; i < 8; ++i) copy(ra, a_off[NN ? i : 0], ka + i * a_step, sb + (i * NW + wave) * 1024);
    if constexpr (NN2) {      // k-tiles never straddle kseg (a multiple of 64)
      const bool seg1 = kt * KB >= p.kseg;
      const __amdgpu_buffer_rsrc_t rq = seg1 ? rb1 : rb;
      const uint32_t kq = (uint32_t)(seg1 ? kt * KB - p.kseg : kt * KB) * ldb_b;
#pragma unroll
      for (int i = 0; i < 8; ++i) copy(rq, b_off[i], kq, sb + q_dst(i));
    } else {
#pragma unroll
      for (int i = 0; i < (NN ? 8 : FN); ++i) {
        if constexpr (SWF)    // Q rows 0..127 gate rows n0.., rows 128..255 up rows n0..
          copy(i < FN / 2 ? rb : rb1, b_off[0], kb + (i & (FN / 2 - 1)) * b_step, sb + q_dst(i));
        else
          copy(rb, b_off[NN ? i : 0], kb + i * b_step, sb + q_dst(i));
      }
    }
  };

  using AccT = typename std::conditional<I8, i32x4, f32x4>::type;
  AccT acc[8][FN];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = AccT{0, 0, 0, 0};

  // fragments of 32-element step ks (P rows wm*128 + 16 i + l16, Q rows or columns
  // wn*128 + 16 j + l16, k = 32 ks + 8 lq ..), read in order of first use: fa[0], fb[0..7], fa[1..7]
  const int a_base0 = g16_off(wm * 128 + l16, lq), a_base1 = g16_off(wm * 128 + l16, 4 + lq);
  const int b_base0 = BM * 128 + g16_off(wn * (BN / 2) + l16, lq), b_base1 = BM * 128 + g16_off(wn * (BN / 2) + l16, 4 + lq);
  auto ldf_rows = [&](const uint8_t* s, int ks, u32x4* fa, u32x4* fb) {   // NT: both tiles k-contiguous rows
    const int a = ks ? a_base1 : a_base0, b = ks ? b_base1 : b_base0;
    fa[0] = lds_ld16(s, a);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[j] = lds_ld16(s, b + j * 2048);
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
      for (int j = 0; j < FN; ++j) {
        if constexpr (I8) acc[i][j] = mfma_i8(fb[j], fa[i], acc[i][j]);
        else acc[i][j] = mfma_bf16(fb[j], fa[i], acc[i][j]);
        // NT 256: keep each result in its accumulator's AGPRs (an empty asm with an AGPR
        // operand); otherwise the allocator moves some accumulators through VGPRs.  (At
        // 192 columns the pins cost ~70 AGPR moves per k-tile and are left out.)
        if constexpr (!NN && BN == 256) asm volatile("" : "+a"(acc[i][j]));
      }
  };

  constexpr int NRQ = NN ? 2 : 1;       // LDS read instructions per Q fragment
  const int KT = K / KB;
  u32x4 fa0[8], fb0[FN], fa1[8], fb1[FN];

  // The low-rank term enters as LR more k-tiles in front ("stages" -LR .. -1, in the stage
  // buffers they would use): their P tile holds s.S[m0 + t][..] as bf16 and their Q tile E in
  // the layout of a regular Q stage, so the k-loop multiplies them with its own code and no
  // MFMA runs before the loop.  Their loads go out first, all at once, branch-free and as
  // 16-byte vectors (indices clamped into range, values zeroed after the load): thread t loads
  // row t of S and, for NT, row t of E ([N, r]); for NN the E tile is the rank rows of E^T
  // ([r, N], E[n][j] at n + j e_ldj), 32 16-byte chunks each.
  //   One segment (LR = 1): rank slots are chunks of 8; with p.seed_hilo (2 r_epi <= 64)
  // chunks [0, r/8) hold the bf16 rounding hi of s.S and chunks [r/8, r/4) the rounding of
  // the remainder s.S - hi, both against the same E ranks, so the low-rank term keeps ~16
  // bits of s.S; otherwise chunks [0, r/8) hold hi only.
  //   Dual tile (LR = 2): k-tile -2 carries the gate term (s_epi.S[.., 0 .. r) against Bg on
  // Q rows 0..127, zero on the up rows) and k-tile -1 the up term (s_epi2.S[.., r .. 2r)
  // against Bu on rows 128..255), r = e_jsplit <= 64, bf16 hi only.
  // The caller guarantees 16-byte aligned S rows and E rows (or rank rows), ranks that are
  // multiples of 8, and (LR = 1) a single E segment (e_jsplit >= r_epi).
  const uint16_t* e0 = static_cast<const uint16_t*>(p.e0);
  const bool live = m0 + tid < M && split == 0;     // (SPLITK blocks past the first: no low-rank term)
  const float* srow = p.S + (size_t)min(m0 + tid, M - 1) * p.ld_s;
  auto pack8 = [](f32x4 a, f32x4 b, float sc, bool lo) {
    const float x[8] = {a[0] * sc, a[1] * sc, a[2] * sc, a[3] * sc, b[0] * sc, b[1] * sc, b[2] * sc, b[3] * sc};
    u32x4 v;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t h0 = f32_to_bf16_bits(x[2 * q]), h1 = f32_to_bf16_bits(x[2 * q + 1]);
      if (lo) {
        h0 = f32_to_bf16_bits(x[2 * q] - __uint_as_float(h0 << 16));
        h1 = f32_to_bf16_bits(x[2 * q + 1] - __uint_as_float(h1 << 16));
      }
      v[q] = h0 | (h1 << 16);
    }
    return v;
  };
  if constexpr (LR == 1) {
    const int cps = p.r_epi >> 3;                     // chunks per part
    const int nparts = p.seed_hilo ? 2 : 1;
    // (LEAF) this thread's output column n0 + t lies in leaf myleaf
    const int nrow = (BN == 256 || tid < BN) ? n0 + tid : n0;
    int myleaf = 0;
    if constexpr (LEAF) {
      for (int l = 0; l + 1 < p.nleaf; ++l) myleaf += nrow >= p.leaf_end[l] ? 1 : 0;
    }
    f32x4 sa[8], sb[8];
    u32x4 ev[8];
    if constexpr (!LEAF && !NN) {
      // only the cps chunks that hold ranks are read (the lo part reuses the hi part's S and E):
      // the loads of every clamped chunk had cost ~3000 cycles of memory-pipeline issue at the
      // start, when every CU issues them at once
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (q < cps) {
          sa[q] = *reinterpret_cast<const f32x4*>(srow + 8 * q);
          sb[q] = *reinterpret_cast<const f32x4*>(srow + 8 * q + 4);
          ev[q] = *reinterpret_cast<const u32x4*>(e0 + (size_t)nrow * p.e_ldn + 8 * q);   // ranks 8q.. of row n0 + t
        }
      copy_stage(0, smem0);
      const u32x4 z = u32x4{0u, 0u, 0u, 0u};
      const float sc = live ? p.s_epi : 0.f;
      auto put_e = [&](int c, u32x4 v) {
        if (BN == 256 || tid < BN) lds_st16(smem1, BM * 128 + g16_off(tid, c), v);
      };
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (q < cps) {
          lds_st16(smem1, g16_off(tid, q), pack8(sa[q], sb[q], sc, false));
          put_e(q, ev[q]);
          if (nparts == 2) {
            lds_st16(smem1, g16_off(tid, q + cps), pack8(sa[q], sb[q], sc, true));
            put_e(q + cps, ev[q]);
          }
        }
#pragma unroll
      for (int c = 0; c < 8; ++c)
        if (c >= cps * nparts) {
          lds_st16(smem1, g16_off(tid, c), z);
          put_e(c, z);
        }
    } else {
      // (NN, leaves) every chunk loaded, clamped into range: branch-free
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int part = c / cps, j0 = 8 * (c - part * cps);
        const int jl = part < nparts ? j0 : 0;           // clamped rank offset
        sa[c] = *reinterpret_cast<const f32x4*>(srow + jl);
        sb[c] = *reinterpret_cast<const f32x4*>(srow + jl + 4);
        if constexpr (NN) {       // rank row jl + t / 32, 16-byte chunk t % 32 of its 256 columns
          ev[c] = *reinterpret_cast<const u32x4*>(e0 + (size_t)(jl + (tid >> 5)) * p.e_ldj + n0 + 8 * (tid & 31));
        } else {                  // ranks jl .. jl + 7 of the leaf's row n0 + t (t < BN)
          ev[c] = *reinterpret_cast<const u32x4*>(e0 + (size_t)nrow * p.e_ldn + jl % p.leaf_r);
        }
      }
      copy_stage(0, smem0);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int part = c / cps, j0 = 8 * (c - part * cps);
        const bool on = part < nparts;
        const u32x4 z = u32x4{0u, 0u, 0u, 0u};
        if constexpr (LEAF) {
          const int lc = j0 / p.leaf_r;                 // leaf of these rank slots
          lds_st16(smem1, g16_off(tid, c), on ? pack8(sa[c], sb[c], live ? p.leaf_s[lc] : 0.f, part == 1) : z);
          if (BN == 256 || tid < BN) lds_st16(smem1, BM * 128 + g16_off(tid, c), (on && lc == myleaf) ? ev[c] : z);
        } else {
          lds_st16(smem1, g16_off(tid, c), on ? pack8(sa[c], sb[c], live ? p.s_epi : 0.f, part == 1) : z);
          const int j = 8 * c + (tid >> 5), ch = tid & 31;
          lds_st16(smem1, BM * 128 + g16_nn_row(j) + ((ch ^ (2 * (j & 3))) << 4), on ? ev[c] : z);
        }
      }
    }
    __syncthreads();
    ldf(smem1, 0, fa0, fb0);
  } else if constexpr (NN2) {
    // two seed k-tiles: segment g (k-tile g - 2) holds s.S[.., g rs .. g rs + rs) (bf16 hi)
    // against the rank rows of E_g (e0, e1: [rs, N] rows at e_ldj), rs = e_jsplit <= 64; one
    // segment at a time, as the dual tile.  The loop starts on smem1 as with one seed k-tile
    // (starting on smem0 made the allocator move the NN loop's accumulators), so segment 0 is
    // staged in smem1 and segment 1 in smem0.
    const int rs = p.e_jsplit;
    const float sc = live ? p.s_epi : 0.f;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const uint16_t* eg = g ? static_cast<const uint16_t*>(p.e1) : e0;
      f32x4 sa[8], sb[8];
      u32x4 ev[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int jl = 8 * c < rs ? 8 * c : 0;
        sa[c] = *reinterpret_cast<const f32x4*>(srow + g * rs + jl);
        sb[c] = *reinterpret_cast<const f32x4*>(srow + g * rs + jl + 4);
        ev[c] = *reinterpret_cast<const u32x4*>(eg + (size_t)(jl + (tid >> 5)) * p.e_ldj + n0 + 8 * (tid & 31));
      }
      uint8_t* buf = g ? smem0 : smem1;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const bool on = 8 * c < rs;
        const u32x4 z = u32x4{0u, 0u, 0u, 0u};
        lds_st16(buf, g16_off(tid, c), on ? pack8(sa[c], sb[c], sc, false) : z);
        const int j = 8 * c + (tid >> 5), ch = tid & 31;
        lds_st16(buf, BM * 128 + g16_nn_row(j) + ((ch ^ (2 * (j & 3))) << 4), on ? ev[c] : z);
      }
    }
    __syncthreads();
    ldf(smem1, 0, fa0, fb0);
  } else if constexpr (LR == 2) {
    const int rs = p.e_jsplit;                        // rank of each segment
    const int own = tid >> 7;                         // segment of this thread's Q row (wave-uniform)
    const uint16_t* erow = (own ? static_cast<const uint16_t*>(p.e1) : e0) + (size_t)(n0 + (tid & 127)) * p.e_ldn;
    // one segment at a time (the loads of both at once do not fit the registers)
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      f32x4 sa[8], sb[8];
      u32x4 ev[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int jl = 8 * c < rs ? 8 * c : 0;
        sa[c] = *reinterpret_cast<const f32x4*>(srow + g * rs + jl);
        sb[c] = *reinterpret_cast<const f32x4*>(srow + g * rs + jl + 4);
        if (own == g) ev[c] = *reinterpret_cast<const u32x4*>(erow + jl);
      }
      uint8_t* buf = g ? smem1 : smem0;
      const float sc = live ? (g ? p.s_epi2 : p.s_epi) : 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const bool on = 8 * c < rs;
        const u32x4 z = u32x4{0u, 0u, 0u, 0u};
        lds_st16(buf, g16_off(tid, c), on ? pack8(sa[c], sb[c], sc, false) : z);
        lds_st16(buf, BM * 128 + g16_off(tid, c), (on && own == g) ? ev[c] : z);
      }
    }
    __syncthreads();
    ldf(smem0, 0, fa0, fb0);
  } else {
    copy_stage(0, smem0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    copy_stage(1, smem1);
    ldf(smem0, 0, fa0, fb0);
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);     // settle the prologue's LDS / scalar reads

  auto tile = [&](auto par_c, int kt) {
    constexpr int PAR = decltype(par_c)::value;
    uint8_t* cur = PAR ? smem1 : smem0;
    uint8_t* nxt = PAR ? smem0 : smem1;
    // The accumulators enter every tile in AGPRs (an empty asm with an AGPR operand):
    // without this the register allocator moves some of them between register files
    // inside the loop and runs out of registers for the fragments.  (Allocation of this
    // loop is fragile: the pins here and in mm were chosen by compiling the variants and
    // counting the AGPR moves and spills left in the loop.)
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) asm volatile("" : "+a"(acc[i][j]));
    // Schedule of a step (8 FN MFMAs): NG groups of {read, 2 MFMAs, read(s), 2 MFMAs} carry
    // the 8 + FN fragment reads (NN: 8 + 16), the other MR MFMAs follow; in the hand-over
    // step one stage copy goes with each group and the other NC2 copies with MPC MFMAs each.
    constexpr int NG = NN ? 8 : (8 + FN) / 2;
    constexpr int MR = 8 * FN - 4 * NG;
    constexpr int NC2 = (NN ? 16 : 8 + FN) - NG;
    constexpr int MPC = (MR + NC2 - 1) / NC2;
    // step 0 of this stage, with the reads of step 1 over its first half
    __builtin_amdgcn_sched_barrier(0);
    ldf(cur, 1, fa1, fb1);
    mm(fa0, fb0);
    for (int q = 0; q < NG; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, NRQ, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, MR, 0);
    __builtin_amdgcn_sched_barrier(0);
    // hand-over: the next stage has landed and every wave is done with this one
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // step 1, with the reads of the next stage's step 0 and this buffer's copies of stage kt+2
    copy_stage(kt + 2, cur);
    ldf(nxt, 0, fa0, fb0);
    mm(fa1, fb1);
    for (int q = 0; q < NG; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, NRQ, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    for (int q = 0; q < NC2; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, MPC, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // One loop body for every k-tile (from the low-rank tile -1 when there is one), so the
  // accumulators keep their registers to the end: an odd count runs one more tile, whose
  // stage the empty copies filled with zeros.
  constexpr int P0 = (LR & 1) || NN2 ? 1 : 0;
  for (int kt = -LR; kt < KT; kt += 2) {
    tile(std::integral_constant<int, P0>{}, kt);
    tile(std::integral_constant<int, 1 - P0>{}, kt + 1);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the last (empty) copies
  __syncthreads();

  // SPLITK: the block's fp32 partial, lane-linear: slot ((wave 8 + i) FN + j) 64 + lane
  // holds acc[i][j]
  auto write_partial = [&]() {
    float* dst = p.part + ((size_t)(bid - p.split_first) * p.split_s + split) * (size_t)(BM * BN);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
      {
        f32x4 v = __builtin_bit_cast(f32x4, acc[i][j]);
        asm volatile("" : "+v"(v));                 // (out of the accumulators first)
        *reinterpret_cast<f32x4*>(dst + ((size_t)((wave * 8 + i) * FN + j) * 64 + lane) * 4) = v;
      }
  };
  if constexpr (SPLITK && !I8) {
    write_partial();
    return;
  }

  // staging rows of SROW bytes; 16-byte chunk c of row rr at c ^ (rr & SWZM) (256 columns: all
  // 32 chunks; 192: within each group of 8, so it stays inside the 24 chunks of the row)
  constexpr int SROW = BN * 2, SWZM = BN == 256 ? 31 : 7, NCH = BN / 8;
  static_assert(128 * SROW <= SB, "half of the output tile fits in a stage buffer");
  // ---- epilogue: bias, bf16, staged through LDS (rows < 128 in smem0, the rest in smem1),
  // written out as whole 16-byte row segments (full 128-byte lines per store instruction;
  // 8-byte stores straight from the accumulator layout touch 16 lines each and were slower).
  // DORA writes z first, then y = z g + bias (both from the fp32 accumulators).
  auto st_ptr = [&](int r, int col) -> uint8_t* {
    uint8_t* base = r < 128 ? smem0 : smem1;
    const int rr = r & 127;
    return base + rr * SROW + ((((col >> 3) ^ (rr & SWZM))) << 4) + ((col & 4) << 1);
  };
  // the staged bf16 tile to dst as 16-byte row segments, eight LDS reads in flight before
  // their stores (one read, wait and store per segment had been bound by the LDS latency:
  // ~6800 cycles per tile)
  // part_c: -1 every row, 0 / 1 (256 columns) the groups of 64 rows with even / odd index
  // (tile rows [0, 64) and [128, 192) / [64, 128) and [192, 256))
  auto write_staged = [&](void* dst, int ldo, auto part_c) __attribute__((always_inline)) {
    constexpr int PART = decltype(part_c)::value;
    uint16_t* out = static_cast<uint16_t*>(dst);
    constexpr int NIT = BM * NCH / 256;
    static_assert(NIT % 8 == 0, "row segments per thread in groups of eight");
    static_assert(PART < 0 || NCH == 32, "row halves: 256 columns");
#pragma unroll
    for (int b = 0; b < NIT; b += 8) {
      if constexpr (PART >= 0) {
        if ((b / 8) % 2 != PART) continue;
      }
      u32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int idx = tid + (b + u) * 256, r = idx / NCH, c = idx % NCH, rr = r & 127;
        v[u] = lds_ld16(r < 128 ? smem0 : smem1, rr * SROW + ((c ^ (rr & SWZM)) << 4));
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int idx = tid + (b + u) * 256, r = idx / NCH, c = idx % NCH;
        if (m0 + r < M) st16(out + (size_t)(m0 + r) * ldo + n0 + c * 8, v[u]);
      }
    }
  };
  // (column blocks outermost: the bias and column scale of the lane's four columns are read
  // once per column block, not once per accumulator block)
  // Staging of the bf16 tile (bias, DORA's column scale).  256 columns: the lane's LDS address
  // is a lane constant plus compile-time parts: row 16 i + l16 of its half (wm), 16-byte chunk
  // (col >> 3) ^ (row & 31) = y ^ ((i & 1) << 4) ^ (j << 1) with y = l16 ^ (lq >> 1) ^ (wn << 4)
  // (col = 128 wn + 16 j + 4 lq), byte 8 (lq & 1) in it.  (A separate path without the bias
  // additions made the allocator move the k-loop's accumulators.)
  // half_c: -1 every accumulator block, 0 / 1 the blocks i < 4 / i >= 4 (rows [0, 64) /
  // [64, 128) of the wave's half)
  auto stage_out = [&](auto z_c, auto half_c) __attribute__((always_inline)) {
    constexpr bool Z = decltype(z_c)::value;       // DORA's unscaled output
    constexpr int HALF = decltype(half_c)::value;
    constexpr bool CS = DORA && !Z;
    [[maybe_unused]] uint8_t* const sb = (wm ? smem1 : smem0) + l16 * SROW + (lq & 1) * 8;
    [[maybe_unused]] const int y = l16 ^ (lq >> 1) ^ (wn << 4);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int cl = wn * (BN / 2) + j * 16 + 4 * lq;
      u32x2 bb = u32x2{0u, 0u};
      if (!Z && p.bias != nullptr) bb = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p.bias) + n0 + cl);
      f32x4 cs = f32x4{1.f, 1.f, 1.f, 1.f};
      if constexpr (CS) cs = *reinterpret_cast<const f32x4*>(p.col_scale + n0 + cl);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (HALF >= 0) {
          if (i / 4 != HALF) continue;
        }
        auto v = __builtin_bit_cast(f32x4, acc[i][j]);   // (fp32 in every kernel that calls this)
        if constexpr (CS) v *= cs;
        u32x2 w;
        w[0] = pack_bf16x2(v[0] + bf16_lo(bb[0]), v[1] + bf16_hi(bb[0]));
        w[1] = pack_bf16x2(v[2] + bf16_lo(bb[1]), v[3] + bf16_hi(bb[1]));
        if constexpr (BN == 256)
          *reinterpret_cast<u32x2*>(sb + ((y ^ ((i & 1) << 4) ^ (j << 1)) << 4) + i * 16 * SROW) = w;
        else
          *reinterpret_cast<u32x2*>(st_ptr(wm * 128 + i * 16 + l16, cl)) = w;
      }
    }
  };
  // 256 columns: the rows of the second halves are staged while the first halves' stores
  // drain (the stores do not hold up the wave; the two halves use different LDS rows)
  auto emit = [&](auto z_c, void* dst, int ldo) __attribute__((always_inline)) {
    using H0 = std::integral_constant<int, 0>;
    using H1 = std::integral_constant<int, 1>;
    using HA = std::integral_constant<int, -1>;
    if constexpr (BN == 256) {
      stage_out(z_c, H0{});
      __syncthreads();
      write_staged(dst, ldo, H0{});
      stage_out(z_c, H1{});
      __syncthreads();
      write_staged(dst, ldo, H1{});
    } else {
      stage_out(z_c, HA{});
      __syncthreads();
      write_staged(dst, ldo, HA{});
    }
  };
  if constexpr (I8) {
    // dequantise the exact int32 products in place: acc . sx[m] . sw[n] in fp32 (the fp32 bits
    // kept in the same registers)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float sxm = p.row_scale[min(m0 + wm * 128 + i * 16 + l16, M - 1)];
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const f32x4 swn = *reinterpret_cast<const f32x4*>(p.col_scale + n0 + wn * (BN / 2) + j * 16 + 4 * lq);
        const i32x4 a = acc[i][j];
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (float)a[e] * sxm * swn[e];
        acc[i][j] = __builtin_bit_cast(i32x4, v);
      }
    }
    if (p.r_epi > 0) {
      // the low-rank term s.S.E^T as one bf16 k-tile in smem0 (layout of the loop's seed tile:
      // hi + lo of s.S where 2 r <= 64, else hi), multiplied into the fp32 accumulators
      const int cps = p.r_epi >> 3;
      const int nparts = p.seed_hilo ? 2 : 1;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int part = c / cps, j0 = 8 * (c - part * cps);
        const bool on = part < nparts;
        const int jl = on ? j0 : 0;
        const f32x4 sa = *reinterpret_cast<const f32x4*>(srow + jl);
        const f32x4 sb = *reinterpret_cast<const f32x4*>(srow + jl + 4);
        const u32x4 ev = *reinterpret_cast<const u32x4*>(e0 + (size_t)(n0 + tid) * p.e_ldn + jl);
        const u32x4 z = u32x4{0u, 0u, 0u, 0u};
        lds_st16(smem0, g16_off(tid, c), on ? pack8(sa, sb, live ? p.s_epi : 0.f, part == 1) : z);
        lds_st16(smem0, BM * 128 + g16_off(tid, c), on ? ev : z);
      }
      __syncthreads();
      u32x4 fa[8], fb[FN];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        ldf_rows(smem0, ks, fa, fb);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_bit_cast(i32x4, mfma_bf16(fb[j], fa[i], __builtin_bit_cast(f32x4, acc[i][j])));
      }
      __syncthreads();
    }
    if constexpr (SPLITK) {         // dequantised partial (the low-rank term with the first split)
      write_partial();
      return;
    }
    emit(std::false_type{}, p.out, p.ldo);
  } else if constexpr (DORA) {
    emit(std::true_type{}, p.out2, p.ldo2);
    __syncthreads();                               // the staging buffers are free again
    emit(std::false_type{}, p.out, p.ldo);
  } else if constexpr (SWB) {
    // two passes through the staging tile: de into out, then du into out2; e and u are read
    // for the lane's four columns of each accumulator block (8 bytes each)
    auto emit_swb = [&](auto o_c, void* dst, int ldo) {
      constexpr int O = decltype(o_c)::value;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = wm * 128 + i * 16 + l16;
        const size_t m = (size_t)min(m0 + r, M - 1);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int cl = wn * 128 + j * 16 + 4 * lq;
          const u32x2 ee = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p.aux0) + m * p.ld_aux0 + n0 + cl);
          const float e4[4] = {bf16_lo(ee[0]), bf16_hi(ee[0]), bf16_lo(ee[1]), bf16_hi(ee[1])};
          const f32x4 v = acc[i][j];
          float r4[4];
          if constexpr (O == 0) {
            const u32x2 uu = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p.aux1) + m * p.ld_aux1 + n0 + cl);
            const float u4[4] = {bf16_lo(uu[0]), bf16_hi(uu[0]), bf16_lo(uu[1]), bf16_hi(uu[1])};
#pragma unroll
            for (int e = 0; e < 4; ++e) r4[e] = v[e] * u4[e] * glu_act_grad(e4[e], p.act);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) r4[e] = v[e] * glu_act(e4[e], p.act);
          }
          u32x2 w;
          w[0] = pack_bf16x2(r4[0], r4[1]);
          w[1] = pack_bf16x2(r4[2], r4[3]);
          *reinterpret_cast<u32x2*>(st_ptr(r, cl)) = w;
        }
      }
      __syncthreads();
      uint16_t* out = static_cast<uint16_t*>(dst);
      for (int idx = tid; idx < BM * 32; idx += 256) {
        const int rr0 = idx >> 5, c = idx & 31;
        if (m0 + rr0 < M) {
          const uint8_t* base = rr0 < 128 ? smem0 : smem1;
          const int rr = rr0 & 127;
          st16(out + (size_t)(m0 + rr0) * ldo + n0 + c * 8, lds_ld16(base, rr * 512 + ((c ^ (rr & 31)) << 4)));
        }
      }
    };
    emit_swb(std::integral_constant<int, 0>{}, p.out, p.ldo);
    __syncthreads();
    emit_swb(std::integral_constant<int, 1>{}, p.out2, p.ldo2);
  } else if constexpr (SWF) {
    // Dual tile: waves wn = 0 hold e, waves wn = 1 hold u of the same (token, unit) in the
    // same lanes.  Pass 1 stages both as bf16 (e in staging columns 0..127, u in 128..255)
    // and writes them to out (e) and out2 (u).  Pass 2 hands the fp32 e to the u waves
    // through LDS (lane-linear: each lane writes and reads 16 contiguous bytes per block),
    // which form h = silu(e) u and stage it; it is then written to out3.
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = wm * 128 + i * 16 + l16;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const f32x4 v = acc[i][j];
        u32x2 w;
        w[0] = pack_bf16x2_int(v[0], v[1]);
        w[1] = pack_bf16x2_int(v[2], v[3]);
        *reinterpret_cast<u32x2*>(st_ptr(r, wn * 128 + j * 16 + 4 * lq)) = w;
      }
    }
    __syncthreads();
    for (int idx = tid; idx < BM * 32; idx += 256) {
      const int r = idx >> 5, c = idx & 31;
      if (m0 + r < M) {
        const uint8_t* base = r < 128 ? smem0 : smem1;
        const int rr = r & 127;
        uint16_t* dst = c < 16 ? static_cast<uint16_t*>(p.out) + (size_t)(m0 + r) * p.ldo
                               : static_cast<uint16_t*>(p.out2) + (size_t)(m0 + r) * p.ldo2;
        st16(dst + n0 + 8 * (c & 15), lds_ld16(base, rr * SROW + ((c ^ (rr & SWZM)) << 4)));
      }
    }
    __syncthreads();
    // pass 2, in quarters of each wave's rows (i = 2q, 2q + 1): every wave writes those fp32
    // accumulators to smem0 (lane-linear, 16 KB per wave); then wave (wm, wn) reads e (from
    // wave (wm, 0)) and u (from wave (wm, 1)) of the column blocks j = 4 wn .. 4 wn + 3, forms
    // h and stages it as bf16 in smem1 ([256 rows][128 units], 256-byte rows, 16-byte chunk c
    // of row r at c ^ (r & 15)).  The accumulators are only read, by every wave alike.
    auto xoff = [&](int w, int i, int j) { return (((w * 2 + i) * 8 + j) * 64 + lane) * 16; };
    auto h_ptr = [&](int r, int col) -> uint8_t* {
      return smem1 + r * 256 + ((((col >> 3) ^ (r & 15))) << 4) + ((col & 4) << 1);
    };
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          // through a VGPR copy: a store straight from the accumulator registers changed how
          // the k-loop's accumulators were allocated (moves inside the loop)
          f32x4 v = acc[2 * q + i][j];
          asm volatile("" : "+v"(v));
          *reinterpret_cast<f32x4*>(smem0 + xoff(wave, i, j)) = v;
        }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 128 + (2 * q + i) * 16 + l16;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int j = 4 * wn + jj;
          const f32x4 e = *reinterpret_cast<const f32x4*>(smem0 + xoff(2 * wm, i, j));
          const f32x4 u = *reinterpret_cast<const f32x4*>(smem0 + xoff(2 * wm + 1, i, j));
          u32x2 w;
          w[0] = pack_bf16x2_int(glu_act(e[0], ACT) * u[0], glu_act(e[1], ACT) * u[1]);
          w[1] = pack_bf16x2_int(glu_act(e[2], ACT) * u[2], glu_act(e[3], ACT) * u[3]);
          *reinterpret_cast<u32x2*>(h_ptr(r, j * 16 + 4 * lq)) = w;
        }
      }
      __syncthreads();
    }
    for (int idx = tid; idx < BM * 16; idx += 256) {
      const int r = idx >> 4, c = idx & 15;
      if (m0 + r < M)
        st16(static_cast<uint16_t*>(p.out3) + (size_t)(m0 + r) * p.ldo3 + n0 + 8 * c,
             lds_ld16(smem1, r * 256 + ((c ^ (r & 15)) << 4)));
    }
  } else {
    emit(std::false_type{}, p.out, p.ldo);
  }
}

}  // namespace ldl
