// Block-tiled MFMA GEMM with a fused rank-r LoRA path, for gfx950.
//
//   acc[m, n] = sum_k P[m, k] * Q[k, n]      (fp32 or exact int32 accumulate)
//   out[m, n] = epilogue(acc[m, n] + s_epi * sum_j S[m, j] * E[n, j])
//
// Layouts (all row-major, the reduction index k):
//   P   : [M, K], k contiguous                      (X, dY, H ...)
//   Q   : NT - [N, K], k contiguous                 (W0 in the forward)
//         NN - [K, N], n contiguous                 (W0 in the input-gradient GEMM),
//              up to two segments along k (rows k >= kseg come from b1)
//   S   : either computed in the same K-loop from the staged P tiles as
//         S = P . side^T with side [r, K] k contiguous (the down-projection
//         U = X.A^T of the forward), or read from a precomputed fp32 [M, r_epi]
//   E   : [N, r_epi] given by element strides (lora_up B in the forward,
//         lora_down A^T in the input-gradient GEMM), up to two segments along j.
//
// This is the fused LoRA linear of "How Unsloth's FastLoRA Kernel Differs from
// Standard LoRA Implementations" (section "Fused Forward Pass Architecture")
// and the rank-tiled low-rank epilogue of the 8-bit core in "nunchaku-style
// kernel fusion - 20-30% faster training" (LoRA-epilogue commit): the [N,K]
// product B.A and the [M,N] low-rank product are never stored.
//
// Tiling: 2 x WN waves (WN = 2 or 4: four or eight waves), block tile BM x BN, wave
// tile (BM/2) x (BN/WN) in 32x32 MFMA blocks (v_mfma_f32_32x32x16_bf16 /
// v_mfma_i32_32x32x32_i8), k-tile of 128 bytes per row (64 bf16 or 128 int8),
// a two-stage LDS ring filled by direct buffer-to-LDS copies, one barrier per
// k-tile.  The NN operand is staged through registers instead, transposed
// 8 x 8 and optionally row-scaled (DoRA g, W8A8 sw) on its way into LDS.
#pragma once

#include "common.hpp"

namespace ldl {

enum EpiKind : int {
  EPI_PLAIN = 0,      // out = acc + lora (+ bias)                         -> bf16
  EPI_DORA = 1,       // z = acc + lora; out = z * g[n] (+ bias); out2 = z -> bf16
  EPI_SWIGLU_BWD = 3, // dh = acc + lora; out = dh*gu*silu'(e), out2 = dh*silu(e)
  EPI_DEQUANT = 4,    // int8: acc * sx[m] * sw[n] + lora (+ bias)        -> bf16
  EPI_RAW_I32 = 5,    // int8: raw int32 product
  EPI_SWIGLU_DUAL = 6,// gate and up in one tile: e, u in registers; out = e, out2 = u, out3 = silu(e)*u
};

struct GemmParams {
  int M, N, K;
  const void* a; int lda;            // P, elements
  const float* a_colscale;           // NN: P[m,k] *= a_colscale[k] on load
  const void* b0; const void* b1; int ldb; int kseg;
  const void* side; int r_side;      // fused down-projection rows [r_side, K]
  const float* S; int ld_s;          // precomputed S (fp32)
  int r_epi;                         // rank of the epilogue update (0: none)
  float s_epi;
  float s_epi2;                      // scale of S columns >= e_jsplit (dual gate/up tile: s_up)
  const void* e0; const void* e1; int e_ldn, e_ldj, e_jsplit;
  const float* row_scale;            // [M]  (int8 sx)
  const float* col_scale;            // [N]  (int8 sw / DoRA g)
  const void* bias;                  // [N] bf16
  void* out; int ldo;
  void* out2; int ldo2;
  void* out3; int ldo3;
  const void* aux0; int ld_aux0;
  const void* aux1; int ld_aux1;
  float* side_save; int ld_side_save;
  int q_fp8;                         // NN with 8-bit Q: the codes are e4m3 (else int8)
  // split reduction of the tiles past the last full round (four-wave plain tiles; set by the
  // launcher when part is given): split_s blocks per tile from tile split_first on, fp32
  // partials in part (split_s x 256 x 256 floats per tile), summed by the fixup pass
  int split_s, split_first;
  float* part;
  int seed_hilo;                     // four-wave tile: low-rank term as bf16 hi + lo (set by the launcher)
  int act;                           // gated MLP activation: ACT_SILU, ACT_GELU, ACT_GELU_TANH
  // several adapters over one concatenated output (four-wave NT seed only): output column n
  // belongs to leaf l for leaf_end[l - 1] <= n < leaf_end[l]; rank slots [l r_leaf, (l + 1) r_leaf)
  // of S hold that leaf's down-projection, scaled by leaf_s[l]; E row n holds its leaf's
  // lora_up row (e_ldn = r_leaf) in those slots and zero in the others
  int nleaf, leaf_r;
  int leaf_end[8];
  float leaf_s[8];
};

template <int BM_, int BN_, bool I8_, bool NN_, bool BINT8_, bool ASCALE_, int SIDE_RSP_, bool SLOAD_, int EPI_,
          int WN_ = 2>
struct GemmCfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int kWN = WN_;           // waves along N (two along M)
  static constexpr int kThreads = 128 * WN_;
  static constexpr bool kI8 = I8_;          // P and Q int8 (NT only)
  static constexpr bool kNN = NN_;          // Q is [K, N]
  static constexpr bool kBInt8 = BINT8_;    // NN: Q int8, upcast to bf16 exactly
  static constexpr bool kAScale = ASCALE_;  // NN: column scale on P
  // NN with a plain bf16 Q: Q copied to LDS as-is ([k][n] rows) and read back
  // transposed by ds_read_b64_tr_b16; otherwise staged through registers
  // (a column scale on P is then applied to the Q fragments after the read, from
  // a 64-float slice of the scale vector copied with each stage)
  static constexpr bool kNNTr = NN_ && (BN_ == 64 || BN_ == 128 || BN_ == 256);
  // int8 Q on the transposed path: its rows copied as stored into an int8 staging tile and
  // widened (times the row scale) into the bf16 Q tile at the stage hand-over (int8 or e4m3
  // codes, p.q_fp8)
  static constexpr bool kQ8 = kNNTr && BINT8_;
  static constexpr int kSideRsp = SIDE_RSP_;// fused side rows (padded to 16), 0: none
  static constexpr bool kSLoad = SLOAD_;    // epilogue S from global
  static constexpr int kEpi = EPI_;
};

template <class C>
struct GemmSmem {
  static constexpr int kRows = C::BM + C::BN + C::kSideRsp + ((C::kNNTr && C::kAScale && !C::kQ8) ? 8 : 0);
  static constexpr int kBuf = kRows * 128;
};

__device__ __forceinline__ u32x4 lds_ld16(const uint8_t* base, int off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}
__device__ __forceinline__ void lds_st16(uint8_t* base, int off, u32x4 v) {
  *reinterpret_cast<u32x4*>(base + off) = v;
}

// Element (n, j) of the epilogue up-matrix as bf16 bits (zero outside [0, r_epi)).
__device__ __forceinline__ uint32_t e_elem(const GemmParams& p, int n, int j) {
  if (j >= p.r_epi) return 0u;
  const uint16_t* src;
  int jj = j;
  if (j < p.e_jsplit) src = static_cast<const uint16_t*>(p.e0);
  else { src = static_cast<const uint16_t*>(p.e1); jj = j - p.e_jsplit; }
  return src[(size_t)n * p.e_ldn + (size_t)jj * p.e_ldj];
}

__device__ __forceinline__ u32x4 e_frag(const GemmParams& p, int n, int j0) {
  // 8 consecutive ranks j0..j0+7 of row n of E
  if (p.e_ldj == 1 && j0 + 8 <= p.r_epi && (j0 >= p.e_jsplit || j0 + 8 <= p.e_jsplit)) {
    const uint16_t* src = (j0 < p.e_jsplit) ? static_cast<const uint16_t*>(p.e0) : static_cast<const uint16_t*>(p.e1);
    int jj = (j0 < p.e_jsplit) ? j0 : j0 - p.e_jsplit;
    const uint16_t* q = src + (size_t)n * p.e_ldn + jj;
    if ((((uintptr_t)q) & 15) == 0) return ld16(q);
  }
  u32x4 v;
#pragma unroll
  for (int t = 0; t < 4; ++t) v[t] = e_elem(p, n, j0 + 2 * t) | (e_elem(p, n, j0 + 2 * t + 1) << 16);
  return v;
}

template <class C>
__global__ __launch_bounds__(C::kThreads, 1) void gemm_kernel(const GemmParams p) {
  constexpr int BM = C::BM, BN = C::BN;
  constexpr bool I8 = C::kI8, NN = C::kNN;
  constexpr int RSP = C::kSideRsp;
  constexpr int WN = C::kWN, WM = 2, NW = WM * WN;   // wave grid
  constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 32, FN = TN / 32;   // 32x32 MFMA blocks per wave
  constexpr int BK = I8 ? 128 : 64;     // elements per k-tile (128 bytes per row)
  constexpr int SPW = RSP ? FM / WN : 1; // fused side: 32-row blocks per wave
  static_assert(FM >= 1 && FN >= 1, "wave tile must hold a 32x32 block");
  static_assert(RSP == 0 || (FM % WN == 0), "fused side rows split evenly over the N waves");
  static_assert(RSP % 32 == 0, "side rows are padded to 32");
  static_assert(!NN || !I8, "NN takes bf16 P");
  using Acc = typename std::conditional<I8, i32x16, f32x16>::type;

  // two LDS stages, each [BM rows of P | BN rows of Q | RSP side rows] x 128 bytes;
  // the epilogue reuses both as one output staging tile
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * GemmSmem<C>::kBuf];
  uint8_t* const smem0 = smem;
  uint8_t* const smem1 = smem + GemmSmem<C>::kBuf;
  // int8 Q: one stage of Q rows as stored ([64][BN] bytes) and its 64 row scales (1 KB copy)
  constexpr bool Q8 = C::kQ8;
  __shared__ __attribute__((aligned(16))) uint8_t s8[Q8 ? 64 * BN + 1024 : 16];

  const int M = p.M, N = p.N, K = p.K;
  // Dual gate/up tile: BN rows of Q = BN/2 gate rows and the BN/2 up rows of the
  // same hidden units, arranged per wave as [gate TN/2 | up TN/2], so that the
  // accumulator blocks j and j + FN/2 of a lane hold e and u of one (m, h).
  constexpr bool DUAL = (C::kEpi == EPI_SWIGLU_DUAL);
  constexpr int OUT_BN = DUAL ? BN / 2 : BN;     // output columns per tile
  const int tiles_m = (M + BM - 1) / BM, tiles_n = N / OUT_BN;

  // Tile order: consecutive workgroups go round-robin over the 8 XCDs, so
  // remap ids so that each XCD receives a contiguous range, then walk that
  // range in groups of GM row-tiles (tiles sharing P rows and Q columns stay
  // on one XCD's L2).
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  constexpr int GM = 4;
  const int group = bid / (GM * tiles_n);
  const int first_m = group * GM;
  const int gm = min(GM, tiles_m - first_m);
  const int in_g = bid - group * GM * tiles_n;
  const int tm = first_m + in_g % gm;
  const int tn = in_g / gm;
  const int m0 = tm * BM, n0 = tn * OUT_BN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 31, lq = lane >> 5;    // fragment row / 16-byte chunk within a step

  const uint32_t lda_b = (uint32_t)p.lda * (I8 ? 1 : 2);
  const uint32_t ldb_b = (uint32_t)p.ldb * ((I8 || C::kBInt8) ? 1 : 2);

  // Per-lane 32-bit source offsets for the direct copies (operands are below
  // 4 GiB, checked on the host).  One wave instruction fills 64 consecutive
  // 16-byte LDS slots = 8 rows; slot (row, phys) receives the logical chunk
  // phys ^ swz(row) of that row.  Rows past the end of an operand (P rows
  // >= M, side rows >= r) read as zero through the buffer bounds.
  const int lrow = lane >> 3, lphys = lane & 7;
  constexpr int A_INST = BM / (8 * NW);       // per wave
  constexpr bool NNTR = C::kNNTr;
  // NN-tr: the Q k-tile is 64 rows of BN bf16 (BN / 8 chunks of 16 bytes per row);
  // chunk c of row k sits at physical chunk c ^ tr_swz(k)
  constexpr int B_INST = NNTR ? (Q8 ? BN / (16 * NW) : BN / (8 * NW)) : (NN ? 0 : BN / (8 * NW));
  static_assert(!Q8 || BN % (16 * NW) == 0, "int8 Q rows split evenly over the waves");
  constexpr int S_INST = (RSP + 8 * NW - 1) / (8 * NW);
  // rows k .. k+3 of one transposing read land on distinct banks
  auto tr_swz = [](int k) { return 2 * (k & 3); };
  // byte offset of element (k, n) (4-column aligned) in the NN-tr Q tile
  auto tr_off = [&](int k, int n) { return k * (BN * 2) + ((((n >> 3) ^ tr_swz(k))) << 4) + ((n & 4) << 1); };
  static_assert(BM % (8 * NW) == 0 && (NN || BN % (8 * NW) == 0), "tile rows split evenly over the waves");
  const __amdgpu_buffer_rsrc_t rs_a = make_rsrc(p.a, (uint32_t)M * lda_b);
  const __amdgpu_buffer_rsrc_t rs_b =
      make_rsrc(p.b0, NNTR ? (uint32_t)p.kseg * ldb_b : (NN ? 0u : (uint32_t)N * ldb_b));
  const __amdgpu_buffer_rsrc_t rs_b2 =
      NNTR ? make_rsrc(p.b1, (uint32_t)(K - p.kseg) * ldb_b)
           : make_rsrc(DUAL ? p.b1 : p.b0, NN ? 0u : (uint32_t)N * ldb_b);
  const __amdgpu_buffer_rsrc_t rs_s = make_rsrc(p.side, RSP ? (uint32_t)p.r_side * (uint32_t)K * 2u : 0u);
  constexpr bool TRSC = NNTR && C::kAScale && !Q8;   // scale slice: 1 KB after the Q tile, first 256 B used
  // copy slices per stage (see issue_loads); the register-staged NN operand is loaded whole
  constexpr int NPART = (NN && !NNTR) ? 1 : 3;
  constexpr bool SPLIT = NPART > 1;
  const __amdgpu_buffer_rsrc_t rs_c = make_rsrc(p.a_colscale, (TRSC || Q8) ? (uint32_t)K * 4u : 0u);
  uint32_t a_off[A_INST];
#pragma unroll
  for (int i = 0; i < A_INST; ++i) {
    const int row = (i * NW + wave) * 8 + lrow;
    a_off[i] = (uint32_t)(m0 + row) * lda_b + ((lphys ^ swz(row)) << 4);
  }
  uint32_t b_off[B_INST ? B_INST : 1];
#pragma unroll
  for (int i = 0; i < B_INST; ++i) {
    if constexpr (Q8) {           // 16 int8 of row krow, stored as is: s8[krow][16 c16 ..]
      const int slot = (i * NW + wave) * 64 + lane;
      const int krow = slot / (BN / 16), c16 = slot % (BN / 16);
      b_off[i] = (uint32_t)krow * ldb_b + (uint32_t)(n0 + 16 * c16);
      continue;
    } else if constexpr (NNTR) {
      const int slot = (i * NW + wave) * 64 + lane;          // 16-byte slot of the k-tile
      const int krow = slot / (BN / 8), phys = slot % (BN / 8);
      b_off[i] = (uint32_t)krow * ldb_b + (uint32_t)(n0 + 8 * (phys ^ tr_swz(krow))) * 2u;
      continue;
    }
    const int row = (i * NW + wave) * 8 + lrow;
    int qrow = n0 + row;
    if constexpr (DUAL) {   // tile row -> (gate | up) row of hidden unit h
      const int within = row % TN;
      qrow = n0 + (row / TN) * (TN / 2) + within % (TN / 2);
    }
    b_off[i] = (uint32_t)qrow * ldb_b + ((lphys ^ swz(row)) << 4);
  }
  uint32_t s_off[S_INST ? S_INST : 1];
#pragma unroll
  for (int i = 0; i < S_INST; ++i) {
    const int row = (i * NW + wave) * 8 + lrow;      // side row
    s_off[i] = (uint32_t)row * (uint32_t)K * 2u + ((lphys ^ swz(BN + row)) << 4);
  }

  Acc acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = Acc{};
  f32x16 sacc[SPW][RSP ? RSP / 32 : 1];
  if constexpr (RSP > 0) {
#pragma unroll
    for (int i = 0; i < SPW; ++i)
#pragma unroll
      for (int j = 0; j < RSP / 32; ++j) sacc[i][j] = f32x16{};
  }

  // NN: each thread stages RPT rows x 8 columns of Q for the transpose; with 512
  // threads the 64 x BN k-tile is covered by 4-row slices (RPT_SLOTS = 2 per column group)
  constexpr int RPT = (NN && NW == 8) ? 4 : 8;
  constexpr int RPT_SLOTS = 8 / RPT;
  static_assert(!NN || BN * RPT_SLOTS <= 64 * NW, "enough threads to stage the NN tile");
  u32x4 rb[NN ? RPT : 1];

  // ---------------------------------------------------------------- loaders
  // the wave's copy instructions of one stage, in order: P tile, Q tile, side rows, scale slice
  constexpr int NCOPY = A_INST + ((NN && !NNTR) ? 0 : B_INST + S_INST + ((TRSC || Q8) ? 1 : 0));
  auto issue_one = [&](int kt, uint8_t* sbuf, int q) {
    const uint32_t koff = (uint32_t)kt * 128u;
    if (q < A_INST) {
      buf2lds16(rs_a, a_off[q], koff, sbuf + (q * NW + wave) * 1024);
      return;
    }
    q -= A_INST;
    uint8_t* sB = sbuf + BM * 128;
    if constexpr (!NN) {
      if (q < B_INST) {
        const bool up = DUAL && ((((q * NW + wave) * 8) % TN) >= TN / 2);
        buf2lds16(up ? rs_b2 : rs_b, b_off[q], koff, sB + (q * NW + wave) * 1024);
        return;
      }
      q -= B_INST;
      if (q < S_INST && (q * NW + wave) * 8 < RSP) buf2lds16(rs_s, s_off[q], koff, sB + BN * 128 + (q * NW + wave) * 1024);
    } else if constexpr (NNTR) {
      const int kk0 = kt * 64;
      const bool seg1 = kk0 >= p.kseg;
      const uint32_t boff = (uint32_t)(seg1 ? kk0 - p.kseg : kk0) * ldb_b;
      if (q < B_INST) {
        buf2lds16(seg1 ? rs_b2 : rs_b, b_off[q], boff, (Q8 ? s8 : sB) + (q * NW + wave) * 1024);
        return;
      }
      if constexpr (TRSC || Q8) {
        if (wave == NW - 1) buf2lds16(rs_c, (uint32_t)lane * 16u, (uint32_t)kt * 256u, Q8 ? s8 + 64 * BN : sB + BN * 128);
      }
    }
  };

  // Copies of a stage are issued in NPART slices (instruction q of this wave goes
  // with slice q % NPART) spread over the MFMA steps, so that a wave never sits
  // through a whole stage's worth of copy issue (the address unit accepts them at
  // a limited rate) while the matrix pipe idles.  part < 0: every slice.
  auto issue_loads = [&](int kt, uint8_t* sbuf, int part) {
    const uint32_t koff = (uint32_t)kt * 128u;
    auto mine = [&](int q) { return part < 0 || q % NPART == part; };
#pragma unroll
    for (int i = 0; i < A_INST; ++i)
      if (mine(i)) buf2lds16(rs_a, a_off[i], koff, sbuf + (i * NW + wave) * 1024);
    if constexpr (!NN) {
      uint8_t* sB = sbuf + BM * 128;
#pragma unroll
      for (int i = 0; i < B_INST; ++i) {
        // the up half of each wave's rows comes from the second matrix (uniform per instruction)
        const bool up = DUAL && ((((i * NW + wave) * 8) % TN) >= TN / 2);
        if (mine(A_INST + i)) buf2lds16(up ? rs_b2 : rs_b, b_off[i], koff, sB + (i * NW + wave) * 1024);
      }
#pragma unroll
      for (int i = 0; i < S_INST; ++i)
        if ((i * NW + wave) * 8 < RSP && mine(A_INST + B_INST + i))
          buf2lds16(rs_s, s_off[i], koff, sB + BN * 128 + (i * NW + wave) * 1024);
    } else if constexpr (NNTR) {
      // Q is [K, N]: rows kt*64 .. +63 of the segment that holds them (k-tiles never straddle kseg)
      uint8_t* sB = sbuf + BM * 128;
      const int kk0 = kt * 64;
      const bool seg1 = kk0 >= p.kseg;
      const uint32_t boff = (uint32_t)(seg1 ? kk0 - p.kseg : kk0) * ldb_b;
#pragma unroll
      for (int i = 0; i < B_INST; ++i)
        if (mine(A_INST + i)) buf2lds16(seg1 ? rs_b2 : rs_b, b_off[i], boff, (Q8 ? s8 : sB) + (i * NW + wave) * 1024);
      // scale[kt*64 ..] -> lanes 0..15 fill the slice; the rest read ahead (or zero past the end)
      if constexpr (TRSC || Q8) {
        if (wave == NW - 1 && mine(A_INST + B_INST))
          buf2lds16(rs_c, (uint32_t)lane * 16u, (uint32_t)kt * 256u, Q8 ? s8 + 64 * BN : sB + BN * 128);
      }
    } else {
      if (part > 0) return;
      // Q is [K, N]: this k-tile covers reduction rows kt*64 .. +63.  Each thread
      // stages RPT rows x 8 columns (RPT = 8 with 256 threads, 4 with 512).
      const int kk0 = kt * 64;
      const uint8_t* pb;
      int krow0;
      if (kk0 < p.kseg) { pb = static_cast<const uint8_t*>(p.b0); krow0 = kk0; }
      else { pb = static_cast<const uint8_t*>(p.b1); krow0 = kk0 - p.kseg; }
      if (tid < BN * RPT_SLOTS) {
        const int kb = tid % (BN / 8), nb = tid / (BN / 8);
#pragma unroll
        for (int e = 0; e < RPT; ++e) {
          const size_t rowoff = (size_t)(krow0 + nb * RPT + e) * (size_t)ldb_b;
          if constexpr (C::kBInt8) {
            u32x2 v = *reinterpret_cast<const u32x2*>(pb + rowoff + (size_t)(n0 + kb * 8));
            rb[e] = i8x8_to_bf16x8(v);
          } else {
            rb[e] = ld16(pb + rowoff + (size_t)(n0 + kb * 8) * 2);
          }
        }
      }
    }
  };

  // NN only: scale (optional) and transpose the staged Q rows into LDS.
  auto store_q = [&](int kt, uint8_t* sbuf) {
    if constexpr (NN && !NNTR) {
      if (tid < BN * RPT_SLOTS) {
        uint8_t* sB = sbuf + BM * 128;
        const int kb = tid % (BN / 8), nb = tid / (BN / 8);
        if constexpr (C::kAScale) {
          const f32x4* sc = reinterpret_cast<const f32x4*>(p.a_colscale + (size_t)kt * 64 + nb * RPT);
          float f[RPT];
#pragma unroll
          for (int q = 0; q < RPT / 4; ++q) {
            const f32x4 v4 = sc[q];
            f[4 * q] = v4[0]; f[4 * q + 1] = v4[1]; f[4 * q + 2] = v4[2]; f[4 * q + 3] = v4[3];
          }
#pragma unroll
          for (int e = 0; e < RPT; ++e) {
            const f32x4 se = f32x4{f[e], f[e], f[e], f[e]};
            rb[e] = scale_bf16x8(rb[e], se, se);
          }
        }
        if constexpr (RPT == 8) {
          u32x4 t[8];
          transpose8x8_b16(rb, t);
#pragma unroll
          for (int c = 0; c < 8; ++c) lds_st16(sB, lds_off(kb * 8 + c, nb), t[c]);
        } else {
          // 4 rows x 8 columns -> 8 columns of 4 values, written as 8-byte halves of a chunk
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) {
            u32x2 lo, hi;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const uint32_t a = rb[2 * j][cc], b = rb[2 * j + 1][cc];
              lo[j] = (a & 0xffffu) | (b << 16);
              hi[j] = (a >> 16) | (b & 0xffff0000u);
            }
            *reinterpret_cast<u32x2*>(sB + lds_off(kb * 8 + 2 * cc, nb >> 1) + (nb & 1) * 8) = lo;
            *reinterpret_cast<u32x2*>(sB + lds_off(kb * 8 + 2 * cc + 1, nb >> 1) + (nb & 1) * 8) = hi;
          }
        }
      }
    }
  };

  // One MFMA step = 16 bf16 (or 32 int8) of the reduction = two 16-byte chunks;
  // a k-tile holds four steps.  Fragments are double-buffered in registers:
  // the LDS reads of step ks+1 are issued before the MFMAs of step ks, so the
  // matrix pipe never waits on LDS inside a k-tile.
  auto load_frags = [&](const uint8_t* sbuf, int ks, u32x4* af, u32x4* bf, u32x4* sf) {
    const uint8_t* sA = sbuf;
    const uint8_t* sB = sbuf + BM * 128;
#pragma unroll
    for (int i = 0; i < FM; ++i) af[i] = lds_ld16(sA, lds_off(wm * TM + i * 32 + lr, ks * 2 + lq));
    if constexpr (NNTR) {
      // lane l needs column wn*TN + 32 j + (l & 31) at k = 16 ks + 8 (l >> 5) + e, e < 8: its
      // 16-lane group reads 4 k rows x 16 columns per instruction (see lds_tr16), twice
      const int g = lane >> 4, jl = lane & 15;
      const int kr = ks * 16 + 8 * (g >> 1) + (jl >> 2);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = wn * TN + j * 32 + 16 * (g & 1) + 4 * (jl & 3);
        const u32x2 lo = lds_tr16(sB, tr_off(kr, n));
        const u32x2 hi = lds_tr16(sB, tr_off(kr + 4, n));
        bf[j] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
      if constexpr (TRSC) {
        // Q row k scaled by scale[k]: this lane's eight reduction indices 16 ks + 8 (l >> 5) + e
        const f32x4* sc = reinterpret_cast<const f32x4*>(sB + BN * 128 + (ks * 16 + 8 * lq) * 4);
        const f32x4 s0 = sc[0], s1 = sc[1];
#pragma unroll
        for (int j = 0; j < FN; ++j) bf[j] = scale_bf16x8(bf[j], s0, s1);
      }
    } else {
#pragma unroll
      for (int j = 0; j < FN; ++j) bf[j] = lds_ld16(sB, lds_off(wn * TN + j * 32 + lr, ks * 2 + lq));
    }
    if constexpr (RSP > 0) {
#pragma unroll
      for (int js = 0; js < RSP / 32; ++js) sf[js] = lds_ld16(sB, lds_off(BN + js * 32 + lr, ks * 2 + lq));
    }
  };
  // Once a wave has started a cluster of MFMAs it takes issue priority over the
  // other wave of its SIMD until the cluster ends, so the two waves alternate
  // between MFMA clusters and their LDS / copy work instead of interleaving both.
  auto mfmas = [&](const u32x4* af, const u32x4* bf, const u32x4* sf, auto&& between) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        between(i * FN + j);
        if constexpr (I8) acc[i][j] = mfma32_i8(bf[j], af[i], acc[i][j]);
        else acc[i][j] = mfma32_bf16(bf[j], af[i], acc[i][j]);
        if (i == 0 && j == 0) {
          __builtin_amdgcn_sched_barrier(0);
          __builtin_amdgcn_s_setprio(1);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    if constexpr (RSP > 0) {
#pragma unroll
      for (int js = 0; js < RSP / 32; ++js) {
#pragma unroll
        for (int w = 0; w < WN; ++w) {
          if (wn == w) {   // uniform branch keeps the fragment index compile-time
#pragma unroll
            for (int i = 0; i < SPW; ++i) sacc[i][js] = mfma32_bf16(sf[js], af[w * SPW + i], sacc[i][js]);
          }
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
  };
  constexpr int SF = RSP ? RSP / 32 : 1;

  // Low-rank update dst[i][jj] += (s_epi * S[m, :]) . E[n, :]^T for the column blocks
  // jc .. jc + NJ - 1 of this wave, in 16-rank MFMA steps (S rounded to bf16 after
  // scaling; the dual gate/up tile masks the ranks of the other half).
  auto lora_update = [&](auto& dst, auto jc_const) {
    constexpr int jc = decltype(jc_const)::value;
    constexpr int NJ = sizeof(dst[0]) / sizeof(dst[0][0]);
    if (p.r_epi <= 0) return;
    const uint16_t* sS = reinterpret_cast<const uint16_t*>(smem0);
    const int nsteps = (p.r_epi + 15) / 16;
    for (int t = 0; t < nsteps; ++t) {
      const int j0 = t * 16 + lq * 8;
      u32x4 sf[FM];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int row = wm * TM + i * 32 + lr;
        sf[i] = u32x4{0, 0, 0, 0};
        if constexpr (RSP > 0) {
          if (j0 < RSP) sf[i] = *reinterpret_cast<const u32x4*>(sS + row * RSP + j0);
        } else if constexpr (C::kSLoad) {
          const int m = m0 + row;
          if (m < M && j0 < p.r_epi) {
            const float* src = p.S + (size_t)m * p.ld_s + j0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              // dual tile: up ranks [r, 2r) take s_up (8-rank groups never straddle r, r % 8 == 0)
              const float sc = (DUAL && j0 >= p.e_jsplit) ? p.s_epi2 : p.s_epi;
              const float lo = (j0 + 2 * e < p.r_epi) ? src[2 * e] * sc : 0.f;
              const float hi = (j0 + 2 * e + 1 < p.r_epi) ? src[2 * e + 1] * sc : 0.f;
              sf[i][e] = pack_bf16x2(lo, hi);
            }
          }
        }
      }
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
        u32x4 ef;
        if constexpr (DUAL) {
          // gate blocks take ranks [0, r) of Bg, up blocks ranks [r, 2r) of Bu
          constexpr int HB = FN / 2;
          const bool upb = (jc + jj) >= HB;
          const int h = n0 + wn * (OUT_BN / WN) + ((jc + jj) % HB) * 32 + lr;
          const bool mine = upb ? (j0 >= p.e_jsplit) : (j0 < p.e_jsplit);
          ef = mine ? e_frag(p, h, j0) : u32x4{0, 0, 0, 0};
        } else {
          ef = e_frag(p, n0 + wn * TN + (jc + jj) * 32 + lr, j0);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) dst[i][jj] = mfma32_bf16(ef, sf[i], dst[i][jj]);
      }
    }
  };
  // bf16 tiles with a precomputed S start their accumulators from the low-rank
  // product (computed while the first stage's copies are in flight) instead of
  // adding it in the epilogue
  constexpr bool SEED = !I8 && RSP == 0 && C::kSLoad;

  // int8 Q: widen the landed stage in s8 into sbuf's Q tile (the transposed-path layout the
  // bf16 copies produce), row k times its scale: (u - 128) s for the biased byte u = q + 128
  // is one fma, rounded once to fp32 and once to bf16 (as bf16(q) * s rounded to bf16).
  // Thread t takes 16-byte units t, t + threads, .. (consecutive lanes, consecutive bytes).
  auto convert_q8 = [&](uint8_t* sbuf) {
    if constexpr (Q8) {
      typedef float f2 __attribute__((ext_vector_type(2)));
      typedef __bf16 b2 __attribute__((ext_vector_type(2)));
      uint8_t* sB = sbuf + BM * 128;
      const float* sc8 = reinterpret_cast<const float*>(s8 + 64 * BN);
      const bool f8 = p.q_fp8 != 0;
#pragma unroll
      for (int u = tid; u < 4 * BN; u += C::kThreads) {
        const int k = u / (BN / 16), c16 = u % (BN / 16);
        const u32x4 v = lds_ld16(s8, u * 16);
        const float sc = sc8[k], c0 = -128.f * sc;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          u32x4 o;
#pragma unroll
          for (int d = 0; d < 2; ++d) {
            f2 lo, hi;
            if (f8) {            // e4m3 codes: exact fp32 values, times the row scale
              const uint32_t w = v[2 * h + d];
              lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false) * sc;
              hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true) * sc;
            } else {
              const uint32_t w = v[2 * h + d] ^ 0x80808080u;
              lo = f2{__builtin_fmaf((float)(w & 0xffu), sc, c0), __builtin_fmaf((float)((w >> 8) & 0xffu), sc, c0)};
              hi = f2{__builtin_fmaf((float)((w >> 16) & 0xffu), sc, c0), __builtin_fmaf((float)(w >> 24), sc, c0)};
            }
            o[2 * d] = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, b2));
            o[2 * d + 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, b2));
          }
          lds_st16(sB, k * (BN * 2) + (((2 * c16 + h) ^ tr_swz(k)) << 4), o);
        }
      }
    }
  };

  // ---------------------------------------------------------------- main loop
  // Stage kt lives in smem[kt & 1].  The hand-over to the next stage sits
  // between the last two MFMA steps of a k-tile: wait for the next stage's
  // copies, barrier (every wave has finished reading this stage, so its
  // buffer can take the copies of stage kt + 2), start those copies and the
  // LDS reads of the next stage's first step, then run this stage's last
  // MFMAs, which hide the barrier and the LDS latency.  (A single call site
  // per step keeps the accumulators in place; unrolling the two stages made
  // the register allocator rotate them every iteration.)
  const int KT = K / BK;
  u32x4 fa0[FM], fb0[FN], fs0[SF], fa1[FM], fb1[FN], fs1[SF];
  issue_loads(0, smem0, -1);
  if constexpr (SEED) lora_update(acc, std::integral_constant<int, 0>{});
  store_q(0, smem0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if constexpr (Q8) {
    convert_q8(smem0);
    __syncthreads();
  }
  if (KT > 1) issue_loads(1, smem1, -1);
  load_frags(smem0, 0, fa0, fb0, fs0);
  // settle every LDS / scalar read of the prologue (not the copies in flight)
  // so that the waits inside the loop can count the fragment reads exactly
  __builtin_amdgcn_s_waitcnt(0xc07f);
  // A stage's copies are spread over three MFMA clusters (the hand-over cluster of
  // stage kt and the first two of stage kt+1), at most CPC per cluster, each copy
  // placed between two MFMAs: a copy instruction holds the issuing wave for a
  // while (the address unit takes them at a limited rate), and in one burst the
  // waves would leave the matrix pipe idle.
  constexpr int NMF = FM * FN;
  constexpr int CPC = (NCOPY + 2) / 3;
  auto copies_between = [&](int kt, uint8_t* sbuf, int cluster, bool on) {
    return [&, kt, sbuf, cluster, on](int t) {
      if (!on) return;
#pragma unroll
      for (int u = 0; u < CPC; ++u) {
        const int q = cluster * CPC + u;
        if (q < NCOPY && t == u * (NMF / CPC)) {
          __builtin_amdgcn_sched_barrier(0);
          issue_one(kt, sbuf, q);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
  };
  auto none = [](int) {};
  // steps 0..2 of stage kt (step 0's fragments already in fa0), leaving step 3's in fa1
  auto first_steps = [&](int kt, uint8_t* cur, uint8_t* nxt, bool more) {
    const bool tail = SPLIT && more && kt >= 1;          // clusters 1, 2 of stage kt+1's copies
    __builtin_amdgcn_sched_barrier(0);
    load_frags(cur, 1, fa1, fb1, fs1);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(fa0, fb0, fs0, copies_between(kt + 1, nxt, 1, tail));
    __builtin_amdgcn_sched_barrier(0);
    load_frags(cur, 2, fa0, fb0, fs0);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(fa1, fb1, fs1, copies_between(kt + 1, nxt, 2, tail));
    __builtin_amdgcn_sched_barrier(0);
    if (more) store_q(kt + 1, nxt);
    load_frags(cur, 3, fa1, fb1, fs1);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(fa0, fb0, fs0, none);
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int kt = 0; kt + 1 < KT; ++kt) {
    uint8_t* cur = (kt & 1) ? smem1 : smem0;
    uint8_t* nxt = (kt & 1) ? smem0 : smem1;
    first_steps(kt, cur, nxt, true);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if constexpr (Q8) {              // stage kt+1's int8 rows have landed; s8 is free after this
      convert_q8(nxt);
      __syncthreads();
    }
    if (!SPLIT && kt + 2 < KT) issue_loads(kt + 2, cur, -1);
    load_frags(nxt, 0, fa0, fb0, fs0);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(fa1, fb1, fs1, copies_between(kt + 2, cur, 0, SPLIT && kt + 2 < KT));
  }
  {
    uint8_t* cur = ((KT - 1) & 1) ? smem1 : smem0;
    first_steps(KT - 1, cur, cur, false);
    mfmas(fa1, fb1, fs1, none);
  }
  __syncthreads();

  // ---------------------------------------------------------------- epilogue
  // acc[i][j] lane l, element v: output row m = mrow_base + 32 i + (l & 31),
  // output columns n = ncol_base + 32 j + 8 (v >> 2) + 4 (l >> 5) + (v & 3).
  const int mrow_base = m0 + wm * TM;
  const int ncol_base = n0 + wn * (OUT_BN / WN) + 4 * lq;   // columns of block j: + 32 j (dual: j < FN/2)

  // Fused side: publish s_epi * U (bf16) to LDS for the rank-r product, save U (fp32).
  if constexpr (RSP > 0) {
    uint16_t* sS = reinterpret_cast<uint16_t*>(smem0);
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int row = wm * TM + (wn * SPW + i) * 32 + lr;
      const int m = m0 + row;
#pragma unroll
      for (int js = 0; js < RSP / 32; ++js) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int j0 = js * 32 + 8 * g + 4 * lq;
          const f32x16 u = sacc[i][js];
          u32x2 w;
          w[0] = pack_bf16x2(u[4 * g] * p.s_epi, u[4 * g + 1] * p.s_epi);
          w[1] = pack_bf16x2(u[4 * g + 2] * p.s_epi, u[4 * g + 3] * p.s_epi);
          *reinterpret_cast<u32x2*>(sS + row * RSP + j0) = w;
          if (p.side_save != nullptr && tn == 0 && m < M) {
            float* dst = p.side_save + (size_t)m * p.ld_side_save;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (j0 + e < p.r_side) dst[j0 + e] = u[4 * g + e];
          }
        }
      }
    }
    __syncthreads();
  }

  // The epilogue walks the accumulator tile in column chunks so that the
  // fp32 copy of an int32 tile never doubles the live registers.
  constexpr int JC = I8 ? 1 : FN;
  static_assert(FN % JC == 0, "column chunking");
  constexpr int EPI = C::kEpi;
  // bf16 outputs go through LDS (one output array at a time) and leave the
  // tile as whole 16-byte row segments; the raw int32 product and the fused
  // side path (whose U tile occupies LDS) store straight from registers.
  constexpr bool STAGE = (RSP == 0) && (EPI != EPI_RAW_I32);
  constexpr int NOUT = (EPI == EPI_SWIGLU_DUAL) ? 3 : ((EPI == EPI_DORA || EPI == EPI_SWIGLU_BWD) ? 2 : 1);
  static_assert(!STAGE || NOUT == 1 || JC == FN, "several staged outputs need the whole tile in registers");
  static_assert(!STAGE || (size_t)BM * OUT_BN * 2 <= 2 * (size_t)GemmSmem<C>::kBuf, "staging tile fits in LDS");
  constexpr int NCH = OUT_BN / 8;                         // 16-byte chunks per staged row
  constexpr int SWM = (NCH & (NCH - 1)) == 0 ? (NCH < 32 ? NCH - 1 : 31) : 7;

  // fp32 tile of column chunk jc: accumulator (dequantised for int8) plus the rank-r update
  auto make_facc = [&](auto jc_const, f32x16 (&facc)[FM][JC]) {
    constexpr int jc = decltype(jc_const)::value;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int jj = 0; jj < JC; ++jj) {
        if constexpr (I8) {
          const int m = mrow_base + i * 32 + lr;
          const float sxm = (m < M) ? p.row_scale[m] : 0.f;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 swn = *reinterpret_cast<const f32x4*>(p.col_scale + ncol_base + (jc + jj) * 32 + 8 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) facc[i][jj][4 * g + e] = float(acc[i][jc + jj][4 * g + e]) * sxm * swn[e];
          }
        } else {
          facc[i][jj] = acc[i][jc + jj];
        }
      }
    if constexpr (!SEED) lora_update(facc, jc_const);
  };

  // Output o of the four columns n .. n+3 of row m (values v), as packed bf16.
  auto out_vals = [&](auto o_const, int m, int n, const float* v, const float* vu) -> u32x2 {
    constexpr int o = decltype(o_const)::value;
    u32x2 w;
    if constexpr (DUAL) {            // o: 0 e, 1 u, 2 act(e) * u
      if constexpr (o == 0) { w[0] = pack_bf16x2(v[0], v[1]); w[1] = pack_bf16x2(v[2], v[3]); }
      else if constexpr (o == 1) { w[0] = pack_bf16x2(vu[0], vu[1]); w[1] = pack_bf16x2(vu[2], vu[3]); }
      else {
        w[0] = pack_bf16x2(glu_act(v[0], p.act) * vu[0], glu_act(v[1], p.act) * vu[1]);
        w[1] = pack_bf16x2(glu_act(v[2], p.act) * vu[2], glu_act(v[3], p.act) * vu[3]);
      }
    } else if constexpr (EPI == EPI_PLAIN || EPI == EPI_DEQUANT || EPI == EPI_DORA) {
      float b4[4] = {0.f, 0.f, 0.f, 0.f};
      if (p.bias != nullptr && !(EPI == EPI_DORA && o == 1)) {
        const u32x2 bb = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p.bias) + n);
        b4[0] = bf16_lo(bb[0]); b4[1] = bf16_hi(bb[0]); b4[2] = bf16_lo(bb[1]); b4[3] = bf16_hi(bb[1]);
      }
      if constexpr (EPI == EPI_DORA && o == 0) {   // y = z * g + bias
        const f32x4 gs = *reinterpret_cast<const f32x4*>(p.col_scale + n);
        w[0] = pack_bf16x2(v[0] * gs[0] + b4[0], v[1] * gs[1] + b4[1]);
        w[1] = pack_bf16x2(v[2] * gs[2] + b4[2], v[3] * gs[3] + b4[3]);
      } else {                                     // plain / dequantised output, or DoRA's z
        w[0] = pack_bf16x2(v[0] + b4[0], v[1] + b4[1]);
        w[1] = pack_bf16x2(v[2] + b4[2], v[3] + b4[3]);
      }
    } else if constexpr (EPI == EPI_SWIGLU_BWD) {  // o: 0 de, 1 dgu
      // rows past M are staged but never written out; their e and u reads stay on row M - 1
      const size_t mr = (size_t)min(m, M - 1);
      const u32x2 ee = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p.aux0) + mr * p.ld_aux0 + n);
      const float e4[4] = {bf16_lo(ee[0]), bf16_hi(ee[0]), bf16_lo(ee[1]), bf16_hi(ee[1])};
      float r4[4];
      if constexpr (o == 0) {
        const u32x2 gg = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p.aux1) + mr * p.ld_aux1 + n);
        const float g4[4] = {bf16_lo(gg[0]), bf16_hi(gg[0]), bf16_lo(gg[1]), bf16_hi(gg[1])};
#pragma unroll
        for (int e = 0; e < 4; ++e) r4[e] = v[e] * g4[e] * glu_act_grad(e4[e], p.act);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) r4[e] = v[e] * glu_act(e4[e], p.act);
      }
      w[0] = pack_bf16x2(r4[0], r4[1]);
      w[1] = pack_bf16x2(r4[2], r4[3]);
    }
    return w;
  };
  auto out_ptr = [&](int o) -> uint16_t* {
    return static_cast<uint16_t*>(o == 0 ? p.out : (o == 1 ? p.out2 : p.out3));
  };
  auto out_ld = [&](int o) -> int { return o == 0 ? p.ldo : (o == 1 ? p.ldo2 : p.ldo3); };

  // Visit the 4-column groups of column chunk jc: f(i, jj, g, m, n_global, col_local, v, vu).
  auto for_groups = [&](auto jc_const, const f32x16 (&facc)[FM][JC], auto&& f) {
    constexpr int jc = decltype(jc_const)::value;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int m = mrow_base + i * 32 + lr;
#pragma unroll
      for (int jj = 0; jj < JC; ++jj) {
        if constexpr (DUAL) {
          if (jc + jj >= FN / 2) continue;
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int cl = wn * (OUT_BN / WN) + (jc + jj) * 32 + 8 * g + 4 * lq;
          const f32x16& va = facc[i][jj];
          const float v[4] = {va[4 * g], va[4 * g + 1], va[4 * g + 2], va[4 * g + 3]};
          float vu[4] = {0.f, 0.f, 0.f, 0.f};
          if constexpr (DUAL) {
            const f32x16& vb = facc[i][jj + FN / 2];
            vu[0] = vb[4 * g]; vu[1] = vb[4 * g + 1]; vu[2] = vb[4 * g + 2]; vu[3] = vb[4 * g + 3];
          }
          f(m, n0 + cl, cl, v, vu);
        }
      }
    }
  };

  if constexpr (STAGE) {
    // staged row r, 16-byte chunk c lives at r * OUT_BN * 2 + ((c ^ (r & SWM)) << 4)
    auto st_off = [&](int r, int col) { return r * (OUT_BN * 2) + (((col >> 3) ^ (r & SWM)) << 4) + ((col & 4) << 1); };
    auto copy_out = [&](int o) {
      uint16_t* dst = out_ptr(o);
      const int ldo = out_ld(o);
      for (int idx = tid; idx < BM * NCH; idx += C::kThreads) {
        const int r = idx / NCH, c = idx - r * NCH;
        if (m0 + r < M)
          st16(dst + (size_t)(m0 + r) * ldo + n0 + c * 8, lds_ld16(smem, r * (OUT_BN * 2) + ((c ^ (r & SWM)) << 4)));
      }
    };
    auto stage_out = [&](auto o_const, auto jc_const, const f32x16 (&facc)[FM][JC]) {
      for_groups(jc_const, facc, [&](int m, int n, int cl, const float* v, const float* vu) {
        const u32x2 w = out_vals(o_const, m, n, v, vu);
        *reinterpret_cast<u32x2*>(smem + st_off(m - m0, cl)) = w;
      });
    };
    if constexpr (JC == FN) {
      f32x16 facc[FM][JC];
      make_facc(std::integral_constant<int, 0>{}, facc);
      auto pass = [&](auto o_const) {
        constexpr int o = decltype(o_const)::value;
        if constexpr (o < NOUT) {
          if (o == 0 || out_ptr(o) != nullptr) {
            if constexpr (o > 0) __syncthreads();       // the previous output has left LDS
            stage_out(o_const, std::integral_constant<int, 0>{}, facc);
            __syncthreads();
            copy_out(o);
          }
        }
      };
      pass(std::integral_constant<int, 0>{});
      pass(std::integral_constant<int, 1>{});
      pass(std::integral_constant<int, 2>{});
    } else {
      // one output (int8 dequantisation): chunk by chunk into the staging tile
      auto chunk = [&](auto jc_const) {
        constexpr int jc = decltype(jc_const)::value;
        if constexpr (jc < FN) {
          f32x16 facc[FM][JC];
          make_facc(jc_const, facc);
          stage_out(std::integral_constant<int, 0>{}, jc_const, facc);
        }
      };
      chunk(std::integral_constant<int, 0>{});
      chunk(std::integral_constant<int, JC>{});
      chunk(std::integral_constant<int, 2 * JC>{});
      chunk(std::integral_constant<int, 3 * JC>{});
      static_assert(FN <= 4 * JC, "at most four column chunks");
      __syncthreads();
      copy_out(0);
    }
  } else if constexpr (EPI == EPI_RAW_I32) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int m = mrow_base + i * 32 + lr;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = ncol_base + j * 32 + 8 * g;
          const Acc& a = acc[i][j];
          *reinterpret_cast<i32x4*>(static_cast<int32_t*>(p.out) + (size_t)m * p.ldo + n) =
              i32x4{a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
        }
    }
  } else {
    // fused side path (plain output only): straight from registers
    static_assert(EPI == EPI_PLAIN, "fused side tiles have the plain epilogue");
    auto chunk = [&](auto jc_const) {
      constexpr int jc = decltype(jc_const)::value;
      if constexpr (jc < FN) {
        f32x16 facc[FM][JC];
        make_facc(jc_const, facc);
        for_groups(jc_const, facc, [&](int m, int n, int cl, const float* v, const float* vu) {
          if (m < M)
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.out) + (size_t)m * p.ldo + n) =
                out_vals(std::integral_constant<int, 0>{}, m, n, v, vu);
        });
      }
    };
    chunk(std::integral_constant<int, 0>{});
    chunk(std::integral_constant<int, JC>{});
    chunk(std::integral_constant<int, 2 * JC>{});
    chunk(std::integral_constant<int, 3 * JC>{});
  }
}

}  // namespace ldl
