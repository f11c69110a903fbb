// Four-wave NT tile for the 8-bit float (e4m3) base: Y = (Xq.Wq^T) . sx[m] . sw[n] +
// s.U.B^T (+ bias), on the block-scaled v_mfma_scale_f32_32x32x64_f8f6f4 with every block
// scale 1.0 (E8M0 127), which computes the plain e4m3 product at the full 8-bit rate ("nunchaku-style
// kernel fusion - 20-30% faster training", MXFP8 commit: the block-scaled instruction with
// unit scales as a drop-in for the plain 8-bit float product; LoRA-epilogue commit: the
// dequant scales plus the rank-tiled low-rank update as the epilogue).
//
// Data path as the bf16 four-wave tile (gemm16.hpp): two LDS stages of 128-byte rows (128
// codes per row and k-tile) filled by direct buffer->LDS copies with the same swizzle, a
// hand-scheduled loop of two steps per k-tile, one wave per SIMD and a 128 x BN/2 wave tile.
// With 32 x 32 blocks a step (64 k) needs 4 + BN/64 fragments of 32 bytes per lane, the
// register footprint the bf16 tile's 16 x 16 blocks need for 32 k; the 16 x 16 x 128 form
// would need twice that.  The e4m3 products accumulate into fp32 (the instruction's own
// internal sums keep about 17 bits relative to the largest term); after the loop the
// accumulators are dequantised and the low-rank term is added as one bf16 k-tile on
// v_mfma_f32_32x32x16_bf16, whose output layout is the same.
#pragma once

#include "gemm16.hpp"

namespace ldl {

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16 mfma_f8_32(const i32x8& a, const i32x8& b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
__device__ __forceinline__ f32x16 mfma_bf16_32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// 32 x 32 blocks: lane l of an operand holds row l & 31 and 32 bytes of the step's 64; the
// result lane l, value v holds D[8 (v >> 2) + 4 (l >> 5) + (v & 3)][l & 31] with D's rows
// from the first operand (here Q: output columns) and its columns from the second (P rows).
// SPLITK (256-wide tiles): the split reduction of the tiles past the last full round, as in
// the bf16 tile: block t S + q takes k-tiles [q KT / S, (q + 1) KT / S) of tile split_first + t
// and writes its dequantised fp32 partial (the low-rank term with q = 0 only) for the fixup
// pass; slot (((wave 4 + i) 4 + j) 4 + q') 64 + lane holds acc[i][j][4 q' .. 4 q' + 3].
template <int BN, bool SPLITK = false>
__global__ __launch_bounds__(256, 1) void gemm_f8_kernel(const GemmParams p) {
  static_assert(BN == 256 || BN == 128, "tile widths 256 and 128");
  static_assert(!SPLITK || BN == 256, "split reduction: 256-wide tiles");
  constexpr int BM = 256, NW = 4, FI = 4, FJ = BN / 64;
  constexpr int SB = BM * 128 + BN * 128;
  constexpr int NCB = BN / 32;                      // Q copies per wave and stage
  __shared__ __attribute__((aligned(16))) uint8_t smem0[SB];
  __shared__ __attribute__((aligned(16))) uint8_t smem1[SB];

  const int M = p.M, N = p.N;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = N / BN;
  int bid = blockIdx.x;
  [[maybe_unused]] int split = 0, kb = 0;
  int KTl = p.K / 128;
  if constexpr (SPLITK) {
    split = bid % p.split_s;
    bid = p.split_first + bid / p.split_s;
    kb = split * KTl / p.split_s;
    KTl = (split + 1) * KTl / p.split_s - kb;
  } else {
    const int nblk = gridDim.x;
    if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  }
  const int K = KTl * 128;                          // this block's reduction length
  constexpr int GM = 4;
  const int group = bid / (GM * tiles_n);
  const int first_m = group * GM;
  const int gm = min(GM, tiles_m - first_m);
  const int in_g = bid - group * GM * tiles_n;
  const int m0 = (first_m + in_g % gm) * BM, n0 = (in_g / gm) * BN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t lda_b = (uint32_t)p.lda, ldb_b = (uint32_t)p.ldb;
  const uint32_t koff = SPLITK ? (uint32_t)kb * 128u : 0u;   // (both operands from k-tile kb on)
  const __amdgpu_buffer_rsrc_t rs_a = make_rsrc(static_cast<const uint8_t*>(p.a) + koff, (uint32_t)M * lda_b - koff);
  const __amdgpu_buffer_rsrc_t rs_b = make_rsrc(static_cast<const uint8_t*>(p.b0) + koff, (uint32_t)N * ldb_b - koff);
  const __amdgpu_buffer_rsrc_t rs_none = make_rsrc(p.a, 0u);

  // copies: 1 KB (8 rows) per instruction; copy i of a wave covers rows 32 i + 8 wave ..
  const int lrow = lane >> 3, lphys = lane & 7;
  const int crow = wave * 8 + lrow;
  const uint32_t a_off = (uint32_t)(m0 + crow) * lda_b + ((lphys ^ swz(crow & 15)) << 4);
  const uint32_t b_off = (uint32_t)(n0 + crow) * ldb_b + ((lphys ^ swz(crow & 15)) << 4);
  const uint32_t a_step = 32u * lda_b, b_step = 32u * ldb_b;
  auto copy = [](__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint8_t* lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
  };
  auto copy_stage = [&](int kt, uint8_t* sb) {
    const bool valid = kt < K / 128;
    const __amdgpu_buffer_rsrc_t ra = valid ? rs_a : rs_none, rb = valid ? rs_b : rs_none;
    const uint32_t ko = (uint32_t)kt * 128u;
#pragma unroll
    for (int i = 0; i < 8; ++i) copy(ra, a_off, ko + i * a_step, sb + (i * NW + wave) * 1024);
#pragma unroll
    for (int i = 0; i < NCB; ++i) copy(rb, b_off, ko + i * b_step, sb + BM * 128 + (i * NW + wave) * 1024);
  };

  f32x16 acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // fragments of step ks: lane l reads logical chunks 4 ks + 2 (l >> 5) and the next of row
  // l & 31 of each 32-row block (rows 32 apart share the swizzle: constant 4 KB offsets)
  const int r32 = lane & 31, hh = lane >> 5;
  int a_base[2][2], b_base[2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      a_base[ks][c] = g16_off(wm * 128 + r32, 4 * ks + 2 * hh + c);
      b_base[ks][c] = BM * 128 + g16_off(wn * (BN / 2) + r32, 4 * ks + 2 * hh + c);
    }
  auto ldf = [&](const uint8_t* s, int ks, i32x8* fa, i32x8* fb) {
#pragma unroll
    for (int i = 0; i < FI; ++i) {
      const u32x4 lo = lds_ld16(s, a_base[ks][0] + i * 4096), hi = lds_ld16(s, a_base[ks][1] + i * 4096);
      fa[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
      const u32x4 lo = lds_ld16(s, b_base[ks][0] + j * 4096), hi = lds_ld16(s, b_base[ks][1] + j * 4096);
      fb[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
  };
  auto mm = [&](const i32x8* fa, const i32x8* fb) {
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        acc[i][j] = mfma_f8_32(fb[j], fa[i], acc[i][j]);
        asm volatile("" : "+a"(acc[i][j]));
      }
  };

  const int KT = K / 128;
  i32x8 fa0[FI], fb0[FJ], fa1[FI], fb1[FJ];
  copy_stage(0, smem0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  copy_stage(1, smem1);
  ldf(smem0, 0, fa0, fb0);
  __builtin_amdgcn_s_waitcnt(0xc07f);

  // a step: FI FJ MFMAs; the 2 (FI + FJ) fragment reads of the next step go two per MFMA
  // over its first MFMAs; in the hand-over step the stage copies (8 + NCB) go one per MFMA
  constexpr int NMF = FI * FJ, NRD = 2 * (FI + FJ), NG = NRD / 2, NCP = 8 + NCB;
  static_assert(NG <= NMF, "two reads per MFMA cover the next step's fragments");
  auto tile = [&](auto par_c, int kt) {
    constexpr int PAR = decltype(par_c)::value;
    uint8_t* cur = PAR ? smem1 : smem0;
    uint8_t* nxt = PAR ? smem0 : smem1;
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
      for (int j = 0; j < FJ; ++j) asm volatile("" : "+a"(acc[i][j]));
    __builtin_amdgcn_sched_barrier(0);
    ldf(cur, 1, fa1, fb1);
    mm(fa0, fb0);
    for (int q = 0; q < NG; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NMF - NG, 0);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    copy_stage(kt + 2, cur);
    ldf(nxt, 0, fa0, fb0);
    mm(fa1, fb1);
    for (int q = 0; q < NG; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    for (int q = 0; q < NCP - NG; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int kt = 0; kt < KT; kt += 2) {
    tile(std::integral_constant<int, 0>{}, kt);
    tile(std::integral_constant<int, 1>{}, kt + 1);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // ---- epilogue: dequantise in place (acc . sx[m] . sw[n])
#pragma unroll
  for (int i = 0; i < FI; ++i) {
    const float sxm = p.row_scale[min(m0 + wm * 128 + 32 * i + r32, M - 1)];
#pragma unroll
    for (int j = 0; j < FJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 swn = *reinterpret_cast<const f32x4*>(p.col_scale + n0 + wn * (BN / 2) + 32 * j + 8 * q + 4 * hh);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][4 * q + e] *= sxm * swn[e];
      }
  }
  // the low-rank term s.S.E^T as one bf16 k-tile in smem0 (P rows: s.S of row m0 + t as
  // bf16 hi + lo where 2 r <= 64, else hi; Q rows: E row n0 + t), four 16-k steps
  if (p.r_epi > 0 && split == 0) {
    const uint16_t* e0 = static_cast<const uint16_t*>(p.e0);
    const bool live = m0 + tid < M;
    const float* srow = p.S + (size_t)min(m0 + tid, M - 1) * p.ld_s;
    const int cps = p.r_epi >> 3;
    const int nparts = p.seed_hilo ? 2 : 1;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int part = c / cps, j0 = 8 * (c - part * cps);
      const bool on = part < nparts;
      const int jl = on ? j0 : 0;
      const f32x4 sa = *reinterpret_cast<const f32x4*>(srow + jl);
      const f32x4 sb = *reinterpret_cast<const f32x4*>(srow + jl + 4);
      const float sc = live ? p.s_epi : 0.f;
      u32x4 hv = u32x4{0u, 0u, 0u, 0u};
      if (on) {
        const float x[8] = {sa[0] * sc, sa[1] * sc, sa[2] * sc, sa[3] * sc, sb[0] * sc, sb[1] * sc, sb[2] * sc, sb[3] * sc};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          uint32_t h0 = f32_to_bf16_bits(x[2 * t]), h1 = f32_to_bf16_bits(x[2 * t + 1]);
          if (part == 1) {
            h0 = f32_to_bf16_bits(x[2 * t] - __uint_as_float(h0 << 16));
            h1 = f32_to_bf16_bits(x[2 * t + 1] - __uint_as_float(h1 << 16));
          }
          hv[t] = h0 | (h1 << 16);
        }
      }
      lds_st16(smem0, g16_off(tid, c), hv);
      if (tid < BN) {
        const u32x4 ev = *reinterpret_cast<const u32x4*>(e0 + (size_t)(n0 + tid) * p.e_ldn + jl);
        lds_st16(smem0, BM * 128 + g16_off(tid, c), on ? ev : u32x4{0u, 0u, 0u, 0u});
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 fa[FI], fb[FJ];
#pragma unroll
      for (int i = 0; i < FI; ++i) fa[i] = lds_ld16(smem0, g16_off(wm * 128 + 32 * i + r32, 2 * ks + hh));
#pragma unroll
      for (int j = 0; j < FJ; ++j) fb[j] = lds_ld16(smem0, BM * 128 + g16_off(wn * (BN / 2) + 32 * j + r32, 2 * ks + hh));
#pragma unroll
      for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j) acc[i][j] = mfma_bf16_32(fb[j], fa[i], acc[i][j]);
    }
    __syncthreads();
  }
  if constexpr (SPLITK) {
    float* dst = p.part + ((size_t)(bid - p.split_first) * p.split_s + split) * (size_t)(BM * BN);
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
      for (int j = 0; j < FJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f32x4 v = f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          asm volatile("" : "+v"(v));               // (out of the accumulators first)
          *reinterpret_cast<f32x4*>(dst + ((size_t)(((wave * FI + i) * FJ + j) * 4 + q) * 64 + lane) * 4) = v;
        }
    return;
  }
  // bias, bf16, staged through LDS (rows < 128 in smem0, the rest in smem1), written out as
  // whole 16-byte row segments
  constexpr int SROW = BN * 2, NCH = BN / 8, SWZM = NCH - 1;
  static_assert(128 * SROW <= SB, "half of the output tile fits in a stage buffer");
  auto st_ptr = [&](int r, int col) -> uint8_t* {
    uint8_t* base = r < 128 ? smem0 : smem1;
    const int rr = r & 127;
    return base + rr * SROW + ((((col >> 3) ^ (rr & SWZM))) << 4) + ((col & 4) << 1);
  };
  // (column groups outermost: the bias of the lane's four columns is read once per group)
#pragma unroll
  for (int j = 0; j < FJ; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int cl = wn * (BN / 2) + 32 * j + 8 * q + 4 * hh;
      u32x2 bb = u32x2{0u, 0u};
      if (p.bias != nullptr) bb = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p.bias) + n0 + cl);
#pragma unroll
      for (int i = 0; i < FI; ++i) {
        const int r = wm * 128 + 32 * i + r32;
        u32x2 w;
        w[0] = pack_bf16x2(acc[i][j][4 * q] + bf16_lo(bb[0]), acc[i][j][4 * q + 1] + bf16_hi(bb[0]));
        w[1] = pack_bf16x2(acc[i][j][4 * q + 2] + bf16_lo(bb[1]), acc[i][j][4 * q + 3] + bf16_hi(bb[1]));
        *reinterpret_cast<u32x2*>(st_ptr(r, cl)) = w;
      }
    }
  __syncthreads();
  // (eight LDS reads in flight before their stores)
  uint16_t* out = static_cast<uint16_t*>(p.out);
  constexpr int NIT = BM * NCH / 256;
  static_assert(NIT % 8 == 0, "row segments per thread in groups of eight");
#pragma unroll
  for (int b = 0; b < NIT; b += 8) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = tid + (b + u) * 256, r = idx / NCH, c = idx % NCH, rr = r & 127;
      v[u] = lds_ld16(r < 128 ? smem0 : smem1, rr * SROW + ((c ^ (rr & SWZM)) << 4));
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = tid + (b + u) * 256, r = idx / NCH, c = idx % NCH;
      if (m0 + r < M) st16(out + (size_t)(m0 + r) * p.ldo + n0 + c * 8, v[u]);
    }
  }
}

}  // namespace ldl
