// Tile table and launches of the MFMA GEMM families.
//
// The block tile is chosen from the output width (it must divide N) and the
// number of rows.  Tiles whose register footprint stays inside the 512
// registers a wave may hold at one wave per SIMD (no scratch spills, checked
// with -Rpass-analysis=kernel-resource-usage) are the only ones listed:
//   NT bf16         256x256, 256x192, 256x128, 128x128, 128x64
//   NT fused side   256x256, 256x128 (down-projection rows computed in the K-loop)
//   NT int8         256x256, 256x128, 128x128, 128x64
//   NN (bf16/int8 Q) 256x256, 256x192, 256x128, 128x128, 128x64
#include "internal.hpp"
#include "gemm16.hpp"
#include "gemm_f8.hpp"

namespace ldl {

// 256x256 tiles run 8 waves (2 x 4 wave grid, two waves per SIMD); the others 4.
template <int BM, int BN, bool I8, bool NN, bool BINT8, bool ASCALE, int RSP, bool SLOAD, int EPI>
static hipError_t run(const GemmParams& p, hipStream_t st) {
  constexpr int WN = (BM == 256 && BN == 256) ? 4 : 2;
  using C = GemmCfg<BM, BN, I8, NN, BINT8, ASCALE, RSP, SLOAD, EPI, WN>;
  const int out_bn = (EPI == EPI_SWIGLU_DUAL) ? BN / 2 : BN;
  const int tiles = ((p.M + BM - 1) / BM) * (p.N / out_bn);
  hipLaunchKernelGGL(gemm_kernel<C>, dim3(tiles), dim3(C::kThreads), 0, st, p);
  return hipGetLastError();
}

static int pick_bn(GemmKind kind, int N) {
  const bool wide_ok = (kind == GK_NT_PLAIN || kind == GK_NT_DORA || kind == GK_NN_PLAIN || kind == GK_NN_DORA ||
                        kind == GK_NN_SCALE || kind == GK_NN_I8_SCALE || kind == GK_NN_SWIGLU || kind == GK_NT_FUSED ||
                        kind == GK_NT_I8_DEQ || kind == GK_NT_I8_RAW);
  const bool b192_ok = (kind == GK_NT_PLAIN || kind == GK_NT_DORA || kind == GK_NN_PLAIN || kind == GK_NN_DORA ||
                        kind == GK_NN_SCALE ||
                        kind == GK_NN_I8_SCALE);
  if (wide_ok && N % 256 == 0) return 256;
  if (b192_ok && N % 192 == 0) return 192;
  if (N % 128 == 0) return 128;
  if (N % 64 == 0) return 64;
  return 0;
}

bool gemm_shape_ok(GemmKind kind, int M, int N, int K) {
  (void)M;
  if (kind == GK_NT_SWIGLU_DUAL) return N % 64 == 0 && K > 0 && K % 64 == 0;
  const bool i8 = (kind == GK_NT_I8_DEQ || kind == GK_NT_I8_RAW);
  if (pick_bn(kind, N) == 0) return false;
  if (kind == GK_NT_FUSED && N % 128 != 0) return false;
  if (K <= 0 || K % (i8 ? 128 : 64) != 0) return false;
  return true;
}

int g_gemm_4wave = 1;

static bool a16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; }

// Four-wave 256x256 tile: plain products, DoRA's row-scaled NT and the SwiGLU-backward NN
// epilogue, over a whole number of 256-column tiles with a low-rank term of rank <= 64
// (NN: Q in one segment).
// The low-rank term takes one k-tile of 64 rank slots; where 2 r fit in it, s.S enters as a
// bf16 pair hi + lo (its rounding error then ~2^-17 relative instead of ~2^-9) at no extra cost.
// Split reduction of the tiles past the last full round of the 256 CUs (plain 256-wide
// four-wave tiles, when the caller gave a partial buffer): the R remaining tiles are each
// computed by S = min(4, 256 / R) blocks over a quarter (third, half) of the k-tiles, so the
// last round is full, and the fixup pass sums the S fp32 partials in order (+ bias, bf16).
// (5120 x 5120 outputs at 4096 tokens: 320 tiles = one full round + 64 tiles.)
static void plan_split(GemmParams& p, int tiles, int kt) {
  p.split_s = 0;
  p.split_first = 0;
  if (p.part == nullptr) return;
  const int full = tiles / 256 * 256, R = tiles - full;
  if (R == 0) return;
  const int S = std::min(4, std::min(256 / R, kt));
  if (S < 2) return;
  p.split_s = S;
  p.split_first = full;
}

// blockIdx.x = 64 * t + c: remaining tile split_first + t, f32x4 slots 256 * c .. 256 * c + 255
// of the lane-linear partial layout of wave (wm, wn) = (wave >> 1, wave & 1).  16x16 blocks
// (L32 = 0): slot ((wave * 8 + i) * 8 + j) * 64 + lane holds row 16 * i + (lane & 15) and the
// four columns from 16 * j + 4 * (lane >> 4).  32x32 blocks (L32 = 1): slot
// (((wave * 4 + i) * 4 + j) * 4 + q) * 64 + lane holds row 32 * i + (lane & 31) and the four
// columns from 32 * j + 8 * q + 4 * (lane >> 5).
template <bool L32>
__global__ __launch_bounds__(256) void split_fixup_kernel(const GemmParams p) {
  const int t = blockIdx.x >> 6, slot = (blockIdx.x & 63) * 256 + threadIdx.x;
  const int tiles_m = (p.M + 255) / 256, tiles_n = p.N / 256;
  const int bid = p.split_first + t;
  constexpr int GM = 4;
  const int group = bid / (GM * tiles_n);
  const int first_m = group * GM;
  const int gm = min(GM, tiles_m - first_m);
  const int in_g = bid - group * GM * tiles_n;
  const int m0 = (first_m + in_g % gm) * 256, n0 = (in_g / gm) * 256;
  const int lane = slot & 63, wave = slot >> 12;
  int row = (wave >> 1) * 128, col = (wave & 1) * 128;
  if constexpr (L32) {
    const int q = (slot >> 6) & 3, j = (slot >> 8) & 3, i = (slot >> 10) & 3;
    row += 32 * i + (lane & 31);
    col += 32 * j + 8 * q + 4 * (lane >> 5);
  } else {
    const int j = (slot >> 6) & 7, i = (slot >> 9) & 7;
    row += 16 * i + (lane & 15);
    col += 16 * j + 4 * (lane >> 4);
  }
  if (m0 + row >= p.M) return;
  const float* src = p.part + (size_t)t * p.split_s * 65536 + (size_t)slot * 4;
  f32x4 v = *reinterpret_cast<const f32x4*>(src);
  for (int q = 1; q < p.split_s; ++q) v += *reinterpret_cast<const f32x4*>(src + (size_t)q * 65536);
  float b4[4] = {0.f, 0.f, 0.f, 0.f};
  if (p.bias != nullptr) {
    const u32x2 bb = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p.bias) + n0 + col);
    b4[0] = bf16_lo(bb[0]); b4[1] = bf16_hi(bb[0]); b4[2] = bf16_lo(bb[1]); b4[3] = bf16_hi(bb[1]);
  }
  u32x2 w;
  w[0] = pack_bf16x2(v[0] + b4[0], v[1] + b4[1]);
  w[1] = pack_bf16x2(v[2] + b4[2], v[3] + b4[3]);
  *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.out) + (size_t)(m0 + row) * p.ldo + n0 + col) = w;
}

static hipError_t launch_split_fixup(const GemmParams& p, int tiles, hipStream_t st, bool l32 = false) {
  const int R = tiles - p.split_first;
  if (l32) hipLaunchKernelGGL(split_fixup_kernel<true>, dim3(R * 64), dim3(256), 0, st, p);
  else hipLaunchKernelGGL(split_fixup_kernel<false>, dim3(R * 64), dim3(256), 0, st, p);
  return hipGetLastError();
}

size_t gemm_split_bytes(int M, int N) {
  if (M <= 128 || N % 256) return 0;
  const int tiles = ((M + 255) / 256) * (N / 256), R = tiles % 256;
  if (R == 0) return 0;
  const int S = std::min(4, 256 / R);
  return S < 2 ? 0 : (size_t)R * S * 65536 * sizeof(float);
}

template <bool NN, bool DORA = false, bool SWB = false, int BN = 256>
static hipError_t run16(const GemmParams& p0, hipStream_t st) {
  GemmParams p = p0;
  p.seed_hilo = (p.r_epi > 0 && 2 * p.r_epi <= 64) ? 1 : 0;
  p.split_s = 0;
  const int tiles = ((p.M + 255) / 256) * (p.N / BN);
  if constexpr (!NN && !DORA && !SWB) {
    if (p.nleaf > 0) {
      hipLaunchKernelGGL((gemm16_kernel<false, 1, false, false, BN, false, false, true>), dim3(tiles), dim3(256), 0, st,
                         p);
      return hipGetLastError();
    }
  }
  if constexpr (!DORA && !SWB && BN == 256) {
    plan_split(p, tiles, p.K / 64);
    if (p.split_s > 1) {            // the full rounds, then the split blocks, then the fixup
      const int nsplit = (tiles - p.split_first) * p.split_s;
      if (p.split_first > 0) {
        if (p.r_epi > 0) hipLaunchKernelGGL((gemm16_kernel<NN, 1, false, false, 256>), dim3(p.split_first), dim3(256), 0, st, p);
        else hipLaunchKernelGGL((gemm16_kernel<NN, 0, false, false, 256>), dim3(p.split_first), dim3(256), 0, st, p);
      }
      if (p.r_epi > 0)
        hipLaunchKernelGGL((gemm16_kernel<NN, 1, false, false, 256, false, false, false, ACT_SILU, true>), dim3(nsplit),
                           dim3(256), 0, st, p);
      else
        hipLaunchKernelGGL((gemm16_kernel<NN, 0, false, false, 256, false, false, false, ACT_SILU, true>), dim3(nsplit),
                           dim3(256), 0, st, p);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      return launch_split_fixup(p, tiles, st);
    }
  }
  if (p.r_epi > 0) hipLaunchKernelGGL((gemm16_kernel<NN, 1, DORA, SWB, BN>), dim3(tiles), dim3(256), 0, st, p);
  else hipLaunchKernelGGL((gemm16_kernel<NN, 0, DORA, SWB, BN>), dim3(tiles), dim3(256), 0, st, p);
  return hipGetLastError();
}

// SwiGLU gate and up in one four-wave tile per 128 hidden units: Q rows = 128 gate rows then
// the 128 up rows of the same units, e = X.Wg^T + s_g.U_g.Bg^T and u = X.Wu^T + s_u.U_u.Bu^T
// in the two column halves, h = silu(e) u formed from the fp32 accumulators in the
// epilogue (outputs e, u, h).  The two low-rank terms are two k-tiles in front of the loop.
// (Measured against two plain four-wave products plus a streaming pass forming h from the
// stored bf16 e and u, 8192 x 4096 x 14336 r = 64: the same step time, 5.41 ms, and h
// rounded once instead of after two other roundings.)
static bool dual16_ok(const GemmParams& p) {
  const int r = p.e_jsplit;
  return g_gemm_4wave && p.M > 128 && p.N % 128 == 0 && p.side == nullptr && p.r_epi == 2 * r &&
         r > 0 && r <= 64 && r % 8 == 0 && p.ld_s % 4 == 0 && a16(p.S) && a16(p.e0) && a16(p.e1) && p.e_ldj == 1 &&
         p.e_ldn % 8 == 0 && p.ldo % 8 == 0 && p.ldo2 % 8 == 0 && p.ldo3 % 8 == 0 && a16(p.out) && a16(p.out2) &&
         a16(p.out3);
}
// W8A8 forward on the four-wave tile: int8 16x16x64 MFMAs into exact int32 accumulators, then
// the dequantisation and the low-rank k-tile on fp32 accumulators after the loop.
// The input gradient over two stacked weights (the gated MLP's gate and up projections):
// the four-wave NN tile with Q rows k < kseg from b0 and the rest from b1, and the rank-(2 r)
// low-rank term as two seed k-tiles (S columns [0, r) against the rank rows of e0, [r, 2 r)
// against e1, bf16 hi).
static bool nn2_ok(const GemmParams& p) {
  const int rs = p.e_jsplit;
  return p.kseg > 0 && p.kseg < p.K && p.kseg % 64 == 0 && (p.K - p.kseg) % 64 == 0 && p.b1 != nullptr &&
         p.r_epi > 0 && p.r_epi == 2 * rs && rs % 8 == 0 && rs <= 64 && p.ld_s % 4 == 0 && a16(p.S) &&
         a16(p.e0) && a16(p.e1) && p.e_ldn == 1 && p.e_ldj % 8 == 0 && p.ldb % 8 == 0 && a16(p.b0) && a16(p.b1);
}

static hipError_t run16_nn2(const GemmParams& p0, hipStream_t st) {
  GemmParams p = p0;
  p.seed_hilo = 0;
  p.split_s = 0;
  const int tiles = ((p.M + 255) / 256) * (p.N / 256);
  hipLaunchKernelGGL((gemm16_kernel<true, 2, false, false, 256>), dim3(tiles), dim3(256), 0, st, p);
  return hipGetLastError();
}

static hipError_t run16_i8(const GemmParams& p0, hipStream_t st) {
  GemmParams p = p0;
  p.seed_hilo = (p.r_epi > 0 && 2 * p.r_epi <= 64) ? 1 : 0;
  const int tiles = ((p.M + 255) / 256) * (p.N / 256);
  plan_split(p, tiles, p.K / 128);
  if (p.split_s > 1) {              // the full rounds, then the split blocks, then the fixup
    if (p.split_first > 0)
      hipLaunchKernelGGL((gemm16_kernel<false, 0, false, false, 256, false, true>), dim3(p.split_first), dim3(256), 0,
                         st, p);
    hipLaunchKernelGGL((gemm16_kernel<false, 0, false, false, 256, false, true, false, ACT_SILU, true>),
                       dim3((tiles - p.split_first) * p.split_s), dim3(256), 0, st, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_split_fixup(p, tiles, st);
  }
  hipLaunchKernelGGL((gemm16_kernel<false, 0, false, false, 256, false, true>), dim3(tiles), dim3(256), 0, st, p);
  return hipGetLastError();
}

static hipError_t run16_dual(const GemmParams& p, hipStream_t st) {
  const int tiles = ((p.M + 255) / 256) * (p.N / 128);
  // the activation is a template argument: a runtime choice inside the epilogue cost ~20 % of
  // the tile's time (8192 x 4096 x 14336: 1878 us against ~1570 us)
  if (p.act == ACT_GELU)
    hipLaunchKernelGGL((gemm16_kernel<false, 2, false, false, 256, true, false, false, ACT_GELU>), dim3(tiles),
                       dim3(256), 0, st, p);
  else if (p.act == ACT_GELU_TANH)
    hipLaunchKernelGGL((gemm16_kernel<false, 2, false, false, 256, true, false, false, ACT_GELU_TANH>), dim3(tiles),
                       dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((gemm16_kernel<false, 2, false, false, 256, true, false, false, ACT_SILU>), dim3(tiles),
                       dim3(256), 0, st, p);
  return hipGetLastError();
}

// 192-column four-wave NT tiles when the 256-column tiles leave CUs idle in their only round
// and the 192-column ones still fit it (3072 columns at 4096 rows: 192 -> 256 tiles), or, over
// several rounds, when the 192-column rounds weighted by their width (3/4) are fewer
// (6144 columns at 4096 rows: two rounds of 256-column tiles, the second half empty, against
// two full rounds of 192-column ones)
static bool b192_fills(int M, int N) {
  if (N % 192) return false;
  const long t256 = (long)((M + 255) / 256) * (N / 256), t192 = (long)((M + 255) / 256) * (N / 192);
  if (t256 < 256 && t192 <= 256 && t192 > t256) return true;
  return N % 256 == 0 && t256 > 256 && 3 * ((t192 + 255) / 256) < 4 * ((t256 + 255) / 256);
}

// 256x128 tiles instead of 256x256 when twice as many tiles still fit one round over the
// 256 CUs (small M): the half-size tiles then keep twice the CUs busy.  With more tiles
// the four-wave 256x128 tile's lower rate per flop outweighs saved tail rounds (measured
// at 4096 and 8192 tokens, 5120 columns).
static bool half_tiles_pay(int M, int N) {
  const long t256 = (long)((M + 255) / 256) * (N / 256);
  return 2 * t256 <= 256;
}


// The four-wave tile's low-rank loads need 16-byte aligned S rows and E rows (NN: rank
// rows of E^T), a rank that is a multiple of 8, and one E segment.
static bool seed_ok(GemmKind kind, const GemmParams& p) {
  return p.r_epi == 0 ||
      (p.r_epi % 8 == 0 && p.ld_s % 4 == 0 && a16(p.S) && a16(p.e0) && p.e_jsplit >= p.r_epi &&
       ((kind == GK_NN_PLAIN || kind == GK_NN_SWIGLU || kind == GK_NN_DORA) ? (p.e_ldn == 1 && p.e_ldj % 8 == 0)
                                                      : (p.e_ldj == 1 && p.e_ldn % 8 == 0)));
}

// The down projection's input gradient as a plain four-wave NN product dh (bf16, written
// into out) followed by the SwiGLU backward in one streaming pass that turns dh into
// de = dh u sigma(e) (1 + e (1 - sigma(e))) in place and writes du = dh silu(e) to out2.
// The fused epilogue reads e and u and writes two outputs with every tile of a round at
// once, which keeps the tile's MFMAs about 40 % busy against about 62 % for the plain tile
// (8192 x 14336 x 4096 bf16); the pass costs the extra write and read of dh.  Taken when
// the plain product runs on the four-wave tile.
static bool swb_split(const GemmParams& p, GemmParams& h) {
  if (!g_gemm_4wave || p.M <= 128 || p.N % 256 != 0 || p.side != nullptr || p.r_epi > 64 || p.kseg != p.K)
    return false;
  if (p.ldo % 8 || p.ldo2 % 8 || p.ld_aux0 % 8 || p.ld_aux1 % 8) return false;
  if (!a16(p.out) || !a16(p.out2) || !a16(p.aux0) || !a16(p.aux1)) return false;
  h = p;
  h.aux0 = nullptr; h.aux1 = nullptr; h.out2 = nullptr;
  return seed_ok(GK_NN_PLAIN, h);
}

// Several adapters over one concatenated output: the leaf-aware low-rank seed exists on the
// four-wave NT tile only (the caller runs one product per leaf otherwise).
bool gemm_multi_leaf_ok(const GemmParams& p) {
  return g_gemm_4wave && p.M > 128 && p.side == nullptr && p.r_epi <= 64 && seed_ok(GK_NT_PLAIN, p) &&
         (p.N % 256 == 0 || b192_fills(p.M, p.N));
}

// e4m3 base: 256-column tiles, or 128-column ones where those fill the chip better or the
// width is not a multiple of 256 (a multiple of 128 is required), K a multiple of 128
static hipError_t run_f8(const GemmParams& p0, hipStream_t st) {
  GemmParams p = p0;
  if (p.N % 128 || p.K % 128 || p.r_epi > 64 || !seed_ok(GK_NT_PLAIN, p) || !a16(p.col_scale))
    return hipErrorInvalidValue;
  p.seed_hilo = (p.r_epi > 0 && 2 * p.r_epi <= 64) ? 1 : 0;
  const int tm = (p.M + 255) / 256;
  p.split_s = 0;
  if (p.N % 256 == 0 && p.part != nullptr) {
    const int tiles = tm * (p.N / 256);
    plan_split(p, tiles, p.K / 128);
    if (p.split_s > 1) {            // the full rounds, then the split blocks, then the fixup
      if (p.split_first > 0) hipLaunchKernelGGL(gemm_f8_kernel<256>, dim3(p.split_first), dim3(256), 0, st, p);
      hipLaunchKernelGGL((gemm_f8_kernel<256, true>), dim3((tiles - p.split_first) * p.split_s), dim3(256), 0, st, p);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      return launch_split_fixup(p, tiles, st, true);
    }
  }
  if (p.N % 256 == 0 && !half_tiles_pay(p.M, p.N))
    hipLaunchKernelGGL(gemm_f8_kernel<256>, dim3(tm * (p.N / 256)), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL(gemm_f8_kernel<128>, dim3(tm * (p.N / 128)), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_gemm(GemmKind kind, const GemmParams& p, hipStream_t st) {
  if (p.M <= 0) return hipSuccess;
  if (kind == GK_NT_F8_DEQ) return run_f8(p, st);
  if (p.nleaf > 0 && (kind != GK_NT_PLAIN || !gemm_multi_leaf_ok(p))) return hipErrorInvalidValue;
  const int bn = pick_bn(kind, p.N);
  const bool big = p.M > 128;
  if (kind == GK_NT_SWIGLU_DUAL && dual16_ok(p)) return run16_dual(p, st);
  if (kind == GK_NN_SWIGLU) {
    GemmParams h;
    if (swb_split(p, h)) {
      hipError_t e = launch_gemm(GK_NN_PLAIN, h, st);
      bool rec = false;
      if (e == hipSuccess) e = hook_start(2, st, &rec);
      if (e == hipSuccess)
        e = launch_swiglu_bwd(p.out, p.ldo, p.aux0, p.ld_aux0, p.aux1, p.ld_aux1, p.out2, p.ldo2, p.M, p.N, p.act, st);
      if (e == hipSuccess) e = hook_stop(2, st, rec);
      return e;
    }
  }
  const bool seed = seed_ok(kind, p);
  // (measured at 5120 x 5120, r = 32: 2048 tokens 88 -> 72 us, 4096 182 -> 145, 8192 303 -> 245,
  // 16384 523 -> 415 us against the eight-wave tile; at 1024 tokens the eight-wave 256 x 128
  // tiles, twice as many in the one round, stay faster: 67 against 71 us)
  if (kind == GK_NT_I8_DEQ && g_gemm_4wave && big && bn == 256 &&
      (g_gemm_4wave == 2 || p.part != nullptr || !half_tiles_pay(p.M, p.N)) &&
      p.side == nullptr &&
      p.r_epi <= 64 && seed && p.K % 128 == 0 && a16(p.col_scale))
    return run16_i8(p, st);
  if (g_gemm_4wave && big && p.side == nullptr && p.r_epi <= 64 && seed &&
      (kind == GK_NT_PLAIN || kind == GK_NT_DORA) && b192_fills(p.M, p.N)) {
    if (kind == GK_NT_PLAIN) return run16<false, false, false, 192>(p, st);
    return run16<false, true, false, 192>(p, st);
  }
  if (kind == GK_NN_PLAIN && g_gemm_4wave && bn == 256 && big && p.side == nullptr && nn2_ok(p))
    return run16_nn2(p, st);
  if (g_gemm_4wave && bn == 256 && big && p.side == nullptr && p.r_epi <= 64 && seed) {
    if (kind == GK_NT_PLAIN) return run16<false>(p, st);
    if (kind == GK_NT_DORA) return run16<false, true>(p, st);
    if (kind == GK_NN_PLAIN && p.kseg == p.K) return run16<true>(p, st);
    if (kind == GK_NN_DORA && p.kseg == p.K) return run16<true, true>(p, st);
    if (kind == GK_NN_SWIGLU && p.kseg == p.K) return run16<true, false, true>(p, st);
  }
  switch (kind) {
    case GK_NT_PLAIN:
      if (bn == 256) return big ? run<256, 256, false, false, false, false, 0, true, EPI_PLAIN>(p, st)
                                : run<128, 128, false, false, false, false, 0, true, EPI_PLAIN>(p, st);
      if (bn == 192) return big ? run<256, 192, false, false, false, false, 0, true, EPI_PLAIN>(p, st)
                                : run<128, 64, false, false, false, false, 0, true, EPI_PLAIN>(p, st);
      if (bn == 128) return big ? run<256, 128, false, false, false, false, 0, true, EPI_PLAIN>(p, st)
                                : run<128, 128, false, false, false, false, 0, true, EPI_PLAIN>(p, st);
      return run<128, 64, false, false, false, false, 0, true, EPI_PLAIN>(p, st);
    case GK_NT_DORA:
      if (bn == 256) return big ? run<256, 256, false, false, false, false, 0, true, EPI_DORA>(p, st)
                                : run<128, 128, false, false, false, false, 0, true, EPI_DORA>(p, st);
      if (bn == 192) return big ? run<256, 192, false, false, false, false, 0, true, EPI_DORA>(p, st)
                                : run<128, 64, false, false, false, false, 0, true, EPI_DORA>(p, st);
      if (bn == 128) return big ? run<256, 128, false, false, false, false, 0, true, EPI_DORA>(p, st)
                                : run<128, 128, false, false, false, false, 0, true, EPI_DORA>(p, st);
      return run<128, 64, false, false, false, false, 0, true, EPI_DORA>(p, st);
    case GK_NT_SWIGLU_DUAL:
      // output width per tile is BN / 2 (hidden units); the tile reads BN/2 gate + BN/2 up rows
      if (p.N % 128 == 0 && big) return run<256, 256, false, false, false, false, 0, true, EPI_SWIGLU_DUAL>(p, st);
      if (p.N % 128 == 0) return run<128, 256, false, false, false, false, 0, true, EPI_SWIGLU_DUAL>(p, st);
      return run<256, 128, false, false, false, false, 0, true, EPI_SWIGLU_DUAL>(p, st);
    case GK_NT_FUSED:
      // down-projection computed in the K-loop; side rows padded to 32 or 64
      if (bn == 256 && big) {
        if (p.r_side <= 32) return run<256, 256, false, false, false, false, 32, false, EPI_PLAIN>(p, st);
        return run<256, 256, false, false, false, false, 64, false, EPI_PLAIN>(p, st);
      }
      if (p.r_side <= 32) return run<256, 128, false, false, false, false, 32, false, EPI_PLAIN>(p, st);
      return run<256, 128, false, false, false, false, 64, false, EPI_PLAIN>(p, st);
    case GK_NT_I8_DEQ:
      if (bn == 256 && big && !half_tiles_pay(p.M, p.N)) return run<256, 256, true, false, false, false, 0, true, EPI_DEQUANT>(p, st);
      if (bn >= 128) return big ? run<256, 128, true, false, false, false, 0, true, EPI_DEQUANT>(p, st)
                                : run<128, 128, true, false, false, false, 0, true, EPI_DEQUANT>(p, st);
      return run<128, 64, true, false, false, false, 0, true, EPI_DEQUANT>(p, st);
    case GK_NT_I8_RAW:
      if (bn == 256 && big) return run<256, 256, true, false, false, false, 0, false, EPI_RAW_I32>(p, st);
      if (bn >= 128) return big ? run<256, 128, true, false, false, false, 0, false, EPI_RAW_I32>(p, st)
                                : run<128, 128, true, false, false, false, 0, false, EPI_RAW_I32>(p, st);
      return run<128, 64, true, false, false, false, 0, false, EPI_RAW_I32>(p, st);
    case GK_NN_PLAIN:
      if (bn == 256 && big) return run<256, 256, false, true, false, false, 0, true, EPI_PLAIN>(p, st);
      if (bn == 192) return big ? run<256, 192, false, true, false, false, 0, true, EPI_PLAIN>(p, st)
                                : run<128, 64, false, true, false, false, 0, true, EPI_PLAIN>(p, st);
      if (bn >= 128) return big ? run<256, 128, false, true, false, false, 0, true, EPI_PLAIN>(p, st)
                                : run<128, 128, false, true, false, false, 0, true, EPI_PLAIN>(p, st);
      return run<128, 64, false, true, false, false, 0, true, EPI_PLAIN>(p, st);
    case GK_NN_DORA:
      if (bn == 256 && big) return run<256, 256, false, true, false, false, 0, true, EPI_DORA>(p, st);
      if (bn == 192) return big ? run<256, 192, false, true, false, false, 0, true, EPI_DORA>(p, st)
                                : run<128, 64, false, true, false, false, 0, true, EPI_DORA>(p, st);
      if (bn >= 128) return big ? run<256, 128, false, true, false, false, 0, true, EPI_DORA>(p, st)
                                : run<128, 128, false, true, false, false, 0, true, EPI_DORA>(p, st);
      return run<128, 64, false, true, false, false, 0, true, EPI_DORA>(p, st);
    case GK_NN_SCALE:
      if (bn == 256 && big) return run<256, 256, false, true, false, true, 0, true, EPI_PLAIN>(p, st);
      if (bn == 192) return big ? run<256, 192, false, true, false, true, 0, true, EPI_PLAIN>(p, st)
                                : run<128, 64, false, true, false, true, 0, true, EPI_PLAIN>(p, st);
      if (bn >= 128) return big ? run<256, 128, false, true, false, true, 0, true, EPI_PLAIN>(p, st)
                                : run<128, 128, false, true, false, true, 0, true, EPI_PLAIN>(p, st);
      return run<128, 64, false, true, false, true, 0, true, EPI_PLAIN>(p, st);
    case GK_NN_I8_SCALE:
      if (bn == 256 && big && !half_tiles_pay(p.M, p.N)) return run<256, 256, false, true, true, true, 0, true, EPI_PLAIN>(p, st);
      if (bn == 192) return big ? run<256, 192, false, true, true, true, 0, true, EPI_PLAIN>(p, st)
                                : run<128, 64, false, true, true, true, 0, true, EPI_PLAIN>(p, st);
      if (bn >= 128) return big ? run<256, 128, false, true, true, true, 0, true, EPI_PLAIN>(p, st)
                                : run<128, 128, false, true, true, true, 0, true, EPI_PLAIN>(p, st);
      return run<128, 64, false, true, true, true, 0, true, EPI_PLAIN>(p, st);
    case GK_NN_SWIGLU:
      if (bn == 256 && big) return run<256, 256, false, true, false, false, 0, true, EPI_SWIGLU_BWD>(p, st);
      if (bn >= 128) return big ? run<256, 128, false, true, false, false, 0, true, EPI_SWIGLU_BWD>(p, st)
                                : run<128, 128, false, true, false, false, 0, true, EPI_SWIGLU_BWD>(p, st);
      return run<128, 64, false, true, false, false, 0, true, EPI_SWIGLU_BWD>(p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace ldl
