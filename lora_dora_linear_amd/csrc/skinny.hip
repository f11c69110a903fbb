// Rank-r ("skinny") contractions on MFMA, and the fixed-order reductions of
// their split partial sums.
//
//   rowproj : out[m, j] = scale * sum_k P[m, k] * Q[j, k]       (U = X.A^T, V = dY.B,
//             P = W0.A^T, G = A.A^T); P, Q bf16 with k contiguous, both read
//             straight from global memory into MFMA fragments.  Q may instead be
//             a [K, R] matrix read in place (lora_up B), optionally with a
//             per-k factor applied and rounded to bf16 (DoRA's diag(g).B).
//   colproj : part[split][c, j] = sum_{m in split} X[m, c] * S[m, j]   (dB = dY^T.U,
//             dA^T = X^T.V and the DoRA norm terms); X bf16 is staged through
//             LDS with an 8x8 register transpose so that each lane holds eight
//             consecutive m; S fp32 is split into bf16 hi + lo parts, so the
//             product keeps ~16 bits of S.  Optionally also the column sums
//             sum_m X[m, c] * Z[m, c] (DoRA dg) or sum_m X[m, c] (bias gradient).
//
// These are the "skinny MFMA contractions" for the factor gradients: each is
// one pass over the [M, *] operand and bound by HBM bandwidth.  Up to three
// independent column projections, and two reductions, share one launch.
#include "internal.hpp"

namespace ldl {

// ============================================================================ rowproj
// 16 output rows per 512-thread block; the eight waves split the reduction
// (wave w takes the 32-element steps w, w+8, ...), each keeping up to eight
// 1 KiB row fragments of P in flight, then reduce through LDS.
constexpr int RP_WAVES = 8;

template <int RP>
__global__ __launch_bounds__(512) void rowproj_kernel(const RowProjParams p) {
  constexpr int NB = RP / 16;
  __shared__ f32x4 red[RP_WAVES][NB][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int m0 = blockIdx.x * 16;
  const int m = m0 + lr;
  const bool mval = m < p.M;
  const uint16_t* prow = (p.P1 != nullptr && m >= p.p_split ? p.P1 + (size_t)(m - p.p_split) * p.ldp1
                                                             : p.P + (size_t)(mval ? m : 0) * p.ldp) + lq * 8;

  const uint16_t* qrow[NB];
  bool qval[NB];
#pragma unroll
  for (int jb = 0; jb < NB; ++jb) {
    const int j = jb * 16 + lr;
    qval[jb] = j < p.R;
    if (p.q_trans) {
      qrow[jb] = p.q0 + (qval[jb] ? j : 0) + (size_t)(lq * 8) * p.ldq;
    } else {
      const uint16_t* base = (j < p.R0) ? (p.q0 + (size_t)j * p.ldq) : (p.q1 + (size_t)(j - p.R0) * p.ldq);
      qrow[jb] = (qval[jb] ? base : p.q0) + lq * 8;
    }
  }
  // Q fragment of step k: 8 consecutive reduction indices k*32 + 8*lq + e of row j
  auto qload = [&](int jb, int k) -> u32x4 {
    if (!qval[jb]) return u32x4{0, 0, 0, 0};
    if (!p.q_trans) return ld16(qrow[jb] + k * 32);
    const uint16_t* q = qrow[jb] + (size_t)(k * 32) * p.ldq;
    u32x4 v;
    if (p.q_kscale == nullptr) {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (uint32_t)q[(size_t)(2 * e) * p.ldq] | ((uint32_t)q[(size_t)(2 * e + 1) * p.ldq] << 16);
    } else {
      const float* sc = p.q_kscale + k * 32 + lq * 8;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[e] = pack_bf16x2(bf16_to_f32(q[(size_t)(2 * e) * p.ldq]) * sc[2 * e],
                           bf16_to_f32(q[(size_t)(2 * e + 1) * p.ldq]) * sc[2 * e + 1]);
    }
    return v;
  };

  f32x4 acc[NB];
#pragma unroll
  for (int jb = 0; jb < NB; ++jb) acc[jb] = f32x4{0, 0, 0, 0};

  const int nsteps = p.K / 32;
  const u32x4 zero = {0, 0, 0, 0};
  // every load of a group (P from HBM, Q from L2) is issued before its MFMAs;
  // each block starts at a different point of the reduction so that the blocks
  // do not all request the same lines of the small Q at the same time
  constexpr int U = NB <= 2 ? 8 : (NB == 4 ? 4 : 2);
  const int groups = nsteps / RP_WAVES;                      // full rounds of 8 steps
  const int rot = groups > 0 ? (int)(blockIdx.x % (unsigned)groups) * RP_WAVES : 0;
  auto step_of = [&](int t) { int k = t + rot; return k >= groups * RP_WAVES ? k - groups * RP_WAVES : k; };
  int ks = wave;
  const int full = groups * RP_WAVES;                        // steps covered by the rotation
  for (; ks + (U - 1) * RP_WAVES < full; ks += U * RP_WAVES) {
    u32x4 pf[U], qf[U][NB];
#pragma unroll
    for (int u = 0; u < U; ++u) pf[u] = mval ? ld16(prow + step_of(ks + u * RP_WAVES) * 32) : zero;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int jb = 0; jb < NB; ++jb)
        qf[u][jb] = qload(jb, step_of(ks + u * RP_WAVES));
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int jb = 0; jb < NB; ++jb) acc[jb] = mfma_bf16(qf[u][jb], pf[u], acc[jb]);
  }
  for (; ks < nsteps; ks += RP_WAVES) {
    const int k = ks < full ? step_of(ks) : ks;
    const u32x4 pf = mval ? ld16(prow + k * 32) : zero;
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) {
      acc[jb] = mfma_bf16(qload(jb, k), pf, acc[jb]);
    }
  }

#pragma unroll
  for (int jb = 0; jb < NB; ++jb) red[wave][jb][lane] = acc[jb];
  __syncthreads();
  // lane holds out[m][jb*16 + 4*lq + i]; waves 0..NB-1 finish one jb each
  for (int jb = wave; jb < NB; jb += RP_WAVES) {
    f32x4 v = red[0][jb][lane];
#pragma unroll
    for (int w = 1; w < RP_WAVES; ++w) v += red[w][jb][lane];
    if (mval) {
      const int j0 = jb * 16 + 4 * lq;
      float* dst = p.out + (size_t)m * p.ldo;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (j0 + i < p.R) dst[j0 + i] = v[i] * p.scale;
    }
  }
}

// ============================================================================ rowproj (streamed)
// Block = 16 rows of P, 4 waves.  The reduction is walked in chunks of KC
// elements; each chunk's P rows, Q slice and k-scale slice are copied to LDS
// by direct buffer->LDS copies (every instruction moves 1 KB of whole cache
// lines) through a ring of STAGES buffers, so STAGES-1 chunks are in flight
// while one is consumed.  The waves split each chunk's 32-element steps and
// combine their partial sums at the end.  P and a row-major Q are stored with
// 16-byte chunk c of row r at physical chunk c ^ (r & 15); a transposed Q
// (a [K, R] matrix, rows of R bf16) is stored as-is and read back with the
// transposing LDS read.
//
// BMR = 32 (rank 64 and 128): a block takes 32 rows, two 16-row MFMA tiles that share each Q
// fragment, so the [K, RP] (or [RP, K]) rank factor is staged once per 32 rows instead of
// per 16; every output row sees the same k-steps on the same wave in the same order as
// with 16-row blocks (identical results).
template <int RP, bool KS, int BMR = 16>
struct RowStream {
  static constexpr int KC = RP <= 32 ? 512 : (RP == 64 ? 256 : 128);   // elements per chunk
  static constexpr int RL = KC * 2;                  // bytes per staged row
  static constexpr int PB = BMR * RL;                // P slice
  static constexpr int QB = RP * RL;                 // Q slice (RP rows of KC, or KC rows of R <= RP)
  static constexpr int GB = KS ? 4096 : 0;           // k-scale slice: KC floats, four 1 KB copies
  static constexpr int SB = PB + QB + GB;
  // as many ring stages as the LDS holds (at most 5): STAGES-1 chunks stay in flight
  static constexpr int STAGES = (160 * 1024) / SB > 5 ? 5 : (160 * 1024) / SB;
  static constexpr int NI = (PB + QB) / 1024 / 4 + (KS ? 1 : 0);  // copy instructions per wave per chunk
  static_assert(STAGES >= 3 && STAGES * SB <= 160 * 1024, "LDS ring fits");
  static_assert((PB + QB) % 4096 == 0, "copies split evenly over the four waves");
  static_assert((STAGES - 2) * NI < 64, "outstanding copies fit the vmcnt counter");
};

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int RP, bool KS, int BMR = 16>
__global__ __launch_bounds__(256) void rowstream_kernel(const RowProjParams p) {
  using T = RowStream<RP, KS, BMR>;
  constexpr int NB = RP / 16, KC = T::KC, RL = T::RL, SB = T::SB, ST = T::STAGES;
  constexpr int NH = BMR / 16;                       // 16-row MFMA tiles per block
  __shared__ __attribute__((aligned(16))) uint8_t smem[ST * SB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lq = lane >> 4;
  const int m0 = blockIdx.x * BMR;
  const int nch = (p.K + KC - 1) / KC;
  const bool tq = p.q_trans != 0;

  // a block's BMR rows lie in one P segment (the splits are multiples of BMR)
  const bool seg2 = p.P2 != nullptr && m0 >= p.p_split2;
  const int end1 = p.P2 != nullptr ? p.p_split2 : p.M;          // end of the first two segments
  const bool seg1 = !seg2 && p.P1 != nullptr && m0 >= p.p_split;
  const uint32_t ldp_b = (uint32_t)(seg2 ? p.ldp2 : seg1 ? p.ldp1 : p.ldp) * 2u, ldq_b = (uint32_t)p.ldq * 2u;
  const int pm0 = seg2 ? m0 - p.p_split2 : seg1 ? m0 - p.p_split : m0;
  const __amdgpu_buffer_rsrc_t rs_p =
      seg2 ? make_rsrc(p.P2, (uint32_t)(p.M - p.p_split2) * ldp_b)
           : seg1 ? make_rsrc(p.P1, (uint32_t)(end1 - p.p_split) * ldp_b)
                  : make_rsrc(p.P, (uint32_t)(p.P1 != nullptr ? p.p_split : end1) * ldp_b);
  const __amdgpu_buffer_rsrc_t rs_q0 =
      make_rsrc(p.q0, tq ? (uint32_t)p.K * (uint32_t)p.R * 2u : (uint32_t)p.R0 * ldq_b);
  const __amdgpu_buffer_rsrc_t rs_q1 = make_rsrc(p.q1, tq ? 0u : (uint32_t)(p.R - p.R0) * ldq_b);
  const __amdgpu_buffer_rsrc_t rs_g = make_rsrc(p.q_kscale, p.q_kscale ? (uint32_t)p.K * 4u : 0u);

  // per-lane source offsets of this wave's copy instructions (chunk independent)
  constexpr int NIP = T::PB / 4096, NIQ = T::QB / 4096;
  uint32_t p_off[NIP], q_off[NIQ];
  bool q_up[NIQ];
#pragma unroll
  for (int i = 0; i < NIP; ++i) {
    const int b = (i * 4 + wave) * 1024 + lane * 16;
    const int row = b / RL, phys = (b % RL) >> 4;
    p_off[i] = (uint32_t)(pm0 + row) * ldp_b + (uint32_t)((phys ^ (row & 15)) << 4);
  }
#pragma unroll
  for (int i = 0; i < NIQ; ++i) {
    const int b = (i * 4 + wave) * 1024 + lane * 16;
    if (tq) {
      q_off[i] = (uint32_t)b;
      q_up[i] = false;
    } else {
      const int row = b / RL, phys = (b % RL) >> 4;
      const int rowb = (i * 4 + wave) * 1024 / RL;             // first row of the instruction
      q_up[i] = rowb >= p.R0;                                    // whole instruction in one segment
      q_off[i] = (uint32_t)(q_up[i] ? row - p.R0 : row) * ldq_b + (uint32_t)((phys ^ (row & 15)) << 4);
    }
  }
  auto issue = [&](int ch) {
    uint8_t* sb = smem + (ch % ST) * SB;
#pragma unroll
    for (int i = 0; i < NIP; ++i) buf2lds16(rs_p, p_off[i], (uint32_t)ch * RL, sb + (i * 4 + wave) * 1024);
    const uint32_t qs = tq ? (uint32_t)ch * (uint32_t)KC * (uint32_t)p.R * 2u : (uint32_t)ch * RL;
#pragma unroll
    for (int i = 0; i < NIQ; ++i) buf2lds16(q_up[i] ? rs_q1 : rs_q0, q_off[i], qs, sb + T::PB + (i * 4 + wave) * 1024);
    if constexpr (KS) buf2lds16(rs_g, (uint32_t)(wave * 1024 + lane * 16), (uint32_t)ch * KC * 4u, sb + T::PB + T::QB + wave * 1024);
  };

  f32x4 acc[NH][NB];
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) acc[h][jb] = f32x4{0, 0, 0, 0};

#pragma unroll
  for (int c = 0; c < ST - 1; ++c)
    if (c < nch) issue(c);
  for (int ch = 0; ch < nch; ++ch) {
    // chunks issued after ch that may stay in flight
    const int after = min(ST - 2, nch - 1 - ch);
    if (after >= 3) wait_vmcnt<(ST > 4 ? 3 : 0) * T::NI>();
    else if (after == 2) wait_vmcnt<2 * T::NI>();
    else if (after == 1) wait_vmcnt<T::NI>();
    else wait_vmcnt<0>();
    __syncthreads();                         // chunk ch visible; chunk ch-1's buffer free
    if (ch + ST - 1 < nch) issue(ch + ST - 1);
    const uint8_t* sb = smem + (ch % ST) * SB;
    const uint8_t* sq = sb + T::PB;
    const float* sg = reinterpret_cast<const float*>(sb + T::PB + T::QB);
    const int nv = min(KC, p.K - ch * KC) / 32;
    for (int st = wave; st < nv; st += 4) {
      const int lc = st * 4 + lq;
      u32x4 pf[NH];
#pragma unroll
      for (int h = 0; h < NH; ++h) pf[h] = *reinterpret_cast<const u32x4*>(sb + (h * 16 + lr) * RL + ((lc ^ lr) << 4));
#pragma unroll
      for (int jb = 0; jb < NB; ++jb) {
        u32x4 qf;
        if (tq) {
          // 8 consecutive k of column jb*16 + lr: two transposing reads of 4 rows each
          const int k0 = st * 32 + 8 * lq + (lr >> 2);
          const int off = k0 * p.R * 2 + (jb * 16 + 4 * (lr & 3)) * 2;
          const u32x2 lo = lds_tr16(sq, off), hi = lds_tr16(sq, off + 4 * p.R * 2);
          qf = u32x4{lo[0], lo[1], hi[0], hi[1]};
          if constexpr (KS) {
            const f32x4* g = reinterpret_cast<const f32x4*>(sg + st * 32 + 8 * lq);
            qf = scale_bf16x8(qf, g[0], g[1]);
          }
        } else {
          const int j = jb * 16 + lr;
          qf = *reinterpret_cast<const u32x4*>(sq + j * RL + ((lc ^ lr) << 4));
        }
#pragma unroll
        for (int h = 0; h < NH; ++h) acc[h][jb] = mfma_bf16(qf, pf[h], acc[h][jb]);
      }
    }
  }

  // combine the four waves' partial sums; lane holds out[m0 + 16h + lr][jb*16 + 4*lq + i]
  __syncthreads();
  f32x4* red = reinterpret_cast<f32x4*>(smem);      // [4][NH][NB][64]
  static_assert(4 * NH * NB * 64 * 16 <= ST * SB, "reduction scratch fits");
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) red[((wave * NH + h) * NB + jb) * 64 + lane] = acc[h][jb];
  __syncthreads();
  for (int it = wave; it < NH * NB; it += 4) {
    const int h = it / NB, jb = it % NB;
    const int m = m0 + h * 16 + lr;
    f32x4 v = red[(h * NB + jb) * 64 + lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) v += red[((w * NH + h) * NB + jb) * 64 + lane];
    if (m < (seg2 ? p.M : end1)) {
      const int j0 = jb * 16 + 4 * lq;
      float* dst = seg2 ? p.out2 + (size_t)(m - p.p_split2) * p.ldo2 : p.out + (size_t)m * p.ldo;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (j0 + i < p.R) dst[j0 + i] = v[i] * p.scale;
    }
    if (p.pk != nullptr && m < ((p.M + 7) & ~7)) {
      // the packed copy: pk_scale * out as bf16 hi and lo (zero past R and past M), 16 bits
      // per value: row m is half (m & 1) of word 4 j + ((m & 7) >> 1) of its 8-row group
      // (hi) and of word 4 (pk_rp + j) + ((m & 7) >> 1) (lo)
      uint16_t* g = p.pk + (size_t)(m >> 3) * (16 * p.pk_rp) + (m & 1);
      const int e = (m & 7) >> 1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = jb * 16 + 4 * lq + i;
        if (j >= p.pk_rp) continue;
        const float x = (m < p.M && j < p.R) ? (v[i] * p.scale) * p.pk_scale : 0.f;
        const uint32_t hi = f32_to_bf16_bits(x);
        g[2 * (4 * j + e)] = (uint16_t)hi;
        g[2 * (4 * (p.pk_rp + j) + e)] = (uint16_t)f32_to_bf16_bits(x - __uint_as_float(hi << 16));
      }
    }
  }
}

// ============================================================================ colproj
// Block = 64 columns of X and one split of rows, walked in sub-tiles of MS rows.
// Per sub-tile: X^T (64 x MS bf16) and S^T as bf16 hi/lo parts (R x MS each) are
// staged in LDS; each of the four waves owns 16 columns.
__device__ __forceinline__ int xt_off(int c, int chunk, int rowbytes) {
  return c * rowbytes + ((chunk ^ swz(c)) << 4);
}

template <int RP>
struct ColProjTile {
  static constexpr int MS = RP <= 64 ? 256 : 128;        // rows per sub-tile
  static constexpr int XBYTES = 64 * MS * 2;
  static constexpr int SBYTES = RP * MS * 2;             // one of hi / lo
};

struct ColProjBatch {
  ColProjParams job[kColProjBatch];
  int first[kColProjBatch + 1];   // grid.y rows [first[i], first[i+1]) are the splits of job i
};

template <int RP>
__global__ __launch_bounds__(256) void colproj_kernel(const ColProjBatch batch) {
  const int y = blockIdx.y;
  const int jobi = y >= batch.first[2] ? 2 : (y >= batch.first[1] ? 1 : 0);
  const ColProjParams& p = batch.job[jobi];
  const int split = y - batch.first[jobi];
  if ((int)blockIdx.x * 64 >= p.C) return;
  using T = ColProjTile<RP>;
  constexpr int NB = RP / 16;
  constexpr int MS = T::MS;
  constexpr int ROWB = MS * 2;          // bytes per transposed row
  __shared__ __attribute__((aligned(16))) uint8_t xt[T::XBYTES];
  __shared__ __attribute__((aligned(16))) uint16_t shi[RP * MS];
  __shared__ __attribute__((aligned(16))) uint16_t slo[RP * MS];
  static_assert(T::XBYTES >= 32 * 65 * 4, "column-sum scratch reuses the X tile");
  float (*csred)[65] = reinterpret_cast<float (*)[65]>(xt);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int c0 = blockIdx.x * 64;
  const int mbeg = split * p.msplit;
  const int mend = min(p.M, mbeg + p.msplit);

  // X loader role: 8 consecutive columns x 8 consecutive rows; the MS/8 row
  // groups x 8 column groups of a sub-tile are spread over the 256 threads
  const int cb = tid & 7, mb = tid >> 3;       // mb in [0, 32)
  const int cl = c0 + cb * 8;
  const bool cval = cl < p.C;                   // C is a multiple of 8

  f32x4 acc[NB];
#pragma unroll
  for (int jb = 0; jb < NB; ++jb) acc[jb] = f32x4{0, 0, 0, 0};
  float cs[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) cs[e] = 0.f;

  for (int sub = mbeg; sub < mend; sub += MS) {
    __syncthreads();   // previous sub-tile fully consumed
    // ---- X[sub .. sub+MS, c0 .. c0+63] -> LDS, transposed (8x8 register transposes)
#pragma unroll
    for (int h = 0; h < (MS + 255) / 256; ++h) {
      const int mg = mb + 32 * h;             // row group of 8
      if (mg >= MS / 8) break;
      u32x4 rows[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int m = sub + mg * 8 + e;
        rows[e] = u32x4{0, 0, 0, 0};
        if (cval && m < mend) {
          rows[e] = ld16(p.X + (size_t)m * p.ldx + cl);
          if (p.colsum_mode == 1) {
            const u32x4 z = ld16(p.Z + (size_t)m * p.ldz + cl);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              cs[2 * t] += bf16_lo(rows[e][t]) * bf16_lo(z[t]);
              cs[2 * t + 1] += bf16_hi(rows[e][t]) * bf16_hi(z[t]);
            }
          } else if (p.colsum_mode == 2) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              cs[2 * t] += bf16_lo(rows[e][t]);
              cs[2 * t + 1] += bf16_hi(rows[e][t]);
            }
          }
        }
      }
      u32x4 cols[8];
      transpose8x8_b16(rows, cols);
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) *reinterpret_cast<u32x4*>(xt + xt_off(cb * 8 + cc, mg, ROWB)) = cols[cc];
    }
    // ---- S[sub .. sub+MS, 0 .. R) -> LDS as bf16 hi / lo, transposed [j][m]:
    // thread t takes row t % MS and a quarter of the columns, 16-byte loads
    {
      constexpr int TPR = 256 / MS;                 // threads per row (1 or 2)
      const int mm = tid % MS, part = tid / MS;
      const int m = sub + mm;
      const bool rv = m < mend;
      const bool vec = (p.lds % 4) == 0;
#pragma unroll
      for (int q = part * 4; q < RP; q += 4 * TPR) {
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        if (rv && q < p.R) {
          const float* src = p.S + (size_t)m * p.lds + q;
          if (vec && q + 4 <= p.R) {
            const f32x4 t = *reinterpret_cast<const f32x4*>(src);
            v[0] = t[0]; v[1] = t[1]; v[2] = t[2]; v[3] = t[3];
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (q + e < p.R) ? src[e] : 0.f;
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = v[e] * p.s_in;
          const uint32_t h = f32_to_bf16_bits(x);
          const int off = (xt_off(q + e, mm >> 3, ROWB) >> 1) + (mm & 7);   // same swizzle as the X tile
          shi[off] = (uint16_t)h;
          slo[off] = (uint16_t)f32_to_bf16_bits(x - __uint_as_float(h << 16));
        }
      }
    }
    __syncthreads();

    // ---- MS/32 reduction steps of 32 rows
    const int c_frag = wave * 16 + lr;
#pragma unroll 2
    for (int s = 0; s < MS / 32; ++s) {
      const u32x4 xf = *reinterpret_cast<const u32x4*>(xt + xt_off(c_frag, s * 4 + lq, ROWB));
#pragma unroll
      for (int jb = 0; jb < NB; ++jb) {
        const int j = jb * 16 + lr;
        const int so = xt_off(j, s * 4 + lq, ROWB);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(shi) + so);
        const u32x4 lo = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(slo) + so);
        acc[jb] = mfma_bf16(hi, xf, acc[jb]);
        acc[jb] = mfma_bf16(lo, xf, acc[jb]);
      }
    }
  }

  // ---- partial product: lane holds (j = jb*16 + 4*lq + i, c = c0 + 16*wave + lr)
  const int c = c0 + wave * 16 + lr;
  if (c < p.C) {
    float* dst = p.part + ((size_t)split * p.C + c) * RP;
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) *reinterpret_cast<f32x4*>(dst + jb * 16 + 4 * lq) = acc[jb];
  }

  // ---- column sums: reduce the row groups of each column
  if (p.colsum_mode != 0) {
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; ++e) csred[mb][cb * 8 + e] = cs[e];
    __syncthreads();
    if (tid < 64 && c0 + tid < p.C) {
      float t = 0.f;
      for (int g = 0; g < 32; ++g) t += csred[g][tid];
      p.cspart[(size_t)split * p.C + c0 + tid] = t;
    }
  }
}

// ============================================================================ colproj (streamed)
// Block = 64 columns of X and one split of rows.  Sub-tiles of MS rows of X
// (and Z for the DoRA column sums) and the matching rows of S (fp32, as
// stored) are copied to LDS through a 3-stage ring of direct buffer->LDS
// copies; X^T fragments come from transposing LDS reads, S^T fragments are
// gathered from the fp32 tile and split into bf16 hi + lo parts.  The four
// waves split each sub-tile's (32-row step, column block) work items and
// combine their partial sums at the end.  X rows are stored with 16-byte
// chunk c of row m at physical chunk c ^ 2 (m & 3).
//
// From rank 32 up (PK) S comes pre-split: pack_s_kernel writes s_in * S once as bf16
// hi + lo parts in MFMA fragment order (per 8-row group g: RP 16-byte chunks of hi, chunk j
// = rows 8g .. 8g+7 of rank column j, then RP chunks of lo), so a sub-tile's S is one
// contiguous copy and each fragment one 16-byte LDS read.  Building the fragments from
// the fp32 tile in every block costs more than the MFMAs at rank 64 (measured: 331 us of
// which ~180 us went to it at 8192 rows x 2 x 14336 columns).  The values fed to the MFMAs
// are the same bits either way.
//
// NH = 2 (no column sums): a block takes 128 columns as two 64-column halves, each staged
// and read exactly as a 64-column block, sharing one S tile; 32-row sub-tiles (64 at rank
// 16, where the S tile of 32 rows would be under one 4 KB copy round) keep the ring small.
template <int RP, int NH = 1>
struct ColStream {
  // rows per sub-tile: 64 from rank 32 up keeps the 3-stage ring at 48 KB, so three blocks
  // share a CU (128 rows measured 15-20 % slower at rank 32, 64 rows slower at rank 16)
  static constexpr int MS = NH == 2 ? (RP <= 16 ? 64 : 32) : (RP <= 16 ? 128 : 64);
  static constexpr int XB = MS * 128;                  // X (or Z) tile: MS rows x 64 columns (one half)
  static constexpr int SBY = MS * RP * 4;              // S tile: MS rows x up to RP fp32
  static constexpr int NSTEP = MS / 32;
  static constexpr int WPS = 4 / NSTEP;                // waves per step
  static constexpr int CFW = 4 / WPS;                  // 16-column blocks per wave
  static constexpr int STAGES = 3;
  static constexpr bool PK = RP >= 32;                 // S pre-split into packed hi / lo fragments
};

template <int RP, bool HASZ, int NH = 1>
__global__ __launch_bounds__(256) void colstream_kernel(const ColProjBatch batch) {
  using T = ColStream<RP, NH>;
  constexpr bool PK = T::PK;
  static_assert(NH == 1 || (NH == 2 && !HASZ), "two halves: no Z");
  constexpr int NB = RP / 16, MS = T::MS, XB = T::XB, SBY = T::SBY, ST = T::STAGES;
  constexpr int SB = XB * NH * (HASZ ? 2 : 1) + SBY;   // bytes per stage
  constexpr int NI = SB / 4096;
  __shared__ __attribute__((aligned(16))) uint8_t smem[ST * SB];
  const int y = blockIdx.y;
  const int jobi = y >= batch.first[2] ? 2 : (y >= batch.first[1] ? 1 : 0);
  const ColProjParams& p = batch.job[jobi];
  const int split = y - batch.first[jobi];
  const int c0 = blockIdx.x * 64 * NH;
  if (c0 >= p.C) return;
  const int mbeg = split * p.msplit;
  const int mend = min(p.M, mbeg + p.msplit);
  const int nsub = mend > mbeg ? (mend - mbeg + MS - 1) / MS : 0;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lq = lane >> 4;
  const bool zmode = HASZ && p.colsum_mode == 1;

  const uint32_t ldx_b = (uint32_t)p.ldx * 2u, lds_b = (uint32_t)p.lds * 4u, ldz_b = (uint32_t)p.ldz * 2u;
  // rows past mend read as zero
  const __amdgpu_buffer_rsrc_t rs_x = make_rsrc(p.X, (uint32_t)mend * ldx_b);
  // packed S: the whole array (rows past mend are finite and meet zero X rows; groups are
  // zero-filled past M)
  const __amdgpu_buffer_rsrc_t rs_s =
      PK ? make_rsrc(p.spk, p.R > 0 ? (uint32_t)((p.M + 7) / 8) * (32u * RP) : 0u)
         : make_rsrc(p.S, p.R > 0 ? (uint32_t)mend * lds_b : 0u);
  const __amdgpu_buffer_rsrc_t rs_z = make_rsrc(p.Z, zmode ? (uint32_t)mend * ldz_b : 0u);
  constexpr int NIX = XB / 4096, NIS = SBY / 4096;
  uint32_t x_off[NH][NIX], s_off[NIS];
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int i = 0; i < NIX; ++i) {
      const int b = (i * 4 + wave) * 1024 + lane * 16;
      const int row = b >> 7, phys = (b >> 4) & 7;
      x_off[h][i] = (uint32_t)row * ldx_b + (uint32_t)(c0 + 64 * h + 8 * (phys ^ (2 * (row & 3)))) * 2u;
    }
  const int rb = p.R > 0 ? p.R * 4 : 16;               // bytes per staged S row
#pragma unroll
  for (int i = 0; i < NIS; ++i) {
    const int b = (i * 4 + wave) * 1024 + lane * 16;
    s_off[i] = PK ? (uint32_t)b : (uint32_t)(b / rb) * lds_b + (uint32_t)(b % rb);
  }
  auto issue = [&](int sub) {
    uint8_t* sb = smem + (sub % ST) * SB;
    const uint32_t m = (uint32_t)(mbeg + sub * MS);
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int i = 0; i < NIX; ++i) buf2lds16(rs_x, x_off[h][i], m * ldx_b, sb + h * XB + (i * 4 + wave) * 1024);
#pragma unroll
    for (int i = 0; i < NIS; ++i)
      buf2lds16(rs_s, s_off[i], PK ? m * (4u * RP) : m * lds_b, sb + NH * XB + (i * 4 + wave) * 1024);
    if constexpr (HASZ) {
#pragma unroll
      for (int i = 0; i < NIX; ++i)   // same element layout as X (Z has its own leading dimension)
        buf2lds16(rs_z, x_off[0][i] / ldx_b * ldz_b + x_off[0][i] % ldx_b, m * ldz_b,
                  sb + XB + SBY + (i * 4 + wave) * 1024);
    }
  };

  constexpr int CFW = T::CFW;
  f32x4 acc[NH * CFW][NB];                              // this wave's column blocks: half h, my_cf0 + q
#pragma unroll
  for (int q = 0; q < NH * CFW; ++q)
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) acc[q][jb] = f32x4{0, 0, 0, 0};
  float cs[4] = {0.f, 0.f, 0.f, 0.f};
  const int my_step = wave % T::NSTEP, my_cf0 = (wave / T::NSTEP) * T::CFW;

#pragma unroll
  for (int c = 0; c < ST - 1; ++c)
    if (c < nsub) issue(c);
  for (int sub = 0; sub < nsub; ++sub) {
    if (sub + 1 < nsub) wait_vmcnt<NI>();
    else wait_vmcnt<0>();
    __syncthreads();                                    // sub-tile visible; sub-1's buffer free
    if (sub + ST - 1 < nsub) issue(sub + ST - 1);
    const uint8_t* sb = smem + (sub % ST) * SB;
    const float* ss = reinterpret_cast<const float*>(sb + NH * XB);
    const int mrow = my_step * 32 + 8 * lq;             // first of this lane's 8 rows
    // S^T fragments (rank j = jb*16 + lr, rows mrow .. mrow+7), hi / lo bf16 parts, pre-scaled
    u32x4 shi[NB], slo[NB];
    if constexpr (PK) {
      const uint8_t* sp = sb + NH * XB + (my_step * 4 + lq) * (32 * RP) + lr * 16;
#pragma unroll
      for (int jb = 0; jb < NB; ++jb) {
        shi[jb] = *reinterpret_cast<const u32x4*>(sp + jb * 256);
        slo[jb] = *reinterpret_cast<const u32x4*>(sp + RP * 16 + jb * 256);
      }
    } else {
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) {
      const int j = jb * 16 + lr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float v0 = 0.f, v1 = 0.f;
        if (j < p.R) {
          v0 = ss[(mrow + 2 * e) * p.R + j] * p.s_in;
          v1 = ss[(mrow + 2 * e + 1) * p.R + j] * p.s_in;
        }
        const uint32_t h0 = f32_to_bf16_bits(v0), h1 = f32_to_bf16_bits(v1);
        shi[jb][e] = h0 | (h1 << 16);
        slo[jb][e] = f32_to_bf16_bits(v0 - __uint_as_float(h0 << 16)) |
                     (f32_to_bf16_bits(v1 - __uint_as_float(h1 << 16)) << 16);
      }
    }
    }
#pragma unroll
    for (int qq = 0; qq < NH * T::CFW; ++qq) {
      const int q = qq % T::CFW;
      const int cf = my_cf0 + q;
      const uint8_t* sx = sb + (qq / T::CFW) * XB;      // this column block's half
      // X^T fragment: column c0 + 64 h + 16 cf + lr, rows mrow .. mrow+7 (two transposing reads)
      const int rr = my_step * 32 + 8 * lq + (lr >> 2);
      const int col = cf * 16 + 4 * (lr & 3);
      auto xoff = [&](int r) { return r * 128 + (((col >> 3) ^ (2 * (r & 3))) << 4) + ((col & 4) << 1); };
      const u32x2 lo = lds_tr16(sx, xoff(rr)), hi = lds_tr16(sx, xoff(rr + 4));
      const u32x4 xf = u32x4{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
      for (int jb = 0; jb < NB; ++jb) {
        acc[qq][jb] = mfma_bf16(shi[jb], xf, acc[qq][jb]);
        acc[qq][jb] = mfma_bf16(slo[jb], xf, acc[qq][jb]);
      }
      if constexpr (NH > 1) {
        // no column sums with two halves
      } else if (p.colsum_mode == 2) {
#pragma unroll
        for (int t = 0; t < 4; ++t) cs[q] += bf16_lo(xf[t]) + bf16_hi(xf[t]);
      } else if (zmode) {
        const uint8_t* sz = sb + XB + SBY;
        const u32x2 zl = lds_tr16(sz, xoff(rr)), zh = lds_tr16(sz, xoff(rr + 4));
        const u32x4 zf = u32x4{zl[0], zl[1], zh[0], zh[1]};
#pragma unroll
        for (int t = 0; t < 4; ++t) cs[q] += bf16_lo(xf[t]) * bf16_lo(zf[t]) + bf16_hi(xf[t]) * bf16_hi(zf[t]);
      }
    }
  }

  // combine the waves: lane holds part[c = c0 + 64 h + 16 cf + lr][j = jb*16 + 4*lq + i]
  __syncthreads();
  f32x4* red = reinterpret_cast<f32x4*>(smem);          // [4 waves][NH][CFW][NB][64]
  static_assert(4 * NH * CFW * NB * 64 * 16 <= ST * SB, "reduction scratch fits");
#pragma unroll
  for (int q = 0; q < NH * CFW; ++q)
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) red[((wave * NH * CFW + q) * NB + jb) * 64 + lane] = acc[q][jb];
  __syncthreads();
  for (int item = wave; item < NH * 4 * NB; item += 4) {
    const int hc = item / NB, jb = item % NB;
    const int h = hc / 4, cf = hc % 4;
    f32x4 v = f32x4{0, 0, 0, 0};
    for (int w = 0; w < 4; ++w) {                       // waves that own column block cf, in order
      const int q = cf - (w / T::NSTEP) * CFW;
      if (q >= 0 && q < CFW) v += red[((w * NH * CFW + h * CFW + q) * NB + jb) * 64 + lane];
    }
    const int c = c0 + 64 * h + cf * 16 + lr;
    if (c < p.C) *reinterpret_cast<f32x4*>(p.part + ((size_t)split * p.C + c) * RP + jb * 16 + 4 * lq) = v;
  }
  if (NH == 1 && p.colsum_mode != 0) {
    // column sums: lanes lr of the four 16-lane groups and the waves sharing a column block
    __syncthreads();
    float* csr = reinterpret_cast<float*>(smem);        // [4 waves][4 q][64 lanes]
#pragma unroll
    for (int q = 0; q < 4; ++q) csr[(wave * 4 + q) * 64 + lane] = cs[q];
    __syncthreads();
    if (tid < 64) {
      const int cf = tid >> 4, l16 = tid & 15;
      float t = 0.f;
      for (int w = 0; w < 4; ++w) {
        const int q = cf - (w / T::NSTEP) * T::CFW;      // this wave's slot for column block cf
        if (q < 0 || q >= T::CFW) continue;
#pragma unroll
        for (int g = 0; g < 4; ++g) t += csr[(w * 4 + q) * 64 + g * 16 + l16];
      }
      if (c0 + tid < p.C) p.cspart[(size_t)split * p.C + c0 + tid] = t;
    }
  }
}

// ============================================================================ reductions
// out[row, col] = alpha * sum_s part[s][...] (+ row scale) (+ alpha2 * sum_l Qm[row, l] * Am[l, col]).
// Threads walk the partial buffer in its own order ([C][rp], j fastest) so the
// split reads are coalesced; `trans` selects whether the partial's column index
// (j) is the output row (dA = part^T) or the output column (dB).
struct ReduceBatch {
  ReduceParams job[2];
  int njobs;
  int blocks0;                    // blocks [0, blocks0) reduce job 0, the rest job 1
};

// One block per 8 partial rows c of one job: the [8][rp] slice of every split is read as
// float4 groups; where the slice has fewer groups than the block has threads, the T threads
// of a group each sum a contiguous run of the splits in order (eight in flight) and the runs
// are added in thread order, so the order of the sum is fixed by the shape alone.  The
// sums are staged in LDS, then written out with the finishing terms, consecutive threads
// on consecutive output columns.  The optional Qm.Am addend (transposed jobs only: the
// partial rows are the output columns) reads both operands from dynamic LDS: Qm
// [rows, rq] (row stride rq + 1) and the block's 8 columns of Am [rq, cols].
constexpr int kReduceRows = 8;

// sum over splits [s0, s1) of the float4 at src (split stride pstride), in split order
__device__ __forceinline__ f32x4 sum_splits(const float* src, size_t pstride, int s0, int s1) {
  f32x4 acc = {0, 0, 0, 0};
  int sp = s0;
  for (; sp + 8 <= s1; sp += 8) {
    f32x4 a[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) a[q] = *reinterpret_cast<const f32x4*>(src + (size_t)(sp + q) * pstride);
#pragma unroll
    for (int q = 0; q < 8; ++q) acc += a[q];
  }
  for (; sp < s1; ++sp) acc += *reinterpret_cast<const f32x4*>(src + (size_t)sp * pstride);
  return acc;
}
__global__ __launch_bounds__(256) void reduce_parts_kernel(const ReduceBatch batch) {
  constexpr int RB = kReduceRows;
  __shared__ float tile[RB * 129];
  extern __shared__ float dyn[];
  const int jobi = (int)blockIdx.x >= batch.blocks0 ? 1 : 0;
  const ReduceParams& p = batch.job[jobi];
  const int c0 = ((int)blockIdx.x - (jobi ? batch.blocks0 : 0)) * RB;
  const int C = p.trans ? p.cols : p.rows;          // partial rows
  const int R = p.trans ? p.rows : p.cols;          // valid partial columns
  if (c0 >= C) return;
  const int tid = threadIdx.x;
  const int ld = p.rp + 1;
  const int nc = C - c0 < RB ? C - c0 : RB;
  const bool addend = p.Qm != nullptr;
  float* sQ = dyn;
  float* sA = dyn + R * (p.rq + 1);
  if (addend) {                                     // stage the addend's operands first
    for (int e = tid; e < R * p.rq; e += 256) {
      const int rr = e / p.rq, l = e % p.rq;
      sQ[rr * (p.rq + 1) + l] = p.Qm[(size_t)rr * p.ldq + l];
    }
    for (int e = tid; e < p.rq * RB; e += 256) {
      const int l = e / RB, cc = e % RB;
      sA[e] = cc < nc ? bf16_to_f32(p.Am[(size_t)l * p.lda + c0 + cc]) : 0.f;
    }
  }
  const int E = RB * p.rp / 4;                     // float4 groups of the slice
  const int T = (E < 256 && 256 % E == 0) ? 256 / E : 1;
  if (T > 1) {
    __shared__ f32x4 runs[256];
    const int e4 = tid % E, t = tid / E;
    const int e = e4 * 4, cc = e / p.rp, j = e % p.rp;
    f32x4 acc = {0, 0, 0, 0};
    if (c0 + cc < C && j < R)                       // columns >= R are padding (or another job's)
      acc = sum_splits(p.part + (size_t)(c0 + cc) * p.rp + j, p.pstride, t * p.nsplit / T,
                       (t + 1) * p.nsplit / T);
    runs[tid] = acc;
    __syncthreads();
    if (tid < E) {
      f32x4 v = runs[tid];
      for (int u = 1; u < T; ++u) v += runs[u * E + tid];
#pragma unroll
      for (int i = 0; i < 4; ++i) tile[cc * ld + j + i] = v[i];
    }
  } else {
    for (int e4 = tid; e4 < E; e4 += 256) {
      const int e = e4 * 4;                         // element offset inside the [RB][rp] slice
      const int cc = e / p.rp, j = e % p.rp;
      f32x4 acc = {0, 0, 0, 0};
      if (c0 + cc < C && j < R) acc = sum_splits(p.part + (size_t)(c0 + cc) * p.rp + j, p.pstride, 0, p.nsplit);
#pragma unroll
      for (int i = 0; i < 4; ++i) tile[cc * ld + j + i] = acc[i];
    }
  }
  __syncthreads();
  for (int e = tid; e < R * RB; e += 256) {
    int cc, j;
    if (p.trans) { j = e / RB; cc = e % RB; } else { cc = e / R; j = e % R; }
    if (cc >= nc) continue;
    const int c = c0 + cc;
    const int row = p.trans ? j : c, col = p.trans ? c : j;
    float v = tile[cc * ld + j] * p.alpha;
    if (p.rowscale != nullptr) v *= p.rowscale[row];
    if (addend) {
      const float* q = sQ + j * (p.rq + 1);
      float t = 0.f;
      for (int l = 0; l < p.rq; ++l) t += q[l] * sA[l * RB + cc];
      v += p.alpha2 * t;
    }
    p.out[(size_t)row * p.ldo + col] = v;
  }
}

__global__ void reduce_colsum_kernel(const float* cspart, int nsplit, int C, float* out) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= C) return;
  float acc = 0.f;
  for (int s = 0; s < nsplit; ++s) acc += cspart[(size_t)s * C + c];
  out[c] = acc;
}

__global__ void fill_zero_kernel(float* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0.f;
}

// ============================================================================ launchers
// The streamed kernel needs 16-byte aligned rows, and for a transposed Q an
// R that keeps its rows 8-byte aligned; a two-segment Q must switch segment
// on a copy-instruction boundary.
static bool rowstream_ok(const RowProjParams& p, int rp) {
  const int rl = rp <= 32 ? 1024 : (rp == 64 ? 512 : 256);
  const int rows_per_inst = 1024 / rl;
  if (p.ldp % 8 || (((uintptr_t)p.P) & 15) || (((uintptr_t)p.q0) & 15)) return false;
  if (p.P1 != nullptr && (p.p_split % 16 || p.ldp1 % 8 || (((uintptr_t)p.P1) & 15))) return false;
  if (p.P2 != nullptr && (p.p_split2 % 16 || p.ldp2 % 8 || (((uintptr_t)p.P2) & 15))) return false;
  if (p.q_kscale && (((uintptr_t)p.q_kscale) & 15)) return false;
  if (p.q_trans) return p.R % 4 == 0 && p.R0 == p.R;
  if (p.ldq % 8 || (((uintptr_t)p.q1) & 15)) return false;
  return p.R0 == p.R || p.R0 % rows_per_inst == 0;
}

template <int RP, bool KS>
static void rowstream_launch(const RowProjParams& p, dim3 grid, dim3 block, hipStream_t st) {
  hipLaunchKernelGGL((rowstream_kernel<RP, KS>), grid, block, 0, st, p);
}

// 32-row blocks at rank 64 and 128 (no k-scale): taken when they still give every CU a
// block (mode 1), always (mode 2, for tests) or never (mode 0)
int g_rowstream32 = 1;
static bool rowstream32(const RowProjParams& p, int rp) {
  if ((rp != 64 && rp != 128) || p.q_kscale != nullptr || g_rowstream32 == 0) return false;
  if (p.P1 != nullptr && p.p_split % 32) return false;
  if (p.P2 != nullptr && p.p_split2 % 32) return false;
  return g_rowstream32 == 2 || (p.M + 31) / 32 >= 256;
}

bool rowproj_packs(const RowProjParams& p) {
  if (p.M <= 0 || p.P2 != nullptr) return false;
  const int rp = p.R <= 16 ? 16 : p.R <= 32 ? 32 : p.R <= 64 ? 64 : 128;
  return rowstream_ok(p, rp) && p.pk_rp == rp;
}

bool rowproj_three_ok(const RowProjParams& p) {
  const int rp = p.R <= 16 ? 16 : p.R <= 32 ? 32 : p.R <= 64 ? 64 : 128;
  return p.P2 != nullptr && rowstream_ok(p, rp);
}

hipError_t launch_rowproj(const RowProjParams& p, hipStream_t st) {
  if (p.M <= 0) return hipSuccess;
  const int rp = p.R <= 16 ? 16 : p.R <= 32 ? 32 : p.R <= 64 ? 64 : 128;
  if ((p.P2 != nullptr || p.pk != nullptr) && !rowstream_ok(p, rp)) return hipErrorInvalidValue;   // (callers check first)
  if (p.pk != nullptr && (p.P2 != nullptr || p.pk_rp != rp)) return hipErrorInvalidValue;
  if (rowstream_ok(p, rp)) {
    if (rowstream32(p, rp)) {
      if (rp == 64) hipLaunchKernelGGL((rowstream_kernel<64, false, 32>), dim3((p.M + 31) / 32), dim3(256), 0, st, p);
      else hipLaunchKernelGGL((rowstream_kernel<128, false, 32>), dim3((p.M + 31) / 32), dim3(256), 0, st, p);
      return hipGetLastError();
    }
    const dim3 grid((p.M + 15) / 16), block(256);
    const bool ks = p.q_kscale != nullptr;
    switch (rp) {
      case 16: ks ? rowstream_launch<16, true>(p, grid, block, st) : rowstream_launch<16, false>(p, grid, block, st); break;
      case 32: ks ? rowstream_launch<32, true>(p, grid, block, st) : rowstream_launch<32, false>(p, grid, block, st); break;
      case 64: ks ? rowstream_launch<64, true>(p, grid, block, st) : rowstream_launch<64, false>(p, grid, block, st); break;
      default: ks ? rowstream_launch<128, true>(p, grid, block, st) : rowstream_launch<128, false>(p, grid, block, st); break;
    }
    return hipGetLastError();
  }
  const dim3 grid((p.M + 15) / 16), block(64 * RP_WAVES);
  switch (rp) {
    case 16: hipLaunchKernelGGL(rowproj_kernel<16>, grid, block, 0, st, p); break;
    case 32: hipLaunchKernelGGL(rowproj_kernel<32>, grid, block, 0, st, p); break;
    case 64: hipLaunchKernelGGL(rowproj_kernel<64>, grid, block, 0, st, p); break;
    default: hipLaunchKernelGGL(rowproj_kernel<128>, grid, block, 0, st, p); break;
  }
  return hipGetLastError();
}

int colproj_rp(int R) { return R <= 16 ? 16 : R <= 32 ? 32 : R <= 64 ? 64 : 128; }

size_t colproj_spk_words(int M, int R) { return M > 0 && R > 0 ? (size_t)((M + 7) / 8) * 8 * colproj_rp(R) : 0; }

// Packed S for the streamed column projection (rank padding RP >= 32): for 8-row group g
// and rank column j < RP, the 8 values v = s_in * S[8g + k, j] (zero past M and for
// j >= R) as bf16 hi = rne(v) at 16-byte chunk g * 2RP + j and lo = rne(v - hi) at chunk
// g * 2RP + RP + j.  One thread per (g, j); blockIdx.y selects the job.
struct PackSBatch {
  const float* S[kColProjBatch];
  const uint16_t* S16[kColProjBatch];              // bf16 S where set (S unused)
  int lds[kColProjBatch], M[kColProjBatch], R[kColProjBatch];
  float s_in[kColProjBatch];
  uint32_t* out[kColProjBatch];
};

template <int RP>
__global__ __launch_bounds__(256) void pack_s_kernel(const PackSBatch b) {
  const int job = blockIdx.y;
  const int M = b.M[job], R = b.R[job];
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= ((M + 7) / 8) * RP) return;
  const int g = t / RP, j = t % RP;
  u32x4 hi, lo;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int m0 = 8 * g + 2 * e;
    float v0 = 0.f, v1 = 0.f;
    if (j < R) {
      const uint16_t* s16 = b.S16[job];
      if (s16 != nullptr) {
        if (m0 < M) v0 = bf16_to_f32(s16[(size_t)m0 * b.lds[job] + j]) * b.s_in[job];
        if (m0 + 1 < M) v1 = bf16_to_f32(s16[(size_t)(m0 + 1) * b.lds[job] + j]) * b.s_in[job];
      } else {
        if (m0 < M) v0 = b.S[job][(size_t)m0 * b.lds[job] + j] * b.s_in[job];
        if (m0 + 1 < M) v1 = b.S[job][(size_t)(m0 + 1) * b.lds[job] + j] * b.s_in[job];
      }
    }
    const uint32_t h0 = f32_to_bf16_bits(v0), h1 = f32_to_bf16_bits(v1);
    hi[e] = h0 | (h1 << 16);
    lo[e] = f32_to_bf16_bits(v0 - __uint_as_float(h0 << 16)) | (f32_to_bf16_bits(v1 - __uint_as_float(h1 << 16)) << 16);
  }
  uint32_t* o = b.out[job] + (size_t)g * (8 * RP);
  *reinterpret_cast<u32x4*>(o + 4 * j) = hi;
  *reinterpret_cast<u32x4*>(o + 4 * (RP + j)) = lo;
}

static hipError_t pack_s_launch(const ColProjParams* jobs, int njobs, int RP, hipStream_t st) {
  PackSBatch b{};
  int nj = 0, maxt = 0;
  for (int i = 0; i < njobs; ++i) {
    if (jobs[i].R <= 0 || jobs[i].M <= 0) continue;
    if (jobs[i].spk_ready) continue;               // packed by the kernel that wrote S
    b.S[nj] = jobs[i].S; b.S16[nj] = jobs[i].S16; b.lds[nj] = jobs[i].lds; b.M[nj] = jobs[i].M; b.R[nj] = jobs[i].R;
    b.s_in[nj] = jobs[i].s_in; b.out[nj] = jobs[i].spk;
    const int tcount = ((jobs[i].M + 7) / 8) * RP;
    if (tcount > maxt) maxt = tcount;
    ++nj;
  }
  if (nj == 0) return hipSuccess;
  const dim3 grid((maxt + 255) / 256, nj);
  if (RP == 32) hipLaunchKernelGGL(pack_s_kernel<32>, grid, dim3(256), 0, st, b);
  else if (RP == 64) hipLaunchKernelGGL(pack_s_kernel<64>, grid, dim3(256), 0, st, b);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

void colproj_plan(int M, int C, int* nsplit, int* msplit, int blocks) {
  if (M <= 0) {
    *nsplit = 1;
    *msplit = 256;
    return;
  }
  // splits are whole multiples of 256 rows (a multiple of every sub-tile height);
  // aim for `blocks` blocks of this job (~512 per launch: two per CU, each streaming
  // several sub-tiles; jobs that share a launch split the target), at most 32 splits
  const int ctiles = (C + 63) / 64;
  const int mchunks = (M + 255) / 256;
  int want = (blocks + ctiles - 1) / ctiles;
  if (want < 1) want = 1;
  if (want > 32) want = 32;
  int ns = mchunks < want ? mchunks : want;
  if (ns < 1) ns = 1;
  const int per = (mchunks + ns - 1) / ns;      // 256-row chunks per split
  *msplit = per * 256;
  *nsplit = (M + *msplit - 1) / *msplit;
  if (*nsplit < 1) *nsplit = 1;
}

static hipError_t colproj_launch(const ColProjBatch& b, int gx, int gy, int R, hipStream_t st) {
  const dim3 grid(gx, gy), block(256);
  switch (colproj_rp(R)) {
    case 16: hipLaunchKernelGGL(colproj_kernel<16>, grid, block, 0, st, b); break;
    case 32: hipLaunchKernelGGL(colproj_kernel<32>, grid, block, 0, st, b); break;
    case 64: hipLaunchKernelGGL(colproj_kernel<64>, grid, block, 0, st, b); break;
    default: hipLaunchKernelGGL(colproj_kernel<128>, grid, block, 0, st, b); break;
  }
  return hipGetLastError();
}

// The streamed kernel copies 16-byte pieces: X, Z and S rows (below rank 32) must be
// 16-byte aligned; from rank 32 up it reads S from the packed copy in spk.
static bool colstream_ok(const ColProjParams& p) {
  if (p.ldx % 8 || (((uintptr_t)p.X) & 15)) return false;
  if (p.R > 0 && colproj_rp(p.R) >= 32) {
    if (p.spk == nullptr || (((uintptr_t)p.spk) & 15)) return false;
  } else if (p.R > 0 && (p.R % 4 || p.lds % 4 || (((uintptr_t)p.S) & 15))) {
    return false;
  }
  if (p.colsum_mode == 1 && (p.ldz % 8 || (((uintptr_t)p.Z) & 15))) return false;
  return p.msplit % 128 == 0;
}

template <bool HASZ>
static hipError_t colstream_launch(const ColProjBatch& b, int gx, int gy, int R, hipStream_t st) {
  const dim3 grid(gx, gy), block(256);
  // without column sums: 128-column blocks of two halves sharing each staged S tile (half
  // the S traffic per X byte; 149 -> 108 us for dBg + dBu at 8192 x 14336, r 64; about
  // 1 us per launch at r 32 and at r 16)
  if (!HASZ && colproj_rp(R) <= 64) {
    bool sums = false;
    for (int i = 0; i < kColProjBatch; ++i) sums = sums || b.job[i].colsum_mode != 0;
    if (!sums) {
      if (colproj_rp(R) == 64) hipLaunchKernelGGL((colstream_kernel<64, false, 2>), dim3((gx + 1) / 2, gy), block, 0, st, b);
      else if (colproj_rp(R) == 32) hipLaunchKernelGGL((colstream_kernel<32, false, 2>), dim3((gx + 1) / 2, gy), block, 0, st, b);
      else hipLaunchKernelGGL((colstream_kernel<16, false, 2>), dim3((gx + 1) / 2, gy), block, 0, st, b);
      return hipGetLastError();
    }
  }
  switch (colproj_rp(R)) {
    case 16: hipLaunchKernelGGL((colstream_kernel<16, HASZ>), grid, block, 0, st, b); break;
    case 32: hipLaunchKernelGGL((colstream_kernel<32, HASZ>), grid, block, 0, st, b); break;
    case 64: hipLaunchKernelGGL((colstream_kernel<64, HASZ>), grid, block, 0, st, b); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_colproj_batch(const ColProjParams* jobs, const int* nsplit, int njobs, hipStream_t st) {
  if (njobs < 1 || njobs > kColProjBatch) return hipErrorInvalidValue;
  for (int i = 1; i < njobs; ++i)
    if (colproj_rp(jobs[i].R) != colproj_rp(jobs[0].R)) {      // one rank padding per launch
      for (int k = 0; k < njobs; ++k) {
        const hipError_t e = launch_colproj_batch(jobs + k, nsplit + k, 1, st);
        if (e != hipSuccess) return e;
      }
      return hipSuccess;
    }
  ColProjBatch b;
  int maxc = 0;
  b.first[0] = 0;
  for (int i = 0; i < kColProjBatch; ++i) {
    b.job[i] = jobs[i < njobs ? i : 0];
    b.first[i + 1] = b.first[i] + (i < njobs ? nsplit[i] : 0);
    if (i < njobs && jobs[i].C > maxc) maxc = jobs[i].C;
  }
  bool stream = true, hasz = false, s16 = false;
  for (int i = 0; i < njobs; ++i) {
    stream = stream && colstream_ok(jobs[i]);
    hasz = hasz || jobs[i].colsum_mode == 1;
    s16 = s16 || jobs[i].S16 != nullptr;
  }
  if (s16 && !colproj_takes_bf16_s(jobs, njobs)) return hipErrorInvalidValue;
  if (stream && colproj_rp(jobs[0].R) <= 64) {      // rank 128: the register-transposing kernel is faster
    if (colproj_rp(jobs[0].R) >= 32) {
      const hipError_t e = pack_s_launch(jobs, njobs, colproj_rp(jobs[0].R), st);
      if (e != hipSuccess) return e;
    }
    return hasz ? colstream_launch<true>(b, (maxc + 63) / 64, b.first[njobs], jobs[0].R, st)
                : colstream_launch<false>(b, (maxc + 63) / 64, b.first[njobs], jobs[0].R, st);
  }
  return colproj_launch(b, (maxc + 63) / 64, b.first[njobs], jobs[0].R, st);
}

bool colproj_takes_bf16_s(const ColProjParams* jobs, int njobs) {
  if (njobs < 1 || njobs > kColProjBatch) return false;
  const int rp = colproj_rp(jobs[0].R);
  if (rp < 32 || rp > 64) return false;              // packed streaming path: rank 17 .. 64
  for (int i = 0; i < njobs; ++i)
    if (colproj_rp(jobs[i].R) != rp || !colstream_ok(jobs[i])) return false;
  return true;
}

hipError_t launch_colproj(const ColProjParams& p, int nsplit, hipStream_t st) {
  return launch_colproj_batch(&p, &nsplit, 1, st);
}

hipError_t launch_colproj2(const ColProjParams& a, int nsplit_a, const ColProjParams& b2, int nsplit_b, hipStream_t st) {
  const ColProjParams jobs[2] = {a, b2};
  const int ns[2] = {nsplit_a, nsplit_b};
  return launch_colproj_batch(jobs, ns, 2, st);
}

static int reduce_blocks(const ReduceParams& p) {
  return ((p.trans ? p.cols : p.rows) + kReduceRows - 1) / kReduceRows;
}
// dynamic LDS of the Qm.Am addend (0 without one)
static size_t reduce_lds(const ReduceParams& p) {
  if (p.Qm == nullptr) return 0;
  return ((size_t)p.rows * (p.rq + 1) + (size_t)p.rq * kReduceRows) * sizeof(float);
}
static hipError_t reduce_launch(const ReduceBatch& b, int blocks, size_t lds, hipStream_t st) {
  for (int i = 0; i < b.njobs; ++i)           // the addend is staged for transposed jobs only
    if (b.job[i].Qm != nullptr && !b.job[i].trans) return hipErrorInvalidValue;
  if (lds > 48 * 1024) {
    static bool raised = false;
    if (!raised) {
      const hipError_t e = hipFuncSetAttribute((const void*)reduce_parts_kernel,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, 120 * 1024);
      if (e != hipSuccess) return e;
      raised = true;
    }
  }
  hipLaunchKernelGGL(reduce_parts_kernel, dim3(blocks), dim3(256), lds, st, b);
  return hipGetLastError();
}

hipError_t launch_reduce2(const ReduceParams& a, const ReduceParams& b2, hipStream_t st) {
  ReduceBatch b;
  b.job[0] = a;
  b.job[1] = b2;
  b.njobs = 2;
  b.blocks0 = reduce_blocks(a);
  const int blocks = b.blocks0 + reduce_blocks(b2);
  if (blocks == 0) return hipSuccess;
  const size_t la = reduce_lds(a), lb = reduce_lds(b2);
  return reduce_launch(b, blocks, la > lb ? la : lb, st);
}

hipError_t launch_reduce(const ReduceParams& p, hipStream_t st) {
  ReduceBatch b;
  b.job[0] = p;
  b.job[1] = p;
  b.njobs = 1;
  b.blocks0 = reduce_blocks(p);
  if (b.blocks0 == 0) return hipSuccess;
  return reduce_launch(b, b.blocks0, reduce_lds(p), st);
}

hipError_t launch_reduce_colsum(const float* cspart, int nsplit, int C, float* out, hipStream_t st) {
  hipLaunchKernelGGL(reduce_colsum_kernel, dim3((C + 255) / 256), dim3(256), 0, st, cspart, nsplit, C, out);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

}  // namespace ldl
