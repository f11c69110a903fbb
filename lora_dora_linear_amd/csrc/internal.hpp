// Internal launch interface between the C entry points and the kernels.
#pragma once

#include "common.hpp"
#include "gemm_tile.hpp"

namespace ldl {

struct RowProjParams {
  int M, K, R, R0;                 // Q rows j < R0 come from q0, rows j >= R0 from q1
  const uint16_t* P; int ldp;      // [M, K] bf16; rows m >= p_split come from P1 (row m - p_split)
  const uint16_t* P1; int p_split; // P1 == nullptr: one segment (p_split = M)
  int ldp1;                        // leading dimension of P1
  const uint16_t* q0; const uint16_t* q1; int ldq;
  int q_trans;                     // 1: Q(j, k) = q0[k * ldq + j] (a [K, R] matrix such as lora_up B)
  const float* q_kscale;           // q_trans only, optional: Q(j, k) *= q_kscale[k] (rounded to bf16)
  float* out; int ldo;             // out[m * ldo + j] = scale * sum_k P[m,k] Q[j,k]
  float scale;
  // optional third segment (streamed kernel only): rows m >= p_split2 come from P2 (row
  // m - p_split2, leading dim ldp2) and go to out2 (row m - p_split2, leading dim ldo2)
  const uint16_t* P2; int p_split2; int ldp2;
  float* out2; int ldo2;
  // optional (streamed kernel, one segment): also write pk_scale * out in the packed bf16
  // hi / lo layout a column projection of rank padding pk_rp reads (pack_s_kernel's layout)
  uint16_t* pk; int pk_rp; float pk_scale;
};

struct ColProjParams {
  int M, C, R;
  const uint16_t* X; int ldx;      // [M, C] bf16, C a multiple of 8
  const float* S; int lds;         // [M, R] fp32
  float s_in;
  const uint16_t* Z; int ldz;      // colsum_mode 1: sum_m X*Z, 2: sum_m X
  int colsum_mode;
  int msplit;                      // rows per split (multiple of 256)
  float* part;                     // [nsplit][C][RP]
  float* cspart;                   // [nsplit][C]
  uint32_t* spk;                   // workspace for S pre-split into bf16 hi / lo fragments,
                                   // colproj_spk_words(M, R) words (used from rank 32 up)
  const uint16_t* S16;             // optional: S given in bf16 (row stride lds) instead of fp32;
                                   // only where colproj_takes_bf16_s says so
  bool spk_ready;                  // spk already holds s_in * S packed (no pack pass)
};

struct ReduceParams {
  int rows, cols;                  // output shape
  const float* part; size_t pstride; int nsplit, rp; int trans;
  float alpha;
  const float* rowscale;           // optional [rows]
  const float* Qm; int ldq, rq;    // optional addend alpha2 * Qm[rows, rq] . Am[rq, cols]
  const uint16_t* Am; int lda;
  float alpha2;
  float* out; int ldo;
};

// GEMM tile families (see gemm_tile.hpp); selected by the entry points.
enum GemmKind : int {
  GK_NT_PLAIN, GK_NT_FUSED, GK_NT_DORA, GK_NT_SWIGLU_DUAL, GK_NT_I8_DEQ, GK_NT_I8_RAW,
  GK_NN_PLAIN, GK_NN_SCALE, GK_NN_I8_SCALE, GK_NN_SWIGLU,
  GK_NN_DORA,    // NN with the two-output column-scale epilogue: out2 = z, out = z * col_scale[n]
  GK_NT_F8_DEQ   // e4m3 P and Q, dequantised by row_scale[m] col_scale[n], + low-rank term (+ bias)
};
hipError_t launch_gemm(GemmKind kind, const GemmParams& p, hipStream_t st);
// timing hook of ldl_set_kernel_events around one launch (rec: whether events were recorded)
hipError_t hook_start(int hook_kind, hipStream_t st, bool* rec);
hipError_t hook_stop(int hook_kind, hipStream_t st, bool rec);
extern int g_gemm_4wave;   // plain bf16 GEMMs on the four-wave 16x16x32 tile (tuning switch)
bool gemm_shape_ok(GemmKind kind, int M, int N, int K);
bool gemm_multi_leaf_ok(const GemmParams& p);
// fp32 partial bytes the split reduction of a plain 256-wide four-wave product of [M, N]
// outputs uses (0: no split for this shape); passed as GemmParams::part
size_t gemm_split_bytes(int M, int N);

hipError_t launch_rowproj(const RowProjParams& p, hipStream_t st);
bool rowproj_three_ok(const RowProjParams& p);   // the streamed kernel takes P2
bool rowproj_packs(const RowProjParams& p);       // the streamed kernel takes p with its pk
int colproj_rp(int R);
// whether a column-projection batch runs on the packed streaming path, which can read S in bf16
bool colproj_takes_bf16_s(const ColProjParams* jobs, int njobs);
extern int g_rowstream32;   // rank 33..128 row projections on 32-row blocks: 0 never, 1 auto, 2 always
// size in 32-bit words of the packed S a column projection of M rows and rank R needs
size_t colproj_spk_words(int M, int R);
// split plan of a column projection over M rows and C columns, aiming at `blocks` blocks
void colproj_plan(int M, int C, int* nsplit, int* msplit, int blocks = 512);
hipError_t launch_colproj(const ColProjParams& p, int nsplit, hipStream_t st);
// up to kColProjBatch independent column projections in one launch (one launch per job when
// their rank paddings differ)
constexpr int kColProjBatch = 3;
hipError_t launch_colproj_batch(const ColProjParams* jobs, const int* nsplit, int njobs, hipStream_t st);
hipError_t launch_colproj2(const ColProjParams& a, int nsplit_a, const ColProjParams& b, int nsplit_b, hipStream_t st);
hipError_t launch_reduce(const ReduceParams& p, hipStream_t st);
hipError_t launch_reduce2(const ReduceParams& a, const ReduceParams& b, hipStream_t st);
hipError_t launch_reduce_colsum(const float* cspart, int nsplit, int C, float* out, hipStream_t st);
hipError_t launch_fill_zero(float* p, size_t n, hipStream_t st);

// DoRA helpers
hipError_t launch_rowsumsq(const void* W0, int dtype_bf16, int N, int K, int ldw, float* out, hipStream_t st);
hipError_t launch_dora_norm(int N, int r, float s, float eps, const float* w0_sumsq, const float* P,
                            const float* G, const uint16_t* B, const float* m, float* norm, float* g, hipStream_t st);
// out = diag(g).W0 [N, K] and out2 = diag(g).B [N, r] (bf16, dense), one launch
hipError_t launch_scale_rows(const void* in, int N, int K, int ld, const void* in2, int r, const float* g, void* out,
                             void* out2, hipStream_t st);
hipError_t launch_scale_cols(const void* in, int M, int N, int ld, const float* g, void* out, int ldo,
                             hipStream_t st);

// gated-MLP backward over bf16 [M, N] arrays: dh (read from dE) -> de in place, du written (act: ACT_*)
hipError_t launch_swiglu_bwd(void* dE, int ld_de, const void* E, int ld_e, const void* U, int ld_u, void* dU,
                             int ld_du, int M, int N, int act, hipStream_t st);
hipError_t launch_dora_finalize(int N, int r, float s, float eps, const float* partT, const float* cspart,
                                int nsplit, int rpT, const float* norm, const float* g, const float* m,
                                const float* P, const float* G, const uint16_t* B,
                                float* dB, float* dm, float* wB, uint16_t* wB_pk, int pk_rp, hipStream_t st);

// LoRA merge: W = W0 + s.B.A (W0 may be null: the delta alone); bf16 or fp32 elements
hipError_t launch_merge(int N, int K, int r, float s, int bf16, const void* W0, int ldw, const void* A, const void* B,
                        void* W, int ldo, hipStream_t st);
hipError_t launch_bf16_to_f32(const void* in, size_t n, float* out, hipStream_t st);

// weight-space dropout: out[j, k] = keep[k] ? in[j, k] : 0 (esz 2: bf16, 4: fp32; in place allowed)
hipError_t launch_col_sumsq(const void* W0, int bf16, int N, int K, int ldw, float* colsq, hipStream_t st);
hipError_t launch_dora_cols_norm(int K, int r, float s, float eps, const float* colsq, const float* m,
                                 const void* A, const float* Pc, const float* Gc, float* norm, float* g,
                                 hipStream_t st);
hipError_t launch_dora_cols_bwd(int K, int r, float s, float eps, const float* dg_part, int dg_nsplit,
                                const float* norm, const float* m, const void* A, const float* Pc, const float* Gc,
                                float* dm, float* dA, void* Aw, hipStream_t st);
hipError_t launch_dora_cols_db(int N, int r, float s, const void* B, const float* T, float* dB, hipStream_t st);
hipError_t launch_mask_cols(const void* in, const uint8_t* keep, int rows, int K, int esz, void* out, hipStream_t st);

// W8A8 helpers
// bf16 [N, K] (dense) = codes [N, K] (row stride ldq) times the row scale; int8 or e4m3 codes
hipError_t launch_dequant8(const void* q, int N, int K, int ldq, const float* scale, int fp8, void* out,
                           hipStream_t st);
// fp8: e4m3 codes (scale absmax / 448) instead of int8 (absmax / 127)
hipError_t launch_quantize_rows(const void* X, int in_f32, int M, int K, int ldx, int8_t* q, float* scale,
                                hipStream_t st, int fp8 = 0);

// fp32 path: C[m, n] = alpha * sum_k A(m, k) B(k, n) + beta * C[m, n] (+ bias[n])
struct F32GemmParams {
  int M, N, K;
  const float* A; long sam, sak;
  const float* B; long sbk, sbn;
  float* C; int ldc;
  float alpha, beta;
  const float* bias;
};
hipError_t launch_f32_gemm(const F32GemmParams& p, hipStream_t st);
// the fp32 LoRA layer at small sizes: forward and backward in one launch each
bool f32_small_ok(int M, int N, int K, int r);
hipError_t launch_f32_small_fwd(int M, int N, int K, int r, float s, const float* X, int ldx, const float* W0,
                                int ldw, const float* A, const float* B, const float* bias, float* Y, int ldy,
                                float* U, int ldu, hipStream_t st);
hipError_t launch_f32_small_bwd(int M, int N, int K, int r, float s, const float* dY, int lddy, const float* X,
                                int ldx, const float* W0, int ldw, const float* A, const float* B, const float* U,
                                int ldu, float* dX, int lddx, float* dA, float* dB, float* dbias, hipStream_t st);
hipError_t launch_f32_colsum(const float* X, int M, int N, int ld, float* out, hipStream_t st);

}  // namespace ldl
