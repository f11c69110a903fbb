/*
 * lora_dora_linear.h - C interface of the fused LoRA / DoRA adapted linear
 * layer for AMD Instinct MI355X (gfx950).
 *
 * Method (sources are web pages; each entry point cites the passage that
 * defines it):
 *   Y = X . W0^T + s . (X . A^T) . B^T              (LoRA bypass, never forming B.A)
 *   DoRA rows:  Y = g (.) (X . W0^T + s . (X . A^T) . B^T) + b,
 *               g_n = m_n / max(||W0_n + s . B_n . A||, eps), the norm from the
 *               closed form rowsum(W0^2)_n + 2s <B_n, (W0 A^T)_n> + s^2 B_n (A A^T) B_n^T.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Shapes: X [M,K], W0 [N,K], A = lora_down [r,K], B = lora_up [N,r],
 *    Y and dY [M,N], dX [M,K].  Every tensor is row-major (last index
 *    contiguous).  Operands passed with a leading-dimension argument (ldx, ldw,
 *    ldy, lddy, lddx, ldu, ldz, ...) may be strided views such as column slices
 *    of a wider buffer: ld is the distance between consecutive rows in elements,
 *    0 selects the row length (dense).  An ld below the row length is
 *    LDL_E_INVAL; for the bf16 / int8 kernels rows must start on 16-byte
 *    boundaries (ld a multiple of 8 bf16 elements, 16 int8 elements, or 4 fp32
 *    elements for U), else LDL_E_UNSUPPORTED.  The fp32 path takes any ld.
 *    Operands without an ld argument (A, B, bias, m, the DoRA state, the SwiGLU
 *    weights and saved activations, the factor gradients) are dense.
 *  - Pointers are DEVICE pointers owned by the caller (inputs, outputs and the
 *    workspace).  The library keeps no state and never allocates.
 *  - dtype: LDL_BF16 (bf16 storage, fp32 accumulation) or LDL_F32.  U, V,
 *    gradients of A, B and the DoRA magnitude are always fp32.
 *  - `stream` is a hipStream_t passed as void* (NULL = default stream).  Calls
 *    only enqueue work; they never synchronise the host.
 *  - Errors: the return value is a status.  Every argument is validated on the
 *    host before anything is enqueued, so an error leaves all outputs
 *    untouched.  LDL_E_INVAL: null required pointer, negative size, bad dtype;
 *    LDL_E_UNSUPPORTED: shape outside what the kernels take (listed per call);
 *    LDL_E_WORKSPACE: ws_bytes below ldl_workspace_bytes() (without its optional
 *    split-reduction partials, see there); LDL_E_HIP: a kernel
 *    launch failed (hipGetLastError is left set).  M == 0 is valid and does
 *    nothing (weight-gradient outputs are zeroed).
 *  - Shape limits of the bf16 / int8 kernels: K and N multiples of 64
 *    (K multiple of 128 for the int8 base), 1 <= r <= 128, every tensor below
 *    2 GiB.  M is arbitrary.  The fp32 path takes any positive N, K, r.
 *  - Determinism: every reduction runs in a fixed order; two calls with the
 *    same inputs give bitwise identical outputs.
 */
#ifndef LORA_DORA_LINEAR_H
#define LORA_DORA_LINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LDL_OK = 0,
  LDL_E_INVAL = -1,
  LDL_E_UNSUPPORTED = -2,
  LDL_E_WORKSPACE = -3,
  LDL_E_HIP = -4
} ldl_status;

typedef enum { LDL_F32 = 0, LDL_BF16 = 1 } ldl_dtype;

/* Operation ids for ldl_workspace_bytes. */
typedef enum {
  LDL_OP_LORA_FWD = 0,
  LDL_OP_LORA_BWD = 1,
  LDL_OP_DORA_FWD = 2,
  LDL_OP_DORA_BWD = 3,
  LDL_OP_SWIGLU_FWD = 4, /* N = hidden size H */
  LDL_OP_SWIGLU_BWD = 5, /* N = hidden size H */
  LDL_OP_W8A8_FWD = 6,
  LDL_OP_W8A8_BWD = 7,
  LDL_OP_MERGE_BWD = 8,  /* M unused; N x K weight */
  LDL_OP_DORA_COLS_FWD = 9,
  LDL_OP_DORA_COLS_BWD = 10
} ldl_op;

/* Human-readable text of a status code (static storage). */
const char* ldl_status_string(int status);

/* Library version as an integer (major*10000 + minor*100 + patch). */
int ldl_version(void);

/* Tuning switches (process-wide; not thread-safe against concurrent calls).
 *   LDL_TUNE_FWD_FUSED_DOWNPROJ (0/1, default 0): compute U = X.A^T inside the
 *     K-loop of the base GEMM from the LDS-staged X tiles (r <= 64, N multiple
 *     of 128) instead of a separate rank-r pass before it.
 *   LDL_TUNE_GEMM_4WAVE (0/1/2, default 1): run the bf16 GEMMs with a low-rank
 *     term of rank <= 64 and M > 128 on the four-wave tile with 16x16x32 MFMAs:
 *     the LoRA forward and input gradient and the DoRA forward (N a multiple of
 *     256, or of 192 when 256-wide tiles would leave CUs idle), the DoRA input
 *     gradient and, in the SwiGLU MLP, the gate/up dual tile (hidden width a
 *     multiple of 128; the activation formed in its epilogue) and the down
 *     projection's input gradient (hidden width a multiple of 256: a plain
 *     product followed by a streaming SwiGLU-backward pass instead of the fused
 *     epilogue), and the W8A8 int8 forward (N a multiple of 256, unless 256 x 128
 *     tiles fit the chip in one round; 2 takes the four-wave int8 tile whenever the
 *     shape allows); 0 selects the eight-wave tiles and fused epilogues for all of them.
 *   LDL_TUNE_ROWSTREAM_32 (0/1/2, default 1): row projections of rank 33..128
 *     (U = X.A^T, V = dY.B and their like) on 32-row blocks that stage the rank
 *     factor once per 32 rows: 1 when those blocks still fill the 256 CUs
 *     (M >= 8161), 2 whenever the rank allows, 0 never.  Results are identical.
 *   LDL_TUNE_PREPACK (0/1, default 1): in the DoRA and gated-MLP backwards, the rank
 *     factors of the last column projections (ranks 17..64) written in their packed
 *     bf16 hi / lo form by the kernels that compute them, instead of by a separate
 *     packing pass (0).  Results are identical.
 * Returns LDL_OK, or LDL_E_INVAL for an unknown key or value. */
typedef enum {
  LDL_TUNE_FWD_FUSED_DOWNPROJ = 0, LDL_TUNE_GEMM_4WAVE = 1, LDL_TUNE_ROWSTREAM_32 = 2, LDL_TUNE_PREPACK = 3
} ldl_tune_key;
int ldl_set_tuning(int key, int value);

/* Kernel timing hook for profilers and benchmarks.  While set, the library
 * records start_events[i] / stop_events[i] (hipEvent_t, passed as void*) on the
 * call's stream around the i-th launch of the kernel `kind`, for i < count, and
 * stops recording after `count` launches.  count = 0 (or NULL arrays) turns it
 * off.  The arrays must stay valid while the hook is set.
 *   kind 0: the base GEMM of the LoRA / DoRA / W8A8 forward (the [M,N] output GEMM)
 *   kind 1: the input-gradient GEMM of the LoRA / DoRA / W8A8 backward (the [M,K] dX GEMM)
 *   kind 2: the gated MLP backward's activation pass (the streaming pass over dH, E and Gu
 *           that writes dE and dGu; recorded only where that pass is a launch of its own)
 * Returns LDL_OK or LDL_E_INVAL. */
int ldl_set_kernel_events(int kind, void** start_events, void** stop_events, int count);

/* Bytes of device workspace the entry point `op` needs for these sizes (256-byte
 * aligned, 0 when none).  Pure host arithmetic; never fails (returns 0 for
 * invalid sizes, which the entry point then rejects).  For the LoRA and 8-bit
 * forward and backward this includes fp32 partials for the split reduction of the
 * output tiles past the last full round of the GPU's compute units; a call given
 * less (but at least what it needs without them) runs those tiles unsplit, with
 * the same results up to fp32 summation order. */
size_t ldl_workspace_bytes(int op, int M, int N, int K, int r, int dtype);

/* ------------------------------------------------------------------------ LoRA
 * Forward of the LoRA bypass linear: the rank-r update is folded into the base
 * GEMM and the [N,K] product B.A is never formed ("How Unsloth's FastLoRA Kernel
 * Differs from Standard LoRA Implementations", section "Fused Forward Pass
 * Architecture"; "LoRA/DoRA fast forward: no weight materialization", commit
 * message; lora_down / lora_up orientation as in "nunchaku-style kernel fusion -
 * 20-30% faster training", LoRA-epilogue commit).
 *   Y = X.W0^T + s.(X.A^T).B^T (+ bias)
 *   X [M,K] (row stride ldx), W0 [N,K] (ldw), A [r,K], B [N,r], bias [N] or NULL
 *   (dtype of X), Y [M,N] (ldy).  U_save [M,r] fp32 (ldu) or NULL: receives
 *   U = X.A^T for the backward.
 */
int lora_linear_fwd(int M, int N, int K, int r, float s, int dtype,
                    const void* X, int ldx, const void* W0, int ldw, const void* A, const void* B,
                    const void* bias, void* Y, int ldy, float* U_save, int ldu,
                    void* ws, size_t ws_bytes, void* stream);

/* Backward of the LoRA linear with W0 frozen.  The LoRA input gradient is folded
 * into the dX GEMM epilogue; dA, dB come from skinny contractions with the factor
 * gradients pre-scaled by s ("How Unsloth's FastLoRA Kernel ...", section "Custom
 * Backward Pass Implementation"; "nunchaku-style kernel fusion ...", LoRA-epilogue
 * commit: neither direction builds an (M, out_features) intermediate).
 *   V = dY.B;  dX = dY.W0 + s.V.A;  dA = s.V^T.X;  dB = s.dY^T.U;  dbias = sum_m dY.
 *   dY [M,N] (lddy); X, W0, A, B as in the forward; U_saved [M,r] fp32 (ldu) from
 *   the forward (NULL: recomputed).  dX [M,K] (dtype, lddx) or NULL; dA [r,K],
 *   dB [N,r] fp32 (overwritten); dbias [N] fp32 or NULL.
 */
int lora_linear_bwd(int M, int N, int K, int r, float s, int dtype,
                    const void* dY, int lddy, const void* X, int ldx, const void* W0, int ldw,
                    const void* A, const void* B, const float* U_saved, int ldu,
                    void* dX, int lddx, float* dA, float* dB, float* dbias,
                    void* ws, size_t ws_bytes, void* stream);

/* The LoRA backward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation and arguments as lora_linear_bwd without the workspace, which comes
 * from a fixed device-resident scratch array of ldl_noalloc_scratch_bytes() bytes
 * (32 MiB) that the library holds on each device it runs on until the process ends.
 * The call makes no allocation of any kind.  The device is the calling thread's
 * current device, which must be the one `stream` belongs to.  Sizes whose workspace
 * (ldl_workspace_bytes(LDL_OP_LORA_BWD, ...)) exceeds the scratch return
 * LDL_E_WORKSPACE before anything is enqueued.  All calls on one device share its
 * scratch, and it keeps the last call's contents: calls that overlap in time on one
 * device (different streams, or different host threads) race and give wrong results;
 * serialise them.  LDL_E_HIP also reports a failed lookup of the device's scratch. */
int lora_linear_bwd_noalloc(int M, int N, int K, int r, float s, int dtype,
                            const void* dY, int lddy, const void* X, int ldx, const void* W0, int ldw,
                            const void* A, const void* B, const float* U_saved, int ldu,
                            void* dX, int lddx, float* dA, float* dB, float* dbias,
                            void* stream);

/* Size in bytes of the per-device scratch array lora_linear_bwd_noalloc uses. */
size_t ldl_noalloc_scratch_bytes(void);

/* ------------------------------------------------------------------------ fused QKV leaves
 * Several LoRA adapters ("leaves", e.g. query / key / value) over one concatenated base
 * weight, computed as one base GEMM in which each output column takes its own leaf's
 * adapter ("How Unsloth's FastLoRA Kernel ...", section "Fused Forward Pass Architecture":
 * a fused Function for the attention projections; "nunchaku-style kernel fusion ...",
 * LoRA-epilogue commit: fused-qkv adapters narrow lora_up to the leaf's rows).  bf16 only.
 *   Leaf l has n_leaf[l] output columns, scale s_leaf[l] and factors A_l [r,K], B_l
 *   [n_leaf[l], r]; W0 = [W0_1; ..; W0_L] [N,K] with N = sum n_leaf (row stride ldw),
 *   A = [A_1; ..; A_L] [L r, K], B = [B_1; ..; B_L] [N, r] (both dense), bias [N] or NULL.
 *   Y[:, leaf l] = X.W0_l^T + s_l.(X.A_l^T).B_l^T (+ bias).  Y [M,N] (ldy); U_save [M, L r]
 *   fp32 (ldu) or NULL receives [X.A_1^T | .. | X.A_L^T].
 *   n_leaf and s_leaf are HOST arrays of nleaf entries, read during the call only.
 *   Limits: 1 <= nleaf <= 8, every n_leaf[l] a multiple of 64, K a multiple of 64, r a
 *   multiple of 8 with L r <= 128.  When L r <= 64 and the shape runs on the four-wave
 *   tile (more than 128 rows, N a multiple of 256 or filling 192-column tiles) the whole
 *   layer is one rank-(L r) projection plus one GEMM; otherwise each leaf runs as
 *   lora_linear_fwd on its column block.
 *   Workspace: ldl_multi_workspace_bytes(LDL_OP_LORA_FWD, ...) (0 needed with U_save). */
size_t ldl_multi_workspace_bytes(int op, int M, int K, int nleaf, const int* n_leaf, int r);

int lora_multi_linear_fwd(int M, int K, int nleaf, const int* n_leaf, int r, const float* s_leaf, int dtype,
                          const void* X, int ldx, const void* W0, int ldw, const void* A, const void* B,
                          const void* bias, void* Y, int ldy, float* U_save, int ldu,
                          void* ws, size_t ws_bytes, void* stream);

/* Backward of the fused leaves (W0 frozen):
 *   V_l = s_l.dY_l.B_l;  dX = dY.W0 + sum_l V_l.A_l (one GEMM of rank L r);
 *   dA_l = V_l^T.X;  dB_l = s_l.dY_l^T.U_l;  dbias = sum_m dY.
 *   dY [M,N] (lddy), X (ldx), W0 (ldw), U_saved [M, L r] (ldu) or NULL (recomputed).
 *   dX [M,K] bf16 (lddx) or NULL; dA [L r, K], dB [N, r] fp32 (overwritten); dbias [N] fp32
 *   or NULL.  Workspace: ldl_multi_workspace_bytes(LDL_OP_LORA_BWD, ...). */
int lora_multi_linear_bwd(int M, int K, int nleaf, const int* n_leaf, int r, const float* s_leaf, int dtype,
                          const void* dY, int lddy, const void* X, int ldx, const void* W0, int ldw,
                          const void* A, const void* B, const float* U_saved, int ldu,
                          void* dX, int lddx, float* dA, float* dB, float* dbias,
                          void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ weight-space dropout
 * Dropout of the adapter drawn once per forward in weight space and shared with the DoRA norm
 * terms ("LoRA/DoRA fast forward: no weight materialization", section "Fidelity"): a keep
 * mask over the input features of lora_down (the same for every rank), drawn by the caller,
 * with the inverted-dropout scale 1 / (1 - p).  The layer with dropout is the plain layer run
 * with A_drop = A . diag(keep) and s / (1 - p) in place of A and s (lora_linear_* ,
 * dora_linear_*, w8a8_lora_linear_*: the DoRA norm then sees the same dropped factor), after
 * which lora_dropout_grad zeroes the dropped columns of the factor gradient dA.  Exact: the
 * kernels copy or zero elements.
 *   lora_dropout_mask: A [r,K] (dtype), keep [K] (0 drops feature k), A_drop [r,K] (dtype;
 *   may be A itself).  lora_dropout_grad: dA [r,K] fp32 masked in place. */
int lora_dropout_mask(int r, int K, int dtype, const void* A, const uint8_t* keep, void* A_drop, void* stream);
int lora_dropout_grad(int r, int K, const uint8_t* keep, float* dA, void* stream);

/* ------------------------------------------------------------------------ LoRA merge
 * The adapted weight formed explicitly, for export or for merging an adapter into its base
 * weight: the merge forward (the delta) and merge backward of the lora family ("Fused
 * Kernels (experimental)", section "What is fused").  The rank-r product is generated tile
 * by tile in registers and written once.
 *   W = W0 + s.B.A   (W0 NULL: W = s.B.A).  W0, W [N,K] (row strides ldw, ldo; W == W0
 *   merges in place and needs ldo == ldw); A [r,K], B [N,r].  dtype LDL_BF16 or LDL_F32.
 *   Limits: K a multiple of 64 (bf16) or 8 (fp32), r <= 128. */
int lora_merge_fwd(int N, int K, int r, float s, int dtype, const void* W0, int ldw,
                   const void* A, const void* B, void* W, int ldo, void* stream);

/* Gradients of the factors from a gradient dW [N,K] (row stride lddw) of the merged weight:
 *   dA = s.B^T.dW [r,K],  dB = s.dW.A^T [N,r]  (fp32, overwritten).
 *   Workspace: ldl_workspace_bytes(LDL_OP_MERGE_BWD, 0, N, K, r, dtype). */
int lora_merge_bwd(int N, int K, int r, float s, int dtype, const void* dW, int lddw,
                   const void* A, const void* B, float* dA, float* dB,
                   void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ DoRA
 * Row-scaled DoRA ("dora-rows"), bf16 only.  The row norm of W' = W0 + s.B.A uses
 * the closed form: the row sums of W0^2 (computed once per frozen weight by
 * dora_prepare) plus the two rank-sized terms
 * P = W0.A^T [N,r] and G = A.A^T [r,r]; the bias is added after the row scale; the
 * norm stays in the autograd graph; eps clamps the norm from below
 * ("LoRA/DoRA fast forward: no weight materialization", commit message, sections
 * "What" and "Fidelity").
 */

/* Once per frozen W0 [N,K] (row stride ldw): w0_sumsq[n] = sum_k W0[n,k]^2 (fp32 [N]).
 * Must be recomputed whenever W0 changes. */
int dora_prepare(int N, int K, int dtype, const void* W0, int ldw, float* w0_sumsq, void* stream);

/* Floats in the DoRA state buffer the forward fills and the backward reads:
 * norm [N] | g [N] | P [N*r] | G [r*r]. */
size_t dora_state_floats(int N, int r);

/*   Z = X.W0^T + s.(X.A^T).B^T;  Y = g (.) Z + bias,  g_n = m_n / max(nu_n, eps).
 *   X [M,K] (ldx), W0 [N,K] (ldw); m [N] fp32 magnitude; w0_sumsq [N] from
 *   dora_prepare; bias [N] or NULL; Y [M,N] (ldy); U_save [M,r] fp32 (ldu, required);
 *   Z_save [M,N] (dtype, ldz, required, read by the backward for the magnitude
 *   gradient); state: dora_state_floats(N,r) fp32 (required). */
int dora_linear_fwd(int M, int N, int K, int r, float s, float eps, int dtype,
                    const void* X, int ldx, const void* W0, int ldw, const void* A, const void* B,
                    const float* m, const float* w0_sumsq, const void* bias,
                    void* Y, int ldy, float* U_save, int ldu, void* Z_save, int ldz, float* state,
                    void* ws, size_t ws_bytes, void* stream);

/* Gradients of the row-scaled DoRA layer, norm kept in the graph:
 *   dZ = dY.diag(g);  dg_n = sum_m dY[m,n] Z[m,n];  dm = dg / max(nu, eps);
 *   w_n = -dg_n m_n / (2 nu_n^3) (0 where nu_n <= eps);
 *   dX = dZ.W0 + s.(dZ.B).A
 *   dB = s.dZ^T.U + w (.) (2s.P + 2s^2.B.G)
 *   dA = s.(dZ.B)^T.X + 2s.(w (.) B)^T.W0 + 2s^2.(B^T diag(w) B).A
 *   Inputs as in the forward plus dY [M,N] (lddy), U_saved (ldu), Z_saved (ldz),
 *   state.  Outputs dX [M,K] (dtype, lddx) or NULL; dA [r,K], dB [N,r], dm [N] fp32;
 *   dbias [N] fp32 or NULL. */
int dora_linear_bwd(int M, int N, int K, int r, float s, float eps, int dtype,
                    const void* dY, int lddy, const void* X, int ldx, const void* W0, int ldw,
                    const void* A, const void* B, const float* m, const float* U_saved, int ldu,
                    const void* Z_saved, int ldz, const float* state,
                    void* dX, int lddx, float* dA, float* dB, float* dm, float* dbias,
                    void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ DoRA, column form
 * Column-scaled DoRA ("dora-cols"), bf16 only: the norm is taken per input column k of
 * W' = W0 + s.B.A and the magnitude m [K] over it scales the layer input per feature
 * ("LoRA/DoRA fast forward: no weight materialization", section "What": lora, dora-rows
 * and dora-cols; section "Fidelity": norm in the graph, eps clamp, bias un-scaled).  The
 * column norm comes from the closed form colsum(W0^2)_k + 2s <A_k, (B^T W0)_k> +
 * s^2 A_k^T (B^T B) A_k with the cached constant colsum(W0^2) and the rank-sized terms
 * Pc = B^T.W0 [r,K] and Gc = B^T.B [r,r]; the adapted weight is never formed.
 */

/* Once per frozen W0 [N,K] (row stride ldw, dtype LDL_F32 or LDL_BF16; bf16 needs K and ldw
 * multiples of 8): w0_colsq[k] = sum_n W0[n,k]^2 (fp32 [K]).  Recompute whenever W0 changes. */
int dora_cols_prepare(int N, int K, int dtype, const void* W0, int ldw, float* w0_colsq, void* stream);

/*   nu_k = ||W'[:,k]||;  g_k = m_k / max(nu_k, eps);  Xs = X.diag(g);
 *   Y = Xs.W0^T + s.(Xs.A^T).B^T (+ bias)   (= X.(W'.diag(g))^T + bias).
 *   X [M,K] (ldx), W0 [N,K] (ldw), A [r,K], B [N,r], m [K] fp32, w0_colsq [K] from
 *   dora_cols_prepare, bias [N] or NULL, Y [M,N] (ldy).  Xs_save [M,K] bf16 (ldxs,
 *   required: the scaled input, read by the backward); U_save [M,r] fp32 (ldu) or NULL
 *   receives Xs.A^T.  state: dora_state_floats(K, r) fp32 (required) = norm [K] | g [K] |
 *   Pc [r*K] | Gc [r*r].  Limits: those of the bf16 layer, r a multiple of 8, r <= 64.
 *   Workspace: ldl_workspace_bytes(LDL_OP_DORA_COLS_FWD, M, N, K, r, dtype). */
int dora_cols_linear_fwd(int M, int N, int K, int r, float s, float eps, int dtype,
                         const void* X, int ldx, const void* W0, int ldw, const void* A, const void* B,
                         const float* m, const float* w0_colsq, const void* bias,
                         void* Y, int ldy, float* U_save, int ldu, void* Xs_save, int ldxs, float* state,
                         void* ws, size_t ws_bytes, void* stream);

/* Gradients of the column-scaled layer, norm kept in the graph:
 *   dXs = dY.W';  dX = dXs.diag(g);  dg_k = sum_m dXs[m,k] X[m,k];  dm = dg / max(nu, eps);
 *   w_k = -dg_k m_k / (2 nu_k^3) (0 where nu_k <= eps);
 *   dA = s.(dY.B)^T.Xs + 2s (Pc + s.Gc.A).diag(w)
 *   dB = s.dY^T.U + 2s W0.diag(w).A^T + 2s^2 B.(A.diag(w).A^T);  dbias = sum_m dY.
 *   Inputs as in the forward plus dY [M,N] (lddy), Xs_saved (ldxs), U_saved (ldu) or NULL
 *   (recomputed), state.  Outputs dX [M,K] bf16 (lddx) or NULL; dA [r,K], dB [N,r], dm [K]
 *   fp32; dbias [N] fp32 or NULL.
 *   Workspace: ldl_workspace_bytes(LDL_OP_DORA_COLS_BWD, M, N, K, r, dtype). */
int dora_cols_linear_bwd(int M, int N, int K, int r, float s, float eps, int dtype,
                         const void* dY, int lddy, const void* X, int ldx, const void* Xs_saved, int ldxs,
                         const void* W0, int ldw, const void* A, const void* B, const float* m,
                         const float* U_saved, int ldu, const float* state,
                         void* dX, int lddx, float* dA, float* dB, float* dm, float* dbias,
                         void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ SwiGLU MLP
 * LoRA MLP with SwiGLU: e = lora(X; gate), u = lora(X; up), h = silu(e) * u,
 * out = lora(h; down) ("How Unsloth's FastLoRA Kernel ...", sections "Fused Forward
 * Pass Architecture" and "Activation Function Fusion").  bf16 only.  Forward: the
 * activation is formed in the epilogue of one GEMM that computes the gate and the up
 * projection of the same hidden units side by side, from its fp32 accumulators.
 * Backward: the down projection's input gradient dh is either followed by one
 * streaming pass over dh, e and u (four-wave route, hidden width a multiple of 256)
 * or has the SwiGLU backward in its epilogue (other shapes).
 *   X [M,K] (ldx); Wg, Wu [H,K]; Ag, Au [r,K]; Bg, Bu [H,r]; Wd [K,H]; Ad [r,H];
 *   Bd [K,r].  Out [M,K] (ldout).  Saved for the backward: E_save, Gu_save, H_save
 *   [M,H] (bf16) and U_save [M,3r] fp32 = [X.Ag^T | X.Au^T | H.Ad^T].  All required.
 *   Limits: K and H multiples of 64, r a multiple of 8 and at most 64.
 */
int swiglu_lora_mlp_fwd(int M, int K, int H, int r, float s_gate, float s_up, float s_down,
                        const void* X, int ldx, const void* Wg, const void* Ag, const void* Bg,
                        const void* Wu, const void* Au, const void* Bu,
                        const void* Wd, const void* Ad, const void* Bd,
                        void* Out, int ldout, void* E_save, void* Gu_save, void* H_save, float* U_save,
                        void* ws, size_t ws_bytes, void* stream);

/* Backward of the SwiGLU LoRA MLP (weights frozen, factor gradients pre-scaled by
 * each adapter's s; "How Unsloth's FastLoRA Kernel ...", section "Custom Backward
 * Pass Implementation").
 *   dH = dOut.Wd + s_d.(dOut.Bd).Ad;  dE = dH (.) u (.) silu'(e);  dU = dH (.) silu(e);
 *   dX = dE.Wg + dU.Wu + s_g.(dE.Bg).Ag + s_u.(dU.Bu).Au; factor gradients as in
 *   lora_linear_bwd for each projection.  dOut [M,K] (lddout), X (ldx); dX [M,K]
 *   bf16 (lddx) or NULL; dAg, dAu [r,K], dBg, dBu [H,r], dAd [r,H], dBd [K,r] fp32. */
int swiglu_lora_mlp_bwd(int M, int K, int H, int r, float s_gate, float s_up, float s_down,
                        const void* dOut, int lddout, const void* X, int ldx,
                        const void* Wg, const void* Ag, const void* Bg,
                        const void* Wu, const void* Au, const void* Bu,
                        const void* Wd, const void* Ad, const void* Bd,
                        const void* E_saved, const void* Gu_saved, const void* H_saved,
                        const float* U_saved,
                        void* dX, int lddx, float* dAg, float* dBg, float* dAu, float* dBu,
                        float* dAd, float* dBd,
                        void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ GeGLU MLP
 * The LoRA MLP with the GeGLU activation: h = gelu(e) * u with gelu(e) = e . Phi(e), Phi the
 * standard normal distribution function (approximate = 0), or its tanh form
 * 0.5 e (1 + tanh(sqrt(2/pi) (e + 0.044715 e^3))) (approximate = 1) ("How Unsloth's FastLoRA
 * Kernel ...", sections "Activation Function Fusion" and "Fused Forward Pass Architecture":
 * the LoRA update injected with the SwiGLU and GeGLU activations computed in the same
 * kernels).  Arguments, outputs, saved tensors, limits and routes as for the SwiGLU MLP;
 * approximate other than 0 or 1 is LDL_E_INVAL. */
int geglu_lora_mlp_fwd(int M, int K, int H, int r, float s_gate, float s_up, float s_down, int approximate,
                       const void* X, int ldx, const void* Wg, const void* Ag, const void* Bg,
                       const void* Wu, const void* Au, const void* Bu,
                       const void* Wd, const void* Ad, const void* Bd,
                       void* Out, int ldout, void* E_save, void* Gu_save, void* H_save, float* U_save,
                       void* ws, size_t ws_bytes, void* stream);

/* Backward of the GeGLU LoRA MLP: dE = dH (.) u (.) gelu'(e), dU = dH (.) gelu(e), the rest as
 * swiglu_lora_mlp_bwd. */
int geglu_lora_mlp_bwd(int M, int K, int H, int r, float s_gate, float s_up, float s_down, int approximate,
                       const void* dOut, int lddout, const void* X, int ldx,
                       const void* Wg, const void* Ag, const void* Bg,
                       const void* Wu, const void* Au, const void* Bu,
                       const void* Wd, const void* Ad, const void* Bd,
                       const void* E_saved, const void* Gu_saved, const void* H_saved,
                       const float* U_saved,
                       void* dX, int lddx, float* dAg, float* dBg, float* dAu, float* dBu,
                       float* dAd, float* dBd,
                       void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ W8A8
 * int8 weight x int8 activation base with per-row (activation) and per-column
 * (weight) dequant scales and the rank-tiled LoRA epilogue; the int32 product is
 * never stored ("nunchaku-style kernel fusion - 20-30% faster training",
 * LoRA-epilogue commit, the comment on activations and the unification commit).
 * Quantisation is symmetric with divisor 127: scale = absmax / 127 (fp32),
 * code = clamp(rint(x / scale), -127, 127) with the quotient in fp32 and ties to
 * even; a zero row has scale 0 and codes 0.
 */

/* Per-output-channel weight quantisation, once per frozen W0 [N,K] (row stride ldw;
 * dtype of W0: LDL_F32 or LDL_BF16): Wq [N,K] int8 (dense), sw [N] fp32. */
int w8a8_quantize_weight(int N, int K, int dtype, const void* W0, int ldw, int8_t* Wq, float* sw, void* stream);

/* Per-row activation quantisation: Xq [M,K] int8 (dense), sx [M] fp32 from bf16 X (ldx). */
int w8a8_quantize_rows(int M, int K, const void* X, int ldx, int8_t* Xq, float* sx, void* stream);

/* Raw int32 product C = Xq.Wq^T (the "raw product" epilogue of the 8-bit core).
 * Xq [M,K] (ldxq), Wq [N,K] (ldwq), C [M,N] int32 (ldc).  Exact. */
int int8_gemm_raw(int M, int N, int K, const int8_t* Xq, int ldxq, const int8_t* Wq, int ldwq,
                  int32_t* C, int ldc, void* stream);

/*   Y = (Xq.Wq^T) . sx[m] . sw[n] + s.(X.A^T).B^T (+ bias), Xq / sx quantised from X
 *   in the call.  X [M,K] bf16 (ldx); Wq [N,K] int8 (ldw); sw [N] fp32; A, B, bias
 *   bf16.  Y [M,N] bf16 (ldy).  Xq_save [M,K] int8 (dense) or NULL, sx_save [M] fp32
 *   or NULL (both NULL or both set), U_save [M,r] fp32 (ldu) or NULL.  The LoRA
 *   branch sees X, not Xq. */
int w8a8_lora_linear_fwd(int M, int N, int K, int r, float s,
                         const void* X, int ldx, const int8_t* Wq, int ldw, const float* sw,
                         const void* A, const void* B, const void* bias,
                         void* Y, int ldy, int8_t* Xq_save, float* sx_save, float* U_save, int ldu,
                         void* ws, size_t ws_bytes, void* stream);

/* Straight-through backward: dX = dY.(diag(sw).Wq + s.B.A) (the dequantised weight,
 * bf16 MFMA), dA = s.(dY.B)^T.X, dB = s.dY^T.U.  dY [M,N] (lddy), X (ldx), Wq (ldw);
 * dX [M,K] bf16 (lddx) or NULL; dA [r,K], dB [N,r] fp32; U_saved [M,r] fp32 (ldu) or
 * NULL (recomputed). */
int w8a8_lora_linear_bwd(int M, int N, int K, int r, float s,
                         const void* dY, int lddy, const void* X, int ldx, const int8_t* Wq, int ldw,
                         const float* sw, const void* A, const void* B, const float* U_saved, int ldu,
                         void* dX, int lddx, float* dA, float* dB,
                         void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ 8-bit float base
 * The same layer over an e4m3 base ("nunchaku-style kernel fusion ...", LoRA-epilogue commit:
 * the per-axis quantiser serves both 8-bit dtypes; MXFP8 commit: the block-scaled 8-bit float
 * instruction with unit block scales computes the plain product at the full 8-bit rate).
 * Codes are e4m3 bytes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, largest
 * finite 448) passed as uint8.  Quantisation is symmetric per row: scale = absmax / 448
 * (fp32), code = e4m3 rounding (nearest, ties to even) of the fp32 quotient x / scale
 * clamped to +-448; a zero row has scale 0 and codes 0.  The product runs on
 * v_mfma_scale_f32_32x32x64_f8f6f4 with every block scale 1.0 (fp32 accumulation; the
 * instruction's internal sums keep about 17 bits relative to the largest term).
 * Arguments, outputs, workspace (ldl_workspace_bytes with LDL_OP_W8A8_FWD / _BWD) and the
 * straight-through backward as for the int8 base, with uint8 codes; the forward also
 * needs N a multiple of 128 and r a multiple of 8 with r <= 64. */
int fp8_quantize_weight(int N, int K, int dtype, const void* W0, int ldw, uint8_t* Wq, float* sw, void* stream);
int fp8_quantize_rows(int M, int K, const void* X, int ldx, uint8_t* Xq, float* sx, void* stream);
int fp8_lora_linear_fwd(int M, int N, int K, int r, float s,
                        const void* X, int ldx, const uint8_t* Wq, int ldw, const float* sw,
                        const void* A, const void* B, const void* bias,
                        void* Y, int ldy, uint8_t* Xq_save, float* sx_save, float* U_save, int ldu,
                        void* ws, size_t ws_bytes, void* stream);
int fp8_lora_linear_bwd(int M, int N, int K, int r, float s,
                        const void* dY, int lddy, const void* X, int ldx, const uint8_t* Wq, int ldw,
                        const float* sw, const void* A, const void* B, const float* U_saved, int ldu,
                        void* dX, int lddx, float* dA, float* dB,
                        void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LORA_DORA_LINEAR_H */
