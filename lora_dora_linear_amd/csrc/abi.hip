// C entry points: host-side validation, workspace layout and the launch
// sequence of each layer.  Nothing here allocates, synchronises or touches an
// output before every argument has been checked.
#include <cstring>
#include <mutex>

#include "../../include/lora_dora_linear.h"
#include "internal.hpp"

using namespace ldl;

namespace {

// Device-resident scratch for lora_linear_bwd_noalloc: callers that cannot allocate (HIP graph
// capture, tight serving loops) pass no workspace.  One copy per device, held until the process
// ends.  Host code never uses the array's name as an address: each device's copy is looked up
// once with hipGetSymbolAddress (with that device current) and that pointer is passed on.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The calling thread's current device's copy of the scratch array, or nullptr on a HIP error.
void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

int g_fwd_fused = 0;   // LDL_TUNE_FWD_FUSED_DOWNPROJ
int g_prepack = 1;     // LDL_TUNE_PREPACK

// Kernel timing hook (ldl_set_kernel_events).
struct EventHook {
  void** start = nullptr;
  void** stop = nullptr;
  int count = 0;
  int next = 0;
};
constexpr int kHooks = 3;
EventHook g_hooks[kHooks];

// Launch a GEMM; when a hook is set for `hook_kind`, bracket it with the caller's events.
hipError_t gemm_timed(int hook_kind, GemmKind kind, const GemmParams& p, hipStream_t st) {
  bool rec = false;
  const hipError_t e0 = hook_start(hook_kind, st, &rec);
  if (e0 != hipSuccess) return e0;
  const hipError_t e = launch_gemm(kind, p, st);
  if (e != hipSuccess) return e;
  return hook_stop(hook_kind, st, rec);
}

constexpr size_t kAlign = 256;
constexpr size_t kMaxBytes = (size_t)1 << 31;   // buffer resources take 31-bit sizes

// Bump allocator over the caller's workspace; with base == nullptr it only sizes.
struct Bump {
  char* base;
  size_t off = 0;
  explicit Bump(void* b) : base(static_cast<char*>(b)) {}
  template <class T>
  T* take(size_t count) {
    off = (off + kAlign - 1) / kAlign * kAlign;
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
  size_t size() const { return (off + kAlign - 1) / kAlign * kAlign; }
};

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
inline bool al(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p && !aligned16(p)) return false;
  return true;
}
inline bool nonnull(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!p) return false;
  return true;
}
inline bool small(size_t rows, size_t cols, size_t elt) { return rows * cols * elt < kMaxBytes; }
inline hipStream_t S(void* st) { return static_cast<hipStream_t>(st); }

#define LDL_TRY(expr)                         \
  do {                                        \
    if ((expr) != hipSuccess) return LDL_E_HIP; \
  } while (0)

// ------------------------------------------------------------------ workspace plans
// From this many rows the 8-bit backward dequantises the weight into a bf16 copy once per call
// and runs the plain four-wave input-gradient product on it (the copy pays for itself against
// widening the codes inside the product at every k-tile of every row tile).
constexpr int kDequantRows = 512;

struct LoraBwdWs {
  float* V; float* U; float* partB; float* csB; float* partA;
  uint32_t* pkB; uint32_t* pkA;    // packed S of the two column projections
  int nsB, msB, nsA, msA, rp;
};
LoraBwdWs plan_lora_bwd(Bump& b, int M, int N, int K, int r, bool need_u) {
  LoraBwdWs w{};
  w.rp = colproj_rp(r);
  // dB and dA share one launch; planned for 512 blocks each against 64-column tiles, which
  // the 128-column blocks of two halves make 256 blocks each (two per CU in all)
  colproj_plan(M, N, &w.nsB, &w.msB, 512);
  colproj_plan(M, K, &w.nsA, &w.msA, 512);
  w.V = b.take<float>((size_t)M * r);
  w.U = need_u ? b.take<float>((size_t)M * r) : nullptr;
  w.partB = b.take<float>((size_t)w.nsB * N * w.rp);
  w.csB = b.take<float>((size_t)w.nsB * N);
  w.partA = b.take<float>((size_t)w.nsA * K * w.rp);
  w.pkB = b.take<uint32_t>(colproj_spk_words(M, r));
  w.pkA = b.take<uint32_t>(colproj_spk_words(M, r));
  return w;
}

struct MergeBwdWs {
  float* Bf; float* part; uint32_t* pk;
  int ns, ms, rp;
};
MergeBwdWs plan_merge_bwd(Bump& b, int N, int K, int r) {
  MergeBwdWs w{};
  w.rp = colproj_rp(r);
  colproj_plan(N, K, &w.ns, &w.ms, 512);
  w.Bf = b.take<float>((size_t)N * r);
  w.part = b.take<float>((size_t)w.ns * K * w.rp);
  w.pk = b.take<uint32_t>(colproj_spk_words(N, r));
  return w;
}

// Column-scaled DoRA.  Forward: B as fp32, the split partials of Pc = B^T.W0 and
// Gc = B^T.B, U when not saved.  Backward: dXs (the gradient of the scaled input) when dX is
// not requested, the LoRA backward's own workspace, the partial column sums of dXs.X, dg,
// A.diag(w) as bf16 hi / lo, and T = [W0; A].(A.diag(w))^T.
struct DoraColsFwdWs {
  float* Bf; float* partP; float* partG; uint32_t* pkP; uint32_t* pkG; float* U;
  int nsP, msP, nsG, msG, rp;
};
DoraColsFwdWs plan_dora_cols_fwd(Bump& b, int M, int N, int K, int r) {
  DoraColsFwdWs w{};
  w.rp = colproj_rp(r);
  colproj_plan(N, K, &w.nsP, &w.msP, 512);
  colproj_plan(N, r, &w.nsG, &w.msG, 64);
  w.Bf = b.take<float>((size_t)N * r);
  w.partP = b.take<float>((size_t)w.nsP * K * w.rp);
  w.partG = b.take<float>((size_t)w.nsG * r * w.rp);
  w.pkP = b.take<uint32_t>(colproj_spk_words(N, r));
  w.pkG = b.take<uint32_t>(colproj_spk_words(N, r));
  w.U = b.take<float>((size_t)M * r);
  return w;
}

struct DoraColsBwdWs {
  uint16_t* dXs; void* lora; size_t lora_bytes; float* partD; float* csD; uint16_t* Aw; float* T;
  int nsD, msD;
};
DoraColsBwdWs plan_dora_cols_bwd(Bump& b, int M, int N, int K, int r) {
  DoraColsBwdWs w{};
  colproj_plan(M, K, &w.nsD, &w.msD, 512);
  w.dXs = b.take<uint16_t>((size_t)M * K);
  Bump lb(nullptr);
  plan_lora_bwd(lb, M, N, K, r, true);
  w.lora_bytes = lb.size();
  w.lora = b.take<uint8_t>(w.lora_bytes);
  w.partD = b.take<float>((size_t)w.nsD * K * 16);
  w.csD = b.take<float>((size_t)w.nsD * K);
  w.Aw = b.take<uint16_t>((size_t)2 * r * K);
  w.T = b.take<float>((size_t)(N + r) * 2 * r);
  return w;
}

struct DoraBwdWs {
  float* V; float* partT; float* cs; float* wB; float* partA; float* partQ; float* Qm;
  uint16_t* gW0; uint16_t* gB;     // diag(g).W0 [N, K] and diag(g).B [N, r] in bf16 (weight-sized)
  float* partbias; float* csbias;
  uint32_t* pkT; uint32_t* pkA; uint32_t* pkW; uint32_t* pkQ;
  int nsT, msT, nsA, msA, nsW, msW, nsQ, msQ, rp;
};
DoraBwdWs plan_dora_bwd(Bump& b, int M, int N, int K, int r) {
  DoraBwdWs w{};
  w.rp = colproj_rp(r);
  colproj_plan(M, N, &w.nsT, &w.msT);
  colproj_plan(M, K, &w.nsA, &w.msA);
  colproj_plan(N, K, &w.nsW, &w.msW);
  colproj_plan(N, r, &w.nsQ, &w.msQ);
  w.V = b.take<float>((size_t)M * r);
  w.partT = b.take<float>((size_t)w.nsT * N * w.rp);
  w.cs = b.take<float>((size_t)w.nsT * N);
  w.wB = b.take<float>((size_t)N * r);
  w.partA = b.take<float>((size_t)(w.nsA + w.nsW) * K * w.rp);
  w.partQ = b.take<float>((size_t)w.nsQ * r * w.rp);
  w.Qm = b.take<float>((size_t)r * r);
  w.partbias = b.take<float>((size_t)w.nsT * N * 16);
  w.csbias = b.take<float>((size_t)w.nsT * N);
  w.gW0 = b.take<uint16_t>((size_t)N * K);
  w.gB = b.take<uint16_t>((size_t)N * r);
  w.pkT = b.take<uint32_t>(colproj_spk_words(M, r));
  w.pkA = b.take<uint32_t>(colproj_spk_words(M, r));
  w.pkW = b.take<uint32_t>(colproj_spk_words(N, r));
  w.pkQ = b.take<uint32_t>(colproj_spk_words(N, r));
  return w;
}

struct MlpBwdWs {
  float* Vd; float* Vgu; uint16_t* dEGu;
  float* partDd; float* partAd; float* partBg; float* partBu; float* partAgu;
  uint32_t* pkDd; uint32_t* pkAd; uint32_t* pkBg; uint32_t* pkBu; uint32_t* pkAgu;
  int nsDd, msDd, nsAd, msAd, nsBg, msBg, nsAgu, msAgu, rp, rp2;
  bool agu_split;                  // dAg, dAu as two rank-r jobs (2r pads to 128)
};
MlpBwdWs plan_mlp_bwd(Bump& b, int M, int K, int H, int r) {
  MlpBwdWs w{};
  w.rp = colproj_rp(r);
  w.rp2 = colproj_rp(2 * r);
  colproj_plan(M, K, &w.nsDd, &w.msDd);
  // dAd (H columns) shares its launch with dBd (K columns): more row splits for the wide
  // job keep its heavy blocks from landing one or two to a CU
  colproj_plan(M, H, &w.nsAd, &w.msAd, 1024);
  colproj_plan(M, H, &w.nsBg, &w.msBg);
  // rank 2r padded to 128 runs on the register-transposing kernel; two rank-r jobs (same
  // partial and packed-factor sizes) run on the streamed one instead
  w.agu_split = w.rp2 > 64;
  colproj_plan(M, K, &w.nsAgu, &w.msAgu, w.agu_split ? 256 : 512);
  w.Vd = b.take<float>((size_t)M * r);
  w.Vgu = b.take<float>((size_t)M * 2 * r);
  w.dEGu = b.take<uint16_t>((size_t)M * 2 * H);
  w.partDd = b.take<float>((size_t)w.nsDd * K * w.rp);
  w.partAd = b.take<float>((size_t)w.nsAd * H * w.rp);
  w.partBg = b.take<float>((size_t)w.nsBg * H * w.rp);
  w.partBu = b.take<float>((size_t)w.nsBg * H * w.rp);
  w.partAgu = b.take<float>((size_t)w.nsAgu * K * w.rp2);
  w.pkDd = b.take<uint32_t>(colproj_spk_words(M, r));
  w.pkAd = b.take<uint32_t>(colproj_spk_words(M, r));
  w.pkBg = b.take<uint32_t>(colproj_spk_words(M, r));
  w.pkBu = b.take<uint32_t>(colproj_spk_words(M, r));
  w.pkAgu = b.take<uint32_t>(colproj_spk_words(M, 2 * r));
  return w;
}

// ------------------------------------------------------------------ small launch helpers
GemmParams gp0() {
  GemmParams p;
  std::memset(&p, 0, sizeof(p));
  p.s_epi = 1.f;
  return p;
}

hipError_t rowproj(int M, int K, int R, const void* P, int ldp, const void* q0, const void* q1, int R0, int ldq,
                   float* out, int ldo, float scale, hipStream_t st) {
  RowProjParams p;
  p.M = M; p.K = K; p.R = R; p.R0 = R0;
  p.P = static_cast<const uint16_t*>(P); p.ldp = ldp;
  p.q0 = static_cast<const uint16_t*>(q0); p.q1 = static_cast<const uint16_t*>(q1 ? q1 : q0); p.ldq = ldq;
  p.P1 = nullptr; p.p_split = M; p.ldp1 = ldp;
  p.q_trans = 0; p.q_kscale = nullptr;
  p.out = out; p.ldo = ldo; p.scale = scale;
  p.P2 = nullptr; p.p_split2 = p.M; p.ldp2 = ldp; p.out2 = nullptr; p.ldo2 = 0;
  p.pk = nullptr; p.pk_rp = 0; p.pk_scale = 1.f;
  return launch_rowproj(p, st);
}

// rowproj over the rows of P (leading dim ldp) followed by the rows of P1 (leading dim ldp1)
hipError_t rowproj2(int M0, int M1, int K, int R, const void* P, int ldp, const void* P1, int ldp1, const void* q0,
                    int ldq, float* out, int ldo, float scale, hipStream_t st) {
  RowProjParams p;
  p.M = M0 + M1; p.K = K; p.R = R; p.R0 = R;
  p.P = static_cast<const uint16_t*>(P); p.ldp = ldp;
  p.P1 = static_cast<const uint16_t*>(P1); p.p_split = M0; p.ldp1 = ldp1;
  p.q0 = p.q1 = static_cast<const uint16_t*>(q0); p.ldq = ldq;
  p.q_trans = 0; p.q_kscale = nullptr;
  p.out = out; p.ldo = ldo; p.scale = scale;
  p.P2 = nullptr; p.p_split2 = p.M; p.ldp2 = ldp; p.out2 = nullptr; p.ldo2 = 0;
  p.pk = nullptr; p.pk_rp = 0; p.pk_scale = 1.f;
  return launch_rowproj(p, st);
}

// rowproj2 over the rows of P then P1 into out, and the rows of P2 against the same Q into out2, in
// one launch when the streamed kernel takes the three segments; otherwise two launches
hipError_t rowproj3(int M0, int M1, int M2, int K, int R, const void* P, int ldp, const void* P1, int ldp1,
                    const void* P2, int ldp2, const void* q0, int ldq, float* out, int ldo, float* out2, int ldo2,
                    hipStream_t st) {
  RowProjParams p;
  p.M = M0 + M1 + M2; p.K = K; p.R = R; p.R0 = R;
  p.P = static_cast<const uint16_t*>(P); p.ldp = ldp;
  p.P1 = static_cast<const uint16_t*>(P1); p.p_split = M0; p.ldp1 = ldp1;
  p.q0 = p.q1 = static_cast<const uint16_t*>(q0); p.ldq = ldq;
  p.q_trans = 0; p.q_kscale = nullptr;
  p.out = out; p.ldo = ldo; p.scale = 1.f;
  p.P2 = static_cast<const uint16_t*>(P2); p.p_split2 = M0 + M1; p.ldp2 = ldp2; p.out2 = out2; p.ldo2 = ldo2;
  p.pk = nullptr; p.pk_rp = 0; p.pk_scale = 1.f;
  if (M2 > 0 && rowproj_three_ok(p)) return launch_rowproj(p, st);
  const hipError_t e = rowproj2(M0, M1, K, R, P, ldp, P1, ldp1, q0, ldq, out, ldo, 1.f, st);
  if (e != hipSuccess || M2 == 0) return e;
  return rowproj(M2, K, R, P2, ldp2, q0, nullptr, R, ldq, out2, ldo2, 1.f, st);
}

// The parameters of a row projection against a transposed Q: out[m, j] = scale * sum_k P[m, k]
// * bf16(Bq[k, j] * kscale[k]) with Bq a [K, R] matrix of leading dim ldb (kscale optional)
static RowProjParams rowproj_t_params(int M, int K, int R, const void* P, int ldp, const void* Bq, int ldb,
                                      const float* kscale, float* out, int ldo, float scale) {
  RowProjParams p;
  p.M = M; p.K = K; p.R = R; p.R0 = R;
  p.P = static_cast<const uint16_t*>(P); p.ldp = ldp;
  p.P1 = nullptr; p.p_split = M; p.ldp1 = ldp;
  p.q0 = p.q1 = static_cast<const uint16_t*>(Bq); p.ldq = ldb;
  p.q_trans = 1; p.q_kscale = kscale;
  p.out = out; p.ldo = ldo; p.scale = scale;
  p.P2 = nullptr; p.p_split2 = p.M; p.ldp2 = ldp; p.out2 = nullptr; p.ldo2 = 0;
  p.pk = nullptr; p.pk_rp = 0; p.pk_scale = 1.f;
  return p;
}

hipError_t rowproj_t(int M, int K, int R, const void* P, int ldp, const void* Bq, int ldb, const float* kscale,
                     float* out, int ldo, float scale, hipStream_t st) {
  return launch_rowproj(rowproj_t_params(M, K, R, P, ldp, Bq, ldb, kscale, out, ldo, scale), st);
}

// rowproj_t with no k-scale that also writes pk_scale * out packed for a column projection of
// rank padding pk_rp, where the streamed kernel takes it (*packed says whether it did)
hipError_t rowproj_t_pk(int M, int K, int R, const void* P, int ldp, const void* Bq, int ldb, float* out, int ldo,
                        float scale, uint16_t* pk, int pk_rp, float pk_scale, bool* packed, hipStream_t st) {
  RowProjParams p = rowproj_t_params(M, K, R, P, ldp, Bq, ldb, nullptr, out, ldo, scale);
  p.pk = pk; p.pk_rp = pk_rp; p.pk_scale = pk_scale;
  *packed = pk != nullptr && rowproj_packs(p);
  if (!*packed) p.pk = nullptr;
  return launch_rowproj(p, st);
}

ColProjParams cpp(int M, int C, int R, const void* X, int ldx, const float* Sm, int lds, float s_in,
                  const void* Z, int ldz, int mode, int msplit, float* part, float* cspart) {
  ColProjParams p;
  p.M = M; p.C = C; p.R = R;
  p.X = static_cast<const uint16_t*>(X); p.ldx = ldx;
  p.S = Sm; p.lds = lds; p.s_in = s_in;
  p.Z = static_cast<const uint16_t*>(Z); p.ldz = ldz; p.colsum_mode = mode;
  p.msplit = msplit; p.part = part; p.cspart = cspart;
  p.spk = nullptr;
  p.S16 = nullptr;
  p.spk_ready = false;
  return p;
}

// the same job with its packed-S workspace
ColProjParams pk(ColProjParams p, uint32_t* spk) {
  p.spk = spk;
  return p;
}

// the same job reading its S operand in bf16 (row stride unchanged)
ColProjParams s16(ColProjParams p, const void* S16) {
  p.S = nullptr;
  p.S16 = static_cast<const uint16_t*>(S16);
  return p;
}

hipError_t colproj(int M, int C, int R, const void* X, int ldx, const float* Sm, int lds, float s_in,
                   const void* Z, int ldz, int mode, int nsplit, int msplit, float* part, float* cspart,
                   hipStream_t st, uint32_t* spk = nullptr) {
  return launch_colproj(pk(cpp(M, C, R, X, ldx, Sm, lds, s_in, Z, ldz, mode, msplit, part, cspart), spk), nsplit,
                        st);
}

// out[rows, cols] = alpha * sum over nsplit partials (+ row scale) (+ addend)
ReduceParams rdp(int rows, int cols, const float* part, size_t pstride, int nsplit, int rp, bool trans, float alpha,
                 float* out, int ldo, const float* rowscale = nullptr,
                 const float* Qm = nullptr, int ldq = 0, int rq = 0, const void* Am = nullptr, int lda = 0,
                 float alpha2 = 0.f) {
  ReduceParams p;
  p.rows = rows; p.cols = cols; p.part = part; p.pstride = pstride; p.nsplit = nsplit; p.rp = rp;
  p.trans = trans ? 1 : 0; p.alpha = alpha; p.rowscale = rowscale;
  p.Qm = Qm; p.ldq = ldq; p.rq = rq; p.Am = static_cast<const uint16_t*>(Am); p.lda = lda; p.alpha2 = alpha2;
  p.out = out; p.ldo = ldo;
  return p;
}

hipError_t reduce(int rows, int cols, const float* part, size_t pstride, int nsplit, int rp, bool trans, float alpha,
                  float* out, int ldo, hipStream_t st, const float* rowscale = nullptr,
                  const float* Qm = nullptr, int ldq = 0, int rq = 0, const void* Am = nullptr, int lda = 0,
                  float alpha2 = 0.f) {
  return launch_reduce(rdp(rows, cols, part, pstride, nsplit, rp, trans, alpha, out, ldo, rowscale, Qm, ldq, rq, Am,
                           lda, alpha2), st);
}

hipError_t zero(float* p, size_t n, hipStream_t st) { return p ? launch_fill_zero(p, n, st) : hipSuccess; }

// Common shape checks of the bf16 layer: N, K multiples of 64, r in [1, 128], sizes < 2 GiB.
int check_bf16_layer(int M, int N, int K, int r) {
  if (M < 0 || N <= 0 || K <= 0 || r <= 0) return LDL_E_INVAL;
  if (r > 128 || N % 64 || K % 64) return LDL_E_UNSUPPORTED;
  if (!small(M + 256, K, 2) || !small(N, K, 2) || !small(M + 256, N, 2) || !small(M, 2 * r, 4)) return LDL_E_UNSUPPORTED;
  return LDL_OK;
}

// Leading dimension (elements) of a row-major operand with `cols` columns: 0 selects `cols`.
// Below `cols` is an invalid argument; rows that are not a whole number of `mult`-element
// groups (16 bytes for the bf16 / int8 kernels, 4 fp32 values for U) are unsupported.
int fix_ld(int& ld, int cols, int mult) {
  if (ld == 0) ld = cols;
  if (ld < cols) return LDL_E_INVAL;
  return ld % mult == 0 ? LDL_OK : LDL_E_UNSUPPORTED;
}

#define LDL_LD(ld, cols, mult)                      \
  do {                                              \
    const int e_ld = fix_ld((ld), (cols), (mult));  \
    if (e_ld != LDL_OK) return e_ld;                \
  } while (0)

// Row-major operands of `rows` rows with leading dimension ld stay below 2 GiB (buffer
// resources take 31-bit sizes; 256 rows of margin for the row tiles past the end).
inline bool fits(int rows, int ld, size_t elt) { return small((size_t)rows + 256, (size_t)ld, elt); }

// ------------------------------------------------------------------ fp32 path
hipError_t f32(int M, int N, int K, const float* A, long sam, long sak, const float* B, long sbk, long sbn,
               float* C, int ldc, float alpha, float beta, const float* bias, hipStream_t st) {
  F32GemmParams p;
  p.M = M; p.N = N; p.K = K; p.A = A; p.sam = sam; p.sak = sak; p.B = B; p.sbk = sbk; p.sbn = sbn;
  p.C = C; p.ldc = ldc; p.alpha = alpha; p.beta = beta; p.bias = bias;
  return launch_f32_gemm(p, st);
}

}  // namespace

// Start / stop of a timed launch: records the caller's events while the hook is set
hipError_t ldl::hook_start(int hook_kind, hipStream_t st, bool* rec) {
  EventHook* h = (hook_kind >= 0 && hook_kind < kHooks) ? &g_hooks[hook_kind] : nullptr;
  *rec = h && h->count > 0 && h->next < h->count;
  return *rec ? hipEventRecord(static_cast<hipEvent_t>(h->start[h->next]), st) : hipSuccess;
}
hipError_t ldl::hook_stop(int hook_kind, hipStream_t st, bool rec) {
  if (!rec) return hipSuccess;
  EventHook* h = &g_hooks[hook_kind];
  const hipError_t e = hipEventRecord(static_cast<hipEvent_t>(h->stop[h->next]), st);
  ++h->next;
  return e;
}


extern "C" {

const char* ldl_status_string(int status) {
  switch (status) {
    case LDL_OK: return "ok";
    case LDL_E_INVAL: return "invalid argument (null pointer, negative size or bad dtype)";
    case LDL_E_UNSUPPORTED: return "unsupported shape or alignment for these kernels";
    case LDL_E_WORKSPACE: return "workspace too small";
    case LDL_E_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int ldl_version(void) { return 100; }

int ldl_set_kernel_events(int kind, void** start_events, void** stop_events, int count) {
  if (kind < 0 || kind >= kHooks || count < 0) return LDL_E_INVAL;
  if (count > 0 && (!start_events || !stop_events)) return LDL_E_INVAL;
  g_hooks[kind].start = count > 0 ? start_events : nullptr;
  g_hooks[kind].stop = count > 0 ? stop_events : nullptr;
  g_hooks[kind].count = count > 0 ? count : 0;
  g_hooks[kind].next = 0;
  return LDL_OK;
}

int ldl_set_tuning(int key, int value) {
  if (key == LDL_TUNE_FWD_FUSED_DOWNPROJ && (value == 0 || value == 1)) {
    g_fwd_fused = value;
    return LDL_OK;
  }
  if (key == LDL_TUNE_GEMM_4WAVE && value >= 0 && value <= 2) {
    g_gemm_4wave = value;
    return LDL_OK;
  }
  if (key == LDL_TUNE_ROWSTREAM_32 && value >= 0 && value <= 2) {
    g_rowstream32 = value;
    return LDL_OK;
  }
  if (key == LDL_TUNE_PREPACK && (value == 0 || value == 1)) {
    g_prepack = value;
    return LDL_OK;
  }

  return LDL_E_INVAL;
}

size_t dora_state_floats(int N, int r) {
  if (N <= 0 || r <= 0) return 0;
  return (size_t)2 * N + (size_t)N * r + (size_t)r * r;
}

}  // extern "C"

// The workspace an op needs (without the split-reduction partials below)
static size_t ws_base(int op, int M, int N, int K, int r, int dtype) {
  if (M < 0 || N <= 0 || K <= 0 || r <= 0) return 0;
  Bump b(nullptr);
  switch (op) {
    case LDL_OP_LORA_FWD:
    case LDL_OP_W8A8_FWD:
      b.take<float>((size_t)M * r);            // U when not saved by the caller
      if (op == LDL_OP_W8A8_FWD) { b.take<int8_t>((size_t)M * K); b.take<float>((size_t)M); }
      break;
    case LDL_OP_LORA_BWD:
    case LDL_OP_W8A8_BWD:
      if (dtype == LDL_F32 && op == LDL_OP_LORA_BWD) { b.take<float>((size_t)M * r); b.take<float>((size_t)M * r); }
      else plan_lora_bwd(b, M, N, K, r, true);
      if (op == LDL_OP_W8A8_BWD && M >= kDequantRows) b.take<uint16_t>((size_t)N * K);   // the dequantised weight
      break;
    case LDL_OP_DORA_FWD:
      break;
    case LDL_OP_DORA_BWD:
      plan_dora_bwd(b, M, N, K, r);
      break;
    case LDL_OP_SWIGLU_FWD:
      break;
    case LDL_OP_SWIGLU_BWD:
      plan_mlp_bwd(b, M, K, N, r);
      break;
    case LDL_OP_MERGE_BWD:   // M unused; N x K weight
      if (dtype != LDL_F32) plan_merge_bwd(b, N, K, r);
      break;
    case LDL_OP_DORA_COLS_FWD:
      plan_dora_cols_fwd(b, M, N, K, r);
      break;
    case LDL_OP_DORA_COLS_BWD:
      plan_dora_cols_bwd(b, M, N, K, r);
      break;
    default:
      return 0;
  }
  return b.size();
}

// Optional fp32 partials of the split reduction of the op's plain four-wave product (the
// tiles past its last full round; 0 when the shape has none): [M, N] forward outputs, [M, K]
// input gradients.  Calls given less workspace than base + this run without the split.
static size_t ws_split(int op, int M, int N, int K, int dtype) {
  if (dtype == LDL_F32) return 0;
  switch (op) {
    case LDL_OP_LORA_FWD:
    case LDL_OP_W8A8_FWD: return gemm_split_bytes(M, N);
    case LDL_OP_LORA_BWD: return gemm_split_bytes(M, K);
    case LDL_OP_W8A8_BWD: return M >= kDequantRows ? gemm_split_bytes(M, K) : 0;
    default: return 0;
  }
}

// The split partials carved from the rest of the workspace, or nullptr if they do not fit.
static float* split_part(Bump& wb, void* ws, size_t ws_bytes, size_t need) {
  if (need == 0 || ws == nullptr) return nullptr;
  if (wb.size() + need > ws_bytes) return nullptr;
  return wb.take<float>(need / sizeof(float));
}

extern "C" {

size_t ldl_workspace_bytes(int op, int M, int N, int K, int r, int dtype) {
  const size_t base = ws_base(op, M, N, K, r, dtype);
  const size_t extra = (M < 0 || N <= 0 || K <= 0 || r <= 0) ? 0 : ws_split(op, M, N, K, dtype);
  return extra ? (base + kAlign - 1) / kAlign * kAlign + extra : base;
}

// =========================================================================== LoRA
int lora_linear_fwd(int M, int N, int K, int r, float s, int dtype, const void* X, int ldx, const void* W0, int ldw,
                    const void* A, const void* B, const void* bias, void* Y, int ldy, float* U_save, int ldu,
                    void* ws, size_t ws_bytes, void* stream) {
  if (!nonnull({W0, A, B}) || (M > 0 && !nonnull({X, Y}))) return LDL_E_INVAL;
  if (dtype != LDL_F32 && dtype != LDL_BF16) return LDL_E_INVAL;
  if (M < 0 || N <= 0 || K <= 0 || r <= 0) return LDL_E_INVAL;
  const int g = dtype == LDL_BF16 ? 8 : 1, gu = dtype == LDL_BF16 ? 4 : 1;
  LDL_LD(ldx, K, g); LDL_LD(ldw, K, g); LDL_LD(ldy, N, g); LDL_LD(ldu, r, gu);
  if (!al({X, W0, A, B, bias, Y, U_save, ws})) return LDL_E_UNSUPPORTED;
  const size_t e = dtype == LDL_BF16 ? 2 : 4;
  if (!fits(M, ldx, e) || !fits(N, ldw, e) || !fits(M, ldy, e) || !fits(M, ldu, 4)) return LDL_E_UNSUPPORTED;
  if (ws_base(LDL_OP_LORA_FWD, M, N, K, r, dtype) > ws_bytes && !U_save) return LDL_E_WORKSPACE;
  if (ws_bytes > 0 && !ws) return LDL_E_INVAL;
  const hipStream_t st = S(stream);
  Bump wb(ws);
  float* U = U_save ? U_save : wb.take<float>((size_t)M * r);
  const int lu = U_save ? ldu : r;
  if (M == 0) return LDL_OK;

  if (dtype == LDL_F32) {
    const float *x = (const float*)X, *w = (const float*)W0, *a = (const float*)A, *bb = (const float*)B;
    if (f32_small_ok(M, N, K, r) && ldx % 4 == 0 && ldw % 4 == 0) {
      LDL_TRY(launch_f32_small_fwd(M, N, K, r, s, x, ldx, w, ldw, a, bb, (const float*)bias, (float*)Y, ldy,
                                   U_save, ldu, st));
      return LDL_OK;
    }
    LDL_TRY(f32(M, r, K, x, ldx, 1, a, 1, K, U, lu, 1.f, 0.f, nullptr, st));
    LDL_TRY(f32(M, N, K, x, ldx, 1, w, 1, ldw, (float*)Y, ldy, 1.f, 0.f, (const float*)bias, st));
    LDL_TRY(f32(M, N, r, U, lu, 1, bb, 1, r, (float*)Y, ldy, s, 1.f, nullptr, st));
    return LDL_OK;
  }

  const int chk = check_bf16_layer(M, N, K, r);
  if (chk != LDL_OK) return chk;
  GemmParams p = gp0();
  p.M = M; p.N = N; p.K = K;
  p.a = X; p.lda = ldx; p.b0 = W0; p.ldb = ldw; p.kseg = K;
  p.r_epi = r; p.s_epi = s; p.e0 = B; p.e1 = B; p.e_ldn = r; p.e_ldj = 1; p.e_jsplit = r;
  p.bias = bias; p.out = Y; p.ldo = ldy;
  p.part = split_part(wb, ws, ws_bytes, ws_split(LDL_OP_LORA_FWD, M, N, K, dtype));
  if (g_fwd_fused && r <= 64 && N % 128 == 0) {
    p.side = A; p.r_side = r; p.side_save = U_save; p.ld_side_save = ldu;
    LDL_TRY(gemm_timed(0, GK_NT_FUSED, p, st));
    return LDL_OK;
  }
  LDL_TRY(rowproj(M, K, r, X, ldx, A, nullptr, r, K, U, lu, 1.f, st));
  p.S = U; p.ld_s = lu;
  LDL_TRY(gemm_timed(0, GK_NT_PLAIN, p, st));
  return LDL_OK;
}

int lora_linear_bwd(int M, int N, int K, int r, float s, int dtype, const void* dY, int lddy, const void* X, int ldx,
                    const void* W0, int ldw, const void* A, const void* B, const float* U_saved, int ldu, void* dX,
                    int lddx, float* dA, float* dB, float* dbias, void* ws, size_t ws_bytes, void* stream) {
  if (!nonnull({W0, A, B, dA, dB}) || (M > 0 && !nonnull({dY, X}))) return LDL_E_INVAL;
  if (dtype != LDL_F32 && dtype != LDL_BF16) return LDL_E_INVAL;
  if (M < 0 || N <= 0 || K <= 0 || r <= 0) return LDL_E_INVAL;
  const int g = dtype == LDL_BF16 ? 8 : 1, gu = dtype == LDL_BF16 ? 4 : 1;
  LDL_LD(lddy, N, g); LDL_LD(ldx, K, g); LDL_LD(ldw, K, g); LDL_LD(ldu, r, gu); LDL_LD(lddx, K, g);
  if (!al({dY, X, W0, A, B, U_saved, dX, dA, dB, dbias, ws})) return LDL_E_UNSUPPORTED;
  const size_t e = dtype == LDL_BF16 ? 2 : 4;
  if (!fits(M, lddy, e) || !fits(M, ldx, e) || !fits(N, ldw, e) || !fits(M, ldu, 4) || !fits(M, lddx, e))
    return LDL_E_UNSUPPORTED;
  if (dtype == LDL_BF16) {
    const int chk = check_bf16_layer(M, N, K, r);
    if (chk != LDL_OK) return chk;
  }
  if (ws_base(LDL_OP_LORA_BWD, M, N, K, r, dtype) > ws_bytes) return LDL_E_WORKSPACE;
  if (!ws) return LDL_E_INVAL;
  const hipStream_t st = S(stream);
  if (M == 0) {
    LDL_TRY(zero(dA, (size_t)r * K, st));
    LDL_TRY(zero(dB, (size_t)N * r, st));
    LDL_TRY(zero(dbias, (size_t)N, st));
    return LDL_OK;
  }

  if (dtype == LDL_F32 && f32_small_ok(M, N, K, r) && lddy % 4 == 0 && ldx % 4 == 0) {
    LDL_TRY(launch_f32_small_bwd(M, N, K, r, s, (const float*)dY, lddy, (const float*)X, ldx, (const float*)W0, ldw,
                                 (const float*)A, (const float*)B, U_saved, ldu, (float*)dX, lddx, dA, dB, dbias, st));
    return LDL_OK;
  }
  if (dtype == LDL_F32) {
    Bump wb(ws);
    float* V = wb.take<float>((size_t)M * r);
    float* Uw = wb.take<float>((size_t)M * r);
    const float *dy = (const float*)dY, *x = (const float*)X, *w = (const float*)W0, *a = (const float*)A,
                *bb = (const float*)B;
    const float* U = U_saved;
    int lu = ldu;
    if (!U) {
      LDL_TRY(f32(M, r, K, x, ldx, 1, a, 1, K, Uw, r, 1.f, 0.f, nullptr, st));
      U = Uw;
      lu = r;
    }
    LDL_TRY(f32(M, r, N, dy, lddy, 1, bb, r, 1, V, r, 1.f, 0.f, nullptr, st));
    if (dX) {
      LDL_TRY(f32(M, K, N, dy, lddy, 1, w, ldw, 1, (float*)dX, lddx, 1.f, 0.f, nullptr, st));
      LDL_TRY(f32(M, K, r, V, r, 1, a, K, 1, (float*)dX, lddx, s, 1.f, nullptr, st));
    }
    LDL_TRY(f32(r, K, M, V, 1, r, x, ldx, 1, dA, K, s, 0.f, nullptr, st));
    LDL_TRY(f32(N, r, M, dy, 1, lddy, U, lu, 1, dB, r, s, 0.f, nullptr, st));
    if (dbias) LDL_TRY(launch_f32_colsum(dy, M, N, lddy, dbias, st));
    return LDL_OK;
  }

  Bump wb(ws);
  LoraBwdWs w = plan_lora_bwd(wb, M, N, K, r, true);
  const float* U = U_saved;
  int lu = ldu;
  if (!U) {
    LDL_TRY(rowproj(M, K, r, X, ldx, A, nullptr, r, K, w.U, r, 1.f, st));
    U = w.U;
    lu = r;
  }
  // V = dY.B  (B read in place as a [N, r] matrix)
  LDL_TRY(rowproj_t(M, N, r, dY, lddy, B, r, nullptr, w.V, r, 1.f, st));
  if (dX) {
    GemmParams p = gp0();
    p.M = M; p.N = K; p.K = N;
    p.a = dY; p.lda = lddy; p.b0 = W0; p.b1 = W0; p.ldb = ldw; p.kseg = N;
    p.S = w.V; p.ld_s = r; p.r_epi = r; p.s_epi = s;
    p.e0 = A; p.e1 = A; p.e_ldn = 1; p.e_ldj = K; p.e_jsplit = r;
    p.out = dX; p.ldo = lddx;
    p.part = split_part(wb, ws, ws_bytes, ws_split(LDL_OP_LORA_BWD, M, N, K, dtype));
    LDL_TRY(gemm_timed(1, GK_NN_PLAIN, p, st));
  }
  // dB = s.dY^T.U (+ dbias = column sums of dY in the same pass) and dA = s.V^T.X: one launch each
  // for the split partial sums and for their fixed-order reduction
  LDL_TRY(launch_colproj2(
      pk(cpp(M, N, r, dY, lddy, U, lu, 1.f, nullptr, 0, dbias ? 2 : 0, w.msB, w.partB, w.csB), w.pkB), w.nsB,
      pk(cpp(M, K, r, X, ldx, w.V, r, 1.f, nullptr, 0, 0, w.msA, w.partA, nullptr), w.pkA), w.nsA, st));
  LDL_TRY(launch_reduce2(rdp(N, r, w.partB, (size_t)N * w.rp, w.nsB, w.rp, false, s, dB, r),
                         rdp(r, K, w.partA, (size_t)K * w.rp, w.nsA, w.rp, true, s, dA, K), st));
  if (dbias) LDL_TRY(launch_reduce_colsum(w.csB, w.nsB, N, dbias, st));
  return LDL_OK;
}

int lora_linear_bwd_noalloc(int M, int N, int K, int r, float s, int dtype, const void* dY, int lddy, const void* X,
                            int ldx, const void* W0, int ldw, const void* A, const void* B, const float* U_saved,
                            int ldu, void* dX, int lddx, float* dA, float* dB, float* dbias, void* stream) {
  if (ws_base(LDL_OP_LORA_BWD, M, N, K, r, dtype) > kScratchBytes) return LDL_E_WORKSPACE;
  void* ws = scratch_for_current_device();
  if (!ws) return LDL_E_HIP;
  return lora_linear_bwd(M, N, K, r, s, dtype, dY, lddy, X, ldx, W0, ldw, A, B, U_saved, ldu, dX, lddx, dA, dB, dbias,
                         ws, kScratchBytes, stream);
}

size_t ldl_noalloc_scratch_bytes(void) { return kScratchBytes; }

}  // extern "C"

namespace {

// =========================================================================== several adapters, one base GEMM
constexpr int kMaxLeaves = 8;

struct MultiBwdWs {
  float* U; float* V; float* partA; uint32_t* pkA;
  float* part[kMaxLeaves]; float* cs[kMaxLeaves]; uint32_t* pk[kMaxLeaves];
  int nsA, msA, rpR, rp, ns[kMaxLeaves], ms[kMaxLeaves];
};
MultiBwdWs plan_multi_bwd(Bump& b, int M, int K, int nleaf, const int* n_leaf, int r) {
  MultiBwdWs w{};
  const int R = nleaf * r;
  w.rpR = colproj_rp(R);
  w.rp = colproj_rp(r);
  colproj_plan(M, K, &w.nsA, &w.msA, 512);
  w.U = b.take<float>((size_t)M * R);
  w.V = b.take<float>((size_t)M * R);
  w.partA = b.take<float>((size_t)w.nsA * K * w.rpR);
  w.pkA = b.take<uint32_t>(colproj_spk_words(M, R));
  for (int l = 0; l < nleaf; ++l) {
    colproj_plan(M, n_leaf[l], &w.ns[l], &w.ms[l], 512);
    w.part[l] = b.take<float>((size_t)w.ns[l] * n_leaf[l] * w.rp);
    w.cs[l] = b.take<float>((size_t)w.ns[l] * n_leaf[l]);
    w.pk[l] = b.take<uint32_t>(colproj_spk_words(M, r));
  }
  return w;
}

// shapes shared by the multi-leaf calls: leaf widths multiples of 64, at most 8 leaves, one rank
int multi_check(int M, int K, int nleaf, const int* n_leaf, int r, int dtype, int* Ntot) {
  if (!n_leaf || nleaf <= 0 || M < 0 || K <= 0 || r <= 0) return LDL_E_INVAL;
  if (dtype != LDL_BF16) return dtype == LDL_F32 ? LDL_E_UNSUPPORTED : LDL_E_INVAL;
  if (nleaf > kMaxLeaves || r % 8 || nleaf * r > 128) return LDL_E_UNSUPPORTED;
  long n = 0;
  for (int l = 0; l < nleaf; ++l) {
    if (n_leaf[l] <= 0) return LDL_E_INVAL;
    if (n_leaf[l] % 64) return LDL_E_UNSUPPORTED;
    n += n_leaf[l];
  }
  if (n > (1 << 30)) return LDL_E_UNSUPPORTED;
  *Ntot = (int)n;
  return check_bf16_layer(M, (int)n, K, nleaf * r);
}

}  // namespace

extern "C" {

size_t ldl_multi_workspace_bytes(int op, int M, int K, int nleaf, const int* n_leaf, int r) {
  int Ntot = 0;
  if (multi_check(M, K, nleaf, n_leaf, r, LDL_BF16, &Ntot) != LDL_OK) return 0;
  Bump b(nullptr);
  if (op == LDL_OP_LORA_FWD) b.take<float>((size_t)M * nleaf * r);
  else if (op == LDL_OP_LORA_BWD) plan_multi_bwd(b, M, K, nleaf, n_leaf, r);
  else return 0;
  return b.size();
}

int lora_multi_linear_fwd(int M, int K, int nleaf, const int* n_leaf, int r, const float* s_leaf, int dtype,
                          const void* X, int ldx, const void* W0, int ldw, const void* A, const void* B,
                          const void* bias, void* Y, int ldy, float* U_save, int ldu, void* ws, size_t ws_bytes,
                          void* stream) {
  int N = 0;
  const int chk = multi_check(M, K, nleaf, n_leaf, r, dtype, &N);
  if (chk != LDL_OK) return chk;
  if (!nonnull({s_leaf, W0, A, B}) || (M > 0 && !nonnull({X, Y}))) return LDL_E_INVAL;
  const int R = nleaf * r;
  LDL_LD(ldx, K, 8); LDL_LD(ldw, K, 8); LDL_LD(ldy, N, 8); LDL_LD(ldu, R, 4);
  if (!al({X, W0, A, B, bias, Y, U_save, ws})) return LDL_E_UNSUPPORTED;
  if (!fits(M, ldx, 2) || !fits(N, ldw, 2) || !fits(M, ldy, 2) || !fits(M, ldu, 4)) return LDL_E_UNSUPPORTED;
  if (!U_save && ldl_multi_workspace_bytes(LDL_OP_LORA_FWD, M, K, nleaf, n_leaf, r) > ws_bytes) return LDL_E_WORKSPACE;
  if (!U_save && !ws) return LDL_E_INVAL;
  if (M == 0) return LDL_OK;
  const hipStream_t st = S(stream);
  Bump wb(ws);
  float* U = U_save ? U_save : wb.take<float>((size_t)M * R);
  const int lu = U_save ? ldu : R;
  GemmParams p = gp0();
  p.M = M; p.N = N; p.K = K;
  p.a = X; p.lda = ldx; p.b0 = W0; p.ldb = ldw; p.kseg = K;
  p.r_epi = R; p.s_epi = 1.f; p.e0 = B; p.e1 = B; p.e_ldn = r; p.e_ldj = 1; p.e_jsplit = R;
  p.bias = bias; p.out = Y; p.ldo = ldy; p.S = U; p.ld_s = lu;
  p.nleaf = nleaf; p.leaf_r = r;
  for (int l = 0, end = 0; l < nleaf; ++l) {
    end += n_leaf[l];
    p.leaf_end[l] = end;
    p.leaf_s[l] = s_leaf[l];
  }
  const uint16_t* Bh = static_cast<const uint16_t*>(B);
  if (gemm_multi_leaf_ok(p)) {
    // U = X.[A_1; ..; A_L]^T in one pass, then one GEMM over the concatenated weight whose
    // low-rank seed takes each output column's leaf
    LDL_TRY(rowproj(M, K, R, X, ldx, A, nullptr, R, K, U, lu, 1.f, st));
    LDL_TRY(gemm_timed(0, GK_NT_PLAIN, p, st));
    return LDL_OK;
  }
  // otherwise one LoRA product per leaf into its column slice of Y
  for (int l = 0, off = 0; l < nleaf; off += n_leaf[l], ++l) {
    const int rc = lora_linear_fwd(M, n_leaf[l], K, r, s_leaf[l], LDL_BF16, X, ldx,
                                   static_cast<const uint16_t*>(W0) + (size_t)off * ldw, ldw,
                                   static_cast<const uint16_t*>(A) + (size_t)l * r * K, Bh + (size_t)off * r,
                                   bias ? static_cast<const uint16_t*>(bias) + off : nullptr,
                                   static_cast<uint16_t*>(Y) + off, ldy, U + (size_t)l * r, lu, nullptr, 0, stream);
    if (rc != LDL_OK) return rc;
  }
  return LDL_OK;
}

int lora_multi_linear_bwd(int M, int K, int nleaf, const int* n_leaf, int r, const float* s_leaf, int dtype,
                          const void* dY, int lddy, const void* X, int ldx, const void* W0, int ldw, const void* A,
                          const void* B, const float* U_saved, int ldu, void* dX, int lddx, float* dA, float* dB,
                          float* dbias, void* ws, size_t ws_bytes, void* stream) {
  int N = 0;
  const int chk = multi_check(M, K, nleaf, n_leaf, r, dtype, &N);
  if (chk != LDL_OK) return chk;
  if (!nonnull({s_leaf, W0, A, B, dA, dB, ws}) || (M > 0 && !nonnull({dY, X}))) return LDL_E_INVAL;
  const int R = nleaf * r;
  LDL_LD(lddy, N, 8); LDL_LD(ldx, K, 8); LDL_LD(ldw, K, 8); LDL_LD(ldu, R, 4); LDL_LD(lddx, K, 8);
  if (!al({dY, X, W0, A, B, U_saved, dX, dA, dB, dbias, ws})) return LDL_E_UNSUPPORTED;
  if (!fits(M, lddy, 2) || !fits(M, ldx, 2) || !fits(N, ldw, 2) || !fits(M, ldu, 4) || !fits(M, lddx, 2))
    return LDL_E_UNSUPPORTED;
  if (ldl_multi_workspace_bytes(LDL_OP_LORA_BWD, M, K, nleaf, n_leaf, r) > ws_bytes) return LDL_E_WORKSPACE;
  const hipStream_t st = S(stream);
  if (M == 0) {
    LDL_TRY(zero(dA, (size_t)R * K, st));
    LDL_TRY(zero(dB, (size_t)N * r, st));
    LDL_TRY(zero(dbias, (size_t)N, st));
    return LDL_OK;
  }
  Bump wb(ws);
  MultiBwdWs w = plan_multi_bwd(wb, M, K, nleaf, n_leaf, r);
  int off[kMaxLeaves];
  for (int l = 0, o = 0; l < nleaf; o += n_leaf[l], ++l) off[l] = o;
  const uint16_t* Bh = static_cast<const uint16_t*>(B);
  const uint16_t* dYh = static_cast<const uint16_t*>(dY);
  const float* U = U_saved;
  int lu = ldu;
  if (!U) {
    LDL_TRY(rowproj(M, K, R, X, ldx, A, nullptr, R, K, w.U, R, 1.f, st));
    U = w.U;
    lu = R;
  }
  // V_l = s_l.dY_l.B_l for each leaf (dY_l: the leaf's columns), side by side in V [M, R]
  for (int l = 0; l < nleaf; ++l)
    LDL_TRY(rowproj_t(M, n_leaf[l], r, dYh + off[l], lddy, Bh + (size_t)off[l] * r, r, nullptr, w.V + (size_t)l * r,
                      R, s_leaf[l], st));
  // dX = dY.W0 + V.[A_1; ..; A_L]: one GEMM over the concatenated weight, rank R
  if (dX) {
    GemmParams p = gp0();
    p.M = M; p.N = K; p.K = N;
    p.a = dY; p.lda = lddy; p.b0 = W0; p.b1 = W0; p.ldb = ldw; p.kseg = N;
    p.S = w.V; p.ld_s = R; p.r_epi = R; p.s_epi = 1.f;
    p.e0 = A; p.e1 = A; p.e_ldn = 1; p.e_ldj = K; p.e_jsplit = R;
    p.out = dX; p.ldo = lddx;
    LDL_TRY(gemm_timed(1, GK_NN_PLAIN, p, st));
  }
  // dA_l = V_l^T.X for every leaf in one column projection of X; dB_l = s_l.dY_l^T.U_l per leaf
  LDL_TRY(colproj(M, K, R, X, ldx, w.V, R, 1.f, nullptr, 0, 0, w.nsA, w.msA, w.partA, nullptr, st, w.pkA));
  for (int l0 = 0; l0 < nleaf; l0 += kColProjBatch) {
    ColProjParams jobs[kColProjBatch];
    int ns[kColProjBatch], nj = 0;
    for (int l = l0; l < nleaf && nj < kColProjBatch; ++l) {
      jobs[nj] = pk(cpp(M, n_leaf[l], r, dYh + off[l], lddy, U + (size_t)l * r, lu, 1.f, nullptr, 0, dbias ? 2 : 0,
                        w.ms[l], w.part[l], w.cs[l]), w.pk[l]);
      ns[nj++] = w.ns[l];
    }
    LDL_TRY(launch_colproj_batch(jobs, ns, nj, st));
  }
  // the fixed-order reductions two per launch: dA with the first leaf's dB, then the other leaves
  // in pairs
  auto dbjob = [&](int l) {
    return rdp(n_leaf[l], r, w.part[l], (size_t)n_leaf[l] * w.rp, w.ns[l], w.rp, false, s_leaf[l],
               dB + (size_t)off[l] * r, r);
  };
  LDL_TRY(launch_reduce2(rdp(R, K, w.partA, (size_t)K * w.rpR, w.nsA, w.rpR, true, 1.f, dA, K), dbjob(0), st));
  for (int l = 1; l < nleaf; l += 2) {
    if (l + 1 < nleaf) LDL_TRY(launch_reduce2(dbjob(l), dbjob(l + 1), st));
    else LDL_TRY(launch_reduce(dbjob(l), st));
  }
  if (dbias)
    for (int l = 0; l < nleaf; ++l) LDL_TRY(launch_reduce_colsum(w.cs[l], w.ns[l], n_leaf[l], dbias + off[l], st));
  return LDL_OK;
}

// =========================================================================== weight-space dropout
int lora_dropout_mask(int r, int K, int dtype, const void* A, const uint8_t* keep, void* A_drop, void* stream) {
  if (!nonnull({A, keep, A_drop})) return LDL_E_INVAL;
  if (dtype != LDL_F32 && dtype != LDL_BF16) return LDL_E_INVAL;
  if (r <= 0 || K <= 0) return LDL_E_INVAL;
  if (!small(r, K, 4)) return LDL_E_UNSUPPORTED;
  LDL_TRY(launch_mask_cols(A, keep, r, K, dtype == LDL_BF16 ? 2 : 4, A_drop, S(stream)));
  return LDL_OK;
}

int lora_dropout_grad(int r, int K, const uint8_t* keep, float* dA, void* stream) {
  if (!nonnull({keep, dA})) return LDL_E_INVAL;
  if (r <= 0 || K <= 0) return LDL_E_INVAL;
  if (!small(r, K, 4)) return LDL_E_UNSUPPORTED;
  LDL_TRY(launch_mask_cols(dA, keep, r, K, 4, dA, S(stream)));
  return LDL_OK;
}

// =========================================================================== LoRA merge
int lora_merge_fwd(int N, int K, int r, float s, int dtype, const void* W0, int ldw, const void* A, const void* B,
                   void* W, int ldo, void* stream) {
  if (!nonnull({A, B, W})) return LDL_E_INVAL;
  if (dtype != LDL_F32 && dtype != LDL_BF16) return LDL_E_INVAL;
  if (N <= 0 || K <= 0 || r <= 0) return LDL_E_INVAL;
  if (r > 128 || K % (dtype == LDL_BF16 ? 64 : 8)) return LDL_E_UNSUPPORTED;
  const int g = dtype == LDL_BF16 ? 8 : 4;
  const size_t e = dtype == LDL_BF16 ? 2 : 4;
  LDL_LD(ldw, K, g); LDL_LD(ldo, K, g);
  if (W0 == W && ldw != ldo) return LDL_E_INVAL;       // in place: the same rows
  if (!al({W0, A, B, W})) return LDL_E_UNSUPPORTED;
  if (!fits(N, ldw, e) || !fits(N, ldo, e) || !small((size_t)N + r, K, e)) return LDL_E_UNSUPPORTED;
  LDL_TRY(launch_merge(N, K, r, s, dtype == LDL_BF16, W0, ldw, A, B, W, ldo, S(stream)));
  return LDL_OK;
}

int lora_merge_bwd(int N, int K, int r, float s, int dtype, const void* dW, int lddw, const void* A, const void* B,
                   float* dA, float* dB, void* ws, size_t ws_bytes, void* stream) {
  if (!nonnull({dW, A, B, dA, dB})) return LDL_E_INVAL;
  if (dtype != LDL_F32 && dtype != LDL_BF16) return LDL_E_INVAL;
  if (N <= 0 || K <= 0 || r <= 0) return LDL_E_INVAL;
  if (r > 128 || K % (dtype == LDL_BF16 ? 64 : 8)) return LDL_E_UNSUPPORTED;
  const int g = dtype == LDL_BF16 ? 8 : 1;
  LDL_LD(lddw, K, g);
  if (!al({dW, A, B, dA, dB, ws})) return LDL_E_UNSUPPORTED;
  if (!fits(N, lddw, dtype == LDL_BF16 ? 2 : 4)) return LDL_E_UNSUPPORTED;
  if (ldl_workspace_bytes(LDL_OP_MERGE_BWD, 0, N, K, r, dtype) > ws_bytes) return LDL_E_WORKSPACE;
  if (ws_bytes > 0 && !ws) return LDL_E_INVAL;
  const hipStream_t st = S(stream);
  if (dtype == LDL_F32) {
    const float *dw = (const float*)dW, *a = (const float*)A, *bb = (const float*)B;
    LDL_TRY(f32(N, r, K, dw, lddw, 1, a, 1, K, dB, r, s, 0.f, nullptr, st));      // dB = s.dW.A^T
    LDL_TRY(f32(r, K, N, bb, 1, r, dw, lddw, 1, dA, K, s, 0.f, nullptr, st));     // dA = s.B^T.dW
    return LDL_OK;
  }
  Bump wb(ws);
  MergeBwdWs w = plan_merge_bwd(wb, N, K, r);
  // dB = s.dW.A^T: a row projection of dW; dA = s.B^T.dW: a column projection of dW against
  // B (as fp32) and the fixed-order reduction of its split partials
  LDL_TRY(rowproj(N, K, r, dW, lddw, A, nullptr, r, K, dB, r, s, st));
  LDL_TRY(launch_bf16_to_f32(B, (size_t)N * r, w.Bf, st));
  LDL_TRY(colproj(N, K, r, dW, lddw, w.Bf, r, 1.f, nullptr, 0, 0, w.ns, w.ms, w.part, nullptr, st, w.pk));
  LDL_TRY(reduce(r, K, w.part, (size_t)K * w.rp, w.ns, w.rp, true, s, dA, K, st));
  return LDL_OK;
}

// =========================================================================== DoRA
int dora_prepare(int N, int K, int dtype, const void* W0, int ldw, float* w0_sumsq, void* stream) {
  if (!nonnull({W0, w0_sumsq})) return LDL_E_INVAL;
  if (N <= 0 || K <= 0) return LDL_E_INVAL;
  if (dtype != LDL_F32 && dtype != LDL_BF16) return LDL_E_INVAL;
  if (!al({W0, w0_sumsq})) return LDL_E_UNSUPPORTED;
  LDL_LD(ldw, K, dtype == LDL_BF16 ? 8 : 1);
  if (!fits(N, ldw, dtype == LDL_BF16 ? 2 : 4)) return LDL_E_UNSUPPORTED;
  if (dtype == LDL_BF16 && K % 8) return LDL_E_UNSUPPORTED;
  LDL_TRY(launch_rowsumsq(W0, dtype == LDL_BF16, N, K, ldw, w0_sumsq, S(stream)));
  return LDL_OK;
}

static int dora_check(int M, int N, int K, int r, int dtype) {
  if (dtype != LDL_BF16) return dtype == LDL_F32 ? LDL_E_UNSUPPORTED : LDL_E_INVAL;
  const int chk = check_bf16_layer(M, N, K, r);
  if (chk != LDL_OK) return chk;
  if (r % 8) return LDL_E_UNSUPPORTED;
  return LDL_OK;
}

int dora_linear_fwd(int M, int N, int K, int r, float s, float eps, int dtype, const void* X, int ldx, const void* W0,
                    int ldw, const void* A, const void* B, const float* m, const float* w0_sumsq, const void* bias,
                    void* Y, int ldy, float* U_save, int ldu, void* Z_save, int ldz, float* state, void* ws,
                    size_t ws_bytes, void* stream) {
  (void)ws; (void)ws_bytes;
  if (!nonnull({W0, A, B, m, w0_sumsq, state}) || (M > 0 && !nonnull({X, Y, U_save, Z_save}))) return LDL_E_INVAL;
  if (M < 0 || N <= 0 || K <= 0 || r <= 0 || !(eps >= 0.f)) return LDL_E_INVAL;
  const int chk = dora_check(M, N, K, r, dtype);
  if (chk != LDL_OK) return chk;
  LDL_LD(ldx, K, 8); LDL_LD(ldw, K, 8); LDL_LD(ldy, N, 8); LDL_LD(ldu, r, 4); LDL_LD(ldz, N, 8);
  if (!al({X, W0, A, B, m, w0_sumsq, bias, Y, U_save, Z_save, state})) return LDL_E_UNSUPPORTED;
  if (!fits(M, ldx, 2) || !fits(N, ldw, 2) || !fits(M, ldy, 2) || !fits(M, ldu, 4) || !fits(M, ldz, 2))
    return LDL_E_UNSUPPORTED;
  const hipStream_t st = S(stream);
  float* norm = state;
  float* g = state + N;
  float* P = state + 2 * (size_t)N;
  float* G = P + (size_t)N * r;
  // the norm terms P = W0.A^T and G = A.A^T (G stored right after P with the same row length)
  // and U = X.A^T: one launch over the rows of W0, A and X; then nu and g
  LDL_TRY(rowproj3(N, r, M, K, r, W0, ldw, A, K, X, ldx, A, K, P, r, U_save, ldu, st));
  LDL_TRY(launch_dora_norm(N, r, s, eps, w0_sumsq, P, G, static_cast<const uint16_t*>(B), m, norm, g, st));
  if (M == 0) return LDL_OK;
  GemmParams p = gp0();
  p.M = M; p.N = N; p.K = K;
  p.a = X; p.lda = ldx; p.b0 = W0; p.ldb = ldw; p.kseg = K;
  p.S = U_save; p.ld_s = ldu; p.r_epi = r; p.s_epi = s;
  p.e0 = B; p.e1 = B; p.e_ldn = r; p.e_ldj = 1; p.e_jsplit = r;
  p.col_scale = g; p.bias = bias;
  p.out = Y; p.ldo = ldy; p.out2 = Z_save; p.ldo2 = ldz;
  LDL_TRY(gemm_timed(0, GK_NT_DORA, p, st));
  return LDL_OK;
}

int dora_linear_bwd(int M, int N, int K, int r, float s, float eps, int dtype, const void* dY, int lddy, const void* X,
                    int ldx, const void* W0, int ldw, const void* A, const void* B, const float* m,
                    const float* U_saved, int ldu, const void* Z_saved, int ldz, const float* state, void* dX,
                    int lddx, float* dA, float* dB, float* dm, float* dbias, void* ws, size_t ws_bytes,
                    void* stream) {
  if (!nonnull({W0, A, B, m, state, dA, dB, dm, ws}) || (M > 0 && !nonnull({dY, X, U_saved, Z_saved})))
    return LDL_E_INVAL;
  if (M < 0 || N <= 0 || K <= 0 || r <= 0 || !(eps >= 0.f)) return LDL_E_INVAL;
  const int chk = dora_check(M, N, K, r, dtype);
  if (chk != LDL_OK) return chk;
  LDL_LD(lddy, N, 8); LDL_LD(ldx, K, 8); LDL_LD(ldw, K, 8); LDL_LD(ldu, r, 4); LDL_LD(ldz, N, 8); LDL_LD(lddx, K, 8);
  if (!al({dY, X, W0, A, B, m, U_saved, Z_saved, state, dX, dA, dB, dm, dbias, ws})) return LDL_E_UNSUPPORTED;
  if (!fits(M, lddy, 2) || !fits(M, ldx, 2) || !fits(N, ldw, 2) || !fits(M, ldu, 4) || !fits(M, ldz, 2) ||
      !fits(M, lddx, 2))
    return LDL_E_UNSUPPORTED;
  if (ldl_workspace_bytes(LDL_OP_DORA_BWD, M, N, K, r, dtype) > ws_bytes) return LDL_E_WORKSPACE;
  const hipStream_t st = S(stream);
  const float* norm = state;
  const float* g = state + N;
  const float* P = state + 2 * (size_t)N;
  const float* G = P + (size_t)N * r;
  Bump wb(ws);
  DoraBwdWs w = plan_dora_bwd(wb, M, N, K, r);
  const uint16_t* Bh = static_cast<const uint16_t*>(B);

  // dg and dZ^T.U in one pass over dY (and Z); M == 0 gives zero partials
  if (M > 0) {
    LDL_TRY(colproj(M, N, r, dY, lddy, U_saved, ldu, 1.f, Z_saved, ldz, 1, w.nsT, w.msT, w.partT, w.cs, st, w.pkT));
  } else {
    LDL_TRY(zero(w.partT, (size_t)w.nsT * N * w.rp, st));
    LDL_TRY(zero(w.cs, (size_t)w.nsT * N, st));
  }
  // The rank-r factors of the last column projections are written pre-packed (bf16 hi / lo,
  // the layout pack_s_kernel writes) by the kernels that form them, where that path applies
  // (ranks 17 .. 64): wB by the finalize pass, V by its row projection.  No pack pass then.
  const bool prepack = g_prepack && w.rp >= 32 && w.rp <= 64;
  // dB, dm and wB = 2s.w.B per output row
  LDL_TRY(launch_dora_finalize(N, r, s, eps, w.partT, w.cs, w.nsT, w.rp, norm, g, m, P, G, Bh, dB, dm, w.wB,
                               prepack ? reinterpret_cast<uint16_t*>(w.pkW) : nullptr, w.rp, st));
  ColProjParams jobs[3];
  int ns[3], nj = 0;
  bool v_packed = false;
  if (M > 0) {
    // dZ = dY.diag(g) is never formed: the row scale goes into bf16 copies of the weight and of
    // lora_up (rounded once, weight-sized), V = dY.(diag(g).B) and dX = dY.(diag(g).W0) + s.V.A
    LDL_TRY(launch_scale_rows(W0, N, dX ? K : 0, ldw, B, r, g, w.gW0, w.gB, st));
    LDL_TRY(rowproj_t_pk(M, N, r, dY, lddy, w.gB, r, w.V, r, 1.f,
                         prepack ? reinterpret_cast<uint16_t*>(w.pkA) : nullptr, w.rp, s, &v_packed, st));
    if (dX) {
      GemmParams p = gp0();
      p.M = M; p.N = K; p.K = N;
      p.a = dY; p.lda = lddy; p.b0 = w.gW0; p.b1 = w.gW0; p.ldb = K; p.kseg = N;
      p.S = w.V; p.ld_s = r; p.r_epi = r; p.s_epi = s;
      p.e0 = A; p.e1 = A; p.e_ldn = 1; p.e_ldj = K; p.e_jsplit = r;
      p.out = dX; p.ldo = lddx;
      LDL_TRY(gemm_timed(1, GK_NN_PLAIN, p, st));
    }
    // s.V^T.X into the first nsA partials of dA
    jobs[nj] = pk(cpp(M, K, r, X, ldx, w.V, r, s, nullptr, 0, 0, w.msA, w.partA, nullptr), w.pkA);
    jobs[nj].spk_ready = v_packed;
    ns[nj++] = w.nsA;
  } else {
    LDL_TRY(zero(w.partA, (size_t)w.nsA * K * w.rp, st));
  }
  // (2s.w.B)^T.W0 into the next nsW partials; Q = B^T.(2s.w.B) (both read the one packed wB)
  jobs[nj] = pk(cpp(N, K, r, W0, ldw, w.wB, r, 1.f, nullptr, 0, 0, w.msW, w.partA + (size_t)w.nsA * K * w.rp,
                    nullptr), w.pkW);
  jobs[nj].spk_ready = prepack;
  ns[nj++] = w.nsW;
  jobs[nj] = pk(cpp(N, r, r, B, r, w.wB, r, 1.f, nullptr, 0, 0, w.msQ, w.partQ, nullptr), prepack ? w.pkW : w.pkQ);
  jobs[nj].spk_ready = prepack;
  ns[nj++] = w.nsQ;
  LDL_TRY(launch_colproj_batch(jobs, ns, nj, st));
  LDL_TRY(reduce(r, r, w.partQ, (size_t)r * w.rp, w.nsQ, w.rp, false, 1.f, w.Qm, r, st));
  // dA = sum of all partials + s.Q.A   (2s^2 B^T diag(w) B A = s.Q.A)
  LDL_TRY(reduce(r, K, w.partA, (size_t)K * w.rp, w.nsA + w.nsW, w.rp, true, 1.f, dA, K, st, nullptr, w.Qm, r, r, A,
                 K, s));
  if (dbias) {
    if (M > 0) {
      LDL_TRY(colproj(M, N, 0, dY, lddy, nullptr, 0, 1.f, nullptr, 0, 2, w.nsT, w.msT, w.partbias, w.csbias, st));
      LDL_TRY(launch_reduce_colsum(w.csbias, w.nsT, N, dbias, st));
    } else {
      LDL_TRY(zero(dbias, (size_t)N, st));
    }
  }
  return LDL_OK;
}

// =========================================================================== DoRA, column form
int dora_cols_prepare(int N, int K, int dtype, const void* W0, int ldw, float* w0_colsq, void* stream) {
  if (!nonnull({W0, w0_colsq})) return LDL_E_INVAL;
  if (N <= 0 || K <= 0) return LDL_E_INVAL;
  if (dtype != LDL_F32 && dtype != LDL_BF16) return LDL_E_INVAL;
  if (!al({W0, w0_colsq})) return LDL_E_UNSUPPORTED;
  LDL_LD(ldw, K, dtype == LDL_BF16 ? 8 : 1);
  if (dtype == LDL_BF16 && K % 8) return LDL_E_UNSUPPORTED;
  if (!fits(N, ldw, dtype == LDL_BF16 ? 2 : 4)) return LDL_E_UNSUPPORTED;
  LDL_TRY(launch_col_sumsq(W0, dtype == LDL_BF16, N, K, ldw, w0_colsq, S(stream)));
  return LDL_OK;
}

static int dora_cols_check(int M, int N, int K, int r, int dtype) {
  const int chk = dora_check(M, N, K, r, dtype);
  if (chk != LDL_OK) return chk;
  return r > 64 ? LDL_E_UNSUPPORTED : LDL_OK;
}

int dora_cols_linear_fwd(int M, int N, int K, int r, float s, float eps, int dtype, const void* X, int ldx,
                         const void* W0, int ldw, const void* A, const void* B, const float* m, const float* w0_colsq,
                         const void* bias, void* Y, int ldy, float* U_save, int ldu, void* Xs_save, int ldxs,
                         float* state, void* ws, size_t ws_bytes, void* stream) {
  if (!nonnull({W0, A, B, m, w0_colsq, state, ws}) || (M > 0 && !nonnull({X, Y, Xs_save}))) return LDL_E_INVAL;
  if (M < 0 || N <= 0 || K <= 0 || r <= 0 || !(eps >= 0.f)) return LDL_E_INVAL;
  const int chk = dora_cols_check(M, N, K, r, dtype);
  if (chk != LDL_OK) return chk;
  LDL_LD(ldx, K, 8); LDL_LD(ldw, K, 8); LDL_LD(ldy, N, 8); LDL_LD(ldu, r, 4); LDL_LD(ldxs, K, 8);
  if (!al({X, W0, A, B, m, w0_colsq, bias, Y, U_save, Xs_save, state, ws})) return LDL_E_UNSUPPORTED;
  if (!fits(M, ldx, 2) || !fits(N, ldw, 2) || !fits(M, ldy, 2) || !fits(M, ldu, 4) || !fits(M, ldxs, 2))
    return LDL_E_UNSUPPORTED;
  if (ldl_workspace_bytes(LDL_OP_DORA_COLS_FWD, M, N, K, r, dtype) > ws_bytes) return LDL_E_WORKSPACE;
  const hipStream_t st = S(stream);
  Bump wb(ws);
  DoraColsFwdWs w = plan_dora_cols_fwd(wb, M, N, K, r);
  float* norm = state;
  float* g = state + K;
  float* Pc = state + 2 * (size_t)K;
  float* Gc = Pc + (size_t)K * r;
  // the norm terms Pc = B^T.W0 and Gc = B^T.B (one column-projection launch over the rows of
  // W0 and of B against B), then nu and g (independent of M)
  {
    ColProjParams jobs[2] = {pk(cpp(N, K, r, W0, ldw, w.Bf, r, 1.f, nullptr, 0, 0, w.msP, w.partP, nullptr), w.pkP),
                             pk(cpp(N, r, r, B, r, w.Bf, r, 1.f, nullptr, 0, 0, w.msG, w.partG, nullptr), w.pkG)};
    int ns[2] = {w.nsP, w.nsG};
    if (colproj_takes_bf16_s(jobs, 2)) {         // B packed from bf16 directly
      jobs[0] = s16(jobs[0], B);
      jobs[1] = s16(jobs[1], B);
    } else {
      LDL_TRY(launch_bf16_to_f32(B, (size_t)N * r, w.Bf, st));
    }
    LDL_TRY(launch_colproj_batch(jobs, ns, 2, st));
  }
  LDL_TRY(launch_reduce2(rdp(r, K, w.partP, (size_t)K * w.rp, w.nsP, w.rp, true, 1.f, Pc, K),
                         rdp(r, r, w.partG, (size_t)r * w.rp, w.nsG, w.rp, true, 1.f, Gc, r), st));
  LDL_TRY(launch_dora_cols_norm(K, r, s, eps, w0_colsq, m, A, Pc, Gc, norm, g, st));
  if (M == 0) return LDL_OK;
  // the layer input scaled per feature, kept for the backward, then the LoRA layer on it
  LDL_TRY(launch_scale_cols(X, M, K, ldx, g, Xs_save, ldxs, st));
  return lora_linear_fwd(M, N, K, r, s, LDL_BF16, Xs_save, ldxs, W0, ldw, A, B, bias, Y, ldy,
                         U_save ? U_save : w.U, U_save ? ldu : r, nullptr, 0, stream);
}

int dora_cols_linear_bwd(int M, int N, int K, int r, float s, float eps, int dtype, const void* dY, int lddy,
                         const void* X, int ldx, const void* Xs_saved, int ldxs, const void* W0, int ldw,
                         const void* A, const void* B, const float* m, const float* U_saved, int ldu,
                         const float* state, void* dX, int lddx, float* dA, float* dB, float* dm, float* dbias,
                         void* ws, size_t ws_bytes, void* stream) {
  if (!nonnull({W0, A, B, m, state, dA, dB, dm, ws}) || (M > 0 && !nonnull({dY, X, Xs_saved}))) return LDL_E_INVAL;
  if (M < 0 || N <= 0 || K <= 0 || r <= 0 || !(eps >= 0.f)) return LDL_E_INVAL;
  const int chk = dora_cols_check(M, N, K, r, dtype);
  if (chk != LDL_OK) return chk;
  LDL_LD(lddy, N, 8); LDL_LD(ldx, K, 8); LDL_LD(ldxs, K, 8); LDL_LD(ldw, K, 8); LDL_LD(ldu, r, 4); LDL_LD(lddx, K, 8);
  if (!al({dY, X, Xs_saved, W0, A, B, m, U_saved, state, dX, dA, dB, dm, dbias, ws})) return LDL_E_UNSUPPORTED;
  if (!fits(M, lddy, 2) || !fits(M, ldx, 2) || !fits(M, ldxs, 2) || !fits(N, ldw, 2) || !fits(M, ldu, 4) ||
      !fits(M, lddx, 2))
    return LDL_E_UNSUPPORTED;
  if (ldl_workspace_bytes(LDL_OP_DORA_COLS_BWD, M, N, K, r, dtype) > ws_bytes) return LDL_E_WORKSPACE;
  const hipStream_t st = S(stream);
  Bump wb(ws);
  DoraColsBwdWs w = plan_dora_cols_bwd(wb, M, N, K, r);
  const float* norm = state;
  const float* g = state + K;
  const float* Pc = state + 2 * (size_t)K;
  const float* Gc = Pc + (size_t)K * r;
  const float* U = U_saved;
  int lu = ldu;
  if (M > 0) {
    // the LoRA layer on the scaled input (V = dY.B; U = Xs.A^T unless saved), with the input
    // gradient's feature scale in the GEMM epilogue from the fp32 accumulators:
    // dXs = dY.W0 + s.V.A (bf16, kept for dg) and dX = dXs.diag(g)
    Bump lb(w.lora);
    LoraBwdWs lw = plan_lora_bwd(lb, M, N, K, r, true);
    if (!U) {
      LDL_TRY(rowproj(M, K, r, Xs_saved, ldxs, A, nullptr, r, K, lw.U, r, 1.f, st));
      U = lw.U;
      lu = r;
    }
    LDL_TRY(rowproj_t(M, N, r, dY, lddy, B, r, nullptr, lw.V, r, 1.f, st));
    GemmParams p = gp0();
    p.M = M; p.N = K; p.K = N;
    p.a = dY; p.lda = lddy; p.b0 = W0; p.b1 = W0; p.ldb = ldw; p.kseg = N;
    p.S = lw.V; p.ld_s = r; p.r_epi = r; p.s_epi = s;
    p.e0 = A; p.e1 = A; p.e_ldn = 1; p.e_ldj = K; p.e_jsplit = r;
    if (dX) {
      p.out = dX; p.ldo = lddx; p.out2 = w.dXs; p.ldo2 = K; p.col_scale = g;
      LDL_TRY(gemm_timed(1, GK_NN_DORA, p, st));
    } else {
      p.out = w.dXs; p.ldo = K;
      LDL_TRY(gemm_timed(1, GK_NN_PLAIN, p, st));
    }
    // dB = s.dY^T.U (+ dbias), dA = s.V^T.Xs, and dg_k = sum_m dXs[m,k] X[m,k] as column
    // sums of the product: split partials, then fixed-order reductions
    {
      ColProjParams jobs[3] = {
          pk(cpp(M, N, r, dY, lddy, U, lu, 1.f, nullptr, 0, dbias ? 2 : 0, lw.msB, lw.partB, lw.csB), lw.pkB),
          pk(cpp(M, K, r, Xs_saved, ldxs, lw.V, r, 1.f, nullptr, 0, 0, lw.msA, lw.partA, nullptr), lw.pkA),
          cpp(M, K, 0, w.dXs, K, nullptr, 0, 1.f, X, ldx, 1, w.msD, w.partD, w.csD)};
      int ns[3] = {lw.nsB, lw.nsA, w.nsD};
      LDL_TRY(launch_colproj_batch(jobs, ns, 3, st));
    }
    LDL_TRY(launch_reduce2(rdp(N, r, lw.partB, (size_t)N * lw.rp, lw.nsB, lw.rp, false, s, dB, r),
                           rdp(r, K, lw.partA, (size_t)K * lw.rp, lw.nsA, lw.rp, true, s, dA, K), st));
    if (dbias) LDL_TRY(launch_reduce_colsum(lw.csB, lw.nsB, N, dbias, st));
  } else {
    LDL_TRY(zero(dA, (size_t)r * K, st));
    LDL_TRY(zero(dB, (size_t)N * r, st));
    LDL_TRY(zero(dbias, (size_t)N, st));
  }
  // dm, and the norm's terms: dA += 2s (Pc + s.Gc.A).diag(w); dB += 2s W0.diag(w).A^T +
  // 2s^2 B.(A.diag(w).A^T), the two products over K as one row projection of [W0; A]
  // (dg_k: the split column sums of dXs.X, summed in split order by the same launch; none at M = 0)
  LDL_TRY(launch_dora_cols_bwd(K, r, s, eps, w.csD, M > 0 ? w.nsD : 0, norm, m, A, Pc, Gc, dm, dA, w.Aw, st));
  LDL_TRY(rowproj2(N, r, K, 2 * r, W0, ldw, A, K, w.Aw, K, w.T, 2 * r, 1.f, st));
  LDL_TRY(launch_dora_cols_db(N, r, s, B, w.T, dB, st));
  return LDL_OK;
}

// =========================================================================== SwiGLU MLP
static int mlp_check(int M, int K, int H, int r) {
  if (M < 0 || K <= 0 || H <= 0 || r <= 0) return LDL_E_INVAL;
  if (r > 64 || r % 8 || K % 64 || H % 64) return LDL_E_UNSUPPORTED;
  if (!small(M + 256, 2 * (size_t)H, 2) || !small(H, K, 2) || !small(M + 256, K, 2)) return LDL_E_UNSUPPORTED;
  return LDL_OK;
}

static int glu_mlp_fwd(int act, int M, int K, int H, int r, float s_gate, float s_up, float s_down, const void* X,
                       int ldx, const void* Wg, const void* Ag, const void* Bg, const void* Wu, const void* Au,
                       const void* Bu, const void* Wd, const void* Ad, const void* Bd, void* Out, int ldout,
                       void* E_save, void* Gu_save, void* H_save, float* U_save, void* ws, size_t ws_bytes,
                       void* stream) {
  (void)ws; (void)ws_bytes;
  if (!nonnull({Wg, Ag, Bg, Wu, Au, Bu, Wd, Ad, Bd}) || (M > 0 && !nonnull({X, Out, E_save, Gu_save, H_save, U_save})))
    return LDL_E_INVAL;
  const int chk = mlp_check(M, K, H, r);
  if (chk != LDL_OK) return chk;
  LDL_LD(ldx, K, 8); LDL_LD(ldout, K, 8);
  if (!fits(M, ldx, 2) || !fits(M, ldout, 2)) return LDL_E_UNSUPPORTED;
  if (!al({X, Wg, Ag, Bg, Wu, Au, Bu, Wd, Ad, Bd, Out, E_save, Gu_save, H_save, U_save})) return LDL_E_UNSUPPORTED;
  if (M == 0) return LDL_OK;
  const hipStream_t st = S(stream);
  const int r3 = 3 * r;
  // [U_g | U_u] = X.[Ag; Au]^T in one pass over X
  LDL_TRY(rowproj(M, K, 2 * r, X, ldx, Ag, Au, r, K, U_save, r3, 1.f, st));
  // gate and up projections in one GEMM (each tile holds e and u of the same hidden units
  // side by side: the four-wave dual tile, or the eight-wave one for 128 tokens or fewer or
  // hidden widths not a multiple of 128) with h = silu(e) * u formed from the fp32
  // accumulators in the epilogue
  GemmParams p = gp0();
  p.M = M; p.N = H; p.K = K;
  p.a = X; p.lda = ldx; p.b0 = Wg; p.b1 = Wu; p.ldb = K; p.kseg = K;
  p.S = U_save; p.ld_s = r3; p.r_epi = 2 * r; p.s_epi = s_gate; p.s_epi2 = s_up;
  p.e0 = Bg; p.e1 = Bu; p.e_ldn = r; p.e_ldj = 1; p.e_jsplit = r;
  p.out = E_save; p.ldo = H; p.out2 = Gu_save; p.ldo2 = H; p.out3 = H_save; p.ldo3 = H;
  p.act = act;
  LDL_TRY(launch_gemm(GK_NT_SWIGLU_DUAL, p, st));
  // U_d = H.Ad^T, then the down projection
  LDL_TRY(rowproj(M, H, r, H_save, H, Ad, nullptr, r, H, U_save + 2 * r, r3, 1.f, st));
  GemmParams q = gp0();
  q.M = M; q.N = K; q.K = H;
  q.a = H_save; q.lda = H; q.b0 = Wd; q.ldb = H; q.kseg = H;
  q.S = U_save + 2 * r; q.ld_s = r3; q.r_epi = r; q.s_epi = s_down;
  q.e0 = Bd; q.e1 = Bd; q.e_ldn = r; q.e_ldj = 1; q.e_jsplit = r;
  q.out = Out; q.ldo = ldout;
  LDL_TRY(gemm_timed(0, GK_NT_PLAIN, q, st));
  return LDL_OK;
}

static int glu_mlp_bwd(int act, int M, int K, int H, int r, float s_gate, float s_up, float s_down,
                       const void* dOut, int lddout, const void* X, int ldx, const void* Wg, const void* Ag,
                       const void* Bg, const void* Wu, const void* Au, const void* Bu, const void* Wd, const void* Ad,
                       const void* Bd, const void* E_saved, const void* Gu_saved, const void* H_saved,
                       const float* U_saved, void* dX, int lddx, float* dAg, float* dBg, float* dAu, float* dBu,
                       float* dAd, float* dBd, void* ws, size_t ws_bytes, void* stream) {
  if (!nonnull({Wg, Ag, Bg, Wu, Au, Bu, Wd, Ad, Bd, dAg, dBg, dAu, dBu, dAd, dBd, ws}) ||
      (M > 0 && !nonnull({dOut, X, E_saved, Gu_saved, H_saved, U_saved})))
    return LDL_E_INVAL;
  const int chk = mlp_check(M, K, H, r);
  if (chk != LDL_OK) return chk;
  LDL_LD(lddout, K, 8); LDL_LD(ldx, K, 8); LDL_LD(lddx, K, 8);
  if (!fits(M, lddout, 2) || !fits(M, ldx, 2) || !fits(M, lddx, 2)) return LDL_E_UNSUPPORTED;
  if (!al({dOut, X, Wg, Ag, Bg, Wu, Au, Bu, Wd, Ad, Bd, E_saved, Gu_saved, H_saved, U_saved, dX, dAg, dBg, dAu, dBu,
           dAd, dBd, ws}))
    return LDL_E_UNSUPPORTED;
  if (ldl_workspace_bytes(LDL_OP_SWIGLU_BWD, M, H, K, r, LDL_BF16) > ws_bytes) return LDL_E_WORKSPACE;
  const hipStream_t st = S(stream);
  if (M == 0) {
    LDL_TRY(zero(dAg, (size_t)r * K, st)); LDL_TRY(zero(dAu, (size_t)r * K, st));
    LDL_TRY(zero(dBg, (size_t)H * r, st)); LDL_TRY(zero(dBu, (size_t)H * r, st));
    LDL_TRY(zero(dAd, (size_t)r * H, st)); LDL_TRY(zero(dBd, (size_t)K * r, st));
    return LDL_OK;
  }
  Bump wb(ws);
  MlpBwdWs w = plan_mlp_bwd(wb, M, K, H, r);
  const int r3 = 3 * r;
  const float* Ug = U_saved;
  const float* Uu = U_saved + r;
  const float* Ud = U_saved + 2 * r;

  // ---- down projection: V_d = dOut.Bd (Bd read in place as a [K, r] matrix)
  LDL_TRY(rowproj_t(M, K, r, dOut, lddout, Bd, r, nullptr, w.Vd, r, 1.f, st));
  // ---- dH = dOut.Wd + s_d.V_d.Ad with the SwiGLU backward in the epilogue -> [dE | dGu]
  {
    GemmParams p = gp0();
    p.M = M; p.N = H; p.K = K;
    p.a = dOut; p.lda = lddout; p.b0 = Wd; p.b1 = Wd; p.ldb = H; p.kseg = K;
    p.S = w.Vd; p.ld_s = r; p.r_epi = r; p.s_epi = s_down;
    p.e0 = Ad; p.e1 = Ad; p.e_ldn = 1; p.e_ldj = H; p.e_jsplit = r;
    p.aux0 = E_saved; p.ld_aux0 = H; p.aux1 = Gu_saved; p.ld_aux1 = H;
    p.out = w.dEGu; p.ldo = 2 * H; p.out2 = w.dEGu + H; p.ldo2 = 2 * H;
    p.act = act;
    LDL_TRY(launch_gemm(GK_NN_SWIGLU, p, st));
  }
  // dBd = s_d.dOut^T.U_d and dAd = s_d.V_d^T.H
  LDL_TRY(launch_colproj2(pk(cpp(M, K, r, dOut, lddout, Ud, r3, 1.f, nullptr, 0, 0, w.msDd, w.partDd, nullptr), w.pkDd),
                          w.nsDd,
                          pk(cpp(M, H, r, H_saved, H, w.Vd, r, 1.f, nullptr, 0, 0, w.msAd, w.partAd, nullptr), w.pkAd),
                          w.nsAd, st));
  LDL_TRY(launch_reduce2(rdp(K, r, w.partDd, (size_t)K * w.rp, w.nsDd, w.rp, false, s_down, dBd, r),
                         rdp(r, H, w.partAd, (size_t)H * w.rp, w.nsAd, w.rp, true, s_down, dAd, H), st));
  // ---- gate / up: V_g = s_g.dE.Bg, V_u = s_u.dGu.Bu (pre-scaled), dBg, dBu
  // (with dAg and dAu as two rank-r column projections, V_g and V_u are also written packed
  // for them by these launches, so that projection needs no pack pass)
  const bool prepack = g_prepack && w.agu_split;
  uint16_t* pk_g = prepack ? reinterpret_cast<uint16_t*>(w.pkAgu) : nullptr;
  uint16_t* pk_u = prepack ? reinterpret_cast<uint16_t*>(w.pkAgu + colproj_spk_words(M, r)) : nullptr;
  bool g_packed = false, u_packed = false;
  LDL_TRY(rowproj_t_pk(M, H, r, w.dEGu, 2 * H, Bg, r, w.Vgu, 2 * r, s_gate, pk_g, w.rp, 1.f, &g_packed, st));
  LDL_TRY(rowproj_t_pk(M, H, r, w.dEGu + H, 2 * H, Bu, r, w.Vgu + r, 2 * r, s_up, pk_u, w.rp, 1.f, &u_packed, st));
  LDL_TRY(launch_colproj2(pk(cpp(M, H, r, w.dEGu, 2 * H, Ug, r3, 1.f, nullptr, 0, 0, w.msBg, w.partBg, nullptr), w.pkBg),
                          w.nsBg,
                          pk(cpp(M, H, r, w.dEGu + H, 2 * H, Uu, r3, 1.f, nullptr, 0, 0, w.msBg, w.partBu, nullptr),
                             w.pkBu),
                          w.nsBg, st));
  LDL_TRY(launch_reduce2(rdp(H, r, w.partBg, (size_t)H * w.rp, w.nsBg, w.rp, false, s_gate, dBg, r),
                         rdp(H, r, w.partBu, (size_t)H * w.rp, w.nsBg, w.rp, false, s_up, dBu, r), st));
  // ---- dX = [dE | dGu].[Wg; Wu] + [V_g | V_u].[Ag; Au]  (one GEMM over the 2H reduction)
  if (dX) {
    GemmParams p = gp0();
    p.M = M; p.N = K; p.K = 2 * H;
    p.a = w.dEGu; p.lda = 2 * H; p.b0 = Wg; p.b1 = Wu; p.ldb = K; p.kseg = H;
    p.S = w.Vgu; p.ld_s = 2 * r; p.r_epi = 2 * r; p.s_epi = 1.f;
    p.e0 = Ag; p.e1 = Au; p.e_ldn = 1; p.e_ldj = K; p.e_jsplit = r;
    p.out = dX; p.ldo = lddx;
    LDL_TRY(gemm_timed(1, GK_NN_PLAIN, p, st));
  }
  // dAg, dAu = [V_g | V_u]^T.X in one pass over X
  if (w.agu_split) {
    float* partAu = w.partAgu + (size_t)w.nsAgu * K * w.rp;
    ColProjParams jg = pk(cpp(M, K, r, X, ldx, w.Vgu, 2 * r, 1.f, nullptr, 0, 0, w.msAgu, w.partAgu, nullptr), w.pkAgu);
    ColProjParams ju = pk(cpp(M, K, r, X, ldx, w.Vgu + r, 2 * r, 1.f, nullptr, 0, 0, w.msAgu, partAu, nullptr),
                          w.pkAgu + colproj_spk_words(M, r));
    jg.spk_ready = g_packed;
    ju.spk_ready = u_packed;
    LDL_TRY(launch_colproj2(jg, w.nsAgu, ju, w.nsAgu, st));
    LDL_TRY(launch_reduce2(rdp(r, K, w.partAgu, (size_t)K * w.rp, w.nsAgu, w.rp, true, 1.f, dAg, K),
                           rdp(r, K, partAu, (size_t)K * w.rp, w.nsAgu, w.rp, true, 1.f, dAu, K), st));
  } else {
    LDL_TRY(colproj(M, K, 2 * r, X, ldx, w.Vgu, 2 * r, 1.f, nullptr, 0, 0, w.nsAgu, w.msAgu, w.partAgu, nullptr, st,
                    w.pkAgu));
    LDL_TRY(launch_reduce2(rdp(r, K, w.partAgu, (size_t)K * w.rp2, w.nsAgu, w.rp2, true, 1.f, dAg, K),
                           rdp(r, K, w.partAgu + r, (size_t)K * w.rp2, w.nsAgu, w.rp2, true, 1.f, dAu, K), st));
  }
  return LDL_OK;
}

int swiglu_lora_mlp_fwd(int M, int K, int H, int r, float s_gate, float s_up, float s_down, const void* X, int ldx,
                        const void* Wg, const void* Ag, const void* Bg, const void* Wu, const void* Au,
                        const void* Bu, const void* Wd, const void* Ad, const void* Bd, void* Out, int ldout,
                        void* E_save, void* Gu_save, void* H_save, float* U_save, void* ws, size_t ws_bytes,
                        void* stream) {
  return glu_mlp_fwd(ACT_SILU, M, K, H, r, s_gate, s_up, s_down, X, ldx, Wg, Ag, Bg, Wu, Au, Bu, Wd, Ad, Bd, Out,
                     ldout, E_save, Gu_save, H_save, U_save, ws, ws_bytes, stream);
}

int swiglu_lora_mlp_bwd(int M, int K, int H, int r, float s_gate, float s_up, float s_down, const void* dOut,
                        int lddout, const void* X, int ldx, const void* Wg, const void* Ag, const void* Bg,
                        const void* Wu, const void* Au, const void* Bu, const void* Wd, const void* Ad, const void* Bd,
                        const void* E_saved, const void* Gu_saved, const void* H_saved, const float* U_saved,
                        void* dX, int lddx, float* dAg, float* dBg, float* dAu, float* dBu, float* dAd, float* dBd,
                        void* ws, size_t ws_bytes, void* stream) {
  return glu_mlp_bwd(ACT_SILU, M, K, H, r, s_gate, s_up, s_down, dOut, lddout, X, ldx, Wg, Ag, Bg, Wu, Au, Bu, Wd, Ad,
                     Bd, E_saved, Gu_saved, H_saved, U_saved, dX, lddx, dAg, dBg, dAu, dBu, dAd, dBd, ws, ws_bytes,
                     stream);
}

int geglu_lora_mlp_fwd(int M, int K, int H, int r, float s_gate, float s_up, float s_down, int approximate,
                       const void* X, int ldx, const void* Wg, const void* Ag, const void* Bg, const void* Wu,
                       const void* Au, const void* Bu, const void* Wd, const void* Ad, const void* Bd, void* Out,
                       int ldout, void* E_save, void* Gu_save, void* H_save, float* U_save, void* ws, size_t ws_bytes,
                       void* stream) {
  if (approximate != 0 && approximate != 1) return LDL_E_INVAL;
  return glu_mlp_fwd(approximate ? ACT_GELU_TANH : ACT_GELU, M, K, H, r, s_gate, s_up, s_down, X, ldx, Wg, Ag, Bg, Wu,
                     Au, Bu, Wd, Ad, Bd, Out, ldout, E_save, Gu_save, H_save, U_save, ws, ws_bytes, stream);
}

int geglu_lora_mlp_bwd(int M, int K, int H, int r, float s_gate, float s_up, float s_down, int approximate,
                       const void* dOut, int lddout, const void* X, int ldx, const void* Wg, const void* Ag,
                       const void* Bg, const void* Wu, const void* Au, const void* Bu, const void* Wd, const void* Ad,
                       const void* Bd, const void* E_saved, const void* Gu_saved, const void* H_saved,
                       const float* U_saved, void* dX, int lddx, float* dAg, float* dBg, float* dAu, float* dBu,
                       float* dAd, float* dBd, void* ws, size_t ws_bytes, void* stream) {
  if (approximate != 0 && approximate != 1) return LDL_E_INVAL;
  return glu_mlp_bwd(approximate ? ACT_GELU_TANH : ACT_GELU, M, K, H, r, s_gate, s_up, s_down, dOut, lddout, X, ldx,
                     Wg, Ag, Bg, Wu, Au, Bu, Wd, Ad, Bd, E_saved, Gu_saved, H_saved, U_saved, dX, lddx, dAg, dBg,
                     dAu, dBu, dAd, dBd, ws, ws_bytes, stream);
}

// =========================================================================== W8A8
static int quantize_weight8(int N, int K, int dtype, const void* W0, int ldw, int8_t* Wq, float* sw, void* stream,
                            int fp8) {
  if (!nonnull({W0, Wq, sw})) return LDL_E_INVAL;
  if (N <= 0 || K <= 0) return LDL_E_INVAL;
  if (dtype != LDL_F32 && dtype != LDL_BF16) return LDL_E_INVAL;
  if (K % 8 || !al({W0, Wq, sw})) return LDL_E_UNSUPPORTED;
  LDL_LD(ldw, K, dtype == LDL_BF16 ? 8 : 1);
  if (!fits(N, ldw, dtype == LDL_BF16 ? 2 : 4) || !fits(N, K, 1)) return LDL_E_UNSUPPORTED;
  LDL_TRY(launch_quantize_rows(W0, dtype == LDL_F32, N, K, ldw, Wq, sw, S(stream), fp8));
  return LDL_OK;
}

static int quantize_rows8(int M, int K, const void* X, int ldx, int8_t* Xq, float* sx, void* stream, int fp8) {
  if (M > 0 && !nonnull({X, Xq, sx})) return LDL_E_INVAL;
  if (M < 0 || K <= 0) return LDL_E_INVAL;
  if (K % 8 || !al({X, Xq, sx})) return LDL_E_UNSUPPORTED;
  LDL_LD(ldx, K, 8);
  if (!fits(M, ldx, 2)) return LDL_E_UNSUPPORTED;
  LDL_TRY(launch_quantize_rows(X, 0, M, K, ldx, Xq, sx, S(stream), fp8));
  return LDL_OK;
}

int w8a8_quantize_weight(int N, int K, int dtype, const void* W0, int ldw, int8_t* Wq, float* sw, void* stream) {
  return quantize_weight8(N, K, dtype, W0, ldw, Wq, sw, stream, 0);
}
int w8a8_quantize_rows(int M, int K, const void* X, int ldx, int8_t* Xq, float* sx, void* stream) {
  return quantize_rows8(M, K, X, ldx, Xq, sx, stream, 0);
}
int fp8_quantize_weight(int N, int K, int dtype, const void* W0, int ldw, uint8_t* Wq, float* sw, void* stream) {
  return quantize_weight8(N, K, dtype, W0, ldw, reinterpret_cast<int8_t*>(Wq), sw, stream, 1);
}
int fp8_quantize_rows(int M, int K, const void* X, int ldx, uint8_t* Xq, float* sx, void* stream) {
  return quantize_rows8(M, K, X, ldx, reinterpret_cast<int8_t*>(Xq), sx, stream, 1);
}

int int8_gemm_raw(int M, int N, int K, const int8_t* Xq, int ldxq, const int8_t* Wq, int ldwq, int32_t* C, int ldc,
                  void* stream) {
  if (!nonnull({Wq}) || (M > 0 && !nonnull({Xq, C}))) return LDL_E_INVAL;
  if (M < 0 || N <= 0 || K <= 0) return LDL_E_INVAL;
  if (N % 64 || K % 128 || !al({Xq, Wq, C})) return LDL_E_UNSUPPORTED;
  LDL_LD(ldxq, K, 16); LDL_LD(ldwq, K, 16); LDL_LD(ldc, N, 4);
  if (!fits(M, ldxq, 1) || !fits(N, ldwq, 1) || !fits(M, ldc, 4)) return LDL_E_UNSUPPORTED;
  GemmParams p = gp0();
  p.M = M; p.N = N; p.K = K; p.a = Xq; p.lda = ldxq; p.b0 = Wq; p.ldb = ldwq; p.kseg = K;
  p.out = C; p.ldo = ldc;
  LDL_TRY(launch_gemm(GK_NT_I8_RAW, p, S(stream)));
  return LDL_OK;
}

static int lora8_fwd(int fp8, int M, int N, int K, int r, float s, const void* X, int ldx, const int8_t* Wq, int ldw,
                     const float* sw, const void* A, const void* B, const void* bias, void* Y, int ldy,
                     int8_t* Xq_save, float* sx_save, float* U_save, int ldu, void* ws, size_t ws_bytes,
                     void* stream) {
  if (!nonnull({Wq, sw, A, B}) || (M > 0 && !nonnull({X, Y}))) return LDL_E_INVAL;
  if ((Xq_save == nullptr) != (sx_save == nullptr)) return LDL_E_INVAL;
  const int chk = check_bf16_layer(M, N, K, r);
  if (chk != LDL_OK) return chk;
  if (K % 128) return LDL_E_UNSUPPORTED;
  if (fp8 && (N % 128 || r % 8 || r > 64)) return LDL_E_UNSUPPORTED;
  LDL_LD(ldx, K, 8); LDL_LD(ldw, K, 16); LDL_LD(ldy, N, 8); LDL_LD(ldu, r, 4);
  if (!fits(M, ldx, 2) || !fits(N, ldw, 1) || !fits(M, ldy, 2) || !fits(M, ldu, 4)) return LDL_E_UNSUPPORTED;
  if (!al({X, Wq, sw, A, B, bias, Y, Xq_save, sx_save, U_save, ws})) return LDL_E_UNSUPPORTED;
  if (ws_base(LDL_OP_W8A8_FWD, M, N, K, r, LDL_BF16) > ws_bytes) return LDL_E_WORKSPACE;
  if (!ws) return LDL_E_INVAL;
  if (M == 0) return LDL_OK;
  const hipStream_t st = S(stream);
  Bump wb(ws);
  float* Uw = wb.take<float>((size_t)M * r);
  int8_t* Xqw = wb.take<int8_t>((size_t)M * K);
  float* sxw = wb.take<float>((size_t)M);
  float* U = U_save ? U_save : Uw;
  const int lu = U_save ? ldu : r;
  int8_t* Xq = Xq_save ? Xq_save : Xqw;
  float* sx = sx_save ? sx_save : sxw;
  LDL_TRY(launch_quantize_rows(X, 0, M, K, ldx, Xq, sx, st, fp8));
  LDL_TRY(rowproj(M, K, r, X, ldx, A, nullptr, r, K, U, lu, 1.f, st));
  GemmParams p = gp0();
  p.M = M; p.N = N; p.K = K;
  p.a = Xq; p.lda = K; p.b0 = Wq; p.ldb = ldw; p.kseg = K;
  p.row_scale = sx; p.col_scale = sw;
  p.S = U; p.ld_s = lu; p.r_epi = r; p.s_epi = s;
  p.e0 = B; p.e1 = B; p.e_ldn = r; p.e_ldj = 1; p.e_jsplit = r;
  p.bias = bias; p.out = Y; p.ldo = ldy;
  p.part = split_part(wb, ws, ws_bytes, ws_split(LDL_OP_W8A8_FWD, M, N, K, LDL_BF16));
  LDL_TRY(gemm_timed(0, fp8 ? GK_NT_F8_DEQ : GK_NT_I8_DEQ, p, st));
  return LDL_OK;
}

int w8a8_lora_linear_fwd(int M, int N, int K, int r, float s, const void* X, int ldx, const int8_t* Wq, int ldw,
                         const float* sw, const void* A, const void* B, const void* bias, void* Y, int ldy,
                         int8_t* Xq_save, float* sx_save, float* U_save, int ldu, void* ws, size_t ws_bytes,
                         void* stream) {
  return lora8_fwd(0, M, N, K, r, s, X, ldx, Wq, ldw, sw, A, B, bias, Y, ldy, Xq_save, sx_save, U_save, ldu, ws,
                   ws_bytes, stream);
}

int fp8_lora_linear_fwd(int M, int N, int K, int r, float s, const void* X, int ldx, const uint8_t* Wq, int ldw,
                        const float* sw, const void* A, const void* B, const void* bias, void* Y, int ldy,
                        uint8_t* Xq_save, float* sx_save, float* U_save, int ldu, void* ws, size_t ws_bytes,
                        void* stream) {
  return lora8_fwd(1, M, N, K, r, s, X, ldx, reinterpret_cast<const int8_t*>(Wq), ldw, sw, A, B, bias, Y, ldy,
                   reinterpret_cast<int8_t*>(Xq_save), sx_save, U_save, ldu, ws, ws_bytes, stream);
}

static int lora8_bwd(int fp8, int M, int N, int K, int r, float s, const void* dY, int lddy, const void* X, int ldx,
                     const int8_t* Wq, int ldw, const float* sw, const void* A, const void* B,
                     const float* U_saved, int ldu, void* dX, int lddx, float* dA, float* dB, void* ws,
                     size_t ws_bytes, void* stream) {
  if (!nonnull({Wq, sw, A, B, dA, dB, ws}) || (M > 0 && !nonnull({dY, X}))) return LDL_E_INVAL;
  const int chk = check_bf16_layer(M, N, K, r);
  if (chk != LDL_OK) return chk;
  LDL_LD(lddy, N, 8); LDL_LD(ldx, K, 8); LDL_LD(ldw, K, 16); LDL_LD(ldu, r, 4); LDL_LD(lddx, K, 8);
  if (!fits(M, lddy, 2) || !fits(M, ldx, 2) || !fits(N, ldw, 1) || !fits(M, ldu, 4) || !fits(M, lddx, 2))
    return LDL_E_UNSUPPORTED;
  if (!al({dY, X, Wq, sw, A, B, U_saved, dX, dA, dB, ws})) return LDL_E_UNSUPPORTED;
  if (ws_base(LDL_OP_W8A8_BWD, M, N, K, r, LDL_BF16) > ws_bytes) return LDL_E_WORKSPACE;
  const hipStream_t st = S(stream);
  if (M == 0) {
    LDL_TRY(zero(dA, (size_t)r * K, st));
    LDL_TRY(zero(dB, (size_t)N * r, st));
    return LDL_OK;
  }
  Bump wb(ws);
  LoraBwdWs w = plan_lora_bwd(wb, M, N, K, r, true);
  const float* U = U_saved;
  int lu = ldu;
  if (!U) {
    LDL_TRY(rowproj(M, K, r, X, ldx, A, nullptr, r, K, w.U, r, 1.f, st));
    U = w.U;
    lu = r;
  }
  LDL_TRY(rowproj_t(M, N, r, dY, lddy, B, r, nullptr, w.V, r, 1.f, st));
  if (dX) {
    GemmParams p = gp0();
    p.M = M; p.N = K; p.K = N;
    p.a = dY; p.lda = lddy; p.a_colscale = sw; p.b0 = Wq; p.b1 = Wq; p.ldb = ldw; p.kseg = N;
    p.S = w.V; p.ld_s = r; p.r_epi = r; p.s_epi = s;
    p.e0 = A; p.e1 = A; p.e_ldn = 1; p.e_ldj = K; p.e_jsplit = r;
    p.out = dX; p.ldo = lddx; p.q_fp8 = fp8;
    if (M >= kDequantRows) {
      // diag(sw).Wq in bf16 (the same rounding as the widening in the tile), then the plain product
      uint16_t* Wd = wb.take<uint16_t>((size_t)N * K);
      LDL_TRY(launch_dequant8(Wq, N, K, ldw, sw, fp8, Wd, st));
      p.a_colscale = nullptr; p.b0 = Wd; p.b1 = Wd; p.ldb = K;
      p.part = split_part(wb, ws, ws_bytes, ws_split(LDL_OP_W8A8_BWD, M, N, K, LDL_BF16));
      LDL_TRY(gemm_timed(1, GK_NN_PLAIN, p, st));
    } else {
      LDL_TRY(gemm_timed(1, GK_NN_I8_SCALE, p, st));
    }
  }
  LDL_TRY(launch_colproj2(
      pk(cpp(M, N, r, dY, lddy, U, lu, 1.f, nullptr, 0, 0, w.msB, w.partB, nullptr), w.pkB), w.nsB,
      pk(cpp(M, K, r, X, ldx, w.V, r, 1.f, nullptr, 0, 0, w.msA, w.partA, nullptr), w.pkA), w.nsA, st));
  LDL_TRY(launch_reduce2(rdp(N, r, w.partB, (size_t)N * w.rp, w.nsB, w.rp, false, s, dB, r),
                         rdp(r, K, w.partA, (size_t)K * w.rp, w.nsA, w.rp, true, s, dA, K), st));
  return LDL_OK;
}

int w8a8_lora_linear_bwd(int M, int N, int K, int r, float s, const void* dY, int lddy, const void* X, int ldx,
                         const int8_t* Wq, int ldw, const float* sw, const void* A, const void* B,
                         const float* U_saved, int ldu, void* dX, int lddx, float* dA, float* dB, void* ws,
                         size_t ws_bytes, void* stream) {
  return lora8_bwd(0, M, N, K, r, s, dY, lddy, X, ldx, Wq, ldw, sw, A, B, U_saved, ldu, dX, lddx, dA, dB, ws,
                   ws_bytes, stream);
}

int fp8_lora_linear_bwd(int M, int N, int K, int r, float s, const void* dY, int lddy, const void* X, int ldx,
                        const uint8_t* Wq, int ldw, const float* sw, const void* A, const void* B,
                        const float* U_saved, int ldu, void* dX, int lddx, float* dA, float* dB, void* ws,
                        size_t ws_bytes, void* stream) {
  return lora8_bwd(1, M, N, K, r, s, dY, lddy, X, ldx, reinterpret_cast<const int8_t*>(Wq), ldw, sw, A, B, U_saved,
                   ldu, dX, lddx, dA, dB, ws, ws_bytes, stream);
}

}  // extern "C"
