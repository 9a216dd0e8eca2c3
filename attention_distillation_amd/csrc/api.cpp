// C ABI of the KVSculpt library: argument checks, workspace carving and the
// host-side schedule that enqueues the HIP kernels on the context's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/kvsculpt.h"
#include "kvs_internal.h"
#include "plan.h"

namespace kvs {
enum ProfClass {
  PROF_FWD, PROF_BWD, PROF_GRAM, PROF_POTRF, PROF_TRAIL, PROF_BACK, PROF_HIST, PROF_DIR,
  PROF_IMP, PROF_REF, PROF_MERGE, PROF_QUERIES, PROF_USE, PROF_PV, PROF_DIGITS, PROF_RESID, PROF_FSUB,
  PROF_GRAM_SPLIT, PROF_RESID_SPLIT, PROF_BWD_SPLIT, PROF_NCLASS
};
const char* const kProfNames[PROF_NCLASS] = {
    "attn_fwd", "attn_bwd", "gram", "potrf_panel", "trailing", "back_subst", "hist_dots",
    "direction", "importance", "ref_attn_fwd", "merge", "build_queries", "use_attn_fwd", "attn_pv",
    "key_digits", "resid_rhs", "fwd_subst", "gram_split", "resid_rhs_split", "attn_bwd_split"};
struct ProfRec {
  int cls;
  hipEvent_t a, b;
  double flops, bytes;
};
struct ProfAcc {
  long long launches = 0;
  double ms = 0, flops = 0, bytes = 0;
};
}  // namespace kvs

struct kvs_ctx_s {
  hipStream_t stream = nullptr;
  std::string err;
  int device = 0;
  int lds_max = 0;          // dynamic LDS bytes per workgroup on this device
  int logit_mode = kvs::LOGIT_I8;   // score arithmetic of the loss forwards
  bool refine_resolves = true;      // refinement step after the schedule's value re-solves
  bool gram_split3 = true;          // large-batch Gram tiles on bf16 MFMA over exact three-piece splits
  int gram_tile256 = 1;             // those tiles 256x256: 0 never, 1 for >= 2048 of them, 2 always
  bool resid_split3 = true;         // refinement residual A^T G on split bf16 products
  bool bwd_split3 = true;           // backward on split bf16 products
  bool prof = false;
  int prof_mask = 0;
  std::vector<hipEvent_t> pool;
  std::vector<kvs::ProfRec> pending;
  kvs::ProfAcc acc[kvs::PROF_NCLASS];
  // pinned host copies of the per-problem status (two buffers of hstat_cap
  // entries) and their completion events, for the pipelined block schedule
  int* hstat = nullptr;
  int hstat_cap = 0;
  hipEvent_t sev[2] = {nullptr, nullptr};
  // device address of this device's copy of the static scratch array (null
  // if it could not be taken; scratch_err says why)
  void* scratch = nullptr;
  std::string scratch_err;
  ~kvs_ctx_s() {
    for (auto& r : pending) { pool.push_back(r.a); pool.push_back(r.b); }
    for (auto e : pool) hipEventDestroy(e);
    if (hstat) {
      hipStreamSynchronize(stream);   // a status copy may still target it
      hipHostFree(hstat);
    }
    for (auto e : sev)
      if (e) hipEventDestroy(e);
  }
};

namespace kvs {

// Scratch memory of the allocation-free entry point (kvs_value_norms_noalloc):
// a file-scope device array, one copy per GPU the library runs on, held until
// the process ends.  In host code its name is only a stand-in: the device
// address of each GPU's copy is taken once per device with that device
// current, and only that address is handed to kernels.
constexpr size_t kNoAllocScratchBytes = size_t(1) << 20;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;        // by device ordinal; null until taken

// Address of the current device's scratch copy (dev must be current).
hipError_t scratch_address(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (dev < 0) return hipErrorInvalidDevice;
  if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

kvs_status fail(kvs_ctx c, kvs_status code, const char* fmt, ...) {
  if (c) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    c->err = buf;
  }
  return code;
}

kvs_status hip_check(kvs_ctx c, const char* where) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(c, KVS_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
  return KVS_OK;
}

hipEvent_t prof_event(kvs_ctx c) {
  if (!c->pool.empty()) {
    hipEvent_t e = c->pool.back();
    c->pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Fold the timings of completed launches into the per-class totals; launches
// still in flight (the schedule drains right after a status copy while the
// next slot runs) stay pending until a later drain.
void prof_drain(kvs_ctx c) {
  const hipError_t before = hipPeekAtLastError();
  size_t keep = 0;
  for (size_t i = 0; i < c->pending.size(); ++i) {
    ProfRec r = c->pending[i];
    float ms = 0.f;
    const hipError_t e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e == hipErrorNotReady) {
      c->pending[keep++] = r;
      continue;
    }
    if (e == hipSuccess) {
      ProfAcc& a = c->acc[r.cls];
      a.launches += 1;
      a.ms += ms;
      a.flops += r.flops;
      a.bytes += r.bytes;
    }
    c->pool.push_back(r.a);
    c->pool.push_back(r.b);
  }
  c->pending.resize(keep);
  // an unfinished event is not an error of the caller's work
  if (before == hipSuccess && hipPeekAtLastError() == hipErrorNotReady) (void)hipGetLastError();
}

// RAII timer around one kernel launch on the context stream (no-op unless
// profiling is enabled).
struct Prof {
  kvs_ctx c;
  ProfRec r{};
  bool on;
  Prof(kvs_ctx ctx, int cls, double flops, double bytes)
      : c(ctx), on(ctx->prof && ((ctx->prof_mask >> cls) & 1)) {
    if (!on) return;
    r.cls = cls; r.flops = flops; r.bytes = bytes;
    r.a = prof_event(c);
    r.b = prof_event(c);
    if (!r.a || !r.b) { on = false; return; }
    hipEventRecord(r.a, c->stream);
  }
  ~Prof() {
    if (!on) return;
    hipEventRecord(r.b, c->stream);
    c->pending.push_back(r);
  }
};

// Algorithmic work of the contraction kernels over the active problems.
// want < 0: the active set is not known at launch (device-driven slots);
// the work is added afterwards from the per-problem trial counters.
double sum_k(const Plan& pl, const std::vector<int>* hs, int want) {
  double s = 0;
  if (want < 0) return 0;
  for (int p = 0; p < pl.P; ++p)
    if (!hs || (*hs)[p] == want) s += pl.info[p].k;
  return s;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

#define KVS_NEED(ptr)                                                                   \
  do {                                                                                  \
    if (!(ptr)) return fail(ctx, KVS_ERR_INVALID, "%s: argument '%s' is NULL", fn, #ptr); \
    if (!aligned((ptr), 16)) return fail(ctx, KVS_ERR_ALIGN, "%s: '%s' not 16-byte aligned", fn, #ptr); \
  } while (0)
#define KVS_OPT(ptr)                                                                    \
  do {                                                                                  \
    if ((ptr) && !aligned((ptr), 16)) return fail(ctx, KVS_ERR_ALIGN, "%s: '%s' not 16-byte aligned", fn, #ptr); \
  } while (0)

kvs_status prepare(kvs_ctx ctx, const char* fn, const kvs_batch* b, const kvs_opts* o, void* ws,
                   size_t ws_bytes, Plan* pl) {
  if (!ctx) return KVS_ERR_INVALID;
  ctx->err.clear();
  std::string e = make_plan(b, o, pl);
  if (!e.empty()) return fail(ctx, KVS_ERR_INVALID, "%s: %s", fn, e.c_str());
  if (!ws) return fail(ctx, KVS_ERR_INVALID, "%s: workspace is NULL", fn);
  if (!aligned(ws, 256)) return fail(ctx, KVS_ERR_ALIGN, "%s: workspace not 256-byte aligned", fn);
  if (ws_bytes < pl->ws_bytes)
    return fail(ctx, KVS_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, pl->ws_bytes);
  launch_write_info(at<ProbInfo>(ws, pl->r_info), pl->info.data(), pl->P, ctx->stream);
  launch_fill_i32(at<int>(ws, pl->r_cnt), 0, 2LL * pl->P, ctx->stream);
  CholArgs c{};
  c.info = at<ProbInfo>(ws, pl->r_info); c.coff = at<int>(ws, pl->r_coff);
  c.P = pl->P; c.kpadmax = pl->kpadmax; c.S = pl->chol_S;
  launch_chol_offsets(c, pl->d, ctx->stream);
  return KVS_OK;
}

// ---------------------------------------------------------------- building blocks

// Reference attention over the compress zone (uniform Z keys per problem).
void run_reference(kvs_ctx ctx, const Plan& pl, const kvs_batch* b, const float* Q, const float* Kz,
                   const float* Vz, float* Y, float* lse, void* ws) {
  FwdArgs f{};
  f.Q = Q; f.K = Kz; f.V = Vz; f.st = nullptr; f.active_mask = 0;
  f.shift = nullptr; f.St = nullptr;
  f.Opart = at<float>(ws, pl.r_Opart); f.Mpart = at<float>(ws, pl.r_Mpart); f.Lpart = at<float>(ws, pl.r_Lpart);
  f.info = nullptr; f.P = pl.P; f.n = pl.n; f.C = pl.Cref; f.kuni = pl.Z; f.kmax = pl.Z; f.scale = b->scale;
  {
    Prof pr(ctx, PROF_REF, 4.0 * pl.n * pl.Z * pl.d * pl.P, 4.0 * pl.P * (2.0 * pl.n * pl.d + 2.0 * pl.Z * pl.d));
    launch_attn_fwd(f, pl.d, LOGIT_F32, ctx->stream);
  }
  MergeArgs m{};
  m.Opart = f.Opart; m.Mpart = f.Mpart; m.Lpart = f.Lpart; m.st = nullptr; m.active_mask = 0;
  m.Yout = Y; m.lse_out = lse; m.P = pl.P; m.n = pl.n; m.C = pl.Cref; m.lambda = b->lambda;
  launch_merge(m, pl.d, false, ctx->stream);
}

// Forward at keys K (+ alpha * dir when dir != NULL) for problems selected by
// (st, mask): stores shifted scores, merges, writes G / e / crow and the loss
// partials, then finalises per-problem losses in the given mode.
// reuse_scores: the keys have not moved since the last forward of every
// selected problem stored its scores (only the values changed), so the
// scores are read back instead of formed again.
void run_forward(kvs_ctx ctx, const Plan& pl, const kvs_batch* b, const float* Q, const float* Y,
                 const float* lse, const float* K, const float* V, LbState* st,
                 int mask, int fin_mode, float* loss, float* mse, const kvs_opts* o, void* ws,
                 const std::vector<int>* hs = nullptr, int want = 0, bool reuse_scores = false) {
  FwdArgs f{};
  f.Q = Q; f.K = K; f.V = V; f.st = st; f.active_mask = mask;
  f.shift = lse;
  f.St = reuse_scores ? nullptr : at<float>(ws, pl.r_St);
  f.Sload = reuse_scores ? at<float>(ws, pl.r_St) : nullptr;
  f.Opart = at<float>(ws, pl.r_Opart); f.Mpart = at<float>(ws, pl.r_Mpart); f.Lpart = at<float>(ws, pl.r_Lpart);
  f.info = at<ProbInfo>(ws, pl.r_info); f.P = pl.P; f.n = pl.n; f.C = pl.C; f.kuni = 0; f.kmax = pl.kmax;
  f.scale = b->scale;
  {
    const double ks = sum_k(pl, hs, want);
    const double np = hs ? 0 : pl.P;
    if (reuse_scores) {
      Prof pr(ctx, PROF_PV, 2.0 * pl.n * pl.d * ks,
              4.0 * (ks * pl.d + ks * pl.npad + (np ? np : 1) * pl.n * pl.d));
      launch_attn_fwd(f, pl.d, ctx->logit_mode, ctx->stream);
    } else {
      if (ctx->logit_mode == LOGIT_I8) {
        // digit planes of the keys (all rows; only the selected problems read them)
        f.K8 = at<int>(ws, pl.r_K8); f.Kscl = at<float>(ws, pl.r_Kscl); f.k8rows = pl.ktot;
        Prof pr(ctx, PROF_DIGITS, 0.0, (double)pl.ktot * pl.d * (4.0 + kDigits) + 4.0 * pl.ktot);
        launch_digit_rows(K, pl.ktot, pl.d, const_cast<int*>(f.K8), const_cast<float*>(f.Kscl), ctx->stream);
      }
      Prof pr(ctx, PROF_FWD, 4.0 * pl.n * pl.d * ks,
              4.0 * (ks * pl.d * 2.0 + ks * pl.npad + (np ? np : 1) * pl.n * pl.d));
      launch_attn_fwd(f, pl.d, ctx->logit_mode, ctx->stream);
    }
  }
  MergeArgs m{};
  m.Opart = f.Opart; m.Mpart = f.Mpart; m.Lpart = f.Lpart; m.st = st; m.active_mask = mask;
  m.Y = Y; m.lse = lse; m.G = at<float>(ws, pl.r_G); m.e = at<float>(ws, pl.r_e);
  m.crow = at<float>(ws, pl.r_crow); m.part = at<double>(ws, pl.r_part);
  m.counter = at<unsigned>(ws, pl.r_cnt);
  m.P = pl.P; m.n = pl.n; m.C = pl.C; m.lambda = b->lambda;
  m.fin_mode = fin_mode; m.c1 = o ? o->c1 : 1e-4; m.shrink = o ? o->shrink : 0.5;
  m.max_bt = o ? o->max_backtracks : 30; m.loss = loss; m.mse = mse;
  m.status_view = at<int>(ws, pl.r_status);
  {
    Prof pr(ctx, PROF_MERGE, 0, 0);
    launch_merge(m, pl.d, true, ctx->stream);
  }
}

// Backward from the last forward's stored scores: split-n partials of dL/dKc
// (reduced by the gradient pass that follows).
void run_backward(kvs_ctx ctx, const Plan& pl, const kvs_batch* b, const float* Q, const float* V,
                  LbState* st, int mask, void* ws, const std::vector<int>* hs = nullptr, int want = 0) {
  BwdArgs bw{};
  bw.Q = Q; bw.St = at<float>(ws, pl.r_St); bw.G = at<float>(ws, pl.r_G); bw.e = at<float>(ws, pl.r_e);
  bw.crow = at<float>(ws, pl.r_crow); bw.K = nullptr; bw.V = V; bw.st = st; bw.active_mask = mask;
  bw.dKpart = at<float>(ws, pl.r_dK); bw.info = at<ProbInfo>(ws, pl.r_info);
  bw.P = pl.P; bw.n = pl.n; bw.Cn = pl.Cn; bw.kmax = pl.kmax; bw.ktot = (int)pl.ktot;
  bw.split3 = ctx->bwd_split3 ? 1 : 0;
  {
    const double ks = sum_k(pl, hs, want);
    Prof pr(ctx, bw.split3 ? PROF_BWD_SPLIT : PROF_BWD, 4.0 * pl.n * pl.d * ks, 4.0 * (ks * pl.npad + ks * pl.d * (1.0 + pl.Cn)));
    launch_attn_bwd(bw, pl.d, ctx->stream);
  }
}

GradUpdArgs grad_args(const Plan& pl, const kvs_batch* b, void* ws, LbState* st, int mask, int mode) {
  GradUpdArgs g{};
  g.dKpart = at<float>(ws, pl.r_dK); g.Cn = pl.Cn; g.scale = b->scale; g.st = st; g.active_mask = mask;
  g.mode = mode; g.info = at<ProbInfo>(ws, pl.r_info); g.P = pl.P; g.d = pl.d; g.ktot = (int)pl.ktot;
  g.nch = pl.nchv;
  return g;
}

// Inputs of the forward that the refinement step of a value solve repeats.
struct RefineIn {
  const float* Q; const float* lse; const float* Kc;
};

// Ridge value solve from the last forward's stored scores (St, e): Gram with
// the A^T Y rows, fixed-order reduction, mu, panel Cholesky, back solve.
// With ref (every problem active, no state), one refinement step follows:
// G = 2 (A Vc - Y) from the stored scores, r = -A^T G / 2 - mu Vc in fp64,
// Vc += (L L^T)^-1 r with the same factor.
void run_value_solve(kvs_ctx ctx, const Plan& pl, const kvs_batch* b, const float* Y, float* Vc,
                     int* flags, LbState* st, int mask, void* ws, const RefineIn* ref = nullptr) {
  float* M = at<float>(ws, pl.r_M);
  // kernels that read the status only to select problems skip that load
  // when every status is selected
  LbState* sel = (mask == kAllStates) ? nullptr : st;
  GramArgs g{};
  g.St = at<float>(ws, pl.r_St); g.e = at<float>(ws, pl.r_e); g.Y = Y; g.st = sel; g.active_mask = mask;
  g.Mpart = pl.Cg > 1 ? at<float>(ws, pl.r_Mg) : M; g.info = at<ProbInfo>(ws, pl.r_info);
  g.P = pl.P; g.n = pl.n; g.Cg = pl.Cg; g.kpadmax = pl.kpadmax; g.mtot = pl.mtot; g.gtot = pl.gtot;
  g.gtot4 = pl.gtot4;
  g.split3 = ctx->gram_split3 ? 1 : 0;
  g.tile256 = ctx->gram_tile256;
  {
    double fl = 0, by = 0;
    for (const auto& q : pl.info) {
      fl += (double)pl.n * q.k * (q.k + 1) + 2.0 * pl.n * q.k * pl.d;
      by += 4.0 * ((double)q.k * pl.npad + (double)pl.n * pl.d + (double)(q.kpad + pl.d) * q.kpad * pl.Cg);
    }
    Prof pr(ctx, gram_split_products(g) ? PROF_GRAM_SPLIT : PROF_GRAM, fl, by);
    launch_gram(g, pl.d, ctx->stream);
  }
  GramReduceArgs r{};
  r.Mpart = g.Mpart; r.M = M; r.trpart = at<double>(ws, pl.r_tr); r.st = sel; r.active_mask = mask;
  r.info = g.info; r.P = pl.P; r.Cg = pl.Cg; r.kpadmax = pl.kpadmax; r.mtot = pl.mtot;
  launch_gram_reduce(r, pl.d, ctx->stream);
  CholArgs c{};
  c.M = M; c.Dinv = at<float>(ws, pl.r_Dinv); c.trpart = r.trpart; c.mu = at<double>(ws, pl.r_mu); c.info_out = at<int>(ws, pl.r_cinfo);
  c.st = sel; c.active_mask = mask; c.info = g.info; c.P = pl.P; c.kpadmax = pl.kpadmax;
  c.ridge_rel = b->ridge_rel; c.coff = at<int>(ws, pl.r_coff); c.S = pl.chol_S;
  launch_mu(c, ctx->stream);
  const int KT = pl.kpadmax / kTile;
  for (int j = -1; j < KT; ++j) {
    Prof pr(ctx, PROF_POTRF, 0, 0);
    launch_chol_step(c, pl.d, j, pl.chol_wgs[j + 1], ctx->stream);
  }
  BackArgs bk{};
  bk.M = M; bk.X = at<float>(ws, pl.r_X); bk.Dinv = c.Dinv; bk.Vc = Vc;
  bk.info_out = c.info_out; bk.flags = flags; bk.st = st; bk.active_mask = mask; bk.info = g.info;
  bk.P = pl.P; bk.d = pl.d; bk.kpadmax = pl.kpadmax; bk.lds_max = ctx->lds_max;
  {
    double fl = 0;
    for (const auto& q : pl.info) fl += 1.0 * q.kpad * q.kpad * pl.d;
    Prof pr(ctx, PROF_BACK, fl, 0);
    launch_back_subst(bk, pl.d, ctx->stream);
  }
  if (!ref) return;
  run_forward(ctx, pl, b, ref->Q, Y, ref->lse, ref->Kc, Vc, nullptr, 0, 0, nullptr, nullptr, nullptr,
              ws, nullptr, 0, true);
  RhsArgs ra{};
  ra.St = g.St; ra.e = g.e; ra.G = at<float>(ws, pl.r_G); ra.info = g.info;
  ra.Rpart = at<double>(ws, pl.r_R); ra.xtot = pl.kpadtot * pl.d;
  ra.P = pl.P; ra.n = pl.n; ra.Cr = pl.Crf; ra.kpadmax = pl.kpadmax;
  ra.split3 = ctx->resid_split3 ? 1 : 0;
  {
    double ks = 0;
    for (const auto& q : pl.info) ks += q.k;
    Prof pr(ctx, ra.split3 ? PROF_RESID_SPLIT : PROF_RESID, 2.0 * pl.n * pl.d * ks,
            4.0 * (ks * pl.npad + (double)pl.P * pl.n * (pl.d + 1)));
    launch_resid_rhs(ra, pl.d, ctx->stream);
  }
  FsubArgs fa{};
  fa.Rpart = ra.Rpart; fa.xtot = ra.xtot; fa.Cr = ra.Cr; fa.mu = c.mu; fa.Vc = Vc; fa.M = M;
  fa.Dinv = c.Dinv; fa.X = bk.X; fa.info_out = c.info_out; fa.info = g.info; fa.P = pl.P;
  fa.kpadmax = pl.kpadmax; fa.lds_max = ctx->lds_max;
  {
    double fl = 0;
    for (const auto& q : pl.info) fl += 1.0 * q.kpad * q.kpad * pl.d;
    Prof pr(ctx, PROF_FSUB, fl, 0);
    launch_fwd_subst(fa, pl.d, ctx->stream);
  }
  bk.accumulate = 1;
  bk.flags = nullptr;
  {
    double fl = 0;
    for (const auto& q : pl.info) fl += 1.0 * q.kpad * q.kpad * pl.d;
    Prof pr(ctx, PROF_BACK, fl, 0);
    launch_back_subst(bk, pl.d, ctx->stream);
  }
}

// Select+Fit: importance, top-k, gather, then the ridge fit at the selected keys.
void run_init_topk(kvs_ctx ctx, const Plan& pl, const kvs_batch* b, const float* Q, const float* Kz,
                   const float* Y, const float* lse, int* idx, float* Kc, float* Vc, int* flags,
                   LbState* st, void* ws, bool refine = false) {
  ImpArgs ia{};
  ia.Q = Q; ia.Kz = Kz; ia.lse = lse;
  ia.Mpart = at<float>(ws, pl.r_imp);
  ia.Spart = ia.Mpart + (size_t)pl.Cq * pl.P * pl.Z;
  ia.P = pl.P; ia.n = pl.n; ia.Z = pl.Z; ia.Cq = pl.Cq; ia.scale = b->scale;
  {
    Prof pr(ctx, PROF_IMP, 2.0 * pl.n * pl.Z * pl.d * pl.P, 4.0 * pl.P * ((double)pl.n * pl.d + (double)pl.Z * pl.d));
    launch_importance(ia, pl.d, ctx->stream);
  }
  TopkArgs ta{};
  ta.Mpart = ia.Mpart; ta.Spart = ia.Spart; ta.Kz = Kz; ta.idx = idx; ta.Kc = Kc;
  ta.info = at<ProbInfo>(ws, pl.r_info); ta.P = pl.P; ta.Z = pl.Z; ta.Cq = pl.Cq; ta.d = pl.d;
  launch_topk(ta, ctx->stream);
  launch_fill_f32(Vc, 0.f, (long long)pl.ktot * pl.d, ctx->stream);
  run_forward(ctx, pl, b, Q, Y, lse, Kc, Vc, nullptr, 0, 0, nullptr, nullptr, nullptr, ws);
  const RefineIn rin{Q, lse, Kc};
  run_value_solve(ctx, pl, b, Y, Vc, flags, st, kAllStates, ws, refine ? &rin : nullptr);
}

constexpr int kAll = kAllStates;

struct LbBuffers {
  LbState* st;
  float *g, *p, *S, *Yh;
  double* hpart;
  int* status_view;
};

LbBuffers lb_in_ws(const Plan& pl, void* ws) {
  return LbBuffers{at<LbState>(ws, pl.r_state), at<float>(ws, pl.r_g), at<float>(ws, pl.r_p),
                   at<float>(ws, pl.r_S), at<float>(ws, pl.r_Yh), at<double>(ws, pl.r_hpart),
                   at<int>(ws, pl.r_status)};
}

LbBuffers lb_in_state(const Plan& pl, void* state, void* ws) {
  return LbBuffers{at<LbState>(state, pl.s_state), at<float>(state, pl.s_g), at<float>(state, pl.s_p),
                   at<float>(state, pl.s_S), at<float>(state, pl.s_Yh), at<double>(ws, pl.r_hpart),
                   at<int>(ws, pl.r_status)};
}

// History inner products and the scalar L-BFGS logic; with grad set, the
// gradient pass (reduction of the backward's split partials, and for an
// accepted step the move of Kc and the staged pair) runs in the same kernel.
void lb_dots(kvs_ctx ctx, const Plan& pl, const kvs_batch* b, const LbBuffers& B, void* ws, int mode,
             int mask, bool grad, float* Kc, int target = 0x7fffffff) {
  DotsArgs d{};
  d.target = target; d.status_view = B.status_view;
  d.grad = grad ? 1 : 0; d.dKpart = at<float>(ws, pl.r_dK); d.Cn = pl.Cn; d.gscale = b->scale;
  d.x = Kc; d.pdir = B.p;
  d.g = B.g; d.S = B.S; d.Yh = B.Yh; d.st = B.st; d.active_mask = mask; d.mode = mode;
  d.history = pl.H; d.curv_eps = 1e-10; d.part = B.hpart; d.counter = at<unsigned>(ws, pl.r_cnt) + pl.P;
  d.info = at<ProbInfo>(ws, pl.r_info); d.P = pl.P; d.d = pl.d; d.ktot = (int)pl.ktot; d.nch = pl.nchd;
  Prof pr(ctx, PROF_HIST, 0, 0);
  launch_dots(d, ctx->stream);
}

// Loss and gradient at the current keys for every problem, then the
// L-BFGS bookkeeping: prep_mode 1 keeps the history, 2 clears it.
void lb_eval_at_x(kvs_ctx ctx, const Plan& pl, const kvs_batch* b, const kvs_opts* o, const float* Q,
                  const float* Y, const float* lse, float* Kc, const float* Vc, const LbBuffers& B,
                  int prep_mode, float* loss_out, float* mse_out, void* ws, bool reuse_scores = false) {
  run_forward(ctx, pl, b, Q, Y, lse, Kc, Vc, B.st, kAll, 2, loss_out, mse_out, o, ws, nullptr, 0,
              reuse_scores);
  run_backward(ctx, pl, b, Q, Vc, B.st, kAll, ws);
  lb_dots(ctx, pl, b, B, ws, prep_mode, kAll, true, Kc);
}

// One L-BFGS iteration for every problem: direction, backtracking Armijo
// rounds (the host reads the per-problem status after each round), then
// gradient at the accepted keys and the history update.  Returns a HIP error
// status; *any_fail reports a failed search (stored scores then stale).
kvs_status lb_iteration(kvs_ctx ctx, const Plan& pl, const kvs_batch* b, const kvs_opts* o,
                        const float* Q, const float* Y, const float* lse, float* Kc, const float* Vc,
                        const LbBuffers& B, void* ws, bool* any_fail, std::vector<int>& hs) {
  DirArgs da{};
  da.p = B.p; da.g = B.g; da.S = B.S; da.Yh = B.Yh; da.st = B.st; da.info = at<ProbInfo>(ws, pl.r_info);
  da.x = Kc; da.kt = at<float>(ws, pl.r_Kt);
  da.P = pl.P; da.d = pl.d; da.ktot = (int)pl.ktot; da.nch = pl.nchv;
  hs.resize(pl.P);
  *any_fail = false;
  for (int round = 0; round < o->max_backtracks; ++round) {
    {
      // direction on the first round; trial keys at the current step on every round
      Prof pr(ctx, PROF_DIR, 0, 0);
      launch_direction(da, ctx->stream);
    }
    run_forward(ctx, pl, b, Q, Y, lse, at<float>(ws, pl.r_Kt), Vc, B.st, 1 << ST_SEARCH, 1, nullptr, nullptr, o, ws,
                round ? &hs : nullptr, ST_SEARCH);
    if (hipMemcpyAsync(hs.data(), B.status_view, sizeof(int) * pl.P, hipMemcpyDeviceToHost,
                       ctx->stream) != hipSuccess ||
        hipStreamSynchronize(ctx->stream) != hipSuccess)
      return fail(ctx, KVS_ERR_HIP, "line search: %s", hipGetErrorString(hipGetLastError()));
    if (ctx->prof) prof_drain(ctx);
    bool searching = false;
    for (int v : hs) searching |= (v == ST_SEARCH);
    if (!searching) break;
  }
  bool any_accept = false;
  for (int v : hs) {
    *any_fail |= (v == ST_FAIL);
    any_accept |= (v == ST_ACCEPT);
  }
  if (any_accept) run_backward(ctx, pl, b, Q, Vc, B.st, 1 << ST_ACCEPT, ws, &hs, ST_ACCEPT);
  lb_dots(ctx, pl, b, B, ws, 0, (1 << ST_ACCEPT) | (1 << ST_FAIL), true, Kc);
  return KVS_OK;
}

// One device-driven slot of the L-BFGS schedule: every kernel acts only on
// the problems whose status asks for it, so a slot advances each problem by
// one step of its own state machine (direction and first trial, or a further
// trial; gradient and history after an accepted or failed search).  A slot
// needs no host decision, so slots are enqueued back to back.
void lb_slot(kvs_ctx ctx, const Plan& pl, const kvs_batch* b, const kvs_opts* o, const float* Q,
             const float* Y, const float* lse, float* Kc, const float* Vc, const LbBuffers& B, void* ws,
             int target) {
  DirArgs da{};
  da.p = B.p; da.g = B.g; da.S = B.S; da.Yh = B.Yh; da.st = B.st; da.info = at<ProbInfo>(ws, pl.r_info);
  da.x = Kc; da.kt = at<float>(ws, pl.r_Kt);
  da.P = pl.P; da.d = pl.d; da.ktot = (int)pl.ktot; da.nch = pl.nchv;
  {
    Prof pr(ctx, PROF_DIR, 0, 0);
    launch_direction(da, ctx->stream);
  }
  std::vector<int> none;
  run_forward(ctx, pl, b, Q, Y, lse, at<float>(ws, pl.r_Kt), Vc, B.st, 1 << ST_SEARCH, 1, nullptr, nullptr, o, ws, &none, -1);
  run_backward(ctx, pl, b, Q, Vc, B.st, 1 << ST_ACCEPT, ws, &none, -1);
  lb_dots(ctx, pl, b, B, ws, 0, (1 << ST_ACCEPT) | (1 << ST_FAIL), true, Kc, target);
}

// Contraction work of the device-driven slots, from the per-problem trial and
// accept counters (profiling only: one state read-back per call).
void prof_add_slot_work(kvs_ctx ctx, const Plan& pl, const LbState* st, const LbState* before) {
  if (!ctx->prof) return;
  std::vector<LbState> h(pl.P);
  if (hipMemcpyAsync(h.data(), st, sizeof(LbState) * pl.P, hipMemcpyDeviceToHost, ctx->stream) != hipSuccess ||
      hipStreamSynchronize(ctx->stream) != hipSuccess)
    return;
  double fw = 0, bw = 0;
  for (int p = 0; p < pl.P; ++p) {
    fw += (double)(h[p].n_trial - (before ? before[p].n_trial : 0)) * pl.info[p].k;
    bw += (double)(h[p].n_accept - (before ? before[p].n_accept : 0)) * pl.info[p].k;
  }
  ctx->acc[PROF_FWD].flops += 4.0 * pl.n * pl.d * fw;
  ctx->acc[ctx->bwd_split3 ? PROF_BWD_SPLIT : PROF_BWD].flops += 4.0 * pl.n * pl.d * bw;
}

// Two pinned status buffers of P entries and their events.
kvs_status status_buffers(kvs_ctx ctx, int P) {
  if (ctx->hstat_cap < P) {
    if (ctx->hstat) {
      if (hipStreamSynchronize(ctx->stream) != hipSuccess)
        return fail(ctx, KVS_ERR_HIP, "status buffers: %s", hipGetErrorString(hipGetLastError()));
      hipHostFree(ctx->hstat);
      ctx->hstat = nullptr;
      ctx->hstat_cap = 0;
    }
    if (hipHostMalloc((void**)&ctx->hstat, sizeof(int) * 2 * (size_t)P, hipHostMallocDefault) != hipSuccess)
      return fail(ctx, KVS_ERR_HIP, "status buffers: %s", hipGetErrorString(hipGetLastError()));
    ctx->hstat_cap = P;
  }
  for (auto& e : ctx->sev)
    if (!e && hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess)
      return fail(ctx, KVS_ERR_HIP, "status events: %s", hipGetErrorString(hipGetLastError()));
  return KVS_OK;
}

// The whole alternating schedule on the plan's batch.  Iterations run in
// blocks that end at the value solves: each block enqueues one slot per
// iteration; problems that needed extra line-search trials get further slots
// until every problem has done the block's iterations.  The status check is
// pipelined: after each copy of the per-problem status one more slot is
// enqueued before the host waits for that copy, so the device keeps working
// while the host decides (a slot leaves a problem that finished its block
// untouched, so the last of these slots runs empty).
// Starting point of a run: Select+Fit, or the caller's keys in Kc with
// ridge-fitted values.
void run_init(kvs_ctx ctx, const Plan& pl, const kvs_batch* b, const float* Q, const float* Kz,
              const float* Y, const float* lse, float* Kc, float* Vc, int* flags, LbState* st,
              bool keys_given, void* ws) {
  // the starting values take the refinement step of the standalone solve,
  // as do the re-solves every vc_every iterations
  if (!keys_given) {
    run_init_topk(ctx, pl, b, Q, Kz, Y, lse, at<int>(ws, pl.r_idx), Kc, Vc, flags, st, ws, true);
    return;
  }
  launch_fill_f32(Vc, 0.f, (long long)pl.ktot * pl.d, ctx->stream);
  run_forward(ctx, pl, b, Q, Y, lse, Kc, Vc, nullptr, 0, 0, nullptr, nullptr, nullptr, ws);
  const RefineIn rin{Q, lse, Kc};
  run_value_solve(ctx, pl, b, Y, Vc, flags, st, kAllStates, ws, &rin);
}

// Everything before the first iteration: reference attention into the
// workspace, the starting point, loss and gradient there with an empty
// history (the state lives in the workspace).
void compress_begin_impl(kvs_ctx ctx, const Plan& pl, const kvs_batch* b, const kvs_opts* o,
                         const float* Q, const float* Kz, const float* Vz, float* Kc, float* Vc,
                         float* init_loss, bool keys_given, void* ws) {
  float* Yr = at<float>(ws, pl.r_yref);
  float* lr = at<float>(ws, pl.r_lseref);
  run_reference(ctx, pl, b, Q, Kz, Vz, Yr, lr, ws);
  LbBuffers B = lb_in_ws(pl, ws);
  launch_state_init(B.st, pl.P, 1, ctx->stream);
  run_init(ctx, pl, b, Q, Kz, Yr, lr, Kc, Vc, nullptr, B.st, keys_given, ws);
  // the init's forward stored the scores at these keys
  lb_eval_at_x(ctx, pl, b, o, Q, Yr, lr, Kc, Vc, B, 2, init_loss, nullptr, ws, true);
}

// Iterations t_begin + 1 .. t_end of the schedule from the state in the
// workspace (t_begin is 0 or follows a value re-solve, so every problem is
// ready for a new search).  Ends with loss, flags and, when asked, the
// output MSE at the current pair.
kvs_status compress_advance_impl(kvs_ctx ctx, const Plan& pl, const kvs_batch* b, const kvs_opts* o,
                                 const float* Q, float* Kc, float* Vc, int t_begin, int t_end,
                                 float* loss, float* mse, int* flags, void* ws) {
  float* Yr = at<float>(ws, pl.r_yref);
  float* lr = at<float>(ws, pl.r_lseref);
  LbBuffers B = lb_in_ws(pl, ws);
  // trial and accept counters before this call, for the profile's work totals
  std::vector<LbState> before;
  if (ctx->prof) {
    before.resize(pl.P);
    if (hipMemcpyAsync(before.data(), B.st, sizeof(LbState) * pl.P, hipMemcpyDeviceToHost, ctx->stream) !=
            hipSuccess ||
        hipStreamSynchronize(ctx->stream) != hipSuccess)
      return fail(ctx, KVS_ERR_HIP, "schedule: %s", hipGetErrorString(hipGetLastError()));
  }
  bool refreshed = false;
  if (kvs_status s = status_buffers(ctx, pl.P); s != KVS_OK) return s;
  int* hbuf[2] = {ctx->hstat, ctx->hstat + pl.P};
  auto copy_status = [&](int i) {
    return hipMemcpyAsync(hbuf[i], B.status_view, sizeof(int) * pl.P, hipMemcpyDeviceToHost, ctx->stream) ==
               hipSuccess &&
           hipEventRecord(ctx->sev[i], ctx->stream) == hipSuccess;
  };
  int done = t_begin;
  while (done < t_end) {
    const int blk = std::min(o->vc_every - done % o->vc_every, t_end - done);
    int slots = 0;
    for (; slots < blk; ++slots) lb_slot(ctx, pl, b, o, Q, Yr, lr, Kc, Vc, B, ws, blk);
    bool any_fail = false;
    int cur = 0;                 // buffer holding the status after `slots` slots
    if (!copy_status(cur)) return fail(ctx, KVS_ERR_HIP, "schedule: %s", hipGetErrorString(hipGetLastError()));
    for (;;) {
      const int checked = slots;
      lb_slot(ctx, pl, b, o, Q, Yr, lr, Kc, Vc, B, ws, blk);
      ++slots;
      if (!copy_status(cur ^ 1) || hipEventSynchronize(ctx->sev[cur]) != hipSuccess)
        return fail(ctx, KVS_ERR_HIP, "schedule: %s", hipGetErrorString(hipGetLastError()));
      if (ctx->prof) prof_drain(ctx);
      bool all = true;
      any_fail = false;
      for (int p = 0; p < pl.P; ++p) {
        const int v = hbuf[cur][p];
        all &= (v == ST_DONE || v == ST_DONE_FAIL);
        any_fail |= (v == ST_DONE_FAIL);
      }
      if (all) break;
      // every slot moves each unfinished problem forward, and a search ends
      // within max_backtracks trials
      if (checked >= blk * (o->max_backtracks + 1))
        return fail(ctx, KVS_ERR_HIP, "schedule: block did not finish in %d slots", checked);
      cur ^= 1;
    }
    done += blk;
    refreshed = false;
    if (done % o->vc_every == 0) {
      if (any_fail) {  // stored scores of a failed search belong to a rejected trial
        const std::vector<int> hs(hbuf[cur], hbuf[cur] + pl.P);
        run_forward(ctx, pl, b, Q, Yr, lr, Kc, Vc, B.st, 1 << ST_DONE_FAIL, 2, nullptr, nullptr, o,
                    ws, &hs, ST_DONE_FAIL);
      }
      // every problem is re-solved (the stored scores are at its current
      // keys), with the refinement step of the standalone solve
      const RefineIn rin{Q, lr, Kc};
      run_value_solve(ctx, pl, b, Yr, Vc, nullptr, B.st, kAll, ws, ctx->refine_resolves ? &rin : nullptr);
      // the value solve used the stored scores at the current keys: valid for
      // every problem, so the loss at the new values reads them back
      lb_eval_at_x(ctx, pl, b, o, Q, Yr, lr, Kc, Vc, B, 1, nullptr, mse, ws, true);
      refreshed = true;
    }
  }
  if (!refreshed)
    run_forward(ctx, pl, b, Q, Yr, lr, Kc, Vc, B.st, kAll, 2, nullptr, mse, o, ws);
  launch_state_flags_out(B.st, flags, loss, pl.P, ctx->stream);
  prof_add_slot_work(ctx, pl, B.st, before.empty() ? nullptr : before.data());
  return KVS_OK;
}

kvs_status compress_impl(kvs_ctx ctx, const Plan& pl, const kvs_batch* b, const kvs_opts* o,
                         const float* Q, const float* Kz, const float* Vz, float* Kc, float* Vc,
                         float* loss, float* mse, float* init_loss, int* flags, void* ws,
                         bool keys_given = false) {
  compress_begin_impl(ctx, pl, b, o, Q, Kz, Vz, Kc, Vc, init_loss, keys_given, ws);
  return compress_advance_impl(ctx, pl, b, o, Q, Kc, Vc, 0, o->iters, loss, mse, flags, ws);
}

// The alternating schedule with Adam on the keys: per iteration loss and
// gradient at the current keys, one Adam step; values re-solved after
// iterations vc_every, 2 vc_every, ... (moments kept).  The moments live in
// the history region, which Adam does not otherwise use.
kvs_status adam_impl(kvs_ctx ctx, const Plan& pl, const kvs_batch* b, const kvs_opts* o,
                     const kvs_adam_opts* ad, const float* Q, const float* Kz, const float* Vz,
                     float* Kc, float* Vc, float* loss, float* mse, float* init_loss, int* flags,
                     bool keys_given, void* ws) {
  float* Yr = at<float>(ws, pl.r_yref);
  float* lr = at<float>(ws, pl.r_lseref);
  launch_fill_i32(flags, 0, pl.P, ctx->stream);
  run_reference(ctx, pl, b, Q, Kz, Vz, Yr, lr, ws);
  run_init(ctx, pl, b, Q, Kz, Yr, lr, Kc, Vc, flags, nullptr, keys_given, ws);
  float* g = at<float>(ws, pl.r_g);
  float* m = at<float>(ws, pl.r_S);
  float* v = at<float>(ws, pl.r_Yh);
  launch_fill_f32(m, 0.f, (long long)pl.ktot * pl.d, ctx->stream);
  launch_fill_f32(v, 0.f, (long long)pl.ktot * pl.d, ctx->stream);
  // loss at the start; its stored scores serve the first gradient
  run_forward(ctx, pl, b, Q, Yr, lr, Kc, Vc, nullptr, 0, 0, init_loss, nullptr, o, ws);
  AdamArgs aa{};
  aa.x = Kc; aa.g = g; aa.m = m; aa.v = v; aa.flags = flags; aa.nonfinite_flag = KVS_FLAG_NONFINITE;
  aa.info = at<ProbInfo>(ws, pl.r_info); aa.P = pl.P; aa.d = pl.d;
  aa.b1 = (float)ad->beta1; aa.b2 = (float)ad->beta2; aa.eps = (float)ad->eps;
  double p1 = 1.0, p2 = 1.0;
  bool fresh = false;   // scores stored at the current keys before a value solve
  for (int t = 1; t <= o->iters; ++t) {
    if (t > 1)
      run_forward(ctx, pl, b, Q, Yr, lr, Kc, Vc, nullptr, 0, 0, nullptr, nullptr, o, ws, nullptr, 0,
                  fresh);
    fresh = false;
    run_backward(ctx, pl, b, Q, Vc, nullptr, 0, ws);
    GradUpdArgs ga = grad_args(pl, b, ws, nullptr, 0, 2);
    ga.gout = g;
    launch_grad_update(ga, ctx->stream);
    p1 *= ad->beta1;
    p2 *= ad->beta2;
    aa.step = (float)(ad->lr / (1.0 - p1));
    aa.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(1.0 - p2));
    launch_adam(aa, pl.kmax, ctx->stream);
    if (t % o->vc_every == 0) {
      // scores at the moved keys for every problem, then the refined solve
      run_forward(ctx, pl, b, Q, Yr, lr, Kc, Vc, nullptr, 0, 0, nullptr, nullptr, o, ws);
      const RefineIn rin{Q, lr, Kc};
      run_value_solve(ctx, pl, b, Yr, Vc, flags, nullptr, kAllStates, ws, ctx->refine_resolves ? &rin : nullptr);
      fresh = true;
    }
  }
  run_forward(ctx, pl, b, Q, Yr, lr, Kc, Vc, nullptr, 0, 0, loss, mse, o, ws, nullptr, 0, fresh);
  return KVS_OK;
}

}  // namespace kvs

using namespace kvs;

extern "C" {

kvs_status kvs_create(kvs_ctx* out, void* hip_stream) {
  if (!out) return KVS_ERR_INVALID;
  kvs_ctx c = new (std::nothrow) kvs_ctx_s();
  if (!c) return KVS_ERR_INVALID;
  c->stream = static_cast<hipStream_t>(hip_stream);
  if (hipGetDevice(&c->device) != hipSuccess) c->device = 0;
  int lds = 0;
  if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, c->device) == hipSuccess)
    c->lds_max = lds;
  (void)hipGetLastError();
  // score arithmetic of the loss forwards, for comparisons: KVS_LOGITS=fp32
  // or fp64 (the default is the exact integer products)
  if (const char* env = getenv("KVS_LOGITS")) {
    if (!strcmp(env, "fp32")) c->logit_mode = kvs::LOGIT_F32;
    else if (!strcmp(env, "fp64")) c->logit_mode = kvs::LOGIT_F64;
  }
  // the schedule's value re-solves without their refinement step, for comparisons
  if (const char* env = getenv("KVS_RESOLVE_REFINE")) c->refine_resolves = env[0] != '0';
  // the Gram's large-batch kernel, for comparisons: KVS_GRAM=fp32 (128x128
  // tiles, fp32 products), split128 or split256 (split bf16 products on
  // 128x128 or 256x256 tiles); the default takes the split products on
  // 256x256 tiles when a batch has at least 2048 of them, else on 128x128
  if (const char* env = getenv("KVS_GRAM")) {
    if (!strcmp(env, "fp32")) c->gram_split3 = false;
    else if (!strcmp(env, "split128")) c->gram_tile256 = 0;
    else if (!strcmp(env, "split256")) c->gram_tile256 = 2;
  }
  // the refinement residual A^T G on fp32 products instead of split bf16 ones, for comparisons
  if (const char* env = getenv("KVS_RESID")) c->resid_split3 = strcmp(env, "fp32") != 0;
  // the backward on fp32 products instead of split bf16 ones, for comparisons
  if (const char* env = getenv("KVS_BWD")) c->bwd_split3 = strcmp(env, "fp32") != 0;
  // the context's device is current here: take its scratch address once
  if (hipError_t e = scratch_address(c->device, &c->scratch); e != hipSuccess) {
    c->scratch = nullptr;
    c->scratch_err = hipGetErrorString(e);
    (void)hipGetLastError();
  }
  *out = c;
  return KVS_OK;
}

kvs_status kvs_destroy(kvs_ctx ctx) {
  delete ctx;
  return KVS_OK;
}

const char* kvs_status_string(kvs_status s) {
  switch (s) {
    case KVS_OK: return "ok";
    case KVS_ERR_INVALID: return "invalid argument";
    case KVS_ERR_ALIGN: return "misaligned pointer";
    case KVS_ERR_WORKSPACE: return "workspace too small";
    case KVS_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* kvs_last_error(kvs_ctx ctx) { return ctx ? ctx->err.c_str() : ""; }

void kvs_default_opts(kvs_opts* o) {
  if (!o) return;
  o->iters = 20;
  o->vc_every = 5;
  o->history = 10;
  o->max_backtracks = 30;
  o->c1 = 1e-4;
  o->shrink = 0.5;
}

size_t kvs_workspace_bytes(const kvs_batch* b, const kvs_opts* o) {
  Plan pl;
  if (!make_plan(b, o, &pl).empty()) return 0;
  return pl.ws_bytes;
}

size_t kvs_lbfgs_state_bytes(const kvs_batch* b, const kvs_opts* o) {
  Plan pl;
  if (!make_plan(b, o, &pl).empty()) return 0;
  return pl.state_bytes;
}

kvs_status kvs_reference_attn(kvs_ctx ctx, const kvs_batch* b, const float* Q, const float* Kz,
                              const float* Vz, float* Y, float* lse, void* ws, size_t ws_bytes) {
  const char* fn = "kvs_reference_attn";
  if (!ctx) return KVS_ERR_INVALID;
  KVS_NEED(Q); KVS_NEED(Kz); KVS_NEED(Vz); KVS_NEED(Y); KVS_NEED(lse);
  // every problem attends over its Z zone keys; b->k only sizes the plan, so
  // a workspace of kvs_workspace_bytes(b) serves this call as any other
  Plan pl;
  kvs_status s = prepare(ctx, fn, b, nullptr, ws, ws_bytes, &pl);
  if (s != KVS_OK) return s;
  run_reference(ctx, pl, b, Q, Kz, Vz, Y, lse, ws);
  return hip_check(ctx, fn);
}

kvs_status kvs_loss_grad(kvs_ctx ctx, const kvs_batch* b, const float* Q, const float* Y,
                         const float* lse, const float* Kc, const float* Vc, float* loss,
                         float* grad, float* mse, void* ws, size_t ws_bytes) {
  const char* fn = "kvs_loss_grad";
  if (!ctx) return KVS_ERR_INVALID;
  KVS_NEED(Q); KVS_NEED(Y); KVS_NEED(lse); KVS_NEED(Kc); KVS_NEED(Vc); KVS_NEED(loss);
  KVS_OPT(grad); KVS_OPT(mse);
  Plan pl;
  kvs_status s = prepare(ctx, fn, b, nullptr, ws, ws_bytes, &pl);
  if (s != KVS_OK) return s;
  run_forward(ctx, pl, b, Q, Y, lse, Kc, Vc, nullptr, 0, 0, loss, mse, nullptr, ws);
  if (grad) {
    run_backward(ctx, pl, b, Q, Vc, nullptr, 0, ws);
    GradUpdArgs g = grad_args(pl, b, ws, nullptr, 0, 2);
    g.gout = grad;
    launch_grad_update(g, ctx->stream);
  }
  return hip_check(ctx, fn);
}

kvs_status kvs_value_solve(kvs_ctx ctx, const kvs_batch* b, const float* Q, const float* Y,
                           const float* lse, const float* Kc, float* Vc, int32_t* flags, void* ws,
                           size_t ws_bytes) {
  const char* fn = "kvs_value_solve";
  if (!ctx) return KVS_ERR_INVALID;
  KVS_NEED(Q); KVS_NEED(Y); KVS_NEED(Kc); KVS_NEED(Vc); KVS_OPT(lse); KVS_OPT(flags);
  Plan pl;
  kvs_status s = prepare(ctx, fn, b, nullptr, ws, ws_bytes, &pl);
  if (s != KVS_OK) return s;
  run_forward(ctx, pl, b, Q, Y, lse, Kc, Vc, nullptr, 0, 0, nullptr, nullptr, nullptr, ws);
  const RefineIn rin{Q, lse, Kc};
  run_value_solve(ctx, pl, b, Y, Vc, flags, nullptr, 0, ws, &rin);
  return hip_check(ctx, fn);
}

}  // extern "C"


extern "C" {

kvs_status kvs_init_topk(kvs_ctx ctx, const kvs_batch* b, const float* Q, const float* Kz,
                         const float* Y, const float* lse, int32_t* idx, float* Kc, float* Vc,
                         int32_t* flags, void* ws, size_t ws_bytes) {
  const char* fn = "kvs_init_topk";
  if (!ctx) return KVS_ERR_INVALID;
  KVS_NEED(Q); KVS_NEED(Kz); KVS_NEED(Y); KVS_NEED(lse); KVS_NEED(idx); KVS_NEED(Kc); KVS_NEED(Vc);
  KVS_OPT(flags);
  Plan pl;
  kvs_status s = prepare(ctx, fn, b, nullptr, ws, ws_bytes, &pl);
  if (s != KVS_OK) return s;
  run_init_topk(ctx, pl, b, Q, Kz, Y, lse, idx, Kc, Vc, flags, nullptr, ws, true);
  return hip_check(ctx, fn);
}

static kvs_status check_state(kvs_ctx ctx, const char* fn, const Plan& pl, void* state, size_t bytes) {
  if (!state) return fail(ctx, KVS_ERR_INVALID, "%s: state is NULL", fn);
  if (!aligned(state, 256)) return fail(ctx, KVS_ERR_ALIGN, "%s: state not 256-byte aligned", fn);
  if (bytes < pl.state_bytes)
    return fail(ctx, KVS_ERR_WORKSPACE, "%s: state %zu bytes < required %zu", fn, bytes, pl.state_bytes);
  return KVS_OK;
}

kvs_status kvs_lbfgs_init(kvs_ctx ctx, const kvs_batch* b, const kvs_opts* o, const float* Q,
                          const float* Y, const float* lse, const float* Kc, const float* Vc,
                          int32_t clear_history, float* loss, int32_t* flags, void* state,
                          size_t state_bytes, void* ws, size_t ws_bytes) {
  const char* fn = "kvs_lbfgs_init";
  if (!ctx) return KVS_ERR_INVALID;
  if (!o) return fail(ctx, KVS_ERR_INVALID, "%s: opts is NULL", fn);
  KVS_NEED(Q); KVS_NEED(Y); KVS_NEED(lse); KVS_NEED(Kc); KVS_NEED(Vc); KVS_OPT(loss); KVS_OPT(flags);
  Plan pl;
  kvs_status s = prepare(ctx, fn, b, o, ws, ws_bytes, &pl);
  if (s != KVS_OK) return s;
  if ((s = check_state(ctx, fn, pl, state, state_bytes)) != KVS_OK) return s;
  LbBuffers B = lb_in_state(pl, state, ws);
  launch_state_init(B.st, pl.P, clear_history ? 1 : 0, ctx->stream);
  lb_eval_at_x(ctx, pl, b, o, Q, Y, lse, const_cast<float*>(Kc), Vc, B, clear_history ? 2 : 1, loss,
               nullptr, ws);
  launch_state_flags_out(B.st, flags, loss, pl.P, ctx->stream);
  return hip_check(ctx, fn);
}

kvs_status kvs_lbfgs_step(kvs_ctx ctx, const kvs_batch* b, const kvs_opts* o, const float* Q,
                          const float* Y, const float* lse, float* Kc, const float* Vc, float* loss,
                          int32_t* flags, void* state, size_t state_bytes, void* ws, size_t ws_bytes) {
  const char* fn = "kvs_lbfgs_step";
  if (!ctx) return KVS_ERR_INVALID;
  if (!o) return fail(ctx, KVS_ERR_INVALID, "%s: opts is NULL", fn);
  KVS_NEED(Q); KVS_NEED(Y); KVS_NEED(lse); KVS_NEED(Kc); KVS_NEED(Vc); KVS_OPT(loss); KVS_OPT(flags);
  Plan pl;
  kvs_status s = prepare(ctx, fn, b, o, ws, ws_bytes, &pl);
  if (s != KVS_OK) return s;
  if ((s = check_state(ctx, fn, pl, state, state_bytes)) != KVS_OK) return s;
  LbBuffers B = lb_in_state(pl, state, ws);
  bool any_fail = false;
  std::vector<int> hs;
  s = lb_iteration(ctx, pl, b, o, Q, Y, lse, Kc, Vc, B, ws, &any_fail, hs);
  if (s != KVS_OK) return s;
  launch_state_flags_out(B.st, flags, loss, pl.P, ctx->stream);
  return hip_check(ctx, fn);
}

kvs_status kvs_compress(kvs_ctx ctx, const kvs_batch* b, const kvs_opts* o, const float* Q,
                        const float* Kz, const float* Vz, float* Kc, float* Vc, float* loss,
                        float* mse, float* init_loss, int32_t* flags, void* ws, size_t ws_bytes) {
  const char* fn = "kvs_compress";
  if (!ctx) return KVS_ERR_INVALID;
  if (!o) return fail(ctx, KVS_ERR_INVALID, "%s: opts is NULL", fn);
  KVS_NEED(Q); KVS_NEED(Kz); KVS_NEED(Vz); KVS_NEED(Kc); KVS_NEED(Vc); KVS_NEED(loss);
  KVS_OPT(mse); KVS_OPT(init_loss); KVS_OPT(flags);
  Plan pl;
  kvs_status s = prepare(ctx, fn, b, o, ws, ws_bytes, &pl);
  if (s != KVS_OK) return s;
  s = compress_impl(ctx, pl, b, o, Q, Kz, Vz, Kc, Vc, loss, mse, init_loss, flags, ws);
  if (s != KVS_OK) return s;
  return hip_check(ctx, fn);
}

kvs_status kvs_compress_from_keys(kvs_ctx ctx, const kvs_batch* b, const kvs_opts* o,
                                  const float* Q, const float* Kz, const float* Vz, float* Kc,
                                  float* Vc, float* loss, float* mse, float* init_loss,
                                  int32_t* flags, void* ws, size_t ws_bytes) {
  const char* fn = "kvs_compress_from_keys";
  if (!ctx) return KVS_ERR_INVALID;
  if (!o) return fail(ctx, KVS_ERR_INVALID, "%s: opts is NULL", fn);
  KVS_NEED(Q); KVS_NEED(Kz); KVS_NEED(Vz); KVS_NEED(Kc); KVS_NEED(Vc); KVS_NEED(loss);
  KVS_OPT(mse); KVS_OPT(init_loss); KVS_OPT(flags);
  Plan pl;
  kvs_status s = prepare(ctx, fn, b, o, ws, ws_bytes, &pl);
  if (s != KVS_OK) return s;
  s = compress_impl(ctx, pl, b, o, Q, Kz, Vz, Kc, Vc, loss, mse, init_loss, flags, ws, true);
  if (s != KVS_OK) return s;
  return hip_check(ctx, fn);
}

kvs_status kvs_compress_begin(kvs_ctx ctx, const kvs_batch* b, const kvs_opts* o, const float* Q,
                              const float* Kz, const float* Vz, int32_t keys_given, float* Kc,
                              float* Vc, float* init_loss, void* ws, size_t ws_bytes) {
  const char* fn = "kvs_compress_begin";
  if (!ctx) return KVS_ERR_INVALID;
  if (!o) return fail(ctx, KVS_ERR_INVALID, "%s: opts is NULL", fn);
  KVS_NEED(Q); KVS_NEED(Kz); KVS_NEED(Vz); KVS_NEED(Kc); KVS_NEED(Vc); KVS_OPT(init_loss);
  Plan pl;
  kvs_status s = prepare(ctx, fn, b, o, ws, ws_bytes, &pl);
  if (s != KVS_OK) return s;
  compress_begin_impl(ctx, pl, b, o, Q, Kz, Vz, Kc, Vc, init_loss, keys_given != 0, ws);
  return hip_check(ctx, fn);
}

kvs_status kvs_compress_advance(kvs_ctx ctx, const kvs_batch* b, const kvs_opts* o, const float* Q,
                                int32_t t_begin, int32_t t_end, float* Kc, float* Vc, float* loss,
                                float* mse, int32_t* flags, void* ws, size_t ws_bytes) {
  const char* fn = "kvs_compress_advance";
  if (!ctx) return KVS_ERR_INVALID;
  if (!o) return fail(ctx, KVS_ERR_INVALID, "%s: opts is NULL", fn);
  KVS_NEED(Q); KVS_NEED(Kc); KVS_NEED(Vc); KVS_NEED(loss); KVS_OPT(mse); KVS_OPT(flags);
  // checked before anything is enqueued (vc_every < 1 is reported by the plan)
  if (t_begin < 0 || t_end < t_begin)
    return fail(ctx, KVS_ERR_INVALID, "%s: need 0 <= t_begin <= t_end (got %d, %d)", fn, t_begin, t_end);
  if (o->vc_every >= 1 && t_begin % o->vc_every != 0)
    return fail(ctx, KVS_ERR_INVALID, "%s: t_begin %d is not a multiple of vc_every %d", fn, t_begin,
                o->vc_every);
  Plan pl;
  kvs_status s = prepare(ctx, fn, b, o, ws, ws_bytes, &pl);
  if (s != KVS_OK) return s;
  s = compress_advance_impl(ctx, pl, b, o, Q, Kc, Vc, t_begin, t_end, loss, mse, flags, ws);
  if (s != KVS_OK) return s;
  return hip_check(ctx, fn);
}

void kvs_default_adam_opts(kvs_adam_opts* a) {
  if (!a) return;
  a->lr = 1e-2;
  a->beta1 = 0.9;
  a->beta2 = 0.999;
  a->eps = 1e-8;
}

kvs_status kvs_compress_adam(kvs_ctx ctx, const kvs_batch* b, const kvs_opts* o,
                             const kvs_adam_opts* a, int32_t keys_given, const float* Q,
                             const float* Kz, const float* Vz, float* Kc, float* Vc, float* loss,
                             float* mse, float* init_loss, int32_t* flags, void* ws,
                             size_t ws_bytes) {
  const char* fn = "kvs_compress_adam";
  if (!ctx) return KVS_ERR_INVALID;
  if (!o) return fail(ctx, KVS_ERR_INVALID, "%s: opts is NULL", fn);
  if (!a) return fail(ctx, KVS_ERR_INVALID, "%s: adam opts is NULL", fn);
  if (!(a->lr > 0.0) || !(a->beta1 >= 0.0 && a->beta1 < 1.0) || !(a->beta2 >= 0.0 && a->beta2 < 1.0) ||
      !(a->eps > 0.0))
    return fail(ctx, KVS_ERR_INVALID, "%s: adam needs lr > 0, beta1 and beta2 in [0, 1), eps > 0", fn);
  KVS_NEED(Q); KVS_NEED(Kz); KVS_NEED(Vz); KVS_NEED(Kc); KVS_NEED(Vc); KVS_NEED(loss);
  KVS_NEED(flags); KVS_OPT(mse); KVS_OPT(init_loss);
  Plan pl;
  kvs_status s = prepare(ctx, fn, b, o, ws, ws_bytes, &pl);
  if (s != KVS_OK) return s;
  s = adam_impl(ctx, pl, b, o, a, Q, Kz, Vz, Kc, Vc, loss, mse, init_loss, flags, keys_given != 0, ws);
  if (s != KVS_OK) return s;
  return hip_check(ctx, fn);
}

kvs_status kvs_pilot_allocate(kvs_ctx ctx, const kvs_batch* b, const kvs_opts* o,
                              int32_t pilot_iters, double alpha, int32_t k_min, int32_t k_max,
                              const float* Q, const float* Kz, const float* Vz, float* pilot_mse,
                              int32_t* k_out, void* ws, size_t ws_bytes) {
  const char* fn = "kvs_pilot_allocate";
  if (!ctx) return KVS_ERR_INVALID;
  if (!o) return fail(ctx, KVS_ERR_INVALID, "%s: opts is NULL", fn);
  KVS_NEED(Q); KVS_NEED(Kz); KVS_NEED(Vz); KVS_NEED(pilot_mse);
  if (!k_out) return fail(ctx, KVS_ERR_INVALID, "%s: k_out is NULL", fn);
  if (pilot_iters < 0) return fail(ctx, KVS_ERR_INVALID, "%s: pilot_iters < 0", fn);
  if (!(alpha >= 0.0)) return fail(ctx, KVS_ERR_INVALID, "%s: alpha < 0", fn);
  kvs_opts po = *o;
  po.iters = pilot_iters;
  Plan pl;
  kvs_status s = prepare(ctx, fn, b, &po, ws, ws_bytes, &pl);
  if (s != KVS_OK) return s;
  if (k_min < 1 || k_max < k_min || k_max > b->Z)
    return fail(ctx, KVS_ERR_INVALID, "%s: need 1 <= k_min <= k_max <= Z", fn);
  int* dflags = at<int>(ws, pl.r_flags);
  float* dloss = at<float>(ws, pl.r_loss);
  launch_fill_i32(dflags, 0, pl.P, ctx->stream);
  s = compress_impl(ctx, pl, b, &po, Q, Kz, Vz, at<float>(ws, pl.r_Kc), at<float>(ws, pl.r_Vc), dloss,
                    pilot_mse, nullptr, dflags, ws);
  if (s != KVS_OK) return s;
  std::vector<float> hm(pl.P);
  if (hipMemcpyAsync(hm.data(), pilot_mse, sizeof(float) * pl.P, hipMemcpyDeviceToHost, ctx->stream) !=
          hipSuccess ||
      hipStreamSynchronize(ctx->stream) != hipSuccess)
    return fail(ctx, KVS_ERR_HIP, "%s: %s", fn, hipGetErrorString(hipGetLastError()));
  std::vector<double> md(hm.begin(), hm.end());
  const int64_t K = pl.ktot;
  s = kvs_allocate_budget(md.data(), pl.P, K, alpha, k_min, k_max, k_out);
  if (s != KVS_OK) return fail(ctx, s, "%s: budget split failed (non-finite pilot MSE?)", fn);
  return hip_check(ctx, fn);
}

}  // extern "C"

extern "C" {

kvs_status kvs_build_queries(kvs_ctx ctx, const kvs_query_geom* q, const float* Qctx,
                             const int32_t* src, float* Q, int32_t* flags) {
  const char* fn = "kvs_build_queries";
  if (!ctx) return KVS_ERR_INVALID;
  ctx->err.clear();
  if (!q) return fail(ctx, KVS_ERR_INVALID, "%s: geometry is NULL", fn);
  const int d = q->d;
  if (q->P < 1 || q->g < 1 || q->N < 1 || q->m < 0 || q->m > q->N || q->F < 0)
    return fail(ctx, KVS_ERR_INVALID, "%s: bad sizes P=%d g=%d N=%d m=%d F=%d", fn, q->P, q->g,
                q->N, q->m, q->F);
  if (d != 8 && d != 16 && d != 32 && d != 64 && d != 128 && d != 256)
    return fail(ctx, KVS_ERR_INVALID, "%s: d=%d is not a power of two in [8, 256]", fn, d);
  if (!(q->theta > 1.0) || !std::isfinite(q->theta))
    return fail(ctx, KVS_ERR_INVALID, "%s: theta must be finite and > 1", fn);
  const long long per_p = (long long)q->g * (q->m + q->F);
  if (per_p < 1) return fail(ctx, KVS_ERR_INVALID, "%s: no queries to build (g (m + F) = 0)", fn);
  if ((long long)q->N + q->F > (1LL << 30))
    return fail(ctx, KVS_ERR_INVALID, "%s: positions beyond 2^30", fn);
  KVS_NEED(Qctx); KVS_NEED(Q);
  if (q->F > 0 && !src) return fail(ctx, KVS_ERR_INVALID, "%s: argument 'src' is NULL", fn);
  if (src && !aligned(src, 4)) return fail(ctx, KVS_ERR_ALIGN, "%s: 'src' not 4-byte aligned", fn);
  if (flags && !aligned(flags, 4)) return fail(ctx, KVS_ERR_ALIGN, "%s: 'flags' not 4-byte aligned", fn);
  QueryArgs a{};
  a.Qctx = Qctx; a.src = src; a.Q = Q; a.flags = flags;
  a.P = q->P; a.g = q->g; a.N = q->N; a.m = q->m; a.F = q->F; a.d = d;
  a.bad_flag = KVS_FLAG_BADINDEX;
  a.log2_theta = std::log2(q->theta);
  a.freq_ratio = std::exp2(-2.0 / d * a.log2_theta);
  {
    // every output element is read once and written once; the future rows
    // also read their source index
    const double rows = (double)q->P * per_p;
    Prof pr(ctx, PROF_QUERIES, 0.0, rows * d * 8.0 + (double)q->P * q->g * q->F * 4.0);
    launch_build_queries(a, ctx->stream);
  }
  return hip_check(ctx, fn);
}

size_t kvs_use_eval_workspace_bytes(const kvs_batch* b, int32_t m) {
  UsePlan u;
  if (!make_use_plan(b, m, &u).empty()) return 0;
  return u.ws_bytes;
}

kvs_status kvs_use_eval(kvs_ctx ctx, const kvs_batch* b, int32_t m, const float* Qh,
                        const float* Kz, const float* Vz, const float* Kr, const float* Vr,
                        const float* Kc, const float* Vc, float* Ofull, float* Ocomp, float* mse,
                        float* rel, void* ws, size_t ws_bytes) {
  const char* fn = "kvs_use_eval";
  if (!ctx) return KVS_ERR_INVALID;
  ctx->err.clear();
  UsePlan u;
  std::string e = make_use_plan(b, m, &u);
  if (!e.empty()) return fail(ctx, KVS_ERR_INVALID, "%s: %s", fn, e.c_str());
  KVS_NEED(Qh); KVS_NEED(Kz); KVS_NEED(Vz); KVS_NEED(Kc); KVS_NEED(Vc); KVS_NEED(mse);
  if (m > 0) { KVS_NEED(Kr); KVS_NEED(Vr); }
  KVS_OPT(Ofull); KVS_OPT(Ocomp); KVS_OPT(rel);
  if (!ws) return fail(ctx, KVS_ERR_INVALID, "%s: workspace is NULL", fn);
  if (!aligned(ws, 256)) return fail(ctx, KVS_ERR_ALIGN, "%s: workspace not 256-byte aligned", fn);
  if (ws_bytes < u.ws_bytes)
    return fail(ctx, KVS_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, ws_bytes,
                u.ws_bytes);
  launch_write_info(at<ProbInfo>(ws, u.r_info), u.info.data(), u.P, ctx->stream);

  const size_t pn = (size_t)u.P * u.n;
  float* Opart = at<float>(ws, u.r_Opart);
  float* Mpart = at<float>(ws, u.r_Mpart);
  float* Lpart = at<float>(ws, u.r_Lpart);
  // split-key partials of one cache into planes [c0, c0 + C)
  auto chunk_fwd = [&](const float* K, const float* V, const ProbInfo* info, int kuni, int kmax,
                       int C, int c0, double keys) {
    FwdArgs f{};
    f.Q = Qh; f.K = K; f.V = V; f.st = nullptr; f.active_mask = 0; f.shift = nullptr;
    f.St = nullptr;
    f.Opart = Opart + (size_t)c0 * pn * u.d;
    f.Mpart = Mpart + (size_t)c0 * pn;
    f.Lpart = Lpart + (size_t)c0 * pn;
    f.info = info; f.P = u.P; f.n = u.n; f.C = C; f.kuni = kuni; f.kmax = kmax;
    f.scale = b->scale;
    Prof pr(ctx, PROF_USE, 4.0 * u.n * u.d * keys, 4.0 * (keys * u.d * 2.0 + (double)pn * u.d));
    launch_attn_fwd(f, u.d, ctx->logit_mode == LOGIT_F32 ? LOGIT_F32 : LOGIT_F64, ctx->stream);
  };
  chunk_fwd(Kz, Vz, nullptr, u.Z, u.Z, u.Cz, 0, (double)u.P * u.Z);
  if (u.Cr) chunk_fwd(Kr, Vr, nullptr, m, m, u.Cr, u.Cz, (double)u.P * m);
  chunk_fwd(Kc, Vc, at<ProbInfo>(ws, u.r_info), 0, u.kmax, u.Cc, u.Cz + u.Cr, (double)u.ktot);

  float* Of = Ofull ? Ofull : at<float>(ws, u.r_Of);
  float* Oc = Ocomp ? Ocomp : at<float>(ws, u.r_Oc);
  auto merge = [&](int c0, int C, float* Y, float* lse) {
    MergeArgs mg{};
    mg.Opart = Opart + (size_t)c0 * pn * u.d;
    mg.Mpart = Mpart + (size_t)c0 * pn;
    mg.Lpart = Lpart + (size_t)c0 * pn;
    mg.st = nullptr; mg.active_mask = 0; mg.Yout = Y; mg.lse_out = lse;
    mg.P = u.P; mg.n = u.n; mg.C = C; mg.lambda = b->lambda;
    launch_merge(mg, u.d, false, ctx->stream);
  };
  merge(0, u.Cz + u.Cr, Of, at<float>(ws, u.r_lf));            // [Kz; Kr]
  merge(u.Cz, u.Cr + u.Cc, Oc, at<float>(ws, u.r_lc));         // [Kr; Kc]

  UseErrArgs ea{};
  ea.Of = Of; ea.Oc = Oc; ea.part = at<double>(ws, u.r_part); ea.mse = mse; ea.rel = rel;
  ea.P = u.P; ea.n = u.n; ea.d = u.d; ea.nblk = u.nblk;
  launch_use_err(ea, ctx->stream);
  return hip_check(ctx, fn);
}

size_t kvs_value_norms_workspace_bytes(int32_t P, int32_t Z) {
  if (P < 1 || Z < 1) return 0;
  const size_t b = (size_t)P * value_norm_chunks(P, Z) * sizeof(double);
  return (b + 255) & ~(size_t)255;
}

kvs_status kvs_value_norms(kvs_ctx ctx, int32_t P, int32_t Z, int32_t d, const float* Vz,
                           double* signal, void* ws, size_t ws_bytes) {
  const char* fn = "kvs_value_norms";
  if (!ctx) return KVS_ERR_INVALID;
  ctx->err.clear();
  if (P < 1 || Z < 1 || (d != 64 && d != 128))
    return fail(ctx, KVS_ERR_INVALID, "%s: bad sizes P=%d Z=%d d=%d", fn, P, Z, d);
  KVS_NEED(Vz);
  if (!signal) return fail(ctx, KVS_ERR_INVALID, "%s: argument 'signal' is NULL", fn);
  if (!aligned(signal, 8)) return fail(ctx, KVS_ERR_ALIGN, "%s: 'signal' not 8-byte aligned", fn);
  if (!ws) return fail(ctx, KVS_ERR_INVALID, "%s: workspace is NULL", fn);
  if (!aligned(ws, 256)) return fail(ctx, KVS_ERR_ALIGN, "%s: workspace not 256-byte aligned", fn);
  const size_t need = kvs_value_norms_workspace_bytes(P, Z);
  if (ws_bytes < need)
    return fail(ctx, KVS_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, need);
  VnormArgs a{};
  a.V = Vz; a.part = static_cast<double*>(ws); a.out = signal; a.P = P; a.Z = Z;
  a.C = value_norm_chunks(P, Z);
  launch_value_norms(a, d, ctx->stream);
  return hip_check(ctx, fn);
}

size_t kvs_value_norms_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

kvs_status kvs_value_norms_noalloc(kvs_ctx ctx, int32_t P, int32_t Z, int32_t d, const float* Vz,
                                   double* signal) {
  const char* fn = "kvs_value_norms_noalloc";
  if (!ctx) return KVS_ERR_INVALID;
  ctx->err.clear();
  if (P < 1 || Z < 1 || (d != 64 && d != 128))
    return fail(ctx, KVS_ERR_INVALID, "%s: bad sizes P=%d Z=%d d=%d", fn, P, Z, d);
  KVS_NEED(Vz);
  if (!signal) return fail(ctx, KVS_ERR_INVALID, "%s: argument 'signal' is NULL", fn);
  if (!aligned(signal, 8)) return fail(ctx, KVS_ERR_ALIGN, "%s: 'signal' not 8-byte aligned", fn);
  const size_t need = kvs_value_norms_workspace_bytes(P, Z);
  if (need > kNoAllocScratchBytes)
    return fail(ctx, KVS_ERR_INVALID, "%s: P=%d needs %zu bytes of scratch, above the %zu-byte static array",
                fn, P, need, kNoAllocScratchBytes);
  if (!ctx->scratch)
    return fail(ctx, KVS_ERR_HIP, "%s: no scratch address for device %d: %s", fn, ctx->device,
                ctx->scratch_err.c_str());
  // the same kernels as kvs_value_norms; the chunk partials go to this
  // device's static scratch (fully written before they are read: nothing
  // to clear between calls)
  VnormArgs a{};
  a.V = Vz; a.part = static_cast<double*>(ctx->scratch); a.out = signal; a.P = P; a.Z = Z;
  a.C = value_norm_chunks(P, Z);
  launch_value_norms(a, d, ctx->stream);
  return hip_check(ctx, fn);
}

kvs_status kvs_profile_enable(kvs_ctx ctx, int32_t enable) {
  if (!ctx) return KVS_ERR_INVALID;
  if (hipStreamSynchronize(ctx->stream) != hipSuccess)
    return fail(ctx, KVS_ERR_HIP, "kvs_profile_enable: %s", hipGetErrorString(hipGetLastError()));
  prof_drain(ctx);
  for (auto& a : ctx->acc) a = ProfAcc();
  ctx->prof = enable != 0;
  ctx->prof_mask = enable;
  return KVS_OK;
}

kvs_status kvs_profile_read(kvs_ctx ctx, kvs_kernel_stats* out, int32_t max, int32_t* count) {
  if (!ctx || !count || (max > 0 && !out)) return KVS_ERR_INVALID;
  if (hipStreamSynchronize(ctx->stream) != hipSuccess)
    return fail(ctx, KVS_ERR_HIP, "kvs_profile_read: %s", hipGetErrorString(hipGetLastError()));
  prof_drain(ctx);
  int n = 0;
  for (int c = 0; c < PROF_NCLASS && n < max; ++c) {
    if (ctx->acc[c].launches == 0) continue;
    kvs_kernel_stats& o = out[n++];
    memset(&o, 0, sizeof o);
    snprintf(o.name, sizeof o.name, "%s", kProfNames[c]);
    o.launches = ctx->acc[c].launches;
    o.total_ms = ctx->acc[c].ms;
    o.flops = ctx->acc[c].flops;
    o.bytes = ctx->acc[c].bytes;
  }
  *count = n;
  return KVS_OK;
}

}  // extern "C"
