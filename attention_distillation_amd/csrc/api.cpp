// C ABI of the KVSculpt library: argument checks, workspace carving and the
// host-side schedule that enqueues the HIP kernels on the context's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/kvsculpt.h"
#include "kvs_internal.h"
#include "plan.h"

struct kvs_ctx_s {
  hipStream_t stream = nullptr;
  std::string err;
  int device = 0;
  bool logit_f64 = true;
};

namespace kvs {

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
  return KVS_OK;
}

// ---------------------------------------------------------------- building blocks

// Reference attention over the compress zone (uniform Z keys per problem).
void run_reference(kvs_ctx ctx, const Plan& pl, const kvs_batch* b, const float* Q, const float* Kz,
                   const float* Vz, float* Y, float* lse, void* ws) {
  FwdArgs f{};
  f.Q = Q; f.K = Kz; f.V = Vz; f.dir = nullptr; f.st = nullptr; f.active_mask = 0;
  f.shift = nullptr; f.St = nullptr;
  f.Opart = at<float>(ws, pl.r_Opart); f.Mpart = at<float>(ws, pl.r_Mpart); f.Lpart = at<float>(ws, pl.r_Lpart);
  f.info = nullptr; f.P = pl.P; f.n = pl.n; f.C = pl.Cref; f.kuni = pl.Z; f.kmax = pl.Z; f.scale = b->scale;
  launch_attn_fwd(f, pl.d, false, ctx->stream);
  MergeArgs m{};
  m.Opart = f.Opart; m.Mpart = f.Mpart; m.Lpart = f.Lpart; m.st = nullptr; m.active_mask = 0;
  m.Yout = Y; m.lse_out = lse; m.P = pl.P; m.n = pl.n; m.C = pl.Cref; m.lambda = b->lambda;
  launch_merge(m, pl.d, false, ctx->stream);
}

// Forward at keys K (+ alpha * dir when dir != NULL) for problems selected by
// (st, mask): stores shifted scores, merges, writes G / e / crow and the loss
// partials, then finalises per-problem losses in the given mode.
void run_forward(kvs_ctx ctx, const Plan& pl, const kvs_batch* b, const float* Q, const float* Y,
                 const float* lse, const float* K, const float* dir, const float* V, LbState* st,
                 int mask, int fin_mode, float* loss, float* mse, const kvs_opts* o, void* ws) {
  FwdArgs f{};
  f.Q = Q; f.K = K; f.V = V; f.dir = dir; f.st = st; f.active_mask = mask;
  f.shift = lse; f.St = at<float>(ws, pl.r_St);
  f.Opart = at<float>(ws, pl.r_Opart); f.Mpart = at<float>(ws, pl.r_Mpart); f.Lpart = at<float>(ws, pl.r_Lpart);
  f.info = at<ProbInfo>(ws, pl.r_info); f.P = pl.P; f.n = pl.n; f.C = pl.C; f.kuni = 0; f.kmax = pl.kmax;
  f.scale = b->scale;
  launch_attn_fwd(f, pl.d, ctx->logit_f64, ctx->stream);
  MergeArgs m{};
  m.Opart = f.Opart; m.Mpart = f.Mpart; m.Lpart = f.Lpart; m.st = st; m.active_mask = mask;
  m.Y = Y; m.lse = lse; m.G = at<float>(ws, pl.r_G); m.e = at<float>(ws, pl.r_e);
  m.crow = at<float>(ws, pl.r_crow); m.part = at<double>(ws, pl.r_part);
  m.P = pl.P; m.n = pl.n; m.C = pl.C; m.lambda = b->lambda;
  launch_merge(m, pl.d, true, ctx->stream);
  FinalizeArgs fa{};
  fa.part = m.part; fa.nblk = pl.nblk; fa.P = pl.P; fa.st = st; fa.loss = loss; fa.mse = mse;
  fa.n = pl.n; fa.d = pl.d; fa.mode = fin_mode;
  fa.c1 = o ? o->c1 : 1e-4; fa.shrink = o ? o->shrink : 0.5; fa.max_bt = o ? o->max_backtracks : 30;
  fa.status_host_view = at<int>(ws, pl.r_status);
  launch_finalize(fa, ctx->stream);
}

// Backward from the last forward's stored scores into grad (scaled, reduced).
void run_backward(kvs_ctx ctx, const Plan& pl, const kvs_batch* b, const float* Q, const float* V,
                  LbState* st, int mask, float* grad, void* ws) {
  BwdArgs bw{};
  bw.Q = Q; bw.St = at<float>(ws, pl.r_St); bw.G = at<float>(ws, pl.r_G); bw.e = at<float>(ws, pl.r_e);
  bw.crow = at<float>(ws, pl.r_crow); bw.K = nullptr; bw.V = V; bw.st = st; bw.active_mask = mask;
  bw.dKpart = at<float>(ws, pl.r_dK); bw.info = at<ProbInfo>(ws, pl.r_info);
  bw.P = pl.P; bw.n = pl.n; bw.Cn = pl.Cn; bw.kmax = pl.kmax; bw.ktot = (int)pl.ktot;
  launch_attn_bwd(bw, pl.d, ctx->stream);
  GradReduceArgs gr{};
  gr.dKpart = bw.dKpart; gr.grad = grad; gr.st = st; gr.active_mask = mask; gr.info = bw.info;
  gr.P = pl.P; gr.Cn = pl.Cn; gr.ktot = (int)pl.ktot; gr.scale = b->scale;
  launch_grad_reduce(gr, pl.d, ctx->stream);
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
  const char* env = getenv("KVS_LOGITS_FP32");
  c->logit_f64 = !(env && env[0] == '1');
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
  kvs_batch bb = *b;
  bb.k = nullptr;   // k is not used here: every problem attends over its Z keys
  Plan pl;
  kvs_status s = prepare(ctx, fn, &bb, nullptr, ws, ws_bytes, &pl);
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
  run_forward(ctx, pl, b, Q, Y, lse, Kc, nullptr, Vc, nullptr, 0, 0, loss, mse, nullptr, ws);
  if (grad) run_backward(ctx, pl, b, Q, Vc, nullptr, 0, grad, ws);
  return hip_check(ctx, fn);
}

}  // extern "C"

// ---- entry points whose kernels are not wired yet -------------------------
extern "C" {
#define KVS_TODO(name) return fail(ctx, KVS_ERR_INVALID, "%s: not available in this build", #name)
kvs_status kvs_init_topk(kvs_ctx ctx, const kvs_batch*, const float*, const float*, const float*,
                         const float*, int32_t*, float*, float*, int32_t*, void*, size_t) { KVS_TODO(kvs_init_topk); }
kvs_status kvs_value_solve(kvs_ctx ctx, const kvs_batch*, const float*, const float*, const float*,
                           const float*, float*, int32_t*, void*, size_t) { KVS_TODO(kvs_value_solve); }
kvs_status kvs_lbfgs_init(kvs_ctx ctx, const kvs_batch*, const kvs_opts*, const float*, const float*,
                          const float*, const float*, const float*, int32_t, float*, int32_t*, void*,
                          size_t, void*, size_t) { KVS_TODO(kvs_lbfgs_init); }
kvs_status kvs_lbfgs_step(kvs_ctx ctx, const kvs_batch*, const kvs_opts*, const float*, const float*,
                          const float*, float*, const float*, float*, int32_t*, void*, size_t, void*,
                          size_t) { KVS_TODO(kvs_lbfgs_step); }
kvs_status kvs_compress(kvs_ctx ctx, const kvs_batch*, const kvs_opts*, const float*, const float*,
                        const float*, float*, float*, float*, float*, float*, int32_t*, void*, size_t) {
  KVS_TODO(kvs_compress);
}
kvs_status kvs_pilot_allocate(kvs_ctx ctx, const kvs_batch*, const kvs_opts*, int32_t, double, int32_t,
                              int32_t, const float*, const float*, const float*, float*, int32_t*,
                              void*, size_t) { KVS_TODO(kvs_pilot_allocate); }
}
