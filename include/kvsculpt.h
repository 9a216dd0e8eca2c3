/*
 * kvsculpt.h -- C ABI of the MI355X (gfx950) KVSculpt cache-distillation library.
 *
 * The method (KVSculpt: KV Cache Compression as Distillation; arXiv abstract
 * and the gist.science page, section 2 "Methodology"): for every (layer,
 * KV-head) problem, the oldest Z = N - m RoPE'd key/value pairs of a cache
 * (the compress zone) are replaced by k free pairs (Kc, Vc) that minimise
 *     L = ||Yhat - Y||_F^2 + lambda * ||lhat - l||^2
 * over a set of training queries Q, where (Y, l) are the compress zone's
 * attention output and log-sum-exp for those queries and (Yhat, lhat) the
 * compressed pairs'.  Kc is updated by L-BFGS; Vc is re-solved in closed
 * form by ridge regression every few iterations; Kc starts at the top-k keys
 * by attention importance.  A short pilot run at uniform k redistributes the
 * total budget across problems in proportion to sqrt(pilot MSE).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Problems p = 0..P-1 (p = layer * kv_heads + head) are batched in one call.
 *  - All tensors are float32, C-contiguous, caller-owned DEVICE pointers with
 *    16-byte alignment, unless marked HOST.
 *      Q   [P][n][d]   training queries (already RoPE'd)
 *      Kz  [P][Z][d]   compress-zone keys     Vz [P][Z][d] values
 *      Y   [P][n][d]   reference attention output over the compress zone
 *      lse [P][n]      reference log-sum-exp (natural log) over the zone
 *      Kc, Vc          packed ragged [sum_p k_p][d]; problem p starts at row
 *                      off_p = k_0 + ... + k_{p-1}
 *  - d is 64 or 128; 1 <= k_p <= Z; n >= 1; Z >= 1.
 *  - Work is enqueued on the context's HIP stream and is complete when that
 *    stream is synchronised.  Only kvs_pilot_allocate synchronises itself.
 *  - The library never allocates device memory: calls that need scratch
 *    take a caller workspace of at least kvs_workspace_bytes() bytes
 *    (256-byte aligned).  Calls on one context must not overlap in time
 *    with other users of the same workspace.
 *  - Errors: every call returns a kvs_status.  Argument errors are found on
 *    the host before anything is enqueued; nothing throws, aborts or prints.
 *    Numerical failures are per problem, reported in a device flags[P] word
 *    (KVS_FLAG_*), and a flagged problem keeps its last good state.
 *  - Results are deterministic: reductions use fixed orders, no float atomics.
 */
#ifndef KVSCULPT_H
#define KVSCULPT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t kvs_status;
#define KVS_OK                 0
#define KVS_ERR_INVALID      (-1)  /* null pointer, bad size or option        */
#define KVS_ERR_ALIGN        (-2)  /* pointer not 16-byte (workspace 256-byte) aligned */
#define KVS_ERR_WORKSPACE    (-3)  /* workspace smaller than required          */
#define KVS_ERR_HIP          (-4)  /* HIP runtime/launch error (see kvs_last_error) */

/* per-problem numerical status bits (device int32 flags[P]) */
#define KVS_FLAG_NONFINITE     1   /* non-finite loss or gradient             */
#define KVS_FLAG_CHOLESKY      2   /* Gram + mu I not positive definite       */
#define KVS_FLAG_LINESEARCH    4   /* no Armijo step found: no move, history cleared */
#define KVS_FLAG_NONDESCENT    8   /* L-BFGS direction not a descent: reset   */

typedef struct kvs_ctx_s* kvs_ctx;

/* Create a context bound to a borrowed HIP stream (hipStream_t; NULL = the
 * null stream) on the current device.  The context owns no device memory. */
kvs_status  kvs_create(kvs_ctx* out, void* hip_stream);
kvs_status  kvs_destroy(kvs_ctx ctx);
const char* kvs_status_string(kvs_status s);
/* Text of the last failing call on ctx (empty if none). */
const char* kvs_last_error(kvs_ctx ctx);

/* Problem batch description.  k points to HOST int32[P].  d is 64 or 128;
 * 1 <= n <= 2097152 training queries per problem (kernels address a tile's
 * rows with 32-bit byte ranges and offsets); every call rejects other values
 * with KVS_ERR_INVALID. */
typedef struct {
  int32_t P, d, Z, n;
  const int32_t* k;     /* HOST [P], 1 <= k[p] <= Z (ragged)                    */
  double  scale;        /* score scale, 1/sqrt(d)                               */
  double  lambda;       /* weight of the LSE term (1.0)                         */
  double  ridge_rel;    /* mu = ridge_rel * trace(A^T A) / k  (1e-3)            */
} kvs_batch;

/* Optimizer schedule. */
typedef struct {
  int32_t iters;          /* L-BFGS iterations T                               */
  int32_t vc_every;       /* Vc re-solved after iterations vc_every, 2*vc_every.. (5) */
  int32_t history;        /* L-BFGS pairs kept, 1..16 (10)                     */
  int32_t max_backtracks; /* Armijo trials per iteration (30)                  */
  double  c1;             /* Armijo constant (1e-4)                            */
  double  shrink;         /* step factor per failed trial (0.5)                */
} kvs_opts;

/* Defaults: iters 20, vc_every 5, history 10, max_backtracks 30, c1 1e-4,
 * shrink 0.5; lambda 1, ridge_rel 1e-3, scale 1/sqrt(d). */
void kvs_default_opts(kvs_opts* o);

/* Workspace that every call below needs for this batch and schedule. */
size_t kvs_workspace_bytes(const kvs_batch* b, const kvs_opts* o);
/* Persistent L-BFGS state for kvs_lbfgs_init / kvs_lbfgs_step. */
size_t kvs_lbfgs_state_bytes(const kvs_batch* b, const kvs_opts* o);

/* Reference chunk attention (gist page, section 2 "Problem Formulation" and
 * "Loss Function"): for each training query, the softmax attention output Y
 * over the compress zone alone and its natural-log log-sum-exp lse, with
 * scores scale * q.k.  Kz/Vz have Z rows per problem.  b->k does not change
 * the result (it may be NULL, meaning k = Z); when given it is validated as
 * for the other calls, and kvs_workspace_bytes(b) is enough for this call. */
kvs_status kvs_reference_attn(kvs_ctx ctx, const kvs_batch* b, const float* Q,
                              const float* Kz, const float* Vz, float* Y, float* lse,
                              void* ws, size_t ws_bytes);

/* Select+Fit warm start (arXiv abstract: attention-score eviction with
 * least-squares value fitting; gist page, "Optimization Strategy",
 * Initialization).  importance_j = sum_i exp(scale*q_i.kz_j - lse_i); the
 * k_p largest (ties to the lower position) are taken in ascending position
 * order: idx [sum k] int32 (positions within the problem's zone), Kc = Kz[idx],
 * then Vc = ridge solve at Kc, refined as in kvs_value_solve.  flags [P]
 * device int32 gets KVS_FLAG_CHOLESKY where the solve failed (Vc then zero). */
kvs_status kvs_init_topk(kvs_ctx ctx, const kvs_batch* b, const float* Q, const float* Kz,
                         const float* Y, const float* lse, int32_t* idx, float* Kc,
                         float* Vc, int32_t* flags, void* ws, size_t ws_bytes);

/* Loss and key gradient (gist page, "Loss Function"): per problem
 * loss[p] = sum_i ||Yhat_i - Y_i||^2 + lambda * sum_i (lhat_i - lse_i)^2 with
 * Yhat = softmax(scale Q Kc^T) Vc and lhat its log-sum-exp; grad = dL/dKc
 * [sum k][d] (NULL to skip); mse[p] = ||Yhat - Y||_F^2 / (n d) (NULL to skip).
 * loss and mse are device float[P].  The scores q.k are exact integer
 * products of base-128 digits of the rows (scaled by powers of two), shifted
 * by lse in float64 before rounding to float32: each carries the truncation
 * of its inputs below 2^-35 of their row maxima (the environment variable
 * KVS_LOGITS=fp64 or fp32, read when the context is created, selects those
 * products instead).  The same holds for every loss forward below. */
kvs_status kvs_loss_grad(kvs_ctx ctx, const kvs_batch* b, const float* Q, const float* Y,
                         const float* lse, const float* Kc, const float* Vc, float* loss,
                         float* grad, float* mse, void* ws, size_t ws_bytes);

/* Closed-form values (gist page, "Optimization Strategy", Value Optimization:
 * ridge regression given the attention weights of the current keys):
 * A = softmax(scale Q Kc^T), mu = ridge_rel * trace(A^T A) / k,
 * (A^T A + mu I) Vc = A^T Y by Cholesky and two triangular solves, then one
 * step of iterative refinement: r = A^T (Y - A Vc) - mu Vc accumulated in
 * fp64 across 64-query tiles, Vc += (L L^T)^-1 r with the same factor (the
 * fp32 solve alone is off by up to 1e-3 relative when mu is small against
 * the largest eigenvalue of A^T A, e.g. k close to Z, or k > n).
 * lse [P][n] is only used as a per-row shift of the scores (it does not
 * change A); NULL means no shift.  flags [P] (device, may be NULL) gets
 * KVS_FLAG_CHOLESKY where the factorisation failed; Vc of that problem is
 * left unchanged.  The value re-solves inside kvs_compress take the same
 * refinement step.  On batches with enough Gram tiles (at least 512 of
 * 128x128) each product of A^T A and Y^T A is taken as six bf16 products
 * of exact three-piece splits of both operands (h = bf16(x),
 * m = bf16(x - h), l = bf16(x - h - m); the terms of weight <= 2), within
 * about 2^-22 of the product, with fp32 accumulation; KVS_GRAM=fp32, read
 * when the context is created, selects fp32 products instead (split128 /
 * split256 force a tile shape).  The refinement residual A^T G takes the
 * same split products (fp32 sums within 64-query tiles, fp64 across them);
 * KVS_RESID=fp32 selects fp32 products. */
kvs_status kvs_value_solve(kvs_ctx ctx, const kvs_batch* b, const float* Q, const float* Y,
                           const float* lse, const float* Kc, float* Vc, int32_t* flags,
                           void* ws, size_t ws_bytes);

/* L-BFGS on the keys (gist page, "Optimization Strategy", Key Optimization).
 * kvs_lbfgs_init evaluates loss and gradient at Kc with the given Vc into the
 * persistent state (clear_history != 0 also empties the history; 0 keeps it,
 * as after a value re-solve).  kvs_lbfgs_step performs one iteration per
 * problem: two-loop direction over the stored pairs (empty history: -g with
 * first step 1/max(1,||g||)), backtracking Armijo search
 * L(x + a p) <= L(x) + c1 a g^T p halving a up to max_backtracks times, then
 * the curvature-guarded pair update (s^T y > 1e-10 ||s|| ||y||).  Kc is
 * updated in place; loss [P] (device float) receives the loss at the new
 * point; flags [P] (device int32) accumulates KVS_FLAG_* bits.  state is
 * caller memory of kvs_lbfgs_state_bytes() bytes, valid between calls with
 * the same batch, Q, Y, lse and Vc.  kvs_lbfgs_step synchronises the stream
 * once per Armijo trial round to decide whether another round is needed. */
kvs_status kvs_lbfgs_init(kvs_ctx ctx, const kvs_batch* b, const kvs_opts* o, const float* Q,
                          const float* Y, const float* lse, const float* Kc, const float* Vc,
                          int32_t clear_history, float* loss, int32_t* flags,
                          void* state, size_t state_bytes, void* ws, size_t ws_bytes);
kvs_status kvs_lbfgs_step(kvs_ctx ctx, const kvs_batch* b, const kvs_opts* o, const float* Q,
                          const float* Y, const float* lse, float* Kc, const float* Vc,
                          float* loss, int32_t* flags, void* state, size_t state_bytes,
                          void* ws, size_t ws_bytes);

/* The whole alternating schedule (arXiv abstract: keys by L-BFGS, values in
 * closed form, alternating every few steps), batched over all problems with
 * ragged k: reference attention, Select+Fit init, then for t = 1..iters one
 * L-BFGS iteration and, when t % vc_every == 0, a value re-solve followed by
 * loss and gradient at the same keys (history kept).  Outputs Kc, Vc packed
 * [sum k][d]; loss [P] final loss; mse [P] final output MSE (may be NULL);
 * init_loss [P] loss at the Select+Fit start (may be NULL); flags [P].
 * All outputs are device memory. */
kvs_status kvs_compress(kvs_ctx ctx, const kvs_batch* b, const kvs_opts* o, const float* Q,
                        const float* Kz, const float* Vz, float* Kc, float* Vc, float* loss,
                        float* mse, float* init_loss, int32_t* flags, void* ws, size_t ws_bytes);

/* kvs_compress from the caller's starting keys: Kc holds them on entry
 * (packed [sum k][d]) and the result on return; the values start as the
 * ridge fit at those keys instead of the Select+Fit choice.  Everything else
 * as kvs_compress.  It serves the comparison with a search over random
 * restarts (gist page, section 4 "Optimizer Efficacy": a single L-BFGS run
 * against the best of 100 restarts): a restart is one more problem of the
 * batch whose starting keys are the caller's random draw. */
kvs_status kvs_compress_from_keys(kvs_ctx ctx, const kvs_batch* b, const kvs_opts* o,
                                  const float* Q, const float* Kz, const float* Vz, float* Kc,
                                  float* Vc, float* loss, float* mse, float* init_loss,
                                  int32_t* flags, void* ws, size_t ws_bytes);

/* kvs_compress in stages, for callers that drive the schedule in pieces
 * (progress reports, early stopping, timing a block of iterations); the
 * same schedule (arXiv abstract; gist page, "Optimization Strategy") with
 * the same kernels, so begin followed by advance(0, iters) gives the bits of
 * kvs_compress.
 * kvs_compress_begin: reference attention over the zone, the start
 * (Select+Fit, or with keys_given != 0 the caller's keys in Kc and their
 * ridge values), loss and gradient there, empty history.  The reference
 * outputs and the L-BFGS state stay in ws; init_loss [P] (device, may be
 * NULL) gets the loss at the start.
 * kvs_compress_advance: iterations t = t_begin + 1 .. t_end, with the
 * value re-solve after every t that is a multiple of vc_every, from the
 * state in ws.  t_begin must be 0 or a multiple of vc_every (a stage ends
 * anywhere, but only a stage that ended after a value re-solve can be
 * continued) and equal to the previous stage's t_end; 0 <= t_begin <= t_end.
 * b, o, Q, Kc, Vc and ws must be those of the begin call and of the earlier
 * stages (o->iters is not used).  On return loss [P] holds the loss at the
 * current pair, mse [P] (may be NULL) its output MSE, flags [P] (may be
 * NULL) the flags accumulated since begin.  Errors: KVS_ERR_INVALID for a
 * bad t_begin / t_end, otherwise as kvs_compress. */
kvs_status kvs_compress_begin(kvs_ctx ctx, const kvs_batch* b, const kvs_opts* o, const float* Q,
                              const float* Kz, const float* Vz, int32_t keys_given, float* Kc,
                              float* Vc, float* init_loss, void* ws, size_t ws_bytes);
kvs_status kvs_compress_advance(kvs_ctx ctx, const kvs_batch* b, const kvs_opts* o, const float* Q,
                                int32_t t_begin, int32_t t_end, float* Kc, float* Vc, float* loss,
                                float* mse, int32_t* flags, void* ws, size_t ws_bytes);

/* The schedule with Adam in place of L-BFGS on the keys (gist page, section 4
 * "Optimizer Efficacy": the ablation that replaces L-BFGS by Adam; section 2
 * "Optimization Strategy": first-order methods get trapped).  Per iteration
 * t = 1..iters: loss and gradient at (Kc, Vc), then the Adam step (Kingma &
 * Ba 2015, Algorithm 1) m = b1 m + (1-b1) g, v = b2 v + (1-b2) g^2,
 * Kc -= lr (m / (1-b1^t)) / (sqrt(v / (1-b2^t)) + eps), in float32; values
 * re-solved after iterations vc_every, 2 vc_every, ... with the moments
 * kept.  The start is Select+Fit (keys_given = 0) or the caller's keys in Kc
 * with ridge values (keys_given != 0).  history, max_backtracks, c1 and
 * shrink of o are validated but unused.  flags [P] (required) is cleared,
 * then gets KVS_FLAG_NONFINITE for a non-finite gradient element (left
 * unchanged) and KVS_FLAG_CHOLESKY for a failed value solve.  Outputs as for
 * kvs_compress. */
typedef struct {
  double lr;      /* step size (1e-2)   */
  double beta1;   /* 0.9                */
  double beta2;   /* 0.999              */
  double eps;     /* 1e-8               */
} kvs_adam_opts;
void kvs_default_adam_opts(kvs_adam_opts* a);
kvs_status kvs_compress_adam(kvs_ctx ctx, const kvs_batch* b, const kvs_opts* o,
                             const kvs_adam_opts* a, int32_t keys_given, const float* Q,
                             const float* Kz, const float* Vz, float* Kc, float* Vc, float* loss,
                             float* mse, float* init_loss, int32_t* flags, void* ws,
                             size_t ws_bytes);

/* Pilot run and budget (gist page, "Adaptive Budget Allocation"): kvs_compress
 * at the batch's uniform k for pilot_iters iterations (60), per-problem output
 * MSE into pilot_mse [P] (device float), then kvs_allocate_budget with
 * K_total = sum of the batch's k.  k_out is HOST int32[P].  Synchronises the
 * stream.  The workspace must fit the pilot batch. */
kvs_status kvs_pilot_allocate(kvs_ctx ctx, const kvs_batch* b, const kvs_opts* o,
                              int32_t pilot_iters, double alpha, int32_t k_min, int32_t k_max,
                              const float* Q, const float* Kz, const float* Vz,
                              float* pilot_mse, int32_t* k_out, void* ws, size_t ws_bytes);

/* Budget split (gist page, "Adaptive Budget Allocation": total budget
 * redistributed in proportion to the square root of the pilot MSE), pure
 * host, IEEE double: weights w_p = sqrt(mse_p) (alpha = 0.5; alpha = 1 uses
 * mse_p; other alpha pow), x_p = clamp(t w_p, k_min, k_max) with sum K_total
 * (bounded water-filling), then floors plus largest remainders, ties to the
 * lower p.  Sums run in problem order so the result is reproducible bit for
 * bit.  mse and k_out are HOST arrays of P entries.  All-zero weights mean a
 * uniform split.  Errors: KVS_ERR_INVALID if P < 1, a weight is negative or
 * not finite, k_min < 1, k_min > k_max or K_total outside
 * [P k_min, P k_max]. */
kvs_status kvs_allocate_budget(const double* mse, int32_t P, int64_t K_total, double alpha,
                               int32_t k_min, int32_t k_max, int32_t* k_out);

/* Two-level budget split (gist page, "Adaptive Budget Allocation":
 * allocation is performed at the layer and the KV-head level), pure host,
 * IEEE double, bit-reproducible like kvs_allocate_budget.  Problem
 * p = layer * heads + head.  A layer's signal is the mean of its heads' mse
 * (summed in head order, divided by heads); the layer budgets split K_total
 * by kvs_allocate_budget with bounds [heads k_min, min(heads k_max,
 * K_total)], then each layer's budget is split over its heads by
 * kvs_allocate_budget on their own mse, same alpha at both levels.  mse and
 * k_out are HOST arrays of layers * heads entries.  Errors as for
 * kvs_allocate_budget, and KVS_ERR_INVALID if a per-layer bound exceeds
 * INT32_MAX. */
kvs_status kvs_allocate_budget_two_level(const double* mse, int32_t layers, int32_t heads,
                                         int64_t K_total, double alpha, int32_t k_min,
                                         int32_t k_max, int32_t* k_out);

/* Static allocation signal (gist page, section 4 "Budget Allocation": static
 * signals such as value norms, compared with the pilot MSE): signal[p] = mean
 * over the Z rows of Vz [P][Z][d] of their Euclidean norm, accumulated in
 * float64 in a fixed order.  signal is DEVICE double[P]; the workspace holds
 * kvs_value_norms_workspace_bytes(P, Z) bytes (256-byte aligned).  Feeding
 * signal to kvs_allocate_budget with alpha = 1 gives the static allocation. */
size_t kvs_value_norms_workspace_bytes(int32_t P, int32_t Z);
kvs_status kvs_value_norms(kvs_ctx ctx, int32_t P, int32_t Z, int32_t d, const float* Vz,
                           double* signal, void* ws, size_t ws_bytes);

/* Allocation-free variant of kvs_value_norms, for callers that cannot
 * allocate device memory or pass a workspace (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Same kernels and
 * the same result bits as kvs_value_norms; the chunk partials live in a
 * static device array of kvs_value_norms_noalloc_max_bytes() bytes (1 MiB),
 * one copy per GPU, held by the library until the process ends, so no call
 * allocates anything.  Sizes needing more scratch than that
 * (kvs_value_norms_workspace_bytes(P, Z) above the limit: P beyond 2048 at
 * the most chunked Z) return KVS_ERR_INVALID.  Every call on one GPU shares
 * that GPU's array: calls that overlap in time on one GPU (two streams, two
 * threads) race and must be serialised by the caller.  KVS_ERR_HIP if the
 * array's device address could not be taken when the context was created. */
size_t kvs_value_norms_noalloc_max_bytes(void);
kvs_status kvs_value_norms_noalloc(kvs_ctx ctx, int32_t P, int32_t Z, int32_t d, const float* Vz,
                                   double* signal);

/* Training queries (gist page, section 2 "Training Query Construction": real
 * queries of the recent context plus synthetic future queries whose content
 * is taken from the context by undoing RoPE and embedded again at future
 * positions, the sources sampled uniformly over the context).
 *   Qctx [P][g][N][d]  device: RoPE'd queries of the g query heads sharing
 *                      KV head p, at context positions 0..N-1
 *   src  [P][g][F]     device int32: source positions of the synthetic
 *                      queries (the caller's uniform draw over [0, N));
 *                      may be NULL when F == 0
 *   Q    [P][g(m+F)][d] device output: per problem the retain block
 *                      (head 0's rows at positions N-m..N-1, head 1's, ...)
 *                      then the future block (head h's query j at row
 *                      g m + h F + j): row Qctx[p][h][s] with s = src[p][h][j],
 *                      turned back by its rotation at s and forward by the
 *                      rotation at position N + j.
 * RoPE: channel c and c + d/2 (c < d/2) form a plane turned by
 * pos * theta^(-2c/d).  Retain rows are exact copies; future rows carry
 * float32 rounding of the turned values (the angle itself is reduced in
 * float64).  A source outside [0, N) gives a zero row and sets
 * KVS_FLAG_BADINDEX in flags[p] (device int32[P], may be NULL; bits are OR'ed
 * in, never cleared).  Errors: KVS_ERR_INVALID for P, g < 1, N < 1, m outside
 * [0, N], F < 0, g (m + F) < 1, d not one of 8, 16, 32, 64, 128, 256 or
 * theta <= 1; KVS_ERR_ALIGN for Qctx or Q not 16-byte aligned.  No workspace
 * is needed. */
#define KVS_FLAG_BADINDEX     16   /* a training-query source outside [0, N)  */
typedef struct {
  int32_t P, g, N, m, F, d;
  double  theta;        /* RoPE base (1e4 .. 1e6 in the Llama / Qwen families) */
} kvs_query_geom;
kvs_status kvs_build_queries(kvs_ctx ctx, const kvs_query_geom* q, const float* Qctx,
                             const int32_t* src, float* Q, int32_t* flags);

/* Use-side evaluation (gist page, section 2 "Problem Formulation": the
 * compressed cache should give the full cache's attention output for future
 * queries, the retain zone kept as is; "Loss Function": the LSE term keeps
 * the chunk's attention mass right when it is combined with other tokens).
 * For held-out queries Qh [P][n][d] (b->n rows per problem, b->k the
 * compressed sizes):
 *   Ofull = softmax(scale Qh [Kz; Kr]^T) [Vz; Vr]    (full cache)
 *   Ocomp = softmax(scale Qh [Kc; Kr]^T) [Vc; Vr]    (compressed cache)
 *   mse[p] = ||Ocomp - Ofull||_F^2 / (n d),  rel[p] = ||Ocomp - Ofull||_F / ||Ofull||_F
 * one softmax over each whole cache, no mask.  Kr, Vr [P][m][d] are the
 * retain zone (m >= 0; may be NULL when m == 0); Kc, Vc packed [sum k][d].
 * Ofull, Ocomp [P][n][d] are optional outputs (NULL: kept in the
 * workspace); mse [P] is required, rel [P] optional (device float).  Scores
 * are float64 products (float32 with KVS_LOGITS=fp32), outputs accumulate in
 * float32, the norms in float64 in a fixed order.  The workspace is
 * kvs_use_eval_workspace_bytes(b, m) bytes (0: invalid batch or m). */
size_t kvs_use_eval_workspace_bytes(const kvs_batch* b, int32_t m);
kvs_status kvs_use_eval(kvs_ctx ctx, const kvs_batch* b, int32_t m, const float* Qh,
                        const float* Kz, const float* Vz, const float* Kr, const float* Vr,
                        const float* Kc, const float* Vc, float* Ofull, float* Ocomp,
                        float* mse, float* rel, void* ws, size_t ws_bytes);

/* Opt-in kernel timing, for measurement tools.  While enabled, the library
 * records a HIP event pair on the context stream around each launch of its
 * main kernels and accumulates, per kernel, the launch count, the summed
 * event time and the algorithmic flops / HBM bytes of those launches (the
 * method's own work, not hardware counters; zero where not tracked).
 * kvs_profile_enable clears the totals; its argument is 0 (off), -1 (all
 * kernels) or a bitmask over attn_fwd (bit 0), attn_bwd, gram, potrf_panel,
 * trailing, back_subst, hist_dots, direction, importance, ref_attn_fwd,
 * merge, build_queries, use_attn_fwd, attn_pv (bit 13: the forward that
 * reads stored scores after a value re-solve), key_digits (bit 14: the digit
 * planes of the keys for the integer score products), resid_rhs and
 * fwd_subst (bits 15, 16: the refinement step of a value solve) and
 * gram_split (bit 17: the Gram's launches whose 128x128 or 256x256 tiles
 * take the products of exact three-piece bf16 splits; "gram" counts the
 * fp32 ones), resid_rhs_split (bit 18: the refinement residual on those
 * products; "resid_rhs" counts the fp32 one) and attn_bwd_split (bit 19:
 * the backward on those products; "attn_bwd" counts the fp32 one).
 * kvs_profile_read
 * synchronises the stream and writes up to max entries (kernels with
 * launches) to out. */
typedef struct {
  char    name[32];
  int64_t launches;
  double  total_ms;
  double  flops;
  double  bytes;
} kvs_kernel_stats;
kvs_status kvs_profile_enable(kvs_ctx ctx, int32_t enable);
kvs_status kvs_profile_read(kvs_ctx ctx, kvs_kernel_stats* out, int32_t max, int32_t* count);

#ifdef __cplusplus
}
#endif
#endif /* KVSCULPT_H */
