// Internal declarations shared by the HIP kernels and the host driver of the
// KVSculpt library (gfx950 only).  Nothing here is part of the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvs {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kHistMax = 16;            // L-BFGS pairs kept at most
constexpr int kSlots = kHistMax + 1;    // ring slots (history + one staging slot)
constexpr int kTile = 64;               // key/query tile edge used across kernels

// Raw buffer resource over `bytes` bytes from `base` (both uniform across the
// wave).  Loads through it at byte offsets at or past `bytes` return zero, so
// the loads of a tile that runs past the end of its range need no clamping.
// The range is a 32-bit count: callers keep it below 2^31 bytes (with at most
// 2^21 training queries per problem every range in the kernels is a tile's
// rows, at most 1 GiB).  The last descriptor word selects untyped 32-bit
// access on gfx9 parts.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, long long bytes) {
  const int nr = bytes <= 0 ? 0 : (bytes >= 0x7fffffffLL ? 0x7fffffff : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nr, 0x00020000);
}
// 16 (4) bytes at byte offset `off` of the resource, as floats
__device__ __forceinline__ f32x4 buf_load4(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ i32x4 buf_load4i(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ float buf_load1(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
// 4 bytes to byte offset voff + soff of the resource (soff uniform); callers
// store only in range
__device__ __forceinline__ void buf_store1(__amdgpu_buffer_rsrc_t r, int voff, int soff, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, voff, soff, 0);
}

// Per-problem geometry, uploaded once per call into the workspace.
struct ProbInfo {
  int k;        // compressed pairs
  int kpad;     // k rounded up to kTile (Gram / Cholesky edge)
  int koff;     // first row of the problem in packed [sum k][d] arrays
  int xorder;   // problem that kernels grouping a problem's workgroups on one XCD
                // run at logical slot p (slots ordered so each XCD gets equal work)
  long long soff;   // offset (floats) of the problem's stored scores [k][n]
  long long moff;   // offset (floats) of the problem's augmented Gram [(kpad+d)][kpad]
  long long xoff;   // offset (floats) of the problem's padded solve rows [kpad][d]
  int gtoff;        // first tile of the problem in the flat order of the 128x128 Gram tiles
  int korder;       // problem that the forwards run at grid row p (largest k first)
  int gtoff4;       // first tile of the problem in the flat order of the 256x256 Gram tiles
};

// L-BFGS / line-search status of one problem.
// ST_DONE / ST_DONE_FAIL: the problem finished the iterations of the current
// block (the last one accepted / failed its search) and waits for the rest.
enum : int { ST_READY = 0, ST_SEARCH = 1, ST_ACCEPT = 2, ST_FAIL = 3, ST_DONE = 4, ST_DONE_FAIL = 5 };
constexpr int kAllStates = 0x3F;   // active_mask selecting every status
constexpr int kMaxChunks = 16;     // key chunks of the split forward (merge unrolls over them)
constexpr int kMaxRefineSplits = 16;   // query splits of the refinement residual (summed unrolled)

// Per-problem optimizer state, kept in device memory between kernels.
struct LbState {
  double L;          // loss at the current keys x
  double Ltrial;     // loss at the last trial point
  double gtp;        // g^T p of the current direction
  double alpha;      // step of the current trial
  double gg;         // g^T g
  int status;        // ST_*
  int trials;        // trials used in the current search
  int flags;         // accumulated KVS_FLAG_* bits
  int count;         // pairs in the history
  int stage;         // ring slot receiving the next (s, y)
  int st_valid;      // stored scores belong to x (not to a rejected trial)
  int iter;          // iterations finished in the current block
  int n_trial;       // line-search trial evaluations since the state was cleared
  int n_accept;      // accepted trials since the state was cleared
  int pad_;
  int order[kHistMax];          // history slots, oldest first
  double rho[kSlots];
  double SY[kSlots][kSlots];    // s_i . y_j by slot
  double YY[kSlots][kSlots];    // y_i . y_j by slot
  double Sg[kSlots], Yg[kSlots];
  double coef_g;                // direction p = coef_g g + sum cs s + sum cy y
  double cs[kSlots], cy[kSlots];
};

static_assert(sizeof(LbState) % 8 == 0, "LbState is copied in 8-byte words");

// Workgroups of a launch go to the 8 XCDs (each with its own L2) round-robin
// by linear index.  xcd_remap turns the hardware linear index into a logical
// one such that each XCD receives a contiguous range of logical indices, so
// neighbouring logical workgroups (which share operands) share an L2.  It is
// a bijection on [0, total).
__device__ __forceinline__ unsigned xcd_remap(unsigned L, unsigned total) {
  const unsigned q = total / 8, r = total % 8;
  const unsigned xcd = L % 8, slot = L / 8;
  return (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}
// Logical (x, y, z) of this workgroup under xcd_remap, x fastest.
__device__ __forceinline__ void xcd_block(unsigned& x, unsigned& y, unsigned& z) {
  const unsigned nx = gridDim.x, ny = gridDim.y, total = nx * ny * gridDim.z;
  const unsigned L = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
  const unsigned Lp = xcd_remap(L, total);
  x = Lp % nx;
  y = (Lp / nx) % ny;
  z = Lp / (nx * ny);
}

// Cross-workgroup partial sums ("last workgroup finalises" reductions).
// Partials are written and read with device-scope relaxed atomics, which are
// coherent across the XCDs' L2 caches, and each wave waits for its own
// stores before the arrival counter is bumped; no workgroup needs a
// device-wide release fence (an L2 write-back on this part).
__device__ __forceinline__ void coherent_store(double* p, double v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double coherent_load(const double* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// all memory operations this wave issued have completed
__device__ __forceinline__ void wait_own_stores() { __builtin_amdgcn_s_waitcnt(0); }
// arrival on a per-problem counter; true for the last of `total` arrivals
__device__ __forceinline__ bool arrive_last(unsigned* counter, unsigned total) {
  const unsigned prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return prev == total - 1;
}

// Number of dot products each WG of the history kernel emits per problem.
constexpr int kDots = 5 * kSlots + 4;

// ---- launchers (device code in the .hip files) ----------------------------

struct FwdArgs {
  const float* Q; const float* K; const float* V;
  const LbState* st;       // per-problem state (status); NULL = all active
  int active_mask;         // bit (1 << status) selects the problems processed
  const float* shift;      // [P][n] per-row score shift, NULL = none
  float* St;               // stored shifted scores (NULL = do not store)
  const float* Sload;      // non-NULL: take the scores from these stored ones
                           // (keys unchanged since they were stored; needs info)
  float* Opart; float* Mpart; float* Lpart;
  const ProbInfo* info;    // NULL: uniform k = kuni rows at K + p*kuni*d
  int P, n, C, kuni, kmax;
  double scale;
  // integer score products (mode LOGIT_I8): digit planes of the keys and their
  // row scales, as written by launch_digit_rows for the rows of K
  const int* K8; const float* Kscl; long long k8rows;
};
// Score (logit) arithmetic of the forward: fp32 MFMA, fp64 MFMA, or exact
// integer products of base-128 digits on int8 MFMA.
enum { LOGIT_F32 = 0, LOGIT_F64 = 1, LOGIT_I8 = 2 };
constexpr int kDigits = 5;   // base-128 digits per element of the integer scores
void launch_attn_fwd(const FwdArgs& a, int d, int logit_mode, hipStream_t s);
// Digit planes of `rows` rows of X (d floats each) for LOGIT_I8 forwards:
// planes [5][rows][d] bytes, scales [rows].
void launch_digit_rows(const float* X, long long rows, int d, int* planes, float* scl, hipStream_t s);

struct MergeArgs {
  const float* Opart; const float* Mpart; const float* Lpart;
  LbState* st; int active_mask;
  const float* Y; const float* lse;   // loss mode: targets; ref mode: NULL
  float* Yout; float* lse_out;        // ref mode outputs
  float* G; float* e; float* crow;    // loss mode outputs
  double* part;                       // [P][nblk][2] loss / output-term partials
  unsigned* counter;                  // [P] arrival counters (zero between launches)
  int P, n, C;
  double lambda;
  // per-problem finalisation, done by the last workgroup of each problem:
  //   0 = write loss / mse, 1 = Armijo trial, 2 = refresh L at the keys
  int fin_mode;
  double c1, shrink; int max_bt;
  float* loss; float* mse;
  int* status_view;                   // device int[P] copy of the status for the host
};
void launch_merge(const MergeArgs& a, int d, bool loss_mode, hipStream_t s);
int merge_blocks(int n);

struct BwdArgs {
  const float* Q; const float* St; const float* G; const float* e; const float* crow;
  const float* K; const float* V;
  const LbState* st; int active_mask;
  float* dKpart;           // [Cn][sum k][d]
  const ProbInfo* info;
  int P, n, Cn, kmax, ktot;
  int split3;              // products of exact three-piece bf16 splits (else fp32)
};
void launch_attn_bwd(const BwdArgs& a, int d, hipStream_t s);

struct GramArgs {
  const float* St; const float* e; const float* Y;
  const LbState* st; int active_mask;
  float* Mpart;            // [Cg][sum M]
  const ProbInfo* info;
  int P, n, Cg, kpadmax; long long mtot;
  long long gtot;          // 128x128 tiles of all problems (flat order, see gram_queue_tile)
  long long gtot4;         // 256x256 tiles of all problems (same order over 256-key tiles)
  int split3;              // products of exact three-piece bf16 splits (else fp32)
  int tile256;             // split products on 256x256 tiles: 0 never, 1 with >= 2048 of them, 2 always
};
void launch_gram(const GramArgs& a, int d, hipStream_t s);
// whether launch_gram takes its large-batch tiles (128x128 or 256x256) with
// the split bf16 products
bool gram_split_products(const GramArgs& a);

// 128x128 Gram tiles of a problem with KT2 = ceil(kpad / 128) key tiles: the
// lower triangle of key rows plus one row of value tiles (Y^T A).
__host__ __device__ inline long long gram128_tiles(int KT2) {
  return (long long)KT2 * (KT2 + 1) / 2 + KT2;
}

// Tile u (0 .. gram128_tiles(KT2) - 1) of a problem in its operand-sharing
// order -> tile row I2 (KT2: the value row) and column J2.  The tile grid
// (rows 0..KT2, columns 0..KT2-1, J2 <= I2 for key rows) is cut into 8x8
// blocks taken row by row, tiles row by row inside a block, so that 64
// consecutive tiles read at most 16 row strips of the stored scores instead
// of up to 128.
__host__ __device__ inline bool gram_queue_tile(long long u, int KT2, int& I2, int& J2) {
  const int NBr = (KT2 + 8) / 8, NBc = (KT2 + 7) / 8;
  for (int BI = 0; BI < NBr; ++BI) {
    const int r0 = 8 * BI, r1 = (r0 + 8 < KT2 + 1) ? r0 + 8 : KT2 + 1;
    const int nbj = (BI + 1 < NBc) ? BI + 1 : NBc;
    for (int BJ = 0; BJ < nbj; ++BJ) {
      const int c0 = 8 * BJ, c1 = (c0 + 8 < KT2) ? c0 + 8 : KT2;
      long long cnt;
      if (BI > BJ) {
        cnt = (long long)(r1 - r0) * (c1 - c0);
      } else {
        // diagonal block: key row r takes columns c0..r, the value row all
        const int m = (r1 < KT2) ? r1 : KT2, t = m - r0;
        cnt = (long long)t * (t + 1) / 2 + (KT2 < r1 ? c1 - c0 : 0);
      }
      if (u >= cnt) {
        u -= cnt;
        continue;
      }
      for (int r = r0; r < r1; ++r) {
        const int cn = (r == KT2) ? c1 - c0 : ((r + 1 < c1 ? r + 1 : c1) - c0);
        if (u < cn) {
          I2 = r;
          J2 = c0 + (int)u;
          return true;
        }
        u -= cn;
      }
      return false;
    }
  }
  return false;
}

struct GramReduceArgs {
  const float* Mpart; float* M; double* trpart; const LbState* st; int active_mask;
  const ProbInfo* info; int P, Cg, kpadmax; long long mtot;
};
void launch_gram_reduce(const GramReduceArgs& a, int d, hipStream_t s);

struct CholArgs {
  float* M; float* Dinv; const double* trpart; double* mu; int* info_out;
  const LbState* st; int active_mask;
  const ProbInfo* info; int P, kpadmax; double ridge_rel;
  int* coff;   // [kpadmax/64 + 1][P + 1]: first workgroup of each problem in launch j (row j + 1)
  int S;       // panels per trailing pass (1 or 2)
};
// Workgroups of Cholesky launch j (-1 .. KT-1) for a problem with KT key
// tiles and DT value-row tiles: the panel rows of column block j (launch -1:
// the look-ahead of block 0 only), then the trailing tiles (I, J), I > J > j,
// that take the pending panels' update (lower triangle, then the value
// rows): at launches j = S, 2S, 3S, .. the S panels j - S .. j - 1 (S = 1, 2
// or 4).
__host__ __device__ inline int chol_pending(int j, int S) {
  // panels that column block j still lacks at launch j: those after the last
  // trailing pass before it (all earlier ones when there was none)
  if (j <= 0) return 0;
  const int m = (j - 1) / S;
  return m >= 1 ? j - S * m : j;
}
__host__ __device__ inline int chol_panel_wgs(int KT, int DT, int j) {
  return j >= KT ? 0 : (j < 0 ? 1 : KT + DT - j - 1);
}
__host__ __device__ inline int chol_trail_wgs(int KT, int DT, int j, int S) {
  if (j >= KT || j < S || j % S != 0) return 0;
  const int nj = KT - j - 1;
  return nj * (nj - 1) / 2 + DT * nj;
}
void launch_mu(const CholArgs& a, hipStream_t s);
void launch_chol_offsets(const CholArgs& a, int d, hipStream_t s);
void launch_chol_step(const CholArgs& a, int d, int panel, int wgs, hipStream_t s);

struct BackArgs {
  const float* M; float* X; const float* Dinv; float* Vc; const int* info_out; int* flags;
  LbState* st; int active_mask;
  const ProbInfo* info; int P, d, kpadmax;
  int lds_max;      // dynamic LDS bytes a workgroup may use (0: solve in global memory)
  int accumulate;   // 0: Vc = X; 1: Vc += X (refinement correction)
};
size_t back_subst_lds_bytes(int kpadmax);
void launch_back_subst(const BackArgs& a, int d, hipStream_t s);

// Refinement step of the value solve: fp64 partials of A^T G per query split
// ([Cr][kpadtot][d], problem p at xoff), then r and the forward substitution
// L Z = r, Z written into the A^T Y rows of M.
struct RhsArgs {
  const float* St; const float* e; const float* G;
  const ProbInfo* info; double* Rpart;
  long long xtot;   // kpadtot * d
  int P, n, Cr, kpadmax;
  int split3;       // products of exact three-piece bf16 splits (else fp32)
};
struct FsubArgs {
  const double* Rpart; long long xtot; int Cr;
  const double* mu; const float* Vc; float* M; const float* Dinv; float* X;
  const int* info_out; const ProbInfo* info; int P, kpadmax, lds_max;
};
int refine_splits(int P, int kpadmax, int n);
void launch_resid_rhs(const RhsArgs& a, int d, hipStream_t s);
void launch_fwd_subst(const FsubArgs& a, int d, hipStream_t s);

struct ImpArgs {
  const float* Q; const float* Kz; const float* lse;
  float* Mpart; float* Spart;   // [Cq][P][Z]
  int P, n, Z, Cq; double scale;
};
void launch_importance(const ImpArgs& a, int d, hipStream_t s);

struct TopkArgs {
  const float* Mpart; const float* Spart; const float* Kz;
  int* idx; float* Kc; const ProbInfo* info;
  int P, Z, Cq, d;
};
void launch_topk(const TopkArgs& a, hipStream_t s);

// Gradient reduction fused with the L-BFGS vector updates.
//   mode 0 (accepted step, problems in ACCEPT): g_new = scale * sum_c dKpart[c],
//          x <- x + alpha p, s = x_new - x, y = g_new - g into the staging slot, g <- g_new
//   mode 1 (refresh, every problem): g <- g_new
//   mode 2 (plain output): gout <- g_new
struct GradUpdArgs {
  const float* dKpart; int Cn; double scale;
  LbState* st; int active_mask; int mode;
  float* x; const float* p; float* g; float* S; float* Yh; float* gout;
  const ProbInfo* info; int P, d, ktot, nch;
};
void launch_grad_update(const GradUpdArgs& a, hipStream_t s);

// Inner products of the history with the staged pair and the gradient, one
// workgroup per (chunk, slot); the last workgroup of each problem then runs
// the scalar L-BFGS logic (history update, two-loop coefficients, first step).
//   mode 0: after a search (ACCEPT: push + coefficients, FAIL: reset)
//   mode 1: gradient refreshed at the same keys; mode 2: history cleared
struct DotsArgs {
  float* g; float* S; float* Yh;   // written by the fused gradient pass
  LbState* st; int active_mask; int mode; int history; double curv_eps;
  double* part;                 // [P][nch][kDots]
  unsigned* counter;            // [P]
  const ProbInfo* info; int P, d, ktot, nch;
  int target;                   // iterations per block: a problem reaching it becomes ST_DONE*
  int* status_view;             // [P] copy of the new status (host-readable), or NULL
  // gradient pass fused in front of the inner products (grad != 0): g is
  // rebuilt as gscale * sum of the backward's Cn split partials; for an
  // accepted step also x <- x + alpha p and the staged s = x_new - x,
  // y = g_new - g.  Applied to the problems the kernel computes for.
  int grad;
  const float* dKpart; int Cn; double gscale; float* x; const float* pdir;
};
void launch_dots(const DotsArgs& a, hipStream_t s);
int dots_chunks(long long kmax_d);
int vec_chunks(long long kmax_d);

// For every problem in search: on its first trial the direction
// p = c_g g + sum (c_s s + c_y y); on every trial the trial keys kt = x + alpha p.
struct DirArgs {
  float* p; const float* g; const float* S; const float* Yh; const LbState* st;
  const float* x; float* kt;
  const ProbInfo* info; int P, d, ktot, nch;
};
void launch_direction(const DirArgs& a, hipStream_t s);

// Training queries: retain rows copied, future rows rotated by (N + j - s).
struct QueryArgs {
  const float* Qctx;       // [P][g][N][d]
  const int* src;          // [P][g][F]
  float* Q;                // [P][g(m+F)][d]
  int* flags;              // [P] or NULL: bad_flag set on an invalid source
  int P, g, N, m, F, d;
  int bad_flag;
  double log2_theta;       // log2 of the RoPE base
  double freq_ratio;       // theta^(-2/d): frequency of plane c+1 over plane c
};
void launch_build_queries(const QueryArgs& a, hipStream_t s);

// Use-side error: per problem sum (Oc - Of)^2 and sum Of^2 over [n][d] rows.
struct UseErrArgs {
  const float* Of; const float* Oc;
  double* part;            // [P][nblk][2]
  float* mse; float* rel;  // [P]; rel may be NULL
  int P, n, d, nblk;
};
int use_err_blocks(int n);
void launch_use_err(const UseErrArgs& a, hipStream_t s);

// One Adam step on the packed keys of every problem.
struct AdamArgs {
  float* x; const float* g; float* m; float* v;
  int* flags; int nonfinite_flag;     // flags [P] or NULL
  const ProbInfo* info; int P, d;
  float b1, b2, eps;
  float step;           // lr / (1 - b1^t)
  float inv_sqrt_bc2;   // 1 / sqrt(1 - b2^t)
};
void launch_adam(const AdamArgs& a, int kmax, hipStream_t s);

// Mean value-row norm per problem: chunk partials, then the per-problem sum.
struct VnormArgs {
  const float* V;          // [P][Z][d]
  double* part;            // [P][C]
  double* out;             // [P]
  int P, Z, C;
};
int value_norm_chunks(int P, int Z);
void launch_value_norms(const VnormArgs& a, int d, hipStream_t s);

void launch_write_info(ProbInfo* dst, const ProbInfo* src, int P, hipStream_t s);
void launch_fill_i32(int* p, int v, long long n, hipStream_t s);
void launch_fill_f32(float* p, float v, long long n, hipStream_t s);
void launch_state_init(LbState* st, int P, int clear, hipStream_t s);
void launch_state_flags_out(const LbState* st, int* flags, float* loss, int P, hipStream_t s);

}  // namespace kvs
