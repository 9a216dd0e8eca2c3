// Workspace layout and launch split factors for a batch of problems.
#include "plan.h"

#include <algorithm>
#include <cstdio>

namespace kvs {

namespace {

constexpr int kTargetWG = 1024;   // ~4 workgroups per CU on a 256-CU part

int split_for(long long base_wgs, int max_split) {
  if (base_wgs <= 0) return 1;
  long long c = (kTargetWG + base_wgs - 1) / base_wgs;
  if (c < 1) c = 1;
  if (c > max_split) c = max_split;
  return (int)c;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

int key_chunks(int P, int n, int keys, int cap) {
  if (keys <= 0) return 0;
  const long long qtiles = (n + 63) / 64;
  const int c = std::max(1, std::min(split_for((long long)P * qtiles, (keys + 63) / 64), cap));
  const int len = (((keys + c - 1) / c) + 63) / 64 * 64;
  return (keys + len - 1) / len;
}

std::string make_plan(const kvs_batch* b, const kvs_opts* o, Plan* pl) {
  if (!b) return "batch is NULL";
  if (b->P < 1) return "P must be >= 1";
  if (b->d != 64 && b->d != 128) return "d must be 64 or 128";
  if (b->Z < 1) return "Z must be >= 1";
  if (b->n < 1) return "n must be >= 1";
  // tile loads address up to 128 rows of the stored scores (and a problem's
  // n rows of targets) through 32-bit byte ranges and offsets
  if (b->n > (1 << 21)) return "n must be <= 2097152";
  if (!(b->scale > 0.0)) return "scale must be > 0";
  if (!(b->lambda >= 0.0)) return "lambda must be >= 0";
  if (!(b->ridge_rel >= 0.0)) return "ridge_rel must be >= 0";
  int H = 10;
  if (o) {
    if (o->history < 1 || o->history > kHistMax) return "history must be in [1, 16]";
    if (o->iters < 0) return "iters must be >= 0";
    if (o->vc_every < 1) return "vc_every must be >= 1";
    if (o->max_backtracks < 1) return "max_backtracks must be >= 1";
    if (!(o->c1 > 0.0 && o->c1 < 1.0)) return "c1 must be in (0, 1)";
    if (!(o->shrink > 0.0 && o->shrink < 1.0)) return "shrink must be in (0, 1)";
    H = o->history;
  }
  Plan& p = *pl;
  p = Plan();
  p.P = b->P; p.d = b->d; p.Z = b->Z; p.n = b->n; p.npad = (b->n + 3) & ~3; p.H = H;
  p.info.resize(p.P);
  long long koff = 0, soff = 0, moff = 0, xoff = 0, gtoff = 0, gtoff4 = 0;
  for (int i = 0; i < p.P; ++i) {
    int k = b->k ? b->k[i] : b->Z;
    if (k < 1 || k > b->Z) return "k[p] must be in [1, Z]";
    ProbInfo& q = p.info[i];
    q.k = k;
    q.kpad = (k + kTile - 1) / kTile * kTile;
    q.koff = (int)koff;
    q.xorder = i;
    q.soff = soff;
    q.moff = moff;
    q.xoff = xoff;
    q.gtoff = (int)gtoff;
    q.gtoff4 = (int)gtoff4;
    q.korder = i;
    gtoff += gram128_tiles((q.kpad / kTile + 1) / 2);
    gtoff4 += gram128_tiles((q.kpad / kTile + 3) / 4);
    koff += k;
    soff += (long long)k * p.npad;
    moff += (long long)(q.kpad + p.d) * q.kpad;
    xoff += (long long)q.kpad * p.d;
    p.kmax = std::max(p.kmax, k);
    p.kpadmax = std::max(p.kpadmax, q.kpad);
  }
  if (koff > 0x7fffffffLL) return "sum of k too large";
  if (gtoff > 0x7fffffffLL / 2) return "too many Gram tiles";
  p.gtot = gtoff;
  p.gtot4 = gtoff4;
  // Slot order for kernels that keep each problem's workgroups on one XCD
  // (a contiguous range of logical slots per XCD): problems by k, largest
  // first, dealt to the 8 XCDs in snake order, so every XCD gets about the
  // same number of problems and the same total k.
  {
    std::vector<int> byk(p.P);
    for (int i = 0; i < p.P; ++i) byk[i] = i;
    std::stable_sort(byk.begin(), byk.end(), [&](int x, int y) { return p.info[x].k > p.info[y].k; });
    std::vector<std::vector<int>> bin(8);
    for (int i = 0; i < p.P; ++i) {
      const int r = i / 8, c = i % 8;
      bin[(r & 1) ? 7 - c : c].push_back(byk[i]);
    }
    int s = 0;
    for (const auto& b : bin)
      for (int prob : b) p.info[s++].xorder = prob;
  }
  // Grid rows of the forwards: a workgroup's work grows with its problem's k,
  // so the largest problems are dispatched first and the last round of
  // workgroups is the shortest.
  {
    std::vector<int> byk(p.P);
    for (int i = 0; i < p.P; ++i) byk[i] = i;
    std::stable_sort(byk.begin(), byk.end(), [&](int x, int y) { return p.info[x].k > p.info[y].k; });
    for (int i = 0; i < p.P; ++i) p.info[i].korder = byk[i];
  }
  p.ktot = koff; p.stot = soff; p.mtot = moff; p.kpadtot = xoff / p.d;

  const long long qtiles = (p.n + 63) / 64;
  p.Cref = key_chunks(p.P, p.n, p.Z, kMaxChunks);
  p.C = key_chunks(p.P, p.n, p.kmax, kMaxChunks);
  // Query splits of the backward.  A workgroup takes one 64-key tile and a
  // chunk of whole 64-query tiles; two run per CU.  Splitting until there are
  // at least six rounds of them (3072) keeps the last round's tail small,
  // while every workgroup keeps at least four query tiles to amortise its
  // fixed cost.  (Measured on the 56-problem full cache: one split 1.86 s,
  // two 1.70 s, four 1.63 s, six 1.63 s, eight 1.64 s per main run.)  No
  // workgroup sweeps more than 64 query tiles: long sweeps leave long tails
  // in the launches of the line-search slots, where only the problems whose
  // trial was accepted run (long-context cache, 280 query tiles: one split
  // 82.6 TF/s, five 93.4 TF/s over the timed blocks).
  {
    long long ktiles = 0;
    for (const ProbInfo& q : p.info) ktiles += (q.k + 63) / 64;
    const long long want = std::max((3072 + ktiles - 1) / std::max(1LL, ktiles), (qtiles + 63) / 64);
    const long long cap = std::max(1LL, qtiles / 4);
    p.Cn = (int)std::max(1LL, std::min(want, cap));
  }
  const int KT = p.kpadmax / kTile;
  const long long gtiles = (long long)KT * (KT + 1) / 2 + (long long)(p.d / kTile) * KT;
  p.Cg = split_for((long long)p.P * gtiles, (int)qtiles);
  p.Cq = split_for((long long)p.P * ((p.Z + 63) / 64), (int)qtiles);
  p.Crf = refine_splits(p.P, p.kpadmax, p.n);
  {
    // Two (four) panels per trailing pass halve (quarter) the trailing
    // read-modify-write; they add panel products to the critical path of
    // some launches, which small batches (latency-bound) do not recover.  (Measured:
    // 2 problems at k = 960 slower by ~1 us per launch; 56 ragged problems
    // at k <= 1920 and 256 at k <= 4680 faster, 104 -> 82 ms and
    // 3.95 -> 1.92 s of Cholesky per run.)
    const int KTm = p.kpadmax / kTile, DT = p.d / kTile;
    long long trail1 = 0;
    for (const ProbInfo& q : p.info)
      for (int j = 1; j < q.kpad / kTile; ++j) trail1 += chol_trail_wgs(q.kpad / kTile, DT, j, 1);
    p.chol_S = trail1 >= 131072 ? 4 : (trail1 >= 16384 ? 2 : 1);
    p.chol_wgs.assign(KTm + 1, 0);
    for (int j = -1; j < KTm; ++j) {
      long long t = 0;
      for (const ProbInfo& q : p.info)
        t += chol_panel_wgs(q.kpad / kTile, DT, j) + chol_trail_wgs(q.kpad / kTile, DT, j, p.chol_S);
      if (t > 0x7fffffffLL) return "Cholesky launch has too many tiles";
      p.chol_wgs[j + 1] = (int)t;
    }
  }
  p.nblk = merge_blocks(p.n);
  p.nchv = vec_chunks((long long)p.kmax * p.d);
  p.nchd = dots_chunks((long long)p.kmax * p.d);
  const int Cmax = std::max(p.Cref, p.C);
  const size_t f = 4;
  size_t off = 0;
  auto take = [&](Region& r, size_t bytes) {
    r.off = off;
    r.bytes = bytes;
    off = align256(off + bytes);
  };
  take(p.r_info, sizeof(ProbInfo) * p.P);
  take(p.r_state, sizeof(LbState) * p.P);
  take(p.r_status, sizeof(int) * p.P);
  take(p.r_flags, sizeof(int) * p.P);
  take(p.r_loss, sizeof(float) * p.P);
  take(p.r_cnt, sizeof(unsigned) * 2 * p.P);
  take(p.r_yref, f * p.P * p.n * p.d);
  take(p.r_lseref, f * p.P * p.n);
  take(p.r_St, f * p.stot);
  take(p.r_Opart, f * Cmax * (size_t)p.P * p.n * p.d);
  take(p.r_Mpart, f * Cmax * (size_t)p.P * p.n);
  take(p.r_Lpart, f * Cmax * (size_t)p.P * p.n);
  take(p.r_G, f * (size_t)p.P * p.n * p.d);
  take(p.r_e, f * (size_t)p.P * p.n);
  take(p.r_crow, f * (size_t)p.P * p.n);
  take(p.r_part, sizeof(double) * 2 * (size_t)p.P * p.nblk);
  take(p.r_dK, f * (size_t)p.Cn * p.ktot * p.d);
  take(p.r_grad, f * (size_t)p.ktot * p.d);
  take(p.r_Mg, p.Cg > 1 ? f * (size_t)p.Cg * p.mtot : 0);
  take(p.r_M, f * (size_t)p.mtot);
  take(p.r_tr, sizeof(double) * (size_t)p.P * KT);
  take(p.r_mu, sizeof(double) * p.P);
  take(p.r_cinfo, sizeof(int) * p.P);
  take(p.r_X, f * (size_t)p.kpadtot * p.d);
  take(p.r_Dinv, f * (size_t)p.kpadtot * kTile);
  take(p.r_R, sizeof(double) * (size_t)p.Crf * p.kpadtot * p.d);
  take(p.r_coff, sizeof(int) * (size_t)(p.kpadmax / kTile + 1) * (p.P + 1));
  take(p.r_imp, f * 2 * (size_t)p.Cq * p.P * p.Z);
  take(p.r_idx, sizeof(int) * (size_t)p.ktot);
  take(p.r_hpart, sizeof(double) * (size_t)p.P * p.nchd * kDots);
  take(p.r_g, f * (size_t)p.ktot * p.d);
  take(p.r_p, f * (size_t)p.ktot * p.d);
  take(p.r_Kt, f * (size_t)p.ktot * p.d);
  // digit planes of the keys and their scales (integer score products)
  take(p.r_K8, (size_t)kDigits * p.ktot * p.d);
  take(p.r_Kscl, f * (size_t)p.ktot);
  take(p.r_S, f * (size_t)(H + 1) * p.ktot * p.d);
  take(p.r_Yh, f * (size_t)(H + 1) * p.ktot * p.d);
  take(p.r_Kc, f * (size_t)p.ktot * p.d);
  take(p.r_Vc, f * (size_t)p.ktot * p.d);
  p.ws_bytes = off;

  off = 0;
  take(p.s_state, sizeof(LbState) * p.P);
  take(p.s_g, f * (size_t)p.ktot * p.d);
  take(p.s_p, f * (size_t)p.ktot * p.d);
  take(p.s_S, f * (size_t)(H + 1) * p.ktot * p.d);
  take(p.s_Yh, f * (size_t)(H + 1) * p.ktot * p.d);
  p.state_bytes = off;
  return std::string();
}

std::string make_use_plan(const kvs_batch* b, int m, UsePlan* up) {
  Plan base;
  std::string e = make_plan(b, nullptr, &base);
  if (!e.empty()) return e;
  if (m < 0) return "m must be >= 0";
  UsePlan& u = *up;
  u = UsePlan();
  u.P = base.P; u.d = base.d; u.Z = base.Z; u.n = base.n; u.m = m; u.kmax = base.kmax;
  u.ktot = base.ktot;
  u.info = base.info;
  // the two merges read planes [0, Cz + Cr) and [Cz, Cz + Cr + Cc): each at
  // most kMaxChunks
  u.Cr = m > 0 ? key_chunks(u.P, u.n, m, 4) : 0;
  u.Cz = key_chunks(u.P, u.n, u.Z, kMaxChunks - u.Cr);
  u.Cc = key_chunks(u.P, u.n, u.kmax, kMaxChunks - u.Cr);
  u.nblk = use_err_blocks(u.n);
  const size_t f = 4, planes = (size_t)(u.Cz + u.Cr + u.Cc), pn = (size_t)u.P * u.n;
  size_t off = 0;
  auto take = [&](Region& r, size_t bytes) {
    r.off = off;
    r.bytes = bytes;
    off = align256(off + bytes);
  };
  take(u.r_info, sizeof(ProbInfo) * u.P);
  take(u.r_Opart, f * planes * pn * u.d);
  take(u.r_Mpart, f * planes * pn);
  take(u.r_Lpart, f * planes * pn);
  take(u.r_Of, f * pn * u.d);
  take(u.r_Oc, f * pn * u.d);
  take(u.r_lf, f * pn);
  take(u.r_lc, f * pn);
  take(u.r_part, sizeof(double) * 2 * (size_t)u.P * u.nblk);
  u.ws_bytes = off;
  return std::string();
}

}  // namespace kvs
