// Training-query construction (KVSculpt: KV Cache Compression as
// Distillation, gist.science page, section 2 "Training Query Construction"):
// the retain-zone queries of every query head, copied, followed by synthetic
// future queries -- a context query with its rotary embedding removed at its
// own position and applied again at a future position.
//
// Removing the rotation at s and applying it at N + j is one rotation of each
// channel plane (c, c + d/2) by (N + j - s) * theta^(-2c/d).  That angle
// reaches ~3.5e4 rad on long contexts, where float32 would lose ~2e-3 rad, so
// it is formed and reduced modulo 2 pi in float64; only the reduced angle
// (|r| <= pi) goes to the float32 sine and cosine.  The kernel streams rows:
// each thread owns four consecutive planes of one row and moves them with
// 16-byte loads and stores, so the cost is the HBM traffic of one read and
// one write per output element.
#include "kvs_internal.h"

namespace kvs {
namespace {

constexpr double kTwoPiHi = 6.283185307179586;         // 2 pi rounded to double
constexpr double kTwoPiLo = 2.4492935982947064e-16;    // 2 pi - kTwoPiHi
constexpr double kInvTwoPi = 0.15915494309189535;

template <int D>
__global__ __launch_bounds__(256) void build_queries_kernel(QueryArgs a) {
  constexpr int TPR = D / 8;          // threads per row, four planes each
  constexpr int RPB = 256 / TPR;      // rows per workgroup
  constexpr int H4 = D / 8;           // float4 offset of the second half of a row
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int t = threadIdx.x % TPR;
  const long long per_p = (long long)a.g * (a.m + a.F);
  if (row >= (long long)a.P * per_p) return;
  const long long p = row / per_p;
  const long long w = row - p * per_p;
  f32x4* out = reinterpret_cast<f32x4*>(a.Q + row * D);

  if (w < (long long)a.g * a.m) {                          // retain query: a copy
    const int hh = (int)(w / a.m), i = (int)(w % a.m);
    const long long srow = (p * a.g + hh) * a.N + (a.N - a.m + i);
    const f32x4* in = reinterpret_cast<const f32x4*>(a.Qctx + srow * D);
    const f32x4 lo = in[t], hi = in[t + H4];
    out[t] = lo;
    out[t + H4] = hi;
    return;
  }
  const long long jj = w - (long long)a.g * a.m;
  const int hh = (int)(jj / a.F), j = (int)(jj % a.F);
  const int s = a.src[(p * a.g + hh) * a.F + j];
  if (s < 0 || s >= a.N) {                                 // invalid source: zero row
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    out[t] = z;
    out[t + H4] = z;
    if (t == 0 && a.flags) atomicOr(a.flags + p, a.bad_flag);
    return;
  }
  const long long srow = (p * a.g + hh) * a.N + s;
  const f32x4* in = reinterpret_cast<const f32x4*>(a.Qctx + srow * D);
  const f32x4 lo = in[t], hi = in[t + H4];

  const double delta = (double)(a.N + j - s);              // exact: |delta| < 2^31
  double f = exp2(-(2.0 * (4 * t) / D) * a.log2_theta);    // theta^(-2c/d), c = 4t
  f32x4 olo, ohi;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const double ang = delta * f;
    const double q = rint(ang * kInvTwoPi);
    double r = fma(-q, kTwoPiHi, ang);
    r = fma(-q, kTwoPiLo, r);
    float sn, cs;
    sincosf((float)r, &sn, &cs);
    olo[k] = lo[k] * cs - hi[k] * sn;
    ohi[k] = lo[k] * sn + hi[k] * cs;
    f *= a.freq_ratio;                                     // next plane's frequency
  }
  out[t] = olo;
  out[t + H4] = ohi;
}

}  // namespace

void launch_build_queries(const QueryArgs& a, hipStream_t s) {
  const long long rows = (long long)a.P * a.g * (a.m + a.F);
  if (rows <= 0) return;
  const int rpb = 256 / (a.d / 8);
  const unsigned blocks = (unsigned)((rows + rpb - 1) / rpb);
  switch (a.d) {
#define KVS_BQ(DD) case DD: hipLaunchKernelGGL((build_queries_kernel<DD>), dim3(blocks), dim3(256), 0, s, a); break;
    KVS_BQ(8) KVS_BQ(16) KVS_BQ(32) KVS_BQ(64) KVS_BQ(128) KVS_BQ(256)
#undef KVS_BQ
    default: break;
  }
}

}  // namespace kvs
