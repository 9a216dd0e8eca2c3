// Adam update of the compressed keys (Kingma & Ba, "Adam: A Method for
// Stochastic Optimization", 2015, Algorithm 1), the first-order optimizer
// that KVSculpt's ablation puts in place of L-BFGS (gist.science page,
// section 4 "Optimizer Efficacy").
//
// Elementwise over the packed keys: moment averages, bias-corrected step.  A
// workgroup row (blockIdx.y) is one problem, so a non-finite gradient can be
// reported in that problem's flag word; such an element is left as it was.
// HBM-bound: reads x, g, m, v and writes x, m, v, 16-byte accesses.
#include "kvs_internal.h"

namespace kvs {
namespace {

__global__ __launch_bounds__(256) void adam_kernel(AdamArgs a) {
  const int p = blockIdx.y;
  const ProbInfo pi = a.info[p];
  const long long base = (long long)pi.koff * a.d;       // multiple of 4: d is 64 or 128
  const long long n4 = (long long)pi.k * a.d / 4;
  bool bad = false;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n4; i += (long long)gridDim.x * 256) {
    f32x4* xp = reinterpret_cast<f32x4*>(a.x + base) + i;
    f32x4* mp = reinterpret_cast<f32x4*>(a.m + base) + i;
    f32x4* vp = reinterpret_cast<f32x4*>(a.v + base) + i;
    const f32x4 g = reinterpret_cast<const f32x4*>(a.g + base)[i];
    f32x4 x = *xp, m = *mp, v = *vp;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (!isfinite(g[j])) {
        bad = true;
        continue;
      }
      m[j] = a.b1 * m[j] + (1.f - a.b1) * g[j];
      v[j] = a.b2 * v[j] + (1.f - a.b2) * (g[j] * g[j]);
      const float denom = sqrtf(v[j]) * a.inv_sqrt_bc2 + a.eps;
      x[j] -= a.step * (m[j] / denom);
    }
    *xp = x;
    *mp = m;
    *vp = v;
  }
  if (bad && a.flags) atomicOr(a.flags + p, a.nonfinite_flag);
}

}  // namespace

void launch_adam(const AdamArgs& a, int kmax, hipStream_t s) {
  const long long n4 = (long long)kmax * a.d / 4;
  const long long want = (n4 + 255) / 256;
  const unsigned bx = (unsigned)(want < 64 ? (want > 0 ? want : 1) : 64);
  hipLaunchKernelGGL(adam_kernel, dim3(bx, a.P), dim3(256), 0, s, a);
}

}  // namespace kvs
