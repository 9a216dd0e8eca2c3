// Use-side error of a compressed cache (KVSculpt: KV Cache Compression as
// Distillation, gist.science page, section 2 "Problem Formulation": the
// compressed cache should reproduce the full cache's attention output for
// future queries).
//
// The two outputs themselves come from the split-key forward and its merge:
// the partials of the compress zone, the retain zone and the compressed
// pairs sit in adjacent planes, so each use-side output is one ordinary
// merge over a contiguous plane range.  What is left is a reduction: per
// problem, the squared Frobenius norm of the difference and of the full
// output, in float64 with a fixed order (block partials, then one workgroup
// per problem), so the result does not depend on scheduling.
#include "kvs_internal.h"

namespace kvs {
namespace {

constexpr int kRowsPerBlock = 16;

// partial sums over 16 rows of one problem: part[p][blk] = (sum D^2, sum F^2)
template <int D>
__global__ __launch_bounds__(256) void use_err_kernel(UseErrArgs a) {
  constexpr int V4 = kRowsPerBlock * D / 4 / 256;   // float4 per thread
  const int p = blockIdx.y, blk = blockIdx.x, tid = threadIdx.x;
  const long long r0 = (long long)blk * kRowsPerBlock;
  const long long base = ((long long)p * a.n + r0) * D;
  const long long lim = (long long)min(kRowsPerBlock, a.n - (int)r0) * D;
  f32x4 fv[V4], cv[V4];
#pragma unroll
  for (int u = 0; u < V4; ++u) {
    const long long i = 4LL * (tid + 256 * u);
    const bool ok = i < lim;
    fv[u] = ok ? *(const f32x4*)(a.Of + base + i) : f32x4{0.f, 0.f, 0.f, 0.f};
    cv[u] = ok ? *(const f32x4*)(a.Oc + base + i) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  double dd = 0.0, ff = 0.0;
#pragma unroll
  for (int u = 0; u < V4; ++u)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double f = fv[u][j], df = (double)cv[u][j] - f;
      dd = fma(df, df, dd);
      ff = fma(f, f, ff);
    }
  __shared__ double red[2][256];
  red[0][tid] = dd;
  red[1][tid] = ff;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) {
      red[0][tid] += red[0][tid + off];
      red[1][tid] += red[1][tid + off];
    }
    __syncthreads();
  }
  if (tid == 0) {
    double* dst = a.part + ((size_t)p * gridDim.x + blk) * 2;
    dst[0] = red[0][0];
    dst[1] = red[1][0];
  }
}

__global__ __launch_bounds__(256) void use_err_final_kernel(UseErrArgs a) {
  const int p = blockIdx.x, tid = threadIdx.x;
  const double* src = a.part + (size_t)p * a.nblk * 2;
  double dd = 0.0, ff = 0.0;
  for (int b = tid; b < a.nblk; b += 256) {
    dd += src[2 * b];
    ff += src[2 * b + 1];
  }
  __shared__ double red[2][256];
  red[0][tid] = dd;
  red[1][tid] = ff;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) {
      red[0][tid] += red[0][tid + off];
      red[1][tid] += red[1][tid + off];
    }
    __syncthreads();
  }
  if (tid == 0) {
    const double s = red[0][0], t = red[1][0];
    a.mse[p] = (float)(s / ((double)a.n * a.d));
    if (a.rel) a.rel[p] = t > 0.0 ? (float)sqrt(s / t) : 0.f;
  }
}

}  // namespace

int use_err_blocks(int n) { return (n + kRowsPerBlock - 1) / kRowsPerBlock; }

void launch_use_err(const UseErrArgs& a, hipStream_t s) {
  dim3 grid(a.nblk, a.P);
  if (a.d == 128) hipLaunchKernelGGL((use_err_kernel<128>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((use_err_kernel<64>), grid, dim3(256), 0, s, a);
  hipLaunchKernelGGL(use_err_final_kernel, dim3(a.P), dim3(256), 0, s, a);
}

}  // namespace kvs
