// Static allocation signal (KVSculpt, gist.science page, section 2 "Adaptive
// Budget Allocation" and section 4 "Budget Allocation": static signals such
// as value norms, against which the pilot MSE is compared): the mean
// Euclidean norm of each problem's compress-zone value rows.
//
// HBM-bound reduction.  A row is read by d/4 lanes with 16-byte loads
// (coalesced, eight rows per thread in flight), its squared norm summed in
// float64 across those lanes, and the row norms accumulated per workgroup
// over a chunk of rows; chunk
// partials are summed per problem in chunk order by a second kernel, so the
// result does not depend on scheduling.
#include "kvs_internal.h"

namespace kvs {
namespace {

template <int D>
__global__ __launch_bounds__(256) void value_norm_kernel(VnormArgs a) {
  constexpr int TPR = D / 4;          // lanes per row
  constexpr int RPI = 256 / TPR;      // rows per iteration of the workgroup
  const int p = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
  const int len = (a.Z + a.C - 1) / a.C;
  const int r0 = c * len, r1 = min(a.Z, r0 + len);
  const int lane = tid % TPR;
  const float* base = a.V + (long long)p * a.Z * D + 4 * lane;
  double acc = 0.0;
  // U rows per thread in flight; rows past the chunk are read clamped and
  // not counted
  constexpr int U = 8;
  for (int rb = r0 + tid / TPR; rb < r1; rb += RPI * U) {
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = min(rb + u * RPI, r1 - 1);
      v[u] = *(const f32x4*)(base + (long long)r * D);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      double s = (double)v[u].x * v[u].x + (double)v[u].y * v[u].y + (double)v[u].z * v[u].z +
                 (double)v[u].w * v[u].w;
#pragma unroll
      for (int off = TPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
      if (lane == 0 && rb + u * RPI < r1) acc += sqrt(s);
    }
  }
  __shared__ double red[256];
  red[tid] = acc;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) red[tid] += red[tid + off];
    __syncthreads();
  }
  if (tid == 0) a.part[(long long)p * a.C + c] = red[0];
}

__global__ void value_norm_final_kernel(VnormArgs a) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= a.P) return;
  double s = 0.0;
  for (int c = 0; c < a.C; ++c) s += a.part[(long long)p * a.C + c];
  a.out[p] = s / (double)a.Z;
}

}  // namespace

int value_norm_chunks(int P, int Z) {
  // enough workgroups for the part, at most one per 64 rows and 64 per problem
  int c = (1024 + P - 1) / P;
  c = c < 64 ? c : 64;
  const int byrows = (Z + 63) / 64;
  c = c < byrows ? c : byrows;
  return c > 0 ? c : 1;
}

void launch_value_norms(const VnormArgs& a, int d, hipStream_t s) {
  dim3 grid(a.C, a.P);
  if (d == 128) hipLaunchKernelGGL((value_norm_kernel<128>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((value_norm_kernel<64>), grid, dim3(256), 0, s, a);
  hipLaunchKernelGGL(value_norm_final_kernel, dim3((a.P + 255) / 256), dim3(256), 0, s, a);
}

}  // namespace kvs
