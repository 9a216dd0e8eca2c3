// One step of iterative refinement for the ridge value solve, gfx950.
//
// The fp32 solve (Gram accumulated over n queries in fp32, fp32 Cholesky)
// loses accuracy when mu is small against the spread of A^T A: relative
// errors of 1e-4 .. 1e-3 at k ~ 1000 .. 2000 keys.  One correction step
//     r  = A^T (Y - A Vc) - mu Vc          (stored scores, G = 2 (A Vc - Y))
//     Vc += (L L^T)^-1 r                   (the factor already computed)
// converges to the solution of the fp32 weights' normal equations, provided
// r is more accurate than the factor: A^T G is accumulated in fp32 over one
// 64-query tile at a time and in fp64 across tiles and query splits, and r
// is formed in fp64 before it is rounded once.
//
// resid_rhs_kernel: fp64 partials of A^T G, one 64-key tile x all d value
// columns per workgroup, split over queries.
// fwd_subst_kernel: r from the partials, then L Z = r (64-row blocks, top
// down, every block step on MFMA); Z replaces the A^T Y rows of M so that
// the back substitution (accumulating into Vc) completes the correction.
#include "../../include/kvsculpt.h"
#include "kvs_internal.h"

namespace kvs {
namespace {

__device__ __forceinline__ f32x4 mfma_r(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Rpart[c][xoff + key * D + dim] = sum over the queries q of split c of
// A[q][key] G[q][dim], A = exp(St - e).  Keys past k read the last key (their
// rows are ignored by the substitution); queries past the split are zero.
template <int D>
__global__ __launch_bounds__(256) void resid_rhs_kernel(RhsArgs a) {
  const int p = blockIdx.y, kt = blockIdx.x, c = blockIdx.z;
  const ProbInfo pi = a.info[p];
  if (64 * kt >= pi.kpad) return;
  const int n = a.n, npad = (n + 3) & ~3;
  const int nq = ((((n + a.Cr - 1) / a.Cr) + 63) / 64) * 64;
  const int qbeg = c * nq, qend = min(n, qbeg + nq);
  constexpr int DB = D / 16;

  __shared__ float As[64][68];   // [key][query]
  __shared__ float Gt[D][68];    // [dim][query]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, lq = lane & 15;
  const float* St = a.St + pi.soff;
  const float* E = a.e + (size_t)p * n;
  const float* Gq = a.G + (size_t)p * n * D;
  const int krow = 64 * kt;

  double acc64[DB][4];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc64[db][r] = 0.0;

  for (int qt = qbeg; qt < qend; qt += 64) {
    // weights: key i >> 4, queries 4 (i % 16) .. + 3 (one 16-byte load)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = tid + 256 * u;
      const int r = i >> 4, q0 = qt + 4 * (i & 15);
      const f32x4 v = *(const f32x4*)(St + (size_t)min(krow + r, pi.k - 1) * npad + min(q0, npad - 4));
      f32x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = (q0 + j < qend) ? __expf(v[j] - E[min(q0 + j, n - 1)]) : 0.f;
      *(f32x4*)&As[r][4 * (i & 15)] = w;
    }
    // G transposed: dim i % D, queries 4 (i / D) .. + 3 (consecutive lanes,
    // consecutive dims)
#pragma unroll
    for (int u = 0; u < D / 16; ++u) {
      const int i = tid + 256 * u;
      const int dim = i % D, q4 = 4 * (i / D);
      f32x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int q = qt + q4 + j;
        w[j] = q < qend ? Gq[(size_t)q * D + dim] : 0.f;
      }
      *(f32x4*)&Gt[dim][q4] = w;
    }
    __syncthreads();
    f32x4 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int qq = 0; qq < 64; qq += 16) {
      const f32x4 av = *(const f32x4*)&As[16 * wave + lq][qq + 4 * g];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const f32x4 bv = *(const f32x4*)&Gt[16 * db + lq][qq + 4 * g];
        acc[db] = mfma_r(av.x, bv.x, acc[db]);
        acc[db] = mfma_r(av.y, bv.y, acc[db]);
        acc[db] = mfma_r(av.z, bv.z, acc[db]);
        acc[db] = mfma_r(av.w, bv.w, acc[db]);
      }
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc64[db][r] += (double)acc[db][r];
    __syncthreads();
  }

  double* out = a.Rpart + (size_t)c * a.xtot + pi.xoff;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      out[(size_t)(krow + 16 * wave + 4 * g + r) * D + 16 * db + lq] = acc64[db][r];
}

// r = -1/2 sum_c Rpart[c] - mu Vc (rows < k; 0 below), then L Z = r for 16
// value columns per workgroup.  Top down, right-looking:
// Z_i = inv(L_ii) W_i, then W_r -= L_ri Z_i for every r > i.  W is held in
// LDS ([kpad][16]) while it fits, else in the per-slab buffer in X.  The
// contraction index of an MFMA step s in lane group g is 16 g + s, so every
// lane reads 16 consecutive floats of a row of L (four 16-byte loads).
template <int D, bool INLDS>
__global__ __launch_bounds__(256) void fwd_subst_kernel(FsubArgs a) {
  extern __shared__ float dyn[];        // INLDS: W [kpadmax][16], then Xs [64][16]
  const int p = blockIdx.y;
  const ProbInfo pi = a.info[p];
  if (a.info_out[p] != 0) return;       // factorisation failed: Vc is not touched
  const int KT = pi.kpad / 64, ld = pi.kpad, k = pi.k;
  float* __restrict__ Mp = a.M + pi.moff;
  const int dim0 = 16 * blockIdx.x;
  const float* __restrict__ Dinv = a.Dinv + (size_t)pi.xoff / D / 64 * 64 * 64;
  float* W = INLDS ? dyn : a.X + pi.xoff + (size_t)blockIdx.x * pi.kpad * 16;
  float* Xs = INLDS ? dyn + (size_t)a.kpadmax * 16 : dyn;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, lq = lane & 15;

  const double mu = a.mu[p];
  for (int e = tid; e < pi.kpad * 16; e += 256) {
    const int row = e >> 4, c = e & 15;
    float v = 0.f;
    if (row < k) {
      const size_t o = pi.xoff + (size_t)row * D + dim0 + c;
      double s = 0.0;
      for (int cc = 0; cc < a.Cr; ++cc) s += a.Rpart[(size_t)cc * a.xtot + o];
      v = (float)(-0.5 * s - mu * (double)a.Vc[(size_t)(pi.koff + row) * D + dim0 + c]);
    }
    W[e] = v;
  }
  __syncthreads();

  for (int i = 0; i < KT; ++i) {
    // Z_i rows b = 16 wave + 4 g + r: sum_a inv(L_ii)[b][a] W_i[a][c]
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    {
      const float* Di = Dinv + (size_t)i * 64 * 64 + (16 * wave + lq) * 64 + 16 * g;
      f32x4 d4[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) d4[t] = *(const f32x4*)(Di + 4 * t);
#pragma unroll
      for (int s = 0; s < 16; ++s) x = mfma_r(d4[s >> 2][s & 3], W[(64 * i + 16 * g + s) * 16 + lq], x);
#pragma unroll
      for (int r = 0; r < 4; ++r) Xs[(16 * wave + 4 * g + r) * 16 + lq] = x[r];
    }
    __syncthreads();
    // every wave has read W_i: it now holds Z_i
#pragma unroll
    for (int r = 0; r < 4; ++r) W[(64 * i + 16 * wave + 4 * g + r) * 16 + lq] = x[r];
    if (i + 1 < KT) {
      float bz[16];
#pragma unroll
      for (int s = 0; s < 16; ++s) bz[s] = Xs[(16 * g + s) * 16 + lq];
      // W_rb -= L_{rb,i} Z_i; wave w owns the blocks rb = i + 1 + w, + 4, ...
      for (int rb = i + 1 + wave; rb < KT; rb += 4) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float* Lr = Mp + (size_t)(64 * rb + 16 * q + lq) * ld + 64 * i + 16 * g;
          f32x4 l4[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) l4[t] = *(const f32x4*)(Lr + 4 * t);
          f32x4 acc;
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[r] = W[(64 * rb + 16 * q + 4 * g + r) * 16 + lq];
#pragma unroll
          for (int s = 0; s < 16; ++s) acc = mfma_r(-l4[s >> 2][s & 3], bz[s], acc);
#pragma unroll
          for (int r = 0; r < 4; ++r) W[(64 * rb + 16 * q + 4 * g + r) * 16 + lq] = acc[r];
        }
      }
    }
    __syncthreads();
  }

  // Z into the A^T Y rows of M: M[kpad + dim0 + c][row] = Z[row][c]
  for (int e = tid; e < pi.kpad * 16; e += 256) {
    const int c = e / pi.kpad, row = e % pi.kpad;
    Mp[(size_t)(pi.kpad + dim0 + c) * ld + row] = W[row * 16 + c];
  }
}

}  // namespace

int refine_splits(int P, int kpadmax, int n) {
  // about four workgroups per CU over the key tiles, each split at least two
  // query tiles long, at most 16 splits
  const long long tiles = (long long)P * (kpadmax / 64);
  const long long qtiles = (n + 63) / 64;
  long long c = tiles > 0 ? (1024 + tiles - 1) / tiles : 1;
  c = std::min(c, std::max(1LL, qtiles / 2));
  c = std::min(c, 16LL);
  return (int)std::max(1LL, c);
}

void launch_resid_rhs(const RhsArgs& a, int d, hipStream_t s) {
  dim3 grid(a.kpadmax / 64, a.P, a.Cr);
  if (d == 128) hipLaunchKernelGGL((resid_rhs_kernel<128>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((resid_rhs_kernel<64>), grid, dim3(256), 0, s, a);
}

void launch_fwd_subst(const FsubArgs& a, int d, hipStream_t s) {
  dim3 grid(d / 16, a.P);
  const size_t lds = back_subst_lds_bytes(a.kpadmax);
  if (lds <= (size_t)a.lds_max) {
    if (d == 128) hipLaunchKernelGGL((fwd_subst_kernel<128, true>), grid, dim3(256), lds, s, a);
    else hipLaunchKernelGGL((fwd_subst_kernel<64, true>), grid, dim3(256), lds, s, a);
    return;
  }
  const size_t xs = 64 * 16 * sizeof(float);
  if (d == 128) hipLaunchKernelGGL((fwd_subst_kernel<128, false>), grid, dim3(256), xs, s, a);
  else hipLaunchKernelGGL((fwd_subst_kernel<64, false>), grid, dim3(256), xs, s, a);
}

}  // namespace kvs
