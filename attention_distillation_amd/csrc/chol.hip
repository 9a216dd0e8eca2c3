// Batched blocked Cholesky of (A^T A + mu I) carried through the A^T Y rows,
// then the back substitution for Vc, gfx950.
//
// Right-looking, 64-column panels, one launch per panel for every problem of
// the batch (problems whose kpad is exhausted exit at once); see
// chol_step_kernel.  The panel solves of the rows below kpad (the Y^T A rows)
// are the forward substitution L W = A^T Y.
// diag_inv_kernel inverts the 64x64 diagonal blocks of L in parallel, then
// back_subst_kernel solves L^T X = W for 16 value columns per workgroup,
// 64-row blocks from the bottom up, every block step on MFMA.
#include "../../include/kvsculpt.h"
#include "kvs_internal.h"

namespace kvs {

__device__ __forceinline__ f32x4 mfma_c(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float bcast(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ __forceinline__ bool chol_active(const LbState* st, int mask, int p) {
  return !st || ((1 << st[p].status) & mask);
}

// mu_p = ridge_rel * trace / k (trace partials summed in tile order)
__global__ __launch_bounds__(64) void mu_kernel(CholArgs a) {
  const int p = blockIdx.x;
  if (!chol_active(a.st, a.active_mask, p)) return;
  const ProbInfo pi = a.info[p];
  const int KT = pi.kpad / 64;
  const int KTmax = a.kpadmax / 64;
  double s = 0.0;
  for (int i = threadIdx.x; i < KT; i += 64) s += a.trpart[(size_t)p * KTmax + i];
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (threadIdx.x == 0) {
    a.mu[p] = a.ridge_rel * s / (double)pi.k;
    a.info_out[p] = 0;
  }
}

void launch_mu(const CholArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(mu_kernel, dim3(a.P), dim3(64), 0, s, a);
}

// 64x64 tile product C -= A B^T (A = rows rowA.., B = rows rowB.., both taking
// columns col0..col0+63 of M), each wave a 32x32 quarter on 16x16x4 fp32 MFMA.
// Results: acc[ib][jb][r] belongs to row rb + 16 ib + 4 g + r, column
// cb + 16 jb + lq of the tile.
__device__ __forceinline__ void tile_aat(const float* __restrict__ Mp, int ld, int rowA, int rowB, int col0,
                                         f32x4 (&acc)[2][2]) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, lq = lane & 15;
  const int rb = 32 * (wave >> 1), cb = 32 * (wave & 1);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) acc[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    f32x4 av[2], bv[2];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
      av[ib] = *(const f32x4*)(Mp + (size_t)(rowA + rb + 16 * ib + lq) * ld + col0 + 16 * t + 4 * g);
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
      bv[jb] = *(const f32x4*)(Mp + (size_t)(rowB + cb + 16 * jb + lq) * ld + col0 + 16 * t + 4 * g);
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        acc[ib][jb] = mfma_c(av[ib].x, bv[jb].x, acc[ib][jb]);
        acc[ib][jb] = mfma_c(av[ib].y, bv[jb].y, acc[ib][jb]);
        acc[ib][jb] = mfma_c(av[ib].z, bv[jb].z, acc[ib][jb]);
        acc[ib][jb] = mfma_c(av[ib].w, bv[jb].w, acc[ib][jb]);
      }
  }
}

// Tile of M (rows row0.., columns col0..) minus the update of panel j-1
// (when j > 0), into LDS.
__device__ __forceinline__ void tile_updated_to_lds(const float* __restrict__ Mp, int ld, int row0,
                                                    int rowJ, int col0, int j, float (*T)[65]) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, lq = lane & 15;
  const int rb = 32 * (wave >> 1), cb = 32 * (wave & 1);
  f32x4 acc[2][2];
  if (j > 0) {
    tile_aat(Mp, ld, row0, rowJ, 64 * (j - 1), acc);
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) acc[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int ib = 0; ib < 2; ++ib)
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rr = rb + 16 * ib + 4 * g + r, cc = cb + 16 * jb + lq;
        T[rr][cc] = Mp[(size_t)(row0 + rr) * ld + col0 + cc] - acc[ib][jb][r];
      }
}

// One step of the right-looking factorisation, per problem, in one launch:
//  - panel workgroups (blockIdx.x < R): row tile I = j + blockIdx.x of column
//    block j.  Each applies the update of panel j-1 to its tile and to the
//    diagonal block (redundantly; nobody writes the diagonal block of M in
//    this launch), factors the diagonal block in one wave (lane r owns row r,
//    each factored column broadcast through LDS), then solves X L_jj^T = tile (right-looking,
//    independent updates per step).  The factored diagonal block goes to
//    Ldiag; the panel tiles are overwritten in place.
//  - trailing workgroups: the update of panel j-1 for the tiles (I, J) with
//    J >= j+1, which no panel workgroup touches.
template <int D>
__global__ __launch_bounds__(256) void chol_step_kernel(CholArgs a, int j, int Rmax, int nJ) {
  const int p = blockIdx.y;
  if (!chol_active(a.st, a.active_mask, p)) return;
  const ProbInfo pi = a.info[p];
  const int KT = pi.kpad / 64, RT = KT + D / 64;
  if (j >= KT) return;
  const int ld = pi.kpad;
  float* __restrict__ Mp = a.M + pi.moff;
  const int tid = threadIdx.x;
  auto rowof = [&](int I) { return (I < KT) ? 64 * I : pi.kpad + 64 * (I - KT); };

  if ((int)blockIdx.x >= Rmax) {
    // trailing update from panel j-1
    if (j == 0) return;
    const int t = blockIdx.x - Rmax;
    const int I = j + 1 + t / nJ, J = j + 1 + t % nJ;
    if (J >= KT || I >= RT || J > I) return;
    const int wave = tid >> 6, lane = tid & 63, g = lane >> 4, lq = lane & 15;
    const int rb = 32 * (wave >> 1), cb = 32 * (wave & 1);
    f32x4 acc[2][2];
    tile_aat(Mp, ld, rowof(I), 64 * J, 64 * (j - 1), acc);
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float* dst = Mp + (size_t)(rowof(I) + rb + 16 * ib + 4 * g + r) * ld + 64 * J + cb + 16 * jb + lq;
          *dst -= acc[ib][jb][r];
        }
    return;
  }

  const int I = j + blockIdx.x;
  if (I >= RT) return;
  __shared__ float Dl[64][65];
  __shared__ float Tl[64][65];
  __shared__ float Lt[64][68];      // Lt[c][t] = L[t][c]: column c as a contiguous row
  tile_updated_to_lds(Mp, ld, 64 * j, 64 * j, 64 * j, j, Dl);
  if (I != j) tile_updated_to_lds(Mp, ld, rowof(I), 64 * j, 64 * j, j, Tl);
  __syncthreads();
  if (tid >= 64) return;

  // one wave from here on: LDS traffic between lanes is ordered by
  // wavefront-scope release/acquire fences
  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  const int r = tid;
  const float mu = (float)a.mu[p];
  float L[64];
#pragma unroll
  for (int c = 0; c < 64; ++c) L[c] = Dl[r][c];
  const bool real_row = (64 * j + r) < pi.k;
#pragma unroll
  for (int c = 0; c < 64; ++c)
    if (c == r && real_row) L[c] += mu;

  int badcol = -1;
#pragma unroll
  for (int c = 0; c < 64; ++c) {
    Lt[c][r] = L[c];
    wave_sync();
    const float piv = Lt[c][c];
    if (!(piv > 0.f) && badcol < 0) badcol = c;
    const float dgn = sqrtf(piv);
    const float inv = __frcp_rn(dgn);
    L[c] = (r == c) ? dgn : ((r > c) ? L[c] * inv : L[c]);
    Lt[c][r] = L[c];
    wave_sync();
    // rank-1 update of the columns to the right with the broadcast column c
#pragma unroll
    for (int t4 = (c + 1) & ~3; t4 < 64; t4 += 4) {
      const f32x4 lc = *(const f32x4*)&Lt[c][t4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (t4 + e > c) L[t4 + e] = fmaf(-L[c], lc[e], L[t4 + e]);
    }
  }

  if (I == j) {
    float* dst = a.Ldiag + ((size_t)pi.xoff / D + 64 * j + r) * 64;
#pragma unroll
    for (int c = 0; c < 64; c += 4) {
      f32x4 v;
      v.x = (c + 0 <= r) ? L[c + 0] : 0.f;
      v.y = (c + 1 <= r) ? L[c + 1] : 0.f;
      v.z = (c + 2 <= r) ? L[c + 2] : 0.f;
      v.w = (c + 3 <= r) ? L[c + 3] : 0.f;
      *(f32x4*)(dst + c) = v;
    }
    if (r == 0 && badcol >= 0 && a.info_out[p] == 0) a.info_out[p] = 64 * j + badcol + 1;
    return;
  }

  // X L^T = T, right-looking: x_c = t_c / L_cc, then t_t -= x_c L_tc (t > c);
  // Lt holds the factored columns
  float x[64];
#pragma unroll
  for (int c = 0; c < 64; ++c) x[c] = Tl[r][c];
#pragma unroll
  for (int c = 0; c < 64; ++c) {
    x[c] = x[c] * __frcp_rn(Lt[c][c]);
#pragma unroll
    for (int t4 = (c + 1) & ~3; t4 < 64; t4 += 4) {
      const f32x4 lc = *(const f32x4*)&Lt[c][t4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (t4 + e > c) x[t4 + e] = fmaf(-x[c], lc[e], x[t4 + e]);
    }
  }
  float* xr = Mp + (size_t)(rowof(I) + r) * ld + 64 * j;
#pragma unroll
  for (int c = 0; c < 64; c += 4) *(f32x4*)(xr + c) = f32x4{x[c], x[c + 1], x[c + 2], x[c + 3]};
}

void launch_chol_step(const CholArgs& a, int d, int j, hipStream_t s) {
  const int KT = a.kpadmax / 64;
  const int Rmax = KT + d / 64 - j;
  const int nI = KT + d / 64 - j - 1, nJ = KT - j - 1;
  const int ntrail = (j > 0 && nI > 0 && nJ > 0) ? nI * nJ : 0;
  dim3 grid(Rmax + ntrail, a.P);
  if (d == 128) hipLaunchKernelGGL((chol_step_kernel<128>), grid, dim3(256), 0, s, a, j, Rmax, nJ > 0 ? nJ : 1);
  else hipLaunchKernelGGL((chol_step_kernel<64>), grid, dim3(256), 0, s, a, j, Rmax, nJ > 0 ? nJ : 1);
}

// Inverse of every 64x64 diagonal block of L (one wave per block, lane c
// computes column c by forward substitution; the block is broadcast from
// LDS).  Padding blocks are the identity.  Dinv is [sum KT][64][64].
__global__ __launch_bounds__(64) void diag_inv_kernel(BackArgs a) {
  const int p = blockIdx.y;
  if (a.st && !((1 << a.st[p].status) & a.active_mask)) return;
  const ProbInfo pi = a.info[p];
  const int KT = pi.kpad / 64;
  const int blk = blockIdx.x;
  if (blk >= KT) return;
  __shared__ float Ls[64][65];
  const int c = threadIdx.x;
  const float* Lb = a.Ldiag + ((size_t)pi.xoff / a.d + 64 * blk) * 64;
  for (int e = c; e < 64 * 64; e += 64) Ls[e >> 6][e & 63] = Lb[e];
  __syncthreads();
  // column c of inv(L): forward substitution L x = e_c; each row's sum is
  // split over four independent accumulators to shorten the dependency chain
  float x[64];
#pragma unroll
  for (int r = 0; r < 64; ++r) {
    float s0 = (r == c) ? 1.f : 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
    for (int t = 0; t + 3 < r; t += 4) {
      s0 = fmaf(-Ls[r][t], x[t], s0);
      s1 = fmaf(-Ls[r][t + 1], x[t + 1], s1);
      s2 = fmaf(-Ls[r][t + 2], x[t + 2], s2);
      s3 = fmaf(-Ls[r][t + 3], x[t + 3], s3);
    }
#pragma unroll
    for (int t = r & ~3; t < r; ++t) s0 = fmaf(-Ls[r][t], x[t], s0);
    x[r] = ((s0 + s1) + (s2 + s3)) / Ls[r][r];
    __asm__ __volatile__("" ::: "memory");   // keep each row's LDS reads in its own step
  }
  // one wave: every lane has finished reading Ls, so it can hold the result
#pragma unroll
  for (int r = 0; r < 64; ++r) Ls[r][c] = x[r];
  __syncthreads();
  float* dst = a.Dinv + ((size_t)pi.xoff / a.d / 64 + blk) * 64 * 64;
  for (int e = c; e < 64 * 64; e += 64) dst[e] = Ls[e >> 6][e & 63];
}

// Solve L^T X = W for 16 value columns per workgroup, 64-row blocks from the
// bottom up, right-looking: X_i = inv(L_ii)^T W_i, then W_r -= L_ir^T X_i for
// every r < i.  W starts as the A^T Y rows left in M by the factorisation
// (forward substitution) and is updated in place in the per-slab solve
// buffer [d/16][kpad][16]; Vc rows < k are written at the end.
template <int D>
__global__ __launch_bounds__(256) void back_subst_kernel(BackArgs a) {
  const int p = blockIdx.y;
  if (a.st && !((1 << a.st[p].status) & a.active_mask)) return;
  const ProbInfo pi = a.info[p];
  const int KT = pi.kpad / 64, ld = pi.kpad;
  const float* __restrict__ Mp = a.M + pi.moff;
  const int dim0 = 16 * blockIdx.x;
  float* __restrict__ W = a.X + pi.xoff + (size_t)blockIdx.x * pi.kpad * 16;
  const float* __restrict__ Dinv = a.Dinv + (size_t)pi.xoff / D / 64 * 64 * 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, lq = lane & 15;
  __shared__ float Xs[64][17];

  // W[row][c] = M[kpad + dim0 + c][row]
  for (int e = tid; e < pi.kpad * 16; e += 256) {
    const int row = e >> 4, c = e & 15;
    W[e] = Mp[(size_t)(pi.kpad + dim0 + c) * ld + row];
  }
  __syncthreads();

  for (int i = KT - 1; i >= 0; --i) {
    // X_i rows b = 16 wave + (4g + r): sum_a inv(L_ii)[a][b] W_i[a][c]
    {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const float* Di = Dinv + (size_t)i * 64 * 64;
      float av[16], bv[16];
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const int arow = 4 * s + g;
        av[s] = Di[arow * 64 + 16 * wave + lq];
        bv[s] = W[(size_t)(64 * i + arow) * 16 + lq];
      }
#pragma unroll
      for (int s = 0; s < 16; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s], bv[s], acc, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) Xs[16 * wave + 4 * g + r][lq] = acc[r];
    }
    __syncthreads();
    // store X_i and update W_r (r < i): block (r, wave) rows 64r + 16 wave + ..
#pragma unroll
    for (int r = 0; r < 4; ++r) W[(size_t)(64 * i + 16 * wave + 4 * g + r) * 16 + lq] = Xs[16 * wave + 4 * g + r][lq];
    if (i > 0) {
      // W_rb -= L_{i,rb}^T X_i for rb < i; wave w owns the blocks rb = w, w+4, ...
      float bv[16];
#pragma unroll
      for (int s = 0; s < 16; ++s) bv[s] = Xs[4 * s + g][lq];
      for (int rb = wave; rb < i; rb += 4) {
        float av[4][16], wv[4][4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
          for (int s = 0; s < 16; ++s)
            av[q][s] = Mp[(size_t)(64 * i + 4 * s + g) * ld + 64 * rb + 16 * q + lq];
#pragma unroll
          for (int r = 0; r < 4; ++r) wv[q][r] = W[(size_t)(64 * rb + 16 * q + 4 * g + r) * 16 + lq];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 16; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[q][s], bv[s], acc, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) W[(size_t)(64 * rb + 16 * q + 4 * g + r) * 16 + lq] = wv[q][r] - acc[r];
        }
      }
    }
    __syncthreads();
  }

  const bool ok = a.info_out[p] == 0;
  if (ok) {
    for (int e = tid; e < pi.k * 16; e += 256) {
      const int row = e >> 4, c = e & 15;
      a.Vc[(size_t)(pi.koff + row) * D + dim0 + c] = W[(size_t)row * 16 + c];
    }
  }
  if (blockIdx.x == 0 && tid == 0 && !ok) {
    if (a.flags) a.flags[p] |= KVS_FLAG_CHOLESKY;
    if (a.st) a.st[p].flags |= KVS_FLAG_CHOLESKY;
  }
}

void launch_back_subst(const BackArgs& a, int d, hipStream_t s) {
  hipLaunchKernelGGL(diag_inv_kernel, dim3(a.kpadmax / 64, a.P), dim3(64), 0, s, a);
  dim3 grid(d / 16, a.P);
  if (d == 128) hipLaunchKernelGGL((back_subst_kernel<128>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((back_subst_kernel<64>), grid, dim3(256), 0, s, a);
}

}  // namespace kvs
