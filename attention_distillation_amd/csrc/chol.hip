// Batched blocked Cholesky of (A^T A + mu I) carried through the A^T Y rows,
// then the back substitution for Vc, gfx950.
//
// Right-looking, 64-column panels, one launch per panel for every problem of
// the batch (problems whose kpad is exhausted exit at once); see
// chol_step_kernel.  The panel solves of the rows below kpad (the Y^T A rows)
// are the forward substitution L W = A^T Y.
// The workgroup that factors a diagonal block also inverts it (for the back
// substitution); back_subst_kernel solves L^T X = W for 16 value columns per workgroup,
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
//    each column broadcast through LDS), then solves X L_jj^T = tile (right-looking,
//    independent updates per step).  The panel tiles are overwritten in
//    place; the diagonal workgroup solves against the identity instead and
//    writes inv(L_jj) to Dinv.
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
  __shared__ float Rd[64];          // 1 / L[c][c]
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

  // Right-looking factorisation with one LDS round trip per column: every
  // lane publishes its entry of the unscaled column c, reads the whole column
  // back (pivot included), and applies a_rt -= a_rc a_tc / a_cc.
  int badcol = -1;
#pragma unroll
  for (int c = 0; c < 64; ++c) {
    Lt[c][r] = L[c];
    wave_sync();
    const int c4 = c & ~3;
    f32x4 col[16];
#pragma unroll
    for (int t4 = c4; t4 < 64; t4 += 4) col[t4 / 4] = *(const f32x4*)&Lt[c][t4];
    const float piv = col[c / 4][c % 4];
    if (!(piv > 0.f) && badcol < 0) badcol = c;
    const float dgn = sqrtf(piv);
    const float inv = __frcp_rn(dgn);
    const float f = L[c] * (inv * inv);
#pragma unroll
    for (int t = c + 1; t < 64; ++t) L[t] = fmaf(-f, col[t / 4][t % 4], L[t]);
    L[c] = (r == c) ? dgn : L[c] * inv;
    __builtin_amdgcn_sched_barrier(0);
  }
  // the factor (zero above the diagonal), column c as row c of Lt
#pragma unroll
  for (int c = 0; c < 64; ++c) Lt[c][r] = (c <= r) ? L[c] : 0.f;
  wave_sync();
  Rd[r] = __frcp_rn(Lt[r][r]);
  wave_sync();

  // X L^T = T, right-looking: x_c = t_c / L_cc, then t_t -= x_c L_tc (t > c).
  // Software-pipelined by hand: the reads of column c+1 are issued at the
  // start of step c (nothing in the loop writes LDS).
  float x[64];
  if (I == j) {
    // diagonal workgroup: T = identity, so lane r ends with row r of
    // inv(L)^T, i.e. column r of inv(L)
#pragma unroll
    for (int c = 0; c < 64; ++c) x[c] = (c == r) ? 1.f : 0.f;
  } else {
#pragma unroll
    for (int c = 0; c < 64; ++c) x[c] = Tl[r][c];
  }
  f32x4 cur[16];
  float rcur = Rd[0];
#pragma unroll
  for (int t4 = 0; t4 < 64; t4 += 4) cur[t4 / 4] = *(const f32x4*)&Lt[0][t4];
#pragma unroll
  for (int c = 0; c < 64; ++c) {
    f32x4 nxt[16];
    float rnxt = 0.f;
    if (c + 1 < 64) {
      rnxt = Rd[c + 1];
#pragma unroll
      for (int t4 = (c + 2) & ~3; t4 < 64; t4 += 4) nxt[t4 / 4] = *(const f32x4*)&Lt[c + 1][t4];
    }
    x[c] = x[c] * rcur;
#pragma unroll
    for (int t = c + 1; t < 64; ++t) x[t] = fmaf(-x[c], cur[t / 4][t % 4], x[t]);
#pragma unroll
    for (int t4 = (c + 2) & ~3; t4 < 64; t4 += 4) cur[t4 / 4] = nxt[t4 / 4];
    rcur = rnxt;
    __builtin_amdgcn_sched_barrier(0);
  }
  if (I == j) {
    // Dinv block j, row-major: Dinv[c][r] = inv(L)[c][r] = x[c] of lane r
    float* dst = a.Dinv + ((size_t)pi.xoff / D + 64 * j) * 64;
#pragma unroll
    for (int c = 0; c < 64; ++c) dst[c * 64 + r] = x[c];
    if (r == 0 && badcol >= 0 && a.info_out[p] == 0) a.info_out[p] = 64 * j + badcol + 1;
    return;
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

// Same solve with the right-hand side W held in LDS ([kpad][16] floats,
// dynamic shared memory) for the whole back substitution: only the L blocks
// and inv(L_ii) come from global memory, and the L-block loads of a step are
// issued before its diagonal solve so their latency overlaps it.
template <int D>
__global__ __launch_bounds__(256) void back_subst_lds_kernel(BackArgs a) {
  extern __shared__ float Wl[];          // [kpadmax][16], then Xs [64][16]
  const int p = blockIdx.y;
  if (a.st && !((1 << a.st[p].status) & a.active_mask)) return;
  const ProbInfo pi = a.info[p];
  const int KT = pi.kpad / 64, ld = pi.kpad;
  const float* __restrict__ Mp = a.M + pi.moff;
  const int dim0 = 16 * blockIdx.x;
  const float* __restrict__ Dinv = a.Dinv + (size_t)pi.xoff / D / 64 * 64 * 64;
  float* Xs = Wl + (size_t)a.kpadmax * 16;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, lq = lane & 15;

  // W[row][c] = M[kpad + dim0 + c][row]: coalesced float4 reads along the row
  for (int e = tid; e < pi.kpad * 4; e += 256) {
    const int c = e / (pi.kpad / 4), r4 = e % (pi.kpad / 4);
    const f32x4 v = *(const f32x4*)(Mp + (size_t)(pi.kpad + dim0 + c) * ld + 4 * r4);
#pragma unroll
    for (int u = 0; u < 4; ++u) Wl[(4 * r4 + u) * 16 + c] = v[u];
  }
  __syncthreads();

  auto load_block = [&](float (&av)[4][16], int i, int rb) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int s2 = 0; s2 < 16; ++s2)
        av[q][s2] = -Mp[(size_t)(64 * i + 4 * s2 + g) * ld + 64 * rb + 16 * q + lq];
  };
  // W_rb += (-L_{i,rb})^T X_i, accumulator seeded with W_rb
  auto update_block = [&](const float (&av)[4][16], const float (&bx)[16], int rb) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x4 acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = Wl[(64 * rb + 16 * q + 4 * g + r) * 16 + lq];
#pragma unroll
      for (int s2 = 0; s2 < 16; ++s2) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[q][s2], bx[s2], acc, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) Wl[(64 * rb + 16 * q + 4 * g + r) * 16 + lq] = acc[r];
    }
  };

  for (int i = KT - 1; i >= 0; --i) {
    float av0[4][16], av1[4][16];
    const int rb0 = wave, rb1 = wave + 4;
    if (rb0 < i) load_block(av0, i, rb0);
    if (rb1 < i) load_block(av1, i, rb1);
    // X_i rows b = 16 wave + (4g + r): sum_a inv(L_ii)[a][b] W_i[a][c]
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    {
      const float* Di = Dinv + (size_t)i * 64 * 64;
      float dv[16], wv[16];
#pragma unroll
      for (int s2 = 0; s2 < 16; ++s2) {
        dv[s2] = Di[(4 * s2 + g) * 64 + 16 * wave + lq];
        wv[s2] = Wl[(64 * i + 4 * s2 + g) * 16 + lq];
      }
#pragma unroll
      for (int s2 = 0; s2 < 16; ++s2) x = __builtin_amdgcn_mfma_f32_16x16x4f32(dv[s2], wv[s2], x, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) Xs[(16 * wave + 4 * g + r) * 16 + lq] = x[r];
    }
    __syncthreads();
    // every wave has read W_i: it now holds X_i
#pragma unroll
    for (int r = 0; r < 4; ++r) Wl[(64 * i + 16 * wave + 4 * g + r) * 16 + lq] = x[r];
    if (i > 0) {
      float bx[16];
#pragma unroll
      for (int s2 = 0; s2 < 16; ++s2) bx[s2] = Xs[(4 * s2 + g) * 16 + lq];
      if (rb0 < i) update_block(av0, bx, rb0);
      if (rb1 < i) update_block(av1, bx, rb1);
      for (int rb = wave + 8; rb < i; rb += 8) {
        load_block(av0, i, rb);
        if (rb + 4 < i) load_block(av1, i, rb + 4);
        update_block(av0, bx, rb);
        if (rb + 4 < i) update_block(av1, bx, rb + 4);
      }
    }
    __syncthreads();
  }

  const bool ok = a.info_out[p] == 0;
  if (ok) {
    for (int e = tid; e < pi.k * 16; e += 256) {
      const int row = e >> 4, c = e & 15;
      a.Vc[(size_t)(pi.koff + row) * D + dim0 + c] = Wl[row * 16 + c];
    }
  }
  if (blockIdx.x == 0 && tid == 0 && !ok) {
    if (a.flags) a.flags[p] |= KVS_FLAG_CHOLESKY;
    if (a.st) a.st[p].flags |= KVS_FLAG_CHOLESKY;
  }
}

size_t back_subst_lds_bytes(int kpadmax) { return ((size_t)kpadmax * 16 + 64 * 16) * sizeof(float); }

void launch_back_subst(const BackArgs& a, int d, hipStream_t s) {
  dim3 grid(d / 16, a.P);
  const size_t lds = back_subst_lds_bytes(a.kpadmax);
  if (lds <= (size_t)a.lds_max) {
    if (d == 128) hipLaunchKernelGGL((back_subst_lds_kernel<128>), grid, dim3(256), lds, s, a);
    else hipLaunchKernelGGL((back_subst_lds_kernel<64>), grid, dim3(256), lds, s, a);
    return;
  }
  if (d == 128) hipLaunchKernelGGL((back_subst_kernel<128>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((back_subst_kernel<64>), grid, dim3(256), 0, s, a);
}

}  // namespace kvs
