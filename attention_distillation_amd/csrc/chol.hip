// Batched blocked Cholesky of (A^T A + mu I) carried through the A^T Y rows,
// then the back substitution for Vc, gfx950.
//
// Right-looking, 64-column panels with a one-block look-ahead, one launch per
// panel for every problem of the batch (problems whose kpad is exhausted exit
// at once); see chol_step_kernel.  The panel solves of the rows below kpad
// (the Y^T A rows) are the forward substitution L W = A^T Y.  The inverted
// diagonal blocks serve the panel solves and the back substitution;
// back_subst_lds_kernel solves L^T X = W for 16 value columns per workgroup,
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

// value of lane T of this lane's 16-lane row (DPP row_newbcast)
template <int T>
__device__ __forceinline__ float row_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + T, 0xF, 0xF, true));
}
// f(integral_constant<int, I>) for I = 0 .. N-1, unrolled at compile time
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
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

// acc += A B^T for 64x64 tiles held in LDS ([64][68], row-major): each wave
// a 32x32 quarter, acc[ib][jb][r] at row rb + 16 ib + 4 g + r, column
// cb + 16 jb + lq of the tile.  Operands are read four k at a time: step t
// takes k = 16 (t / 4) + 4 g + t % 4 on both sides.
__device__ __forceinline__ void tile_abt_acc(const float (*A)[68], const float (*B)[68], f32x4 (&acc)[2][2]) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, lq = lane & 15;
  const int rb = 32 * (wave >> 1), cb = 32 * (wave & 1);
#pragma unroll
  for (int t4 = 0; t4 < 4; ++t4) {
    f32x4 av[2], bv[2];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) av[ib] = *(const f32x4*)&A[rb + 16 * ib + lq][16 * t4 + 4 * g];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) bv[jb] = *(const f32x4*)&B[cb + 16 * jb + lq][16 * t4 + 4 * g];
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) acc[ib][jb] = mfma_c(av[ib][e], bv[jb][e], acc[ib][jb]);
  }
}

// Launch j of the right-looking factorisation with look-ahead (j = -1 .. KT-1),
// all problems of the batch at once.  The trailing matrix takes the panels'
// updates S at a time (S = 1, 2 or 4 by batch size): launches j = S, 2S, ..
// apply panels j-S .. j-1 in one read-modify-write of every trailing tile.
//  - panel workgroups: row tile I = j+1+w of column block j (w: the
//    workgroup's index within its problem's range of the grid).  Each
//    applies to its tile the panels the trailing passes have not
//    (chol_pending), solves it against L_jj by
//    one MFMA product with inv(L_jj) (computed one launch earlier), stores
//    L_Ij in place and subtracts L_Ij L_Ij^T from its row's diagonal tile
//    (I, I).  Rows below kpad are the A^T Y rows: their panel solves are the
//    forward substitution L W = A^T Y.
//  - the workgroup of I = j+1 keeps that diagonal tile in LDS instead (all
//    earlier panels are already applied), factors it and writes
//    inv(L_{j+1,j+1}) for the next launch and the back substitution.  Launch
//    -1 does only this for block 0.
//  - trailing workgroups: the update of the pending panels for the tiles
//    (I, J) with I > J >= j+1 (diagonal tiles are left to the panel
//    workgroups).
// The grid of launch j lists only the workgroups that have work: problem p
// owns [coff[j+1][p], coff[j+1][p+1]), its panel rows first, then its
// trailing tiles (a ragged batch would otherwise launch the largest
// problem's square of tiles for every problem).
template <int D>
__global__ __launch_bounds__(256) void chol_step_kernel(CholArgs a, int j) {
  const int* __restrict__ off = a.coff + (size_t)(j + 1) * (a.P + 1);
  const int x = blockIdx.x;
  int lo = 0, hi = a.P;           // largest lo with off[lo] <= x (off[P] > x)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= x) lo = mid;
    else hi = mid;
  }
  const int p = lo;
  if (!chol_active(a.st, a.active_mask, p)) return;
  const ProbInfo pi = a.info[p];
  const int KT = pi.kpad / 64, RT = KT + D / 64;
  if (j >= KT) return;
  const int wid = x - off[p];                      // workgroup within the problem
  const int npanel = chol_panel_wgs(KT, D / 64, j);
  const int ld = pi.kpad;
  float* __restrict__ Mp = a.M + pi.moff;
  float* __restrict__ Dinv = a.Dinv + (size_t)pi.xoff / D * 64;   // [KT][64][64]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, lq = lane & 15;
  const int rb = 32 * (wave >> 1), cb = 32 * (wave & 1);
  auto rowof = [&](int I) { return (I < KT) ? 64 * I : pi.kpad + 64 * (I - KT); };
  __shared__ float Tl[64][68];      // panel tile, then L_Ij (trailing: a panel block of row I)
  __shared__ float Dl[64][68];      // diagonal tile of the look-ahead, then its factor (trailing: of row J)

  if (wid >= npanel) {
    // trailing update from the pending panels: strictly lower tiles among the
    // columns j+1 .. KT-1 row by row, then the value rows (diagonal tiles
    // are left to the panel workgroups)
    const int nj = KT - j - 1;
    const int u = wid - npanel;
    const int ntri = nj * (nj - 1) / 2;
    int I, J;
    if (u < ntri) {
      int i = (int)((sqrt(8.0 * (double)u + 1.0) + 1.0) * 0.5);   // i (i - 1) / 2 <= u < i (i + 1) / 2
      while (i * (i - 1) / 2 > u) --i;
      while (i * (i + 1) / 2 <= u) ++i;
      I = j + 1 + i;
      J = j + 1 + (u - i * (i - 1) / 2);
    } else {
      const int v = u - ntri;
      I = KT + v / nj;
      J = j + 1 + v % nj;
    }
    if (J >= KT || I >= RT || J >= I) return;   // not reached: the count lists only these
    // the tile itself is loaded first so its latency overlaps the operands'
    float cv[2][2][4];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          cv[ib][jb][r] = Mp[(size_t)(rowof(I) + rb + 16 * ib + 4 * g + r) * ld + 64 * J + cb + 16 * jb + lq];
    // T -= sum over the pending panels of L_{I,p} L_{J,p}^T: each panel's two
    // 64x64 blocks are staged in LDS once for the four waves (each wave would
    // otherwise read its own 32 rows of both from L2), the next panel's
    // blocks loaded during the current panel's products
    f32x4 acc[2][2];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) acc[ib][jb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int rA = rowof(I), rB = 64 * J, c00 = 64 * (j - a.S);
    f32x4 pa[4], pb[4];
    auto load_blocks = [&](int c0) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = tid + 256 * u, r = i >> 4, c4 = 4 * (i & 15);
        pa[u] = *(const f32x4*)(Mp + (size_t)(rA + r) * ld + c0 + c4);
        pb[u] = *(const f32x4*)(Mp + (size_t)(rB + r) * ld + c0 + c4);
      }
    };
    load_blocks(c00);
    for (int pn = 0; pn < a.S; ++pn) {
      __syncthreads();   // the previous panel's blocks are read
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = tid + 256 * u, r = i >> 4, c4 = 4 * (i & 15);
        *(f32x4*)&Tl[r][c4] = pa[u];
        *(f32x4*)&Dl[r][c4] = pb[u];
      }
      __syncthreads();
      if (pn + 1 < a.S) load_blocks(c00 + 64 * (pn + 1));
      tile_abt_acc(Tl, Dl, acc);
    }
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          Mp[(size_t)(rowof(I) + rb + 16 * ib + 4 * g + r) * ld + 64 * J + cb + 16 * jb + lq] =
              cv[ib][jb][r] - acc[ib][jb][r];
    return;
  }

  const int I = j + 1 + wid;
  if (I >= RT) return;
  const bool look = (I == j + 1) && (I < KT);
  __shared__ float Xr[4][16][20];   // inverses of the factor's 16x16 diagonal blocks

  const int rowI = rowof(I);
  // The diagonal tile (I, I) receives the update of panel j from the panel
  // workgroup of row I in launch j (it holds the fresh L_Ij); trailing
  // workgroups never touch diagonal tiles.  So the look-ahead workgroup finds
  // panels 0..j-1 already applied and subtracts only panel j.
  const bool diag = (I < KT) && j >= 0;      // row I has a diagonal tile to update
  float dv[2][2][4];
  if (j >= 0) {
    // every global load of the workgroup is issued here, before any use:
    // the panel tile (I, j), the diagonal tile (I, I), the operands of the
    // panel tile's update by its np pending panels, and inv(L_jj) as MFMA B
    // operand
    const int np = chol_pending(j, a.S);
    const int np0 = np < 2 ? np : 2;   // the newest two: loaded with the tiles
    const bool upd = np > 0;
    float tv[2][2][4], dj[16][2];
    f32x4 av[8][2], bt[8][2];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rr = rb + 16 * ib + 4 * g + r, cc = cb + 16 * jb + lq;
          tv[ib][jb][r] = Mp[(size_t)(rowI + rr) * ld + 64 * j + cc];
          dv[ib][jb][r] = diag ? Mp[(size_t)(rowI + rr) * ld + 64 * I + cc] : 0.f;
        }
    if (upd) {
      const int c0 = 64 * (j - np0);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if (t >= 4 * np0) break;
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
          av[t][ib] = *(const f32x4*)(Mp + (size_t)(rowI + rb + 16 * ib + lq) * ld + c0 + 16 * t + 4 * g);
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
          bt[t][jb] = *(const f32x4*)(Mp + (size_t)(64 * j + cb + 16 * jb + lq) * ld + c0 + 16 * t + 4 * g);
      }
    }
    // inv(L_jj) as B operand, four k per load: step t takes
    // k = 16 (t / 4) + 4 g + t % 4 (the A operand below uses the same order)
    const float* Dj = Dinv + (size_t)j * 64 * 64;
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        const f32x4 v = *(const f32x4*)&Dj[(cb + 16 * jb + lq) * 64 + 16 * t4 + 4 * g];
#pragma unroll
        for (int e = 0; e < 4; ++e) dj[4 * t4 + e][jb] = v[e];
      }

    // update by the pending panels: T -= sum_p L_{I,p} L_{j,p}^T
    f32x4 accT[2][2];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) accT[ib][jb] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (upd) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if (t >= 4 * np0) break;
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
          for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int e = 0; e < 4; ++e) accT[ib][jb] = mfma_c(av[t][ib][e], bt[t][jb][e], accT[ib][jb]);
      }
    }
    // older pending panels (S = 4), two at a time
    for (int e2 = np0; e2 < np; e2 += 2) {
      const int nq = np - e2 < 2 ? np - e2 : 2;
      const int c1 = 64 * (j - np + e2 - np0);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if (t >= 4 * nq) break;
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
          av[t][ib] = *(const f32x4*)(Mp + (size_t)(rowI + rb + 16 * ib + lq) * ld + c1 + 16 * t + 4 * g);
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
          bt[t][jb] = *(const f32x4*)(Mp + (size_t)(64 * j + cb + 16 * jb + lq) * ld + c1 + 16 * t + 4 * g);
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if (t >= 4 * nq) break;
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
          for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int e = 0; e < 4; ++e) accT[ib][jb] = mfma_c(av[t][ib][e], bt[t][jb][e], accT[ib][jb]);
      }
    }
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rr = rb + 16 * ib + 4 * g + r, cc = cb + 16 * jb + lq;
          Tl[rr][cc] = tv[ib][jb][r] - accT[ib][jb][r];
        }
    __syncthreads();

    // L_Ij = T inv(L_jj)^T
    f32x4 acc[2][2];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) acc[ib][jb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      f32x4 a4[2];
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) a4[ib] = *(const f32x4*)&Tl[rb + 16 * ib + lq][16 * t4 + 4 * g];
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
          for (int jb = 0; jb < 2; ++jb) acc[ib][jb] = mfma_c(a4[ib][e], dj[4 * t4 + e][jb], acc[ib][jb]);
    }
    __syncthreads();
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rr = rb + 16 * ib + 4 * g + r, cc = cb + 16 * jb + lq;
          Tl[rr][cc] = acc[ib][jb][r];
          Mp[(size_t)(rowI + rr) * ld + 64 * j + cc] = acc[ib][jb][r];
        }
    if (diag) {
      // D_II -= L_Ij L_Ij^T: into LDS for the look-ahead factor, else back to M
      __syncthreads();
      f32x4 acc2[2][2];
#pragma unroll
      for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) acc2[ib][jb] = f32x4{0.f, 0.f, 0.f, 0.f};
      tile_abt_acc(Tl, Tl, acc2);
#pragma unroll
      for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int rr = rb + 16 * ib + 4 * g + r, cc = cb + 16 * jb + lq;
            const float v = dv[ib][jb][r] - acc2[ib][jb][r];
            if (look) Dl[rr][cc] = v;
            else Mp[(size_t)(rowI + rr) * ld + 64 * I + cc] = v;
          }
    }
  }
  if (!look) return;

  if (j < 0) {
    // block 0: nothing to update
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rr = rb + 16 * ib + 4 * g + r, cc = cb + 16 * jb + lq;
          Dl[rr][cc] = Mp[(size_t)rr * ld + cc];
        }
  }
  __syncthreads();

  // Factor the diagonal tile and invert the factor, in 16-column panels.
  //  - wave 0 factors panel b (rows 16b..63, columns 16b..16b+15) in
  //    registers, one row per lane: the pivot column is broadcast by readlane
  //    (by symmetry, entry c of the rows below the pivot), and the 16x16
  //    diagonal block is inverted in the same sweep (X L_bb^T = I, lane r
  //    keeping column r of inv(L_bb)).  It then applies panel b to the tiles
  //    of panel b+1 on MFMA and goes on with that panel.
  //  - waves 1..3 meanwhile apply panel b to the rest of the trailing tiles
  //    and carry block column q = wave-1 of X = inv(L) by blocked forward
  //    substitution: X_bq = inv(L_bb) B_bq, then B_iq -= L_ib X_bq for i > b,
  //    with B starting as the identity.  Block column 3 is inv(L_33) itself.
  // One barrier per panel; every tile is 16x16 and MFMA operands are read
  // four k at a time (k = 4 g + s in step s), results of one product feeding
  // the next as its B operand in the same k order.
  const float mu = (float)a.mu[p];
  if (tid < 64 && 64 * I + tid < pi.k) Dl[tid][tid] += mu;
  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  // Dl tile (ti, tj) -= L_{ti,b} L_{tj,b}^T
  auto tile_update = [&](int ti, int tj, int b) {
    const f32x4 av = *(const f32x4*)&Dl[16 * ti + lq][16 * b + 4 * g];
    const f32x4 bv = *(const f32x4*)&Dl[16 * tj + lq][16 * b + 4 * g];
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma_c(av[s], bv[s], acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) Dl[16 * ti + 4 * g + r][16 * tj + lq] -= acc[r];
  };
  float* dst = Dinv + (size_t)I * 64 * 64;   // inv(L_II), row-major
  const int q = wave - 1;                    // block column carried by waves 1..3
  f32x4 Bq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) Bq[i][r] = (i == q && 4 * g + r == lq) ? 1.f : 0.f;
  // X_bq from B_bq, then B_iq -= L_ib X_bq (i > b)
  auto column_step = [&](auto bc) {
    constexpr int b = decltype(bc)::value;
    const f32x4 xa = *(const f32x4*)&Xr[b][lq][4 * g];
    f32x4 X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) X = mfma_c(xa[s], Bq[b][s], X);
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[(16 * b + 4 * g + r) * 64 + 16 * q + lq] = X[r];
#pragma unroll
    for (int i = b + 1; i < 4; ++i) {
      const f32x4 la = *(const f32x4*)&Dl[16 * i + lq][16 * b + 4 * g];
#pragma unroll
      for (int s = 0; s < 4; ++s) Bq[i] = mfma_c(-la[s], X[s], Bq[i]);
    }
  };
  int badcol = -1;
  auto panel_step = [&](auto bc) {
    constexpr int b = decltype(bc)::value;
    if (wave == 0) {
      if constexpr (b > 0) {
        // panel b-1 applied to the tiles of panel b
#pragma unroll
        for (int ti = b; ti < 4; ++ti) tile_update(ti, b, b - 1);
      }
      wave_sync();
      // Lane layout: li = lane % 16 names a row of the 16x16 diagonal block,
      // held by every 16-lane row of the wave (Db) so that entry t of any
      // column is one row broadcast away.  Each lane also carries one row
      // of the augmented panel (P): a row below the block (lane < nb) or
      // row li of the identity (nb <= lane < nb + 16).  The sweep turns the
      // rows below into L_ib and the identity rows into inv(L_bb)^T.
      constexpr int nb = 48 - 16 * b;
      float Db[16], P[16], iv[16];
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const f32x4 v = *(const f32x4*)&Dl[16 * b + lq][16 * b + 4 * c4];
        const f32x4 w = *(const f32x4*)&Dl[min(16 * (b + 1) + lane, 63)][16 * b + 4 * c4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          Db[4 * c4 + e] = v[e];
          P[4 * c4 + e] = (lane < nb) ? w[e] : ((lane < nb + 16 && 4 * c4 + e == lq) ? 1.f : 0.f);
        }
      }
      // right-looking sweep: with col the pivot column (unscaled) and
      // inv = 1/sqrt(pivot), a_t -= a_c col_t / pivot (t > c) for every row;
      // row r of the result is P_c inv_c
      // Column c+1 is updated first and its pivot's 1/sqrt started before
      // the rest of step c, so that latency hides behind step c's updates.
      float piv = row_bcast<0>(Db[0]);
      float inv = __builtin_amdgcn_rsqf(piv);   // hardware 1/sqrt (about 1 ulp)
      static_for<16>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        if (!(piv > 0.f) && badcol < 0) badcol = 16 * b + c;
        iv[c] = inv;
        const float i2 = inv * inv;
        const float fD = Db[c] * i2, fP = P[c] * i2;
        if constexpr (c + 1 < 16) {
          const float col = row_bcast<c + 1>(Db[c]);
          Db[c + 1] = fmaf(-fD, col, Db[c + 1]);
          P[c + 1] = fmaf(-fP, col, P[c + 1]);
          piv = row_bcast<c + 1>(Db[c + 1]);
          inv = __builtin_amdgcn_rsqf(piv);
        }
        static_for<16>([&](auto tt) {
          constexpr int t = decltype(tt)::value;
          if constexpr (t > c + 1) {
            const float col = row_bcast<t>(Db[c]);
            Db[t] = fmaf(-fD, col, Db[t]);
            P[t] = fmaf(-fP, col, P[t]);
          }
        });
      });
      if (lane < nb) {
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)
          *(f32x4*)&Dl[16 * (b + 1) + lane][16 * b + 4 * c4] =
              f32x4{P[4 * c4] * iv[4 * c4], P[4 * c4 + 1] * iv[4 * c4 + 1], P[4 * c4 + 2] * iv[4 * c4 + 2],
                    P[4 * c4 + 3] * iv[4 * c4 + 3]};
      } else if (lane < nb + 16) {
        // identity row li became column li of inv(L_bb)
#pragma unroll
        for (int c = 0; c < 16; ++c) Xr[b][c][lq] = P[c] * iv[c];
        if constexpr (b == 3) {
#pragma unroll
          for (int c = 0; c < 16; ++c) dst[(48 + c) * 64 + 48 + lq] = P[c] * iv[c];
        }
      }
    } else if constexpr (b == 0) {
      // blocks above the diagonal of inv(L_II) are zero
      const int t = tid - 64;                 // 0..191
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int u = t + 192 * e;            // 384 float4 = 6 blocks of 16x16
        if (u < 384) {
          const int blk = u / 64, w = u % 64, row = w / 4, c4 = w % 4;
          const int rbk = blk < 3 ? 0 : (blk < 5 ? 1 : 2);
          const int cbk = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
          *(f32x4*)&dst[(16 * rbk + row) * 64 + 16 * cbk + 4 * c4] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    } else {
      // panel b-1 applied to the tiles right of panel b, then block column q
      constexpr int pb = b - 1;
      int k = 0;
#pragma unroll
      for (int tj = pb + 2; tj < 4; ++tj)
#pragma unroll
        for (int ti = tj; ti < 4; ++ti, ++k)
          if (k == q) tile_update(ti, tj, pb);
      if (q <= pb) column_step(std::integral_constant<int, pb>{});
    }
    __syncthreads();
  };
  panel_step(std::integral_constant<int, 0>{});
  panel_step(std::integral_constant<int, 1>{});
  panel_step(std::integral_constant<int, 2>{});
  panel_step(std::integral_constant<int, 3>{});
  if (wave > 0) column_step(std::integral_constant<int, 3>{});
  if (tid == 0 && badcol >= 0 && a.info_out[p] == 0) a.info_out[p] = 64 * I + badcol + 1;
}

// coff rows for every launch j = -1 .. KTmax-1: one workgroup per launch, an
// exclusive scan of the per-problem workgroup counts (each thread sums a
// contiguous segment of problems, the segment totals are scanned in LDS).
template <int D>
__global__ __launch_bounds__(256) void chol_offsets_kernel(CholArgs a) {
  const int j = (int)blockIdx.x - 1, tid = threadIdx.x;
  int* off = a.coff + (size_t)blockIdx.x * (a.P + 1);
  const int seg = (a.P + 255) / 256;
  const int p0 = min(a.P, tid * seg), p1 = min(a.P, p0 + seg);
  auto count = [&](int p) {
    const int KT = a.info[p].kpad / 64;
    return chol_panel_wgs(KT, D / 64, j) + chol_trail_wgs(KT, D / 64, j, a.S);
  };
  int sum = 0;
  for (int p = p0; p < p1; ++p) sum += count(p);
  __shared__ int sc[256];
  sc[tid] = sum;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int v = tid >= o ? sc[tid - o] : 0;
    __syncthreads();
    sc[tid] += v;
    __syncthreads();
  }
  int run = sc[tid] - sum;          // exclusive prefix of this segment
  for (int p = p0; p < p1; ++p) {
    off[p] = run;
    run += count(p);
  }
  if (tid == 255) off[a.P] = sc[255];
}

void launch_chol_offsets(const CholArgs& a, int d, hipStream_t s) {
  dim3 grid(a.kpadmax / 64 + 1);
  if (d == 128) hipLaunchKernelGGL((chol_offsets_kernel<128>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((chol_offsets_kernel<64>), grid, dim3(256), 0, s, a);
}

void launch_chol_step(const CholArgs& a, int d, int j, int wgs, hipStream_t s) {
  if (wgs <= 0) return;
  if (d == 128) hipLaunchKernelGGL((chol_step_kernel<128>), dim3(wgs), dim3(256), 0, s, a, j);
  else hipLaunchKernelGGL((chol_step_kernel<64>), dim3(wgs), dim3(256), 0, s, a, j);
}

// Solve L^T X = W for 16 value columns per workgroup, 64-row blocks from the
// bottom up, right-looking: X_i = inv(L_ii)^T W_i, then W_r -= L_ir^T X_i for
// every r < i.  W starts as the A^T Y rows left in M by the factorisation
// (forward substitution); Vc rows < k are written at the end.  Eight waves:
// four solve the diagonal block, all share the block updates.  W is held in
// LDS ([kpad][16] floats, dynamic shared memory) while it fits (INLDS), else
// in the per-slab solve buffer [d/16][kpad][16] in X: only the L blocks and
// inv(L_ii) come from global memory, and the L-block loads of a step are
// issued before its diagonal solve so their latency overlaps it.
template <int D, bool INLDS>
__global__ __launch_bounds__(512) void back_subst_lds_kernel(BackArgs a) {
  extern __shared__ float dyn[];         // INLDS: W [kpadmax][16], then Xs [64][16]
  const int p = blockIdx.y;
  if (a.st && !((1 << a.st[p].status) & a.active_mask)) return;
  const ProbInfo pi = a.info[p];
  const int KT = pi.kpad / 64, ld = pi.kpad;
  const float* __restrict__ Mp = a.M + pi.moff;
  const int dim0 = 16 * blockIdx.x;
  const float* __restrict__ Dinv = a.Dinv + (size_t)pi.xoff / D / 64 * 64 * 64;
  float* Wl = INLDS ? dyn : a.X + pi.xoff + (size_t)blockIdx.x * pi.kpad * 16;
  float* Xs = INLDS ? dyn + (size_t)a.kpadmax * 16 : dyn;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, lq = lane & 15;

  // W[row][c] = M[kpad + dim0 + c][row]: coalesced float4 reads along the row
  for (int e = tid; e < pi.kpad * 4; e += 512) {
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

  // inv(L_ii) as A operand of X_i, loaded one step ahead
  auto load_dinv = [&](float (&dv)[16], int i) {
    const float* Di = Dinv + (size_t)i * 64 * 64;
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2) dv[s2] = Di[(4 * s2 + g) * 64 + 16 * wave + lq];
  };
  // waves 0..3 solve the diagonal block (16 rows each); all eight update
  const bool dw = wave < 4;
  float dv[16];
  if (dw) load_dinv(dv, KT - 1);
  // the two first L blocks of a step (rb = wave, wave + 8) are loaded while
  // the previous step finishes, into the registers its updates have freed
  float av0[4][16], av1[4][16];
  const int rb0 = wave, rb1 = wave + 8;
  if (rb0 < KT - 1) load_block(av0, KT - 1, rb0);
  if (rb1 < KT - 1) load_block(av1, KT - 1, rb1);
  for (int i = KT - 1; i >= 0; --i) {
    // X_i rows b = 16 wave + (4g + r): sum_a inv(L_ii)[a][b] W_i[a][c]
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (dw) {
      float wv[16];
#pragma unroll
      for (int s2 = 0; s2 < 16; ++s2) wv[s2] = Wl[(64 * i + 4 * s2 + g) * 16 + lq];
#pragma unroll
      for (int s2 = 0; s2 < 16; ++s2) x = __builtin_amdgcn_mfma_f32_16x16x4f32(dv[s2], wv[s2], x, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) Xs[(16 * wave + 4 * g + r) * 16 + lq] = x[r];
    }
    if (dw && i > 0) load_dinv(dv, i - 1);
    __syncthreads();
    // every wave has read W_i: it now holds X_i
    if (dw) {
#pragma unroll
      for (int r = 0; r < 4; ++r) Wl[(64 * i + 16 * wave + 4 * g + r) * 16 + lq] = x[r];
    }
    if (i > 0) {
      float bx[16];
#pragma unroll
      for (int s2 = 0; s2 < 16; ++s2) bx[s2] = Xs[(4 * s2 + g) * 16 + lq];
      if (rb0 < i) update_block(av0, bx, rb0);
      if (rb1 < i) update_block(av1, bx, rb1);
      for (int rb = wave + 16; rb < i; rb += 16) {
        load_block(av0, i, rb);
        if (rb + 8 < i) load_block(av1, i, rb + 8);
        update_block(av0, bx, rb);
        if (rb + 8 < i) update_block(av1, bx, rb + 8);
      }
      // next step's first blocks
      if (rb0 < i - 1) load_block(av0, i - 1, rb0);
      if (rb1 < i - 1) load_block(av1, i - 1, rb1);
    }
    __syncthreads();
  }

  const bool ok = a.info_out[p] == 0;
  if (ok) {
    for (int e = tid; e < pi.k * 16; e += 512) {
      const int row = e >> 4, c = e & 15;
      float* v = a.Vc + (size_t)(pi.koff + row) * D + dim0 + c;
      *v = a.accumulate ? *v + Wl[row * 16 + c] : Wl[row * 16 + c];
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
    if (d == 128) hipLaunchKernelGGL((back_subst_lds_kernel<128, true>), grid, dim3(512), lds, s, a);
    else hipLaunchKernelGGL((back_subst_lds_kernel<64, true>), grid, dim3(512), lds, s, a);
    return;
  }
  const size_t xs = 64 * 16 * sizeof(float);
  if (d == 128) hipLaunchKernelGGL((back_subst_lds_kernel<128, false>), grid, dim3(512), xs, s, a);
  else hipLaunchKernelGGL((back_subst_lds_kernel<64, false>), grid, dim3(512), xs, s, a);
}

}  // namespace kvs
