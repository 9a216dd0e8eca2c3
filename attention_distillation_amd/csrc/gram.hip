// Normal equations of the ridge value solve, gfx950.
//
// The softmax weights are rebuilt from the stored shifted scores while the
// Gram tiles are staged (the scores themselves stay untouched).
//
// For A = exp(St - e) (the softmax weights rebuilt from the stored shifted
// scores, n x k) the kernel forms the augmented lower-trapezoidal matrix
//     M = [ A^T A ]   rows 0..kpad-1  (lower triangle, 64x64 tiles)
//         [ Y^T A ]   rows kpad..kpad+d-1
// so that a Cholesky factorisation of the top block, carried through the
// bottom rows, also performs the forward substitution L W = A^T Y.
// Tiles are 64x64; 4 waves each compute a 32x32 quarter with 16x16x4 fp32
// MFMA, operands staged in LDS along the query (contraction) axis.  The
// query axis can be split over gridDim.z; partial tiles are then summed in
// a fixed order by gram_reduce_kernel, which also pads rows/columns k..kpad-1
// with the identity and emits per-diagonal-tile trace partials.
#include "kvs_internal.h"

namespace kvs {

__device__ __forceinline__ f32x4 mfma_g(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// tile t of a problem with KT key tiles and DT = d/64 value tiles -> (I, J)
__device__ __forceinline__ bool gram_tile(long long t, int KT, int DT, int& I, int& J) {
  const long long tri = (long long)KT * (KT + 1) / 2;
  if (t < tri) {
    int i = (int)((sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
    while ((long long)(i + 1) * (i + 2) / 2 <= t) ++i;
    while ((long long)i * (i + 1) / 2 > t) --i;
    I = i;
    J = (int)(t - (long long)i * (i + 1) / 2);
    return true;
  }
  const long long u = t - tri;
  if (u >= (long long)DT * KT) return false;
  I = KT + (int)(u / KT);
  J = (int)(u % KT);
  return true;
}

template <int D>
__global__ __launch_bounds__(256) void gram_kernel(GramArgs a) {
  // logical block: tile bx of problem p, query split bz; consecutive tiles
  // (same row block of A) share an XCD
  unsigned bx, by, bz;
  xcd_block(bx, by, bz);
  const int p = by;
  if (a.st && !((1 << a.st[p].status) & a.active_mask)) return;
  const ProbInfo pi = a.info[p];
  const int KT = pi.kpad / 64, DT = D / 64;
  int I, J;
  if (!gram_tile(bx, KT, DT, I, J)) return;
  const int n = a.n, npad = (n + 3) & ~3;
  const int nq = ((((n + a.Cg - 1) / a.Cg) + 63) / 64) * 64;
  const int qbeg = bz * nq, qend = min(n, qbeg + nq);

  __shared__ float Ra[64][68];
  __shared__ float Ca[64][68];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, lq = lane & 15;
  const int rb = 32 * (wave >> 1), cb = 32 * (wave & 1);
  const bool diag = (I == J);
  const float* St = a.St + pi.soff;      // stored shifted scores
  const float* E = a.e + (size_t)p * n;
  const float* Y = a.Y + (size_t)p * n * D;

  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Operand tiles of 64 queries, software-pipelined: the loads of the next
  // tile are issued before the MFMA work of this one.  Element u of a thread
  // (i = tid + 256 u) is, for a key tile, key i / 16 and queries 4 (i % 16)
  // .. + 3 (one 16-byte load); for the value rows of YᵀA, dim i % 64 and
  // queries 4 (i / 64) .. + 3, read as four 4-byte loads (consecutive lanes,
  // consecutive dims) so that the tile lands transposed with one 16-byte LDS
  // store.  Keys past k read the last key (their rows and columns are
  // replaced by the identity later); queries past qend are zeroed.
  const bool yrows = I >= KT;
  const int keyR = 64 * I, keyC = 64 * J;
  const int dim0 = 64 * (I - KT);
  f32x4 pr[4], pc[4], ev;
  auto prefetch = [&](int qt) {
    // e of this thread's four key-tile queries (clamped past n)
#pragma unroll
    for (int j = 0; j < 4; ++j) ev[j] = E[min(qt + 4 * (tid & 15) + j, n - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = tid + 256 * u;
      const int r = i >> 4, q4 = 4 * (i & 15);
      if (yrows) {
        const int qy = qt + 4 * (i >> 6);
#pragma unroll
        for (int j = 0; j < 4; ++j) pr[u][j] = Y[(size_t)min(qy + j, n - 1) * D + dim0 + (i & 63)];
      } else {
        pr[u] = *(const f32x4*)(St + (size_t)min(keyR + r, pi.k - 1) * npad + min(qt + q4, npad - 4));
      }
      if (!diag) pc[u] = *(const f32x4*)(St + (size_t)min(keyC + r, pi.k - 1) * npad + min(qt + q4, npad - 4));
    }
  };
  // softmax weights A = exp(St - e) of staged scores (queries past qend: 0);
  // exp in its hardware exp2 form: the arguments are <= 0 up to rounding
  auto weights = [&](f32x4 v, int q0) {
    f32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = (q0 + j < qend) ? __expf(v[j] - ev[j]) : 0.f;
    return w;
  };
  if (qbeg < qend) prefetch(qbeg);
  for (int qt = qbeg; qt < qend; qt += 64) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = tid + 256 * u;
      const int r = yrows ? (i & 63) : (i >> 4), q4 = yrows ? 4 * (i >> 6) : 4 * (i & 15);
      f32x4 v;
      if (yrows) {
        v = pr[u];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (qt + q4 + j >= qend) v[j] = 0.f;
      } else {
        v = weights(pr[u], qt + q4);
      }
      *(f32x4*)&Ra[r][q4] = v;
      if (!diag) *(f32x4*)&Ca[i >> 4][4 * (i & 15)] = weights(pc[u], qt + 4 * (i & 15));
    }
    __syncthreads();
    if (qt + 64 < qend) prefetch(qt + 64);
    float (*C)[68] = diag ? Ra : Ca;
#pragma unroll
    for (int qq = 0; qq < 64; qq += 16) {
      f32x4 av[2], bv[2];
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) av[ib] = *(const f32x4*)&Ra[rb + 16 * ib + lq][qq + 4 * g];
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) bv[jb] = *(const f32x4*)&C[cb + 16 * jb + lq][qq + 4 * g];
#pragma unroll
      for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
          acc[ib][jb] = mfma_g(av[ib].x, bv[jb].x, acc[ib][jb]);
          acc[ib][jb] = mfma_g(av[ib].y, bv[jb].y, acc[ib][jb]);
          acc[ib][jb] = mfma_g(av[ib].z, bv[jb].z, acc[ib][jb]);
          acc[ib][jb] = mfma_g(av[ib].w, bv[jb].w, acc[ib][jb]);
        }
    }
  }

  float* Mout = a.Mpart + (size_t)bz * a.mtot + pi.moff;
  const int ld = pi.kpad;
#pragma unroll
  for (int ib = 0; ib < 2; ++ib)
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 64 * I + rb + 16 * ib + 4 * g + r;
        const int col = 64 * J + cb + 16 * jb + lq;
        Mout[(size_t)row * ld + col] = acc[ib][jb][r];
      }
}

// 128x128 output tiles for batches with many tiles: each staged weight is
// used by 128 outputs instead of 64, which halves the exp work and the LDS
// operand reads per flop.  Tile t of a problem with KT2 = ceil(KT / 2)
// 128-key tiles is (I2, J2) of the lower triangle, then (KT2, J2) for the d
// value rows of Y^T A (one 128-row tile).  Results go to the same 64-tile
// layout of M as gram_kernel's; rows and columns past kpad (odd KT) and the
// strictly upper quadrant of a diagonal tile are not written.
__device__ __forceinline__ bool gram_tile128(long long t, int KT2, int& I2, int& J2) {
  const long long tri = (long long)KT2 * (KT2 + 1) / 2;
  if (t < tri) {
    int i = (int)((sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
    while ((long long)(i + 1) * (i + 2) / 2 <= t) ++i;
    while ((long long)i * (i + 1) / 2 > t) --i;
    I2 = i;
    J2 = (int)(t - (long long)i * (i + 1) / 2);
    return true;
  }
  const long long u = t - tri;
  if (u >= KT2) return false;
  I2 = KT2;
  J2 = (int)u;
  return true;
}

template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4, 4))) void gram128_kernel(GramArgs a) {
  // plain dispatch order: the tiles of every problem spread over all XCDs,
  // so ragged batches load them evenly (the tiles share little in L2 either
  // way: they do not sweep the query axis in step)
  const unsigned bx = blockIdx.x, by = blockIdx.y, bz = blockIdx.z;
  const int p = by;
  if (a.st && !((1 << a.st[p].status) & a.active_mask)) return;
  const ProbInfo pi = a.info[p];
  const int KT = pi.kpad / 64, KT2 = (KT + 1) / 2;
  int I2, J2;
  if (!gram_tile128(bx, KT2, I2, J2)) return;
  const int n = a.n, npad = (n + 3) & ~3;
  const int nq = ((((n + a.Cg - 1) / a.Cg) + 63) / 64) * 64;
  const int qbeg = bz * nq, qend = min(n, qbeg + nq);

  __shared__ float Ra[128][68];
  __shared__ float Ca[128][68];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, lq = lane & 15;
  const int wr = wave >> 2, wc = wave & 3;     // rows 64 wr .. +63, columns 32 wc .. +31 of the tile
  const bool yrows = I2 >= KT2;
  const bool diag = !yrows && I2 == J2;
  // waves with nothing to write skip their MFMA work (they still stage)
  const bool idle = (diag && wr == 0 && wc >= 2) || (yrows && 64 * wr >= D) ||
                    (!yrows && 128 * I2 + 64 * wr >= pi.kpad) || (128 * J2 + 32 * wc >= pi.kpad);
  const float* St = a.St + pi.soff;
  const float* E = a.e + (size_t)p * n;
  const float* Y = a.Y + (size_t)p * n * D;
  const int keyR = 128 * I2, keyC = 128 * J2;

  f32x4 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Operand tiles of 64 queries, loads of the next tile issued before the
  // MFMA work of this one.  Key tiles: element u of a thread (i = tid + 512 u)
  // is key i / 16, queries 4 (i % 16) .. + 3 (one 16-byte load); value rows:
  // dim i % 128, queries 4 (i / 128) .. + 3 (four 4-byte loads), landing
  // transposed with one 16-byte LDS store.  Keys past k read the last key;
  // queries past qend are zeroed; dims past d are zero.
  const int qk4 = 4 * (tid & 15);
  f32x4 pr[4], pc[4], ev;
  auto prefetch = [&](int qt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) ev[j] = E[min(qt + qk4 + j, n - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = tid + 512 * u;
      if (yrows) {
        const int dim = i & 127, qy = qt + 4 * (i >> 7);
#pragma unroll
        for (int j = 0; j < 4; ++j) pr[u][j] = dim < D ? Y[(size_t)min(qy + j, n - 1) * D + dim] : 0.f;
      } else {
        pr[u] = *(const f32x4*)(St + (size_t)min(keyR + (i >> 4), pi.k - 1) * npad + min(qt + qk4, npad - 4));
      }
      if (!diag) pc[u] = *(const f32x4*)(St + (size_t)min(keyC + (i >> 4), pi.k - 1) * npad + min(qt + qk4, npad - 4));
    }
  };
  auto weights = [&](f32x4 v, int q0) {
    f32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = (q0 + j < qend) ? __expf(v[j] - ev[j]) : 0.f;
    return w;
  };
  if (qbeg < qend) prefetch(qbeg);
  for (int qt = qbeg; qt < qend; qt += 64) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = tid + 512 * u;
      if (yrows) {
        const int q4 = 4 * (i >> 7);
        f32x4 v = pr[u];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (qt + q4 + j >= qend) v[j] = 0.f;
        *(f32x4*)&Ra[i & 127][q4] = v;
      } else {
        *(f32x4*)&Ra[i >> 4][qk4] = weights(pr[u], qt + qk4);
      }
      if (!diag) *(f32x4*)&Ca[i >> 4][qk4] = weights(pc[u], qt + qk4);
    }
    __syncthreads();
    if (qt + 64 < qend) prefetch(qt + 64);
    if (idle) continue;
    float (*C)[68] = diag ? Ra : Ca;
#pragma unroll
    for (int qq = 0; qq < 64; qq += 16) {
      f32x4 av[4], bv[2];
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) av[ib] = *(const f32x4*)&Ra[64 * wr + 16 * ib + lq][qq + 4 * g];
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) bv[jb] = *(const f32x4*)&C[32 * wc + 16 * jb + lq][qq + 4 * g];
#pragma unroll
      for (int ib = 0; ib < 4; ++ib)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
          acc[ib][jb] = mfma_g(av[ib].x, bv[jb].x, acc[ib][jb]);
          acc[ib][jb] = mfma_g(av[ib].y, bv[jb].y, acc[ib][jb]);
          acc[ib][jb] = mfma_g(av[ib].z, bv[jb].z, acc[ib][jb]);
          acc[ib][jb] = mfma_g(av[ib].w, bv[jb].w, acc[ib][jb]);
        }
    }
  }
  if (idle) return;

  float* Mout = a.Mpart + (size_t)bz * a.mtot + pi.moff;
  const int ld = pi.kpad;
  const int row0 = yrows ? pi.kpad + 64 * wr : keyR + 64 * wr;
  const int col0 = keyC + 32 * wc;
#pragma unroll
  for (int ib = 0; ib < 4; ++ib)
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + 16 * ib + 4 * g + r;
        const int col = col0 + 16 * jb + lq;
        Mout[(size_t)row * ld + col] = acc[ib][jb][r];
      }
}

void launch_gram(const GramArgs& a, int d, hipStream_t s) {
  const long long KT = a.kpadmax / 64;
  // 128-row tiles when the batch has enough of them to fill the chip
  const long long KT2 = (KT + 1) / 2;
  const long long T2 = KT2 * (KT2 + 1) / 2 + KT2;
  if ((long long)a.P * T2 * a.Cg >= 512) {
    dim3 grid2((unsigned)T2, a.P, a.Cg);
    if (d == 128) hipLaunchKernelGGL((gram128_kernel<128>), grid2, dim3(512), 0, s, a);
    else hipLaunchKernelGGL((gram128_kernel<64>), grid2, dim3(512), 0, s, a);
    return;
  }
  const long long T = KT * (KT + 1) / 2 + (long long)(d / 64) * KT;
  dim3 grid((unsigned)T, a.P, a.Cg);
  if (d == 128) hipLaunchKernelGGL((gram_kernel<128>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((gram_kernel<64>), grid, dim3(256), 0, s, a);
}

// Sum split partials (fixed order), pad with the identity beyond k, trace.
template <int D>
__global__ __launch_bounds__(256) void gram_reduce_kernel(GramReduceArgs a) {
  const int p = blockIdx.y;
  if (a.st && !((1 << a.st[p].status) & a.active_mask)) return;
  const ProbInfo pi = a.info[p];
  const int KT = pi.kpad / 64, DT = D / 64;
  int I, J;
  if (!gram_tile(blockIdx.x, KT, DT, I, J)) return;
  const int ld = pi.kpad, k = pi.k;
  const int tid = threadIdx.x;
  __shared__ double red[256];
  double tr = 0.0;
  for (int i = tid; i < 64 * 16; i += 256) {
    const int r = i >> 4, c4 = i & 15;
    const int row = 64 * I + r;
    const int col = 64 * J + 4 * c4;
    const size_t off = pi.moff + (size_t)row * ld + col;
    f32x4 v = *(const f32x4*)(a.Mpart + off);
    for (int c = 1; c < a.Cg; ++c) v += *(const f32x4*)(a.Mpart + (size_t)c * a.mtot + off);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int cc = col + e;
      if (I < KT) {
        if (row >= k || cc >= k) v[e] = (row == cc) ? 1.f : 0.f;
        else if (row == cc) tr += (double)v[e];
      } else if (cc >= k) {
        v[e] = 0.f;
      }
    }
    *(f32x4*)(a.M + off) = v;
  }
  if (I == J) {
    red[tid] = tr;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
      if (tid < off) red[tid] += red[tid + off];
      __syncthreads();
    }
    if (tid == 0) a.trpart[(size_t)p * (a.kpadmax / 64) + I] = red[0];
  }
}

void launch_gram_reduce(const GramReduceArgs& a, int d, hipStream_t s) {
  const long long KT = a.kpadmax / 64;
  const long long T = KT * (KT + 1) / 2 + (long long)(d / 64) * KT;
  dim3 grid((unsigned)T, a.P);
  if (d == 128) hipLaunchKernelGGL((gram_reduce_kernel<128>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((gram_reduce_kernel<64>), grid, dim3(256), 0, s, a);
}

}  // namespace kvs
