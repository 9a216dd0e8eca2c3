// Normal equations of the ridge value solve, gfx950.
//
// Three kernels form them: gram_kernel (64x64 tiles, fp32 MFMA; small
// batches), gram128_kernel (128x128 tiles, fp32 MFMA) and gram128s_kernel
// (128x128 tiles, bf16 MFMA over exact three-piece splits of the operands;
// the default for large batches, KVS_GRAM=fp32 selects gram128_kernel).
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
// gram_kernel: 64x64 tiles; 4 waves each compute a 32x32 quarter with 16x16x4 fp32
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
// operand reads per flop.  A problem with KT2 = ceil(KT / 2) 128-key tiles
// has the tiles (I2, J2) of the lower triangle plus (KT2, J2) for the d value
// rows of Y^T A (one 128-row tile).  Results go to the same 64-tile layout of
// M as gram_kernel's; rows and columns past kpad (odd KT) and the strictly
// upper quadrant of a diagonal tile are not written.
template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4, 4))) void gram128_kernel(GramArgs a) {
  // Workgroup L runs on XCD L % 8 (hardware round-robin) as that XCD's
  // (L / 8)-th workgroup, and an XCD holds 64 of these (two per CU).  The
  // flat tile order (problems in order, each in gram_queue_tile's 8x8-block
  // order) is cut into rounds of 64 tiles dealt to the XCDs in turn, so the
  // tiles that run together on one XCD come from one or two blocks: they
  // start together, sweep the query axis at the same pace and share their
  // score strips in that XCD's L2.  Every XCD gets the same number of
  // rounds, give or take one.
  const unsigned L = blockIdx.x, bz = blockIdx.z;
  const unsigned slot = L >> 3;
  const long long f = ((long long)(slot >> 6) * 8 + (L & 7)) * 64 + (slot & 63);
  if (f >= a.gtot) return;
  // problem of flat tile f: the last one whose first tile is <= f
  int lo = 0, hi = a.P - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.info[mid].gtoff <= f) lo = mid;
    else hi = mid - 1;
  }
  const int p = lo;
  if (a.st && !((1 << a.st[p].status) & a.active_mask)) return;
  const ProbInfo pi = a.info[p];
  const int KT = pi.kpad / 64, KT2 = (KT + 1) / 2;
  int I2, J2;
  if (!gram_queue_tile(f - pi.gtoff, KT2, I2, J2)) return;
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
  // transposed with one 16-byte LDS store.  The loads go through buffer
  // resources over the tile's score rows (keys past k read zero; those rows
  // and columns are replaced by the identity later), the problem's e and Y
  // rows (queries past n read zero); queries past qend are zeroed; dims past
  // d are zero.  Every offset that the range check needs is in the lane
  // offset.
  const int qk4 = 4 * (tid & 15);
  const auto rE = buf_rsrc(E, (long long)n * 4);
  const auto rY = buf_rsrc(Y, (long long)n * D * 4);
  const auto rR = buf_rsrc(St + (size_t)keyR * npad, (long long)min(128, pi.k - keyR) * npad * 4);
  const auto rC = buf_rsrc(St + (size_t)keyC * npad, (long long)min(128, pi.k - keyC) * npad * 4);
  f32x4 pr[4], pc[4], ev;
  auto prefetch = [&](int qt) {
    ev = buf_load4(rE, (qt + qk4) * 4);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = tid + 512 * u;
      if (yrows) {
        const int dim = i & 127, qy = qt + 4 * (i >> 7);
#pragma unroll
        for (int j = 0; j < 4; ++j) pr[u][j] = dim < D ? buf_load1(rY, ((qy + j) * D + dim) * 4) : 0.f;
      } else {
        pr[u] = buf_load4(rR, ((i >> 4) * npad + qt + qk4) * 4);
      }
      if (!diag) pc[u] = buf_load4(rC, ((i >> 4) * npad + qt + qk4) * 4);
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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Two floats as a pair of bf16 rounded to nearest even (element 0 in the low
// half); the two halves back as floats.
__device__ __forceinline__ uint32_t pk_bf16(float x0, float x1) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((float __attribute__((ext_vector_type(2)))){x0, x1}, bf16x2));
}
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// x = h + m + l for two floats, each piece a bf16: h = bf16(x), m = bf16(x - h),
// l = bf16(x - h - m).  Both differences are exact in fp32 (each piece keeps
// the leading 8 bits of what is left), so |x - h - m - l| <= 2^-24 |x| up to
// the underflow of l.
__device__ __forceinline__ void split3_pair(float x0, float x1, uint32_t& h, uint32_t& m, uint32_t& l) {
  h = pk_bf16(x0, x1);
  const float r0 = x0 - bf_lo(h), r1 = x1 - bf_hi(h);
  m = pk_bf16(r0, r1);
  l = pk_bf16(r0 - bf_lo(m), r1 - bf_hi(m));
}

__device__ __forceinline__ f32x4 mfma_b(i32x4 a, i32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// gram128_kernel's tiles and tile order with the products on bf16 MFMA: every
// staged operand x (a softmax weight, or an element of Y for the value rows)
// is split into three bf16 pieces h + m + l (|x - h - m - l| <= 2^-24 |x|),
// and a product x y is taken as the six piece products of weight at most 2,
//     hh + hm + mh + hl + lh + mm,
// which differ from x y by at most about 2^-22 |x y| (the dropped ml, lm, ll
// terms and the two residuals, of either sign), the size of a few fp32
// roundings.  Each 16x16x32 product sums 32 queries into the fp32
// accumulator, so a 32-query step rounds the accumulator 6 times where the
// fp32 16x16x4 products round it 8 times.  The six products take 6 x 16 = 96
// matrix-pipe cycles per 16x16x32 block against 256 for fp32.
// Operand strips of 32 queries (planes h, m, l of 128 rows, 20 words a row:
// 16 bf16 pairs and 4 words of padding so that the 16-byte operand reads of
// 16 rows fall on distinct banks).
template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4, 4))) void gram128s_kernel(GramArgs a) {
  const unsigned L = blockIdx.x, bz = blockIdx.z;
  const unsigned slot = L >> 3;
  const long long f = ((long long)(slot >> 6) * 8 + (L & 7)) * 64 + (slot & 63);
  if (f >= a.gtot) return;
  int lo = 0, hi = a.P - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.info[mid].gtoff <= f) lo = mid;
    else hi = mid - 1;
  }
  const int p = lo;
  if (a.st && !((1 << a.st[p].status) & a.active_mask)) return;
  const ProbInfo pi = a.info[p];
  const int KT = pi.kpad / 64, KT2 = (KT + 1) / 2;
  int I2, J2;
  if (!gram_queue_tile(f - pi.gtoff, KT2, I2, J2)) return;
  const int n = a.n, npad = (n + 3) & ~3;
  const int nq = ((((n + a.Cg - 1) / a.Cg) + 63) / 64) * 64;
  const int qbeg = bz * nq, qend = min(n, qbeg + nq);

  constexpr int LW = 20;
  __shared__ __align__(16) uint32_t Rs[3][128][LW];
  __shared__ __align__(16) uint32_t Cs[3][128][LW];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, lq = lane & 15;
  const int wr = wave >> 2, wc = wave & 3;
  const bool yrows = I2 >= KT2;
  const bool diag = !yrows && I2 == J2;
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

  // Staging of a 32-query step: element u of a thread (i = tid + 512 u) is,
  // for a key strip, key i / 8 and queries 4 (i % 8) .. + 3 (one 16-byte
  // load); for the value rows, dim i % 128 and queries 4 (i / 128) .. + 3
  // (four 4-byte loads).  Resources and range checks as in gram128_kernel.
  const int qk4 = 4 * (tid & 7);
  const auto rE = buf_rsrc(E, (long long)n * 4);
  const auto rY = buf_rsrc(Y, (long long)n * D * 4);
  const auto rR = buf_rsrc(St + (size_t)keyR * npad, (long long)min(128, pi.k - keyR) * npad * 4);
  const auto rC = buf_rsrc(St + (size_t)keyC * npad, (long long)min(128, pi.k - keyC) * npad * 4);
  f32x4 pr[2], pc[2], ev;
  auto prefetch = [&](int qt) {
    ev = buf_load4(rE, (qt + qk4) * 4);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = tid + 512 * u;
      if (yrows) {
        const int dim = i & 127, qy = qt + 4 * (i >> 7);
#pragma unroll
        for (int j = 0; j < 4; ++j) pr[u][j] = dim < D ? buf_load1(rY, ((qy + j) * D + dim) * 4) : 0.f;
      } else {
        pr[u] = buf_load4(rR, ((i >> 3) * npad + qt + qk4) * 4);
      }
      if (!diag) pc[u] = buf_load4(rC, ((i >> 3) * npad + qt + qk4) * 4);
    }
  };
  auto weights = [&](f32x4 v, int q0) {
    f32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = (q0 + j < qend) ? __expf(v[j] - ev[j]) : 0.f;
    return w;
  };
  // the three pieces of four consecutive queries of one row, as 8-byte stores
  auto stage = [&](uint32_t (*S)[128][LW], int row, int q4, f32x4 v) {
    uint32_t h0, m0, l0, h1, m1, l1;
    split3_pair(v[0], v[1], h0, m0, l0);
    split3_pair(v[2], v[3], h1, m1, l1);
    *(u32x2*)&S[0][row][q4 / 2] = u32x2{h0, h1};
    *(u32x2*)&S[1][row][q4 / 2] = u32x2{m0, m1};
    *(u32x2*)&S[2][row][q4 / 2] = u32x2{l0, l1};
  };
  if (qbeg < qend) prefetch(qbeg);
  for (int qt = qbeg; qt < qend; qt += 32) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = tid + 512 * u;
      if (yrows) {
        const int q4 = 4 * (i >> 7);
        f32x4 v = pr[u];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (qt + q4 + j >= qend) v[j] = 0.f;
        stage(Rs, i & 127, q4, v);
      } else {
        stage(Rs, i >> 3, qk4, weights(pr[u], qt + qk4));
      }
      if (!diag) stage(Cs, i >> 3, qk4, weights(pc[u], qt + qk4));
    }
    __syncthreads();
    if (qt + 32 < qend) prefetch(qt + 32);
    if (idle) continue;
    uint32_t (*C)[128][LW] = diag ? Rs : Cs;
    i32x4 bv[2][3];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int s = 0; s < 3; ++s) bv[jb][s] = *(const i32x4*)&C[s][32 * wc + 16 * jb + lq][4 * g];
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      i32x4 av[3];
#pragma unroll
      for (int s = 0; s < 3; ++s) av[s] = *(const i32x4*)&Rs[s][64 * wr + 16 * ib + lq][4 * g];
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        f32x4 c = acc[ib][jb];
        c = mfma_b(av[1], bv[jb][1], c);   // mm
        c = mfma_b(av[2], bv[jb][0], c);   // lh
        c = mfma_b(av[0], bv[jb][2], c);   // hl
        c = mfma_b(av[1], bv[jb][0], c);   // mh
        c = mfma_b(av[0], bv[jb][1], c);   // hm
        c = mfma_b(av[0], bv[jb][0], c);   // hh
        acc[ib][jb] = c;
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

// gram128s_kernel's products on 256x256 tiles: a tile sweeps two 256-key
// strips, so each staged score feeds 256 outputs instead of 128 and the
// strips are read half as often per flop.  One workgroup of eight waves per
// CU (the two split strips take 120 KB of LDS); wave (wr, wc) owns rows
// 64 wr .. + 63 and columns 128 wc .. + 127 of the tile as two 64-column
// halves (4 x 4 blocks of 16x16 each).  A half is skipped when it lies past
// kpad or strictly above the diagonal (64-tile granularity, as the 64-tile
// layout of M stores); the value tile (Y^T A, d rows) leaves the waves of
// rows past d idle.  Tiles are dealt to the XCDs in rounds of 32 (one per CU).
template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void gram256s_kernel(GramArgs a) {
  const unsigned L = blockIdx.x, bz = blockIdx.z;
  const unsigned slot = L >> 3;
  const long long f = ((long long)(slot >> 5) * 8 + (L & 7)) * 32 + (slot & 31);
  if (f >= a.gtot4) return;
  int lo = 0, hi = a.P - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.info[mid].gtoff4 <= f) lo = mid;
    else hi = mid - 1;
  }
  const int p = lo;
  if (a.st && !((1 << a.st[p].status) & a.active_mask)) return;
  const ProbInfo pi = a.info[p];
  const int KT = pi.kpad / 64, KT4 = (KT + 3) / 4;
  int I4, J4;
  if (!gram_queue_tile(f - pi.gtoff4, KT4, I4, J4)) return;
  const int n = a.n, npad = (n + 3) & ~3;
  const int nq = ((((n + a.Cg - 1) / a.Cg) + 63) / 64) * 64;
  const int qbeg = bz * nq, qend = min(n, qbeg + nq);

  constexpr int LW = 20;
  __shared__ __align__(16) uint32_t Rs[3][256][LW];
  __shared__ __align__(16) uint32_t Cs[3][256][LW];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, lq = lane & 15;
  const int wr = wave >> 1, wc = wave & 1;
  const bool yrows = I4 >= KT4;
  const bool diag = !yrows && I4 == J4;
  const int keyR = 256 * I4, keyC = 256 * J4;
  // 64-tile row and column of the wave's halves
  const int trow = 4 * I4 + wr;
  const bool rows_live = yrows ? 64 * wr < D : 64 * trow < pi.kpad;
  bool live[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int tcol = 4 * J4 + 2 * wc + h;
    live[h] = rows_live && 64 * tcol < pi.kpad && !(diag && tcol > trow);
  }
  const bool idle = !live[0] && !live[1];
  const float* St = a.St + pi.soff;
  const float* E = a.e + (size_t)p * n;
  const float* Y = a.Y + (size_t)p * n * D;

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Staging of a 32-query step: element u of a thread (i = tid + 512 u) is,
  // for a key strip, key i / 8 and queries 4 (i % 8) .. + 3 (one 16-byte
  // load); for the value rows (u < 2 only), dim i % 128 and queries
  // 4 (i / 128) .. + 3 (four 4-byte loads).
  const int qk4 = 4 * (tid & 7);
  const auto rE = buf_rsrc(E, (long long)n * 4);
  const auto rY = buf_rsrc(Y, (long long)n * D * 4);
  const auto rR = buf_rsrc(St + (size_t)keyR * npad, (long long)min(256, pi.k - keyR) * npad * 4);
  const auto rC = buf_rsrc(St + (size_t)keyC * npad, (long long)min(256, pi.k - keyC) * npad * 4);
  f32x4 pr[4], pc[4], ev;
  auto prefetch = [&](int qt) {
    ev = buf_load4(rE, (qt + qk4) * 4);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = tid + 512 * u;
      if (yrows) {
        if (u < 2) {
          const int dim = i & 127, qy = qt + 4 * (i >> 7);
#pragma unroll
          for (int j = 0; j < 4; ++j) pr[u][j] = dim < D ? buf_load1(rY, ((qy + j) * D + dim) * 4) : 0.f;
        }
      } else {
        pr[u] = buf_load4(rR, ((i >> 3) * npad + qt + qk4) * 4);
      }
      if (!diag) pc[u] = buf_load4(rC, ((i >> 3) * npad + qt + qk4) * 4);
    }
  };
  auto weights = [&](f32x4 v, int q0) {
    f32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = (q0 + j < qend) ? __expf(v[j] - ev[j]) : 0.f;
    return w;
  };
  auto stage = [&](uint32_t (*S)[256][LW], int row, int q4, f32x4 v) {
    uint32_t h0, m0, l0, h1, m1, l1;
    split3_pair(v[0], v[1], h0, m0, l0);
    split3_pair(v[2], v[3], h1, m1, l1);
    *(u32x2*)&S[0][row][q4 / 2] = u32x2{h0, h1};
    *(u32x2*)&S[1][row][q4 / 2] = u32x2{m0, m1};
    *(u32x2*)&S[2][row][q4 / 2] = u32x2{l0, l1};
  };
  if (qbeg < qend) prefetch(qbeg);
  for (int qt = qbeg; qt < qend; qt += 32) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = tid + 512 * u;
      if (yrows) {
        if (u < 2) {
          const int q4 = 4 * (i >> 7);
          f32x4 v = pr[u];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (qt + q4 + j >= qend) v[j] = 0.f;
          stage(Rs, i & 127, q4, v);
        }
      } else {
        stage(Rs, i >> 3, qk4, weights(pr[u], qt + qk4));
      }
      if (!diag) stage(Cs, i >> 3, qk4, weights(pc[u], qt + qk4));
    }
    __syncthreads();
    if (qt + 32 < qend) prefetch(qt + 32);
    if (idle) continue;
    uint32_t (*C)[256][LW] = diag ? Rs : Cs;
    i32x4 av[4][3];
#pragma unroll
    for (int ib = 0; ib < 4; ++ib)
#pragma unroll
      for (int s = 0; s < 3; ++s) av[ib][s] = *(const i32x4*)&Rs[s][64 * wr + 16 * ib + lq][4 * g];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (!live[h]) continue;
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const int jb = 4 * h + j4;
        i32x4 bv[3];
#pragma unroll
        for (int s = 0; s < 3; ++s) bv[s] = *(const i32x4*)&C[s][128 * wc + 16 * jb + lq][4 * g];
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
          f32x4 c = acc[ib][jb];
          c = mfma_b(av[ib][1], bv[1], c);   // mm
          c = mfma_b(av[ib][2], bv[0], c);   // lh
          c = mfma_b(av[ib][0], bv[2], c);   // hl
          c = mfma_b(av[ib][1], bv[0], c);   // mh
          c = mfma_b(av[ib][0], bv[1], c);   // hm
          c = mfma_b(av[ib][0], bv[0], c);   // hh
          acc[ib][jb] = c;
        }
      }
    }
  }
  if (idle) return;

  float* Mout = a.Mpart + (size_t)bz * a.mtot + pi.moff;
  const int ld = pi.kpad;
  const int row0 = yrows ? pi.kpad + 64 * wr : keyR + 64 * wr;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (!live[h]) continue;
#pragma unroll
    for (int ib = 0; ib < 4; ++ib)
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int jb = 4 * h + j4;
          const int row = row0 + 16 * ib + 4 * g + r;
          const int col = keyC + 128 * wc + 16 * jb + lq;
          Mout[(size_t)row * ld + col] = acc[ib][jb][r];
        }
  }
}

// 128-row tiles when the batch has enough of them to fill the chip
static bool gram_big_tiles(const GramArgs& a) {
  const long long KT2 = (a.kpadmax / 64 + 1) / 2;
  const long long T2 = KT2 * (KT2 + 1) / 2 + KT2;
  return (long long)a.P * T2 * a.Cg >= 512;
}

bool gram_split_products(const GramArgs& a) { return a.split3 && gram_big_tiles(a); }

void launch_gram(const GramArgs& a, int d, hipStream_t s) {
  const long long KT = a.kpadmax / 64;
  // 256x256 tiles when there are at least eight per CU (one workgroup per
  // CU: with fewer, the 128x128 tiles' two workgroups per CU hide more; the
  // full cache at k = 960 has three); n <= 2^20 keeps the lane offsets of a
  // 256-row strip below 2^31 bytes
  const bool t256 = a.tile256 == 2 || (a.tile256 == 1 && a.gtot4 * a.Cg >= 2048);
  if (gram_big_tiles(a) && a.split3 && t256 && a.n <= (1 << 20)) {
    // whole rounds of 32 tiles on each of the 8 XCDs
    const long long rounds = (a.gtot4 + 32 * 8 - 1) / (32 * 8);
    dim3 grid4((unsigned)(rounds * 32 * 8), 1, a.Cg);
    if (d == 128) hipLaunchKernelGGL((gram256s_kernel<128>), grid4, dim3(512), 0, s, a);
    else hipLaunchKernelGGL((gram256s_kernel<64>), grid4, dim3(512), 0, s, a);
    return;
  }
  if (gram_big_tiles(a)) {
    // whole rounds of 64 tiles on each of the 8 XCDs
    const long long rounds = (a.gtot + 64 * 8 - 1) / (64 * 8);
    dim3 grid2((unsigned)(rounds * 64 * 8), 1, a.Cg);
    if (a.split3) {
      if (d == 128) hipLaunchKernelGGL((gram128s_kernel<128>), grid2, dim3(512), 0, s, a);
      else hipLaunchKernelGGL((gram128s_kernel<64>), grid2, dim3(512), 0, s, a);
      return;
    }
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
