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
// A[q][key] G[q][dim], A = exp(St - e).  One workgroup = 4 wave64s = 64 keys
// (16 per wave) x one query split.  The layout is the backward's with dS
// replaced by A: a lane's stored scores (key kw + lq, queries 16 qb + 4 g ..
// + 3 of a 64-query tile) are the A operand of the product as they are
// loaded, G is staged transposed in LDS as the B operand.  The loads of the
// next query tile (G, scores, e) are issued inside the MFMA work of this one
// through buffer resources: G and e over the tile's rows (queries past the
// split's end read zero), the scores over the wave's 16 key rows (keys past
// k read zero and weigh zero; their rows are ignored by the substitution).
// Products are summed in fp32 within a tile and in fp64 across tiles.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void resid_rhs_kernel(RhsArgs a) {
  const int p = blockIdx.y, kt0 = 64 * blockIdx.x, c = blockIdx.z;
  const ProbInfo pi = a.info[p];
  if (kt0 >= pi.kpad) return;
  const int n = a.n, npad = (n + 3) & ~3;
  const int nq = ((((n + a.Cr - 1) / a.Cr) + 63) / 64) * 64;
  const int qbeg = c * nq, qend = min(n, qbeg + nq);
  constexpr int DB = D / 16;

  __shared__ float Gt[D][64 + 4];    // [dim][query]
  __shared__ __align__(16) float es[64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, lq = lane & 15;
  const size_t prow = (size_t)p * n;
  const float* Gp = a.G + prow * D;

  double acc64[DB][4];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc64[db][r] = 0.0;

  // G transposed: lane l of a quad covering queries 4 m .. 4 m + 3 and dims
  // 4 c .. 4 c + 3 reads dim 4 c + l of the four queries (coalesced 4-byte
  // loads across the quads of a wave) and writes them as one 16-byte row
  // segment of Gt
  constexpr int NL = 64 * (D / 4) / 256;
  // first key row of this wave (uniform across it: the resource base needs that)
  const int kw = kt0 + 16 * __builtin_amdgcn_readfirstlane(wave);
  const auto rS = buf_rsrc(a.St + pi.soff + (size_t)kw * npad, (long long)max(0, min(16, pi.k - kw)) * npad * 4);
  const int soff_l = (lq * npad + 4 * g) * 4;
  const bool kok = kw + lq < pi.k;     // this lane's key (rows past k stay zero)
  f32x4 gpre[NL], spre[4];
  float epre = 0.f;
  auto prefetch = [&](int qt) {
    const long long rows = min(64, qend - qt);
    const auto rG = buf_rsrc(Gp + (size_t)qt * D, rows * D * 4);
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int i = tid + 256 * u;
      const int rq = 4 * (i / (4 * (D / 4))), dq = 4 * ((i >> 2) % (D / 4)) + (i & 3);
#pragma unroll
      for (int j = 0; j < 4; ++j) gpre[u][j] = buf_load1(rG, ((rq + j) * D + dq) * 4);
    }
    const int so = soff_l + qt * 4;
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) spre[qb] = buf_load4(rS, so + 64 * qb);
    if (tid < 64) epre = buf_load1(buf_rsrc(a.e + prow + qt, rows * 4), tid * 4);
  };
  if (qbeg < qend) prefetch(qbeg);
  for (int qt = qbeg; qt < qend; qt += 64) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int i = tid + 256 * u;
      const int rq = 4 * (i / (4 * (D / 4))), dq = 4 * ((i >> 2) % (D / 4)) + (i & 3);
      *(f32x4*)&Gt[dq][rq] = gpre[u];
    }
    if (tid < 64) es[tid] = epre;
    f32x4 svv[4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) svv[qb] = spre[qb];
    __syncthreads();
    if (qt + 64 < qend) prefetch(qt + 64);

    f32x4 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const f32x4 e4 = *(const f32x4*)&es[16 * qb + 4 * g];
      float w[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = __expf(svv[qb][r] - e4[r]);
        w[r] = (kok && qt + 16 * qb + 4 * g + r < qend) ? v : 0.f;
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const f32x4 gv = *(const f32x4*)&Gt[16 * db + lq][16 * qb + 4 * g];
        acc[db] = mfma_r(w[0], gv.x, acc[db]);
        acc[db] = mfma_r(w[1], gv.y, acc[db]);
        acc[db] = mfma_r(w[2], gv.z, acc[db]);
        acc[db] = mfma_r(w[3], gv.w, acc[db]);
      }
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc64[db][r] += (double)acc[db][r];
  }

  // acc64[db][r] = sum A[q][key = kt0 + 16 wave + 4 g + r] G[q][dim = 16 db + lq]
  double* out = a.Rpart + (size_t)c * a.xtot + pi.xoff;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      out[(size_t)(kt0 + 16 * wave + 4 * g + r) * D + 16 * db + lq] = acc64[db][r];
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_bf16r(float x0, float x1) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((float __attribute__((ext_vector_type(2)))){x0, x1}, bf16x2));
}
// x = h + m + l for two floats (bf16 pieces, round to nearest even, the
// differences exact in fp32)
__device__ __forceinline__ void split3_pair_r(float x0, float x1, uint32_t& h, uint32_t& m, uint32_t& l) {
  h = pk_bf16r(x0, x1);
  const float r0 = x0 - __uint_as_float(h << 16), r1 = x1 - __uint_as_float(h & 0xffff0000u);
  m = pk_bf16r(r0, r1);
  l = pk_bf16r(r0 - __uint_as_float(m << 16), r1 - __uint_as_float(m & 0xffff0000u));
}
__device__ __forceinline__ f32x4 mfma_rb(i32x4 a, i32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// resid_rhs_kernel with the products of the Gram's large-batch kernels: the
// weights and G split into three bf16 pieces each, six piece products per
// multiply-add on 16x16x32 bf16 MFMA, fp32 sums within a 64-query tile and
// fp64 across tiles as before.  G is split once per tile while it is staged
// (three planes, [dim][query position], 36 words a row); a 32-query product
// t takes, in K slot s of lane group g, query 16 (2t + s / 4) + 4 g + s % 4,
// so the weights a lane already holds (key lq, queries 16 qb + 4 g .. + 3 of
// each 16-query block qb) form its A operand as they are, and the planes
// store query 16 qb + 4 g + r at position 32 (qb / 2) + 8 g + 4 (qb % 2) + r,
// making each lane's eight B values one 16-byte read per plane.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void resid_rhs_split_kernel(RhsArgs a) {
  const int p = blockIdx.y, kt0 = 64 * blockIdx.x, c = blockIdx.z;
  const ProbInfo pi = a.info[p];
  if (kt0 >= pi.kpad) return;
  const int n = a.n, npad = (n + 3) & ~3;
  const int nq = ((((n + a.Cr - 1) / a.Cr) + 63) / 64) * 64;
  const int qbeg = c * nq, qend = min(n, qbeg + nq);
  constexpr int DB = D / 16;
  constexpr int QW = 36;

  __shared__ __align__(16) uint32_t Gs3[3][D][QW];   // pieces of G^T, permuted query positions
  __shared__ __align__(16) float es[64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, lq = lane & 15;
  const size_t prow = (size_t)p * n;
  const float* Gp = a.G + prow * D;

  double acc64[DB][4];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc64[db][r] = 0.0;

  constexpr int NL = 64 * (D / 4) / 256;
  const int kw = kt0 + 16 * __builtin_amdgcn_readfirstlane(wave);
  const auto rS = buf_rsrc(a.St + pi.soff + (size_t)kw * npad, (long long)max(0, min(16, pi.k - kw)) * npad * 4);
  const int soff_l = (lq * npad + 4 * g) * 4;
  const bool kok = kw + lq < pi.k;
  f32x4 gpre[NL], spre[4];
  float epre = 0.f;
  auto prefetch = [&](int qt) {
    const long long rows = min(64, qend - qt);
    const auto rG = buf_rsrc(Gp + (size_t)qt * D, rows * D * 4);
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int i = tid + 256 * u;
      const int rq = 4 * (i / (4 * (D / 4))), dq = 4 * ((i >> 2) % (D / 4)) + (i & 3);
#pragma unroll
      for (int j = 0; j < 4; ++j) gpre[u][j] = buf_load1(rG, ((rq + j) * D + dq) * 4);
    }
    const int so = soff_l + qt * 4;
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) spre[qb] = buf_load4(rS, so + 64 * qb);
    if (tid < 64) epre = buf_load1(buf_rsrc(a.e + prow + qt, rows * 4), tid * 4);
  };
  if (qbeg < qend) prefetch(qbeg);
  for (int qt = qbeg; qt < qend; qt += 64) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int i = tid + 256 * u;
      // queries 4 m .. 4 m + 3 (m = 4 qb + gg) of dim dq
      const int m = i / (4 * (D / 4)), dq = 4 * ((i >> 2) % (D / 4)) + (i & 3);
      const int qb = m >> 2, gg = m & 3;
      const int wpos = 16 * (qb >> 1) + 4 * gg + 2 * (qb & 1);
      uint32_t h0, m0, l0, h1, m1, l1;
      split3_pair_r(gpre[u][0], gpre[u][1], h0, m0, l0);
      split3_pair_r(gpre[u][2], gpre[u][3], h1, m1, l1);
      *(u32x2*)&Gs3[0][dq][wpos] = u32x2{h0, h1};
      *(u32x2*)&Gs3[1][dq][wpos] = u32x2{m0, m1};
      *(u32x2*)&Gs3[2][dq][wpos] = u32x2{l0, l1};
    }
    if (tid < 64) es[tid] = epre;
    f32x4 svv[4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) svv[qb] = spre[qb];
    __syncthreads();
    if (qt + 64 < qend) prefetch(qt + 64);

    f32x4 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      // this lane's weights at queries 16 (2t + h) + 4 g + r, h = 0, 1
      float w[8];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int qb = 2 * t + hh;
        const f32x4 e4 = *(const f32x4*)&es[16 * qb + 4 * g];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = __expf(svv[qb][r] - e4[r]);
          w[4 * hh + r] = (kok && qt + 16 * qb + 4 * g + r < qend) ? v : 0.f;
        }
      }
      uint32_t ah[4], am[4], al[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) split3_pair_r(w[2 * j], w[2 * j + 1], ah[j], am[j], al[j]);
      const i32x4 Ah = {(int)ah[0], (int)ah[1], (int)ah[2], (int)ah[3]};
      const i32x4 Am = {(int)am[0], (int)am[1], (int)am[2], (int)am[3]};
      const i32x4 Al = {(int)al[0], (int)al[1], (int)al[2], (int)al[3]};
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int row = 16 * db + lq, wo = 16 * t + 4 * g;
        const i32x4 Bh = *(const i32x4*)&Gs3[0][row][wo];
        const i32x4 Bm = *(const i32x4*)&Gs3[1][row][wo];
        const i32x4 Bl = *(const i32x4*)&Gs3[2][row][wo];
        f32x4 cc = acc[db];
        cc = mfma_rb(Am, Bm, cc);
        cc = mfma_rb(Al, Bh, cc);
        cc = mfma_rb(Ah, Bl, cc);
        cc = mfma_rb(Am, Bh, cc);
        cc = mfma_rb(Ah, Bm, cc);
        cc = mfma_rb(Ah, Bh, cc);
        acc[db] = cc;
      }
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc64[db][r] += (double)acc[db][r];
  }

  double* out = a.Rpart + (size_t)c * a.xtot + pi.xoff;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      out[(size_t)(kt0 + 16 * wave + 4 * g + r) * D + 16 * db + lq] = acc64[db][r];
}

// r = -1/2 sum_c Rpart[c] - mu Vc (rows < k; 0 below), then L Z = r for 16
// value columns per workgroup.  Top down, right-looking:
// Z_i = inv(L_ii) W_i, then W_r -= L_ri Z_i for every r > i.  W is held in
// LDS ([kpad][16]) while it fits, else in the per-slab buffer in X.  The
// contraction index of an MFMA step s in lane group g is 16 g + s, so every
// lane reads 16 consecutive floats of a row of L (four 16-byte loads).  Eight
// waves: waves 0..3 solve the diagonal block (16 rows each, inv(L_ii) loaded
// one step ahead), all eight share the step's block updates, and the first
// two L blocks a wave updates in a step are loaded while the previous step
// finishes.
template <int D, bool INLDS>
__global__ __launch_bounds__(512) void fwd_subst_kernel(FsubArgs a) {
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

  // every partial of an element is loaded before the first addition (a
  // dependent load per partial left this prologue latency-bound at small
  // batches); the sum keeps the split order
  const double mu = a.mu[p];
  const int Cr = a.Cr;
  constexpr int EU = 2;                 // elements per thread per round
  for (int e0 = tid; e0 < pi.kpad * 16; e0 += EU * 512) {
    double part[EU][kMaxRefineSplits];
    float vc[EU];
#pragma unroll
    for (int u = 0; u < EU; ++u) {
      const int e = e0 + 512 * u, row = e >> 4, c = e & 15;
      const bool live = e < pi.kpad * 16 && row < k;
      const size_t o = pi.xoff + (size_t)row * D + dim0 + c;
#pragma unroll
      for (int cc = 0; cc < kMaxRefineSplits; ++cc)
        part[u][cc] = (live && cc < Cr) ? a.Rpart[(size_t)cc * a.xtot + o] : 0.0;
      vc[u] = live ? a.Vc[(size_t)(pi.koff + row) * D + dim0 + c] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < EU; ++u) {
      const int e = e0 + 512 * u, row = e >> 4;
      if (e >= pi.kpad * 16) break;
      float v = 0.f;
      if (row < k) {
        double s = 0.0;
#pragma unroll
        for (int cc = 0; cc < kMaxRefineSplits; ++cc)
          if (cc < Cr) s += part[u][cc];
        v = (float)(-0.5 * s - mu * (double)vc[u]);
      }
      W[e] = v;
    }
  }

  // -L_{rb,i} as A operands: rows 64 rb + 16 q + lq, columns 64 i + 16 g + s
  auto load_block = [&](float (&lv)[4][16], int rb, int i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float* Lr = Mp + (size_t)(64 * rb + 16 * q + lq) * ld + 64 * i + 16 * g;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const f32x4 v = *(const f32x4*)(Lr + 4 * t);
#pragma unroll
        for (int u = 0; u < 4; ++u) lv[q][4 * t + u] = -v[u];
      }
    }
  };
  // W_rb -= L_{rb,i} Z_i, accumulator seeded with W_rb
  auto update_block = [&](const float (&lv)[4][16], const float (&bz)[16], int rb) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x4 acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = W[(64 * rb + 16 * q + 4 * g + r) * 16 + lq];
#pragma unroll
      for (int s2 = 0; s2 < 16; ++s2) acc = mfma_r(lv[q][s2], bz[s2], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) W[(64 * rb + 16 * q + 4 * g + r) * 16 + lq] = acc[r];
    }
  };
  // inv(L_ii) rows 16 wave + lq, columns 16 g + s
  auto load_dinv = [&](float (&dv)[16], int i) {
    const float* Di = Dinv + (size_t)i * 64 * 64 + (16 * wave + lq) * 64 + 16 * g;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const f32x4 v = *(const f32x4*)(Di + 4 * t);
#pragma unroll
      for (int u = 0; u < 4; ++u) dv[4 * t + u] = v[u];
    }
  };
  const bool dw = wave < 4;
  float dv[16];
  if (dw) load_dinv(dv, 0);
  float l0[4][16], l1[4][16];
  if (1 + wave < KT) load_block(l0, 1 + wave, 0);
  if (9 + wave < KT) load_block(l1, 9 + wave, 0);
  __syncthreads();

  for (int i = 0; i < KT; ++i) {
    // Z_i rows b = 16 wave + 4 g + r: sum_a inv(L_ii)[b][a] W_i[a][c]
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (dw) {
#pragma unroll
      for (int s2 = 0; s2 < 16; ++s2) x = mfma_r(dv[s2], W[(64 * i + 16 * g + s2) * 16 + lq], x);
#pragma unroll
      for (int r = 0; r < 4; ++r) Xs[(16 * wave + 4 * g + r) * 16 + lq] = x[r];
      if (i + 1 < KT) load_dinv(dv, i + 1);
    }
    __syncthreads();
    // every wave has read W_i: it now holds Z_i
    if (dw) {
#pragma unroll
      for (int r = 0; r < 4; ++r) W[(64 * i + 16 * wave + 4 * g + r) * 16 + lq] = x[r];
    }
    if (i + 1 < KT) {
      float bz[16];
#pragma unroll
      for (int s2 = 0; s2 < 16; ++s2) bz[s2] = Xs[(16 * g + s2) * 16 + lq];
      const int r0 = i + 1 + wave, r1 = r0 + 8;
      if (r0 < KT) update_block(l0, bz, r0);
      if (r1 < KT) update_block(l1, bz, r1);
      for (int rb = r0 + 16; rb < KT; rb += 16) {
        load_block(l0, rb, i);
        if (rb + 8 < KT) load_block(l1, rb + 8, i);
        update_block(l0, bz, rb);
        if (rb + 8 < KT) update_block(l1, bz, rb + 8);
      }
      // the next step's first blocks
      if (r0 + 1 < KT) load_block(l0, r0 + 1, i + 1);
      if (r1 + 1 < KT) load_block(l1, r1 + 1, i + 1);
    }
    __syncthreads();
  }

  // Z into the A^T Y rows of M: M[kpad + dim0 + c][row] = Z[row][c]
  for (int e = tid; e < pi.kpad * 16; e += 512) {
    const int c = e / pi.kpad, row = e % pi.kpad;
    Mp[(size_t)(pi.kpad + dim0 + c) * ld + row] = W[row * 16 + c];
  }
}

}  // namespace

int refine_splits(int P, int kpadmax, int n) {
  // about four workgroups per CU over the key tiles and no split longer than
  // 64 query tiles (long sweeps leave long tails), each split at least two
  // query tiles long, at most 16 splits
  const long long tiles = (long long)P * (kpadmax / 64);
  const long long qtiles = (n + 63) / 64;
  long long c = tiles > 0 ? (1024 + tiles - 1) / tiles : 1;
  c = std::max(c, (qtiles + 63) / 64);
  c = std::min(c, std::max(1LL, qtiles / 2));
  c = std::min(c, (long long)kMaxRefineSplits);
  return (int)std::max(1LL, c);
}

void launch_resid_rhs(const RhsArgs& a, int d, hipStream_t s) {
  dim3 grid(a.kpadmax / 64, a.P, a.Cr);
  if (a.split3) {
    if (d == 128) hipLaunchKernelGGL((resid_rhs_split_kernel<128>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((resid_rhs_split_kernel<64>), grid, dim3(256), 0, s, a);
    return;
  }
  if (d == 128) hipLaunchKernelGGL((resid_rhs_kernel<128>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((resid_rhs_kernel<64>), grid, dim3(256), 0, s, a);
}

void launch_fwd_subst(const FsubArgs& a, int d, hipStream_t s) {
  dim3 grid(d / 16, a.P);
  const size_t lds = back_subst_lds_bytes(a.kpadmax);
  if (lds <= (size_t)a.lds_max) {
    if (d == 128) hipLaunchKernelGGL((fwd_subst_kernel<128, true>), grid, dim3(512), lds, s, a);
    else hipLaunchKernelGGL((fwd_subst_kernel<64, true>), grid, dim3(512), lds, s, a);
    return;
  }
  const size_t xs = 64 * 16 * sizeof(float);
  if (d == 128) hipLaunchKernelGGL((fwd_subst_kernel<128, false>), grid, dim3(512), xs, s, a);
  else hipLaunchKernelGGL((fwd_subst_kernel<64, false>), grid, dim3(512), xs, s, a);
}

}  // namespace kvs
