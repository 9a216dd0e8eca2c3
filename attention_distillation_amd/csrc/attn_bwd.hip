// Gradient of the distillation loss with respect to the compressed keys, gfx950.
//
// With G = 2 (Yhat - Y), e = lhat - l and crow_i = -G_i.Yhat_i + 2 lam e_i
// (all produced by the forward merge), and A = exp(St - e) rebuilt from the
// stored shifted scores:
//     dA = G Vc^T,   dS = A * (dA + crow 1^T),   dL/dKc = scale * dS^T Q.
// One workgroup = 4 wave64s = 64 keys (16 per wave) x one chunk of queries.
// Each wave keeps its 16 value rows in VGPRs (B operand of dA), the query
// tile is staged in LDS twice: G row-major (A operand of dA) and Q transposed
// (B operand of dK).  dA comes out with query rows 4g+r and key column lq,
// which is the A-operand layout of dK = dS^T Q, so dS never leaves VGPRs.
// Partial dK per query chunk is written out and summed in a fixed order by
// the gradient pass of the optimizer (no float atomics).
#include "kvs_internal.h"

namespace kvs {

__device__ __forceinline__ f32x4 mfma_f32b(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int D>
// two waves per SIMD (its LDS tiles allow two workgroups per CU); the
// register budget that leaves is 256
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attn_bwd_kernel(BwdArgs a) {
  // logical block: key tile bx of problem p, query chunk bz; the key tiles of
  // one query chunk (same G, Q and score rows) share an XCD
  unsigned bx, by, bz;
  xcd_block(bx, by, bz);
  // logical slot -> problem: the slots of one XCD carry equal total work
  const int p = a.info[by].xorder;
  // the problem table is read before the status test, which uses it, so the
  // two loads share one round trip
  const ProbInfo pi = a.info[p];
  if ((a.st && !((1 << a.st[p].status) & a.active_mask)) || pi.k < 0) return;
  const int k = pi.k;
  const int kt0 = bx * 64;
  if (kt0 >= k) return;
  const int n = a.n, npad = (n + 3) & ~3;
  const int nq = ((((n + a.Cn - 1) / a.Cn) + 63) / 64) * 64;
  const int qbeg = bz * nq;
  const int qend = min(n, qbeg + nq);

  __shared__ float Gs[64][D + 4];
  __shared__ float Qt[D][64 + 4];
  __shared__ __align__(16) float es[64];
  __shared__ __align__(16) float cs[64];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, lq = lane & 15;
  const int key = kt0 + wave * 16 + lq;
  const bool kok = key < k;

  float vr[D / 4];
#pragma unroll
  for (int j = 0; j < D / 16; ++j) {
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (kok) v = *(const f32x4*)(a.V + (size_t)(pi.koff + key) * D + 16 * j + 4 * g);
    vr[4 * j + 0] = v.x; vr[4 * j + 1] = v.y; vr[4 * j + 2] = v.z; vr[4 * j + 3] = v.w;
  }
  f32x4 dk[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) dk[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const size_t prow = (size_t)p * n;

  // Software-pipelined over query tiles: the global loads of tile t+1 (G, Q,
  // the stored scores and the row terms) are issued inside the MFMA work of
  // tile t.  They go through buffer resources: G, Q and the row terms over
  // the rows qt .. qend-1 of the tile, so rows past qend read zero (their dS
  // is zero anyway), and the scores over this wave's 16 key rows, so keys
  // past k read zero; the lane offsets are fixed.  G is staged row-major; Q
  // transposed: lane l of a quad covering rows 4 m .. 4 m + 3 and dims
  // 4 c .. 4 c + 3 reads dim 4 c + l of the four rows (coalesced 4-byte loads
  // across the quads of a wave) and writes them as one 16-byte row segment
  // of Qt.
  constexpr int NL = 64 * (D / 4) / 256;   // float4 of G (and of Q) per thread per tile
  const float* Gp = a.G + prow * D;
  const float* Qp = a.Q + prow * D;
  // first key row of this wave (uniform across it: the resource base needs that)
  const int kw = kt0 + 16 * __builtin_amdgcn_readfirstlane(wave);
  const auto rS = buf_rsrc(a.St + pi.soff + (size_t)kw * npad, (long long)min(16, k - kw) * npad * 4);
  const int soff_l = (lq * npad + 4 * g) * 4;
  f32x4 gpre[NL], qpre[NL], spre[4];
  float epre = 0.f, cpre = 0.f;
  auto prefetch = [&](int qt) {
    const long long rows = min(64, qend - qt);   // the tile's rows
    const auto rG = buf_rsrc(Gp + (size_t)qt * D, rows * D * 4);
    const auto rQ = buf_rsrc(Qp + (size_t)qt * D, rows * D * 4);
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int i = tid + 256 * u;
      const int rg = i / (D / 4), cg = i % (D / 4);
      gpre[u] = buf_load4(rG, (rg * D + 4 * cg) * 4);
      const int rq = 4 * (i / (4 * (D / 4))), dq = 4 * ((i >> 2) % (D / 4)) + (i & 3);
#pragma unroll
      for (int j = 0; j < 4; ++j) qpre[u][j] = buf_load1(rQ, ((rq + j) * D + dq) * 4);
    }
    const int so = soff_l + qt * 4;
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) spre[qb] = buf_load4(rS, so + 64 * qb);
    if (tid < 64) {
      epre = buf_load1(buf_rsrc(a.e + prow + qt, rows * 4), tid * 4);
      cpre = buf_load1(buf_rsrc(a.crow + prow + qt, rows * 4), tid * 4);
    }
  };
  if (qbeg < qend) prefetch(qbeg);
  for (int qt = qbeg; qt < qend; qt += 64) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int i = tid + 256 * u;
      const int rg = i / (D / 4), cg = i % (D / 4);
      *(f32x4*)&Gs[rg][4 * cg] = gpre[u];
      const int rq = 4 * (i / (4 * (D / 4))), dq = 4 * ((i >> 2) % (D / 4)) + (i & 3);
      *(f32x4*)&Qt[dq][rq] = qpre[u];
    }
    if (tid < 64) {
      es[tid] = epre;
      cs[tid] = cpre;
    }
    f32x4 svv[4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) svv[qb] = spre[qb];
    __syncthreads();

#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      // the next tile's loads are issued inside the MFMA work of this one
      if (qb == 1 && qt + 64 < qend) prefetch(qt + 64);
      const f32x4 sv = svv[qb];
      // row terms of this lane's four query rows, read ahead of the dA chain
      const f32x4 e4 = *(const f32x4*)&es[16 * qb + 4 * g];
      const f32x4 c4 = *(const f32x4*)&cs[16 * qb + 4 * g];
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < D / 16; ++j) {
        const f32x4 gv = *(const f32x4*)&Gs[16 * qb + lq][16 * j + 4 * g];
        acc = mfma_f32b(gv.x, vr[4 * j + 0], acc);
        acc = mfma_f32b(gv.y, vr[4 * j + 1], acc);
        acc = mfma_f32b(gv.z, vr[4 * j + 2], acc);
        acc = mfma_f32b(gv.w, vr[4 * j + 3], acc);
      }
      // dS without branches; rows past qend are selected away (their stored
      // scores may be padding).  Keys past k need no mask: a key's dS only
      // reaches its own row of dK, and those rows are not written.
      float ds[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = __expf(sv[r] - e4[r]) * (acc[r] + c4[r]);
        ds[r] = (qt + 16 * qb + 4 * g + r < qend) ? v : 0.f;
      }
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        const f32x4 qv = *(const f32x4*)&Qt[16 * db + lq][16 * qb + 4 * g];
        dk[db] = mfma_f32b(ds[0], qv.x, dk[db]);
        dk[db] = mfma_f32b(ds[1], qv.y, dk[db]);
        dk[db] = mfma_f32b(ds[2], qv.z, dk[db]);
        dk[db] = mfma_f32b(ds[3], qv.w, dk[db]);
      }
    }
  }

  // dk[db][r] = dK[key = kt0 + 16 wave + 4g + r][dim = 16 db + lq]
  float* out = a.dKpart + (size_t)bz * a.ktot * D;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int kr = kt0 + wave * 16 + 4 * g + r;
    if (kr < k) {
#pragma unroll
      for (int db = 0; db < D / 16; ++db) out[(size_t)(pi.koff + kr) * D + 16 * db + lq] = dk[db][r];
    }
  }
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_bf16b(float x0, float x1) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((float __attribute__((ext_vector_type(2)))){x0, x1}, bf16x2));
}
// x = h + m + l for two floats (bf16 pieces, round to nearest even, the
// differences exact in fp32)
__device__ __forceinline__ void split3_pair_b(float x0, float x1, uint32_t& h, uint32_t& m, uint32_t& l) {
  h = pk_bf16b(x0, x1);
  const float r0 = x0 - __uint_as_float(h << 16), r1 = x1 - __uint_as_float(h & 0xffff0000u);
  m = pk_bf16b(r0, r1);
  l = pk_bf16b(r0 - __uint_as_float(m << 16), r1 - __uint_as_float(m & 0xffff0000u));
}
__device__ __forceinline__ f32x4 mfma_bb(i32x4 a, i32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// acc += a b as the six piece products of weight <= 2 (smallest first)
__device__ __forceinline__ f32x4 mfma6(const i32x4 (&a)[3], const i32x4 (&b)[3], f32x4 c) {
  c = mfma_bb(a[1], b[1], c);   // mm
  c = mfma_bb(a[2], b[0], c);   // lh
  c = mfma_bb(a[0], b[2], c);   // hl
  c = mfma_bb(a[1], b[0], c);   // mh
  c = mfma_bb(a[0], b[1], c);   // hm
  return mfma_bb(a[0], b[0], c);   // hh
}

// attn_bwd_kernel with the products of the Gram's large-batch kernels: G,
// Vc, dS and Q split into three bf16 pieces each, six piece products per
// multiply-add on 16x16x32 bf16 MFMA with fp32 accumulation.  Query tiles of
// 32 (the two staged planes sets fit twice per CU): G is staged row-major
// (three planes [query][dim], 68 words a row), Q transposed (three planes
// [dim][query position], 20 words a row).
//  - dA = G Vc^T per 16-query block: A = G rows (8 consecutive dims per
//    lane group), B = this lane's value row, split once per workgroup;
//    dA comes out with query rows 4 g + r and key column lq, as before.
//  - dK += dS^T Q per 32-query tile: in K slot s of lane group g the query
//    16 (s / 4) + 4 g + s % 4, so the dS values a lane holds (key lq, queries
//    16 qb + 4 g .. + 3) form its A operand as they are; the Q planes store
//    query 16 qb + 4 g + r at position 8 g + 4 qb + r, making a lane's eight
//    B values one 16-byte read per plane.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attn_bwd_split_kernel(BwdArgs a) {
  unsigned bx, by, bz;
  xcd_block(bx, by, bz);
  const int p = a.info[by].xorder;
  const ProbInfo pi = a.info[p];
  if ((a.st && !((1 << a.st[p].status) & a.active_mask)) || pi.k < 0) return;
  const int k = pi.k;
  const int kt0 = bx * 64;
  if (kt0 >= k) return;
  const int n = a.n, npad = (n + 3) & ~3;
  const int nq = ((((n + a.Cn - 1) / a.Cn) + 63) / 64) * 64;
  const int qbeg = bz * nq;
  const int qend = min(n, qbeg + nq);
  constexpr int GW = D / 2 + 4;     // words per G plane row
  constexpr int QW = 20;            // words per Q plane row (32 positions + padding)

  __shared__ __align__(16) uint32_t Gs3[3][32][GW];
  __shared__ __align__(16) uint32_t Qs3[3][D][QW];
  __shared__ __align__(16) float es[32];
  __shared__ __align__(16) float cs[32];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, lq = lane & 15;
  const int key = kt0 + wave * 16 + lq;
  const bool kok = key < k;

  // value row of this lane's key, dims 32 kk + 8 g .. + 7, as B pieces
  i32x4 vb[D / 32][3];
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    f32x4 v0 = {0.f, 0.f, 0.f, 0.f}, v1 = v0;
    if (kok) {
      const float* vp = a.V + (size_t)(pi.koff + key) * D + 32 * kk + 8 * g;
      v0 = *(const f32x4*)vp;
      v1 = *(const f32x4*)(vp + 4);
    }
    uint32_t h[4], m[4], l[4];
    split3_pair_b(v0.x, v0.y, h[0], m[0], l[0]);
    split3_pair_b(v0.z, v0.w, h[1], m[1], l[1]);
    split3_pair_b(v1.x, v1.y, h[2], m[2], l[2]);
    split3_pair_b(v1.z, v1.w, h[3], m[3], l[3]);
    vb[kk][0] = i32x4{(int)h[0], (int)h[1], (int)h[2], (int)h[3]};
    vb[kk][1] = i32x4{(int)m[0], (int)m[1], (int)m[2], (int)m[3]};
    vb[kk][2] = i32x4{(int)l[0], (int)l[1], (int)l[2], (int)l[3]};
  }
  f32x4 dk[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) dk[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const size_t prow = (size_t)p * n;
  // per 32-query tile: G row-major and Q transposed, float4 per thread each
  constexpr int NL = 32 * (D / 4) / 256;
  const float* Gp = a.G + prow * D;
  const float* Qp = a.Q + prow * D;
  const int kw = kt0 + 16 * __builtin_amdgcn_readfirstlane(wave);
  const auto rS = buf_rsrc(a.St + pi.soff + (size_t)kw * npad, (long long)min(16, k - kw) * npad * 4);
  const int soff_l = (lq * npad + 4 * g) * 4;
  f32x4 gpre[NL], qpre[NL], spre[2];
  float epre = 0.f, cpre = 0.f;
  auto prefetch = [&](int qt) {
    const long long rows = min(32, qend - qt);
    const auto rG = buf_rsrc(Gp + (size_t)qt * D, rows * D * 4);
    const auto rQ = buf_rsrc(Qp + (size_t)qt * D, rows * D * 4);
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int i = tid + 256 * u;
      const int rg = i / (D / 4), cg = i % (D / 4);
      gpre[u] = buf_load4(rG, (rg * D + 4 * cg) * 4);
      const int rq = 4 * (i / (4 * (D / 4))), dq = 4 * ((i >> 2) % (D / 4)) + (i & 3);
#pragma unroll
      for (int j = 0; j < 4; ++j) qpre[u][j] = buf_load1(rQ, ((rq + j) * D + dq) * 4);
    }
    const int so = soff_l + qt * 4;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) spre[qb] = buf_load4(rS, so + 64 * qb);
    if (tid < 32) {
      epre = buf_load1(buf_rsrc(a.e + prow + qt, rows * 4), tid * 4);
      cpre = buf_load1(buf_rsrc(a.crow + prow + qt, rows * 4), tid * 4);
    }
  };
  if (qbeg < qend) prefetch(qbeg);
  for (int qt = qbeg; qt < qend; qt += 32) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int i = tid + 256 * u;
      uint32_t h0, m0, l0, h1, m1, l1;
      // G row rg, dims 4 cg .. + 3
      const int rg = i / (D / 4), cg = i % (D / 4);
      split3_pair_b(gpre[u][0], gpre[u][1], h0, m0, l0);
      split3_pair_b(gpre[u][2], gpre[u][3], h1, m1, l1);
      *(u32x2*)&Gs3[0][rg][2 * cg] = u32x2{h0, h1};
      *(u32x2*)&Gs3[1][rg][2 * cg] = u32x2{m0, m1};
      *(u32x2*)&Gs3[2][rg][2 * cg] = u32x2{l0, l1};
      // Q queries 4 mq .. + 3 (mq = 4 qb + gg) of dim dq at positions 8 gg + 4 qb
      const int mq = i / (4 * (D / 4)), dq = 4 * ((i >> 2) % (D / 4)) + (i & 3);
      const int wq = 4 * (mq & 3) + 2 * (mq >> 2);
      split3_pair_b(qpre[u][0], qpre[u][1], h0, m0, l0);
      split3_pair_b(qpre[u][2], qpre[u][3], h1, m1, l1);
      *(u32x2*)&Qs3[0][dq][wq] = u32x2{h0, h1};
      *(u32x2*)&Qs3[1][dq][wq] = u32x2{m0, m1};
      *(u32x2*)&Qs3[2][dq][wq] = u32x2{l0, l1};
    }
    if (tid < 32) {
      es[tid] = epre;
      cs[tid] = cpre;
    }
    f32x4 svv[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) svv[qb] = spre[qb];
    __syncthreads();
    if (qt + 32 < qend) prefetch(qt + 32);

    float ds[8];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const f32x4 e4 = *(const f32x4*)&es[16 * qb + 4 * g];
      const f32x4 c4 = *(const f32x4*)&cs[16 * qb + 4 * g];
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        i32x4 ga[3];
#pragma unroll
        for (int sp = 0; sp < 3; ++sp) ga[sp] = *(const i32x4*)&Gs3[sp][16 * qb + lq][16 * kk + 4 * g];
        acc = mfma6(ga, vb[kk], acc);
      }
      // dS without branches; rows past qend are selected away (their stored
      // scores may be padding); keys past k only reach their own rows of
      // dK, which are not written
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = __expf(svv[qb][r] - e4[r]) * (acc[r] + c4[r]);
        ds[4 * qb + r] = (qt + 16 * qb + 4 * g + r < qend) ? v : 0.f;
      }
    }
    i32x4 da[3];
    {
      uint32_t h[4], m[4], l[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) split3_pair_b(ds[2 * j], ds[2 * j + 1], h[j], m[j], l[j]);
      da[0] = i32x4{(int)h[0], (int)h[1], (int)h[2], (int)h[3]};
      da[1] = i32x4{(int)m[0], (int)m[1], (int)m[2], (int)m[3]};
      da[2] = i32x4{(int)l[0], (int)l[1], (int)l[2], (int)l[3]};
    }
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      i32x4 qv[3];
#pragma unroll
      for (int sp = 0; sp < 3; ++sp) qv[sp] = *(const i32x4*)&Qs3[sp][16 * db + lq][4 * g];
      dk[db] = mfma6(da, qv, dk[db]);
    }
  }

  // dk[db][r] = dK[key = kt0 + 16 wave + 4g + r][dim = 16 db + lq]
  float* out = a.dKpart + (size_t)bz * a.ktot * D;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int kr = kt0 + wave * 16 + 4 * g + r;
    if (kr < k) {
#pragma unroll
      for (int db = 0; db < D / 16; ++db) out[(size_t)(pi.koff + kr) * D + 16 * db + lq] = dk[db][r];
    }
  }
}

void launch_attn_bwd(const BwdArgs& a, int d, hipStream_t s) {
  dim3 grid((a.kmax + 63) / 64, a.P, a.Cn);
  if (a.split3) {
    if (d == 128) hipLaunchKernelGGL((attn_bwd_split_kernel<128>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((attn_bwd_split_kernel<64>), grid, dim3(256), 0, s, a);
    return;
  }
  if (d == 128) hipLaunchKernelGGL((attn_bwd_kernel<128>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((attn_bwd_kernel<64>), grid, dim3(256), 0, s, a);
}

}  // namespace kvs
