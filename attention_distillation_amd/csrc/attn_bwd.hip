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
__global__ __launch_bounds__(256) void attn_bwd_kernel(BwdArgs a) {
  // logical block: key tile bx of problem p, query chunk bz; the key tiles of
  // one query chunk (same G, Q and score rows) share an XCD
  unsigned bx, by, bz;
  xcd_block(bx, by, bz);
  const int p = by;
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
  __shared__ float es[64], cs[64];

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
  const float* strow = a.St + pi.soff + (size_t)(kok ? key : 0) * npad;

  // Software-pipelined over query tiles: the global loads of tile t+1 (G, Q,
  // the stored scores and the row terms) are issued inside the MFMA work of
  // tile t.  Rows past qend read the last valid row; their dS is zero, so
  // they never count.  G is staged row-major; Q transposed: lane l of a quad
  // covering rows 4 m .. 4 m + 3 and dims 4 c .. 4 c + 3 reads dim 4 c + l of
  // the four rows (coalesced 4-byte loads across the quads of a wave) and
  // writes them as one 16-byte row segment of Qt.
  constexpr int NL = 64 * (D / 4) / 256;   // float4 of G (and of Q) per thread per tile
  const float* Gp = a.G + prow * D;
  const float* Qp = a.Q + prow * D;
  f32x4 gpre[NL], qpre[NL], spre[4];
  float epre = 0.f, cpre = 0.f;
  auto prefetch = [&](int qt) {
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int i = tid + 256 * u;
      const int rg = i / (D / 4), cg = i % (D / 4);
      gpre[u] = *(const f32x4*)(Gp + (unsigned)(min(qt + rg, qend - 1) * D + 4 * cg));
      const int rq = 4 * (i / (4 * (D / 4))), dq = 4 * ((i >> 2) % (D / 4)) + (i & 3);
#pragma unroll
      for (int j = 0; j < 4; ++j) qpre[u][j] = Qp[(unsigned)(min(qt + rq + j, qend - 1) * D + dq)];
    }
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const int qrow = qt + 16 * qb + 4 * g;
      spre[qb] = *(const f32x4*)(strow + (qrow < qend ? qrow : 0));
    }
    if (tid < 64) {
      const int qq = min(qt + tid, qend - 1);
      epre = a.e[prow + qq];
      cpre = a.crow[prow + qq];
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
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < D / 16; ++j) {
        const f32x4 gv = *(const f32x4*)&Gs[16 * qb + lq][16 * j + 4 * g];
        acc = mfma_f32b(gv.x, vr[4 * j + 0], acc);
        acc = mfma_f32b(gv.y, vr[4 * j + 1], acc);
        acc = mfma_f32b(gv.z, vr[4 * j + 2], acc);
        acc = mfma_f32b(gv.w, vr[4 * j + 3], acc);
      }
      float ds[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int li = 16 * qb + 4 * g + r;
        const bool ok = kok && (qt + li) < qend;
        ds[r] = ok ? expf(sv[r] - es[li]) * (acc[r] + cs[li]) : 0.f;
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

void launch_attn_bwd(const BwdArgs& a, int d, hipStream_t s) {
  dim3 grid((a.kmax + 63) / 64, a.P, a.Cn);
  if (d == 128) hipLaunchKernelGGL((attn_bwd_kernel<128>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((attn_bwd_kernel<64>), grid, dim3(256), 0, s, a);
}

}  // namespace kvs
