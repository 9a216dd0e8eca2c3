// Select+Fit warm start, gfx950: attention importance of every compress-zone
// key and the top-k selection.
//
// importance_kernel: log imp_j = log sum_i exp(scale q_i.kz_j - lse_i), a
// column log-sum-exp over all training queries (no underflow where the
// softmax weights are tiny).  One workgroup = 64 keys (16 per wave, kept in
// VGPRs as the A operand of S^T = Kz Q^T) x one chunk of queries (staged in
// LDS); each lane keeps a running (max, sum) for its 4 keys and the 16 lanes
// of a key merge by xor shuffles.  Query chunks are merged in topk_kernel.
//
// topk_kernel (one 1024-thread workgroup per problem): radix select of the
// k-th largest importance on an order-preserving 32-bit key, then an
// ascending compaction that keeps every key above the threshold and the
// lowest-positioned ties, and finally the row gather Kc = Kz[idx].
#include "kvs_internal.h"

namespace kvs {

__device__ __forceinline__ f32x4 mfma_t(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float mm = fmaxf(m, m2);
  if (mm == -INFINITY) {
    s = 0.f;
  } else {
    s = s * expf(m - mm) + s2 * expf(m2 - mm);
  }
  m = mm;
}

template <int D>
__global__ __launch_bounds__(256) void importance_kernel(ImpArgs a) {
  const int p = blockIdx.y;
  const int n = a.n, Z = a.Z;
  const int kt0 = blockIdx.x * 64;
  const int nq = ((((n + a.Cq - 1) / a.Cq) + 63) / 64) * 64;
  const int qbeg = blockIdx.z * nq, qend = min(n, qbeg + nq);
  __shared__ float Qs[64][D + 4];
  __shared__ float ls[64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, lq = lane & 15;
  const int key = kt0 + 16 * wave + lq;
  const bool kok = key < Z;
  float kf[D / 4];
#pragma unroll
  for (int j = 0; j < D / 16; ++j) {
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (kok) v = *(const f32x4*)(a.Kz + ((size_t)p * Z + key) * D + 16 * j + 4 * g);
    kf[4 * j] = v.x; kf[4 * j + 1] = v.y; kf[4 * j + 2] = v.z; kf[4 * j + 3] = v.w;
  }
  float m[4], s[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) { m[r] = -INFINITY; s[r] = 0.f; }
  const float* Qp = a.Q + (size_t)p * n * D;
  const float* lp = a.lse + (size_t)p * n;
  const float sc = (float)a.scale;

  for (int qt = qbeg; qt < qend; qt += 64) {
    __syncthreads();
    for (int i = tid; i < 64 * (D / 4); i += 256) {
      const int r = i / (D / 4), c4 = i % (D / 4);
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (qt + r < qend) v = *(const f32x4*)(Qp + (size_t)(qt + r) * D + 4 * c4);
      *(f32x4*)&Qs[r][4 * c4] = v;
    }
    if (tid < 64) ls[tid] = (qt + tid < qend) ? lp[qt + tid] : 0.f;
    __syncthreads();
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < D / 16; ++j) {
        const f32x4 qv = *(const f32x4*)&Qs[16 * qb + lq][16 * j + 4 * g];
        acc = mfma_t(kf[4 * j], qv.x, acc);
        acc = mfma_t(kf[4 * j + 1], qv.y, acc);
        acc = mfma_t(kf[4 * j + 2], qv.z, acc);
        acc = mfma_t(kf[4 * j + 3], qv.w, acc);
      }
      // acc[r] = S^T[key = kt0 + 16 wave + 4g + r][q = qt + 16 qb + lq]
      const int q = qt + 16 * qb + lq;
      if (q < qend) {
        const float lq_ = ls[16 * qb + lq];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = acc[r] * sc - lq_;
          if (v > m[r]) {
            s[r] = s[r] * expf(m[r] - v) + 1.f;
            m[r] = v;
          } else {
            s[r] += expf(v - m[r]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const float m2 = __shfl_xor(m[r], off), s2 = __shfl_xor(s[r], off);
      lse_merge(m[r], s[r], m2, s2);
    }
  }
  if (lq == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int kk = kt0 + 16 * wave + 4 * g + r;
      if (kk < Z) {
        const size_t o = ((size_t)blockIdx.z * a.P + p) * Z + kk;
        a.Mpart[o] = m[r];
        a.Spart[o] = s[r];
      }
    }
  }
}

void launch_importance(const ImpArgs& a, int d, hipStream_t s) {
  dim3 grid((a.Z + 63) / 64, a.P, a.Cq);
  if (d == 128) hipLaunchKernelGGL((importance_kernel<128>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((importance_kernel<64>), grid, dim3(256), 0, s, a);
}

__device__ __forceinline__ unsigned order_key(float x) {
  const unsigned u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(1024) void topk_kernel(TopkArgs a) {
  const int p = blockIdx.x;
  const ProbInfo pi = a.info[p];
  const int Z = a.Z, k = pi.k, tid = threadIdx.x;
  __shared__ unsigned hist[256];
  __shared__ unsigned sh_prefix, sh_need;
  __shared__ int scan[1024];
  __shared__ int sh_base_sel, sh_base_tie;
  // 1) merge query-chunk partials into order keys (kept in Mpart of chunk 0)
  unsigned* keys = reinterpret_cast<unsigned*>(const_cast<float*>(a.Mpart)) + (size_t)p * Z;
  for (int j = tid; j < Z; j += 1024) {
    float m = -INFINITY, s = 0.f;
    for (int c = 0; c < a.Cq; ++c) {
      const size_t o = ((size_t)c * a.P + p) * Z + j;
      lse_merge(m, s, a.Mpart[o], a.Spart[o]);
    }
    // same thread, same address as its chunk-0 read: no cross-thread hazard
    keys[j] = order_key(m + logf(s));
  }
  __syncthreads();
  // 2) radix select (MSB first) of the k-th largest key
  unsigned prefix = 0, need = (unsigned)k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += 1024) hist[i] = 0;
    __syncthreads();
    const unsigned hmask = (shift == 24) ? 0u : (0xFFFFFFFFu << (shift + 8));
    for (int j = tid; j < Z; j += 1024) {
      const unsigned kv = keys[j];
      if ((kv & hmask) == (prefix & hmask)) atomicAdd(&hist[(kv >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      unsigned acc = 0;
      int b = 255;
      for (; b > 0; --b) {
        if (acc + hist[b] >= need) break;
        acc += hist[b];
      }
      sh_prefix = prefix | ((unsigned)b << shift);
      sh_need = need - acc;
    }
    __syncthreads();
    prefix = sh_prefix;
    need = sh_need;
    __syncthreads();
  }
  const unsigned T = prefix;          // k-th largest key; 'need' ties at T are taken
  // 3) ascending compaction
  if (tid == 0) { sh_base_sel = 0; sh_base_tie = 0; }
  __syncthreads();
  for (int j0 = 0; j0 < Z; j0 += 1024) {
    const int j = j0 + tid;
    const unsigned kv = (j < Z) ? keys[j] : 0u;
    const int gt = (j < Z && kv > T) ? 1 : 0;
    const int eq = (j < Z && kv == T) ? 1 : 0;
    // exclusive scan of eq (tie rank)
    scan[tid] = eq;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int v = (tid >= off) ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const int tie_rank = sh_base_tie + scan[tid] - eq;
    const int tot_eq = scan[1023];
    const int sel = gt | (eq && tie_rank < (int)need);
    __syncthreads();
    scan[tid] = sel;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int v = (tid >= off) ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const int pos = sh_base_sel + scan[tid] - sel;
    if (sel && pos < k) a.idx[pi.koff + pos] = j;
    const int tot_sel = scan[1023];
    __syncthreads();
    if (tid == 0) {
      sh_base_sel += tot_sel;
      sh_base_tie += tot_eq;
    }
    __syncthreads();
  }
  __syncthreads();
  // 4) gather the selected rows
  const int d4 = a.d / 4;
  for (int e = tid; e < k * d4; e += 1024) {
    const int row = e / d4, c4 = e % d4;
    const int j = a.idx[pi.koff + row];
    *(f32x4*)(a.Kc + (size_t)(pi.koff + row) * a.d + 4 * c4) =
        *(const f32x4*)(a.Kz + ((size_t)p * Z + j) * a.d + 4 * c4);
  }
}

void launch_topk(const TopkArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(topk_kernel, dim3(a.P), dim3(1024), 0, s, a);
}

}  // namespace kvs
