// Batched blocked Cholesky of (A^T A + mu I) carried through the A^T Y rows,
// then the back substitution for Vc, gfx950.
//
// Right-looking, 64-column panels, one launch pair per panel for every
// problem of the batch (problems whose kpad is exhausted exit at once):
//   potrf_panel_kernel  one wave per 64-row tile of the panel: the wave
//                       factors the 64x64 diagonal block in VGPRs (lane r
//                       owns row r, column broadcasts by v_readlane) and,
//                       for tiles below it, solves X L^T = M_I by forward
//                       substitution -- the rows below kpad are the Y^T A
//                       rows, so this is the forward solve L W = A^T Y.
//   trailing_kernel     M_IJ -= L_I L_J^T for the trailing tiles (fp32 MFMA).
// back_subst_kernel then solves L^T X = W for 16 value columns per
// workgroup, 64-row blocks from the bottom up.
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

template <int D>
__global__ __launch_bounds__(64) void potrf_panel_kernel(CholArgs a, int j) {
  const int p = blockIdx.y;
  if (!chol_active(a.st, a.active_mask, p)) return;
  const ProbInfo pi = a.info[p];
  const int KT = pi.kpad / 64;
  if (j >= KT) return;
  const int I = j + blockIdx.x;
  if (I >= KT + D / 64) return;
  const int ld = pi.kpad;
  float* Mp = a.M + pi.moff;
  const int r = threadIdx.x;
  const float mu = (float)a.mu[p];

  float L[64];
  {
    const float* src = Mp + (size_t)(64 * j + r) * ld + 64 * j;
#pragma unroll
    for (int c = 0; c < 64; c += 4) {
      const f32x4 v = *(const f32x4*)(src + c);
      L[c] = v.x; L[c + 1] = v.y; L[c + 2] = v.z; L[c + 3] = v.w;
    }
  }
  const bool real_row = (64 * j + r) < pi.k;
#pragma unroll
  for (int c = 0; c < 64; ++c)
    if (c == r && real_row) L[c] += mu;

  int badcol = -1;
#pragma unroll
  for (int c = 0; c < 64; ++c) {
    const float piv = bcast(L[c], c);
    if (!(piv > 0.f) && badcol < 0) badcol = c;
    const float dgn = sqrtf(piv);
    const float inv = 1.f / dgn;
    L[c] = (r == c) ? dgn : ((r > c) ? L[c] * inv : L[c]);
#pragma unroll
    for (int t = c + 1; t < 64; ++t) L[t] = fmaf(-L[c], bcast(L[c], t), L[t]);
  }

  if (blockIdx.x == 0) {
    float* dst = Mp + (size_t)(64 * j + r) * ld + 64 * j;
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

  // forward substitution of this lane's row against L (64x64, lower)
  const int row = (I < KT) ? 64 * I + r : pi.kpad + 64 * (I - KT) + r;
  float* xr = Mp + (size_t)row * ld + 64 * j;
  float x[64];
#pragma unroll
  for (int c = 0; c < 64; c += 4) {
    const f32x4 v = *(const f32x4*)(xr + c);
    x[c] = v.x; x[c + 1] = v.y; x[c + 2] = v.z; x[c + 3] = v.w;
  }
#pragma unroll
  for (int c = 0; c < 64; ++c) {
    float s = x[c];
#pragma unroll
    for (int t = 0; t < c; ++t) s = fmaf(-x[t], bcast(L[t], c), s);
    x[c] = s / bcast(L[c], c);
  }
#pragma unroll
  for (int c = 0; c < 64; c += 4) *(f32x4*)(xr + c) = f32x4{x[c], x[c + 1], x[c + 2], x[c + 3]};
}

void launch_potrf_panel(const CholArgs& a, int d, int panel, hipStream_t s) {
  const int KT = a.kpadmax / 64;
  dim3 grid(KT + d / 64 - panel, a.P);
  if (d == 128) hipLaunchKernelGGL((potrf_panel_kernel<128>), grid, dim3(64), 0, s, a, panel);
  else hipLaunchKernelGGL((potrf_panel_kernel<64>), grid, dim3(64), 0, s, a, panel);
}

// M_IJ -= L_Ij L_Jj^T for j < J <= I (J a key tile, I any row tile)
template <int D>
__global__ __launch_bounds__(256) void trailing_kernel(CholArgs a, int j, int nJ) {
  const int p = blockIdx.y;
  if (!chol_active(a.st, a.active_mask, p)) return;
  const ProbInfo pi = a.info[p];
  const int KT = pi.kpad / 64;
  if (j >= KT) return;
  const int I = j + 1 + blockIdx.x / nJ;
  const int J = j + 1 + blockIdx.x % nJ;
  if (J >= KT || I >= KT + D / 64 || J > I) return;
  const int ld = pi.kpad;
  float* Mp = a.M + pi.moff;
  const int rowI = (I < KT) ? 64 * I : pi.kpad + 64 * (I - KT);
  const int rowJ = 64 * J;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, lq = lane & 15;
  const int rb = 32 * (wave >> 1), cb = 32 * (wave & 1);

  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) acc[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    f32x4 av[2], bv[2];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
      av[ib] = *(const f32x4*)(Mp + (size_t)(rowI + rb + 16 * ib + lq) * ld + 64 * j + 16 * t + 4 * g);
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
      bv[jb] = *(const f32x4*)(Mp + (size_t)(rowJ + cb + 16 * jb + lq) * ld + 64 * j + 16 * t + 4 * g);
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
#pragma unroll
  for (int ib = 0; ib < 2; ++ib)
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float* dst = Mp + (size_t)(rowI + rb + 16 * ib + 4 * g + r) * ld + rowJ + cb + 16 * jb + lq;
        *dst -= acc[ib][jb][r];
      }
}

void launch_trailing(const CholArgs& a, int d, int panel, hipStream_t s) {
  const int KT = a.kpadmax / 64;
  const int nI = KT + d / 64 - panel - 1;
  const int nJ = KT - panel - 1;
  if (nI <= 0 || nJ <= 0) return;
  dim3 grid(nI * nJ, a.P);
  if (d == 128) hipLaunchKernelGGL((trailing_kernel<128>), grid, dim3(256), 0, s, a, panel, nJ);
  else hipLaunchKernelGGL((trailing_kernel<64>), grid, dim3(256), 0, s, a, panel, nJ);
}

// Solve L^T X = W (W^T sits in rows kpad.. of M), 16 columns per workgroup.
// X is kept in the padded solve buffer, grouped by 16-column slab so each
// workgroup owns whole cache lines; Vc rows < k are written at the end.
template <int D>
__global__ __launch_bounds__(256) void back_subst_kernel(BackArgs a) {
  const int p = blockIdx.y;
  if (a.st && !((1 << a.st[p].status) & a.active_mask)) return;
  const ProbInfo pi = a.info[p];
  const int KT = pi.kpad / 64, ld = pi.kpad;
  const float* Mp = a.M + pi.moff;
  const int dim0 = 16 * blockIdx.x;
  float* Xg = a.X + pi.xoff + (size_t)blockIdx.x * pi.kpad * 16;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, lq = lane & 15;

  __shared__ float Lii[64][65];
  __shared__ float accs[64][17];

  for (int i = KT - 1; i >= 0; --i) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int col = 64 * i + 16 * wave + lq;    // row b of the block (column of L)
    for (int t = i + 1; t < KT; ++t) {
      float av[16], bv[16];
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const int arow = 64 * t + 4 * s + g;
        av[s] = Mp[(size_t)arow * ld + col];
        bv[s] = Xg[(size_t)arow * 16 + lq];
      }
#pragma unroll
      for (int s = 0; s < 16; ++s) acc = mfma_c(av[s], bv[s], acc);
    }
    // acc[r] -> (b = 16 wave + 4 g + r, dim = lq)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int b = 16 * wave + 4 * g + r;
      const float w = Mp[(size_t)(pi.kpad + dim0 + lq) * ld + 64 * i + b];
      accs[b][lq] = w - acc[r];
    }
    for (int e = tid; e < 64 * 64; e += 256) {
      const int rr = e >> 6, cc = e & 63;
      Lii[rr][cc] = (cc <= rr) ? Mp[(size_t)(64 * i + rr) * ld + 64 * i + cc] : 0.f;
    }
    __syncthreads();
    if (tid < 16) {
      float x[64];
#pragma unroll
      for (int b = 63; b >= 0; --b) {
        float s = accs[b][tid];
#pragma unroll
        for (int aa = b + 1; aa < 64; ++aa) s = fmaf(-Lii[aa][b], x[aa], s);
        x[b] = s / Lii[b][b];
      }
#pragma unroll
      for (int b = 0; b < 64; ++b) Xg[(size_t)(64 * i + b) * 16 + tid] = x[b];
    }
    __threadfence();
    __syncthreads();
  }

  const bool ok = a.info_out[p] == 0;
  if (ok) {
    for (int e = tid; e < pi.k * 16; e += 256) {
      const int row = e >> 4, c = e & 15;
      a.Vc[(size_t)(pi.koff + row) * D + dim0 + c] = Xg[(size_t)row * 16 + c];
    }
  }
  if (blockIdx.x == 0 && tid == 0 && !ok) {
    if (a.flags) a.flags[p] |= KVS_FLAG_CHOLESKY;
    if (a.st) a.st[p].flags |= KVS_FLAG_CHOLESKY;
  }
}

void launch_back_subst(const BackArgs& a, int d, hipStream_t s) {
  dim3 grid(d / 16, a.P);
  if (d == 128) hipLaunchKernelGGL((back_subst_kernel<128>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((back_subst_kernel<64>), grid, dim3(256), 0, s, a);
}

}  // namespace kvs
