// L-BFGS on the compressed keys, batched over problems, gfx950.
//
// The two-loop recursion (Nocedal & Wright, Numerical Optimization,
// Algorithm 7.4) is evaluated from inner products: every scalar it needs is
// a combination of s_i.y_j, y_i.y_j, s_i.g and y_i.g, so the recursion runs
// in a few hundred scalar flops per problem (prepare_kernel) and the vectors
// are touched in two streaming passes per iteration:
//   hist_dots_kernel   accepted step: x <- x + a p, s = x_new - x, y = g_new - g,
//                      g <- g_new, and the new inner products (fixed-order
//                      partials per workgroup, double accumulation);
//   direction_kernel   p = c_g g + sum_j (cs_j s_j + cy_j y_j).
// Pairs live in a ring of history+1 slots; the spare slot stages the next
// (s, y) before the curvature test decides whether it enters the history.
#include <float.h>

#include "../../include/kvsculpt.h"
#include "kvs_internal.h"

namespace kvs {

constexpr int kVecPerWG = 1024;   // float4 per workgroup in the vector passes

__device__ __forceinline__ double dsum_wave(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Sum of NV doubles over the 256-thread workgroup (fixed tree), result in out[0..NV).
template <int NV>
__device__ __forceinline__ void wg_sum(double (&v)[NV], double* out, double (*sh)[NV]) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = dsum_wave(v[i]);
  if (lane == 0)
#pragma unroll
    for (int i = 0; i < NV; ++i) sh[wave][i] = v[i];
  __syncthreads();
  if (tid == 0)
#pragma unroll
    for (int i = 0; i < NV; ++i) out[i] = ((sh[0][i] + sh[1][i]) + sh[2][i]) + sh[3][i];
  __syncthreads();
}

__device__ __forceinline__ double dot4(f32x4 a, f32x4 b) {
  return (double)a.x * b.x + (double)a.y * b.y + (double)a.z * b.z + (double)a.w * b.w;
}

__global__ __launch_bounds__(256) void hist_dots_kernel(HistArgs a) {
  const int p = blockIdx.y;
  LbState* st = a.st + p;
  if (!((1 << st->status) & a.active_mask)) return;
  const ProbInfo pi = a.info[p];
  const long long n4 = (long long)pi.k * a.d / 4;
  const long long base4 = (long long)pi.koff * a.d / 4;
  const long long stride4 = (long long)a.ktot * a.d / 4;
  const long long beg = (long long)blockIdx.x * kVecPerWG;
  if (beg >= n4) {
    // keep the partial layout complete: zero contributions
    if (threadIdx.x < kDots) a.part[((size_t)p * a.nwg + blockIdx.x) * kDots + threadIdx.x] = 0.0;
    return;
  }
  const int tid = threadIdx.x;
  const int stg = st->stage;
  const float alpha = (float)st->alpha;
  f32x4* X = reinterpret_cast<f32x4*>(a.x) + base4;
  const f32x4* Pd = reinterpret_cast<const f32x4*>(a.p) + base4;
  f32x4* G = reinterpret_cast<f32x4*>(a.g) + base4;
  const f32x4* Gn = reinterpret_cast<const f32x4*>(a.gnew) + base4;
  f32x4* S = reinterpret_cast<f32x4*>(a.S) + base4;
  f32x4* Yv = reinterpret_cast<f32x4*>(a.Yh) + base4;

  constexpr int PER = kVecPerWG / 256;
  f32x4 sv[PER], yv[PER], gv[PER];
  bool ok[PER];
  double gg = 0.0, ss = 0.0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const long long e = beg + tid + 256 * i;
    ok[i] = e < n4;
    sv[i] = yv[i] = gv[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (!ok[i]) continue;
    const f32x4 gn = Gn[e];
    if (a.mode == 0) {
      const f32x4 xv = X[e], pv = Pd[e], go = G[e];
      f32x4 xn;
      xn.x = __fmaf_rn(alpha, pv.x, xv.x);
      xn.y = __fmaf_rn(alpha, pv.y, xv.y);
      xn.z = __fmaf_rn(alpha, pv.z, xv.z);
      xn.w = __fmaf_rn(alpha, pv.w, xv.w);
      sv[i] = xn - xv;
      yv[i] = gn - go;
      X[e] = xn;
      S[(size_t)stg * stride4 + e] = sv[i];
      Yv[(size_t)stg * stride4 + e] = yv[i];
    }
    G[e] = gn;
    gv[i] = gn;
    gg += dot4(gn, gn);
    ss += dot4(sv[i], sv[i]);
  }
  __shared__ double sh5[4][5];
  __shared__ double sh2[4][2];
  double* out = a.part + ((size_t)p * a.nwg + blockIdx.x) * kDots;
  {
    double v[2] = {gg, ss};
    wg_sum<2>(v, out + 5 * kSlots, sh2);
  }
  // slots to visit: the history plus (accept mode) the staged pair
  const int cnt = st->count;
  const int nvis = cnt + (a.mode == 0 ? 1 : 0);
  for (int t = 0; t < nvis; ++t) {
    const int j = (t < cnt) ? st->order[t] : stg;
    double v[5] = {0.0, 0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (!ok[i]) continue;
      const long long e = beg + tid + 256 * i;
      const f32x4 sj = S[(size_t)j * stride4 + e];
      const f32x4 yj = Yv[(size_t)j * stride4 + e];
      v[0] += dot4(sv[i], yj);   // s_stage . y_j
      v[1] += dot4(sj, yv[i]);   // s_j . y_stage
      v[2] += dot4(yv[i], yj);   // y_stage . y_j
      v[3] += dot4(gv[i], sj);   // g . s_j
      v[4] += dot4(gv[i], yj);   // g . y_j
    }
    wg_sum<5>(v, out + 5 * j, sh5);
  }
}

void launch_hist_dots(const HistArgs& a, hipStream_t s) {
  dim3 grid(a.nwg, a.P);
  hipLaunchKernelGGL(hist_dots_kernel, grid, dim3(256), 0, s, a);
}

// Scalar L-BFGS logic per problem: reduce the inner products, update the
// history, and derive the next direction's coefficients from the two-loop
// recursion; sets status = SEARCH with the first trial step.
//   mode 0: after an accepted (or failed) search; 1: gradient refreshed at
//   the same keys; 2: start (history cleared).
__global__ __launch_bounds__(64) void prepare_kernel(PrepArgs a) {
  const int p = blockIdx.x;
  LbState* st = a.st + p;
  const int status = st->status;
  if (a.mode == 0 && status != ST_ACCEPT && status != ST_FAIL) return;
  __shared__ double d[kDots];
  const int tid = threadIdx.x;
  const bool use_dots = !(a.mode == 0 && status == ST_FAIL);
  if (use_dots) {
    for (int i = tid; i < kDots; i += 64) {
      double s = 0.0;
      for (int b = 0; b < a.nwg; ++b) s += a.part[((size_t)p * a.nwg + b) * kDots + i];
      d[i] = s;
    }
  }
  __syncthreads();
  if (tid != 0) return;
  const int H = a.history;
  if (a.mode == 2 || (a.mode == 0 && status == ST_FAIL)) {
    if (a.mode == 0) st->flags |= KVS_FLAG_LINESEARCH;
    st->count = 0;
    st->stage = 0;
  }
  if (a.mode == 0 && status == ST_ACCEPT) {
    const int stg = st->stage;
    const double sy = d[5 * stg + 0], yy = d[5 * stg + 2], ss = d[5 * kSlots + 1];
    if (sy > a.curv_eps * sqrt(ss) * sqrt(yy)) {
      st->rho[stg] = 1.0 / sy;
      for (int t = 0; t < st->count; ++t) {
        const int j = st->order[t];
        st->SY[stg][j] = d[5 * j + 0];
        st->SY[j][stg] = d[5 * j + 1];
        st->YY[stg][j] = d[5 * j + 2];
        st->YY[j][stg] = d[5 * j + 2];
      }
      st->SY[stg][stg] = sy;
      st->YY[stg][stg] = yy;
      if (st->count < H) {
        st->order[st->count++] = stg;
        // next free slot: the smallest not in the history
        int fr = 0;
        for (; fr < kSlots; ++fr) {
          bool used = false;
          for (int t = 0; t < st->count; ++t) used |= (st->order[t] == fr);
          if (!used) break;
        }
        st->stage = fr;
      } else {
        const int old = st->order[0];
        for (int t = 1; t < H; ++t) st->order[t - 1] = st->order[t];
        st->order[H - 1] = stg;
        st->stage = old;
      }
    }
  }
  if (use_dots) {
    for (int j = 0; j < kSlots; ++j) {
      st->Sg[j] = d[5 * j + 3];
      st->Yg[j] = d[5 * j + 4];
    }
    st->gg = d[5 * kSlots];
  }

  // two-loop recursion through inner products
  const int m = st->count;
  const double gg = st->gg;
  double gtp, a0;
  for (int j = 0; j < kSlots; ++j) { st->cs[j] = 0.0; st->cy[j] = 0.0; }
  if (m > 0) {
    double al[kHistMax], be[kHistMax];
    for (int i = m - 1; i >= 0; --i) {
      const int oi = st->order[i];
      double t = st->Sg[oi];
      for (int j = i + 1; j < m; ++j) t -= al[j] * st->SY[oi][st->order[j]];
      al[i] = st->rho[oi] * t;
    }
    const int on = st->order[m - 1];
    const double gamma = st->SY[on][on] / st->YY[on][on];
    for (int i = 0; i < m; ++i) {
      const int oi = st->order[i];
      double t = st->Yg[oi];
      for (int j = 0; j < m; ++j) t -= al[j] * st->YY[oi][st->order[j]];
      double yr = gamma * t;
      for (int j = 0; j < i; ++j) yr += (al[j] - be[j]) * st->SY[st->order[j]][oi];
      be[i] = st->rho[oi] * yr;
    }
    double gtr = gamma * gg;
    for (int j = 0; j < m; ++j) {
      const int oj = st->order[j];
      gtr += -gamma * al[j] * st->Yg[oj] + (al[j] - be[j]) * st->Sg[oj];
      st->cy[oj] = gamma * al[j];
      st->cs[oj] = -(al[j] - be[j]);
    }
    st->coef_g = -gamma;
    gtp = -gtr;
    a0 = 1.0;
    if (!(gtp < 0.0)) {
      st->flags |= KVS_FLAG_NONDESCENT;
      st->count = 0;
      st->stage = 0;
      for (int j = 0; j < kSlots; ++j) { st->cs[j] = 0.0; st->cy[j] = 0.0; }
    }
  }
  if (st->count == 0) {
    st->coef_g = -1.0;
    gtp = -gg;
    a0 = 1.0 / fmax(1.0, sqrt(gg));
  }
  st->gtp = gtp;
  st->alpha = a0;
  st->trials = 0;
  st->status = ST_SEARCH;
}

void launch_prepare(const PrepArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(prepare_kernel, dim3(a.P), dim3(64), 0, s, a);
}

__global__ __launch_bounds__(256) void direction_kernel(DirArgs a) {
  const int p = blockIdx.y;
  const LbState* st = a.st + p;
  if (st->status != ST_SEARCH) return;
  const ProbInfo pi = a.info[p];
  const long long n4 = (long long)pi.k * a.d / 4;
  const long long base4 = (long long)pi.koff * a.d / 4;
  const long long stride4 = (long long)a.ktot * a.d / 4;
  const long long beg = (long long)blockIdx.x * kVecPerWG;
  if (beg >= n4) return;
  const int m = st->count;
  const float cg = (float)st->coef_g;
  f32x4* Pd = reinterpret_cast<f32x4*>(a.p) + base4;
  const f32x4* G = reinterpret_cast<const f32x4*>(a.g) + base4;
  const f32x4* S = reinterpret_cast<const f32x4*>(a.S) + base4;
  const f32x4* Yv = reinterpret_cast<const f32x4*>(a.Yh) + base4;
  constexpr int PER = kVecPerWG / 256;
  f32x4 acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const long long e = beg + threadIdx.x + 256 * i;
    acc[i] = (e < n4) ? G[e] * cg : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int t = 0; t < m; ++t) {
    const int j = st->order[t];
    const float cs = (float)st->cs[j], cy = (float)st->cy[j];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const long long e = beg + threadIdx.x + 256 * i;
      if (e < n4) acc[i] += S[(size_t)j * stride4 + e] * cs + Yv[(size_t)j * stride4 + e] * cy;
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const long long e = beg + threadIdx.x + 256 * i;
    if (e < n4) Pd[e] = acc[i];
  }
}

void launch_direction(const DirArgs& a, hipStream_t s) {
  dim3 grid(a.nwg, a.P);
  hipLaunchKernelGGL(direction_kernel, grid, dim3(256), 0, s, a);
}

__global__ void state_init_kernel(LbState* st, int P, int clear) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= P) return;
  st[p].status = ST_READY;
  st[p].trials = 0;
  st[p].alpha = 0.0;
  if (clear) {
    st[p].count = 0;
    st[p].stage = 0;
    st[p].flags = 0;
  }
}

void launch_state_init(LbState* st, int P, int clear, hipStream_t s) {
  hipLaunchKernelGGL(state_init_kernel, dim3((P + 63) / 64), dim3(64), 0, s, st, P, clear);
}

__global__ void state_out_kernel(const LbState* st, int* flags, float* loss, int P) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= P) return;
  if (flags) flags[p] |= st[p].flags;
  if (loss) loss[p] = (float)st[p].L;
}

void launch_state_flags_out(const LbState* st, int* flags, float* loss, int P, hipStream_t s) {
  hipLaunchKernelGGL(state_out_kernel, dim3((P + 63) / 64), dim3(64), 0, s, st, flags, loss, P);
}

}  // namespace kvs
