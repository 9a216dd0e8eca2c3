// L-BFGS on the compressed keys, batched over problems, gfx950.
//
// The two-loop recursion (Nocedal & Wright, Numerical Optimization,
// Algorithm 7.4) is evaluated from inner products: every scalar it needs is
// a combination of s_i.y_j, y_i.y_j, s_i.g and y_i.g, so the recursion runs
// in a few hundred scalar flops per problem and the vectors are streamed in
// three bandwidth-bound passes per iteration:
//   dots_kernel         g_new = scale * sum of the backward's split partials,
//                       and for an accepted step x <- x + a p, s = x_new - x,
//                       y = g_new - g (into the staging slot), g <- g_new;
//                       then, one workgroup per chunk, the five inner products of
//                       every history slot with the staged pair and g, kept
//                       in registers and reduced per wave after each of the
//                       chunk's sub-chunks; the last workgroup of each problem
//                       (arrival counter) reduces them in chunk order and runs
//                       the scalar logic (curvature test, ring update, two-loop
//                       coefficients, descent check, first step) on a copy of
//                       the state in LDS, lane-parallel over the history;
//   direction_kernel    p = c_g g + sum_j (cs_j s_j + cy_j y_j) on a search's first
//                       trial, and the trial keys x + alpha p on every trial.
// Pairs live in a ring of history+1 slots; the spare slot stages the next
// (s, y) before the curvature test decides whether it enters the history.
#include "../../include/kvsculpt.h"
#include "kvs_internal.h"

namespace kvs {

static_assert(sizeof(LbState) % 8 == 0, "state is copied to LDS in 8-byte words");

constexpr int kVec4PerWG = 256;     // float4 per workgroup in the streaming passes
constexpr int kDotSub = 2;          // 256-float4 sub-chunks per workgroup in the dot pass
constexpr int kDotVec4PerWG = 256 * kDotSub;  // float4 per workgroup in the dot pass

int vec_chunks(long long kmax_d) {
  const long long v4 = (kmax_d + 3) / 4;
  return (int)std::max<long long>(1, (v4 + kVec4PerWG - 1) / kVec4PerWG);
}
int dots_chunks(long long kmax_d) {
  const long long v4 = (kmax_d + 3) / 4;
  return (int)std::max<long long>(1, (v4 + kDotVec4PerWG - 1) / kDotVec4PerWG);
}

__device__ __forceinline__ double dot4(f32x4 a, f32x4 b) {
  return (double)a.x * b.x + (double)a.y * b.y + (double)a.z * b.z + (double)a.w * b.w;
}

__device__ __forceinline__ bool active(const LbState* st, int mask) {
  return (1 << st->status) & mask;
}

// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 4))) void grad_update_kernel(GradUpdArgs a) {
  const int p = blockIdx.y;
  LbState* st = a.st ? a.st + p : nullptr;
  if (st && !active(st, a.active_mask)) return;
  const ProbInfo pi = a.info[p];
  const long long n4 = (long long)pi.k * a.d / 4;
  const long long e = (long long)blockIdx.x * kVec4PerWG + threadIdx.x;
  if (e >= n4) return;
  const long long base4 = (long long)pi.koff * a.d / 4;
  const long long stride4 = (long long)a.ktot * a.d / 4;
  const f32x4* dK = reinterpret_cast<const f32x4*>(a.dKpart) + base4;
  // split partials in a fixed order, loads issued eight at a time
  f32x4 gn = dK[e];
  for (int c0 = 1; c0 < a.Cn; c0 += 8) {
    f32x4 t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] = dK[(size_t)(c0 + j < a.Cn ? c0 + j : 0) * stride4 + e];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (c0 + j < a.Cn) gn += t[j];
  }
  gn *= (float)a.scale;
  if (a.mode == 2) {
    reinterpret_cast<f32x4*>(a.gout)[base4 + e] = gn;
    return;
  }
  f32x4* G = reinterpret_cast<f32x4*>(a.g) + base4;
  if (a.mode == 0) {
    f32x4* X = reinterpret_cast<f32x4*>(a.x) + base4;
    const f32x4* Pd = reinterpret_cast<const f32x4*>(a.p) + base4;
    const float alpha = (float)st->alpha;
    const int stg = st->stage;
    const f32x4 xv = X[e], pv = Pd[e], go = G[e];
    f32x4 xn;
    xn.x = __fmaf_rn(alpha, pv.x, xv.x);
    xn.y = __fmaf_rn(alpha, pv.y, xv.y);
    xn.z = __fmaf_rn(alpha, pv.z, xv.z);
    xn.w = __fmaf_rn(alpha, pv.w, xv.w);
    X[e] = xn;
    reinterpret_cast<f32x4*>(a.S)[(size_t)stg * stride4 + base4 + e] = xn - xv;
    reinterpret_cast<f32x4*>(a.Yh)[(size_t)stg * stride4 + base4 + e] = gn - go;
  }
  G[e] = gn;
}

void launch_grad_update(const GradUpdArgs& a, hipStream_t s) {
  dim3 grid(a.nch, a.P);
  hipLaunchKernelGGL(grad_update_kernel, grid, dim3(256), 0, s, a);
}

// --------------------------------------------------------------------------
// value of v in lane `src` (uniform), through two 32-bit readlanes
__device__ __forceinline__ double lane_value(double v, int src) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)(b & 0xffffffffLL), src);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), src);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

// Scalar L-BFGS logic of one problem on the LDS copy of its state, spread
// over the first wave of the workgroup (lane i owns history position i).
// d holds the reduced inner products by ring slot: 5 j + r for slot j,
// r = 0..4 as in dots_kernel, then g.g at 5 MS and s.s at 5 MS + 1.
// Every thread of the workgroup calls it (barriers), lanes of wave 0 work.
template <int MS>
__device__ void lbfgs_scalar(LbState* st, const double* d, int mode, int H, double curv_eps, int target) {
  const int tid = threadIdx.x;
  const bool w0 = tid < 64;
  const int lane = tid & 63;
  __syncthreads();
  const int status = st->status;
  const bool use_dots = !(mode == 0 && status == ST_FAIL);
  const bool reset = (mode == 2 || (mode == 0 && status == ST_FAIL));
  const bool accept = (mode == 0 && status == ST_ACCEPT);
  const int cnt0 = st->count, stg0 = st->stage;
  __syncthreads();
  // inner products with g, by slot (slots outside the history are
  // rewritten before they are read)
  if (use_dots && w0 && lane < MS) {
    st->Sg[lane] = d[5 * lane + 3];
    st->Yg[lane] = d[5 * lane + 4];
  }
  if (use_dots && tid == 0) {
    st->gg = d[5 * MS];
    // a fresh loss and gradient (start, accepted step, or after a value
    // re-solve): record a non-finite one; the problem then keeps failing its
    // searches and stays where it is
    if (!(isfinite(st->L) && isfinite(st->gg))) st->flags |= KVS_FLAG_NONFINITE;
  }
  __syncthreads();
  if (reset && tid == 0) {
    if (mode == 0) st->flags |= KVS_FLAG_LINESEARCH;
    st->count = 0;
    st->stage = 0;
  }
  __syncthreads();
  if (accept) {
    const int stg = stg0, cnt = cnt0;
    const double sy = d[5 * stg + 0], yy = d[5 * stg + 2], ss = d[5 * MS + 1];
    const bool push = sy > curv_eps * sqrt(ss) * sqrt(yy);
    if (push) {
      if (w0 && lane < cnt) {
        const int j = st->order[lane];
        st->SY[stg][j] = d[5 * j + 0];
        st->SY[j][stg] = d[5 * j + 1];
        st->YY[stg][j] = d[5 * j + 2];
        st->YY[j][stg] = d[5 * j + 2];
      }
      __syncthreads();
      if (tid == 0) {
        st->rho[stg] = 1.0 / sy;
        st->SY[stg][stg] = sy;
        st->YY[stg][stg] = yy;
        if (cnt < H) {
          st->order[cnt] = stg;
          st->count = cnt + 1;
          unsigned used = 0;                  // smallest slot not in the history
          for (int t = 0; t <= cnt; ++t) used |= 1u << st->order[t];
          st->stage = __builtin_ctz(~used);
        } else {
          const int old = st->order[0];
          for (int t = 1; t < H; ++t) st->order[t - 1] = st->order[t];
          st->order[H - 1] = stg;
          st->stage = old;
        }
      }
    }
  }
  if (w0 && lane < kSlots) { st->cs[lane] = 0.0; st->cy[lane] = 0.0; }
  __syncthreads();

  // two-loop recursion through inner products: two triangular solves of
  // size m <= 16 with lane-parallel updates
  const int m = st->count;
  const double gg = st->gg;
  double gtp = -gg, coef_g = -1.0;
  bool nondescent = false;
  if (m > 0 && w0) {
    const bool mine = lane < m;
    const int oi = mine ? st->order[lane] : 0;
    double row[kHistMax], col[kHistMax], yyr[kHistMax];
#pragma unroll
    for (int j = 0; j < kHistMax; ++j) {
      const int oj = (j < m) ? st->order[j] : 0;
      row[j] = (mine && j < m) ? st->SY[oi][oj] : 0.0;   // s_i . y_j
      col[j] = (mine && j < m) ? st->SY[oj][oi] : 0.0;   // s_j . y_i
      yyr[j] = (mine && j < m) ? st->YY[oi][oj] : 0.0;
    }
    const double rho = mine ? st->rho[oi] : 0.0;
    const double sg = mine ? st->Sg[oi] : 0.0, yg = mine ? st->Yg[oi] : 0.0;
    double al[kHistMax], be[kHistMax];
    // newest -> oldest: a_i = rho_i (s_i.g - sum_{j>i} a_j s_i.y_j)
    double acc = sg;
#pragma unroll
    for (int j = kHistMax - 1; j >= 0; --j) {
      al[j] = 0.0;
      if (j < m) {
        const double mine_al = rho * acc;
        al[j] = lane_value(mine_al, j);
        if (lane < j) acc -= al[j] * row[j];
      }
    }
    const int on = st->order[m - 1];
    const double gamma = st->SY[on][on] / st->YY[on][on];
    // oldest -> newest: b_i = rho_i y_i.r, r = gamma (g - sum a_j y_j) + sum_{j<i} (a_j - b_j) s_j
    double c = yg;
#pragma unroll
    for (int j = 0; j < kHistMax; ++j)
      if (j < m) c -= al[j] * yyr[j];
    c *= gamma;
    double acc2 = 0.0;
#pragma unroll
    for (int j = 0; j < kHistMax; ++j) {
      be[j] = 0.0;
      if (j < m) {
        const double mine_be = rho * (c + acc2);
        be[j] = lane_value(mine_be, j);
        if (lane > j) acc2 += (al[j] - be[j]) * col[j];
      }
    }
    double my_al = 0.0, my_be = 0.0;
#pragma unroll
    for (int j = 0; j < kHistMax; ++j)
      if (j == lane) { my_al = al[j]; my_be = be[j]; }
    double term = mine ? (-gamma * my_al * yg + (my_al - my_be) * sg) : 0.0;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) term += __shfl_xor(term, off);
    gtp = -(gamma * gg + term);
    coef_g = -gamma;
    if (gtp < 0.0) {
      if (mine) {
        st->cy[oi] = gamma * my_al;
        st->cs[oi] = -(my_al - my_be);
      }
    } else {
      nondescent = true;
    }
  }
  __syncthreads();
  if (tid == 0) {
    double a0 = 1.0;
    if (nondescent) {
      st->flags |= KVS_FLAG_NONDESCENT;
      st->count = 0;
      st->stage = 0;
    }
    if (st->count == 0) {
      coef_g = -1.0;
      gtp = -gg;
      a0 = 1.0 / fmax(1.0, sqrt(gg));
    }
    st->coef_g = coef_g;
    st->gtp = gtp;
    st->alpha = a0;
    st->trials = 0;
    int next = ST_SEARCH;
    if (mode == 0) {
      st->iter += 1;
      if (st->iter >= target) next = (status == ST_FAIL) ? ST_DONE_FAIL : ST_DONE;
    } else {
      st->iter = 0;
    }
    st->status = next;
  }
  __syncthreads();
}

// One workgroup per chunk of kDotSub 256-float4 sub-chunks of a problem's
// vectors, one float4 per thread per sub-chunk.  The five inner products are
// taken per ring slot (not per history position), so no vector load waits for
// the history order: the problem table and the state header are read
// together, then every vector load of the thread for a sub-chunk is issued at
// once.  Each sub-chunk's products are reduced across the wave and added to
// the lane's running total (the two waves of a SIMD overlap one's loads with
// the other's arithmetic, and the partial store and arrival are paid once per
// chunk).  The history slots and the gradient partials are read once per
// iteration, with non-temporal loads (3.5% faster on the long-context heads,
// the direction pass after it reading the slots 2% slower), and only the
// Cn partials that exist.  The last workgroup of the problem sums the chunk
// partials in a fixed order and runs the scalar logic.  MS bounds the ring
// slots in use (history + 1).
template <int MS>
__global__ __launch_bounds__(256) void dots_kernel(DotsArgs a) {
  constexpr int E = 5 * MS + 2;            // partial entries per chunk
  const int p = blockIdx.y;
  LbState* gst = a.st + p;
  const ProbInfo pi = a.info[p];
  const int status = gst->status;
  const int stg = gst->stage;
  const float alpha = (float)gst->alpha;
  if (!((1 << status) & a.active_mask) || pi.k < 0) return;   // both loads before the test
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const long long n4 = (long long)pi.k * a.d / 4;
  const long long base4 = (long long)pi.koff * a.d / 4;
  const long long stride4 = (long long)a.ktot * a.d / 4;
  const int nslot = a.history + 1;         // ring slots in use
  const bool accept = (a.mode == 0 && status == ST_ACCEPT);
  const bool compute = !(a.mode == 0 && status == ST_FAIL);
  double* out = a.part + ((size_t)p * a.nch + blockIdx.x) * E;
  constexpr int NV = (E + 63) / 64;       // reduced values per lane
  __shared__ double red[4][64 * NV];
  __shared__ int s_last;

  if (compute) {
    // per-lane running totals of the wave-reduced values over the sub-chunks
    double tot[NV];
#pragma unroll
    for (int gi = 0; gi < NV; ++gi) tot[gi] = 0.0;
    for (int sub = 0; sub < kDotSub; ++sub) {
      const long long e0 = ((long long)blockIdx.x * kDotSub + sub) * 256;
      if (e0 >= n4) break;                 // uniform across the workgroup
      const long long e = e0 + tid;
      const bool ok = e < n4;
      const long long ec = ok ? e : 0;       // in-range index for the loads of idle lanes
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      const f32x4* S = reinterpret_cast<const f32x4*>(a.S) + base4;
      const f32x4* Yv = reinterpret_cast<const f32x4*>(a.Yh) + base4;
      f32x4 sj[MS], yj[MS];
#pragma unroll
      for (int t = 0; t < MS; ++t) {
        const bool use = t < nslot;
        sj[t] = use ? __builtin_nontemporal_load(S + (size_t)t * stride4 + ec) : z;
        yj[t] = use ? __builtin_nontemporal_load(Yv + (size_t)t * stride4 + ec) : z;
      }
      f32x4 gv = z, sv = z, yv = z;
      if (a.grad) {
        // gradient from the split partials (fixed order), then the accepted
        // step and its (s, y) pair, staged in slot stg
        const f32x4* dK = reinterpret_cast<const f32x4*>(a.dKpart) + base4;
        f32x4* G = reinterpret_cast<f32x4*>(a.g) + base4;
        f32x4* X = reinterpret_cast<f32x4*>(a.x) + base4;
        const f32x4 go = G[ec];
        const f32x4 xv = accept ? X[ec] : z;
        const f32x4 pv = accept ? reinterpret_cast<const f32x4*>(a.pdir)[base4 + ec] : z;
        f32x4 t0[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) t0[j] = j < a.Cn ? __builtin_nontemporal_load(dK + (size_t)j * stride4 + ec) : z;
        f32x4 gn = t0[0];
#pragma unroll
        for (int j = 1; j < 8; ++j)
          if (j < a.Cn) gn += t0[j];
        for (int c0 = 8; c0 < a.Cn; c0 += 8) {
          f32x4 t[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) t[j] = c0 + j < a.Cn ? __builtin_nontemporal_load(dK + (size_t)(c0 + j) * stride4 + ec) : z;
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (c0 + j < a.Cn) gn += t[j];
        }
        gn *= (float)a.gscale;
        if (ok) {
          if (accept) {
            f32x4 xn;
            xn.x = __fmaf_rn(alpha, pv.x, xv.x);
            xn.y = __fmaf_rn(alpha, pv.y, xv.y);
            xn.z = __fmaf_rn(alpha, pv.z, xv.z);
            xn.w = __fmaf_rn(alpha, pv.w, xv.w);
            X[e] = xn;
            sv = xn - xv;
            yv = gn - go;
            reinterpret_cast<f32x4*>(a.S)[(size_t)stg * stride4 + base4 + e] = sv;
            reinterpret_cast<f32x4*>(a.Yh)[(size_t)stg * stride4 + base4 + e] = yv;
          }
          G[e] = gn;
          gv = gn;
        }
      } else {
        gv = ok ? reinterpret_cast<const f32x4*>(a.g)[base4 + e] : z;
        sv = (ok && accept) ? S[(size_t)stg * stride4 + e] : z;
        yv = (ok && accept) ? Yv[(size_t)stg * stride4 + e] : z;
      }
      if (!ok) {
#pragma unroll
        for (int t = 0; t < MS; ++t) sj[t] = yj[t] = z;
      }
      // the staged slot holds the new pair (its loads above may predate the
      // stores): take it from registers
#pragma unroll
      for (int t = 0; t < MS; ++t)
        if (accept && t == stg) {
          sj[t] = sv;
          yj[t] = yv;
        }
      // all E values of this lane, padded to a multiple of 64, then a
      // butterfly reduction per group of 64: at each level a lane keeps one
      // half of its values and adds the partner's copy of that half, so lane l
      // ends with the wave total of value l of the group (63 exchanges per
      // group instead of a full reduction per value)
      double v[64 * NV];
#pragma unroll
      for (int t = 0; t < MS; ++t) {
        v[5 * t + 0] = dot4(sv, yj[t]);   // s_new . y_t
        v[5 * t + 1] = dot4(sj[t], yv);   // s_t . y_new
        v[5 * t + 2] = dot4(yv, yj[t]);   // y_new . y_t
        v[5 * t + 3] = dot4(gv, sj[t]);   // g . s_t
        v[5 * t + 4] = dot4(gv, yj[t]);   // g . y_t
      }
      v[5 * MS] = dot4(gv, gv);
      v[5 * MS + 1] = dot4(sv, sv);
#pragma unroll
      for (int i = E; i < 64 * NV; ++i) v[i] = 0.0;
#pragma unroll
      for (int gi = 0; gi < NV; ++gi) {
        double* w = v + 64 * gi;
#pragma unroll
        for (int L = 32; L > 0; L >>= 1) {
          const bool hi = (lane & L) != 0;
#pragma unroll
          for (int i = 0; i < L; ++i) {
            const double send = hi ? w[i] : w[i + L];
            const double keep = hi ? w[i + L] : w[i];
            w[i] = keep + __shfl_xor(send, L);
          }
        }
        tot[gi] += w[0];
      }
    }
#pragma unroll
    for (int gi = 0; gi < NV; ++gi) red[wave][64 * gi + lane] = tot[gi];
    __syncthreads();
    if (tid < E) coherent_store(out + tid, ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid]);
  }
  // arrival: the last workgroup of this problem runs the scalar logic
  wait_own_stores();
  __syncthreads();
  if (tid == 0) s_last = arrive_last(a.counter + p, gridDim.x);
  __syncthreads();
  if (!s_last) return;

  __shared__ double fold[256];
  __shared__ double d[E];
  __shared__ LbState ls;
  // state copy to LDS; its loads go out together with the partial loads below
  {
    const unsigned long long* s8 = reinterpret_cast<const unsigned long long*>(gst);
    unsigned long long* d8 = reinterpret_cast<unsigned long long*>(&ls);
    for (int i = tid; i < (int)(sizeof(LbState) / 8); i += 256) d8[i] = s8[i];
  }
  if (compute) {
    // value i is summed by G threads, thread q over chunks q, q + G, ...
    // (up to 32 loads in flight), then the G sums in order of q
    constexpr int G = 256 / E;
    const int i = tid % E, q = tid / E;
    const double* src = a.part + (size_t)p * a.nch * E;
    double acc = 0.0;
    if (q < G) {
      for (int c0 = q; c0 < a.nch; c0 += 32 * G) {
        double t[32];
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          const int c = c0 + j * G;
          t[j] = coherent_load(src + (size_t)(c < a.nch ? c : 0) * E + i);
        }
#pragma unroll
        for (int j = 0; j < 32; ++j)
          if (c0 + j * G < a.nch) acc += t[j];
      }
      fold[tid] = acc;
    }
    __syncthreads();
    if (tid < E) {
      double sum = fold[tid];
#pragma unroll
      for (int r = 1; r < G; ++r) sum += fold[tid + r * E];
      d[tid] = sum;
    }
  }
  lbfgs_scalar<MS>(&ls, d, a.mode, a.history, a.curv_eps, a.target);
  {
    const unsigned long long* s8 = reinterpret_cast<const unsigned long long*>(&ls);
    unsigned long long* d8 = reinterpret_cast<unsigned long long*>(gst);
    for (int i = tid; i < (int)(sizeof(LbState) / 8); i += 256) d8[i] = s8[i];
  }
  if (tid == 0) {
    if (a.status_view) a.status_view[p] = ls.status;
    a.counter[p] = 0u;
  }
}

void launch_dots(const DotsArgs& a, hipStream_t s) {
  dim3 grid(a.nch, a.P);
  if (a.history <= 10) hipLaunchKernelGGL((dots_kernel<11>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((dots_kernel<kSlots>), grid, dim3(256), 0, s, a);
}

// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void direction_kernel(DirArgs a) {
  const int p = blockIdx.y;
  const LbState* st = a.st + p;
  const ProbInfo pi = a.info[p];
  // problems in search; the table load joins the state load before the test
  if (st->status != ST_SEARCH || pi.k < 0) return;
  const long long n4 = (long long)pi.k * a.d / 4;
  const long long e = (long long)blockIdx.x * kVec4PerWG + threadIdx.x;
  if (e >= n4) return;
  const long long base4 = (long long)pi.koff * a.d / 4;
  const long long stride4 = (long long)a.ktot * a.d / 4;
  f32x4* Pd = reinterpret_cast<f32x4*>(a.p) + base4;
  f32x4 pv;
  if (st->trials == 0) {   // once per iteration
    const int m = st->count;
    const f32x4* G = reinterpret_cast<const f32x4*>(a.g) + base4;
    const f32x4* S = reinterpret_cast<const f32x4*>(a.S) + base4;
    const f32x4* Yv = reinterpret_cast<const f32x4*>(a.Yh) + base4;
    f32x4 acc = G[e] * (float)st->coef_g;
    for (int t = 0; t < m; ++t) {
      const int j = st->order[t];
      acc += S[(size_t)j * stride4 + e] * (float)st->cs[j] + Yv[(size_t)j * stride4 + e] * (float)st->cy[j];
    }
    Pd[e] = acc;
    pv = acc;
  } else {
    pv = Pd[e];
  }
  // trial keys at the current step (the same fma the accepted step applies)
  const float alpha = (float)st->alpha;
  const f32x4 xv = reinterpret_cast<const f32x4*>(a.x)[base4 + e];
  f32x4 kv;
  kv.x = __fmaf_rn(alpha, pv.x, xv.x);
  kv.y = __fmaf_rn(alpha, pv.y, xv.y);
  kv.z = __fmaf_rn(alpha, pv.z, xv.z);
  kv.w = __fmaf_rn(alpha, pv.w, xv.w);
  reinterpret_cast<f32x4*>(a.kt)[base4 + e] = kv;
}

void launch_direction(const DirArgs& a, hipStream_t s) {
  dim3 grid(a.nch, a.P);
  hipLaunchKernelGGL(direction_kernel, grid, dim3(256), 0, s, a);
}

// --------------------------------------------------------------------------
__global__ void state_init_kernel(LbState* st, int P, int clear) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= P) return;
  st[p].status = ST_READY;
  st[p].trials = 0;
  st[p].alpha = 0.0;
  st[p].iter = 0;
  if (clear) {
    st[p].count = 0;
    st[p].stage = 0;
    st[p].flags = 0;
    st[p].n_trial = 0;
    st[p].n_accept = 0;
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
