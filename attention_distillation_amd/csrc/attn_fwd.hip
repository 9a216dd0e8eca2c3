// Forward attention over compressed (or compress-zone) keys, gfx950.
//
// One workgroup = 4 wave64s = 64 training queries of one problem and one
// chunk of its keys.  Each wave owns 16 queries: their rows stay in VGPRs as
// the B operand of S^T = K Q^T (16x16x4 MFMA, keys as rows), so the score
// tile comes out with one query per lane column, which is exactly the B
// operand layout that O^T += V^T P^T needs next.  K and V tiles (64 keys)
// are staged in LDS; V transposed, with the key order inside each 16-key
// block permuted to match the score layout of the MFMA variant in use.
//
// Scores (logits) run on fp32 MFMA, on fp64 MFMA, or as exact integer
// products on int8 MFMA, and are shifted by a per-row value (the target
// log-sum-exp) in fp64 before rounding to fp32: the stored
// St = scale*q.k - shift keeps small magnitudes, so the exp() of later
// kernels sees a well-conditioned argument.  Softmax is online (running max
// per query, per-lane partial sums), partial O / max / sum per key chunk are
// merged by merge_kernel.
//
// Integer scores.  Every query row and key row is scaled by a power of two
// 2^-e (e: the exponent of its largest magnitude, so each scaled element x
// lies in (-1, 1)) and written as five base-128 digits of its magnitude,
// each carrying the element's sign,
//     x = sign(x) (a_0/128 + a_1/128^2 + ... + a_4/128^5 + r),   0 <= r < 128^-5,
// a_0..a_4 in [0, 127], so every signed digit fits int8 (peeling the digits
// of |x| is exact: the fraction of a non-negative float is representable,
// which a floor of a negative value close to zero would not keep).  Then
//     sum_j x_j y_j = sum_{s,t} 128^-(s+t+2) sum_j a_s,j b_t,j + O(128^-5),
// every digit product sum_j a_s,j b_t,j is an int8 MFMA with exact int32
// accumulation, products of one weight s + t share an accumulator, and the
// 19 products with s + t <= 5 are kept (the dropped ones add less than
// 2^-33 * 2^(e_q + e_k) at d = 128).  The sums are combined in fp64 and
// scaled by 2^(e_q + e_k), so a score carries only the truncation of each
// input element below 2^-35 of its row's largest magnitude: far below the
// accumulation rounding of fp32 MFMA, whose error grows with the partial
// sums of the outlier channels.  (The splitting of floating-point products
// into exact integer ones is the scheme of Ozaki, Ogita, Oishi and Rump.)
#include "kvs_internal.h"

namespace kvs {

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f64x4 mfma_f64(double a, double b, f64x4 c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}
// 16x16x64 int8 product: lane (g, lq) supplies row lq of A and column lq of
// B, bytes b of both being the same contraction index (any order that A and
// B share), and receives C[4 g + r][lq]
__device__ __forceinline__ i32x4 mfma_i8(i32x4 a, i32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// The five digits of t = x * 128 (|t| < 128), each with the sign of t,
// packed into byte c of w[0..4].
__device__ __forceinline__ void put_digits(float t, int c, unsigned (&w)[kDigits]) {
  const bool neg = t < 0.f;
  float u = fabsf(t);
#pragma unroll
  for (int s = 0; s < kDigits; ++s) {
    const float a = floorf(u);
    const int q = (int)a;
    w[s] |= ((unsigned)(neg ? -q : q) & 0xffu) << (8 * c);
    u = (u - a) * 128.f;
  }
}

// Byte order of a row's digits, shared by the key planes and the query
// operands: the 16-byte chunk 4 h + g holds dims 16 (4 h + j) + 4 g + c at
// byte 4 j + c (j, c = 0..3), which is what lane group g supplies to the
// integer product over dims 64 h .. 64 h + 63.  Dword of the four dims
// 4 c4 .. 4 c4 + 3 inside a row:
__device__ __forceinline__ int digit_dword(int c4) {
  const int j = c4 >> 2, g = c4 & 3;
  return (4 * (j >> 2) + g) * 4 + (j & 3);
}

// One thread per float4 of X (D / 4 threads per row, consecutive lanes):
// the row's largest magnitude by lane exchange, its exponent e (that
// magnitude < 2^e; 0 for a zero row), the digits of x = X * 2^-e into the
// five planes, and scl = 2^e (NaN if the row has a non-finite element).
template <int D>
__global__ __launch_bounds__(256) void digit_rows_kernel(const float* X, long long rows, int* planes, float* scl) {
  const long long i4 = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = i4 / (D / 4);
  const int c4 = (int)(i4 % (D / 4));
  const bool ok = row < rows;
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  if (ok) v = reinterpret_cast<const f32x4*>(X)[i4];
  float m = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  int bad = !(isfinite(v.x) && isfinite(v.y) && isfinite(v.z) && isfinite(v.w));
#pragma unroll
  for (int o = 1; o < D / 4; o <<= 1) {
    m = fmaxf(m, __shfl_xor(m, o));
    bad |= __shfl_xor(bad, o);
  }
  int e = 0;
  if (!bad) frexpf(m, &e);
  unsigned w[kDigits] = {0u, 0u, 0u, 0u, 0u};
  if (!bad) {
#pragma unroll
    for (int c = 0; c < 4; ++c) put_digits(ldexpf(v[c], 7 - e), c, w);
  }
  if (ok) {
    const int dw = digit_dword(c4);
#pragma unroll
    for (int s = 0; s < kDigits; ++s) planes[((size_t)s * rows + row) * (D / 4) + dw] = (int)w[s];
    if (c4 == 0) scl[row] = bad ? __builtin_nanf("") : ldexpf(1.f, e);
  }
}

void launch_digit_rows(const float* X, long long rows, int d, int* planes, float* scl, hipStream_t s) {
  const long long n4 = rows * (d / 4);
  if (n4 <= 0) return;
  dim3 grid((unsigned)((n4 + 255) / 256));
  if (d == 128) hipLaunchKernelGGL((digit_rows_kernel<128>), grid, dim3(256), 0, s, X, rows, planes, scl);
  else hipLaunchKernelGGL((digit_rows_kernel<64>), grid, dim3(256), 0, s, X, rows, planes, scl);
}

// Key (row) index held in register r by lane group g of a 16x16 MFMA result.
template <bool F64>
__device__ __forceinline__ constexpr int out_row(int g, int r) {
  return F64 ? (g + 4 * r) : (4 * g + r);
}
// LDS column of key kk (0..15) inside its 16-key block of the transposed V
// tile, so that lane group g finds its four keys (r = 0..3) contiguous.
template <bool F64>
__device__ __forceinline__ int vt_col(int kk) {
  return F64 ? ((kk & 3) * 4 + (kk >> 2)) : kk;
}

// V staging: a quad of lanes covers dims 4 c4 .. 4 c4 + 3 of four keys of one
// 16-key block (group vg: block vg / 4, slot vg % 4).  The keys are the four
// that vt_col places in consecutive LDS columns, so each lane writes one
// 16-byte row segment of Vt.
template <bool F64>
__device__ __forceinline__ int vt_key(int vg, int j) {
  return 16 * (vg >> 2) + (F64 ? (vg & 3) + 4 * j : 4 * (vg & 3) + j);
}

template <int D, bool STORE, int SM>
// waves_per_eu(2): at least two waves per SIMD, whose register budget the
// interleaved score accumulators of d = 128 fill (its LDS tiles allow two
// workgroups per CU)
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attn_fwd_kernel(FwdArgs a) {
  // score arithmetic; the integer scores come out in the fp32 product's layout
  constexpr bool F64 = SM == LOGIT_F64, I8 = SM == LOGIT_I8;
  // grid row -> problem: largest k first (a workgroup's work grows with k)
  const int p = a.info ? a.info[blockIdx.y].korder : (int)blockIdx.y;
  const int c = blockIdx.z;
  // the problem table and the state are read before the status test, which
  // uses both, so the two loads share one round trip
  int k, koff;
  long long soff;
  if (a.info) {
    k = a.info[p].k; koff = a.info[p].koff; soff = a.info[p].soff;
  } else {
    k = a.kuni; koff = p * a.kuni; soff = 0;
  }
  if (a.st && (!((1 << a.st[p].status) & a.active_mask) || k < 0)) return;
  const int n = a.n;
  const int npad = (n + 3) & ~3;
  const int chunk = (((k + a.C - 1) / a.C) + 63) & ~63;
  const int kbeg = c * chunk;
  const int kend = min(k, kbeg + chunk);

  __shared__ float Ks[I8 ? 1 : 64][D + 4];
  __shared__ float Vt[D][64 + 4];
  // integer scores: the key tile's digit planes (a row's D bytes with its
  // 16-byte chunks permuted by the row, so that the 16 rows one lane group
  // reads fall in distinct banks) and the keys' scales
  __shared__ __align__(16) int Ks8[I8 ? kDigits : 1][I8 ? 64 : 1][D / 4];
  __shared__ __align__(16) float Kscl[I8 ? 64 : 4];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, lq = lane & 15;
  const int q = blockIdx.x * 64 + wave * 16 + lq;
  const bool qok = q < n;
  const size_t prow = (size_t)p * n;

  // query rows as MFMA B operand: lane (g, lq) holds dims 16j+4g..+3 of query lq
  float qf[D / 4];
#pragma unroll
  for (int j = 0; j < D / 16; ++j) {
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (qok) v = *(const f32x4*)(a.Q + (prow + q) * D + 16 * j + 4 * g);
    qf[4 * j + 0] = v.x; qf[4 * j + 1] = v.y; qf[4 * j + 2] = v.z; qf[4 * j + 3] = v.w;
  }
  // fp64 query operands of the score MFMA, converted once
  double qd[F64 ? D / 4 : 1];
  if constexpr (F64) {
#pragma unroll
    for (int i = 0; i < D / 4; ++i) qd[i] = (double)qf[i];
  }
  // integer scores: this lane's query digits as B operands (digit s, dims
  // 64 h .. 64 h + 63 in the shared byte order: dword j of half h holds dims
  // 16 (4 h + j) + 4 g + c, i.e. qf[16 h + 4 j + c]) and the query's factor
  // scale * 2^(e_q - 49); a query with a non-finite element gets NaN scores
  i32x4 qb[I8 ? kDigits : 1][I8 ? D / 64 : 1];
  double qfac = 0.0;
  if constexpr (I8) {
    float m = 0.f;
    int bad = 0;
#pragma unroll
    for (int i = 0; i < D / 4; ++i) {
      m = fmaxf(m, fabsf(qf[i]));
      bad |= !isfinite(qf[i]);
    }
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    bad |= __shfl_xor(bad, 16);
    bad |= __shfl_xor(bad, 32);
    int e = 0;
    if (!bad) frexpf(m, &e);
#pragma unroll
    for (int h = 0; h < D / 64; ++h)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        unsigned w[kDigits] = {0u, 0u, 0u, 0u, 0u};
        if (!bad) {
#pragma unroll
          for (int c = 0; c < 4; ++c) put_digits(ldexpf(qf[16 * h + 4 * j + c], 7 - e), c, w);
        }
#pragma unroll
        for (int sd = 0; sd < kDigits; ++sd) qb[sd][h][j] = (int)w[sd];
      }
    qfac = bad ? __builtin_nan("") : ldexp(a.scale, e - 49);
  }
  const double shift = (a.shift && qok) ? (double)a.shift[prow + q] : 0.0;

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 oacc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // K/V tile staging, pipelined over the two phases of a tile: the next
  // tile's K is loaded into registers during this tile's score products and
  // written to LDS once every wave has finished reading K; its V is loaded
  // during the P V products and written once every wave has finished reading
  // V.  Two barriers per tile separate the phases, and only LDS stores sit
  // between them.  The loads go through buffer resources that end at kend:
  // rows past kend read zero, their scores are replaced by -inf, so their
  // softmax weights are exactly zero and the values they carry never count.
  // Every load of a thread uses one lane offset: K batch u (RPU rows) has a
  // resource of its own, V batch u is an immediate offset.  Each resource
  // covers one tile (or batch), so its range stays far below 2^31 bytes.
  constexpr int NL = 64 * (D / 4) / 256;     // float4 of K (and V) per thread per tile
  constexpr int RPU = 1024 / D;              // K rows per batch of 256 float4
  const float* Kp = a.K + (size_t)koff * D;
  const float* Vp = a.V + (size_t)koff * D;
  const int k_lane = ((tid / (D / 4)) * D + 4 * (tid % (D / 4))) * 4;
  auto load_k = [&](int kt, f32x4 (&kr)[NL]) {
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int r0 = kt + RPU * u;
      kr[u] = buf_load4(buf_rsrc(Kp + (size_t)r0 * D, (long long)min(RPU, kend - r0) * D * 4), k_lane);
    }
  };
  auto store_k = [&](const f32x4 (&kr)[NL]) {
#pragma unroll
    for (int u = 0; u < NL; ++u) *(f32x4*)&Ks[RPU * u + tid / (D / 4)][4 * (tid % (D / 4))] = kr[u];
  };
  // integer scores: 16-byte chunk u of a thread is chunk tid % (D / 16) of
  // row r of digit plane s (a plane's tile is 64 rows of D bytes, one
  // resource per plane over the tile's rows; rows past kend read zero), and
  // the first 64 threads take the keys' scales
  constexpr int CPP = 64 * (D / 16) / 256;   // chunks per thread per plane
  constexpr int NL8 = kDigits * CPP;
  const int ch8 = tid % (D / 16);
  auto k8_row = [&](int u) { return (tid + 256 * (u % CPP)) / (D / 16); };
  auto load_k8 = [&](int kt, i32x4 (&kr)[NL8], float& ks) {
    const long long rows = min(64, kend - kt);
#pragma unroll
    for (int sd = 0; sd < kDigits; ++sd) {
      const auto rK = buf_rsrc(a.K8 + ((size_t)sd * a.k8rows + koff + kt) * (D / 4), rows * D);
#pragma unroll
      for (int v = 0; v < CPP; ++v) kr[sd * CPP + v] = buf_load4i(rK, k8_row(v) * D + 16 * ch8);
    }
    if (tid < 64) ks = buf_load1(buf_rsrc(a.Kscl + koff + kt, rows * 4), tid * 4);
  };
  auto store_k8 = [&](const i32x4 (&kr)[NL8], float ks) {
#pragma unroll
    for (int u = 0; u < NL8; ++u) {
      const int r = k8_row(u);
      *(i32x4*)&Ks8[u / CPP][r][4 * (ch8 ^ ((r / (256 / D)) & (D / 16 - 1)))] = kr[u];
    }
    if (tid < 64) Kscl[tid] = ks;
  };
  // V: wave w stages keys 16 w .. 16 w + 15, lane l key 16 w + (l & 15) and
  // dims 16 u + 4 (l >> 4) .. + 3 of batch u (one 16-byte load); the four
  // floats go to the four Vt rows of those dims, in the column that vt_col
  // gives the key (the 64 lanes of each store hit 64 different banks)
  const int v_key = 16 * (tid >> 6) + (lane & 15);
  const int v_lane = (v_key * D + 4 * (lane >> 4)) * 4;
  const int v_col = 16 * (tid >> 6) + vt_col<F64>(lane & 15);
  auto load_v = [&](int kt, f32x4 (&vr)[NL]) {
    const auto rV = buf_rsrc(Vp + (size_t)kt * D, (long long)min(64, kend - kt) * D * 4);
#pragma unroll
    for (int u = 0; u < NL; ++u) vr[u] = buf_load4(rV, v_lane + 64 * u);
  };
  auto store_v = [&](const f32x4 (&vr)[NL]) {
#pragma unroll
    for (int u = 0; u < NL; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) Vt[16 * u + 4 * (lane >> 4) + j][v_col] = vr[u][j];
  };
  // stored scores: row (key) kt + 16 b + out_row(g, r) of this lane's query;
  // the lane's part of the byte offset is fixed, the row part is uniform
  const int st_lane = ((F64 ? g : 4 * g) * npad + q) * 4;
  f32x4 kpre[NL], vpre[NL];
  i32x4 kpre8[I8 ? NL8 : 1];
  float kspre = 0.f;
  if (kbeg < kend) {
    if constexpr (I8) load_k8(kbeg, kpre8, kspre);
    else load_k(kbeg, kpre);
    load_v(kbeg, vpre);
    if constexpr (I8) store_k8(kpre8, kspre);
    else store_k(kpre);
    store_v(vpre);
  }
  __syncthreads();
  for (int kt = kbeg; kt < kend; kt += 64) {
    const bool more = kt + 64 < kend;
    const bool tail = !more && kt + 64 > kend;   // the chunk's last tile may hold keys past kend
    if (more) {
      if constexpr (I8) load_k8(kt + 64, kpre8, kspre);
      else load_k(kt + 64, kpre);
    }

    float sv[4][4];
    if constexpr (I8) {
      // per 16-key block: the 19 digit products into six accumulators by
      // weight s + t, pairs of weights joined exactly in int32 (each below
      // 2^31), the three pairs in fp64, then the scale 2^(e_q + e_k - 49)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        i32x4 acc[6];
#pragma unroll
        for (int w = 0; w < 6; ++w) acc[w] = i32x4{0, 0, 0, 0};
        const int row = 16 * b + lq;
#pragma unroll
        for (int h = 0; h < D / 64; ++h) {
          const int ch = (4 * h + g) ^ ((row / (256 / D)) & (D / 16 - 1));
#pragma unroll
          for (int sd = 0; sd < kDigits; ++sd) {
            const i32x4 av = *(const i32x4*)&Ks8[sd][row][4 * ch];
#pragma unroll
            for (int t = 0; t < kDigits; ++t)
              if (sd + t <= 5) acc[sd + t] = mfma_i8(av, qb[t][h], acc[sd + t]);
          }
        }
        const f32x4 ks = *(const f32x4*)&Kscl[16 * b + 4 * g];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int hi = acc[0][r] * 128 + acc[1][r];
          const int mid = acc[2][r] * 128 + acc[3][r];
          const int lo = acc[4][r] * 128 + acc[5][r];
          const double v = fma(fma((double)hi, 16384.0, (double)mid), 16384.0, (double)lo);
          sv[b][r] = (float)fma(v, qfac * (double)ks[r], -shift);
        }
      }
    } else if constexpr (F64) {
      // the four 16-key blocks' score products interleaved: each column
      // group of K is read from LDS once for 16 products (3% faster than
      // block by block on the long-context heads)
      f64x4 acc[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) acc[w] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int j = 0; j < D / 16; ++j) {
        f32x4 kv[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) kv[w] = *(const f32x4*)&Ks[16 * w + lq][16 * j + 4 * g];
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int w = 0; w < 4; ++w) acc[w] = mfma_f64((double)kv[w][c], qd[4 * j + c], acc[w]);
      }
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int r = 0; r < 4; ++r) sv[w][r] = (float)(acc[w][r] * a.scale - shift);
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if constexpr (!F64 && !I8) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < D / 16; ++j) {
          const f32x4 kv = *(const f32x4*)&Ks[16 * b + lq][16 * j + 4 * g];
          acc = mfma_f32(kv.x, qf[4 * j + 0], acc);
          acc = mfma_f32(kv.y, qf[4 * j + 1], acc);
          acc = mfma_f32(kv.z, qf[4 * j + 2], acc);
          acc = mfma_f32(kv.w, qf[4 * j + 3], acc);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) sv[b][r] = (float)((double)acc[r] * a.scale - shift);
      }
    }
    // the scores of the tile's keys go to St (queries past n have no row);
    // keys past kend are not stored and get -inf
    if (STORE && qok) {
      const auto rSt = buf_rsrc(a.St + soff + (size_t)kt * npad, (long long)min(64, kend - kt) * npad * 4);
      if (!tail) {
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r) buf_store1(rSt, st_lane, (16 * b + (F64 ? 4 * r : r)) * npad * 4, sv[b][r]);
      } else {
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (kt + 16 * b + out_row<F64>(g, r) < kend)
              buf_store1(rSt, st_lane, (16 * b + (F64 ? 4 * r : r)) * npad * 4, sv[b][r]);
      }
    }
    if (tail) {
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (kt + 16 * b + out_row<F64>(g, r) >= kend) sv[b][r] = -INFINITY;
    }
    __syncthreads();   // every wave is done with this tile's K
    if (more) {
      if constexpr (I8) store_k8(kpre8, kspre);
      else store_k(kpre);
      load_v(kt + 64, vpre);
    }

    float tmax = sv[0][0];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, sv[b][r]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);   // finite: the tile holds a valid key
    // The running sums are rescaled only when some query's maximum moved (a
    // factor of exactly 1 elsewhere); exponentials in the hardware exp2 form
    // of arguments relative to the running maximum, so only weights far below
    // the largest carry its product rounding.
    if (__builtin_amdgcn_ballot_w64(m_new != m_run)) {
      const float corr = __expf(m_run - m_new);
      l_run *= corr;
#pragma unroll
      for (int i = 0; i < D / 16; ++i) oacc[i] *= corr;
    }
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sv[b][r] = __expf(sv[b][r] - m_new);
        l_run += sv[b][r];
      }
    m_run = m_new;

#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        const f32x4 vv = *(const f32x4*)&Vt[16 * db + lq][16 * b + 4 * g];
        oacc[db] = mfma_f32(vv.x, sv[b][0], oacc[db]);
        oacc[db] = mfma_f32(vv.y, sv[b][1], oacc[db]);
        oacc[db] = mfma_f32(vv.z, sv[b][2], oacc[db]);
        oacc[db] = mfma_f32(vv.w, sv[b][3], oacc[db]);
      }
    __syncthreads();   // every wave is done with this tile's V (and the next K is in)
    if (more) store_v(vpre);
  }

  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (qok) {
    const size_t orow = (size_t)c * a.P * n + prow + q;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) *(f32x4*)(a.Opart + orow * D + 16 * db + 4 * g) = oacc[db];
    if (g == 0) {
      a.Mpart[orow] = m_run;
      a.Lpart[orow] = l_run;
    }
  }
}

// Forward at keys whose shifted scores are already stored: the keys have not
// moved since the forward that stored them, only the values have (the loss
// after a value re-solve).  The scores are read from St instead of formed on
// MFMA; staging, softmax and P V are the forward's, in the same layout (F64:
// the layout of the fp64 score product).  A stored score is exactly the float
// that product rounded to, so the partials equal the full forward's bit for bit.
template <int D, bool F64>
__global__ __launch_bounds__(256) void attn_pv_kernel(FwdArgs a) {
  const int p = a.info[blockIdx.y].korder, c = blockIdx.z;   // largest k first
  const int k = a.info[p].k, koff = a.info[p].koff;
  const long long soff = a.info[p].soff;
  if (a.st && (!((1 << a.st[p].status) & a.active_mask) || k < 0)) return;
  const int n = a.n;
  const int npad = (n + 3) & ~3;
  const int chunk = (((k + a.C - 1) / a.C) + 63) & ~63;
  const int kbeg = c * chunk;
  const int kend = min(k, kbeg + chunk);

  __shared__ float Vt[D][64 + 4];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, lq = lane & 15;
  const int q = blockIdx.x * 64 + wave * 16 + lq;
  const bool qok = q < n;
  const size_t prow = (size_t)p * n;

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 oacc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int NL = 64 * (D / 4) / 256;     // float4 of V per thread per tile
  const float* Vp = a.V + (size_t)koff * D;
  // this lane's scores: fixed lane part of the byte offset, uniform row part
  const int st_lane = ((F64 ? g : 4 * g) * npad + q) * 4;
  for (int kt = kbeg; kt < kend; kt += 64) {
    const long long rows = min(64, kend - kt);
    const auto rS = buf_rsrc(a.Sload + soff + (size_t)kt * npad, rows * npad * 4);
    const auto rV = buf_rsrc(Vp + (size_t)kt * D, rows * D * 4);
    const bool tail = kt + 64 > kend;
    // this lane's scores (query q, keys of the score layout); rows past kend
    // are -inf, queries past n 0 (as the forward forms them), neither is
    // loaded.  The bound between the PV products and these loads is the MFMA
    // work and the partial outputs, not the scores' 64-byte segments.
    float sv[4][4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (tail && kt + 16 * b + out_row<F64>(g, r) >= kend) sv[b][r] = -INFINITY;
        else sv[b][r] = qok ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                  rS, st_lane, (16 * b + (F64 ? 4 * r : r)) * npad * 4, 0))
                            : 0.f;
      }
    __syncthreads();
    // V rows past kend read zero (their weights are exactly zero)
    f32x4 vv[NL];
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int i = tid + 256 * u;
      const int q4 = i >> 2, vg = q4 / (D / 4), dim = 4 * (q4 % (D / 4)) + (i & 3);
#pragma unroll
      for (int j = 0; j < 4; ++j) vv[u][j] = buf_load1(rV, (vt_key<F64>(vg, j) * D + dim) * 4);
    }
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int i = tid + 256 * u;
      const int q4 = i >> 2, vg = q4 / (D / 4), dim = 4 * (q4 % (D / 4)) + (i & 3);
      *(f32x4*)&Vt[dim][16 * (vg >> 2) + 4 * (vg & 3)] = vv[u];
    }
    __syncthreads();

    float tmax = sv[0][0];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, sv[b][r]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);   // finite: the tile holds a valid key
    // The running sums are rescaled only when some query's maximum moved (a
    // factor of exactly 1 elsewhere); exponentials in the hardware exp2 form
    // of arguments relative to the running maximum, so only weights far below
    // the largest carry its product rounding.
    if (__builtin_amdgcn_ballot_w64(m_new != m_run)) {
      const float corr = __expf(m_run - m_new);
      l_run *= corr;
#pragma unroll
      for (int i = 0; i < D / 16; ++i) oacc[i] *= corr;
    }
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sv[b][r] = __expf(sv[b][r] - m_new);
        l_run += sv[b][r];
      }
    m_run = m_new;

#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        const f32x4 vv4 = *(const f32x4*)&Vt[16 * db + lq][16 * b + 4 * g];
        oacc[db] = mfma_f32(vv4.x, sv[b][0], oacc[db]);
        oacc[db] = mfma_f32(vv4.y, sv[b][1], oacc[db]);
        oacc[db] = mfma_f32(vv4.z, sv[b][2], oacc[db]);
        oacc[db] = mfma_f32(vv4.w, sv[b][3], oacc[db]);
      }
  }

  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (qok) {
    const size_t orow = (size_t)c * a.P * n + prow + q;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) *(f32x4*)(a.Opart + orow * D + 16 * db + 4 * g) = oacc[db];
    if (g == 0) {
      a.Mpart[orow] = m_run;
      a.Lpart[orow] = l_run;
    }
  }
}

void launch_attn_fwd(const FwdArgs& a, int d, int logit_mode, hipStream_t s) {
  dim3 grid((a.n + 63) / 64, a.P, a.C);
  if (a.Sload) {
    // the stored scores are in the layout of the product that formed them
    const bool f64 = logit_mode == LOGIT_F64;
#define KVS_PV(DD, FF) hipLaunchKernelGGL((attn_pv_kernel<DD, FF>), grid, dim3(256), 0, s, a)
    if (d == 128) { if (f64) KVS_PV(128, true); else KVS_PV(128, false); }
    else { if (f64) KVS_PV(64, true); else KVS_PV(64, false); }
#undef KVS_PV
    return;
  }
  const bool store = a.St != nullptr;
#define KVS_FWD(DD, SS, MM) hipLaunchKernelGGL((attn_fwd_kernel<DD, SS, MM>), grid, dim3(256), 0, s, a)
#define KVS_FWD_M(DD, SS)                                           \
  do {                                                              \
    if (logit_mode == LOGIT_I8) KVS_FWD(DD, SS, LOGIT_I8);          \
    else if (logit_mode == LOGIT_F64) KVS_FWD(DD, SS, LOGIT_F64);   \
    else KVS_FWD(DD, SS, LOGIT_F32);                                \
  } while (0)
  if (d == 128) {
    if (store) KVS_FWD_M(128, true);
    else KVS_FWD_M(128, false);
  } else {
    if (store) KVS_FWD_M(64, true);
    else KVS_FWD_M(64, false);
  }
#undef KVS_FWD_M
#undef KVS_FWD
}

// --------------------------------------------------------------------------
// merge of key-chunk partials + epilogue.  16 queries per workgroup, 16
// threads per query, each owning d/16 consecutive dims.
//   reference mode: Y = O, lse = m + log l
//   loss mode (scores were shifted by the target lse, so m + log l = lhat - l):
//     R = O - Y, G = 2R, e = lhat - l, crow = -G.O + 2 lam e,
//     per-WG partials of sum(R^2) + lam sum(e^2) and of sum(R^2); the last
//     workgroup of a problem (arrival counter) sums them in block order and
//     finalises: loss / mse outputs, or the Armijo test of a line-search trial.

// Fixed-order sum of the per-block partials, then the per-problem decision.
template <int D>
__device__ void finalize_problem(const MergeArgs& a, int p, int nblk) {
  __shared__ double r0[4], r1[4];
  const int t = threadIdx.x;
  double sL = 0.0, sO = 0.0;
  for (int i = t; i < nblk; i += 256) {
    const double* src = a.part + ((size_t)p * nblk + i) * 2;
    sL += coherent_load(src);
    sO += coherent_load(src + 1);
  }
  // fixed xor tree within each wave, then the four waves in order
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    sL += __shfl_xor(sL, off);
    sO += __shfl_xor(sO, off);
  }
  if ((t & 63) == 0) {
    r0[t >> 6] = sL;
    r1[t >> 6] = sO;
  }
  __syncthreads();
  if (t != 0) return;
  sL = ((r0[0] + r0[1]) + r0[2]) + r0[3];
  sO = ((r1[0] + r1[1]) + r1[2]) + r1[3];
  LbState* st = a.st ? a.st + p : nullptr;
  if (a.fin_mode == 1) {
    st->Ltrial = sL;
    st->n_trial += 1;
    if (sL <= st->L + a.c1 * st->alpha * st->gtp) {
      st->n_accept += 1;
      st->status = ST_ACCEPT;
      st->L = sL;
      st->st_valid = 1;
    } else {
      st->st_valid = 0;
      st->trials += 1;
      st->alpha *= a.shrink;
      if (st->trials >= a.max_bt) st->status = ST_FAIL;
    }
    if (a.status_view) a.status_view[p] = st->status;
  } else {
    if (st) {
      st->L = sL;
      st->st_valid = 1;
    }
    if (a.loss) a.loss[p] = (float)sL;
    if (a.mse) a.mse[p] = (float)(sO / ((double)a.n * (double)D));
  }
}

// waves_per_eu: let the scheduler keep the batched loads in flight instead
// of trading them for occupancy
template <int D, bool LOSS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 4))) void merge_kernel(MergeArgs a) {
  const int p = blockIdx.y;
  if (a.st && !((1 << a.st[p].status) & a.active_mask)) return;
  constexpr int DPT = D / 16;
  const int tid = threadIdx.x, qi = tid >> 4, part = tid & 15;
  const int n = a.n;
  const int q = blockIdx.x * 16 + qi;
  const bool ok = q < n;
  const size_t row = (size_t)p * n + q;
  const size_t plane = (size_t)a.P * n;

  // all chunk maxima and sums first, then the partial outputs four chunks at
  // a time; loads are branch-free (rows past n read row 0 and are dropped).
  // The targets of the loss are loaded first so their latency overlaps the
  // partials'.
  const size_t rrow = ok ? row : (size_t)p * n;
  f32x4 yv[DPT / 4];
  if constexpr (LOSS) {
    const float* y = a.Y + rrow * D + part * DPT;
#pragma unroll
    for (int i = 0; i < DPT / 4; ++i) yv[i] = *(const f32x4*)(y + 4 * i);
  }
  float m, l;
  float o[DPT];
  if (a.C == 1) {
    // one chunk: its output is already merged (the general path would scale
    // it by exp(0) = 1, so the result is the same bit for bit)
    m = a.Mpart[rrow];
    l = a.Lpart[rrow];
    const float* src = a.Opart + rrow * D + part * DPT;
#pragma unroll
    for (int i = 0; i < DPT / 4; ++i) {
      const f32x4 v = *(const f32x4*)(src + 4 * i);
      o[4 * i + 0] = v.x; o[4 * i + 1] = v.y; o[4 * i + 2] = v.z; o[4 * i + 3] = v.w;
    }
  } else {
    float mv[kMaxChunks], lv[kMaxChunks];
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      const size_t off = (c < a.C ? c : 0) * plane + rrow;
      mv[c] = a.Mpart[off];
      lv[c] = a.Lpart[off];
    }
    m = -INFINITY;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c)
      if (c < a.C) m = fmaxf(m, mv[c]);
    l = 0.f;
#pragma unroll
    for (int i = 0; i < DPT; ++i) o[i] = 0.f;
#pragma unroll
    for (int c0 = 0; c0 < kMaxChunks; c0 += 4) {
      if (c0 >= a.C) break;
      f32x4 ov[4][DPT / 4];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const int c = c0 + cc < a.C ? c0 + cc : 0;
        const float* src = a.Opart + (c * plane + rrow) * D + part * DPT;
#pragma unroll
        for (int i = 0; i < DPT / 4; ++i) ov[cc][i] = *(const f32x4*)(src + 4 * i);
      }
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const int c = c0 + cc;
        const float w = (c < a.C) ? expf(mv[c] - m) : 0.f;
        l += w * ((c < a.C) ? lv[c] : 0.f);
#pragma unroll
        for (int i = 0; i < DPT / 4; ++i) {
          o[4 * i + 0] += w * ov[cc][i].x; o[4 * i + 1] += w * ov[cc][i].y;
          o[4 * i + 2] += w * ov[cc][i].z; o[4 * i + 3] += w * ov[cc][i].w;
        }
      }
    }
  }
  const float inv = ok ? 1.f / l : 0.f;
#pragma unroll
  for (int i = 0; i < DPT; ++i) o[i] *= inv;
  const float lse = ok ? m + logf(l) : 0.f;

  if constexpr (!LOSS) {
    if (ok) {
      float* dst = a.Yout + row * D + part * DPT;
#pragma unroll
      for (int i = 0; i < DPT; i += 4) *(f32x4*)(dst + i) = f32x4{o[i], o[i + 1], o[i + 2], o[i + 3]};
      if (part == 0) a.lse_out[row] = lse;
    }
  } else {
    __shared__ double red[2][4];
    __shared__ int s_last;
    float rr = 0.f, dl = 0.f;
    if (ok) {
      float* gout = a.G + row * D + part * DPT;
#pragma unroll
      for (int i = 0; i < DPT; i += 4) {
        const f32x4 y4 = yv[i / 4];
        f32x4 gv;
        const float r0 = o[i] - y4.x, r1 = o[i + 1] - y4.y, r2 = o[i + 2] - y4.z, r3 = o[i + 3] - y4.w;
        rr += r0 * r0 + r1 * r1 + r2 * r2 + r3 * r3;
        gv.x = 2.f * r0; gv.y = 2.f * r1; gv.z = 2.f * r2; gv.w = 2.f * r3;
        dl += gv.x * o[i] + gv.y * o[i + 1] + gv.z * o[i + 2] + gv.w * o[i + 3];
        *(f32x4*)(gout + i) = gv;
      }
    }
    // reduce over the 16 threads of this query (fixed xor tree)
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      rr += __shfl_xor(rr, off);
      dl += __shfl_xor(dl, off);
    }
    const float e = lse;   // lhat - l
    if (ok && part == 0) {
      a.e[row] = e;
      a.crow[row] = -dl + (float)(2.0 * a.lambda) * e;
    }
    // every lane of a query holds its row terms; a wave holds four queries:
    // their sum by two xor steps, then the four waves in order
    double lrow = ok ? (double)rr + a.lambda * (double)e * (double)e : 0.0;
    double orow = ok ? (double)rr : 0.0;
    lrow += __shfl_xor(lrow, 16);
    orow += __shfl_xor(orow, 16);
    lrow += __shfl_xor(lrow, 32);
    orow += __shfl_xor(orow, 32);
    if ((tid & 63) == 0) {
      red[0][tid >> 6] = lrow;
      red[1][tid >> 6] = orow;
    }
    __syncthreads();
    if (tid == 0) {
      double* dst = a.part + ((size_t)p * gridDim.x + blockIdx.x) * 2;
      coherent_store(dst, ((red[0][0] + red[0][1]) + red[0][2]) + red[0][3]);
      coherent_store(dst + 1, ((red[1][0] + red[1][1]) + red[1][2]) + red[1][3]);
      wait_own_stores();
      s_last = arrive_last(a.counter + p, gridDim.x);
    }
    __syncthreads();
    if (!s_last) return;
    finalize_problem<D>(a, p, gridDim.x);
    if (tid == 0) a.counter[p] = 0u;
  }
}

// Loss-mode merge when the forward used one key chunk (its partial output is
// already the merged one): 64 queries per workgroup, the loads of all four
// 16-query groups issued before any use, so a workgroup moves enough bytes to
// cover its fixed cost (status test, partial store, arrival).  The row terms,
// G, e and crow are those of merge_kernel, bit for bit; the loss partials
// are summed over four times fewer, larger blocks.
template <int D>
__global__ __launch_bounds__(256) void merge1_loss_kernel(MergeArgs a) {
  const int p = blockIdx.y;
  if (a.st && !((1 << a.st[p].status) & a.active_mask)) return;
  constexpr int DPT = D / 16, SUB = 4;
  const int tid = threadIdx.x, qi = tid >> 4, part = tid & 15;
  const int n = a.n;
  bool ok[SUB];
  size_t row[SUB];
  float mv[SUB], lv[SUB];
  f32x4 ov[SUB][DPT / 4], yv[SUB][DPT / 4];
#pragma unroll
  for (int u = 0; u < SUB; ++u) {
    const int q = blockIdx.x * 64 + 16 * u + qi;
    ok[u] = q < n;
    row[u] = (size_t)p * n + (ok[u] ? q : 0);
    mv[u] = a.Mpart[row[u]];
    lv[u] = a.Lpart[row[u]];
    const float* src = a.Opart + row[u] * D + part * DPT;
    const float* y = a.Y + row[u] * D + part * DPT;
#pragma unroll
    for (int i = 0; i < DPT / 4; ++i) {
      ov[u][i] = *(const f32x4*)(src + 4 * i);
      yv[u][i] = *(const f32x4*)(y + 4 * i);
    }
  }
  double lsum = 0.0, osum = 0.0;
#pragma unroll
  for (int u = 0; u < SUB; ++u) {
    const float inv = ok[u] ? 1.f / lv[u] : 0.f;
    const float e = ok[u] ? mv[u] + logf(lv[u]) : 0.f;   // lhat - l
    float rr = 0.f, dl = 0.f;
    float* gout = a.G + row[u] * D + part * DPT;
#pragma unroll
    for (int i = 0; i < DPT / 4; ++i) {
      const float o0 = ov[u][i].x * inv, o1 = ov[u][i].y * inv, o2 = ov[u][i].z * inv, o3 = ov[u][i].w * inv;
      const float r0 = o0 - yv[u][i].x, r1 = o1 - yv[u][i].y, r2 = o2 - yv[u][i].z, r3 = o3 - yv[u][i].w;
      rr += r0 * r0 + r1 * r1 + r2 * r2 + r3 * r3;
      f32x4 gv;
      gv.x = 2.f * r0; gv.y = 2.f * r1; gv.z = 2.f * r2; gv.w = 2.f * r3;
      dl += gv.x * o0 + gv.y * o1 + gv.z * o2 + gv.w * o3;
      if (ok[u]) *(f32x4*)(gout + 4 * i) = gv;
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      rr += __shfl_xor(rr, off);
      dl += __shfl_xor(dl, off);
    }
    if (ok[u] && part == 0) {
      a.e[row[u]] = e;
      a.crow[row[u]] = -dl + (float)(2.0 * a.lambda) * e;
    }
    lsum += ok[u] ? (double)rr + a.lambda * (double)e * (double)e : 0.0;
    osum += ok[u] ? (double)rr : 0.0;
  }
  // each lane of a query group holds the group's sums; a wave holds four
  // groups: two xor steps, then the four waves in order
  __shared__ double red[2][4];
  __shared__ int s_last;
  lsum += __shfl_xor(lsum, 16);
  osum += __shfl_xor(osum, 16);
  lsum += __shfl_xor(lsum, 32);
  osum += __shfl_xor(osum, 32);
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = lsum;
    red[1][tid >> 6] = osum;
  }
  __syncthreads();
  if (tid == 0) {
    double* dst = a.part + ((size_t)p * gridDim.x + blockIdx.x) * 2;
    coherent_store(dst, ((red[0][0] + red[0][1]) + red[0][2]) + red[0][3]);
    coherent_store(dst + 1, ((red[1][0] + red[1][1]) + red[1][2]) + red[1][3]);
    wait_own_stores();
    s_last = arrive_last(a.counter + p, gridDim.x);
  }
  __syncthreads();
  if (!s_last) return;
  finalize_problem<D>(a, p, gridDim.x);
  if (tid == 0) a.counter[p] = 0u;
}

int merge_blocks(int n) { return (n + 15) / 16; }

void launch_merge(const MergeArgs& a, int d, bool loss_mode, hipStream_t s) {
  if (loss_mode && a.C == 1) {
    dim3 grid((a.n + 63) / 64, a.P);
    if (d == 128) hipLaunchKernelGGL((merge1_loss_kernel<128>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((merge1_loss_kernel<64>), grid, dim3(256), 0, s, a);
    return;
  }
  dim3 grid(merge_blocks(a.n), a.P);
#define KVS_MERGE(DD, LL) hipLaunchKernelGGL((merge_kernel<DD, LL>), grid, dim3(256), 0, s, a)
  if (d == 128) { if (loss_mode) KVS_MERGE(128, true); else KVS_MERGE(128, false); }
  else { if (loss_mode) KVS_MERGE(64, true); else KVS_MERGE(64, false); }
#undef KVS_MERGE
}

// --------------------------------------------------------------------------
__global__ void fill_i32_kernel(int* p, int v, long long n) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x) p[i] = v;
}
__global__ void fill_f32_kernel(float* p, float v, long long n) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x) p[i] = v;
}
void launch_fill_i32(int* p, int v, long long n, hipStream_t s) {
  if (n <= 0) return;
  int blocks = (int)std::min<long long>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(fill_i32_kernel, dim3(blocks), dim3(256), 0, s, p, v, n);
}
void launch_fill_f32(float* p, float v, long long n, hipStream_t s) {
  if (n <= 0) return;
  int blocks = (int)std::min<long long>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(fill_f32_kernel, dim3(blocks), dim3(256), 0, s, p, v, n);
}

struct InfoChunk {
  int first, count;
  ProbInfo e[48];
};
__global__ void write_info_kernel(ProbInfo* dst, InfoChunk c) {
  const int i = threadIdx.x;
  if (i < c.count) dst[c.first + i] = c.e[i];
}
void launch_write_info(ProbInfo* dst, const ProbInfo* src, int P, hipStream_t s) {
  for (int first = 0; first < P; first += 48) {
    InfoChunk c;
    c.first = first;
    c.count = std::min(48, P - first);
    for (int i = 0; i < c.count; ++i) c.e[i] = src[first + i];
    hipLaunchKernelGGL(write_info_kernel, dim3(1), dim3(64), 0, s, dst, c);
  }
}

}  // namespace kvs
