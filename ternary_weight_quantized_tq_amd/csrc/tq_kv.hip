// TurboQuant-style KV-cache quantiser: quantise K/V rows of dimension 128,
// score queries against quantised keys, and take probability-weighted sums
// of quantised values, all on the packed records.
//
// Source: "Mac users can use TurboQuant in oMLX, with Gemma-4-31B" (aitntnews),
// section "What TurboQuant is and what problem it solves": each KV vector is
// rotated by a random orthogonal matrix and put in polar form with a
// high-precision radius (PolarQuant); a 1-bit Johnson-Lindenstrauss
// projection (QJL) then removes the remaining bias of inner products; the
// method is data-oblivious (no per-block scale).  Section "Why these
// results": decoding costs a coordinate rotation and table lookups.
//
// Readings where the page is silent: d = 128; rotation Pi = H diag(sigma)
// (normalised Sylvester Hadamard after random signs); radius r = |x| in fp16;
// direction u = Pi x / r quantised per coordinate with the Lloyd-Max
// codebook of N(0, 1/d), nearest level, a tie to the lower level; keys keep
// bits - 1 codebook bits and z = sign(S e) of the residual e = u - u~ with
// gamma = |e| in fp16; score = r (<Pi q, u~> + gamma sqrt(pi/2)/d <S Pi q, z>);
// values keep bits codebook bits, v^ = r Pi^T u~.  A record stores the codes
// as packed little-endian fields (code j at bits m j .. m j + m - 1), then
// for keys the 128 bits of z (set where z = +1): 16 bytes per bit of the
// mode in both cases.
#include "tq_internal.h"

#include <limits.h>

#include <cmath>
#include <utility>
#include <vector>

using namespace tq;

namespace {

constexpr int kD = TQ_KV_DIM;
constexpr double kInvSqrtD = 0.08838834764831845;  // 1/sqrt(128)

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------ codebook ---
// The Lloyd-Max levels of N(0, 1) with L = 2^bits levels: each level the
// mean of its nearest-level cell (Lloyd's and Max's optimality conditions).
// By symmetry only the positive half y_1 < ... < y_h (h = L/2) is solved:
// y_j = E[X | a_j < X < b_j] with a_1 = 0, a_j = (y_{j-1} + y_j)/2,
// b_j = (y_j + y_{j+1})/2 and b_h = infinity, by damped Newton steps from
// the companding start (levels at the quantiles of N(0, 3), the asymptotic
// optimum of Panter and Dite).  The Jacobian is tridiagonal: a cell mean m
// moves by phi(a)(m - a)/P with its lower end a and by phi(b)(b - m)/P with
// its upper end b, and each end by half of each neighbouring level's step.
double upper_tail(double x) {
  if (std::isinf(x)) return x > 0 ? 0.0 : 1.0;
  return 0.5 * std::erfc(x / std::sqrt(2.0));
}
double normal_pdf(double x) { return std::isinf(x) ? 0.0 : std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI); }

// x >= 0 with upper_tail(x) = p, 0 < p <= 1/2, by bisection.
double upper_tail_inverse(double p) {
  double lo = 0.0, hi = 40.0;
  for (int i = 0; i < 200; ++i) {
    const double mid = 0.5 * (lo + hi);
    if (upper_tail(mid) > p)
      lo = mid;
    else
      hi = mid;
  }
  return 0.5 * (lo + hi);
}

// Residual f_j = y_j - m_j and the three diagonals of its Jacobian.
double half_residual(const std::vector<double>& y, std::vector<double>* f, std::vector<double>* sub,
                     std::vector<double>* dia, std::vector<double>* sup) {
  const int h = static_cast<int>(y.size());
  double worst = 0.0;
  for (int j = 0; j < h; ++j) {
    const double a = j == 0 ? 0.0 : 0.5 * (y[j - 1] + y[j]);
    const double b = j == h - 1 ? INFINITY : 0.5 * (y[j] + y[j + 1]);
    const double p = upper_tail(a) - upper_tail(b);
    const double m = (normal_pdf(a) - normal_pdf(b)) / p;
    (*f)[j] = y[j] - m;
    worst = std::fmax(worst, std::fabs((*f)[j]));
    if (sub) {
      const double dma = j == 0 ? 0.0 : normal_pdf(a) * (m - a) / p;
      const double dmb = j == h - 1 ? 0.0 : normal_pdf(b) * (b - m) / p;
      (*sub)[j] = -0.5 * dma;
      (*sup)[j] = -0.5 * dmb;
      (*dia)[j] = 1.0 - 0.5 * dma - 0.5 * dmb;
    }
  }
  return worst;
}

bool lloyd_max_half(int h, std::vector<double>* yout) {
  const int levels = 2 * h;
  std::vector<double> y(h), f(h), sub(h), dia(h), sup(h), step(h), trial(h), ftrial(h), cp(h), dp(h);
  for (int j = 0; j < h; ++j) y[j] = std::sqrt(3.0) * upper_tail_inverse(0.5 - (j + 0.5) / levels);
  double res = half_residual(y, &f, &sub, &dia, &sup);
  for (int it = 0; it < 200 && res > 1e-15; ++it) {
    // Thomas algorithm for J step = -f.
    cp[0] = sup[0] / dia[0];
    dp[0] = -f[0] / dia[0];
    for (int j = 1; j < h; ++j) {
      const double den = dia[j] - sub[j] * cp[j - 1];
      cp[j] = sup[j] / den;
      dp[j] = (-f[j] - sub[j] * dp[j - 1]) / den;
    }
    step[h - 1] = dp[h - 1];
    for (int j = h - 2; j >= 0; --j) step[j] = dp[j] - cp[j] * step[j + 1];
    // Halve the step until the levels stay ordered and positive and the
    // residual does not grow.
    double t = 1.0, rt = res;
    for (int k = 0; k < 60; ++k, t *= 0.5) {
      bool ordered = true;
      for (int j = 0; j < h; ++j) {
        trial[j] = y[j] + t * step[j];
        if (trial[j] <= (j ? trial[j - 1] : 0.0)) ordered = false;
      }
      if (!ordered) continue;
      rt = half_residual(trial, &ftrial, nullptr, nullptr, nullptr);
      if (rt <= res || rt < 1e-15) break;
    }
    double moved = 0.0;
    for (int j = 0; j < h; ++j) moved = std::fmax(moved, std::fabs(trial[j] - y[j]));
    y = trial;
    res = half_residual(y, &f, &sub, &dia, &sup);
    if (moved < 1e-16) break;
  }
  for (double v : y)
    if (!std::isfinite(v)) return false;
  *yout = y;
  return res < 1e-12;
}

// ---------------------------------------------------- record fields ---
// Field of W bits at bit offset O of a record held in registers (O and W
// compile-time; a field may straddle two words).
template <int O, int W, int N>
__device__ __forceinline__ uint32_t field(const uint32_t (&w)[N]) {
  constexpr int wi = O / 32, sh = O % 32;
  constexpr uint32_t mask = (1u << W) - 1u;
  if constexpr (sh + W <= 32) {
    return (w[wi] >> sh) & mask;
  } else {
    return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & mask;
  }
}

template <int N>
__device__ __forceinline__ void load_record(const uint32_t* p, uint32_t (&w)[N]) {
#pragma unroll
  for (int i = 0; i < N / 4; ++i) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p) + i);
    w[4 * i] = v.x;
    w[4 * i + 1] = v.y;
    w[4 * i + 2] = v.z;
    w[4 * i + 3] = v.w;
  }
}

__device__ __forceinline__ float half_bits_to_f32(uint16_t b) { return static_cast<float>(__builtin_bit_cast(_Float16, b)); }

// Sum over groups g of tab[g * TE + field g], in group order.
template <int TE, int IB, int O, int N, int... G>
__device__ __forceinline__ float lut_sum(const float* tab, const uint32_t (&w)[N], std::integer_sequence<int, G...>) {
  return (0.0f + ... + tab[G * TE + field<O + IB * G, IB>(w)]);
}

// acc[C g + t] += wt * level t of the C-tuple that field g selects.
template <int C, int IB, int G, int N>
__device__ __forceinline__ void lut_fma_one(const float* tab, const uint32_t (&w)[N], float wt, float (&acc)[kD]) {
  const uint32_t idx = field<IB * G, IB>(w);
  if constexpr (C == 2) {
    const float2 lv = *reinterpret_cast<const float2*>(&tab[2 * idx]);
    acc[2 * G] = fmaf(wt, lv.x, acc[2 * G]);
    acc[2 * G + 1] = fmaf(wt, lv.y, acc[2 * G + 1]);
  } else {
    acc[G] = fmaf(wt, tab[idx], acc[G]);
  }
}
template <int C, int IB, int N, int... G>
__device__ __forceinline__ void lut_fma(const float* tab, const uint32_t (&w)[N], float wt, float (&acc)[kD],
                                        std::integer_sequence<int, G...>) {
  (lut_fma_one<C, IB, G>(tab, w, wt, acc), ...);
}

// acc[32 q + C g + t] += wt[q] * level t of the C-tuple that field g of w
// selects (32 codes of one record quarter, GQ queries).
template <int C, int IB, int GQ, int G, int N, int NV>
__device__ __forceinline__ void kv_values_g_one(const float* tab, const uint32_t (&w)[N], const float (&wt)[GQ],
                                                float (&acc)[NV]) {
  const uint32_t idx = field<IB * G, IB>(w);
  if constexpr (C == 2) {
    const float2 lv = *reinterpret_cast<const float2*>(&tab[2 * idx]);
#pragma unroll
    for (int q = 0; q < GQ; ++q) {
      acc[32 * q + 2 * G] = fmaf(wt[q], lv.x, acc[32 * q + 2 * G]);
      acc[32 * q + 2 * G + 1] = fmaf(wt[q], lv.y, acc[32 * q + 2 * G + 1]);
    }
  } else {
    const float lv = tab[idx];
#pragma unroll
    for (int q = 0; q < GQ; ++q) acc[32 * q + G] = fmaf(wt[q], lv, acc[32 * q + G]);
  }
}
template <int C, int IB, int N, int GQ, int NV, int... G>
__device__ __forceinline__ void kv_values_g_decode(const float* tab, const uint32_t (&w)[N], const float (&wt)[GQ],
                                                   float (&acc)[NV], std::integer_sequence<int, G...>) {
  (kv_values_g_one<C, IB, GQ, G>(tab, w, wt, acc), ...);
}

// ------------------------------------------------------------ quantise ---
// One wavefront per vector, lane l holding coordinates 2l and 2l + 1, all
// in FP64: radius, sign flip and block-128 transform, direction, nearest
// level (binary search over the cell boundaries, a value on a boundary to
// the lower level), and for keys the residual, its norm and z = sign(S e)
// with S^T staged in LDS.  The workgroup's four wavefronts walk the vectors
// together so that the barriers around the shared staging are uniform.
// Orders a wavefront's LDS stores before its later LDS loads of other
// lanes' values (and those loads before the next stores): the wavefront's
// LDS operations are waited for and the compiler keeps them on their side.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();
}

constexpr int kQWaves = 8;  // wavefronts per quantise workgroup (one copy of S^T in LDS for all)
constexpr int kQVecs = 4;   // vectors per wavefront and pass

// Each wavefront quantises kQVecs vectors per pass: their loads first, then
// per vector the radius, sign flip and block-128 butterfly, the nearest
// levels (binary search over the cell boundaries) and, for keys, the
// residual e, its norm and S e.  The projection reads S^T from LDS once per
// pass for all kQVecs vectors (row lane and lane + 64 per lane), so its LDS
// traffic per vector is a quarter of one vector at a time.  Everything a
// wavefront exchanges through LDS is its own: no workgroup barrier in the
// loop.
template <bool KEYS>
__global__ __launch_bounds__(kQWaves * 64) void kv_quantize_kernel(const void* __restrict__ x, int x_dtype, long long n,
                                                                 const float* __restrict__ signs,
                                                                 const float* __restrict__ jl,
                                                                 const double* __restrict__ levels, int mb,
                                                                 long long stride, int rec_words,
                                                                 uint32_t* __restrict__ rec,
                                                                 uint16_t* __restrict__ radius,
                                                                 uint16_t* __restrict__ gamma) {
  __shared__ float st[KEYS ? kD * kD : 1];  // st[k][row] = S[row][k]
  __shared__ double lv[256];
  __shared__ double mids[256];
  __shared__ __attribute__((aligned(16))) double ebuf[KEYS ? kQWaves : 1][kQVecs][KEYS ? kD : 2];
  __shared__ uint32_t chunk[kQWaves][kQVecs][64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nl = 1 << mb;
  for (int i = tid; i < nl; i += kQWaves * 64) lv[i] = levels[i];
  for (int i = tid; i < nl - 1; i += kQWaves * 64) mids[i] = (levels[i] + levels[i + 1]) / 2.0;
  if constexpr (KEYS) {
    for (int i = tid; i < kD * kD; i += kQWaves * 64) st[(i % kD) * kD + i / kD] = jl[i];
  }
  __syncthreads();
  const double sg0 = signs[2 * lane], sg1 = signs[2 * lane + 1];
  const int code_words = 4 * mb;
  constexpr long long kPass = kQWaves * kQVecs;
  for (long long base = static_cast<long long>(blockIdx.x) * kPass; base < n;
       base += static_cast<long long>(gridDim.x) * kPass) {
    const long long v0 = base + static_cast<long long>(wv) * kQVecs;
    double xa[kQVecs], xb[kQVecs];
#pragma unroll
    for (int q = 0; q < kQVecs; ++q) {
      xa[q] = 0.0;
      xb[q] = 0.0;
      if (v0 + q < n) {
        xa[q] = static_cast<double>(load_act(x, x_dtype, static_cast<size_t>(v0 + q) * kD + 2 * lane));
        xb[q] = static_cast<double>(load_act(x, x_dtype, static_cast<size_t>(v0 + q) * kD + 2 * lane + 1));
      }
    }
    double rq[kQVecs], gq[kQVecs];
#pragma unroll
    for (int q = 0; q < kQVecs; ++q) {
      const double r = sqrt(wave_sum_f64(xa[q] * xa[q] + xb[q] * xb[q], lane));
      double y0 = sg0 * xa[q], y1 = sg1 * xb[q];
      wave_fwht128<double>(y0, y1, lane, kInvSqrtD);
      const double u0 = r > 0.0 ? y0 / r : 0.0;
      const double u1 = r > 0.0 ? y1 / r : 0.0;
      int c0 = 0, c1 = 0;
      for (int s = nl >> 1; s >= 1; s >>= 1) {
        if (mids[c0 + s - 1] < u0) c0 += s;
        if (mids[c1 + s - 1] < u1) c1 += s;
      }
      chunk[wv][q][lane] = static_cast<uint32_t>(c0) | (static_cast<uint32_t>(c1) << mb);
      double gam = 0.0;
      if constexpr (KEYS) {
        const double e0 = u0 - lv[c0], e1 = u1 - lv[c1];
        *reinterpret_cast<double2*>(&ebuf[wv][q][2 * lane]) = make_double2(e0, e1);
        gam = sqrt(wave_sum_f64(e0 * e0 + e1 * e1, lane));
      }
      rq[q] = r;
      gq[q] = gam;
    }
    wave_lds_sync();
    if constexpr (KEYS) {
      double sa[kQVecs], sb[kQVecs];
#pragma unroll
      for (int q = 0; q < kQVecs; ++q) sa[q] = sb[q] = 0.0;
      for (int k = 0; k < kD; k += 2) {
        const double s0 = st[k * kD + lane], s1 = st[k * kD + lane + 64];
        const double t0 = st[(k + 1) * kD + lane], t1 = st[(k + 1) * kD + lane + 64];
#pragma unroll
        for (int q = 0; q < kQVecs; ++q) {
          const double2 e = *reinterpret_cast<const double2*>(&ebuf[wv][q][k]);
          sa[q] = fma(t0, e.y, fma(s0, e.x, sa[q]));
          sb[q] = fma(t1, e.y, fma(s1, e.x, sb[q]));
        }
      }
#pragma unroll
      for (int q = 0; q < kQVecs; ++q) {
        const unsigned long long za = __ballot(sa[q] >= 0.0);
        const unsigned long long zb = __ballot(sb[q] >= 0.0);
        const int zi = lane - code_words;
        if (v0 + q < n && zi >= 0 && zi < 4) {
          const unsigned long long zm = zi < 2 ? za : zb;
          rec[static_cast<size_t>(v0 + q) * static_cast<size_t>(stride) * rec_words + code_words + zi] =
              static_cast<uint32_t>((zi & 1) ? (zm >> 32) : zm);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kQVecs; ++q) {
      if (v0 + q >= n) break;
      const size_t rbase = static_cast<size_t>(v0 + q) * static_cast<size_t>(stride);
      if (lane < code_words) {
        // Word `lane` of the code fields: bits 32 lane .. 32 lane + 31, from
        // the 2 mb-bit chunks of the lanes that overlap them.
        const int cw = 2 * mb;
        const int l0 = (32 * lane) / cw, l1 = (32 * lane + 31) / cw;
        uint32_t word = 0;
        for (int l = l0; l <= l1; ++l) {
          const uint32_t c = chunk[wv][q][l];
          const int off = l * cw - 32 * lane;
          word |= off >= 0 ? (c << off) : (c >> (-off));
        }
        rec[rbase * rec_words + lane] = word;
      }
      if (lane == 0) {
        radius[rbase] = f64_to_f16_rne(rq[q]);
        if constexpr (KEYS) gamma[rbase] = f64_to_f16_rne(gq[q]);
      }
    }
    wave_lds_sync();  // this pass's reads are done before the next pass's stores
  }
}

// --------------------------------------------------- score: the query ---
// One workgroup per query: q' = Pi q (sign flip, block-128 transform) and
// S q', both FP32, to the workspace as [q' (128) | S q' (128)].  Thread t
// takes half of row t mod 128 of S (64 contiguous entries, 16-byte loads);
// the two halves meet in LDS.
__global__ __launch_bounds__(256) void kv_query_kernel(const float* __restrict__ q, const float* __restrict__ signs,
                                                       const float* __restrict__ jl, float* __restrict__ qws) {
  __shared__ float qr[kD];
  __shared__ float part[kD];
  const int tid = threadIdx.x, lane = tid & 63;
  const size_t qi = blockIdx.x;
  const int row = tid & (kD - 1), half = tid >> 7;
  // This thread's 64 entries of S, loaded before the transform so that the
  // two memory latencies overlap.
  const float4* srow = reinterpret_cast<const float4*>(jl + row * kD + half * 64);
  float4 sv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) sv[i] = srow[i];
  if (tid < 64) {
    float y0 = signs[2 * lane] * q[qi * kD + 2 * lane];
    float y1 = signs[2 * lane + 1] * q[qi * kD + 2 * lane + 1];
    wave_fwht128<float>(y0, y1, lane, static_cast<float>(kInvSqrtD));
    qr[2 * lane] = y0;
    qr[2 * lane + 1] = y1;
    qws[qi * 256 + 2 * lane] = y0;
    qws[qi * 256 + 2 * lane + 1] = y1;
  }
  __syncthreads();
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float4 v = sv[i];
    const int k = half * 64 + 4 * i;
    acc = fmaf(v.x, qr[k], acc);
    acc = fmaf(v.y, qr[k + 1], acc);
    acc = fmaf(v.z, qr[k + 2], acc);
    acc = fmaf(v.w, qr[k + 3], acc);
  }
  if (half) part[row] = acc;
  __syncthreads();
  if (!half) qws[qi * 256 + kD + row] = acc + part[row];
}

// Codes per table lookup: as many as fit in 8 index bits (a power of two).
template <int MB>
constexpr int codes_per_lookup() {
  return MB == 1 ? 8 : MB == 2 ? 4 : MB <= 4 ? 2 : 1;
}

// ----------------------------------------------------- score: the keys ---
// Lane per key; a workgroup serves GQ queries of one KV head (the query
// heads that share its keys), so each key is fetched and split into its
// fields once for all of them.  Tables in LDS, built once per workgroup:
// for every group g of C adjacent codes, T_g[i] = sum_t q'_{Cg+t} c[code_t(i)]
// over the 2^(C mb) concatenations i of C codes, and for every ZB bits of
// z, Z_g[beta] = sum_t (+-1) (S q')_{ZB g + t}; each entry holds the GQ
// queries' values side by side, so one LDS read serves all of them.  A
// key's score is one table read per group plus one per ZB bits of z:
// r (sum_g T_g + gamma kappa sum_g Z_g), kappa = sqrt(pi/2)/128.
template <int GQ>
struct QVec;
template <>
struct QVec<1> {
  typedef float T;
};
template <>
struct QVec<2> {
  typedef float T __attribute__((ext_vector_type(2)));
};
template <>
struct QVec<4> {
  typedef float T __attribute__((ext_vector_type(4)));
};
template <typename V>
__device__ __forceinline__ V vsplat(float x) {
  return (V)(x);
}
template <int GQ>
__device__ __forceinline__ float vget(const typename QVec<GQ>::T& v, int i) {
  if constexpr (GQ == 1) {
    return v;
  } else {
    return v[i];
  }
}
template <typename V, int TE, int IB, int O, int N, int... G>
__device__ __forceinline__ V lut_sum_v(const V* tab, const uint32_t (&w)[N], std::integer_sequence<int, G...>) {
  return (vsplat<V>(0.0f) + ... + tab[G * TE + field<O + IB * G, IB>(w)]);
}

// GQ queries per workgroup: the largest of 4, 2, 1 that divides the query
// heads per KV head and whose tables fit the LDS.
template <int MB, int GQ>
constexpr bool kv_scores_fits() {
  constexpr int C = codes_per_lookup<MB>();
  constexpr int ZB = GQ == 1 ? 8 : 4;
  return static_cast<long>((kD / C) * (1 << (C * MB)) + (kD / ZB) * (1 << ZB) + 2 * kD) * GQ * 4 <= 150 * 1024;
}
template <int GQ>
constexpr int kv_scores_threads() {
  return GQ == 1 ? 256 : 512;
}

// q' and S q' of each query come from the workspace, formed once per query
// by kv_query_kernel.  (Forming them inside every workgroup instead, S read
// from L2 by each, made this kernel 7 us slower than the launch it saved.)
template <int MB, int GQ>
__global__ __launch_bounds__(kv_scores_threads<GQ>()) void kv_scores_kernel(
    const float* __restrict__ qws, int nq, const uint32_t* __restrict__ keys, const uint16_t* __restrict__ radius,
    const uint16_t* __restrict__ gamma, long long n, const double* __restrict__ levels, int kpt,
    float* __restrict__ scores) {
  typedef typename QVec<GQ>::T V;
  constexpr int BS = kv_scores_threads<GQ>();
  constexpr int C = codes_per_lookup<MB>();
  constexpr int IB = C * MB;
  constexpr int NG = kD / C;
  constexpr int TE = 1 << IB;
  constexpr int ZB = GQ == 1 ? 8 : 4;  // bits of z per lookup
  constexpr int NZ = kD / ZB;
  constexpr int RW = 4 * (MB + 1);
  constexpr float kKappa = 0.0097916731f;  // sqrt(pi/2) / 128
  static_assert(kv_scores_fits<MB, GQ>(), "tables exceed the LDS");
  __shared__ V tab[NG * TE];
  __shared__ V ztab[NZ << ZB];
  __shared__ V qv[2 * kD];  // [q' | S q'] of the GQ queries, side by side
  __shared__ float lvf[1 << MB];
  const int tid = threadIdx.x;
  const int groups_per_head = nq / GQ;
  const int head = blockIdx.y / groups_per_head;
  const int q0 = head * nq + (blockIdx.y % groups_per_head) * GQ;  // first query of this workgroup
  for (int e = tid; e < 2 * kD * GQ; e += BS) {
    const int k = e % (2 * kD), qq = e / (2 * kD);
    reinterpret_cast<float*>(qv)[k * GQ + qq] = qws[static_cast<size_t>(q0 + qq) * 256 + k];
  }
  if (tid < (1 << MB)) lvf[tid] = static_cast<float>(levels[tid]);
  __syncthreads();
  for (int e = tid; e < NG * TE; e += BS) {
    const int g = e / TE, idx = e % TE;
    V acc = vsplat<V>(0.0f);
#pragma unroll
    for (int t = 0; t < C; ++t) acc += qv[C * g + t] * lvf[(idx >> (MB * t)) & ((1 << MB) - 1)];
    tab[e] = acc;
  }
  for (int e = tid; e < (NZ << ZB); e += BS) {
    const int g = e >> ZB, beta = e & ((1 << ZB) - 1);
    V acc = vsplat<V>(0.0f);
#pragma unroll
    for (int t = 0; t < ZB; ++t) {
      const V s = qv[kD + ZB * g + t];
      acc += ((beta >> t) & 1) ? s : -s;
    }
    ztab[e] = acc;
  }
  __syncthreads();
  const size_t hn = static_cast<size_t>(head) * static_cast<size_t>(n);
  const long long k0 = static_cast<long long>(blockIdx.x) * BS * kpt + tid;
  for (int i = 0; i < kpt; ++i) {
    const long long k = k0 + static_cast<long long>(i) * BS;
    if (k >= n) break;
    uint32_t w[RW];
    load_record(keys + (hn + k) * RW, w);
    const V mse = lut_sum_v<V, TE, IB, 0>(tab, w, std::make_integer_sequence<int, NG>{});
    const V qjl = lut_sum_v<V, 1 << ZB, ZB, 128 * MB>(ztab, w, std::make_integer_sequence<int, NZ>{});
    const float r = half_bits_to_f32(radius[hn + k]);
    const float gk = half_bits_to_f32(gamma[hn + k]) * kKappa;
    const V sc = r * (mse + gk * qjl);
#pragma unroll
    for (int qq = 0; qq < GQ; ++qq) scores[static_cast<size_t>(q0 + qq) * static_cast<size_t>(n) + k] = vget<GQ>(sc, qq);
  }
}

// ------------------------------------------------------------ values ---
// Lane per value vector; each lane accumulates p_i r_i c[code] into 128
// registers (a table of C-level tuples turns C adjacent codes into C
// levels with one LDS read).  The workgroup then reduces its lanes by
// recursive halving (each exchange hands half of the remaining coordinates
// to the partner lane, so lane l ends with coordinates 2l, 2l + 1), sums
// its four wavefronts in LDS and writes one partial vector per key chunk.
template <int M, int H, int N>
__device__ __forceinline__ void halve(float (&a)[N], int lane) {
  const bool up = (lane & M) != 0;
#pragma unroll
  for (int i = 0; i < H; ++i) {
    const float send = up ? a[i] : a[i + H];
    const float keep = up ? a[i + H] : a[i];
    a[i] = keep + lane_xor_f32<M>(send, lane);
  }
}

// Softmax form (SM, tq_kv_attend): p holds the scores s, and the kernels
// work in base 2: z = scale2 * s with scale2 = scale log2(e), so that
// exp(scale s) = 2^z and each weight is one hardware exp2.  Value i is
// weighed by 2^(z_i - o) r_i with a running offset o, one per wavefront and
// query (a uniform value).  o starts at -inf; whenever a lane meets
// z > o + kOffsetSlack, o moves up to that z and the wavefront's running
// sums of the query are scaled by 2^(o_old - o_new).  Weights so stay below
// 2^kOffsetSlack (chunk sums far inside FP32 range) and the rescaling is
// rare: never again once o is within kOffsetSlack of the chunk's maximum.
// Each lane also sums its weights (l).  At the end the workgroup scales
// every wavefront to the largest offset m of its four, and (m, l) per
// (query, chunk) go beside the partial vectors; the finishing launch
// rescales the chunks to their common maximum.  The loop ends for a whole
// wavefront at once, so every lane takes part in the rescaling.
constexpr float kOffsetSlack = 24.0f;
constexpr double kLog2E = 1.4426950408889634;

// The offset the exponentials take: o itself, or 0 while o is -inf (every
// score so far masked), so that they come out 0 rather than NaN.
__device__ __forceinline__ float exp_offset(float o) { return o == -INFINITY ? 0.0f : o; }

// Raise the wavefront's offset o until no lane has z > o + kOffsetSlack;
// returns the factor 2^(o_before - o_after) for the running sums (1 when
// o is unchanged, 0 when it was -inf: nothing has been summed yet).
// Only lanes with `mine` set take part (the lanes whose z is a score of
// this query).
__device__ __forceinline__ float raise_offset(float z, float& o, bool mine = true) {
  float f = 1.0f;
  uint64_t need = __builtin_amdgcn_ballot_w64(mine && z > o + kOffsetSlack);
  while (need) {
    const float zn = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z), __builtin_ctzll(need)));
    f = o == -INFINITY ? 0.0f : f * exp2f(o - zn);
    o = zn;
    need = __builtin_amdgcn_ballot_w64(mine && z > o + kOffsetSlack);
  }
  return f;
}

// The softmax form's weights of one value for GQ queries: x holds the
// scores s on entry and 2^(scale2 s - o) on return (0 for a lane whose
// value is past the end, valid false).  The common path has one uniform
// branch; the rescaling path (rare) raises each query's offset and scales
// its NA running sums acc[NA qq ..] and weight sum.
template <int GQ, int NA, int NV>
__device__ __forceinline__ void softmax_weights(float (&x)[GQ], bool valid, float scale, float (&off)[GQ],
                                                float (&acc)[NV], float (&l)[GQ]) {
  bool need = false;
#pragma unroll
  for (int qq = 0; qq < GQ; ++qq) {
    x[qq] = valid ? scale * x[qq] : -INFINITY;
    need = need || x[qq] > off[qq] + kOffsetSlack;
  }
  if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
    for (int qq = 0; qq < GQ; ++qq) {
      const float f = raise_offset(x[qq], off[qq]);
      if (f != 1.0f) {
#pragma unroll
        for (int j = 0; j < NA; ++j) acc[NA * qq + j] *= f;
        l[qq] *= f;
      }
    }
  }
#pragma unroll
  for (int qq = 0; qq < GQ; ++qq) {
    x[qq] = __builtin_amdgcn_exp2f(x[qq] - exp_offset(off[qq]));
    l[qq] += x[qq];
  }
}

// wt[q] = x of part q of the lane's four-lane group (DPP quad permutations;
// the four lanes of a value are active or inactive together).
template <int GQ>
__device__ __forceinline__ void quad_spread(float x, float (&wt)[GQ]) {
  static_assert(GQ == 2 || GQ == 4, "four lanes per value serve 2 or 4 queries");
  wt[0] = dpp_f32<0x00>(x);  // quad_perm(0,0,0,0)
  wt[1] = dpp_f32<0x55>(x);  // quad_perm(1,1,1,1)
  if constexpr (GQ == 4) {
    wt[2] = dpp_f32<0xAA>(x);
    wt[3] = dpp_f32<0xFF>(x);
  }
}

// The grouped kernel's softmax weights of one value, the work split over
// the value's four lanes: lane part p loads the score of query p % GQ and
// takes its exponential (one load and one exponential per lane), then the
// GQ weights are broadcast across the four lanes.  l is the lane's weight
// sum of its own query.  The common path has one uniform branch.
template <int GQ, int NV>
__device__ __forceinline__ void softmax_weights_quad(float z, bool valid, int part, float scale, float (&off)[GQ],
                                                     float (&acc)[NV], float& l, float (&wt)[GQ]) {
  const int mq = part & (GQ - 1);
  z = valid ? scale * z : -INFINITY;
  float om = off[0];
#pragma unroll
  for (int qq = 1; qq < GQ; ++qq) om = mq == qq ? off[qq] : om;
  if (__builtin_amdgcn_ballot_w64(z > om + kOffsetSlack)) {
#pragma unroll
    for (int qq = 0; qq < GQ; ++qq) {
      const float f = raise_offset(z, off[qq], mq == qq);
      if (f != 1.0f) {
#pragma unroll
        for (int j = 0; j < 32; ++j) acc[32 * qq + j] *= f;
        l = mq == qq ? l * f : l;
      }
    }
    om = off[0];
#pragma unroll
    for (int qq = 1; qq < GQ; ++qq) om = mq == qq ? off[qq] : om;
  }
  const float w = __builtin_amdgcn_exp2f(z - exp_offset(om));
  l += w;
  quad_spread<GQ>(w, wt);
}

// End of the softmax form: the workgroup's offset m = max over its four
// wavefronts, every wavefront's sums scaled to it, and the weight sums l
// (lane's l belongs to query lq) added per query over the workgroup into
// lout.  Lanes S0 apart hold different values (1: one value per lane; 4:
// the four lanes of a value, whose parts p and p + GQ repeat a query), so
// the lane sums run over strides S0 .. 32 and lane q < GQ then holds
// query q's wavefront sum.
template <int GQ, int NV, int S0>
__device__ __forceinline__ void softmax_merge(float (&off)[GQ], float (&acc)[NV], float l, int lq, float (&lout)[GQ],
                                              float (*sbuf)[GQ]) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  constexpr int NA = NV / GQ;
  if (lane == 0)
#pragma unroll
    for (int qq = 0; qq < GQ; ++qq) sbuf[wv][qq] = off[qq];
  __syncthreads();
#pragma unroll
  for (int qq = 0; qq < GQ; ++qq) {
    const float m = fmaxf(fmaxf(sbuf[0][qq], sbuf[1][qq]), fmaxf(sbuf[2][qq], sbuf[3][qq]));
    const float f = off[qq] == -INFINITY ? 0.0f : exp2f(off[qq] - m);
    if (f != 1.0f) {
#pragma unroll
      for (int j = 0; j < NA; ++j) acc[NA * qq + j] *= f;
      l = lq == qq ? l * f : l;
    }
    off[qq] = m;
  }
  if constexpr (S0 <= 1) l += lane_xor_f32<1>(l, lane);
  if constexpr (S0 <= 2) l += lane_xor_f32<2>(l, lane);
  l += lane_xor_f32<4>(l, lane);
  l += lane_xor_f32<8>(l, lane);
  l += lane_xor_f32<16>(l, lane);
  l += lane_xor_f32<32>(l, lane);
  __syncthreads();  // every wavefront has read the offsets
  if (lane < GQ) sbuf[wv][lane] = l;
  __syncthreads();
#pragma unroll
  for (int qq = 0; qq < GQ; ++qq) lout[qq] = (sbuf[0][qq] + sbuf[1][qq]) + (sbuf[2][qq] + sbuf[3][qq]);
}

template <int MB, bool SM>
__global__ __launch_bounds__(256) void kv_values_kernel(const float* __restrict__ p, int nq,
                                                        const uint32_t* __restrict__ vals,
                                                        const uint16_t* __restrict__ radius, long long n,
                                                        const double* __restrict__ levels, int kpt,
                                                        float* __restrict__ partial, float scale,
                                                        float2* __restrict__ ml) {
  constexpr int C = MB <= 4 ? 2 : 1;
  constexpr int IB = C * MB;
  constexpr int NG = kD / C;
  constexpr int TE = 1 << IB;
  constexpr int RW = 4 * MB;
  __shared__ __align__(16) float tab[TE * C];
  __shared__ float red[4][kD];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int qi = blockIdx.y;
  const int head = qi / nq;
  for (int e = tid; e < TE; e += 256) {
#pragma unroll
    for (int t = 0; t < C; ++t) tab[e * C + t] = static_cast<float>(levels[(e >> (MB * t)) & ((1 << MB) - 1)]);
  }
  __syncthreads();
  float off[1] = {-INFINITY}, lsum[1] = {0.0f};
  float acc[kD];
#pragma unroll
  for (int j = 0; j < kD; ++j) acc[j] = 0.0f;
  const size_t hn = static_cast<size_t>(head) * static_cast<size_t>(n);
  const long long kbeg = static_cast<long long>(blockIdx.x) * 256 * kpt;
  const long long k0 = kbeg + tid;
  for (int i = 0; i < kpt; ++i) {
    long long k = k0 + static_cast<long long>(i) * 256;
    bool valid = true;
    if constexpr (SM) {
      if (kbeg + 64 * wv + static_cast<long long>(i) * 256 >= n) break;  // whole wavefront past n
      valid = k < n;
      k = valid ? k : n - 1;  // an in-bounds stand-in, weighed 0
    } else {
      if (k >= n) break;
    }
    uint32_t w[RW];
    load_record(vals + (hn + k) * RW, w);
    const float r = half_bits_to_f32(radius[hn + k]);
    float pk[1] = {p[static_cast<size_t>(qi) * static_cast<size_t>(n) + k]};
    if constexpr (SM) softmax_weights<1, kD>(pk, valid, scale, off, acc, lsum);
    lut_fma<C, IB>(tab, w, pk[0] * r, acc, std::make_integer_sequence<int, NG>{});
  }
  if constexpr (SM) {
    __shared__ float sml[4][1];
    softmax_merge<1, kD, 1>(off, acc, lsum[0], 0, lsum, sml);
    if (tid == 0) ml[static_cast<size_t>(qi) * gridDim.x + blockIdx.x] = make_float2(off[0], lsum[0]);
  }
  halve<32, 64>(acc, lane);
  halve<16, 32>(acc, lane);
  halve<8, 16>(acc, lane);
  halve<4, 8>(acc, lane);
  halve<2, 4>(acc, lane);
  halve<1, 2>(acc, lane);
  red[wv][2 * lane] = acc[0];
  red[wv][2 * lane + 1] = acc[1];
  __syncthreads();
  if (wv == 0) {
    const float s0 = (red[0][2 * lane] + red[1][2 * lane]) + (red[2][2 * lane] + red[3][2 * lane]);
    const float s1 = (red[0][2 * lane + 1] + red[1][2 * lane + 1]) + (red[2][2 * lane + 1] + red[3][2 * lane + 1]);
    float2* out = reinterpret_cast<float2*>(partial + (static_cast<size_t>(qi) * gridDim.x + blockIdx.x) * kD);
    out[lane] = make_float2(s0, s1);
  }
}

// GQ queries per workgroup (the query heads of one KV head): four lanes per
// value, lane part p taking coordinates 32 p .. 32 p + 31 (its m words of
// the record) for all GQ queries, 32 GQ running sums.  Each value is
// fetched and split once for all GQ queries.  The wavefront's lanes of one
// part are reduced by recursive halving over lane strides 32, 16, 8, 4
// (lane l then holds entries f = (GQ 32 / 16)(l / 4) + i of the flattened
// [query][coordinate] sums of part l % 4), the four wavefronts in LDS.
template <int MB, int GQ, bool SM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void kv_values_g_kernel(
    const float* __restrict__ p, int nq, const uint32_t* __restrict__ vals, const uint16_t* __restrict__ radius,
    long long n, const double* __restrict__ levels, int kpt, float* __restrict__ partial, float scale,
    float2* __restrict__ ml) {
  constexpr int C = MB <= 4 ? 2 : 1;
  constexpr int IB = C * MB;
  constexpr int TE = 1 << IB;
  constexpr int RW = 4 * MB;   // record words
  constexpr int PW = MB;       // words of one quarter (32 codes)
  constexpr int NV = 32 * GQ;  // running sums per lane
  constexpr int FIN = NV / 16;  // sums per lane after the halving
  __shared__ __align__(16) float tab[TE * C];
  __shared__ float red[4][GQ][kD];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, part = tid & 3;
  const int groups_per_head = nq / GQ;
  const int head = blockIdx.y / groups_per_head;
  const int q0 = head * nq + (blockIdx.y % groups_per_head) * GQ;
  for (int e = tid; e < TE; e += 256) {
#pragma unroll
    for (int t = 0; t < C; ++t) tab[e * C + t] = static_cast<float>(levels[(e >> (MB * t)) & ((1 << MB) - 1)]);
  }
  __syncthreads();
  float off[GQ], lsum = 0.0f;
#pragma unroll
  for (int qq = 0; qq < GQ; ++qq) off[qq] = -INFINITY;
  float acc[NV];
#pragma unroll
  for (int f = 0; f < NV; ++f) acc[f] = 0.0f;
  const size_t hn = static_cast<size_t>(head) * static_cast<size_t>(n);
  const long long kbeg = static_cast<long long>(blockIdx.x) * 64 * kpt;
  const long long k0 = kbeg + (tid >> 2);
  for (int i = 0; i < kpt; ++i) {
    long long k = k0 + static_cast<long long>(i) * 64;
    bool valid = true;
    if constexpr (SM) {
      if (kbeg + 16 * wv + static_cast<long long>(i) * 64 >= n) break;  // whole wavefront past n
      valid = k < n;
      k = valid ? k : n - 1;  // an in-bounds stand-in, weighed 0
    } else {
      if (k >= n) break;
    }
    uint32_t w[PW];
    const uint32_t* rp = vals + (hn + k) * RW + PW * part;
#pragma unroll
    for (int x = 0; x < PW; ++x) w[x] = __builtin_nontemporal_load(rp + x);
    const float r = half_bits_to_f32(radius[hn + k]);
    // Lane part q loads the weight (or score) of query q % GQ; the quad
    // shares them.
    float wt[GQ];
    const float pq = p[static_cast<size_t>(q0 + (part & (GQ - 1))) * static_cast<size_t>(n) + k];
    if constexpr (SM)
      softmax_weights_quad<GQ>(pq, valid, part, scale, off, acc, lsum, wt);
    else
      quad_spread<GQ>(pq, wt);
#pragma unroll
    for (int qq = 0; qq < GQ; ++qq) wt[qq] *= r;
    kv_values_g_decode<C, IB>(tab, w, wt, acc, std::make_integer_sequence<int, 32 / C>{});
  }
  if constexpr (SM) {
    __shared__ float sml[4][GQ];
    float lq[GQ];
    softmax_merge<GQ, NV, 4>(off, acc, lsum, part & (GQ - 1), lq, sml);
    if (tid == 0) {
#pragma unroll
      for (int qq = 0; qq < GQ; ++qq)
        ml[static_cast<size_t>(q0 + qq) * gridDim.x + blockIdx.x] = make_float2(off[qq], lq[qq]);
    }
  }
  halve<32, NV / 2>(acc, lane);
  halve<16, NV / 4>(acc, lane);
  halve<8, NV / 8>(acc, lane);
  halve<4, NV / 16>(acc, lane);
#pragma unroll
  for (int x = 0; x < FIN; ++x) {
    const int f = FIN * (lane >> 2) + x;
    red[wv][f >> 5][32 * part + (f & 31)] = acc[x];
  }
  __syncthreads();
  for (int o = tid; o < GQ * kD; o += 256) {
    const int qq = o / kD, c = o % kD;
    const float v = (red[0][qq][c] + red[1][qq][c]) + (red[2][qq][c] + red[3][qq][c]);
    partial[(static_cast<size_t>(q0 + qq) * gridDim.x + blockIdx.x) * kD + c] = v;
  }
}

// Sum of the chunks' partial vectors, then Pi^T: the block-128 transform
// (H is symmetric) and the sign flip.  Wavefront w of 16 adds chunks w,
// w + 16, ... into four running sums (four independent loads in flight per
// step), then wavefront 0 adds the wavefronts' sums in order: a fixed order,
// so the result is deterministic.
// With SM, chunk c's partial vector and its l_c are first scaled by
// 2^(m_c - M) (offsets in base 2), M the largest m_c of the query, and the
// sum divided by the scaled l's sum; no chunks (n = 0) give zeros.
// 2^(m_c - M); a chunk whose scores are all -inf has nothing to add.
__device__ __forceinline__ float chunk_weight(float mc, float mx) { return mc == -INFINITY ? 0.0f : exp2f(mc - mx); }
constexpr int kFinishWaves = 16;
template <bool SM>
__global__ __launch_bounds__(kFinishWaves * 64) void kv_values_finish_kernel(const float* __restrict__ partial,
                                                                            int chunks,
                                                                            const float* __restrict__ signs,
                                                                            float* __restrict__ out,
                                                                            const float2* __restrict__ ml) {
  constexpr int W = kFinishWaves;
  __shared__ float2 red[W][64];
  __shared__ float sm[W];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const size_t qi = blockIdx.x;
  const float2* base = reinterpret_cast<const float2*>(partial + qi * static_cast<size_t>(chunks) * kD) + lane;
  const float2* mq = ml + qi * static_cast<size_t>(chunks);
  float mx = 0.0f;
  if constexpr (SM) {
    float v = -INFINITY;
    for (int c = tid; c < chunks; c += W * 64) v = fmaxf(v, mq[c].x);
    v = wave_max(v, lane);
    if (lane == 0) sm[wv] = v;
    __syncthreads();
    mx = sm[0];
#pragma unroll
    for (int w = 1; w < W; ++w) mx = fmaxf(mx, sm[w]);
  }
  float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f, l = 0.f;
  int c = wv;
  for (; c + W < chunks; c += 2 * W) {
    const float2 pa = base[static_cast<size_t>(c) * (kD / 2)];
    const float2 pb = base[static_cast<size_t>(c + W) * (kD / 2)];
    if constexpr (SM) {
      const float2 ma = mq[c], mb = mq[c + W];
      const float ea = chunk_weight(ma.x, mx), eb = chunk_weight(mb.x, mx);
      a0 = fmaf(ea, pa.x, a0), a1 = fmaf(ea, pa.y, a1), b0 = fmaf(eb, pb.x, b0), b1 = fmaf(eb, pb.y, b1);
      l = fmaf(ea, ma.y, fmaf(eb, mb.y, l));
    } else {
      a0 += pa.x, a1 += pa.y, b0 += pb.x, b1 += pb.y;
    }
  }
  for (; c < chunks; c += W) {
    const float2 pa = base[static_cast<size_t>(c) * (kD / 2)];
    if constexpr (SM) {
      const float2 ma = mq[c];
      const float ea = chunk_weight(ma.x, mx);
      a0 = fmaf(ea, pa.x, a0), a1 = fmaf(ea, pa.y, a1);
      l = fmaf(ea, ma.y, l);
    } else {
      a0 += pa.x, a1 += pa.y;
    }
  }
  if constexpr (SM) __syncthreads();  // sm is reused for the l sums
  red[wv][lane] = make_float2(a0 + b0, a1 + b1);
  if (SM && lane == 0) sm[wv] = l;  // every lane of a wavefront holds the same l
  __syncthreads();
  if (wv == 0) {
    float v0 = 0.0f, v1 = 0.0f, lt = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      v0 += red[w][lane].x;
      v1 += red[w][lane].y;
      if constexpr (SM) lt += sm[w];
    }
    if constexpr (SM) {
      const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
      v0 *= inv;
      v1 *= inv;
    }
    wave_fwht128<float>(v0, v1, lane, static_cast<float>(kInvSqrtD));
    out[qi * kD + 2 * lane] = signs[2 * lane] * v0;
    out[qi * kD + 2 * lane + 1] = signs[2 * lane + 1] * v1;
  }
}

// --------------------------------------------------------------- plans ---
// Keys (values) per thread: enough chunks for about 2048 workgroups over
// all queries, at least 2 (4) keys per thread so that building the tables
// (reducing the lanes) stays a small part of a workgroup's work.
int kv_kpt(long long n, long long rows, int lo, int hi, int bs = 256, long long target = 2048) {
  const long long per_row = (target + rows - 1) / rows;
  long long kpt = (n + bs * per_row - 1) / (bs * per_row);
  if (kpt < lo) kpt = lo;
  if (kpt > hi) kpt = hi;
  return static_cast<int>(kpt);
}
constexpr int kScoreKptLo = 2, kScoreKptHi = 16;
constexpr int kValueKptLo = 4, kValueKptHi = 32;

long long kv_chunks(long long n, int kpt, int bs = 256) { return (n + static_cast<long long>(bs) * kpt - 1) / (static_cast<long long>(bs) * kpt); }

bool kv_dtype_ok(int d) { return d == TQ_F32 || d == TQ_BF16 || d == TQ_F16; }

// Scores: GQ queries per workgroup (see kv_scores_kernel); the grid is
// (key chunks, heads * nq / GQ), one workgroup per CU when GQ > 1, so a
// workgroup then takes at least four keys per thread.
template <int MB, int GQ>
int launch_scores_g(long long queries, int nq, hipStream_t s, const float* qws, const uint32_t* keys,
                    const uint16_t* r, const uint16_t* g, long long n, const double* levels, float* scores) {
  constexpr int BS = kv_scores_threads<GQ>();
  const long long rows = queries / GQ;
  const int kpt = kv_kpt(n, rows, GQ == 1 ? kScoreKptLo : 4, kScoreKptHi, BS, GQ == 1 ? 2048 : 256);
  const long long chunks = kv_chunks(n, kpt, BS);
  if (chunks > INT_MAX) return TQ_ESHAPE;
  hipLaunchKernelGGL((kv_scores_kernel<MB, GQ>), dim3(static_cast<unsigned>(chunks), static_cast<unsigned>(rows)),
                     dim3(BS), 0, s, qws, nq, keys, r, g, n, levels, kpt, scores);
  return TQ_OK;
}
template <int MB>
int launch_scores(long long queries, int nq, hipStream_t s, const float* qws, const uint32_t* keys,
                  const uint16_t* r, const uint16_t* g, long long n, const double* levels, float* scores) {
  if constexpr (kv_scores_fits<MB, 4>()) {
    if (nq % 4 == 0) return launch_scores_g<MB, 4>(queries, nq, s, qws, keys, r, g, n, levels, scores);
  }
  if (nq % 2 == 0) return launch_scores_g<MB, 2>(queries, nq, s, qws, keys, r, g, n, levels, scores);
  return launch_scores_g<MB, 1>(queries, nq, s, qws, keys, r, g, n, levels, scores);
}

// Value sums: GQ queries per workgroup when the query heads per KV head
// allow (4, 2, else 1); keys per workgroup 64 kpt (GQ > 1, four lanes per
// value) or 256 kpt (GQ = 1, a lane per value), chosen for about 768 (GQ > 1:
// three per CU of the 256, one round; sweeps over 192..4096 at 128K tokens
// had their minimum there) or 2048 workgroups.  The workspace holds one
// partial vector per (query, key chunk).
struct ValuesPlan {
  int gq, kpt;
  long long chunks;
};
ValuesPlan kv_values_plan(long long n, long long queries, int nq) {
  ValuesPlan v;
  v.gq = nq % 4 == 0 ? 4 : (nq % 2 == 0 ? 2 : 1);
  if (v.gq == 1) {
    v.kpt = kv_kpt(n, queries, kValueKptLo, kValueKptHi);
    v.chunks = kv_chunks(n, v.kpt);
  } else {
    v.kpt = kv_kpt(n, queries / v.gq, 8, 256, 64, 768);
    v.chunks = kv_chunks(n, v.kpt, 64);
  }
  return v;
}

template <int MB, bool SM>
void launch_values(const ValuesPlan& v, long long queries, hipStream_t s, const float* p, int nq,
                   const uint32_t* vals, const uint16_t* r, long long n, const double* levels, float* partial,
                   float scale, float2* ml) {
  const unsigned gx = static_cast<unsigned>(v.chunks);
  if (v.gq == 4)
    hipLaunchKernelGGL((kv_values_g_kernel<MB, 4, SM>), dim3(gx, static_cast<unsigned>(queries / 4)), dim3(256), 0, s,
                       p, nq, vals, r, n, levels, v.kpt, partial, scale, ml);
  else if (v.gq == 2)
    hipLaunchKernelGGL((kv_values_g_kernel<MB, 2, SM>), dim3(gx, static_cast<unsigned>(queries / 2)), dim3(256), 0, s,
                       p, nq, vals, r, n, levels, v.kpt, partial, scale, ml);
  else
    hipLaunchKernelGGL((kv_values_kernel<MB, SM>), dim3(gx, static_cast<unsigned>(queries)), dim3(256), 0, s, p, nq,
                       vals, r, n, levels, v.kpt, partial, scale, ml);
}

}  // namespace

extern "C" {

int tq_kv_codebook(int bits, double* levels) {
  if (!levels || bits < 1 || bits > TQ_KV_MAX_BITS) return TQ_EINVAL;
  const int h = 1 << (bits - 1);
  std::vector<double> y;
  if (!lloyd_max_half(h, &y)) return TQ_EUNSUPPORTED;
  for (int j = 0; j < h; ++j) {
    levels[h + j] = y[j] * kInvSqrtD;
    levels[h - 1 - j] = -y[j] * kInvSqrtD;
  }
  return TQ_OK;
}

size_t tq_kv_record_bytes(int bits) { return bits >= 1 && bits <= TQ_KV_MAX_BITS ? 16u * bits : 0; }

int tq_kv_quantize(const void* x, int x_dtype, int64_t n, const float* signs, const float* jl, const double* levels,
                   int bits, int keys, int64_t stride, uint32_t* records, uint16_t* radius, uint16_t* gamma,
                   void* stream) {
  if (!x || !signs || !levels || !records || !radius) return TQ_EINVAL;
  if (keys && (!jl || !gamma)) return TQ_EINVAL;
  if (!kv_dtype_ok(x_dtype)) return TQ_EINVAL;
  if (bits < (keys ? 2 : 1) || bits > TQ_KV_MAX_BITS) return TQ_EINVAL;
  if (!tq_aligned(x, tq_act_align(x_dtype)) || !tq_aligned(signs, 4) || !tq_aligned(levels, 8) ||
      !tq_aligned(records, 16) || !tq_aligned(radius, 2) || (jl && !tq_aligned(jl, 4)) ||
      (gamma && !tq_aligned(gamma, 2)))
    return TQ_EINVAL;
  if (n < 0 || stride < 1) return TQ_ESHAPE;
  if (n == 0) return TQ_OK;
  const int mb = keys ? bits - 1 : bits;
  const long long groups = (n + kQWaves * kQVecs - 1) / (kQWaves * kQVecs);
  const unsigned grid = static_cast<unsigned>(groups < 2048 ? groups : 2048);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int rw = 4 * bits;
  if (keys)
    hipLaunchKernelGGL(kv_quantize_kernel<true>, dim3(grid), dim3(kQWaves * 64), 0, s, x, x_dtype, n, signs, jl, levels, mb,
                       stride, rw, records, radius, gamma);
  else
    hipLaunchKernelGGL(kv_quantize_kernel<false>, dim3(grid), dim3(kQWaves * 64), 0, s, x, x_dtype, n, signs, jl, levels, mb,
                       stride, rw, records, radius, gamma);
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}

size_t tq_kv_workspace(int op, int64_t n, int heads, int nq) {
  if (n < 0 || heads < 1 || nq < 1) return SIZE_MAX;
  const long long queries = static_cast<long long>(heads) * nq;
  if (op == TQ_KV_OP_SCORES) return static_cast<size_t>(queries) * 256 * sizeof(float);
  if (op == TQ_KV_OP_VALUES || op == TQ_KV_OP_ATTEND) {
    const long long chunks = kv_values_plan(n, queries, nq).chunks;
    const size_t vecs = static_cast<size_t>(queries) * static_cast<size_t>(chunks > 0 ? chunks : 1);
    return vecs * kD * sizeof(float) + (op == TQ_KV_OP_ATTEND ? vecs * sizeof(float2) : 0);
  }
  return SIZE_MAX;
}

int tq_kv_scores(const float* q, int heads, int nq, const uint32_t* keys, const uint16_t* radius,
                 const uint16_t* gamma, int64_t n, int bits, const float* signs, const float* jl,
                 const double* levels, float* scores, void* workspace, size_t ws_bytes, void* stream) {
  if (!q || !keys || !radius || !gamma || !signs || !jl || !levels || !scores || !workspace) return TQ_EINVAL;
  if (bits < 2 || bits > TQ_KV_MAX_BITS) return TQ_EINVAL;
  if (!tq_aligned(q, 8) || !tq_aligned(keys, 16) || !tq_aligned(radius, 2) || !tq_aligned(gamma, 2) ||
      !tq_aligned(signs, 4) || !tq_aligned(jl, 16) || !tq_aligned(levels, 8) || !tq_aligned(scores, 4) ||
      !tq_aligned(workspace, 16))
    return TQ_EINVAL;
  if (heads < 1 || nq < 1 || n < 0) return TQ_ESHAPE;
  const long long queries = static_cast<long long>(heads) * nq;
  if (queries > 65535) return TQ_ESHAPE;
  if (ws_bytes < tq_kv_workspace(TQ_KV_OP_SCORES, n, heads, nq)) return TQ_ENOSPACE;
  if (n == 0) return TQ_OK;
  if (n > static_cast<long long>(INT_MAX) * 256) return TQ_ESHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* qws = static_cast<float*>(workspace);
  hipLaunchKernelGGL(kv_query_kernel, dim3(static_cast<unsigned>(queries)), dim3(256), 0, s, q, signs, jl, qws);
  TQ_LAUNCH_CHECK();
  int st;
#define TQ_KVS(MB) launch_scores<MB>(queries, nq, s, qws, keys, radius, gamma, n, levels, scores)
  switch (bits - 1) {
    case 1: st = TQ_KVS(1); break;
    case 2: st = TQ_KVS(2); break;
    case 3: st = TQ_KVS(3); break;
    case 4: st = TQ_KVS(4); break;
    case 5: st = TQ_KVS(5); break;
    case 6: st = TQ_KVS(6); break;
    default: st = TQ_KVS(7); break;
  }
#undef TQ_KVS
  if (st != TQ_OK) return st;
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}

namespace {
int kv_values_impl(bool attend, const float* p, float scale, int heads, int nq, const uint32_t* values,
                   const uint16_t* radius, int64_t n, int bits, const float* signs, const double* levels, float* out,
                   void* workspace, size_t ws_bytes, void* stream) {
  if (!p || !values || !radius || !signs || !levels || !out || !workspace) return TQ_EINVAL;
  if (bits < 1 || bits > TQ_KV_MAX_BITS) return TQ_EINVAL;
  if (attend && !std::isfinite(scale)) return TQ_EINVAL;
  if (!tq_aligned(p, 4) || !tq_aligned(values, 16) || !tq_aligned(radius, 2) || !tq_aligned(signs, 4) ||
      !tq_aligned(levels, 8) || !tq_aligned(out, 8) || !tq_aligned(workspace, 16))
    return TQ_EINVAL;
  if (heads < 1 || nq < 1 || n < 0) return TQ_ESHAPE;
  const long long queries = static_cast<long long>(heads) * nq;
  if (queries > 65535) return TQ_ESHAPE;
  if (ws_bytes < tq_kv_workspace(attend ? TQ_KV_OP_ATTEND : TQ_KV_OP_VALUES, n, heads, nq)) return TQ_ENOSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const ValuesPlan v = kv_values_plan(n, queries, nq);
  const long long chunks = v.chunks;
  if (chunks > INT_MAX) return TQ_ESHAPE;
  float* partial = static_cast<float*>(workspace);
  float2* ml = reinterpret_cast<float2*>(partial + static_cast<size_t>(queries) * static_cast<size_t>(chunks) * kD);
  const float scale2 = static_cast<float>(static_cast<double>(scale) * kLog2E);
  if (chunks > 0) {
#define TQ_KVV(MB)                                                                                        \
  (attend ? launch_values<MB, true>(v, queries, s, p, nq, values, radius, n, levels, partial, scale2, ml) \
          : launch_values<MB, false>(v, queries, s, p, nq, values, radius, n, levels, partial, 0.0f, ml))
    switch (bits) {
      case 1: TQ_KVV(1); break;
      case 2: TQ_KVV(2); break;
      case 3: TQ_KVV(3); break;
      case 4: TQ_KVV(4); break;
      case 5: TQ_KVV(5); break;
      case 6: TQ_KVV(6); break;
      case 7: TQ_KVV(7); break;
      default: TQ_KVV(8); break;
    }
#undef TQ_KVV
    TQ_LAUNCH_CHECK();
  }
  if (attend)
    hipLaunchKernelGGL(kv_values_finish_kernel<true>, dim3(static_cast<unsigned>(queries)), dim3(kFinishWaves * 64),
                       0, s, partial, static_cast<int>(chunks), signs, out, ml);
  else
    hipLaunchKernelGGL(kv_values_finish_kernel<false>, dim3(static_cast<unsigned>(queries)), dim3(kFinishWaves * 64),
                       0, s, partial, static_cast<int>(chunks), signs, out, ml);
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}
}  // namespace

int tq_kv_values(const float* p, int heads, int nq, const uint32_t* values, const uint16_t* radius, int64_t n,
                 int bits, const float* signs, const double* levels, float* out, void* workspace, size_t ws_bytes,
                 void* stream) {
  return kv_values_impl(false, p, 0.0f, heads, nq, values, radius, n, bits, signs, levels, out, workspace, ws_bytes,
                        stream);
}

int tq_kv_attend(const float* scores, float scale, int heads, int nq, const uint32_t* values,
                 const uint16_t* radius, int64_t n, int bits, const float* signs, const double* levels, float* out,
                 void* workspace, size_t ws_bytes, void* stream) {
  return kv_values_impl(true, scores, scale, heads, nq, values, radius, n, bits, signs, levels, out, workspace,
                        ws_bytes, stream);
}

}  // extern "C"
