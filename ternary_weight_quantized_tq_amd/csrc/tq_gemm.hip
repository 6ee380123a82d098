// Prefill GEMM on packed ternary weights:
//   Y[m][n] = sum_k fp32(s[n][k/128]) t[n][k] x'[m][k],  x' = H_128 x.
//
// Two launches on the caller's stream:
//   1. prep: block-128 transform of every activation row (FP32), scaled by
//      a power of two 2^e per row (max |x'| 2^e in [2^13, 2^14), so neither
//      part overflows or goes subnormal whatever the activations' scale),
//      split into hi = fp16(x' 2^e) and lo = fp16(x' 2^e - hi), written to the
//      workspace padded to whole tiles (zeros outside M x K) with e per
//      row.  hi + lo carries ~22 bits of x'; the epilogue multiplies by 2^-e.
//   2. gemm: each workgroup computes a 64 x 256 tile of Y on the matrix cores
//      (v_mfma_f32_16x16x32_f16; see gemm_kernel).  The weights' B operands
//      are decoded from the packed words straight into registers as fp16
//      s*t, which is exact because t is in {-1, 0, 1}, so the per-group
//      scale is applied before the product and no separate FP32 scale pass
//      is needed; hi and lo of x' are separate A rows.  FP32 accumulation.
// Weights stream once per 64-row M tile; tiles are ordered so that all N
// tiles of one M tile run on one XCD, keeping that activation tile (64 x K x
// 4 bytes) in the XCD's L2.
#include "tq_internal.h"

#include <limits.h>

using namespace tq;

namespace {

constexpr int BM = 64;          // rows of Y per workgroup with x' in two fp16 parts (128 with one)
constexpr int BN = 256;         // columns of Y per workgroup (4 wavefronts x 64)
constexpr int BK = 160;         // trits per K step = 2 quads = 8 words
constexpr int kThreads = 256;
// Wavefronts per row block in gemm_kernel: with x' in two fp16 parts one
// (the in-wavefront software pipeline; two measured 0.864 against 0.854
// ms), with one part (TQ_FAST_F16) two (0.481 against 0.506 ms).
template <int P>
constexpr int gemm_ts() { return P == 2 ? 1 : 2; }

#define TQ_LDS_BARRIER() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")

// ------------------------------------------------------------------ prep ---
// One workgroup per row of the padded [mpad][kpad] A rows; wavefront w takes
// blocks of 128 w, w + 4, ...  Pass 1 finds the row's max |x'|, pass 2
// transforms again (the row is in L2 by then), scales by 2^e and splits.
__device__ __forceinline__ void prep_block(const void* __restrict__ x, int dtype, int row, int m, int k, int kb,
                                           int fused, int lane, float& v0, float& v1) {
  v0 = 0.0f;
  v1 = 0.0f;
  if (row < m && kb < k) {
    load_act2(x, dtype, static_cast<size_t>(row) * k + kb + 2 * lane, v0, v1);
    if (fused) wave_fwht128<float>(v0, v1, lane, kInvSqrt128);
  }
}

__global__ __launch_bounds__(256) void gemm_prep_kernel(const void* __restrict__ x, int dtype, int m, int k,
                                                        int kpad, int fused, int parts, _Float16* __restrict__ xh,
                                                        _Float16* __restrict__ xl, int* __restrict__ xe) {
  __shared__ float wmax[4];
  const int row = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nblk = kpad / 128;
  float mx = 0.0f;
  for (int b = wave; b < nblk; b += 4) {
    float v0, v1;
    prep_block(x, dtype, row, m, k, b * 128, fused, lane, v0, v1);
    mx = fmaxf(mx, fmaxf(fabsf(v0), fabsf(v1)));
  }
  mx = wave_max(mx, lane);
  if (lane == 0) wmax[wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const int e = mx > 0.0f ? 14 - __builtin_amdgcn_frexp_expf(mx) : 0;
  if (threadIdx.x == 0) xe[row] = e;
  for (int b = wave; b < nblk; b += 4) {
    float v0, v1;
    prep_block(x, dtype, row, m, k, b * 128, fused, lane, v0, v1);
    const float s0 = ldexpf(v0, e), s1 = ldexpf(v1, e);
    const _Float16 h0 = static_cast<_Float16>(s0), h1 = static_cast<_Float16>(s1);
    const half2_t hh = {h0, h1};
    const half2_t ll = {static_cast<_Float16>(s0 - static_cast<float>(h0)),
                        static_cast<_Float16>(s1 - static_cast<float>(h1))};
    const size_t o = static_cast<size_t>(row) * kpad + b * 128 + 2 * lane;
    *reinterpret_cast<half2_t*>(xh + o) = hh;
    if (parts == 2) *reinterpret_cast<half2_t*>(xl + o) = ll;
  }
}

struct GemmArgs {
  const uint4* words;
  const uint16_t* scales;
  const _Float16* xh;
  const _Float16* xl;
  const int* xe;  // per padded row: the power of two applied to x' before the split
  float* y;
  int m, n, k, kpad, nb, groups, mtiles, ntiles, steps, xcd_map;
  int accumulate;  // TQ_ACCUMULATE: y += (one workgroup per output tile: no atomics)
};

// Tile of this workgroup: all N tiles of an M tile on one XCD (workgroups
// are dispatched to the 8 XCDs round-robin by id) when M tiles divide by 8.
__device__ __forceinline__ void tile_of(const GemmArgs& a, int& mt, int& nt) {
  const int b = blockIdx.x;
  if (a.xcd_map) {
    const int xcd = b & 7, j = b >> 3;
    mt = xcd + 8 * (j / a.ntiles);
    nt = j % a.ntiles;
  } else {
    mt = b / a.ntiles;
    nt = b % a.ntiles;
  }
}

// Main kernel.  Workgroup (M tile of 64 tokens, N tile of 256 weight rows);
// wavefront w owns weight rows 64 (4 nt + w) .. + 63 and all 64 tokens.
// Per 160-trit unit (K step) and row quarter h, a lane decodes its row's
// word pair exactly as the M >= 2 decode GEMV does (lane j = l % 16 takes
// row 16 h + j, lane group kb = l / 16 words 2 kb, 2 kb + 1 of the unit),
// giving the B operands of the unit's five 32-trit steps of
// v_mfma_f32_16x16x32_f16 straight in registers: fp16 codes from the
// 81-entry table, times the row's fp16 group scale (s*t is exact in fp16).
// Each B operand then serves eight A tiles (8 tokens x {hi, lo} each), so
// one table read feeds eight MFMAs.  The activation tile of the unit (64
// tokens x 160 trits, hi and lo rows) is double-buffered in LDS; the next
// unit's activations, word pairs and (at a slice boundary) scales are
// loaded while the current unit's MFMAs run.  One barrier per unit.
constexpr int kATiles = 8;                // A tiles of 16 A rows
constexpr int kAStride = BK + 8;          // halves per A row in LDS (16-byte pad)
constexpr int kARows = 16 * kATiles;      // 128 A rows: 64 tokens x (hi, lo), or 128 tokens (one fp16 part)
constexpr int kAVecs = kARows * BK / 8 / kThreads;  // uint4 per thread per unit (10)
// A rows of a workgroup: with P = 2 parts (the default), A row 2 t + p is
// part p (hi, lo) of token t, 64 tokens; with P = 1 (TQ_FAST_F16) A row t is
// token t, 128 tokens.
template <int P>
__device__ __forceinline__ void a_row_of(int idx, int& t, int& part, int& c) {
  constexpr int kTok = kARows / P;
  part = P == 2 ? idx / (kTok * BK / 8) : 0;
  const int rem = P == 2 ? idx % (kTok * BK / 8) : idx;
  t = rem / (BK / 8);
  c = rem % (BK / 8);
}

__device__ __forceinline__ uint2 load_pair_cached(const uint32_t* p) { return *reinterpret_cast<const uint2*>(p); }

// G: scale groups per slice (5 at group 128, 10 at group 64).  TS: wavefronts
// per row block (1: one wavefront takes all eight A tiles; 2: wavefronts w
// and w + 4 share row block w % 4, A tiles 0-3 and 4-7, and both decode its
// words, so that two wavefronts per SIMD hide each other's latencies).
template <int G, int P, int TS>
__global__ __launch_bounds__(kThreads * TS) void gemm_kernel(GemmArgs a) {
  constexpr int kT = kThreads * TS;        // threads per workgroup
  constexpr int kTiles = kATiles / TS;     // A tiles per wavefront
  constexpr int kAV = kARows * BK / 8 / kT;  // uint4 of the activation tile per thread per unit
  constexpr int kTok = kARows / P;  // tokens per workgroup
  constexpr int kGroup = kSliceTrits / G;
  constexpr int kScaleVecs = G * 64 / 8;  // 16-byte vectors of one block's slice scales
  constexpr int kScaleLoads = (kScaleVecs + 63) / 64;
  __shared__ __attribute__((aligned(16))) _Float16 As[2][kARows * kAStride];   // 86,016 B
  __shared__ __attribute__((aligned(16))) uint2 codes[81];
  __shared__ __attribute__((aligned(16))) uint16_t ssc[kT / 64][G * 64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, j = lane & 15, kb = lane >> 4;
  const int t0 = (wave / 4) * kTiles;  // this wavefront's first A tile
  int mt, nt;
  tile_of(a, mt, nt);
  const int rb = nt * (BN / 64) + wave % 4;
  const bool active = rb < a.nb;
  const int rbc = active ? rb : a.nb - 1;
  const int nsl = slices_per_row(a.k);
  build_code_table(codes, tid, kT);

  // Loaders.  Unit u: slice u / 4, unit u % 4 of the slice.
  auto a_src = [&](int u, int i) {  // i-th uint4 of this thread in unit u
    const int idx = tid + i * kT;                     // 0 .. 2559
    int t, part, c;
    a_row_of<P>(idx, t, part, c);
    const _Float16* src = part ? a.xl : a.xh;
    return reinterpret_cast<const uint4*>(src + static_cast<size_t>(mt * kTok + t) * a.kpad + u * BK + 8 * c);
  };
  auto a_dst = [&](int buf, int i) {
    const int idx = tid + i * kT;
    int t, part, c;
    a_row_of<P>(idx, t, part, c);
    return reinterpret_cast<uint4*>(&As[buf][(P * t + part) * kAStride + 8 * c]);
  };
  auto pair_ptr = [&](int u, int h) {
    const int s = u >> 2, uu = u & 3;
    return reinterpret_cast<const uint32_t*>(a.words) +
           (row64_quad_base(s, rbc, a.nb) + (2 * uu + (kb >> 1)) * 64 + 16 * h + j) * 4 + 2 * (kb & 1);
  };
  // A block's slice scales are kScaleVecs 16-byte vectors: lane l loads
  // vector l (clamped; every lane loads, since a load under a lane condition
  // is waited for at once) and, at group 64, vector 64 + l.
  static_assert(kScaleLoads <= 2, "at most two scale vectors per lane");
  const int sl = lane < kScaleVecs ? lane : 0;
  const int sl2 = lane + 64 < kScaleVecs ? lane + 64 : 0;
  auto scale_ptr = [&](int s, int v) {
    return reinterpret_cast<const uint4*>(a.scales + row64_scale_base(s, rbc, a.nb, G) + 8 * v);
  };

  // Unit 0 into buffer 0, slice 0's scales.
  uint4 av[kAV];
  uint2 wq[4], wn[4];
#pragma unroll
  for (int i = 0; i < kAV; ++i) av[i] = *a_src(0, i);
#pragma unroll
  for (int h = 0; h < 4; ++h) wq[h] = load_pair_cached(pair_ptr(0, h));
  uint4 scq = *scale_ptr(0, sl), scq2 = scq;
  if constexpr (kScaleLoads > 1) scq2 = *scale_ptr(0, sl2);
#pragma unroll
  for (int i = 0; i < kAV; ++i) *a_dst(0, i) = av[i];
  if (lane < kScaleVecs) *reinterpret_cast<uint4*>(&ssc[wave][8 * lane]) = scq;
  if constexpr (kScaleLoads > 1)
    if (lane + 64 < kScaleVecs) *reinterpret_cast<uint4*>(&ssc[wave][8 * (lane + 64)]) = scq2;
  TQ_LDS_BARRIER();

  float4_t acc[4][kTiles];
#pragma unroll
  for (int h = 0; h < 4; ++h)
#pragma unroll
    for (int t = 0; t < kTiles; ++t) acc[h][t] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const char* cbase = reinterpret_cast<const char*>(codes);
  // Code-table reads of row quarter h of a unit from its word pair.
  auto decode = [&](uint2 w, uint2 (&cv)[10]) {
    uint32_t o[10];
    word_offsets_s<3, false>(w.x, o);  // no inline asm next to MFMAs
    word_offsets_s<3, false>(w.y, o + 5);
#pragma unroll
    for (int c = 0; c < 10; ++c) cv[c] = *reinterpret_cast<const uint2*>(cbase + o[c]);
  };

  // Software pipeline (TS = 1): while unit u's MFMAs run, row quarter st of
  // unit u + 1 is decoded (its words were loaded during unit u - 1), unit
  // u + 1's activations are loaded for the other LDS buffer and unit u + 2's
  // words are requested.  With TS = 2 the registers do not hold two units'
  // codes: a wavefront decodes its unit at the unit's start and requests
  // the next unit's words, and the other wavefront on its SIMD covers the
  // wait.
  uint2 cv[4][10];
  if constexpr (TS == 1) {
#pragma unroll
    for (int h = 0; h < 4; ++h) decode(wq[h], cv[h]);
#pragma unroll
    for (int h = 0; h < 4; ++h) wq[h] = load_pair_cached(pair_ptr(min(1, a.steps - 1), h));  // unit 1
  }
  for (int s = 0; s < nsl; ++s) {
    _Float16 sc[4][G];  // this lane's rows 16 h + j, the slice's G groups
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int g = 0; g < G; ++g)
        sc[h][g] = __builtin_bit_cast(_Float16, ssc[wave][g * 64 + 16 * h + j]);
#pragma unroll
    for (int uu = 0; uu < 4; ++uu) {
      const int u = 4 * s + uu;
      if (u >= a.steps) break;
      const int buf = u & 1;
      const bool more = u + 1 < a.steps;
      const int un = more ? u + 1 : u;  // clamped to this unit on the last one
#pragma unroll
      for (int i = 0; i < kAV; ++i) av[i] = *a_src(un, i);
      if (uu == 3) {
        scq = *scale_ptr(min(s + 1, nsl - 1), sl);
        if constexpr (kScaleLoads > 1) scq2 = *scale_ptr(min(s + 1, nsl - 1), sl2);
      }
      uint2 cvn[4][10];
      if constexpr (TS == 2) {
#pragma unroll
        for (int h = 0; h < 4; ++h) decode(wq[h], cv[h]);
#pragma unroll
        for (int h = 0; h < 4; ++h) wq[h] = load_pair_cached(pair_ptr(un, h));
      }
      const _Float16* abase = &As[buf][j * kAStride + 8 * kb];
#pragma unroll
      for (int st = 0; st < 5; ++st) {
        const int g = (160 * uu + 32 * st) / kGroup;  // compile-time: one scale group per step
        half8_t af[kTiles];
#pragma unroll
        for (int t = 0; t < kTiles; ++t)
          af[t] = *reinterpret_cast<const half8_t*>(abase + 16 * (t0 + t) * kAStride + 32 * st);
        if constexpr (TS == 1) {
          if (st < 4) {
            decode(wq[st], cvn[st]);
          } else {
#pragma unroll
            for (int h = 0; h < 4; ++h) wn[h] = load_pair_cached(pair_ptr(min(u + 2, a.steps - 1), h));
          }
        }
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const uint4 bq = make_uint4(cv[h][2 * st].x, cv[h][2 * st].y, cv[h][2 * st + 1].x, cv[h][2 * st + 1].y);
          const half8_t b = __builtin_bit_cast(half8_t, bq) * sc[h][g];
#pragma unroll
          for (int t = 0; t < kTiles; ++t)
            acc[h][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[t], b, acc[h][t], 0, 0, 0);
        }
      }
      if (more) {
#pragma unroll
        for (int i = 0; i < kAV; ++i) *a_dst(buf ^ 1, i) = av[i];
      }
      if (uu == 3) {
        if (lane < kScaleVecs) *reinterpret_cast<uint4*>(&ssc[wave][8 * lane]) = scq;
        if constexpr (kScaleLoads > 1)
          if (lane + 64 < kScaleVecs) *reinterpret_cast<uint4*>(&ssc[wave][8 * (lane + 64)]) = scq2;
      }
      if constexpr (TS == 1) {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          wq[h] = wn[h];
#pragma unroll
          for (int c = 0; c < 10; ++c) cv[h][c] = cvn[h][c];
        }
      }
      TQ_LDS_BARRIER();
    }
  }

  // D rows 4 kb + v of A tile t: v = 0, 1 the parts of token 8 t + 2 kb,
  // v = 2, 3 those of token 8 t + 2 kb + 1; column j = row 16 h + j.
  if (!active) return;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int col = rb * 64 + 16 * h + j;
    if (col >= a.n) continue;
#pragma unroll
    for (int t = 0; t < kTiles; ++t)
#pragma unroll
      for (int q = 0; q < 4 / P; ++q) {
        // D row 4 kb + v of A tile t0 + t: P = 2, token 8 (t0 + t) + 2 kb + q
        // from v = 2q (hi) and 2q + 1 (lo); P = 1, token 16 (t0 + t) + 4 kb + q.
        const int row = mt * kTok + (16 / P) * (t0 + t) + (4 / P) * kb + q;
        if (row < a.m) {
          float* yp = a.y + static_cast<size_t>(row) * a.n + col;
          const float sum = P == 2 ? acc[h][t][2 * q] + acc[h][t][2 * q + 1] : acc[h][t][q];
          const float v = ldexpf(sum, -a.xe[row]);
          *yp = a.accumulate ? *yp + v : v;
        }
      }
  }
}

// Binary {-c, +c} variant (32 sign bits per word, bit i of slice word w is
// weight 32 w + i).  Same tile and A staging as gemm_kernel; the B operand of
// step s (weights 32 s .. 32 s + 31 of the slice) for lane group kb is byte
// kb of word s of the lane's row, mapped by a 256-entry LDS table to its
// eight fp16 signs and multiplied by the row's fp16 scale (exact).  Each
// lane loads its five bytes of a unit directly (byte loads of the words'
// cache lines); the next unit's bytes and activations are loaded while the
// current unit's MFMAs run.
template <int G, int P>
__global__ __launch_bounds__(kThreads) void gemm_bin_kernel(GemmArgs a) {
  constexpr int kTok = kARows / P;  // tokens per workgroup
  constexpr int kStepsPerGroup = kSliceTrits / G / 32;
  constexpr int kScaleVecs = G * 64 / 8;
  __shared__ __attribute__((aligned(16))) _Float16 As[2][kARows * kAStride];
  __shared__ __attribute__((aligned(16))) uint4 codes[256];
  __shared__ __attribute__((aligned(16))) uint16_t ssc[kThreads / 64][G * 64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, j = lane & 15, kb = lane >> 4;
  int mt, nt;
  tile_of(a, mt, nt);
  const int rb = nt * (BN / 64) + wave;
  const bool active = rb < a.nb;
  const int rbc = active ? rb : a.nb - 1;
  const int nsl = slices_per_row(a.k);
  for (int c = tid; c < 256; c += kThreads) {
    uint32_t d[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      d[i] = (((c >> (2 * i)) & 1) ? 0x3c00u : 0xbc00u) | ((((c >> (2 * i + 1)) & 1) ? 0x3c00u : 0xbc00u) << 16);
    codes[c] = make_uint4(d[0], d[1], d[2], d[3]);
  }
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  auto a_src = [&](int u, int i) {
    const int idx = tid + i * kThreads;
    int t, part, c;
    a_row_of<P>(idx, t, part, c);
    const _Float16* src = part ? a.xl : a.xh;
    return reinterpret_cast<const u32x4_t*>(src + static_cast<size_t>(mt * kTok + t) * a.kpad + u * BK + 8 * c);
  };
  auto a_dst = [&](int buf, int i) {
    const int idx = tid + i * kThreads;
    int t, part, c;
    a_row_of<P>(idx, t, part, c);
    return reinterpret_cast<u32x4_t*>(&As[buf][(P * t + part) * kAStride + 8 * c]);
  };
  // Byte kb of word 5 (u % 4) + st of slice u / 4, row 64 rb + 16 h + j.
  const uint8_t* wbytes = reinterpret_cast<const uint8_t*>(a.words);
  auto byte_ptr = [&](int u, int h, int st) {
    const int w = 5 * (u & 3) + st;
    const size_t qb = row64_quad_base_bin(u >> 2, rbc, a.nb);
    return wbytes + ((qb + (w >> 2) * 64 + 16 * h + j) * 4 + (w & 3)) * 4 + kb;
  };
  auto stage_scales = [&](int sl) {
    const uint16_t* sb = a.scales + row64_scale_base(sl, rbc, a.nb, G);
    for (int v = lane; v < kScaleVecs; v += 64)
      *reinterpret_cast<uint4*>(&ssc[wave][8 * v]) = *reinterpret_cast<const uint4*>(sb + 8 * v);
  };
  auto scale16 = [&](int h, int g) {
    const uint16_t v = reinterpret_cast<const volatile uint16_t*>(&ssc[wave][0])[g * 64 + 16 * h + j];
    return active ? __builtin_bit_cast(_Float16, v) : static_cast<_Float16>(0.0f);
  };

  u32x4_t av[kAVecs];
  uint32_t bcur[4][5], bnext[4][5];
#pragma unroll
  for (int i = 0; i < kAVecs; ++i) av[i] = *a_src(0, i);
#pragma unroll
  for (int h = 0; h < 4; ++h)
#pragma unroll
    for (int st = 0; st < 5; ++st) bcur[h][st] = *byte_ptr(0, h, st);
#pragma unroll
  for (int i = 0; i < kAVecs; ++i) *a_dst(0, i) = av[i];
  stage_scales(0);
  __syncthreads();

  float4_t acc[4][kATiles];
#pragma unroll
  for (int h = 0; h < 4; ++h)
#pragma unroll
    for (int t = 0; t < kATiles; ++t) acc[h][t] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const char* cbase = reinterpret_cast<const char*>(codes);
  for (int u = 0; u < a.steps; ++u) {
    const int buf = u & 1, uu = u & 3, sl = u >> 2;
    const bool more = u + 1 < a.steps;
    const int un = more ? u + 1 : u;
#pragma unroll
    for (int i = 0; i < kAVecs; ++i) av[i] = *a_src(un, i);
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int st = 0; st < 5; ++st) bnext[h][st] = *byte_ptr(un, h, st);
    const _Float16* abase = &As[buf][j * kAStride + 8 * kb];
#pragma unroll
    for (int st = 0; st < 5; ++st) {
      const int step = 5 * uu + st;  // step of the slice
      half8_t af[kATiles];
#pragma unroll
      for (int t = 0; t < kATiles; ++t) af[t] = *reinterpret_cast<const half8_t*>(abase + 16 * t * kAStride + 32 * st);
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const half8_t b = *reinterpret_cast<const half8_t*>(cbase + (bcur[h][st] << 4)) *
                          scale16(h, step / kStepsPerGroup);
#pragma unroll
        for (int t = 0; t < kATiles; ++t)
          acc[h][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[t], b, acc[h][t], 0, 0, 0);
      }
    }
    __syncthreads();  // every wavefront is done with buffer buf ^ 1 and with this slice's scales
    if (more) {
#pragma unroll
      for (int i = 0; i < kAVecs; ++i) *a_dst(buf ^ 1, i) = av[i];
      if (uu == 3) stage_scales(min(sl + 1, nsl - 1));
    }
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int st = 0; st < 5; ++st) bcur[h][st] = bnext[h][st];
    __syncthreads();
  }

  if (!active) return;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int col = rb * 64 + 16 * h + j;
    if (col >= a.n) continue;
#pragma unroll
    for (int t = 0; t < kATiles; ++t)
#pragma unroll
      for (int q = 0; q < 4 / P; ++q) {
        // D row 4 kb + v of A tile t: P = 2, token 8 t + 2 kb + q from v = 2q (hi)
        // and 2q + 1 (lo); P = 1, token 16 t + 4 kb + q.
        const int row = mt * kTok + (16 / P) * t + (4 / P) * kb + q;
        if (row < a.m) {
          float* yp = a.y + static_cast<size_t>(row) * a.n + col;
          const float sum = P == 2 ? acc[h][t][2 * q] + acc[h][t][2 * q + 1] : acc[h][t][q];
          const float v = ldexpf(sum, -a.xe[row]);
          *yp = a.accumulate ? *yp + v : v;
        }
      }
  }
}

struct GemmPlan {
  int mpad, kpad, mtiles, ntiles, steps;
  size_t xh_bytes, xe_bytes, total;
};

GemmPlan plan_gemm(int n, int k, int m) {
  GemmPlan p;
  p.mtiles = (m + BM - 1) / BM;
  p.ntiles = (n + BN - 1) / BN;
  p.mpad = (m + kARows - 1) / kARows * kARows;  // whole tiles of either A-row mode
  p.steps = (k + BK - 1) / BK;
  p.kpad = p.steps * BK;
  if (p.kpad % 128) p.kpad = (p.kpad + 127) / 128 * 128;  // prep works in blocks of 128
  p.xh_bytes = (static_cast<size_t>(p.mpad) * p.kpad * 2 + 255) & ~static_cast<size_t>(255);
  p.xe_bytes = (static_cast<size_t>(p.mpad) * 4 + 255) & ~static_cast<size_t>(255);
  p.total = 2 * p.xh_bytes + p.xe_bytes;
  return p;
}

}  // namespace

size_t tq_gemm_workspace(int n, int k, int m) { return plan_gemm(n, k, m).total; }

extern "C" int tq_gemm(const tq_weights* w, const void* x, int x_dtype, int m, float* y, unsigned flags,
                       void* workspace, size_t ws_bytes, void* stream) {
  int st = tq_check_weights(w, 1);
  if (st != TQ_OK) return st;
  if (!x || !y || !workspace) return TQ_EINVAL;
  if (x_dtype != TQ_F32 && x_dtype != TQ_BF16 && x_dtype != TQ_F16) return TQ_EINVAL;
  if (!tq_aligned(x, tq_act_align(x_dtype)) || !tq_aligned(y, 4) || !tq_aligned(workspace, 16)) return TQ_EINVAL;
  if (flags & ~static_cast<unsigned>(TQ_FWHT_FUSED | TQ_ACCUMULATE | TQ_FAST_F16)) return TQ_EINVAL;
  if (!tq_dim_ok(m)) return TQ_ESHAPE;
  GemmPlan p = plan_gemm(w->n, w->k, m);
  const int parts = (flags & TQ_FAST_F16) ? 1 : 2;
  p.mtiles = (m + kARows / parts - 1) / (kARows / parts);
  if (ws_bytes < p.total) return TQ_ENOSPACE;
  if (static_cast<long long>(p.mtiles) * p.ntiles > INT_MAX) return TQ_ESHAPE;
  _Float16* xh = static_cast<_Float16*>(workspace);
  _Float16* xl = reinterpret_cast<_Float16*>(static_cast<char*>(workspace) + p.xh_bytes);
  int* xe = reinterpret_cast<int*>(static_cast<char*>(workspace) + 2 * p.xh_bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(gemm_prep_kernel, dim3(static_cast<unsigned>(p.mpad)), dim3(256), 0, s, x, x_dtype, m, w->k,
                     p.kpad, (flags & TQ_FWHT_FUSED) ? 1 : 0, parts, xh, xl, xe);
  TQ_LAUNCH_CHECK();
  GemmArgs a;
  a.words = reinterpret_cast<const uint4*>(w->words);
  a.scales = w->scales;
  a.xh = xh;
  a.xl = xl;
  a.xe = xe;
  a.y = y;
  a.m = m;
  a.n = w->n;
  a.k = w->k;
  a.kpad = p.kpad;
  a.nb = row_blocks(w->n);
  a.groups = w->k / TQ_GROUP;
  a.mtiles = p.mtiles;
  a.ntiles = p.ntiles;
  a.steps = p.steps;
  a.xcd_map = (p.mtiles % 8 == 0) ? 1 : 0;
  a.accumulate = (flags & TQ_ACCUMULATE) ? 1 : 0;
  const dim3 grid(p.mtiles * p.ntiles);
  const bool g5 = slice_groups(w->group) == 5;
  const dim3 blk(kThreads);
  if (w->levels == 2) {
    if (parts == 2) {
      if (g5) hipLaunchKernelGGL((gemm_bin_kernel<5, 2>), grid, blk, 0, s, a);
      else hipLaunchKernelGGL((gemm_bin_kernel<10, 2>), grid, blk, 0, s, a);
    } else {
      if (g5) hipLaunchKernelGGL((gemm_bin_kernel<5, 1>), grid, blk, 0, s, a);
      else hipLaunchKernelGGL((gemm_bin_kernel<10, 1>), grid, blk, 0, s, a);
    }
  } else {
    if (parts == 2) {
      const dim3 b2(kThreads * gemm_ts<2>());
      if (g5) hipLaunchKernelGGL((gemm_kernel<5, 2, gemm_ts<2>()>), grid, b2, 0, s, a);
      else hipLaunchKernelGGL((gemm_kernel<10, 2, gemm_ts<2>()>), grid, b2, 0, s, a);
    } else {
      const dim3 b1(kThreads * gemm_ts<1>());
      if (g5) hipLaunchKernelGGL((gemm_kernel<5, 1, gemm_ts<1>()>), grid, b1, 0, s, a);
      else hipLaunchKernelGGL((gemm_kernel<10, 1, gemm_ts<1>()>), grid, b1, 0, s, a);
    }
  }
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}
