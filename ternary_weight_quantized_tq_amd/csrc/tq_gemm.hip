// Prefill GEMM on packed ternary weights:
//   Y[m][n] = sum_k fp32(s[n][k/128]) t[n][k] x'[m][k],  x' = H_128 x.
//
// Two launches on the caller's stream:
//   1. prep: block-128 transform of every activation row (FP32), split into
//      hi = fp16(x') and lo = fp16(x' - hi), written to the workspace padded
//      to whole tiles (zeros outside M x K).  hi + lo carries ~22 bits of x'.
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

constexpr int BM = 64;          // rows of Y per workgroup
constexpr int BN = 256;         // columns of Y per workgroup (4 wavefronts x 64)
constexpr int BK = 160;         // trits per K step = 2 quads = 8 words
constexpr int kThreads = 256;

#define TQ_LDS_BARRIER() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")

// ------------------------------------------------------------------ prep ---
// One wavefront per (row, block of 128) of the padded [mpad][kpad] output.
__global__ __launch_bounds__(256) void gemm_prep_kernel(const void* __restrict__ x, int dtype, int m, int k,
                                                        int mpad, int kpad, int fused, _Float16* __restrict__ xh,
                                                        _Float16* __restrict__ xl) {
  const int bpr = kpad / 128;
  const long long job = static_cast<long long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (job >= static_cast<long long>(mpad) * bpr) return;
  const int lane = threadIdx.x & 63;
  const int row = static_cast<int>(job / bpr);
  const int kb = static_cast<int>(job % bpr) * 128;
  float v0 = 0.0f, v1 = 0.0f;
  if (row < m && kb < k) {
    load_act2(x, dtype, static_cast<size_t>(row) * k + kb + 2 * lane, v0, v1);
    if (fused) wave_fwht128<float>(v0, v1, lane, kInvSqrt128);
  }
  const _Float16 h0 = static_cast<_Float16>(v0), h1 = static_cast<_Float16>(v1);
  const _Float16 l0 = static_cast<_Float16>(v0 - static_cast<float>(h0));
  const _Float16 l1 = static_cast<_Float16>(v1 - static_cast<float>(h1));
  const size_t o = static_cast<size_t>(row) * kpad + kb + 2 * lane;
  half2_t hh = {h0, h1}, ll = {l0, l1};
  *reinterpret_cast<half2_t*>(xh + o) = hh;
  *reinterpret_cast<half2_t*>(xl + o) = ll;
}

struct GemmArgs {
  const uint4* words;
  const uint16_t* scales;
  const _Float16* xh;
  const _Float16* xl;
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
constexpr int kATiles = BM / 8;           // A tiles of 8 tokens (16 A rows)
constexpr int kAStride = BK + 8;          // halves per A row in LDS (16-byte pad)
constexpr int kARows = 2 * BM;            // A row 2 t + p: part p (hi, lo) of token t
constexpr int kAVecs = kARows * BK / 8 / kThreads;  // uint4 per thread per unit (10)

__device__ __forceinline__ uint2 load_pair_cached(const uint32_t* p) { return *reinterpret_cast<const uint2*>(p); }

__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 As[2][kARows * kAStride];   // 86,016 B
  __shared__ __attribute__((aligned(16))) uint2 codes[81];
  __shared__ __attribute__((aligned(16))) uint16_t ssc[kThreads / 64][kSliceGroups * 64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, j = lane & 15, kb = lane >> 4;
  int mt, nt;
  tile_of(a, mt, nt);
  const int rb = nt * (BN / 64) + wave;
  const bool active = rb < a.nb;
  const int rbc = active ? rb : a.nb - 1;
  const int nsl = slices_per_row(a.k);
  build_code_table(codes, tid, kThreads);

  // Loaders.  Unit u: slice u / 4, unit u % 4 of the slice.
  auto a_src = [&](int u, int i) {  // i-th uint4 of this thread in unit u
    const int idx = tid + i * kThreads;               // 0 .. 2559
    const int part = idx / (BM * BK / 8), rem = idx % (BM * BK / 8);
    const int t = rem / (BK / 8), c = rem % (BK / 8);
    const _Float16* src = part ? a.xl : a.xh;
    return reinterpret_cast<const uint4*>(src + static_cast<size_t>(mt * BM + t) * a.kpad + u * BK + 8 * c);
  };
  auto a_dst = [&](int buf, int i) {
    const int idx = tid + i * kThreads;
    const int part = idx / (BM * BK / 8), rem = idx % (BM * BK / 8);
    const int t = rem / (BK / 8), c = rem % (BK / 8);
    return reinterpret_cast<uint4*>(&As[buf][(2 * t + part) * kAStride + 8 * c]);
  };
  auto pair_ptr = [&](int u, int h) {
    const int s = u >> 2, uu = u & 3;
    return reinterpret_cast<const uint32_t*>(a.words) +
           (row64_quad_base(s, rbc, a.nb) + (2 * uu + (kb >> 1)) * 64 + 16 * h + j) * 4 + 2 * (kb & 1);
  };
  const int sl = lane < kSliceGroups * 8 ? lane : 0;
  auto scale_ptr = [&](int s) {
    return reinterpret_cast<const uint4*>(a.scales + row64_scale_base(s, rbc, a.nb) + 8 * sl);
  };

  // Unit 0 into buffer 0, slice 0's scales.
  uint4 av[kAVecs];
  uint2 wq[4], wn[4];
#pragma unroll
  for (int i = 0; i < kAVecs; ++i) av[i] = *a_src(0, i);
#pragma unroll
  for (int h = 0; h < 4; ++h) wq[h] = load_pair_cached(pair_ptr(0, h));
  uint4 scq = *scale_ptr(0);
#pragma unroll
  for (int i = 0; i < kAVecs; ++i) *a_dst(0, i) = av[i];
  if (lane < kSliceGroups * 8) *reinterpret_cast<uint4*>(&ssc[wave][8 * lane]) = scq;
  TQ_LDS_BARRIER();

  float4_t acc[4][kATiles];
#pragma unroll
  for (int h = 0; h < 4; ++h)
#pragma unroll
    for (int t = 0; t < kATiles; ++t) acc[h][t] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const char* cbase = reinterpret_cast<const char*>(codes);
  // Code-table reads of row quarter h of a unit from its word pair.
  auto decode = [&](uint2 w, uint2 (&cv)[10]) {
    uint32_t o[10];
    word_offsets_s<3, false>(w.x, o);  // no inline asm next to MFMAs
    word_offsets_s<3, false>(w.y, o + 5);
#pragma unroll
    for (int c = 0; c < 10; ++c) cv[c] = *reinterpret_cast<const uint2*>(cbase + o[c]);
  };

  // Software pipeline: while unit u's MFMAs run, row quarter st of unit
  // u + 1 is decoded (its words were loaded during unit u - 1), unit u + 1's
  // activations are loaded for the other LDS buffer and unit u + 2's words
  // are requested.
  uint2 cv[4][10];
#pragma unroll
  for (int h = 0; h < 4; ++h) decode(wq[h], cv[h]);
#pragma unroll
  for (int h = 0; h < 4; ++h) wq[h] = load_pair_cached(pair_ptr(min(1, a.steps - 1), h));  // unit 1
  for (int s = 0; s < nsl; ++s) {
    _Float16 sc[4][kSliceGroups];  // this lane's rows 16 h + j, the slice's five groups
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int g = 0; g < kSliceGroups; ++g)
        sc[h][g] = __builtin_bit_cast(_Float16, ssc[wave][g * 64 + 16 * h + j]);
#pragma unroll
    for (int uu = 0; uu < 4; ++uu) {
      const int u = 4 * s + uu;
      if (u >= a.steps) break;
      const int buf = u & 1;
      const bool more = u + 1 < a.steps;
      const int un = more ? u + 1 : u;  // clamped to this unit on the last one
#pragma unroll
      for (int i = 0; i < kAVecs; ++i) av[i] = *a_src(un, i);
      if (uu == 3) scq = *scale_ptr(min(s + 1, nsl - 1));
      uint2 cvn[4][10];
      const _Float16* abase = &As[buf][j * kAStride + 8 * kb];
#pragma unroll
      for (int st = 0; st < 5; ++st) {
        const int g = (160 * uu + 32 * st) / 128;  // compile-time: one scale group per step
        half8_t af[kATiles];
#pragma unroll
        for (int t = 0; t < kATiles; ++t)
          af[t] = *reinterpret_cast<const half8_t*>(abase + 16 * t * kAStride + 32 * st);
        if (st < 4) {
          decode(wq[st], cvn[st]);
        } else {
#pragma unroll
          for (int h = 0; h < 4; ++h) wn[h] = load_pair_cached(pair_ptr(min(u + 2, a.steps - 1), h));
        }
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const uint4 bq = make_uint4(cv[h][2 * st].x, cv[h][2 * st].y, cv[h][2 * st + 1].x, cv[h][2 * st + 1].y);
          const half8_t b = __builtin_bit_cast(half8_t, bq) * sc[h][g];
#pragma unroll
          for (int t = 0; t < kATiles; ++t)
            acc[h][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[t], b, acc[h][t], 0, 0, 0);
        }
      }
      if (more) {
#pragma unroll
        for (int i = 0; i < kAVecs; ++i) *a_dst(buf ^ 1, i) = av[i];
      }
      if (uu == 3 && lane < kSliceGroups * 8) *reinterpret_cast<uint4*>(&ssc[wave][8 * lane]) = scq;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        wq[h] = wn[h];
#pragma unroll
        for (int c = 0; c < 10; ++c) cv[h][c] = cvn[h][c];
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
    for (int t = 0; t < kATiles; ++t)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int row = mt * BM + 8 * t + 2 * kb + q;
        if (row < a.m) {
          float* yp = a.y + static_cast<size_t>(row) * a.n + col;
          const float v = acc[h][t][2 * q] + acc[h][t][2 * q + 1];
          *yp = a.accumulate ? *yp + v : v;
        }
      }
  }
}

struct GemmPlan {
  int mpad, kpad, mtiles, ntiles, steps;
  size_t xh_bytes, total;
};

GemmPlan plan_gemm(int n, int k, int m) {
  GemmPlan p;
  p.mtiles = (m + BM - 1) / BM;
  p.ntiles = (n + BN - 1) / BN;
  p.mpad = p.mtiles * BM;
  p.steps = (k + BK - 1) / BK;
  p.kpad = p.steps * BK;
  if (p.kpad % 128) p.kpad = (p.kpad + 127) / 128 * 128;  // prep works in blocks of 128
  p.xh_bytes = (static_cast<size_t>(p.mpad) * p.kpad * 2 + 255) & ~static_cast<size_t>(255);
  p.total = 2 * p.xh_bytes;
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
  if (flags & ~static_cast<unsigned>(TQ_FWHT_FUSED | TQ_ACCUMULATE)) return TQ_EINVAL;
  if (m < 1) return TQ_ESHAPE;
  const GemmPlan p = plan_gemm(w->n, w->k, m);
  if (ws_bytes < p.total) return TQ_ENOSPACE;
  if (static_cast<long long>(p.mtiles) * p.ntiles > INT_MAX) return TQ_ESHAPE;
  _Float16* xh = static_cast<_Float16*>(workspace);
  _Float16* xl = reinterpret_cast<_Float16*>(static_cast<char*>(workspace) + p.xh_bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const long long jobs = static_cast<long long>(p.mpad) * (p.kpad / 128);
  hipLaunchKernelGGL(gemm_prep_kernel, dim3(static_cast<unsigned>((jobs + 3) / 4)), dim3(256), 0, s, x, x_dtype, m,
                     w->k, p.mpad, p.kpad, (flags & TQ_FWHT_FUSED) ? 1 : 0, xh, xl);
  TQ_LAUNCH_CHECK();
  GemmArgs a;
  a.words = reinterpret_cast<const uint4*>(w->words);
  a.scales = w->scales;
  a.xh = xh;
  a.xl = xl;
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
  hipLaunchKernelGGL(gemm_kernel, dim3(p.mtiles * p.ntiles), dim3(kThreads), 0, s, a);
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}
