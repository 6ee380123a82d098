// Routed ternary expert MLP (TurboQuant-MLX page, section "Why 1.58 bit did
// not turn into gibberish", point 1: 256 routed experts, 8 active per token,
// only the experts ternary, the router gate at full precision).
//
// tq_moe_route: softmax over the expert logits, top-k, renormalised weights.
// tq_moe_gemv with at most 64 (token, slot) pairs, two launches:
//   1. gate/up:  grid (pair, 64-row block of the intermediate dimension,
//                640-trit slice of the hidden size), no bucketing; the
//                slice's partial sums are stored.
//   2. down:     below four tokens, grid (pair, 64-row block of the hidden
//                size), one wavefront per unit: adds the gate/up partials in
//                order, h = silu(gate) * up, the block-128 transform, the
//                down rows, the route weight; the last slot of a token to
//                finish adds the slots' rows in slot order and stores y.
//                From four tokens on, grid (token, 64-row block), one
//                wavefront per slot, the slots' rows added in LDS.
// Otherwise four launches on the caller's stream:
//   1. bucket:   one workgroup groups the (token, slot) pairs by expert and
//                lists the experts that received tokens (ascending id).
//   2. gate/up:  grid (active expert slot, 64-row block of the intermediate
//                dimension, 640-trit slice of K = the hidden size).
//                Wavefronts 0, 1 own the gate rows 64b..64b+63, 2, 3 the up
//                rows I+64b.., each half of the slice's 160-trit units.
//                Tokens of the expert go 1..8 at a time through the matrix
//                cores as in the M >= 2 decode GEMV: the block-128
//                transformed activations as two fp16 parts in the A rows (a
//                power of two per token and slice keeps them in range),
//                fp16 trit codes from an 81-entry table as B; stores
//                h = silu(gate) * up.
//   3. down:     grid (active expert slot, 4 row blocks of the hidden size),
//                one row block per wavefront, the same contraction after
//                the block-128 transform of h; each (token, slot) pair's
//                output row is stored.
//   4. combine:  y[t] = sum_j route_w[t][j] * o[t][j] in slot order.
// Only experts that received tokens are read; every pair's arithmetic is
// independent of which other pairs share its tile, so results do not depend
// on the order the bucket step lists pairs in.
#include "tq_internal.h"

#include <limits.h>

using namespace tq;

namespace {

constexpr int kTile = 8;          // tokens per pass
constexpr int kFusedMaxPairs = 64;  // the one-launch and per-pair paths: at most 64 (token, slot) pairs
constexpr int kMoeG = 5;          // scale groups per slice: the expert path takes group 128
constexpr int kMaxExperts = 1024;


struct MoeArgs {
  const uint4* gu_words;
  const uint16_t* gu_scales;
  const uint4* dn_words;
  const uint16_t* dn_scales;
  size_t gu_wstride, gu_sstride, dn_wstride, dn_sstride;  // per expert, in quads / scales
  const void* x;
  int x_dtype;
  const int32_t* ids;
  const float* route_w;
  float* y;
  int t, topk, experts, hidden, inter;
  int fused;
  int accumulate;    // TQ_ACCUMULATE: y += the layer's output
  // workspace
  int* bad;          // [1] number of (token, slot) ids outside [0, E) (written by one workgroup per call)
  int* num_active;   // [1]
  int* active;       // [experts]   expert id of active slot a
  int* seg;          // [experts+1] pair range of slot a
  int* pairs;        // [t*topk]    pair indices grouped by expert
  float* gu;         // few pairs: [gu_parts][t*topk][2*inter] gate/up partial sums per
                     // hidden slice; otherwise [t*topk][inter] h = silu(gate) * up
  int gu_parts;
  float* o;          // [t*topk][hidden]
  int* cnt;          // few pairs: [t][row_blocks(hidden)] arrival counters
  int* pcnt;         // one launch: [t*topk] pair counters, self-resetting
  int* tcnt;         // one launch: [t] token counters, self-resetting
};


// ----------------------------------------------------------- bucket ---
__global__ __launch_bounds__(1024) void moe_bucket_kernel(MoeArgs a) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int fill[kMaxExperts];
  __shared__ int start[kMaxExperts];
  __shared__ int wsum_c[kMaxExperts / 64], wsum_f[kMaxExperts / 64];
  __shared__ int nbad;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P = a.t * a.topk;
  for (int e = tid; e < a.experts; e += blockDim.x) {
    cnt[e] = 0;
    fill[e] = 0;
  }
  if (tid == 0) nbad = 0;
  __syncthreads();
  for (int p = tid; p < P; p += blockDim.x) {
    const int e = a.ids[p];
    if (e >= 0 && e < a.experts) atomicAdd(&cnt[e], 1);
    else atomicAdd(&nbad, 1);
  }
  __syncthreads();
  if (tid == 0) *a.bad = nbad;
  // Exclusive prefix sums over experts (one per thread, blockDim >= experts)
  // of the pair counts (segment starts) and of "has pairs" (active slots).
  const int e = tid;
  const int ce = e < a.experts ? cnt[e] : 0;
  const int fe = ce > 0 ? 1 : 0;
  int c = ce, f = fe;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int tc = __shfl_up(c, d);
    const int tf = __shfl_up(f, d);
    if (lane >= d) {
      c += tc;
      f += tf;
    }
  }
  if (lane == 63) {
    wsum_c[wave] = c;
    wsum_f[wave] = f;
  }
  __syncthreads();
  int oc = 0, of = 0;
  for (int w = 0; w < wave; ++w) {
    oc += wsum_c[w];
    of += wsum_f[w];
  }
  const int off = oc + c - ce;   // pairs of the experts before e
  const int slot = of + f - fe;  // active experts before e
  if (e < a.experts) {
    start[e] = off;
    if (fe) {
      a.active[slot] = e;
      a.seg[slot] = off;
    }
    if (e == a.experts - 1) {
      a.seg[slot + fe] = off + ce;
      a.num_active[0] = slot + fe;
    }
  }
  __syncthreads();
  for (int p = tid; p < P; p += blockDim.x) {
    const int ep = a.ids[p];
    if (ep >= 0 && ep < a.experts) a.pairs[start[ep] + atomicAdd(&fill[ep], 1)] = p;
  }
}

constexpr int kXStride = kSliceTrits + 8;  // A rows padded by 16 bytes (LDS banks)

// Units u0 .. u1-1 of one 640-trit slice of one 64-row block on the matrix
// cores (see gemv_mfma_kernel; u0, u1 are wavefront-uniform).  wb: this
// lane's word-pair pointer of unit 0, row quarter 0 (quad kb / 2, words
// 2 (kb % 2), +1 of row j); the pairs are loaded ahead by mfma_load.
__device__ __forceinline__ void mfma_load(const uint32_t* wb, int u0, int u1, uint2 (&wq)[4][4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (u >= u0 && u < u1)
#pragma unroll
      for (int h = 0; h < 4; ++h) wq[u][h] = load_pair(wb + ((2 * u) * 64 + 16 * h) * 4);
}
// ssc: the block's scales of the slice in LDS ([group][64 rows], fp16 bits);
// xrow: this lane's A row at offset 8 kb; tot[h][v] += the group-scaled D
// rows 4 kb + v of row quarter h.
__device__ __forceinline__ void mfma_units(const uint2 (&wq)[4][4], const uint16_t* ssc, const _Float16* xrow,
                                           const char* cbase, int j, int u0, int u1, float (&tot)[4][4]) {
  float4_t acc[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) acc[h] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (u >= u0 && u < u1) {
      half8_t af[5];
#pragma unroll
      for (int s = 0; s < 5; ++s) af[s] = *reinterpret_cast<const half8_t*>(xrow + 160 * u + 32 * s);
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        uint32_t o[10];
        word_offsets_s<3, false>(wq[u][h].x, o);  // no inline asm next to MFMAs
        word_offsets_s<3, false>(wq[u][h].y, o + 5);
        uint2 cv[10];
#pragma unroll
        for (int c = 0; c < 10; ++c) cv[c] = *reinterpret_cast<const uint2*>(cbase + o[c]);
#pragma unroll
        for (int s = 0; s < 5; ++s) {
          const int step = 5 * u + s;  // scale group step / 4
          const uint4 bq = make_uint4(cv[2 * s].x, cv[2 * s].y, cv[2 * s + 1].x, cv[2 * s + 1].y);
          acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[s], __builtin_bit_cast(half8_t, bq), acc[h], 0, 0, 0);
          if ((step & 3) == 3 || (s == 4 && u == u1 - 1)) {
            const float sc = f16_to_f32(ssc[(step >> 2) * 64 + 16 * h + j]);
#pragma unroll
            for (int v = 0; v < 4; ++v) tot[h][v] = fmaf(sc, acc[h][v], tot[h][v]);
            acc[h] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
          }
        }
      }
    }
  }
}

// Activation row m of the tile, slice s: the five blocks of 128 (lane l
// holds elements 2l, 2l + 1 of each; zero past K).  load(i, v0, v1) reads
// elements i, i + 1 of the row.  Split into a load and a transform so that
// the weight loads can be issued in between: loads complete in order, and
// the transform should wait for the activations only.
struct SliceAct {
  float v[kSliceBlocks][2];
  bool ok[kSliceBlocks];
};
template <typename Load>
__device__ __forceinline__ void load_slice(SliceAct& x, int s, int K, int lane, Load load) {
#pragma unroll
  for (int b = 0; b < kSliceBlocks; ++b) {
    const int k0 = s * kSliceTrits + b * 128;
    x.ok[b] = k0 < K;
    load((x.ok[b] ? k0 : 0) + 2 * lane, x.v[b][0], x.v[b][1]);
  }
}
// Transforms a loaded slice and splits it into A rows 2m, 2m + 1 of xh.
__device__ __forceinline__ void transform_slice(SliceAct& x, _Float16 (*xh)[kXStride], int* xexp, int m, bool fused,
                                                int lane) {
  if (fused) wave_fwht128_batch<kSliceBlocks>(x.v, lane, kInvSqrt128);
#pragma unroll
  for (int b = 0; b < kSliceBlocks; ++b) {
    if (!x.ok[b]) {
      x.v[b][0] = 0.0f;
      x.v[b][1] = 0.0f;
    }
  }
  const int e = split_two_fp16<kSliceBlocks>(x.v, lane, &xh[2 * m][0], &xh[2 * m + 1][0]);
  if (lane == 0) xexp[m] = e;
}

// tot[h][q] += the slice sums of activation row 2 kb + q, scaled back by its
// power of two.
__device__ __forceinline__ void add_slice(const float (&ts)[4][4], const int* xexp, int kb, int M, float (&tot)[4][2]) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int m = 2 * kb + q;
    const int e = m < M ? xexp[m] : 0;
#pragma unroll
    for (int h = 0; h < 4; ++h) tot[h][q] += ldexpf(ts[h][2 * q] + ts[h][2 * q + 1], -e);
  }
}

// ---------------------------------------------------------- gate/up ---
// Workgroup (active expert slot, 64-row block b of I): wavefronts 0, 1 take
// the gate rows 64b.., units 0-1 and 2-3 of each slice, wavefronts 2, 3 the
// up rows I + 64b..; the expert's tokens 8 at a time, all slices;
// h = silu(g) * u is stored to gu[pair][0, I).
// Three wavefronts per SIMD (at most 168 registers): three workgroups per
// CU instead of two, fewer rounds of this latency-bound loop.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void moe_gate_up_kernel(MoeArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 xh[2 * kTile][kXStride];
  __shared__ __attribute__((aligned(16))) _Float16 zeros[kSliceTrits];
  __shared__ __attribute__((aligned(16))) uint2 codes[81];
  __shared__ __attribute__((aligned(16))) uint16_t ssc[2][kMoeG * 64];  // gate, up block
  __shared__ int xexp[kTile];
  __shared__ float red[4][kTile][64];
  const int slot = blockIdx.x;
  if (slot >= a.num_active[0]) return;
  const int e = a.active[slot];
  const int p0 = a.seg[slot], p1 = a.seg[slot + 1];
  auto pair_of = [&](int i) { return a.pairs[i]; };
  const int b = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, j = lane & 15, kb = lane >> 4;
  const int K = a.hidden, nb = row_blocks(2 * a.inter);
  const uint32_t* wexp = reinterpret_cast<const uint32_t*>(a.gu_words + static_cast<size_t>(e) * a.gu_wstride);
  const uint16_t* sexp = a.gu_scales + static_cast<size_t>(e) * a.gu_sstride;
  const int rb = wave < 2 ? b : b + a.inter / 64;  // this wavefront's gate or up block
  const int u0 = 2 * (wave & 1);
  build_code_table(codes, tid, blockDim.x);
  for (int i = tid; i < kSliceTrits; i += blockDim.x) zeros[i] = static_cast<_Float16>(0.0f);
  const char* cbase = reinterpret_cast<const char*>(codes);
  for (int q = p0; q < p1; q += kTile) {
    const int M = min(kTile, p1 - q);
    const _Float16* xrow = (j < 2 * M ? &xh[j < 2 * M ? j : 0][0] : &zeros[0]) + 8 * kb;
    float tot[4][2] = {{0.0f, 0.0f}, {0.0f, 0.0f}, {0.0f, 0.0f}, {0.0f, 0.0f}};
    for (int s = 0; s < slices_per_row(K); ++s) {
      __syncthreads();  // the previous slice's readers are done
      const int u1 = __builtin_amdgcn_readfirstlane(min(u0 + 2, row64_slice_quads(K, s) / 2));
      const uint32_t* wb = wexp + (row64_quad_base(s, rb, nb) + (kb >> 1) * 64 + j) * 4 + 2 * (kb & 1);
      uint2 wq[4][4];
      // The block's scales first, by every lane (a load under a lane
      // condition is waited for at once), staged after the transform.
      const uint4 scq = *reinterpret_cast<const uint4*>(sexp + row64_scale_base(s, rb, nb, kMoeG) +
                                                       8 * (lane < kMoeG * 8 ? lane : 0));
      for (int m = wave; m < M; m += 4) {
        SliceAct xa;
        const size_t base = static_cast<size_t>(pair_of(q + m) / a.topk) * K;
        load_slice(xa, s, K, lane, [&](int i, float& v0, float& v1) { load_act2(a.x, a.x_dtype, base + i, v0, v1); });
        transform_slice(xa, xh, xexp, m, a.fused != 0, lane);
      }
      if ((wave & 1) == 0 && lane < kMoeG * 8) *reinterpret_cast<uint4*>(&ssc[wave >> 1][8 * lane]) = scq;
      __syncthreads();
      // Many workgroups in flight: the weights are requested here, after the
      // barrier (requesting them before the transform measured 1-2 % slower).
      mfma_load(wb, u0, u1, wq);
      float ts[4][4] = {};
      mfma_units(wq, ssc[wave >> 1], xrow, cbase, j, u0, u1, ts);
      add_slice(ts, xexp, kb, M, tot);
    }
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      const int m = 2 * kb + qq;
      if (m < M)
#pragma unroll
        for (int h = 0; h < 4; ++h) red[wave][m][16 * h + j] = tot[h][qq];
    }
    __syncthreads();
    {
      for (int idx = tid; idx < M * 64; idx += blockDim.x) {
        const int m = idx >> 6, l = idx & 63;
        const float g = red[0][m][l] + red[1][m][l];
        const float u = red[2][m][l] + red[3][m][l];
        a.gu[static_cast<size_t>(pair_of(q + m)) * a.inter + b * 64 + l] = g / (1.0f + __expf(-g)) * u;
      }
    }
  }
}

// ------------------------------------------------------------- down ---
// Three wavefronts per SIMD, as for gate/up.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void moe_down_kernel(MoeArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 xh[2 * kTile][kXStride];
  __shared__ __attribute__((aligned(16))) _Float16 zeros[kSliceTrits];
  __shared__ __attribute__((aligned(16))) uint2 codes[81];
  __shared__ __attribute__((aligned(16))) uint16_t ssc[4][kMoeG * 64];
  __shared__ int xexp[kTile];
  const int slot = blockIdx.x;
  if (slot >= a.num_active[0]) return;
  const int e = a.active[slot];
  const int p0 = a.seg[slot], p1 = a.seg[slot + 1];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, j = lane & 15, kb = lane >> 4;
  const int K = a.inter, nsl = slices_per_row(K), nb = row_blocks(a.hidden);
  const int rb = blockIdx.y * 4 + wave;
  const int rbc = min(rb, nb - 1);
  const uint32_t* wexp = reinterpret_cast<const uint32_t*>(a.dn_words + static_cast<size_t>(e) * a.dn_wstride);
  const uint16_t* sexp = a.dn_scales + static_cast<size_t>(e) * a.dn_sstride;
  build_code_table(codes, tid, blockDim.x);
  for (int i = tid; i < kSliceTrits; i += blockDim.x) zeros[i] = static_cast<_Float16>(0.0f);
  const char* cbase = reinterpret_cast<const char*>(codes);
  for (int q = p0; q < p1; q += kTile) {
    const int M = min(kTile, p1 - q);
    const _Float16* xrow = (j < 2 * M ? &xh[j < 2 * M ? j : 0][0] : &zeros[0]) + 8 * kb;
    float tot[4][2] = {{0.0f, 0.0f}, {0.0f, 0.0f}, {0.0f, 0.0f}, {0.0f, 0.0f}};
    const float* h0 = a.gu + static_cast<size_t>(a.pairs[q + min(wave, M - 1)]) * K;
    const float* h1 = a.gu + static_cast<size_t>(a.pairs[q + min(wave + 4, M - 1)]) * K;
    for (int s = 0; s < nsl; ++s) {
      __syncthreads();
      // h rows wave, wave + 4 of the tile, the scales, then the weights, all
      // before the transform (which waits for h only); every load
      // unconditional (rows clamped, slices stored whole).
      SliceAct x0, x1;
      load_slice(x0, s, K, lane, [&](int i, float& v0, float& v1) {
        const float2 v = *reinterpret_cast<const float2*>(h0 + i);
        v0 = v.x;
        v1 = v.y;
      });
      load_slice(x1, s, K, lane, [&](int i, float& v0, float& v1) {
        const float2 v = *reinterpret_cast<const float2*>(h1 + i);
        v0 = v.x;
        v1 = v.y;
      });
      const uint4 scq = *reinterpret_cast<const uint4*>(sexp + row64_scale_base(s, rbc, nb, kMoeG) +
                                                       8 * (lane < kMoeG * 8 ? lane : 0));
      const uint32_t* wb = wexp + (row64_quad_base(s, rbc, nb) + (kb >> 1) * 64 + j) * 4 + 2 * (kb & 1);
      uint2 wq[4][4];
      mfma_load(wb, 0, 4, wq);
      if (wave < M) transform_slice(x0, xh, xexp, wave, true, lane);
      if (wave + 4 < M) transform_slice(x1, xh, xexp, wave + 4, true, lane);
      if (lane < kMoeG * 8) *reinterpret_cast<uint4*>(&ssc[wave][8 * lane]) = scq;
      __syncthreads();
      const int u1 = __builtin_amdgcn_readfirstlane(row64_slice_quads(K, s) / 2);
      if (rb < nb) {
        float ts[4][4] = {};
        mfma_units(wq, ssc[wave], xrow, cbase, j, 0, u1, ts);
        add_slice(ts, xexp, kb, M, tot);
      }
    }
    if (rb < nb) {
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const int m = 2 * kb + qq;
        if (m < M)
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const int row = rb * 64 + 16 * h + j;
            if (row < a.hidden) a.o[static_cast<size_t>(a.pairs[q + m]) * a.hidden + row] = tot[h][qq];
          }
      }
    }
  }
}

// -------------------------------------------------------- few pairs ---
// Gate/up: workgroup (pair, 64-row block b of I, 640-trit slice s of the
// hidden size), 8 wavefronts: wavefront w decodes unit w % 4 of the gate
// (w < 4) or up (w >= 4) block; wavefront 0 transforms the activations,
// wavefronts 3 and 7 stage the scales.  The four units' sums are added
// in order and stored to gu[s][pair][.] (gate in [0, I), up in [I, 2I)).
// Workgroup (0, 0, 0) also clears the arrival counters of the down launch.
constexpr int kPairGuWaves = 8;
__global__ __launch_bounds__(kPairGuWaves * 64) void moe_gate_up_pairs_kernel(MoeArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 xh[2][kXStride];
  __shared__ __attribute__((aligned(16))) _Float16 zeros[kSliceTrits];
  __shared__ __attribute__((aligned(16))) uint2 codes[81];
  __shared__ __attribute__((aligned(16))) uint16_t ssc[2][kMoeG * 64];
  __shared__ int xexp[1];
  __shared__ float red[kPairGuWaves][64];
  const int pair = blockIdx.x, b = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, j = lane & 15, kb = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int up = wave >> 2, unit = wave & 3;
  const int K = a.hidden, I = a.inter, nb = row_blocks(2 * I);
  const size_t P = static_cast<size_t>(a.t) * a.topk;
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0) {
    for (int i = tid; i < a.t * row_blocks(a.hidden); i += blockDim.x) a.cnt[i] = 0;
    // The call's count of ids outside [0, E) (at most 64 pairs: one wavefront).
    if (tid < 64) {
      int c = 0;
      if (tid < P) {
        const int ei = a.ids[tid];
        c = (ei < 0 || ei >= a.experts) ? 1 : 0;
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off);
      if (tid == 0) *a.bad = c;
    }
  }
  const int e = a.ids[pair];
  if (e < 0 || e >= a.experts) return;  // contributes nothing; its partials are never read
  SliceAct xa;
  if (wave == 0) {
    const size_t base = static_cast<size_t>(pair / a.topk) * K;
    load_slice(xa, s, K, lane, [&](int i, float& v0, float& v1) { load_act2(a.x, a.x_dtype, base + i, v0, v1); });
  }
  const int rb = up ? b + I / 64 : b;
  const int u1 = __builtin_amdgcn_readfirstlane(min(unit + 1, row64_slice_quads(K, s) / 2));
  const uint32_t* wexp = reinterpret_cast<const uint32_t*>(a.gu_words + static_cast<size_t>(e) * a.gu_wstride);
  const uint16_t* sexp = a.gu_scales + static_cast<size_t>(e) * a.gu_sstride;
  const uint32_t* wb = wexp + (row64_quad_base(s, rb, nb) + (kb >> 1) * 64 + j) * 4 + 2 * (kb & 1);
  uint2 wq[4][4];
  mfma_load(wb, unit, u1, wq);
  build_code_table(codes, tid, blockDim.x);
  for (int i = tid; i < kSliceTrits; i += blockDim.x) zeros[i] = static_cast<_Float16>(0.0f);
  if (unit == 3 && lane < kMoeG * 8)  // not wavefront 0: its transform waits for nothing else
    *reinterpret_cast<uint4*>(&ssc[up][8 * lane]) =
        *reinterpret_cast<const uint4*>(sexp + row64_scale_base(s, rb, nb, kMoeG) + 8 * lane);
  if (wave == 0) transform_slice(xa, xh, xexp, 0, a.fused != 0, lane);
  __syncthreads();
  const _Float16* xrow = (j < 2 ? &xh[j < 2 ? j : 0][0] : &zeros[0]) + 8 * kb;
  float ts[4][4] = {};
  mfma_units(wq, ssc[up], xrow, reinterpret_cast<const char*>(codes), j, unit, u1, ts);
  float tot[4][2] = {{0.0f, 0.0f}, {0.0f, 0.0f}, {0.0f, 0.0f}, {0.0f, 0.0f}};
  add_slice(ts, xexp, kb, 1, tot);
  if (kb == 0)
#pragma unroll
    for (int h = 0; h < 4; ++h) red[wave][16 * h + j] = tot[h][0];
  __syncthreads();
  if (tid < 128) {
    const int g = tid >> 6, l = tid & 63;  // g = 0: gate, 1: up
    const float v = ((red[4 * g][l] + red[4 * g + 1][l]) + red[4 * g + 2][l]) + red[4 * g + 3][l];
    a.gu[(static_cast<size_t>(s) * P + pair) * 2 * I + g * I + b * 64 + l] = v;
  }
}

// Down + combine: workgroup (pair, 64-row block rb of the hidden size), 4
// wavefronts: wavefront w decodes unit w of each slice of the intermediate
// dimension; wavefront 0 assembles h = silu(g) * u from the gate/up partials
// (added in order) and transforms it.  The units' sums are added in order,
// scaled by the route weight and stored to o[pair][.]; the arrival is
// counted, and the last of the token's slots to arrive adds the slots' rows
// in slot order and stores y.  The o rows are written and read with
// device-scope atomic accesses (coherent across the dies); each slot waits
// for its row's stores to complete before it counts its arrival, and the
// last slot reads the rows only after its count has returned.
constexpr int kPairDnWaves = 4;
__global__ __launch_bounds__(kPairDnWaves * 64) void moe_down_pairs_kernel(MoeArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 xh[2][kXStride];
  __shared__ __attribute__((aligned(16))) _Float16 zeros[kSliceTrits];
  __shared__ __attribute__((aligned(16))) uint2 codes[81];
  __shared__ __attribute__((aligned(16))) uint16_t ssc[kMoeG * 64];
  __shared__ int xexp[1];
  __shared__ float red[kPairDnWaves][64];
  const int pair = blockIdx.x, rb = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, j = lane & 15, kb = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = a.inter, nsl = slices_per_row(K), nb = row_blocks(a.hidden);
  const int tok = pair / a.topk;
  const size_t P = static_cast<size_t>(a.t) * a.topk;
  const int e = a.ids[pair];
  const float wgt = a.route_w[pair];
  const bool valid = e >= 0 && e < a.experts;
  build_code_table(codes, tid, blockDim.x);
  for (int i = tid; i < kSliceTrits; i += blockDim.x) zeros[i] = static_cast<_Float16>(0.0f);
  float tot[4][2] = {{0.0f, 0.0f}, {0.0f, 0.0f}, {0.0f, 0.0f}, {0.0f, 0.0f}};
  if (valid) {
    const uint32_t* wexp = reinterpret_cast<const uint32_t*>(a.dn_words + static_cast<size_t>(e) * a.dn_wstride);
    const uint16_t* sexp = a.dn_scales + static_cast<size_t>(e) * a.dn_sstride;
    const float* grow = a.gu + static_cast<size_t>(pair) * 2 * K;
    const _Float16* xrow = (j < 2 ? &xh[j < 2 ? j : 0][0] : &zeros[0]) + 8 * kb;
    for (int s = 0; s < nsl; ++s) {
      if (s > 0) __syncthreads();  // the previous slice's readers are done
      // This wavefront's weights first, then (wavefront 0) h of this slice:
      // the gate/up partials added in order, four partials' loads in
      // flight at a time.
      const uint32_t* wb = wexp + (row64_quad_base(s, rb, nb) + (kb >> 1) * 64 + j) * 4 + 2 * (kb & 1);
      const int u1 = __builtin_amdgcn_readfirstlane(min(wave + 1, row64_slice_quads(K, s) / 2));
      uint2 wq[4][4];
      mfma_load(wb, wave, u1, wq);
      if (wave == 0) {
        const uint4 scq = *reinterpret_cast<const uint4*>(sexp + row64_scale_base(s, rb, nb, kMoeG) +
                                                         8 * (lane < kMoeG * 8 ? lane : 0));
        float g[kSliceBlocks][2] = {}, u[kSliceBlocks][2] = {};
        for (int z0 = 0; z0 < a.gu_parts; z0 += 4) {
          float2 gv[4][kSliceBlocks], uv[4][kSliceBlocks];
#pragma unroll
          for (int dz = 0; dz < 4; ++dz) {
            const float* src = grow + static_cast<size_t>(min(z0 + dz, a.gu_parts - 1)) * P * 2 * K;
#pragma unroll
            for (int bb = 0; bb < kSliceBlocks; ++bb) {
              const int k0 = s * kSliceTrits + bb * 128;
              const int i = (k0 < K ? k0 : 0) + 2 * lane;
              gv[dz][bb] = *reinterpret_cast<const float2*>(src + i);
              uv[dz][bb] = *reinterpret_cast<const float2*>(src + K + i);
            }
          }
#pragma unroll
          for (int dz = 0; dz < 4; ++dz)
            if (z0 + dz < a.gu_parts)
#pragma unroll
              for (int bb = 0; bb < kSliceBlocks; ++bb) {
                g[bb][0] += gv[dz][bb].x;
                g[bb][1] += gv[dz][bb].y;
                u[bb][0] += uv[dz][bb].x;
                u[bb][1] += uv[dz][bb].y;
              }
        }
        SliceAct xa;
#pragma unroll
        for (int bb = 0; bb < kSliceBlocks; ++bb) {
          xa.ok[bb] = s * kSliceTrits + bb * 128 < K;
#pragma unroll
          for (int c = 0; c < 2; ++c) xa.v[bb][c] = g[bb][c] / (1.0f + __expf(-g[bb][c])) * u[bb][c];
        }
        transform_slice(xa, xh, xexp, 0, true, lane);
        if (lane < kMoeG * 8) *reinterpret_cast<uint4*>(&ssc[8 * lane]) = scq;
      }
      __syncthreads();
      float ts[4][4] = {};
      mfma_units(wq, ssc, xrow, reinterpret_cast<const char*>(codes), j, wave, u1, ts);
      add_slice(ts, xexp, kb, 1, tot);
    }
  }
  if (kb == 0)
#pragma unroll
    for (int h = 0; h < 4; ++h) red[wave][16 * h + j] = tot[h][0];
  __syncthreads();
  if (wave != 0) return;
  const int row = rb * 64 + lane;
  const int rowc = row < a.hidden ? row : 0;
  if (a.accumulate) {  // y += w o with device atomics: no arrival count, no combine
    if (valid && row < a.hidden)
      atomicAdd(a.y + static_cast<size_t>(tok) * a.hidden + row,
                wgt * (((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane]));
    return;
  }
  if (valid && row < a.hidden) {
    const float v = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
    __hip_atomic_store(a.o + static_cast<size_t>(pair) * a.hidden + row, wgt * v, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  // Publication without a release fence (a device-scope release writes back
  // the whole L2 and measured +2.5 us per launch at one token): the row was
  // stored with device-scope atomic stores, which gfx950 writes through to
  // the device-coherent level; waiting for their completion (vmcnt 0) before
  // the counter's device-scope read-modify-write orders them before the
  // count.  The last arriver reads the rows with device-scope atomic loads,
  // which read the device-coherent level, issued only after its
  // read-modify-write has returned (the branch on its result, and a compiler
  // barrier that keeps the loads below it).
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  int prev = 0;
  if (lane == 0) prev = __hip_atomic_fetch_add(&a.cnt[tok * nb + rb], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  prev = __shfl(prev, 0);
  if (prev != a.topk - 1) return;
  asm volatile("" ::: "memory");
  const int32_t* tok_ids = a.ids + static_cast<size_t>(tok) * a.topk;
  float* orow = a.o + static_cast<size_t>(tok) * a.topk * a.hidden + rowc;
  float v = 0.0f;
  for (int j0 = 0; j0 < a.topk; j0 += 8) {
    float ov[8];
#pragma unroll
    for (int d = 0; d < 8; ++d)
      ov[d] = __hip_atomic_load(orow + static_cast<size_t>(min(j0 + d, a.topk - 1)) * a.hidden, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const int ej = tok_ids[min(j0 + d, a.topk - 1)];
      if (j0 + d < a.topk && ej >= 0 && ej < a.experts) v += ov[d];
    }
  }
  if (row < a.hidden) a.y[static_cast<size_t>(tok) * a.hidden + row] = v;
}

// Down + combine: workgroup (token, 64-row block rb of the hidden size),
// the token's slots eight at a time, one wavefront per slot: it adds the
// gate/up partials in order, forms h = silu(g) * u, transforms it, stages
// the expert's scales and decodes the four units of each slice of the
// intermediate dimension.  A slot's row (times the route weight) stays in
// LDS; y = the valid slots' rows added in slot order.  Nothing leaves the
// workgroup but y.
// Used from kTokMinTokens tokens on: with fewer, its workgroups are too few
// and each slot's four units on one wavefront too long a chain (256-expert
// layer, top-8: 24.9 against 23.9 us at three tokens, 26.5 against 28.3 at
// four, 37.5 against 49.7 at eight, for the per-pair kernel).
constexpr int kTokSlots = 8;
constexpr int kMaxTopk = 32;
constexpr int kTokMinTokens = 4;
__global__ __launch_bounds__(kTokSlots * 64) void moe_down_tok_kernel(MoeArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 xh[kTokSlots][2][kXStride];
  __shared__ __attribute__((aligned(16))) _Float16 zeros[kSliceTrits];
  __shared__ __attribute__((aligned(16))) uint2 codes[81];
  __shared__ __attribute__((aligned(16))) uint16_t ssc[kTokSlots][kMoeG * 64];
  __shared__ int xexp[kTokSlots];
  __shared__ float orow[kMaxTopk][64];
  const int tok = blockIdx.x, rb = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, j = lane & 15, kb = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = a.inter, nsl = slices_per_row(K), nb = row_blocks(a.hidden);
  const size_t P = static_cast<size_t>(a.t) * a.topk;
  build_code_table(codes, tid, blockDim.x);
  for (int i = tid; i < kSliceTrits; i += blockDim.x) zeros[i] = static_cast<_Float16>(0.0f);
  const _Float16* xrow = (j < 2 ? &xh[wave][j < 2 ? j : 0][0] : &zeros[0]) + 8 * kb;
  const int sl = lane < kMoeG * 8 ? lane : 0;
  __syncthreads();
  for (int j0 = 0; j0 < a.topk; j0 += kTokSlots) {
    const int slot = j0 + wave;
    const int pair = tok * a.topk + min(slot, a.topk - 1);
    const int e = a.ids[pair];
    const bool valid = slot < a.topk && e >= 0 && e < a.experts;  // wavefront-uniform
    float tot[4][2] = {{0.0f, 0.0f}, {0.0f, 0.0f}, {0.0f, 0.0f}, {0.0f, 0.0f}};
    if (valid) {  // this wavefront's slot only: no barrier inside
      const uint32_t* wexp = reinterpret_cast<const uint32_t*>(a.dn_words + static_cast<size_t>(e) * a.dn_wstride);
      const uint16_t* sexp = a.dn_scales + static_cast<size_t>(e) * a.dn_sstride;
      const float* grow = a.gu + static_cast<size_t>(pair) * 2 * K;
      for (int s = 0; s < nsl; ++s) {
        // The weights, the scales, then h of this slice: the gate/up
        // partials added in order, four partials' loads in flight at a time.
        const uint32_t* wb = wexp + (row64_quad_base(s, rb, nb) + (kb >> 1) * 64 + j) * 4 + 2 * (kb & 1);
        const int u1 = __builtin_amdgcn_readfirstlane(row64_slice_quads(K, s) / 2);
        uint2 wq[4][4];
        mfma_load(wb, 0, 4, wq);  // slices are stored whole: every unit can be read
        const uint4 scq = *reinterpret_cast<const uint4*>(sexp + row64_scale_base(s, rb, nb, kMoeG) + 8 * sl);
        float g[kSliceBlocks][2] = {}, u[kSliceBlocks][2] = {};
        for (int z0 = 0; z0 < a.gu_parts; z0 += 4) {
          float2 gv[4][kSliceBlocks], uv[4][kSliceBlocks];
#pragma unroll
          for (int dz = 0; dz < 4; ++dz) {
            const float* src = grow + static_cast<size_t>(min(z0 + dz, a.gu_parts - 1)) * P * 2 * K;
#pragma unroll
            for (int bb = 0; bb < kSliceBlocks; ++bb) {
              const int k0 = s * kSliceTrits + bb * 128;
              const int i = (k0 < K ? k0 : 0) + 2 * lane;
              gv[dz][bb] = *reinterpret_cast<const float2*>(src + i);
              uv[dz][bb] = *reinterpret_cast<const float2*>(src + K + i);
            }
          }
#pragma unroll
          for (int dz = 0; dz < 4; ++dz)
            if (z0 + dz < a.gu_parts)
#pragma unroll
              for (int bb = 0; bb < kSliceBlocks; ++bb) {
                g[bb][0] += gv[dz][bb].x;
                g[bb][1] += gv[dz][bb].y;
                u[bb][0] += uv[dz][bb].x;
                u[bb][1] += uv[dz][bb].y;
              }
        }
        SliceAct xa;
#pragma unroll
        for (int bb = 0; bb < kSliceBlocks; ++bb) {
          xa.ok[bb] = s * kSliceTrits + bb * 128 < K;
#pragma unroll
          for (int c = 0; c < 2; ++c) xa.v[bb][c] = g[bb][c] / (1.0f + __expf(-g[bb][c])) * u[bb][c];
        }
        transform_slice(xa, xh[wave], &xexp[wave], 0, true, lane);
        if (lane < kMoeG * 8) *reinterpret_cast<uint4*>(&ssc[wave][8 * lane]) = scq;
        // The wavefront's own LDS writes are complete before its reads.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        float ts[4][4] = {};
        mfma_units(wq, ssc[wave], xrow, reinterpret_cast<const char*>(codes), j, 0, u1, ts);
        add_slice(ts, &xexp[wave], kb, 1, tot);
      }
    }
    if (slot < a.topk && kb == 0)
#pragma unroll
      for (int h = 0; h < 4; ++h) orow[slot][16 * h + j] = a.route_w[pair] * tot[h][0];
  }
  __syncthreads();
  if (tid < 64) {
    const int row = rb * 64 + tid;
    float v = 0.0f;
    for (int s2 = 0; s2 < a.topk; ++s2) {
      const int e2 = a.ids[tok * a.topk + s2];
      if (e2 >= 0 && e2 < a.experts) v += orow[s2][tid];
    }
    if (row < a.hidden) {
      float* yp = a.y + static_cast<size_t>(tok) * a.hidden + row;
      *yp = a.accumulate ? *yp + v : v;
    }
  }
}

// ------------------------------------------------ one launch (few pairs) ---
// The whole expert MLP in one launch, with no workgroup ever waiting for
// another (so dispatch order cannot deadlock it).  Grid and phase 1 as
// moe_gate_up_pairs_kernel: workgroup (pair, 64-row block b of I, hidden
// slice s), eight wavefronts, the slice's gate and up sums of the block
// stored with device-scope atomic stores.  Each workgroup then counts its
// arrival on its pair's counter; the last of the pair's (I / 64) x slices
// workgroups to arrive runs phase 2 for the whole pair: it adds the gate/up
// partials in slice order, forms h = silu(gate) * up, transforms h (all
// slices of I into LDS), and computes all of the pair's down rows (row
// blocks spread over its eight wavefronts, every unit of a block on one
// wavefront), scaled by the route weight.  The rows are published as in
// moe_down_pairs_kernel, and the last of the token's slots to arrive adds
// them in slot order into y (TQ_ACCUMULATE: each row is added into y with
// device atomics instead).  The counters reset themselves: the workspace's
// counter area must be zero before the first call and every call leaves it
// zero.
constexpr int kFusedMaxInterSlices = 4;  // I <= 2560
__global__ __launch_bounds__(kPairGuWaves * 64) void moe_fused_pairs_kernel(MoeArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 xh[kFusedMaxInterSlices][2][kXStride];
  __shared__ __attribute__((aligned(16))) _Float16 zeros[kSliceTrits];
  __shared__ __attribute__((aligned(16))) uint2 codes[81];
  __shared__ __attribute__((aligned(16))) uint16_t ssc[kPairGuWaves][kMoeG * 64];
  __shared__ __attribute__((aligned(16))) float hs[kFusedMaxInterSlices * kSliceTrits];
  __shared__ int xexp[kFusedMaxInterSlices];
  __shared__ float red[kPairGuWaves][64];
  __shared__ int last;
  const int pair = blockIdx.x, b = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, j = lane & 15, kb = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int up = wave >> 2, unit = wave & 3;
  const int K = a.hidden, I = a.inter, nb = row_blocks(2 * I);
  const size_t P = static_cast<size_t>(a.t) * a.topk;
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && tid < 64) {
    int c = 0;
    if (tid < P) {
      const int ei = a.ids[tid];
      c = (ei < 0 || ei >= a.experts) ? 1 : 0;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off);
    if (tid == 0) *a.bad = c;
  }
  const int e = a.ids[pair];
  const bool valid = e >= 0 && e < a.experts;  // workgroup-uniform
  build_code_table(codes, tid, blockDim.x);
  for (int i = tid; i < kSliceTrits; i += blockDim.x) zeros[i] = static_cast<_Float16>(0.0f);

  // ---- phase 1: this workgroup's gate and up sums for the slice
  if (valid) {
    SliceAct xa;
    if (wave == 0) {
      const size_t base = static_cast<size_t>(pair / a.topk) * K;
      load_slice(xa, s, K, lane, [&](int i, float& v0, float& v1) { load_act2(a.x, a.x_dtype, base + i, v0, v1); });
    }
    const int rb = up ? b + I / 64 : b;
    const int u1 = __builtin_amdgcn_readfirstlane(min(unit + 1, row64_slice_quads(K, s) / 2));
    const uint32_t* wexp = reinterpret_cast<const uint32_t*>(a.gu_words + static_cast<size_t>(e) * a.gu_wstride);
    const uint16_t* sexp = a.gu_scales + static_cast<size_t>(e) * a.gu_sstride;
    const uint32_t* wb = wexp + (row64_quad_base(s, rb, nb) + (kb >> 1) * 64 + j) * 4 + 2 * (kb & 1);
    uint2 wq[4][4];
    mfma_load(wb, unit, u1, wq);
    if (unit == 3 && lane < kMoeG * 8)
      *reinterpret_cast<uint4*>(&ssc[up][8 * lane]) =
          *reinterpret_cast<const uint4*>(sexp + row64_scale_base(s, rb, nb, kMoeG) + 8 * lane);
    if (wave == 0) transform_slice(xa, xh[0], xexp, 0, a.fused != 0, lane);
    __syncthreads();
    const _Float16* xrow = (j < 2 ? &xh[0][j < 2 ? j : 0][0] : &zeros[0]) + 8 * kb;
    float ts[4][4] = {};
    mfma_units(wq, ssc[up], xrow, reinterpret_cast<const char*>(codes), j, unit, u1, ts);
    float tot[4][2] = {{0.0f, 0.0f}, {0.0f, 0.0f}, {0.0f, 0.0f}, {0.0f, 0.0f}};
    add_slice(ts, xexp, kb, 1, tot);
    if (kb == 0)
#pragma unroll
      for (int h = 0; h < 4; ++h) red[wave][16 * h + j] = tot[h][0];
    __syncthreads();
    if (tid < 128) {
      const int g = tid >> 6, l = tid & 63;  // g = 0: gate, 1: up
      const float v = ((red[4 * g][l] + red[4 * g + 1][l]) + red[4 * g + 2][l]) + red[4 * g + 3][l];
      __hip_atomic_store(a.gu + (static_cast<size_t>(s) * P + pair) * 2 * I + g * I + b * 64 + l, v,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // Arrival on the pair's counter (stores complete first; see
  // moe_down_pairs_kernel for why this ordering suffices on gfx950).
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  const int parts = (I / 64) * slices_per_row(K);
  if (tid == 0) {
    const int prev = __hip_atomic_fetch_add(&a.pcnt[pair], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = prev == parts - 1;
    if (last) __hip_atomic_store(&a.pcnt[pair], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // for the next call
  }
  __syncthreads();
  if (!last) return;
  asm volatile("" ::: "memory");

  // ---- phase 2 (the pair's last workgroup): h, its transform, all down rows
  const int tok = pair / a.topk;
  const int KI = I, nsl_i = slices_per_row(KI), nbd = row_blocks(a.hidden);
  if (valid) {
    for (int k = tid; k < KI; k += blockDim.x) {
      float g = 0.0f, u = 0.0f;
      for (int z = 0; z < a.gu_parts; ++z) {  // slice order
        const float* src = a.gu + (static_cast<size_t>(z) * P + pair) * 2 * I;
        g += __hip_atomic_load(src + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        u += __hip_atomic_load(src + I + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      hs[k] = g / (1.0f + __expf(-g)) * u;
    }
    __syncthreads();
    if (wave < nsl_i) {  // wavefront si transforms slice si of h
      SliceAct xa;
      load_slice(xa, wave, KI, lane, [&](int i, float& v0, float& v1) {
        v0 = hs[i];
        v1 = hs[i + 1];
      });
      transform_slice(xa, xh[wave], &xexp[wave], 0, true, lane);
    }
    __syncthreads();
  }
  const float wgt = a.route_w[pair];
  float* orow = a.o + static_cast<size_t>(pair) * a.hidden;
  if (valid) {
    const uint32_t* wexp = reinterpret_cast<const uint32_t*>(a.dn_words + static_cast<size_t>(e) * a.dn_wstride);
    const uint16_t* sexp = a.dn_scales + static_cast<size_t>(e) * a.dn_sstride;
    for (int rbd = wave; rbd < nbd; rbd += kPairGuWaves) {
      float tot[4][2] = {{0.0f, 0.0f}, {0.0f, 0.0f}, {0.0f, 0.0f}, {0.0f, 0.0f}};
      for (int si = 0; si < nsl_i; ++si) {
        const uint32_t* wb = wexp + (row64_quad_base(si, rbd, nbd) + (kb >> 1) * 64 + j) * 4 + 2 * (kb & 1);
        const int u1 = __builtin_amdgcn_readfirstlane(row64_slice_quads(KI, si) / 2);
        uint2 wq[4][4];
        mfma_load(wb, 0, 4, wq);  // slices are stored whole
        const uint4 scq = *reinterpret_cast<const uint4*>(sexp + row64_scale_base(si, rbd, nbd, kMoeG) +
                                                         8 * (lane < kMoeG * 8 ? lane : 0));
        if (lane < kMoeG * 8) *reinterpret_cast<uint4*>(&ssc[wave][8 * lane]) = scq;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wavefront's own scale stores, before its reads
        const _Float16* xrow = (j < 2 ? &xh[si][j < 2 ? j : 0][0] : &zeros[0]) + 8 * kb;
        float ts[4][4] = {};
        mfma_units(wq, ssc[wave], xrow, reinterpret_cast<const char*>(codes), j, 0, u1, ts);
        add_slice(ts, &xexp[si], kb, 1, tot);
      }
      if (kb == 0)
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const int row = rbd * 64 + 16 * h + j;
          if (row < a.hidden) {
            if (a.accumulate)
              atomicAdd(a.y + static_cast<size_t>(tok) * a.hidden + row, wgt * tot[h][0]);
            else
              __hip_atomic_store(orow + row, wgt * tot[h][0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
    }
  }
  if (a.accumulate) return;
  // ---- the token's combine: the last of its slots adds the rows in slot order
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    const int prev = __hip_atomic_fetch_add(&a.tcnt[tok], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = prev == a.topk - 1;
    if (last) __hip_atomic_store(&a.tcnt[tok], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!last) return;
  asm volatile("" ::: "memory");
  const int32_t* tok_ids = a.ids + static_cast<size_t>(tok) * a.topk;
  const float* obase = a.o + static_cast<size_t>(tok) * a.topk * a.hidden;
  for (int row = tid; row < a.hidden; row += blockDim.x) {
    float v = 0.0f;
    for (int sj = 0; sj < a.topk; ++sj) {
      const int ej = tok_ids[sj];
      if (ej >= 0 && ej < a.experts)
        v += __hip_atomic_load(obase + static_cast<size_t>(sj) * a.hidden + row, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    a.y[static_cast<size_t>(tok) * a.hidden + row] = v;
  }
}

// ---------------------------------------------------------- combine ---
__global__ __launch_bounds__(256) void moe_combine_kernel(MoeArgs a) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<size_t>(a.t) * a.hidden) return;
  const int tok = static_cast<int>(idx / a.hidden);
  const int n = static_cast<int>(idx % a.hidden);
  float acc = 0.0f;
  // Eight slots' loads in flight at a time (unconditional, slots clamped),
  // then added in slot order.
  for (int j0 = 0; j0 < a.topk; j0 += 8) {
    int ev[8];
    float wv[8], ov[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const int p = tok * a.topk + min(j0 + d, a.topk - 1);
      ev[d] = a.ids[p];
      wv[d] = a.route_w[p];
      ov[d] = a.o[static_cast<size_t>(p) * a.hidden + n];
    }
#pragma unroll
    for (int d = 0; d < 8; ++d)
      if (j0 + d < a.topk && ev[d] >= 0 && ev[d] < a.experts) acc = fmaf(wv[d], ov[d], acc);
  }
  a.y[idx] = a.accumulate ? a.y[idx] + acc : acc;
}

// ----------------------------------------------------------- router ---
// One wavefront per token: softmax in FP32 (max-subtracted), then topk
// rounds of wavefront argmax (larger p first, lower id on ties).
__global__ __launch_bounds__(256) void moe_route_kernel(const float* __restrict__ logits, int t, int e, int topk,
                                                        int32_t* __restrict__ ids, float* __restrict__ weights) {
  const int tok = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tok >= t) return;
  const int lane = threadIdx.x & 63;
  const float* z = logits + static_cast<size_t>(tok) * e;
  constexpr int kPer = kMaxExperts / 64;
  float p[kPer];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int id = i * 64 + lane;
    p[i] = id < e ? z[id] : -INFINITY;
    mx = fmaxf(mx, p[i]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    p[i] = (i * 64 + lane) < e ? __expf(p[i] - mx) : -1.0f;
    if (p[i] > 0.0f) sum += p[i];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  float chosen_sum = 0.0f;
  float mine = 0.0f;  // lane j keeps the j-th chosen probability
  int mine_id = 0;
  for (int r = 0; r < topk; ++r) {
    float bv = -2.0f;
    int bi = INT_MAX;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int id = i * 64 + lane;
      if (p[i] > bv || (p[i] == bv && id < bi)) {
        bv = p[i];
        bi = id;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) p[bi >> 6] = -2.0f;  // remove the winner
    chosen_sum += bv / sum;
    if (lane == r) {
      mine = bv / sum;
      mine_id = bi;
    }
  }
  if (lane < topk) {
    ids[static_cast<size_t>(tok) * topk + lane] = mine_id;
    weights[static_cast<size_t>(tok) * topk + lane] = mine / chosen_sum;
  }
}

inline size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

struct MoeLayout {
  size_t bad, num_active, active, seg, pairs, gu, o, cnt, fcnt, total;
};

// Few (token, slot) pairs: no bucketing, one workgroup per pair for gate/up
// (split over hidden slices), down and combine in one launch.
bool moe_pairs(int t, int topk) { return static_cast<long long>(t) * topk <= kFusedMaxPairs; }

MoeLayout moe_layout(int experts, int t, int topk, int hidden, int inter) {
  const bool pairs = moe_pairs(t, topk);
  MoeLayout l;
  const size_t P = static_cast<size_t>(t) * topk;
  size_t off = 0;
  l.bad = off;  // first: tq_moe_bad_ids reads it at offset 0
  off += align256(sizeof(int));
  // One launch: pair then token counters, at a fixed place whatever the
  // call's size (they must stay zero between calls on one workspace).
  l.fcnt = off;
  off += align256(sizeof(int) * 2 * kFusedMaxPairs);
  l.num_active = off;
  off += align256(sizeof(int));
  l.active = off;
  off += align256(sizeof(int) * experts);
  l.seg = off;
  off += align256(sizeof(int) * (experts + 1));
  l.pairs = off;
  off += align256(sizeof(int) * P);
  l.gu = off;
  off += align256(sizeof(float) * (pairs ? slices_per_row(hidden) * P * 2 * inter : P * inter));
  l.o = off;
  off += align256(sizeof(float) * P * hidden);
  l.cnt = off;
  off += align256(sizeof(int) * t * row_blocks(hidden));
  l.total = off;
  return l;
}


}  // namespace

size_t tq_moe_workspace(const tq_weights* gu, int t, int topk) {
  const int inter = gu->n / 2, hidden = gu->k;
  return moe_layout(gu->num_experts, t, topk, hidden, inter).total;
}

extern "C" int tq_moe_bad_ids(const void* workspace, size_t ws_bytes, int32_t* count, void* stream) {
  if (!workspace || !count || !tq_aligned(workspace, 16)) return TQ_EINVAL;
  if (ws_bytes < sizeof(int32_t)) return TQ_ENOSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, workspace, sizeof(v), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    tq_set_hip_error(e, __func__);
    return TQ_EHIP;
  }
  *count = v;
  return v ? TQ_EDATA : TQ_OK;
}

extern "C" int tq_moe_route(const float* logits, int t, int e, int topk, int32_t* ids, float* weights,
                            void* stream) {
  if (!logits || !ids || !weights) return TQ_EINVAL;
  if (!tq_aligned(logits, 4) || !tq_aligned(ids, 4) || !tq_aligned(weights, 4)) return TQ_EINVAL;
  if (t < 1 || e < 1 || e > kMaxExperts || topk < 1 || topk > 32 || topk > e) return TQ_ESHAPE;
  hipLaunchKernelGGL(moe_route_kernel, dim3((t + 3) / 4), dim3(256), 0, static_cast<hipStream_t>(stream), logits,
                     t, e, topk, ids, weights);
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}

extern "C" int tq_moe_gemv(const tq_weights* w_gate_up, const tq_weights* w_down, const void* x, int x_dtype, int t,
                           int topk, const int32_t* expert_ids, const float* route_w, float* y, unsigned flags,
                           void* workspace, size_t ws_bytes, void* stream) {
  int st = tq_check_weights(w_gate_up, 0);
  if (st != TQ_OK) return st;
  st = tq_check_weights(w_down, w_gate_up->num_experts);
  if (st != TQ_OK) return st;
  if (!x || !expert_ids || !route_w || !y || !workspace) return TQ_EINVAL;
  if (x_dtype != TQ_F32 && x_dtype != TQ_BF16 && x_dtype != TQ_F16) return TQ_EINVAL;
  if (!tq_aligned(x, tq_act_align(x_dtype)) || !tq_aligned(y, 4) || !tq_aligned(workspace, 16) ||
      !tq_aligned(expert_ids, 4) || !tq_aligned(route_w, 4))
    return TQ_EINVAL;
  if (flags & ~static_cast<unsigned>(TQ_FWHT_FUSED | TQ_ACCUMULATE | TQ_MOE_ONE_LAUNCH)) return TQ_EINVAL;
  // The expert path takes the ternary format at group 128.
  if (w_gate_up->levels != 3 || w_down->levels != 3 || w_gate_up->group != 128 || w_down->group != 128)
    return TQ_EUNSUPPORTED;
  const int E = w_gate_up->num_experts, hidden = w_gate_up->k, inter = w_gate_up->n / 2;
  if (w_gate_up->n % 2 || inter % 64 || w_down->n != hidden || w_down->k != inter) return TQ_ESHAPE;
  if (t < 1 || topk < 1 || topk > 32 || static_cast<long long>(t) * topk > INT_MAX / 4) return TQ_ESHAPE;
  if (E > kMaxExperts && !moe_pairs(t, topk)) return TQ_EUNSUPPORTED;  // the bucket step holds E counters in LDS
  const MoeLayout l = moe_layout(E, t, topk, hidden, inter);
  if (ws_bytes < l.total) return TQ_ENOSPACE;
  char* ws = static_cast<char*>(workspace);
  MoeArgs a;
  a.gu_words = reinterpret_cast<const uint4*>(w_gate_up->words);
  a.gu_scales = w_gate_up->scales;
  a.dn_words = reinterpret_cast<const uint4*>(w_down->words);
  a.dn_scales = w_down->scales;
  a.gu_wstride = tq_row64_words(w_gate_up->n, hidden, 3) / 4;
  a.gu_sstride = tq_row64_scales(w_gate_up->n, hidden, 128);
  a.dn_wstride = tq_row64_words(hidden, inter, 3) / 4;
  a.dn_sstride = tq_row64_scales(hidden, inter, 128);
  a.x = x;
  a.x_dtype = x_dtype;
  a.ids = expert_ids;
  a.route_w = route_w;
  a.y = y;
  a.t = t;
  a.topk = topk;
  a.experts = E;
  a.hidden = hidden;
  a.inter = inter;
  a.fused = (flags & TQ_FWHT_FUSED) ? 1 : 0;
  a.accumulate = (flags & TQ_ACCUMULATE) ? 1 : 0;
  a.bad = reinterpret_cast<int*>(ws + l.bad);
  a.num_active = reinterpret_cast<int*>(ws + l.num_active);
  a.active = reinterpret_cast<int*>(ws + l.active);
  a.seg = reinterpret_cast<int*>(ws + l.seg);
  a.pairs = reinterpret_cast<int*>(ws + l.pairs);
  a.gu = reinterpret_cast<float*>(ws + l.gu);
  a.gu_parts = slices_per_row(hidden);
  a.cnt = reinterpret_cast<int*>(ws + l.cnt);
  a.pcnt = reinterpret_cast<int*>(ws + l.fcnt);
  a.tcnt = a.pcnt + kFusedMaxPairs;
  a.o = reinterpret_cast<float*>(ws + l.o);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int P = t * topk;
  if (flags & TQ_MOE_ONE_LAUNCH) {
    if (!moe_pairs(t, topk) || slices_per_row(inter) > kFusedMaxInterSlices) return TQ_EUNSUPPORTED;
    hipLaunchKernelGGL(moe_fused_pairs_kernel, dim3(P, inter / 64, slices_per_row(hidden)), dim3(kPairGuWaves * 64),
                       0, s, a);
    TQ_LAUNCH_CHECK();
    return TQ_OK;
  }
  if (moe_pairs(t, topk)) {
    hipLaunchKernelGGL(moe_gate_up_pairs_kernel, dim3(P, inter / 64, slices_per_row(hidden)), dim3(kPairGuWaves * 64), 0,
                       s, a);
    TQ_LAUNCH_CHECK();
    if (t >= kTokMinTokens)
      hipLaunchKernelGGL(moe_down_tok_kernel, dim3(t, row_blocks(hidden)), dim3(kTokSlots * 64), 0, s, a);
    else
      hipLaunchKernelGGL(moe_down_pairs_kernel, dim3(P, row_blocks(hidden)), dim3(kPairDnWaves * 64), 0, s, a);
    TQ_LAUNCH_CHECK();
    return TQ_OK;
  }
  const int slots = P < E ? P : E;
  hipLaunchKernelGGL(moe_bucket_kernel, dim3(1), dim3(1024), 0, s, a);
  TQ_LAUNCH_CHECK();
  hipLaunchKernelGGL(moe_gate_up_kernel, dim3(slots, inter / 64), dim3(256), 0, s, a);
  TQ_LAUNCH_CHECK();
  hipLaunchKernelGGL(moe_down_kernel, dim3(slots, (row_blocks(hidden) + 3) / 4), dim3(256), 0, s, a);
  TQ_LAUNCH_CHECK();
  const size_t outs = static_cast<size_t>(t) * hidden;
  hipLaunchKernelGGL(moe_combine_kernel, dim3(static_cast<unsigned>((outs + 255) / 256)), dim3(256), 0, s, a);
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}
