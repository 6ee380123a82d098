// Routed ternary expert MLP (TurboQuant-MLX page, section "Why 1.58 bit did
// not turn into gibberish", point 1: 256 routed experts, 8 active per token,
// only the experts ternary, the router gate at full precision).
//
// tq_moe_route: softmax over the expert logits, top-k, renormalised weights.
// tq_moe_gemv, four launches on the caller's stream:
//   1. bucket:   one workgroup groups the (token, slot) pairs by expert and
//                lists the experts that received tokens (ascending id).
//   2. gate/up:  grid (active expert slot, 64-row block of the intermediate
//                dimension).  Lane r of every wavefront owns gate row 64b+r
//                and up row I+64b+r of its expert; the four wavefronts split
//                K (the hidden size) into 640-trit slices.  Tokens of the
//                expert are processed 1..8 at a time against the block-128
//                transformed activations (fp16, in LDS), accumulated with
//                v_dot2_f32_f16 on fp16 trit codes; the slices are summed in
//                LDS in a fixed order and h = silu(gate) * up is stored.
//   3. down:     grid (active expert slot, 256-row group of the hidden
//                size); the block-128 transform of h is fused in, and each
//                (token, slot) pair's output row is stored.
//   4. combine:  y[t] = sum_j route_w[t][j] * o[t][j] in slot order.
// Only experts that received tokens are read; every pair's arithmetic is
// independent of which other pairs share its tile, so results do not depend
// on the order the bucket step lists pairs in.
#include "tq_internal.h"

#include <limits.h>

using namespace tq;

namespace {

constexpr int kTile = 8;          // tokens per pass
constexpr int kMaxK = 4096;       // largest hidden / intermediate size held in LDS
constexpr int kMaxExperts = 1024;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

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
  // workspace
  int* num_active;   // [1]
  int* active;       // [experts]   expert id of active slot a
  int* seg;          // [experts+1] pair range of slot a
  int* pairs;        // [t*topk]    pair indices grouped by expert
  float* h;          // [t*topk][inter]
  float* o;          // [t*topk][hidden]
};

__device__ __forceinline__ uint4 zero_quad() { return make_uint4(kZeroWord, kZeroWord, kZeroWord, kZeroWord); }

// ----------------------------------------------------------- bucket ---
__global__ __launch_bounds__(1024) void moe_bucket_kernel(MoeArgs a) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int fill[kMaxExperts];
  __shared__ int start[kMaxExperts];
  __shared__ int wsum_c[kMaxExperts / 64], wsum_f[kMaxExperts / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P = a.t * a.topk;
  for (int e = tid; e < a.experts; e += blockDim.x) {
    cnt[e] = 0;
    fill[e] = 0;
  }
  __syncthreads();
  for (int p = tid; p < P; p += blockDim.x) {
    const int e = a.ids[p];
    if (e >= 0 && e < a.experts) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
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

// Transform `len` (multiple of 128) values of one row into fp16 LDS, by
// wavefront-sized blocks; `load(i)` gives element i, dst row padded to dlen.
template <typename Load>
__device__ __forceinline__ void transform_row_f16(_Float16* dst, int len, int dlen, int wave, int nwaves, int lane,
                                                  bool fused, Load load) {
  for (int b = wave; b * 128 < dlen; b += nwaves) {
    float v0 = 0.0f, v1 = 0.0f;
    if (b * 128 < len) {
      load(b * 128 + 2 * lane, v0, v1);
      if (fused) wave_fwht128<float>(v0, v1, lane, kInvSqrt128);
    }
    dst[b * 128 + 2 * lane] = static_cast<_Float16>(v0);
    dst[b * 128 + 2 * lane + 1] = static_cast<_Float16>(v1);
  }
}

// Accumulate one 640-trit slice of R rows per lane against M activation rows.
// wp[r]: this lane's quad 0 of the slice for row r (quads 64 apart); nq_here:
// quads holding trits below K (whole units); sc[r][g]: scales; xs: LDS fp16
// activations of the slice, row stride xstride (elements).  A 160-trit unit
// (quads 2u, 2u + 1, loaded one unit ahead) spans scale groups g0 = 5u / 4
// and g0 + 1; its chunks come in ROW64 order, so each is summed into the
// accumulator of its group and both are scaled at the end of the unit.
template <int M, int R>
__device__ __forceinline__ void slice_dot2(const uint4* const (&wp)[R], const float (&sc)[R][kSliceGroups],
                                           int nq_here, const _Float16* xs, int xstride, const uint32_t* codes_lo,
                                           const uint32_t* codes_hi, float (&tot)[R][M]) {
  uint4 cur[R][2];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int q = 0; q < 2; ++q) cur[r][q] = wp[r][q * 64];
#pragma unroll
  for (int u = 0; u < kSliceQuads / 2; ++u) {
    if (2 * u < nq_here) {
      uint4 nxt[R][2];
      if (u + 1 < kSliceQuads / 2) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int q = 0; q < 2; ++q) nxt[r][q] = wp[r][min(2 * u + 2 + q, nq_here - 1) * 64];
      }
      float acc[R][M][2];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m][0] = acc[r][m][1] = 0.0f;
      const int g0 = (5 * u) / 4;
#pragma unroll
      for (int wl = 0; wl < 8; ++wl) {
        const int j = wl & 3;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint4 qv = cur[r][wl >> 2];
          const uint32_t wv = j == 0 ? qv.x : j == 1 ? qv.y : j == 2 ? qv.z : qv.w;
          uint32_t o[5];
          word_offsets(wv, o);
#pragma unroll
          for (int hh = 0; hh < 5; ++hh) {
            const int p = 40 * u + row64_chunk(wl, hh);  // chunk of the slice
            const int gi = p / 32 - g0;
            const half2_t lo = __builtin_bit_cast(
                half2_t, *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(codes_lo) + o[hh]));
            const half2_t hi = __builtin_bit_cast(
                half2_t, *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(codes_hi) + o[hh]));
#pragma unroll
            for (int m = 0; m < M; ++m) {
              const uint2 xv = *reinterpret_cast<const uint2*>(xs + m * xstride + 4 * p);
              float t = acc[r][m][gi];
              t = __builtin_amdgcn_fdot2(lo, __builtin_bit_cast(half2_t, xv.x), t, false);
              t = __builtin_amdgcn_fdot2(hi, __builtin_bit_cast(half2_t, xv.y), t, false);
              acc[r][m][gi] = t;
            }
          }
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m)
          tot[r][m] = fmaf(sc[r][g0], acc[r][m][0], fmaf(sc[r][g0 + 1], acc[r][m][1], tot[r][m]));
      if (u + 1 < kSliceQuads / 2) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int q = 0; q < 2; ++q) cur[r][q] = nxt[r][q];
      }
    }
  }
}

__device__ __forceinline__ void build_codes(uint32_t* codes_lo, uint32_t* codes_hi) {
  const int tid = threadIdx.x;
  if (tid < 81) {
    uint16_t hv[4];
    int c = tid;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hv[i] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(static_cast<float>(c % 3) - 1.0f));
      c /= 3;
    }
    codes_lo[tid] = hv[0] | (static_cast<uint32_t>(hv[1]) << 16);
    codes_hi[tid] = hv[2] | (static_cast<uint32_t>(hv[3]) << 16);
  }
}

__device__ __forceinline__ void load_scales(const uint16_t* sbase, int nb, int rb, int lane, int s,
                                            float (&dst)[kSliceGroups]) {
  const uint16_t* sp = sbase + row64_scale_base(s, rb, nb) + lane;
#pragma unroll
  for (int j = 0; j < kSliceGroups; ++j) dst[j] = f16_to_f32(sp[j * 64]);
}

// ---------------------------------------------------------- gate/up ---
template <int M>
__device__ __forceinline__ void gate_up_tile(const MoeArgs& a, int e, int b, const int* tile_pairs, _Float16* xh,
                                             float* red, const uint32_t* codes_lo, const uint32_t* codes_hi) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int K = a.hidden;
  const int nslices = slices_per_row(K), nb = row_blocks(2 * a.inter);
  const int xstride = nslices * kSliceTrits;
  const uint4* wbase = a.gu_words + static_cast<size_t>(e) * a.gu_wstride;
  const uint16_t* sbase = a.gu_scales + static_cast<size_t>(e) * a.gu_sstride;
  const int rb_gate = b, rb_up = b + a.inter / 64;
  float tot[2][M];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) tot[r][m] = 0.0f;
  for (int s = wave; s < nslices; s += 4) {
    // Gate row, then up row (two accumulators per activation row and unit
    // leave no room for both rows at once).
    const int nh = row64_slice_quads(K, s);
    {
      float sc[1][kSliceGroups];
      const uint4* const wp[1] = {wbase + row64_quad_base(s, rb_gate, nb) + lane};
      load_scales(sbase, nb, rb_gate, lane, s, sc[0]);
      slice_dot2<M, 1>(wp, sc, nh, xh + s * kSliceTrits, xstride, codes_lo, codes_hi,
                       *reinterpret_cast<float(*)[1][M]>(&tot[0][0]));
    }
    asm volatile("" ::: "memory");
    {
      float sc[1][kSliceGroups];
      const uint4* const wp[1] = {wbase + row64_quad_base(s, rb_up, nb) + lane};
      load_scales(sbase, nb, rb_up, lane, s, sc[0]);
      slice_dot2<M, 1>(wp, sc, nh, xh + s * kSliceTrits, xstride, codes_lo, codes_hi,
                       *reinterpret_cast<float(*)[1][M]>(&tot[1][0]));
    }
  }
  // red[w][r][m][lane]; slices summed in wavefront order.
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) red[((wave * 2 + r) * kTile + m) * 64 + lane] = tot[r][m];
  __syncthreads();
  for (int idx = threadIdx.x; idx < M * 64; idx += blockDim.x) {
    const int m = idx >> 6, l = idx & 63;
    float g = 0.0f, u = 0.0f;
    for (int w = 0; w < 4; ++w) {
      g += red[((w * 2 + 0) * kTile + m) * 64 + l];
      u += red[((w * 2 + 1) * kTile + m) * 64 + l];
    }
    const float hv = g / (1.0f + __expf(-g)) * u;
    a.h[static_cast<size_t>(tile_pairs[m]) * a.inter + b * 64 + l] = hv;
  }
}

__global__ __launch_bounds__(256) void moe_gate_up_kernel(MoeArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ uint32_t codes_lo[81], codes_hi[81];
  const int slot = blockIdx.x;
  if (slot >= a.num_active[0]) return;
  const int e = a.active[slot];
  const int p0 = a.seg[slot], p1 = a.seg[slot + 1];
  const int b = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int xstride = slices_per_row(a.hidden) * kSliceTrits;
  _Float16* xh = reinterpret_cast<_Float16*>(smem);                        // [kTile][xstride]
  float* red = reinterpret_cast<float*>(smem + kTile * xstride * 2);       // [4][2][kTile][64]
  build_codes(codes_lo, codes_hi);
  for (int q = p0; q < p1; q += kTile) {
    const int M = min(kTile, p1 - q);
    __syncthreads();  // previous tile's readers are done
    for (int m = 0; m < M; ++m) {
      const int tok = a.pairs[q + m] / a.topk;
      transform_row_f16(xh + m * xstride, a.hidden, xstride, wave, 4, lane, a.fused != 0,
                        [&](int i, float& v0, float& v1) {
                          load_act2(a.x, a.x_dtype, static_cast<size_t>(tok) * a.hidden + i, v0, v1);
                        });
    }
    __syncthreads();
    const int* tp = a.pairs + q;
    switch (M) {
      case 1: gate_up_tile<1>(a, e, b, tp, xh, red, codes_lo, codes_hi); break;
      case 2: gate_up_tile<2>(a, e, b, tp, xh, red, codes_lo, codes_hi); break;
      case 3: gate_up_tile<3>(a, e, b, tp, xh, red, codes_lo, codes_hi); break;
      case 4: gate_up_tile<4>(a, e, b, tp, xh, red, codes_lo, codes_hi); break;
      case 5: gate_up_tile<5>(a, e, b, tp, xh, red, codes_lo, codes_hi); break;
      case 6: gate_up_tile<6>(a, e, b, tp, xh, red, codes_lo, codes_hi); break;
      case 7: gate_up_tile<7>(a, e, b, tp, xh, red, codes_lo, codes_hi); break;
      default: gate_up_tile<8>(a, e, b, tp, xh, red, codes_lo, codes_hi); break;
    }
  }
}

// ------------------------------------------------------------- down ---
template <int M>
__device__ __forceinline__ void down_tile(const MoeArgs& a, int e, int rb, const int* tile_pairs, const _Float16* xh,
                                          const uint32_t* codes_lo, const uint32_t* codes_hi) {
  const int lane = threadIdx.x & 63;
  const int K = a.inter;
  const int nslices = slices_per_row(K);
  const int xstride = nslices * kSliceTrits;
  const int nb = row_blocks(a.hidden);
  if (rb >= nb) return;
  const uint4* wbase = a.dn_words + static_cast<size_t>(e) * a.dn_wstride;
  const uint16_t* sbase = a.dn_scales + static_cast<size_t>(e) * a.dn_sstride;
  float tot[1][M];
#pragma unroll
  for (int m = 0; m < M; ++m) tot[0][m] = 0.0f;
  for (int s = 0; s < nslices; ++s) {
    float sc[1][kSliceGroups];
    const int nh = row64_slice_quads(K, s);
    const uint4* const wp[1] = {wbase + row64_quad_base(s, rb, nb) + lane};
    load_scales(sbase, nb, rb, lane, s, sc[0]);
    slice_dot2<M, 1>(wp, sc, nh, xh + s * kSliceTrits, xstride, codes_lo,
                     codes_hi, tot);
  }
  const int row = rb * 64 + lane;
  if (row < a.hidden) {
#pragma unroll
    for (int m = 0; m < M; ++m) a.o[static_cast<size_t>(tile_pairs[m]) * a.hidden + row] = tot[0][m];
  }
}

__global__ __launch_bounds__(256) void moe_down_kernel(MoeArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ uint32_t codes_lo[81], codes_hi[81];
  const int slot = blockIdx.x;
  if (slot >= a.num_active[0]) return;
  const int e = a.active[slot];
  const int p0 = a.seg[slot], p1 = a.seg[slot + 1];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rb = blockIdx.y * 4 + wave;
  const int xstride = slices_per_row(a.inter) * kSliceTrits;
  _Float16* xh = reinterpret_cast<_Float16*>(smem);  // [kTile][xstride]
  build_codes(codes_lo, codes_hi);
  for (int q = p0; q < p1; q += kTile) {
    const int M = min(kTile, p1 - q);
    __syncthreads();
    for (int m = 0; m < M; ++m) {
      const float* hrow = a.h + static_cast<size_t>(a.pairs[q + m]) * a.inter;
      transform_row_f16(xh + m * xstride, a.inter, xstride, wave, 4, lane, true, [&](int i, float& v0, float& v1) {
        const float2 v = *reinterpret_cast<const float2*>(hrow + i);
        v0 = v.x;
        v1 = v.y;
      });
    }
    __syncthreads();
    const int* tp = a.pairs + q;
    switch (M) {
      case 1: down_tile<1>(a, e, rb, tp, xh, codes_lo, codes_hi); break;
      case 2: down_tile<2>(a, e, rb, tp, xh, codes_lo, codes_hi); break;
      case 3: down_tile<3>(a, e, rb, tp, xh, codes_lo, codes_hi); break;
      case 4: down_tile<4>(a, e, rb, tp, xh, codes_lo, codes_hi); break;
      case 5: down_tile<5>(a, e, rb, tp, xh, codes_lo, codes_hi); break;
      case 6: down_tile<6>(a, e, rb, tp, xh, codes_lo, codes_hi); break;
      case 7: down_tile<7>(a, e, rb, tp, xh, codes_lo, codes_hi); break;
      default: down_tile<8>(a, e, rb, tp, xh, codes_lo, codes_hi); break;
    }
  }
}

// ---------------------------------------------------------- combine ---
__global__ __launch_bounds__(256) void moe_combine_kernel(MoeArgs a) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<size_t>(a.t) * a.hidden) return;
  const int tok = static_cast<int>(idx / a.hidden);
  const int n = static_cast<int>(idx % a.hidden);
  float acc = 0.0f;
  for (int j = 0; j < a.topk; ++j) {
    const int p = tok * a.topk + j;
    const int e = a.ids[p];
    if (e >= 0 && e < a.experts) acc = fmaf(a.route_w[p], a.o[static_cast<size_t>(p) * a.hidden + n], acc);
  }
  a.y[idx] = acc;
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
  size_t num_active, active, seg, pairs, h, o, total;
};

MoeLayout moe_layout(int experts, int t, int topk, int hidden, int inter) {
  MoeLayout l;
  const size_t P = static_cast<size_t>(t) * topk;
  size_t off = 0;
  l.num_active = off;
  off += align256(sizeof(int));
  l.active = off;
  off += align256(sizeof(int) * experts);
  l.seg = off;
  off += align256(sizeof(int) * (experts + 1));
  l.pairs = off;
  off += align256(sizeof(int) * P);
  l.h = off;
  off += align256(sizeof(float) * P * inter);
  l.o = off;
  off += align256(sizeof(float) * P * hidden);
  l.total = off;
  return l;
}

size_t moe_smem_gate_up(int hidden) {
  const int xstride = slices_per_row(hidden) * kSliceTrits;
  return static_cast<size_t>(kTile) * xstride * 2 + 4 * 2 * kTile * 64 * sizeof(float);
}
size_t moe_smem_down(int inter) {
  const int xstride = slices_per_row(inter) * kSliceTrits;
  return static_cast<size_t>(kTile) * xstride * 2;
}

}  // namespace

size_t tq_moe_workspace(const tq_weights* gu, int t, int topk) {
  const int inter = gu->n / 2, hidden = gu->k;
  return moe_layout(gu->num_experts, t, topk, hidden, inter).total;
}

extern "C" int tq_moe_route(const float* logits, int t, int e, int topk, int32_t* ids, float* weights,
                            void* stream) {
  if (!logits || !ids || !weights) return TQ_EINVAL;
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
  if (flags & ~static_cast<unsigned>(TQ_FWHT_FUSED)) return TQ_EINVAL;
  const int E = w_gate_up->num_experts, hidden = w_gate_up->k, inter = w_gate_up->n / 2;
  if (w_gate_up->n % 2 || inter % 64 || w_down->n != hidden || w_down->k != inter) return TQ_ESHAPE;
  if (hidden > kMaxK || inter > kMaxK || E > kMaxExperts) return TQ_EUNSUPPORTED;
  if (t < 1 || topk < 1 || topk > 32 || static_cast<long long>(t) * topk > INT_MAX / 4) return TQ_ESHAPE;
  const MoeLayout l = moe_layout(E, t, topk, hidden, inter);
  if (ws_bytes < l.total) return TQ_ENOSPACE;
  char* ws = static_cast<char*>(workspace);
  MoeArgs a;
  a.gu_words = reinterpret_cast<const uint4*>(w_gate_up->words);
  a.gu_scales = w_gate_up->scales;
  a.dn_words = reinterpret_cast<const uint4*>(w_down->words);
  a.dn_scales = w_down->scales;
  a.gu_wstride = tq_layout_words(w_gate_up->n, hidden, TQ_LAYOUT_ROW64) / 4;
  a.gu_sstride = tq_layout_scales(w_gate_up->n, hidden, TQ_LAYOUT_ROW64);
  a.dn_wstride = tq_layout_words(hidden, inter, TQ_LAYOUT_ROW64) / 4;
  a.dn_sstride = tq_layout_scales(hidden, inter, TQ_LAYOUT_ROW64);
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
  a.num_active = reinterpret_cast<int*>(ws + l.num_active);
  a.active = reinterpret_cast<int*>(ws + l.active);
  a.seg = reinterpret_cast<int*>(ws + l.seg);
  a.pairs = reinterpret_cast<int*>(ws + l.pairs);
  a.h = reinterpret_cast<float*>(ws + l.h);
  a.o = reinterpret_cast<float*>(ws + l.o);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int P = t * topk;
  const int slots = P < E ? P : E;
  hipLaunchKernelGGL(moe_bucket_kernel, dim3(1), dim3(1024), 0, s, a);
  TQ_LAUNCH_CHECK();
  // Dynamic LDS above the default 64 KiB needs an explicit per-kernel limit.
  const size_t smem_gu = moe_smem_gate_up(hidden), smem_dn = moe_smem_down(inter);
  if (smem_gu > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(moe_gate_up_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem_gu));
    if (e != hipSuccess) {
      tq_set_hip_error(e, "tq_moe_gemv (gate/up LDS limit)");
      return TQ_EHIP;
    }
  }
  if (smem_dn > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(moe_down_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem_dn));
    if (e != hipSuccess) {
      tq_set_hip_error(e, "tq_moe_gemv (down LDS limit)");
      return TQ_EHIP;
    }
  }
  hipLaunchKernelGGL(moe_gate_up_kernel, dim3(slots, inter / 64), dim3(256), smem_gu, s, a);
  TQ_LAUNCH_CHECK();
  hipLaunchKernelGGL(moe_down_kernel, dim3(slots, (row_blocks(hidden) + 3) / 4), dim3(256), smem_dn, s, a);
  TQ_LAUNCH_CHECK();
  const size_t outs = static_cast<size_t>(t) * hidden;
  hipLaunchKernelGGL(moe_combine_kernel, dim3(static_cast<unsigned>((outs + 255) / 256)), dim3(256), 0, s, a);
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}
