// Decode GEMV on packed ternary weights: y = W_hat . (H_128 x), M = 1..8.
//
// Work split (TQ_LAYOUT_ROW64, slice-major): a workgroup owns one 640-trit K
// slice (8 quads, 5 scale groups) of W consecutive 64-row blocks; lane r of
// wavefront w owns row 64*(W*blockIdx.y + w) + r.  W is chosen on the host so
// that (row groups) x (slices) fills the compute units in a single round;
// partial sums of the slices of a row are then combined (see finish()).
// Small matrices (few row blocks per workgroup): an M == 1 workgroup still
// has five wavefronts, one per transform block of the prologue; an M >= 2
// workgroup of one or two row blocks splits each block's four units over
// four wavefronts.
// All lanes of a wavefront sit at the same K position, so activations and
// lookup tables are wavefront-uniform and scale-group boundaries fall at
// compile-time chunk positions.
//
// M == 1 (single-stream decode) uses a partial-sum table in LDS: for every
// 4-trit position p of the slice and every chunk value c in [0, 81),
// T[p][c] = sum_{i<4} (d_i(c) - 1) x'[4p + i] in FP32.  Each 4 trits then
// cost one LDS read and one add: with weights in {-1, 0, 1} the product
// reduces to sign tests and additions/subtractions ("Ternary-Bonsai2-27B vs
// Qwen3.8-27B-GSQ-RCO" page, section 1.1).  Order of work, chosen so that
// nothing waits on the weight stream before it has to:
//   1. load this wavefront's block of activations (the dtype is a template
//      parameter, so the load is branch-free and the transform waits for it
//      alone), then kLookahead quads of weights (non-temporal: streamed
//      once), then the scales (needed last; loads complete in order);
//   2. block-128 transform in registers (lane exchanges on the VALU), the
//      transformed slice staged in LDS, and the table built by every
//      wavefront of the workgroup;
//   3. decode, software-pipelined: the table reads of word w + 2 are in
//      flight while the sums of word w are formed, and quad i + kLookahead
//      is loaded while quad i is decoded.
// The two barriers wait for LDS only (a plain __syncthreads() would also
// wait for every outstanding weight load).
//
// M >= 2 runs on the matrix cores (v_mfma_f32_16x16x32_f16): x' split into
// two fp16 parts in LDS is the A operand, fp16 trit codes read from an
// 81-entry LDS table are the B operand (see gemv_mfma_kernel).
#include "tq_internal.h"

#include <atomic>
#include <mutex>

using namespace tq;

namespace {

constexpr int kSliceChunks = 160;
constexpr int kLutEntries = 81;
constexpr int kMaxWaves = 16;
constexpr int kLookahead = 3;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

struct GemvArgs {
  const uint4* words;       // ROW64 words, as quads
  const uint16_t* scales;   // ROW64 scales
  const void* x;            // [m][k]
  float* y;                 // [m][n]
  float* partial;           // [nsl][m][npad] (mode kPartial)
  int mode;                 // kDirect, kPartial or kAtomic (see finish())
  int x_dtype;
  int n, k, groups, nb, npad, nsl;
  int bpg;                  // row blocks per workgroup (wavefronts past bpg only help with the prologue)
  int fused;
};

// s_barrier after this wavefront's LDS traffic has completed; outstanding
// global loads are left in flight.
#define TQ_LDS_BARRIER() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")
// Keeps the compiler from hoisting later loads above this point.
#define TQ_ORDER() asm volatile("" ::: "memory")

__device__ __forceinline__ uint4 load_quad(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

struct Tile {
  int slice, rg, tid, wave, lane, waves, rb, rbc, nq_here, k0;
  bool active;
};

__device__ __forceinline__ Tile make_tile(const GemvArgs& a) {
  Tile t;
  t.slice = blockIdx.x;
  t.rg = blockIdx.y;
  t.tid = threadIdx.x;
  t.wave = t.tid >> 6;
  t.lane = t.tid & 63;
  t.waves = blockDim.x >> 6;
  t.rb = t.rg * a.bpg + t.wave;
  t.active = t.wave < a.bpg && t.rb < a.nb;
  t.rbc = t.active ? t.rb : a.nb - 1;
  t.nq_here = row64_slice_quads(a.k, t.slice);
  t.k0 = t.slice * kSliceTrits;
  return t;
}

template <int G>
__device__ __forceinline__ void load_scales(const GemvArgs& a, const Tile& t, float (&sc)[G]) {
  const uint16_t* sp = a.scales + row64_scale_base(t.slice, t.rbc, a.nb, G) + t.lane;
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float v = f16_to_f32(sp[j * 64]);
    sc[j] = t.active ? v : 0.0f;
  }
}

// Activations of block `blk` (0..4) of the slice for row m; zero past K.
__device__ __forceinline__ void load_block(const GemvArgs& a, const Tile& t, int m, int blk, float& v0, float& v1,
                                           bool& valid) {
  const int kb = t.k0 + blk * 128;
  valid = kb < a.k;
  load_act2(a.x, a.x_dtype, static_cast<size_t>(m) * a.k + (valid ? kb : 0) + 2 * t.lane, v0, v1);
}

// Same with the activation dtype fixed at compile time (no branch around
// the load, so later loads need not wait for it).
template <int XT>
__device__ __forceinline__ void load_block_t(const GemvArgs& a, const Tile& t, int m, int blk, float& v0, float& v1,
                                             bool& valid) {
  const int kb = t.k0 + blk * 128;
  valid = kb < a.k;
  load_act2(a.x, XT, static_cast<size_t>(m) * a.k + (valid ? kb : 0) + 2 * t.lane, v0, v1);
}

__device__ __forceinline__ void transform(const GemvArgs& a, float& v0, float& v1, bool valid, int lane) {
  if (a.fused) wave_fwht128<float>(v0, v1, lane, kInvSqrt128);
  if (!valid) {
    v0 = 0.0f;
    v1 = 0.0f;
  }
}

// How a workgroup delivers its per-row partial sums:
//   kDirect  (one slice per row):  y = partial;
//   kPartial (default):            partial[slice][m][row] = partial, summed in
//                                  slice order by reduce_kernel (deterministic);
//   kAtomic  (TQ_ACCUMULATE):      y += partial with device-scope float
//                                  atomics (single launch; the order of the
//                                  slice additions is not fixed).
enum { kDirect = 0, kPartial = 1, kAtomic = 2 };

template <int M>
__device__ __forceinline__ void finish(const GemvArgs& a, const Tile& t, const float (&part)[M]) {
  const int row = t.rb * 64 + t.lane;
  if (!t.active || row >= a.n) return;
  if (a.mode == kPartial) {
#pragma unroll
    for (int m = 0; m < M; ++m) a.partial[(static_cast<size_t>(t.slice) * M + m) * a.npad + row] = part[m];
  } else if (a.mode == kAtomic) {
#pragma unroll
    for (int m = 0; m < M; ++m) atomicAdd(&a.y[static_cast<size_t>(m) * a.n + row], part[m]);
  } else {
#pragma unroll
    for (int m = 0; m < M; ++m) a.y[static_cast<size_t>(m) * a.n + row] = part[m];
  }
}

// y[m][row] = sum over slices, in slice order, of partial[slice][m][row].
__global__ __launch_bounds__(256) void reduce_kernel(const float* __restrict__ partial, float* __restrict__ y, int m,
                                                     int n, int npad, int nsl) {
  const int row = blockIdx.x * 256 + threadIdx.x;
  const int mm = blockIdx.y;
  if (row >= n) return;
  const float* p = partial + static_cast<size_t>(mm) * npad + row;
  const size_t stride = static_cast<size_t>(m) * npad;
  float v[8];
  float sum = 0.0f;
  for (int s0 = 0; s0 < nsl; s0 += 8) {
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = (s0 + q < nsl) ? p[(s0 + q) * stride] : 0.0f;
#pragma unroll
    for (int q = 0; q < 8; ++q) sum += v[q];
  }
  y[static_cast<size_t>(mm) * n + row] = sum;
}

// ------------------------------------------------------------ M == 1 ---
// Slice chunk (0..159, trits 4p .. 4p + 3 of the slice) held by chunk h of
// slice word w in the ROW64 layout.
__host__ __device__ constexpr int slice_chunk(int w, int h) { return 40 * (w >> 3) + row64_chunk(w & 7, h); }

// Table values of the five chunks of word w (0..31) of the slice.
__device__ __forceinline__ void word_lookups(const float* lut, uint32_t word, int w, float (&v)[5]) {
  uint32_t o[5];
  word_offsets(word, o);
#pragma unroll
  for (int h = 0; h < 5; ++h) {
    const int p = slice_chunk(w, h);  // compile-time after unrolling
    v[h] = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(lut) + p * kLutEntries * 4 + o[h]);
  }
}

// The partial-sum table of the slice from its transformed activations xs
// (640 floats in LDS): T[p][c] = sum_i (d_i - 1) x'[4p + i] for position p
// (0..159) and chunk c = d0 + 3 d1 + 9 d2 + 27 d3.  Work item i (< 480):
// position i / 3, entries 27 t .. 27 t + 26 with t = i % 3 = d3.  Consecutive
// items write at a stride of 27 words, so a wavefront's stores spread over
// all banks.  Entries are A[d0 + 3 d1] + ((d2 - 1) x2 + (d3 - 1) x3), the
// products by -1, 0, 1 being exact.
__device__ __forceinline__ void build_table(float* lut, const float* xs, int tid, int nthreads) {
  for (int i = tid; i < kSliceChunks * 3; i += nthreads) {
    const int p = i / 3, t = i - 3 * p;
    const float4 x = *reinterpret_cast<const float4*>(xs + 4 * p);
    const float A[9] = {-x.x - x.y, -x.y, x.x - x.y, -x.x, 0.0f, x.x, x.y - x.x, x.y, x.x + x.y};
    const float x3 = t == 0 ? -x.w : (t == 1 ? 0.0f : x.w);
    float* row = lut + p * kLutEntries + 27 * t;
    const float base[3] = {x3 - x.z, x3, x3 + x.z};
#pragma unroll
    for (int d2 = 0; d2 < 3; ++d2)
#pragma unroll
      for (int s2 = 0; s2 < 9; ++s2) row[9 * d2 + s2] = A[s2] + base[d2];
  }
}

// G: scale groups per slice (5 at group 128, 10 at group 64).
template <int XT, int G>
__global__ __launch_bounds__(kMaxWaves * 64) void gemv_lut_m1_kernel(GemvArgs a) {
  constexpr int kChunksPerGroup = kSliceChunks / G;  // 4-trit chunks per scale group
  __shared__ float lut[kSliceChunks * kLutEntries];                   // 51840 B
  __shared__ __attribute__((aligned(16))) float xs[kSliceTrits];       // transformed activations
  const Tile t = make_tile(a);

  // Activations first (every wavefront loads a block, branch-free, so that
  // the transform below waits for this load only), then the first weights,
  // then the scales, which are needed last.
  float v0 = 0.0f, v1 = 0.0f;
  bool valid = false;
  load_block_t<XT>(a, t, 0, min(t.wave, kSliceBlocks - 1), v0, v1, valid);
  TQ_ORDER();
  const uint4* wp = a.words + row64_quad_base(t.slice, t.rbc, a.nb) + t.lane;
  uint4 wq[kSliceQuads];
#pragma unroll
  for (int i = 0; i < kLookahead; ++i) wq[i] = load_quad(wp + min(i, t.nq_here - 1) * 64);
  TQ_ORDER();
  float sc[G];
  load_scales<G>(a, t, sc);
  TQ_ORDER();

  // The slice's five transform blocks (one per wavefront, wavefronts 0..4
  // when there are five or more), staged in LDS; then every wavefront
  // builds a share of the table.
  for (int blk = t.wave; blk < kSliceBlocks; blk += t.waves) {
    if (blk != t.wave) load_block_t<XT>(a, t, 0, blk, v0, v1, valid);
    transform(a, v0, v1, valid, t.lane);
    *reinterpret_cast<float2*>(&xs[128 * blk + 2 * t.lane]) = make_float2(v0, v1);
  }
  TQ_LDS_BARRIER();
  build_table(lut, xs, t.tid, blockDim.x);
  TQ_LDS_BARRIER();
  if (t.wave >= a.bpg) return;  // a prologue-only wavefront (small matrices)

  float acc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) acc[g] = 0.0f;
  if (t.nq_here == kSliceQuads) {
    // Software-pipelined: the table reads of word w + 2 are in flight while
    // the sums of word w are formed, so the LDS and VALU pipes overlap
    // within the wavefront.
    float v[3][5];
    word_lookups(lut, wq[0].x, 0, v[0]);
    word_lookups(lut, wq[0].y, 1, v[1]);
#pragma unroll
    for (int w = 0; w < kSliceWords; ++w) {
      const int i = w >> 2;
      if ((w & 3) == 0 && i + kLookahead < kSliceQuads) wq[i + kLookahead] = load_quad(wp + (i + kLookahead) * 64);
      if (w + 2 < kSliceWords) {
        const uint4 q = wq[(w + 2) >> 2];
        const uint32_t wn = ((w + 2) & 3) == 0 ? q.x : ((w + 2) & 3) == 1 ? q.y : ((w + 2) & 3) == 2 ? q.z : q.w;
        word_lookups(lut, wn, w + 2, v[(w + 2) % 3]);
      }
#pragma unroll
      for (int h = 0; h < 5; ++h) acc[slice_chunk(w, h) / kChunksPerGroup] += v[w % 3][h];
      if ((w & 3) == 3) TQ_ORDER();
    }
  } else {
#pragma unroll
    for (int i = 0; i < kSliceQuads; ++i) {
      if (i + kLookahead < kSliceQuads) wq[i + kLookahead] = load_quad(wp + min(i + kLookahead, t.nq_here - 1) * 64);
      if (i < t.nq_here) {
        const uint32_t wv[4] = {wq[i].x, wq[i].y, wq[i].z, wq[i].w};
        float v[20];
#pragma unroll
        for (int j = 0; j < 4; ++j) word_lookups(lut, wv[j], i * 4 + j, *reinterpret_cast<float(*)[5]>(&v[j * 5]));
#pragma unroll
        for (int c = 0; c < 20; ++c) acc[slice_chunk(4 * i + c / 5, c % 5) / kChunksPerGroup] += v[c];
      }
      TQ_ORDER();
    }
  }
  float part[1] = {0.0f};
#pragma unroll
  for (int g = 0; g < G; ++g) part[0] = fmaf(sc[g], acc[g], part[0]);
  finish<1>(a, t, part);
}

// ------------------------------------------- 2 <= M <= 8 on the matrix cores ---
// v_mfma_f32_16x16x32_f16 with A = x' and B = trit codes (16 columns =
// output rows).  A row i = 2 m + p holds part p of activation row m: x'
// scaled by 2^e_m (a power of two per row and slice that puts max |x'| in
// [2^13, 2^14)) is split into p = 0: its fp16 rounding and p = 1: the fp16
// rounding of the remainder, so the 16 A rows carry all eight activation
// rows at about 22 significant bits and no fp16 overflow or underflow.
// Lane l, j = l % 16, kb = l / 16 (0..3), row quarter h (0..3) of the
// wavefront's 64-row block: output row 64 rb + 16 h + j.  In unit u (0..3,
// quads 2u and 2u + 1 of the slice) the lane decodes the unit's words 2 kb,
// 2 kb + 1 of its row; by the ROW64 chunk order (row64_chunk) their ten
// chunks are, in digit order, the chunk pairs that step s (0..4) needs:
// trits 160 u + 32 s + 8 kb .. + 7.  An 81-entry LDS table maps a chunk to
// its four fp16 codes (d - 1), so B costs one 8-byte table read per chunk.
// A step covers 32 consecutive trits and never crosses a scale group: sums
// are scaled by the row's FP32 scale every four steps.
// Lane l ends with D rows 4 kb .. 4 kb + 3: both parts of activation rows
// 2 kb and 2 kb + 1.
constexpr int kMfmaMaxWaves = 9;  // 3 per SIMD at most: ~168 registers per lane
constexpr int kXStride = kSliceTrits + 8;
constexpr int kMfmaLookahead = 10;  // of 16 word pairs per lane: weights in flight during the prologue

// kUs > 1 (small matrices): the four units of a row block's slice are
// split over kUs wavefronts (wavefront w: block w / kUs, units
// (w % kUs) 4 / kUs ..), which shortens each wavefront's dependent chain;
// their sums are added in LDS in a fixed order before the epilogue.
template <int M, int XT, int kUs, int G>
__global__ __launch_bounds__(kMfmaMaxWaves * 64) void gemv_mfma_kernel(GemvArgs a) {
  constexpr int kStepsPerGroup = kSliceTrits / G / 32;  // 32-trit matrix-core steps per scale group (4 or 2)
  constexpr int kScaleVecs = G * 64 / 8;                // 16-byte vectors of one block's scales (40 or 80)
  // A rows padded by 16 bytes: the 16 lanes of a lane group read 16 rows at
  // one offset, which then fall on 16 different 4-bank groups.
  __shared__ __attribute__((aligned(16))) _Float16 xh[2 * M][kXStride];
  __shared__ __attribute__((aligned(16))) _Float16 zeros[kSliceTrits];
  __shared__ __attribute__((aligned(16))) uint2 codes[kLutEntries];
  __shared__ __attribute__((aligned(16))) uint16_t ssc[kMfmaMaxWaves][G * 64];
  __shared__ int xexp[M];
  __shared__ float red[kUs > 1 ? kMfmaMaxWaves : 1][16][64];  // unit-split partial sums
  Tile t = make_tile(a);
  constexpr int kUnits = 4;                       // 8-word units per slice
  constexpr int kIters = 4 * kUnits;              // (unit, row quarter)
  const int j = t.lane & 15, kb = t.lane >> 4;
  const int part = t.wave % kUs;                  // this wavefront's units: u0 .. u1 - 1
  const int u0 = part * (kUnits / kUs), u1 = u0 + kUnits / kUs;
  if (kUs > 1) {  // row block of this wavefront: t.wave / kUs
    t.rb = t.rg * a.bpg + t.wave / kUs;
    t.active = t.wave / kUs < a.bpg && t.rb < a.nb;
    t.rbc = t.active ? t.rb : a.nb - 1;
  }

  // Wavefront w transforms activation row w (and w + waves, ... when there
  // are fewer wavefronts than rows): the slice's five blocks at once, loaded
  // before the weights.
  float xv[kSliceBlocks][2];
  bool xok[kSliceBlocks];
  {
    const int m = t.wave < M ? t.wave : 0;
#pragma unroll
    for (int r = 0; r < kSliceBlocks; ++r) load_block_t<XT>(a, t, m, r, xv[r][0], xv[r][1], xok[r]);
  }
  TQ_ORDER();
  // Word pair of (row quarter h, unit u): quad 2u + kb / 2, words 2 (kb % 2)
  // and + 1.  Slices are stored whole (quads past the row's end hold
  // all-zero words), so every unit is read and no clamp is needed.
  // Wavefronts past the workgroup's row blocks (small matrices: more
  // wavefronts than blocks, for the prologue) read one cached line instead.
  const bool decodes = __builtin_amdgcn_readfirstlane(t.wave < a.bpg * kUs ? 1 : 0) != 0;
  const uint32_t* wbase = reinterpret_cast<const uint32_t*>(a.words) +
                          (decodes ? (row64_quad_base(t.slice, t.rbc, a.nb) + (kb >> 1) * 64 + j) * 4 + 2 * (kb & 1)
                                   : 0);
  const int pstride = decodes ? 1 : 0;
  auto pair_at = [&](int it) { return wbase + pstride * ((2 * (it / 4)) * 64 + 16 * (it % 4)) * 4; };  // it = 4 u + h
  uint2 wq[kIters];
  if (kUs == 1) {
#pragma unroll
    for (int i = 0; i < kMfmaLookahead; ++i) wq[i] = load_pair(pair_at(i));
  } else {  // all of this wavefront's pairs (at most 8)
#pragma unroll
    for (int i = 0; i < kIters; ++i)
      if (i >= 4 * u0 && i < 4 * u1) wq[i] = load_pair(pair_at(i));
  }
  TQ_ORDER();
  // The block's G x 64 scales (640 or 1280 contiguous bytes) in 16-byte
  // loads (lanes 0..39, or all lanes and then lanes 0..15), staged in LDS;
  // each lane needs 4 G of them.  (Every lane loads, indices clamped: a load
  // under a lane condition is waited for at once.)
  constexpr int kScaleLoads = (kScaleVecs + 63) / 64;
  static_assert(kScaleLoads <= 2, "at most two scale vectors per lane");
  const uint16_t* sbase = a.scales + row64_scale_base(t.slice, t.rbc, a.nb, G);
  const uint4 scq = *reinterpret_cast<const uint4*>(sbase + 8 * (t.lane < kScaleVecs ? t.lane : 0));
  uint4 scq2 = scq;
  if constexpr (kScaleLoads > 1)
    scq2 = *reinterpret_cast<const uint4*>(sbase + 8 * (t.lane + 64 < kScaleVecs ? t.lane + 64 : 0));
  TQ_ORDER();

  build_code_table(codes, t.tid, blockDim.x);
  for (int i = t.tid; i < kSliceTrits; i += blockDim.x) zeros[i] = static_cast<_Float16>(0.0f);
  for (int m = t.wave; m < M; m += t.waves) {
    if (m != t.wave) {
#pragma unroll
      for (int r = 0; r < kSliceBlocks; ++r) load_block_t<XT>(a, t, m, r, xv[r][0], xv[r][1], xok[r]);
    }
    if (a.fused) wave_fwht128_batch<kSliceBlocks>(xv, t.lane, kInvSqrt128);
#pragma unroll
    for (int r = 0; r < kSliceBlocks; ++r) {
      if (!xok[r]) {
        xv[r][0] = 0.0f;
        xv[r][1] = 0.0f;
      }
    }
    const int e = split_two_fp16<kSliceBlocks>(xv, t.lane, &xh[2 * m][0], &xh[2 * m + 1][0]);
    if (t.lane == 0) xexp[m] = e;
  }
  // Stored after the transform, which then waits for the activations only.
  if (t.lane < kScaleVecs) *reinterpret_cast<uint4*>(&ssc[t.wave][8 * t.lane]) = scq;
  if constexpr (kScaleLoads > 1)
    if (t.lane + 64 < kScaleVecs) *reinterpret_cast<uint4*>(&ssc[t.wave][8 * (t.lane + 64)]) = scq2;
  TQ_LDS_BARRIER();

  // Scales of this lane's rows.  Five groups per slice (group 128): FP32 in
  // registers, each group's sum scaled when its last step is done.  Ten
  // (group 64): the B operand itself is scaled, s * t being exact in fp16,
  // so the accumulation runs through the slice without per-group closes
  // (closing every two steps needs more registers than the kernel has).
  constexpr bool kScaleB = G > 5;
  float sc[4][kScaleB ? 1 : G];
  if constexpr (!kScaleB) {
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float v = f16_to_f32(ssc[t.wave][g * 64 + 16 * h + j]);
        sc[h][g] = t.active ? v : 0.0f;
      }
  }
  // fp16 scale of row quarter h, group g (read at its use: volatile keeps
  // the compiler from hoisting all of them into registers).
  auto scale16 = [&](int h, int g) {
    const uint16_t v = reinterpret_cast<const volatile uint16_t*>(&ssc[t.wave][0])[g * 64 + 16 * h + j];
    return t.active ? __builtin_bit_cast(_Float16, v) : static_cast<_Float16>(0.0f);
  };

  // This lane's A row (part j % 2 of activation row j / 2, at its 8-trit
  // offset of each step), or the zero row past the M activation rows.
  const _Float16* xrow = (j < 2 * M ? &xh[j < 2 * M ? j : 0][0] : &zeros[0]) + 8 * kb;
  const char* cbase = reinterpret_cast<const char*>(codes);

  if (kUs == 1 && !decodes) return;
  float4_t acc[4];
  float tot[4][4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    acc[h] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int v = 0; v < 4; ++v) tot[h][v] = 0.0f;
  }
  // Units outer, row quarters inner: each activation operand read serves the
  // four quarters' independent accumulation chains.
#pragma unroll
  for (int u = 0; u < kUnits; ++u) {
    if (kUs > 1 && (!decodes || u < u0 || u >= u1)) continue;
    half8_t af[5];
#pragma unroll
    for (int s = 0; s < 5; ++s) af[s] = *reinterpret_cast<const half8_t*>(xrow + 160 * u + 32 * s);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int it = u * 4 + h;
      if (kUs == 1 && it + kMfmaLookahead < kIters) wq[it + kMfmaLookahead] = load_pair(pair_at(it + kMfmaLookahead));
      uint32_t o[10];
      word_offsets_s<3, false>(wq[it].x, o);
      word_offsets_s<3, false>(wq[it].y, o + 5);
      uint2 cv[10];
#pragma unroll
      for (int c = 0; c < 10; ++c) cv[c] = *reinterpret_cast<const uint2*>(cbase + o[c]);
      _Float16 s16 = static_cast<_Float16>(0.0f);
#pragma unroll
      for (int s = 0; s < 5; ++s) {
        const int step = 5 * u + s;  // scale group step / kStepsPerGroup
        const uint4 bq = make_uint4(cv[2 * s].x, cv[2 * s].y, cv[2 * s + 1].x, cv[2 * s + 1].y);
        if constexpr (kScaleB) {
          if (s == 0 || step % kStepsPerGroup == 0) s16 = scale16(h, step / kStepsPerGroup);
          const half8_t b = __builtin_bit_cast(half8_t, bq) * s16;
          acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[s], b, acc[h], 0, 0, 0);
        } else {
          acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[s], __builtin_bit_cast(half8_t, bq), acc[h], 0, 0, 0);
          // A scale group's steps can span two units; with the units split
          // over wavefronts, the last step of a wavefront's range also
          // closes its share of the group.
          if (step % kStepsPerGroup == kStepsPerGroup - 1 || (kUs > 1 && s == 4 && u == u1 - 1)) {
#pragma unroll
            for (int v = 0; v < 4; ++v) tot[h][v] = fmaf(sc[h][step / kStepsPerGroup], acc[h][v], tot[h][v]);
            acc[h] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
          }
        }
      }
    }
    TQ_ORDER();
  }
  if constexpr (kScaleB) {
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int v = 0; v < 4; ++v) tot[h][v] = acc[h][v];
  }
  if (kUs > 1) {
    // The units' sums of a row block, added in unit order by the wavefront
    // with the first units.
    if (decodes)
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[t.wave][4 * h + v][t.lane] = tot[h][v];
    __syncthreads();
    if (!decodes || part != 0) return;
#pragma unroll
    for (int p = 1; p < kUs; ++p)
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int v = 0; v < 4; ++v) tot[h][v] += red[t.wave + p][4 * h + v][t.lane];
  }
  // D rows 4 kb + v: v = 0, 1 are the two parts of activation row 2 kb,
  // v = 2, 3 those of row 2 kb + 1.
  const int mrow[2] = {2 * kb, 2 * kb + 1};
  int mexp[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) mexp[q] = mrow[q] < M ? -xexp[mrow[q] < M ? mrow[q] : 0] : 0;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int row = t.rb * 64 + 16 * h + j;
    if (t.active && row < a.n) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int m = mrow[q];
        if (m < M) {
          const float val = ldexpf(tot[h][2 * q] + tot[h][2 * q + 1], mexp[q]);
          if (a.mode == kPartial) a.partial[(static_cast<size_t>(t.slice) * M + m) * a.npad + row] = val;
          else if (a.mode == kAtomic) atomicAdd(&a.y[static_cast<size_t>(m) * a.n + row], val);
          else a.y[static_cast<size_t>(m) * a.n + row] = val;
        }
      }
    }
  }
}

// ------------------------------------------- binary {-c, +c}, M == 1 ---
// The pure 1-bit variant the TurboQuant-MLX page compares ternary against
// (point 3): 32 sign bits per word, bit i of slice word w is weight 32 w + i.
// Partial-sum table over bytes: for byte position p (0..79, weights
// 8p .. 8p + 7 of the slice) and byte value c, T[p][c] = sum_{i<8} (2 bit_i(c)
// - 1) x'[8p + i] in FP32 (81,920 B of LDS); each 8 weights then cost one
// table read and one add.  Work split and prologue as for the ternary M == 1
// kernel; a lane's 20 words of the slice (5 quads) are all requested up front.
constexpr int kBinBytes = 80;  // byte positions per slice

// T[p][c] = L(p, c & 15) + Hl(p, (c >> 4) & 3) + Hh(p, c >> 6), each part a
// sum of +-x' over 4, 2 and 2 weights.  Work item (p, lane pair hl, lo)
// writes the four entries c = 16 (4 hh + hl) + lo, hh = 0..3: the 64 lanes of
// one store touch every bank twice.
__device__ __forceinline__ void build_bin_table(float* lut, const float* xs, int tid, int nthreads) {
  for (int i = tid; i < kBinBytes * 64; i += nthreads) {
    const int p = i >> 6, hl = (i >> 4) & 3, lo = i & 15;
    const float* x = xs + 8 * p;
    float l = 0.0f;
#pragma unroll
    for (int b = 0; b < 4; ++b) l += ((lo >> b) & 1) ? x[b] : -x[b];
    const float mid = l + (((hl & 1) ? x[4] : -x[4]) + ((hl & 2) ? x[5] : -x[5]));
    float* row = lut + p * 256 + 16 * hl + lo;
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) row[64 * hh] = mid + (((hh & 1) ? x[6] : -x[6]) + ((hh & 2) ? x[7] : -x[7]));
  }
}

template <int XT, int G>
__global__ __launch_bounds__(kMaxWaves * 64) void gemv_bin_m1_kernel(GemvArgs a) {
  constexpr int kBytesPerGroup = kBinBytes / G;  // 16 at group 128, 8 at 64
  __shared__ float lut[kBinBytes * 256];                               // 81920 B
  __shared__ __attribute__((aligned(16))) float xs[kSliceTrits];
  const Tile t = make_tile(a);
  float v0 = 0.0f, v1 = 0.0f;
  bool valid = false;
  load_block_t<XT>(a, t, 0, min(t.wave, kSliceBlocks - 1), v0, v1, valid);
  TQ_ORDER();
  const uint4* wp = a.words + row64_quad_base_bin(t.slice, t.rbc, a.nb) + t.lane;
  uint4 wq[kSliceQuadsBin];
#pragma unroll
  for (int i = 0; i < kSliceQuadsBin; ++i) wq[i] = load_quad(wp + i * 64);
  TQ_ORDER();
  float sc[G];
  load_scales<G>(a, t, sc);
  TQ_ORDER();
  for (int blk = t.wave; blk < kSliceBlocks; blk += t.waves) {
    if (blk != t.wave) load_block_t<XT>(a, t, 0, blk, v0, v1, valid);
    transform(a, v0, v1, valid, t.lane);
    *reinterpret_cast<float2*>(&xs[128 * blk + 2 * t.lane]) = make_float2(v0, v1);
  }
  TQ_LDS_BARRIER();
  build_bin_table(lut, xs, t.tid, blockDim.x);
  TQ_LDS_BARRIER();
  if (t.wave >= a.bpg) return;
  float acc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) acc[g] = 0.0f;
  // Words past K hold zero bits, and x' past K is zero, so their table
  // entries are zero: the whole slice is read unconditionally.
#pragma unroll
  for (int q = 0; q < kSliceQuadsBin; ++q) {
    const uint32_t wv[4] = {wq[q].x, wq[q].y, wq[q].z, wq[q].w};
#pragma unroll
    for (int jw = 0; jw < 4; ++jw)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int p = 4 * (4 * q + jw) + b;  // compile-time
        const uint32_t c = (wv[jw] >> (8 * b)) & 0xffu;
        acc[p / kBytesPerGroup] += lut[p * 256 + c];
      }
  }
  float part[1] = {0.0f};
#pragma unroll
  for (int g = 0; g < G; ++g) part[0] = fmaf(sc[g], acc[g], part[0]);
  finish<1>(a, t, part);
}

// --------------------------------- binary {-c, +c}, 2 <= M <= 8, matrix cores ---
// As gemv_mfma_kernel (x' as two fp16 parts in the A rows, one wavefront per
// 64-row block, lane j = l % 16 on row 16 h + j of row quarter h, lane group
// kb = l / 16), with the B operand of step s (weights 32 s .. 32 s + 31 of the
// slice) taken from byte kb of word s: a 256-entry LDS table maps a byte to
// its eight fp16 signs (+-1), multiplied by the row's fp16 scale (exact).
// Lanes of one row read the same quads (four lane groups, one cache line).
template <int M, int XT, int G>
__global__ __launch_bounds__(kMfmaMaxWaves * 64) void gemv_bin_mfma_kernel(GemvArgs a) {
  constexpr int kStepsPerGroup = kSliceTrits / G / 32;
  constexpr int kScaleVecs = G * 64 / 8;
  __shared__ __attribute__((aligned(16))) _Float16 xh[2 * M][kXStride];
  __shared__ __attribute__((aligned(16))) _Float16 zeros[kSliceTrits];
  __shared__ __attribute__((aligned(16))) uint4 codes[256];
  __shared__ __attribute__((aligned(16))) uint16_t ssc[kMfmaMaxWaves][G * 64];
  __shared__ int xexp[M];
  const Tile t = make_tile(a);
  const int j = t.lane & 15, kb = t.lane >> 4;
  float xv[kSliceBlocks][2];
  bool xok[kSliceBlocks];
  {
    const int m = t.wave < M ? t.wave : 0;
#pragma unroll
    for (int r = 0; r < kSliceBlocks; ++r) load_block_t<XT>(a, t, m, r, xv[r][0], xv[r][1], xok[r]);
  }
  TQ_ORDER();
  // Quads 0..2 of the four row quarters now; quad q + 3 after unit q.
  const uint4* qbase = a.words + row64_quad_base_bin(t.slice, t.rbc, a.nb) + j;
  uint4 wq[4][kSliceQuadsBin];
#pragma unroll
  for (int q = 0; q < 3; ++q)
#pragma unroll
    for (int h = 0; h < 4; ++h) wq[h][q] = load_quad(qbase + q * 64 + 16 * h);
  TQ_ORDER();
  const uint16_t* sbase = a.scales + row64_scale_base(t.slice, t.rbc, a.nb, G);
  const uint4 scq = *reinterpret_cast<const uint4*>(sbase + 8 * (t.lane < kScaleVecs ? t.lane : 0));
  uint4 scq2 = scq;
  if constexpr (kScaleVecs > 64)
    scq2 = *reinterpret_cast<const uint4*>(sbase + 8 * (t.lane + 64 < kScaleVecs ? t.lane + 64 : 0));
  TQ_ORDER();
  for (int c = t.tid; c < 256; c += blockDim.x) {
    uint32_t d[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      d[i] = (((c >> (2 * i)) & 1) ? 0x3c00u : 0xbc00u) | ((((c >> (2 * i + 1)) & 1) ? 0x3c00u : 0xbc00u) << 16);
    codes[c] = make_uint4(d[0], d[1], d[2], d[3]);
  }
  for (int i = t.tid; i < kSliceTrits; i += blockDim.x) zeros[i] = static_cast<_Float16>(0.0f);
  for (int m = t.wave; m < M; m += t.waves) {
    if (m != t.wave) {
#pragma unroll
      for (int r = 0; r < kSliceBlocks; ++r) load_block_t<XT>(a, t, m, r, xv[r][0], xv[r][1], xok[r]);
    }
    if (a.fused) wave_fwht128_batch<kSliceBlocks>(xv, t.lane, kInvSqrt128);
#pragma unroll
    for (int r = 0; r < kSliceBlocks; ++r)
      if (!xok[r]) {
        xv[r][0] = 0.0f;
        xv[r][1] = 0.0f;
      }
    const int e = split_two_fp16<kSliceBlocks>(xv, t.lane, &xh[2 * m][0], &xh[2 * m + 1][0]);
    if (t.lane == 0) xexp[m] = e;
  }
  if (t.lane < kScaleVecs) *reinterpret_cast<uint4*>(&ssc[t.wave][8 * t.lane]) = scq;
  if constexpr (kScaleVecs > 64)
    if (t.lane + 64 < kScaleVecs) *reinterpret_cast<uint4*>(&ssc[t.wave][8 * (t.lane + 64)]) = scq2;
  TQ_LDS_BARRIER();
  if (t.wave >= a.bpg) return;  // a prologue-only wavefront

  const _Float16* xrow = (j < 2 * M ? &xh[j < 2 * M ? j : 0][0] : &zeros[0]) + 8 * kb;
  const char* cbase = reinterpret_cast<const char*>(codes);
  auto scale16 = [&](int h, int g) {
    const uint16_t v = reinterpret_cast<const volatile uint16_t*>(&ssc[t.wave][0])[g * 64 + 16 * h + j];
    return t.active ? __builtin_bit_cast(_Float16, v) : static_cast<_Float16>(0.0f);
  };
  float4_t acc[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) acc[h] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  // Unit u: steps 5u .. 5u + 4, words 5u .. 5u + 4, quads u and u + 1.
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    half8_t af[5];
#pragma unroll
    for (int s = 0; s < 5; ++s) af[s] = *reinterpret_cast<const half8_t*>(xrow + 160 * u + 32 * s);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      _Float16 s16 = static_cast<_Float16>(0.0f);
#pragma unroll
      for (int s = 0; s < 5; ++s) {
        const int step = 5 * u + s, w = step;  // word w of the slice
        const uint4 q = wq[h][w >> 2];
        const uint32_t word = (w & 3) == 0 ? q.x : (w & 3) == 1 ? q.y : (w & 3) == 2 ? q.z : q.w;
        const uint32_t off = ((word >> (8 * kb)) & 0xffu) << 4;
        if (s == 0 || step % kStepsPerGroup == 0) s16 = scale16(h, step / kStepsPerGroup);
        const half8_t b = *reinterpret_cast<const half8_t*>(cbase + off) * s16;
        acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[s], b, acc[h], 0, 0, 0);
      }
    }
    if (u + 3 < kSliceQuadsBin) {
#pragma unroll
      for (int h = 0; h < 4; ++h) wq[h][u + 3] = load_quad(qbase + (u + 3) * 64 + 16 * h);
    }
    TQ_ORDER();
  }
  // D rows 4 kb + v: v = 0, 1 the parts of activation row 2 kb, 2, 3 those of 2 kb + 1.
  const int mrow[2] = {2 * kb, 2 * kb + 1};
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int row = t.rb * 64 + 16 * h + j;
    if (t.active && row < a.n) {
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        const int m = mrow[q2];
        if (m < M) {
          const float val = ldexpf(acc[h][2 * q2] + acc[h][2 * q2 + 1], -xexp[m]);
          if (a.mode == kPartial) a.partial[(static_cast<size_t>(t.slice) * M + m) * a.npad + row] = val;
          else if (a.mode == kAtomic) atomicAdd(&a.y[static_cast<size_t>(m) * a.n + row], val);
          else a.y[static_cast<size_t>(m) * a.n + row] = val;
        }
      }
    }
  }
}

inline size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

struct GemvPlan {
  int nb, npad, nsl, waves, bpg, ngroups;
  size_t partial_bytes;
};

// Workspace: the per-slice partial sums (only when K spans several slices).
GemvPlan plan_sizes(int n, int k, int m) {
  GemvPlan p;
  p.nb = row_blocks(n);
  p.npad = p.nb * 64;
  p.nsl = slices_per_row(k);
  p.waves = 0;
  p.ngroups = 0;
  p.partial_bytes = p.nsl > 1 ? static_cast<size_t>(p.nsl) * m * p.npad * sizeof(float) : 0;
  return p;
}

// Wavefronts per workgroup: enough row blocks per workgroup that
// (row groups) x (slices) fits the compute units in one round.
void plan_waves(GemvPlan& p, int min_waves, int max_waves) {
  const int cus = tq_device_cus();
  const int per_slice = cus / p.nsl > 0 ? cus / p.nsl : 1;
  int w = (p.nb + per_slice - 1) / per_slice;
  if (w < min(min_waves, p.nb)) w = min(min_waves, p.nb);
  if (w < 1) w = 1;
  if (w > max_waves) w = max_waves;
  p.waves = w;
  p.bpg = w;
  p.ngroups = (p.nb + w - 1) / w;
}

template <int M, int kUs, int G>
void launch_mfma_us(int x_dtype, dim3 grid, dim3 block, hipStream_t s, const GemvArgs& a) {
  if (x_dtype == TQ_F32) hipLaunchKernelGGL((gemv_mfma_kernel<M, TQ_F32, kUs, G>), grid, block, 0, s, a);
  else if (x_dtype == TQ_BF16) hipLaunchKernelGGL((gemv_mfma_kernel<M, TQ_BF16, kUs, G>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((gemv_mfma_kernel<M, TQ_F16, kUs, G>), grid, block, 0, s, a);
}

template <int M>
void launch_mfma(int x_dtype, int us, int G, dim3 grid, dim3 block, hipStream_t s, const GemvArgs& a) {
  if (G == 5) {
    if (us == 4) launch_mfma_us<M, 4, 5>(x_dtype, grid, block, s, a);
    else launch_mfma_us<M, 1, 5>(x_dtype, grid, block, s, a);
  } else {
    if (us == 4) launch_mfma_us<M, 4, 10>(x_dtype, grid, block, s, a);
    else launch_mfma_us<M, 1, 10>(x_dtype, grid, block, s, a);
  }
}

template <int G>
void launch_bin_m1(int x_dtype, dim3 grid, dim3 block, hipStream_t s, const GemvArgs& a) {
  if (x_dtype == TQ_F32) hipLaunchKernelGGL((gemv_bin_m1_kernel<TQ_F32, G>), grid, block, 0, s, a);
  else if (x_dtype == TQ_BF16) hipLaunchKernelGGL((gemv_bin_m1_kernel<TQ_BF16, G>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((gemv_bin_m1_kernel<TQ_F16, G>), grid, block, 0, s, a);
}

template <int M, int G>
void launch_bin_mfma_g(int x_dtype, dim3 grid, dim3 block, hipStream_t s, const GemvArgs& a) {
  if (x_dtype == TQ_F32) hipLaunchKernelGGL((gemv_bin_mfma_kernel<M, TQ_F32, G>), grid, block, 0, s, a);
  else if (x_dtype == TQ_BF16) hipLaunchKernelGGL((gemv_bin_mfma_kernel<M, TQ_BF16, G>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((gemv_bin_mfma_kernel<M, TQ_F16, G>), grid, block, 0, s, a);
}

template <int M>
void launch_bin_mfma(int x_dtype, int G, dim3 grid, dim3 block, hipStream_t s, const GemvArgs& a) {
  if (G == 5) launch_bin_mfma_g<M, 5>(x_dtype, grid, block, s, a);
  else launch_bin_mfma_g<M, 10>(x_dtype, grid, block, s, a);
}

template <int G>
void launch_m1(int x_dtype, dim3 grid, dim3 block, hipStream_t s, const GemvArgs& a) {
  if (x_dtype == TQ_F32) hipLaunchKernelGGL((gemv_lut_m1_kernel<TQ_F32, G>), grid, block, 0, s, a);
  else if (x_dtype == TQ_BF16) hipLaunchKernelGGL((gemv_lut_m1_kernel<TQ_BF16, G>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((gemv_lut_m1_kernel<TQ_F16, G>), grid, block, 0, s, a);
}

}  // namespace

// Compute units of the current device (queried once per device).
// (A cache of a device constant: concurrent first calls store the same value,
// through atomics so that no thread reads a torn one.)
int tq_device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cus[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cus[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// Shared by the C entry points: validates a compute descriptor.
size_t tq_row64_words(int n, int k, int levels) {
  return static_cast<size_t>(slices_per_row(k)) * row_blocks(n) * (levels == 3 ? kSliceQuads : kSliceQuadsBin) * 256;
}

size_t tq_row64_scales(int n, int k, int group) {
  return static_cast<size_t>(slices_per_row(k)) * row_blocks(n) * slice_groups(group) * 64;
}

int tq_check_weights(const tq_weights* w, int experts_expected) {
  if (!w) return TQ_EINVAL;
  if (w->magic != TQ_MAGIC || w->version != TQ_VERSION) return TQ_EFORMAT;
  if (!tq_group_ok(w->group) || !tq_levels_ok(w->levels)) return TQ_EFORMAT;
  if (w->layout != TQ_LAYOUT_ROW64) return w->layout == TQ_LAYOUT_ROWMAJOR ? TQ_EUNSUPPORTED : TQ_EFORMAT;
  if (experts_expected > 0 && w->num_experts != experts_expected) return TQ_EFORMAT;
  if (w->num_experts < 1) return TQ_EFORMAT;
  if (!tq_dim_ok(w->n) || !tq_dim_ok(w->k) || w->k % TQ_GROUP) return TQ_ESHAPE;
  if (!w->words || !w->scales) return TQ_EINVAL;
  if (!tq_aligned(w->words, 16) || !tq_aligned(w->scales, 16)) return TQ_EINVAL;
  return TQ_OK;
}

size_t tq_gemv_workspace(int n, int k, int m) { return plan_sizes(n, k, m).partial_bytes; }

namespace {
int gemv_impl(const tq_weights* w, const void* x, int x_dtype, int m, float* y, unsigned flags, void* workspace,
              size_t ws_bytes, void* stream) {
  int st = tq_check_weights(w, 1);
  if (st != TQ_OK) return st;
  if (!x || !y) return TQ_EINVAL;
  if (x_dtype != TQ_F32 && x_dtype != TQ_BF16 && x_dtype != TQ_F16) return TQ_EINVAL;
  if (!tq_aligned(x, tq_act_align(x_dtype)) || !tq_aligned(y, 4)) return TQ_EINVAL;
  if (flags & ~static_cast<unsigned>(TQ_FWHT_FUSED | TQ_ACCUMULATE)) return TQ_EINVAL;
  if (m < 1 || m > 8) return TQ_ESHAPE;
  const bool binary = w->levels == 2;
  GemvPlan p = plan_sizes(w->n, w->k, m);
  int us = 1;
  const bool accumulate = (flags & TQ_ACCUMULATE) != 0;
  const int mode = accumulate ? kAtomic : (p.nsl > 1 ? kPartial : kDirect);
  if (mode == kPartial) {
    if (!workspace || !tq_aligned(workspace, 16)) return TQ_EINVAL;
    if (ws_bytes < p.partial_bytes) return TQ_ENOSPACE;
  }
  if (m == 1) {
    // Row blocks per workgroup as above; at least one wavefront per
    // transform block, so that a small matrix's prologue runs in parallel.
    plan_waves(p, 1, kMaxWaves);
    p.waves = max(p.waves, kSliceBlocks);
  } else {
    // Row blocks per workgroup so that the grid fills the compute units in
    // one round; every activation row gets a wavefront for the prologue
    // (one transform per row).
    plan_waves(p, 1, kMfmaMaxWaves);
    // One or two row blocks per workgroup (small matrices): split each
    // block's units over four wavefronts.  (A split over two wavefronts at
    // three or four row blocks measured no faster.)
    us = (!binary && 4 * p.bpg <= kMfmaMaxWaves) ? 4 : 1;
    p.waves = max(us * p.bpg, m);
  }
  GemvArgs a;
  a.words = reinterpret_cast<const uint4*>(w->words);
  a.scales = w->scales;
  a.x = x;
  a.y = y;
  a.partial = static_cast<float*>(workspace);
  a.mode = mode;
  a.x_dtype = x_dtype;
  a.n = w->n;
  a.k = w->k;
  a.groups = w->k / TQ_GROUP;
  a.nb = p.nb;
  a.npad = p.npad;
  a.nsl = p.nsl;
  a.fused = (flags & TQ_FWHT_FUSED) ? 1 : 0;
  a.bpg = p.bpg;
  const dim3 grid(p.nsl, p.ngroups);
  const dim3 block(p.waves * 64);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int G = slice_groups(w->group);
  if (binary) {
    if (m == 1) {
      if (G == 5) launch_bin_m1<5>(x_dtype, grid, block, s, a);
      else launch_bin_m1<10>(x_dtype, grid, block, s, a);
    } else {
      switch (m) {
        case 2: launch_bin_mfma<2>(x_dtype, G, grid, block, s, a); break;
        case 3: launch_bin_mfma<3>(x_dtype, G, grid, block, s, a); break;
        case 4: launch_bin_mfma<4>(x_dtype, G, grid, block, s, a); break;
        case 5: launch_bin_mfma<5>(x_dtype, G, grid, block, s, a); break;
        case 6: launch_bin_mfma<6>(x_dtype, G, grid, block, s, a); break;
        case 7: launch_bin_mfma<7>(x_dtype, G, grid, block, s, a); break;
        default: launch_bin_mfma<8>(x_dtype, G, grid, block, s, a); break;
      }
    }
    TQ_LAUNCH_CHECK();
    if (mode == kPartial) {
      hipLaunchKernelGGL(reduce_kernel, dim3((w->n + 255) / 256, m), dim3(256), 0, s, a.partial, y, m, w->n, p.npad,
                         p.nsl);
      TQ_LAUNCH_CHECK();
    }
    return TQ_OK;
  }
  switch (m) {
    case 1:
      if (G == 5) launch_m1<5>(x_dtype, grid, block, s, a);
      else launch_m1<10>(x_dtype, grid, block, s, a);
      break;
    case 2: launch_mfma<2>(x_dtype, us, G, grid, block, s, a); break;
    case 3: launch_mfma<3>(x_dtype, us, G, grid, block, s, a); break;
    case 4: launch_mfma<4>(x_dtype, us, G, grid, block, s, a); break;
    case 5: launch_mfma<5>(x_dtype, us, G, grid, block, s, a); break;
    case 6: launch_mfma<6>(x_dtype, us, G, grid, block, s, a); break;
    case 7: launch_mfma<7>(x_dtype, us, G, grid, block, s, a); break;
    default: launch_mfma<8>(x_dtype, us, G, grid, block, s, a); break;
  }
  TQ_LAUNCH_CHECK();
  if (mode == kPartial) {
    hipLaunchKernelGGL(reduce_kernel, dim3((w->n + 255) / 256, m), dim3(256), 0, s, a.partial, y, m, w->n, p.npad,
                       p.nsl);
    TQ_LAUNCH_CHECK();
  }
  return TQ_OK;
}
}  // namespace

extern "C" int tq_gemv(const tq_weights* w, const void* x, int x_dtype, int m, float* y, unsigned flags,
                       void* workspace, size_t ws_bytes, void* stream) {
  return gemv_impl(w, x, x_dtype, m, y, flags, workspace, ws_bytes, stream);
}

// ------------------------------------------ no-allocation entry point ---
// For callers that cannot allocate device memory (a workspace included):
// the slice partial sums go to one library-owned array per GPU.  In host
// code `scratch` names a host-side stand-in, never the device array: its
// device address comes from hipGetSymbolAddress, taken once per device with
// that device current, and only that address is passed to kernels.
namespace {
constexpr size_t kScratchBytes = size_t{16} << 20;
__device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

struct ScratchAddr {
  std::atomic<void*> ptr{nullptr};
  std::mutex mu;
};
ScratchAddr g_scratch_addr[64];

// Device address of this device's scratch array (looked up on the first
// call on each device).
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  ScratchAddr& slot = g_scratch_addr[dev];
  void* p = slot.ptr.load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(slot.mu);
    p = slot.ptr.load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      slot.ptr.store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}
}  // namespace

extern "C" int tq_gemv_noalloc(const tq_weights* w, const void* x, int x_dtype, int m, float* y, unsigned flags,
                               void* stream) {
  const int st = tq_check_weights(w, 1);
  if (st != TQ_OK) return st;
  if (m < 1 || m > 8) return TQ_ESHAPE;
  // The partial sums of the default (deterministic) mode must fit the array;
  // checked before any HIP call.
  const size_t need = (flags & TQ_ACCUMULATE) ? 0 : plan_sizes(w->n, w->k, m).partial_bytes;
  if (need > kScratchBytes) return TQ_ENOSPACE;
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) {
      tq_set_hip_error(e, __func__);
      return TQ_EHIP;
    }
  }
  return gemv_impl(w, x, x_dtype, m, y, flags, ws, need > 0 ? kScratchBytes : 0, stream);
}
