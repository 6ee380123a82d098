// Offline conversion (rotate + ternarise), base-3 pack/unpack, scale
// re-layout, and the standalone block-128 transform.
#include "tq_internal.h"

#include <limits.h>

using namespace tq;

namespace {

// ------------------------------------------------------------ quantize ---
// A wavefront takes kQuantBlocks consecutive (row, block of 128) jobs: the
// blocks' loads are all issued first (so that enough bytes are in flight),
// then each block is transformed in FP64 (27B ternary page, section 2 (1))
// and, per scale group (the whole block at group 128; lanes 0..31 and
// 32..63 at group 64, since lane l holds elements 2l, 2l + 1), gets
// gamma = mean |w'| with an fp16 scale (section 2 (2)) and is ternarised
// with the absmean threshold (the TurboQuant-MLX page's {-c, 0, +c}) or
// takes signs (levels 2, its pure 1-bit variant).
constexpr int kQuantBlocks = 8;

template <typename T>
__global__ __launch_bounds__(256) void quantize_kernel(const T* __restrict__ w, int n, int k, int group, int levels,
                                                       int8_t* __restrict__ trits,
                                                       uint16_t* __restrict__ scales) {
  const int blocks = k / 128, groups = k / group;
  const long long jobs = static_cast<long long>(n) * blocks;
  const long long job0 = (static_cast<long long>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * kQuantBlocks;
  if (job0 >= jobs) return;
  const int lane = threadIdx.x & 63;
  double v[kQuantBlocks][2];
#pragma unroll
  for (int jb = 0; jb < kQuantBlocks; ++jb) {
    const long long job = min(job0 + jb, jobs - 1);  // past the end: a repeat, not stored
    const size_t base = static_cast<size_t>(job) * 128 + 2 * lane;  // rows are whole blocks: job * 128
    v[jb][0] = static_cast<double>(w[base]);
    v[jb][1] = static_cast<double>(w[base + 1]);
  }
#pragma unroll
  for (int jb = 0; jb < kQuantBlocks; ++jb) {
    const long long job = job0 + jb;
    if (job >= jobs) break;
    const int row = static_cast<int>(job / blocks);
    const int blk = static_cast<int>(job % blocks);
    const size_t base = static_cast<size_t>(job) * 128 + 2 * lane;
    double v0 = v[jb][0], v1 = v[jb][1];
    wave_fwht128<double>(v0, v1, lane, 0.08838834764831845 /* 1/sqrt(128) */);
    double s = fabs(v0) + fabs(v1);
    // Sum over the lanes of one group: all 64 lanes at group 128, 32 at 64.
    s += lane_xor_f64<16>(s, lane);
    s += lane_xor_f64<8>(s, lane);
    s += lane_xor_f64<4>(s, lane);
    s += lane_xor_f64<2>(s, lane);
    s += lane_xor_f64<1>(s, lane);
    const double s_other_half = lane_xor_f64<32>(s, lane);
    if (group == 128) s += s_other_half;
    const double gamma = s / static_cast<double>(group);
    int8_t t0, t1;
    if (levels == 2) {
      t0 = v0 >= 0.0 ? 1 : -1;
      t1 = v1 >= 0.0 ? 1 : -1;
    } else {
      const double thr = gamma * 0.5;
      t0 = v0 > thr ? 1 : (v0 < -thr ? -1 : 0);
      t1 = v1 > thr ? 1 : (v1 < -thr ? -1 : 0);
    }
    const uint16_t pair = static_cast<uint16_t>(static_cast<uint8_t>(t0)) |
                          static_cast<uint16_t>(static_cast<uint16_t>(static_cast<uint8_t>(t1)) << 8);
    reinterpret_cast<uint16_t*>(trits + base)[0] = pair;
    const int g = group == 128 ? blk : 2 * blk + (lane >> 5);
    if ((lane & (group == 128 ? 63 : 31)) == 0)
      scales[static_cast<size_t>(row) * groups + g] = f64_to_f16_rne(gamma);
  }
}

// ---------------------------------------------------------------- pack ---
// word = sum_{i<20} (t_{20w+i} + 1) 3^i, evaluated by Horner from the top
// digit (TurboQuant-MLX, "Why 1.58 bit...", point 3).  One thread per word
// of the destination layout, padding included.  A value outside {-1, 0, 1}
// (a caller error, counted by tq_pack_checked) is packed as 0, so every
// word stays below 3^20.
__device__ __forceinline__ uint32_t digit_of(int8_t t) {
  return (t >= -1 && t <= 1) ? static_cast<uint32_t>(t + 1) : 1u;
}

__device__ __forceinline__ uint32_t pack_word(const int8_t* __restrict__ row, int k, int w) {
  uint32_t acc = 0;
  const int k0 = w * TQ_TRITS_PER_WORD;
#pragma unroll
  for (int i = TQ_TRITS_PER_WORD - 1; i >= 0; --i) {
    const int kk = k0 + i;
    const uint32_t d = kk < k ? digit_of(row[kk]) : 1u;
    acc = acc * 3u + d;
  }
  return acc;
}

// tq_pack_checked: the number of input values outside {-1, 0, 1}.  One
// thread per 16 trits (the last thread of a ragged end reads fewer); one
// atomic per wavefront that saw any.
__global__ __launch_bounds__(64) void clear_count_kernel(int32_t* __restrict__ bad) { *bad = 0; }

__global__ __launch_bounds__(256) void count_bad_trits_kernel(const int8_t* __restrict__ t, size_t total, int levels,
                                                              int32_t* __restrict__ bad) {
  const size_t i0 = (static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 16;
  int c = 0;
  for (int i = 0; i < 16; ++i)
    if (i0 + i < total) {
      const int8_t v = t[i0 + i];
      c += (levels == 2 ? (v != -1 && v != 1) : (v < -1 || v > 1)) ? 1 : 0;
    }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off);
  if ((threadIdx.x & 63) == 0 && c) atomicAdd(bad, c);
}

__global__ __launch_bounds__(256) void pack_rowmajor_kernel(const int8_t* __restrict__ trits, int n,
                                                            int k, int wpr, uint32_t* __restrict__ words) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<size_t>(n) * wpr) return;
  const int row = static_cast<int>(idx / wpr);
  const int w = static_cast<int>(idx % wpr);
  words[idx] = pack_word(trits + static_cast<size_t>(row) * k, k, w);
}

// ROW64 (slice-major, see row64_word_index; chunk order row64_chunk): one
// thread per destination word, padding included (padded rows and trits
// past k are zero trits, so a word of padding only is the all-zero word).
__device__ __forceinline__ uint32_t pack_word_row64(const int8_t* __restrict__ row, int k, int s, int qi, int j) {
  const int wl = 4 * (qi & 1) + j;
  const int k0 = s * kSliceTrits + (qi >> 1) * 160;
  uint32_t acc = 0;
#pragma unroll
  for (int c = 4; c >= 0; --c) {
    const int kc = k0 + 4 * row64_chunk(wl, c);
#pragma unroll
    for (int d = 3; d >= 0; --d) {
      const int kk = kc + d;
      acc = acc * 3u + (kk < k ? digit_of(row[kk]) : 1u);
    }
  }
  return acc;
}

__global__ __launch_bounds__(256) void pack_row64_kernel(const int8_t* __restrict__ trits, int n, int k, int nsl,
                                                         int nb, uint32_t* __restrict__ words) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const size_t total = static_cast<size_t>(nsl) * nb * kSliceQuads * 256;
  if (idx >= total) return;
  const int j = static_cast<int>(idx & 3);
  const int r = static_cast<int>((idx >> 2) & 63);
  const int qi = static_cast<int>((idx >> 8) & 7);
  const size_t sb = idx >> 11;
  const int b = static_cast<int>(sb % nb);
  const int s = static_cast<int>(sb / nb);
  const int row = b * 64 + r;
  words[idx] = row < n ? pack_word_row64(trits + static_cast<size_t>(row) * k, k, s, qi, j) : kZeroWord;
}

// ROW64 pack through LDS: one workgroup per (slice, row block).  The
// block's 64 rows x 640 trits are staged with 16-byte loads (rows 16-byte
// aligned: k is a multiple of 128 and the caller's pointer is checked), zero
// trits past n and k, and each thread then forms 8 of the block's 2048
// words from 4-trit chunks read back as 32-bit LDS words (a chunk never
// straddles: 4 divides every chunk offset); the words leave in layout
// order, one coalesced store per thread and word.
constexpr int kTileStride = kSliceTrits + 16;  // bytes per staged row (16-byte pad against bank conflicts)

// Chunk value sum_d (t_d + 1) 3^d of four int8 trits in one 32-bit word:
// one 4-way int8 dot product with (1, 3, 9, 27) plus 40 when all four are in
// {-1, 0, 1} (chunk_trits_valid); a chunk holding another value takes the
// per-digit rule (packed as a zero trit).
__device__ __forceinline__ uint32_t chunk_value(uint32_t four) {
  if (chunk_trits_valid(four))
    return static_cast<uint32_t>(__builtin_amdgcn_sdot4(static_cast<int>(four), 0x1b090301, 40, false));
  uint32_t c = 0;
#pragma unroll
  for (int d = 3; d >= 0; --d) c = c * 3u + digit_of(static_cast<int8_t>((four >> (8 * d)) & 0xffu));
  return c;
}

__global__ __launch_bounds__(256) void pack_row64_tile_kernel(const int8_t* __restrict__ trits, int n, int k,
                                                              int nb, uint32_t* __restrict__ words) {
  __shared__ __attribute__((aligned(16))) int8_t tile[64 * kTileStride];
  const int tid = threadIdx.x;
  const int b = blockIdx.x % nb, s = blockIdx.x / nb;
  const int cols = min(kSliceTrits, k - s * kSliceTrits);  // a multiple of 128
  for (int i = tid; i < 64 * (kSliceTrits / 16); i += 256) {
    const int r = i / (kSliceTrits / 16), c16 = i % (kSliceTrits / 16);
    const int row = b * 64 + r;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (row < n && 16 * c16 < cols)
      v = *reinterpret_cast<const uint4*>(trits + static_cast<size_t>(row) * k + s * kSliceTrits + 16 * c16);
    *reinterpret_cast<uint4*>(&tile[r * kTileStride + 16 * c16]) = v;
  }
  __syncthreads();
  uint32_t* out = words + row64_quad_base(s, b, nb) * 4;
#pragma unroll
  for (int i = 0; i < kSliceQuads; ++i) {
    const int idx = tid + 256 * i;  // layout order within the block: (quad, row, word)
    const int j = idx & 3, r = (idx >> 2) & 63, qi = idx >> 8;
    const int wl = 4 * (qi & 1) + j;
    const int8_t* trow = tile + r * kTileStride + (qi >> 1) * 160;
    uint32_t acc = 0;
#pragma unroll
    for (int c = 4; c >= 0; --c)
      acc = acc * 81u + chunk_value(*reinterpret_cast<const uint32_t*>(trow + 4 * row64_chunk(wl, c)));
    out[idx] = acc;
  }
}

// ROW64 unpack through LDS, the inverse: each thread decodes 8 words of the
// block (coalesced loads) into 4-trit chunks, each written as one 32-bit
// LDS word of int8 trits (an 81-entry table maps a chunk to its four
// trits), then the staged rows leave with 16-byte stores (rows < n, columns
// < k).
__global__ __launch_bounds__(256) void unpack_row64_tile_kernel(const uint32_t* __restrict__ words, int n, int k,
                                                                int nb, int8_t* __restrict__ trits) {
  __shared__ __attribute__((aligned(16))) int8_t tile[64 * kTileStride];
  __shared__ uint32_t four[81];
  const int tid = threadIdx.x;
  const int b = blockIdx.x % nb, s = blockIdx.x / nb;
  const int cols = min(kSliceTrits, k - s * kSliceTrits);
  if (tid < 81) {
    uint32_t v = 0, c = tid;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      v |= (static_cast<uint32_t>(static_cast<int>(c % 3u) - 1) & 0xffu) << (8 * d);
      c /= 3u;
    }
    four[tid] = v;
  }
  const uint32_t* in = words + row64_quad_base(s, b, nb) * 4;
  uint32_t wv[kSliceQuads];
#pragma unroll
  for (int i = 0; i < kSliceQuads; ++i) wv[i] = in[tid + 256 * i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kSliceQuads; ++i) {
    const int idx = tid + 256 * i;
    const int j = idx & 3, r = (idx >> 2) & 63, qi = idx >> 8;
    const int wl = 4 * (qi & 1) + j;
    int8_t* trow = tile + r * kTileStride + (qi >> 1) * 160;
    uint32_t v = wv[i];
#pragma unroll
    for (int c = 0; c < 5; ++c) {
      const uint32_t q = v / 81u;
      *reinterpret_cast<uint32_t*>(trow + 4 * row64_chunk(wl, c)) = four[min(v - 81u * q, 80u)];  // < 81 unless the word is >= 3^20
      v = q;
    }
  }
  __syncthreads();
  for (int i = tid; i < 64 * (kSliceTrits / 16); i += 256) {
    const int r = i / (kSliceTrits / 16), c16 = i % (kSliceTrits / 16);
    const int row = b * 64 + r;
    if (row < n && 16 * c16 < cols)
      *reinterpret_cast<uint4*>(trits + static_cast<size_t>(row) * k + s * kSliceTrits + 16 * c16) =
          *reinterpret_cast<const uint4*>(&tile[r * kTileStride + 16 * c16]);
  }
}

// Binary words (levels 2): bit i of word w is weight 32w + i, 1 for +1; any
// value other than -1 packs as 1 (the sign rule's side for 0); bits past k
// are 0.
__device__ __forceinline__ uint32_t pack_bits(const int8_t* __restrict__ row, int k, int k0) {
  uint32_t acc = 0;
#pragma unroll
  for (int i = 0; i < TQ_BITS_PER_WORD; ++i) {
    const int kk = k0 + i;
    if (kk < k && row[kk] != -1) acc |= 1u << i;
  }
  return acc;
}

__global__ __launch_bounds__(256) void pack_bin_rowmajor_kernel(const int8_t* __restrict__ trits, int n, int k,
                                                                int wpr, uint32_t* __restrict__ words) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<size_t>(n) * wpr) return;
  const int row = static_cast<int>(idx / wpr);
  const int w = static_cast<int>(idx % wpr);
  words[idx] = pack_bits(trits + static_cast<size_t>(row) * k, k, w * TQ_BITS_PER_WORD);
}

// Binary ROW64: 20 words (5 quads) per slice, one thread per destination
// word, padding included (0).
__global__ __launch_bounds__(256) void pack_bin_row64_kernel(const int8_t* __restrict__ trits, int n, int k, int nsl,
                                                             int nb, uint32_t* __restrict__ words) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const size_t total = static_cast<size_t>(nsl) * nb * kSliceQuadsBin * 256;
  if (idx >= total) return;
  const int j = static_cast<int>(idx & 3);
  const int r = static_cast<int>((idx >> 2) & 63);
  const size_t rest = idx >> 8;
  const int qi = static_cast<int>(rest % kSliceQuadsBin);
  const size_t sb = rest / kSliceQuadsBin;
  const int b = static_cast<int>(sb % nb);
  const int s = static_cast<int>(sb / nb);
  const int row = b * 64 + r;
  const int w = s * kSliceWordsBin + 4 * qi + j;
  words[idx] = row < n ? pack_bits(trits + static_cast<size_t>(row) * k, k, w * TQ_BITS_PER_WORD) : 0u;
}

// ROW64 scale re-layout through LDS, one workgroup per row block: its 64
// rows' scales (groups contiguous per row) are read once, coalesced, and
// every slice's [group][64 rows] piece is written contiguously.  For
// blocks whose scales fit kScaleTileBytes of LDS; larger ones take
// scales_row64_kernel.
constexpr int kScaleTileBytes = 32 * 1024;
__global__ __launch_bounds__(256) void scales_row64_tile_kernel(const uint16_t* __restrict__ s, int n, int groups,
                                                                int nsl, int nb, int G, uint16_t* __restrict__ out) {
  __shared__ uint16_t tile[kScaleTileBytes / 2];  // [row][group]
  const int b = blockIdx.x, tid = threadIdx.x;
  const int rows = min(64, n - b * 64);
  const uint16_t* src = s + static_cast<size_t>(b) * 64 * groups;
  for (int i = tid; i < rows * groups; i += 256) tile[i] = src[i];  // contiguous: the block's rows are adjacent
  __syncthreads();
  for (int sl = 0; sl < nsl; ++sl) {
    uint16_t* dst = out + (static_cast<size_t>(sl) * nb + b) * G * 64;
    for (int i = tid; i < G * 64; i += 256) {
      const int gi = i >> 6, r = i & 63, g = sl * G + gi;
      dst[i] = (r < rows && g < groups) ? tile[r * groups + g] : static_cast<uint16_t>(0);
    }
  }
}

__global__ __launch_bounds__(256) void scales_row64_kernel(const uint16_t* __restrict__ s, int n, int groups,
                                                           int nsl, int nb, int G, uint16_t* __restrict__ out) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<size_t>(nsl) * nb * G * 64) return;
  const int r = static_cast<int>(idx & 63);
  const size_t rest = idx >> 6;
  const int gi = static_cast<int>(rest % G);
  const size_t sb = rest / G;
  const int b = static_cast<int>(sb % nb);
  const int sl = static_cast<int>(sb / nb);
  const int row = b * 64 + r;
  const int g = sl * G + gi;
  out[idx] = (row < n && g < groups) ? s[static_cast<size_t>(row) * groups + g] : static_cast<uint16_t>(0);
}

// -------------------------------------------------------------- unpack ---
// t = ((word / 3^i) mod 3) - 1 for digit i, peeled by repeated division.
// One thread per word: wpr words per row (ROWMAJOR), or the nsl * 32 words
// of a ROW64 row, each digit written to the column its chunk maps to.
__global__ __launch_bounds__(256) void unpack_bin_kernel(const uint32_t* __restrict__ words, int n, int k,
                                                         int layout, int wpr, int nb, int8_t* __restrict__ trits) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<size_t>(n) * wpr) return;
  const int row = static_cast<int>(idx / wpr);
  const int w = static_cast<int>(idx % wpr);
  const uint32_t v = layout == TQ_LAYOUT_ROW64 ? words[row64_word_index_bin(row, w, nb)] : words[idx];
  int8_t* out = trits + static_cast<size_t>(row) * k;
  for (int i = 0; i < TQ_BITS_PER_WORD; ++i) {
    const int kk = w * TQ_BITS_PER_WORD + i;
    if (kk < k) out[kk] = static_cast<int8_t>(2 * static_cast<int>((v >> i) & 1u) - 1);
  }
}

__global__ __launch_bounds__(256) void unpack_kernel(const uint32_t* __restrict__ words, int n, int k,
                                                     int layout, int wpr, int nb,
                                                     int8_t* __restrict__ trits) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<size_t>(n) * wpr) return;
  const int row = static_cast<int>(idx / wpr);
  const int w = static_cast<int>(idx % wpr);
  const bool r64 = layout == TQ_LAYOUT_ROW64;
  uint32_t v = r64 ? words[row64_word_index(row, w, nb)] : words[idx];
  const int wl = w & 7;
  const int k0 = (w >> 3) * 160;  // ROW64: first column of the word's unit
  int8_t* out = trits + static_cast<size_t>(row) * k;
  for (int i = 0; i < TQ_TRITS_PER_WORD; ++i) {
    const int kk = r64 ? k0 + 4 * row64_chunk(wl, i >> 2) + (i & 3) : w * TQ_TRITS_PER_WORD + i;
    const uint32_t q3 = v / 3u;
    if (kk < k) out[kk] = static_cast<int8_t>(static_cast<int>(v - 3u * q3) - 1);
    v = q3;
  }
}

// ---------------------------------------------------------------- FWHT ---
// One wavefront per block of 128 of one activation row.
__global__ __launch_bounds__(256) void fwht_kernel(const void* __restrict__ x, int dtype, int m, int k,
                                                   float* __restrict__ out) {
  const int blocks_per_row = k / 128;
  const long long job = static_cast<long long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (job >= static_cast<long long>(m) * blocks_per_row) return;
  const int lane = threadIdx.x & 63;
  const size_t base = static_cast<size_t>(job) * 128 + 2 * lane;
  float v0, v1;
  load_act2(x, dtype, base, v0, v1);
  wave_fwht128<float>(v0, v1, lane, kInvSqrt128);
  *reinterpret_cast<float2*>(out + base) = make_float2(v0, v1);
}

inline bool bad_dtype(int d) { return d != TQ_F32 && d != TQ_BF16 && d != TQ_F16; }
inline unsigned grid_for(size_t threads) { return static_cast<unsigned>((threads + 255) / 256); }

}  // namespace

extern "C" {

size_t tq_words_per_row(int k) { return tq_dim_ok(k) ? static_cast<size_t>(words_per_row(k)) : 0; }

size_t tq_packed_bytes(int n, int k) {
  if (!tq_dim_ok(n) || !tq_dim_ok(k)) return 0;
  return 4ull * n * words_per_row(k) + 2ull * n * (k / TQ_GROUP);
}

size_t tq_format_bytes(int n, int k, int group, int levels) {
  if (!tq_dim_ok(n) || !tq_dim_ok(k) || !tq_group_ok(group) || !tq_levels_ok(levels) || k % group) return 0;
  const size_t wpr = levels == 3 ? words_per_row(k) : words_per_row_bin(k);
  return 4ull * n * wpr + 2ull * n * (k / group);
}

size_t tq_layout_words(int n, int k, int layout, int levels) {
  if (!tq_dim_ok(n) || !tq_dim_ok(k) || !tq_levels_ok(levels)) return 0;
  if (layout == TQ_LAYOUT_ROWMAJOR)
    return static_cast<size_t>(n) * (levels == 3 ? words_per_row(k) : words_per_row_bin(k));
  if (layout == TQ_LAYOUT_ROW64) return tq_row64_words(n, k, levels);
  return 0;
}

size_t tq_layout_scales(int n, int k, int layout, int group) {
  if (!tq_dim_ok(n) || !tq_dim_ok(k) || !tq_group_ok(group) || k % TQ_GROUP) return 0;
  if (layout == TQ_LAYOUT_ROWMAJOR) return static_cast<size_t>(n) * (k / group);
  if (layout == TQ_LAYOUT_ROW64) return tq_row64_scales(n, k, group);
  return 0;
}

const char* tq_strerror(int status) {
  switch (status) {
    case TQ_OK: return "ok";
    case TQ_EINVAL: return "invalid argument (null pointer, dtype, flag or enum)";
    case TQ_ESHAPE: return "invalid shape (sizes out of range or K not a multiple of 128)";
    case TQ_EFORMAT: return "weight descriptor does not match (magic, version, layout or expert count)";
    case TQ_ENOSPACE: return "workspace too small";
    case TQ_EHIP: return "HIP kernel launch failed";
    case TQ_EUNSUPPORTED: return "request not supported by the library";
    case TQ_EDATA: return "input values out of range (trits outside {-1,0,1} or expert ids outside [0, E))";
    default: return "unknown tq status";
  }
}

int tq_quantize(const void* w, int w_dtype, int n, int k, int group, int levels, int8_t* trits, uint16_t* scales,
                void* stream) {
  if (!w || !trits || !scales) return TQ_EINVAL;
  if (w_dtype != TQ_F64 && w_dtype != TQ_F32) return TQ_EINVAL;
  if (!tq_group_ok(group) || !tq_levels_ok(levels)) return TQ_EINVAL;
  if (!tq_aligned(w, w_dtype == TQ_F64 ? 8 : 4) || !tq_aligned(trits, 2) || !tq_aligned(scales, 2)) return TQ_EINVAL;
  if (!tq_dim_ok(n) || !tq_dim_ok(k) || k % TQ_GROUP) return TQ_ESHAPE;
  const size_t jobs = static_cast<size_t>(n) * (k / 128);
  const size_t waves = (jobs + kQuantBlocks - 1) / kQuantBlocks;
  if (waves > (static_cast<size_t>(UINT_MAX) / 4)) return TQ_ESHAPE;
  const unsigned grid = static_cast<unsigned>((waves + 3) / 4);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (w_dtype == TQ_F64)
    hipLaunchKernelGGL(quantize_kernel<double>, dim3(grid), dim3(256), 0, s, static_cast<const double*>(w), n, k,
                       group, levels, trits, scales);
  else
    hipLaunchKernelGGL(quantize_kernel<float>, dim3(grid), dim3(256), 0, s, static_cast<const float*>(w), n, k,
                       group, levels, trits, scales);
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}

int tq_pack(const int8_t* trits, int n, int k, int layout, int levels, uint32_t* words, void* stream) {
  if (!trits || !words) return TQ_EINVAL;
  if (layout != TQ_LAYOUT_ROWMAJOR && layout != TQ_LAYOUT_ROW64) return TQ_EINVAL;
  if (!tq_levels_ok(levels)) return TQ_EINVAL;
  if (!tq_aligned(words, 4)) return TQ_EINVAL;
  if (!tq_dim_ok(n) || !tq_dim_ok(k)) return TQ_ESHAPE;
  if (layout == TQ_LAYOUT_ROW64 && k % TQ_GROUP) return TQ_ESHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (levels == 2) {
    if (layout == TQ_LAYOUT_ROWMAJOR) {
      const int wpr = words_per_row_bin(k);
      hipLaunchKernelGGL(pack_bin_rowmajor_kernel, dim3(grid_for(static_cast<size_t>(n) * wpr)), dim3(256), 0, s,
                         trits, n, k, wpr, words);
    } else {
      const int nsl = slices_per_row(k), nb = row_blocks(n);
      hipLaunchKernelGGL(pack_bin_row64_kernel, dim3(grid_for(static_cast<size_t>(nsl) * nb * kSliceQuadsBin * 256)),
                         dim3(256), 0, s, trits, n, k, nsl, nb, words);
    }
    TQ_LAUNCH_CHECK();
    return TQ_OK;
  }
  const int wpr = words_per_row(k);
  if (layout == TQ_LAYOUT_ROWMAJOR) {
    hipLaunchKernelGGL(pack_rowmajor_kernel, dim3(grid_for(static_cast<size_t>(n) * wpr)), dim3(256), 0, s,
                       trits, n, k, wpr, words);
  } else {
    const int nsl = slices_per_row(k), nb = row_blocks(n);
    if (tq_aligned(trits, 16) && static_cast<size_t>(nsl) * nb <= UINT_MAX)
      hipLaunchKernelGGL(pack_row64_tile_kernel, dim3(static_cast<unsigned>(static_cast<size_t>(nsl) * nb)),
                         dim3(256), 0, s, trits, n, k, nb, words);
    else
      hipLaunchKernelGGL(pack_row64_kernel, dim3(grid_for(static_cast<size_t>(nsl) * nb * kSliceQuads * 256)),
                         dim3(256), 0, s, trits, n, k, nsl, nb, words);
  }
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}

int tq_pack_checked(const int8_t* trits, int n, int k, int layout, int levels, uint32_t* words, int32_t* bad,
                    void* stream) {
  if (!bad || !tq_aligned(bad, 4)) return TQ_EINVAL;
  const int st = tq_pack(trits, n, k, layout, levels, words, stream);
  if (st != TQ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t total = static_cast<size_t>(n) * k;
  const size_t threads = (total + 15) / 16;
  if (threads > static_cast<size_t>(UINT_MAX)) return TQ_ESHAPE;
  hipLaunchKernelGGL(clear_count_kernel, dim3(1), dim3(64), 0, s, bad);
  TQ_LAUNCH_CHECK();
  hipLaunchKernelGGL(count_bad_trits_kernel, dim3(grid_for(threads)), dim3(256), 0, s, trits, total, levels, bad);
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}

int tq_pack_scales(const uint16_t* scales, int n, int k, int layout, int group, uint16_t* scales_out, void* stream) {
  if (!scales || !scales_out) return TQ_EINVAL;
  if (layout != TQ_LAYOUT_ROWMAJOR && layout != TQ_LAYOUT_ROW64) return TQ_EINVAL;
  if (!tq_group_ok(group)) return TQ_EINVAL;
  if (!tq_aligned(scales, 2) || !tq_aligned(scales_out, 2)) return TQ_EINVAL;
  if (!tq_dim_ok(n) || !tq_dim_ok(k) || k % TQ_GROUP) return TQ_ESHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int groups = k / group, G = slice_groups(group);
  if (layout == TQ_LAYOUT_ROWMAJOR) {
    const hipError_t e =
        hipMemcpyAsync(scales_out, scales, static_cast<size_t>(n) * groups * 2, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) {
      tq_set_hip_error(e, __func__);
      return TQ_EHIP;
    }
    return TQ_OK;
  }
  const int nb = row_blocks(n), nsl = slices_per_row(k);
  if (static_cast<size_t>(64) * groups * 2 <= kScaleTileBytes)
    hipLaunchKernelGGL(scales_row64_tile_kernel, dim3(static_cast<unsigned>(nb)), dim3(256), 0, s, scales, n, groups,
                       nsl, nb, G, scales_out);
  else
    hipLaunchKernelGGL(scales_row64_kernel, dim3(grid_for(static_cast<size_t>(nsl) * nb * G * 64)), dim3(256), 0, s,
                       scales, n, groups, nsl, nb, G, scales_out);
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}

int tq_unpack(const uint32_t* words, int n, int k, int layout, int levels, int8_t* trits, void* stream) {
  if (!words || !trits) return TQ_EINVAL;
  if (layout != TQ_LAYOUT_ROWMAJOR && layout != TQ_LAYOUT_ROW64) return TQ_EINVAL;
  if (!tq_levels_ok(levels)) return TQ_EINVAL;
  if (!tq_aligned(words, 4)) return TQ_EINVAL;
  if (!tq_dim_ok(n) || !tq_dim_ok(k)) return TQ_ESHAPE;
  if (layout == TQ_LAYOUT_ROW64 && k % TQ_GROUP) return TQ_ESHAPE;
  if (levels == 2) {
    const int wpr = layout == TQ_LAYOUT_ROW64 ? slices_per_row(k) * kSliceWordsBin : words_per_row_bin(k);
    hipLaunchKernelGGL(unpack_bin_kernel, dim3(grid_for(static_cast<size_t>(n) * wpr)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), words, n, k, layout, wpr, row_blocks(n), trits);
    TQ_LAUNCH_CHECK();
    return TQ_OK;
  }
  const int wpr = layout == TQ_LAYOUT_ROW64 ? slices_per_row(k) * kSliceWords : words_per_row(k);
  const size_t tiles = static_cast<size_t>(slices_per_row(k)) * row_blocks(n);
  if (layout == TQ_LAYOUT_ROW64 && tq_aligned(trits, 16) && tiles <= UINT_MAX)
    hipLaunchKernelGGL(unpack_row64_tile_kernel, dim3(static_cast<unsigned>(tiles)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), words, n, k, row_blocks(n), trits);
  else
    hipLaunchKernelGGL(unpack_kernel, dim3(grid_for(static_cast<size_t>(n) * wpr)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), words, n, k, layout, wpr, row_blocks(n), trits);
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}

int tq_fwht(const void* x, int x_dtype, int m, int k, float* x_rot, void* stream) {
  if (!x || !x_rot) return TQ_EINVAL;
  if (bad_dtype(x_dtype)) return TQ_EINVAL;
  if (!tq_aligned(x, tq_act_align(x_dtype)) || !tq_aligned(x_rot, 8)) return TQ_EINVAL;
  if (!tq_dim_ok(m) || !tq_dim_ok(k) || k % TQ_GROUP) return TQ_ESHAPE;
  const size_t jobs = static_cast<size_t>(m) * (k / 128);
  if (jobs > (static_cast<size_t>(UINT_MAX) / 4)) return TQ_ESHAPE;
  hipLaunchKernelGGL(fwht_kernel, dim3(static_cast<unsigned>((jobs + 3) / 4)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), x, x_dtype, m, k, x_rot);
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}

}  // extern "C"
