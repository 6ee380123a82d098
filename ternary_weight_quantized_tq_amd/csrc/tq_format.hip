// Offline conversion (rotate + ternarise), base-3 pack/unpack, scale
// re-layout, and the standalone block-128 transform.
#include "tq_internal.h"

#include <limits.h>

using namespace tq;

namespace {

// ------------------------------------------------------------ quantize ---
// One wavefront per (row, group of 128): load the group in FP64, transform
// it (27B ternary page, section 2 (1)), then absmean-ternarise with an fp16
// scale (section 2 (2); the TurboQuant-MLX page's {-c, 0, +c}).
template <typename T>
__global__ __launch_bounds__(256) void quantize_kernel(const T* __restrict__ w, int n, int k,
                                                       int8_t* __restrict__ trits,
                                                       uint16_t* __restrict__ scales) {
  const int groups = k / TQ_GROUP;
  const long long job = static_cast<long long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (job >= static_cast<long long>(n) * groups) return;
  const int lane = threadIdx.x & 63;
  const int row = static_cast<int>(job / groups);
  const int g = static_cast<int>(job % groups);
  const size_t base = static_cast<size_t>(row) * k + static_cast<size_t>(g) * TQ_GROUP + 2 * lane;
  double v0 = static_cast<double>(w[base]);
  double v1 = static_cast<double>(w[base + 1]);
  wave_fwht128<double>(v0, v1, lane, 0.08838834764831845 /* 1/sqrt(128) */);
  double s = fabs(v0) + fabs(v1);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  const double gamma = s / 128.0;
  const double thr = gamma * 0.5;
  const int8_t t0 = v0 > thr ? 1 : (v0 < -thr ? -1 : 0);
  const int8_t t1 = v1 > thr ? 1 : (v1 < -thr ? -1 : 0);
  const uint16_t pair = static_cast<uint16_t>(static_cast<uint8_t>(t0)) |
                        static_cast<uint16_t>(static_cast<uint16_t>(static_cast<uint8_t>(t1)) << 8);
  reinterpret_cast<uint16_t*>(trits + base)[0] = pair;
  if (lane == 0) scales[static_cast<size_t>(row) * groups + g] = f64_to_f16_rne(gamma);
}

// ---------------------------------------------------------------- pack ---
// word = sum_{i<20} (t_{20w+i} + 1) 3^i, evaluated by Horner from the top
// digit (TurboQuant-MLX, "Why 1.58 bit...", point 3).  One thread per word
// of the destination layout, padding included.
__device__ __forceinline__ uint32_t pack_word(const int8_t* __restrict__ row, int k, int w) {
  uint32_t acc = 0;
  const int k0 = w * TQ_TRITS_PER_WORD;
#pragma unroll
  for (int i = TQ_TRITS_PER_WORD - 1; i >= 0; --i) {
    const int kk = k0 + i;
    const uint32_t d = kk < k ? static_cast<uint32_t>(row[kk] + 1) : 1u;
    acc = acc * 3u + d;
  }
  return acc;
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
      acc = acc * 3u + (kk < k ? static_cast<uint32_t>(row[kk] + 1) : 1u);
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

__global__ __launch_bounds__(256) void scales_row64_kernel(const uint16_t* __restrict__ s, int n, int groups,
                                                           int nsl, int nb, uint16_t* __restrict__ out) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<size_t>(nsl) * nb * kSliceGroups * 64) return;
  const int r = static_cast<int>(idx & 63);
  const size_t rest = idx >> 6;
  const int gi = static_cast<int>(rest % kSliceGroups);
  const size_t sb = rest / kSliceGroups;
  const int b = static_cast<int>(sb % nb);
  const int sl = static_cast<int>(sb / nb);
  const int row = b * 64 + r;
  const int g = sl * kSliceGroups + gi;
  out[idx] = (row < n && g < groups) ? s[static_cast<size_t>(row) * groups + g] : static_cast<uint16_t>(0);
}

// -------------------------------------------------------------- unpack ---
// t = ((word / 3^i) mod 3) - 1 for digit i, peeled by repeated division.
// One thread per word: wpr words per row (ROWMAJOR), or the nsl * 32 words
// of a ROW64 row, each digit written to the column its chunk maps to.
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

size_t tq_words_per_row(int k) { return k > 0 ? static_cast<size_t>(words_per_row(k)) : 0; }

size_t tq_packed_bytes(int n, int k) {
  if (n <= 0 || k <= 0) return 0;
  return 4ull * n * words_per_row(k) + 2ull * n * (k / TQ_GROUP);
}

size_t tq_layout_words(int n, int k, int layout) {
  if (n <= 0 || k <= 0) return 0;
  if (layout == TQ_LAYOUT_ROWMAJOR) return static_cast<size_t>(n) * words_per_row(k);
  if (layout == TQ_LAYOUT_ROW64) return static_cast<size_t>(slices_per_row(k)) * row_blocks(n) * kSliceQuads * 256;
  return 0;
}

size_t tq_layout_scales(int n, int k, int layout) {
  if (n <= 0 || k <= 0 || k % TQ_GROUP) return 0;
  if (layout == TQ_LAYOUT_ROWMAJOR) return static_cast<size_t>(n) * (k / TQ_GROUP);
  if (layout == TQ_LAYOUT_ROW64) return static_cast<size_t>(slices_per_row(k)) * row_blocks(n) * kSliceGroups * 64;
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
    default: return "unknown tq status";
  }
}

int tq_quantize(const void* w, int w_dtype, int n, int k, int8_t* trits, uint16_t* scales, void* stream) {
  if (!w || !trits || !scales) return TQ_EINVAL;
  if (w_dtype != TQ_F64 && w_dtype != TQ_F32) return TQ_EINVAL;
  if (n <= 0 || k <= 0 || k % TQ_GROUP) return TQ_ESHAPE;
  const size_t jobs = static_cast<size_t>(n) * (k / TQ_GROUP);
  if (jobs > (static_cast<size_t>(UINT_MAX) / 4)) return TQ_ESHAPE;
  const unsigned grid = static_cast<unsigned>((jobs + 3) / 4);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (w_dtype == TQ_F64)
    hipLaunchKernelGGL(quantize_kernel<double>, dim3(grid), dim3(256), 0, s, static_cast<const double*>(w), n, k,
                       trits, scales);
  else
    hipLaunchKernelGGL(quantize_kernel<float>, dim3(grid), dim3(256), 0, s, static_cast<const float*>(w), n, k,
                       trits, scales);
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}

int tq_pack(const int8_t* trits, int n, int k, int layout, uint32_t* words, void* stream) {
  if (!trits || !words) return TQ_EINVAL;
  if (layout != TQ_LAYOUT_ROWMAJOR && layout != TQ_LAYOUT_ROW64) return TQ_EINVAL;
  if (n <= 0 || k <= 0) return TQ_ESHAPE;
  if (layout == TQ_LAYOUT_ROW64 && k % TQ_GROUP) return TQ_ESHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int wpr = words_per_row(k);
  if (layout == TQ_LAYOUT_ROWMAJOR) {
    hipLaunchKernelGGL(pack_rowmajor_kernel, dim3(grid_for(static_cast<size_t>(n) * wpr)), dim3(256), 0, s,
                       trits, n, k, wpr, words);
  } else {
    const int nsl = slices_per_row(k), nb = row_blocks(n);
    hipLaunchKernelGGL(pack_row64_kernel, dim3(grid_for(static_cast<size_t>(nsl) * nb * kSliceQuads * 256)),
                       dim3(256), 0, s, trits, n, k, nsl, nb, words);
  }
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}

int tq_pack_scales(const uint16_t* scales, int n, int k, int layout, uint16_t* scales_out, void* stream) {
  if (!scales || !scales_out) return TQ_EINVAL;
  if (layout != TQ_LAYOUT_ROWMAJOR && layout != TQ_LAYOUT_ROW64) return TQ_EINVAL;
  if (n <= 0 || k <= 0 || k % TQ_GROUP) return TQ_ESHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int groups = k / TQ_GROUP;
  if (layout == TQ_LAYOUT_ROWMAJOR) {
    if (hipMemcpyAsync(scales_out, scales, static_cast<size_t>(n) * groups * 2, hipMemcpyDeviceToDevice, s) !=
        hipSuccess)
      return TQ_EHIP;
    return TQ_OK;
  }
  const int nb = row_blocks(n), nsl = slices_per_row(k);
  hipLaunchKernelGGL(scales_row64_kernel, dim3(grid_for(static_cast<size_t>(nsl) * nb * kSliceGroups * 64)),
                     dim3(256), 0, s, scales, n, groups, nsl, nb, scales_out);
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}

int tq_unpack(const uint32_t* words, int n, int k, int layout, int8_t* trits, void* stream) {
  if (!words || !trits) return TQ_EINVAL;
  if (layout != TQ_LAYOUT_ROWMAJOR && layout != TQ_LAYOUT_ROW64) return TQ_EINVAL;
  if (n <= 0 || k <= 0) return TQ_ESHAPE;
  if (layout == TQ_LAYOUT_ROW64 && k % TQ_GROUP) return TQ_ESHAPE;
  const int wpr = layout == TQ_LAYOUT_ROW64 ? slices_per_row(k) * kSliceWords : words_per_row(k);
  hipLaunchKernelGGL(unpack_kernel, dim3(grid_for(static_cast<size_t>(n) * wpr)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), words, n, k, layout, wpr, row_blocks(n), trits);
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}

int tq_fwht(const void* x, int x_dtype, int m, int k, float* x_rot, void* stream) {
  if (!x || !x_rot) return TQ_EINVAL;
  if (bad_dtype(x_dtype)) return TQ_EINVAL;
  if (!tq_aligned(x, tq_act_align(x_dtype)) || !tq_aligned(x_rot, 8)) return TQ_EINVAL;
  if (m <= 0 || k <= 0 || k % TQ_GROUP) return TQ_ESHAPE;
  const size_t jobs = static_cast<size_t>(m) * (k / 128);
  if (jobs > (static_cast<size_t>(UINT_MAX) / 4)) return TQ_ESHAPE;
  hipLaunchKernelGGL(fwht_kernel, dim3(static_cast<unsigned>((jobs + 3) / 4)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), x, x_dtype, m, k, x_rot);
  TQ_LAUNCH_CHECK();
  return TQ_OK;
}

}  // extern "C"
