// Internal helpers shared by the HIP kernels and the C-ABI host layer.
#pragma once
#include <type_traits>

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq.h"
#include "tq_decode.h"

namespace tq {

constexpr uint32_t kZeroWord = 1743392200u;  // every digit 1: twenty zero trits
constexpr int kWave = 64;
constexpr float kInvSqrt128 = 0.08838834764831845f;

// ---------------------------------------------------------------- sizes ---
// A slice is 640 trits = 32 words = 8 quads of 4 words = 5 transform blocks
// of 128 = G scale groups (G = 640 / group: 5 at group 128, 10 at group 64);
// 640 = lcm(20, 128), so slices start on word, block and group boundaries.
// Binary words: a slice is 20 words = 5 quads.
constexpr int kSliceTrits = 640;
constexpr int kSliceWords = 32;
constexpr int kSliceQuads = 8;
constexpr int kSliceBlocks = 5;
constexpr int kSliceWordsBin = 20;
constexpr int kSliceQuadsBin = 5;
__host__ __device__ constexpr int slice_groups(int group) { return kSliceTrits / group; }
inline bool tq_group_ok(int group) { return group == 64 || group == 128; }
inline bool tq_levels_ok(int levels) { return levels == 2 || levels == 3; }
// A matrix or activation dimension the library takes: 1 .. TQ_MAX_DIM.
inline bool tq_dim_ok(int v) { return v > 0 && v <= TQ_MAX_DIM; }

// Pointer alignment checks of the entry points: p is a multiple of a bytes
// (a a power of two); activations are read two elements at a time.
inline bool tq_aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
inline size_t tq_act_align(int dtype) { return dtype == TQ_F32 ? 8 : 4; }

__host__ __device__ inline int words_per_row(int k) { return (k + TQ_TRITS_PER_WORD - 1) / TQ_TRITS_PER_WORD; }
__host__ __device__ inline int words_per_row_bin(int k) { return (k + TQ_BITS_PER_WORD - 1) / TQ_BITS_PER_WORD; }
__host__ __device__ inline int row_blocks(int n) { return (n + 63) / 64; }
__host__ __device__ inline int slices_per_row(int k) { return (words_per_row(k) + kSliceWords - 1) / kSliceWords; }

// TQ_LAYOUT_ROW64 addressing: slice s, row block b (64 rows), quad qi of
// the slice, row r of the block, word j of the quad:
//   word index  = (((s*nb + b)*Q + qi)*64 + r)*4 + j   (Q = 8, binary 5)
//   scale index = ((s*nb + b)*G + gi)*64 + r           (group g = Gs + gi)
// so the words of one slice of one row block are contiguous (8 KiB, binary
// 5 KiB) and a wavefront reading quad qi of its 64 rows reads 1 KiB
// contiguously.
__host__ __device__ inline size_t row64_word_index(int row, int w, int nb) {
  const int s = w / kSliceWords, qi = (w % kSliceWords) >> 2, j = w & 3, b = row >> 6, r = row & 63;
  return ((((static_cast<size_t>(s) * nb + b) * kSliceQuads + qi) * 64 + r) << 2) + j;
}
__host__ __device__ inline size_t row64_word_index_bin(int row, int w, int nb) {
  const int s = w / kSliceWordsBin, qi = (w % kSliceWordsBin) >> 2, j = w & 3, b = row >> 6, r = row & 63;
  return ((((static_cast<size_t>(s) * nb + b) * kSliceQuadsBin + qi) * 64 + r) << 2) + j;
}
__host__ __device__ inline size_t row64_scale_index(int row, int g, int nb, int G) {
  const int s = g / G, gi = g % G, b = row >> 6, r = row & 63;
  return ((static_cast<size_t>(s) * nb + b) * G + gi) * 64 + r;
}
// Quad / scale base of (slice, row block) in units of uint4 / uint16.
__host__ __device__ inline size_t row64_quad_base(int s, int b, int nb) {
  return (static_cast<size_t>(s) * nb + b) * kSliceQuads * 64;
}
__host__ __device__ inline size_t row64_quad_base_bin(int s, int b, int nb) {
  return (static_cast<size_t>(s) * nb + b) * kSliceQuadsBin * 64;
}
__host__ __device__ inline size_t row64_scale_base(int s, int b, int nb, int G) {
  return (static_cast<size_t>(s) * nb + b) * G * 64;
}
// Quads of slice s that hold trits below k: whole 160-trit units (a unit's
// chunks are reordered within it, see row64_chunk), 2 quads each.
__host__ __device__ inline int row64_slice_quads(int k, int s) {
  const int rem = k - s * kSliceTrits;
  return rem >= kSliceTrits ? kSliceQuads : 2 * ((rem + 159) / 160);
}

// ------------------------------------------------------ element loads ---
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float f16_to_f32(uint16_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, b));
}
__device__ __forceinline__ float load_act(const void* x, int dtype, size_t i) {
  if (dtype == TQ_F32) return static_cast<const float*>(x)[i];
  if (dtype == TQ_BF16) return bf16_to_f32(static_cast<const uint16_t*>(x)[i]);
  return f16_to_f32(static_cast<const uint16_t*>(x)[i]);
}
// Two consecutive activations (i even).
__device__ __forceinline__ void load_act2(const void* x, int dtype, size_t i, float& a, float& b) {
  if (dtype == TQ_F32) {
    const float2 v = *reinterpret_cast<const float2*>(static_cast<const float*>(x) + i);
    a = v.x;
    b = v.y;
  } else {
    const uint32_t v = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(x) + i);
    if (dtype == TQ_BF16) {
      a = __uint_as_float(v << 16);
      b = __uint_as_float(v & 0xffff0000u);
    } else {
      a = f16_to_f32(static_cast<uint16_t>(v & 0xffffu));
      b = f16_to_f32(static_cast<uint16_t>(v >> 16));
    }
  }
}

// ----------------------------------------------- block-128 transform ---
// Value of lane (lane ^ S) for S = 1..32, all on the VALU (no LDS queue, so
// the exchanges never wait behind another wavefront's LDS traffic): DPP
// inside 16-lane rows for S <= 8 (quad_perm for 1 and 2, row shifts for 4,
// row rotate for 8), v_permlane16_swap for 16 and v_permlane32_swap for 32.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int S>
__device__ __forceinline__ float lane_xor_f32(float v, int lane) {
  if constexpr (S == 1) return dpp_f32<0xB1>(v);         // quad_perm(1,0,3,2)
  else if constexpr (S == 2) return dpp_f32<0x4E>(v);    // quad_perm(2,3,0,1)
  else if constexpr (S == 4) {
    const float up = dpp_f32<0x104>(v);                  // row_shl:4, lane i <- i + 4
    const float dn = dpp_f32<0x114>(v);                  // row_shr:4, lane i <- i - 4
    return (lane & 4) ? dn : up;
  } else if constexpr (S == 8) return dpp_f32<0x128>(v);  // row_ror:8
  else if constexpr (S == 16) {
    // Both operands v: the first result holds v's rows 0, 0, 2, 2 and the
    // second v's rows 1, 1, 3, 3 (16-lane rows 0..3).
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((lane & 16) ? r[0] : r[1]);
  } else {
    static_assert(S == 32, "lane strides 1..32");
    // Both operands v: the first result holds v's lanes 0..31 twice, the
    // second v's lanes 32..63 twice.
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((lane & 32) ? r[0] : r[1]);
  }
}

// The same exchange for a double: its two 32-bit halves moved by the
// 32-bit exchange (bit moves and selects only, so the value is exact).
template <int S>
__device__ __forceinline__ double lane_xor_f64(double v, int lane) {
  const unsigned long long b = static_cast<unsigned long long>(__double_as_longlong(v));
  const uint32_t lo = __float_as_uint(lane_xor_f32<S>(__uint_as_float(static_cast<uint32_t>(b)), lane));
  const uint32_t hi = __float_as_uint(lane_xor_f32<S>(__uint_as_float(static_cast<uint32_t>(b >> 32)), lane));
  return __longlong_as_double(static_cast<long long>((static_cast<unsigned long long>(hi) << 32) | lo));
}
// Sum of v over the wavefront, lane strides 32, 16, .., 1 in that order
// (every lane gets it).
__device__ __forceinline__ double wave_sum_f64(double v, int lane) {
  v += lane_xor_f64<32>(v, lane);
  v += lane_xor_f64<16>(v, lane);
  v += lane_xor_f64<8>(v, lane);
  v += lane_xor_f64<4>(v, lane);
  v += lane_xor_f64<2>(v, lane);
  v += lane_xor_f64<1>(v, lane);
  return v;
}

// Walsh-Hadamard transform of B independent blocks of 128 (one per v[r]),
// each held by the wavefront with lane l owning elements 2l and 2l+1.
// Stage stride 1 is inside the lane; strides 2..64 pair lane l with lane
// l ^ (stride/2).  Scaled by 1/sqrt(128).  The blocks go stage by stage, so
// that their lane exchanges are in flight together.
template <int S, int B>
__device__ __forceinline__ void fwht_batch_stage(float (&a)[B], float (&b)[B], int lane) {
  float pa[B], pb[B];
#pragma unroll
  for (int r = 0; r < B; ++r) {
    pa[r] = lane_xor_f32<S>(a[r], lane);
    pb[r] = lane_xor_f32<S>(b[r], lane);
  }
  // Lower lane of a pair: a + p; upper lane: p - a.  Both are p + sgn * a.
  const float sgn = (lane & S) ? -1.0f : 1.0f;
#pragma unroll
  for (int r = 0; r < B; ++r) {
    a[r] = fmaf(sgn, a[r], pa[r]);
    b[r] = fmaf(sgn, b[r], pb[r]);
  }
}
template <int B>
__device__ __forceinline__ void wave_fwht128_batch(float (&v)[B][2], int lane, float scale) {
  float a[B], b[B];
#pragma unroll
  for (int r = 0; r < B; ++r) {
    a[r] = v[r][0] + v[r][1];
    b[r] = v[r][0] - v[r][1];
  }
  fwht_batch_stage<1>(a, b, lane);
  fwht_batch_stage<2>(a, b, lane);
  fwht_batch_stage<4>(a, b, lane);
  fwht_batch_stage<8>(a, b, lane);
  fwht_batch_stage<16>(a, b, lane);
  fwht_batch_stage<32>(a, b, lane);
#pragma unroll
  for (int r = 0; r < B; ++r) {
    v[r][0] = a[r] * scale;
    v[r][1] = b[r] * scale;
  }
}

// One block: float on the VALU exchanges above; other types (the FP64
// quantiser) through ds_bpermute.
template <typename T>
__device__ __forceinline__ void wave_fwht128(T& v0, T& v1, int lane, T scale) {
  if constexpr (sizeof(T) == sizeof(float)) {
    float v[1][2] = {{v0, v1}};
    wave_fwht128_batch<1>(v, lane, scale);
    v0 = v[0][0];
    v1 = v[0][1];
  } else {
    T a = v0 + v1, b = v0 - v1;
    // Stage of stride S: the lower lane of a pair keeps a + p, the upper p - a.
    auto stage = [&](auto tag) {
      constexpr int S = decltype(tag)::value;
      const T pa = lane_xor_f64<S>(a, lane);
      const T pb = lane_xor_f64<S>(b, lane);
      const T sgn = (lane & S) ? T(-1) : T(1);
      a = sgn * a + pa;
      b = sgn * b + pb;
    };
    stage(std::integral_constant<int, 1>{});
    stage(std::integral_constant<int, 2>{});
    stage(std::integral_constant<int, 4>{});
    stage(std::integral_constant<int, 8>{});
    stage(std::integral_constant<int, 16>{});
    stage(std::integral_constant<int, 32>{});
    v0 = a * scale;
    v1 = b * scale;
  }
}

// ------------------------------------------- matrix-core decode helpers ---
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// Two consecutive words, streamed once (non-temporal).
__device__ __forceinline__ uint2 load_pair(const uint32_t* p) {
  typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v.x, v.y);
}

// Maximum of v over the wavefront (every lane gets it).
__device__ __forceinline__ float wave_max(float v, int lane) {
  v = fmaxf(v, lane_xor_f32<1>(v, lane));
  v = fmaxf(v, lane_xor_f32<2>(v, lane));
  v = fmaxf(v, lane_xor_f32<4>(v, lane));
  v = fmaxf(v, lane_xor_f32<8>(v, lane));
  v = fmaxf(v, lane_xor_f32<16>(v, lane));
  return fmaxf(v, lane_xor_f32<32>(v, lane));
}

// Entry c of the 81-entry table of a 4-trit chunk: its four fp16 codes
// (d_i - 1), digits 0, 1 in .x and 2, 3 in .y.
__device__ __forceinline__ void build_code_table(uint2* codes, int tid, int nthreads) {
  for (int e = tid; e < 81; e += nthreads) {
    uint16_t hv[4];
    int c = e;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hv[i] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(static_cast<float>(c % 3) - 1.0f));
      c /= 3;
    }
    codes[e] = make_uint2(hv[0] | (static_cast<uint32_t>(hv[1]) << 16), hv[2] | (static_cast<uint32_t>(hv[3]) << 16));
  }
}

// A wavefront's NB transformed blocks of one activation row (lane l holds
// elements 2l, 2l+1 of each) as the two fp16 parts of the matrix-core A
// operand: with e from the wavefront maximum so that max |x'| 2^e lies in
// [2^13, 2^14), hi = fp16(x' 2^e) and lo = fp16(x' 2^e - hi), both finite
// and normal down to |x'| 2^e ~ 2^-3; together about 22 significant bits.
// Writes hi[128 b + 2l], lo[128 b + 2l] (and + 1); returns e.
template <int NB>
__device__ __forceinline__ int split_two_fp16(const float (&xv)[NB][2], int lane, _Float16* hi, _Float16* lo) {
  float mx = 0.0f;
#pragma unroll
  for (int b = 0; b < NB; ++b) mx = fmaxf(mx, fmaxf(fabsf(xv[b][0]), fabsf(xv[b][1])));
  mx = wave_max(mx, lane);
  const int e = mx > 0.0f ? 14 - __builtin_amdgcn_frexp_expf(mx) : 0;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const float s0 = ldexpf(xv[b][0], e), s1 = ldexpf(xv[b][1], e);
    const _Float16 h0 = static_cast<_Float16>(s0), h1 = static_cast<_Float16>(s1);
    const half2_t hv = {h0, h1};
    const half2_t lv = {static_cast<_Float16>(s0 - static_cast<float>(h0)),
                        static_cast<_Float16>(s1 - static_cast<float>(h1))};
    *reinterpret_cast<half2_t*>(hi + b * 128 + 2 * lane) = hv;
    *reinterpret_cast<half2_t*>(lo + b * 128 + 2 * lane) = lv;
  }
  return e;
}

// ------------------------------------------------- fp16 bit patterns ---
// Round a double to the nearest fp16 (ties to even) in a single rounding.
__host__ __device__ inline uint16_t f64_to_f16_rne(double d) {
  uint64_t b;
  __builtin_memcpy(&b, &d, 8);
  const uint16_t sign = static_cast<uint16_t>((b >> 48) & 0x8000u);
  const int exp = static_cast<int>((b >> 52) & 0x7ff);
  const uint64_t mant = b & ((1ull << 52) - 1);
  if (exp == 0x7ff) return sign | 0x7c00u | (mant ? 0x200u : 0u);
  if (exp == 0) return sign;  // fp64 subnormals are far below fp16's range
  const int e = exp - 1023;
  const uint64_t m = mant | (1ull << 52);  // 53-bit significand, value m * 2^(e-52)
  int shift;
  int he;
  if (e >= -14) {  // normal fp16 candidate: 11-bit significand
    shift = 42;
    he = e + 15;
  } else {  // subnormal: units of 2^-24
    shift = 42 + (-14 - e);
    he = 0;
    if (shift > 63) return sign;
  }
  uint64_t q = m >> shift;
  const uint64_t r = m & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (r > half || (r == half && (q & 1))) ++q;
  if (he == 0) {
    // q <= 1024; q == 1024 is the smallest normal, which the encoding below
    // produces naturally (exponent field 1, mantissa 0).
    return sign | static_cast<uint16_t>(q);
  }
  if (q == (1ull << 11)) {  // significand overflow
    q >>= 1;
    ++he;
  }
  if (he >= 31) return sign | 0x7c00u;
  return sign | static_cast<uint16_t>(he << 10) | static_cast<uint16_t>(q & 0x3ffu);
}

}  // namespace tq

// Records a HIP failure for tq_last_error() (per host thread).
void tq_set_hip_error(hipError_t e, const char* where);

// Host-side launch check shared by all entry points.
#define TQ_LAUNCH_CHECK()                      \
  do {                                         \
    const hipError_t tq_e_ = hipGetLastError(); \
    if (tq_e_ != hipSuccess) {                 \
      tq_set_hip_error(tq_e_, __func__);       \
      return TQ_EHIP;                          \
    }                                          \
  } while (0)

// Host-side helpers defined in the kernel sources.
int tq_check_weights(const tq_weights* w, int experts_expected);
// Words / scales of one matrix in the ROW64 layout.
size_t tq_row64_words(int n, int k, int levels);
size_t tq_row64_scales(int n, int k, int group);
int tq_device_cus();
size_t tq_gemv_workspace(int n, int k, int m);
size_t tq_moe_workspace(const tq_weights* gu, int t, int topk);
size_t tq_gemm_workspace(int n, int k, int m);
