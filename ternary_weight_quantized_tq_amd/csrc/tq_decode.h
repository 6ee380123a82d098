// Splitting a packed base-3 word into base-81 chunks (as LDS byte offsets).
//
// A word holds 20 ternary digits d_0..d_19 (d = t + 1), least significant
// first: w = sum_i d_i 3^i < 3^20.  The kernels consume it four digits at a
// time: chunk c_j = d_{4j} + 3 d_{4j+1} + 9 d_{4j+2} + 27 d_{4j+3} in [0, 81),
// so w = sum_j c_j 81^j.  Because 4 divides both 20 and 128, a chunk never
// straddles a scale group.  word_offsets() returns 4*c_j, the byte offset of
// entry c_j in a table of 4-byte entries.
//
// Every step is one full-rate instruction (no division, no 64-bit
// arithmetic beyond one FP64 FMA):
//   a  = floor(w / 3^8):  one FP64 FMA, floor(w * (1/6561) + 0.5/6561).  For
//        w < 3^20 the FMA is within 1.3e-10 of (w + 0.5)/6561, which lies at
//        least 0.5/6561 = 7.6e-5 from an integer, so truncation is exact.
//   e  = floor(a / 6561) = mulhi_u24(a, 654622): 654622 = ceil(2^32/6561),
//        exact while a * (654622*6561 - 2^32) < 2^32, i.e. a < 561736, and
//        a < 3^12 = 531441.
//   4b = 4w - 26244 a (digits 0..7, times 4) and 4m = 4a - 26244 e (digits
//        8..15, times 4) by 24-bit multiply-add, exact modulo 2^32.
//   floor(b / 81) = mulhi_u24(4b, 13256072): 13256072 = ceil(2^30/81) and
//        81 * 13256072 = 2^30 + 8, so the error stays below 6e-7 < 1/81.
//   4 c_even = 4v - 324 floor(v/81), 4 c_odd = floor(v/81) << 2.
// 15 VALU instructions per word for five offsets.  The host build of this
// header emulates the same instructions (24-bit operands) so that a CPU test
// can check every step exhaustively against plain division.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define TQ_HD __host__ __device__ __forceinline__
#else
#define TQ_HD static inline
#endif

namespace tq {

// Low 32 bits of sext24(a) * sext24(b) + c  (v_mad_i32_i24).
// kAsm: emit the instruction as inline asm, one instruction; the compiler
// otherwise emits v_mul_lo_u32 and an add (on gfx950 v_mul_lo_u32 issues
// at the rate of v_add_u32: measured 5.3 against 5.3 clocks per
// instruction on one wavefront).  Inline asm is hidden from the compiler's
// hazard tracking, so kernels that issue matrix-core (MFMA) instructions
// must use kAsm = false: an asm write can land on a register an MFMA is
// still reading.
template <bool kAsm = true>
TQ_HD uint32_t mad_i24(uint32_t a, int32_t b, uint32_t c) {
#if defined(__HIP_DEVICE_COMPILE__)
  if constexpr (kAsm) {
    uint32_t r;
    asm("v_mad_i32_i24 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(b), "v"(c));
    return r;
  } else {
    return static_cast<uint32_t>(static_cast<int32_t>(a) * b) + c;  // operands fit 24 bits at every call
  }
#else
  const int64_t sa = static_cast<int64_t>(static_cast<int32_t>(a << 8) >> 8);
  const int64_t sb = static_cast<int64_t>(static_cast<int32_t>(static_cast<uint32_t>(b) << 8) >> 8);
  return static_cast<uint32_t>(static_cast<uint64_t>(sa * sb) + c);
#endif
}

// Bits 32..47 of (a & 0xffffff) * (b & 0xffffff)  (v_mul_hi_u32_u24; the
// compiler selects it from this form).
TQ_HD uint32_t mulhi_u24(uint32_t a, uint32_t b) {
  return static_cast<uint32_t>((static_cast<uint64_t>(a & 0xffffffu) * (b & 0xffffffu)) >> 32);
}

// o[j] = 2^S * chunk j (digits 4j..4j+3) of the word: the byte offset of
// entry c_j in a table of 2^S-byte entries (S = 2: 4-byte entries, S = 3:
// 8-byte entries).  The constants scale with 2^S: 4b = 4w - 26244 a becomes
// 2^S b = 2^S w - 6561 * 2^S a, and floor(b / 81) = mulhi_u24(2^S b,
// ceil(2^(32-S) / 81)), exact for b < 6561 (the multiplier exceeds
// 2^(32-S)/81 by less than 1, so the error stays below 6561 * 2^S / 2^32).
template <int S, bool kAsm = true>
TQ_HD void word_offsets_s(uint32_t w, uint32_t o[5]) {
  constexpr int32_t k6561 = -6561 * (1 << S);
  constexpr int32_t k81 = -81 * (1 << S);
  constexpr uint32_t kInv81 = S == 2 ? 13256072u : 6628036u;  // ceil(2^(32-S) / 81)
  static_assert(S == 2 || S == 3, "table entries of 4 or 8 bytes");
  const double wd = static_cast<double>(w);
  const uint32_t a = static_cast<uint32_t>(__builtin_fma(wd, 1.0 / 6561.0, 0.5 / 6561.0));
  const uint32_t e = mulhi_u24(a, 654622u);
  const uint32_t bs = mad_i24<kAsm>(a, k6561, w << S);
  const uint32_t ms = mad_i24<kAsm>(e, k6561, a << S);
  const uint32_t b1 = mulhi_u24(bs, kInv81);
  const uint32_t m1 = mulhi_u24(ms, kInv81);
  o[0] = mad_i24<kAsm>(b1, k81, bs);
  o[1] = b1 << S;
  o[2] = mad_i24<kAsm>(m1, k81, ms);
  o[3] = m1 << S;
  o[4] = e << S;
}

// o[j] = 4 * chunk j (digits 4j..4j+3) of the word.
TQ_HD void word_offsets(uint32_t w, uint32_t o[5]) { word_offsets_s<2>(w, o); }

// True when all four bytes of `four` (int8 trits of a chunk, lowest digit in
// the low byte) are -1, 0 or 1: each byte plus 1 without carries between
// bytes must be 0, 1 or 2 (no bit above the low two, and not 3).
TQ_HD bool chunk_trits_valid(uint32_t four) {
  const uint32_t y = ((four & 0x7f7f7f7fu) + 0x01010101u) ^ (four & 0x80808080u);
  return ((y & 0xfcfcfcfcu) | (y & (y >> 1) & 0x01010101u)) == 0u;
}

// Chunk order of the ROW64 layout.  A unit is 160 trits of a row = 8 words
// = 40 chunks of 4 trits; its words hold its own trits only, but chunk j of
// unit word wl (0..7) is unit chunk row64_chunk(wl, j), i.e. unit trits
// 4c .. 4c + 3.  With kb = wl / 2 and q = 5 (wl % 2) + j (0..9):
//   c = 8 (q / 2) + 2 kb + q % 2,
// so the word pair 2kb, 2kb + 1 holds, in digit order, the chunk pairs
// (8s + 2kb, 8s + 2kb + 1) for s = 0..4: a 32-trit step 32s .. 32s + 31 takes
// two consecutive chunks from each of the four pairs and lies in a single
// scale group (128 is a multiple of 32).
constexpr int row64_chunk(int wl, int j) {
  return 8 * ((5 * (wl & 1) + j) >> 1) + 2 * (wl >> 1) + ((5 * (wl & 1) + j) & 1);
}
// Inverse: unit word and chunk-in-word of unit chunk c (0..39).
constexpr int row64_chunk_word(int c) { return 2 * ((c & 7) >> 1) + (2 * (c >> 3) + (c & 1)) / 5; }
constexpr int row64_chunk_index(int c) { return (2 * (c >> 3) + (c & 1)) % 5; }

}  // namespace tq
