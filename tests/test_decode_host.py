"""Host build of the kernels' word decoder (the same header, with each GPU
instruction emulated bit-exactly) checked against plain division: every
step over its full input range, the word boundaries of both FP64 divisions,
and a large random sample of words."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "ternary_weight_quantized_tq_amd", "csrc")

PROG = r'''
#include <stdio.h>
#include <stdint.h>
#include "tq_decode.h"
using namespace tq;
static int check(uint32_t w) {
  uint32_t o[5], o8[5];
  word_offsets(w, o);
  word_offsets_s<3>(w, o8);
  uint32_t v = w;
  for (int j = 0; j < 5; ++j) {
    if (o[j] != 4u * (v % 81u) || o8[j] != 8u * (v % 81u)) return 1;
    v /= 81u;
  }
  return 0;
}
int main() {
  const uint32_t N = 3486784401u;  /* 3^20 */
  long bad = 0;
  /* 24-bit steps over their whole ranges */
  for (uint32_t a = 0; a < 531441u; ++a) bad += mulhi_u24(a, 654622u) != a / 6561u;
  for (uint32_t b = 0; b < 6561u; ++b) bad += mulhi_u24(4u * b, 13256072u) != b / 81u;
  for (uint32_t b = 0; b < 6561u; ++b) bad += mulhi_u24(8u * b, 6628036u) != b / 81u;
  /* both FP64 divisions at every multiple boundary */
  for (uint32_t q = 0; q < 531441u; ++q) {
    uint32_t lo = q * 6561u;
    bad += check(lo) + check(lo + 6560u);
    if (q) bad += check(lo - 1u);
  }
  for (uint32_t q = 0; q < 81u; ++q) bad += check(q * 43046721u) + check(q * 43046721u + 43046720u);
  bad += check(0) + check(N - 1u) + check(1743392200u);
  /* a dense sweep of words */
  for (uint64_t w = 0; w < N; w += 1009u) bad += check((uint32_t)w);
  printf("%ld\n", bad);
  return bad != 0;
}
'''


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_word_decoder_exhaustive():
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "t.cpp")
        exe = os.path.join(d, "t")
        open(src, "w").write(PROG)
        subprocess.run(["g++", "-O2", "-std=c++17", f"-I{CSRC}", src, "-o", exe], check=True)
        p = subprocess.run([exe], capture_output=True, text=True, timeout=600)
        assert p.returncode == 0 and p.stdout.strip() == "0", p.stdout + p.stderr


CHUNK_PROG = r'''
#include <stdio.h>
#include "tq_decode.h"
using namespace tq;
int main() {
  for (int wl = 0; wl < 8; ++wl)
    for (int j = 0; j < 5; ++j) {
      const int c = row64_chunk(wl, j);
      printf("%d %d %d %d\n", c, row64_chunk_word(c), row64_chunk_index(c), wl * 5 + j);
    }
  return 0;
}
'''


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_row64_chunk_order():
    """The kernels' ROW64 chunk order is a permutation of a unit's 40 chunks,
    its inverse is exact, it equals the test-side definition, and every
    32-trit step 32s .. 32s + 31 is made of chunk pairs (8s + 2kb, +1) that
    sit in digit order in words 2kb, 2kb + 1 (one scale group per step)."""
    import sys
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from tqgpu import row64_chunk
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "c.cpp")
        exe = os.path.join(d, "c")
        open(src, "w").write(CHUNK_PROG)
        subprocess.run(["g++", "-O2", "-std=c++17", f"-I{CSRC}", src, "-o", exe], check=True)
        rows = [list(map(int, l.split())) for l in subprocess.run([exe], capture_output=True, text=True,
                                                                    check=True).stdout.split("\n") if l]
    assert sorted(r[0] for r in rows) == list(range(40))
    for c, wl, j, idx in rows:
        assert (wl, j) == divmod(idx, 5)
        assert c == row64_chunk(wl, j)
    for kb in range(4):
        digits = [row64_chunk(2 * kb + h, j) for h in range(2) for j in range(5)]
        assert digits == [8 * s + 2 * kb + e for s in range(5) for e in range(2)]


VALID_PROG = r'''
#include <stdio.h>
#include <stdint.h>
#include "tq_decode.h"
using namespace tq;
int main() {
  long bad = 0;
  /* every byte value at every position, the other bytes each of -1, 0, 1 */
  const uint32_t ok3[3] = {0xffu, 0x00u, 0x01u};
  for (int pos = 0; pos < 4; ++pos)
    for (uint32_t b = 0; b < 256u; ++b)
      for (int f = 0; f < 81; ++f) {
        uint32_t four = 0;
        int g = f;
        for (int i = 0; i < 4; ++i) {
          uint32_t byte = ok3[g % 3];
          g /= 3;
          if (i == pos) byte = b;
          four |= byte << (8 * i);
        }
        const int8_t sb = (int8_t)b;
        const bool want = sb >= -1 && sb <= 1;
        bad += chunk_trits_valid(four) != want;
      }
  /* two invalid bytes at once */
  for (uint32_t a = 0; a < 256u; ++a)
    for (uint32_t b = 0; b < 256u; ++b) {
      const uint32_t four = a | (b << 16);
      const bool want = ((int8_t)a >= -1 && (int8_t)a <= 1) && ((int8_t)b >= -1 && (int8_t)b <= 1);
      bad += chunk_trits_valid(four) != want;
    }
  printf("%ld\n", bad);
  return bad != 0;
}
'''


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_chunk_trits_valid_exhaustive():
    """The pack kernel's test that a chunk's four int8 values are trits (its
    fast path then takes one int8 dot product): every byte value at every
    position beside every valid combination of the others, and every pair of
    bytes at two positions, against the plain range test."""
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "v.cpp")
        exe = os.path.join(d, "v")
        open(src, "w").write(VALID_PROG)
        subprocess.run(["g++", "-O2", "-std=c++17", f"-I{CSRC}", src, "-o", exe], check=True)
        p = subprocess.run([exe], capture_output=True, text=True, timeout=60)
        assert p.returncode == 0 and p.stdout.strip() == "0", p.stdout + p.stderr
