"""Pins for the oracle's format variants: scale groups of 64 (the model id
"-g64" on the TurboQuant-MLX page) and the binary {-c, +c} ablation (pure
1-bit experts, the same page's point 3).  As for the main format: closed
forms, page constants, special values, exhaustive round trips, invariants
and planted mistakes, never a re-typed formula."""
import json
import math
import os

import numpy as np
import pytest

from oracle import tq_oracle as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))
G64 = GOLD["group_size_variant"]["value"]


# ------------------------------------------------------------ group 64 ---
def test_group64_bits_per_weight_closed_form():
    rng = np.random.default_rng(1)
    for n, k in [(3, 5120), (2, 17408), (4, 2048), (5, 512), (2, 128)]:
        t, s, _ = O.ternarize(rng.normal(size=(n, k)), G64)
        assert s.shape == (n, k // 64)
        assert O.pack(t).nbytes + s.nbytes == O.packed_bytes(n, k, G64)
    # 32/20 bits on the words plus 16/64 on the scales
    assert 8.0 * O.packed_bytes(1, 5120, G64) / 5120 == pytest.approx(1.6 + 0.25, abs=1e-12)
    assert O.packed_bytes(1, 5120, G64) - O.packed_bytes(1, 5120) == 2 * 5120 // 128


def test_group64_scale_invariance_per_group():
    """Multiplying one 64-wide group by a power of two scales only its own
    scale (exactly) and leaves every trit unchanged: the groups are 64
    weights wide, not 128."""
    rng = np.random.default_rng(2)
    w = rng.normal(size=(6, 1024))
    t0, s0, _ = O.ternarize(w, G64)
    for g in (0, 1, 7, 15):
        w2 = w.copy()
        w2[:, 64 * g:64 * (g + 1)] *= 1024.0
        t1, s1, _ = O.ternarize(w2, G64)
        assert np.array_equal(t1, t0)
        others = [c for c in range(16) if c != g]
        assert np.array_equal(s1[:, others], s0[:, others])
        assert np.allclose(s1[:, g].astype(np.float64), 1024.0 * s0[:, g].astype(np.float64), rtol=1e-3)
    # at group 128 the same scaling moves the threshold of the neighbouring half
    t128, _, _ = O.ternarize(w, 128)
    w3 = w.copy()
    w3[:, :64] *= 1024.0
    assert not np.array_equal(O.ternarize(w3, 128)[0][:, 64:128], t128[:, 64:128])


def test_group64_zero_fraction_gaussian():
    # the absmean threshold's zero fraction on Gaussian data,
    # erf(sqrt(2/pi) / (2 sqrt 2)), up to the finite-group effect at 64
    w = np.random.default_rng(3).normal(size=(400, 4096))
    t, _, _ = O.ternarize(w, G64)
    want = math.erf(math.sqrt(2 / math.pi) / (2 * math.sqrt(2)))
    assert abs(np.mean(t == 0) - want) < 0.01


def test_group64_matvec_one_hot_and_group_ones_exact():
    rng = np.random.default_rng(4)
    n, k = 9, 640
    t = rng.integers(-1, 2, size=(n, k)).astype(np.int8)
    s = rng.uniform(0.01, 0.03, size=(n, k // 64)).astype(np.float16)
    words = O.pack(t)
    for c in (0, 63, 64, 127, 128, 191, 639):
        x = np.zeros(k)
        x[c] = 1.0
        y = O.gemv(words, s, k, x, False, G64)[0]
        assert np.array_equal(y, s[:, c // 64].astype(np.float64) * t[:, c])
    for g in (0, 1, 9):
        x = np.zeros(k)
        x[64 * g:64 * (g + 1)] = 1.0
        y = O.gemv(words, s, k, x, False, G64)[0]
        assert np.array_equal(y, s[:, g].astype(np.float64) * t[:, 64 * g:64 * (g + 1)].sum(axis=1))


def test_group64_quantize_rotation_identity():
    """quantize at group 64 rotates with the same block-128 Hadamard: with
    no quantisation error (weights already ternary times a group-constant
    scale after rotation) the matvec on the rotated activation reproduces W x."""
    rng = np.random.default_rng(5)
    n, k = 4, 256
    t = rng.choice(np.array([-1, 1], np.int8), size=(n, k))
    c = np.repeat(rng.choice([0.5, 1.0, 2.0], size=(n, k // 64)), 64, axis=1)
    w_rot = t * c                                  # exactly representable: gamma = c, all |w'| > gamma/2
    w = O.block_transform(w_rot)                   # H is its own inverse
    tq, s, gamma = O.quantize(w, G64)
    assert np.array_equal(tq, t)
    assert np.allclose(gamma, c[:, ::64])
    x = rng.normal(size=(2, k))
    assert np.allclose(O.gemv(O.pack(tq), s, k, x, True, G64), x @ w.T, rtol=1e-12, atol=1e-12)


# -------------------------------------------------------------- binary ---
def test_binary_bits_per_weight_closed_form():
    assert GOLD["binary_bits_per_weight"]["value"] == 32 // O.BITS_PER_WORD
    rng = np.random.default_rng(6)
    for n, k in [(3, 5120), (2, 17408), (1, 100)]:
        t = rng.choice(np.array([-1, 1], np.int8), size=(n, k))
        assert O.pack_binary(t).shape == (n, -(-k // 32))
    assert 8.0 * O.packed_bytes_binary(1, 5120) / 5120 == pytest.approx(1.0 + 16 / 128, abs=1e-12)
    assert 8.0 * O.packed_bytes_binary(1, 5120, G64) / 5120 == pytest.approx(1.0 + 16 / 64, abs=1e-12)
    # ternary at 20 per word costs 0.6 bit per weight more on the words
    assert 8.0 * (O.packed_bytes(1, 5120) - O.packed_bytes_binary(1, 5120)) / 5120 == pytest.approx(0.6)


def test_binary_special_words():
    ones = np.ones((1, 32), np.int8)
    assert int(O.pack_binary(ones)[0, 0]) == 0xFFFFFFFF
    assert int(O.pack_binary(-ones)[0, 0]) == 0
    for i in range(32):
        t = -ones.copy()
        t[0, i] = 1
        assert int(O.pack_binary(t)[0, 0]) == 1 << i
    t = -np.ones((1, 64), np.int8)
    t[0, 37] = 1                                   # word 1, bit 5
    w = O.pack_binary(t)
    assert int(w[0, 0]) == 0 and int(w[0, 1]) == 32
    # a ragged row: bits past K are 0 and read back as nothing
    t = np.ones((1, 40), np.int8)
    w = O.pack_binary(t)
    assert int(w[0, 1]) == 0xFF
    assert O.unpack_binary(w, 40).tolist() == t.tolist()


def test_binary_round_trip_exhaustive_halves():
    rng = np.random.default_rng(7)
    lo = np.arange(1 << 16, dtype=np.int64)
    t_lo = (2 * ((lo[:, None] >> np.arange(16)) & 1) - 1).astype(np.int8)
    t_hi = rng.choice(np.array([-1, 1], np.int8), size=(1 << 16, 16))
    t = np.concatenate([t_lo, t_hi], axis=1)
    w = O.pack_binary(t)
    assert np.array_equal(w[:, 0] & 0xFFFF, lo.astype(np.uint32))
    assert np.array_equal(O.unpack_binary(w, 32), t)


def test_binarize_values_ties_and_least_squares_scale():
    rng = np.random.default_rng(8)
    w = rng.normal(size=(5, 512))
    w[0, 3] = 0.0
    t, s, gamma = O.binarize(w)
    assert set(np.unique(t)) <= {-1, 1}
    assert t[0, 3] == 1                              # an exact zero goes to +1
    assert np.array_equal(O.binarize(-w)[0][w != 0], -t[w != 0])
    # gamma = mean |w| minimises sum (w - c sign w)^2 over c (closed form of
    # the 1-bit least-squares scale): any other c does worse
    g = w.reshape(5, 4, 128)
    sg = np.where(g >= 0, 1.0, -1.0)
    for c_scale in (0.98, 0.999, 1.001, 1.02):
        e_best = ((g - gamma[:, :, None] * sg) ** 2).sum(axis=2)
        e_other = ((g - c_scale * gamma[:, :, None] * sg) ** 2).sum(axis=2)
        assert np.all(e_other > e_best)
    assert np.array_equal(s, gamma.astype(np.float16))


def test_binary_matvec_one_hot_exact():
    rng = np.random.default_rng(9)
    n, k = 7, 384
    t = rng.choice(np.array([-1, 1], np.int8), size=(n, k))
    s = rng.uniform(0.01, 0.03, size=(n, k // 128)).astype(np.float16)
    words = O.pack_binary(t)
    for c in (0, 31, 32, 127, 128, 383):
        x = np.zeros(k)
        x[c] = 1.0
        y = O.gemv(words, s, k, x, False, 128, 2)[0]
        assert np.array_equal(y, s[:, c // 128].astype(np.float64) * t[:, c])
    # every weight is +-s: a row of ones sums the signs times the scales exactly
    y = O.gemv(words, s, k, np.ones(k), False, 128, 2)[0]
    want = (t.reshape(n, 3, 128).sum(axis=2) * s.astype(np.float64)).sum(axis=1)
    assert np.array_equal(y, want)


def test_binary_reconstruction_worse_than_ternary_on_gaussian():
    """The page's point 3 compares the two value sets; on Gaussian weights
    the ternary reconstruction error (absmean, zero level) is below the
    binary one (the quality claims themselves need trained models)."""
    w = np.random.default_rng(10).normal(size=(64, 1024))
    tt, st, _ = O.ternarize(w)
    tb, sb, _ = O.binarize(w)
    e_t = np.linalg.norm(w - tt * np.repeat(st.astype(np.float64), 128, axis=1))
    e_b = np.linalg.norm(w - tb * np.repeat(sb.astype(np.float64), 128, axis=1))
    assert e_t < e_b


# --------------------------------------------- planted-mistake checks ---
def _expect_pin_failure(monkeypatch, attr, bad, pins):
    monkeypatch.setattr(O, attr, bad)
    failed = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, f"no pin caught the planted mistake in {attr}"


def test_pins_catch_big_endian_bits(monkeypatch):
    good = O.pack_binary

    def bad(t):
        t = np.asarray(t)
        n, k = t.shape
        nw = -(-k // 32)
        tt = -np.ones((n, nw * 32), np.int8)
        tt[:, :k] = t
        return good(tt.reshape(n, nw, 32)[:, :, ::-1].reshape(n, nw * 32))
    _expect_pin_failure(monkeypatch, "pack_binary", bad, [test_binary_special_words])


def test_pins_catch_binary_zero_level(monkeypatch):
    good = O.binarize

    def bad(w_rot, group=128):
        t, s, g = good(w_rot, group)
        t = t.copy()
        t[np.asarray(w_rot) == 0] = 0                  # a zero level sneaking back in
        return t, s, g
    _expect_pin_failure(monkeypatch, "binarize", bad, [test_binarize_values_ties_and_least_squares_scale])


def test_pins_catch_group64_read_as_128(monkeypatch):
    good = O.dequantize

    def bad(words, scales, k, group=128, levels=3):
        # one scale per 128 weights: every other 64-group scale, used twice
        return good(words, np.repeat(np.asarray(scales)[:, ::2], 2, axis=1), k, group, levels)
    _expect_pin_failure(monkeypatch, "dequantize", bad, [test_group64_matvec_one_hot_and_group_ones_exact])
