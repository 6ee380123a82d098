"""Pins for the CPU oracle: page constants, closed forms, invariants, library
routines and brute force on tiny inputs.  None of these re-types the
oracle's own formula; each is chosen so that a plausible mistake (a dropped
term, a wrong sign, digit order or index, a transposed operand, a missing
normalisation, a double rounding) fails at least one of them.  The
``test_pins_catch_*`` tests plant such mistakes in the oracle (on the CPU)
and check that a pin fails.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg

import synth
from oracle import tq_oracle as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))
ALL_ZERO_WORD = (3 ** 20 - 1) // 2      # every digit 1 (t = 0)


# ---------------------------------------------------------------- format ---
def test_word_capacity_closed_form():
    n = GOLD["trits_per_word"]["value"]
    bits = GOLD["word_bits"]["value"]
    assert 3 ** n < 2 ** bits            # 20 trits fit a 32-bit word ...
    assert 3 ** (n + 1) > 2 ** bits      # ... and 21 would not
    assert abs(bits / n - GOLD["approx_bits_per_weight_words"]["value"]) < 1e-12
    assert abs(math.log2(3) - GOLD["info_bits_per_trit"]["value"]) < GOLD["info_bits_per_trit"]["tol"]


def test_bits_per_weight_matches_pages():
    # words + fp16 scales per 128 -> 32/20 + 16/128 = 1.725 bpw when 20 | K
    rng = np.random.default_rng(0)
    for n, k in [(4, 5120), (3, 17408), (2, 2048), (5, 1024), (2, 512), (1, 128)]:
        t = rng.integers(-1, 2, size=(n, k)).astype(np.int8)
        words = O.pack(t)
        _, s, _ = O.ternarize(rng.normal(size=(n, k)))
        assert words.dtype == np.uint32 and s.dtype == np.float16
        assert words.nbytes + s.nbytes == O.packed_bytes(n, k)
        bpw = 8.0 * O.packed_bytes(n, k) / (n * k)
        exact = (GOLD["word_bits"]["value"] * math.ceil(k / 20) / k
                 + GOLD["scale_bits"]["value"] / GOLD["group_size"]["value"])
        assert abs(bpw - exact) < 1e-12
    assert O.packed_bytes(1, 5120) * 8 / 5120 == pytest.approx(1.725, abs=1e-12)
    # 27B params at 1.725 bpw lands at the page's "5.9 GB level"
    gb = GOLD["params_billion"]["value"] * 1e9 * 1.725 / 8 / 1e9
    assert abs(gb - GOLD["approx_ternary_gb"]["value"]) / GOLD["approx_ternary_gb"]["value"] < 0.02 + 1e-9
    # the page's 1.76 is a file-level average: 5.93 GB over 27B weights
    file_bpw = GOLD["total_file_gb"]["value"] * 8 / GOLD["params_billion"]["value"]
    assert abs(file_bpw - GOLD["avg_bits_per_weight_file"]["value"]) < GOLD["avg_bits_per_weight_file"]["tol"]
    # 53.8 GB at 2 bytes per weight is the same ~27B parameters
    assert abs(GOLD["fp16_weights_gb"]["value"] / 2 - GOLD["params_billion"]["value"]) < 0.2


def test_special_words():
    z = np.zeros((1, 20), np.int8)
    assert int(O.pack(z - 1)[0, 0]) == 0
    assert int(O.pack(z)[0, 0]) == ALL_ZERO_WORD == 1743392200
    assert int(O.pack(z + 1)[0, 0]) == 3 ** 20 - 1 == 3486784400
    for i in range(20):
        t = z.copy()
        t[0, i] = 1
        assert int(O.pack(t)[0, 0]) == ALL_ZERO_WORD + 3 ** i
        t[0, i] = -1
        assert int(O.pack(t)[0, 0]) == ALL_ZERO_WORD - 3 ** i
    # second word of a row holds trits 20..39
    t = np.zeros((1, 40), np.int8)
    t[0, 23] = 1
    w = O.pack(t)
    assert int(w[0, 0]) == ALL_ZERO_WORD and int(w[0, 1]) == ALL_ZERO_WORD + 27


def test_unpack_special_words():
    for i in range(20):
        t = O.unpack(np.array([[ALL_ZERO_WORD + 3 ** i]], np.uint32), 20)[0]
        want = np.zeros(20, np.int8)
        want[i] = 1
        assert np.array_equal(t, want)
    assert np.array_equal(O.unpack(np.array([[0]], np.uint32), 20)[0], -np.ones(20, np.int8))


def test_round_trip_exhaustive_halves():
    rng = np.random.default_rng(1)
    lo = np.arange(3 ** 10, dtype=np.int64)
    digits_lo = np.stack([(lo // 3 ** i) % 3 for i in range(10)], axis=1)
    digits_hi = rng.integers(0, 3, size=(lo.size, 10))
    for d in (np.concatenate([digits_lo, digits_hi], 1), np.concatenate([digits_hi, digits_lo], 1)):
        t = (d - 1).astype(np.int8)
        # 59049 rows of one word each
        words = O.pack(t)
        assert np.array_equal(O.unpack(words, 20), t)


def test_pack_is_bijection_onto_range():
    rng = np.random.default_rng(2)
    w = rng.integers(0, 3 ** 20, size=(200, 7), dtype=np.int64).astype(np.uint32)
    w[0, :3] = [0, 3 ** 20 - 1, ALL_ZERO_WORD]
    t = O.unpack(w, 140)
    assert set(np.unique(t)) <= {-1, 0, 1}
    assert np.array_equal(O.pack(t), w)


def test_row_tail_padding():
    rng = np.random.default_rng(3)
    for k in (1, 19, 20, 21, 27, 127, 128, 129, 1000):
        t = rng.integers(-1, 2, size=(3, k)).astype(np.int8)
        w = O.pack(t)
        assert w.shape == (3, -(-k // 20))
        full = O.unpack(w, w.shape[1] * 20)
        assert np.array_equal(full[:, :k], t)
        assert np.all(full[:, k:] == 0)


def test_pack_rejects_non_ternary():
    with pytest.raises(ValueError):
        O.pack(np.array([[2]], np.int8))


# ------------------------------------------------------------- Hadamard ---
def test_hadamard_textbook_and_library():
    assert np.allclose(O.hadamard(2), np.array([[1, 1], [1, -1]]) / math.sqrt(2), atol=0, rtol=0)
    for n in (2, 4, 16, 128):
        assert np.array_equal(O.hadamard(n) * math.sqrt(n), scipy.linalg.hadamard(n).astype(float))


def test_hadamard_orthonormal_symmetric():
    h = O.hadamard(128)
    assert np.abs(h @ h - np.eye(128)).max() < 1e-14
    assert np.array_equal(h, h.T)
    ones = np.ones(128)
    e0 = np.zeros(128)
    e0[0] = math.sqrt(128)
    assert np.abs(h @ ones - e0).max() < 1e-12


def _butterfly(x):
    """Textbook in-place fast Walsh-Hadamard transform, O(n log n)."""
    x = np.array(x, dtype=np.float64)
    n = x.shape[-1]
    hlen = 1
    while hlen < n:
        for i in range(0, n, 2 * hlen):
            a = x[..., i:i + hlen].copy()
            b = x[..., i + hlen:i + 2 * hlen].copy()
            x[..., i:i + hlen] = a + b
            x[..., i + hlen:i + 2 * hlen] = a - b
        hlen *= 2
    return x / math.sqrt(n)


def test_fwht_equals_butterfly_and_preserves_norm():
    rng = np.random.default_rng(4)
    x = rng.normal(size=(3, 640))
    xr = O.fwht(x)
    bf = np.concatenate([_butterfly(x[:, b * 128:(b + 1) * 128]) for b in range(5)], axis=1)
    assert np.abs(xr - bf).max() < 1e-13
    for b in range(5):
        blk = slice(b * 128, (b + 1) * 128)
        assert np.allclose(np.linalg.norm(xr[:, blk], axis=1), np.linalg.norm(x[:, blk], axis=1), rtol=1e-14)
    assert np.abs(O.fwht(xr) - x).max() < 1e-13          # involution: H H = I
    e = np.zeros((1, 256))
    e[0, 130] = 1.0                                       # column 2 of block 1
    col = O.fwht(e)[0]
    assert np.all(col[:128] == 0)
    assert np.allclose(col[128:], scipy.linalg.hadamard(128)[2] / math.sqrt(128), rtol=0, atol=1e-16)


def test_rotation_identity_brute_force():
    """W.x == (W.H)(H.x): the rotation is a lossless change of basis."""
    rng = np.random.default_rng(5)
    for n, k in [(3, 128), (5, 256), (64, 1024)]:
        w = rng.normal(size=(n, k))
        x = rng.normal(size=(2, k))
        lhs = x @ w.T
        rhs = O.fwht(x) @ O.rotate_weights(w).T
        assert np.abs(lhs - rhs).max() / np.abs(lhs).max() < 1e-13


# ------------------------------------------------------------ quantizer ---
def test_quantizer_zero_fraction_gaussian():
    """Pure Gaussian: P(|z| <= E|z|/2) = erf(sqrt(2/pi)/(2 sqrt 2)) = 0.3101."""
    rng = np.random.default_rng(6)
    w = rng.normal(0, 0.02, size=(2048, 1024))
    t, s, gamma = O.ternarize(w)
    assert set(np.unique(t)) <= {-1, 0, 1}
    frac0 = float(np.mean(t == 0))
    expect = math.erf(math.sqrt(2 / math.pi) / (2 * math.sqrt(2)))
    assert abs(expect - 0.3101) < 1e-4
    assert abs(frac0 - expect) < 0.004
    # symmetric: +1 and -1 equally likely
    assert abs(float(np.mean(t == 1)) - float(np.mean(t == -1))) < 0.003
    # mean |w| of N(0, s^2) is s sqrt(2/pi)
    assert abs(float(gamma.mean()) - 0.02 * math.sqrt(2 / math.pi)) < 2e-5


def test_quantizer_threshold_tie_and_zero_group():
    g = np.concatenate([np.full(64, 3.0), np.full(64, 1.0)])     # gamma = 2, gamma/2 = 1
    w = np.stack([g, -g, np.zeros(128)])
    t, s, gamma = O.ternarize(w)
    assert np.all(t[0, :64] == 1) and np.all(t[0, 64:] == 0)    # exact tie -> 0
    assert np.all(t[1, :64] == -1) and np.all(t[1, 64:] == 0)
    assert np.all(t[2] == 0) and float(s[2, 0]) == 0.0
    assert float(s[0, 0]) == 2.0 and float(s[1, 0]) == 2.0


def test_scale_single_rounding_from_fp64():
    """A double rounding (fp64 -> fp32 -> fp16) would land on the tie and round
    to even (1.0); one rounding from fp64 must give 1 + 2^-10."""
    v = 1.0 + 2.0 ** -11 + 2.0 ** -40
    _, s, _ = O.ternarize(np.full((1, 128), v))
    assert float(s[0, 0]) == 1.0 + 2.0 ** -10
    _, s, _ = O.ternarize(np.full((1, 128), 1.0 + 2.0 ** -11))   # exact tie -> even
    assert float(s[0, 0]) == 1.0


def test_quantizer_symmetries():
    rng = np.random.default_rng(7)
    w = synth.weights(9, 16, 512)
    t, s, _ = O.quantize(w)
    t2, s2, _ = O.quantize(-w)
    assert np.array_equal(t2, -t) and np.array_equal(s2, s)
    t4, s4, _ = O.quantize(4.0 * w)
    assert np.array_equal(t4, t) and np.array_equal(s4.astype(np.float64), 4.0 * s.astype(np.float64))
    perm = rng.permutation(16)
    t5, s5, _ = O.quantize(w[perm])
    assert np.array_equal(t5, t[perm]) and np.array_equal(s5, s[perm])


def test_rotation_reduces_quantization_error_with_outliers():
    """Rotating before ternarising spreads the x20 outliers (the pages' reason
    for the rotation): the quantised product is closer to W.x than without it."""
    w = synth.weights(1001, 512, 1024)
    x = synth.activations(1002, 1, 1024, "f32").values
    y_fp = O.unquantized(w, x)
    t, s, _ = O.quantize(w)
    y_rot = O.gemv(O.pack(t), s, 1024, x, True)
    tu, su, _ = O.ternarize(w)                       # no rotation
    y_plain = O.gemv(O.pack(tu), su, 1024, x, False)
    e_rot, e_plain = O.rel_l2(y_rot, y_fp), O.rel_l2(y_plain, y_fp)
    assert e_rot < 0.6 and e_rot < 0.8 * e_plain


# --------------------------------------------------------------- matvec ---
def _small_packed(seed, n, k):
    t = synth.trits(seed, n, k)
    s = synth.scales(seed + 1, n, k // 128)
    return t, s, O.pack(t)


def test_matvec_one_hot_exact():
    n, k = 7, 384
    t, s, w = _small_packed(11, n, k)
    for kk in (0, 19, 20, 127, 128, 255, 383):
        x = np.zeros((1, k))
        x[0, kk] = 1.0
        y = O.gemv(w, s, k, x, fused_fwht=False)[0]
        want = s[:, kk // 128].astype(np.float64) * t[:, kk]
        assert np.array_equal(y, want)


def test_matvec_group_ones_exact():
    n, k = 5, 512
    t, s, w = _small_packed(12, n, k)
    for g in range(4):
        x = np.zeros((1, k))
        x[0, g * 128:(g + 1) * 128] = 1.0
        y = O.gemv(w, s, k, x, fused_fwht=False)[0]
        want = s[:, g].astype(np.float64) * t[:, g * 128:(g + 1) * 128].sum(axis=1)
        assert np.array_equal(y, want)


def test_matvec_brute_force_tiny():
    """Pure-Python loops straight from the definition on a tiny case."""
    n, k = 3, 256
    t, s, w = _small_packed(13, n, k)
    rng = np.random.default_rng(14)
    x = rng.normal(size=k)
    xr = [0.0] * k
    for b in range(k // 128):
        for j in range(128):
            acc = 0.0
            for i in range(128):
                sign = -1.0 if bin(i & j).count("1") % 2 else 1.0
                acc += x[128 * b + i] * sign
            xr[128 * b + j] = acc / math.sqrt(128)
    want = []
    for r in range(n):
        acc = 0.0
        for kk in range(k):
            word = int(w[r, kk // 20])
            d = (word // 3 ** (kk % 20)) % 3
            acc += float(s[r, kk // 128]) * (d - 1) * xr[kk]
        want.append(acc)
    y = O.gemv(w, s, k, x[None, :], True)[0]
    assert np.abs(y - np.array(want)).max() < 1e-12


def test_matvec_linear_and_batched():
    n, k = 33, 640
    t, s, w = _small_packed(15, n, k)
    rng = np.random.default_rng(16)
    x = rng.normal(size=(8, k))
    y8 = O.gemv(w, s, k, x, True)
    for m in range(8):
        assert np.allclose(O.gemv(w, s, k, x[m:m + 1], True)[0], y8[m], rtol=1e-13, atol=1e-13)
    y_sum = O.gemv(w, s, k, x[0:1] + 2.0 * x[1:2], True)[0]
    assert np.allclose(y_sum, y8[0] + 2.0 * y8[1], rtol=1e-12, atol=1e-12)
    assert np.array_equal(O.gemm_rows(w, s, k, x, [5, 2]), O.gemv(w, s, k, x[[5, 2]], True))


# ------------------------------------------------------------------ MoE ---
def test_silu_textbook():
    assert O.silu(0.0) == 0.0
    assert abs(float(O.silu(1.0)) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert abs(float(O.silu(40.0)) - 40.0) < 1e-12 and abs(float(O.silu(-40.0))) < 1e-15


def test_route_properties():
    lg = synth.logits(4903, 64, 256)
    ids, w = O.route(lg, 8)
    assert ids.shape == (64, 8) and np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    for t in range(64):
        order = np.argsort(-lg[t].astype(np.float64), kind="stable")[:8]   # softmax is monotone
        assert np.array_equal(ids[t], order)
        p = np.exp(lg[t].astype(np.float64))
        assert np.allclose(w[t], p[ids[t]] / p[ids[t]].sum(), rtol=1e-14)
        assert np.all(np.diff(w[t]) <= 0)
    tie = np.zeros((1, 256), np.float32)
    tie[0, [200, 7, 100]] = 5.0
    ids, w = O.route(tie, 2)
    assert list(ids[0]) == [7, 100] and np.allclose(w[0], [0.5, 0.5])


def _tiny_moe(seed, e_count=6, hidden=256, inter=128):
    gu_w, gu_s, dn_w, dn_s = [], [], [], []
    for e in range(e_count):
        t, s, w = _small_packed(seed + 10 * e, 2 * inter, hidden)
        gu_w.append(w), gu_s.append(s)
        t, s, w = _small_packed(seed + 10 * e + 5, hidden, inter)
        dn_w.append(w), dn_s.append(s)
    return gu_w, gu_s, dn_w, dn_s


def test_moe_top1_reduces_to_dense_and_is_linear():
    hidden, inter = 256, 128
    gu_w, gu_s, dn_w, dn_s = _tiny_moe(100)
    rng = np.random.default_rng(17)
    x = rng.normal(size=(3, hidden))
    ids = np.array([[2], [0], [5]], np.int32)
    w1 = np.ones((3, 1))
    y = O.moe(x, ids, w1, gu_w, gu_s, dn_w, dn_s, hidden, inter)
    for t in range(3):
        e = ids[t, 0]
        gu = O.gemv(gu_w[e], gu_s[e], hidden, x[t:t + 1], True)[0]
        h = O.silu(gu[:inter]) * gu[inter:]
        o = O.gemv(dn_w[e], dn_s[e], inter, h[None, :], True)[0]
        assert np.allclose(y[t], o, rtol=1e-13, atol=1e-13)
    # combine is linear in the routing weights; tokens are independent
    ids2 = np.array([[2, 4], [0, 1], [5, 3]], np.int32)
    wa = rng.random((3, 2))
    ya = O.moe(x, ids2, wa, gu_w, gu_s, dn_w, dn_s, hidden, inter)
    yb = O.moe(x, ids2, 3.0 * wa, gu_w, gu_s, dn_w, dn_s, hidden, inter)
    assert np.allclose(yb, 3.0 * ya, rtol=1e-13, atol=1e-13)
    y_t1 = O.moe(x[1:2], ids2[1:2], wa[1:2], gu_w, gu_s, dn_w, dn_s, hidden, inter)
    assert np.allclose(y_t1[0], ya[1], rtol=1e-13, atol=1e-13)
    sep = sum(O.moe(x, ids2[:, j:j + 1], wa[:, j:j + 1], gu_w, gu_s, dn_w, dn_s, hidden, inter) for j in range(2))
    assert np.allclose(sep, ya, rtol=1e-12, atol=1e-12)


# ---------------------------------------------- planted-mistake checks ---
def _expect_pin_failure(monkeypatch, attr, bad, pins):
    monkeypatch.setattr(O, attr, bad)
    failed = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, f"no pin caught the planted mistake in {attr}"


def test_pins_catch_big_endian_digits(monkeypatch):
    good = O.pack

    def bad(t):
        t = np.asarray(t)
        n, k = t.shape
        nw = -(-k // 20)
        tt = np.zeros((n, nw * 20), np.int8)
        tt[:, :k] = t
        return good(tt.reshape(n, nw, 20)[:, :, ::-1].reshape(n, nw * 20))
    _expect_pin_failure(monkeypatch, "pack", bad, [test_special_words])


def test_pins_catch_wrong_threshold(monkeypatch):
    good = O.ternarize

    def bad(w_rot, group=128):
        t, s, g = good(w_rot, group)
        w = np.asarray(w_rot).reshape(t.shape[0], -1, group)
        thr = g[:, :, None]                             # threshold at gamma, not gamma/2
        tb = np.where(w > thr, 1, np.where(w < -thr, -1, 0)).astype(np.int8)
        return tb.reshape(t.shape), s, g
    _expect_pin_failure(monkeypatch, "ternarize", bad, [test_quantizer_zero_fraction_gaussian])


def test_pins_catch_unnormalised_hadamard(monkeypatch):
    monkeypatch.setattr(O, "_H_CACHE", {})
    good = O.hadamard
    _expect_pin_failure(monkeypatch, "hadamard", lambda n=128: good(n) * math.sqrt(n),
                        [test_hadamard_orthonormal_symmetric, test_fwht_equals_butterfly_and_preserves_norm])


def test_pins_catch_wrong_group_index(monkeypatch):
    good = O.dequantize

    def bad(words, scales, k, *rest):
        s = np.asarray(scales)
        return good(words, np.roll(s, 1, axis=1), k, *rest)    # off-by-one group
    _expect_pin_failure(monkeypatch, "dequantize", bad,
                        [test_matvec_one_hot_exact, test_matvec_group_ones_exact])


def test_pins_catch_double_rounded_scale(monkeypatch):
    good = O.ternarize

    def bad(w_rot, group=128):
        t, s, g = good(w_rot, group)
        return t, g.astype(np.float32).astype(np.float16), g
    _expect_pin_failure(monkeypatch, "ternarize", bad, [test_scale_single_rounding_from_fp64])


# ------------------------------------------------------- parity metrics ---
def test_rel_l2_hand_values():
    # reference (3, 4) has norm 5; the difference (0.6, 0.8) has norm 1
    assert O.rel_l2([3.6, 4.8], [3.0, 4.0]) == pytest.approx(0.2, abs=1e-15)
    # the reference is the denominator: swapping the arguments gives 1/6
    assert O.rel_l2([3.0, 4.0], [3.6, 4.8]) == pytest.approx(1.0 / 6.0, abs=1e-15)
    # a sign flip doubles every element's error: 2, whatever the vector
    assert O.rel_l2([-1.0, 2.0, -2.0], [1.0, -2.0, 2.0]) == pytest.approx(2.0, abs=1e-15)
    # a whole-tensor norm, not a per-row mean: rows (1, 0), (0, 1) against
    # (1, 0), (0, 0) -> sqrt(1) / sqrt(2)
    assert O.rel_l2([[1.0, 0.0], [0.0, 0.0]], [[1.0, 0.0], [0.0, 1.0]]) == pytest.approx(
        1.0 / math.sqrt(2.0), abs=1e-15)
    # exact equality, and invariance under a common scale
    assert O.rel_l2([5.0, -7.0], [5.0, -7.0]) == 0.0
    a, b = np.array([1.5, -2.0, 0.25]), np.array([1.0, -2.5, 0.5])
    assert O.rel_l2(1e-30 * a, 1e-30 * b) == pytest.approx(O.rel_l2(a, b), rel=1e-12)
    # a zero reference reports the plain norm of y
    assert O.rel_l2([3.0, 4.0], [0.0, 0.0]) == pytest.approx(5.0, abs=1e-15)


def test_rel_l2_small_errors_are_not_squared():
    # a relative error of 1e-4 must read 1e-4 (a squared ratio reads 1e-8,
    # which would loosen every 1e-5 gate to ~3e-3)
    ref = np.ones(10000)
    assert O.rel_l2(ref * (1 + 1e-4), ref) == pytest.approx(1e-4, rel=1e-9)


def test_row_max_rel_hand_values():
    y_ref = np.array([[1.0, -4.0, 2.0], [0.5, 0.25, -0.125]])
    y = y_ref.copy()
    y[0, 2] += 0.02        # row 0: 0.02 / 4
    y[1, 0] -= 0.01        # row 1: 0.01 / 0.5 = 0.02, the worst row
    assert O.row_max_rel(y, y_ref) == pytest.approx(0.02, abs=1e-15)
    # the whole-tensor rel-L2 of the same pair is far smaller: a local error
    # that the norm dilutes
    assert O.rel_l2(y, y_ref) < 0.006
    # one row, and the reference in the denominator
    assert O.row_max_rel([2.0, 0.0], [1.0, 0.0]) == pytest.approx(1.0, abs=1e-15)
    assert O.row_max_rel([1.0, 0.0], [2.0, 0.0]) == pytest.approx(0.5, abs=1e-15)
    assert O.row_max_rel(y_ref, y_ref) == 0.0


def test_pins_catch_squared_rel_l2(monkeypatch):
    good = O.rel_l2
    _expect_pin_failure(monkeypatch, "rel_l2", lambda y, r: good(y, r) ** 2,
                        [test_rel_l2_hand_values, test_rel_l2_small_errors_are_not_squared])


def test_pins_catch_rel_l2_wrong_denominator(monkeypatch):
    def bad(y, y_ref):
        y = np.asarray(y, dtype=np.float64)
        y_ref = np.asarray(y_ref, dtype=np.float64)
        return float(np.linalg.norm((y - y_ref).ravel()) / np.linalg.norm(y.ravel()))
    _expect_pin_failure(monkeypatch, "rel_l2", bad, [test_rel_l2_hand_values])


def test_pins_catch_rel_l2_per_row_mean(monkeypatch):
    def bad(y, y_ref):
        y = np.atleast_2d(np.asarray(y, dtype=np.float64))
        y_ref = np.atleast_2d(np.asarray(y_ref, dtype=np.float64))
        num = np.linalg.norm(y - y_ref, axis=1)
        den = np.linalg.norm(y_ref, axis=1)
        return float(np.mean(np.where(den > 0, num / np.where(den > 0, den, 1), num)))
    _expect_pin_failure(monkeypatch, "rel_l2", bad, [test_rel_l2_hand_values])
