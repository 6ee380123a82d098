"""Pins for the KV-cache quantiser oracle (oracle/kv_oracle.py): textbook
values of the Gaussian Lloyd-Max quantiser, its optimality conditions, the
rotation's orthogonality, the 1-bit projection's closed-form expectation,
the score estimator's unbiasedness (Monte Carlo), the pages' compression
figures, and planted mistakes that a pin must catch."""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg

import synth
from oracle import kv_oracle as K

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))

# J. Max, "Quantizing for minimum distortion", IRE Trans. Information Theory,
# 1960, Table I (normal density): output levels and mean-square error.
MAX_1960 = {2: ([0.7980], 0.3634), 4: ([0.4528, 1.5104], 0.1175), 8: ([0.2451, 0.7560, 1.3440, 2.1520], 0.03455),
             16: ([0.1284, 0.3881, 0.6568, 0.9424, 1.2562, 1.6180, 2.0690, 2.7326], 0.009497)}


@pytest.mark.parametrize("levels", [2, 4, 8, 16])
def test_lloyd_max_matches_published_table(levels):
    c, b, mse = K.lloyd_max_gaussian(levels)
    want, want_mse = MAX_1960[levels]
    assert np.allclose(c[levels // 2:], want, atol=2e-4)
    assert np.allclose(c, -c[::-1], atol=1e-12)          # symmetric
    assert mse == pytest.approx(want_mse, rel=2e-3)


@pytest.mark.parametrize("levels", [2, 4, 8, 16, 32, 128, 256])
def test_lloyd_max_optimality_conditions(levels):
    """Each level is the mean of its cell and each boundary the midpoint of
    its two levels (checked by numerical integration, not by the closed
    forms the iteration uses); the distortion matches Monte Carlo."""
    c, b, mse = K.lloyd_max_gaussian(levels)
    assert np.array_equal(c, -c[::-1]) and b[levels // 2 - 1] == 0.0
    assert np.allclose(b, (c[:-1] + c[1:]) / 2, atol=1e-12)
    edges = np.concatenate([[-12.0], b, [12.0]])
    pts = 200001 if levels <= 16 else 20001
    for i in range(levels):
        xs = np.linspace(edges[i], edges[i + 1], pts)
        w = np.exp(-xs ** 2 / 2)
        assert np.trapezoid(xs * w, xs) / np.trapezoid(w, xs) == pytest.approx(c[i], abs=1e-6)
    # the distortion against the integral of (x - c_i)^2 over each cell
    dist = 0.0
    for i in range(levels):
        xs = np.linspace(edges[i], edges[i + 1], pts)
        dist += np.trapezoid((xs - c[i]) ** 2 * np.exp(-xs ** 2 / 2), xs) / math.sqrt(2 * math.pi)
    assert dist == pytest.approx(mse, rel=1e-5)
    if levels <= 16:
        x = np.random.default_rng(levels).standard_normal(2_000_000)
        q = c[K.nearest_level(x, c)]
        assert np.mean((x - q) ** 2) == pytest.approx(mse, rel=0.01)


def test_nearest_level_ties_and_order():
    lv = np.array([-1.0, 0.0, 2.0])
    got = K.nearest_level([-0.5, -0.49, 1.0, 1.01, -9.0, 9.0], lv)
    assert got.tolist() == [0, 1, 1, 2, 0, 2]            # exactly halfway goes to the lower level


def test_rotation_is_orthogonal_and_random_signs_matter():
    s = synth.kv_signs(1, K.D)
    pi = K.rotation(s)
    assert np.allclose(pi @ pi.T, np.eye(K.D), atol=1e-13)
    x = np.random.default_rng(2).normal(size=(5, K.D))
    assert np.allclose(np.linalg.norm(K.rotate(x, s), axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    assert np.allclose(K.unrotate(K.rotate(x, s), s), x, atol=1e-12)
    # with all signs +1 it is the plain Hadamard: e_0 -> the constant vector
    e0 = np.zeros(K.D)
    e0[0] = 1.0
    assert np.allclose(K.rotate(e0, np.ones(K.D))[0], np.full(K.D, 1 / math.sqrt(K.D)))
    # the sign flip acts first: Pi e_i = sigma_i H e_i (column i of the
    # textbook Hadamard, scipy's, times sigma_i)
    h = scipy.linalg.hadamard(K.D) / math.sqrt(K.D)
    for i in (3, 77):
        assert np.allclose(K.rotate(np.eye(K.D)[i], s)[0], s[i] * h[:, i], atol=1e-14)


def test_rotated_coordinates_are_near_gaussian():
    """After the random rotation a unit vector's coordinates have variance
    1/d whatever the input (a spike, a constant, a Gaussian draw)."""
    s = synth.kv_signs(3, K.D)
    for x in (np.eye(K.D)[7], np.ones(K.D), np.random.default_rng(4).normal(size=K.D)):
        u = K.rotate(x / np.linalg.norm(x), s)[0]
        assert np.sum(u ** 2) == pytest.approx(1.0)
    # a spike's rotation spreads it over all coordinates: max |u_i| = 1/sqrt(d)
    u = K.rotate(np.eye(K.D)[7], s)[0]
    assert np.allclose(np.abs(u), 1 / math.sqrt(K.D))


def test_one_bit_projection_closed_form():
    """For s ~ N(0, I): E[sign(<s, e>) <s, y>] = sqrt(2/pi) <y, e> / |e|, the
    identity that makes sqrt(pi/2)/m <S y, sign(S e)> unbiased (Monte Carlo
    over 400,000 rows, 5 sigma)."""
    rng = np.random.default_rng(5)
    e, y = rng.normal(size=16), rng.normal(size=16)
    s = rng.normal(size=(400_000, 16))
    v = np.sign(s @ e) * (s @ y)
    want = math.sqrt(2 / math.pi) * (y @ e) / np.linalg.norm(e)
    assert abs(v.mean() - want) < 5 * v.std() / math.sqrt(len(v))


@pytest.mark.parametrize("along_residual", [False, True])
def test_score_estimator_is_unbiased(along_residual):
    """Over independent JL matrices the key score's mean is the exact <q, k>
    up to the fp16 radius and residual norm (Monte Carlo, 5 sigma).  A query
    along the residual (q = Pi^T e) makes the 1-bit term's spread small
    (about 7 % of it per draw), so its scale is pinned tightly."""
    rng = np.random.default_rng(6)
    s = synth.kv_signs(7, K.D)
    k = rng.normal(size=(1, K.D))
    u = K.rotate(k, s)[0] / np.linalg.norm(k)
    cb = K.codebook(2)
    ut = cb[K.nearest_level(u, cb)]
    e = u - ut
    q = K.unrotate(e, s)[0] * 10.0 if along_residual else rng.normal(size=K.D)
    est = []
    for t in range(300 if along_residual else 600):
        jl = synth.kv_jl(1000 + t, K.D)
        kq = K.kv_quantize(k, s, 3, True, jl)
        est.append(K.kv_scores(q, kq, s, jl)[0])
    est = np.array(est)
    # the exact value with the stored (fp16) r and gamma: r^ (<q', u~> + (gamma^/gamma) <q', e>)
    qr = K.rotate(q, s)[0]
    r_hat = float(np.float16(np.linalg.norm(k)))
    g, g_hat = np.linalg.norm(e), float(np.float16(np.linalg.norm(e)))
    want = r_hat * (qr @ ut + g_hat / g * (qr @ e))
    assert abs(est.mean() - want) < 5 * est.std() / math.sqrt(len(est))
    assert want == pytest.approx(float(q @ k[0]), rel=2e-3)          # fp16 r and gamma only


def test_more_bits_converge_to_exact():
    rng = np.random.default_rng(8)
    s = synth.kv_signs(9, K.D)
    x = rng.normal(size=(20, K.D))
    errs = []
    for b in (2, 3, 4, 6):
        vq = K.kv_quantize(x, s, b, False)
        errs.append(np.linalg.norm(K.kv_dequantize_values(vq, s) - x) / np.linalg.norm(x))
    assert all(e2 < e1 for e1, e2 in zip(errs, errs[1:]))
    # relative error near sqrt of the Lloyd-Max distortion: 3 bits -> sqrt(0.0345)
    assert errs[1] == pytest.approx(math.sqrt(K.lloyd_max_gaussian(8)[2]), rel=0.1)


def test_values_weighted_sum_matches_dequantised():
    rng = np.random.default_rng(10)
    s = synth.kv_signs(11, K.D)
    v = rng.normal(size=(30, K.D))
    p = rng.random(30)
    vq = K.kv_quantize(v, s, 3, False)
    assert np.allclose(K.kv_values(p, vq, s), p @ K.kv_dequantize_values(vq, s), atol=1e-12)


def test_attend_special_cases():
    """Equal scores average the dequantised values; one score far above the
    rest selects its value; the result matches scipy's softmax weights."""
    import scipy.special
    rng = np.random.default_rng(14)
    s = synth.kv_signs(15, K.D)
    v = rng.normal(size=(50, K.D))
    vq = K.kv_quantize(v, s, 3, False)
    vhat = K.kv_dequantize_values(vq, s)
    assert np.allclose(K.kv_attend(np.full(50, 3.7), 0.1, vq, s), vhat.mean(axis=0), atol=1e-12)
    sc = rng.normal(size=50)
    sc[17] = 1e4
    assert np.allclose(K.kv_attend(sc, 1.0, vq, s), vhat[17], atol=1e-12)
    sc = rng.normal(size=50) * 30
    want = scipy.special.softmax(0.25 * sc) @ vhat
    assert np.allclose(K.kv_attend(sc, 0.25, vq, s), want, atol=1e-12)


def test_zero_vector():
    s = synth.kv_signs(12, K.D)
    jl = synth.kv_jl(13, K.D)
    kq = K.kv_quantize(np.zeros((1, K.D)), s, 3, True, jl)
    assert float(kq["r"][0]) == 0.0
    assert K.kv_scores(np.ones(K.D), kq, s, jl)[0] == 0.0


def test_compression_matches_pages():
    """3 bits per coordinate: about 4-5x against fp16 (oMLX/Gemma page,
    'What TurboQuant is...'); no per-block scales, only the per-vector norms."""
    fp16 = 16 * K.D
    lo, hi = GOLD["kv_ratio_3bit"]["value"]
    assert lo <= fp16 / K.stored_bits(3, True) <= hi
    assert lo <= fp16 / K.stored_bits(3, False) <= hi * 1.03
    # 3 bits keep about a fifth: the 128K figure of the same page, 8.14 GB -> 1.70 GB
    kept = GOLD["kv_128k_gb"]["value"]
    assert K.stored_bits(3, True) / fp16 == pytest.approx(kept[1] / kept[0], abs=0.01)
    # the TurboQuant+ range 1/4 .. 1/6 spans 4 bits down to 2.5 bits
    a, b = GOLD["kv_ratio_range_plus"]["value"]
    assert a <= fp16 / K.stored_bits(4, True) * 1.07 and fp16 / K.stored_bits(2, True) >= b


def test_key_record_fields():
    """A key record holds the (bits - 1)-bit codes as packed fields, then z."""
    kq = {"bits": 3, "keys": True, "codes": np.zeros((2, K.D), np.int64), "z": -np.ones((2, K.D), np.int8)}
    kq["codes"][1, 40] = 3                               # bits 80, 81: word 2, bits 16, 17
    kq["codes"][1, 15] = 2                               # bit 31 of word 0
    kq["z"][1, 127] = 1                                  # last bit of the record
    rec = K.kv_records(kq)
    assert rec.shape == (2, 12) and rec.dtype == np.uint32
    assert rec[0].sum() == 0
    assert rec[1, 2] == 3 << 16 and rec[1, 0] == 1 << 31 and rec[1, 11] == 1 << 31
    assert rec[1].astype(np.int64).sum() == (3 << 16) + 2 * (1 << 31)
    vq = {"bits": 2, "keys": False, "codes": np.full((1, K.D), 2, np.int64)}
    assert K.kv_records(vq)[0].tolist() == [0xAAAAAAAA] * 8


def test_fields_straddle_words():
    """3-bit fields cross word boundaries (code 10 spans bits 30..32)."""
    codes = np.zeros((1, K.D), np.int64)
    codes[0, 10] = 0b111
    f = K.pack_fields(codes, 3)
    assert f.shape == (1, 12)
    assert f[0, 0] == 0b11 << 30 and f[0, 1] == 1 and f[0].astype(np.int64).sum() == (0b11 << 30) + 1
    # every code recovered by reading its bits back
    rng = np.random.default_rng(3)
    for nb in (1, 2, 3, 5, 7, 8):
        c = rng.integers(0, 2 ** nb, size=(4, K.D))
        f = K.pack_fields(c, nb).astype(np.uint64)
        bits = ((f[:, :, None] >> np.arange(32, dtype=np.uint64)) & np.uint64(1)).reshape(4, -1)
        back = sum(bits[:, t::nb].astype(np.int64) << t for t in range(nb))
        assert np.array_equal(back, c)


# --------------------------------------------- planted-mistake checks ---
def _expect_pin_failure(monkeypatch, attr, bad, pins):
    monkeypatch.setattr(K, attr, bad)
    failed = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, f"no pin caught the planted mistake in {attr}"


def test_pins_catch_missing_sqrt_pi_over_2(monkeypatch):
    good = K.kv_scores

    def bad(q, kq, signs, jl):
        kq2 = dict(kq)
        kq2["gamma"] = (kq["gamma"].astype(np.float64) / math.sqrt(math.pi / 2)).astype(np.float16)
        return good(q, kq2, signs, jl)
    _expect_pin_failure(monkeypatch, "kv_scores", bad, [lambda: test_score_estimator_is_unbiased(True)])


def test_pins_catch_unscaled_codebook(monkeypatch):
    good = K.codebook
    _expect_pin_failure(monkeypatch, "codebook", lambda bits, d=K.D: good(bits, d) * math.sqrt(d),
                        [test_more_bits_converge_to_exact])


def test_pins_catch_newton_sign_error(monkeypatch):
    """A wrong-sign Newton step leaves a point that is not the fixed point
    (or diverges); the optimality pin at 32 levels catches it."""
    good_solve = np.linalg.solve
    monkeypatch.setattr(K, "_LM_CACHE", {})
    monkeypatch.setattr(K.np.linalg, "solve", lambda a, b: -good_solve(a, b))
    failed = 0
    try:
        test_lloyd_max_optimality_conditions(32)
    except (AssertionError, ValueError, FloatingPointError, ZeroDivisionError):
        failed = 1
    assert failed, "no pin caught the wrong-sign Newton step"


def test_pins_catch_transposed_rotation(monkeypatch):
    """Pi^T in place of Pi (the sign flip after the transform, not before)."""
    def bad(x, s):
        return (np.atleast_2d(np.asarray(x, np.float64)) @ K._hadamard_pm1(len(s))) / np.sqrt(len(s)) * s
    _expect_pin_failure(monkeypatch, "rotate", bad, [test_rotation_is_orthogonal_and_random_signs_matter])
