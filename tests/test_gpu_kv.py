"""GPU parity of the KV-cache quantiser (TurboQuant KV page) through the C
ABI against the FP64 oracle (oracle/kv_oracle.py).

* Quantisation runs in FP64 on both sides, so records, radii and residual
  norms are compared bit for bit.
* Scores and value sums are FP32 table sums on the GPU.  Bounds: a score is
  r times a sum of 48 (3-bit keys) to 144 table entries, each a short FP32
  sum of terms no larger than |q| in total, so its rounding error is below
  about 50 * 2^-24 * r |q| * (a few); each score is held to 2e-5 r |q|
  (a score itself can be far smaller than r |q| when its terms cancel, so
  a relative bound per score would not hold), and every (head, query) row
  to rel-L2 2e-5 and its largest error to 1e-4 of its largest score.  A
  value sum adds n FP32 products per coordinate (chunked, then the chunks
  in order): rel-L2 1e-5.
* The fused attend (softmax of scale * scores, then the value sum) takes
  scale * s and its exponential in FP32: each weight is off by a relative
  few times 2^-24 |scale s|, under 1e-6 for the logits used here, and the
  normalising sum of the same weights cancels most of it: rel-L2 2e-5.
"""
import numpy as np
import pytest

import synth
import ternary_weight_quantized_tq_amd as tq
from oracle import kv_oracle as K
from tests.parity import assert_parity
from tests.tqgpu import act_tensor, dev, torch

pytestmark = pytest.mark.gpu

SCORE_REL_L2, SCORE_ROW_MAX, SCORE_ABS = 2e-5, 1e-4, 2e-5
VALUE_REL_L2, VALUE_ROW_MAX = 1e-5, 1e-4
ATTEND_REL_L2, ATTEND_ROW_MAX = 2e-5, 1e-4
SCALE = 1.0 / np.sqrt(128.0)


def _setup(sign_seed=21, jl_seed=22):
    signs = synth.kv_signs(sign_seed, K.D)
    jl = synth.kv_jl(jl_seed, K.D)
    return signs, jl, dev(signs), dev(jl)


def _levels(bits, keys):
    return dev(tq.tq_kv_codebook(bits - 1 if keys else bits))


def _gpu_quantize(x, n, bits, keys, signs_d, jl_d, stride=1):
    t = torch()
    rec = t.zeros((n * stride, 4 * bits), dtype=t.int32, device="cuda")
    r = t.zeros(n * stride, dtype=t.int16, device="cuda")
    g = t.zeros(n * stride, dtype=t.int16, device="cuda") if keys else None
    tq.tq_kv_quantize(x, n, signs_d, jl_d if keys else None, _levels(bits, keys), bits, keys, rec, r, g, stride)
    t.cuda.synchronize()
    return rec, r, g


def _oracle_store(kq):
    out = {"rec": K.kv_records(kq), "r": kq["r"].view(np.uint16)}
    if kq["keys"]:
        out["g"] = kq["gamma"].view(np.uint16)
    return out


@pytest.mark.parametrize("keys,bits", [(True, b) for b in range(2, 9)] + [(False, b) for b in range(1, 9)])
def test_quantize_bit_exact(keys, bits):
    """1001 vectors (a ragged last workgroup), three of them zero."""
    signs, jl, sd, jd = _setup()
    act = synth.kv_vectors(31 + bits, 1001, K.D, "bf16")
    ref = act.values.copy()
    raw = act.raw.copy()
    for i in (0, 500, 1000):
        ref[i] = 0.0
        raw[i] = 0
    act = synth.Activations(ref, raw, "bf16")
    rec, r, g = _gpu_quantize(act_tensor(act), 1001, bits, keys, sd, jd)
    want = _oracle_store(K.kv_quantize(act.values, signs, bits, keys, jl))
    got_rec = rec.cpu().numpy().view(np.uint32)
    bad = np.argwhere(got_rec != want["rec"])
    assert bad.size == 0, f"{len(bad)} record words differ, first at {bad[:3].tolist()}"
    assert np.array_equal(r.cpu().numpy().view(np.uint16), want["r"])
    if keys:
        assert np.array_equal(g.cpu().numpy().view(np.uint16), want["g"])


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_quantize_input_dtypes(dtype):
    signs, jl, sd, jd = _setup()
    act = synth.kv_vectors(41, 300, K.D, "f32")
    if dtype == "f16":
        x16 = act.raw.astype(np.float16)
        act = synth.Activations(x16.astype(np.float64), x16.view(np.uint16), "f16")
    for keys in (True, False):
        rec, r, g = _gpu_quantize(act_tensor(act), 300, 3, keys, sd, jd)
        want = _oracle_store(K.kv_quantize(act.values, signs, 3, keys, jl))
        assert np.array_equal(rec.cpu().numpy().view(np.uint32), want["rec"])
        assert np.array_equal(r.cpu().numpy().view(np.uint16), want["r"])


def test_quantize_strided_into_head_major_cache():
    """One token of 5 heads written at position 7 of a 20-token cache."""
    t = torch()
    signs, jl, sd, jd = _setup()
    act = synth.kv_vectors(43, 5, K.D, "bf16")
    cap, pos, bits = 20, 7, 4
    rec = t.zeros((5 * cap, 4 * bits), dtype=t.int32, device="cuda")
    r = t.zeros(5 * cap, dtype=t.int16, device="cuda")
    g = t.zeros(5 * cap, dtype=t.int16, device="cuda")
    tq.tq_kv_quantize(act_tensor(act), 5, sd, jd, _levels(bits, True), bits, True, rec[pos:], r[pos:], g[pos:], cap)
    t.cuda.synchronize()
    want = _oracle_store(K.kv_quantize(act.values, signs, bits, True, jl))
    got = rec.cpu().numpy().view(np.uint32)
    rows = [h * cap + pos for h in range(5)]
    assert np.array_equal(got[rows], want["rec"])
    assert np.array_equal(r.cpu().numpy().view(np.uint16)[rows], want["r"])
    assert np.array_equal(g.cpu().numpy().view(np.uint16)[rows], want["g"])
    others = np.setdiff1d(np.arange(5 * cap), rows)
    assert not got[others].any()


def _assert_scores(got, want, r16, q, what=""):
    """Each score within SCORE_ABS * r * |q|; rows of many scores also by
    rel-L2 and per-row maximum."""
    bound = SCORE_ABS * r16.astype(np.float64) * np.linalg.norm(q)
    err = np.abs(np.asarray(got, np.float64) - want)
    assert np.all(err <= bound + 1e-30), f"{what}: worst {np.max(err / (bound + 1e-30)):.2f} of the bound"
    if len(want) >= 100:
        assert_parity(np.asarray(got)[None], want[None], SCORE_REL_L2, SCORE_ROW_MAX, what)


def _upload_store(stores):
    """Per-head oracle stores -> device records [heads][n][4 bits], radius and gamma [heads][n]."""
    rec = dev(np.ascontiguousarray(np.stack([s["rec"] for s in stores])))
    r = dev(np.ascontiguousarray(np.stack([s["r"] for s in stores])))
    g = dev(np.ascontiguousarray(np.stack([s["g"] for s in stores]))) if "g" in stores[0] else None
    return rec, r, g


def _run_scores(q, heads, nq, rec, r, g, n, bits, sd, jd, lv):
    t = torch()
    out = t.empty((heads, nq, n), dtype=t.float32, device="cuda")
    ws, nb = tq.kv_workspace(tq.TQ_KV_OP_SCORES, n, heads, nq)
    tq.tq_kv_scores(q, heads, nq, rec, r, g, n, bits, sd, jd, lv, out, ws, nb)
    t.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _run_values(p, heads, nq, rec, r, n, bits, sd, lv):
    t = torch()
    out = t.empty((heads, nq, K.D), dtype=t.float32, device="cuda")
    ws, nb = tq.kv_workspace(tq.TQ_KV_OP_VALUES, n, heads, nq)
    tq.tq_kv_values(p, heads, nq, rec, r, n, bits, sd, lv, out, ws, nb)
    t.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _run_attend(s, scale, heads, nq, rec, r, n, bits, sd, lv):
    t = torch()
    out = t.full((heads, nq, K.D), 7.0, dtype=t.float32, device="cuda")
    ws, nb = tq.kv_workspace(tq.TQ_KV_OP_ATTEND, n, heads, nq)
    tq.tq_kv_attend(s, scale, heads, nq, rec, r, n, bits, sd, lv, out, ws, nb)
    t.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _value_store(heads, n, bits, signs, seed=70):
    stores, vqs = [], []
    for h in range(heads):
        vq = K.kv_quantize(synth.kv_vectors(seed + h, n, K.D, "bf16").values, signs, bits, False)
        vqs.append(vq)
        stores.append(_oracle_store(vq))
    rec, r, _ = _upload_store(stores)
    return rec, r, vqs


@pytest.mark.parametrize("bits", range(2, 9))
@pytest.mark.parametrize("heads,nq,n", [(2, 3, 1), (2, 3, 700), (2, 4, 700), (1, 2, 700), (3, 8, 1500), (1, 4, 3)])
def test_scores_parity(bits, heads, nq, n):
    """Keys quantised by the oracle; scores of `heads` KV heads x `nq`
    queries each (query groups of 1, 2 and 4 per workgroup)."""
    signs, jl, sd, jd = _setup()
    stores, kqs = [], []
    for h in range(heads):
        kq = K.kv_quantize(synth.kv_vectors(50 + h, n, K.D, "bf16").values, signs, bits, True, jl)
        kqs.append(kq)
        stores.append(_oracle_store(kq))
    rec, r, g = _upload_store(stores)
    q = synth.kv_vectors(60, heads * nq, K.D, "f32")
    got = _run_scores(dev(q.raw.astype(np.float32)), heads, nq, rec, r, g, n, bits, sd, jd, _levels(bits, True))
    for h in range(heads):
        for j in range(nq):
            want = K.kv_scores(q.values[h * nq + j], kqs[h], signs, jl)
            _assert_scores(got[h, j], want, kqs[h]["r"], q.values[h * nq + j], f"h{h} q{j}")


@pytest.mark.parametrize("bits", range(1, 9))
@pytest.mark.parametrize("heads,nq,n", [(2, 3, 1), (2, 3, 3000), (2, 4, 3000), (1, 2, 3000), (3, 8, 5000), (1, 4, 3)])
def test_values_parity(bits, heads, nq, n):
    """Values quantised by the oracle; softmax-like weights, `heads` KV heads
    x `nq` queries each (query groups of 1, 2 and 4 per workgroup)."""
    signs, jl, sd, jd = _setup()
    stores, vqs = [], []
    for h in range(heads):
        vq = K.kv_quantize(synth.kv_vectors(70 + h, n, K.D, "bf16").values, signs, bits, False)
        vqs.append(vq)
        stores.append(_oracle_store(vq))
    rec, r, _ = _upload_store(stores)
    rng = np.random.default_rng(80 + bits)
    logits = rng.normal(size=(heads, nq, n)) * 2.0
    p = np.exp(logits - logits.max(axis=-1, keepdims=True))
    p = (p / p.sum(axis=-1, keepdims=True)).astype(np.float32)
    got = _run_values(dev(p), heads, nq, rec, r, n, bits, sd, _levels(bits, False))
    want = np.stack([np.stack([K.kv_values(p[h, j].astype(np.float64), vqs[h], signs) for j in range(nq)])
                     for h in range(heads)])
    assert_parity(got.reshape(heads * nq, K.D), want.reshape(heads * nq, K.D), VALUE_REL_L2, VALUE_ROW_MAX)


@pytest.mark.parametrize("nq", [3, 4])
def test_values_of_no_tokens_are_zero(nq):
    t = torch()
    signs, jl, sd, jd = _setup()
    out = t.full((2, nq, K.D), 7.0, dtype=t.float32, device="cuda")
    ws, nb = tq.kv_workspace(tq.TQ_KV_OP_VALUES, 0, 2, nq)
    rec = t.zeros((1, 12), dtype=t.int32, device="cuda")
    r = t.zeros(1, dtype=t.int16, device="cuda")
    p = t.zeros(1, dtype=t.float32, device="cuda")
    tq.tq_kv_values(p, 2, nq, rec, r, 0, 3, sd, _levels(3, False), out, ws, nb)
    t.cuda.synchronize()
    assert not out.cpu().numpy().any()


@pytest.mark.parametrize("bits", range(1, 9))
@pytest.mark.parametrize("heads,nq,n", [(2, 3, 1), (2, 3, 3000), (2, 4, 3000), (1, 2, 3000), (3, 8, 5000), (1, 4, 3)])
def test_attend_parity(bits, heads, nq, n):
    """Fused softmax + value sum against the oracle's softmax of scale *
    scores and value sum; scores of attention size (|scale s| up to ~12)."""
    signs, _, sd, _ = _setup()
    rec, r, vqs = _value_store(heads, n, bits, signs)
    rng = np.random.default_rng(90 + bits)
    s = (rng.normal(size=(heads, nq, n)) * 30.0).astype(np.float32)
    got = _run_attend(dev(s), SCALE, heads, nq, rec, r, n, bits, sd, _levels(bits, False))
    want = np.stack([np.stack([K.kv_attend(s[h, j], SCALE, vqs[h], signs) for j in range(nq)])
                     for h in range(heads)])
    assert_parity(got.reshape(heads * nq, K.D), want.reshape(heads * nq, K.D), ATTEND_REL_L2, ATTEND_ROW_MAX)


@pytest.mark.parametrize("nq", [1, 2, 4])
def test_attend_rescales_chunks(nq):
    """The key chunks' maxima differ by far more than FP32's exponent range
    once exponentiated: a ramp of scores (rising or falling) with one narrow
    peak in the middle, or a sawtooth whose teeth rise steeply enough that
    the running offset inside a chunk moves every few keys; masked (-inf)
    tokens including whole chunks.  The merge must rescale each chunk to the
    common maximum.  A query whose scores are all -inf gives zeros."""
    signs, _, sd, _ = _setup()
    heads, n, bits = 2, 40000, 3
    rec, r, vqs = _value_store(heads, n, bits, signs, seed=75)
    s = np.empty((heads, nq, n), np.float32)
    ramps = [np.linspace(-4000.0, 400.0, n, dtype=np.float32), np.linspace(400.0, -4000.0, n, dtype=np.float32),
             (450.0 / 256.0 * (np.arange(n) % 256)).astype(np.float32)]
    for h in range(heads):
        for j in range(nq):
            row = ramps[(h + j) % 3].copy()
            if (h + j) % 3 != 2:
                row[n // 2 - 3:n // 2 + 3] = 600.0 + np.arange(6, dtype=np.float32)
            row[1000:9000] = -np.inf
            row[::7] = -np.inf
            s[h, j] = row
    s[1, nq - 1] = -np.inf
    got = _run_attend(dev(s), SCALE, heads, nq, rec, r, n, bits, sd, _levels(bits, False))
    for h in range(heads):
        for j in range(nq):
            if h == 1 and j == nq - 1:
                assert not got[h, j].any()
                continue
            want = K.kv_attend(s[h, j], SCALE, vqs[h], signs)
            assert_parity(got[h, j][None], want[None], ATTEND_REL_L2, ATTEND_ROW_MAX, f"h{h} q{j}")


@pytest.mark.parametrize("nq", [3, 4])
def test_attend_of_no_tokens_is_zero(nq):
    t = torch()
    signs, jl, sd, jd = _setup()
    rec = t.zeros((1, 12), dtype=t.int32, device="cuda")
    r = t.zeros(1, dtype=t.int16, device="cuda")
    s = t.zeros(1, dtype=t.float32, device="cuda")
    got = _run_attend(s, SCALE, 2, nq, rec, r, 0, 3, sd, _levels(3, False))
    assert not got.any()


def test_attend_matches_values_of_softmax():
    """tq_kv_attend against tq_kv_values fed torch's FP32 softmax of the same
    scores: the two GPU paths agree to FP32 rounding."""
    t = torch()
    signs, _, sd, _ = _setup()
    heads, nq, n, bits = 2, 4, 20000, 3
    rec, r, _ = _value_store(heads, n, bits, signs)
    rng = np.random.default_rng(95)
    s = dev((rng.normal(size=(heads, nq, n)) * 30.0).astype(np.float32))
    lv = _levels(bits, False)
    p = t.softmax(s * SCALE, dim=-1).contiguous()
    a = _run_attend(s, SCALE, heads, nq, rec, r, n, bits, sd, lv)
    b = _run_values(p, heads, nq, rec, r, n, bits, sd, lv)
    assert_parity(a.reshape(-1, K.D), b.reshape(-1, K.D), ATTEND_REL_L2, ATTEND_ROW_MAX)


def test_attention_pipeline_small():
    """Quantise keys and values on the GPU, score, softmax (torch, FP32),
    weighted value sum; against the oracle doing the same from x."""
    t = torch()
    wl = synth.KV_SMALL
    signs, jl, sd, jd = synth.kv_signs(wl.sign_seed), synth.kv_jl(wl.jl_seed), None, None
    sd, jd = dev(signs), dev(jl)
    n, heads, nq, bits = wl.tokens, wl.heads, wl.queries, wl.bits
    kx = synth.kv_vectors(wl.key_seed, heads * n, K.D, "bf16")
    vx = synth.kv_vectors(wl.value_seed, heads * n, K.D, "bf16")
    q = synth.kv_vectors(wl.query_seed, heads * nq, K.D, "f32")
    krec, kr, kg = _gpu_quantize(act_tensor(kx), heads * n, bits, True, sd, jd)
    vrec, vr, _ = _gpu_quantize(act_tensor(vx), heads * n, bits, False, sd, jd)
    s = _run_scores(dev(q.raw.astype(np.float32)), heads, nq, krec, kr, kg, n, bits, sd, jd, _levels(bits, True))
    sdev = t.from_numpy(s).float().cuda()
    p = t.softmax(sdev / np.sqrt(K.D), dim=-1).contiguous()
    got = _run_values(p, heads, nq, vrec, vr, n, bits, sd, _levels(bits, False))
    fused = _run_attend(sdev, SCALE, heads, nq, vrec, vr, n, bits, sd, _levels(bits, False))
    for h in range(heads):
        kq = K.kv_quantize(kx.values[h * n:(h + 1) * n], signs, bits, True, jl)
        vq = K.kv_quantize(vx.values[h * n:(h + 1) * n], signs, bits, False)
        assert np.array_equal(krec.cpu().numpy().view(np.uint32)[h * n:(h + 1) * n], K.kv_records(kq))
        for j in range(nq):
            sc = K.kv_scores(q.values[h * nq + j], kq, signs, jl)
            _assert_scores(s[h, j], sc, kq["r"], q.values[h * nq + j], f"scores h{h} q{j}")
            pr = np.exp(sc / np.sqrt(K.D) - (sc / np.sqrt(K.D)).max())
            pr /= pr.sum()
            want = K.kv_values(pr, vq, signs)
            assert_parity(got[h, j][None], want[None], 1e-4, 1e-4, f"out h{h} q{j}")
            assert_parity(fused[h, j][None], want[None], 1e-4, 1e-4, f"fused h{h} q{j}")


@pytest.mark.slow
def test_full_size_sampled():
    """The 128K-token, 8-head, 4-query, 3-bit decode workload in the launch
    configuration the benchmark times: sampled records bit-exact, sampled
    scores, and value sums whose weights are nonzero only on a sample (the
    GPU still reads every record)."""
    t = torch()
    wl = synth.KV_DECODE_128K
    n, heads, nq, bits = wl.tokens, wl.heads, wl.queries, wl.bits
    signs, jl = synth.kv_signs(wl.sign_seed), synth.kv_jl(wl.jl_seed)
    sd, jd = dev(signs), dev(jl)
    kx = synth.kv_vectors(wl.key_seed, heads * n, K.D, "bf16")
    krec, kr, kg = _gpu_quantize(act_tensor(kx), heads * n, bits, True, sd, jd)
    vx = synth.kv_vectors(wl.value_seed, heads * n, K.D, "bf16")
    vrec, vr, _ = _gpu_quantize(act_tensor(vx), heads * n, bits, False, sd, jd)
    q = synth.kv_vectors(wl.query_seed, heads * nq, K.D, "f32")
    s = _run_scores(dev(q.raw.astype(np.float32)), heads, nq, krec, kr, kg, n, bits, sd, jd, _levels(bits, True))
    rng = np.random.default_rng(7)
    kh = krec.cpu().numpy().view(np.uint32)
    vh = vrec.cpu().numpy().view(np.uint32)
    p = np.zeros((heads, nq, n), np.float32)
    for h in range(heads):
        idx = np.sort(rng.choice(n, 64, replace=False))
        rows = h * n + idx
        kq = K.kv_quantize(kx.values[rows], signs, bits, True, jl)
        vq = K.kv_quantize(vx.values[rows], signs, bits, False)
        assert np.array_equal(kh[rows], K.kv_records(kq))
        assert np.array_equal(vh[rows], K.kv_records(vq))
        assert np.array_equal(kr.cpu().numpy().view(np.uint16)[rows], kq["r"].view(np.uint16))
        for j in range(nq):
            want = K.kv_scores(q.values[h * nq + j], kq, signs, jl)
            _assert_scores(s[h, j, idx], want, kq["r"], q.values[h * nq + j], f"h{h} q{j}")
            p[h, j, idx] = rng.random(64).astype(np.float32)
    got = _run_values(dev(p), heads, nq, vrec, vr, n, bits, sd, _levels(bits, False))
    # Fused attend on the same sample: every other score masked to -inf.
    sm = np.where(p > 0, s.astype(np.float32), -np.inf).astype(np.float32)
    fused = _run_attend(dev(sm), SCALE, heads, nq, vrec, vr, n, bits, sd, _levels(bits, False))
    for h in range(heads):
        nz = np.nonzero(p[h, 0])[0]
        vq = K.kv_quantize(vx.values[h * n + nz], signs, bits, False)
        for j in range(nq):
            want = K.kv_values(p[h, j, nz].astype(np.float64), vq, signs)
            assert_parity(got[h, j][None], want[None], VALUE_REL_L2, VALUE_ROW_MAX, f"values h{h} q{j}")
            want = K.kv_attend(sm[h, j, nz], SCALE, vq, signs)
            assert_parity(fused[h, j][None], want[None], ATTEND_REL_L2, ATTEND_ROW_MAX, f"attend h{h} q{j}")
