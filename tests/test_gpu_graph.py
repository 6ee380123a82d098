"""The entry points inside HIP graphs, as bench.py times them: each call is
captured once, the graph replayed several times with eager work and
synchronisations between the replays, and every replay compared with the
eager result (bit-exact for the deterministic paths)."""
import numpy as np
import pytest

import synth
import ternary_weight_quantized_tq_amd as tq

from tqgpu import act_tensor, dev, gpu_pack, gpu_pack_expert, torch

pytestmark = pytest.mark.gpu


def _replays_match(call, out, exact=True, replays=3):
    """call() writes out; eager result first, then replays of its graph."""
    th = torch()
    out.fill_(float("nan"))
    call()
    th.cuda.synchronize()
    ref = out.clone()
    g = th.cuda.CUDAGraph()
    with th.cuda.graph(g):
        call()
    for r in range(replays):
        out.fill_(float("nan"))
        busy = th.randn(1 << 16, device="cuda")  # unrelated eager work between replays
        busy.mul_(2.0)
        th.cuda.synchronize()
        g.replay()
        th.cuda.synchronize()
        if exact:
            assert th.equal(out, ref), f"replay {r}"
        else:
            assert th.allclose(out, ref, rtol=1e-6, atol=1e-6), f"replay {r}"


def _weights(seed, n, k):
    t = synth.trits(seed, n, k)
    s = synth.scales(seed + 1, n, k // 128)
    return gpu_pack(t, s)


@pytest.mark.parametrize("m", [1, 8])
def test_gemv_in_graph(m):
    th = torch()
    w = _weights(5, 2176, 5120)
    x = act_tensor(synth.activations(6, m, 5120, "bf16"))
    y = th.empty((m, w.n), dtype=th.float32, device="cuda")
    ws, nb = tq.workspace(tq.TQ_OP_GEMV, w, m)
    _replays_match(lambda: tq.tq_gemv(w, x, m, y, tq.TQ_FWHT_FUSED, ws, nb), y)


def test_gemv_accumulate_in_graph():
    """The bench step: a fill kernel, then TQ_ACCUMULATE (atomics, so the
    order of the slice additions may differ between replays)."""
    th = torch()
    w = _weights(7, 2176, 5120)
    x = act_tensor(synth.activations(8, 1, 5120, "bf16"))
    y = th.empty((1, w.n), dtype=th.float32, device="cuda")

    def step():
        y.zero_()
        tq.tq_gemv(w, x, 1, y, tq.TQ_FWHT_FUSED | tq.TQ_ACCUMULATE)
    _replays_match(step, y, exact=False)


@pytest.mark.parametrize("T", [1, 5, 40])
def test_moe_in_graph(T):
    """Per-pair (T = 1), per-token (T = 5) and bucketed (T = 40) paths; the
    per-pair path's arrival counters are cleared inside the graph."""
    th = torch()
    E, hidden, inter, topk = 12, 640, 256, 2
    w_gu = tq.empty_weights(2 * inter, hidden, num_experts=E)
    w_dn = tq.empty_weights(hidden, inter, num_experts=E)
    for e in range(E):
        gpu_pack_expert(w_gu, e, trits=synth.trits(50 + e, 2 * inter, hidden),
                        scales=synth.scales(70 + e, 2 * inter, hidden // 128))
        gpu_pack_expert(w_dn, e, trits=synth.trits(90 + e, hidden, inter),
                        scales=synth.scales(110 + e, hidden, inter // 128))
    rng = np.random.default_rng(T)
    ids = dev(np.stack([rng.choice(E, topk, replace=False) for _ in range(T)]).astype(np.int32))
    rw = dev(rng.random((T, topk)).astype(np.float32))
    x = act_tensor(synth.activations(9, T, hidden, "bf16"))
    y = th.empty((T, hidden), dtype=th.float32, device="cuda")
    ws, nb = tq.workspace(tq.TQ_OP_MOE, w_gu, T, topk)
    _replays_match(lambda: tq.tq_moe_gemv(w_gu, w_dn, x, T, topk, ids, rw, y, tq.TQ_FWHT_FUSED, ws, nb), y)


def test_gemm_in_graph():
    th = torch()
    w = _weights(11, 640, 1280)
    m = 96
    x = act_tensor(synth.activations(12, m, 1280, "bf16"))
    y = th.empty((m, w.n), dtype=th.float32, device="cuda")
    ws, nb = tq.workspace(tq.TQ_OP_GEMM, w, m)
    _replays_match(lambda: tq.tq_gemm(w, x, m, y, tq.TQ_FWHT_FUSED, ws, nb), y)


@pytest.mark.parametrize("nq", [3, 4])
def test_kv_cache_in_graph(nq):
    """KV quantise, scores, value sums and attend (query groups of 1 and 4
    per workgroup), each captured and replayed; all deterministic."""
    th = torch()
    heads, n, bits = 2, 3000, 3
    sd, jd = dev(synth.kv_signs(91)), dev(synth.kv_jl(92))
    lk, lv = dev(tq.tq_kv_codebook(bits - 1)), dev(tq.tq_kv_codebook(bits))
    x = act_tensor(synth.kv_vectors(93, heads * n, 128, "bf16"))
    rec = th.zeros((heads * n, 4 * bits), dtype=th.int32, device="cuda")
    r = th.zeros(heads * n, dtype=th.int16, device="cuda")
    g = th.zeros(heads * n, dtype=th.int16, device="cuda")
    quant = lambda: tq.tq_kv_quantize(x, heads * n, sd, jd, lk, bits, True, rec, r, g)
    quant()
    th.cuda.synchronize()
    ref = (rec.clone(), r.clone(), g.clone())
    gq = th.cuda.CUDAGraph()
    with th.cuda.graph(gq):
        quant()
    for rep in range(3):
        for t_ in (rec, r, g):
            t_.fill_(-1)
        th.cuda.synchronize()
        gq.replay()
        th.cuda.synchronize()
        assert all(th.equal(a, b) for a, b in zip((rec, r, g), ref)), f"quantise replay {rep}"
    q = dev(synth.kv_vectors(94, heads * nq, 128, "f32").raw.astype(np.float32))
    scores = th.empty((heads, nq, n), dtype=th.float32, device="cuda")
    ws, nb = tq.kv_workspace(tq.TQ_KV_OP_SCORES, n, heads, nq)
    _replays_match(lambda: tq.tq_kv_scores(q, heads, nq, rec, r, g, n, bits, sd, jd, lk, scores, ws, nb), scores)
    p = th.softmax(scores, dim=-1).contiguous()
    out = th.empty((heads, nq, 128), dtype=th.float32, device="cuda")
    wv, nbv = tq.kv_workspace(tq.TQ_KV_OP_VALUES, n, heads, nq)
    _replays_match(lambda: tq.tq_kv_values(p, heads, nq, rec, r, n, bits, sd, lv, out, wv, nbv), out)
    wa, nba = tq.kv_workspace(tq.TQ_KV_OP_ATTEND, n, heads, nq)
    att = th.empty((heads, nq, 128), dtype=th.float32, device="cuda")
    _replays_match(lambda: tq.tq_kv_attend(scores, 0.125, heads, nq, rec, r, n, bits, sd, lv, att, wa, nba), att)
