"""GPU parity of the MoE path (router, grouped expert MLP) against the oracle."""
import numpy as np
import pytest

import synth
import ternary_weight_quantized_tq_amd as tq
from oracle import tq_oracle as O

from parity import assert_parity
from tqgpu import act_tensor, dev, gpu_pack_expert, run_moe, torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("t,e,topk,seed", [(64, 256, 8, 4903), (1, 256, 8, 4901), (5, 40, 3, 7), (3, 1000, 32, 9)])
def test_router_matches_oracle(t, e, topk, seed):
    lg = synth.logits(seed, t, e)
    ids_ref, w_ref = O.route(lg, topk)
    th = torch()
    ids = th.empty((t, topk), dtype=th.int32, device="cuda")
    w = th.empty((t, topk), dtype=th.float32, device="cuda")
    tq.tq_moe_route(dev(lg), t, e, topk, ids, w)
    th.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert np.abs(w.cpu().numpy() - w_ref).max() < 1e-5


def test_router_ties_go_to_the_lower_id():
    """Equal logits: the chosen ids ascend from 0 and the weights are equal;
    a block of tied maxima is taken in id order before lower logits."""
    th = torch()
    e, topk = 48, 6
    lg = np.zeros((2, e), np.float32)
    lg[1, [40, 7, 23, 31]] = 3.0      # four tied maxima, then the zeros tie
    ids = th.empty((2, topk), dtype=th.int32, device="cuda")
    w = th.empty((2, topk), dtype=th.float32, device="cuda")
    tq.tq_moe_route(dev(lg), 2, e, topk, ids, w)
    th.cuda.synchronize()
    ids_ref, w_ref = O.route(lg, topk)
    assert ids.cpu().numpy().tolist() == ids_ref.tolist()
    assert ids_ref[0].tolist() == list(range(topk)) and ids_ref[1].tolist() == [7, 23, 31, 40, 0, 1]
    assert np.abs(w.cpu().numpy() - w_ref).max() < 1e-6


def _random_experts(seed, E, hidden, inter):
    w_gu = tq.empty_weights(2 * inter, hidden, num_experts=E)
    w_dn = tq.empty_weights(hidden, inter, num_experts=E)
    host = {"gu_w": [], "gu_s": [], "dn_w": [], "dn_s": []}
    for e in range(E):
        t = synth.trits(seed + 10 * e, 2 * inter, hidden)
        s = synth.scales(seed + 10 * e + 1, 2 * inter, hidden // 128)
        gpu_pack_expert(w_gu, e, trits=t, scales=s)
        host["gu_w"].append(O.pack(t)), host["gu_s"].append(s)
        t = synth.trits(seed + 10 * e + 2, hidden, inter)
        s = synth.scales(seed + 10 * e + 3, hidden, inter // 128)
        gpu_pack_expert(w_dn, e, trits=t, scales=s)
        host["dn_w"].append(O.pack(t)), host["dn_s"].append(s)
    return w_gu, w_dn, host


@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
def test_moe_small_random(dtype):
    E, hidden, inter, T, topk = 6, 256, 128, 5, 2
    w_gu, w_dn, h = _random_experts(300, E, hidden, inter)
    act = synth.activations(31, T, hidden, dtype)
    rng = np.random.default_rng(32)
    ids = np.stack([rng.choice(E, topk, replace=False) for _ in range(T)]).astype(np.int32)
    rw = rng.random((T, topk))
    rw /= rw.sum(axis=1, keepdims=True)
    y = run_moe(w_gu, w_dn, act_tensor(act), T, topk, ids, rw)
    y_ref = O.moe(act.values, ids, rw, h["gu_w"], h["gu_s"], h["dn_w"], h["dn_s"], hidden, inter)
    assert_parity(y, y_ref)


@pytest.mark.parametrize("T", [2, 40])
@pytest.mark.parametrize("scale", [3e-6, 2e4])
def test_moe_activation_range(T, scale):
    """Activations of scale 2e4 and 3e-6 through both launch shapes (4 pairs:
    per-pair launches; 80 pairs: bucketed by expert), with a hidden size of
    3.2 slices."""
    E, hidden, inter, topk = 4, 2048, 256, 2
    w_gu, w_dn, h = _random_experts(700, E, hidden, inter)
    act = synth.activations(71, T, hidden, "bf16", scale=scale)
    rng = np.random.default_rng(72)
    ids = np.stack([rng.choice(E, topk, replace=False) for _ in range(T)]).astype(np.int32)
    rw = rng.random((T, topk))
    rw /= rw.sum(axis=1, keepdims=True)
    y = run_moe(w_gu, w_dn, act_tensor(act), T, topk, ids, rw)
    with np.errstate(over="ignore"):  # silu of large negative gates: exp overflows to inf, silu -> 0
        y_ref = O.moe(act.values, ids, rw, h["gu_w"], h["gu_s"], h["dn_w"], h["dn_s"], hidden, inter)
    assert np.all(np.isfinite(y))
    assert_parity(y, y_ref)


@pytest.mark.parametrize("T", [21, 40])
def test_moe_many_tokens_per_expert_and_bad_ids(T):
    """More than 8 tokens on one expert (several tiles when bucketed: 80
    pairs; 42 pairs take the per-pair launches), and ids outside [0, E) that
    must contribute nothing."""
    E, hidden, inter, topk = 3, 384, 256, 2
    w_gu, w_dn, h = _random_experts(500, E, hidden, inter)
    act = synth.activations(51, T, hidden, "bf16")
    ids = np.zeros((T, topk), np.int32)
    ids[:, 1] = np.arange(T) % E
    ids[3, 1] = -1
    ids[7, 0] = E + 4
    rw = np.full((T, topk), 0.5)
    y = run_moe(w_gu, w_dn, act_tensor(act), T, topk, ids, rw)
    ok = (ids >= 0) & (ids < E)
    y_ref = np.zeros_like(y)
    for t in range(T):
        for j in range(topk):
            if ok[t, j]:
                y_ref[t] += O.moe(act.values[t:t + 1], ids[t:t + 1, j:j + 1], rw[t:t + 1, j:j + 1], h["gu_w"],
                                  h["gu_s"], h["dn_w"], h["dn_s"], hidden, inter)[0]
    assert_parity(y, y_ref)


@pytest.mark.parametrize("T,topk", [(2, 12), (2, 32), (3, 22), (4, 16), (5, 9)])
def test_moe_wide_topk(T, topk):
    """9 to 32 slots per token with two invalid ids: below four tokens the
    slots' rows are combined by whichever slot finishes last, from four on
    in one workgroup per token and row block, eight slots at a time (64
    pairs is the largest per-pair launch, 66 pairs are bucketed)."""
    E, hidden, inter = 40, 640, 384
    w_gu, w_dn, h = _random_experts(900, E, hidden, inter)
    act = synth.activations(91, T, hidden, "f32")
    rng = np.random.default_rng(92)
    ids = np.stack([rng.choice(E, topk, replace=False) for _ in range(T)]).astype(np.int32)
    ids[0, topk - 1] = -3
    ids[T - 1, 1] = E
    rw = rng.random((T, topk))
    rw /= rw.sum(axis=1, keepdims=True)
    y = run_moe(w_gu, w_dn, act_tensor(act), T, topk, ids, rw)
    ok = (ids >= 0) & (ids < E)
    y_ref = O.moe(act.values, np.where(ok, ids, 0), np.where(ok, rw, 0.0), h["gu_w"], h["gu_s"], h["dn_w"], h["dn_s"],
                  hidden, inter)
    assert_parity(y, y_ref)


@pytest.mark.parametrize("wl", [synth.MOE_T1, synth.MOE_T64], ids=["t1", "t64"])
def test_moe_expert_layer_workload(wl):
    """256 experts (hidden 2048, intermediate 512), top-8 from seeded logits,
    experts quantised on the GPU; the oracle recomputes sampled tokens."""
    lg = synth.logits(wl.logit_seed, wl.tokens, wl.experts)
    ids, rw = O.route(lg, wl.topk)
    act = synth.activations(wl.x_seed, wl.tokens, wl.hidden, "bf16")
    w_gu = tq.empty_weights(2 * wl.inter, wl.hidden, num_experts=wl.experts)
    w_dn = tq.empty_weights(wl.hidden, wl.inter, num_experts=wl.experts)
    tokens = list(range(wl.tokens)) if wl.tokens <= 4 else [0, 17, 42, wl.tokens - 1]
    need = sorted(set(ids.ravel().tolist()))
    check = sorted(set(ids[tokens].ravel().tolist()))
    host = {}
    for e in need:
        gu64, dn64 = synth.expert_weights(e, wl.hidden, wl.inter)
        gpu_pack_expert(w_gu, e, weights64=gu64)
        gpu_pack_expert(w_dn, e, weights64=dn64)
        if e in check:
            t, s, _ = O.quantize(gu64)
            t2, s2, _ = O.quantize(dn64)
            host[e] = (O.pack(t), s, O.pack(t2), s2)
    y = run_moe(w_gu, w_dn, act_tensor(act), wl.tokens, wl.topk, ids, rw)
    gu_w = {e: v[0] for e, v in host.items()}
    gu_s = {e: v[1] for e, v in host.items()}
    dn_w = {e: v[2] for e, v in host.items()}
    dn_s = {e: v[3] for e, v in host.items()}
    y_ref = O.moe(act.values, ids, rw, gu_w, gu_s, dn_w, dn_s, wl.hidden, wl.inter, tokens=tokens)
    assert_parity(y[tokens], y_ref[tokens])


def test_moe_many_experts_few_pairs():
    """1500 experts (past the bucket step's 1024) on the per-pair path; only
    the experts in use are packed."""
    E, hidden, inter, T, topk = 1500, 256, 128, 2, 4
    ids = np.array([[1499, 1024, 3, 700], [1025, 1499, 0, 1100]], np.int32)
    w_gu = tq.empty_weights(2 * inter, hidden, num_experts=E)
    w_dn = tq.empty_weights(hidden, inter, num_experts=E)
    h = {"gu_w": {}, "gu_s": {}, "dn_w": {}, "dn_s": {}}
    for e in sorted(set(ids.ravel().tolist())):
        t = synth.trits(1100 + e, 2 * inter, hidden)
        s = synth.scales(1101 + e, 2 * inter, hidden // 128)
        gpu_pack_expert(w_gu, e, trits=t, scales=s)
        h["gu_w"][e], h["gu_s"][e] = O.pack(t), s
        t = synth.trits(1102 + e, hidden, inter)
        s = synth.scales(1103 + e, hidden, inter // 128)
        gpu_pack_expert(w_dn, e, trits=t, scales=s)
        h["dn_w"][e], h["dn_s"][e] = O.pack(t), s
    act = synth.activations(111, T, hidden, "bf16")
    rw = np.full((T, topk), 0.25)
    y = run_moe(w_gu, w_dn, act_tensor(act), T, topk, ids, rw)
    y_ref = O.moe(act.values, ids, rw, h["gu_w"], h["gu_s"], h["dn_w"], h["dn_s"], hidden, inter)
    assert_parity(y, y_ref)


@pytest.mark.parametrize("T", [1, 3, 5, 40])
def test_moe_accumulate(T):
    """TQ_ACCUMULATE adds the layer into y (a residual stream): per-pair
    (T = 1, 3: device atomics), per-token (T = 5) and bucketed (T = 40)."""
    th = torch()
    E, hidden, inter, topk = 10, 640, 256, 2
    w_gu, w_dn, h = _random_experts(700, E, hidden, inter)
    act = synth.activations(71, T, hidden, "bf16")
    rng = np.random.default_rng(72)
    ids = np.stack([rng.choice(E, topk, replace=False) for _ in range(T)]).astype(np.int32)
    rw = rng.random((T, topk))
    rw /= rw.sum(axis=1, keepdims=True)
    base = rng.normal(size=(T, hidden)).astype(np.float32)
    y = dev(base.copy())
    ws, nbytes = tq.workspace(tq.TQ_OP_MOE, w_gu, T, topk)
    tq.tq_moe_gemv(w_gu, w_dn, act_tensor(act), T, topk, dev(ids), dev(rw.astype(np.float32)), y,
                   tq.TQ_FWHT_FUSED | tq.TQ_ACCUMULATE, ws, nbytes)
    th.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64) - base
    y_ref = O.moe(act.values, ids, rw, h["gu_w"], h["gu_s"], h["dn_w"], h["dn_s"], hidden, inter)
    assert_parity(got, y_ref)


@pytest.mark.parametrize("T,topk", [(3, 2), (5, 4), (40, 2)])
def test_moe_reports_bad_ids(T, topk):
    """Ids outside [0, E) are counted on the device and reported by
    tq_moe_bad_ids (per-pair, per-token and bucketed paths); a following
    call with valid ids on the same workspace reports zero."""
    th = torch()
    E, hidden, inter = 5, 256, 128
    w_gu, w_dn, h = _random_experts(1300, E, hidden, inter)
    act = synth.activations(131, T, hidden, "bf16")
    rng = np.random.default_rng(132)
    ids = np.stack([rng.choice(E, topk, replace=False) for _ in range(T)]).astype(np.int32)
    good_ids = ids.copy()
    ids[0, 0] = -1
    ids[T - 1, topk - 1] = E
    ids[T // 2, 0] = 1 << 30
    rw = np.full((T, topk), 1.0 / topk)
    y = th.empty((T, hidden), dtype=th.float32, device="cuda")
    ws, nbytes = tq.workspace(tq.TQ_OP_MOE, w_gu, T, topk)
    x = act_tensor(act)
    tq.tq_moe_gemv(w_gu, w_dn, x, T, topk, dev(ids), dev(rw.astype(np.float32)), y, tq.TQ_FWHT_FUSED, ws, nbytes)
    assert tq.tq_moe_bad_ids(ws, nbytes) == 3
    st = tq.lib().tq_moe_bad_ids(ws.data_ptr(), nbytes, tq.ctypes.byref(tq.ctypes.c_int32()), None)
    assert st == tq.TQ_EDATA
    tq.tq_moe_gemv(w_gu, w_dn, x, T, topk, dev(good_ids), dev(rw.astype(np.float32)), y, tq.TQ_FWHT_FUSED, ws,
                   nbytes)
    assert tq.tq_moe_bad_ids(ws, nbytes) == 0
    y_ref = O.moe(act.values, good_ids, rw, h["gu_w"], h["gu_s"], h["dn_w"], h["dn_s"], hidden, inter)
    assert_parity(y.cpu().numpy(), y_ref)


def _run_moe_flags(w_gu, w_dn, x, t, topk, ids, rw, flags, ws=None, nbytes=None, y=None):
    th = torch()
    if y is None:
        y = th.empty((t, w_dn.n), dtype=th.float32, device="cuda")
    if ws is None:
        ws, nbytes = tq.workspace(tq.TQ_OP_MOE, w_gu, t, topk)
    tq.tq_moe_gemv(w_gu, w_dn, x, t, topk, dev(ids.astype(np.int32)), dev(rw.astype(np.float32)), y, flags, ws,
                   nbytes)
    th.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("T,topk", [(1, 2), (3, 4), (2, 12), (5, 9), (8, 8)])
def test_moe_one_launch_matches_oracle(T, topk):
    """TQ_MOE_ONE_LAUNCH: the last gate/up workgroup of a pair runs its down
    projection, the last slot of a token combines; with invalid ids."""
    E, hidden, inter = 12, 640, 384
    w_gu, w_dn, h = _random_experts(1700, E, hidden, inter)
    act = synth.activations(171, T, hidden, "bf16")
    rng = np.random.default_rng(172)
    ids = np.stack([rng.choice(E, topk, replace=False) for _ in range(T)]).astype(np.int32)
    ids[0, topk - 1] = -2
    rw = rng.random((T, topk))
    rw /= rw.sum(axis=1, keepdims=True)
    y = _run_moe_flags(w_gu, w_dn, act_tensor(act), T, topk, ids, rw, tq.TQ_FWHT_FUSED | tq.TQ_MOE_ONE_LAUNCH)
    ok = (ids >= 0) & (ids < E)
    y_ref = O.moe(act.values, np.where(ok, ids, 0), np.where(ok, rw, 0.0), h["gu_w"], h["gu_s"], h["dn_w"],
                  h["dn_s"], hidden, inter)
    assert_parity(y, y_ref)


def test_moe_one_launch_repeated_calls_and_accumulate():
    """Counters reset themselves: three calls in a row on one workspace
    (different token counts), then TQ_ACCUMULATE, all against the oracle and
    bit-identical across repeats."""
    th = torch()
    E, hidden, inter, topk = 6, 1280, 512, 4
    w_gu, w_dn, h = _random_experts(1800, E, hidden, inter)
    ws, nbytes = tq.workspace(tq.TQ_OP_MOE, w_gu, 16, topk)   # sized for the largest call
    outs = []
    for T in (3, 1, 3):
        act = synth.activations(181 + T, T, hidden, "bf16")
        rng = np.random.default_rng(182 + T)
        ids = np.stack([rng.choice(E, topk, replace=False) for _ in range(T)]).astype(np.int32)
        rw = rng.random((T, topk))
        rw /= rw.sum(axis=1, keepdims=True)
        y = _run_moe_flags(w_gu, w_dn, act_tensor(act), T, topk, ids, rw, tq.TQ_FWHT_FUSED | tq.TQ_MOE_ONE_LAUNCH,
                           ws, nbytes)
        assert_parity(y, O.moe(act.values, ids, rw, h["gu_w"], h["gu_s"], h["dn_w"], h["dn_s"], hidden, inter))
        outs.append(y)
    assert np.array_equal(outs[0], outs[2])
    base = np.random.default_rng(190).normal(size=(3, hidden)).astype(np.float32)
    yd = dev(base.copy())
    act = synth.activations(184, 3, hidden, "bf16")
    rng = np.random.default_rng(185)
    ids = np.stack([rng.choice(E, topk, replace=False) for _ in range(3)]).astype(np.int32)
    rw = np.full((3, topk), 1.0 / topk)
    got = _run_moe_flags(w_gu, w_dn, act_tensor(act), 3, topk, ids, rw,
                         tq.TQ_FWHT_FUSED | tq.TQ_MOE_ONE_LAUNCH | tq.TQ_ACCUMULATE, ws, nbytes, y=yd) - base
    assert_parity(got, O.moe(act.values, ids, rw, h["gu_w"], h["gu_s"], h["dn_w"], h["dn_s"], hidden, inter))


def test_moe_one_launch_expert_layer_t1():
    """256 experts (hidden 2048, intermediate 512), top-8, one token, experts
    quantised on the GPU: one launch against the oracle and equal to the
    two-launch path up to rounding order."""
    wl = synth.MOE_T1
    lg = synth.logits(wl.logit_seed, 1, wl.experts)
    ids, rw = O.route(lg, wl.topk)
    act = synth.activations(wl.x_seed, 1, wl.hidden, "bf16")
    w_gu = tq.empty_weights(2 * wl.inter, wl.hidden, num_experts=wl.experts)
    w_dn = tq.empty_weights(wl.hidden, wl.inter, num_experts=wl.experts)
    host = {}
    for e in sorted(set(ids.ravel().tolist())):
        gu64, dn64 = synth.expert_weights(e, wl.hidden, wl.inter)
        gpu_pack_expert(w_gu, e, weights64=gu64)
        gpu_pack_expert(w_dn, e, weights64=dn64)
        t, s, _ = O.quantize(gu64)
        t2, s2, _ = O.quantize(dn64)
        host[e] = (O.pack(t), s, O.pack(t2), s2)
    x = act_tensor(act)
    y1 = _run_moe_flags(w_gu, w_dn, x, 1, wl.topk, ids, rw, tq.TQ_FWHT_FUSED | tq.TQ_MOE_ONE_LAUNCH)
    y2 = _run_moe_flags(w_gu, w_dn, x, 1, wl.topk, ids, rw, tq.TQ_FWHT_FUSED)
    y_ref = O.moe(act.values, ids, rw, {e: v[0] for e, v in host.items()}, {e: v[1] for e, v in host.items()},
                  {e: v[2] for e, v in host.items()}, {e: v[3] for e, v in host.items()}, wl.hidden, wl.inter)
    assert_parity(y1, y_ref)
    assert_parity(y1, y2, rel_l2=1e-6, row_max=1e-5)


def test_moe_one_launch_limits():
    lib = tq.lib()
    E = 4
    w_gu = tq.empty_weights(2 * 256, 512, num_experts=E)
    w_dn = tq.empty_weights(512, 256, num_experts=E)
    for t, topk, inter_ok in ((9, 8, True), (2, 2, False)):
        gu, dn = w_gu.desc(), w_dn.desc()
        if not inter_ok:   # intermediate 3200: five slices of 640
            gu = tq.tq_weights(tq.TQ_MAGIC, tq.TQ_VERSION, 6400, 512, E, tq.TQ_LAYOUT_ROW64, 128, 3, gu.words, gu.scales)
            dn = tq.tq_weights(tq.TQ_MAGIC, tq.TQ_VERSION, 512, 3200, E, tq.TQ_LAYOUT_ROW64, 128, 3, dn.words, dn.scales)
        st = lib.tq_moe_gemv(tq.ctypes.byref(gu), tq.ctypes.byref(dn), 0x3000, tq.TQ_BF16, t, topk, 0x4000, 0x5000,
                             0x6000, tq.TQ_FWHT_FUSED | tq.TQ_MOE_ONE_LAUNCH, 0x7000, 1 << 30, None)
        assert st == tq.TQ_EUNSUPPORTED, (t, topk, st)
