"""GPU parity of the prefill GEMM (matrix cores) against the oracle."""
import numpy as np
import pytest

import synth
import ternary_weight_quantized_tq_amd as tq
from oracle import tq_oracle as O

from parity import assert_parity
from tqgpu import act_tensor, dev, gpu_pack, gpu_quantize_pack, run_gemm, run_gemv, torch

pytestmark = pytest.mark.gpu


def _rand(seed, n, k):
    t = synth.trits(seed, n, k)
    s = synth.scales(seed + 1, n, k // 128)
    return t, s, gpu_pack(t, s)


@pytest.mark.parametrize("m,n,k", [(70, 256, 384), (64, 300, 1280), (3, 257, 640)])
def test_gemm_one_hot_exact(m, n, k):
    t, s, w = _rand(40 + n, n, k)
    rng = np.random.default_rng(41)
    cols = rng.integers(0, k, m)
    x = np.zeros((m, k), np.float32)
    x[np.arange(m), cols] = 1.0
    y = run_gemm(w, dev(x), m, fused=False)
    want = (s[:, cols // 128].astype(np.float64) * t[:, cols]).T
    assert np.array_equal(y, want)


@pytest.mark.parametrize("m,n,k,dtype", [(130, 300, 1280, "bf16"), (64, 512, 2048, "f32"), (1, 256, 640, "bf16"),
                                         (200, 1024, 5120, "bf16"), (65, 320, 17408, "f16")])
def test_gemm_random_vs_oracle(m, n, k, dtype):
    t, s, w = _rand(60 + m + n, n, k)
    act = synth.activations(61 + m, m, k, dtype)
    y = run_gemm(w, act_tensor(act), m)
    y_ref = O.gemv(O.pack(t), s, k, act.values, True)
    assert_parity(y, y_ref)


def test_gemm_row_equals_gemv():
    t, s, w = _rand(80, 512, 1280)
    act = synth.activations(81, 4, 1280, "bf16")
    yg = run_gemm(w, act_tensor(act), 4)
    yv = run_gemv(w, act_tensor(synth.Activations(act.values[:1], act.raw[:1], "bf16")), 1)
    assert np.abs(yg[0] - yv[0]).max() <= 1e-5 * np.abs(yv[0]).max()


def test_gemm_prefill_full_size_sampled():
    """2048 x 5120 x 17408, weights quantised on the GPU; the oracle checks
    8 rows x 192 columns."""
    wl = synth.PREFILL_GEMM.linears[0]
    w64 = synth.weights(wl.w_seed, wl.n, wl.k)
    act = synth.activations(wl.x_seed, 2048, wl.k, "bf16")
    w = gpu_quantize_pack(w64)
    y = run_gemm(w, act_tensor(act), 2048)
    rng = np.random.default_rng(5)
    rows = np.concatenate([rng.choice(2048, 6, replace=False), [0, 2047]])
    cols = np.concatenate([rng.choice(wl.n, 190, replace=False), [0, wl.n - 1]])
    t, s, _ = O.quantize(w64[cols])
    y_ref = O.gemv(O.pack(t), s, wl.k, act.values[rows], True)
    assert_parity(y[np.ix_(rows, cols)], y_ref)


def test_gemm_accumulate():
    """TQ_ACCUMULATE adds the product into Y (a residual stream)."""
    th = torch()
    t, s, w = _rand(95, 300, 1280)
    m = 70
    act = synth.activations(96, m, 1280, "bf16")
    base = np.random.default_rng(97).normal(size=(m, 300)).astype(np.float32)
    y = dev(base.copy())
    ws, nbytes = tq.workspace(tq.TQ_OP_GEMM, w, m)
    tq.tq_gemm(w, act_tensor(act), m, y, tq.TQ_FWHT_FUSED | tq.TQ_ACCUMULATE, ws, nbytes)
    th.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64) - base
    y_ref = O.gemv(O.pack(t), s, 1280, act.values, True)
    assert_parity(got, y_ref)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("scale", [3e-6, 2e4])
def test_gemm_activation_range(dtype, scale):
    """Activations of scale 2e4 (x' past fp16's largest value) and 3e-6 (x'
    below fp16's normal range): the prep step scales each row by a power of
    two before splitting it into fp16 parts, and the epilogue undoes it."""
    t, s, w = _rand(120, 300, 1920)
    m = 70
    act = synth.activations(121, m, 1920, dtype, scale=scale)
    y = run_gemm(w, act_tensor(act), m)
    y_ref = O.gemv(O.pack(t), s, 1920, act.values, True)
    assert_parity(y, y_ref)


def test_gemm_rows_of_very_different_scales():
    """Each activation row gets its own power of two: rows of scale 1e-5, 1
    and 3e4 in one call."""
    t, s, w = _rand(130, 257, 1280)
    m = 66
    act = synth.activations(131, m, 1280, "f32")
    x = act.raw.copy()
    x[::3] *= 1e-5
    x[1::3] *= 3e4
    y = run_gemm(w, dev(x), m)
    y_ref = O.gemv(O.pack(t), s, 1280, x.astype(np.float64), True)
    for r in range(m):
        assert_parity(y[r:r + 1], y_ref[r:r + 1], what=f"row {r}")


# TQ_FAST_F16: x' as one fp16 part after the per-row power of two.  fp16
# rounding is at most 2^-11 relative, about 2.8e-4 RMS, so the output error
# sits near 3e-4: the tests hold it to 6e-4 rel-L2 (the path's bound is 1e-3)
# and 3e-3 of each row's largest value.
FAST = dict(rel_l2=6e-4, row_max=3e-3)


def _run_gemm_flags(w, x, m, flags):
    th = torch()
    y = th.empty((m, w.n), dtype=th.float32, device="cuda")
    ws, nbytes = tq.workspace(tq.TQ_OP_GEMM, w, m)
    tq.tq_gemm(w, x, m, y, flags, ws, nbytes)
    th.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("m,n,k,dtype", [(1, 256, 640, "bf16"), (70, 300, 1280, "bf16"), (130, 257, 2048, "f32"),
                                         (200, 1024, 5120, "bf16"), (129, 320, 17408, "f16")])
def test_gemm_fast_f16_vs_oracle(m, n, k, dtype):
    t, s, w = _rand(160 + m + n, n, k)
    act = synth.activations(161 + m, m, k, dtype)
    y = _run_gemm_flags(w, act_tensor(act), m, tq.TQ_FWHT_FUSED | tq.TQ_FAST_F16)
    assert_parity(y, O.gemv(O.pack(t), s, k, act.values, True), **FAST)


@pytest.mark.parametrize("scale", [3e-6, 2e4])
def test_gemm_fast_f16_activation_range(scale):
    t, s, w = _rand(170, 300, 1920)
    act = synth.activations(171, 130, 1920, "bf16", scale=scale)
    y = _run_gemm_flags(w, act_tensor(act), 130, tq.TQ_FWHT_FUSED | tq.TQ_FAST_F16)
    assert_parity(y, O.gemv(O.pack(t), s, 1920, act.values, True), **FAST)


def test_gemm_fast_f16_one_hot_exact():
    """A one-hot row is exact in one fp16 part too (1 * 2^e is a power of two)."""
    n, k, m = 300, 1280, 140
    t, s, w = _rand(180, n, k)
    cols = np.random.default_rng(181).integers(0, k, m)
    x = np.zeros((m, k), np.float32)
    x[np.arange(m), cols] = 1.0
    y = _run_gemm_flags(w, dev(x), m, tq.TQ_FAST_F16)
    assert np.array_equal(y, (s[:, cols // 128].astype(np.float64) * t[:, cols]).T)


@pytest.mark.parametrize("group,levels", [(64, 3), (128, 2), (64, 2)])
def test_gemm_fast_f16_variants(group, levels):
    n, k, m = 320, 2560, 150
    if levels == 3:
        t = synth.trits(190, n, k)
    else:
        t = np.where(np.random.default_rng(190).random((n, k)) < 0.5, -1, 1).astype(np.int8)
    s = synth.scales(191, n, k // group)
    w = gpu_pack(t, s, group=group, levels=levels)
    act = synth.activations(192, m, k, "bf16")
    y = _run_gemm_flags(w, act_tensor(act), m, tq.TQ_FWHT_FUSED | tq.TQ_FAST_F16)
    words = O.pack(t) if levels == 3 else O.pack_binary(t)
    assert_parity(y, O.gemv(words, s, k, act.values, True, group, levels), **FAST)


def test_gemm_fast_f16_prefill_full_size_sampled():
    """2048 x 5120 x 17408 with TQ_FAST_F16, weights quantised on the GPU;
    8 rows x 192 columns against the oracle."""
    wl = synth.PREFILL_GEMM.linears[0]
    w64 = synth.weights(wl.w_seed, wl.n, wl.k)
    act = synth.activations(wl.x_seed, 2048, wl.k, "bf16")
    w = gpu_quantize_pack(w64)
    y = _run_gemm_flags(w, act_tensor(act), 2048, tq.TQ_FWHT_FUSED | tq.TQ_FAST_F16)
    rng = np.random.default_rng(6)
    rows = np.concatenate([rng.choice(2048, 6, replace=False), [0, 2047]])
    cols = np.concatenate([rng.choice(wl.n, 190, replace=False), [0, wl.n - 1]])
    t, s, _ = O.quantize(w64[cols])
    assert_parity(y[np.ix_(rows, cols)], O.gemv(O.pack(t), s, wl.k, act.values[rows], True), **FAST)
