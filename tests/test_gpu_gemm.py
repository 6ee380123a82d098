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
