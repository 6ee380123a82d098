"""tq_gemv_noalloc (no allocation: library-owned scratch array per GPU)
against tq_gemv with a caller workspace, called through the C ABI: two
calls in a row on the shared array, the second with a smaller input (it
must not see the first call's partial sums), bit-identical to the
workspace entry point (same kernels, deterministic reduction)."""
import ctypes

import numpy as np
import pytest

import synth
import ternary_weight_quantized_tq_amd as tq

from tqgpu import act_tensor, gpu_pack, torch

pytestmark = pytest.mark.gpu


def _via_workspace(w, x, m, flags):
    th = torch()
    y = th.empty((m, w.n), dtype=th.float32, device="cuda")
    ws, nbytes = tq.workspace(tq.TQ_OP_GEMV, w, m)
    tq.tq_gemv(w, x, m, y, flags, ws, nbytes)
    return y


def _via_noalloc(w, x, m, flags):
    th = torch()
    y = th.full((m, w.n), float("nan"), dtype=th.float32, device="cuda")
    st = tq.lib().tq_gemv_noalloc(ctypes.byref(w.desc()), x.data_ptr(), tq.dtype_code(x), m, y.data_ptr(), flags,
                                  th.cuda.current_stream().cuda_stream)
    assert st == tq.TQ_OK, tq.tq_strerror(st)
    return y


def _case(seed, n, k, m):
    t = synth.trits(seed, n, k)
    s = synth.scales(seed + 1, n, k // 128)
    return gpu_pack(t, s), act_tensor(synth.activations(seed + 2, m, k, "bf16"))


@pytest.mark.parametrize("flags", [tq.TQ_FWHT_FUSED, 0])
def test_noalloc_matches_workspace_entry_point_twice(flags):
    th = torch()
    first = (5120, 17408, 8)      # 28 slices x 8 rows x 5120: 4.6 MB of partial sums
    second = (700, 2560, 3)       # smaller: 4 slices, fewer rows, fewer activation rows
    outs = []
    for seed, (n, k, m) in ((11, first), (23, second)):
        w, x = _case(seed, n, k, m)
        y_nw = _via_noalloc(w, x, m, flags)
        th.cuda.synchronize()
        y_ws = _via_workspace(w, x, m, flags)
        th.cuda.synchronize()
        a, b = y_nw.cpu().numpy(), y_ws.cpu().numpy()
        assert np.all(np.isfinite(a))
        assert np.array_equal(a, b), f"{n}x{k} m={m}: max diff {np.abs(a - b).max()}"
        outs.append(a)
    assert outs[1].shape == (3, 700)


def test_noalloc_single_slice_and_m1():
    th = torch()
    for seed, (n, k, m) in ((31, (17408, 5120, 1)), (37, (300, 640, 2))):
        w, x = _case(seed, n, k, m)
        y_nw = _via_noalloc(w, x, m, tq.TQ_FWHT_FUSED)
        y_ws = _via_workspace(w, x, m, tq.TQ_FWHT_FUSED)
        th.cuda.synchronize()
        assert np.array_equal(y_nw.cpu().numpy(), y_ws.cpu().numpy())


def test_noalloc_accumulate_needs_no_array():
    th = torch()
    w, x = _case(41, 1000, 5120, 4)
    base = th.ones((4, 1000), dtype=th.float32, device="cuda")
    y = base.clone()
    tq.tq_gemv_noalloc(w, x, 4, y, tq.TQ_FWHT_FUSED | tq.TQ_ACCUMULATE)
    ref = _via_workspace(w, x, 4, tq.TQ_FWHT_FUSED)
    th.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64) - 1.0
    want = ref.cpu().numpy().astype(np.float64)
    assert np.abs(got - want).max() <= 1e-5 * np.abs(want).max()


def test_noalloc_rejects_partials_beyond_the_array():
    """34816 x 17408 at M = 8 needs 28 x 8 x 34816 x 4 B = 31 MB of partial
    sums: rejected before any GPU work (descriptor pointers are never read)."""
    d = tq.tq_weights(tq.TQ_MAGIC, tq.TQ_VERSION, 34816, 17408, 1, tq.TQ_LAYOUT_ROW64, 128, 3, 0x1000, 0x2000)
    st = tq.lib().tq_gemv_noalloc(ctypes.byref(d), 0x3000, tq.TQ_BF16, 8, 0x4000, tq.TQ_FWHT_FUSED, None)
    assert st == tq.TQ_ENOSPACE
