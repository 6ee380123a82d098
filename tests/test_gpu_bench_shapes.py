"""GPU parity of tq_gemv at the exact shapes and launch forms the benchmark
times: the dense 27B block's fused projections and the single-stream decode
linears, at M = 1 (single stream), 2 and 8 (eight concurrent streams), in
both output modes (default: slice partials + ordered reduction;
TQ_ACCUMULATE: device atomics into y).

At 256 compute units these shapes take launch forms that small test shapes
never reach:
  * M >= 2 with three or more 64-row blocks per workgroup (every matrix here)
    runs the matrix-core kernel with one wavefront per row block, the
    ten-pair weight lookahead and prologue-only wavefronts (5120 x 5120:
    3 blocks per workgroup, 8 wavefronts at M = 8);
  * M = 1 at 34816 x 5120 (gate||up) runs 16 wavefronts per workgroup, and
    at 5120 x 17408 28 slices with 9 row blocks per workgroup.
Weights are random trits (uniform over {-1, 0, 1}) with random fp16 scales,
packed on the GPU; the oracle recomputes about 200 sampled output rows
(random ones plus row-block and workgroup boundaries) for every activation
row, and each activation row's sampled outputs are held to rel-L2 1e-5 and a
per-row max error of 1e-4 of its largest reference value."""
import numpy as np
import pytest

import synth
import ternary_weight_quantized_tq_amd as tq
from oracle import tq_oracle as O

from parity import assert_parity
from tqgpu import act_tensor, dev, gpu_pack, torch

pytestmark = pytest.mark.gpu

# (n, k): o / q (5120x5120), q||k||v (7168x5120), up or gate (17408x5120),
# down (5120x17408), gate||up (34816x5120).
SHAPES = [(5120, 5120), (7168, 5120), (17408, 5120), (5120, 17408), (34816, 5120)]
_CACHE = {}


def _packed(n, k):
    if (n, k) not in _CACHE:
        _CACHE.clear()  # one shape resident at a time
        t = synth.trits_uniform(9000 + n + k, n, k)
        s = synth.scales(9100 + n + k, n, k // 128)
        _CACHE[(n, k)] = (t, s, gpu_pack(t, s))
    return _CACHE[(n, k)]


def _rows(n):
    rng = np.random.default_rng(n)
    fixed = [0, 1, 63, 64, 191, 192, 575, 576, n // 2, n - 65, n - 64, n - 1]
    return np.unique(np.concatenate([rng.choice(n, 192, replace=False), [r for r in fixed if 0 <= r < n]]))


@pytest.mark.parametrize("mode", ["partial", "accumulate"])
@pytest.mark.parametrize("m", [1, 2, 8])
@pytest.mark.parametrize("n,k", SHAPES)
def test_gemv_bench_shape(n, k, m, mode):
    th = torch()
    t, s, w = _packed(n, k)
    act = synth.activations(9200 + m, m, k, "bf16")
    x = act_tensor(act)
    if mode == "accumulate":
        base = np.random.default_rng(9300 + m).normal(size=(m, n)).astype(np.float32)
        y = dev(base.copy())
        tq.tq_gemv(w, x, m, y, tq.TQ_FWHT_FUSED | tq.TQ_ACCUMULATE)
        th.cuda.synchronize()
        got = y.cpu().numpy().astype(np.float64) - base
    else:
        y = th.empty((m, n), dtype=th.float32, device="cuda")
        ws, nbytes = tq.workspace(tq.TQ_OP_GEMV, w, m)
        tq.tq_gemv(w, x, m, y, tq.TQ_FWHT_FUSED, ws, nbytes)
        th.cuda.synchronize()
        got = y.cpu().numpy().astype(np.float64)
    rows = _rows(n)
    y_ref = O.gemv(O.pack(t[rows]), s[rows], k, act.values, True)
    assert_parity(got[:, rows], y_ref, what=f"{n}x{k} m={m} {mode}")
