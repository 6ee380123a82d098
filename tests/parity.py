"""Parity assertions shared by the GPU tests: the FP64 oracle's metrics
(whole-tensor rel-L2 and the per-row max |d| / max |y_ref|) against the
bounds the tests hold."""
from __future__ import annotations

import numpy as np

from oracle import tq_oracle as O

# The path's bound is 1e-3 relative L2; the kernels keep x' at FP32-level
# precision (FP32, or two fp16 parts after a power-of-two scaling), so the
# tests hold them to 1e-5, and every output row to 1e-4 of its largest
# reference value.
REL_L2 = 1e-5
ROW_MAX = 1e-4


def assert_parity(y, y_ref, rel_l2=REL_L2, row_max=ROW_MAX, what=""):
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    assert y.shape == y_ref.shape, (what, y.shape, y_ref.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite outputs"
    e = O.rel_l2(y, y_ref)
    r = O.row_max_rel(y, y_ref)
    assert e <= rel_l2, f"{what}: rel-L2 {e:.3e} > {rel_l2:.1e}"
    assert r <= row_max, f"{what}: per-row max error {r:.3e} > {row_max:.1e}"
    return e, r
