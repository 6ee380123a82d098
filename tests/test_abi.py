"""CPU checks of the boundary: the library loads, exports every function
include/tq.h declares, sizes follow the closed forms, and malformed
requests are rejected synchronously (before any HIP call)."""
import ctypes

import pytest

import ternary_weight_quantized_tq_amd as tq
from oracle import tq_oracle as O


def test_library_exports_every_header_function():
    names = tq.header_functions()
    assert {"tq_pack", "tq_fwht", "tq_gemv", "tq_moe_gemv", "tq_gemm"} <= set(names)
    lib = tq.lib()
    for name in names:
        assert hasattr(lib, name), name


def test_sizes_match_closed_forms():
    for n, k in [(512, 1024), (17408, 5120), (5120, 17408), (1024, 2048), (2048, 512), (3, 20), (1, 1)]:
        assert tq.tq_words_per_row(k) == O.words_per_row(k)
        if k % 128 == 0:
            assert tq.tq_packed_bytes(n, k) == O.packed_bytes(n, k)
        assert tq.tq_layout_words(n, k, tq.TQ_LAYOUT_ROWMAJOR) == n * O.words_per_row(k)
        nb, nsl = -(-n // 64), -(-O.words_per_row(k) // 32)   # 64-row blocks, 640-trit slices
        assert tq.tq_layout_words(n, k, tq.TQ_LAYOUT_ROW64) == nsl * nb * 64 * 32
        if k % 128 == 0:
            assert tq.tq_layout_scales(n, k, tq.TQ_LAYOUT_ROW64) == nsl * nb * 64 * 5
    assert tq.tq_packed_bytes(17408, 5120) == 19218432
    assert tq.tq_packed_bytes(5120, 17408) == 19230720
    assert tq.tq_layout_scales(10, 100, tq.TQ_LAYOUT_ROWMAJOR) == 0      # K % 128 != 0
    assert tq.tq_layout_words(10, 128, 7) == 0


def _desc(**kw):
    d = dict(magic=tq.TQ_MAGIC, version=tq.TQ_VERSION, n=256, k=1280, num_experts=1,
             layout=tq.TQ_LAYOUT_ROW64, words=0x1000, scales=0x2000)
    d.update(kw)
    return tq.tq_weights(d["magic"], d["version"], d["n"], d["k"], d["num_experts"], d["layout"],
                         d["words"], d["scales"])


@pytest.mark.parametrize("kw,status", [
    (dict(magic=0), tq.TQ_EFORMAT),
    (dict(version=2), tq.TQ_EFORMAT),
    (dict(layout=5), tq.TQ_EFORMAT),
    (dict(layout=tq.TQ_LAYOUT_ROWMAJOR), tq.TQ_EUNSUPPORTED),
    (dict(num_experts=4), tq.TQ_EFORMAT),
    (dict(k=1000), tq.TQ_ESHAPE),
    (dict(n=0), tq.TQ_ESHAPE),
    (dict(words=None), tq.TQ_EINVAL),
    (dict(words=0x1004), tq.TQ_EINVAL),
    (dict(scales=0x2002), tq.TQ_EINVAL),
])
def test_gemv_rejects_bad_descriptor(kw, status):
    lib = tq.lib()
    w = _desc(**kw)
    st = lib.tq_gemv(ctypes.byref(w), 0x3000, tq.TQ_BF16, 1, 0x4000, tq.TQ_FWHT_FUSED, 0x5000, 1 << 20, None)
    assert st == status


def test_gemv_rejects_bad_arguments():
    lib = tq.lib()
    w = _desc()
    call = lambda x=0x3000, dt=tq.TQ_BF16, m=1, y=0x4000, fl=1, ws=0x5000, nb=1 << 20: lib.tq_gemv(
        ctypes.byref(w), x, dt, m, y, fl, ws, nb, None)
    assert call(x=None) == tq.TQ_EINVAL
    assert call(y=None) == tq.TQ_EINVAL
    assert call(dt=9) == tq.TQ_EINVAL
    assert call(fl=8) == tq.TQ_EINVAL
    assert call(fl=4) == tq.TQ_EINVAL
    assert call(m=0) == tq.TQ_ESHAPE
    assert call(m=9) == tq.TQ_ESHAPE
    assert call(nb=16) == tq.TQ_ENOSPACE
    assert call(ws=None) == tq.TQ_EINVAL
    # alignment: activations two elements, outputs 4 bytes, workspaces 16
    assert call(x=0x3002) == tq.TQ_EINVAL
    assert call(x=0x3004, dt=tq.TQ_F32) == tq.TQ_EINVAL
    assert call(y=0x4002) == tq.TQ_EINVAL
    assert call(ws=0x5004) == tq.TQ_EINVAL
    need = lib.tq_workspace_bytes(tq.TQ_OP_GEMV, ctypes.byref(w), 1, 0)
    assert 0 < need < 1 << 20
    assert lib.tq_workspace_bytes(tq.TQ_OP_GEMV, ctypes.byref(_desc(magic=1)), 1, 0) == tq.SIZE_MAX


def test_format_calls_reject_bad_arguments():
    lib = tq.lib()
    assert lib.tq_pack(None, 4, 20, 0, 0x10, None) == tq.TQ_EINVAL
    assert lib.tq_pack(0x10, 4, 20, 3, 0x10, None) == tq.TQ_EINVAL
    assert lib.tq_pack(0x10, 0, 20, 0, 0x10, None) == tq.TQ_ESHAPE
    assert lib.tq_pack(0x10, 4, 100, tq.TQ_LAYOUT_ROW64, 0x10, None) == tq.TQ_ESHAPE
    assert lib.tq_unpack(0x10, 4, 100, tq.TQ_LAYOUT_ROW64, 0x10, None) == tq.TQ_ESHAPE
    assert lib.tq_quantize(0x10, tq.TQ_BF16, 4, 128, 0x10, 0x10, None) == tq.TQ_EINVAL
    assert lib.tq_quantize(0x10, tq.TQ_F64, 4, 100, 0x10, 0x10, None) == tq.TQ_ESHAPE
    assert lib.tq_fwht(0x10, tq.TQ_F32, 2, 129, 0x10, None) == tq.TQ_ESHAPE
    assert lib.tq_fwht(0x10, tq.TQ_F64, 2, 128, 0x10, None) == tq.TQ_EINVAL
    assert lib.tq_fwht(0x12, tq.TQ_BF16, 2, 128, 0x10, None) == tq.TQ_EINVAL
    assert lib.tq_fwht(0x10, tq.TQ_BF16, 2, 128, 0x14, None) == tq.TQ_EINVAL
    assert lib.tq_strerror(-2).decode().startswith("invalid shape")


def test_binding_raises_with_message():
    w = tq.Weights(0x1000, 0x2000, 256, 1280, magic=0)
    with pytest.raises(tq.TQError) as e:
        tq._check("tq_gemv", tq.lib().tq_gemv(ctypes.byref(w.desc()), 0x3000, tq.TQ_BF16, 1, 0x4000, 1, 0x5000,
                                              1 << 20, None))
    assert e.value.status == tq.TQ_EFORMAT


def test_binding_refuses_host_and_strided_tensors():
    import torch
    with pytest.raises(ValueError, match="device memory"):
        tq._ptr(torch.zeros(8))
    assert tq._ptr(None) is None and tq._ptr(0x1000) == 0x1000


@pytest.mark.parametrize("experts,t,topk,status", [
    (1500, 20, 4, tq.TQ_EUNSUPPORTED),   # 80 pairs: bucketed, at most 1024 experts
    (1500, 16, 4, tq.TQ_ENOSPACE),       # 64 pairs: per-pair path, no expert limit (then: no workspace)
    (64, 0, 4, tq.TQ_ESHAPE),
    (64, 2, 33, tq.TQ_ESHAPE),
])
def test_moe_limits(experts, t, topk, status):
    lib = tq.lib()
    gu = _desc(n=256, k=512, num_experts=experts)
    dn = _desc(n=512, k=128, num_experts=experts)
    st = lib.tq_moe_gemv(ctypes.byref(gu), ctypes.byref(dn), 0x3000, tq.TQ_BF16, t, topk, 0x4000, 0x5000, 0x6000,
                         tq.TQ_FWHT_FUSED, 0x7000, 0, None)
    assert st == status


def test_moe_and_gemm_check_alignment():
    lib = tq.lib()
    gu = _desc(n=256, k=512)
    dn = _desc(n=512, k=128)
    moe = lambda x=0x3000, ids=0x4000, rw=0x5000, y=0x6000, ws=0x7000: lib.tq_moe_gemv(
        ctypes.byref(gu), ctypes.byref(dn), x, tq.TQ_BF16, 1, 1, ids, rw, y, tq.TQ_FWHT_FUSED, ws, 1 << 24, None)
    assert moe(x=0x3002) == tq.TQ_EINVAL
    assert moe(ids=0x4002) == tq.TQ_EINVAL
    assert moe(rw=0x5001) == tq.TQ_EINVAL
    assert moe(y=0x6002) == tq.TQ_EINVAL
    assert moe(ws=0x7008) == tq.TQ_EINVAL
    w = _desc()
    gemm = lambda x=0x3000, y=0x4000, ws=0x5000: lib.tq_gemm(ctypes.byref(w), x, tq.TQ_F32, 4, y, tq.TQ_FWHT_FUSED,
                                                           ws, 1 << 24, None)
    assert gemm(x=0x3004) == tq.TQ_EINVAL
    assert gemm(y=0x4002) == tq.TQ_EINVAL
    assert gemm(ws=0x5008) == tq.TQ_EINVAL
