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
        assert tq.tq_layout_words(n, k, tq.TQ_LAYOUT_ROWMAJOR, 3) == n * O.words_per_row(k)
        assert tq.tq_layout_words(n, k, tq.TQ_LAYOUT_ROWMAJOR, 2) == n * O.words_per_row_binary(k)
        nb, nsl = -(-n // 64), -(-O.words_per_row(k) // 32)   # 64-row blocks, 640-trit slices
        assert tq.tq_layout_words(n, k, tq.TQ_LAYOUT_ROW64, 3) == nsl * nb * 64 * 32
        assert tq.tq_layout_words(n, k, tq.TQ_LAYOUT_ROW64, 2) == nsl * nb * 64 * 20
        if k % 128 == 0:
            assert tq.tq_layout_scales(n, k, tq.TQ_LAYOUT_ROW64, 128) == nsl * nb * 64 * 5
            assert tq.tq_layout_scales(n, k, tq.TQ_LAYOUT_ROW64, 64) == nsl * nb * 64 * 10
            for g in (64, 128):
                assert tq.tq_format_bytes(n, k, g, 3) == O.packed_bytes(n, k, g)
                assert tq.tq_format_bytes(n, k, g, 2) == O.packed_bytes_binary(n, k, g)
    assert tq.tq_packed_bytes(17408, 5120) == 19218432
    assert tq.tq_packed_bytes(5120, 17408) == 19230720
    assert tq.tq_layout_scales(10, 100, tq.TQ_LAYOUT_ROWMAJOR, 128) == 0      # K % 128 != 0
    assert tq.tq_layout_scales(10, 128, tq.TQ_LAYOUT_ROWMAJOR, 32) == 0       # group not 64 or 128
    assert tq.tq_layout_words(10, 128, 7, 3) == 0
    assert tq.tq_layout_words(10, 128, tq.TQ_LAYOUT_ROW64, 4) == 0
    assert tq.tq_format_bytes(10, 128, 96, 3) == 0 and tq.tq_format_bytes(10, 128, 128, 1) == 0


def _desc(**kw):
    d = dict(magic=tq.TQ_MAGIC, version=tq.TQ_VERSION, n=256, k=1280, num_experts=1,
             layout=tq.TQ_LAYOUT_ROW64, words=0x1000, scales=0x2000)
    d.update(kw)
    return tq.tq_weights(d["magic"], d["version"], d["n"], d["k"], d["num_experts"], d["layout"],
                         d.get("group", 128), d.get("levels", 3), d["words"], d["scales"])


@pytest.mark.parametrize("kw,status", [
    (dict(magic=0), tq.TQ_EFORMAT),
    (dict(version=1), tq.TQ_EFORMAT),
    (dict(group=32), tq.TQ_EFORMAT),
    (dict(levels=4), tq.TQ_EFORMAT),
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
    assert lib.tq_pack(None, 4, 20, 0, 3, 0x10, None) == tq.TQ_EINVAL
    assert lib.tq_pack(0x10, 4, 20, 3, 3, 0x10, None) == tq.TQ_EINVAL
    assert lib.tq_pack(0x10, 4, 20, 0, 1, 0x10, None) == tq.TQ_EINVAL         # levels
    assert lib.tq_pack(0x10, 0, 20, 0, 3, 0x10, None) == tq.TQ_ESHAPE
    assert lib.tq_pack(0x10, 4, 100, tq.TQ_LAYOUT_ROW64, 3, 0x10, None) == tq.TQ_ESHAPE
    assert lib.tq_unpack(0x10, 4, 100, tq.TQ_LAYOUT_ROW64, 3, 0x10, None) == tq.TQ_ESHAPE
    assert lib.tq_unpack(0x10, 4, 128, tq.TQ_LAYOUT_ROW64, 5, 0x10, None) == tq.TQ_EINVAL
    assert lib.tq_quantize(0x10, tq.TQ_BF16, 4, 128, 128, 3, 0x10, 0x10, None) == tq.TQ_EINVAL
    assert lib.tq_quantize(0x10, tq.TQ_F64, 4, 100, 128, 3, 0x10, 0x10, None) == tq.TQ_ESHAPE
    assert lib.tq_quantize(0x10, tq.TQ_F64, 4, 128, 32, 3, 0x10, 0x10, None) == tq.TQ_EINVAL   # group
    assert lib.tq_quantize(0x10, tq.TQ_F64, 4, 128, 64, 1, 0x10, 0x10, None) == tq.TQ_EINVAL   # levels
    assert lib.tq_pack_scales(0x10, 4, 128, 1, 100, 0x10, None) == tq.TQ_EINVAL              # group
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


def test_dimensions_above_the_limit_are_rejected():
    """n, k and m up to TQ_MAX_DIM pass the shape checks (the size queries
    return finite sizes), one step beyond is TQ_ESHAPE or a zero / SIZE_MAX
    size, before any device work."""
    lib = tq.lib()
    top, big = tq.TQ_MAX_DIM, tq.TQ_MAX_DIM + 128
    assert 0 < tq.tq_packed_bytes(top, top) < tq.SIZE_MAX
    assert tq.tq_packed_bytes(big, 128) == 0 and tq.tq_packed_bytes(128, big) == 0
    assert tq.tq_format_bytes(big, 128, 64, 2) == 0
    assert tq.tq_layout_words(top, top, tq.TQ_LAYOUT_ROW64, 3) > 0
    assert tq.tq_layout_words(big, 128, tq.TQ_LAYOUT_ROW64, 3) == 0
    assert tq.tq_layout_scales(128, big, tq.TQ_LAYOUT_ROWMAJOR, 128) == 0
    assert lib.tq_words_per_row(big) == 0
    for kw in (dict(n=big), dict(k=big)):
        w = _desc(**kw)
        assert lib.tq_gemv(ctypes.byref(w), 0x3000, tq.TQ_BF16, 1, 0x4000, 0, 0x5000, 1 << 20, None) == tq.TQ_ESHAPE
        assert lib.tq_workspace_bytes(tq.TQ_OP_GEMV, ctypes.byref(w), 1, 0) == tq.SIZE_MAX
    w = _desc()
    assert lib.tq_workspace_bytes(tq.TQ_OP_GEMM, ctypes.byref(w), big, 0) == tq.SIZE_MAX
    assert lib.tq_workspace_bytes(tq.TQ_OP_MOE, ctypes.byref(_desc(num_experts=4)), 1 << 28, 8) == tq.SIZE_MAX
    assert lib.tq_gemm(ctypes.byref(w), 0x3000, tq.TQ_F32, big, 0x4000, 0, 0x5000, 1 << 24, None) == tq.TQ_ESHAPE
    assert lib.tq_pack(0x10, big, 20, tq.TQ_LAYOUT_ROWMAJOR, 3, 0x10, None) == tq.TQ_ESHAPE
    assert lib.tq_pack(0x10, 4, big, tq.TQ_LAYOUT_ROW64, 3, 0x10, None) == tq.TQ_ESHAPE
    assert lib.tq_unpack(0x10, big, 128, tq.TQ_LAYOUT_ROW64, 3, 0x10, None) == tq.TQ_ESHAPE
    assert lib.tq_pack_scales(0x10, big, 128, tq.TQ_LAYOUT_ROW64, 128, 0x10, None) == tq.TQ_ESHAPE
    assert lib.tq_quantize(0x10, tq.TQ_F64, big, 128, 128, 3, 0x10, 0x10, None) == tq.TQ_ESHAPE
    assert lib.tq_fwht(0x10, tq.TQ_F32, big, 128, 0x10, None) == tq.TQ_ESHAPE
    assert lib.tq_fwht(0x10, tq.TQ_F32, 2, big, 0x10, None) == tq.TQ_ESHAPE


def test_offline_calls_check_alignment():
    lib = tq.lib()
    assert lib.tq_pack(0x10, 4, 20, 0, 3, 0x12, None) == tq.TQ_EINVAL             # words 4 bytes
    assert lib.tq_unpack(0x12, 4, 20, 0, 3, 0x10, None) == tq.TQ_EINVAL           # words 4 bytes
    assert lib.tq_quantize(0x14, tq.TQ_F64, 4, 128, 128, 3, 0x10, 0x10, None) == tq.TQ_EINVAL   # f64 8 bytes
    assert lib.tq_quantize(0x12, tq.TQ_F32, 4, 128, 128, 3, 0x10, 0x10, None) == tq.TQ_EINVAL   # f32 4 bytes
    assert lib.tq_quantize(0x10, tq.TQ_F32, 4, 128, 128, 3, 0x11, 0x10, None) == tq.TQ_EINVAL   # trits 2 bytes
    assert lib.tq_quantize(0x10, tq.TQ_F32, 4, 128, 128, 3, 0x10, 0x11, None) == tq.TQ_EINVAL   # scales 2 bytes
    assert lib.tq_pack_scales(0x11, 4, 128, 1, 128, 0x10, None) == tq.TQ_EINVAL
    assert lib.tq_pack_scales(0x10, 4, 128, 1, 128, 0x11, None) == tq.TQ_EINVAL
    assert lib.tq_moe_route(0x12, 1, 8, 2, 0x10, 0x10, None) == tq.TQ_EINVAL
    assert lib.tq_moe_route(0x10, 1, 8, 2, 0x12, 0x10, None) == tq.TQ_EINVAL
    assert lib.tq_moe_route(0x10, 1, 8, 2, 0x10, 0x13, None) == tq.TQ_EINVAL


def test_checking_calls_reject_bad_arguments():
    lib = tq.lib()
    assert lib.tq_pack_checked(0x10, 4, 20, 0, 3, 0x10, None, None) == tq.TQ_EINVAL
    assert lib.tq_pack_checked(0x10, 4, 20, 0, 3, 0x10, 0x22, None) == tq.TQ_EINVAL
    assert lib.tq_pack_checked(0x10, 0, 20, 0, 3, 0x10, 0x20, None) == tq.TQ_ESHAPE
    c = ctypes.c_int32(5)
    assert lib.tq_moe_bad_ids(None, 256, ctypes.byref(c), None) == tq.TQ_EINVAL
    assert lib.tq_moe_bad_ids(0x1008, 256, ctypes.byref(c), None) == tq.TQ_EINVAL
    assert lib.tq_moe_bad_ids(0x1000, 2, ctypes.byref(c), None) == tq.TQ_ENOSPACE
    assert lib.tq_moe_bad_ids(0x1000, 256, None, None) == tq.TQ_EINVAL
    assert lib.tq_strerror(tq.TQ_EDATA).decode().startswith("input values out of range")


def test_moe_rejects_variant_formats():
    """The expert path takes the ternary format at group 128 only."""
    d = lambda g, lv: tq.tq_weights(tq.TQ_MAGIC, tq.TQ_VERSION, 256, 512, 4, tq.TQ_LAYOUT_ROW64, g, lv, 0x1000, 0x2000)
    lib = tq.lib()
    for g, lv in ((64, 3), (128, 2)):
        gu, dn = d(g, lv), tq.tq_weights(tq.TQ_MAGIC, tq.TQ_VERSION, 512, 128, 4, tq.TQ_LAYOUT_ROW64, g, lv, 0x1000,
                                         0x2000)
        st = lib.tq_moe_gemv(tq.ctypes.byref(gu), tq.ctypes.byref(dn), 0x3000, tq.TQ_BF16, 1, 1, 0x4000, 0x5000, 0x6000,
                             tq.TQ_FWHT_FUSED, 0x7000, 1 << 24, None)
        assert st == tq.TQ_EUNSUPPORTED


def test_kv_calls_reject_bad_arguments():
    lib = tq.lib()
    A = 0x1000  # aligned stand-in address (nothing is launched)
    q = lambda **kw: lib.tq_kv_quantize(*[kw.get(k, v) for k, v in (
        ("x", A), ("dt", tq.TQ_BF16), ("n", 4), ("signs", A), ("jl", A), ("levels", A), ("bits", 3), ("keys", 1),
        ("stride", 1), ("rec", A), ("r", A), ("g", A), ("s", None))])
    assert q(x=None) == tq.TQ_EINVAL
    assert q(jl=None) == tq.TQ_EINVAL and q(g=None) == tq.TQ_EINVAL          # keys need S and gamma
    assert q(dt=tq.TQ_F64) == tq.TQ_EINVAL
    assert q(bits=1) == tq.TQ_EINVAL and q(bits=9) == tq.TQ_EINVAL           # keys: 2..8
    assert q(rec=A + 4) == tq.TQ_EINVAL and q(levels=A + 4) == tq.TQ_EINVAL and q(x=A + 2) == tq.TQ_EINVAL
    assert q(n=-1) == tq.TQ_ESHAPE and q(stride=0) == tq.TQ_ESHAPE
    assert q(n=0) == tq.TQ_OK                                                  # no-op, nothing launched
    sc = lambda **kw: lib.tq_kv_scores(*[kw.get(k, v) for k, v in (
        ("q", A), ("h", 2), ("nq", 2), ("keys", A), ("r", A), ("g", A), ("n", 100), ("bits", 3), ("signs", A),
        ("jl", A), ("levels", A), ("out", A), ("ws", A), ("wsb", 1 << 20), ("s", None))])
    assert sc(keys=None) == tq.TQ_EINVAL and sc(bits=1) == tq.TQ_EINVAL and sc(keys=A + 8) == tq.TQ_EINVAL
    assert sc(h=0) == tq.TQ_ESHAPE and sc(h=300, nq=300) == tq.TQ_ESHAPE
    assert sc(wsb=tq.tq_kv_workspace(tq.TQ_KV_OP_SCORES, 100, 2, 2) - 1) == tq.TQ_ENOSPACE
    assert sc(n=0) == tq.TQ_OK
    va = lambda **kw: lib.tq_kv_values(*[kw.get(k, v) for k, v in (
        ("p", A), ("h", 2), ("nq", 2), ("vals", A), ("r", A), ("n", 100), ("bits", 3), ("signs", A),
        ("levels", A), ("out", A), ("ws", A), ("wsb", 1 << 20), ("s", None))])
    assert va(vals=None) == tq.TQ_EINVAL and va(bits=0) == tq.TQ_EINVAL and va(out=A + 4) == tq.TQ_EINVAL
    assert va(wsb=tq.tq_kv_workspace(tq.TQ_KV_OP_VALUES, 100, 2, 2) - 1) == tq.TQ_ENOSPACE
    at = lambda **kw: lib.tq_kv_attend(*[kw.get(k, v) for k, v in (
        ("s", A), ("scale", 0.125), ("h", 2), ("nq", 2), ("vals", A), ("r", A), ("n", 100), ("bits", 3),
        ("signs", A), ("levels", A), ("out", A), ("ws", A), ("wsb", 1 << 20), ("st", None))])
    assert at(s=None) == tq.TQ_EINVAL and at(bits=9) == tq.TQ_EINVAL and at(vals=A + 4) == tq.TQ_EINVAL
    assert at(scale=float("nan")) == tq.TQ_EINVAL and at(scale=float("inf")) == tq.TQ_EINVAL
    assert at(h=0) == tq.TQ_ESHAPE and at(n=-1) == tq.TQ_ESHAPE and at(h=300, nq=300) == tq.TQ_ESHAPE
    # the attend workspace also holds a (maximum, sum) pair per partial vector
    vb, ab = (tq.tq_kv_workspace(op, 100, 2, 2) for op in (tq.TQ_KV_OP_VALUES, tq.TQ_KV_OP_ATTEND))
    assert ab > vb and at(wsb=ab - 1) == tq.TQ_ENOSPACE
    assert lib.tq_kv_workspace(tq.TQ_KV_OP_SCORES, 10, 0, 1) == tq.SIZE_MAX
    assert lib.tq_kv_workspace(7, 10, 1, 1) == tq.SIZE_MAX
    assert [tq.tq_kv_record_bytes(b) for b in (0, 1, 3, 8, 9)] == [0, 16, 48, 128, 0]
    buf = (ctypes.c_double * 512)()
    assert lib.tq_kv_codebook(0, buf) == tq.TQ_EINVAL and lib.tq_kv_codebook(9, buf) == tq.TQ_EINVAL


@pytest.mark.parametrize("bits", range(1, 9))
def test_kv_codebook_matches_oracle(bits):
    """The library's codebook (its own Newton solve on the positive half) is
    the oracle's Lloyd-Max fixed point, exactly symmetric."""
    from oracle import kv_oracle as K
    got = tq.tq_kv_codebook(bits)
    want = K.codebook(bits)
    assert got.shape == want.shape
    assert abs(got - want).max() <= 1e-12 * abs(want).max()
    assert (got == -got[::-1]).all() and (got[1:] > got[:-1]).all()
