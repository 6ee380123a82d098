"""Python binding of libtq.so (the ternary-weight packed GEMV library).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/tq.h.  PyTorch supplies device
memory and streams.  The entry points keep the C names and argument order;
tensors are passed by pointer, and a negative status raises TQError.  There
is no CPU fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "tq.h")

TQ_MAGIC = 0x30325154
TQ_VERSION = 2
TQ_TRITS_PER_WORD = 20
TQ_GROUP = 128
TQ_BITS_PER_WORD = 32
TQ_MAX_DIM = 1 << 30
TQ_OK, TQ_EINVAL, TQ_ESHAPE, TQ_EFORMAT, TQ_ENOSPACE, TQ_EHIP, TQ_EUNSUPPORTED, TQ_EDATA = 0, -1, -2, -3, -4, -5, -6, -7
TQ_F32, TQ_BF16, TQ_F16, TQ_F64 = 0, 1, 2, 3
TQ_LAYOUT_ROWMAJOR, TQ_LAYOUT_ROW64 = 0, 1
TQ_FWHT_FUSED = 1
TQ_ACCUMULATE = 2
TQ_MOE_ONE_LAUNCH = 4
TQ_FAST_F16 = 8
TQ_OP_GEMV, TQ_OP_MOE, TQ_OP_GEMM = 0, 1, 2
TQ_KV_DIM = 128
TQ_KV_MAX_BITS = 8
TQ_KV_OP_SCORES, TQ_KV_OP_VALUES, TQ_KV_OP_ATTEND = 0, 1, 2
SIZE_MAX = 2 ** 64 - 1


class TQError(RuntimeError):
    def __init__(self, func: str, status: int, message: str):
        super().__init__(f"{func}: {message} (status {status})")
        self.status = status


class tq_weights(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint32), ("version", ctypes.c_uint32), ("n", ctypes.c_int32),
                ("k", ctypes.c_int32), ("num_experts", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("group", ctypes.c_int32), ("levels", ctypes.c_int32),
                ("words", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_I64 = ctypes.c_int64
_W = ctypes.POINTER(tq_weights)
_SIGNATURES = {
    "tq_words_per_row": (_SZ, [_I]),
    "tq_packed_bytes": (_SZ, [_I, _I]),
    "tq_format_bytes": (_SZ, [_I, _I, _I, _I]),
    "tq_layout_words": (_SZ, [_I, _I, _I, _I]),
    "tq_layout_scales": (_SZ, [_I, _I, _I, _I]),
    "tq_quantize": (_I, [_P, _I, _I, _I, _I, _I, _P, _P, _P]),
    "tq_pack": (_I, [_P, _I, _I, _I, _I, _P, _P]),
    "tq_pack_checked": (_I, [_P, _I, _I, _I, _I, _P, _P, _P]),
    "tq_moe_bad_ids": (_I, [_P, _SZ, ctypes.POINTER(ctypes.c_int32), _P]),
    "tq_pack_scales": (_I, [_P, _I, _I, _I, _I, _P, _P]),
    "tq_unpack": (_I, [_P, _I, _I, _I, _I, _P, _P]),
    "tq_fwht": (_I, [_P, _I, _I, _I, _P, _P]),
    "tq_gemv": (_I, [_W, _P, _I, _I, _P, ctypes.c_uint, _P, _SZ, _P]),
    "tq_gemv_noalloc": (_I, [_W, _P, _I, _I, _P, ctypes.c_uint, _P]),
    "tq_moe_route": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "tq_moe_gemv": (_I, [_W, _W, _P, _I, _I, _I, _P, _P, _P, ctypes.c_uint, _P, _SZ, _P]),
    "tq_gemm": (_I, [_W, _P, _I, _I, _P, ctypes.c_uint, _P, _SZ, _P]),
    "tq_workspace_bytes": (_SZ, [_I, _W, _I, _I]),
    "tq_read_bytes": (_I, [_P, _SZ, _P, _P]),
    "tq_kv_codebook": (_I, [_I, ctypes.POINTER(ctypes.c_double)]),
    "tq_kv_record_bytes": (_SZ, [_I]),
    "tq_kv_quantize": (_I, [_P, _I, _I64, _P, _P, _P, _I, _I, _I64, _P, _P, _P, _P]),
    "tq_kv_workspace": (_SZ, [_I, _I64, _I, _I]),
    "tq_kv_scores": (_I, [_P, _I, _I, _P, _P, _P, _I64, _I, _P, _P, _P, _P, _P, _SZ, _P]),
    "tq_kv_values": (_I, [_P, _I, _I, _P, _P, _I64, _I, _P, _P, _P, _P, _SZ, _P]),
    "tq_kv_attend": (_I, [_P, ctypes.c_float, _I, _I, _P, _P, _I64, _I, _P, _P, _P, _P, _SZ, _P]),
    "tq_strerror": (ctypes.c_char_p, [_I]),
    "tq_last_error": (ctypes.c_char_p, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libtq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "or python ternary_weight_quantized_tq_amd/build.py")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/tq.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z0-9_]+)\s*\(", text)))


# ------------------------------------------------------------- helpers ---
def _ptr(t) -> int | None:
    """Device address of a tensor (or a raw address passed as int).  Host
    tensors and non-contiguous views are refused: the kernels read device
    memory densely."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError(f"tensor on {t.device}: the library reads device memory only")
    if not t.is_contiguous():
        raise ValueError("non-contiguous tensor: pass a contiguous one")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(name: str, st: int) -> int:
    if st != TQ_OK:
        msg = tq_strerror(st)
        if st == TQ_EHIP:
            msg += ": " + tq_last_error()
        raise TQError(name, st, msg)
    return st


def dtype_code(t) -> int:
    import torch
    return {torch.float32: TQ_F32, torch.bfloat16: TQ_BF16, torch.float16: TQ_F16,
            torch.float64: TQ_F64}[t.dtype]


# ----------------------------------------------------------- sizes ---
def tq_words_per_row(k: int) -> int:
    return lib().tq_words_per_row(k)


def tq_packed_bytes(n: int, k: int) -> int:
    return lib().tq_packed_bytes(n, k)


def tq_format_bytes(n: int, k: int, group: int, levels: int) -> int:
    return lib().tq_format_bytes(n, k, group, levels)


def tq_layout_words(n: int, k: int, layout: int, levels: int) -> int:
    return lib().tq_layout_words(n, k, layout, levels)


def tq_layout_scales(n: int, k: int, layout: int, group: int) -> int:
    return lib().tq_layout_scales(n, k, layout, group)


def tq_strerror(status: int) -> str:
    return lib().tq_strerror(status).decode()


def tq_last_error() -> str:
    return lib().tq_last_error().decode()


# --------------------------------------------------- entry points ---
def tq_quantize(w, n, k, group, levels, trits, scales, stream=None):
    return _check("tq_quantize", lib().tq_quantize(_ptr(w), dtype_code(w), n, k, group, levels, _ptr(trits),
                                                   _ptr(scales), _stream(stream)))


def tq_pack(trits, n, k, layout, levels, words, stream=None):
    return _check("tq_pack", lib().tq_pack(_ptr(trits), n, k, layout, levels, _ptr(words), _stream(stream)))


def tq_pack_checked(trits, n, k, layout, levels, words, bad, stream=None):
    """tq_pack plus the count of input values outside the format's set
    written to `bad` (a one-element int32 device tensor)."""
    return _check("tq_pack_checked", lib().tq_pack_checked(_ptr(trits), n, k, layout, levels, _ptr(words),
                                                           _ptr(bad), _stream(stream)))


def tq_moe_bad_ids(workspace, ws_bytes, stream=None) -> int:
    """Number of expert ids outside [0, E) seen by the last tq_moe_gemv on
    this workspace (waits for the stream).  Returns the count; TQ_EDATA is
    not raised here, it is what a nonzero count means."""
    c = ctypes.c_int32(0)
    st = lib().tq_moe_bad_ids(_ptr(workspace), ws_bytes, ctypes.byref(c), _stream(stream))
    if st not in (TQ_OK, TQ_EDATA):
        _check("tq_moe_bad_ids", st)
    return int(c.value)


def tq_pack_scales(scales, n, k, layout, group, scales_out, stream=None):
    return _check("tq_pack_scales", lib().tq_pack_scales(_ptr(scales), n, k, layout, group, _ptr(scales_out),
                                                         _stream(stream)))


def tq_unpack(words, n, k, layout, levels, trits, stream=None):
    return _check("tq_unpack", lib().tq_unpack(_ptr(words), n, k, layout, levels, _ptr(trits), _stream(stream)))


def tq_fwht(x, m, k, x_rot, stream=None):
    return _check("tq_fwht", lib().tq_fwht(_ptr(x), dtype_code(x), m, k, _ptr(x_rot), _stream(stream)))


def tq_gemv(w, x, m, y, flags=TQ_FWHT_FUSED, workspace=None, ws_bytes=0, stream=None):
    return _check("tq_gemv", lib().tq_gemv(ctypes.byref(_desc(w)), _ptr(x), dtype_code(x), m, _ptr(y), flags,
                                           _ptr(workspace), ws_bytes, _stream(stream)))


def tq_gemv_noalloc(w, x, m, y, flags=TQ_FWHT_FUSED, stream=None):
    return _check("tq_gemv_noalloc", lib().tq_gemv_noalloc(ctypes.byref(_desc(w)), _ptr(x), dtype_code(x), m,
                                                           _ptr(y), flags, _stream(stream)))


def tq_moe_route(logits, t, e, topk, ids, weights, stream=None):
    return _check("tq_moe_route", lib().tq_moe_route(_ptr(logits), t, e, topk, _ptr(ids), _ptr(weights),
                                                     _stream(stream)))


def tq_moe_gemv(w_gate_up, w_down, x, t, topk, expert_ids, route_w, y, flags=TQ_FWHT_FUSED,
                workspace=None, ws_bytes=0, stream=None):
    return _check("tq_moe_gemv", lib().tq_moe_gemv(
        ctypes.byref(_desc(w_gate_up)), ctypes.byref(_desc(w_down)), _ptr(x), dtype_code(x), t, topk,
        _ptr(expert_ids), _ptr(route_w), _ptr(y), flags, _ptr(workspace), ws_bytes, _stream(stream)))


def tq_gemm(w, x, m, y, flags=TQ_FWHT_FUSED, workspace=None, ws_bytes=0, stream=None):
    return _check("tq_gemm", lib().tq_gemm(ctypes.byref(_desc(w)), _ptr(x), dtype_code(x), m, _ptr(y), flags,
                                           _ptr(workspace), ws_bytes, _stream(stream)))


def tq_read_bytes(src, nbytes, sink, stream=None):
    """Measurement aid: one plain read pass over nbytes of src."""
    return _check("tq_read_bytes", lib().tq_read_bytes(_ptr(src), nbytes, _ptr(sink), _stream(stream)))


def tq_kv_codebook(bits) -> "numpy.ndarray":
    """The 2^bits codebook levels (host float64 array)."""
    import numpy as np
    buf = (ctypes.c_double * (1 << TQ_KV_MAX_BITS))()
    _check("tq_kv_codebook", lib().tq_kv_codebook(bits, buf))
    return np.array(buf[:1 << bits], dtype=np.float64)


def tq_kv_record_bytes(bits) -> int:
    return lib().tq_kv_record_bytes(bits)


def tq_kv_quantize(x, n, signs, jl, levels, bits, keys, records, radius, gamma=None, stride=1, stream=None):
    return _check("tq_kv_quantize", lib().tq_kv_quantize(
        _ptr(x), dtype_code(x), n, _ptr(signs), _ptr(jl), _ptr(levels), bits, int(bool(keys)), stride,
        _ptr(records), _ptr(radius), _ptr(gamma), _stream(stream)))


def tq_kv_workspace(op, n, heads, nq) -> int:
    return lib().tq_kv_workspace(op, n, heads, nq)


def tq_kv_scores(q, heads, nq, keys, radius, gamma, n, bits, signs, jl, levels, scores, workspace, ws_bytes,
                 stream=None):
    return _check("tq_kv_scores", lib().tq_kv_scores(
        _ptr(q), heads, nq, _ptr(keys), _ptr(radius), _ptr(gamma), n, bits, _ptr(signs), _ptr(jl), _ptr(levels),
        _ptr(scores), _ptr(workspace), ws_bytes, _stream(stream)))


def tq_kv_values(p, heads, nq, values, radius, n, bits, signs, levels, out, workspace, ws_bytes, stream=None):
    return _check("tq_kv_values", lib().tq_kv_values(
        _ptr(p), heads, nq, _ptr(values), _ptr(radius), n, bits, _ptr(signs), _ptr(levels), _ptr(out),
        _ptr(workspace), ws_bytes, _stream(stream)))


def tq_kv_attend(scores, scale, heads, nq, values, radius, n, bits, signs, levels, out, workspace, ws_bytes,
                 stream=None):
    return _check("tq_kv_attend", lib().tq_kv_attend(
        _ptr(scores), float(scale), heads, nq, _ptr(values), _ptr(radius), n, bits, _ptr(signs), _ptr(levels),
        _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)))


def kv_workspace(op, n, heads, nq, device="cuda"):
    """Workspace of the size tq_kv_scores / tq_kv_values / tq_kv_attend needs."""
    import torch
    nbytes = tq_kv_workspace(op, n, heads, nq)
    if nbytes == SIZE_MAX:
        raise TQError("tq_kv_workspace", TQ_EINVAL, "invalid request")
    return torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device), nbytes


def tq_workspace_bytes(op, w, m_or_t, topk=0) -> int:
    return lib().tq_workspace_bytes(op, ctypes.byref(_desc(w)), m_or_t, topk)


# ------------------------------------------------ weight containers ---
@dataclass
class Weights:
    """Device buffers of one packed matrix (or E experts) and its shape."""
    words: object       # torch.int32 tensor holding uint32 words
    scales: object      # torch.int16 tensor holding fp16 bits
    n: int
    k: int
    layout: int = TQ_LAYOUT_ROW64
    num_experts: int = 1
    group: int = TQ_GROUP
    levels: int = 3
    magic: int = TQ_MAGIC
    version: int = TQ_VERSION

    def desc(self) -> tq_weights:
        return tq_weights(self.magic, self.version, self.n, self.k, self.num_experts, self.layout, self.group,
                          self.levels, _ptr(self.words), _ptr(self.scales))

    def clone(self) -> "Weights":
        return Weights(self.words.clone(), self.scales.clone(), self.n, self.k, self.layout, self.num_experts,
                       self.group, self.levels)


def _desc(w) -> tq_weights:
    return w if isinstance(w, tq_weights) else w.desc()


def empty_weights(n, k, layout=TQ_LAYOUT_ROW64, num_experts=1, device="cuda", group=TQ_GROUP,
                  levels=3) -> Weights:
    import torch
    nw = tq_layout_words(n, k, layout, levels)
    ns = tq_layout_scales(n, k, layout, group)
    return Weights(torch.empty(num_experts * nw, dtype=torch.int32, device=device),
                   torch.empty(num_experts * ns, dtype=torch.int16, device=device), n, k, layout, num_experts,
                   group, levels)


def workspace(op, w, m_or_t, topk=0, device="cuda"):
    """Zero-filled workspace of the size the operation needs (may be empty)."""
    import torch
    nbytes = tq_workspace_bytes(op, w, m_or_t, topk)
    if nbytes == SIZE_MAX:
        raise TQError("tq_workspace_bytes", TQ_EINVAL, "invalid request")
    return torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device), nbytes
