"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

This module holds NO arithmetic of the method (no rotation, ternarisation,
packing, transform or matvec): only random draws, the rounding of
activations to their storage dtype, and the workload shapes and seeds.
Both sides receive the same arrays from here.

Weights follow the workload recipe: N(0, 0.02^2) drawn row-major, then an
outlier mask drawn from the same generator (Bernoulli 0.001 per entry) whose
entries are multiplied by 20 (sign kept).  Activations are N(0, 1), stored
as fp32 or rounded to bf16 (round-to-nearest-even from fp32).  Router
logits are N(0, 1) fp32.  Expert weights use one generator per expert,
seeded by the sequence (4, e).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def _gen(seed) -> np.random.Generator:
    if isinstance(seed, (tuple, list)):
        return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(seed))))
    return np.random.Generator(np.random.PCG64(seed))


def weights(seed, n: int, k: int, std: float = 0.02, outlier_p: float = 0.001,
            outlier_mult: float = 20.0) -> np.ndarray:
    """float64 [n][k]: Gaussian weights with sparse x20 outliers."""
    g = _gen(seed)
    w = g.normal(0.0, std, size=(n, k))
    mask = g.random((n, k)) < outlier_p
    w[mask] *= outlier_mult
    return w


def expert_weights(e: int, hidden: int, inter: int):
    """(w_gate_up float64 [2*inter][hidden], w_down float64 [hidden][inter]) for
    expert e; gate rows first, then up rows."""
    g = _gen((4, e))
    out = []
    for n, k in ((2 * inter, hidden), (hidden, inter)):
        w = g.normal(0.0, 0.02, size=(n, k))
        mask = g.random((n, k)) < 0.001
        w[mask] *= 20.0
        out.append(w)
    return out[0], out[1]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns of float32 values, round-to-nearest-even."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


def f16_bits(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float16).view(np.uint16)


@dataclass
class Activations:
    """values: float64 copy of exactly what the device sees; raw: the device
    array (float32, or uint16 bit patterns for bf16/f16); dtype name."""
    values: np.ndarray
    raw: np.ndarray
    dtype: str


def activations(seed, m: int, k: int, dtype: str = "bf16", scale: float = 1.0) -> Activations:
    """N(0, scale^2) activations, rounded to `dtype`."""
    g = _gen(seed)
    x = (g.standard_normal((m, k)) * scale).astype(np.float32)
    if dtype == "f32":
        return Activations(x.astype(np.float64), x, "f32")
    if dtype == "bf16":
        bits = bf16_bits(x)
        return Activations(bf16_to_f32(bits).astype(np.float64), bits, "bf16")
    if dtype == "f16":
        h = x.astype(np.float16)
        return Activations(h.astype(np.float64), h.view(np.uint16), "f16")
    raise ValueError(dtype)


def logits(seed, t: int, e: int) -> np.ndarray:
    return _gen(seed).standard_normal((t, e)).astype(np.float32)


def trits(seed, n: int, k: int, p_zero: float = 0.31) -> np.ndarray:
    """Random trits (int8 in {-1,0,1}) for kernel-level tests."""
    g = _gen(seed)
    u = g.random((n, k))
    t = np.where(u < p_zero, 0, np.where(u < (1 + p_zero) / 2, -1, 1))
    return t.astype(np.int8)


def trits_uniform(seed, n: int, k: int) -> np.ndarray:
    """Trits uniform over {-1, 0, 1} (int8), drawn as bytes: cheap at the
    full decode shapes (hundreds of millions of trits)."""
    return (_gen(seed).integers(0, 3, size=(n, k), dtype=np.int8) - np.int8(1)).astype(np.int8)


def scales(seed, n: int, groups: int, lo: float = 0.005, hi: float = 0.03) -> np.ndarray:
    """Random fp16 scales for kernel-level tests."""
    return _gen(seed).uniform(lo, hi, size=(n, groups)).astype(np.float16)


# ---------------------------------------------------------------------------
# Workloads (shapes and seeds)
# ---------------------------------------------------------------------------
@dataclass
class Linear:
    name: str
    n: int
    k: int
    w_seed: object
    x_seed: object


@dataclass
class Workload:
    name: str
    m: int
    x_dtype: str
    linears: list = field(default_factory=list)


SINGLE_LINEAR = Workload("linear-512x1024-m1", 1, "f32",
                         [Linear("w", 512, 1024, 1001, 1002)])

DENSE_DECODE_27B = Workload("dense-27b-decode-up-down-m1", 1, "bf16", [
    Linear("up", 17408, 5120, 2001, 2003),
    Linear("down", 5120, 17408, 2002, 2004),
])

# One dense 27B-class decoder block's linears; q, k, v share the attention
# input, gate and up the MLP input.
BLOCK_LINEARS = [
    Linear("q", 5120, 5120, 3001, 3010),
    Linear("k", 1024, 5120, 3002, 3010),
    Linear("v", 1024, 5120, 3003, 3010),
    Linear("o", 5120, 5120, 3004, 3011),
    Linear("gate", 17408, 5120, 3005, 3012),
    Linear("up", 17408, 5120, 3006, 3012),
    Linear("down", 5120, 17408, 3007, 3013),
]
DENSE_BLOCK_M8 = Workload("dense-27b-block-m8", 8, "bf16", BLOCK_LINEARS)
DENSE_BLOCK_M1 = Workload("dense-27b-block-m1", 1, "bf16", BLOCK_LINEARS)  # single-stream decode

@dataclass
class MoEWorkload:
    name: str
    tokens: int
    experts: int = 256
    topk: int = 8
    hidden: int = 2048
    inter: int = 512
    logit_seed: int = 4901
    x_seed: int = 4902


MOE_T1 = MoEWorkload("moe-256x-top8-h2048-i512-t1", 1, logit_seed=4901, x_seed=4902)
MOE_T64 = MoEWorkload("moe-256x-top8-h2048-i512-t64", 64, logit_seed=4903, x_seed=4904)

PREFILL_GEMM = Workload("prefill-gemm-2048x5120x17408", 2048, "bf16",
                        [Linear("up", 17408, 5120, 5001, 5002)])


# ---------------------------------------------------------------------------
# KV-cache quantiser inputs: the random rotation's sign flips and the
# Johnson-Lindenstrauss projection matrix are random draws of the method,
# passed to both sides as inputs.
# ---------------------------------------------------------------------------
def kv_signs(seed, d: int = 128) -> np.ndarray:
    """Random +-1 (float32) of the KV rotation."""
    return np.where(_gen(seed).random(d) < 0.5, -1.0, 1.0).astype(np.float32)


def kv_jl(seed, d: int = 128) -> np.ndarray:
    """d x d projection matrix with N(0, 1) entries (float32, row-major)."""
    return _gen(seed).standard_normal((d, d)).astype(np.float32)


def kv_vectors(seed, n: int, d: int = 128, dtype: str = "bf16") -> Activations:
    """n K or V rows of N(0, 1) with a per-row scale drawn log-uniformly in
    [0.25, 4] (rows of different norms, as keys and values of real layers)."""
    g = _gen(seed)
    x = (g.standard_normal((n, d)) * np.exp(g.uniform(np.log(0.25), np.log(4.0), size=(n, 1)))).astype(np.float32)
    if dtype == "f32":
        return Activations(x.astype(np.float64), x, "f32")
    bits = bf16_bits(x)
    return Activations(bf16_to_f32(bits).astype(np.float64), bits, "bf16")


@dataclass
class KVWorkload:
    """Decode attention over a quantised KV cache: `tokens` cached K and V
    vectors (d = 128) for each of `heads` KV heads, `queries` query heads per
    KV head, `bits` bits per coordinate for keys and for values."""
    name: str
    tokens: int
    heads: int
    queries: int
    bits: int
    key_seed: int
    value_seed: int
    query_seed: int
    sign_seed: int
    jl_seed: int


# 128K context at 3 bits (the oMLX/Gemma page's long-context case), 8 KV
# heads with 4 query heads each.
KV_DECODE_128K = KVWorkload("kv-decode-128k-h8-g4-3bit", 131072, 8, 4, 3, 6001, 6002, 6003, 6004, 6005)
KV_SMALL = KVWorkload("kv-small-3000-h2-g3-3bit", 3000, 2, 3, 3, 6101, 6102, 6103, 6104, 6105)
