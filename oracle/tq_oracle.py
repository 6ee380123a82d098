"""Plain CPU oracle for the ternary-weight (1.58-bit) packed matvec path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, tables, constants or helpers) and imports
nothing from the package; the seeded input generators in ``synth/`` are the
only thing both sides consume.

Everything is computed in FP64 (integers exactly) straight from the
definitions, in the order the pages give the method:

  offline:  W  -> W' = W . H_B          (block-128 Hadamard along K)
               -> per group of 128: gamma = mean|W'|, t in {-1,0,+1},
                  s = fp16(gamma)
               -> base-3 pack, 20 trits per uint32
  online:   x  -> x' = H_B . x          (the matching transform)
               -> y = sum_k s[n][k/128] * t[n][k] * x'[k]

Sources (web pages; cited by title and section):

* [TQ-MLX]  "16GB Mac runs Qwen3.6-35B-A3B: the TurboQuant-MLX 1.58-bit
  build" (tantan.ink/?p=490).  Section "Why 1.58 bit did not turn into
  gibberish": weights take one of three values -c, 0, +c; only the routed
  experts (256, top-8 per token) are ternary while the router gate stays at
  full precision (point 1); base-3 coding puts 20 ternary indices in one
  32-bit integer, about 1.6 bits per weight (point 3).
* [Bonsai]  "27B model in 5.9 GB: ternary quantization, why does it not
  collapse?" (cosmocat.dev).  Section 2 (1) "flatten first, then compress":
  a Hadamard rotation is applied to the weights before compression, it is an
  orthogonal change of basis, and a matching fast transform costing
  O(n log n) undoes it at inference.  Section 2 (2) "a ruler for every 128
  weights": 128 weights share one FP16 scale that restores the magnitude.
  Section 2 (3): kernels compute on the packed format directly.
* [GSQ-cmp] "Ternary-Bonsai2-27B vs Qwen3.8-27B-GSQ-RCO" (nxmr.cn), §1.1:
  with weights in {-1,0,1} times a scale the matmul reduces to sign tests
  and additions/subtractions.

Readings where the pages are silent:

* scale estimator: absmean, gamma = mean |w'| over the group (the BitNet
  b1.58 rule; BitNet is named as the lineage in [Bonsai] section 1);
* threshold: t = sign(w') if |w'| > gamma/2 else 0 (exact tie -> 0);
* stored scale: fp16 round-to-nearest-even of gamma in ONE rounding from
  FP64; the threshold uses the unrounded gamma; gamma == 0 -> t = 0, s = 0;
* digit d = t + 1; trit k of a row is base-3 digit (k mod 20) of word
  floor(k / 20) (little-endian); rows are packed contiguously, so words may
  straddle group boundaries; the row tail is padded with t = 0 (digit 1);
* Hadamard: Sylvester, natural order, normalised by 1/sqrt(128), no random
  sign diagonal; rotation blocks coincide with the scale groups;
* group size: 128 ([Bonsai] section 2 (2)); 64 as the finer-scale variant
  that [TQ-MLX]'s model id ("...-g64") hints at.  The rotation stays
  block-128 either way: only the scale granularity changes;
* binary variant ([TQ-MLX] point 3, pure 1-bit {-c, +c}): the same rotation
  and absmean scale, t = +1 where w' >= 0 else -1, 32 signs per uint32
  (bit i of word w is weight 32w + i, 1 for +1);
* MoE: softmax over all expert logits, top-k (ties to the lower id), weights
  renormalised to sum 1; expert MLP is SwiGLU, h = silu(gate) * up, and the
  block-128 transform is applied to h before the down projection.

Parity status: every function here is pinned by ``tests/test_oracle.py``
against closed forms, page constants, library routines or brute force.
"""
from __future__ import annotations

import numpy as np

TRITS_PER_WORD = 20          # [TQ-MLX] point 3
GROUP = 128                  # [Bonsai] section 2 (2)
HBLOCK = 128                 # rotation block = scale group (reading)
POW3 = [3 ** i for i in range(TRITS_PER_WORD + 1)]


# --------------------------------------------------------------------------
# Hadamard matrix and the block transform  ([Bonsai] section 2 (1))
# --------------------------------------------------------------------------
def hadamard(n: int = HBLOCK) -> np.ndarray:
    """Dense Sylvester Hadamard matrix of order n (a power of two), scaled by
    1/sqrt(n): H[i][j] = (-1)^popcount(i & j) / sqrt(n)."""
    if n <= 0 or n & (n - 1):
        raise ValueError("n must be a power of two")
    h = np.empty((n, n), dtype=np.float64)
    for i in range(n):
        for j in range(n):
            h[i, j] = -1.0 if bin(i & j).count("1") % 2 else 1.0
    return h / np.sqrt(float(n))


_H_CACHE: dict[int, np.ndarray] = {}


def _h(n: int) -> np.ndarray:
    if n not in _H_CACHE:
        _H_CACHE[n] = hadamard(n)
    return _H_CACHE[n]


def block_transform(a: np.ndarray, block: int = HBLOCK) -> np.ndarray:
    """Apply H along the last axis, independently on each aligned block:
    out[..., block*b + j] = sum_i a[..., block*b + i] * H[i][j].

    Used both for the offline weight rotation W' = W . H_B and the online
    activation transform x' = H_B . x (H is symmetric, so the two coincide).
    Dense product per block in FP64: the plain definition that the fast
    O(n log n) butterfly reaches faster."""
    a = np.asarray(a, dtype=np.float64)
    k = a.shape[-1]
    if k % block:
        raise ValueError("last dimension must be a multiple of the block")
    h = _h(block)
    blocks = a.reshape(a.shape[:-1] + (k // block, block))
    return (blocks @ h).reshape(a.shape)


def rotate_weights(w: np.ndarray) -> np.ndarray:
    """Offline rotation of W [N][K] along K ([Bonsai] section 2 (1))."""
    return block_transform(w)


def fwht(x: np.ndarray) -> np.ndarray:
    """Online transform of activations x [..][K] ([Bonsai] section 2 (1))."""
    return block_transform(x)


# --------------------------------------------------------------------------
# Ternarisation with a group FP16 scale  ([TQ-MLX] intro; [Bonsai] 2 (2))
# --------------------------------------------------------------------------
def ternarize(w_rot: np.ndarray, group: int = GROUP):
    """Per (row n, group g): gamma = mean |w'|, t = sign(w') where
    |w'| > gamma/2 else 0, s = fp16(gamma) rounded once from FP64.

    Returns (t int8 [N][K], s float16 [N][K/group], gamma float64 [N][K/group])."""
    w_rot = np.asarray(w_rot, dtype=np.float64)
    n, k = w_rot.shape
    if k % group:
        raise ValueError("K must be a multiple of the group size")
    g = w_rot.reshape(n, k // group, group)
    gamma = np.abs(g).mean(axis=2)
    thr = (gamma / 2.0)[:, :, None]
    t = np.zeros(g.shape, dtype=np.int8)
    t[g > thr] = 1
    t[g < -thr] = -1
    s = gamma.astype(np.float16)          # one RNE rounding from FP64
    return t.reshape(n, k), s, gamma


def quantize(w: np.ndarray, group: int = GROUP):
    """Offline conversion: rotate (blocks of 128), then ternarise per group
    of `group` weights (128, or 64 for the finer-scale variant). Returns
    (t, s, gamma)."""
    return ternarize(rotate_weights(w), group)


# --------------------------------------------------------------------------
# Binary {-c, +c} variant  ([TQ-MLX] point 3: pure 1-bit experts, only -c and
# +c, compared against ternary)
# --------------------------------------------------------------------------
def binarize(w_rot: np.ndarray, group: int = GROUP):
    """Per (row n, group g): gamma = mean |w'| (for signs this is also the
    least-squares scale, argmin_c sum (w' - c sign w')^2), t = +1 where
    w' >= 0 else -1 (no zero level; an exact 0 goes to +1), s = fp16(gamma)
    rounded once from FP64.  Returns (t int8, s float16, gamma float64)."""
    w_rot = np.asarray(w_rot, dtype=np.float64)
    n, k = w_rot.shape
    if k % group:
        raise ValueError("K must be a multiple of the group size")
    g = w_rot.reshape(n, k // group, group)
    gamma = np.abs(g).mean(axis=2)
    t = np.where(g >= 0.0, 1, -1).astype(np.int8)
    return t.reshape(n, k), gamma.astype(np.float16), gamma


def quantize_binary(w: np.ndarray, group: int = GROUP):
    """Offline conversion of the binary variant: rotate, then binarise."""
    return binarize(rotate_weights(w), group)


BITS_PER_WORD = 32


def words_per_row_binary(k: int) -> int:
    return -(-k // BITS_PER_WORD)


def pack_binary(t: np.ndarray) -> np.ndarray:
    """word[n][w] = sum_{i<32} b[n][32w+i] 2^i with b = 1 for +1, 0 for -1;
    bits past K are 0."""
    t = np.asarray(t)
    n, k = t.shape
    if t.size and not np.all((t == 1) | (t == -1)):
        raise ValueError("binary weights must be -1 or +1")
    nw = words_per_row_binary(k)
    bits = np.zeros((n, nw * BITS_PER_WORD), dtype=np.uint64)
    bits[:, :k] = (t > 0).astype(np.uint64)
    bits = bits.reshape(n, nw, BITS_PER_WORD)
    acc = np.zeros((n, nw), dtype=np.uint64)
    for i in range(BITS_PER_WORD):
        acc += bits[:, :, i] * np.uint64(1 << i)
    return acc.astype(np.uint32)


def unpack_binary(words: np.ndarray, k: int) -> np.ndarray:
    """t[n][k] = 2 ((word[n][k // 32] // 2^(k mod 32)) mod 2) - 1."""
    words = np.asarray(words, dtype=np.int64)
    kk = np.arange(k)
    w = words[:, kk // BITS_PER_WORD]
    p = np.array([1 << int(i) for i in (kk % BITS_PER_WORD)], dtype=np.int64)
    return (2 * ((w // p) % 2) - 1).astype(np.int8)


def packed_bytes_binary(n: int, k: int, group: int = GROUP) -> int:
    """Bytes of 1-bit words plus fp16 scales: 4*N*ceil(K/32) + 2*N*K/group."""
    return 4 * n * words_per_row_binary(k) + 2 * n * (k // group)


# --------------------------------------------------------------------------
# Base-3 packing, 20 trits per uint32  ([TQ-MLX] point 3)
# --------------------------------------------------------------------------
def words_per_row(k: int) -> int:
    return -(-k // TRITS_PER_WORD)


def pack(t: np.ndarray) -> np.ndarray:
    """word[n][w] = sum_{i<20} (t[n][20w+i] + 1) * 3^i, with t = 0 beyond K."""
    t = np.asarray(t)
    n, k = t.shape
    if t.size and (t.min() < -1 or t.max() > 1):
        raise ValueError("trits must be in {-1, 0, 1}")
    nw = words_per_row(k)
    digits = np.ones((n, nw * TRITS_PER_WORD), dtype=np.uint64)   # pad t=0
    digits[:, :k] = (t.astype(np.int64) + 1).astype(np.uint64)
    digits = digits.reshape(n, nw, TRITS_PER_WORD)
    acc = np.zeros((n, nw), dtype=np.uint64)
    for i in range(TRITS_PER_WORD):
        acc += digits[:, :, i] * np.uint64(POW3[i])
    if acc.size and int(acc.max()) >= POW3[TRITS_PER_WORD]:
        raise AssertionError("packed word out of range")
    return acc.astype(np.uint32)


def unpack(words: np.ndarray, k: int) -> np.ndarray:
    """t[n][k] = ((word[n][k // 20] // 3^(k mod 20)) mod 3) - 1, plain / and %."""
    words = np.asarray(words, dtype=np.int64)
    n = words.shape[0]
    kk = np.arange(k)
    w = words[:, kk // TRITS_PER_WORD]
    p = np.array([POW3[i] for i in (kk % TRITS_PER_WORD)], dtype=np.int64)
    return ((w // p) % 3 - 1).astype(np.int8)


def packed_bytes(n: int, k: int, group: int = GROUP) -> int:
    """Bytes of words plus fp16 scales: 4*N*ceil(K/20) + 2*N*K/group."""
    return 4 * n * words_per_row(k) + 2 * n * (k // group)


# --------------------------------------------------------------------------
# Dequantised matvec on packed weights  ([Bonsai] 2 (2)(3); [GSQ-cmp] §1.1)
# --------------------------------------------------------------------------
def dequantize(words: np.ndarray, scales: np.ndarray, k: int, group: int = GROUP,
               levels: int = 3) -> np.ndarray:
    """W_hat[n][k] = fp64(s[n][k // group]) * t[n][k]  (FP64, dense, [N][K]);
    t from base-3 words (levels 3) or 1-bit words (levels 2)."""
    t = (unpack(words, k) if levels == 3 else unpack_binary(words, k)).astype(np.float64)
    s = np.asarray(scales).astype(np.float64)
    return t * np.repeat(s, group, axis=1)[:, :k]


def matvec(words, scales, k, x_rot, group: int = GROUP, levels: int = 3) -> np.ndarray:
    """y[m][n] = sum_k s[n][k/group] t[n][k] x'[m][k] for x' already rotated."""
    x_rot = np.atleast_2d(np.asarray(x_rot, dtype=np.float64))
    return x_rot @ dequantize(words, scales, k, group, levels).T


def gemv(words, scales, k, x, fused_fwht: bool = True, group: int = GROUP, levels: int = 3) -> np.ndarray:
    """Online path: x -> (optional) block-128 transform -> dequantised matvec."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    xr = fwht(x) if fused_fwht else x
    return matvec(words, scales, k, xr, group, levels)


def gemm_rows(words, scales, k, x, rows, group: int = GROUP, levels: int = 3) -> np.ndarray:
    """Selected rows of Y = fwht(X) . W_hat^T (the prefill GEMM)."""
    x = np.asarray(x, dtype=np.float64)[np.asarray(rows)]
    return gemv(words, scales, k, x, True, group, levels)


def unquantized(w: np.ndarray, x: np.ndarray) -> np.ndarray:
    """Context only (never parity): y = x . W^T with the original weights."""
    return np.atleast_2d(np.asarray(x, dtype=np.float64)) @ np.asarray(w, dtype=np.float64).T


# --------------------------------------------------------------------------
# MoE expert layer  ([TQ-MLX] point 1: 256 routed experts, top-8, FP gate)
# --------------------------------------------------------------------------
def route(logits: np.ndarray, topk: int):
    """Full-precision router: p = softmax over all experts (FP64); the top-k
    by p, ties to the lower id; weights renormalised over the chosen k."""
    z = np.asarray(logits, dtype=np.float64)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p = p / p.sum(axis=1, keepdims=True)
    ids = np.argsort(-p, axis=1, kind="stable")[:, :topk]
    w = np.take_along_axis(p, ids, axis=1)
    w = w / w.sum(axis=1, keepdims=True)
    return ids.astype(np.int32), w


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def moe(x, ids, route_w, gu_words, gu_scales, dn_words, dn_scales, hidden, inter,
        tokens=None, group: int = GROUP):
    """Expert MLP over routed tokens.  Per token t and slot j with e = ids[t][j]:
    g||u = W_gu[e] . H x_t  (rows [0, I) gate, [I, 2I) up),
    h = silu(g) * u,  o = W_dn[e] . H h,  y_t = sum_j w[t][j] * o.

    gu_words[e] / dn_words[e] etc. are indexable per expert (list, dict or
    array).  ``tokens`` restricts the computation to those token rows (the
    result still has one row per token; others stay zero).  Dequantised
    experts are memoised within the call only."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    t_count = x.shape[0]
    y = np.zeros((t_count, hidden), dtype=np.float64)
    gu_cache, dn_cache = {}, {}
    for t in (range(t_count) if tokens is None else tokens):
        xr = fwht(x[t:t + 1])[0]
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            if e not in gu_cache:
                gu_cache[e] = dequantize(gu_words[e], gu_scales[e], hidden, group)
                dn_cache[e] = dequantize(dn_words[e], dn_scales[e], inter, group)
            gu = gu_cache[e] @ xr
            h = silu(gu[:inter]) * gu[inter:]
            o = dn_cache[e] @ fwht(h[None, :])[0]
            y[t] += float(route_w[t, j]) * o
    return y


# --------------------------------------------------------------------------
# Parity metric
# --------------------------------------------------------------------------
def rel_l2(y, y_ref) -> float:
    """||y - y_ref||_2 / ||y_ref||_2 over the whole tensor, in FP64 (the
    ratio of norms, not of squared norms; the reference in the denominator).
    A zero reference gives the plain norm of y."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    den = np.linalg.norm(y_ref.ravel())
    num = np.linalg.norm((y - y_ref).ravel())
    return float(num / den) if den > 0 else float(num)


def row_max_rel(y, y_ref) -> float:
    """Largest, over the rows of a [rows][cols] pair (a 1-D pair is one row),
    of max_c |y - y_ref| / max_c |y_ref|: a local error that a whole-tensor
    norm would dilute.  A row whose reference is all zero contributes
    max |y| of that row."""
    y = np.atleast_2d(np.asarray(y, dtype=np.float64))
    y_ref = np.atleast_2d(np.asarray(y_ref, dtype=np.float64))
    if y.shape != y_ref.shape:
        raise ValueError("shape mismatch")
    worst = 0.0
    for r in range(y.shape[0]):
        num = float(np.max(np.abs(y[r] - y_ref[r]))) if y.shape[1] else 0.0
        den = float(np.max(np.abs(y_ref[r]))) if y.shape[1] else 0.0
        worst = max(worst, num / den if den > 0 else num)
    return worst
