"""Plain CPU oracle for the TurboQuant-style KV-cache quantiser.

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` (and nothing on the product
path).  It shares no code with the HIP library and imports nothing from the
package; the random rotation signs and the JL matrix are inputs drawn by
``synth``.  FP64 throughout, straight from the definitions.

What the pages say (cited by title and section):

* [oMLX-Gemma] "Mac users can use TurboQuant in oMLX, with Gemma-4-31B"
  (aitntnews), section "What TurboQuant is and what problem it solves":
  it compresses the KV cache (not the weights) in two steps: a random
  orthogonal rotation of each KV vector and a conversion to polar form
  (PolarQuant) with the radius kept at high precision; then a 1-bit
  Johnson-Lindenstrauss projection (QJL) that removes the remaining bias.
  It is data-oblivious (no per-block scale), giving about 4-5x at 3 bits.
  The decode path does "coordinate rotation and table lookups" (section
  "Why these results").
* [TQ+] "TurboQuant+" (hugong.cc): the KV cache shrinks to 1/4 - 1/6.

Readings (where the pages are silent):

* vectors are per-head K or V rows of dimension d = 128;
* rotation Pi x = H (sigma * x): the Sylvester Hadamard of order 128
  (normalised) after a seeded random sign flip sigma, a fast random
  orthogonal transform; Pi^T y = sigma * (H y);
* polar form: radius r = |x|_2 stored in fp16 (round to nearest even once),
  direction u = Pi x / r (u = 0 when r = 0);
* the direction's coordinates are quantised with a fixed codebook, the
  Lloyd-Max quantiser of N(0, 1/d) (a coordinate of a random unit vector in
  R^d is close to N(0, 1/d) at d = 128), nearest level, a tie to the lower
  level;
* keys (inner products with queries): b - 1 bits of codebook, then the
  residual e = u - u~ through the 1-bit projection: z = sign(S e) with
  S in R^{d x d} of N(0, 1) entries (sign(0) = +1), and gamma = |e|_2 in fp16;
  score(q, k) = r (<Pi q, u~> + gamma sqrt(pi/2) / d <S Pi q, z>);
* values (reconstructed): b bits of codebook; v^ = r Pi^T u~;
* storage: the codes as packed little-endian fields (the code of
  coordinate j in bits m j .. m j + m - 1 of the record, m bits per code,
  word w holding record bits 32 w .. 32 w + 31), then for keys the signs z
  as 128 more bits (bit j set where z_j = +1); per vector only r (and gamma
  for keys) beside the codes.
"""
from __future__ import annotations

import math

import numpy as np

D = 128


# --------------------------------------------------------------------------
# rotation  ([oMLX-Gemma]: random orthogonal rotation)
# --------------------------------------------------------------------------
def hadamard(n: int = D) -> np.ndarray:
    h = np.empty((n, n))
    for i in range(n):
        for j in range(n):
            h[i, j] = -1.0 if bin(i & j).count("1") % 2 else 1.0
    return h / math.sqrt(n)


def rotation(signs) -> np.ndarray:
    """Pi = H diag(sigma) as a dense d x d matrix."""
    s = np.asarray(signs, dtype=np.float64)
    return hadamard(len(s)) * s[None, :]


_PM1: dict = {}


def _hadamard_pm1(n: int) -> np.ndarray:
    """The Sylvester Hadamard matrix with its +-1 entries (unscaled)."""
    if n not in _PM1:
        _PM1[n] = hadamard(n) * math.sqrt(n)
    return _PM1[n]


def rotate(x, signs) -> np.ndarray:
    """Rows of x mapped by Pi: y = H (sigma * x), summed with the exact +-1
    entries and scaled by 1/sqrt(d) once, so that a coordinate whose terms
    cancel exactly (bf16 inputs can) is exactly 0 rather than a rounding
    residue of the scaled entries."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    s = np.asarray(signs, dtype=np.float64)
    return ((x * s[None, :]) @ _hadamard_pm1(len(s)).T) / math.sqrt(len(s))


def unrotate(y, signs) -> np.ndarray:
    """Rows of y mapped by Pi^T: sigma * (H y), scaled the same way."""
    y = np.atleast_2d(np.asarray(y, dtype=np.float64))
    s = np.asarray(signs, dtype=np.float64)
    return ((y @ _hadamard_pm1(len(s))) / math.sqrt(len(s))) * s[None, :]


# --------------------------------------------------------------------------
# the codebook: Lloyd-Max quantiser of a Gaussian (data-oblivious)
# --------------------------------------------------------------------------
def _phi(x):
    return math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi) if math.isfinite(x) else 0.0


def _upper(x):
    """P(X > x) for X ~ N(0, 1), from erfc so that far tails keep full precision."""
    if not math.isfinite(x):
        return 0.0 if x > 0 else 1.0
    return 0.5 * math.erfc(x / math.sqrt(2.0))


def _cell_prob(a, b):
    """P(a < X < b); cells on one side of 0 use tail differences there."""
    if a >= 0.0:
        return _upper(a) - _upper(b)
    if b <= 0.0:
        return _upper(-b) - _upper(-a)
    return 1.0 - _upper(b) - _upper(-a)


def _cells(c):
    """Boundaries (midpoints, with -inf and +inf at the ends), cell
    probabilities and cell means E[X | cell] = (phi(a) - phi(b)) / P."""
    b = np.concatenate([[-math.inf], (c[:-1] + c[1:]) / 2.0, [math.inf]])
    p = np.array([_cell_prob(b[i], b[i + 1]) for i in range(len(c))])
    m = np.array([(_phi(b[i]) - _phi(b[i + 1])) / p[i] for i in range(len(c))])
    return b, p, m


def lloyd_max_gaussian(levels: int, iters: int = 2000):
    """The Lloyd-Max quantiser of N(0, 1): levels that are the means of their
    nearest-level cells.  Lloyd's iteration (cells from the levels, levels
    from the cell means) from uniform starting levels, at most `iters`
    steps; from 16 levels up it approaches the fixed point too slowly, so
    Newton's method on the same equations c_i = E[X | cell_i(c)] finishes
    it (the Jacobian of a cell mean with respect to its ends a, b is
    phi(a)(m - a)/P and phi(b)(b - m)/P, and each end moves by half of each
    neighbouring level's step).  Returns (levels ascending, boundaries, mse)."""
    c = np.linspace(-2.0, 2.0, levels) if levels > 1 else np.zeros(1)
    for _ in range(iters):
        new = _cells(c)[2]
        done = np.max(np.abs(new - c)) < 1e-15
        c = new
        if done:
            break
    for _ in range(100):
        b, p, m = _cells(c)
        if np.max(np.abs(c - m)) < 1e-15:
            break
        jac = np.eye(levels)
        for i in range(levels):
            da = _phi(b[i]) * (m[i] - b[i]) / p[i] if math.isfinite(b[i]) else 0.0
            db = _phi(b[i + 1]) * (b[i + 1] - m[i]) / p[i] if math.isfinite(b[i + 1]) else 0.0
            if i > 0:
                jac[i, i - 1] -= da / 2.0
            jac[i, i] -= (da + db) / 2.0
            if i + 1 < levels:
                jac[i, i + 1] -= db / 2.0
        step = np.linalg.solve(jac, m - c)
        c = c + step
        if np.max(np.abs(step)) < 1e-15:
            break
    # N(0, 1) is symmetric, and so is its quantiser; rounding in the solves
    # leaves a mismatch near 1e-13, removed here so that 0 sits exactly on
    # the middle boundary (a zero vector then takes the lower middle level).
    c = (c - c[::-1]) / 2.0
    b = _cells(c)[0]
    # E[(X - c)^2] over each cell: E[X^2 | cell] - 2 c E[X | cell] + c^2, with
    # E[X^2 1(a<X<b)] = P(a<X<b) + a phi(a) - b phi(b)
    mse = 0.0
    for i in range(levels):
        a, bb = b[i], b[i + 1]
        p = _cell_prob(a, bb)
        m1 = _phi(a) - _phi(bb)
        m2 = p + (a * _phi(a) if math.isfinite(a) else 0.0) - (bb * _phi(bb) if math.isfinite(bb) else 0.0)
        mse += m2 - 2.0 * c[i] * m1 + c[i] * c[i] * p
    return c, b[1:-1], mse


_LM_CACHE: dict = {}


def codebook(bits: int, d: int = D) -> np.ndarray:
    """Levels of the b-bit quantiser of one rotated unit-vector coordinate:
    Lloyd-Max of N(0, 1) scaled by 1/sqrt(d)."""
    if bits not in _LM_CACHE:
        _LM_CACHE[bits] = lloyd_max_gaussian(2 ** bits)[0]
    return _LM_CACHE[bits] / math.sqrt(d)


def nearest_level(u, levels) -> np.ndarray:
    """Index of the nearest level (levels ascending); a value exactly halfway
    between two levels goes to the lower one."""
    u = np.asarray(u, dtype=np.float64)
    mids = (levels[:-1] + levels[1:]) / 2.0
    return np.searchsorted(mids, u, side="left").astype(np.int64)


# --------------------------------------------------------------------------
# quantise, estimate, reconstruct
# --------------------------------------------------------------------------
def kv_quantize(x, signs, bits: int, keys: bool, jl=None):
    """Quantise rows of x.  keys=True: (bits - 1)-bit codes, the residual's
    1-bit projection z = sign(S e) and gamma = |e|; keys=False: bits-bit codes.
    Returns a dict of r (fp16), codes (int), and for keys gamma (fp16), z (+-1)."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    d = x.shape[1]
    r = np.linalg.norm(x, axis=1)
    y = rotate(x, signs)
    u = np.where(r[:, None] > 0, y / np.where(r > 0, r, 1.0)[:, None], 0.0)
    mb = bits - 1 if keys else bits
    cb = codebook(mb, d)
    codes = nearest_level(u, cb)
    out = {"r": r.astype(np.float16), "codes": codes, "bits": bits, "keys": keys}
    if keys:
        e = u - cb[codes]
        s = np.asarray(jl, dtype=np.float64) @ e.T           # [d][n]
        out["z"] = np.where(s.T >= 0.0, 1, -1).astype(np.int8)
        out["gamma"] = np.linalg.norm(e, axis=1).astype(np.float16)
    return out


def kv_scores(q, kq, signs, jl) -> np.ndarray:
    """score(q, k_i) = r_i (<Pi q, u~_i> + gamma_i sqrt(pi/2) / d <S Pi q, z_i>)
    for one query q against the quantised keys kq (stored r, gamma)."""
    q = np.asarray(q, dtype=np.float64).reshape(-1)
    d = q.shape[0]
    qr = rotate(q, signs)[0]
    cb = codebook(kq["bits"] - 1, d)
    mse = cb[kq["codes"]] @ qr
    sq = np.asarray(jl, dtype=np.float64) @ qr
    qjl = kq["gamma"].astype(np.float64) * math.sqrt(math.pi / 2.0) / d * (kq["z"].astype(np.float64) @ sq)
    return kq["r"].astype(np.float64) * (mse + qjl)


def kv_values(p, vq, signs) -> np.ndarray:
    """sum_i p_i v^_i with v^_i = r_i Pi^T u~_i (accumulated in the rotated
    frame, one Pi^T at the end)."""
    p = np.asarray(p, dtype=np.float64).reshape(-1)
    d = vq["codes"].shape[1]
    cb = codebook(vq["bits"], d)
    acc = (p * vq["r"].astype(np.float64)) @ cb[vq["codes"]]
    return unrotate(acc, signs)[0]


def kv_attend(scores, scale: float, vq, signs) -> np.ndarray:
    """Attention output for one query: p = softmax(scale * scores) over the
    keys (max subtracted, FP64), then sum_i p_i v^_i (kv_values)."""
    z = float(scale) * np.asarray(scores, dtype=np.float64).reshape(-1)
    p = np.exp(z - z.max())
    return kv_values(p / p.sum(), vq, signs)


def kv_dequantize_values(vq, signs) -> np.ndarray:
    d = vq["codes"].shape[1]
    return vq["r"].astype(np.float64)[:, None] * unrotate(codebook(vq["bits"], d)[vq["codes"]], signs)


def pack_fields(codes, nbits: int) -> np.ndarray:
    """Codes as packed little-endian nbits-bit fields: out[n][w] holds bits
    32 w .. 32 w + 31 of the concatenation, code j in bits nbits j ..
    nbits j + nbits - 1."""
    codes = np.asarray(codes, dtype=np.int64)
    n, d = codes.shape
    words = d * nbits // 32
    out = np.zeros((n, words), dtype=np.uint64)
    for j in range(d):
        for t in range(nbits):
            bit = nbits * j + t
            out[:, bit // 32] |= ((codes[:, j] >> t) & 1).astype(np.uint64) << np.uint64(bit % 32)
    return out.astype(np.uint32)


def kv_records(kq) -> np.ndarray:
    """The stored record of each vector, uint32 [n][4 bits]: the codebook
    codes as packed fields, then (keys) the 128 bits of z (set where
    z = +1)."""
    mb = kq["bits"] - 1 if kq["keys"] else kq["bits"]
    rec = pack_fields(kq["codes"], mb)
    if kq["keys"]:
        rec = np.concatenate([rec, pack_fields((kq["z"] > 0).astype(np.int64), 1)], axis=1)
    return rec


def stored_bits(bits: int, keys: bool, d: int = D) -> int:
    """Bits per stored vector: d b code and sign bits, plus the fp16 radius
    (and the fp16 residual norm for keys)."""
    return d * bits + (32 if keys else 16)
