"""Test helpers: move synthetic inputs to the GPU and run the HIP path through
the C ABI.  Nothing here computes any step of the method."""
from __future__ import annotations

import numpy as np

import synth
import ternary_weight_quantized_tq_amd as tq

ZERO_WORD = 1743392200


def torch():
    import torch as _t
    return _t


def dev(a: np.ndarray):
    t = torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        return t.from_numpy(a.view(np.int32)).cuda()
    if a.dtype == np.uint16:
        return t.from_numpy(a.view(np.int16)).cuda()
    return t.from_numpy(a).cuda()


def act_tensor(act: synth.Activations):
    t = torch()
    if act.dtype == "f32":
        return dev(act.raw.astype(np.float32))
    x = dev(act.raw.astype(np.uint16))
    return x.view(t.bfloat16) if act.dtype == "bf16" else x.view(t.float16)


def host_u32(x) -> np.ndarray:
    return x.cpu().numpy().view(np.uint32)


def host_f16(x) -> np.ndarray:
    return x.cpu().numpy().view(np.float16)


def gpu_pack(trits: np.ndarray, scales: np.ndarray, layout=tq.TQ_LAYOUT_ROW64, group=128, levels=3) -> tq.Weights:
    """Pack given trits (or signs) and scales on the GPU into `layout`."""
    n, k = trits.shape
    w = tq.empty_weights(n, k, layout, group=group, levels=levels)
    tq.tq_pack(dev(trits), n, k, layout, levels, w.words)
    tq.tq_pack_scales(dev(scales.view(np.uint16)), n, k, layout, group, w.scales)
    return w


def gpu_quantize(weights: np.ndarray, dtype="f64", group=128, levels=3):
    """Offline conversion on the GPU: returns (trits tensor [n][k] int8, scales tensor int16)."""
    t = torch()
    n, k = weights.shape
    w = dev(weights.astype(np.float64 if dtype == "f64" else np.float32))
    trits = t.empty((n, k), dtype=t.int8, device="cuda")
    scales = t.empty((n, k // group), dtype=t.int16, device="cuda")
    tq.tq_quantize(w, n, k, group, levels, trits, scales)
    del w
    return trits, scales


def gpu_quantize_pack(weights: np.ndarray, layout=tq.TQ_LAYOUT_ROW64, group=128, levels=3) -> tq.Weights:
    n, k = weights.shape
    trits, scales = gpu_quantize(weights, group=group, levels=levels)
    w = tq.empty_weights(n, k, layout, group=group, levels=levels)
    tq.tq_pack(trits, n, k, layout, levels, w.words)
    tq.tq_pack_scales(scales, n, k, layout, group, w.scales)
    return w


def run_gemv(w: tq.Weights, x, m: int, fused=True) -> np.ndarray:
    t = torch()
    y = t.empty((m, w.n), dtype=t.float32, device="cuda")
    ws, nbytes = tq.workspace(tq.TQ_OP_GEMV, w, m)
    tq.tq_gemv(w, x, m, y, tq.TQ_FWHT_FUSED if fused else 0, ws, nbytes)
    t.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def row64_to_rowmajor(words: np.ndarray, n: int, k: int) -> np.ndarray:
    """Re-index ROW64 words per the layout definition in tq.h: word
    (((s*nb + b)*8 + qi)*64 + r)*4 + j is word 32s + 4qi + j of row 64b + r.
    Returns [nb*64][nsl*32] (padding included)."""
    nsl = -(-k // 640)
    nb = -(-n // 64)
    return words.reshape(nsl, nb, 8, 64, 4).transpose(1, 3, 0, 2, 4).reshape(nb * 64, nsl * 32)


def row64_chunk(wl: int, j: int) -> int:
    """Unit chunk held by chunk j (digits 4j..4j+3) of unit word wl, per the
    ROW64 chunk order in tq.h: q = 5 (wl % 2) + j, c = 8 (q // 2) + 2 (wl // 2) + q % 2."""
    q = 5 * (wl % 2) + j
    return 8 * (q // 2) + 2 * (wl // 2) + q % 2


def row64_word_order(t: np.ndarray) -> np.ndarray:
    """Trits [n][k] rearranged so that trits 20w .. 20w + 19 are the digits of
    ROW64 word w of the row (w = 32s + 8u + wl, unit u of slice s), zero trits
    past k: packing this array row by row gives the ROW64 word values.  Index
    bookkeeping only."""
    n, k = t.shape
    nsl = -(-k // 640)
    src = np.empty(nsl * 640, np.int64)
    for w in range(nsl * 32):
        base = 640 * (w // 32) + 160 * ((w % 32) // 8)
        for j in range(5):
            c = row64_chunk(w % 8, j)
            src[20 * w + 4 * j: 20 * w + 4 * j + 4] = base + 4 * c + np.arange(4)
    padded = np.zeros((n, nsl * 640), np.int8)
    padded[:, :k] = t
    return padded[:, src]


def row64_scales_to_rowmajor(s: np.ndarray, n: int, k: int) -> np.ndarray:
    """Scale (s*nb + b)*5 + gi, row r  ->  [n][k/128]."""
    g = k // 128
    wpr = -(-k // 20)
    nsl = -(-wpr // 32)
    nb = -(-n // 64)
    a = s.reshape(nsl, nb, 5, 64).transpose(1, 3, 0, 2).reshape(nb * 64, nsl * 5)
    return a[:n, :g], a


def gpu_pack_expert(w: "tq.Weights", e: int, weights64: np.ndarray = None, trits=None, scales=None):
    """Quantise (or take given trits/scales) and pack one expert into slot e
    of an E-expert ROW64 buffer."""
    n, k = w.n, w.k
    nw = tq.tq_layout_words(n, k, tq.TQ_LAYOUT_ROW64, 3)
    ns = tq.tq_layout_scales(n, k, tq.TQ_LAYOUT_ROW64, 128)
    if weights64 is not None:
        t_dev, s_dev = gpu_quantize(weights64)
    else:
        t_dev, s_dev = dev(trits), dev(scales.view(np.uint16))
    tq.tq_pack(t_dev, n, k, tq.TQ_LAYOUT_ROW64, 3, w.words.data_ptr() + 4 * nw * e)
    tq.tq_pack_scales(s_dev, n, k, tq.TQ_LAYOUT_ROW64, 128, w.scales.data_ptr() + 2 * ns * e)
    torch().cuda.synchronize()


def run_moe(w_gu, w_dn, x, t, topk, ids: np.ndarray, route_w: np.ndarray) -> np.ndarray:
    th = torch()
    y = th.empty((t, w_dn.n), dtype=th.float32, device="cuda")
    ws, nbytes = tq.workspace(tq.TQ_OP_MOE, w_gu, t, topk)
    tq.tq_moe_gemv(w_gu, w_dn, x, t, topk, dev(ids.astype(np.int32)), dev(route_w.astype(np.float32)), y,
                   tq.TQ_FWHT_FUSED, ws, nbytes)
    th.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def run_gemm(w: "tq.Weights", x, m: int, fused=True) -> np.ndarray:
    th = torch()
    y = th.empty((m, w.n), dtype=th.float32, device="cuda")
    ws, nbytes = tq.workspace(tq.TQ_OP_GEMM, w, m)
    tq.tq_gemm(w, x, m, y, tq.TQ_FWHT_FUSED if fused else 0, ws, nbytes)
    th.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)
