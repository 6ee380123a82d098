"""GPU parity of the offline format kernels against the oracle: pack/unpack
bit-exact, scale re-layout exact, GPU quantiser identical except at exact
threshold ties, and the block transform within FP32 rounding."""
import numpy as np
import pytest

import synth
import ternary_weight_quantized_tq_amd as tq
from oracle import tq_oracle as O

from tqgpu import (ZERO_WORD, act_tensor, dev, gpu_pack, gpu_quantize, host_f16, host_u32, row64_scales_to_rowmajor,
                   row64_to_rowmajor, row64_word_order, torch)

pytestmark = pytest.mark.gpu

ROWMAJOR_SHAPES = [(1, 1), (3, 19), (5, 20), (7, 21), (4, 127), (4, 128), (3, 129), (2, 1000), (64, 640),
                   (65, 5120), (2, 17408)]
ROW64_SHAPES = [(1, 128), (63, 256), (64, 640), (65, 768), (130, 1024), (7, 2048), (3, 17408), (200, 512)]


@pytest.mark.parametrize("n,k", ROWMAJOR_SHAPES)
def test_pack_rowmajor_bit_exact(n, k):
    t = synth.trits(10 + n + k, n, k)
    want = O.pack(t)
    words = torch().empty(tq.tq_layout_words(n, k, tq.TQ_LAYOUT_ROWMAJOR, 3), dtype=torch().int32, device="cuda")
    tq.tq_pack(dev(t), n, k, tq.TQ_LAYOUT_ROWMAJOR, 3, words)
    got = host_u32(words).reshape(n, -1)
    assert np.array_equal(got, want)
    back = torch().empty((n, k), dtype=torch().int8, device="cuda")
    tq.tq_unpack(words, n, k, tq.TQ_LAYOUT_ROWMAJOR, 3, back)
    assert np.array_equal(back.cpu().numpy(), t)


@pytest.mark.parametrize("n,k", ROW64_SHAPES)
def test_pack_row64_layout(n, k):
    t = synth.trits(20 + n + k, n, k)
    s = synth.scales(21 + n, n, k // 128)
    w = gpu_pack(t, s, tq.TQ_LAYOUT_ROW64)
    full = row64_to_rowmajor(host_u32(w.words), n, k)
    assert np.array_equal(full[:n], O.pack(row64_word_order(t)))
    assert np.all(full[n:] == ZERO_WORD)
    sc = host_f16(w.scales)
    sc_canon, sc_full = row64_scales_to_rowmajor(sc, n, k)
    assert np.array_equal(sc_canon.view(np.uint16), s.view(np.uint16))
    spad = np.ones(sc_full.shape, bool)
    spad[:n, :k // 128] = False
    assert np.all(sc_full[spad].view(np.uint16) == 0)
    back = torch().empty((n, k), dtype=torch().int8, device="cuda")
    tq.tq_unpack(w.words, n, k, tq.TQ_LAYOUT_ROW64, 3, back)
    assert np.array_equal(back.cpu().numpy(), t)


@pytest.mark.parametrize("n,k", [(65, 768), (3, 17408)])
def test_pack_row64_unaligned_trits(n, k):
    """Trits at an address that is not 16-byte aligned take the per-word
    kernels (the staged ones need aligned rows); same words, same trits
    back."""
    th = torch()
    t = synth.trits(40 + n + k, n, k)
    buf = th.zeros(n * k + 16, dtype=th.int8, device="cuda")
    src = buf[3:3 + n * k]
    src.copy_(th.from_numpy(t.ravel()).cuda())
    words = th.empty(tq.tq_layout_words(n, k, tq.TQ_LAYOUT_ROW64, 3), dtype=th.int32, device="cuda")
    tq.tq_pack(src, n, k, tq.TQ_LAYOUT_ROW64, 3, words)
    full = row64_to_rowmajor(host_u32(words), n, k)
    assert np.array_equal(full[:n], O.pack(row64_word_order(t)))
    assert np.all(full[n:] == ZERO_WORD)
    out = th.zeros(n * k + 16, dtype=th.int8, device="cuda")
    tq.tq_unpack(words, n, k, tq.TQ_LAYOUT_ROW64, 3, out[5:5 + n * k])
    got = out.cpu().numpy()
    assert np.array_equal(got[5:5 + n * k].reshape(n, k), t)
    assert not got[:5].any() and not got[5 + n * k:].any()


def _near_tie(w_rot, gamma, rel=1e-12):
    n, k = w_rot.shape
    g = np.repeat(gamma, 128, axis=1)
    return np.abs(np.abs(w_rot) - g / 2) <= rel * g


@pytest.mark.parametrize("seed,n,k", [(1001, 512, 1024), (77, 100, 384), (78, 3, 17408)])
@pytest.mark.parametrize("dtype", ["f64", "f32"])
def test_quantize_matches_oracle(seed, n, k, dtype):
    w = synth.weights(seed, n, k)
    if dtype == "f32":
        w = w.astype(np.float32).astype(np.float64)
    w_rot = O.rotate_weights(w)
    t_ref, s_ref, gamma = O.ternarize(w_rot)
    trits, scales = gpu_quantize(w, dtype)
    t_gpu = trits.cpu().numpy()
    s_gpu = scales.cpu().numpy().view(np.float16)
    diff = t_gpu != t_ref
    assert not np.any(diff & ~_near_tie(w_rot, gamma)), "trit decisions differ away from a threshold tie"
    assert diff.sum() <= 2
    assert np.array_equal(s_gpu.view(np.uint16), s_ref.view(np.uint16))


def test_quantize_tie_and_zero_groups():
    g = np.concatenate([np.full(64, 3.0), np.full(64, 1.0)])
    h = O.hadamard(128)
    w = np.stack([g @ h, -(g @ h), np.zeros(128)])   # rotates back to g, -g, 0
    trits, scales = gpu_quantize(w)
    t_ref, s_ref, _ = O.quantize(w)
    assert np.array_equal(scales.cpu().numpy().view(np.uint16), s_ref.view(np.uint16))
    tie = _near_tie(O.rotate_weights(w), O.ternarize(O.rotate_weights(w))[2], rel=1e-9)
    t = trits.cpu().numpy()
    assert np.array_equal(t[~tie], t_ref[~tie])
    assert np.all(t[2] == 0)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_fwht_matches_oracle(dtype):
    act = synth.activations(5, 3, 640, dtype)
    x = act_tensor(act)
    out = torch().empty((3, 640), dtype=torch().float32, device="cuda")
    tq.tq_fwht(x, 3, 640, out)
    got = out.cpu().numpy().astype(np.float64)
    want = O.fwht(act.values)
    assert O.rel_l2(got, want) < 1e-6
    assert np.abs(got - want).max() < 1e-5


def test_fwht_one_hot_exact_columns():
    x = np.zeros((1, 256), np.float32)
    x[0, 131] = 1.0
    out = torch().empty((1, 256), dtype=torch().float32, device="cuda")
    tq.tq_fwht(dev(x), 1, 256, out)
    got = out.cpu().numpy()[0]
    assert np.all(got[:128] == 0)
    assert np.allclose(got[128:], O.hadamard(128)[3], rtol=0, atol=1e-7)


@pytest.mark.parametrize("layout", [tq.TQ_LAYOUT_ROWMAJOR, tq.TQ_LAYOUT_ROW64])
def test_pack_checked_counts_bad_trits(layout):
    """Values outside {-1, 0, 1} are counted by tq_pack_checked and packed
    as 0 by both pack calls (every word stays a base-3 number below 3^20)."""
    th = torch()
    n, k = 70, 1280
    t = synth.trits(31, n, k)
    bad = t.copy()
    rng = np.random.default_rng(32)
    pos = rng.choice(n * k, 37, replace=False)
    bad.ravel()[pos] = rng.choice(np.array([2, -2, 5, 127, -128], np.int8), 37)
    clean = bad.copy()
    clean.ravel()[pos] = 0
    count = th.full((1,), -1, dtype=th.int32, device="cuda")
    w_checked = th.empty(tq.tq_layout_words(n, k, layout, 3), dtype=th.int32, device="cuda")
    w_plain = th.empty_like(w_checked)
    w_clean = th.empty_like(w_checked)
    tq.tq_pack_checked(dev(bad), n, k, layout, 3, w_checked, count)
    tq.tq_pack(dev(bad), n, k, layout, 3, w_plain)
    tq.tq_pack(dev(clean), n, k, layout, 3, w_clean)
    th.cuda.synchronize()
    assert int(count.item()) == 37
    assert np.array_equal(host_u32(w_checked), host_u32(w_clean))
    assert np.array_equal(host_u32(w_plain), host_u32(w_clean))
    assert host_u32(w_checked).max() < 3 ** 20
    # a clean input reports zero, on the same counter
    tq.tq_pack_checked(dev(clean), n, k, layout, 3, w_checked, count)
    th.cuda.synchronize()
    assert int(count.item()) == 0
