"""Benchmark of the ternary packed-weight decode path on one MI355X.

Main metric (one JSON line on stdout).  A step is one single-stream decode
pass through a 27B-class dense MLP's two ternary linears at M = 1: the
block-128 transform fused into each GEMV, up (K=5120 -> N=17408) then down
(K=17408 -> N=5120), bf16 activations, FP32 outputs.  The outputs are
accumulated into one zeroed buffer (one fill kernel per step, then each
GEMV is a single launch in TQ_ACCUMULATE mode).  Weights are seeded
synthetic (N(0, 0.02^2) with 0.1% x20 outliers) and quantised and packed on
the GPU before timing; the step cycles through R copies of the packed
weights (R * bytes >= 1 GiB) so that HBM, not the 256 MB Infinity Cache,
serves them.

  value     packed-weight GB/s over the whole timed step (fill, launch gaps
            and both GEMVs included)
  roofline  the GEMV kernel alone: algorithmic packed bytes per launch over
            the mean launch duration from HIP events recorded around each
            launch on its stream, against the 8 TB/s HBM peak; `traffic` is
            the measured HBM bytes per launch from the committed rocprofv3
            counter summary when it was taken on the current kernel sources
  cpu_baseline  the FP64 CPU oracle (unpack + transform + dequantised
            matvec) on a bounded row sample, in packed-weight GB/s: all
            cores (one process per usable core, one BLAS thread each) as
            `value`, one thread beside it
  read_only_same_bytes  one plain read pass over one launch's bytes (the
            read ceiling at this launch size; context)
  isolated_launch_us_p10_p50_p90  one GEMV launched alone between two HIP
            events (dispatch and ramp-up included; context)
  mall_hot_single_copy   the same step on one weight copy (cache-resident,
            labelled; context, not the metric)

`extras` adds the other workloads: one transformer block's seven linears at
M = 1 (single stream) and M = 8, the 256-expert MoE layer at T = 1 and
T = 64, the prefill GEMM, and the format variants (ternary at group 64,
binary {-c, +c} at groups 128 and 64) on the decode step's two linears.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
VALU_F32_PEAK_TFLOPS = 157.3
ROTATE_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_m1_dense27b_traffic.md")
GEMV_SOURCES = ["ternary_weight_quantized_tq_amd/csrc/tq_gemv.hip", "ternary_weight_quantized_tq_amd/csrc/tq_decode.h",
                "ternary_weight_quantized_tq_amd/csrc/tq_internal.h"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-extras", action="store_true", help="only the main metric")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--only-extra", choices=["block_m1", "block_m8", "moe", "prefill_gemm", "variants", "kv_cache",
                                            "format"],
                   help="run one extra workload alone and print its JSON (for profiling)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 256 MiB device copy (for scaling rocprofv3 byte counters)")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def sources_digest() -> str:
    """Hash of the GEMV kernel sources with comments and whitespace removed,
    so that it changes with the code and not with its comments."""
    h = hashlib.sha256()
    for f in GEMV_SOURCES:
        text = open(os.path.join(ROOT, f)).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic():
    """Bytes per GEMV launch from the committed counter summary, or None if
    it is missing or was taken on different kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m = re.search(r"sources_digest:\s*([0-9a-f]+)", text)
    b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not b or m.group(1) != sources_digest():
        return None
    return float(b.group(1))


def quantize_pack(tq, torch, w64, n, k, w_out=None, expert=0):
    wt = torch.from_numpy(w64).cuda()
    trits = torch.empty((n, k), dtype=torch.int8, device="cuda")
    scales = torch.empty((n, k // 128), dtype=torch.int16, device="cuda")
    tq.tq_quantize(wt, n, k, 128, 3, trits, scales)
    del wt
    w = w_out if w_out is not None else tq.empty_weights(n, k)
    nw, ns = tq.tq_layout_words(n, k, tq.TQ_LAYOUT_ROW64, 3), tq.tq_layout_scales(n, k, tq.TQ_LAYOUT_ROW64, 128)
    tq.tq_pack(trits, n, k, tq.TQ_LAYOUT_ROW64, 3, w.words.data_ptr() + 4 * nw * expert)
    tq.tq_pack_scales(scales, n, k, tq.TQ_LAYOUT_ROW64, 128, w.scales.data_ptr() + 2 * ns * expert)
    return w


def bf16(torch, act):
    import numpy as np
    return torch.from_numpy(act.raw.view(np.int16)).cuda().view(torch.bfloat16)


def clone_w(tq, w):
    return w.clone()


def capture(torch, n, fn, *extra):
    """A HIP graph holding n steps (fn(i, *extra) for i < n)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i, *extra)
    return g


def timed(torch, steps, warmup, fn):
    """Mean ms per step: `warmup` eager steps, then `steps` steps captured in
    one HIP graph, replayed once untimed and once between two events."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    g = capture(torch, steps, fn)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def _oracle_worker(chunks, seconds, barrier, out):
    """One all-cores worker: the oracle on its row chunks, repeated for
    `seconds` after every worker is ready; BLAS limited to one thread."""
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except Exception:
        pass
    from oracle import tq_oracle as O
    barrier.wait()
    done, reps, t0 = 0, 0, time.perf_counter()
    while True:
        for words, s, k, x, nbytes in chunks:
            O.gemv(words, s, k, x, True)
            done += nbytes
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    out.put((done, reps, time.perf_counter() - t0))


def cpu_model_name():
    """The host processor as lscpu names it (model name, family, model and
    stepping), or /proc/cpuinfo's model name if lscpu is missing."""
    try:
        import subprocess
        txt = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        f = {ln.split(":", 1)[0].strip(): ln.split(":", 1)[1].strip() for ln in txt.splitlines() if ":" in ln}
        if "Model name" in f:
            return (f"{f['Model name']} (vendor {f.get('Vendor ID', '?')}, family {f.get('CPU family', '?')}, "
                    f"model {f.get('Model', '?')}, stepping {f.get('Stepping', '?')})")
    except Exception:
        pass
    try:
        with open("/proc/cpuinfo") as fh:
            return next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), None)
    except OSError:
        return None


def cpu_baseline(O, synth, lins, w64s, seconds, max_workers=16):
    """The FP64 oracle (unpack + dense block-128 transform + dequantised
    matvec) on row samples of the step's linears, in packed bytes per
    second.  Two legs: one thread (this process, BLAS limited to one
    thread), and all cores: the same rows cut into one chunk per usable core
    (at most `max_workers`), each chunk in its own process with one BLAS
    thread, all started together and run for the same time."""
    import multiprocessing as mp
    samples = []
    for lin, w64 in zip(lins, w64s):
        rows = 1024 if lin.k <= 8192 else 512
        t, s, _ = O.quantize(w64[:rows])
        x = synth.activations(lin.x_seed, 1, lin.k, "bf16").values
        samples.append((O.pack(t), s, lin.k, x, rows))
    desc = " + ".join(f"{smp[4]} rows of {lin.name} ({lin.n}x{lin.k})" for smp, lin in zip(samples, lins))

    # one thread
    one = {}
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            done, reps, t0 = 0, 0, time.perf_counter()
            while True:
                for words, s, k, x, rows in samples:
                    O.gemv(words, s, k, x, True)
                    done += O.packed_bytes(rows, k)
                reps += 1
                if time.perf_counter() - t0 >= seconds / 2:
                    break
            dt = time.perf_counter() - t0
        one = {"value": round(done / dt / 1e9, 5), "threads": 1, "reps": reps, "seconds": round(dt, 1)}
    except Exception as e:  # report, never hide
        one = {"error": f"{type(e).__name__}: {e}"}

    # all cores: one process per usable core, each on its share of the rows
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    workers = max(1, min(affinity, max_workers))
    chunks = [[] for _ in range(workers)]
    for words, s, k, x, rows in samples:
        for i, idx in enumerate(np_array_split(rows, workers)):
            if len(idx):
                chunks[i].append((words[idx], s[idx], k, x, O.packed_bytes(len(idx), k)))
    ctx = mp.get_context("spawn")
    barrier, out = ctx.Barrier(workers), ctx.Queue()
    procs = [ctx.Process(target=_oracle_worker, args=(chunks[i], seconds / 2, barrier, out)) for i in range(workers)]
    for p in procs:
        p.start()
    res = [out.get(timeout=600) for _ in procs]
    for p in procs:
        p.join()
    total = sum(r[0] for r in res)
    wall = max(r[2] for r in res)
    all_cores = total / wall / 1e9
    return {"value": round(all_cores, 5), "unit": "GB/s", "cores": workers, "kind": "oracle",
            "sample": f"{desc}: all cores = {workers} processes, one BLAS thread each, each on 1/{workers} of "
                      f"the rows, run together for {wall:.1f} s (FP64 unpack + dense block-128 transform + "
                      f"dequantised matvec), packed bytes per second",
            "one_thread": one, "nproc": os.cpu_count(), "affinity_cpus": affinity, "workers": workers,
            "cpu_model": cpu_model_name()}


def np_array_split(n, parts):
    """Index ranges of n rows in `parts` nearly equal consecutive chunks."""
    import numpy as np
    return np.array_split(np.arange(n), parts)


def cpu_gemm_rows(O, synth, rows=64):
    """The oracle on a row subset of the prefill GEMM: `rows` rows of X
    against the whole weight matrix (offline quantise and pack untimed), one
    timed call; the full-batch time is extrapolated linearly and flagged."""
    wl = synth.PREFILL_GEMM
    lin = wl.linears[0]
    t, s, _ = O.quantize(synth.weights(lin.w_seed, lin.n, lin.k))
    words = O.pack(t)
    del t
    x = synth.activations(lin.x_seed, rows, lin.k, "bf16").values
    t0 = time.perf_counter()
    O.gemm_rows(words, s, lin.k, x, list(range(rows)))
    dt = time.perf_counter() - t0
    return {"workload": wl.name, "rows_timed": rows, "seconds": round(dt, 2),
            "tok_s": round(rows / dt, 2), "useful_gflops": round(2.0 * rows * lin.n * lin.k / dt / 1e9, 2),
            "extrapolated_ms_full_batch": round(dt * wl.m / rows * 1e3, 1),
            "note": "extrapolated linearly from the row subset (the dequantised matrix is rebuilt per call)"}


def cpu_moe_t1(O, synth):
    """The oracle on the single-token MoE layer: route the T = 1 logits,
    quantise and pack the eight routed experts (untimed), then one timed
    expert-MLP call, in layer tok/s."""
    wl = synth.MOE_T1
    ids, rw = O.route(synth.logits(wl.logit_seed, wl.tokens, wl.experts), wl.topk)
    gu_w, gu_s, dn_w, dn_s = {}, {}, {}, {}
    for e in sorted(set(int(v) for v in ids.ravel())):
        gu64, dn64 = synth.expert_weights(e, wl.hidden, wl.inter)
        t, s_, _ = O.quantize(gu64)
        gu_w[e], gu_s[e] = O.pack(t), s_
        t, s_, _ = O.quantize(dn64)
        dn_w[e], dn_s[e] = O.pack(t), s_
    x = synth.activations(wl.x_seed, wl.tokens, wl.hidden, "bf16").values
    t0 = time.perf_counter()
    O.moe(x, ids, rw, gu_w, gu_s, dn_w, dn_s, wl.hidden, wl.inter)
    dt = time.perf_counter() - t0
    return {"workload": wl.name, "seconds": round(dt, 3), "us_per_layer": round(dt * 1e6, 1),
            "tok_s": round(wl.tokens / dt, 2)}


def cpu_kv_sample(K, synth, tokens=65536):
    """The KV oracle on a sample of the 128K decode workload: one KV head's
    first `tokens` keys and values (quantised untimed), its 4 queries'
    scores and one weighted value sum per query, timed; in (key, query)
    pairs per second, with the full step (8 heads x 131,072 tokens)
    extrapolated linearly and flagged."""
    import numpy as np
    wl = synth.KV_DECODE_128K
    signs, jl = synth.kv_signs(wl.sign_seed), synth.kv_jl(wl.jl_seed)
    kq = K.kv_quantize(synth.kv_vectors(wl.key_seed, tokens, 128, "bf16").values, signs, wl.bits, True, jl)
    vq = K.kv_quantize(synth.kv_vectors(wl.value_seed, tokens, 128, "bf16").values, signs, wl.bits, False)
    q = synth.kv_vectors(wl.query_seed, wl.queries, 128, "f32").values
    t0 = time.perf_counter()
    for j in range(wl.queries):
        sc = K.kv_scores(q[j], kq, signs, jl)
        p = np.exp(sc / np.sqrt(128.0) - (sc / np.sqrt(128.0)).max())
        K.kv_values(p / p.sum(), vq, signs)
    dt = time.perf_counter() - t0
    pairs = tokens * wl.queries
    return {"workload": wl.name, "tokens_sampled": tokens, "heads_sampled": 1, "seconds": round(dt, 3),
            "pairs_per_s": round(pairs / dt, 1),
            "extrapolated_ms_full_step": round(dt * (wl.tokens / tokens) * wl.heads * 1e3, 1),
            "note": "scores, softmax and value sum of one head's 4 queries; extrapolated linearly to 8 heads "
                    "x 131,072 tokens"}


# --------------------------------------------------------------- extras ---
def extra_block(tq, torch, synth, np, wl):
    """One dense block's seven linears at wl.m activation rows (1: single
    stream, 8: eight streams).  Linears that share an input (q, k, v; gate,
    up) are also packed as one matrix of concatenated rows (the usual fused
    projections, same bytes and the same per-row quantisation): one launch
    per input instead of seven."""
    m = wl.m
    nbytes = sum(tq.tq_packed_bytes(l.n, l.k) for l in wl.linears)
    groups = {}
    for lin in wl.linears:
        groups.setdefault(lin.x_seed, []).append(lin)
    xs = {s: bf16(torch, synth.activations(s, m, g[0].k, "bf16")) for s, g in groups.items()}

    def run(mats, label):
        """mats: [(name, n, k, x_seed, w64)]; timed step and per-matrix kernel time."""
        base = [quantize_pack(tq, torch, w64, n, k) for _, n, k, _, w64 in mats]
        torch.cuda.synchronize()
        copies = max(1, -(-ROTATE_BYTES // nbytes))
        sets = [base] + [[clone_w(tq, w) for w in base] for _ in range(copies - 1)]
        y_all = torch.empty(m * sum(mt[1] for mt in mats), dtype=torch.float32, device="cuda")
        offs = np.cumsum([0] + [m * mt[1] for mt in mats])
        ys = [y_all[offs[i]:offs[i + 1]].view(m, mt[1]) for i, mt in enumerate(mats)]

        def step(i):
            y_all.zero_()
            for j, (mt, w) in enumerate(zip(mats, sets[i % copies])):
                tq.tq_gemv(w, xs[mt[3]], m, ys[j], tq.TQ_FWHT_FUSED | tq.TQ_ACCUMULATE)
        ms = timed(torch, 32, 4, step)
        per = {}
        for j, mt in enumerate(mats):
            g = capture(torch, copies, lambda i: tq.tq_gemv(sets[i][j], xs[mt[3]], m, ys[j],
                                                             tq.TQ_FWHT_FUSED | tq.TQ_ACCUMULATE))
            g.replay()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            per[mt[0]] = round(1e3 * a.elapsed_time(b) / copies, 3)
        del sets
        torch.cuda.empty_cache()
        return {"launches": len(mats), "ms_per_step": round(ms, 4), "gb_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                "frac_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "layer_tok_s": round(m / (ms * 1e-3), 1), "kernel_us": per, "weight_copies_rotated": copies}

    w64 = {l.name: synth.weights(l.w_seed, l.n, l.k) for l in wl.linears}
    fused = run([("|".join(l.name for l in g), sum(l.n for l in g), g[0].k, s,
                  np.concatenate([w64[l.name] for l in g], axis=0)) for s, g in groups.items()], "fused")
    separate = run([(l.name, l.n, l.k, l.x_seed, w64[l.name]) for l in wl.linears], "separate")
    out = {"workload": wl.name, "m": m, "packed_bytes_per_step": nbytes}
    out.update(fused)
    out["separate_linears"] = separate
    out["compute"] = ("LDS partial-sum table, FP32" if m == 1 else
                      "v_mfma_f32_16x16x32_f16 (x' as two fp16 parts in the A rows, fp16 trit codes, FP32 accumulate)")
    # The block's three floors beside its measured step: HBM (packed bytes at
    # the peak), the matrix cores (2 M N K flops; M >= 2 issues them twice,
    # for the hi and lo parts of x', at the dense fp16 peak) and the FP32
    # vector ALU (the same flops at its peak), in microseconds.
    flops = 2.0 * m * sum(l.n * l.k for l in wl.linears)
    out["floors_us"] = {"hbm": round(nbytes / (HBM_PEAK_GBS * 1e9) * 1e6, 2),
                        "mfma_fp16": round((flops * (2 if m > 1 else 1)) / (MFMA_F16_PEAK_TFLOPS * 1e12) * 1e6, 2),
                        "valu_fp32": round(flops / (VALU_F32_PEAK_TFLOPS * 1e12) * 1e6, 2),
                        "measured": round(fused["ms_per_step"] * 1e3, 2)}
    return out


def extra_variants(tq, torch, synth, np):
    """The format variants on the single-stream decode step's two linears
    (up 5120 -> 17408, down 17408 -> 5120): ternary at group 64, and binary
    {-c, +c} at group 128 and 64, at M = 1 and M = 8.  Each variant's own
    algorithmic bytes (words + scales) over the kernel time; weights
    quantised on the GPU from the same seeded matrices, rotated over copies
    of >= 1 GiB."""
    lins = synth.DENSE_DECODE_27B.linears
    w64s = [synth.weights(l.w_seed, l.n, l.k) for l in lins]
    out = []
    for name, group, levels in (("ternary-g64", 64, 3), ("binary-g128", 128, 2), ("binary-g64", 64, 2)):
        base = []
        for lin, w64 in zip(lins, w64s):
            wt = torch.from_numpy(w64).cuda()
            t = torch.empty((lin.n, lin.k), dtype=torch.int8, device="cuda")
            sc = torch.empty((lin.n, lin.k // group), dtype=torch.int16, device="cuda")
            tq.tq_quantize(wt, lin.n, lin.k, group, levels, t, sc)
            del wt
            w = tq.empty_weights(lin.n, lin.k, group=group, levels=levels)
            tq.tq_pack(t, lin.n, lin.k, tq.TQ_LAYOUT_ROW64, levels, w.words)
            tq.tq_pack_scales(sc, lin.n, lin.k, tq.TQ_LAYOUT_ROW64, group, w.scales)
            base.append(w)
        torch.cuda.synchronize()
        nbytes = [tq.tq_format_bytes(l.n, l.k, group, levels) for l in lins]
        copies = max(1, -(-ROTATE_BYTES // sum(nbytes)))
        sets = [base] + [[w.clone() for w in base] for _ in range(copies - 1)]
        row = {"variant": name, "group": group, "levels": levels, "bytes_per_step": sum(nbytes),
               "weight_copies_rotated": copies}
        for m in (1, 8):
            xs = [bf16(torch, synth.activations(l.x_seed, m, l.k, "bf16")) for l in lins]
            ys = [torch.zeros((m, l.n), dtype=torch.float32, device="cuda") for l in lins]
            us = []
            for j in range(len(lins)):
                g = capture(torch, copies, lambda i: tq.tq_gemv(sets[i][j], xs[j], m, ys[j],
                                                                 tq.TQ_FWHT_FUSED | tq.TQ_ACCUMULATE))
                g.replay()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                g.replay()
                b.record()
                torch.cuda.synchronize()
                us.append(1e3 * a.elapsed_time(b) / copies)
            gbs = sum(nbytes) / (sum(us) * 1e-6) / 1e9
            row[f"m{m}"] = {"kernel_us": {l.name: round(u, 3) for l, u in zip(lins, us)}, "gb_s": round(gbs, 1),
                            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                            "layer_tok_s": round(m / (sum(us) * 1e-6), 1)}
        del sets
        torch.cuda.empty_cache()
        out.append(row)
    return out


def extra_block_m1(tq, torch, synth, np):
    return extra_block(tq, torch, synth, np, synth.DENSE_BLOCK_M1)


def extra_block_m8(tq, torch, synth, np):
    return extra_block(tq, torch, synth, np, synth.DENSE_BLOCK_M8)


def extra_moe(tq, torch, synth, np):
    out = []
    wl = synth.MOE_T1
    E, H, I = wl.experts, wl.hidden, wl.inter
    w_gu = tq.empty_weights(2 * I, H, num_experts=E)
    w_dn = tq.empty_weights(H, I, num_experts=E)
    for e in range(E):
        gu64, dn64 = synth.expert_weights(e, H, I)
        quantize_pack(tq, torch, gu64, 2 * I, H, w_gu, e)
        quantize_pack(tq, torch, dn64, H, I, w_dn, e)
    torch.cuda.synchronize()
    per_expert = tq.tq_packed_bytes(2 * I, H) + tq.tq_packed_bytes(H, I)
    copies = max(1, -(-ROTATE_BYTES // (E * per_expert)))
    sets = [(w_gu, w_dn)] + [(clone_w(tq, w_gu), clone_w(tq, w_dn)) for _ in range(copies - 1)]
    for wl in (synth.MOE_T1, synth.MOE_T64):
        T = wl.tokens
        lg = torch.from_numpy(synth.logits(wl.logit_seed, T, E)).cuda()
        ids = torch.empty((T, wl.topk), dtype=torch.int32, device="cuda")
        rw = torch.empty((T, wl.topk), dtype=torch.float32, device="cuda")
        tq.tq_moe_route(lg, T, E, wl.topk, ids, rw)
        x = bf16(torch, synth.activations(wl.x_seed, T, H, "bf16"))
        y = torch.empty((T, H), dtype=torch.float32, device="cuda")
        ws, nb = tq.workspace(tq.TQ_OP_MOE, w_gu, T, wl.topk)
        active = len(set(ids.cpu().numpy().ravel().tolist()))

        def step(i, flags=tq.TQ_FWHT_FUSED):
            g, d = sets[i % copies]
            tq.tq_moe_gemv(g, d, x, T, wl.topk, ids, rw, y, flags, ws, nb)
        ms = timed(torch, 50, 5, step)
        ms_acc = timed(torch, 50, 5, lambda i: step(i, tq.TQ_FWHT_FUSED | tq.TQ_ACCUMULATE))
        bytes_ = active * per_expert
        row = {"workload": wl.name, "tokens": T, "active_experts": active, "expert_bytes_read": bytes_,
               "weight_copies_rotated": copies, "us_per_layer": round(ms * 1e3, 2),
               "us_per_layer_accumulate": round(ms_acc * 1e3, 2),
               "gb_s": round(bytes_ / (ms * 1e-3) / 1e9, 1), "tok_s": round(T / (ms * 1e-3), 1),
               "launches": 2 if T * wl.topk <= 64 else 4}  # per-pair launches up to 64 pairs
        if T * wl.topk <= 64:  # the one-launch form (its counters start zeroed in this workspace)
            ms1 = timed(torch, 50, 5, lambda i: step(i, tq.TQ_FWHT_FUSED | tq.TQ_MOE_ONE_LAUNCH))
            row["us_per_layer_one_launch"] = round(ms1 * 1e3, 2)
        out.append(row)
    return out


def extra_gemm(tq, torch, synth, np):
    wl = synth.PREFILL_GEMM
    lin = wl.linears[0]
    w = quantize_pack(tq, torch, synth.weights(lin.w_seed, lin.n, lin.k), lin.n, lin.k)
    x = bf16(torch, synth.activations(lin.x_seed, wl.m, lin.k, "bf16"))
    y = torch.empty((wl.m, lin.n), dtype=torch.float32, device="cuda")
    ws, nb = tq.workspace(tq.TQ_OP_GEMM, w, wl.m)
    ms = timed(torch, 10, 2, lambda i: tq.tq_gemm(w, x, wl.m, y, tq.TQ_FWHT_FUSED, ws, nb))
    ms_fast = timed(torch, 10, 2, lambda i: tq.tq_gemm(w, x, wl.m, y, tq.TQ_FWHT_FUSED | tq.TQ_FAST_F16, ws, nb))
    useful = 2.0 * wl.m * lin.n * lin.k
    return {"workload": wl.name, "ms": round(ms, 4), "tok_s": round(wl.m / (ms * 1e-3), 1),
            "useful_tflops": round(useful / (ms * 1e-3) / 1e12, 1),
            "frac_f16_mfma_peak_useful": round(useful / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
            "mfma_tflops_hi_lo": round(2 * useful / (ms * 1e-3) / 1e12, 1),
            "frac_f16_mfma_peak": round(2 * useful / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
            "compute": "v_mfma_f32_16x16x32_f16, x' split into fp16 hi + lo A rows, B = fp16 s*t decoded into registers, FP32 accumulate",
            "fast_f16": {"ms": round(ms_fast, 4), "tok_s": round(wl.m / (ms_fast * 1e-3), 1),
                         "useful_tflops": round(useful / (ms_fast * 1e-3) / 1e12, 1),
                         "frac_f16_mfma_peak": round(useful / (ms_fast * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
                         "compute": "TQ_FAST_F16: x' as one fp16 part (128 tokens per workgroup), rel-L2 ~3e-4"}}


def extra_kv(tq, torch, synth, np):
    """TurboQuant KV cache at 128K tokens, 8 KV heads, 4 queries per head,
    3 bits: quantisation of the whole cache (prefill rate), then one decode
    step's scores and value sums over copies of the cache rotated past the
    caches (>= 1 GiB).  Algorithmic bytes: every record, radius and gamma
    once, plus the scores written (scores) or the weights read (values);
    the fused attend (softmax folded into the value sums) reads the scores
    in place of the weights, the same bytes."""
    wl = synth.KV_DECODE_128K
    n, H, G, bits = wl.tokens, wl.heads, wl.queries, wl.bits
    signs = torch.from_numpy(synth.kv_signs(wl.sign_seed)).cuda()
    jl = torch.from_numpy(synth.kv_jl(wl.jl_seed)).cuda()
    lk = torch.from_numpy(tq.tq_kv_codebook(bits - 1)).cuda()
    lv = torch.from_numpy(tq.tq_kv_codebook(bits)).cuda()
    rb = tq.tq_kv_record_bytes(bits)

    def cache():
        return (torch.empty((H * n, rb // 4), dtype=torch.int32, device="cuda"),
                torch.empty(H * n, dtype=torch.int16, device="cuda"),
                torch.empty(H * n, dtype=torch.int16, device="cuda"))
    kx = bf16(torch, synth.kv_vectors(wl.key_seed, H * n, 128, "bf16"))
    kc = cache()
    ms_qk = timed(torch, 3, 1, lambda i: tq.tq_kv_quantize(kx, H * n, signs, jl, lk, bits, True, *kc))
    del kx
    vx = bf16(torch, synth.kv_vectors(wl.value_seed, H * n, 128, "bf16"))
    vc = cache()
    ms_qv = timed(torch, 3, 1, lambda i: tq.tq_kv_quantize(vx, H * n, signs, None, lv, bits, False, vc[0], vc[1]))
    del vx
    torch.cuda.synchronize()
    cache_bytes = H * n * (2 * rb + 6)
    copies = max(1, -(-ROTATE_BYTES // cache_bytes))
    sets = [(kc, vc)] + [(tuple(t.clone() for t in kc), tuple(t.clone() for t in vc)) for _ in range(copies - 1)]
    q = torch.from_numpy(synth.kv_vectors(wl.query_seed, H * G, 128, "f32").raw.astype(np.float32)).cuda()
    scores = torch.empty((H, G, n), dtype=torch.float32, device="cuda")
    out = torch.empty((H, G, 128), dtype=torch.float32, device="cuda")
    ws_s, nb_s = tq.kv_workspace(tq.TQ_KV_OP_SCORES, n, H, G)
    ws_v, nb_v = tq.kv_workspace(tq.TQ_KV_OP_VALUES, n, H, G)

    def score(i):
        k = sets[i % copies][0]
        tq.tq_kv_scores(q, H, G, k[0], k[1], k[2], n, bits, signs, jl, lk, scores, ws_s, nb_s)
    ms_s = timed(torch, copies, 2, score)
    p = torch.softmax(scores / float(np.sqrt(128.0)), dim=-1).contiguous()

    def values(i):
        v = sets[i % copies][1]
        tq.tq_kv_values(p, H, G, v[0], v[1], n, bits, signs, lv, out, ws_v, nb_v)
    ms_v = timed(torch, copies, 2, values)
    ms_sm = timed(torch, 10, 2, lambda i: torch.softmax(scores, dim=-1))
    ws_a, nb_a = tq.kv_workspace(tq.TQ_KV_OP_ATTEND, n, H, G)
    scale = 1.0 / float(np.sqrt(128.0))

    def attend(i):
        v = sets[i % copies][1]
        tq.tq_kv_attend(scores, scale, H, G, v[0], v[1], n, bits, signs, lv, out, ws_a, nb_a)
    ms_a = timed(torch, copies, 2, attend)
    b_s = H * n * (rb + 4) + H * G * n * 4
    b_v = H * n * (rb + 2) + H * G * n * 4
    row = lambda ms, b: {"us": round(ms * 1e3, 2), "bytes": b, "gb_s": round(b / (ms * 1e-3) / 1e9, 1),
                         "frac_hbm_peak": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    fp16_bytes = 2 * H * n * 128 * 2
    return {"workload": wl.name, "tokens": n, "kv_heads": H, "queries_per_head": G, "bits": bits,
            "cache_bytes": cache_bytes, "fp16_cache_bytes": fp16_bytes,
            "compression_vs_fp16": round(fp16_bytes / cache_bytes, 3), "cache_copies_rotated": copies,
            "scores": row(ms_s, b_s), "values": row(ms_v, b_v), "attend": row(ms_a, b_v),
            "softmax_torch_us": round(ms_sm * 1e3, 2),
            "decode_attention_us": round((ms_s + ms_v + ms_sm) * 1e3, 2),
            "decode_attention_fused_us": round((ms_s + ms_a) * 1e3, 2),
            "quantize_keys": {"ms": round(ms_qk, 3), "vectors_per_s": round(H * n / (ms_qk * 1e-3), 1)},
            "quantize_values": {"ms": round(ms_qv, 3), "vectors_per_s": round(H * n / (ms_qv * 1e-3), 1)},
            "note": "a workgroup serves the 4 query heads of a KV head, so each record is fetched once per "
                    "call; the query launch (scores) and the chunk-sum launch (values, attend) are included; "
                    "decode_attention_us = scores + torch softmax + values, decode_attention_fused_us = scores + "
                    "attend"}


def extra_format(tq, torch, synth, np):
    """The format kernels at the up projection's size (17408 x 5120), HBM
    bytes each moves over its time: quantise (FP32 weights in; trits and
    fp16 scales out), pack and unpack in the ROW64 layout, the scale
    re-layout; and the standalone block-128 transform of a prefill batch
    (2048 x 5120 bf16 in, FP32 out).  Offline conversion except the
    transform."""
    lin = synth.DENSE_DECODE_27B.linears[0]
    n, k = lin.n, lin.k
    w = torch.from_numpy(synth.weights(lin.w_seed, n, k).astype(np.float32)).cuda()
    t = torch.empty((n, k), dtype=torch.int8, device="cuda")
    sc = torch.empty((n, k // 128), dtype=torch.int16, device="cuda")
    wts = tq.empty_weights(n, k)
    t2 = torch.empty_like(t)
    rows = {}

    def row(name, ms, nbytes):
        gbs = nbytes / (ms * 1e-3) / 1e9
        rows[name] = {"us": round(ms * 1e3, 2), "bytes": nbytes, "gb_s": round(gbs, 1),
                      "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    row("quantize_f32", timed(torch, 5, 1, lambda i: tq.tq_quantize(w, n, k, 128, 3, t, sc)),
        n * k * 4 + n * k + n * (k // 128) * 2)
    wb = tq.tq_packed_bytes(n, k) - tq.tq_layout_scales(n, k, tq.TQ_LAYOUT_ROW64, 128) * 2
    row("pack_row64", timed(torch, 10, 1, lambda i: tq.tq_pack(t, n, k, tq.TQ_LAYOUT_ROW64, 3, wts.words)),
        n * k + wb)
    row("pack_scales_row64", timed(torch, 10, 1, lambda i: tq.tq_pack_scales(sc, n, k, tq.TQ_LAYOUT_ROW64, 128,
                                                                              wts.scales)),
        2 * n * (k // 128) * 2)
    row("unpack_row64", timed(torch, 10, 1, lambda i: tq.tq_unpack(wts.words, n, k, tq.TQ_LAYOUT_ROW64, 3, t2)),
        wb + n * k)
    del w
    m = 2048
    x = bf16(torch, synth.activations(5002, m, k, "bf16"))
    xr = torch.empty((m, k), dtype=torch.float32, device="cuda")
    row("fwht_bf16_to_f32", timed(torch, 20, 2, lambda i: tq.tq_fwht(x, m, k, xr)), m * k * 2 + m * k * 4)
    return {"workload": f"format-{n}x{k}", "rows": n, "cols": k, "fwht_rows": m, "kernels": rows,
            "note": "one launch each, timed in a graph of back-to-back launches on the same buffers"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the decode GEMV shards by "
              "output rows with no reduction across GPUs).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import synth
    import ternary_weight_quantized_tq_amd as tq

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    if args.only_extra:
        fn = {"block_m1": extra_block_m1, "block_m8": extra_block_m8, "moe": extra_moe,
              "prefill_gemm": extra_gemm, "variants": extra_variants, "kv_cache": extra_kv,
              "format": extra_format}[args.only_extra]
        print(json.dumps({args.only_extra: fn(tq, torch, synth, np)}), flush=True)
        return

    if args.copy_calibration:
        src = torch.empty(64 << 20, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4, "launches": 5}))
        return

    wl = synth.DENSE_DECODE_27B
    lins = wl.linears
    log("building weights ...")
    base, w64s = [], []
    for lin in lins:
        w64 = synth.weights(lin.w_seed, lin.n, lin.k)
        base.append(quantize_pack(tq, torch, w64, lin.n, lin.k))
        w64s.append(w64)
    torch.cuda.synchronize()
    lin_bytes = [tq.tq_packed_bytes(l.n, l.k) for l in lins]
    step_bytes = sum(lin_bytes)
    copies = max(1, -(-ROTATE_BYTES // step_bytes))
    sets = [base] + [[clone_w(tq, w) for w in base] for _ in range(copies - 1)]
    xs = [bf16(torch, synth.activations(l.x_seed, 1, l.k, "bf16")) for l in lins]
    y_all = torch.empty(sum(l.n for l in lins), dtype=torch.float32, device="cuda")
    ys = [y_all[:lins[0].n].view(1, -1), y_all[lins[0].n:].view(1, -1)]
    log(f"weights ready: {copies} copies x {step_bytes / 1e6:.1f} MB")

    def step(i, evs=None):
        y_all.zero_()
        for j, w in enumerate(sets[i % copies]):
            if evs is not None:
                evs[j][0].record()
            tq.tq_gemv(w, xs[j], 1, ys[j], tq.TQ_FWHT_FUSED | tq.TQ_ACCUMULATE)
            if evs is not None:
                evs[j][1].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # The timed steps run as one HIP graph so that host launch cost does not
    # pace the GPU.  (HIP graphs on ROCm take no timing events as nodes.)
    g = capture(torch, args.steps, step)
    g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    g.replay()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    # Mean launch time of each GEMV: a graph of its back-to-back launches over
    # the rotated copies, HIP events on its stream around the replay, divided
    # by the launch count.
    kernel_timing = "graph of back-to-back launches of one linear, divided by the launch count"
    mean_us = []
    for j in range(len(lins)):
        kg = capture(torch, copies, lambda i: tq.tq_gemv(sets[i][j], xs[j], 1, ys[j],
                                                          tq.TQ_FWHT_FUSED | tq.TQ_ACCUMULATE))
        kg.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        kg.replay()
        b.record()
        torch.cuda.synchronize()
        mean_us.append(1e3 * a.elapsed_time(b) / copies)
    # Isolated launches: eager, each between two events on an otherwise idle
    # stream, so each time includes the dispatch and ramp-up that back-to-back
    # launches overlap (context; per-kernel percentiles come from the trace).
    per = [[] for _ in lins]
    for i in range(args.steps):
        for j in range(len(lins)):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            tq.tq_gemv(sets[i % copies][j], xs[j], 1, ys[j], tq.TQ_FWHT_FUSED | tq.TQ_ACCUMULATE)
            b.record()
            per[j].append((a, b))
    torch.cuda.synchronize()
    spread = {l.name: [round(float(np.percentile([1e3 * a.elapsed_time(b) for a, b in v], q)), 3) for q in (10, 50, 90)]
              for l, v in zip(lins, per)}
    # Context for the roofline: a plain device copy moving the same bytes per
    # launch (half read, half written), timed the same way, sources rotated.
    half = lin_bytes[0] // 8
    srcs = [sets[i][0].words.view(-1)[:half] for i in range(copies)]
    dst = torch.empty(half, dtype=srcs[0].dtype, device="cuda")
    cg = capture(torch, copies, lambda i: dst.copy_(srcs[i]))
    cg.replay()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    cg.replay()
    b.record()
    torch.cuda.synchronize()
    copy_us = 1e3 * a.elapsed_time(b) / copies
    # The read ceiling at this launch size: one plain read pass over the
    # bytes of one GEMV launch (16-byte non-temporal loads, the GEMV's load
    # form), over rotated buffers, timed the same way.
    rd_bytes = lin_bytes[0] // 16 * 16
    rd_stride = (rd_bytes + 255) // 256 * 256
    rd_copies = max(1, -(-ROTATE_BYTES // rd_stride))
    rd_buf = torch.ones(rd_copies * rd_stride // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    rd = lambda i: tq.tq_read_bytes(rd_buf.data_ptr() + i * rd_stride, rd_bytes, sink)
    for i in range(rd_copies):
        rd(i)
    rg = capture(torch, rd_copies, rd)
    rg.replay()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    rg.replay()
    b.record()
    torch.cuda.synchronize()
    read_us = 1e3 * a.elapsed_time(b) / rd_copies
    del rd_buf
    # The same step on one copy of the weights (no rotation): they then sit
    # in the 256 MB Infinity Cache, so this shows the kernels off HBM.
    hot = capture(torch, args.steps, lambda i: step(0))
    hot.replay()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    hot.replay()
    b.record()
    torch.cuda.synchronize()
    hot_ms = a.elapsed_time(b) / args.steps
    # The default deterministic path (no TQ_ACCUMULATE): per-slice partials
    # in a workspace, then the reduction launch in slice order.
    wss = [tq.workspace(tq.TQ_OP_GEMV, w, 1) for w in base]

    def det_step(i):
        for j, w in enumerate(sets[i % copies]):
            tq.tq_gemv(w, xs[j], 1, ys[j], tq.TQ_FWHT_FUSED, wss[j][0], wss[j][1])
    det_ms = timed(torch, args.steps, args.warmup, det_step)
    gbs = step_bytes / (ms * 1e-3) / 1e9
    kern_gbs = sum(lin_bytes) / (sum(mean_us) * 1e-6) / 1e9
    traffic = measured_traffic()

    result = {
        "metric": "packed-weight HBM GB/s (% of peak) for ternary GEMV at M=1/8; layer tok/s",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,0.02^2) weights with 0.1% x20 outliers, quantised and packed on the GPU; "
                "N(0,1) bf16 activations)",
        "config": {"workload": wl.name, "linears": [f"{l.name} {l.k}->{l.n}" for l in lins], "m": 1,
                   "x_dtype": "bf16", "weight_copies_rotated": copies, "packed_bytes_per_step": step_bytes,
                   "output": "one zero-fill per step, then each GEMV accumulates (TQ_ACCUMULATE)"},
        "layer_tok_s": round(1e3 / ms, 1),
        "frac_hbm_peak_step": round(gbs / HBM_PEAK_GBS, 4),
        "kernel_us": {l.name: round(u, 3) for l, u in zip(lins, mean_us)},
        "kernel_timing": kernel_timing,
        "isolated_launch_us_p10_p50_p90": spread,
        "deterministic_step": {"ms_per_step": round(det_ms, 5),
                               "gb_s": round(step_bytes / (det_ms * 1e-3) / 1e9, 1),
                               "note": "default flags: partials in a workspace + the in-order reduction launch"},
        "mall_hot_single_copy": {"ms_per_step": round(hot_ms, 5),
                                 "gb_s": round(step_bytes / (hot_ms * 1e-3) / 1e9, 1),
                                 "note": "one weight copy, cache-resident; not the metric"},
        "plain_copy_same_bytes": {"bytes_moved": 8 * half, "us": round(copy_us, 3),
                                  "gb_s": round(8 * half / (copy_us * 1e-6) / 1e9, 1),
                                  "frac_hbm_peak": round(8 * half / (copy_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        "read_only_same_bytes": {"bytes_read": rd_bytes, "us": round(read_us, 3),
                                 "gb_s": round(rd_bytes / (read_us * 1e-6) / 1e9, 1),
                                 "frac_hbm_peak": round(rd_bytes / (read_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                 "buffers_rotated": rd_copies,
                                 "note": "one plain read pass (tq_read_bytes) over one launch's bytes: the read "
                                         "ceiling at this launch size; context"},
        "roofline": {"bound": "hbm", "achieved": round(kern_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(kern_gbs / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic)},
    }
    if not args.no_extras:
        extras = {}
        for name, fn in (("block_m1", extra_block_m1), ("block_m8", extra_block_m8), ("moe", extra_moe),
                         ("prefill_gemm", extra_gemm), ("variants", extra_variants), ("kv_cache", extra_kv),
                         ("format", extra_format)):
            log(f"extra: {name} ...")
            try:
                extras[name] = fn(tq, torch, synth, np)
            except Exception as e:  # report, never hide
                extras[name] = {"error": f"{type(e).__name__}: {e}"}
        result["extras"] = extras
    if not args.no_cpu:
        from oracle import tq_oracle as O
        log("timing the CPU oracle ...")
        result["cpu_baseline"] = cpu_baseline(O, synth, lins, w64s, args.cpu_seconds)
        if not args.no_extras:
            log("timing the CPU oracle on prefill GEMM rows ...")
            try:
                result["cpu_baseline"]["prefill_gemm_rows"] = cpu_gemm_rows(O, synth)
            except Exception as e:  # report, never hide
                result["cpu_baseline"]["prefill_gemm_rows"] = {"error": f"{type(e).__name__}: {e}"}
            log("timing the CPU oracle on the MoE layer (T = 1) and a KV sample ...")
            try:
                result["cpu_baseline"]["moe_t1"] = cpu_moe_t1(O, synth)
            except Exception as e:  # report, never hide
                result["cpu_baseline"]["moe_t1"] = {"error": f"{type(e).__name__}: {e}"}
            try:
                from oracle import kv_oracle as K
                result["cpu_baseline"]["kv_sample"] = cpu_kv_sample(K, synth)
            except Exception as e:  # report, never hide
                result["cpu_baseline"]["kv_sample"] = {"error": f"{type(e).__name__}: {e}"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
