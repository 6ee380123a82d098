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
            matvec) on a bounded row sample, in packed-weight GB/s
  isolated_launch_us_p10_p50_p90  one GEMV launched alone between two HIP
            events (dispatch and ramp-up included; context)
  mall_hot_single_copy   the same step on one weight copy (cache-resident,
            labelled; context, not the metric)

`extras` adds the other workloads: one transformer block's seven linears at
M = 1 (single stream) and M = 8, the 256-expert MoE layer at T = 1 and
T = 64, and the prefill GEMM.
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
    p.add_argument("--only-extra", choices=["block_m1", "block_m8", "moe", "prefill_gemm"],
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
    tq.tq_quantize(wt, n, k, trits, scales)
    del wt
    w = w_out if w_out is not None else tq.empty_weights(n, k)
    nw, ns = tq.tq_layout_words(n, k, tq.TQ_LAYOUT_ROW64), tq.tq_layout_scales(n, k, tq.TQ_LAYOUT_ROW64)
    tq.tq_pack(trits, n, k, tq.TQ_LAYOUT_ROW64, w.words.data_ptr() + 4 * nw * expert)
    tq.tq_pack_scales(scales, n, k, tq.TQ_LAYOUT_ROW64, w.scales.data_ptr() + 2 * ns * expert)
    return w


def bf16(torch, act):
    import numpy as np
    return torch.from_numpy(act.raw.view(np.int16)).cuda().view(torch.bfloat16)


def clone_w(tq, w):
    return tq.Weights(w.words.clone(), w.scales.clone(), w.n, w.k, w.layout, w.num_experts)


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


def cpu_baseline(O, synth, lins, w64s, seconds):
    """Oracle unpack + transform + matvec on row samples, repeated for about
    `seconds`; reported as packed bytes per second."""
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    samples = []
    for lin, w64 in zip(lins, w64s):
        rows = 1024 if lin.k <= 8192 else 512
        t, s, _ = O.quantize(w64[:rows])
        x = synth.activations(lin.x_seed, 1, lin.k, "bf16").values
        samples.append((O.pack(t), s, lin.k, x, O.packed_bytes(rows, lin.k), rows))
    def run(budget):
        done, t0, reps = 0, time.perf_counter(), 0
        while True:
            for words, s, k, x, nbytes, _ in samples:
                O.gemv(words, s, k, x, True)
                done += nbytes
            reps += 1
            if time.perf_counter() - t0 >= budget:
                break
        dt = time.perf_counter() - t0
        return done / dt / 1e9, reps, dt

    gbs, reps, dt = run(seconds)
    try:  # the same sample on one thread, for a third of the time
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            gbs1, reps1, dt1 = run(seconds / 3)
        one = {"value": round(gbs1, 4), "reps": reps1, "seconds": round(dt1, 1)}
    except Exception as e:  # report, never hide
        one = {"error": f"{type(e).__name__}: {e}"}
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    desc = " + ".join(f"{smp[5]} rows of {lin.name} ({lin.n}x{lin.k})" for smp, lin in zip(samples, lins))
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{desc}, repeated {reps}x over {dt:.1f} s (FP64 unpack + dense block-128 transform + "
                      f"dequantised matvec), packed bytes per second",
            "one_thread": one, "cpu_model": model}


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
        out.append({"workload": wl.name, "tokens": T, "active_experts": active, "expert_bytes_read": bytes_,
                    "weight_copies_rotated": copies, "us_per_layer": round(ms * 1e3, 2),
                    "us_per_layer_accumulate": round(ms_acc * 1e3, 2),
                    "gb_s": round(bytes_ / (ms * 1e-3) / 1e9, 1), "tok_s": round(T / (ms * 1e-3), 1),
                    "launches": 2 if T * wl.topk <= 64 else 4})  # per-pair launches up to 64 pairs
    return out


def extra_gemm(tq, torch, synth, np):
    wl = synth.PREFILL_GEMM
    lin = wl.linears[0]
    w = quantize_pack(tq, torch, synth.weights(lin.w_seed, lin.n, lin.k), lin.n, lin.k)
    x = bf16(torch, synth.activations(lin.x_seed, wl.m, lin.k, "bf16"))
    y = torch.empty((wl.m, lin.n), dtype=torch.float32, device="cuda")
    ws, nb = tq.workspace(tq.TQ_OP_GEMM, w, wl.m)
    ms = timed(torch, 10, 2, lambda i: tq.tq_gemm(w, x, wl.m, y, tq.TQ_FWHT_FUSED, ws, nb))
    useful = 2.0 * wl.m * lin.n * lin.k
    return {"workload": wl.name, "ms": round(ms, 4), "tok_s": round(wl.m / (ms * 1e-3), 1),
            "useful_tflops": round(useful / (ms * 1e-3) / 1e12, 1),
            "mfma_tflops_hi_lo": round(2 * useful / (ms * 1e-3) / 1e12, 1),
            "frac_f16_mfma_peak": round(2 * useful / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
            "compute": "v_mfma_f32_16x16x32_f16, x' split into fp16 hi + lo A rows, B = fp16 s*t decoded into registers, FP32 accumulate"}


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
              "prefill_gemm": extra_gemm}[args.only_extra]
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
        "mall_hot_single_copy": {"ms_per_step": round(hot_ms, 5),
                                 "gb_s": round(step_bytes / (hot_ms * 1e-3) / 1e9, 1),
                                 "note": "one weight copy, cache-resident; not the metric"},
        "plain_copy_same_bytes": {"bytes_moved": 8 * half, "us": round(copy_us, 3),
                                  "gb_s": round(8 * half / (copy_us * 1e-6) / 1e9, 1),
                                  "frac_hbm_peak": round(8 * half / (copy_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        "roofline": {"bound": "hbm", "achieved": round(kern_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(kern_gbs / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic)},
    }
    if not args.no_extras:
        extras = {}
        for name, fn in (("block_m1", extra_block_m1), ("block_m8", extra_block_m8), ("moe", extra_moe),
                         ("prefill_gemm", extra_gemm)):
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
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
