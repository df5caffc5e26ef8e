#!/usr/bin/env python3
"""Benchmark of the predictor-gated sparse FFN decode step on one MI355X.

A step is one decode token through one FFN layer: predict (h = A x, logits, threshold,
compaction) then the sparse FFN over the predicted neurons, as one psffn_layer call.  The timed
steps are replayed from HIP graphs (64 steps per graph); a second pass times the two halves
(psffn_predict, psffn_sparse_ffn), each replayed from a graph of the same steps, with HIP events for the
per-call breakdown.  The default workload is the
OPT-30B-shaped ReLU layer: d = 7168, F = 28672, predictor rank 1024, fp16 weights with fp32
accumulation, batch 1, Zipf(1.1) firing at mean density 0.03, neurons permuted hot-first by a
512-token profile.  Weights are random (synthetic); inputs are resident in HBM before timing.

To measure HBM and not the 256 MB Infinity Cache, the steps rotate over `--copies` independent
copies of the layer (8 copies: ~7 GB, the predictor alone 590 MB), as a decode through a deep
layer stack would.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-FFN µs/layer and achieved HBM GB/s (% of roofline) at batch 1"
HBM_PEAK_GBPS = 8000.0


# HBM bytes per psffn_layer step (every kernel of the call), from two rocprofv3 --pmc passes over
# this script (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch, summed over the step's kernels and
# averaged over the steps).  A plain device copy of 512 MiB reads as 262156 KiB of FETCH_SIZE and
# 524288 KiB of WRITE_SIZE, so FETCH_SIZE is scaled by 2.0 and WRITE_SIZE by 1.0.  A figure holds
# only for the kernel sources it was measured on (hash below); after any change to them the
# traffic is reported as null until measured again.
TRAFFIC_SOURCES = ("activation_sparse_ffn_psffn_amd/csrc/common.h", "activation_sparse_ffn_psffn_amd/csrc/chunk.h",
                   "activation_sparse_ffn_psffn_amd/csrc/fused.hip", "activation_sparse_ffn_psffn_amd/csrc/stream.hip")
BATCH_TRAFFIC_SOURCES = ("activation_sparse_ffn_psffn_amd/csrc/common.h", "activation_sparse_ffn_psffn_amd/csrc/batch.hip")
TRAFFIC = {
    # profiles/opt30b_relu_f16_b1_hbm_traffic.md: k_h1 + k_qu + k_dn, 1.038x the algorithmic bytes
    ("opt30b_relu_f16", 1): {"sources": "5c0be3841a1ba240", "bytes": 101962538},
    # profiles/opt175b_relu_i4_b1_hbm_traffic.md: k_h1 + k_qu + k_dn (4-bit rows), 1.046x
    ("opt175b_relu_i4", 1): {"sources": "5c0be3841a1ba240", "bytes": 217132358},
    # profiles/llama2_13b_swiglu_f16_b1_hbm_traffic.md: k_h1 + k_q + k_ud + k_reduce_ud, 1.040x
    ("llama2_13b_swiglu_f16", 1): {"sources": "5c0be3841a1ba240", "bytes": 292497549},
    # profiles/falcon40b_stack_f16_b1_hbm_traffic.md: per layer call, k_h with the LayerNorm + k_qu + k_dn, 1.035x
    ("falcon40b_stack_f16", 1): {"sources": "5c0be3841a1ba240", "bytes": 157800685},
    # profiles/opt175b_relu_i4_b8_hbm_traffic.md: the eight batch kernels, 1.17x
    ("opt175b_relu_i4", 8): {"files": BATCH_TRAFFIC_SOURCES, "sources": "4381b58d6eb1cfba", "bytes": 318682435},
}


def sources_hash(files=TRAFFIC_SOURCES):
    """Hash of the traffic sources with comments and whitespace removed: an edit to comments alone
    leaves the kernels, and so the figure, unchanged."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f)) as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload, B):
    rec = TRAFFIC.get((workload, B))
    if rec is None or rec["sources"] != sources_hash(rec.get("files", TRAFFIC_SOURCES)):
        return None
    return rec["bytes"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# A bounded GPU spin queued right before a start event: the host then enqueues the event and the
# timed graph replays while the GPU is still busy, so the events time the K steps on the GPU and not
# the host's launch latency before the first of them (which a short run, such as 20 steps in one
# graph, would otherwise spread over its steps).  About a millisecond at the shader clock.
SPIN_CYCLES = 2_000_000


def gpu_busy(torch):
    torch.cuda._sleep(SPIN_CYCLES)


def graph_plan(steps, graph_steps):
    """Partition of the K timed steps into consecutive captured HIP graphs: (first step, length)
    pairs covering [0, steps) in order.  Full graphs of graph_steps steps, then one shorter graph
    for the remainder; graph_steps <= 0 means no graphs (eager launches: an empty plan)."""
    if steps < 1:
        raise ValueError("steps must be >= 1")
    if graph_steps <= 0:
        return []
    plan, t = [], 0
    while t < steps:
        n = min(graph_steps, steps - t)
        plan.append((t, n))
        t += n
    return plan


def host_cpu():
    """(logical CPUs this process may use, CPU model name) of the host the bench runs on."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return n, model


def device_copy_gbps(torch, mib=512, reps=5, trials=3):
    """The GPU's measured copy bandwidth, as context for the fraction of the 8 TB/s nominal peak: a
    device-to-device copy of `mib` MiB (read + written bytes) timed with events over `reps` copies,
    the best of `trials` such batches."""
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    st = torch.cuda.current_stream()
    best = float("inf")
    for _ in range(trials):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gpu_busy(torch)
        e0.record(st)
        for _ in range(reps):
            dst.copy_(src)
        e1.record(st)
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) / reps)
    del src, dst
    return round(2 * n / (best * 1e-3) / 1e9, 1)


def hot_prefix_len(counts, tokens, p_hot):
    """Length of the hot prefix of a hot-first layer (the neurons computed without prediction): the
    number of neurons whose profiled firing frequency counts[i] / tokens is at least p_hot.  counts
    are in the layer's hot-first order, so these are exactly the first ones."""
    if tokens < 1 or not (0.0 < p_hot <= 1.0):
        raise ValueError("hot_prefix_len: tokens >= 1 and 0 < p_hot <= 1")
    c = counts.detach().to("cpu").long()
    need = math.ceil(p_hot * tokens - 1e-9)
    n = int((c >= need).sum().item())
    if n and int(c[:n].min().item()) < need:
        raise ValueError("hot_prefix_len: counts are not in hot-first (descending) order")
    return n


def algorithmic_bytes(spec, B, n_active, n_hot=0):
    """Bytes the method must move for one step with n_active listed neurons (per-step mean).
    With a hot prefix, the small-batch predictor (fp32 up to 4 tokens; fp16 at 1 token, and at 2
    up to 1024 ranks) reads the Q rows and biases of the other F - n_hot neurons only."""
    e_p = 4 if spec.storage == "f32" else 2
    e_x = 4 if spec.storage == "f32" else 2
    d, F, r = spec.d, spec.F, spec.r
    small = B <= 4 if spec.storage == "f32" else (B == 1 or (B == 2 and r <= 1024))
    Fq = F - n_hot if small else F
    pred = (r * d + Fq * r) * e_p + 4 * Fq + B * d * e_x
    if spec.storage == "i4":
        rowb = d // 2 + 2 * (d // 128)
    else:
        rowb = d * e_x
    m = 3 if spec.act == "swiglu" else 2
    rows = m * n_active * rowb + 4 * n_active
    out = B * d * 4
    return pred, rows + out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1024)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--copies", type=int, default=8)
    ap.add_argument("--workload", default="opt30b_relu_f16")
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU oracle baseline: decode steps are timed until about this much CPU time is spent")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="CPU oracle baseline: at most this many decode steps (0: every token of the workload)")
    ap.add_argument("--no-events", action="store_true", help="skip the per-call event pass")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-MiB buffer 8 times with a plain device copy and exit (reference "
                         "kernel of known traffic for scaling hardware byte counters)")
    ap.add_argument("--hot", type=float, default=0.0, metavar="P_HOT",
                    help="hot prefix: neurons profiled to fire on at least this fraction of the profile tokens "
                         "are computed without prediction (psffn_layer_hot); the layer is profiled and permuted "
                         "hot-first first.  0 = off")
    ap.add_argument("--study", default="", choices=["", "predictor", "sizing", "drift"],
                    help="predictor: accuracy and speed of predictors aligned with the layer (rank-r "
                         "approximations of the deciding weights) at several ranks, against the generated one")
    ap.add_argument("--ranks", default="128,256,512,1024", help="ranks of the aligned predictors (--study)")
    ap.add_argument("--sizing-tokens", type=int, default=16, help="calibration tokens per layer (--study sizing)")
    ap.add_argument("--sizing-price", type=float, default=1.0,
                    help="--study sizing: MB of predictor worth spending to find one more firing neuron per token")
    ap.add_argument("--graph-steps", type=int, default=64,
                    help="steps per captured HIP graph in the timed region (0: eager launches)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        log("bench.py: measures one GPU only (the path is a single-GPU decode step); "
            "--gpus %d is not supported" % args.gpus)
        sys.exit(2)

    import numpy as np
    import torch

    import activation_sparse_ffn_psffn_amd as ps
    import synth

    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(8):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "copies": 8}), flush=True)
        return

    spec = synth.CONFIGS[args.workload]
    B = args.batch
    dev = "cuda"
    torch.cuda.init()
    if args.study == "predictor":
        return bench_study(args, spec, ps, synth, np, torch)
    if args.study == "sizing":
        return bench_sizing(args, spec, ps, synth, np, torch)
    if args.study == "drift":
        return bench_drift(args, spec, ps, synth, np, torch)
    if spec.layers > 1:
        return bench_stack(args, spec, ps, synth, np, torch)
    log("workload", spec.name, "B", B)
    t0 = time.time()
    L = synth.make_layer(spec, seed=0, device=dev)
    W = ps.FFN(spec.act, L.w_up, L.w_dT, w_gate=L.w_gate, s_up=L.s_up, s_gate=L.s_gate, s_dT=L.s_dT, b_up=L.b_up,
               b_gate=L.b_gate, b_down=L.b_down)
    P = ps.Predictor(L.A, L.Q, L.c)
    n_hot = 0
    if spec.hot_first or args.hot > 0:
        T = spec.profile_tokens or 512
        Xp = synth.make_tokens(spec, T, seed=0, stream="profile", device=dev)
        counts = ps.profile_counts(W, Xp)
        perm, W, P = ps.permute_hot_first(counts, W, P)
        if args.hot > 0:
            n_hot = hot_prefix_len(counts[perm.long()], T, args.hot)
            log("hot prefix: %d neurons fire on >= %.3f of %d profile tokens" % (n_hot, args.hot, T))
        del Xp, L
    torch.cuda.synchronize()
    log("layer ready in %.1f s" % (time.time() - t0))

    def clone(W, P):
        c = lambda t: None if t is None else t.clone()
        return (ps.FFN(W.act, c(W.w_up), c(W.w_dT), w_gate=c(W.w_gate), s_up=c(W.s_up), s_gate=c(W.s_gate),
                       s_dT=c(W.s_dT), b_up=c(W.b_up), b_gate=c(W.b_gate), b_down=c(W.b_down)),
                ps.Predictor(c(P.A), c(P.Q), c(P.c)))

    copies = [(W, P)] + [clone(W, P) for _ in range(args.copies - 1)]
    ntok = spec.tokens
    X = synth.make_tokens(spec, ntok * B, seed=0, device=dev).reshape(ntok, B, spec.d)
    ws = ps.new_workspace(P, W, B)
    F = spec.F
    idx = torch.empty(F, dtype=torch.int32, device=dev)
    K, Wm = args.steps, args.warmup
    counts_all = torch.zeros(K, dtype=torch.int32, device=dev)
    y = torch.empty(B, spec.d, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    def step(t, cnt, stream):
        # one decode step of one layer: predict + sparse FFN in one library call
        Wc, Pc = copies[t % len(copies)]
        ps.layer(Pc, Wc, X[t % ntok], ws, idx=idx, count=cnt, y=y, stream=stream, n_hot=n_hot)

    scratch_cnt = torch.zeros(1, dtype=torch.int32, device=dev)
    for t in range(Wm):
        step(t, scratch_cnt, stream)
    torch.cuda.synchronize()

    # the timed region: K steps replayed from HIP graphs of G consecutive steps (distinct tokens,
    # rotating layer copies), so that host launch overhead is not part of the step
    plan = graph_plan(K, args.graph_steps)
    graphs = []
    if plan:
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        for g0, gn in plan:
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.stream(cap):
                with torch.cuda.graph(gr, stream=cap):
                    for t in range(g0, g0 + gn):
                        step(Wm + t, counts_all[t:t + 1], cap)
            graphs.append(gr)
        stream.wait_stream(cap)
        torch.cuda.synchronize()
        graphs[0].replay()  # warm the replay path (outside the timed region)
        torch.cuda.synchronize()
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    gpu_busy(torch)
    e_start.record(stream)
    if graphs:
        for gr in graphs:
            gr.replay()
    else:
        for t in range(K):
            step(Wm + t, counts_all[t:t + 1], stream)
    e_end.record(stream)
    torch.cuda.synchronize()
    total_ms = e_start.elapsed_time(e_end)
    us_per_step = total_ms * 1e3 / K

    counts_np = counts_all.cpu().numpy().astype(np.float64)
    n_mean = float(counts_np.mean())
    pred_bytes, ffn_bytes = algorithmic_bytes(spec, B, n_mean, n_hot)
    step_bytes = pred_bytes + ffn_bytes
    layer_gbps = step_bytes / (us_per_step * 1e-6) / 1e9

    # per-call durations with HIP events on the launch stream: the same K steps as two calls,
    # psffn_predict then psffn_sparse_ffn on its list, each call sequence captured in a HIP graph
    # and timed over its replay (no host launch gaps, like the timed region)
    roof = None
    breakdown = None
    if not args.no_events:
        idx_all = torch.empty(K, F, dtype=torch.int32, device=dev)
        cnt_all = torch.zeros(K, dtype=torch.int32, device=dev)
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        g_pred, g_ffn = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g_pred, stream=cap):
                for t in range(K):
                    Wc, Pc = copies[(Wm + t) % len(copies)]
                    ps.predict(Pc, X[(Wm + t) % ntok], ws, idx=idx_all[t], count=cnt_all[t:t + 1], stream=cap,
                               n_hot=n_hot)
            with torch.cuda.graph(g_ffn, stream=cap):
                for t in range(K):
                    Wc, Pc = copies[(Wm + t) % len(copies)]
                    ps.sparse_ffn(Wc, X[(Wm + t) % ntok], idx_all[t], cnt_all[t:t + 1], ws, y=y, stream=cap)
        stream.wait_stream(cap)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        g_pred.replay()  # lists for the FFN replay, and warm
        torch.cuda.synchronize()
        gpu_busy(torch)
        ev[0].record(stream)
        g_pred.replay()
        ev[1].record(stream)
        g_ffn.replay()
        ev[2].record(stream)
        torch.cuda.synchronize()
        pred_us = ev[0].elapsed_time(ev[1]) * 1e3 / K
        ffn_us = ev[1].elapsed_time(ev[2]) * 1e3 / K
        breakdown = {"predict_us": round(pred_us, 3), "sparse_ffn_us": round(ffn_us, 3),
                     "two_call_step_us": round(pred_us + ffn_us, 3),
                     "predict_bytes": int(pred_bytes), "sparse_ffn_bytes": int(ffn_bytes),
                     "predict_gbps": round(pred_bytes / (pred_us * 1e-6) / 1e9, 1),
                     "sparse_ffn_gbps": round(ffn_bytes / (ffn_us * 1e-6) / 1e9, 1)}
        del g_pred, g_ffn, idx_all

    # the roofline covers the timed launch sequence itself: one psffn_layer call per step, its
    # algorithmic bytes over its average duration (HIP events on the stream the calls run on)
    traffic = measured_traffic(spec.name, B) if not n_hot else None
    roof = {"bound": "hbm", "achieved": round(layer_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(layer_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
            "kernel": "psffn_layer (%s)" % layer_kernels(spec, B),
            "bytes_per_launch": int(step_bytes), "avg_launch_us": round(us_per_step, 3)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(spec, copies[0], X, B, args.cpu_tokens, args.cpu_seconds)

    out = {
        "metric": METRIC, "value": round(us_per_step, 3), "unit": "us/layer", "n_gpus": 1, "steps": K,
        "warmup": Wm, "ms_per_step": round(total_ms / K, 6), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16" if spec.storage != "f32" else "f32", "data": "synthetic",
        "config": {"workload": "%s: d=%d F=%d r=%d %s %s batch %d, Zipf(%.1f) density %.2f%s, %d layer copies" % (
            spec.name, spec.d, spec.F, spec.r, spec.storage, spec.act, B, spec.zipf, spec.density,
            ", hot-first" if (spec.hot_first or n_hot) else "", len(copies)) + (
            ", hot prefix of %d neurons (profiled firing >= %g) computed without prediction" % (n_hot, args.hot)
            if n_hot else ""), "batch": B, "d": spec.d, "F": spec.F, "r": spec.r, "n_hot": n_hot},
        "layer": {"gbps": round(layer_gbps, 1), "frac_of_hbm_peak": round(layer_gbps / HBM_PEAK_GBPS, 4),
                  "algorithmic_bytes_per_step": int(step_bytes), "mean_active": round(n_mean, 2),
                  "tokens_per_s": round(1e6 / us_per_step * B, 1), "breakdown": breakdown,
                  "device_copy_gbps": device_copy_gbps(torch)},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def layer_kernels(spec, B, ln=False):
    """The kernels one psffn_layer (ln: psffn_layer_ln) call launches for this workload and batch (as
    the library picks its pipeline: small-batch kernels at one token and for the shapes they take,
    MFMA batch kernels otherwise)."""
    if ln and B == 1 and spec.storage == "f16" and spec.act == "relu" and spec.d <= 8192:
        return "k_h with the LayerNorm, k_qu, k_dn"
    if ln and B == 2 and spec.storage == "f16" and spec.act == "relu" and spec.r <= 1024:
        return "k_h with the LayerNorm, k_q, k_ud, k_reduce_ud"
    if ln and B > 1:
        return "the LayerNorm kernel, then " + layer_kernels(spec, B)
    if B == 1 and spec.storage == "f16" and spec.act == "relu" and spec.d <= 8192:
        return "k_h1, k_qu, k_dn"
    if B == 1 and spec.storage == "i4" and spec.act == "relu" and spec.d <= 16384:
        return ("k_h1, " if spec.d <= 12288 else "k_h, ") + "k_qu (4-bit up rows), k_dn (4-bit rows)"
    if B == 1 or spec.storage == "f32":
        return "k_h, k_q, k_ud, k_reduce_ud"
    pred_batch = B > 4 or B >= 3 or spec.r > 1024
    ffn_batch = B > 4 or spec.storage == "i4" or (spec.act == "relu" and B >= 3)
    if pred_batch and ffn_batch and B <= 32 and spec.r <= 1536:
        if spec.storage == "i4":
            return "MFMA batch kernels: k_bh, k_bhred, k_bq_full, k_bscan, k_bup, k_bact, k_bdown, k_breduce"
        if spec.act == "relu":
            return "MFMA batch kernels: k_bh, k_bhred, k_bq_full, k_bup (orders the list), k_bact, k_bdown, k_breduce"
    return "small-batch or MFMA batch kernels by batch size"


def bench_stack(args, spec, ps, synth, np, torch):
    """Decode through a stack of FFN layers: per layer x <- x + FFN(fp16(LayerNorm(x))), the FFN
    restricted to the batch's predicted union set; one step moves B tokens through all layers.
    Reported as tokens/s through the stack (higher is better)."""
    B, dev, L = args.batch, "cuda", spec.layers
    t0 = time.time()
    layers = []
    for l in range(L):
        Ly = synth.make_layer(spec, seed=0, layer=l, device=dev)
        layers.append((ps.Predictor(Ly.A, Ly.Q, Ly.c), ps.FFN(spec.act, Ly.w_up, Ly.w_dT, b_up=Ly.b_up), Ly.p))
        del Ly
    torch.cuda.synchronize()
    log("stack of %d layers ready in %.1f s" % (L, time.time() - t0))
    P0, W0, _ = layers[0]
    ws = ps.new_workspace(P0, W0, B)
    F, d = spec.F, spec.d
    idx = torch.empty(F, dtype=torch.int32, device=dev)
    cnts = torch.zeros(L, dtype=torch.int32, device=dev)
    x0 = synth.make_residual(spec, B, seed=0, device=dev)
    x = x0.clone()
    hbuf = torch.empty(B, d, dtype=torch.float16, device=dev)
    stream = torch.cuda.current_stream()

    def step(st):
        for l, (P, W, _) in enumerate(layers):
            # x <- x + FFN(fp16(LayerNorm(x))) in one library call
            ps.layer_ln(P, W, x, ws, eps=1e-5, h=hbuf, idx=idx, count=cnts[l:l + 1], stream=st)

    for _ in range(max(1, args.warmup)):
        step(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            step(cap)
    stream.wait_stream(cap)
    g.replay()
    torch.cuda.synchronize()
    K = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gpu_busy(torch)
    e0.record(stream)
    for _ in range(K):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    tok_s = B / (ms * 1e-3)
    n = cnts.cpu().numpy().astype(np.float64)
    byt = sum(sum(algorithmic_bytes(spec, B, n[l])) for l in range(L))
    # the union a batch of B independent tokens would have: sum_i 1 - (1 - p_i)^B per layer
    exp_union = [float((1.0 - (1.0 - pl) ** B).sum()) for (_, _, pl) in layers]
    gbps = byt / (ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": measured_traffic(spec.name, B),
            "kernel": "psffn_layer_ln (%s), 48 calls per step" % layer_kernels(spec, B, ln=True),
            "bytes_per_launch": int(byt / L), "avg_launch_us": round(ms * 1e3 / L, 3)}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_stack(spec, layers, x0, B, L, budget_s=args.cpu_seconds)
    out = {"metric": "decode tokens/s through a stack of sparse FFN layers", "value": round(tok_s, 1),
           "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(ms, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
           "config": {"workload": "%s: %d layers d=%d F=%d r=%d f16 relu, batch %d, per-layer density U(0.02,0.10) "
                                  "Zipf(1.0), residual + LayerNorm between layers" % (spec.name, L, d, F, spec.r, B),
                      "batch": B},
           "layer": {"us_per_layer": round(ms * 1e3 / L, 3), "gbps": round(gbps, 1),
                     "device_copy_gbps": device_copy_gbps(torch),
                     "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                     "mean_union_active_per_layer": round(float(n.mean()), 1),
                     "union_active_per_layer_min_max": [int(n.min()), int(n.max())],
                     "mean_union_if_tokens_independent": round(float(np.mean(exp_union)), 1),
                     "algorithmic_bytes_per_step": int(byt)},
           "roofline": roof, "cpu_baseline": cpu}
    print(json.dumps(out), flush=True)


def cpu_baseline_stack(spec, layers, x0, B, L, budget_s=12.0):
    """The oracle timed on this host on a bounded sample of the stack: layer by layer from the
    stack's input (x <- x + FFN(fp16(LayerNorm(x))) per layer), until about budget_s seconds of CPU
    work or every layer is done; the mean time per layer is scaled to the whole stack."""
    import numpy as np

    import oracle

    oracle.build()
    g = lambda t: t.detach().cpu().numpy()
    x = x0.cpu().numpy()
    spent, done = 0.0, 0
    for l in range(L):
        P, W, _ = layers[l]
        lay = [(g(P.A), g(P.Q), g(P.c), oracle.Layer(spec.act, g(W.w_up), g(W.w_dT), b_up=g(W.b_up)))]
        t0 = time.perf_counter()
        x = oracle.stack_step(lay, x)
        spent += time.perf_counter() - t0
        done += 1
        if spent >= budget_s:
            break
    per_layer = spent / done
    log("cpu baseline: %d of %d layers in %.2f s" % (done, L, spent))
    nproc, model = host_cpu()
    return {"value": round(B / (per_layer * L), 4), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "host_nproc": nproc, "host_cpu": model,
            "sample": "the first %d of %d layers at batch %d (LayerNorm, predict, compact, sparse FFN, residual), "
                      "time per layer scaled to the %d-layer stack; single-threaded fp64 C (one of the host's %d "
                      "logical CPUs)" % (done, L, B, L, nproc)}


def set_stats(pred_idx, fired):
    """Recall and precision of a predicted neuron list against the truly firing set (bool [F])."""
    import numpy as np
    hit = int(fired[pred_idx].sum()) if len(pred_idx) else 0
    nf, npred = int(fired.sum()), len(pred_idx)
    return (hit / nf if nf else 1.0), (hit / npred if npred else 1.0)


def cosine(a, b):
    import numpy as np
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    return float(a @ b / (na * nb)) if na > 0 and nb > 0 else float(na == nb)


def bench_drift(args, spec, ps, synth, np, torch):
    """Drift of the decode stack from the oracle (reported, not graded): the GPU chain (psffn_layer_ln
    per layer) and the oracle's own chain (oracle.stack_step, fp64) from the same x0, one layer at a
    time, with ||x_gpu - x_oracle||inf / ||x_oracle||inf and the two sets' symmetric difference after
    every layer (a set may differ inside the logit band, and the chains then go their own ways)."""
    import oracle

    B, dev, L = args.batch, "cuda", spec.layers
    x0 = synth.make_residual(spec, B, seed=7, device=dev)
    x = x0.clone()
    xr = x0.cpu().numpy()
    g = lambda t: t.detach().cpu().numpy()
    rows = []
    t0 = time.time()
    for l in range(L):
        Ly = synth.make_layer(spec, seed=0, layer=l, device=dev)
        P, W = ps.Predictor(Ly.A, Ly.Q, Ly.c), ps.FFN(spec.act, Ly.w_up, Ly.w_dT, b_up=Ly.b_up)
        ws = ps.new_workspace(P, W, B)
        idx, cnt, h = ps.layer_ln(P, W, x, ws)
        torch.cuda.synchronize()
        gpu_set = g(idx[:int(cnt.item())])
        A, Q, c = g(Ly.A), g(Ly.Q), g(Ly.c)
        orc = oracle.Layer(spec.act, g(Ly.w_up), g(Ly.w_dT), b_up=g(Ly.b_up))
        h_ref = oracle.round_to_f16(oracle.layernorm(xr))
        ref_set = oracle.compact(oracle.predict_logits(A, Q, c, h_ref))
        xr = oracle.stack_step([(A, Q, c, orc)], xr)
        xg = g(x).astype(np.float64)
        drift = float(np.abs(xg - xr).max() / max(np.abs(xr).max(), 1e-30))
        rows.append({"layer": l, "rel_drift": drift, "set_sym_diff": int(len(np.setxor1d(gpu_set, ref_set))),
                     "count": int(len(gpu_set))})
        log("layer %2d drift %.3e set diff %d (%d listed)" % (l, drift, rows[-1]["set_sym_diff"], len(gpu_set)))
        del Ly, P, W, ws, orc, A, Q, c
    print(json.dumps({"study": "decode-stack drift from the oracle", "workload": spec.name, "layers": L, "batch": B,
                      "final_rel_drift": rows[-1]["rel_drift"], "max_rel_drift": max(r["rel_drift"] for r in rows),
                      "seconds": round(time.time() - t0, 1), "per_layer": rows}), flush=True)


def bench_sizing(args, spec, ps, synth, np, torch):
    """Per-layer predictor sizing for the decode stack (Elamur summary, Interesting ideas I3: each
    layer's predictor is sized by that layer's sparsity and skew).

    For every layer: the predictor aligned with the layer (synth.make_aligned_predictor) at the
    configured rank r_max, and its leading-r truncations for r in --ranks; recall of the predicted set
    against the neurons that truly fire, on --sizing-tokens calibration tokens (psffn_predict and
    psffn_profile_counts on each token).  The layer's rank r_l grows from the smallest rank tried to
    the next while the firing neurons the larger predictor additionally finds per token,
    (recall(r') - recall(r)) x the layer's mean firing count, are worth its extra bytes at a price of
    --sizing-price MB of predictor per neuron found: a layer with more firing neurons (lower
    sparsity) or firing spread over more neurons (lower skew) gains more from a larger predictor and
    gets one, a sparse, skewed layer keeps a small one.  Then the whole stack
    (x <- x + FFN(fp16(LN(x))), psffn_layer_ln per layer, one HIP graph per step) is timed with the
    aligned predictors at r_max and at r_l, and both are reported with the recall they give."""
    B, dev, L = args.batch, "cuda", spec.layers
    d, F = spec.d, spec.F
    ranks = sorted({int(v) for v in args.ranks.split(",") if v} | {spec.r})
    T = args.sizing_tokens
    Xc = synth.make_tokens(spec, T, seed=1, stream="profile", device=dev).reshape(T, 1, d)
    t0 = time.time()
    layers, rows = [], []
    for l in range(L):
        Ly = synth.make_layer(spec, seed=0, layer=l, device=dev)
        W = ps.FFN(spec.act, Ly.w_up, Ly.w_dT, b_up=Ly.b_up)
        A, Q, c = synth.make_aligned_predictor(Ly, spec.r, seed=l)
        if l == 0:
            ws = ps.new_workspace(ps.Predictor(A, Q, c), W, max(B, 1))
        fired = [ps.profile_counts(W, Xc[t]).cpu().numpy() > 0 for t in range(T)]
        n_fire = float(np.mean([f.sum() for f in fired]))
        rec = {}
        preds = {}
        for r in ranks:
            P = ps.Predictor(A[:r].contiguous(), Q[:, :r].contiguous(), c)
            preds[r] = P
            vals = []
            for t in range(T):
                idx, cnt = ps.predict(P, Xc[t], ws)
                vals.append(set_stats(idx[:int(cnt.item())].cpu().numpy(), fired[t])[0])
            rec[r] = float(np.mean(vals))
        r_l = ranks[0]
        for r_next in ranks[1:]:
            found = (rec[r_next] - rec[r_l]) * n_fire  # extra firing neurons found per token
            cost_mb = (r_next - r_l) * (d + F) * 2 / 1e6  # extra predictor bytes (fp16 A rows + Q columns)
            if found * args.sizing_price < cost_mb:
                break
            r_l = r_next
        layers.append((preds[spec.r], preds[r_l], W))
        rows.append({"layer": l, "density": round(synth.layer_density(spec, 0, l), 4), "rank": r_l,
                     "mean_firing": round(n_fire, 1),
                     "recall_by_rank": {str(r): round(v, 4) for r, v in rec.items()}})
        log("layer %2d density %.4f recall %s -> rank %d" % (l, rows[-1]["density"], rows[-1]["recall_by_rank"], r_l))
        del Ly, A, Q
    log("sizing done in %.1f s" % (time.time() - t0))
    x0 = synth.make_residual(spec, B, seed=0, device=dev)
    hbuf = torch.empty(B, d, dtype=torch.float16, device=dev)
    idx = torch.empty(F, dtype=torch.int32, device=dev)
    cnts = torch.zeros(L, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def timed(which):
        x = x0.clone()

        def step(st):
            for l, lay in enumerate(layers):
                ps.layer_ln(lay[which], lay[2], x, ws, eps=1e-5, h=hbuf, idx=idx, count=cnts[l:l + 1], stream=st)

        step(stream)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                step(cap)
        stream.wait_stream(cap)
        g.replay()
        torch.cuda.synchronize()
        K = max(1, min(args.steps, 64))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gpu_busy(torch)
        e0.record(stream)
        for _ in range(K):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        del g
        return B / (e0.elapsed_time(e1) / K * 1e-3)

    tok_full, tok_sized = timed(0), timed(1)
    esz = 2
    pbytes = lambda r: (r * d + F * r) * esz + 4 * F
    full_b = sum(pbytes(spec.r) for _ in range(L))
    sized_b = sum(pbytes(rw["rank"]) for rw in rows)
    out = {"study": "per-layer predictor sizing (aligned predictors)", "workload": spec.name, "layers": L, "batch": B,
           "calibration_tokens": T, "price_mb_per_neuron": args.sizing_price, "ranks_tried": ranks,
           "ranks": [rw["rank"] for rw in rows], "densities": [rw["density"] for rw in rows],
           "mean_recall_at_rmax": round(float(np.mean([rw["recall_by_rank"][str(spec.r)] for rw in rows])), 4),
           "mean_recall_sized": round(float(np.mean([rw["recall_by_rank"][str(rw["rank"])] for rw in rows])), 4),
           "predictor_bytes_per_step_rmax": full_b, "predictor_bytes_per_step_sized": sized_b,
           "tokens_per_s_rmax": round(tok_full, 1), "tokens_per_s_sized": round(tok_sized, 1), "per_layer": rows}
    print(json.dumps(out), flush=True)


def bench_study(args, spec, ps, synth, np, torch):
    """Predictor accuracy against predictor size (one layer, batch 1).

    For the generated predictor (independent of the weights, equal firing rates) and for
    predictors aligned with the layer at each rank of --ranks (synth.make_aligned_predictor):
    recall and precision of the predicted set against the neurons that truly fire (the ReLU or
    gate pre-activation > 0, from psffn_profile_counts on each token alone), the cosine between the
    predicted-set output and the dense FFN output (psffn_sparse_ffn over every neuron), and the
    layer time (psffn_layer, graph replay over 8 rotating copies of the layer).  Every step runs
    in the library's kernels; the statistics are host arithmetic on their outputs."""
    dev = "cuda"
    t0 = time.time()
    L = synth.make_layer(spec, seed=0, device=dev)
    W = ps.FFN(spec.act, L.w_up, L.w_dT, w_gate=L.w_gate, b_up=L.b_up, b_gate=L.b_gate, b_down=L.b_down)
    F, d = spec.F, spec.d
    T = min(64, spec.tokens)
    X = synth.make_tokens(spec, T, seed=0, device=dev).reshape(T, 1, d)
    ws = ps.new_workspace(ps.Predictor(L.A, L.Q, L.c), W, 1)
    all_idx = torch.arange(F, dtype=torch.int32, device=dev)
    all_cnt = torch.tensor([F], dtype=torch.int32, device=dev)
    fired, dense = [], []
    for t in range(T):
        fired.append(ps.profile_counts(W, X[t]).cpu().numpy() > 0)
        dense.append(ps.sparse_ffn(W, X[t], all_idx, all_cnt, ws).cpu().numpy())
    log("layer and dense outputs ready in %.1f s" % (time.time() - t0))
    variants = [("generated", spec.r, (L.A, L.Q, L.c))]
    for r in [int(v) for v in args.ranks.split(",") if v]:
        variants.append(("aligned", r, synth.make_aligned_predictor(L, r)))
    esz = 4 if spec.storage == "f32" else 2
    copies_w = [W] + [ps.FFN(spec.act, L.w_up.clone(), L.w_dT.clone(), w_gate=None if L.w_gate is None else
                             L.w_gate.clone(), b_up=L.b_up, b_gate=L.b_gate) for _ in range(7)]
    rows = []
    for kind, r, (A, Q, c) in variants:
        P = ps.Predictor(A, Q, c)
        rec, prec, cos, nact = [], [], [], []
        for t in range(T):
            idx, cnt, y = ps.layer(P, W, X[t], ws)
            n = int(cnt.item())
            rc, pr = set_stats(idx[:n].cpu().numpy(), fired[t])
            rec.append(rc)
            prec.append(pr)
            cos.append(cosine(y.cpu().numpy(), dense[t]))
            nact.append(n)
        # timing: 8 rotating copies (FFN weights and predictor), graph replay of K steps
        Ps = [P] + [ps.Predictor(A.clone(), Q.clone(), c.clone()) for _ in range(7)]
        K = 256
        idx = torch.empty(F, dtype=torch.int32, device=dev)
        cnt = torch.zeros(1, dtype=torch.int32, device=dev)
        y = torch.empty(1, d, dtype=torch.float32, device=dev)
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(gr, stream=cap):
                for k in range(K):
                    ps.layer(Ps[k % 8], copies_w[k % 8], X[k % T], ws, idx=idx, count=cnt, y=y, stream=cap)
        torch.cuda.current_stream().wait_stream(cap)
        gr.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gpu_busy(torch)
        e0.record()
        gr.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / K
        del gr, Ps
        row = {"predictor": kind, "rank": r, "predictor_bytes": (r * d + F * r) * esz + 4 * F,
               "recall": round(float(np.mean(rec)), 4), "precision": round(float(np.mean(prec)), 4),
               "cosine_vs_dense": round(float(np.mean(cos)), 5), "mean_listed": round(float(np.mean(nact)), 1),
               "mean_firing": round(float(np.mean([f.sum() for f in fired])), 1), "us_per_layer": round(us, 3)}
        log(json.dumps(row))
        rows.append(row)
    print(json.dumps({"study": "predictor accuracy against rank", "workload": spec.name, "tokens": T, "batch": 1,
                      "rows": rows}), flush=True)


def cpu_baseline(spec, copy0, X, B, max_steps, budget_s):
    """The oracle (single-threaded fp64 C loops) timed on this host on decode steps of the same
    workload (predict, compact, sparse FFN over its own list), one after another until about
    `budget_s` seconds are spent, at most `max_steps` (0: every token) and at least one."""
    import numpy as np

    import oracle

    W, P = copy0
    g = lambda t: None if t is None else t.detach().cpu().numpy()
    A, Q, c = g(P.A), g(P.Q), g(P.c)
    lay = oracle.Layer(spec.act, g(W.w_up), g(W.w_dT), w_gate=g(W.w_gate), s_up=g(W.s_up), s_gate=g(W.s_gate),
                       s_dT=g(W.s_dT), b_up=g(W.b_up), b_gate=g(W.b_gate), b_down=g(W.b_down))
    n = X.shape[0] if max_steps <= 0 else min(max_steps, X.shape[0])
    Xn = X[:n].cpu().numpy()
    oracle.build()
    t0 = time.perf_counter()
    ntok = 0
    while ntok < n:
        oracle.predicted_layer(A, Q, c, lay, Xn[ntok])
        ntok += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    log("cpu baseline: %d steps in %.2f s" % (ntok, dt))
    nproc, model = host_cpu()
    return {"value": round(dt / ntok * 1e6, 1), "unit": "us/layer", "cores": 1, "kind": "oracle",
            "host_nproc": nproc, "host_cpu": model,
            "sample": "%d decode steps (batch %d) of the same layer: predict, compact, sparse FFN; "
                      "single-threaded fp64 C (one of the host's %d logical CPUs)" % (ntok, B, nproc)}


if __name__ == "__main__":
    main()
