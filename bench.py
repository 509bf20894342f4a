#!/usr/bin/env python3
"""Medusa verify-step benchmark on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
medusa_heads -> medusa_tree_candidates -> medusa_tree_attention for every
layer (each layer on its own Q/K/V buffers) -> medusa_accept_paths.  All
inputs are resident in HBM before timing starts.  The step is captured once
as a HIP graph and replayed (the host never sits in the timed loop).  For the
per-stage and per-kernel figures every stage is captured as a graph of its
own and replayed between HIP events on the launch stream; the attention
stage's graph holds all layers, so its time / L is one layer's launch.  The
commit of the accepted path (medusa_commit_accepted, KV rollback over all
layers) closes a step in a decoding loop; it is timed as a stage of its own
and reported beside the step, not inside it.

Prints one JSON line (see the keys at the end of main()).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "verify steps/sec + tree_attention HBM GB/s & head-GEMM MFMA % of peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense bf16


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="zephyr7b-shaped",
                   help="default: the largest single-GPU workload (B=8, GQA, ctx 16384)")
    p.add_argument("--eager", action="store_true", help="time eager launches instead of a graph")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-layers", type=int, default=1,
                   help="attention layers the CPU oracle runs (scaled to all L layers)")
    p.add_argument("--cpu-seqs", type=int, default=1,
                   help="sequences of those layers the CPU oracle runs (scaled to all B)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="CPU work to time (whole sampled steps, repeated)")
    p.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                   help="run only a plain device copy of MIB MiB (4 times) and exit: the "
                        "calibration run for HBM byte counters")
    return p.parse_args()


def copy_probe(mib: int) -> None:
    """A plain device-to-device copy of known size, for scaling the HBM byte
    counters (FETCH_SIZE / WRITE_SIZE) of a profiler run."""
    import torch
    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(4):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n * 4, "repeats": 4}), flush=True)


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def read_probe(gib: int = 2, reps: int = 5) -> dict:
    """Read bandwidth of the library's streaming read probe
    (medusa_read_probe: every 16-byte piece of a buffer larger than the
    chip's last-level cache read once, coalesced), timed between two events
    on the launch stream; it sets the roofline's 8 TB/s beside what a
    streaming kernel reaches on this chip."""
    import torch
    from medusa_tree_verification_amd import api
    n = gib * (1 << 30) // 4
    x = torch.ones(n, dtype=torch.int32, device="cuda")
    parts = api.read_probe(x)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        api.read_probe(x, parts)
    e1.record()
    torch.cuda.synchronize()
    us = 1000.0 * e0.elapsed_time(e1) / reps
    del x
    torch.cuda.empty_cache()
    return {"gbs": round(n * 4 / (us * 1e-6) / 1e9, 1), "bytes": n * 4,
            "method": f"medusa_read_probe over {gib} GiB, {reps} launches"}


def counter_traffic(w, label: str, source: str):
    """HBM bytes per launch measured by the FETCH_SIZE / WRITE_SIZE counter runs
    recorded in profiles/hbm_counters_<workload>.txt (scaled by a plain copy
    of known size), or None when there is no record for this workload or the
    kernel source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"hbm_counters_{w.name}.txt")
    try:
        with open(path) as f:
            rec = [json.loads(l[len("record: "):]) for l in f if l.startswith("record: ")][-1]
        with open(os.path.join(ROOT, "medusa_tree_verification_amd", "csrc", source), "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, IndexError, ValueError):
        return None
    if rec.get("sources", {}).get(source) != sha:
        return None
    return rec.get("traffic_bytes_per_launch", {}).get(label)


def attention_bytes(w) -> int:
    """Algorithmic HBM bytes of one tree-attention layer: every K and V row of
    every sequence's context + tree (read once), Q read and O written once."""
    kv = w.B * w.Hkv * (w.ctx + w.T) * w.D * 2 * 2
    qo = 2 * w.B * w.T * w.Hq * w.D * 2
    return kv + qo


def heads_bytes(w) -> int:
    """Algorithmic HBM bytes of the heads: both weight matrices of every head
    read once (bf16) plus hidden in, r round trip and fp32 logits out."""
    weights = w.K * (w.H * w.H + w.H * w.V) * 2
    acts = w.B * w.H * 2 + 2 * w.K * w.B * w.H * 2 + w.B * w.K * w.V * 4
    return weights + acts


def heads_flops(w) -> int:
    return 2 * w.B * w.K * (w.H * w.H + w.H * w.V)


def build_step(w, dev):
    import torch
    from medusa_tree_verification_amd import api, synth

    log("generating inputs for", w.name)
    hidden, w1, wlm = synth.head_inputs(w, dev)
    parent, rank = synth.cost_ordered_tree(w.topk, w.T)
    tree = api.Tree(parent, rank, w.topk)
    root = synth.roots(w, dev)
    ctx = torch.full((w.B,), w.ctx, dtype=torch.int32, device=dev)
    # every layer's K/V in one [L][B][Hkv][S_cap][D] pair (own buffers per
    # layer, uniform layer stride for the commit)
    q0, k0, v0 = synth.attention_inputs(w, 0, dev)[:3]
    k_all = torch.empty((w.L,) + tuple(k0.shape), dtype=k0.dtype, device=dev)
    v_all = torch.empty_like(k_all)
    q_all = torch.empty((w.L,) + tuple(q0.shape), dtype=q0.dtype, device=dev)
    q_all[0], k_all[0], v_all[0] = q0, k0, v0
    del q0, k0, v0
    for l in range(1, w.L):
        q, k, v = synth.attention_inputs(w, l, dev)[:3]
        q_all[l], k_all[l], v_all[l] = q, k, v
        del q, k, v
    layers = [(q_all[l], k_all[l], v_all[l]) for l in range(w.L)]
    base = synth.normal((w.B, w.T, w.V), w.base_logit_std, synth.seed_for(w.cfg_id, synth.T_BASE), dev)
    ua = synth.uniform((w.B, w.T), synth.seed_for(w.cfg_id, synth.T_UACC), dev)
    us = synth.uniform((w.B, w.T), synth.seed_for(w.cfg_id, synth.T_USMP), dev)

    logits = torch.empty((w.B, w.K, w.V), dtype=torch.float32, device=dev)
    topk = torch.empty((w.B, w.K, tree.kmax), dtype=torch.int32, device=dev)
    toks = torch.empty((w.B, w.T), dtype=torch.int32, device=dev)
    pos = torch.empty((w.B, w.T), dtype=torch.int32, device=dev)
    out_all = torch.empty((w.L, w.B, w.T, w.Hq, w.D), dtype=torch.bfloat16, device=dev)
    outs = [out_all[l] for l in range(w.L)]
    acc_outs = {tau: (torch.empty(w.B, dtype=torch.int32, device=dev),
                      torch.empty((w.B, w.K + 1), dtype=torch.int32, device=dev),
                      torch.empty((w.B, w.K + 1), dtype=torch.int32, device=dev))
                for tau in w.temperature}

    def ws(n):
        return torch.zeros(max(n, 256), dtype=torch.uint8, device=dev)

    ws_heads = ws(api.heads_workspace_size(w.B, w.H, w.K, torch.bfloat16))
    ws_attn = ws(api.tree_attention_workspace_size(w.B, w.Hq, w.Hkv, w.D, w.ctx, tree, torch.bfloat16))
    ws_attn_layers = ws(api.tree_attention_layers_workspace_size(w.L, w.B, w.Hq, w.Hkv, w.D, w.ctx,
                                                                 tree, torch.bfloat16))
    ws_cand = ws(api.tree_candidates_workspace_size(w.B, w.V, tree))
    ws_acc = ws(max(api.accept_workspace_size(w.B, w.V, tree, t) for t in w.temperature))

    def stage_heads():
        api.heads(hidden, w1, wlm, logits=logits, ws=ws_heads)

    def stage_candidates():
        api.tree_candidates(logits, root, ctx, tree, topk, toks, pos, ws=ws_cand)

    def stage_attention(l):
        q, k, v = layers[l]
        api.tree_attention(q, k, v, ctx, w.ctx, tree, out=outs[l], ws=ws_attn)

    def stage_attention_batched():  # every layer in one grid (secondary figure)
        api.tree_attention_layers(q_all, k_all, v_all, ctx, w.ctx, tree, out=out_all,
                                  ws=ws_attn_layers)

    # dense variant of the heads (every tree row, M = B*T), a figure of its own
    dense_rows = synth.normal((w.B * w.T, w.H), 1.0, synth.seed_for(w.cfg_id, synth.T_HIDDEN, 0, 1), dev,
                              torch.bfloat16)
    dense_idx = torch.empty((w.B * w.T, w.K, tree.kmax), dtype=torch.int32, device=dev)
    dense_val = torch.empty((w.B * w.T, w.K, tree.kmax), dtype=torch.float32, device=dev)
    ws_dense = ws(api._lib.load().medusa_heads_dense_workspace_size(w.B * w.T, w.H, w.V, w.K, tree.handle, 1))

    def stage_heads_dense():
        api.heads_dense(dense_rows, w1, wlm, tree, outs=(dense_idx, dense_val), ws=ws_dense)

    def stage_accept():
        for tau, o in acc_outs.items():
            api.accept_paths(base, logits, toks, tree, ua, us, tau, outs=o, ws=ws_acc)

    ctx_next = torch.empty_like(ctx)
    root_next = torch.empty_like(root)
    acc0 = acc_outs[w.temperature[0]]

    def stage_commit():  # after the step: KV rollback / compaction of the accepted path
        api.commit_accepted(k_all, v_all, acc0[0], acc0[2], acc0[1], ctx, tree, ctx_next, root_next)

    def step():
        stage_heads()
        stage_candidates()
        for l in range(w.L):
            stage_attention(l)
        stage_accept()

    keep = dict(hidden=hidden, w1=w1, wlm=wlm, tree=tree, layers=layers, base=base)
    return step, (stage_heads, stage_candidates, stage_attention, stage_accept, stage_commit,
                  stage_attention_batched, stage_heads_dense), keep


def _capture(fn):
    """Capture fn's launches (on torch's current stream) as one HIP graph."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _time_mean(run, reps):
    """Mean ms per call of reps back-to-back calls of run(), between two
    events on the launch stream (nothing else inside the timed region)."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _time_each(run, reps):
    """ms of each of reps calls of run(), from an event recorded after every
    call (a separate pass: the events themselves add a little time between
    calls, so means come from _time_mean)."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        run()
        ev[i + 1].record()
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]


def _pct(xs, scale=1.0, nd=2):
    """p10 / median / p90 of xs (times scale)."""
    import numpy as np
    a = np.asarray(xs, dtype=np.float64) * scale
    return {"p10": round(float(np.percentile(a, 10)), nd), "p50": round(float(np.median(a)), nd),
            "p90": round(float(np.percentile(a, 90)), nd)}


def time_gpu(w, args):
    import torch

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    step, stages, keep = build_step(w, dev)
    torch.cuda.synchronize()
    (stage_heads, stage_candidates, stage_attention, stage_accept, stage_commit,
     stage_attention_batched, stage_heads_dense) = stages

    run = step if args.eager else _capture(step).replay
    log(f"warmup {args.warmup}, timing {args.steps} steps ({'eager' if args.eager else 'graph'})")
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    # exactly args.steps steps between two synchronisations and two events
    t_wall = time.perf_counter()
    ms_per_step = _time_mean(run, args.steps)
    wall_s = time.perf_counter() - t_wall
    # the per-step distribution from a second pass of as many steps, with an
    # event after every step (not part of the timed region above)
    step_ms = _time_each(run, args.steps)

    # per-stage figures: each stage captured as its own graph and replayed
    # between events on the launch stream (no host time inside)
    def all_layers():
        for l in range(w.L):
            stage_attention(l)

    graphs = {"heads": _capture(stage_heads), "candidates": _capture(stage_candidates),
              "attention": _capture(all_layers), "accept": _capture(stage_accept),
              "commit": _capture(stage_commit),
              "attention_batched": _capture(stage_attention_batched),
              "heads_dense": _capture(stage_heads_dense)}
    reps = max(5, args.steps)
    stages_us, stages_pct = {}, {}
    for n, g in graphs.items():
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        stages_us[n] = 1000.0 * _time_mean(g.replay, reps)
        stages_pct[n] = _pct(_time_each(g.replay, reps), 1000.0)
    attn_call_us = stages_us["attention"] / w.L
    return ms_per_step, wall_s, stages_us, attn_call_us, _pct(step_ms, 1.0, 4), stages_pct


def host_cpu() -> dict:
    """The host's CPU model (from /proc/cpuinfo) and logical core count."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "os_cpu_count": os.cpu_count()}


def cpu_baseline(w, n_layers, n_seqs, min_seconds=10.0, max_steps=40):
    """The oracle as it stands (NumPy, fp64: the precision its parity role
    fixes; it is not tuned for speed) on the host cores, on a bounded sample
    of one step of the same workload: heads, top-k/tree and acceptance in
    full, tree attention on n_layers layers of n_seqs sequences scaled by
    (L / n_layers) * (B / n_seqs) -- every layer and sequence has the same
    shape and they are independent.  Sampled steps are repeated until about
    min_seconds of CPU work have been timed."""
    import numpy as np
    import torch
    from medusa_tree_verification_amd import synth
    from oracle import accept as oaccept
    from oracle import attention as oattn
    from oracle import heads as oheads
    from oracle import topk as otopk
    from oracle import tree as otree

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    n_layers = max(1, min(n_layers, w.L))
    n_seqs = max(1, min(n_seqs, w.B))
    parent, rank = synth.cost_ordered_tree(w.topk, w.T)
    f64 = lambda t: t.to(torch.float64).numpy()
    hidden, w1, wlm = synth.head_inputs(w, "cpu")
    h64, w1_64, wlm64 = f64(hidden), f64(w1), f64(wlm)
    del w1, wlm
    layers = []
    for l in range(n_layers):
        q, k, v, ctx = synth.attention_inputs(w, l, "cpu")
        layers.append((f64(q[:n_seqs]), f64(k[:n_seqs]), f64(v[:n_seqs]), ctx.numpy()[:n_seqs]))
        del q, k, v
    base = synth.normal((w.B, w.T, w.V), w.base_logit_std, synth.seed_for(w.cfg_id, synth.T_BASE)).numpy()
    ua = synth.uniform((w.B, w.T), synth.seed_for(w.cfg_id, synth.T_UACC)).numpy()
    us = synth.uniform((w.B, w.T), synth.seed_for(w.cfg_id, synth.T_USMP)).numpy()
    roots = synth.roots(w, "cpu").numpy()
    scale_attn = (w.L / n_layers) * (w.B / n_seqs)
    tot = {"heads": 0.0, "candidates": 0.0, "attention": 0.0, "accept": 0.0}
    timed = 0.0
    steps = 0
    while steps < max_steps and (steps == 0 or timed < min_seconds):
        t0 = time.perf_counter()
        logits = oheads.medusa_heads(h64, w1_64, wlm64, round_r=w.dtype == "bf16")
        t1 = time.perf_counter()
        tk = otopk.head_topk(logits, w.topk)
        toks = otree.tree_tokens(tk, roots, parent, rank)
        vis = otree.visible_bruteforce(parent)
        t2 = time.perf_counter()
        for (qd, kd, vd, cl) in layers:
            oattn.tree_attention(qd, kd, vd, cl, vis)
        t3 = time.perf_counter()
        for tau in w.temperature:
            oaccept.accept_paths(base, logits, toks, parent, rank, ua, us, tau, w.K)
        t4 = time.perf_counter()
        tot["heads"] += t1 - t0
        tot["candidates"] += t2 - t1
        tot["attention"] += (t3 - t2) * scale_attn
        tot["accept"] += t4 - t3
        timed += t4 - t0
        steps += 1
    per_step = sum(tot.values()) / steps
    return {
        "value": 1.0 / per_step,
        "unit": "verify steps/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"{steps} sampled {w.name} step(s) in fp64 NumPy: heads, top-k/tree and "
                   f"acceptance in full; tree attention on {n_layers} of {w.L} layers x "
                   f"{n_seqs} of {w.B} sequences, scaled x{scale_attn:g} (layers and sequences "
                   f"are identical in shape and independent); {timed:.1f} s of CPU work timed"),
        "stage_s": {k: round(v / steps, 3) for k, v in tot.items()},
        "host": host_cpu(),
    }


def main():
    args = parse()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the library runs the "
              "verify step on one GPU and has no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    from medusa_tree_verification_amd import synth
    w = synth.WORKLOADS[args.workload]
    if w.dtype != "bf16":
        sys.exit("bench.py times the bf16 workloads")

    ms, wall_s, stages_us, attn_us, step_pct, stages_pct = time_gpu(w, args)
    a_bytes = attention_bytes(w)
    h_bytes = heads_bytes(w)
    attn_gbs = a_bytes / (attn_us * 1e-6) / 1e9
    heads_gbs = h_bytes / (stages_us["heads"] * 1e-6) / 1e9
    heads_tflops = heads_flops(w) / (stages_us["heads"] * 1e-6) / 1e12
    attn_total = stages_us["attention"]
    dominant_attention = attn_total >= stages_us["heads"]
    if dominant_attention:
        # more than 128 query rows per K/V head (T x query heads per K/V head)
        # run the grouped-query kernel
        attn_kernel = "tree_attn_gqa" if (w.Hq // w.Hkv) * w.T > 128 else "tree_attn_bf16"
        roof = {"kernel": f"tree attention, one layer ({attn_kernel} + merge_splits)", "bound": "hbm",
                "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                "traffic": counter_traffic(w, "tree_attention", "attention.hip"),
                "bytes_per_launch": a_bytes, "us_per_launch": round(attn_us, 2)}
    else:
        roof = {"kernel": "skinny_gemm_bf16 x2 (residual block + vocab projection)", "bound": "hbm",
                "achieved": round(heads_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(heads_gbs / HBM_PEAK_GBS, 4),
                "traffic": counter_traffic(w, "heads", "heads.hip"),
                "bytes_per_launch": h_bytes, "us_per_launch": round(stages_us["heads"], 2)}
    result = {
        "metric": METRIC,
        "value": round(1000.0 / ms, 2),
        "unit": "verify steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "hidden": w.H, "vocab": w.V, "heads": w.K,
                   "tree_nodes": w.T, "topk": list(w.topk), "layers": w.L, "q_heads": w.Hq,
                   "kv_heads": w.Hkv, "head_dim": w.D, "context": w.ctx,
                   "acceptance": ["greedy" if t == 0 else f"rejection tau={t}" for t in w.temperature],
                   "timing": "eager" if args.eager else "hip graph replay"},
        "roofline": roof,
        "tree_attention_hbm_gbs": round(attn_gbs, 1),
        "heads": {"hbm_gbs": round(heads_gbs, 1), "hbm_frac": round(heads_gbs / HBM_PEAK_GBS, 4),
                  "mfma_tflops": round(heads_tflops, 2),
                  "mfma_frac": round(heads_tflops / BF16_MFMA_PEAK_TFLOPS, 5)},
        "tree_attention_batched": {
            "us_all_layers": round(stages_us["attention_batched"], 2),
            "us_per_layer": round(stages_us["attention_batched"] / w.L, 2),
            "hbm_gbs": round(a_bytes * w.L / (stages_us["attention_batched"] * 1e-6) / 1e9, 1),
            "hbm_frac": round(a_bytes * w.L / (stages_us["attention_batched"] * 1e-6) / 1e9
                              / HBM_PEAK_GBS, 4)},
        "heads_dense": {
            "rows": w.B * w.T,
            "us": round(stages_us["heads_dense"], 2),
            "mfma_tflops": round(heads_flops(w) * w.T / (stages_us["heads_dense"] * 1e-6) / 1e12, 1),
            "mfma_frac": round(heads_flops(w) * w.T / (stages_us["heads_dense"] * 1e-6) / 1e12
                               / BF16_MFMA_PEAK_TFLOPS, 4),
            # weights read once dominate its bytes (the logits never leave the chip)
            "hbm_gbs": round(w.K * (w.H * w.H + w.H * w.V) * 2 / (stages_us["heads_dense"] * 1e-6) / 1e9, 1),
            "hbm_frac": round(w.K * (w.H * w.H + w.H * w.V) * 2 / (stages_us["heads_dense"] * 1e-6) / 1e9
                              / HBM_PEAK_GBS, 4)},
        "stages_us": {k: round(v, 2) for k, v in stages_us.items()},
        "step_ms_pct": step_pct,
        "stages_us_pct": stages_pct,
        "wall_s_timed": round(wall_s, 4),
    }
    probe = read_probe()
    probe["tree_attention_frac"] = round(attn_gbs / probe["gbs"], 4)
    probe["tree_attention_batched_frac"] = round(result["tree_attention_batched"]["hbm_gbs"] / probe["gbs"], 4)
    probe["heads_frac"] = round(heads_gbs / probe["gbs"], 4)
    result["hbm_read_probe"] = probe
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_layers, args.cpu_seqs, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
