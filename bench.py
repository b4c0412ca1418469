#!/usr/bin/env python3
"""CommunityKV decode-step benchmark on one MI355X.

A step is one pass of the whole decode path over the layer: centroid scoring,
budgeted community selection, gather + exact attention, top-kappa edges with
assignment and centroid update (four C-ABI calls, all HIP kernels).  The
default workload is the Llama-3.1-8B-shaped layer at 131072 tokens of context
(batch 1, 32 query heads over 8 kv heads, head_dim 128, bf16 K/V, one graph
per query head, token budget 4096, kappa 8), drawn synthetically.

Inputs for every step are generated and copied to the GPU before timing.
Timed passes restore the same starting state, so every pass runs the same
steps.  Output: one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode steps/s + gathered-KV HBM GB/s (% roofline) at 128K ctx, budget 4096"
HBM_PEAK_GBPS = 8000.0
# HBM traffic of one gather launch, from rocprofv3 FETCH_SIZE / WRITE_SIZE runs
# scaled by a plain copy kernel; valid only for the sources it names.
PMC_SUMMARY = os.path.join(ROOT, "profiles", "gather_attend_llama31_8b_128k_pmc.txt")
GATHER_SOURCES = ("attend.hip", "combine.h", "ckv_device.h", "ckv_internal.h")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama31_8b_128k")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--windows", type=int, default=1,
                    help="graph windows per step, each on its own stream (1 = one launch per call)")
    ap.add_argument("--no-defer", action="store_true",
                    help="complete gathers (combine inside the gather kernel) instead of the deferred combine")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU work budget of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--recall-steps", type=int, default=16,
                    help="steps per budget of the attention-mass recall sweep (0: skip)")
    ap.add_argument("--profile", action="store_true", help="only warm-up + timed steps (for rocprofv3 runs)")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill graph-construction leg")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the prefill graph construction of the workload's first sequence (profiling)")
    ap.add_argument("--eager-only", action="store_true", help="with --profile: no HIP graph (counter runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB copy kernel 5 times (scale for rocprofv3 byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the CommunityKV step runs on a single MI355X "
              "(multi-GPU sharding is described in the design notes, not launched)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from community_kv_retrieval_amd import ckv, runner, synth

    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
        return
    w = synth.preset(args.workload)
    if w.n_layers > 1:
        bench_stack(args, w)
        return
    W, K = args.warmup, args.steps
    total = W + K
    if args.prefill_only:
        slices = synth.gen_layer(w, args.seed)
        layer = runner.load_layer(w, args.seed, extra=1, slices=slices)
        print(json.dumps({"prefill_graph": bench_prefill(w, args.seed, layer.kv, slices, reps=args.steps)}),
              flush=True)
        return
    log(f"[bench] workload {w.name}: generating")
    t0 = time.time()
    slices = synth.gen_layer(w, args.seed)
    layer = runner.load_layer(w, args.seed, extra=total + 1, slices=slices)
    dec, buf, idx, kv = layer.dec, layer.dec.buf, layer.idx, layer.kv
    dec.set_windows(args.windows)
    dec.defer = not args.no_defer
    steps_in = [synth.gen_step(w, args.seed, t, slices) for t in range(total)]
    Q = torch.stack([s.q for s in steps_in]).cuda()
    KN = torch.stack([s.k_new for s in steps_in]).cuda()
    VN = torch.stack([s.v_new for s in steps_in]).cuda()
    torch.cuda.synchronize()
    log(f"[bench] setup {time.time() - t0:.1f}s; G={idx.n_graphs} c_cap={idx.c_cap} t_cap={buf.t_cap}")

    snap = (idx.state_dict(), kv.kv.clone(), kv.seq_len.clone())

    def restore():
        idx.load_state_dict(snap[0])
        kv.kv.copy_(snap[1])
        kv.seq_len.copy_(snap[2])
        torch.cuda.synchronize()

    # Accounting pass: tokens gathered per step (results are deterministic,
    # so the timed passes below gather exactly these).
    restore()
    tok = []
    for t in range(total):
        dec.step(Q[t], KN[t], VN[t])
        tok.append(buf.tok_n.clone())
    torch.cuda.synchronize()
    tok = torch.stack(tok).cpu().numpy().astype(np.int64)  # [total][G]
    assert int(idx.status.item()) == 0, f"device status {int(idx.status.item())}"
    esz = 2 if w.dtype == "bf16" else 4
    row_bytes = 2 * w.head_dim * esz  # K row + V row
    gathered = tok[W:].sum(axis=1) * row_bytes  # bytes per timed step
    n_comm = np.array(synth.graph_n_comm(w, slices), dtype=np.int64)
    # the scoring kernel streams the int16 screening copy of every used
    # centroid column plus its scale and member count
    score_bytes = int(n_comm.sum()) * (w.head_dim * 2 + 8)

    # Eager pass: K steps launched one call at a time from Python.
    restore()
    for t in range(W):
        dec.step(Q[t], KN[t], VN[t])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for t in range(W, total):
        dec.step(Q[t], KN[t], VN[t])
    e1.record()
    torch.cuda.synchronize()
    ms_eager = e0.elapsed_time(e1) / K
    ref = [x.clone() for x in (buf.out, buf.edges, buf.assign, idx.cent, idx.size, idx.tail_len, kv.seq_len)]
    if args.profile and args.eager_only:
        log(f"[bench] profile run (eager only): {ms_eager * 1e3:.1f} us/step")
        return

    # Headline pass: the same K steps captured once as one HIP graph (how a
    # decode loop is launched in serving) and replayed, bracketed by
    # synchronisation.  The replay must reproduce the eager pass bit for bit.
    restore()
    for t in range(W):
        dec.step(Q[t], KN[t], VN[t])
    torch.cuda.synchronize()
    snap_w = (idx.state_dict(), kv.kv.clone(), kv.seq_len.clone())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for t in range(W, total):
            dec.step(Q[t], KN[t], VN[t])
    idx.load_state_dict(snap_w[0])
    kv.kv.copy_(snap_w[1])
    kv.seq_len.copy_(snap_w[2])
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = e0.elapsed_time(e1) / K
    got = (buf.out, buf.edges, buf.assign, idx.cent, idx.size, idx.tail_len, kv.seq_len)
    assert all(torch.equal(a, b) for a, b in zip(ref, got)), "graph replay differs from the eager steps"
    del graph
    if args.profile:
        log(f"[bench] profile run: {ms_step * 1e3:.1f} us/step (graph), {ms_eager * 1e3:.1f} us/step (eager)")
        return

    # Host-input pass: the same steps launched eagerly, each step's query and
    # new key/value rows first copied from pinned host memory (a caller that
    # holds them on the host).  Compare with ms_eager; never the headline.
    restore()
    Qh, KNh, VNh = (torch.empty(x.shape, dtype=x.dtype, pin_memory=True) for x in (Q, KN, VN))
    for hx, dx in ((Qh, Q), (KNh, KN), (VNh, VN)):
        hx.copy_(dx)
    qd, knd, vnd = torch.empty_like(Q[0]), torch.empty_like(KN[0]), torch.empty_like(VN[0])
    for t in range(W):
        dec.step(Q[t], KN[t], VN[t])
    torch.cuda.synchronize()
    e0.record()
    for t in range(W, total):
        qd.copy_(Qh[t], non_blocking=True)
        knd.copy_(KNh[t], non_blocking=True)
        vnd.copy_(VNh[t], non_blocking=True)
        dec.step(qd, knd, vnd)
    e1.record()
    torch.cuda.synchronize()
    ms_host = e0.elapsed_time(e1) / K
    got = (buf.out, buf.edges, buf.assign, idx.cent, idx.size, idx.tail_len, kv.seq_len)
    assert all(torch.equal(a, b) for a, b in zip(ref, got)), "host-input steps differ from the eager steps"
    host_bytes = int(Q[0].numel() * Q.element_size() + 2 * KN[0].numel() * KN.element_size())
    del Qh, KNh, VNh

    # Breakdown pass: the same steps, each of the four kernels stamping its own
    # start/stop events from its dispatch (ckv_time_next_launch), so these are
    # kernel execution times on the stream the kernels run on.
    b = buf

    def stamp_events():
        ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(4)]
              for _ in range(K)]
        for row in ev:  # torch creates the underlying HIP events on first record
            for a, c in row:
                a.record()
                c.record()
        return ev

    def stamped_step(t, row):
        """One step as its four calls, each stamping row[k] from its dispatch."""
        q = Q[t]
        ckv.ckv_time_next_launch(*row[0])
        ckv.ckv_score_centroids(kv, idx, q, b.scores)
        ckv.ckv_time_next_launch(*row[1])
        ckv.ckv_select_communities(kv, idx, q, b.scores, dec.budget, dec.max_comm, b.sel, b.sel_n, b.top,
                                   b.tok_list, b.tok_n)
        ckv.ckv_time_next_launch(*row[2])
        out, ml = (None, None) if dec.defer else (b.out, b.ml)
        ckv.ckv_gather_attend(kv, idx, q, b.tok_list, b.tok_n, dec.sm_scale, out, b.logits, ml, b.ws)
        ckv.ckv_time_next_launch(*row[3])
        ckv.ckv_assign_update(kv, idx, b.tok_list, b.tok_n, b.logits, b.ml, b.top, dec.kappa, KN[t], VN[t],
                              b.edges, b.assign, b.ws, out=b.out if dec.defer else None)

    restore()
    for t in range(W):
        dec.step(Q[t], KN[t], VN[t])
    ev = stamp_events()
    torch.cuda.synchronize()
    for i, t in enumerate(range(W, total)):
        stamped_step(t, ev[i])
    torch.cuda.synchronize()
    dt = np.array([[a.elapsed_time(c) for a, c in ev[i]] for i in range(K)]) * 1e3  # us
    names = ["score_centroids", "select_communities", "gather_attend", "assign_update"]
    gather_us = dt[:, 2]
    gather_gbps = float(gathered.sum() / (gather_us.sum() * 1e-6) / 1e9)
    score_gbps = float(score_bytes * K / (dt[:, 0].sum() * 1e-6) / 1e9)
    ceiling = read_ceiling(w, kv, idx, buf, row_bytes, K)

    # Cold passes: a 512 MB read between steps evicts the 256 MB MALL (a read,
    # so the step does not also pay for writing dirty lines back); only the
    # step itself is timed.  The first pass times whole steps; the second stamps
    # each kernel as in the breakdown pass (its extra event calls can slow the
    # host's launches past the flush, so it does not time whole steps).
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    restore()
    for t in range(W):
        dec.step(Q[t], KN[t], VN[t])
    cold = []
    for t in range(W, total):
        flush.amax()
        a, c = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dec.step(Q[t], KN[t], VN[t])
        c.record()
        cold.append((a, c))
    torch.cuda.synchronize()
    cold_us = np.array([a.elapsed_time(c) for a, c in cold]) * 1e3
    restore()
    for t in range(W):
        dec.step(Q[t], KN[t], VN[t])
    evc = stamp_events()
    torch.cuda.synchronize()
    for i, t in enumerate(range(W, total)):
        flush.amax()
        stamped_step(t, evc[i])
    torch.cuda.synchronize()
    cold_dt = np.array([[a.elapsed_time(c) for a, c in evc[i]] for i in range(K)]) * 1e3  # us
    del flush

    # Dense flash-decode over every cached token of the same state.
    dense = None
    if not args.no_dense:
        restore()
        out = torch.empty_like(buf.out)
        for _ in range(3):
            dec.dense(Q[W], out)
        torch.cuda.synchronize()
        reps = 20
        a, c = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            dec.dense(Q[W], out)
        c.record()
        torch.cuda.synchronize()
        d_us = a.elapsed_time(c) / reps * 1e3
        d_bytes = int(kv.seq_len.sum().item()) * w.n_kv_heads * row_bytes
        dense = {"us_per_call": round(d_us, 2), "bytes": d_bytes, "gbps": round(d_bytes / (d_us * 1e-6) / 1e9, 1),
                 "frac_of_8tbps": round(d_bytes / (d_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}

    # Attention-mass recall (the page's Figure 3 quality proxy): the share of
    # each head's dense softmax mass that the attended tokens carry, per budget.
    recall = None
    if args.recall_steps > 0:
        recall = {}
        budget0 = dec.budget
        dec.defer = False  # recall reads the gather's ml before the update
        dml = torch.empty((w.batch, w.n_q_heads, 2), dtype=torch.float32, device="cuda")
        dout = torch.empty_like(buf.out)
        for B in [b for b in (128, 512, 1024, 2048, 4096) if b <= budget0]:
            restore()
            dec.budget = B
            vals = []
            for t in range(min(args.recall_steps, total)):
                dec.retrieve(Q[t])
                dec.attend(Q[t])
                dec.dense(Q[t], dout, ml=dml)
                vals.append(dec.recall(dml).flatten())
                dec.update(KN[t], VN[t])
            v = torch.cat(vals).cpu().numpy()
            recall[str(B)] = {"mean": round(float(v.mean()), 4), "p10": round(float(np.percentile(v, 10)), 4),
                              "min": round(float(v.min()), 4)}
        dec.budget = budget0
        dec.defer = True

    prefill = None
    if not args.no_prefill:
        prefill = bench_prefill(w, args.seed, kv, slices,
                                cpu_seconds=0.0 if args.no_cpu_baseline else args.cpu_seconds / 2)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.seed, slices, steps_in, args.cpu_seconds)

    avg_gather = float(gathered.mean())
    src_hash = gather_source_hash()
    traffic = measured_traffic(w.name, src_hash)
    res = {
        "metric": METRIC,
        "value": round(1e3 / ms_step, 1),
        "unit": "decode steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "ctx": w.n_ctx, "budget": w.budget, "kappa": w.kappa,
                   "graphs": "per_query_head" if w.mode == synth.PER_HEAD else "query_group",
                   "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
                   "kv_dtype": w.dtype, "n_graphs": idx.n_graphs, "seed": args.seed,
                   "windows": dec.windows, "deferred_combine": dec.defer},
        "gathered_kv_gbps": round(gather_gbps, 1),
        "gathered_kv_frac_of_hbm": round(gather_gbps / HBM_PEAK_GBPS, 4),
        "roofline": {"bound": "hbm", "kernel": "gather_attend", "achieved": round(gather_gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gather_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "bytes_per_launch": int(avg_gather),
                     "avg_launch_us": round(float(gather_us.mean()), 2), "kernel_sources": src_hash,
                     "read_ceiling_gbps": ceiling["gbps"],
                     "frac_of_read_ceiling": round(gather_gbps / ceiling["gbps"], 4)},
        "read_ceiling": ceiling,
        "score_roofline": {"bound": "hbm", "achieved": round(score_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                           "frac": round(score_gbps / HBM_PEAK_GBPS, 4), "bytes_per_launch": score_bytes,
                           "avg_launch_us": round(float(dt[:, 0].mean()), 2)},
        "breakdown_us": {n: round(float(dt[:, j].mean()), 2) for j, n in enumerate(names)},
        "breakdown_step_us": round(float(dt.sum(axis=1).mean()), 2),
        "cold_step_us": {"median": round(float(np.median(cold_us)), 2),
                         "p10": round(float(np.percentile(cold_us, 10)), 2),
                         "p90": round(float(np.percentile(cold_us, 90)), 2),
                         "kernels_median": {n: round(float(np.median(cold_dt[:, k])), 2) for k, n in enumerate(names)}},
        "tokens_per_step": round(float(tok[W:].sum(axis=1).mean()), 1),
        "dense_flash_decode": dense,
        "attention_mass_recall": recall,
        "prefill_graph": prefill,
        "cpu_baseline": cpu,
        "ms_per_step_eager": round(ms_eager, 5),
        "host_inputs": {"ms_per_step": round(ms_host, 5), "steps_per_s": round(1e3 / ms_host, 1),
                        "bytes_per_step": host_bytes,
                        "how": "eager launches; q, k_new and v_new copied from pinned host memory before each step"},
        "launch": "hip_graph",
        "wall_s_timed": round(wall, 4),
    }
    print(json.dumps(res), flush=True)


MFMA_BF16_PEAK_TFLOPS = 2500.0


def bench_prefill(w, seed, kv, slices, reps=3, cpu_seconds=0.0):
    """Prefill graph construction (top-kappa edges per query, matrix cores) of
    the first sequence's whole prompt: per head with weights, per head
    without, and per query group.  Algorithmic work: n(n+1)/2 causal pairs x
    2 d flop per query head (the group mode's second pass is not counted)."""
    import numpy as np
    import torch

    from community_kv_retrieval_amd import ckv, synth

    n = int(slices[0][0].part.labels.shape[0])
    parts = [slices[0][kh].part for kh in range(w.n_kv_heads)]
    q = synth.gen_prefill_queries_device(w, seed, 0, 0, parts)
    flops = n * (n + 1) / 2 * 2 * w.head_dim * w.n_q_heads
    out = {"workload": w.name, "prompt_tokens": n, "q_heads": w.n_q_heads, "kappa": w.kappa,
           "algorithmic_tflop": round(flops / 1e12, 3)}
    for name, mode, with_w in (("per_head", ckv.CKV_MODE_PER_HEAD, True),
                               ("per_head_edges_only", ckv.CKV_MODE_PER_HEAD, False),
                               ("query_group", ckv.CKV_MODE_QUERY_GROUP, True)):
        graphs = w.n_q_heads if mode == ckv.CKV_MODE_PER_HEAD else w.n_kv_heads
        edges = torch.empty((graphs, n, w.kappa), dtype=torch.int32, device="cuda")
        weights = torch.empty((graphs, n, w.kappa), dtype=torch.float32, device="cuda") if with_w else None
        ws = ckv.prefill_workspace(kv, mode, n)
        ckv.ckv_prefill_topk(kv, mode, 0, q, w.n_sinks, w.kappa, w.sm_scale, edges, weights, ws)
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()  # torch creates the underlying HIP events on first record
            e1.record()
            torch.cuda.synchronize()
            if mode == ckv.CKV_MODE_PER_HEAD:  # the call's one kernel, dispatch-stamped
                ckv.ckv_time_next_launch(e0, e1)
                ckv.ckv_prefill_topk(kv, mode, 0, q, w.n_sinks, w.kappa, w.sm_scale, edges, weights, ws)
            else:  # two kernels: events around the call
                e0.record()
                ckv.ckv_prefill_topk(kv, mode, 0, q, w.n_sinks, w.kappa, w.sm_scale, edges, weights, ws)
                e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        t = float(np.median(ms))
        tf = flops / (t * 1e-3) / 1e12
        out[name] = {"ms_per_layer": round(t, 3), "tflops": round(tf, 1),
                     "frac_of_bf16_mfma_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
        del edges, weights, ws
    if cpu_seconds > 0:
        out["cpu_baseline"] = prefill_cpu_baseline(w, q, slices, cpu_seconds)
    out["roofline"] = {"bound": "mfma", "kernel": "prefill_topk (per head, weights)",
                       "achieved": out["per_head"]["tflops"], "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                       "frac": out["per_head"]["frac_of_bf16_mfma_peak"], "traffic": None}
    return out


def bench_stack(args, w):
    """Streaming multi-layer decode: every layer of the stack runs the four
    calls per step, the batch's sequences growing by one token per step.  The
    stack holds the whole capacity resident (no copy of it fits), so the
    passes run forward one after another instead of from a restored state:
    eager warm-up, K steps captured as one graph and replayed (timed), more
    steps with per-kernel stamps, then one dense step."""
    import numpy as np
    import torch

    from community_kv_retrieval_amd import ckv, runner, synth
    W, K, KB = args.warmup, args.steps, 4
    total = W + K + KB
    t0 = time.time()
    stack = runner.load_stack(w, args.seed, total, log=log)
    lens0 = [int(x) for x in stack[0].kv.seq_len.cpu()]
    resident = sum(L.kv.kv.numel() * L.kv.kv.element_size() for L in stack)
    log(f"[bench] stack of {len(stack)} layers ready in {time.time() - t0:.1f}s; pool {resident / 1e9:.1f} GB")

    def step(t):
        for L in stack:
            L.dec.step(L.q[t], L.k_new[t], L.v_new[t])

    for t in range(W):
        step(t)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for t in range(W, W + K):
            step(t)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = e0.elapsed_time(e1) / K
    del graph
    for L in stack:
        assert int(L.idx.status.item()) == 0, "device status set"
    assert [int(x) for x in stack[0].kv.seq_len.cpu()] == [n + W + K for n in lens0]

    # Per-kernel times (dispatch-stamped) and gathered bytes over KB more steps.
    names = ["score_centroids", "select_communities", "gather_attend", "assign_update"]
    ev = [[[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(4)]
           for _ in stack] for _ in range(KB)]
    for a in ev:
        for row in a:
            for x, y in row:
                x.record()
                y.record()
    torch.cuda.synchronize()
    tok = []
    for i, t in enumerate(range(W + K, total)):
        for li, L in enumerate(stack):
            b, q = L.dec.buf, L.q[t]
            ckv.ckv_time_next_launch(*ev[i][li][0])
            ckv.ckv_score_centroids(L.kv, L.idx, q, b.scores)
            ckv.ckv_time_next_launch(*ev[i][li][1])
            ckv.ckv_select_communities(L.kv, L.idx, q, b.scores, L.dec.budget, L.dec.max_comm, b.sel, b.sel_n,
                                       b.top, b.tok_list, b.tok_n)
            ckv.ckv_time_next_launch(*ev[i][li][2])
            ckv.ckv_gather_attend(L.kv, L.idx, q, b.tok_list, b.tok_n, L.dec.sm_scale, None, b.logits, None, b.ws)
            ckv.ckv_time_next_launch(*ev[i][li][3])
            ckv.ckv_assign_update(L.kv, L.idx, b.tok_list, b.tok_n, b.logits, b.ml, b.top, L.dec.kappa,
                                  L.k_new[t], L.v_new[t], b.edges, b.assign, b.ws, out=b.out)
            tok.append(b.tok_n.sum())
    torch.cuda.synchronize()
    dt = np.array([[[a.elapsed_time(c) for a, c in ev[i][li]] for li in range(len(stack))]
                   for i in range(KB)]) * 1e3  # [step][layer][kernel] us
    row_bytes = 2 * w.head_dim * (2 if w.dtype == "bf16" else 4)
    gathered = float(torch.stack(tok).double().sum().item()) * row_bytes / KB  # bytes per step
    gather_us = float(dt[:, :, 2].sum(axis=1).mean())  # per step, all layers
    gbps = gathered / (gather_us * 1e-6) / 1e9

    # One dense step over every cached token of every layer.
    dense = None
    if not args.no_dense:
        out = torch.empty_like(stack[0].dec.buf.out)
        a, c = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for L in stack:
            L.dec.dense(L.q[total - 1], out)
        c.record()
        torch.cuda.synchronize()
        d_us = a.elapsed_time(c) * 1e3
        d_bytes = sum(int(L.kv.seq_len.sum().item()) * w.n_kv_heads * row_bytes for L in stack)
        dense = {"us_per_step": round(d_us, 1), "bytes": d_bytes, "gbps": round(d_bytes / (d_us * 1e-6) / 1e9, 1)}

    res = {
        "metric": METRIC,
        "value": round(1e3 / ms_step, 2),
        "unit": "decode steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "layers": len(stack), "ctx": [w.min_ctx, w.n_ctx],
                   "seq_len_at_start": lens0, "budget": w.budget, "kappa": w.kappa,
                   "graphs": "per_query_head" if w.mode == synth.PER_HEAD else "query_group",
                   "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "kv_dtype": w.dtype,
                   "seed": args.seed},
        "tokens_per_s": round(1e3 / ms_step * w.batch, 1),
        "resident_kv_gb": round(resident / 1e9, 1),
        "gathered_kv_gbps": round(gbps, 1),
        "roofline": {"bound": "hbm", "kernel": "gather_attend", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "bytes_per_launch": int(gathered / len(stack)),
                     "avg_launch_us": round(float(dt[:, :, 2].mean()), 2)},
        "breakdown_us_per_layer": {n: round(float(dt[:, :, j].mean()), 2) for j, n in enumerate(names)},
        "breakdown_step_us": round(float(dt.sum(axis=(1, 2)).mean()), 1),
        "dense_flash_decode": dense,
        "cpu_baseline": None,
        "launch": "hip_graph",
        "wall_s_timed": round(wall, 4),
    }
    print(json.dumps(res), flush=True)


def gather_source_hash():
    h = hashlib.sha256()
    for f in GATHER_SOURCES:
        with open(os.path.join(ROOT, "community_kv_retrieval_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, src_hash):
    """Bytes per gather launch from the committed counter summary, or None when
    it was taken on other kernel sources or another workload."""
    try:
        with open(PMC_SUMMARY) as fh:
            kv = dict(line.split(":", 1) for line in fh.read().splitlines() if ":" in line)
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("kernel_sources") != src_hash or kv.get("workload") != workload:
        return None
    try:
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def read_ceiling(w, kv, idx, buf, row_bytes, reps):
    """The practical read rate of the gather's access pattern: ckv_read_rows
    (the gather's loads, no arithmetic) over the rows the last step's token
    lists name, timed with dispatch-stamped events like the gather."""
    import numpy as np
    import torch
    from community_kv_retrieval_amd import ckv, synth
    G, T = buf.tok_list.shape
    gi = torch.arange(G, device="cuda")[:, None].expand(G, T)
    mask = torch.arange(T, device="cuda")[None, :] < buf.tok_n[:, None]
    pos, g = buf.tok_list[mask].long(), gi[mask]
    if w.mode == synth.PER_HEAD:
        b, kh = g // w.n_q_heads, (g % w.n_q_heads) // (w.n_q_heads // w.n_kv_heads)
    else:
        b, kh = g // w.n_kv_heads, g % w.n_kv_heads
    ps = kv.page_size
    page = kv.page_table[b, pos // ps].long()
    rows = ((page * w.n_kv_heads + kh) * ps + pos % ps).to(torch.int32).contiguous()
    n = rows.numel()
    part = torch.zeros(((n + 255) // 256,), dtype=torch.int32, device="cuda")
    for _ in range(5):
        ckv.ckv_read_rows(kv, rows, part)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, c in ev:
        a.record()
        c.record()
    torch.cuda.synchronize()
    for a, c in ev:
        ckv.ckv_time_next_launch(a, c)
        ckv.ckv_read_rows(kv, rows, part)
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(c) for a, c in ev]) * 1e3
    gbps = n * row_bytes / (float(us.mean()) * 1e-6) / 1e9
    return {"kernel": "read_rows", "rows": n, "bytes_per_launch": n * row_bytes,
            "avg_launch_us": round(float(us.mean()), 2), "gbps": round(gbps, 1),
            "frac_of_8tbps": round(gbps / HBM_PEAK_GBPS, 4)}


def copy_calibration():
    """A plain copy kernel of known size: 256 MiB read and 256 MiB written per launch."""
    import torch
    n = (256 << 20) // 4
    src = torch.empty(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1.0)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: 5 launches of neg over {n * 4} bytes")


def cpu_baseline(w, seed, slices, steps_in, seconds):
    """The CPU oracle, as it stands, on the first steps of the same workload."""
    import numpy as np

    from community_kv_retrieval_amd import synth
    from oracle import ckv_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count() or 1
    kvh = [[(s.k.float().numpy(), s.v.float().numpy()) for s in row] for row in slices]
    orc = O.Oracle(w, kvh, dict(enumerate(synth.graph_labels(w, slices))),
                   dict(enumerate(synth.graph_n_comm(w, slices))), extra=len(steps_in) + 1)
    n, t_used = 0, 0.0
    while t_used < seconds and n < len(steps_in):
        s = steps_in[n]
        t0 = time.perf_counter()
        orc.step(s.q.float().numpy(), s.k_new.float().numpy(), s.v_new.float().numpy())
        t_used += time.perf_counter() - t0
        n += 1
    return {"value": round(n / t_used, 3), "unit": "decode steps/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n} decode steps of the same workload, all {w.n_graphs} graphs, float64 numpy "
                      f"({t_used:.1f}s of CPU time; setup not timed)"}


def prefill_cpu_baseline(w, q, slices, seconds):
    """The CPU oracle's prefill graph (prefill_edges_rows, float64 numpy) on a
    random sample of (position, query head) rows of the same prompt, timed and
    extrapolated to the whole layer by the number of query-key pairs."""
    import numpy as np

    from oracle import ckv_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count() or 1
    n = q.shape[0]
    G = w.n_q_heads // w.n_kv_heads
    rng = np.random.default_rng(5)
    rows = np.sort(rng.integers(0, n, size=256))
    qh = q[torch_index(rows)].float().cpu().numpy().astype(np.float64)  # [R][Hq][d]
    t_used, pairs, done = 0.0, 0, 0
    for kh in range(w.n_kv_heads):
        keys = slices[0][kh].k.float().numpy().astype(np.float64)
        for h in range(kh * G, (kh + 1) * G):
            for r, i in enumerate(rows):
                t0 = time.perf_counter()
                O.prefill_edges_rows(qh[r:r + 1, h:h + 1], [int(i)], keys, w.n_sinks, w.kappa, w.sm_scale)
                t_used += time.perf_counter() - t0
                pairs += int(i) + 1
                done += 1
                if t_used >= seconds:
                    break
            if t_used >= seconds:
                break
        if t_used >= seconds:
            break
    total_pairs = n * (n + 1) / 2 * w.n_q_heads
    return {"value": round(t_used * total_pairs / pairs, 1), "unit": "s per layer (extrapolated)",
            "cores": int(threads), "kind": "oracle",
            "sample": f"{done} random (position, query head) rows of the {n}-token prompt, float64 numpy "
                      f"({t_used:.1f}s of CPU time), scaled by query-key pairs to all {w.n_q_heads} heads"}


def torch_index(rows):
    import torch
    return torch.as_tensor(rows, dtype=torch.long, device="cuda")


if __name__ == "__main__":
    main()
