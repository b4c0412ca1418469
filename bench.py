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
    ap.add_argument("--no-group", action="store_true", help="skip the batch-8 query-group leg")
    ap.add_argument("--no-centroid", action="store_true", help="skip the centroid-budget leg")
    ap.add_argument("--centroid-only", type=int, default=0,
                    help="with --profile: only the centroid-budget layer at this budget (for rocprofv3 runs)")
    ap.add_argument("--recall-steps", type=int, default=16,
                    help="steps per budget of the attention-mass recall sweep (0: skip)")
    ap.add_argument("--profile", action="store_true", help="only warm-up + timed steps (for rocprofv3 runs)")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill graph-construction leg")
    ap.add_argument("--no-refresh", action="store_true", help="skip the refresh-vs-incremental leg")
    ap.add_argument("--refresh-only", action="store_true", help="only the refresh-vs-incremental leg")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the prefill graph construction of the workload's first sequence (profiling)")
    ap.add_argument("--eager-only", action="store_true", help="with --profile: no HIP graph (counter runs)")
    ap.add_argument("--cold-only", action="store_true",
                    help="with --profile: only eager steps, each after the MALL flush (cold kernel averages)")
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
    if args.centroid_only > 0:
        bench_centroid(args, w, args.warmup, args.steps, budgets=(args.centroid_only,), profile=True)
        return
    if w.n_layers > 1:
        bench_stack(args, w)
        return
    W, K = args.warmup, args.steps
    total = W + K
    if args.refresh_only:
        print(json.dumps({"refresh_vs_incremental": bench_refresh(args, synth.preset("qwen3_8b_32k"), **REFRESH_LEG),
                          "refresh_vs_incremental_128k": bench_refresh(args, synth.preset("llama31_8b_128k"),
                                                                       **REFRESH_LEG_128K)}),
              flush=True)
        return
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
    aux = aux_memory(kv, idx)

    snap = (idx.state_dict(), kv.kv.clone(), kv.seq_len.clone())

    def restore():
        idx.load_state_dict(snap[0])
        kv.kv.copy_(snap[1])
        kv.seq_len.copy_(snap[2])
        torch.cuda.synchronize()

    if args.profile:
        passes = time_layer(w, dec, kv, idx, Q, KN, VN, W, K, restore, profile=True, eager_only=args.eager_only,
                            cold_only=args.cold_only)
        return
    L = time_layer(w, dec, kv, idx, Q, KN, VN, W, K, restore)
    gathered, score_bytes, row_bytes = L["gathered"], L["score_bytes"], L["row_bytes"]
    ref = L["ref"]

    # Host-input pass: the same steps launched eagerly, each step's query and
    # new key/value rows first copied from pinned host memory (a caller that
    # holds them on the host).  Compare with the eager rate; never the headline.
    restore()
    Qh, KNh, VNh = (torch.empty(x.shape, dtype=x.dtype, pin_memory=True) for x in (Q, KN, VN))
    for hx, dx in ((Qh, Q), (KNh, KN), (VNh, VN)):
        hx.copy_(dx)
    qd, knd, vnd = torch.empty_like(Q[0]), torch.empty_like(KN[0]), torch.empty_like(VN[0])
    for t in range(W):
        dec.step(Q[t], KN[t], VN[t])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
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

    ceiling = read_ceiling(w, kv, idx, buf, row_bytes, K)
    dense = None if args.no_dense else dense_baseline(w, dec, kv, Q[W], restore)

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
        dec.defer = not args.no_defer

    prefill = None
    if not args.no_prefill:
        prefill = bench_prefill(w, args.seed, kv, slices,
                                cpu_seconds=0.0 if args.no_cpu_baseline else args.cpu_seconds / 2)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.seed, slices, steps_in, args.cpu_seconds)
    del layer, dec, buf, idx, kv, snap, Q, KN, VN
    torch.cuda.empty_cache()

    group = None
    if not args.no_group and w.name == "llama31_8b_128k":
        group = bench_group(args, synth.preset("llama31_8b_128k_group_b8"), W, K)
    centroid = None
    if not args.no_centroid and w.name == "llama31_8b_128k":
        centroid = bench_centroid(args, w, W, K)

    refresh = refresh_128k = None
    if not args.no_refresh and w.name == "llama31_8b_128k":
        refresh = bench_refresh(args, synth.preset("qwen3_8b_32k"), **REFRESH_LEG)
        refresh_128k = bench_refresh(args, synth.preset("llama31_8b_128k"), **REFRESH_LEG_128K)

    src_hash = gather_source_hash()
    traffic = measured_traffic(w.name, src_hash)
    cold_step_us = float(L["cold_us"].mean())
    res = {
        "metric": METRIC,
        "value": round(1e6 / cold_step_us, 1),
        "unit": "decode steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(cold_step_us * 1e-3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "ctx": w.n_ctx, "budget": w.budget, "kappa": w.kappa,
                   "graphs": "per_query_head" if w.mode == synth.PER_HEAD else "query_group",
                   "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
                   "kv_dtype": w.dtype, "n_graphs": L["n_graphs"], "seed": args.seed,
                   "windows": args.windows, "deferred_combine": not args.no_defer},
        "timing": "each of the K steps timed alone after a 512 MB read that evicts the 256 MB MALL (cold); "
                  "'warm' is the same K steps replayed back to back as one HIP graph",
        "step_us": L["step_us"],
        "warm": {"steps_per_s": round(1e3 / L["ms_warm"], 1), "ms_per_step": round(L["ms_warm"], 5),
                 "ms_per_step_eager": round(L["ms_eager"], 5), "launch": "hip_graph"},
        "gathered_kv_gbps": L["gather"]["cold"]["gbps"],
        "gathered_kv_frac_of_hbm": L["gather"]["cold"]["frac"],
        "roofline": {"bound": "hbm", "kernel": "gather_attend", "achieved": L["gather"]["cold"]["gbps"],
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": L["gather"]["cold"]["frac"],
                     "traffic": traffic, "bytes_per_launch": int(gathered.mean()),
                     "avg_launch_us": L["gather"]["cold"]["avg_launch_us"], "kernel_sources": src_hash,
                     "mall": "flushed", "warm": L["gather"]["warm"],
                     "read_ceiling_gbps": ceiling["gbps"],
                     "frac_of_read_ceiling_warm": round(L["gather"]["warm"]["gbps"] / ceiling["gbps"], 4),
                     "read_ceiling_gbps_cold": ceiling["cold"]["gbps"],
                     "frac_of_read_ceiling_cold": round(L["gather"]["cold"]["gbps"] / ceiling["cold"]["gbps"], 4)},
        "read_ceiling": ceiling,
        "score_roofline": {"bound": "hbm", "kernel": "score_centroids", "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                           "bytes_per_launch": score_bytes, "cold": L["score"]["cold"], "warm": L["score"]["warm"]},
        "breakdown_us": L["breakdown_cold"],
        "breakdown_us_warm": L["breakdown_warm"],
        "tokens_per_step": round(float(L["tok"][W:].sum(axis=1).mean()), 1),
        "aux_memory": aux,
        "dense_flash_decode": dense,
        "attention_mass_recall": recall,
        "prefill_graph": prefill,
        "group_b8": group,
        "centroid_budget": centroid,
        "refresh_vs_incremental": refresh,
        "refresh_vs_incremental_128k": refresh_128k,
        "cpu_baseline": cpu,
        "host_inputs": {"ms_per_step": round(ms_host, 5), "steps_per_s": round(1e3 / ms_host, 1),
                        "bytes_per_step": host_bytes,
                        "how": "eager launches; q, k_new and v_new copied from pinned host memory before each step"},
        "launch": "eager per step (cold); hip_graph (warm)",
        "wall_s_timed": L["wall_s"],
    }
    if dense is not None:
        res["dense_flash_decode"]["dense_over_sparse_step_cold"] = round(dense["us_per_call"] / cold_step_us, 3)
        res["dense_flash_decode"]["dense_over_sparse_step_warm"] = round(dense["us_per_call"] / (L["ms_warm"] * 1e3), 3)
    print(json.dumps(res), flush=True)


STEP_KERNELS = ["score_centroids", "select_communities", "gather_attend", "assign_update"]


def time_layer(w, dec, kv, idx, Q, KN, VN, W, K, restore, profile=False, eager_only=False, cold_only=False):
    """Every timing pass of one layer over steps W .. W + K - 1 (after W
    untimed warm-up steps, from the same restored state each time):
    accounting (tokens gathered per step), eager, the K steps captured as one
    HIP graph and replayed (warm; must equal the eager pass bit for bit),
    each kernel stamped from its own dispatch (warm), and the cold passes
    (a 512 MB read before every step evicts the 256 MB MALL: whole steps, and
    per kernel)."""
    import numpy as np
    import torch

    from community_kv_retrieval_amd import ckv
    total = W + K
    buf = dec.buf
    if profile and cold_only:
        # For a profiler: every launch of every step kernel follows the 512 MB
        # read that evicts the MALL (as in the cold passes), so a kernel's
        # average over all its dispatches is its cold time.
        flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
        for _ in range(2):  # the flush's own first launches
            flush.amax()
        restore()
        for t in range(total):
            flush.amax()
            dec.step(Q[t], KN[t], VN[t])
        torch.cuda.synchronize()
        log(f"[bench] cold profile run: {total} steps, each after a MALL flush")
        return None
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
    n_comm = np.array(idx.n_comm.cpu().numpy(), dtype=np.int64)
    # the scoring kernel streams the int8 screening copy of every used
    # centroid column plus its scale and member count
    score_bytes = int(n_comm.sum()) * (w.head_dim + 8)

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
    if profile and eager_only:
        log(f"[bench] profile run (eager only): {ms_eager * 1e3:.1f} us/step")
        return None

    # Warm pass: the same K steps captured once as one HIP graph and replayed,
    # bracketed by synchronisation; it must reproduce the eager pass bit for bit.
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
    del snap_w
    torch.cuda.synchronize()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_warm = e0.elapsed_time(e1) / K
    got = (buf.out, buf.edges, buf.assign, idx.cent, idx.size, idx.tail_len, kv.seq_len)
    assert all(torch.equal(a, b) for a, b in zip(ref, got)), "graph replay differs from the eager steps"
    del graph
    if profile:
        log(f"[bench] profile run: {ms_warm * 1e3:.1f} us/step (graph), {ms_eager * 1e3:.1f} us/step (eager)")
        return None

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
        ckv.ckv_score_centroids(kv, idx, q, b.scores, b.ws)
        ckv.ckv_time_next_launch(*row[1])
        ckv.ckv_select_communities(kv, idx, q, b.scores, dec.budget, dec.max_comm, b.sel, b.sel_n, b.top,
                                   b.tok_list, b.tok_n, b.ws)
        ckv.ckv_time_next_launch(*row[2])
        out, ml = (None, None) if dec.defer else (b.out, b.ml)
        ckv.ckv_gather_attend(kv, idx, q, b.tok_list, b.tok_n, dec.sm_scale, out, b.logits, ml, b.ws)
        ckv.ckv_time_next_launch(*row[3])
        ckv.ckv_assign_update(kv, idx, b.tok_list, b.tok_n, b.logits, b.ml, b.top, dec.kappa, KN[t], VN[t],
                              b.edges, b.assign, b.ws, out=b.out if dec.defer else None)

    # Warm per-kernel pass: each kernel stamps its own start/stop from its
    # dispatch (ckv_time_next_launch), on the stream it runs on.
    restore()
    for t in range(W):
        dec.step(Q[t], KN[t], VN[t])
    ev = stamp_events()
    torch.cuda.synchronize()
    for i, t in enumerate(range(W, total)):
        stamped_step(t, ev[i])
    torch.cuda.synchronize()
    dt = np.array([[a.elapsed_time(c) for a, c in ev[i]] for i in range(K)]) * 1e3  # us

    # Cold passes: a 512 MB read between steps evicts the 256 MB MALL (a read,
    # so the step does not also pay for writing dirty lines back); only the
    # step itself is timed.  The first pass times whole steps (the headline);
    # the second stamps each kernel (its extra event calls can slow the host's
    # launches past the flush, so it does not time whole steps).
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    for _ in range(2):  # the flush's own first launches (its reduction's set-up), untimed
        flush.amax()
    restore()
    for t in range(W):
        dec.step(Q[t], KN[t], VN[t])
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    cold = []
    for t in range(W, total):
        flush.amax()
        a, c = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dec.step(Q[t], KN[t], VN[t])
        c.record()
        cold.append((a, c))
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    cold_us = np.array([a.elapsed_time(c) for a, c in cold]) * 1e3
    got = (buf.out, buf.edges, buf.assign, idx.cent, idx.size, idx.tail_len, kv.seq_len)
    assert all(torch.equal(a, b) for a, b in zip(ref, got)), "cold steps differ from the eager steps"
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

    def kernel_rate(times_us, nbytes):
        gbps = float(nbytes / (times_us.sum() * 1e-6) / 1e9)
        return {"gbps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4),
                "avg_launch_us": round(float(times_us.mean()), 2)}

    return {
        "tok": tok, "gathered": gathered, "score_bytes": score_bytes, "row_bytes": row_bytes, "ref": ref,
        "n_graphs": idx.n_graphs, "ms_eager": ms_eager, "ms_warm": ms_warm, "cold_us": cold_us,
        "wall_s": round(wall, 4),
        "step_us": {"cold_mean": round(float(cold_us.mean()), 2), "cold_median": round(float(np.median(cold_us)), 2),
                    "cold_p10": round(float(np.percentile(cold_us, 10)), 2),
                    "cold_p90": round(float(np.percentile(cold_us, 90)), 2), "warm": round(ms_warm * 1e3, 2)},
        "breakdown_cold": {n: round(float(cold_dt[:, j].mean()), 2) for j, n in enumerate(STEP_KERNELS)},
        "breakdown_warm": {n: round(float(dt[:, j].mean()), 2) for j, n in enumerate(STEP_KERNELS)},
        "gather": {"cold": kernel_rate(cold_dt[:, 2], gathered.sum()), "warm": kernel_rate(dt[:, 2], gathered.sum())},
        "score": {"cold": kernel_rate(cold_dt[:, 0], score_bytes * K), "warm": kernel_rate(dt[:, 0], score_bytes * K)},
    }


def aux_memory(kv, idx):
    """Bytes of the community index (everything the method keeps beside the
    K/V cache) against the K/V bytes of the cached tokens, as the page's
    Table 5 reports auxiliary memory against the KV cache."""
    parts = {k: int(getattr(idx, k).numel() * getattr(idx, k).element_size())
             for k in idx.STATE + ("n_comm",) if k != "status"}
    kv_filled = int(kv.seq_len.sum().item()) * kv.n_kv_heads * 2 * kv.head_dim * kv.kv.element_size()
    kv_alloc = int(kv.kv.numel() * kv.kv.element_size())
    total = sum(parts.values())
    return {"index_bytes": total, "kv_bytes_cached": kv_filled, "kv_bytes_allocated": kv_alloc,
            "aux_over_kv": round(total / kv_filled, 4), "parts": parts}


def dense_baseline(w, dec, kv, q, restore, reps=20):
    """Dense flash-decode over every cached token of the same state."""
    import torch
    restore()
    out = torch.empty_like(dec.buf.out)
    for _ in range(3):
        dec.dense(q, out)
    torch.cuda.synchronize()
    a, c = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dec.dense(q, out)
    c.record()
    torch.cuda.synchronize()
    d_us = a.elapsed_time(c) / reps * 1e3
    row_bytes = 2 * w.head_dim * (2 if w.dtype == "bf16" else 4)
    d_bytes = int(kv.seq_len.sum().item()) * w.n_kv_heads * row_bytes
    # The read ceiling of the same rows (every cached token of every kv head,
    # in the dense kernel's order) with the gather's loads and no arithmetic.
    ps = kv.page_size
    rows = []
    for b in range(w.batch):
        pos = torch.arange(int(kv.seq_len[b].item()), device="cuda")
        page = kv.page_table[b, pos // ps].long()
        for kh in range(w.n_kv_heads):
            rows.append((page * w.n_kv_heads + kh) * ps + pos % ps)
    rows = torch.cat(rows).to(torch.int32).contiguous()
    ceiling = rows_read_rate(kv, rows, row_bytes, reps)
    del rows
    gbps = d_bytes / (d_us * 1e-6) / 1e9
    return {"us_per_call": round(d_us, 2), "bytes": d_bytes, "gbps": round(gbps, 1),
            "frac_of_8tbps": round(gbps / HBM_PEAK_GBPS, 4), "read_ceiling": ceiling,
            "frac_of_read_ceiling": round(gbps / ceiling["gbps"], 4)}


def bench_group(args, w, W, K):
    """The batch-8 query-group layer (one graph per kv head, the group's four
    query heads share its selection): keys, values and step inputs drawn on
    the device with the recipe of the host generator, then every timing pass
    of time_layer, the gather roofline, auxiliary memory and the dense
    baseline."""
    import torch

    from community_kv_retrieval_amd import runner
    t0 = time.time()
    L0 = runner.load_stack(w, args.seed, W + K, layers=[0])[0]
    dec, kv, idx = L0.dec, L0.kv, L0.idx
    dec.defer = not args.no_defer
    log(f"[bench] group leg {w.name}: setup {time.time() - t0:.1f}s; G={idx.n_graphs}")
    aux = aux_memory(kv, idx)
    snap = (idx.state_dict(), kv.kv.clone(), kv.seq_len.clone())

    def restore():
        idx.load_state_dict(snap[0])
        kv.kv.copy_(snap[1])
        kv.seq_len.copy_(snap[2])
        torch.cuda.synchronize()

    L = time_layer(w, dec, kv, idx, L0.q, L0.k_new, L0.v_new, W, K, restore)
    dense = None if args.no_dense else dense_baseline(w, dec, kv, L0.q[W], restore, reps=5)
    cold_step_us = float(L["cold_us"].mean())
    out = {"workload": w.name, "batch": w.batch, "ctx": w.n_ctx, "budget": w.budget, "graphs": "query_group",
           "n_graphs": idx.n_graphs, "data": "synthetic, drawn on the device",
           "steps_per_s": round(1e6 / cold_step_us, 1), "tokens_per_s": round(1e6 / cold_step_us * w.batch, 1),
           "step_us": L["step_us"], "warm_steps_per_s": round(1e3 / L["ms_warm"], 1),
           "breakdown_us": L["breakdown_cold"], "breakdown_us_warm": L["breakdown_warm"],
           "gathered_bytes_per_step": int(L["gathered"].mean()),
           "gather_roofline": {"bound": "hbm", "kernel": "gather_attend (matrix-core group kernel)",
                               "peak": HBM_PEAK_GBPS, "unit": "GB/s", "cold": L["gather"]["cold"],
                               "warm": L["gather"]["warm"]},
           "score_roofline": {"bytes_per_launch": L["score_bytes"], "cold": L["score"]["cold"],
                              "warm": L["score"]["warm"]},
           "aux_memory": aux, "dense_flash_decode": dense}
    if dense is not None:
        out["dense_flash_decode"]["dense_over_sparse_step_cold"] = round(dense["us_per_call"] / cold_step_us, 3)
    del L0, dec, kv, idx, snap
    torch.cuda.empty_cache()
    return out


def bench_centroid(args, w, W, K, budgets=(0, 16, 256), profile=False):
    """The centroid budget of the page's Table 6 on this workload's layer
    (drawn on the device): every timing pass of time_layer at each budget
    (0 = off, the same layer and steps), the step's cost over budget 0, and the
    bytes the centroid-term kernel reads (a float64 key sum and value sum per
    centroid term)."""
    import torch

    from community_kv_retrieval_amd import runner
    t0 = time.time()
    wc = w.replace(cent_budget=max(budgets))
    L0 = runner.load_stack(wc, args.seed, W + K, layers=[0])[0]
    dec, kv, idx = L0.dec, L0.kv, L0.idx
    dec.defer = not args.no_defer
    log(f"[bench] centroid leg {w.name}: setup {time.time() - t0:.1f}s; G={idx.n_graphs}")
    snap = (idx.state_dict(), kv.kv.clone(), kv.seq_len.clone())

    def restore():
        idx.load_state_dict(snap[0])
        kv.kv.copy_(snap[1])
        kv.seq_len.copy_(snap[2])
        torch.cuda.synchronize()

    out = {"workload": w.name, "budget": w.budget, "n_graphs": idx.n_graphs, "data": "synthetic, drawn on the device",
           "reading": "next-ranked communities after the selection, one softmax term each (key: stored centroid, "
                      "value: mean member value, logit: scale * q . mu + ln n)",
           "value_sum_bytes": int(idx.vsum.numel() * 8), "by_budget": {}}
    for n in budgets:
        idx.desc.cent_budget = n
        L = time_layer(wc, dec, kv, idx, L0.q, L0.k_new, L0.v_new, W, K, restore, profile=profile,
                       eager_only=args.eager_only)
        if profile:
            continue
        cold = float(L["cold_us"].mean())
        out["by_budget"][str(n)] = {
            "steps_per_s": round(1e6 / cold, 1), "step_us": L["step_us"], "breakdown_us": L["breakdown_cold"],
            "centroid_terms_per_step": idx.n_graphs * n,
            "centroid_kernel_bytes_per_step": idx.n_graphs * n * 12 * w.head_dim}  # fp32 row + fp64 value sum
    if not profile and "0" in out["by_budget"]:
        base = out["by_budget"]["0"]["step_us"]
        for n in budgets:
            if n:
                st = out["by_budget"][str(n)]["step_us"]
                out["by_budget"][str(n)]["extra_us_over_budget_0"] = {
                    "cold": round(st["cold_mean"] - base["cold_mean"], 2), "warm": round(st["warm"] - base["warm"], 2)}
    idx.desc.cent_budget = max(budgets)
    del L0, dec, kv, idx, snap
    torch.cuda.empty_cache()
    return out


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
        if name == "per_head":
            out["leiden"] = leiden_timing(w, edges, n, oracle=cpu_seconds > 0)
        del edges, weights, ws
    if cpu_seconds > 0:
        out["cpu_baseline"] = prefill_cpu_baseline(w, q, slices, cpu_seconds)
    out["roofline"] = {"bound": "mfma", "kernel": "prefill_topk (per head, weights)",
                       "achieved": out["per_head"]["tflops"], "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                       "frac": out["per_head"]["frac_of_bf16_mfma_peak"], "traffic": None}
    return out


# The refresh leg: per-head graphs of the 32K layer, resolution 512 (Leiden's
# communities then average about 14 tokens at this size, near the planted 16;
# modularity's community count grows like sqrt(n) at a fixed resolution),
# 1024 drifting steps, a re-partition every 256.
REFRESH_LEG = dict(steps=1024, interval=256, gamma=(512, 1))
# The same at the headline's length (131 072 tokens): a resolution four times
# higher keeps the communities near the same size.
REFRESH_LEG_128K = dict(steps=1024, interval=256, gamma=(2048, 1))


def host_threads() -> int:
    """Host threads for the library's Leiden: the job's CPU share as the
    environment states it (OMP_NUM_THREADS), else the visible cores, at most 16."""
    try:
        return max(1, int(os.environ["OMP_NUM_THREADS"]))
    except (KeyError, ValueError):
        return max(1, min(16, os.cpu_count() or 1))


def leiden_timing(w, edges, n, reps=2, oracle=False):
    """Leiden partition (Figure 1 panel (2); ckv_leiden_partition, host threads)
    of the prompt's per-head graphs from the prefill edges just computed; with
    oracle set, the CPU oracle's Leiden timed on the first graph beside it
    (a baseline, one graph, one thread)."""
    import time

    import numpy as np

    from community_kv_retrieval_amd import ckv

    e = edges.cpu().numpy()
    n_tok = np.full(e.shape[0], n, dtype=np.int32)
    secs = []
    for _ in range(reps):
        t0 = time.perf_counter()
        _, n_comm, q = ckv.ckv_leiden_partition(n_tok, w.n_sinks, e, (1, 1), host_threads())
        secs.append(time.perf_counter() - t0)
    return {"graphs": int(e.shape[0]), "tokens_per_graph": int(n), "gamma": 1, "host_threads": host_threads(),
            "s_per_layer": round(min(secs), 4), "communities_mean": round(float(n_comm.mean()), 1),
            "community_size_mean": round(float((n - w.n_sinks) / n_comm.mean()), 1),
            "modularity_mean": round(float(q.mean()), 4),
            "context": "the page's Table 10 lists 0.37-0.45 s of exposed Leiden time per prefill (its hardware)",
            **(leiden_oracle_baseline(w, e[0], n) if oracle else {})}


def leiden_oracle_baseline(w, rows, n):
    """The oracle's Leiden (pure Python, one thread) on one graph, against the
    library's on the same graph with one thread."""
    import time

    import numpy as np

    from community_kv_retrieval_amd import ckv
    from oracle import leiden_oracle as LO
    t0 = time.perf_counter()
    LO.partition_tokens(rows, n, w.n_sinks)
    t_orc = time.perf_counter() - t0
    one = np.ascontiguousarray(rows[None])
    t0 = time.perf_counter()
    ckv.ckv_leiden_partition(np.array([n], dtype=np.int32), w.n_sinks, one, (1, 1), 1)
    t_lib = time.perf_counter() - t0
    return {"cpu_baseline": {"kind": "oracle", "value": round(t_orc, 3), "unit": "s per graph", "cores": 1,
                             "sample": f"Leiden of the first head's {n}-token prompt graph, pure Python"},
            "library_s_per_graph_one_thread": round(t_lib, 4)}


def bench_refresh(args, base, steps=512, interval=128, gamma=(1, 1), drift_topics=16, drift_rate=0.5):
    """Refresh against incremental assignment (Tables 8 and 9) on a decode
    stream that drifts to topics the prompt never had: both runs start from
    the Leiden partition of the prompt's graph (prefill top-kappa edges,
    ckv_prefill_topk); "incremental" only assigns new tokens, "refresh" also
    re-partitions the grown graph every `interval` steps.  Reported per run:
    attention-mass recall and the output's relative error against dense
    attention over every cached token (all heads, and the heads whose query is
    a drift topic), the modularity of the partition on the grown graph, and
    the cost of each refresh (host Leiden + index rebuild, wall clock)."""
    import time

    import numpy as np
    import torch

    from community_kv_retrieval_amd import ckv, runner, synth

    w = base.replace(name=base.name + "_drift", drift_topics=drift_topics, drift_rate=drift_rate)
    slices = synth.gen_layer(w, args.seed)
    steps_in = [synth.gen_step(w, args.seed, t, slices) for t in range(steps)]
    Q = torch.stack([s.q for s in steps_in]).cuda()
    KN = torch.stack([s.k_new for s in steps_in]).cuda()
    VN = torch.stack([s.v_new for s in steps_in]).cuda()
    drift = np.stack([s.target for s in steps_in])[:, 0] < 0          # [steps][Hq] (batch 1)
    parts = [slices[0][kh].part for kh in range(w.n_kv_heads)]
    qp = synth.gen_prefill_queries_device(w, args.seed, 0, 0, parts)
    n = int(qp.shape[0])
    mode = ckv.CKV_MODE_PER_HEAD if w.mode == synth.PER_HEAD else ckv.CKV_MODE_QUERY_GROUP
    out = {"workload": w.name, "ctx": w.n_ctx, "budget": w.budget, "steps": steps, "refresh_every": interval,
           "gamma": gamma[0] / gamma[1], "drift_topics_per_kv_head": w.drift_topics, "drift_rate": w.drift_rate,
           "quality": "synthetic stand-in for the page's NLL/KL/top-1 (no model): recall and output error "
                      "against dense attention"}
    for name in ("incremental", "refresh", "refresh_async"):
        do_refresh = name != "incremental"
        layer = runner.load_layer(w, args.seed, extra=steps + 1, slices=slices)
        dec, kv = layer.dec, layer.kv
        dec.defer = False
        table = ckv.EdgeTable(kv, dec.idx.mode, dec.idx.l_cap, w.kappa)
        graphs = w.n_q_heads if mode == ckv.CKV_MODE_PER_HEAD else w.n_kv_heads
        pe = torch.empty((graphs, n, w.kappa), dtype=torch.int32, device="cuda")
        ws = ckv.prefill_workspace(kv, mode, n)
        ckv.ckv_prefill_topk(kv, mode, 0, qp, w.n_sinks, w.kappa, w.sm_scale, pe, None, ws)
        table.put_prefill(0, pe)
        del pe, ws
        t0 = time.perf_counter()
        q_init = dec.refresh(table, gamma, n_threads=host_threads())
        torch.cuda.synchronize()
        init_ms = (time.perf_counter() - t0) * 1e3
        dec.edge_table = table
        dml = torch.empty((w.batch, w.n_q_heads, 2), dtype=torch.float32, device="cuda")
        dout = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
        rec, err, qual, ref_ms, ncomm, phases = [], [], [], [], [], []
        pend, pend_t, lags = None, 0, []
        threads = max(1, host_threads() - 2)   # leave cores to the thread launching steps

        def apply_pending(t):
            tm = {}
            dec.refresh_apply(pend, table, timings=tm)
            ref_ms.append(round(tm["snapshot"] + tm["wait"] + tm["place"] + tm["build"], 1))  # not the drain
            phases.append({k: round(v, 1) for k, v in tm.items()})
            lags.append(t - pend_t)

        for t in range(steps):
            dec.retrieve(Q[t])
            dec.attend(Q[t])
            dec.dense(Q[t], dout, ml=dml)
            rec.append(dec.recall(dml).flatten())
            d = torch.linalg.vector_norm(dec.buf.out - dout, dim=-1) / torch.linalg.vector_norm(dout, dim=-1)
            err.append(d.flatten())
            dec.update(KN[t], VN[t])
            if pend is not None and (pend.done() or t + 1 - pend_t >= interval // 2):
                apply_pending(t + 1)
                pend = None
            if (t + 1) % interval == 0:
                if name == "refresh_async":
                    if pend is not None:
                        apply_pending(t + 1)
                        pend = None
                    if t + 1 < steps:
                        pend, pend_t = dec.refresh_async(table, gamma, n_threads=threads), t + 1
                    idx = dec.idx
                    lens = kv.seq_len.cpu().numpy()
                    n_tok = lens[table.graph_seq.cpu().numpy()].astype(np.int32)
                    qv = ckv.ckv_partition_quality(n_tok, idx.n_sinks, table.e[:, :idx.l_cap].cpu().numpy(),
                                                   np.ascontiguousarray(idx.label.cpu().numpy()), gamma)
                elif do_refresh and t + 1 < steps:
                    torch.cuda.synchronize()
                    t0 = time.perf_counter()
                    tm = {}
                    qv = dec.refresh(table, gamma, n_threads=host_threads(), timings=tm)
                    torch.cuda.synchronize()
                    ref_ms.append(round((time.perf_counter() - t0) * 1e3, 1))
                    phases.append({k: round(v, 1) for k, v in tm.items()})
                else:
                    idx = dec.idx
                    lens = kv.seq_len.cpu().numpy()
                    n_tok = lens[table.graph_seq.cpu().numpy()].astype(np.int32)
                    qv = ckv.ckv_partition_quality(n_tok, idx.n_sinks, table.e[:, :idx.l_cap].cpu().numpy(),
                                                   np.ascontiguousarray(idx.label.cpu().numpy()), gamma)
                qual.append(round(float(np.mean(qv)), 4))
                ncomm.append(round(float(dec.idx.n_comm.float().mean()), 1))
        R = torch.stack(rec).cpu().numpy()            # [steps][G * hpg] = [steps][Hq] per head
        E = torch.stack(err).cpu().numpy()
        win = [round(float(R[i:i + interval].mean()), 4) for i in range(0, steps, interval)]
        out[name] = {"recall_mean": round(float(R.mean()), 4), "recall_drift_heads": round(float(R[drift].mean()), 4),
                     "recall_prompt_topic_heads": round(float(R[~drift].mean()), 4),
                     "recall_by_window": win,
                     "out_rel_err_mean": round(float(E.mean()), 4),
                     "out_rel_err_drift_heads": round(float(E[drift].mean()), 4),
                     "modularity_by_window": qual, "communities_by_window": ncomm,
                     "initial_partition": {"modularity_mean": round(float(np.mean(q_init)), 4), "ms": round(init_ms, 1)}}
        if do_refresh:
            out[name]["refresh_ms"] = ref_ms
            out[name]["refresh_phases_ms"] = phases
            out[name]["refresh_ms_per_step_amortised"] = round(float(np.mean(ref_ms)) / interval, 3) if ref_ms else None
        if name == "refresh_async":
            out[name]["how"] = ("partition of a snapshot on host threads while steps go on; applied at the first "
                                "step after it is ready, at most interval/2 steps after the snapshot (then waiting "
                                "for it), the tokens decoded meanwhile placed by the vote of their edges; refresh_ms "
                                "is the time the step loop spent on it (snapshot, wait, place, build; not the drain "
                                "of the steps already queued on the GPU)")
            out[name]["applied_after_steps"] = lags
        del layer, dec, kv, table
        torch.cuda.empty_cache()
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
            ckv.ckv_score_centroids(L.kv, L.idx, q, b.scores, b.ws)
            ckv.ckv_time_next_launch(*ev[i][li][1])
            ckv.ckv_select_communities(L.kv, L.idx, q, b.scores, L.dec.budget, L.dec.max_comm, b.sel, b.sel_n,
                                       b.top, b.tok_list, b.tok_n, b.ws)
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
    import torch
    from community_kv_retrieval_amd import synth
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
    return rows_read_rate(kv, rows, row_bytes, reps)


def rows_read_rate(kv, rows, row_bytes, reps, cold=True):
    """ckv_read_rows over the given row ids, timed with dispatch-stamped events:
    back to back (warm), and with cold=True also each launch after the 512 MB
    read that evicts the MALL, as the cold step passes do."""
    import numpy as np
    import torch
    from community_kv_retrieval_amd import ckv
    n = rows.numel()
    part = torch.zeros(((n + 255) // 256,), dtype=torch.int32, device="cuda")
    for _ in range(5):
        ckv.ckv_read_rows(kv, rows, part)
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda") if cold else None
    if flush is not None:
        for _ in range(2):  # the flush's own first launches, untimed
            flush.amax()

    def timed(flushed):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, c in ev:
            a.record()
            c.record()
        torch.cuda.synchronize()
        for a, c in ev:
            if flushed:
                flush.amax()
            ckv.ckv_time_next_launch(a, c)
            ckv.ckv_read_rows(kv, rows, part)
        torch.cuda.synchronize()
        return float((np.array([a.elapsed_time(c) for a, c in ev]) * 1e3).mean())

    us = timed(False)
    gbps = n * row_bytes / (us * 1e-6) / 1e9
    out = {"kernel": "read_rows", "rows": n, "bytes_per_launch": n * row_bytes,
           "avg_launch_us": round(us, 2), "gbps": round(gbps, 1), "frac_of_8tbps": round(gbps / HBM_PEAK_GBPS, 4)}
    if cold:
        us_c = timed(True)
        gbps_c = n * row_bytes / (us_c * 1e-6) / 1e9
        out["cold"] = {"avg_launch_us": round(us_c, 2), "gbps": round(gbps_c, 1),
                       "frac_of_8tbps": round(gbps_c / HBM_PEAK_GBPS, 4)}
    del flush
    return out


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
