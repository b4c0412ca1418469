"""Load a synthetic workload onto the GPU through the C ABI.

Uploads the generator's keys and values into a paged store (ckv_kv_write),
builds the community index from the planted labels (ckv_index_build) and
returns a Decoder ready to run steps.  Setup only: no step of the decode
path runs here.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

from . import ckv, synth


@dataclass
class Layer:
    kv: ckv.KVStore
    idx: ckv.CommunityIndex
    dec: ckv.Decoder
    slices: list
    lens: List[int]


def load_layer(w: synth.Workload, seed: int, extra: int, layer: int = 0, device: str = "cuda",
               page_size: int = 16, c_cap: Optional[int] = None, slices=None,
               budget: Optional[int] = None, tail_cap: Optional[int] = None) -> Layer:
    """Paged store + index for one layer of workload `w` with room for `extra`
    decode steps."""
    if slices is None:
        slices = synth.gen_layer(w, seed, layer)
    lens = [int(slices[b][0].part.labels.shape[0]) for b in range(w.batch)]
    cap = max(lens) + max(extra, 1)
    kv = ckv.KVStore(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.torch_dtype, cap, page_size,
                     device, shuffle_pages=True, seed=seed + 1000 * layer, seq_len=lens)
    for b in range(w.batch):
        for kh in range(w.n_kv_heads):
            s = slices[b][kh]
            ckv.ckv_kv_write(kv, b, kh, 0, s.k.to(device), s.v.to(device))
    mode = ckv.CKV_MODE_PER_HEAD if w.mode == synth.PER_HEAD else ckv.CKV_MODE_QUERY_GROUP
    labels = np.full((w.n_graphs, cap), -1, dtype=np.int32)
    for g, lab in enumerate(synth.graph_labels(w, slices)):
        labels[g, :lab.shape[0]] = lab
    n_comm = synth.graph_n_comm(w, slices)
    if tail_cap is None:
        tail_cap = max(1, min(4096, extra))
    idx = ckv.CommunityIndex(kv, mode, n_comm, l_cap=cap, tail_cap=tail_cap,
                             n_sinks=w.n_sinks, c_cap=c_cap, device=device, cent_budget=w.cent_budget)
    dec = ckv.Decoder(kv, idx, w.budget if budget is None else budget, w.max_comm, w.kappa, w.sm_scale, device)
    dec.build(torch.from_numpy(labels).to(device))
    return Layer(kv, idx, dec, slices, lens)


@dataclass
class StackLayer:
    """One layer of a multi-layer stack, with its step inputs on the device."""
    kv: ckv.KVStore
    idx: ckv.CommunityIndex
    dec: ckv.Decoder
    parts: list          # parts[b][kh]: host Partition (labels, n_comm; no centres)
    q: torch.Tensor      # [steps][B][Hq][d]
    k_new: torch.Tensor  # [steps][B][Hkv][d]
    v_new: torch.Tensor


def load_stack(w: synth.Workload, seed: int, steps: int, device: str = "cuda", page_size: int = 16,
               layers: Optional[List[int]] = None, log=None) -> List[StackLayer]:
    """Every layer of workload `w` (or the listed ones) with keys and values
    drawn on the device, the store sized for n_ctx + steps tokens per sequence,
    and `steps` decode steps of inputs per layer."""
    lens = synth.seq_lengths(w, seed)
    cap = w.n_ctx + max(steps, 1)
    mode = ckv.CKV_MODE_PER_HEAD if w.mode == synth.PER_HEAD else ckv.CKV_MODE_QUERY_GROUP
    out = []
    for layer in (range(w.n_layers) if layers is None else layers):
        parts = [[synth.gen_partition(w, seed, layer, b, kh, lens[b], with_centers=False)
                  for kh in range(w.n_kv_heads)] for b in range(w.batch)]
        n_comm = np.array([[p.n_comm for p in row] for row in parts], dtype=np.int64)
        offsets = np.concatenate([[0], np.cumsum(n_comm.ravel())[:-1]]).reshape(n_comm.shape)
        kv = ckv.KVStore(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.torch_dtype, cap, page_size,
                         device, shuffle_pages=True, seed=seed + 1000 * layer, seq_len=lens)
        cents = []
        for b in range(w.batch):
            for kh in range(w.n_kv_heads):
                c, k, v = synth.gen_slice_device(w, seed, layer, b, kh, parts[b][kh], device)
                ckv.ckv_kv_write(kv, b, kh, 0, k, v)
                cents.append(c)
                del k, v
        centers = torch.cat(cents)
        del cents
        q, kn, vn = synth.gen_steps_device(w, seed, layer, steps, centers, offsets, n_comm, device)
        del centers
        labels = torch.full((w.n_graphs, cap), -1, dtype=torch.int32)
        for g in range(w.n_graphs):
            b, kh, _, _ = w.graph_coords(g)
            lab = parts[b][kh].labels
            labels[g, :lab.shape[0]] = torch.from_numpy(lab)
        gn = [int(n_comm[w.graph_coords(g)[0], w.graph_coords(g)[1]]) for g in range(w.n_graphs)]
        idx = ckv.CommunityIndex(kv, mode, gn, l_cap=cap, tail_cap=max(1, min(4096, steps)),
                                 n_sinks=w.n_sinks, device=device, cent_budget=w.cent_budget)
        dec = ckv.Decoder(kv, idx, w.budget, w.max_comm, w.kappa, w.sm_scale, device)
        dec.build(labels.to(device))
        out.append(StackLayer(kv, idx, dec, parts, q, kn, vn))
        if log is not None:
            log(f"layer {layer}: {sum(lens)} tokens, {int(n_comm.sum())} communities")
    torch.cuda.synchronize()
    return out
