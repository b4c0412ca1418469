"""Seeded synthetic workloads for the CommunityKV decode step.

This module only draws inputs: planted community labels, keys, values and
the per-step queries and new tokens.  It holds none of the method's
arithmetic (no centroids, scores, selection, attention or assignment), so
that both the HIP path and the CPU oracle can consume exactly the same
tensors without sharing any computation.

The planted partition stands in for the prefill-time Leiden partition that
the CommunityKV page (Figure 1, panel 2) computes from the top-kappa token
graph: tokens of one community are noisy copies of one random centre, so
keys of a community are close to each other and far from other centres.

Every tensor is a deterministic function of (workload, seed, layer, batch
row, kv head, step) through numpy's SeedSequence spawn keys, so any slice can
be regenerated on its own.  Float data is drawn in fp32 and then rounded to
the workload's storage dtype (bf16 rounding is round-to-nearest-even, done by
torch); the oracle reads those rounded values exactly.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np
import torch

# stream tags for SeedSequence spawn keys
_T_PART, _T_KEY, _T_VAL, _T_STEP, _T_LEN, _T_DEV, _T_DEV_STEP, _T_PREFILL, _T_DRIFT = 1, 2, 3, 4, 5, 6, 7, 8, 9

PER_HEAD = "per_head"
GROUP = "group"


@dataclass(frozen=True)
class Workload:
    """Shape and distribution of one synthetic decode workload."""

    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str                 # storage dtype of K/V/q: "f32" or "bf16"
    n_ctx: int                 # prefill length (upper bound when lengths vary)
    n_sinks: int
    mode: str                  # PER_HEAD (one graph per query head) or GROUP (one per kv head)
    budget: int                # token budget for the selected communities (sinks not counted)
    max_comm: int              # cap on the number of selected communities (0 = no cap)
    kappa: int
    steps: int
    sm_scale: float            # softmax scale applied to q.k
    key_scale: float           # keys are (centre + noise) * key_scale
    noise: float               # std of the per-token noise around a centre
    partition: str             # "iid" (uniform labels) or "geometric"
    n_components: int = 0      # for partition == "iid"
    mean_size: int = 16        # for partition == "geometric"
    min_size: int = 4
    max_size: int = 64
    n_layers: int = 1
    min_ctx: int = 0           # > 0: per-sequence lengths uniform in [min_ctx, n_ctx]
    cent_budget: int = 0       # centroid entries of next-ranked communities (Table 6; 0 = none)
    drift_topics: int = 0      # > 0: decode steps also draw from this many centres absent from the prompt
    drift_rate: float = 0.0    # chance that a head's decode query (and the new key) takes such a centre

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_graphs(self) -> int:
        per = self.n_q_heads if self.mode == PER_HEAD else self.n_kv_heads
        return self.batch * per

    @property
    def heads_per_graph(self) -> int:
        return 1 if self.mode == PER_HEAD else self.group

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def graph_of(self, b: int, qh: int) -> int:
        """Graph id that query head qh of sequence b reads."""
        if self.mode == PER_HEAD:
            return b * self.n_q_heads + qh
        return b * self.n_kv_heads + qh // self.group

    def graph_coords(self, g: int):
        """(sequence, kv head, first query head, number of query heads) of graph g."""
        if self.mode == PER_HEAD:
            b, qh = divmod(g, self.n_q_heads)
            return b, qh // self.group, qh, 1
        b, kh = divmod(g, self.n_kv_heads)
        return b, kh, kh * self.group, self.group

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads.  Names describe the shape, not a model checkpoint: no
# weights are involved, only the attention-layer geometry.
PRESETS = {
    "tiny": Workload(
        name="tiny", batch=1, n_q_heads=1, n_kv_heads=1, head_dim=64, dtype="f32",
        n_ctx=1024, n_sinks=4, mode=PER_HEAD, budget=1 << 30, max_comm=4, kappa=4,
        steps=16, sm_scale=1.0 / 8.0, key_scale=1.0, noise=0.3, partition="iid",
        n_components=32),
    "qwen3_8b_32k": Workload(
        name="qwen3_8b_32k", batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128,
        dtype="bf16", n_ctx=32768, n_sinks=4, mode=PER_HEAD, budget=2048, max_comm=0,
        kappa=8, steps=64, sm_scale=1.0, key_scale=1.0 / math.sqrt(128), noise=0.25,
        partition="geometric"),
    "llama31_8b_128k": Workload(
        name="llama31_8b_128k", batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128,
        dtype="bf16", n_ctx=131072, n_sinks=4, mode=PER_HEAD, budget=4096, max_comm=0,
        kappa=8, steps=128, sm_scale=1.0, key_scale=1.0 / math.sqrt(128), noise=0.25,
        partition="geometric"),
    "llama31_8b_128k_group_b8": Workload(
        name="llama31_8b_128k_group_b8", batch=8, n_q_heads=32, n_kv_heads=8,
        head_dim=128, dtype="bf16", n_ctx=131072, n_sinks=4, mode=GROUP, budget=4096,
        max_comm=0, kappa=8, steps=128, sm_scale=1.0, key_scale=1.0 / math.sqrt(128),
        noise=0.25, partition="geometric"),
    "qwen3_8b_stream_36l": Workload(
        name="qwen3_8b_stream_36l", batch=8, n_q_heads=32, n_kv_heads=8, head_dim=128,
        dtype="bf16", n_ctx=131072, min_ctx=16384, n_sinks=4, mode=GROUP, budget=4096,
        max_comm=0, kappa=8, steps=256, sm_scale=1.0, key_scale=1.0 / math.sqrt(128),
        noise=0.25, partition="geometric", n_layers=36),
}


def preset(name: str) -> Workload:
    return PRESETS[name]


def _rng(seed: int, tag: int, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(entropy=seed, spawn_key=(tag,) + tuple(key)))


def _to_storage(x: np.ndarray, w: Workload) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t if w.dtype == "f32" else t.to(torch.bfloat16)


def seq_lengths(w: Workload, seed: int, layer: int = 0) -> List[int]:
    """Prefill length of each sequence (all equal unless min_ctx > 0)."""
    if w.min_ctx <= 0:
        return [w.n_ctx] * w.batch
    r = _rng(seed, _T_LEN)
    return [int(x) for x in r.integers(w.min_ctx, w.n_ctx + 1, size=w.batch)]


@dataclass
class Partition:
    """Planted partition of one (layer, sequence, kv head) slice."""

    centers: np.ndarray   # [C][d] float32, unscaled
    labels: np.ndarray    # [n] int32, -1 for sinks
    n_comm: int


def gen_partition(w: Workload, seed: int, layer: int, b: int, kh: int, n: int,
                  with_centers: bool = True) -> Partition:
    """Draw centres and labels for positions 0..n-1 (0..n_sinks-1 are sinks).
    The centres are the last draw, so with_centers=False gives the same labels."""
    r = _rng(seed, _T_PART, layer, b, kh)
    d = w.head_dim
    labels = np.full(n, -1, dtype=np.int32)
    m = n - w.n_sinks
    if w.partition == "iid":
        C = w.n_components
        centers = r.standard_normal((C, d), dtype=np.float32)
        labels[w.n_sinks:] = r.integers(0, C, size=m, dtype=np.int32)
        return Partition(centers, labels, C)
    # geometric sizes on {1,2,...} with the given mean, clamped, drawn until
    # they cover the non-sink positions; the last run takes the remainder.
    p = 1.0 / w.mean_size
    sizes: List[int] = []
    total = 0
    while total < m:
        chunk = np.clip(r.geometric(p, size=max(16, (m - total) // w.mean_size + 16)),
                        w.min_size, w.max_size)
        for s in chunk:
            s = int(min(s, m - total))
            sizes.append(s)
            total += s
            if total >= m:
                break
    C = len(sizes)
    perm = r.permutation(np.arange(w.n_sinks, n, dtype=np.int32))
    lab = np.repeat(np.arange(C, dtype=np.int32), sizes)
    labels[perm] = lab
    centers = r.standard_normal((C, d), dtype=np.float32) if with_centers else None
    return Partition(centers, labels, C)


def gen_kv(w: Workload, seed: int, layer: int, b: int, kh: int, part: Partition):
    """Keys and values [n][d] in the storage dtype for one slice."""
    n = part.labels.shape[0]
    d = w.head_dim
    rk = _rng(seed, _T_KEY, layer, b, kh)
    rv = _rng(seed, _T_VAL, layer, b, kh)
    noise = rk.standard_normal((n, d), dtype=np.float32)
    k = np.empty((n, d), dtype=np.float32)
    s = w.n_sinks
    k[:s] = noise[:s]
    k[s:] = part.centers[part.labels[s:]] + np.float32(w.noise) * noise[s:]
    k *= np.float32(w.key_scale)
    v = rv.standard_normal((n, d), dtype=np.float32)
    return _to_storage(k, w), _to_storage(v, w)


@dataclass
class Slice:
    b: int
    kh: int
    part: Partition
    k: torch.Tensor  # [n][d] storage dtype (CPU)
    v: torch.Tensor


def gen_layer(w: Workload, seed: int, layer: int = 0, with_kv: bool = True) -> List[List[Slice]]:
    """All (sequence, kv head) slices of one layer: result[b][kh]."""
    lens = seq_lengths(w, seed)
    out = []
    for b in range(w.batch):
        row = []
        for kh in range(w.n_kv_heads):
            part = gen_partition(w, seed, layer, b, kh, lens[b])
            if with_kv:
                k, v = gen_kv(w, seed, layer, b, kh, part)
            else:
                k = v = None
            row.append(Slice(b, kh, part, k, v))
        out.append(row)
    return out


def graph_labels(w: Workload, slices: List[List[Slice]]) -> List[np.ndarray]:
    """Initial labels of every graph (query heads of one kv head share the kv
    head's planted partition in per-head mode)."""
    res = []
    for g in range(w.n_graphs):
        b, kh, _, _ = w.graph_coords(g)
        res.append(slices[b][kh].part.labels)
    return res


def graph_n_comm(w: Workload, slices: List[List[Slice]]) -> List[int]:
    return [slices[w.graph_coords(g)[0]][w.graph_coords(g)[1]].part.n_comm for g in range(w.n_graphs)]


@dataclass
class StepInput:
    q: torch.Tensor      # [B][Hq][d] storage dtype
    k_new: torch.Tensor  # [B][Hkv][d]
    v_new: torch.Tensor  # [B][Hkv][d]
    target: np.ndarray   # [B][Hq] planted community each query head was drawn around


def gen_step(w: Workload, seed: int, step: int, slices: List[List[Slice]], layer: int = 0) -> StepInput:
    """Query, new key and new value for decode step `step`.

    Each query head is a planted centre of its kv head plus noise.  In
    per-head mode every query head picks its own centre; in group mode the
    heads of a group share one.  The new key is drawn around the centre of
    the group's first query head, scaled like the prefill keys.
    """
    B, Hq, Hkv, d, G = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.group
    if w.drift_topics > 0:
        return _gen_step_drift(w, seed, step, slices, layer)
    q = np.empty((B, Hq, d), dtype=np.float32)
    kn = np.empty((B, Hkv, d), dtype=np.float32)
    vn = np.empty((B, Hkv, d), dtype=np.float32)
    tgt = np.empty((B, Hq), dtype=np.int32)
    for b in range(B):
        for kh in range(Hkv):
            part = slices[b][kh].part
            r = _rng(seed, _T_STEP, layer, b, kh, step)
            if w.mode == PER_HEAD:
                cs = r.integers(0, part.n_comm, size=G)
            else:
                cs = np.repeat(r.integers(0, part.n_comm, size=1), G)
            qn = r.standard_normal((G, d), dtype=np.float32)
            for j in range(G):
                q[b, kh * G + j] = part.centers[cs[j]] + np.float32(w.noise) * qn[j]
                tgt[b, kh * G + j] = cs[j]
            kk = r.standard_normal(d, dtype=np.float32)
            kn[b, kh] = (part.centers[cs[0]] + np.float32(w.noise) * kk) * np.float32(w.key_scale)
            vn[b, kh] = r.standard_normal(d, dtype=np.float32)
    return StepInput(_to_storage(q, w), _to_storage(kn, w), _to_storage(vn, w), tgt)


def drift_centers(w: Workload, seed: int, layer: int, b: int, kh: int) -> np.ndarray:
    """The drift_topics centres of one slice that the prompt never uses [T][d]."""
    return _rng(seed, _T_DRIFT, layer, b, kh).standard_normal((w.drift_topics, w.head_dim), dtype=np.float32)


def _gen_step_drift(w: Workload, seed: int, step: int, slices, layer: int) -> StepInput:
    """gen_step with topic drift: each head's centre is, with chance
    drift_rate, one of the slice's drift centres (target -1 - topic), else a
    planted community's.  The new key follows the group's first head, so the
    cache grows with tokens of topics the prompt's partition has no community
    for: the case a re-partition (Tables 8 and 9, "Refresh") addresses."""
    B, Hq, Hkv, d, G = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.group
    q = np.empty((B, Hq, d), dtype=np.float32)
    kn = np.empty((B, Hkv, d), dtype=np.float32)
    vn = np.empty((B, Hkv, d), dtype=np.float32)
    tgt = np.empty((B, Hq), dtype=np.int32)
    for b in range(B):
        for kh in range(Hkv):
            part = slices[b][kh].part
            extra = drift_centers(w, seed, layer, b, kh)
            r = _rng(seed, _T_STEP, layer, b, kh, step)
            nh = G if w.mode == PER_HEAD else 1
            drift = r.random(nh) < w.drift_rate
            cs = np.where(drift, -1 - r.integers(0, w.drift_topics, size=nh), r.integers(0, part.n_comm, size=nh))
            if w.mode != PER_HEAD:
                cs = np.repeat(cs, G)
            qn = r.standard_normal((G, d), dtype=np.float32)
            cen = [extra[-1 - c] if c < 0 else part.centers[c] for c in cs]
            for j in range(G):
                q[b, kh * G + j] = cen[j] + np.float32(w.noise) * qn[j]
                tgt[b, kh * G + j] = cs[j]
            kk = r.standard_normal(d, dtype=np.float32)
            kn[b, kh] = (cen[0] + np.float32(w.noise) * kk) * np.float32(w.key_scale)
            vn[b, kh] = r.standard_normal(d, dtype=np.float32)
    return StepInput(_to_storage(q, w), _to_storage(kn, w), _to_storage(vn, w), tgt)


# --------------------------------------------------------------------------
# Device-side streams for the multi-layer workload.  The key, value and centre
# draws of one slice come from a torch generator on the GPU seeded from the
# slice's SeedSequence key, so any slice can be regenerated (and copied to
# the host for the oracle) on its own; the labels use the host partition
# stream above.
# --------------------------------------------------------------------------

def torch_generator(seed: int, tag: int, *key: int, device="cuda") -> torch.Generator:
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(tag,) + tuple(key))
    g = torch.Generator(device=device)
    g.manual_seed(int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64(0x7FFFFFFFFFFFFFFF)))
    return g


def gen_slice_device(w: Workload, seed: int, layer: int, b: int, kh: int, part: Partition, device="cuda"):
    """Centres [C][d] (float32) and keys, values [n][d] (storage dtype) of one
    slice, drawn on the device: keys are (centre of the label + noise) *
    key_scale, sinks pure noise * key_scale, values N(0, I)."""
    n, d, s = part.labels.shape[0], w.head_dim, w.n_sinks
    g = torch_generator(seed, _T_DEV, layer, b, kh, device=device)
    centers = torch.randn((part.n_comm, d), generator=g, device=device)
    k = torch.randn((n, d), generator=g, device=device)
    v = torch.randn((n, d), generator=g, device=device)
    lab = torch.from_numpy(part.labels[s:].astype(np.int64)).to(device)
    k[s:] = centers[lab] + float(w.noise) * k[s:]
    k.mul_(float(w.key_scale))
    return centers, k.to(w.torch_dtype), v.to(w.torch_dtype)


def gen_steps_device(w: Workload, seed: int, layer: int, steps: int, centers: torch.Tensor,
                     offsets: np.ndarray, n_comm: np.ndarray, device="cuda"):
    """Queries, new keys and new values of `steps` decode steps of one layer,
    as device tensors [steps][B][Hq][d], [steps][B][Hkv][d], [steps][B][Hkv][d].
    `centers` holds the layer's centres, slice (b, kh) at rows
    offsets[b, kh] .. offsets[b, kh] + n_comm[b, kh].  Same rules as gen_step:
    every query head draws a planted centre of its kv head (the heads of a
    group share one in group mode), the new key follows the group's first
    head's centre."""
    B, Hq, Hkv, d, G = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.group
    r = _rng(seed, _T_DEV_STEP, layer)
    u = r.random((steps, B, Hkv, G))
    if w.mode != PER_HEAD:
        u[..., 1:] = u[..., :1]
    cs = np.minimum((u * n_comm[None, :, :, None]).astype(np.int64), n_comm[None, :, :, None] - 1)
    rows = torch.from_numpy((cs + offsets[None, :, :, None]).reshape(steps, B, Hq)).to(device)
    g = torch_generator(seed, _T_DEV_STEP, layer, device=device)
    q = centers[rows] + float(w.noise) * torch.randn((steps, B, Hq, d), generator=g, device=device)
    first = rows.view(steps, B, Hkv, G)[..., 0]
    kn = (centers[first] + float(w.noise) * torch.randn((steps, B, Hkv, d), generator=g, device=device)) \
        * float(w.key_scale)
    vn = torch.randn((steps, B, Hkv, d), generator=g, device=device)
    return q.to(w.torch_dtype), kn.to(w.torch_dtype), vn.to(w.torch_dtype)


def gen_prefill_queries(w: Workload, seed: int, layer: int, b: int, slices_b, n: Optional[int] = None) -> torch.Tensor:
    """Queries of the prompt positions 0..n-1 of sequence b, [n][Hq][d] in the
    storage dtype: a head of kv head kh asks at position i for the centre of
    i's planted community in that slice plus N(0, noise^2) (the decode query
    rule), a sink position asks N(0, I).  slices_b: gen_layer(...)[b] (or
    partitions with centres, indexed by kv head)."""
    G = w.n_q_heads // w.n_kv_heads
    parts = [getattr(x, "part", x) for x in slices_b]
    n = parts[0].labels.shape[0] if n is None else n
    r = _rng(seed, _T_PREFILL, layer, b)
    out = np.empty((n, w.n_q_heads, w.head_dim), dtype=np.float32)
    for kh, part in enumerate(parts):
        lab = part.labels[:n]
        base = part.centers[np.maximum(lab, 0)]
        sink = lab < 0
        for g in range(G):
            noise = r.standard_normal((n, w.head_dim), dtype=np.float32)
            q = base + np.float32(w.noise) * noise
            q[sink] = noise[sink]
            out[:, kh * G + g] = q
    return _to_storage(out, w)


def gen_prefill_queries_device(w: Workload, seed: int, layer: int, b: int, parts, device="cuda") -> torch.Tensor:
    """gen_prefill_queries' rule drawn on the device (long prompts): [n][Hq][d]
    in the storage dtype, noise from a torch generator keyed like the host
    stream.  parts: the sequence's partitions with centres, by kv head."""
    G = w.n_q_heads // w.n_kv_heads
    n = parts[0].labels.shape[0]
    g = torch_generator(seed, _T_PREFILL, layer, b, device=device)
    out = torch.empty((n, w.n_q_heads, w.head_dim), dtype=w.torch_dtype, device=device)
    for kh, part in enumerate(parts):
        lab = torch.from_numpy(part.labels.astype(np.int64)).to(device)
        cent = torch.from_numpy(part.centers).to(device)
        base = cent[lab.clamp(min=0)]
        sink = (lab < 0)[:, None]
        for h in range(G):
            noise = torch.randn((n, w.head_dim), generator=g, device=device)
            out[:, kh * G + h] = torch.where(sink, noise, base + float(w.noise) * noise).to(w.torch_dtype)
    return out
