"""CPU oracle for the CommunityKV sparse decode step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
module: only the tests, the smoke check and the benchmark's CPU-baseline leg
use it.  It shares no code with the HIP library; the two meet only in the
seeded inputs.

Source: "CommunityKV: Efficient Long-Context Decoding via Graph Partitioning"
(McKenna, Alexandridis, Susanj, Liu), Figure 1 caption, panel (3), the
incremental update.  Each decoding step compares the query with the community
centroids and keeps the best communities.  Attention over their tokens and
the sinks is computed exactly.  The tokens it weights most become the new
token's edges, and they decide its community at a cost independent of the
context length.  Table 1 gives the per-step update as O(d) and the retrieval as a pass
over the centroids.  Table 6 fixes the defaults (kappa = 8, per-head graphs,
sinks excluded from the top-kappa pool).

Table 6 also ablates a centroid budget: the attention then takes, besides the
exact tokens, the centroids of the next-ranked communities (centroid_communities,
attend_with_centroids).

The same caption's panel (1), the prefill graph construction, is here too:
every prompt token is linked to the earlier non-sink tokens it attends to
most (prefill_edges).

Everything is computed in float64 with plain numpy, one graph at a time, in
the order the caption describes.  Where the page leaves a step open, the
reading taken is stated at the function that implements it.

Decision precision.  Two integer decisions rest on floating point:
  * community selection compares centroid scores.  The centroid table is held
    in float32 (the mean of the members' keys, computed exactly in float64,
    rounded once to float32); a score is the float64 dot product of the
    aggregated query with that float32 centroid, rounded once to float32.
    Ties of the float32 score go to the lower community id.
  * the top-kappa edge choice compares attention weights, computed here in
    float64; ties go to the lower token position.
A checker compares a device decision with these under a 1e-6 tie window.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

NEG_INF32 = np.float32(-np.inf)


# --------------------------------------------------------------------------
# Centroids (Figure 1, panel (2): one centroid, drawn as a star, per community)
# --------------------------------------------------------------------------

def community_sums(keys: np.ndarray, labels: np.ndarray, n_comm: int):
    """Exact float64 key sum and member count of every community.

    keys: [n][d]; labels: [n] with -1 for tokens in no community (sinks).
    Sums of bf16/fp32 keys in float64 are exact for these magnitudes.
    """
    keys = np.asarray(keys, dtype=np.float64)
    labels = np.asarray(labels)
    d = keys.shape[1]
    m = labels >= 0
    sums = np.zeros((n_comm, d), dtype=np.float64)
    np.add.at(sums, labels[m], keys[m])
    counts = np.bincount(labels[m], minlength=n_comm).astype(np.int64)
    return sums, counts


def community_means(sums: np.ndarray, counts: np.ndarray) -> np.ndarray:
    """float64 centroid = mean of the members' keys (0 for an empty community)."""
    out = np.zeros_like(sums)
    nz = counts > 0
    out[nz] = sums[nz] / counts[nz, None].astype(np.float64)
    return out


def scoring_centroids(sums: np.ndarray, counts: np.ndarray) -> np.ndarray:
    """The centroid table as stored for scoring: the float64 mean rounded once to float32."""
    return community_means(sums, counts).astype(np.float32)


# --------------------------------------------------------------------------
# Retrieval (Figure 1, panel (3): the query is compared with every centroid and
# the best communities are kept, within a token budget)
# --------------------------------------------------------------------------

def aggregate_query(q_heads: np.ndarray) -> np.ndarray:
    """Query vector a graph scores with.

    One graph per query head: the head's own query.  Query-group graphs (the
    page's "query group" aggregation, Table 5 / Table 6): the score of a
    community is the sum over the group's heads of q_h . centroid, which by
    linearity is (sum_h q_h) . centroid.
    """
    q = np.asarray(q_heads, dtype=np.float64).reshape(-1, np.shape(q_heads)[-1])
    return q.sum(axis=0)


def score_communities(qbar: np.ndarray, cent32: np.ndarray, counts: np.ndarray) -> np.ndarray:
    """s[c] = qbar . centroid[c] (float64 sum, rounded to float32); -inf for empty c."""
    s = (cent32.astype(np.float64) @ np.asarray(qbar, dtype=np.float64)).astype(np.float32)
    s[np.asarray(counts) <= 0] = NEG_INF32
    return s


def rank_communities(scores: np.ndarray, counts: np.ndarray) -> np.ndarray:
    """Non-empty communities ordered by score, highest first; ties: lower id first."""
    ids = np.nonzero(np.asarray(counts) > 0)[0]
    order = np.lexsort((ids, -scores[ids].astype(np.float64)))
    return ids[order]


def select_communities(scores: np.ndarray, counts: np.ndarray, budget: int,
                       max_comm: int = 0) -> np.ndarray:
    """Communities retrieved for attention, as ascending ids.

    Reading of the budgeted retrieval of a subset of communities: walk the
    communities from the best score down and keep each one while the running
    member count stays within the budget; the first community that would
    exceed it ends the walk (no skipping ahead to smaller ones).  Sink tokens
    are not counted against the budget.  With max_comm > 0 the walk also stops
    after max_comm communities (the tiny workload's fixed top-4).
    """
    taken: List[int] = []
    total = 0
    for c in rank_communities(scores, counts):
        if max_comm > 0 and len(taken) == max_comm:
            break
        if total + int(counts[c]) > budget:
            break
        taken.append(int(c))
        total += int(counts[c])
    return np.array(sorted(taken), dtype=np.int64)


def attended_positions(labels: np.ndarray, n_sinks: int, selected: np.ndarray) -> np.ndarray:
    """Token set of the exact attention: the sinks plus every member of a
    selected community, as ascending positions.  `labels` covers exactly the
    tokens already in the cache (the new token is not among them)."""
    labels = np.asarray(labels)
    members = np.nonzero(np.isin(labels, np.asarray(selected)) & (labels >= 0))[0]
    sinks = np.arange(min(n_sinks, labels.shape[0]))
    return np.union1d(sinks, members)


def centroid_communities(scores: np.ndarray, counts: np.ndarray, selected: np.ndarray,
                         n_cent: int) -> np.ndarray:
    """Communities whose centroid the attention takes besides the exact tokens
    (Table 6, "Centroid Budget": 0, 4, 16, 64 or 256; 0, the default, takes
    none), as ascending ids.

    Reading (the page gives only the budget values): the n_cent best-ranked
    non-empty communities that the budget walk did not take, in the ranking of
    rank_communities; all of them when fewer are left.  After a plain walk
    these are the ranks just past the taken prefix, starting with the
    community that ended the walk.
    """
    if n_cent <= 0:
        return np.zeros(0, dtype=np.int64)
    taken = {int(c) for c in np.asarray(selected)}
    rest = [int(c) for c in rank_communities(scores, counts) if int(c) not in taken]
    return np.array(sorted(rest[:n_cent]), dtype=np.int64)


# --------------------------------------------------------------------------
# Exact attention on the subset (Figure 1, panel (3))
# --------------------------------------------------------------------------

def attend(q_heads: np.ndarray, keys: np.ndarray, values: np.ndarray, sm_scale: float):
    """Softmax attention of each query head over the given keys and values.

    Returns (out [h][d], probs [h][T], logits [h][T]) with
    logits = sm_scale * q . k, probs = softmax(logits) per head, out = probs @ V.
    With no token at all (no sinks and no community within the budget, a case
    the page never meets) the output is the empty sum, zero (reading R23).
    """
    q = np.asarray(q_heads, dtype=np.float64).reshape(-1, np.shape(q_heads)[-1])
    K = np.asarray(keys, dtype=np.float64)
    V = np.asarray(values, dtype=np.float64)
    if K.shape[0] == 0:
        empty = np.zeros((q.shape[0], 0))
        return np.zeros((q.shape[0], V.shape[-1])), empty, empty
    z = float(sm_scale) * (q @ K.T)
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    p = e / e.sum(axis=1, keepdims=True)
    return p @ V, p, z


def attend_with_centroids(q_heads: np.ndarray, keys: np.ndarray, values: np.ndarray,
                          cent_keys: np.ndarray, cent_values: np.ndarray, cent_counts: np.ndarray,
                          sm_scale: float):
    """Softmax attention over the attended tokens and the centroid entries of
    the centroid budget (Table 6).

    Reading: a centroid entry stands for its n members as if every member's
    key were the centroid mu, so it enters the softmax as one term of logit
    sm_scale * q . mu + ln n (the mass n exp(sm_scale q . mu)) with the
    members' mean value as its value.  It is not a token: it never becomes an
    edge, but its mass is in the normaliser of every token's probability.
    cent_keys: [N][d] the stored (float32) centroids; cent_values: [N][d] the
    mean member values; cent_counts: [N] member counts (> 0).
    Returns (out [h][d], token probs [h][T], token logits [h][T],
    centroid probs [h][N], centroid logits [h][N]).
    """
    q = np.asarray(q_heads, dtype=np.float64).reshape(-1, np.shape(q_heads)[-1])
    K = np.asarray(keys, dtype=np.float64).reshape(-1, q.shape[1])
    V = np.asarray(values, dtype=np.float64).reshape(-1, q.shape[1])
    MU = np.asarray(cent_keys, dtype=np.float64).reshape(-1, q.shape[1])
    NU = np.asarray(cent_values, dtype=np.float64).reshape(-1, q.shape[1])
    n = np.asarray(cent_counts, dtype=np.float64)
    T = K.shape[0]
    zt = float(sm_scale) * (q @ K.T)
    zc = float(sm_scale) * (q @ MU.T) + np.log(n)[None, :]
    z = np.concatenate([zt, zc], axis=1)
    if z.shape[1] == 0:
        return np.zeros((q.shape[0], V.shape[1])), zt, zt, zc, zc
    e = np.exp(z - z.max(axis=1, keepdims=True))
    p = e / e.sum(axis=1, keepdims=True)
    out = p[:, :T] @ V + p[:, T:] @ NU
    return out, p[:, :T], zt, p[:, T:], zc


def dense_attend(q_heads: np.ndarray, keys: np.ndarray, values: np.ndarray, sm_scale: float,
                 chunk: int = 1 << 15) -> np.ndarray:
    """Full attention over every cached token, in float64 (chunked so large
    contexts fit in memory; the chunks merge exactly by rescaling)."""
    q = np.asarray(q_heads, dtype=np.float64).reshape(-1, np.shape(q_heads)[-1])
    n = keys.shape[0]
    z = np.concatenate([float(sm_scale) * (q @ np.asarray(keys[i:i + chunk], dtype=np.float64).T)
                        for i in range(0, n, chunk)], axis=1)
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    out = np.zeros((q.shape[0], values.shape[1]))
    for i in range(0, n, chunk):
        out += e[:, i:i + chunk] @ np.asarray(values[i:i + chunk], dtype=np.float64)
    return out / e.sum(axis=1, keepdims=True)


def attention_mass_recall(q_heads: np.ndarray, keys: np.ndarray, positions: np.ndarray,
                          sm_scale: float) -> np.ndarray:
    """Share of each head's dense softmax mass over every cached token that
    the attended positions carry (the page's attention-mass recall, Figure 3):
    sum over j in positions of softmax_j(sm_scale * q . K^T).  One value per
    head; 1 when every cached token is attended."""
    q = np.asarray(q_heads, dtype=np.float64).reshape(-1, np.shape(q_heads)[-1])
    z = float(sm_scale) * (q @ np.asarray(keys, dtype=np.float64).T)
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return p[:, np.asarray(positions, dtype=np.int64)].sum(axis=1)


# --------------------------------------------------------------------------
# Incremental update (Figure 1, panel (3); Table 1 "Per-step Update O(d)")
# --------------------------------------------------------------------------

def edge_weights(probs: np.ndarray) -> np.ndarray:
    """Attention weight of each attended token for the graph.

    One graph per query head: that head's softmax probability.  Query-group
    graphs: the sum of the group's per-head probabilities (reading: the group
    graph's edge weight is the summed attention of its heads).
    """
    return np.atleast_2d(np.asarray(probs, dtype=np.float64)).sum(axis=0)


def top_kappa(weights: np.ndarray, positions: np.ndarray, kappa: int, n_sinks: int) -> np.ndarray:
    """The new token's edges: the kappa attended tokens of largest weight.

    Sinks are excluded from the pool (Figure 1, panel (1); Table 6 "sinks
    excluded").  Ties go to the lower position.  Fewer than kappa candidates:
    all of them.  Returned in rank order.
    """
    positions = np.asarray(positions)
    pool = positions >= n_sinks
    w = np.asarray(weights, dtype=np.float64)[pool]
    pos = positions[pool]
    order = np.lexsort((pos, -w))
    return pos[order[:kappa]]


def majority_vote(edge_labels: Sequence[int]) -> int:
    """Community holding most of the edges; ties go to the lowest id.
    Returns -1 when there are no labelled edges."""
    lab = np.asarray([x for x in edge_labels if x >= 0], dtype=np.int64)
    if lab.size == 0:
        return -1
    vals, cnt = np.unique(lab, return_counts=True)
    return int(vals[np.argmax(cnt)])  # unique() sorts ids, argmax takes the first maximum


# --------------------------------------------------------------------------
# Whole-step loop over many graphs
# --------------------------------------------------------------------------

# --------------------------------------------------------------------------
# Prefill graph construction (Figure 1, panel (1)): each query is connected to
# the keys it attends to most, sinks left out of the pool.  It precedes the
# partition (panel (2)) and the decode path; Table 10 times it as the prefill's
# fused top-kappa selection.
# --------------------------------------------------------------------------

def causal_probs(q_heads: np.ndarray, keys: np.ndarray, sm_scale: float) -> np.ndarray:
    """Causal softmax of every query position over the keys at or before it.

    q_heads: [n][h][d] (the heads of one graph), keys: [n][d].  Returns
    p [h][n][n] with p[h, i, j] = softmax_j(sm_scale * q[i, h] . k[j]) over
    j <= i (reading: the prefill attention is the model's causal attention,
    the token itself included) and 0 for j > i.
    """
    q = np.asarray(q_heads, dtype=np.float64)
    K = np.asarray(keys, dtype=np.float64)
    n = K.shape[0]
    z = float(sm_scale) * np.einsum("ihd,jd->hij", q, K)
    future = np.triu(np.ones((n, n), dtype=bool), k=1)
    z[:, future] = -np.inf
    e = np.exp(z - z.max(axis=2, keepdims=True))
    return e / e.sum(axis=2, keepdims=True)


def prefill_edges(q_heads: np.ndarray, keys: np.ndarray, n_sinks: int, kappa: int, sm_scale: float):
    """Top-kappa edges of every query position of one graph.

    The weight of key j for query i is the graph's attention weight: the
    head's probability (one head) or the sum of the group's probabilities
    (query group; as in the decode step).  Candidates are the keys
    n_sinks <= j < i: sinks never become edges (Table 6) and a token is not
    its own edge (reading: an edge links two tokens), while the token itself
    stays in the softmax normaliser.  Ties go to the lower position; fewer
    than kappa candidates: all of them.

    Returns edges [n][kappa] (int64, -1 padded) and weights [n][kappa]
    (float64, 0 padded), each row in rank order.
    """
    w = causal_probs(q_heads, keys, sm_scale).sum(axis=0)
    n = w.shape[0]
    edges = np.full((n, kappa), -1, dtype=np.int64)
    weights = np.zeros((n, kappa), dtype=np.float64)
    for i in range(n):
        cand = np.arange(n_sinks, i)
        if cand.size == 0:
            continue
        wi = w[i, n_sinks:i]
        order = np.lexsort((cand, -wi))[:kappa]
        edges[i, :order.size] = cand[order]
        weights[i, :order.size] = wi[order]
    return edges, weights


def prefill_row_weights(q_heads_row: np.ndarray, i: int, keys: np.ndarray, sm_scale: float) -> np.ndarray:
    """The graph weight of every key j <= i for query position i: the causal
    softmax over keys 0..i of each head (q_heads_row: [h][d]), summed over
    the heads.  Returns [i + 1] float64."""
    K = np.asarray(keys, dtype=np.float64)[:i + 1]
    z = float(sm_scale) * (np.asarray(q_heads_row, dtype=np.float64) @ K.T)  # [h][i+1]
    e = np.exp(z - z.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)).sum(axis=0)


def prefill_edges_rows(q_heads_rows: np.ndarray, rows: Sequence[int], keys: np.ndarray, n_sinks: int,
                       kappa: int, sm_scale: float):
    """prefill_edges for selected query positions only (long prefixes).

    q_heads_rows: [len(rows)][h][d], the queries of those positions; keys:
    [>= max(rows) + 1][d].  Same definition, one row at a time.
    """
    edges = np.full((len(rows), kappa), -1, dtype=np.int64)
    weights = np.zeros((len(rows), kappa), dtype=np.float64)
    for r, i in enumerate(rows):
        w = prefill_row_weights(q_heads_rows[r], i, keys, sm_scale)
        cand = np.arange(n_sinks, i)
        if cand.size == 0:
            continue
        wi = w[n_sinks:i]
        order = np.lexsort((cand, -wi))[:kappa]
        edges[r, :order.size] = cand[order]
        weights[r, :order.size] = wi[order]
    return edges, weights


@dataclass
class GraphState:
    """Community state of one graph."""

    b: int                   # sequence
    kh: int                  # kv head whose keys the graph indexes
    qh0: int                 # first query head of the graph
    nh: int                  # query heads of the graph
    labels: np.ndarray       # [cap] int64, -1 = sink / not yet cached
    sums: np.ndarray         # [C][d] float64
    counts: np.ndarray       # [C] int64
    vsums: np.ndarray        # [C][d] float64 exact value sums (the centroid entries' values)


@dataclass
class GraphStep:
    scores: np.ndarray
    selected: np.ndarray
    positions: np.ndarray
    out: np.ndarray          # [nh][d]
    probs: np.ndarray        # [nh][T]
    logits: np.ndarray       # [nh][T]
    weights: np.ndarray      # [T] (graph edge weight of every attended token)
    edges: np.ndarray
    assign: int
    top: int                 # best-scoring community
    cent: np.ndarray = field(default_factory=lambda: np.zeros(0, dtype=np.int64))  # centroid entries
    cent_logits: np.ndarray = field(default_factory=lambda: np.zeros((0, 0)))      # [nh][len(cent)]


class Oracle:
    """Decode-step oracle for a set of graphs of one layer.

    shape: any object with batch, n_q_heads, n_kv_heads, head_dim, n_sinks,
    mode ("per_head" | "group"), budget, max_comm, kappa, sm_scale, and
    optionally cent_budget (default 0).
    kv[b][kh] = (keys [n_b][d], values [n_b][d]) as float32-representable
    arrays (bf16 and fp32 storage both read exactly).
    graphs: which graphs to track (default: all).
    """

    def __init__(self, shape, kv, labels: Dict[int, np.ndarray], n_comm: Dict[int, int],
                 graphs: Optional[Sequence[int]] = None, extra: int = 1024):
        self.w = shape
        B, Hq, Hkv = shape.batch, shape.n_q_heads, shape.n_kv_heads
        self.group = Hq // Hkv
        per_head = shape.mode == "per_head"
        self.n_graphs = B * (Hq if per_head else Hkv)
        self.graph_ids = list(range(self.n_graphs)) if graphs is None else list(graphs)
        self.len: Dict[int, int] = {}
        self.K: Dict[tuple, np.ndarray] = {}
        self.V: Dict[tuple, np.ndarray] = {}
        self.g: Dict[int, GraphState] = {}
        for gid in self.graph_ids:
            if per_head:
                b, qh = divmod(gid, Hq)
                kh, qh0, nh = qh // self.group, qh, 1
            else:
                b, kh = divmod(gid, Hkv)
                qh0, nh = kh * self.group, self.group
            if (b, kh) not in self.K:
                k, v = kv[b][kh]
                n = k.shape[0]
                self.len[b] = n
                self.K[(b, kh)] = np.zeros((n + extra, k.shape[1]), dtype=np.float32)
                self.V[(b, kh)] = np.zeros((n + extra, v.shape[1]), dtype=np.float32)
                self.K[(b, kh)][:n] = np.asarray(k, dtype=np.float32)
                self.V[(b, kh)][:n] = np.asarray(v, dtype=np.float32)
            n = self.len[b]
            lab = np.full(n + extra, -1, dtype=np.int64)
            lab[:n] = labels[gid]
            sums, counts = community_sums(self.K[(b, kh)][:n], lab[:n], n_comm[gid])
            vsums, _ = community_sums(self.V[(b, kh)][:n], lab[:n], n_comm[gid])
            self.g[gid] = GraphState(b, kh, qh0, nh, lab, sums, counts, vsums)

    # -- pieces a checker may call on their own -----------------------------
    def centroids32(self, gid: int) -> np.ndarray:
        st = self.g[gid]
        return scoring_centroids(st.sums, st.counts)

    def graph_query(self, gid: int, q: np.ndarray) -> np.ndarray:
        st = self.g[gid]
        return np.asarray(q[st.b, st.qh0:st.qh0 + st.nh], dtype=np.float64)

    def step_graph(self, gid: int, q: np.ndarray, force_sel=None, force_edges=None,
                   force_cent=None) -> GraphStep:
        """Retrieval, attention and edge choice for one graph (no state change).
        With a centroid budget (shape.cent_budget > 0) the attention also takes
        the centroid entries of centroid_communities."""
        w, st = self.w, self.g[gid]
        n = self.len[st.b]
        qh = self.graph_query(gid, q)
        scores = score_communities(aggregate_query(qh), self.centroids32(gid), st.counts)
        ranked = rank_communities(scores, st.counts)
        top = int(ranked[0]) if ranked.size else -1
        sel = select_communities(scores, st.counts, w.budget, w.max_comm)
        if force_sel is not None:
            sel = np.array(sorted(int(c) for c in force_sel), dtype=np.int64)
        pos = attended_positions(st.labels[:n], w.n_sinks, sel)
        K = self.K[(st.b, st.kh)][pos]
        V = self.V[(st.b, st.kh)][pos]
        cent = centroid_communities(scores, st.counts, sel, getattr(w, "cent_budget", 0))
        if force_cent is not None:
            cent = np.array(sorted(int(c) for c in force_cent), dtype=np.int64)
        zc = np.zeros((qh.shape[0], 0))
        if cent.size:
            nc = st.counts[cent]
            out, p, z, _, zc = attend_with_centroids(qh, K, V, self.centroids32(gid)[cent],
                                                     st.vsums[cent] / nc[:, None].astype(np.float64), nc,
                                                     w.sm_scale)
        else:
            out, p, z = attend(qh, K, V, w.sm_scale)
        wts = edge_weights(p)
        edges = top_kappa(wts, pos, w.kappa, w.n_sinks)
        if force_edges is not None:
            edges = np.asarray(force_edges, dtype=np.int64)
        a = majority_vote(st.labels[edges])
        if a < 0:
            a = top  # no attended non-sink token: fall back to the best-scoring community
        return GraphStep(scores, sel, pos, out, p, z, wts, edges, a, top, cent, zc)

    def apply_update(self, gid: int, assign: int, k_new: np.ndarray, v_new: Optional[np.ndarray] = None):
        """label[P] = a, member count and key sum of a grow by the new token
        (so the centroid becomes the running mean (n*mu + k)/(n + 1)); the
        value sum grows by its value."""
        st = self.g[gid]
        P = self.len[st.b]
        if assign < 0:
            return
        st.labels[P] = assign
        st.sums[assign] += np.asarray(k_new, dtype=np.float64)
        if v_new is not None:
            st.vsums[assign] += np.asarray(v_new, dtype=np.float64)
        st.counts[assign] += 1

    def step(self, q, k_new, v_new, force_sel: Optional[Dict[int, Sequence[int]]] = None,
             force_edges: Optional[Dict[int, Sequence[int]]] = None) -> Dict[int, GraphStep]:
        """One decode step for every tracked graph, then append the new token.

        q: [B][Hq][d]; k_new, v_new: [B][Hkv][d] (any float dtype).
        force_sel / force_edges: per-graph decisions to adopt in place of the
        oracle's own (used after a near-tie was accepted).
        """
        q = np.asarray(q, dtype=np.float64)
        res = {}
        for gid in self.graph_ids:
            res[gid] = self.step_graph(gid, q, (force_sel or {}).get(gid), (force_edges or {}).get(gid))
        for gid in self.graph_ids:
            st = self.g[gid]
            self.apply_update(gid, res[gid].assign, k_new[st.b][st.kh], v_new[st.b][st.kh])
        self.append(k_new, v_new)
        return res

    def append(self, k_new, v_new):
        """Store the new token's key and value at position P of every tracked
        sequence and advance the cached length (after every graph's update)."""
        for (b, kh) in self.K:
            P = self.len[b]
            self.K[(b, kh)][P] = np.asarray(k_new[b][kh], dtype=np.float32)
            self.V[(b, kh)][P] = np.asarray(v_new[b][kh], dtype=np.float32)
        for b in {b for (b, _) in self.K}:
            self.len[b] += 1

    def repartition(self, gid: int, labels: np.ndarray, n_comm: int):
        """Replace graph gid's partition by `labels` (one per cached position,
        -1 for sinks) as a re-partition does ("Refresh", Tables 8 and 9): the
        community state is rebuilt from scratch, each centroid the mean of its
        members' keys (Figure 1, panel (2)), the value sums likewise."""
        st = self.g[gid]
        n = self.len[st.b]
        lab = np.full(st.labels.shape[0], -1, dtype=np.int64)
        lab[:n] = np.asarray(labels, dtype=np.int64)[:n]
        sums, counts = community_sums(self.K[(st.b, st.kh)][:n], lab[:n], n_comm)
        vsums, _ = community_sums(self.V[(st.b, st.kh)][:n], lab[:n], n_comm)
        st.labels, st.sums, st.counts, st.vsums = lab, sums, counts, vsums

    def recall(self, gid: int, q, positions) -> np.ndarray:
        """Attention-mass recall of graph gid's heads for the given attended positions."""
        st = self.g[gid]
        n = self.len[st.b]
        return attention_mass_recall(self.graph_query(gid, q), self.K[(st.b, st.kh)][:n], positions,
                                     self.w.sm_scale)

    def dense(self, q, b: int, kh: int) -> np.ndarray:
        """Dense attention of kv head kh's query heads over all cached tokens of sequence b."""
        n = self.len[b]
        qh = np.asarray(q, dtype=np.float64)[b, kh * self.group:(kh + 1) * self.group]
        return dense_attend(qh, self.K[(b, kh)][:n], self.V[(b, kh)][:n], self.w.sm_scale)
