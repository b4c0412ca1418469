"""CPU oracle for the token graph, its Leiden partition and the refresh step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
module: only the tests, the smoke check and the benchmark's CPU-baseline leg
use it.  It shares no code with the library; the two meet only in the edge
tables they are given.

Sources.
  * "CommunityKV: Efficient Long-Context Decoding via Graph Partitioning",
    Figure 1 caption: panel (1) links every prompt token to the earlier
    tokens it attends to most (sinks excluded), panel (2) partitions that
    graph with the Leiden algorithm, panel (3) gives every decoded token its
    edges the same way.  Figure 2 (left): a resolution parameter gamma sets
    the community size.  Figure 3 (left): the modularity Q of the partition
    over generation.  Tables 8 and 9: incremental assignment ("Incr.")
    against re-partitioning the grown graph ("Refresh").
  * The algorithm itself is not on the page.  It is restated here from its
    publication: Traag, Waltman and van Eck, "From Louvain to Leiden:
    guaranteeing well-connected communities", Scientific Reports 9, 5233
    (2019), section "Leiden algorithm" and its supplementary pseudo-code:
    fast local moving of nodes, refinement of every community into
    well-connected sub-communities, aggregation of the refined partition
    with the unrefined one as the aggregate's starting partition, repeated
    until every community of the current level is one node.

Readings (the page fixes none of them):
  * The graph is undirected with integer weights.  A[u][v] counts the edges
    u -> v and v -> u in the tokens' top-kappa lists (0, 1 or 2); a token is
    never its own edge and sinks are not nodes.  Node i is token
    n_sinks + i.  The weights are the direct-attention relation Figure 1
    draws, not the attention values.
  * Quality is modularity at resolution gamma = num / den:
      H = sum_C [E_C - gamma K_C^2 / 2m],  Q = H / 2m,
    E_C = sum of A[u][v] over ordered pairs inside C (a self-loop once),
    K_C = sum of the degrees k_v = sum_u A[v][u] of C's nodes, 2m = sum_v k_v.
    Every decision compares integers (the gains times 2m * den), so it is
    exact.
  * Deterministic choices where the Leiden paper draws at random:
      - the queue of the local moving starts with the nodes in increasing
        index order and neighbours join its back in increasing index order;
      - a node moves to the candidate community of largest gain, staying
        unless some candidate is strictly better, the lower community id
        among equal gains, and a new (the lowest-numbered empty) community
        only when that is strictly better than every other choice;
      - the refinement takes the limit theta -> 0 of the paper's randomised
        merge: a singleton joins the well-connected sub-community of largest
        strictly positive gain (lowest id among equal gains), else stays;
      - aggregate nodes are numbered by their refined community's id (a
        node index) in increasing order, the aggregate's starting
        communities by their previous id in increasing order;
      - when the refinement merges nothing the partition is final (the
        aggregate would be the same graph and the loop would not end).
  * Communities of the result are numbered in order of their first token.

Parity: pinned (brute-force optimum on small graphs, closed forms of the
quality, connected components at gamma = 0, exact recovery of planted
cliques, hand-computed refinement and aggregation, and the partition
invariants the Leiden paper proves), see tests/test_leiden_pins.py.
"""
from __future__ import annotations

import heapq
from collections import deque
from typing import Dict, List, Sequence, Tuple

import numpy as np

Graph = List[Dict[int, int]]   # adjacency: node -> {neighbour: weight}, symmetric


# --------------------------------------------------------------------------
# The token graph (Figure 1, panels (1) and (3))
# --------------------------------------------------------------------------

def token_graph(edge_rows: np.ndarray, n_tokens: int, n_sinks: int) -> Graph:
    """Undirected graph of tokens n_sinks .. n_tokens - 1 from their edge rows.

    edge_rows[i] lists token i's edges (earlier non-sink tokens, -1 = none).
    Each listed edge i -> j adds one to A[i][j] and to A[j][i].
    """
    n = max(0, n_tokens - n_sinks)
    adj: Graph = [dict() for _ in range(n)]
    for i in range(n_sinks, n_tokens):
        for j in np.asarray(edge_rows[i]).tolist():
            if j < 0:
                continue
            if not (n_sinks <= j < n_tokens) or j == i:
                raise ValueError(f"token {i}: edge to {j} is not a non-sink token other than itself")
            a, b = i - n_sinks, j - n_sinks
            adj[a][b] = adj[a].get(b, 0) + 1
            adj[b][a] = adj[b].get(a, 0) + 1
    return adj


def degrees(adj: Graph) -> List[int]:
    return [sum(nb.values()) for nb in adj]


# --------------------------------------------------------------------------
# Quality (Figure 3, left: modularity Q; Figure 2: resolution gamma)
# --------------------------------------------------------------------------

def quality_terms(adj: Graph, labels: Sequence[int], gnum: int, gden: int) -> Tuple[int, int]:
    """(H * 2m * den, 2m) as exact integers for the partition `labels`."""
    k = degrees(adj)
    two_m = sum(k)
    E: Dict[int, int] = {}
    K: Dict[int, int] = {}
    for v, nb in enumerate(adj):
        c = labels[v]
        K[c] = K.get(c, 0) + k[v]
        for u, wt in nb.items():
            if labels[u] == c:
                E[c] = E.get(c, 0) + wt
    h = sum(E.get(c, 0) * two_m * gden - gnum * K[c] * K[c] for c in K)
    return h, two_m


def modularity(adj: Graph, labels: Sequence[int], gnum: int = 1, gden: int = 1) -> float:
    """Q = H / 2m of the partition (0 for a graph without edges)."""
    h, two_m = quality_terms(adj, labels, gnum, gden)
    if two_m == 0:
        return 0.0
    return h / (two_m * two_m * gden)


# --------------------------------------------------------------------------
# Leiden, phase 1: fast local moving of nodes
# --------------------------------------------------------------------------

def move_nodes_fast(adj: Graph, k: List[int], two_m: int, comm: List[int], empty: List[int],
                    gnum: int, gden: int) -> None:
    """Visit nodes from a queue; move each to the community of largest gain.

    The gain of putting v (degree k_v) into community C, v itself left out of
    every community, is proportional to A(v, C) * 2m * den - num * k_v * K_C;
    a move from D to C gains the difference of C's and D's values.  A moved
    node's neighbours outside its new community rejoin the queue.  `comm` is
    updated in place; `empty` is a min-heap of the unused community ids.
    """
    n = len(adj)
    Kc = [0] * n
    size = [0] * n
    for v in range(n):
        Kc[comm[v]] += k[v]
        size[comm[v]] += 1
    queue = deque(range(n))
    queued = [True] * n
    while queue:
        v = queue.popleft()
        queued[v] = False
        D = comm[v]
        to: Dict[int, int] = {}
        for u, wt in adj[v].items():
            if u != v:
                to[comm[u]] = to.get(comm[u], 0) + wt
        kv = k[v]
        best = D
        best_s = to.get(D, 0) * two_m * gden - gnum * kv * (Kc[D] - kv)
        for C in sorted(to):
            if C == D:
                continue
            s = to[C] * two_m * gden - gnum * kv * Kc[C]
            if s > best_s:
                best, best_s = C, s
        if best_s < 0:
            best = heapq.heappop(empty)
        if best == D:
            continue
        Kc[D] -= kv
        size[D] -= 1
        if size[D] == 0:
            heapq.heappush(empty, D)
        Kc[best] += kv
        size[best] += 1
        comm[v] = best
        for u in sorted(adj[v]):
            if u != v and comm[u] != best and not queued[u]:
                queue.append(u)
                queued[u] = True


# --------------------------------------------------------------------------
# Leiden, phase 2: refinement into well-connected sub-communities
# --------------------------------------------------------------------------

def refine(adj: Graph, k: List[int], two_m: int, comm: Sequence[int], gnum: int, gden: int) -> List[int]:
    """Refined partition of `comm`: ids are node indices, every refined
    community lies inside one community of `comm`.

    Inside a community S every node starts alone.  A node v that is
    well-connected to S (A(v, S - v) * 2m * den >= num * k_v * (K_S - k_v))
    and still alone joins, among the refined communities R inside S that are
    well-connected to S (ext(R) * 2m * den >= num * K_R * (K_S - K_R), ext(R)
    the weight from R to S - R) and adjacent to v, the one of largest
    positive gain A(v, R) * 2m * den - num * k_v * K_R.
    """
    n = len(adj)
    ref = list(range(n))
    Kr = list(k)
    size = [1] * n
    ext = [0] * n
    members: Dict[int, List[int]] = {}
    for v in range(n):
        members.setdefault(comm[v], []).append(v)
    for C in sorted(members):
        S = members[C]
        KS = sum(k[v] for v in S)
        inside = {}
        for v in S:
            inside[v] = sum(wt for u, wt in adj[v].items() if u != v and comm[u] == C)
            ext[v] = inside[v]
        for v in S:
            kv = k[v]
            if inside[v] * two_m * gden < gnum * kv * (KS - kv):
                continue
            if size[ref[v]] != 1:
                continue
            to: Dict[int, int] = {}
            for u, wt in adj[v].items():
                if u != v and comm[u] == C:
                    to[ref[u]] = to.get(ref[u], 0) + wt
            best, best_g = -1, 0
            for R in sorted(to):
                if R == ref[v]:
                    continue
                if ext[R] * two_m * gden < gnum * Kr[R] * (KS - Kr[R]):
                    continue
                g = to[R] * two_m * gden - gnum * kv * Kr[R]
                if g > best_g:
                    best, best_g = R, g
            if best < 0:
                continue
            old = ref[v]
            ext[best] += inside[v] - 2 * to[best]
            Kr[best] += kv
            size[best] += 1
            Kr[old], size[old], ext[old] = 0, 0, 0
            ref[v] = best
    return ref


# --------------------------------------------------------------------------
# Leiden, phase 3: aggregation
# --------------------------------------------------------------------------

def aggregate(adj: Graph, ref: Sequence[int], comm: Sequence[int]):
    """Graph of the refined communities and its starting partition.

    Node a of the aggregate is the a-th refined id in increasing order; its
    weight to node b sums A[u][v] over u in a, v in b (so an edge inside a
    refined community adds to a's self-loop from both ends).  Its starting
    community is the rank of its members' community of `comm` among the
    communities in use.  Returns (graph, starting communities, map from old
    node to aggregate node).
    """
    ids = sorted(set(ref))
    at = {r: a for a, r in enumerate(ids)}
    node_map = [at[ref[v]] for v in range(len(adj))]
    new: Graph = [dict() for _ in ids]
    for v, nb in enumerate(adj):
        a = node_map[v]
        for u, wt in nb.items():
            b = node_map[u]
            new[a][b] = new[a].get(b, 0) + wt
    cids = {c: i for i, c in enumerate(sorted(set(comm)))}
    start = [0] * len(ids)
    for v in range(len(adj)):
        start[node_map[v]] = cids[comm[v]]
    return new, start, node_map


# --------------------------------------------------------------------------
# The whole algorithm
# --------------------------------------------------------------------------

def first_token_order(labels: Sequence[int]) -> List[int]:
    """Renumber communities 0, 1, ... in order of their first node."""
    out, seen = [], {}
    for c in labels:
        if c not in seen:
            seen[c] = len(seen)
        out.append(seen[c])
    return out


def leiden(adj: Graph, gnum: int = 1, gden: int = 1) -> List[int]:
    """Leiden partition of `adj` at resolution gnum / gden (community per node,
    numbered in order of first node)."""
    if gnum < 0 or gden <= 0:
        raise ValueError("resolution must be num >= 0, den > 0")
    n0 = len(adj)
    k = degrees(adj)
    two_m = sum(k)
    if two_m == 0:
        return list(range(n0))
    comm = list(range(n0))
    empty: List[int] = []
    node_of = list(range(n0))
    while True:
        move_nodes_fast(adj, k, two_m, comm, empty, gnum, gden)
        n_comm = len(set(comm))
        if n_comm == len(adj):
            break
        ref = refine(adj, k, two_m, comm, gnum, gden)
        if len(set(ref)) == len(adj):
            break
        adj, comm, node_map = aggregate(adj, ref, comm)
        node_of = [node_map[a] for a in node_of]
        k = degrees(adj)
        empty = list(range(n_comm, len(adj)))
        heapq.heapify(empty)
    return first_token_order([comm[node_of[i]] for i in range(n0)])


def partition_tokens(edge_rows: np.ndarray, n_tokens: int, n_sinks: int, gnum: int = 1,
                     gden: int = 1) -> Tuple[np.ndarray, int]:
    """Community label of every token 0 .. n_tokens - 1 (-1 for the sinks)
    from the token graph of `edge_rows`, and the number of communities."""
    lab = leiden(token_graph(edge_rows, n_tokens, n_sinks), gnum, gden)
    out = np.full(n_tokens, -1, dtype=np.int64)
    out[n_sinks:] = lab
    return out, (max(lab) + 1 if lab else 0)


# --------------------------------------------------------------------------
# Tokens decoded while a partition was computed (Figure 4: the partitioning
# runs beside the model; Figure 1 panel (3): a new token joins by its edges)
# --------------------------------------------------------------------------

def extend_by_vote(labels: np.ndarray, n_comm: int, edge_rows: np.ndarray, first: int, stop: int):
    """Labels of tokens first .. stop - 1, in order, from the partition of the
    tokens before them: each joins the community most of its edges' targets
    are in (ties to the lower id), as a decode step assigns a new token; a
    token none of whose edges has a community starts one of its own (as the
    partition places a node without edges).  labels: [>= stop] int64, filled
    below `first`; returns (labels, n_comm) with rows first .. stop - 1 set."""
    out = np.array(labels, dtype=np.int64, copy=True)
    for i in range(first, stop):
        votes: Dict[int, int] = {}
        for j in np.asarray(edge_rows[i]).tolist():
            if j >= 0 and out[j] >= 0:
                votes[int(out[j])] = votes.get(int(out[j]), 0) + 1
        if votes:
            best = max(votes.values())
            out[i] = min(c for c, v in votes.items() if v == best)
        else:
            out[i] = n_comm
            n_comm += 1
    return out, n_comm
