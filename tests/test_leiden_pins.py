"""Pins of the Leiden oracle (oracle/leiden_oracle.py) to things other than
itself: hand-computed token graphs and quality values, closed forms, the
brute-force optimum over every partition of small graphs, connected
components (resolution 0), planted cliques, the resolution-limit result for
a ring of cliques, hand-computed refinement and aggregation steps, and the
guarantees the Leiden paper proves for every iteration (connected
communities, no pair of communities worth merging).  Planted mistakes in
the oracle must fail at least one of them.
"""
from __future__ import annotations

import random
from fractions import Fraction

import numpy as np
import pytest

from oracle import leiden_oracle as L


def graph(n, edges):
    adj = [dict() for _ in range(n)]
    for a, b in edges:
        adj[a][b] = adj[a].get(b, 0) + 1
        adj[b][a] = adj[b].get(a, 0) + 1
    return adj


def clique(nodes):
    return [(a, b) for i, a in enumerate(nodes) for b in nodes[i + 1:]]


def ring_of_cliques(n_cliques, m):
    e = []
    for c in range(n_cliques):
        e += clique(list(range(c * m, c * m + m)))
        e.append((c * m + m - 1, ((c + 1) % n_cliques) * m))
    return graph(n_cliques * m, e)


def partitions(n):
    """Every partition of 0..n-1 as a restricted growth string."""
    def rec(i, cur, m):
        if i == n:
            yield list(cur)
            return
        for c in range(m + 1):
            cur.append(c)
            yield from rec(i + 1, cur, max(m, c + 1))
            cur.pop()
    yield from rec(0, [], 0)


def components(adj):
    """Connected components by breadth-first search, numbered by first node."""
    lab = [-1] * len(adj)
    c = 0
    for s in range(len(adj)):
        if lab[s] >= 0:
            continue
        lab[s], todo = c, [s]
        while todo:
            v = todo.pop()
            for u in adj[v]:
                if lab[u] < 0:
                    lab[u] = c
                    todo.append(u)
        c += 1
    return lab


def q_exact(adj, labels, gamma=Fraction(1)):
    """Modularity from its definition with exact fractions: the sum over
    ordered node pairs of the same community of A_uv - gamma k_u k_v / 2m,
    divided by 2m."""
    n = len(adj)
    k = [sum(nb.values()) for nb in adj]
    two_m = sum(k)
    s = Fraction(0)
    for u in range(n):
        for v in range(n):
            if labels[u] == labels[v]:
                s += adj[u].get(v, 0) - gamma * Fraction(k[u] * k[v], two_m)
    return s / two_m


def sbm(rng, sizes, p_in, p_out):
    n = sum(sizes)
    block = np.repeat(np.arange(len(sizes)), sizes)
    perm = rng.permutation(n)          # nodes of a block are scattered
    lab = block[perm]
    e = []
    for a in range(n):
        for b in range(a + 1, n):
            if rng.random() < (p_in if lab[a] == lab[b] else p_out):
                e.append((a, b))
    return graph(n, e), lab


def token_rows(rng, n, n_sinks, kappa, n_topics):
    """Edge rows shaped like a prefill graph: token i links to earlier
    tokens of its own topic and, now and then, to a random earlier one."""
    topic = rng.integers(0, n_topics, n)
    rows = np.full((n, kappa), -1, dtype=np.int64)
    for i in range(n_sinks + 1, n):
        same = [j for j in range(n_sinks, i) if topic[j] == topic[i]][-(kappa - 1):]
        other = [int(rng.integers(n_sinks, i))] if rng.random() < 0.5 else []
        c = list(dict.fromkeys(same + other))[:kappa]
        rows[i, :len(c)] = c
    return rows


# -- the token graph ----------------------------------------------------------

def test_token_graph_hand_example():
    # 2 sinks; token 3 -> 2, token 4 -> 2 and 3, token 5 -> 4; token 4 is
    # also named by 5, token 3 by 4.  Nodes are tokens 2..5.
    rows = np.array([[-1, -1], [-1, -1], [-1, -1], [2, -1], [3, 2], [4, -1]])
    adj = L.token_graph(rows, 6, 2)
    assert adj == [{1: 1, 2: 1}, {0: 1, 2: 1}, {1: 1, 0: 1, 3: 1}, {2: 1}]
    # both directions listed: weight 2
    rows2 = np.array([[-1], [-1], [3], [2]])
    assert L.token_graph(rows2, 4, 1) == [{}, {2: 2}, {1: 2}]
    with pytest.raises(ValueError):
        L.token_graph(np.array([[-1], [0]]), 2, 1)   # an edge to a sink


# -- the quality ----------------------------------------------------------------

def test_quality_hand_value_two_triangles():
    adj = graph(6, clique([0, 1, 2]) + clique([3, 4, 5]) + [(2, 3)])
    # 2m = 14; each triangle: E = 6 ordered pairs, K = 7: H = 2 (6 - 49/14) = 5
    assert L.quality_terms(adj, [0, 0, 0, 1, 1, 1], 1, 1) == (70, 14)
    assert L.modularity(adj, [0, 0, 0, 1, 1, 1]) == pytest.approx(5 / 14, abs=1e-15)


@pytest.mark.parametrize("n_cliques,m", [(30, 5), (8, 4), (3, 6)])
def test_quality_closed_form_ring_of_cliques(n_cliques, m):
    adj = ring_of_cliques(n_cliques, m)
    L_edges = n_cliques * (m * (m - 1) // 2 + 1)
    per = Fraction(m * (m - 1) // 2, L_edges) - Fraction(m * (m - 1) + 2, 2 * L_edges) ** 2
    labels = [v // m for v in range(n_cliques * m)]
    assert L.modularity(adj, labels) == pytest.approx(float(n_cliques * per), abs=1e-14)
    assert L.modularity(adj, labels) == pytest.approx(float(q_exact(adj, labels)), abs=1e-14)
    # everything in one community: Q = 0; singletons: -sum k^2 / (2m)^2
    assert L.modularity(adj, [0] * len(adj)) == pytest.approx(0.0, abs=1e-15)
    k = [sum(nb.values()) for nb in adj]
    assert L.modularity(adj, list(range(len(adj)))) == pytest.approx(-sum(x * x for x in k) / sum(k) ** 2, abs=1e-15)


def test_quality_resolution_against_definition():
    rng = np.random.default_rng(5)
    adj, lab = sbm(rng, [6, 5, 7], 0.7, 0.1)
    for g in (Fraction(1, 3), Fraction(1), Fraction(5, 2)):
        got = L.modularity(adj, lab.tolist(), g.numerator, g.denominator)
        assert got == pytest.approx(float(q_exact(adj, lab.tolist(), g)), abs=1e-14)


# -- the algorithm against brute force and closed forms ----------------------------

STRUCTURED = {
    "two triangles and a bridge": (6, clique([0, 1, 2]) + clique([3, 4, 5]) + [(2, 3)]),
    "two K4 and a bridge": (8, clique([0, 1, 2, 3]) + clique([4, 5, 6, 7]) + [(3, 4)]),
    "K4, triangle, K2 in a chain": (9, clique([0, 1, 2, 3]) + clique([4, 5, 6]) + [(7, 8), (3, 4), (6, 7)]),
    "star and a disjoint triangle": (8, [(0, i) for i in range(1, 5)] + clique([5, 6, 7])),
    "interleaved triangles": (9, clique([0, 4, 8]) + clique([1, 5, 6]) + clique([2, 3, 7]) + [(8, 1), (6, 2)]),
}


@pytest.mark.parametrize("name", sorted(STRUCTURED))
def test_brute_force_optimum(name):
    n, e = STRUCTURED[name]
    adj = graph(n, e)
    best = max(L.quality_terms(adj, p, 1, 1)[0] for p in partitions(n))
    lab = L.leiden(adj)
    assert L.quality_terms(adj, lab, 1, 1)[0] == best


def test_brute_force_optimum_at_other_resolutions():
    n, e = STRUCTURED["K4, triangle, K2 in a chain"]
    adj = graph(n, e)
    for num, den in ((1, 4), (3, 1)):
        best = max(L.quality_terms(adj, p, num, den)[0] for p in partitions(n))
        assert L.quality_terms(adj, L.leiden(adj, num, den), num, den)[0] == best


def test_resolution_zero_gives_connected_components():
    rnd = random.Random(2)
    for _ in range(150):
        n = rnd.randint(1, 50)
        e = [(a, b) for a in range(n) for b in range(a + 1, n) if rnd.random() < 1.5 / n]
        adj = graph(n, e)
        assert L.leiden(adj, 0, 1) == components(adj)


def test_planted_disjoint_cliques_recovered():
    rng = np.random.default_rng(3)
    sizes = [3, 4, 5, 6, 7, 8, 3, 9]
    n = sum(sizes)
    perm = rng.permutation(n)
    e, owner, at = [], np.empty(n, dtype=np.int64), 0
    for c, s in enumerate(sizes):
        nodes = perm[at:at + s].tolist()
        owner[nodes] = c
        e += clique(nodes)
        at += s
    lab = L.leiden(graph(n, e))
    assert lab == L.first_token_order(owner.tolist())


def test_ring_of_cliques_resolution_limit():
    # 30 five-cliques in a ring: modularity prefers pairs of neighbouring
    # cliques (the resolution limit); at resolution 2 the single cliques win.
    adj = ring_of_cliques(30, 5)
    lab = L.leiden(adj)
    assert max(lab) + 1 == 15
    for c in range(15):
        cl = sorted({v // 5 for v in range(150) if lab[v] == c})
        assert len(cl) == 2 and (cl[1] - cl[0]) % 30 in (1, 29)
        assert all(lab[v] == c for q in cl for v in range(5 * q, 5 * q + 5))
    assert L.leiden(adj, 2, 1) == [v // 5 for v in range(150)]


def test_planted_blocks_recovered():
    rng = np.random.default_rng(11)
    adj, lab = sbm(rng, [20] * 8, 0.6, 0.004)
    assert L.leiden(adj) == L.first_token_order(lab.tolist())


# -- the local moving on its own -------------------------------------------------------

def test_move_nodes_hand_trace():
    # Edges 0-2, 0-3, 0-5, 1-3, 1-4, 2-5, 4-5; degrees 3 2 2 2 2 3, 2m = 14;
    # a value is A(v, C) * 14 - k_v * K_C.  From singletons:
    #  0: {2} and {3} give 8, {5} gives 5: -> 2 (lower id of the tie)
    #  1: {3} and {4} give 10: -> 3
    #  2: stays (8 in {0,2}, {5} also 8); 3: stays (10 against 4)
    #  4: {3} gives 6, {5} gives 8: -> 5, requeues 1
    #  5: {5} keeps 8, {2} gives 2 * 14 - 3 * 5 = 13: -> 2, requeues 4
    #  1: stays (10 against 10); 4, now alone: {2} gives -2, {3} gives 6: -> 3
    #  5: stays (13 against -4)
    adj = graph(6, [(0, 2), (0, 3), (0, 5), (1, 3), (1, 4), (2, 5), (4, 5)])
    k = L.degrees(adj)
    comm = list(range(6))
    L.move_nodes_fast(adj, k, sum(k), comm, [], 1, 1)
    assert comm == [2, 3, 2, 3, 3, 2]


def test_move_nodes_to_an_empty_community():
    # Three nodes with self-loops of 20 in a path (aggregate nodes), all in
    # community 0, ids 1 and 2 unused; degrees 21 22 21, 2m = 64.
    #  0: staying gives 64 - 21 * 43 < 0 and there is no other neighbour
    #     community: -> the lowest empty id, 1
    #  1: staying gives 64 - 22 * 21 = -398, {0} gives the same: -> 2
    #  2 (now alone) and 0 (requeued) stay: every neighbour gives < 0
    adj = [{0: 20, 1: 1}, {1: 20, 0: 1, 2: 1}, {2: 20, 1: 1}]
    k = L.degrees(adj)
    comm = [0, 0, 0]
    L.move_nodes_fast(adj, k, sum(k), comm, [1, 2], 1, 1)
    assert comm == [1, 2, 0]


def test_quality_with_self_loops_against_definition():
    adj = [{0: 4, 1: 1}, {1: 2, 0: 1, 2: 3}, {2: 6, 1: 3, 3: 1}, {3: 0, 2: 1}]
    for lab in ([0, 0, 1, 1], [0, 1, 1, 2], [0, 0, 0, 0]):
        for g in (Fraction(1), Fraction(2, 3)):
            got = L.modularity(adj, lab, g.numerator, g.denominator)
            assert got == pytest.approx(float(q_exact(adj, lab, g)), abs=1e-14)


# -- the refinement and the aggregation on their own --------------------------------

def test_refine_splits_what_is_not_connected():
    # One community holding two disjoint triangles; 2m = 12, K_S = 12.
    # Node 0 (inside weight 2 >= 2 * 10 / 12) joins node 2 (gain 1 * 12 -
    # 2 * 2 = 8, the lower of two equal candidates), node 1 joins node 3.
    # Node 4 would gain joining {0, 2}, but that pair is not well-connected
    # to the rest of S (2 < 4 * 8 / 12), so it stays alone; so does 5.
    adj = graph(6, clique([0, 2, 4]) + clique([1, 3, 5]))
    k = L.degrees(adj)
    ref = L.refine(adj, k, sum(k), [0] * 6, 1, 1)
    assert ref == [2, 3, 2, 3, 4, 5]
    # never a refined community across the two triangles, whatever the order
    for comm in ([0] * 6, [1, 0, 1, 0, 1, 0]):
        ref = L.refine(adj, k, sum(k), comm, 1, 1)
        assert all((ref[u] == ref[v]) <= (u % 2 == v % 2) for u in range(6) for v in range(6))


def test_refine_hand_example():
    # One community holding two K4s, {0,2,4,6} and {1,3,5,7}, joined by the
    # edge 6-1: degrees 3 (4 for nodes 1 and 6), 2m = K_S = 26.
    #  node 0 -> {2} (gain 26 - 3*3 = 17; {4} ties, {6} gives 14); {0,2}: K 6, ext 4
    #  node 1 -> {3} (26 - 4*3 = 14, lowest of 3, 5, 7; {6} gives 10); {1,3}: K 7, ext 5
    #  node 4: {0,2} is not well-connected (4 * 26 < 6 * 20), so -> {6} (14)
    #  node 5: {1,3} is not well-connected (5 * 26 < 7 * 19), so -> {7} (17)
    #  nodes 2, 3, 6, 7 are no longer alone.
    a, b = [0, 2, 4, 6], [1, 3, 5, 7]
    adj = graph(8, clique(a) + clique(b) + [(6, 1)])
    k = L.degrees(adj)
    ref = L.refine(adj, k, sum(k), [0] * 8, 1, 1)
    assert ref == [2, 3, 2, 3, 6, 7, 6, 7]
    # inside two separate communities nothing crosses over
    ref2 = L.refine(adj, k, sum(k), [0, 1, 0, 1, 0, 1, 0, 1], 1, 1)
    assert L.first_token_order(ref2) == [0, 1, 0, 1, 0, 1, 0, 1]


def test_refine_skips_a_node_not_well_connected():
    # Path 0-1-2-3 in community 0, leaves 4 and 5 on node 0 in community 1;
    # degrees 3 2 2 1 1 1, 2m = 10, K_S = 8.
    #  0: inside weight 1, 1 * 10 < 3 * 5: not well-connected, stays alone
    #  1: {0} is not well-connected (1 * 10 < 3 * 5); {2}: gain 10 - 4 = 6 -> 2
    #  2: no longer alone; 3: {1,2} (ext 2, K 4: 20 >= 16) gains 6 -> 2
    #  4, 5: no weight inside their community, not well-connected
    adj = graph(6, [(0, 1), (1, 2), (2, 3), (0, 4), (0, 5)])
    k = L.degrees(adj)
    assert L.refine(adj, k, sum(k), [0, 0, 0, 0, 1, 1], 1, 1) == [0, 2, 2, 2, 4, 5]


def test_aggregate_hand_example():
    adj = graph(5, [(0, 1), (1, 2), (2, 3), (3, 4), (0, 4), (1, 3)])
    ref = [3, 3, 2, 3, 4]          # refined communities {0,1,3}, {2}, {4}
    comm = [7, 7, 7, 7, 9]
    new, start, node_map = L.aggregate(adj, ref, comm)
    # aggregate nodes in refined-id order: 2 -> {2}, 3 -> {0,1,3}, 4 -> {4}
    assert node_map == [1, 1, 0, 1, 2]
    assert new == [{1: 2}, {1: 4, 0: 2, 2: 2}, {1: 2}]
    assert start == [0, 0, 1]
    assert sum(L.degrees(new)) == sum(L.degrees(adj))


# -- what the Leiden paper guarantees after every iteration ---------------------------

def _check_guarantees(adj, lab, gnum=1, gden=1):
    k = L.degrees(adj)
    two_m = sum(k)
    comms = {}
    for v, c in enumerate(lab):
        comms.setdefault(c, []).append(v)
    assert sorted(comms) == list(range(len(comms)))
    for c, mem in comms.items():
        sub = set(mem)
        seen, todo = {mem[0]}, [mem[0]]
        while todo:
            v = todo.pop()
            for u in adj[v]:
                if u in sub and u not in seen:
                    seen.add(u)
                    todo.append(u)
        assert seen == sub, f"community {c} is not connected"
    K = {c: sum(k[v] for v in mem) for c, mem in comms.items()}
    between = {}
    for v, nb in enumerate(adj):
        for u, wt in nb.items():
            if lab[u] != lab[v]:
                key = (min(lab[u], lab[v]), max(lab[u], lab[v]))
                between[key] = between.get(key, 0) + wt
    for (c, d), w2 in between.items():   # w2 counts each edge from both ends
        assert w2 * two_m * gden <= 2 * gnum * K[c] * K[d], f"merging {c} and {d} would gain"


def test_guarantees_on_random_graphs():
    rng = np.random.default_rng(7)
    for t in range(12):
        sizes = rng.integers(3, 25, rng.integers(2, 9)).tolist()
        adj, _ = sbm(rng, sizes, 0.3 + 0.05 * t, 0.03)
        for gnum, gden in ((1, 1), (1, 2), (3, 1)):
            _check_guarantees(adj, L.leiden(adj, gnum, gden), gnum, gden)


def test_guarantees_on_token_graphs():
    rng = np.random.default_rng(8)
    rows = token_rows(rng, 1200, 4, 8, 60)
    lab, nc = L.partition_tokens(rows, 1200, 4)
    assert (lab[:4] == -1).all() and nc == lab.max() + 1
    _check_guarantees(L.token_graph(rows, 1200, 4), lab[4:].tolist())


def test_no_edges_and_degenerate_graphs():
    assert L.leiden([]) == []
    assert L.leiden([{}, {}, {}]) == [0, 1, 2]
    adj = graph(4, [(1, 2)])
    assert L.leiden(adj) == [0, 1, 1, 2]
    lab, nc = L.partition_tokens(np.full((4, 2), -1), 4, 4)
    assert lab.tolist() == [-1] * 4 and nc == 0


# -- tokens decoded during a partition: joined by the vote of their edges ---------------

def test_extend_by_vote_hand_example():
    # tokens 0-1 sinks, 2-5 partitioned as [0, -, 1, 1] (token 3 in no
    # community, as a full tail leaves a token); then
    #  6 -> 2, 4, 5: communities 0, 1, 1 -> 1
    #  7 -> 2, 4: one vote each -> 0 (lower id)
    #  8 -> 6, 7, 3: communities 1, 0 and none: one vote each -> 0
    #  9 -> no edges -> a new community 2; 10 -> 9, 9 -> 2
    rows = np.full((11, 3), -1)
    rows[6] = [2, 4, 5]
    rows[7, :2] = [2, 4]
    rows[8] = [6, 7, 3]
    rows[10, :2] = [9, 9]
    lab = np.array([-1, -1, 0, -1, 1, 1] + [-1] * 5)
    out, nc = L.extend_by_vote(lab, 2, rows, 6, 11)
    assert out.tolist() == [-1, -1, 0, -1, 1, 1, 1, 0, 0, 2, 2] and nc == 3
    assert lab[6] == -1  # the input is not changed


def test_extend_by_vote_matches_partition_of_isolated_growth():
    # a new token whose edges all point into one community joins it, so
    # extending a partition by tokens linked to one clique each keeps the
    # cliques (checked against the Leiden result of the whole graph)
    rows = np.full((40, 4), -1)
    for c in range(4):                      # four 8-cliques over tokens 4..35
        mem = [4 + c + 4 * i for i in range(8)]
        for a in range(1, 8):
            rows[mem[a], :min(a, 4)] = mem[max(0, a - 4):a][::-1][:4]
    for t in range(36, 40):                 # four late tokens, one per clique
        rows[t, :3] = [4 + (t - 36) + 4 * i for i in (0, 3, 5)]
    full, nc_full = L.partition_tokens(rows, 40, 4)
    part, nc = L.partition_tokens(rows[:36], 36, 4)
    lab = np.concatenate([part, np.full(4, -1)])
    ext, nc2 = L.extend_by_vote(lab, nc, rows, 36, 40)
    assert nc2 == nc and np.array_equal(ext, full)
