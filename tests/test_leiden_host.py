"""The library's host Leiden (ckv_leiden_partition, ckv_partition_quality)
against the oracle on the same edge tables: labels bit-identical, community
counts equal, modularity within rounding.  Host calls only: no GPU.
"""
import numpy as np
import pytest

from community_kv_retrieval_amd import ckv
from oracle import leiden_oracle as L


def prefill_like_rows(rng, n, n_sinks, kappa, n_topics, p_other=0.5):
    """Rows shaped like a prefill graph: each token's edges go to earlier
    tokens of its own topic and, now and then, to a random earlier token."""
    topic = rng.integers(0, n_topics, n)
    rows = np.full((n, kappa), -1, dtype=np.int32)
    last = {}
    for i in range(n_sinks, n):
        same = last.get(topic[i], [])[-(kappa - 1):] if kappa > 1 else []
        other = [int(rng.integers(n_sinks, i))] if i > n_sinks and rng.random() < p_other else []
        c = list(dict.fromkeys(same + other))[:kappa]
        rows[i, :len(c)] = c
        last.setdefault(topic[i], []).append(i)
    return rows


def random_rows(rng, n, n_sinks, kappa, density):
    rows = np.full((n, kappa), -1, dtype=np.int32)
    for i in range(n_sinks + 1, n):
        m = min(kappa, i - n_sinks, int(rng.binomial(kappa, density)))
        if m:
            rows[i, :m] = rng.choice(np.arange(n_sinks, i), size=m, replace=False)
    return rows


def _pack(tables, stride):
    G = len(tables)
    kappa = tables[0].shape[1]
    e = np.full((G, stride, kappa), -1, dtype=np.int32)
    n = np.zeros(G, dtype=np.int32)
    for g, t in enumerate(tables):
        e[g, :t.shape[0]] = t
        n[g] = t.shape[0]
    return n, e


CASES = [
    # (seed, n, sinks, kappa, kind, gamma)
    (1, 600, 4, 8, "prefill", (1, 1)),
    (2, 1500, 4, 8, "prefill", (1, 1)),
    (3, 2500, 4, 8, "prefill", (3, 2)),
    (4, 900, 4, 4, "random", (1, 1)),
    (5, 900, 0, 3, "random", (1, 3)),
    (6, 700, 4, 1, "random", (1, 1)),
    (7, 1200, 4, 16, "prefill", (2, 1)),
    (8, 500, 2, 32, "random", (1, 1)),
    (9, 400, 4, 8, "random", (0, 1)),
    (10, 3000, 4, 8, "prefill", (1, 4)),
]


@pytest.mark.parametrize("seed,n,sinks,kappa,kind,gamma", CASES)
def test_host_leiden_matches_oracle(seed, n, sinks, kappa, kind, gamma):
    rng = np.random.default_rng(seed)
    tables = []
    for g in range(3):    # graphs of different lengths in one call
        m = n - 97 * g
        tables.append(prefill_like_rows(rng, m, sinks, kappa, max(2, m // 20)) if kind == "prefill"
                      else random_rows(rng, m, sinks, kappa, 0.6))
    n_tok, edges = _pack(tables, n + 5)
    labels, n_comm, q = ckv.ckv_leiden_partition(n_tok, sinks, edges, gamma, n_threads=3)
    for g, t in enumerate(tables):
        ref, nc = L.partition_tokens(t, t.shape[0], sinks, *gamma)
        assert n_comm[g] == nc
        assert np.array_equal(labels[g, :t.shape[0]], ref.astype(np.int32))
        assert (labels[g, t.shape[0]:] == -1).all()
        adj = L.token_graph(t, t.shape[0], sinks)
        assert q[g] == pytest.approx(L.modularity(adj, ref[sinks:].tolist(), *gamma), abs=1e-12)


def test_host_quality_of_given_labels():
    rng = np.random.default_rng(21)
    t = prefill_like_rows(rng, 800, 4, 8, 40)
    n_tok, edges = _pack([t, t], 800)
    lab = np.full((2, 800), -1, dtype=np.int32)
    lab[0, 4:] = rng.integers(0, 30, 796)
    lab[1, 4:] = np.arange(796) // 7
    q = ckv.ckv_partition_quality(n_tok, 4, edges, lab, (1, 1))
    adj = L.token_graph(t, 800, 4)
    for g in range(2):
        assert q[g] == pytest.approx(L.modularity(adj, lab[g, 4:].tolist()), abs=1e-12)
    q2 = ckv.ckv_partition_quality(n_tok, 4, edges, lab, (5, 2))
    assert q2[1] == pytest.approx(L.modularity(adj, lab[1, 4:].tolist(), 5, 2), abs=1e-12)


def test_host_leiden_degenerate_graphs():
    e = np.full((4, 10, 2), -1, dtype=np.int32)
    n_tok = np.array([0, 3, 6, 10], dtype=np.int32)     # empty, all sinks, no edges, one edge
    e[3, 7] = [5, -1]
    labels, n_comm, q = ckv.ckv_leiden_partition(n_tok, 4, e)
    assert (labels[0] == -1).all() and n_comm[0] == 0
    assert (labels[1] == -1).all() and n_comm[1] == 0
    assert labels[2].tolist() == [-1] * 4 + [0, 1] + [-1] * 4 and n_comm[2] == 2 and q[2] == 0.0
    assert labels[3].tolist() == [-1] * 4 + [0, 1, 2, 1, 3, 4] and n_comm[3] == 5


@pytest.mark.parametrize("bad", ["sink", "self", "future", "kappa", "gamma", "n_tokens"])
def test_host_leiden_rejects_bad_input(bad):
    e = np.full((1, 8, 2), -1, dtype=np.int32)
    n_tok = np.array([8], dtype=np.int32)
    gamma = (1, 1)
    if bad == "sink":
        e[0, 6, 0] = 1
    elif bad == "self":
        e[0, 6, 0] = 6
    elif bad == "future":
        e[0, 6, 0] = 9
    elif bad == "kappa":
        e = np.full((1, 8, 33), -1, dtype=np.int32)
    elif bad == "gamma":
        gamma = (1, 0)
    elif bad == "n_tokens":
        n_tok = np.array([9], dtype=np.int32)
    with pytest.raises(ckv.CkvError) as ei:
        ckv.ckv_leiden_partition(n_tok, 4, e, gamma)
    assert ei.value.code == ckv.CKV_E_INVALID


def test_host_extend_partition_matches_oracle():
    rng = np.random.default_rng(31)
    tables, firsts, ref = [], [], []
    for g in range(3):
        n = 700 + 50 * g
        t = prefill_like_rows(rng, n, 4, 8, 30)
        first = 500 + 20 * g
        lab, nc = L.partition_tokens(t[:first], first, 4)
        lab = np.concatenate([lab, np.full(n - first, -1)])
        if g == 1:
            lab[10] = -1            # a token without a community: its edges do not vote
        if g == 2:
            t[first + 3] = -1       # a token without edges starts a community
        want, nc2 = L.extend_by_vote(lab, nc, t, first, n)
        tables.append(t)
        firsts.append(first)
        ref.append((lab, nc, want, nc2))
    n_tok, edges = _pack(tables, 900)
    labels = np.full((3, 900), -1, dtype=np.int32)
    n_comm = np.zeros(3, dtype=np.int32)
    for g, (lab, nc, _, _) in enumerate(ref):
        labels[g, :lab.size] = lab
        n_comm[g] = nc
    ckv.ckv_extend_partition(np.array(firsts, dtype=np.int32), n_tok, edges, labels, n_comm)
    for g, (_, _, want, nc2) in enumerate(ref):
        assert np.array_equal(labels[g, :want.size], want.astype(np.int32))
        assert n_comm[g] == nc2
    bad = edges.copy()
    bad[0, 600, 0] = 650           # an edge to a later token
    with pytest.raises(ckv.CkvError):
        ckv.ckv_extend_partition(np.array(firsts, dtype=np.int32), n_tok, bad, labels.copy(), n_comm.copy())


@pytest.mark.parametrize("gamma", [(1, 1), (512, 1)])
def test_host_leiden_full_size_prompt_graph(gamma):
    """A graph of the benchmark's prompt length (131 072 tokens, kappa 8,
    communities of about 16 planted tokens plus stray edges): the library's
    labels equal the oracle's at the resolution of the prefill timing (1) and
    of the refresh leg (512); several aggregation levels run at this size."""
    rng = np.random.default_rng(2026)
    n = 131072
    rows = prefill_like_rows(rng, n, 4, 8, n // 16, p_other=0.3)
    ref, nc = L.partition_tokens(rows, n, 4, *gamma)
    labels, n_comm, _ = ckv.ckv_leiden_partition(np.array([n], dtype=np.int32), 4, rows[None].copy(), gamma, 4)
    assert n_comm[0] == nc and np.array_equal(labels[0], ref.astype(np.int32))


def test_host_leiden_resolution_extremes_and_overflow_guard():
    rng = np.random.default_rng(41)
    t = prefill_like_rows(rng, 600, 4, 8, 30)
    n_tok, edges = _pack([t], 600)
    # a resolution far above every gain: no merge pays, every token alone
    labels, n_comm, _ = ckv.ckv_leiden_partition(n_tok, 4, edges, (10 ** 6, 1))
    assert n_comm[0] == 596 and labels[0, 4:].tolist() == list(range(596))
    ref, nc = L.partition_tokens(t, 600, 4, 10 ** 6, 1)
    assert nc == 596
    # resolution 0: the connected components
    labels0, n0, _ = ckv.ckv_leiden_partition(n_tok, 4, edges, (0, 1))
    ref0, nc0 = L.partition_tokens(t, 600, 4, 0, 1)
    assert n0[0] == nc0 and np.array_equal(labels0[0], ref0.astype(np.int32))
    # products that could leave int64 are refused: (2m)^2 * 4 * max(num, den) >= 2^62
    with pytest.raises(ckv.CkvError) as ei:
        ckv.ckv_leiden_partition(n_tok, 4, edges, (1 << 44, 1))
    assert ei.value.code == ckv.CKV_E_INVALID
