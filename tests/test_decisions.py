"""The GPU parity checker's acceptance rules for selections and edges
(tests/decisions.py), fed planted device results on the CPU: every genuine
mistake (a community dropped or added at the cut, a walk that stops early or
runs over the budget, an edge too few, edges out of rank order, a sink or a
duplicate as an edge) must be rejected, and every decision that a
tie-consistent ranking yields must be accepted."""
import numpy as np
import pytest

from oracle import ckv_oracle as O
from tests import decisions as D


def _sel(scores, counts, budget, max_comm=0):
    s = np.asarray(scores, dtype=np.float32)
    c = np.asarray(counts, dtype=np.int64)
    return s, c, O.select_communities(s, c, budget, max_comm)


# --- selection -------------------------------------------------------------

def test_identical_selection_passes():
    s, c, so = _sel([5, 4, 3, 2, 1], [10] * 5, 35)
    assert so.tolist() == [0, 1, 2]
    assert D.selection_ok(s, c, so, [2, 0, 1], 35) is True


@pytest.mark.parametrize("dev", [
    [0, 1],            # the last community of the prefix dropped
    [0, 1, 3],         # the cut community replaced by a worse one
    [0, 1, 2, 3],      # one past the budget
    [0, 1, 2, 2],      # duplicate
    [1, 2, 3],         # the best community missing
    [0, 1, 2, 7],      # an id past the communities
])
def test_selection_mistakes_rejected(dev):
    s, c, so = _sel([5, 4, 3, 2, 1], [10] * 5, 35)
    with pytest.raises(AssertionError):
        D.selection_ok(s, c, so, dev, 35)


def test_selection_dropping_last_rejected_with_ties_elsewhere():
    """Near-ties away from the cut do not excuse a dropped last community."""
    s, c, so = _sel([5, 5 - 4e-7, 3, 2, 1], [10] * 5, 35)
    assert so.tolist() == [0, 1, 2]
    with pytest.raises(AssertionError):
        D.selection_ok(s, c, so, [0, 1], 35)
    assert D.selection_ok(s, c, so, [0, 1, 2], 35) is True


def test_selection_empty_community_rejected():
    s, c, so = _sel([5, 4, -np.inf, 2], [10, 10, 0, 10], 35)
    with pytest.raises(AssertionError):
        D.selection_ok(s, c, so, [0, 1, 2], 35)


def test_selection_cap_respected():
    s, c, so = _sel([5, 4, 3, 2, 1], [1] * 5, 100, max_comm=2)
    assert so.tolist() == [0, 1]
    with pytest.raises(AssertionError):
        D.selection_ok(s, c, so, [0, 1, 2], 100, max_comm=2)
    with pytest.raises(AssertionError):  # stops before the cap with room left
        D.selection_ok(s, c, so, [0], 100, max_comm=2)


def test_selection_tie_at_cut_accepted_either_way():
    """Two communities 5e-7 apart at the cut, the better one too large to fit
    after the first two: the oracle stops before it; a device that ranked the
    (tied) smaller one first takes it and stops at the larger."""
    s, c, so = _sel([5, 4, 3, 3 + 5e-7, 1], [10, 10, 10, 20, 10], 35)
    assert so.tolist() == [0, 1]
    gaps = []
    assert D.selection_ok(s, c, so, [0, 1, 2], 35, gaps=gaps) is False
    assert gaps and gaps[0] <= D.TIE


def test_selection_tie_dropping_last_accepted_when_tied_next_overflows():
    """The oracle takes the last fitting community; a device ranking a tied,
    larger community first stops before it: a valid budget prefix."""
    s, c, so = _sel([5, 4, 3, 3 - 5e-7], [10, 10, 10, 20], 35)
    assert so.tolist() == [0, 1, 2]
    assert D.selection_ok(s, c, so, [0, 1], 35) is False


def test_selection_swap_beyond_tie_rejected():
    s, c, so = _sel([5, 4, 3, 3 + 5e-6, 1], [10, 10, 10, 20, 10], 35)
    with pytest.raises(AssertionError):
        D.selection_ok(s, c, so, [0, 1, 2], 35)


def test_selection_exact_ties_any_valid_prefix():
    """Every score equal: any set that fills the budget walk of some order of
    the ids and stops at a community that does not fit is valid."""
    s = np.zeros(6, dtype=np.float32)
    c = np.array([3, 5, 2, 4, 1, 6])
    so = O.select_communities(s, c, 10)
    assert so.tolist() == [0, 1, 2]
    assert D.selection_ok(s, c, so, [1, 3, 4], 10) is False  # 5 + 4 + 1, every outsider overflows
    assert D.selection_ok(s, c, so, [0, 2], 10) is False     # 5 tokens, then community 5 (size 6) overflows
    with pytest.raises(AssertionError):
        D.selection_ok(s, c, so, [3, 4, 5], 10)             # 11 tokens: over the budget
    with pytest.raises(AssertionError):
        D.selection_ok(s, c, so, [0], 10)                   # 3 tokens, and every outsider would still fit


# --- edges -----------------------------------------------------------------

POS = np.array([0, 1, 2, 3, 10, 11, 12, 13, 14])
WTS = np.array([0.3, 0.2, 0.1, 0.05, 0.11, 0.09, 0.07, 0.05, 0.03])


def test_identical_edges_pass():
    eo = O.top_kappa(WTS, POS, 3, 4)
    assert eo.tolist() == [10, 11, 12]
    assert D.edges_ok(POS, WTS, 4, 3, eo, [10, 11, 12]) is True


@pytest.mark.parametrize("dev", [
    [10, 11],            # kappa - 1 edges
    [11, 10, 12],        # out of rank order
    [10, 12, 11],        # out of rank order at the end
    [10, 11, 13],        # third replaced by a lighter one
    [0, 10, 11],         # a sink as an edge
    [10, 10, 11],        # duplicate
    [10, 11, 12, 13],    # kappa + 1
    [10, 11, 99],        # a token that was not attended
])
def test_edge_mistakes_rejected(dev):
    eo = O.top_kappa(WTS, POS, 3, 4)
    with pytest.raises(AssertionError):
        D.edges_ok(POS, WTS, 4, 3, eo, dev)


def test_fewer_candidates_than_kappa_needs_all():
    pos = np.array([0, 1, 2, 3, 10, 11])
    w = np.array([0.5, 0.2, 0.1, 0.1, 0.06, 0.04])
    eo = O.top_kappa(w, pos, 8, 4)
    assert eo.tolist() == [10, 11]
    assert D.edges_ok(pos, w, 4, 8, eo, [10, 11]) is True
    with pytest.raises(AssertionError):
        D.edges_ok(pos, w, 4, 8, eo, [10])


def test_edge_tie_swaps_accepted():
    w = WTS.copy()
    w[6] = w[5] + 4e-7  # 12 and 11 within the tie window
    eo = O.top_kappa(w, POS, 3, 4)
    assert eo.tolist() == [10, 12, 11]
    assert D.edges_ok(POS, w, 4, 3, eo, [10, 11, 12]) is False
    w2 = WTS.copy()
    w2[7] = w2[6] - 4e-7  # 13 ties 12 at the cut
    eo2 = O.top_kappa(w2, POS, 3, 4)
    assert D.edges_ok(POS, w2, 4, 3, eo2, [10, 11, 13]) is False


def test_edge_order_chain_of_small_ties_rejected():
    """Each neighbour within the window, the ends not: rank order is checked on
    every pair, not only neighbours."""
    pos = np.array([0, 10, 11, 12])
    w = np.array([0.5, 1.0, 1.0 + 0.9e-6, 1.0 + 1.8e-6])
    eo = O.top_kappa(w, pos, 3, 1)
    assert eo.tolist() == [12, 11, 10]
    with pytest.raises(AssertionError):
        D.edges_ok(pos, w, 1, 3, eo, [10, 11, 12])


# --- planted mistakes on real oracle steps -----------------------------------

def _oracle_steps(mode, budget, seed=5, steps=8):
    from community_kv_retrieval_amd import synth
    w = synth.preset("qwen3_8b_32k").replace(name="decisions", n_ctx=3000, n_q_heads=4, n_kv_heads=1,
                                               budget=budget, mode=mode)
    sl = synth.gen_layer(w, seed)
    kv = [[(s.k.float().numpy(), s.v.float().numpy()) for s in row] for row in sl]
    orc = O.Oracle(w, kv, dict(enumerate(synth.graph_labels(w, sl))), dict(enumerate(synth.graph_n_comm(w, sl))),
                   extra=steps + 1)
    res = []
    for t in range(steps):
        inp = synth.gen_step(w, seed, t, sl)
        before = {g: st.counts.copy() for g, st in orc.g.items()}  # the step's own update grows one
        out = orc.step(inp.q.float().numpy(), inp.k_new.float().numpy(), inp.v_new.float().numpy())
        res += [(w, before[g], r) for g, r in out.items()]
    return res


@pytest.mark.parametrize("mode", ["per_head", "group"])
def test_off_by_one_on_oracle_steps_rejected(mode):
    """On seeded 3000-token graphs (budget 256, kappa 8), a device result that
    drops the last selected community, adds the next one, drops the last edge,
    or swaps the first two edges is rejected; the oracle's own is accepted."""
    checked = 0
    for w, counts, r in _oracle_steps(mode, 256):
        assert D.selection_ok(r.scores, counts, r.selected, r.selected, w.budget) is True
        assert D.edges_ok(r.positions, r.weights, w.n_sinks, w.kappa, r.edges, r.edges) is True
        ranked = O.rank_communities(r.scores, counts)
        k = r.selected.size
        assert k >= 2 and ranked[k - 1] in r.selected
        with pytest.raises(AssertionError):
            D.selection_ok(r.scores, counts, r.selected, [c for c in r.selected if c != ranked[k - 1]], w.budget)
        with pytest.raises(AssertionError):
            D.selection_ok(r.scores, counts, r.selected, list(r.selected) + [int(ranked[k])], w.budget)
        e = [int(x) for x in r.edges]
        assert len(e) == w.kappa
        with pytest.raises(AssertionError):
            D.edges_ok(r.positions, r.weights, w.n_sinks, w.kappa, r.edges, e[:-1])
        with pytest.raises(AssertionError):
            D.edges_ok(r.positions, r.weights, w.n_sinks, w.kappa, r.edges, [e[1], e[0]] + e[2:])
        checked += 1
    assert checked >= 8


# --- prefill rows --------------------------------------------------------------

def _prefill_case():
    rng = np.random.default_rng(3)
    n, d, sinks, kappa = 40, 16, 4, 5
    keys = rng.standard_normal((n, d))
    q = rng.standard_normal((n, 2, d))
    e, wts = O.prefill_edges(q, keys, sinks, kappa, 0.5)
    return q, keys, sinks, kappa, e, wts


def test_prefill_rows_identical_and_mistakes():
    q, keys, sinks, kappa, e, wts = _prefill_case()
    for i in (4, 5, 7, 20, 39):
        W = O.prefill_row_weights(q[i], i, keys, 0.5)
        row, wrow = e[i], wts[i]
        k = int((row >= 0).sum())
        assert k == min(kappa, i - sinks)
        assert D.prefill_row_ok(W, i, sinks, kappa, row, row, wrow.astype(np.float32)) is True
        if k == 0:
            with pytest.raises(AssertionError):
                D.prefill_row_ok(W, i, sinks, kappa, row, np.r_[[sinks], -np.ones(kappa - 1, int)], None)
            continue
        bad = []
        bad.append(np.r_[row[:k - 1], -np.ones(kappa - k + 1, int)])        # an edge too few
        bad.append(np.r_[row[:k - 1], [i], -np.ones(kappa - k, int)])       # the token itself
        bad.append(np.r_[row[:k - 1], [0], -np.ones(kappa - k, int)])       # a sink
        if k >= 2:
            sw = row.copy()
            sw[0], sw[1] = sw[1], sw[0]
            bad.append(sw)                                                  # out of rank order
        for b in bad:
            with pytest.raises(AssertionError):
                D.prefill_row_ok(W, i, sinks, kappa, row, b, None)
        wbad = wrow.astype(np.float32).copy()
        wbad[0] *= 1.01
        with pytest.raises(AssertionError):
            D.prefill_row_ok(W, i, sinks, kappa, row, row, wbad)


def test_prefill_pair_window_is_relative_to_the_pair():
    """A swap of two heavy edges 6e-7 apart relatively is a tie; the same
    absolute gap between light edges is not (window relative to the pair)."""
    pos = np.arange(10)
    w = np.array([0.3, 0.2, 0.1, 0.05, 0.0239383, 0.0239382, 0.0100, 2e-5, 1e-5, 1e-5 * (1 - 1e-4)])
    W = np.r_[w, 0.0]  # weight of the query's own position (never a candidate)
    orow = np.array([4, 5, 6, 7])
    i = 10
    assert D.prefill_row_ok(W, i, 4, 4, orow, orow, None) is True
    assert D.prefill_row_ok(W, i, 4, 4, orow, np.array([5, 4, 6, 7]), None) is False
    six = np.array([4, 5, 6, 7, 8, 9])
    assert D.prefill_row_ok(W, i, 4, 6, six, np.array([4, 5, 6, 7, 9, 8]), None) is False  # 1e-9 of 1e-5
    with pytest.raises(AssertionError):
        D.prefill_row_ok(W, i, 4, 6, six, np.array([4, 5, 6, 8, 7, 9]), None)  # 1e-5 of 2e-5


# --- centroid budget ---------------------------------------------------------

def _cent(scores, counts, sel, n):
    s = np.asarray(scores, dtype=np.float32)
    c = np.asarray(counts, dtype=np.int64)
    return s, c, O.centroid_communities(s, c, np.asarray(sel, dtype=np.int64), n)


def test_identical_centroids_pass():
    s, c, co = _cent([5, 4, 3, 2, 1], [1] * 5, [0, 1], 2)
    assert co.tolist() == [2, 3]
    assert D.centroids_ok(s, c, [0, 1], co, [3, 2], 2) is True


@pytest.mark.parametrize("dev", [
    [2],           # one too few
    [2, 3, 4],     # one too many
    [2, 4],        # the second replaced by a worse one
    [1, 2],        # a selected community
    [2, 2],        # duplicate
    [2, 9],        # out of range
    [3, 4],        # the walk's stopper left out
])
def test_centroid_mistakes_rejected(dev):
    s, c, co = _cent([5, 4, 3, 2, 1], [1] * 5, [0, 1], 2)
    with pytest.raises(AssertionError):
        D.centroids_ok(s, c, [0, 1], co, dev, 2)


def test_centroid_near_tie_accepted_and_empty_rejected():
    s, c, co = _cent([5, 4, 3, 2 - 4e-7, 2, -np.inf], [1, 1, 1, 1, 1, 0], [0, 1], 2)
    assert co.tolist() == [2, 4]
    assert D.centroids_ok(s, c, [0, 1], co, [2, 3], 2) is False
    with pytest.raises(AssertionError):
        D.centroids_ok(s, c, [0, 1], co, [2, 5], 2)


def test_centroid_all_left_taken_when_short():
    s, c, co = _cent([5, 4, 3], [1, 1, 1], [0], 8)
    assert co.tolist() == [1, 2]
    assert D.centroids_ok(s, c, [0], co, [1, 2], 8) is True
    with pytest.raises(AssertionError):
        D.centroids_ok(s, c, [0], co, [1], 8)
