"""Acceptance rules for the two integer decisions of a decode step that rest
on floating point: which communities are retrieved, and which attended tokens
become the new token's edges.

The oracle decides both in float64; the device decides the selection on the
same exact float32 scores and the edges on float32 attention weights.  A
device decision that differs from the oracle's is accepted only when it is
the decision of *some* ranking that differs from the oracle's by swaps of
items whose oracle values lie within TIE of each other ("tie-consistent":
an item may precede another only if its value is at least the other's minus
TIE).  Such a ranking exists for the given device decision exactly when the
conditions checked below hold; anything else (a dropped or extra community,
an edge too few, an edge out of rank order) is an error.

Imports only numpy, so the CPU tests can plant device results here.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np

TIE = 1e-6


def selection_ok(scores: np.ndarray, counts: np.ndarray, oracle_sel: Sequence[int], dev_sel: Sequence[int],
                 budget: int, max_comm: int = 0, where: str = "", gaps: Optional[List[float]] = None) -> bool:
    """True when the device's selection equals the oracle's; False when it
    differs but is the budget walk of a tie-consistent ranking (the caller
    then adopts it); AssertionError otherwise.

    The budget walk (Figure 1 panel (3) with the token budget of Tables 2-3,
    read as: take communities best first while the running member count stays
    within the budget, stop at the first that does not fit; optionally at most
    max_comm of them) yields the device set S from a ranking pi exactly when
      1. S fits: sum of sizes <= budget (and |S| <= max_comm when capped);
      2. S is a prefix of pi: every member of S may precede every non-empty
         community outside S (score >= outside score - TIE);
      3. the walk stops right after S: every non-empty community is in S, or
         the cap is reached, or some community c outside S that may come first
         among the outsiders (score >= best outside score - TIE) does not fit
         (sum of sizes of S + size[c] > budget).
    scores: the oracle's exact float32 scores (-inf for empty communities).
    """
    so = sorted(int(c) for c in oracle_sel)
    sg = [int(c) for c in dev_sel]
    assert len(set(sg)) == len(sg), f"{where}: duplicate community in the device selection {sg}"
    sg = sorted(sg)
    if so == sg:
        return True
    counts = np.asarray(counts)
    C = counts.size
    s = np.asarray(scores, dtype=np.float64)[:C]
    live = counts > 0
    for c in sg:
        assert 0 <= c < C and live[c], f"{where}: device selected community {c}, empty or out of range"
    inside = np.zeros(C, dtype=bool)
    inside[sg] = True
    total = int(counts[sg].sum())
    assert total <= budget, f"{where}: device selection holds {total} tokens, budget {budget}"
    if max_comm > 0:
        assert len(sg) <= max_comm, f"{where}: device selection holds {len(sg)} communities, cap {max_comm}"
    outside = np.nonzero(live & ~inside)[0]
    if outside.size == 0:
        best_out = -np.inf
    else:
        best_out = float(s[outside].max())
        worst_in = float(s[sg].min()) if sg else np.inf
        inversion = best_out - worst_in
        assert inversion <= TIE, (f"{where}: device selection is not a prefix of any tie-consistent ranking "
                                  f"(community {int(outside[np.argmax(s[outside])])} scores {inversion:.3g} above "
                                  f"selected community {sg[int(np.argmin(s[sg]))]})")
        if gaps is not None:
            gaps.append(max(inversion, 0.0))
    capped = max_comm > 0 and len(sg) == max_comm
    if outside.size and not capped:
        first = outside[s[outside] >= best_out - TIE]
        stops = first[total + counts[first] > budget]
        assert stops.size > 0, (f"{where}: device selection stops early: community "
                                f"{int(first[0])} (size {int(counts[first[0]])}) would still fit "
                                f"({total} of {budget} tokens taken)")
    return False


def edges_ok(positions: np.ndarray, weights: np.ndarray, n_sinks: int, kappa: int, oracle_edges: Sequence[int],
             dev_edges: Sequence[int], where: str = "", gaps: Optional[List[float]] = None,
             tie: float = TIE, rel: float = 0.0) -> bool:
    """True when the device's edges equal the oracle's, in rank order; False
    when they differ but are the first kappa of a tie-consistent ranking of the
    pool (the caller then adopts them); AssertionError otherwise.

    The pool is the attended non-sink tokens (Table 6: sinks excluded), ranked
    by weight, higher first.  The device must return exactly min(kappa, |pool|)
    distinct pool tokens, in an order where each may precede the next
    (weight >= next weight - window), each of weight >= every unchosen pool
    token's weight - window.
    positions: the attended positions (sinks included); weights: the oracle's
    float64 graph weight of each.  Two weights a, b count as tied when they
    differ by at most tie + rel * max(a, b) (TIE absolute by default).
    """
    positions = np.asarray(positions)
    w = dict(zip(positions.tolist(), np.asarray(weights, dtype=np.float64).tolist()))
    pool = [int(p) for p in positions if p >= n_sinks]
    want = min(kappa, len(pool))
    eo = [int(x) for x in oracle_edges]
    eg = [int(x) for x in dev_edges]
    assert len(eo) == want, f"{where}: oracle gave {len(eo)} edges, expected {want}"
    assert len(eg) == want, f"{where}: device gave {len(eg)} edges, expected min(kappa, pool) = {want}"
    if eg == eo:
        return True
    assert len(set(eg)) == len(eg), f"{where}: duplicate edge {eg}"
    inpool = set(pool)
    for p in eg:
        assert p in inpool, f"{where}: edge {p} is not an attended non-sink token"
    worst = 0.0
    we = [w[p] for p in eg]
    for i in range(len(eg) - 1):
        j = i + 1 + int(np.argmax(we[i + 1:]))
        inv = we[j] - we[i]
        assert inv <= tie + rel * we[j], (f"{where}: edges out of rank order: position {eg[j]} (rank {j}) "
                                          f"outweighs {eg[i]} (rank {i}) by {inv:.3g}")
        worst = max(worst, inv)
    chosen = set(eg)
    rest = [p for p in pool if p not in chosen]
    if rest and eg:
        best_rest = max(w[p] for p in rest)
        inv = best_rest - min(we)
        assert inv <= tie + rel * best_rest, f"{where}: an unchosen pool token outweighs a device edge by {inv:.3g}"
        worst = max(worst, inv)
    if gaps is not None:
        gaps.append(worst)
    return False


def centroids_ok(scores: np.ndarray, counts: np.ndarray, selected: Sequence[int], oracle_cent: Sequence[int],
                 dev_cent: Sequence[int], n_cent: int, where: str = "", gaps: Optional[List[float]] = None) -> bool:
    """The communities whose centroids a step attends (Table 6's centroid
    budget, read as the n_cent best-ranked non-empty communities the budget
    walk did not take).  True when the device's set equals the oracle's;
    False when it differs but is the head of a tie-consistent ranking of the
    communities outside the selection (the caller then adopts it);
    AssertionError otherwise.  The device must return exactly
    min(n_cent, non-empty communities outside the selection) distinct such
    communities, each scoring at least every other outsider's score - TIE.
    selected: the selection the step used (the device's, once accepted)."""
    so = sorted(int(c) for c in oracle_cent)
    sg = [int(c) for c in dev_cent]
    assert len(set(sg)) == len(sg), f"{where}: duplicate centroid community {sg}"
    sg = sorted(sg)
    counts = np.asarray(counts)
    C = counts.size
    live = counts > 0
    taken = np.zeros(C, dtype=bool)
    taken[[int(c) for c in selected]] = True
    outside = np.nonzero(live & ~taken)[0]
    want = min(max(n_cent, 0), outside.size)
    assert len(sg) == want, f"{where}: device attends {len(sg)} centroids, expected {want}"
    if so == sg:
        return True
    s = np.asarray(scores, dtype=np.float64)[:C]
    for c in sg:
        assert 0 <= c < C and live[c] and not taken[c], \
            f"{where}: centroid community {c} is empty, out of range or already selected"
    chosen = np.zeros(C, dtype=bool)
    chosen[sg] = True
    rest = np.nonzero(live & ~taken & ~chosen)[0]
    if rest.size and sg:
        inv = float(s[rest].max() - s[sg].min())
        assert inv <= TIE, (f"{where}: community {int(rest[np.argmax(s[rest])])} outranks centroid community "
                            f"{sg[int(np.argmin(s[sg]))]} by {inv:.3g}")
        if gaps is not None:
            gaps.append(max(inv, 0.0))
    return False


# Prefill graph (Figure 1 panel (1)): the logits come from bf16 operands on
# the matrix cores with float32 accumulation, |dz| <= (d - 1) 2^-24
# sum_i |q_i k_i| (about 6e-5 at d = 128 with these magnitudes, sum |q k| up
# to ~10), and a weight exp(z - lse) carries the error of z and of lse:
# relative eps <= ~1.7e-4 per weight (a sum of a group's positive weights keeps
# that bound).  Two weights can therefore change order when they differ by at
# most eps (a + b) <= 2 eps max(a, b): the pair window is relative to the
# larger weight compared.  Each device weight matches the oracle's within eps.
PREFILL_TIE_REL = 3.5e-4
PREFILL_WRT, PREFILL_WAT = 2e-4, 1e-9


def prefill_row_ok(W: np.ndarray, i: int, n_sinks: int, kappa: int, oracle_row: np.ndarray, dev_row: np.ndarray,
                   dev_weights: Optional[np.ndarray], where: str = "") -> bool:
    """One query position i of the prefill graph: dev_row (kappa entries, -1
    padded) against the oracle's, under the edge rules of edges_ok over the
    pool n_sinks <= j < i with a pair window relative to the larger weight
    (PREFILL_TIE_REL); dev_weights (or None) must match the oracle weight of each chosen
    edge within PREFILL_WRT / PREFILL_WAT and be 0 past the edges.
    W: the oracle's float64 weight of every key j <= i.
    Returns True when identical, False for an accepted near tie."""
    o = np.asarray(oracle_row)
    a = np.asarray(dev_row)
    k = int((o >= 0).sum())
    assert (o[k:] == -1).all()
    ka = int((a >= 0).sum())
    assert (a[ka:] == -1).all(), f"{where} row {i}: edges not -1 padded"
    same = edges_ok(np.arange(i), W[:i], n_sinks, kappa, o[:k], a[:ka], f"{where} row {i}", tie=1e-12,
                    rel=PREFILL_TIE_REL)
    if dev_weights is not None:
        assert (dev_weights[ka:] == 0).all(), f"{where} row {i}: padding weight"
        np.testing.assert_allclose(dev_weights[:ka], W[a[:ka]], rtol=PREFILL_WRT, atol=PREFILL_WAT,
                                   err_msg=f"{where} row {i}: weights")
    return same
