"""The pins must catch plausible mistakes in the oracle.

Each mutant below plants one mistake into a copy of an oracle function (a
dropped term, a wrong sign, a flipped comparison, a swapped operand, a wrong
tie rule).  The pin suite is then run against the mutated oracle on the CPU
and at least one pin has to fail.
"""
import numpy as np
import pytest

from oracle import ckv_oracle as O
from tests import test_oracle_pins as P


def _pins():
    """The pin checks, called directly (parametrised ones over a few params)."""
    fx = P._hand()
    checks = [lambda c=c["name"]: P.test_hand_fixture_case(c) for c in fx["cases"]]
    checks += [P.test_hand_fixture_sequence, P.test_centroid_brute_force_means,
               P.test_centroid_zero_noise_is_center, P.test_score_exact_small_integers,
               P.test_score_brute_force_fsum, P.test_group_score_is_sum_of_head_scores,
               P.test_select_no_skip_ahead, P.test_select_everything_under_large_budget,
               P.test_select_top_k_cap_matches_heap, P.test_attend_two_tokens_closed_form,
               P.test_attend_matches_torch_sdpa_float64, P.test_dense_chunking_is_exact,
               P.test_attended_positions_brute_force,
               P.test_top_kappa_excludes_sinks_and_takes_all_when_short,
               P.test_group_weights_explicit_loop, P.test_budget_walk_invariants_on_workload,
               P.test_recall_two_tokens_closed_form, P.test_recall_brute_force_loops,
               P.test_recall_full_set_is_one_and_complements_add_up,
               P.test_prefill_identical_keys_closed_form, P.test_prefill_one_hot_target_closed_form,
               P.test_prefill_subsets_brute_force, P.test_prefill_per_head_matches_decode_edges,
               P.test_prefill_invariants_and_rows, P.test_centroid_entry_two_term_closed_form,
               P.test_centroid_budget_past_the_walk_on_workload]
    checks += [lambda a=a: P.test_centroid_communities_hand_cases(*a) for a in P.CENT_HAND_CASES]
    checks += [lambda b=b, h=h: P.test_centroid_entries_equal_attention_over_identical_members(b, h)
               for b in (1, 3, 64) for h in (1, 4)]
    checks += [lambda m=m: P.test_value_sums_stay_member_sums(m) for m in ("per_head", "group")]
    checks += [lambda s=s: P.test_select_matches_definition(s) for s in range(40)]
    checks += [lambda s=s: P.test_top_kappa_matches_heap(s) for s in range(20)]
    checks += [lambda s=s: P.test_vote_matches_counter(s) for s in range(20)]
    checks += [lambda m=m: P.test_centroid_stays_member_mean(m) for m in ("per_head", "group")]
    checks += [lambda m=m: P.test_full_budget_equals_dense(m) for m in ("per_head", "group")]
    return checks


def _failures(monkeypatch, name, fn):
    monkeypatch.setattr(O, name, fn)
    failed = 0
    for chk in _pins():
        try:
            chk()
        except Exception:
            failed += 1
    return failed


_orig = {k: getattr(O, k) for k in dir(O) if not k.startswith("_")}


def m_score_sign(qbar, cent32, counts):
    return -_orig["score_communities"](qbar, cent32, counts)


def m_score_no_empty_mask(qbar, cent32, counts):
    return (cent32.astype(np.float64) @ np.asarray(qbar, np.float64)).astype(np.float32)


def m_select_overflow_included(scores, counts, budget, max_comm=0):
    taken, total = [], 0
    for c in O.rank_communities(scores, counts):
        if max_comm > 0 and len(taken) == max_comm:
            break
        taken.append(int(c))
        total += int(counts[c])
        if total > budget:
            break
    return np.array(sorted(taken), dtype=np.int64)


def m_select_skip_ahead(scores, counts, budget, max_comm=0):
    taken, total = [], 0
    for c in O.rank_communities(scores, counts):
        if max_comm > 0 and len(taken) == max_comm:
            break
        if total + int(counts[c]) > budget:
            continue
        taken.append(int(c))
        total += int(counts[c])
    return np.array(sorted(taken), dtype=np.int64)


def m_rank_tie_high_id(scores, counts):
    ids = np.nonzero(np.asarray(counts) > 0)[0]
    order = np.lexsort((-ids, -scores[ids].astype(np.float64)))
    return ids[order]


def m_rank_ascending(scores, counts):
    return _orig["rank_communities"](scores, counts)[::-1]


def m_attend_no_norm(q_heads, keys, values, sm_scale):
    q = np.asarray(q_heads, np.float64).reshape(-1, np.shape(q_heads)[-1])
    z = sm_scale * (q @ np.asarray(keys, np.float64).T)
    e = np.exp(z - z.max(axis=1, keepdims=True))
    return e @ np.asarray(values, np.float64), e, z


def m_attend_no_scale(q_heads, keys, values, sm_scale):
    return _orig["attend"](q_heads, keys, values, 1.0)


def m_attend_kv_swapped(q_heads, keys, values, sm_scale):
    return _orig["attend"](q_heads, values, keys, sm_scale)


def m_attend_transposed_q(q_heads, keys, values, sm_scale):
    q = np.asarray(q_heads, np.float64).reshape(-1, np.shape(q_heads)[-1])
    return _orig["attend"](q[:, ::-1], keys, values, sm_scale)


def m_positions_no_sinks(labels, n_sinks, selected):
    return _orig["attended_positions"](labels, 0, selected)


def m_topk_with_sinks(weights, positions, kappa, n_sinks):
    return _orig["top_kappa"](weights, positions, kappa, 0)


def m_topk_smallest(weights, positions, kappa, n_sinks):
    return _orig["top_kappa"](-np.asarray(weights), positions, kappa, n_sinks)


def m_topk_tie_high_pos(weights, positions, kappa, n_sinks):
    positions = np.asarray(positions)
    pool = positions >= n_sinks
    w, pos = np.asarray(weights)[pool], positions[pool]
    return pos[np.lexsort((-pos, -w))[:kappa]]


def m_topk_off_by_one(weights, positions, kappa, n_sinks):
    return _orig["top_kappa"](weights, positions, kappa + 1, n_sinks)


def m_vote_high_id(edge_labels):
    lab = np.asarray([x for x in edge_labels if x >= 0])
    if lab.size == 0:
        return -1
    vals, cnt = np.unique(lab, return_counts=True)
    return int(vals[::-1][np.argmax(cnt[::-1])])


def m_vote_first_edge(edge_labels):
    lab = [x for x in edge_labels if x >= 0]
    return int(lab[0]) if lab else -1


def m_weights_max(probs):
    return np.asarray(probs, np.float64).reshape(-1, np.shape(probs)[-1]).max(axis=0)


def m_agg_mean(q_heads):
    q = np.asarray(q_heads, np.float64).reshape(-1, np.shape(q_heads)[-1])
    return q.mean(axis=0)


def m_means_off_by_one(sums, counts):
    out = np.zeros_like(sums)
    nz = counts > 0
    out[nz] = sums[nz] / (counts[nz, None] + 1.0)
    return out


def m_sums_skip_first(keys, labels, n_comm):
    keys = np.asarray(keys, np.float64)
    labels = np.asarray(labels).copy()
    first = np.nonzero(labels >= 0)[0]
    if first.size:
        labels[first[0]] = -1
    return _orig["community_sums"](keys, labels, n_comm)


def m_dense_last_chunk_only(q_heads, keys, values, sm_scale, chunk=1 << 15):
    n = keys.shape[0]
    lo = max(0, n - 1 - ((n - 1) % chunk)) if n > chunk else 0
    return _orig["attend"](q_heads, keys[lo:], values[lo:], sm_scale)[0]


def m_recall_unnormalised(q_heads, keys, positions, sm_scale):
    q = np.asarray(q_heads, np.float64).reshape(-1, np.shape(q_heads)[-1])
    z = float(sm_scale) * (q @ np.asarray(keys, np.float64).T)
    p = np.exp(z - z.max(axis=1, keepdims=True))
    return p[:, np.asarray(positions, np.int64)].sum(axis=1)


def m_recall_no_scale(q_heads, keys, positions, sm_scale):
    return _orig["attention_mass_recall"](q_heads, keys, positions, 1.0)


def _prefill_from(w, n_sinks, kappa, cand_hi=0, tie_sign=1):
    # top-kappa rows from a weight matrix w [n][n]; candidates [n_sinks, i + cand_hi)
    n = w.shape[0]
    edges = np.full((n, kappa), -1, dtype=np.int64)
    weights = np.zeros((n, kappa))
    for i in range(n):
        cand = np.arange(n_sinks, min(i + cand_hi, n))
        if cand.size == 0:
            continue
        wi = w[i, cand]
        order = np.lexsort((tie_sign * cand, -wi))[:kappa]
        edges[i, :order.size] = cand[order]
        weights[i, :order.size] = wi[order]
    return edges, weights


def m_prefill_self_candidate(q_heads, keys, n_sinks, kappa, sm_scale):
    return _prefill_from(O.causal_probs(q_heads, keys, sm_scale).sum(axis=0), n_sinks, kappa, cand_hi=1)


def m_prefill_sinks_in_pool(q_heads, keys, n_sinks, kappa, sm_scale):
    return _orig["prefill_edges"](q_heads, keys, 0, kappa, sm_scale)


def m_prefill_tie_high_pos(q_heads, keys, n_sinks, kappa, sm_scale):
    return _prefill_from(O.causal_probs(q_heads, keys, sm_scale).sum(axis=0), n_sinks, kappa, tie_sign=-1)


def m_prefill_group_max(q_heads, keys, n_sinks, kappa, sm_scale):
    return _prefill_from(O.causal_probs(q_heads, keys, sm_scale).max(axis=0), n_sinks, kappa)


def m_causal_self_excluded(q_heads, keys, sm_scale):
    q, K = np.asarray(q_heads, np.float64), np.asarray(keys, np.float64)
    n = K.shape[0]
    z = float(sm_scale) * np.einsum("ihd,jd->hij", q, K)
    z[:, np.triu(np.ones((n, n), dtype=bool), k=0)] = -np.inf
    z[:, 0, 0] = 0.0  # row 0 keeps one term
    e = np.exp(z - z.max(axis=2, keepdims=True))
    return e / e.sum(axis=2, keepdims=True)


def m_causal_no_mask(q_heads, keys, sm_scale):
    q, K = np.asarray(q_heads, np.float64), np.asarray(keys, np.float64)
    z = float(sm_scale) * np.einsum("ihd,jd->hij", q, K)
    e = np.exp(z - z.max(axis=2, keepdims=True))
    return e / e.sum(axis=2, keepdims=True)


def m_causal_no_scale(q_heads, keys, sm_scale):
    return _orig["causal_probs"](q_heads, keys, 1.0)


def m_prefill_rows_self_excluded(q_heads_rows, rows, keys, n_sinks, kappa, sm_scale):
    K = np.asarray(keys, np.float64)
    edges = np.full((len(rows), kappa), -1, dtype=np.int64)
    weights = np.zeros((len(rows), kappa))
    for r, i in enumerate(rows):
        if i == 0:
            continue
        z = float(sm_scale) * (np.asarray(q_heads_rows[r], np.float64) @ K[:i].T)
        e = np.exp(z - z.max(axis=1, keepdims=True))
        w = (e / e.sum(axis=1, keepdims=True)).sum(axis=0)
        cand = np.arange(n_sinks, i)
        if cand.size == 0:
            continue
        order = np.lexsort((cand, -w[n_sinks:i]))[:kappa]
        edges[r, :order.size] = cand[order]
        weights[r, :order.size] = w[n_sinks:i][order]
    return edges, weights


def m_row_weights_no_scale(q_heads_row, i, keys, sm_scale):
    return _orig["prefill_row_weights"](q_heads_row, i, keys, 1.0)


def m_cent_includes_taken(scores, counts, selected, n_cent):
    return _orig["centroid_communities"](scores, counts, np.zeros(0, dtype=np.int64), n_cent)


def m_cent_lowest_ranked(scores, counts, selected, n_cent):
    if n_cent <= 0:
        return np.zeros(0, dtype=np.int64)
    taken = {int(c) for c in selected}
    rest = [int(c) for c in O.rank_communities(scores, counts) if int(c) not in taken]
    return np.array(sorted(rest[::-1][:n_cent]), dtype=np.int64)


def m_cent_skip_stopper(scores, counts, selected, n_cent):
    if n_cent <= 0:
        return np.zeros(0, dtype=np.int64)
    taken = {int(c) for c in selected}
    rest = [int(c) for c in O.rank_communities(scores, counts) if int(c) not in taken]
    return np.array(sorted(rest[1:n_cent + 1]), dtype=np.int64)


def m_cent_one_short(scores, counts, selected, n_cent):
    return _orig["centroid_communities"](scores, counts, selected, n_cent)[:max(n_cent - 1, 0)]


def m_cent_no_count(q, K, V, MU, NU, n, sm_scale):
    return _orig["attend_with_centroids"](q, K, V, MU, NU, np.ones_like(np.asarray(n)), sm_scale)


def m_cent_value_sum(q, K, V, MU, NU, n, sm_scale):
    nn = np.asarray(n, dtype=np.float64).reshape(-1, 1)
    return _orig["attend_with_centroids"](q, K, V, MU, np.asarray(NU) * nn, n, sm_scale)


def m_cent_unscaled(q, K, V, MU, NU, n, sm_scale):
    return _orig["attend_with_centroids"](q, K, V, np.asarray(MU) / sm_scale, NU, n, sm_scale)


def m_cent_token_only_norm(q, K, V, MU, NU, n, sm_scale):
    out, p, z, pc, zc = _orig["attend_with_centroids"](q, K, V, MU, NU, n, sm_scale)
    return out, p / p.sum(axis=1, keepdims=True), z, pc, zc


MUTANTS = {
    "centroid_communities": [m_cent_includes_taken, m_cent_lowest_ranked, m_cent_skip_stopper, m_cent_one_short],
    "attend_with_centroids": [m_cent_no_count, m_cent_value_sum, m_cent_unscaled, m_cent_token_only_norm],
    "prefill_row_weights": [m_row_weights_no_scale],
    "prefill_edges": [m_prefill_self_candidate, m_prefill_sinks_in_pool, m_prefill_tie_high_pos,
                      m_prefill_group_max],
    "causal_probs": [m_causal_self_excluded, m_causal_no_mask, m_causal_no_scale],
    "prefill_edges_rows": [m_prefill_rows_self_excluded],
    "score_communities": [m_score_sign, m_score_no_empty_mask],
    "select_communities": [m_select_overflow_included, m_select_skip_ahead],
    "rank_communities": [m_rank_tie_high_id, m_rank_ascending],
    "attend": [m_attend_no_norm, m_attend_no_scale, m_attend_kv_swapped, m_attend_transposed_q],
    "attended_positions": [m_positions_no_sinks],
    "top_kappa": [m_topk_with_sinks, m_topk_smallest, m_topk_tie_high_pos, m_topk_off_by_one],
    "majority_vote": [m_vote_high_id, m_vote_first_edge],
    "edge_weights": [m_weights_max],
    "aggregate_query": [m_agg_mean],
    "community_means": [m_means_off_by_one],
    "community_sums": [m_sums_skip_first],
    "dense_attend": [m_dense_last_chunk_only],
    "attention_mass_recall": [m_recall_unnormalised, m_recall_no_scale],
}


@pytest.mark.parametrize("name,mutant", [(k, f) for k, fs in MUTANTS.items() for f in fs],
                         ids=[f.__name__ for fs in MUTANTS.values() for f in fs])
def test_pins_catch_mutant(monkeypatch, name, mutant):
    assert _failures(monkeypatch, name, mutant) > 0


def test_apply_update_mutant_caught(monkeypatch):
    def bad(self, gid, assign, k_new, v_new=None):  # overwrite instead of accumulate
        st = self.g[gid]
        P_ = self.len[st.b]
        if assign < 0:
            return
        st.labels[P_] = assign
        st.sums[assign] = np.asarray(k_new, np.float64) * st.counts[assign]
        st.counts[assign] += 1
    monkeypatch.setattr(O.Oracle, "apply_update", bad)
    assert _count_failures() > 0


def test_value_sum_update_mutant_caught(monkeypatch):
    orig = O.Oracle.apply_update

    def bad(self, gid, assign, k_new, v_new=None):  # the value sum is left as it was
        orig(self, gid, assign, k_new, None)
    monkeypatch.setattr(O.Oracle, "apply_update", bad)
    assert _count_failures() > 0


def _count_failures():
    failed = 0
    for chk in _pins():
        try:
            chk()
        except Exception:
            failed += 1
    return failed


def test_unmutated_oracle_passes_every_pin():
    for chk in _pins():
        chk()
