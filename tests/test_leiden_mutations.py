"""The Leiden pins must catch plausible mistakes in the Leiden oracle.

Each mutant plants one mistake into the source of one oracle function (a
dropped term, a wrong operand, a flipped comparison, a lost guard, a wrong
tie rule); the mutated function replaces the original and the pin suite of
tests/test_leiden_pins.py runs on the CPU: at least one pin has to fail.
"""
import inspect
import signal
import textwrap

import pytest

from oracle import leiden_oracle as L
from tests import test_leiden_pins as P


def _pins():
    checks = [P.test_token_graph_hand_example, P.test_quality_hand_value_two_triangles,
              P.test_quality_resolution_against_definition, P.test_brute_force_optimum_at_other_resolutions,
              P.test_resolution_zero_gives_connected_components, P.test_planted_disjoint_cliques_recovered,
              P.test_ring_of_cliques_resolution_limit, P.test_planted_blocks_recovered,
              P.test_refine_splits_what_is_not_connected, P.test_refine_hand_example,
              P.test_aggregate_hand_example, P.test_guarantees_on_random_graphs,
              P.test_guarantees_on_token_graphs, P.test_no_edges_and_degenerate_graphs,
              P.test_move_nodes_hand_trace, P.test_move_nodes_to_an_empty_community,
              P.test_quality_with_self_loops_against_definition, P.test_refine_skips_a_node_not_well_connected,
              P.test_extend_by_vote_hand_example, P.test_extend_by_vote_matches_partition_of_isolated_growth]
    checks += [lambda a=a: P.test_quality_closed_form_ring_of_cliques(*a) for a in ((30, 5), (8, 4), (3, 6))]
    checks += [lambda nm=nm: P.test_brute_force_optimum(nm) for nm in sorted(P.STRUCTURED)]
    return checks


# (function, text in its source, replacement)
MUTANTS = [
    ("token_graph", "adj[b][a] = adj[b].get(a, 0) + 1", "pass"),                       # one direction only
    ("token_graph", "if j < 0:", "if j < n_sinks:"),                                   # silently drops bad edges
    ("quality_terms", "gnum * K[c] * K[c]", "gnum * K[c]"),                            # K not squared
    ("quality_terms", "if labels[u] == c:", "if labels[u] == c and u != v:"),          # self-loops dropped
    ("move_nodes_fast", "(Kc[D] - kv)", "Kc[D]"),                                      # v not taken out of D
    ("move_nodes_fast", "gnum * kv * Kc[C]", "gnum * Kc[C]"),                          # k_v missing
    ("move_nodes_fast", "if s > best_s:", "if s >= best_s:"),                          # ties to the higher id
    ("move_nodes_fast", "if best_s < 0:", "if best_s < -10 ** 30:"),                   # never a new community
    ("move_nodes_fast", "if u != v and comm[u] != best and not queued[u]:", "if False:"),  # no re-queue
    ("refine", "if inside[v] * two_m * gden < gnum * kv * (KS - kv):", "if False:"),  # v need not be well-connected
    ("refine", "if ext[R] * two_m * gden < gnum * Kr[R] * (KS - Kr[R]):", "if False:"),  # R need not be
    ("refine", "ext[best] += inside[v] - 2 * to[best]", "ext[best] += inside[v]"),    # ext not updated right
    ("refine", "if size[ref[v]] != 1:", "if False:"),                                  # merged nodes move again
    ("refine", "if g > best_g:", "if g >= best_g:"),                                   # zero-gain merges
    ("aggregate", "new[a][b] = new[a].get(b, 0) + wt", "new[a][b] = new[a].get(b, 0) + (wt if a != b else 0)"),
    ("aggregate", "start[node_map[v]] = cids[comm[v]]", "start[node_map[v]] = node_map[v]"),  # P not carried
    ("move_nodes_fast", "best = heapq.heappop(empty)", "best = empty.pop()"),         # not the lowest empty id
    ("leiden", "empty = list(range(n_comm, len(adj)))", "empty = []"),                  # no free ids past level 0
    ("leiden", "if len(set(ref)) == len(adj):", "if True:"),                            # stops after level 0
    ("first_token_order", "seen[c] = len(seen)", "seen[c] = -len(seen) - 1"),
    ("extend_by_vote", "out[i] = min(c for c, v in votes.items() if v == best)",
     "out[i] = max(c for c, v in votes.items() if v == best)"),                     # ties to the higher id
    ("extend_by_vote", "if j >= 0 and out[j] >= 0:", "if j >= 0:"),                # unlabelled targets vote
    ("extend_by_vote", "out[i] = n_comm\n", "out[i] = 0\n"),                        # no new community

]


def _mutate(name, old, new):
    src = textwrap.dedent(inspect.getsource(getattr(L, name)))
    assert src.count(old) == 1, f"{name}: '{old}' must occur once"
    ns = dict(L.__dict__)
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), ns)
    return ns[name]


class _Slow(Exception):
    pass


def _run_limited(chk, seconds=5.0):
    """Run one pin; a mutant that never ends (a node moving back and forth)
    counts as caught once the pin takes longer than `seconds`."""
    def _alarm(signum, frame):
        raise _Slow()
    old = signal.signal(signal.SIGALRM, _alarm)
    signal.setitimer(signal.ITIMER_REAL, seconds)
    try:
        chk()
    finally:
        signal.setitimer(signal.ITIMER_REAL, 0)
        signal.signal(signal.SIGALRM, old)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[f"{m[0]}:{m[1][:30]}" for m in MUTANTS])
def test_pins_catch_mutant(monkeypatch, name, old, new):
    monkeypatch.setattr(L, name, _mutate(name, old, new))
    failed = 0
    for chk in _pins():
        try:
            _run_limited(chk)
        except KeyboardInterrupt:
            raise
        except BaseException:      # pytest.raises reports through a BaseException
            failed += 1
            break
    assert failed > 0, f"no pin catches the mutant of {name}: {old!r} -> {new!r}"


def test_unmutated_oracle_passes_every_pin():
    for chk in _pins():
        chk()
