"""Parity harness: runs decode steps through the C ABI on the GPU and checks
every output against the CPU oracle on the same seeded inputs.

Bars (written here once, used by every GPU test):
  * community selection, token lists, assignments, labels, sizes, CSR and
    tail state: bit-exact; a selected set or edge set may differ from the
    oracle's only by members whose oracle score / weight lies within TIE of
    the cut, and then the oracle adopts the device's decision and goes on;
  * attention outputs: |gpu - ref| <= ATOL + RTOL * |ref| element-wise;
  * float32 centroids and float64 key sums after every update: bit-exact
    (both sides hold the exact float64 sum of bf16/fp32 keys and round the
    mean once).
"""
from __future__ import annotations

import sys
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional

import numpy as np
import torch

from community_kv_retrieval_amd import ckv, runner, synth
from oracle import ckv_oracle as O
from tests import decisions as D

ATOL, RTOL = 2e-3, 1e-2
TIE = D.TIE
LOGIT_ATOL = 1e-4
# The int8 screening copy (as the library documents it): codes in [-SCREEN_MAX, SCREEN_MAX]
SCREEN_MAX = 127


def screen_factor(D: int) -> float:
    """Bound factor of a screening score, in units of cscale * |qbar|_1: half a
    code for the rounding of the codes, plus (D + 4) SCREEN_MAX 2^-24 for the
    float32 accumulation of D products of |q_d| with codes up to SCREEN_MAX and
    the float32 rounding of qbar."""
    return 0.5 + (D + 4) * SCREEN_MAX * 2.0 ** -24


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


@dataclass
class Stats:
    steps: int = 0
    graphs: int = 0
    near_sel: int = 0
    near_edges: int = 0
    max_abs: float = 0.0
    max_rel: float = 0.0
    dense_equal: int = 0
    near_cent: int = 0
    cent_terms: int = 0
    cent_visible: int = 0   # graphs whose output the centroid terms move beyond the output tolerance
    band_min: int = 0       # largest lower bound of a selection's band seen (_band_lower_bound)
    gaps: List[float] = field(default_factory=list)


def host_kv(slices, wanted):
    """kv[b][kh] = (K, V) float32 arrays for the wanted (b, kh) pairs."""
    return [[(s.k.float().numpy(), s.v.float().numpy()) if (s.b, s.kh) in wanted else None for s in row]
            for row in slices]


def make_pair(w: synth.Workload, seed: int, steps: int, graphs: Optional[List[int]] = None, **kw):
    layer = runner.load_layer(w, seed, extra=steps + 1, **kw)
    gids = list(range(w.n_graphs)) if graphs is None else list(graphs)
    wanted = {tuple(w.graph_coords(g)[:2]) for g in gids}
    labels = synth.graph_labels(w, layer.slices)
    n_comm = synth.graph_n_comm(w, layer.slices)
    orc = O.Oracle(w, host_kv(layer.slices, wanted), {g: labels[g] for g in gids}, {g: n_comm[g] for g in gids},
                   graphs=gids, extra=steps + 1)
    return layer, orc


def check_index_state(layer, orc: O.Oracle, w: synth.Workload, full: bool = False):
    """Device index == oracle state: sizes, centroids and sums bit-exact."""
    idx = layer.idx
    size = idx.size.cpu().numpy()
    for g, st in orc.g.items():
        C = st.counts.size
        np.testing.assert_array_equal(size[g, :C], st.counts, err_msg=f"size g={g}")
        assert (size[g, C:] == 0).all()
        cent = idx.cent[g, :C].cpu().numpy()
        np.testing.assert_array_equal(cent, orc.centroids32(g), err_msg=f"centroids g={g}")
        check_screening_copy(idx, g, C, cent)
        if full:
            np.testing.assert_array_equal(idx.csum[g, :C].cpu().numpy(), st.sums, err_msg=f"csum g={g}")
            if idx.cent_budget > 0:
                np.testing.assert_array_equal(idx.vsum[g, :C].cpu().numpy(), st.vsums, err_msg=f"vsum g={g}")
            n = orc.len[st.b]
            np.testing.assert_array_equal(idx.label[g, :n].cpu().numpy(), st.labels[:n], err_msg=f"label g={g}")


def check_screening_copy(idx, g: int, C: int, cent: np.ndarray):
    """The int8 screening copy of the centroid table (stored tile-major,
    [c_cap / 256][D][256] per graph): per community scale = max |cent| / 127
    (float32) and code = round(cent / scale), clamped to +-127 (0 for a zero
    column), as the library documents it."""
    scale = idx.cscale[g, :C].cpu().numpy()
    D = idx.cq.shape[2]
    code = idx.cq[g].permute(1, 0, 2).reshape(D, -1)[:, :C].t().cpu().numpy().astype(np.int32)
    want_scale = (np.abs(cent).max(axis=1).astype(np.float32) / np.float32(SCREEN_MAX)).astype(np.float32)
    np.testing.assert_array_equal(scale, want_scale, err_msg=f"cscale g={g}")
    with np.errstate(divide="ignore", invalid="ignore"):
        want = np.clip(np.rint(cent / want_scale[:, None]), -SCREEN_MAX, SCREEN_MAX)
    want = np.where(want_scale[:, None] > 0, want, 0).astype(np.int32)
    np.testing.assert_array_equal(code, want, err_msg=f"cq g={g}")


def check_csr(layer, orc: O.Oracle):
    """Base CSR right after the build: members of every community, ascending."""
    idx = layer.idx
    offs = idx.offs.cpu().numpy()
    toks = idx.toks.cpu().numpy()
    for g, st in orc.g.items():
        n = orc.len[st.b]
        lab = st.labels[:n]
        order = np.argsort(lab, kind="stable")
        order = order[lab[order] >= 0]
        C = st.counts.size
        np.testing.assert_array_equal(offs[g, 1:C + 1] - offs[g, :C], st.counts)
        np.testing.assert_array_equal(toks[g, :order.size], order)


def _check_screening(scores, cscale, q_heads, exact, counts, where: str):
    """The scoring kernel's screening scores against the oracle's exact ones.
    The int8 copy rounds every centroid entry to within cscale / 2, and the
    float32 dot product over D dimensions (with the query rounded to float32)
    adds at most 127 (D + 4) 2^-24 cscale |qbar|_1 (screen_factor); the two float32 roundings
    of the screening score and the one of the exact score stay under
    2^-21 |s~|.  The selection's certain-taken / certain-not decisions rest on
    this bound.  Empty communities and ids at or past the count score -inf."""
    C, D = counts.size, q_heads.shape[-1]
    live = counts > 0
    assert np.all(scores[:C][~live] == -np.inf) and np.all(scores[C:] == -np.inf), f"{where}: dead ids not -inf"
    qbar = q_heads.astype(np.float64).sum(axis=0).astype(np.float32).astype(np.float64)
    s = scores[:C][live].astype(np.float64)
    bound = cscale[:C][live].astype(np.float64) * np.abs(qbar).sum() * screen_factor(D) \
        + np.abs(s) * 2.0 ** -21
    err = np.abs(s - exact[live].astype(np.float64))
    assert np.all(err <= bound), f"{where}: screening error {err.max():.3g} beyond its bound"


def _band_lower_bound(r: O.GraphStep, counts, cscale, q_heads) -> int:
    """Live communities whose screening interval holds the exact score of the
    walk's stopper (the best-ranked live community not taken).  Their upper
    bounds reach the cut and their lower bounds do not clear it, so each of them
    is in the selection's band of undecided communities however the score bins
    fall: the count is a lower bound of the band's size (0 when every live
    community is taken)."""
    C, D = counts.size, q_heads.shape[-1]
    live = counts > 0
    out = live.copy()
    out[np.asarray(r.selected, dtype=np.int64)] = False
    if not out.any():
        return 0
    s = r.scores[:C].astype(np.float64)
    ids = np.flatnonzero(out)
    stop = ids[np.lexsort((ids, -s[ids]))[0]]  # highest score, then lowest id
    qbar = q_heads.astype(np.float64).sum(axis=0).astype(np.float32).astype(np.float64)
    E = cscale[:C].astype(np.float64) * np.abs(qbar).sum() * screen_factor(D)
    return int((live & (np.abs(s - s[stop]) <= E)).sum())


def _selection_ok(r: O.GraphStep, counts, gpu_sel, w, stats: Stats, where: str) -> bool:
    return D.selection_ok(r.scores, counts, r.selected, gpu_sel, w.budget, w.max_comm, where, stats.gaps) or \
        _count(stats, "near_sel")


def _edges_ok(r: O.GraphStep, gpu_edges, w, stats: Stats, where: str) -> bool:
    return D.edges_ok(r.positions, r.weights, w.n_sinks, w.kappa, r.edges, gpu_edges, where, stats.gaps) or \
        _count(stats, "near_edges")


def _count(stats: Stats, field_name: str) -> bool:
    setattr(stats, field_name, getattr(stats, field_name) + 1)
    return False


def _check_logits(H, g, tl, r, where):
    """Token logits of every slot, and the softmax state (max, sum) over the
    tokens and the centroid terms of a centroid budget."""
    if r.positions.size:
        slot = {int(p): i for i, p in enumerate(tl)}
        idxs = np.array([slot[int(p)] for p in r.positions])
        gl = H["logits"][g][:, idxs]
        assert np.abs(gl - r.logits).max() <= LOGIT_ATOL * max(1.0, np.abs(r.logits).max()), f"{where}: logits"
    z = np.concatenate([r.logits, r.cent_logits], axis=1) if r.cent.size else r.logits
    np.testing.assert_allclose(H["ml"][g][:, 0], z.max(axis=1), atol=LOGIT_ATOL * 20, err_msg=f"{where}: ml max")
    lsum = np.exp(z - z.max(axis=1, keepdims=True)).sum(axis=1)
    np.testing.assert_allclose(H["ml"][g][:, 1], lsum, rtol=1e-4, err_msg=f"{where}: ml sum")


def snapshot(buf, cscale, idx=None) -> Dict[str, np.ndarray]:
    """Host copies of a decoder's step outputs, plus the screening scales the
    step scored with (taken before its update changed them) and, with a
    centroid budget, the index's centroid communities of the step."""
    H = {k: getattr(buf, k).cpu().numpy() for k in
         ("sel", "sel_n", "top", "tok_list", "tok_n", "out", "logits", "ml", "edges", "assign", "scores")}
    H["cscale"] = cscale.cpu().numpy()
    if idx is not None and idx.cent_budget > 0:
        H["cent_sel"] = idx.cent_sel.cpu().numpy()
        H["cent_n"] = idx.cent_n.cpu().numpy()
    return H


def check_graph(H, g: int, orc: O.Oracle, qn: np.ndarray, k_new: np.ndarray, w: synth.Workload, stats: Stats,
                where: str, dense: Optional[torch.Tensor] = None, v_new: Optional[np.ndarray] = None):
    """Every output of graph g's step against the oracle's step on the same
    query, then the oracle applies the device's (checked) assignment.
    qn: [B][Hq][d] the step's queries; k_new, v_new: [B][Hkv][d] the new keys
    and values (v_new: for the value sums of a centroid budget)."""
    st = orc.g[g]
    gsel = H["sel"][g, :H["sel_n"][g]]
    assert (np.diff(gsel) > 0).all(), f"{where}: sel not ascending"
    r = orc.step_graph(g, qn)
    _check_screening(H["scores"][g], H["cscale"][g], qn[st.b, st.qh0:st.qh0 + st.nh], r.scores, st.counts, where)
    if w.max_comm == 0:
        stats.band_min = max(stats.band_min, _band_lower_bound(r, st.counts, H["cscale"][g],
                                                               qn[st.b, st.qh0:st.qh0 + st.nh]))
    assert H["top"][g] == r.top, f"{where}: top {H['top'][g]} != {r.top}"
    if not _selection_ok(r, st.counts, gsel, w, stats, where):
        r = orc.step_graph(g, qn, force_sel=gsel)
    gcent = None
    if w.cent_budget > 0:
        gcent = H["cent_sel"][g, :H["cent_n"][g]]
        assert (np.diff(gcent) > 0).all(), f"{where}: centroid communities not ascending"
        if not D.centroids_ok(r.scores, st.counts, gsel, r.cent, gcent, w.cent_budget, where, stats.gaps):
            stats.near_cent += 1
            r = orc.step_graph(g, qn, force_sel=gsel, force_cent=gcent)
        stats.cent_terms += int(gcent.size)
    tl = H["tok_list"][g, :H["tok_n"][g]]
    assert tl.size == np.unique(tl).size, f"{where}: duplicate token"
    np.testing.assert_array_equal(np.sort(tl), r.positions, err_msg=f"{where}: token set")
    gout = H["out"][st.b, st.qh0:st.qh0 + st.nh].astype(np.float64)
    err = np.abs(gout - r.out)
    assert np.all(err <= ATOL + RTOL * np.abs(r.out)), f"{where}: attention max abs err {err.max():.3g}"
    if r.cent.size:  # would the check above see the centroid terms?  (the test's power)
        r0 = orc.step_graph(g, qn, force_sel=gsel, force_cent=[])
        if np.any(np.abs(r0.out - r.out) > ATOL + RTOL * np.abs(r.out)):
            stats.cent_visible += 1
    stats.max_abs = max(stats.max_abs, float(err.max()))
    stats.max_rel = max(stats.max_rel, float((err / np.maximum(np.abs(r.out), 1e-3)).max()))
    if dense is not None:
        grp = w.n_q_heads // w.n_kv_heads
        dref = orc.dense(qn, st.b, st.kh)[st.qh0 - st.kh * grp:st.qh0 - st.kh * grp + st.nh]
        dn = dense.cpu().numpy()[st.b, st.qh0:st.qh0 + st.nh]
        assert np.all(np.abs(dn - dref) <= ATOL + RTOL * np.abs(dref)), f"{where}: dense baseline"
        if r.positions.size == orc.len[st.b]:  # every cached token attended: sparse == dense
            assert np.all(np.abs(gout - dref) <= ATOL + RTOL * np.abs(dref)), f"{where}: sparse vs dense"
            stats.dense_equal += 1
    # logits of every slot, and the softmax state (empty: max -inf, sum 0)
    if r.positions.size == 0 and r.cent.size == 0:
        assert np.all(H["ml"][g][:, 0] == -np.inf) and np.all(H["ml"][g][:, 1] == 0), f"{where}: empty ml"
    else:
        _check_logits(H, g, tl, r, where)
    ge = H["edges"][g]
    ne = int((ge >= 0).sum())
    assert (ge[ne:] == -1).all(), f"{where}: edges not -1 padded"
    if not _edges_ok(r, ge[:ne], w, stats, where):
        r = orc.step_graph(g, qn, force_sel=gsel, force_edges=ge[:ne], force_cent=gcent)
    assert H["assign"][g] == r.assign, f"{where}: assign {H['assign'][g]} != {r.assign}"
    orc.apply_update(g, int(H["assign"][g]), k_new[st.b, st.kh], None if v_new is None else v_new[st.b, st.kh])
    stats.graphs += 1
    return r


def run_steps(w: synth.Workload, seed: int, steps: int, graphs: Optional[List[int]] = None,
              check_state_every: int = 1, layer_kw: Optional[dict] = None, check_dense: bool = False,
              pair=None, windows: int = 1, defer: bool = True, q_fn=None, first_step: int = 0,
              edge_log: Optional[Dict] = None) -> Stats:
    """Steps the library and the oracle side by side and checks every output.
    windows > 1 runs each step as the decoder's windowed multi-stream step;
    defer=False runs complete gathers (combine inside the gather kernel).
    q_fn(t, q) -> q replaces step t's queries (both sides see the same ones).
    Steps are numbered first_step .. first_step + steps - 1 (the inputs of
    step t are drawn for t), continuing a pair that has already run.
    edge_log (a dict) receives edge_log[(t, g)] = the oracle's edges of graph
    g at step t (after adopting an accepted near tie)."""
    layer, orc = pair if pair is not None else make_pair(w, seed, steps, graphs, **(layer_kw or {}))
    dev = layer.kv.kv.device
    dec, buf = layer.dec, layer.dec.buf
    dec.defer = defer
    dec.set_windows(windows)
    assert not (check_dense and windows > 1), "the dense check runs between the calls of one window"
    if first_step == 0:
        check_csr(layer, orc)
        check_index_state(layer, orc, w, full=True)
    stats = Stats()
    for t in range(first_step, first_step + steps):
        inp = synth.gen_step(w, seed, t, layer.slices)
        if q_fn is not None:
            inp = replace(inp, q=q_fn(t, inp.q))
        q, kn, vn = inp.q.to(dev), inp.k_new.to(dev), inp.v_new.to(dev)
        cscale = layer.idx.cscale.clone()  # the scales the step scores with (its update changes them)
        dense = None
        if windows > 1:
            dec.step(q, kn, vn)
        else:
            dec.retrieve(q)
            dec.attend(q)
            if check_dense:
                dense = torch.empty_like(buf.out)
                dec.dense(q, dense)
            dec.update(kn, vn)
        torch.cuda.synchronize()
        H = snapshot(buf, cscale, layer.idx)
        assert int(layer.idx.status.item()) == 0, f"step {t}: device status {int(layer.idx.status.item())}"
        qn = inp.q.float().numpy()
        kn_host = inp.k_new.float().numpy()
        vn_host = inp.v_new.float().numpy()
        for g in orc.graph_ids:
            r = check_graph(H, g, orc, qn, kn_host, w, stats, f"{w.name} seed={seed} step={t} graph={g}", dense,
                            vn_host)
            if edge_log is not None:
                edge_log[(t, g)] = np.asarray(r.edges, dtype=np.int64)
        orc.append(kn_host, vn_host)
        stats.steps += 1
        done = t + 1 - first_step
        if check_state_every and done % check_state_every == 0:
            check_index_state(layer, orc, w, full=(done == steps))
        if done % 32 == 0:
            log(f"  {w.name}: {done} of {steps} steps checked")
    lens = layer.kv.seq_len.cpu().numpy()
    for b in {st.b for st in orc.g.values()}:
        assert lens[b] == orc.len[b]
    return stats
