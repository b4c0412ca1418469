"""Prefill graph construction (the CommunityKV page, Figure 1 panel (1)) on
the GPU against the oracle: every query position's top-kappa edges and their
weights, per head and per query group.

Edge rows are compared exactly.  A differing row is accepted only as a near
tie under tests/decisions.prefill_row_ok: the right number of edges, each a
pool key, in a rank order and with a set that a ranking within the window
(relative to the oracle's kappa-th weight) yields; the float32 logits of the
matrix cores differ from the float64 ones by about d * 2^-24 * sum|q k| (up
to ~1e-4 relative in the weight at these magnitudes).
"""
import numpy as np
import pytest
import torch

from community_kv_retrieval_amd import ckv, synth
from oracle import ckv_oracle as O
from tests import decisions as D
from tests import parity as PY

pytestmark = pytest.mark.gpu


def _layer(w, seed):
    slices = synth.gen_layer(w, seed)
    lens = [int(slices[b][0].part.labels.shape[0]) for b in range(w.batch)]
    kv = ckv.KVStore(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.torch_dtype, max(lens) + 1, 16, "cuda",
                     shuffle_pages=True, seed=seed + 77, seq_len=lens)
    for b in range(w.batch):
        for kh in range(w.n_kv_heads):
            ckv.ckv_kv_write(kv, b, kh, 0, slices[b][kh].k.cuda(), slices[b][kh].v.cuda())
    return kv, slices, lens


def _run(kv, mode, b, q, n_sinks, kappa, sm_scale, with_w=True):
    graphs = kv.n_q_heads if mode == ckv.CKV_MODE_PER_HEAD else kv.n_kv_heads
    n = q.shape[0]
    edges = torch.full((graphs, n, kappa), -7, dtype=torch.int32, device="cuda")
    weights = torch.full((graphs, n, kappa), -7.0, dtype=torch.float32, device="cuda") if with_w else None
    ws = ckv.prefill_workspace(kv, mode, n)
    ckv.ckv_prefill_topk(kv, mode, b, q.cuda(), n_sinks, kappa, sm_scale, edges, weights, ws)
    torch.cuda.synchronize()
    return edges.cpu().numpy(), (weights.cpu().numpy() if with_w else None)


def _heads(w, mode, g):
    G = w.n_q_heads // w.n_kv_heads
    return [g] if mode == ckv.CKV_MODE_PER_HEAD else list(range(g * G, (g + 1) * G))


def _kv_head(w, mode, g):
    return g // (w.n_q_heads // w.n_kv_heads) if mode == ckv.CKV_MODE_PER_HEAD else g


def _check_rows(ge, gw, re_, rw, rows, qh, keys, n_sinks, sm_scale, where, stats):
    """ge/gw: device edges/weights of the rows; re_/rw: the oracle's.  Rows
    equal to the oracle's only need their weights checked (against the
    oracle's weights of the same edges); any other row is judged by
    decisions.prefill_row_ok on the oracle's weights of every key."""
    kappa = re_.shape[1]
    for r, i in enumerate(rows):
        if (ge[r] == re_[r]).all():
            k = int((re_[r] >= 0).sum())
            if gw is not None:
                assert (gw[r, k:] == 0).all(), f"{where} row {i}: padding weight"
                np.testing.assert_allclose(gw[r, :k], rw[r, :k], rtol=D.PREFILL_WRT, atol=D.PREFILL_WAT,
                                           err_msg=f"{where} row {i}")
            continue
        W = O.prefill_row_weights(qh[r], i, keys, sm_scale)
        D.prefill_row_ok(W, i, n_sinks, kappa, re_[r], ge[r], None if gw is None else gw[r], where)
        stats["near"] += 1


def _compare_all(w, kv, slices, b, q, mode, n_sinks, kappa, sm_scale, with_w=True, graphs=None):
    e, wt = _run(kv, mode, b, q, n_sinks, kappa, sm_scale, with_w)
    qf = q.float().numpy().astype(np.float64)
    n = q.shape[0]
    stats = {"near": 0}
    all_g = range(kv.n_q_heads if mode == ckv.CKV_MODE_PER_HEAD else kv.n_kv_heads)
    for g in (all_g if graphs is None else graphs):
        keys = slices[b][_kv_head(w, mode, g)].k[:n].float().numpy().astype(np.float64)
        qh = qf[:, _heads(w, mode, g)]
        re_, rw = O.prefill_edges(qh, keys, n_sinks, kappa, sm_scale)
        _check_rows(e[g], None if wt is None else wt[g], re_, rw, range(n), qh, keys, n_sinks, sm_scale,
                    f"mode={mode} g={g} kappa={kappa}", stats)
    PY.log(f"  prefill mode={mode} n={n} kappa={kappa}: near ties {stats['near']}")
    return stats


def _small(**kw):
    base = dict(name="prefill_small", batch=2, n_ctx=1500, min_ctx=0, n_q_heads=8, n_kv_heads=2)
    base.update(kw)
    return synth.preset("qwen3_8b_32k").replace(**base)


@pytest.mark.parametrize("kappa,with_w", [(8, True), (8, False), (16, True), (32, True), (3, True)])
def test_prefill_per_head_matches_oracle(kappa, with_w):
    w = _small()
    kv, slices, lens = _layer(w, 41)
    q = synth.gen_prefill_queries(w, 41, 0, 1, slices[1])
    PY.log(f"prefill per head kappa={kappa} weights={with_w}")
    _compare_all(w, kv, slices, 1, q, ckv.CKV_MODE_PER_HEAD, w.n_sinks, kappa, w.sm_scale, with_w)


@pytest.mark.parametrize("kappa", [8, 16, 5])
def test_prefill_group_matches_oracle(kappa):
    w = _small(n_ctx=1300)
    kv, slices, lens = _layer(w, 42)
    q = synth.gen_prefill_queries(w, 42, 0, 0, slices[0])
    PY.log(f"prefill group kappa={kappa}")
    _compare_all(w, kv, slices, 0, q, ckv.CKV_MODE_QUERY_GROUP, w.n_sinks, kappa, w.sm_scale)


@pytest.mark.parametrize("d,group", [(64, False), (64, True)])
def test_prefill_head_dim_64(d, group):
    w = _small(head_dim=d, n_ctx=900, key_scale=1.0 / np.sqrt(d))
    kv, slices, lens = _layer(w, 43)
    q = synth.gen_prefill_queries(w, 43, 0, 1, slices[1])
    PY.log(f"prefill d={d} group={group}")
    _compare_all(w, kv, slices, 1, q, ckv.CKV_MODE_QUERY_GROUP if group else ckv.CKV_MODE_PER_HEAD,
                 w.n_sinks, 8, w.sm_scale)


@pytest.mark.parametrize("n,n_sinks", [(1, 4), (5, 4), (33, 0), (65, 4), (129, 40)])
def test_prefill_short_prompts_and_sinks(n, n_sinks):
    # fewer candidates than kappa, a prompt shorter than one tile, no sinks,
    # more sinks than a tile: rows with nothing to link are all -1
    w = _small(n_ctx=200)
    kv, slices, lens = _layer(w, 44)
    q = synth.gen_prefill_queries(w, 44, 0, 0, slices[0], n=n)
    for mode in (ckv.CKV_MODE_PER_HEAD, ckv.CKV_MODE_QUERY_GROUP):
        _compare_all(w, kv, slices, 0, q, mode, n_sinks, 8, w.sm_scale)


def test_prefill_scale_and_sequence_rows():
    # another sm_scale, and the prompt of the second sequence read through its
    # own page-table row: the result must not depend on the first
    w = _small(n_ctx=700)
    kv, slices, lens = _layer(w, 45)
    q = synth.gen_prefill_queries(w, 45, 0, 1, slices[1])
    _compare_all(w, kv, slices, 1, q, ckv.CKV_MODE_PER_HEAD, w.n_sinks, 8, 0.37)


@pytest.mark.parametrize("mode", [ckv.CKV_MODE_PER_HEAD, ckv.CKV_MODE_QUERY_GROUP])
def test_prefill_32k_sampled_rows(mode):
    # the full 32K prompt of the Qwen3-8B-shaped layer, every graph computed on
    # the device; sampled rows of sampled graphs against the oracle
    w = synth.preset("qwen3_8b_32k")
    kv, slices, lens = _layer(w, 46)
    n = lens[0]
    q = synth.gen_prefill_queries(w, 46, 0, 0, slices[0])
    PY.log(f"prefill 32K mode={mode}")
    e, wt = _run(kv, mode, 0, q, w.n_sinks, w.kappa, w.sm_scale)
    rng = np.random.default_rng(7)
    rows = sorted(set([0, 3, 4, 5, 31, 32, 63, 64, 127, 128, 4095, 4096, n // 2, n - 2, n - 1] +
                      rng.integers(0, n, size=12).tolist()))
    qf = q.float().numpy().astype(np.float64)
    graphs = [0, 13, 31] if mode == ckv.CKV_MODE_PER_HEAD else [0, 5, 7]
    stats = {"near": 0}
    for g in graphs:
        keys = slices[0][_kv_head(w, mode, g)].k.float().numpy().astype(np.float64)
        qh = qf[rows][:, _heads(w, mode, g)]
        re_, rw = O.prefill_edges_rows(qh, rows, keys, w.n_sinks, w.kappa, w.sm_scale)
        _check_rows(e[g][rows], wt[g][rows], re_, rw, rows, qh, keys, w.n_sinks, w.sm_scale,
                    f"32K mode={mode} g={g}", stats)
    # every row of every graph: structurally valid
    graphs_all = e.shape[0]
    pos = np.arange(n)[None, :, None]
    valid = e >= 0
    assert ((~valid) | ((e >= w.n_sinks) & (e < pos))).all()
    assert (np.diff(valid.astype(np.int8), axis=2) <= 0).all()  # padding only at the end
    assert ((wt >= 0) & (wt <= (1 if mode == ckv.CKV_MODE_PER_HEAD else 4) + 1e-5)).all()
    assert (np.diff(np.where(valid, wt, -1.0), axis=2) <= 1e-7).all()  # rank order
    PY.log(f"  32K mode={mode}: graphs {graphs_all}, near ties {stats['near']}")


@pytest.mark.parametrize("mode", [ckv.CKV_MODE_PER_HEAD, ckv.CKV_MODE_QUERY_GROUP])
def test_prefill_128k_bench_configuration_sampled_rows(mode):
    # the benchmark's prefill leg as it runs: the 128K layer loaded by the
    # runner, queries drawn on the device, every graph computed; sampled rows
    # of sampled graphs against the oracle
    from community_kv_retrieval_amd import runner
    w = synth.preset("llama31_8b_128k")
    slices = synth.gen_layer(w, 1)
    layer = runner.load_layer(w, 1, extra=1, slices=slices)
    n = int(slices[0][0].part.labels.shape[0])
    q = synth.gen_prefill_queries_device(w, 1, 0, 0, [slices[0][kh].part for kh in range(w.n_kv_heads)])
    PY.log(f"prefill 128K bench configuration mode={mode}")
    e, wt = _run(layer.kv, mode, 0, q, w.n_sinks, w.kappa, w.sm_scale)
    rng = np.random.default_rng(9)
    rows = sorted(set([4, 5, 63, 64, 65536, n - 1] + rng.integers(0, n, size=8).tolist()))
    qh_all = q[rows].float().cpu().numpy().astype(np.float64)
    graphs = [0, 17, 31] if mode == ckv.CKV_MODE_PER_HEAD else [0, 6]
    stats = {"near": 0}
    for g in graphs:
        keys = slices[0][_kv_head(w, mode, g)].k.float().numpy().astype(np.float64)
        qh = qh_all[:, _heads(w, mode, g)]
        re_, rw = O.prefill_edges_rows(qh, rows, keys, w.n_sinks, w.kappa, w.sm_scale)
        _check_rows(e[g][rows], wt[g][rows], re_, rw, rows, qh, keys, w.n_sinks, w.sm_scale,
                    f"128K mode={mode} g={g}", stats)
    PY.log(f"  128K mode={mode}: near ties {stats['near']}")


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 4), (16, 2)])
def test_prefill_per_head_group_sizes(hq, hkv):
    # one, two and eight query heads per kv head: blocks then hold four query
    # tiles of one head, two tiles of two heads, or half a group
    w = _small(n_q_heads=hq, n_kv_heads=hkv, n_ctx=777)
    kv, slices, lens = _layer(w, 47)
    q = synth.gen_prefill_queries(w, 47, 0, 1, slices[1])
    PY.log(f"prefill per head {hq}/{hkv}")
    _compare_all(w, kv, slices, 1, q, ckv.CKV_MODE_PER_HEAD, w.n_sinks, 8, w.sm_scale)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 4)])
def test_prefill_group_sizes(hq, hkv):
    w = _small(n_q_heads=hq, n_kv_heads=hkv, n_ctx=650)
    kv, slices, lens = _layer(w, 48)
    q = synth.gen_prefill_queries(w, 48, 0, 0, slices[0])
    PY.log(f"prefill group {hq}/{hkv}")
    _compare_all(w, kv, slices, 0, q, ckv.CKV_MODE_QUERY_GROUP, w.n_sinks, 8, w.sm_scale)


def test_prefill_group_of_eight_is_unsupported():
    w = _small(n_q_heads=16, n_kv_heads=2, n_ctx=100)
    kv, slices, lens = _layer(w, 49)
    q = synth.gen_prefill_queries(w, 49, 0, 0, slices[0]).cuda()
    edges = torch.empty((2, 100, 8), dtype=torch.int32, device="cuda")
    ws = ckv.prefill_workspace(kv, ckv.CKV_MODE_QUERY_GROUP, 100)
    with pytest.raises(ckv.CkvError):
        ckv.ckv_prefill_topk(kv, ckv.CKV_MODE_QUERY_GROUP, 0, q, 4, 8, 1.0, edges, None, ws)
