"""ckv_gather_attend_noalloc through the C ABI against ckv_gather_attend
(complete mode, caller workspace) on the same token lists: out, ml and every
logit of every graph must be bit-identical (the same kernels run on the
library's static scratch instead of the workspace).  Two calls in a row, the
second on a smaller input (fewer graphs, a shorter list capacity), so the
second call reuses scratch that the first left behind."""
import pytest
import torch

from community_kv_retrieval_amd import ckv, runner, synth
from tests import parity as PY

pytestmark = pytest.mark.gpu


def _compare(w, seed, steps=2):
    layer = runner.load_layer(w, seed, extra=steps + 1)
    dec, buf, kv, idx = layer.dec, layer.dec.buf, layer.kv, layer.idx
    G, nh = idx.n_graphs, idx.heads_per_graph(kv)
    for t in range(steps):
        inp = synth.gen_step(w, seed, t, layer.slices)
        q = inp.q.cuda()
        dec.retrieve(q)
        outs = []
        for noalloc in (False, True):
            out = torch.full_like(buf.out, float("nan"))
            logits = torch.full_like(buf.logits, float("nan"))
            ml = torch.full((G, nh, 2), float("nan"), dtype=torch.float32, device="cuda")
            if noalloc:
                ckv.ckv_gather_attend_noalloc(kv, idx, q, buf.tok_list, buf.tok_n, dec.sm_scale, out, logits, ml)
            else:
                ckv.ckv_gather_attend(kv, idx, q, buf.tok_list, buf.tok_n, dec.sm_scale, out, logits, ml, buf.ws)
            outs.append((out, logits, ml))
        torch.cuda.synchronize()
        (oa, la, ma), (ob, lb, mb) = outs
        assert torch.equal(oa, ob), f"{w.name} step {t}: out differs"
        assert torch.equal(ma, mb), f"{w.name} step {t}: ml differs"
        n = buf.tok_n.cpu()
        for g in range(G):
            assert torch.equal(la[g, :, :n[g]], lb[g, :, :n[g]]), f"{w.name} step {t} graph {g}: logits differ"
        # advance the index so the next step's lists differ
        dec.attend(q)
        dec.update(inp.k_new.cuda(), inp.v_new.cuda())
    torch.cuda.synchronize()
    return G, buf.t_cap


def test_noalloc_gather_matches_workspace_gather_twice():
    big = synth.preset("llama31_8b_128k_group_b8").replace(name="noalloc_big", batch=4, n_ctx=20000,
                                                            min_ctx=9000, budget=3000)
    small = synth.preset("qwen3_8b_32k").replace(name="noalloc_small", n_ctx=3000, n_q_heads=8, n_kv_heads=2,
                                                 budget=500)
    PY.log("noalloc: first call (group, 32 graphs), then a smaller one (per head, 8 graphs)")
    g1, t1 = _compare(big, 61)
    g2, t2 = _compare(small, 62)
    assert g2 < g1 and t2 < t1


def test_noalloc_gather_with_centroid_terms():
    """With a centroid budget both gathers first write the centroid terms'
    records (into the static scratch or the workspace) and combine them after
    the spans: still bit-identical."""
    w = synth.preset("qwen3_8b_32k").replace(name="noalloc_cent", n_ctx=6000, n_q_heads=8, n_kv_heads=2,
                                             budget=600, cent_budget=64)
    PY.log("noalloc with centroid terms (8 graphs, budget 64)")
    _compare(w, 64)


def test_noalloc_rejects_oversized_shape():
    """A shape whose records exceed the static scratch is refused on the host."""
    w = synth.preset("qwen3_8b_32k").replace(name="noalloc_reject", n_ctx=1000, n_q_heads=8, n_kv_heads=2,
                                             budget=200)
    layer = runner.load_layer(w, 63, extra=2)
    kv, idx = layer.kv, layer.idx
    G = idx.n_graphs
    t_cap = 250_000  # 8 graphs x ceil(250000 / 256) spans x 640 bytes: 5.0 MB of records, past 4 MiB
    tok_list = torch.zeros((G, t_cap), dtype=torch.int32, device="cuda")
    tok_n = torch.zeros((G,), dtype=torch.int32, device="cuda")
    logits = torch.zeros((G, 1, t_cap), dtype=torch.float32, device="cuda")
    out = torch.zeros((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    ml = torch.zeros((G, 1, 2), dtype=torch.float32, device="cuda")
    q = torch.zeros((w.batch, w.n_q_heads, w.head_dim), dtype=w.torch_dtype, device="cuda")
    with pytest.raises(ckv.CkvError) as e:
        ckv.ckv_gather_attend_noalloc(kv, idx, q, tok_list, tok_n, w.sm_scale, out, logits, ml)
    assert e.value.code == ckv.CKV_E_WORKSPACE
