"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Sizes span several kernel tiles (score tiles of 256 communities, gather
blocks of 128 tokens, select blocks of 1024 threads) with ragged tails, plus
the edge cases of the method: budget 0 (sinks only), a budget that takes
every community (equals dense attention), fewer candidates than kappa, a
community cap, empty communities, a full tail, page sizes 1..64, fp32 and
bf16 storage at d = 64 and 128, one and several query heads per graph.
"""
import numpy as np
import pytest
import torch

from community_kv_retrieval_amd import ckv, runner, synth
from tests import parity as PY

pytestmark = pytest.mark.gpu


def small_per_head(**kw):
    base = dict(name="small_per_head", n_ctx=9000, budget=600, steps=6)
    base.update(kw)
    return synth.preset("qwen3_8b_32k").replace(**base)


def small_group(**kw):
    base = dict(name="small_group", batch=3, n_ctx=7000, min_ctx=2500, budget=700, steps=6)
    base.update(kw)
    return synth.preset("llama31_8b_128k_group_b8").replace(**base)


@pytest.mark.parametrize("seed", [1, 2])
def test_tiny_workload_16_steps(seed):
    w = synth.preset("tiny")
    PY.log(f"tiny seed={seed}")
    st = PY.run_steps(w, seed, w.steps, check_dense=True, defer=seed == 1)
    PY.log(f"  near-tie selections {st.near_sel}, edges {st.near_edges}, max abs {st.max_abs:.2e}")
    assert st.steps == 16


def test_small_per_head():
    w = small_per_head()
    PY.log("small per-head")
    st = PY.run_steps(w, 3, w.steps)
    PY.log(f"  graphs {st.graphs} near {st.near_sel}/{st.near_edges} max abs {st.max_abs:.2e}")


def test_small_group_mixed_lengths():
    w = small_group()
    PY.log("small group, mixed lengths")
    st = PY.run_steps(w, 4, w.steps)
    PY.log(f"  graphs {st.graphs} near {st.near_sel}/{st.near_edges} max abs {st.max_abs:.2e}")


@pytest.mark.parametrize("mode", [synth.PER_HEAD, synth.GROUP])
def test_budget_takes_everything_equals_dense(mode):
    w = small_per_head(mode=mode, n_ctx=3000, budget=1 << 20, steps=3)
    PY.log(f"full budget {mode}")
    st = PY.run_steps(w, 5, w.steps, check_dense=True)
    assert st.dense_equal == st.graphs


@pytest.mark.parametrize("mode", [synth.PER_HEAD, synth.GROUP])
def test_budget_zero_sinks_only(mode):
    w = small_per_head(mode=mode, n_ctx=2000, budget=0, steps=3)
    PY.log(f"budget 0 {mode}")
    PY.run_steps(w, 6, w.steps)


def test_fewer_candidates_than_kappa():
    w = small_per_head(n_ctx=2000, budget=12, kappa=32, steps=3)
    PY.log("budget 12, kappa 32")
    PY.run_steps(w, 7, w.steps)


@pytest.mark.parametrize("n_ctx,budget", [(14000, 9000), (40000, 1 << 20)])
def test_long_token_lists(n_ctx, budget):
    # more member slots than the select kernel maps in LDS, and (second case)
    # more taken communities than it stages: the fallback copies
    w = small_per_head(n_ctx=n_ctx, budget=budget, n_kv_heads=2, n_q_heads=8, steps=2)
    PY.log(f"long token lists n={n_ctx} budget={budget}")
    PY.run_steps(w, 18, w.steps, check_dense=budget > n_ctx)


@pytest.mark.parametrize("mode", [synth.PER_HEAD, synth.GROUP])
@pytest.mark.parametrize("budget", [2500, 4200])
def test_selection_beyond_the_candidates(mode, budget):
    """Budgets near half of a 9000-token context: about half of every group of
    64 communities bears on the cut, more than the 15 candidates the scoring
    kernel keeps per group, so the selection falls back from the candidates to
    every community (with the cut still inside the walk: the L walk overflows);
    a budget of 2500 mixes groups that fit in their candidates and groups
    that do not."""
    w = small_per_head(mode=mode, n_ctx=9000, budget=budget, steps=3)
    PY.log(f"selection beyond the candidates {mode} budget {budget}")
    PY.run_steps(w, 9, w.steps)


@pytest.mark.parametrize("budget,mean_size,max_size", [(30000, 6, 24), (8000, 5, 20)])
def test_long_band(budget, mean_size, max_size):
    """About 10 000 small communities over 60 000 tokens: more than 512
    communities' screening intervals hold the score where the walk stops (a
    lower bound of the band, counted on the host), so the selection cuts a band
    of hundreds of members through its score bins, with crowded cut bins left
    to the radix select."""
    w = small_per_head(n_ctx=60000, n_q_heads=8, n_kv_heads=2, budget=budget, mean_size=mean_size, min_size=1,
                       max_size=max_size, steps=2)
    PY.log(f"long band: budget {budget}, mean community size {mean_size}")
    stats = PY.run_steps(w, 19, w.steps)
    assert stats.band_min > 512, f"band lower bound {stats.band_min}: the long-band cut was not reached"


def test_community_cap():
    w = small_per_head(n_ctx=3000, budget=1 << 20, max_comm=5, steps=3)
    PY.log("max_comm 5")
    PY.run_steps(w, 8, w.steps)


@pytest.mark.parametrize("seed", range(16))
def test_random_configuration(seed):
    """Seeded random mixes of the shape parameters, a few steps each against
    the oracle: graph mode, storage dtype, head dim, batch with ragged lengths,
    group size (one, two, four or eight heads per kv head), budget, kappa,
    sinks, community sizes and page size."""
    r = np.random.default_rng(1000 + seed)
    mode = [synth.PER_HEAD, synth.GROUP][int(r.integers(2))]
    dtype = ["bf16", "f32"][int(r.integers(2))]
    d = [64, 128][int(r.integers(2))]
    hkv, grp = int(r.choice([1, 2, 4])), int(r.choice([1, 2, 4, 8]))
    batch, n_ctx = int(r.integers(1, 4)), int(r.integers(600, 5000))
    w = synth.preset("qwen3_8b_32k").replace(
        name=f"random{seed}", batch=batch, n_q_heads=hkv * grp, n_kv_heads=hkv, head_dim=d, dtype=dtype,
        n_ctx=n_ctx, min_ctx=int(r.integers(0, n_ctx // 2)), n_sinks=int(r.integers(0, 9)), mode=mode,
        budget=int(r.integers(1, n_ctx)), kappa=int(r.integers(1, 33)), key_scale=1.0 / np.sqrt(d),
        mean_size=int(r.integers(4, 33)), min_size=1, max_size=64, steps=3)
    page_size = int(r.choice([1, 4, 16, 64]))
    PY.log(f"random {seed}: {mode} {dtype} d={d} batch={batch} kv_heads={hkv} group={grp} ctx={n_ctx} "
           f"budget={w.budget} kappa={w.kappa} sinks={w.n_sinks} mean_size={w.mean_size} page={page_size}")
    PY.run_steps(w, 50 + seed, w.steps, layer_kw={"page_size": page_size})


def test_max_community_capacity():
    """c_cap at its maximum (16384) over about 550 communities: the selection's
    four-slab path, and scoring tiles that lie wholly past the community count."""
    w = small_per_head(n_ctx=9000, steps=3)
    PY.log("c_cap 16384")
    PY.run_steps(w, 33, w.steps, layer_kw={"c_cap": ckv.CKV_MAX_C_CAP})


@pytest.mark.parametrize("n_ctx,c_cap,budget,max_comm,d,mode", [
    (18000, 4352, 600, 0, 128, synth.PER_HEAD),    # one slab of 4096 and one column of 1024
    (18000, 4352, 600, 0, 64, synth.GROUP),        # the same, d = 64, query groups
    (35500, 8448, 600, 0, 128, synth.PER_HEAD),    # two slabs and a column: the 128K capacity
    (35500, 8448, 600, 40, 128, synth.PER_HEAD),   # the same, exact scores of every community
    (35500, 8448, 20000, 0, 128, synth.PER_HEAD),  # more taken communities than the LDS copy holds
    (35500, 8448, 1200, 0, 64, synth.GROUP),       # two slabs and a column, d = 64, query groups
    (52800, 12544, 900, 0, 64, synth.PER_HEAD),    # three slabs and a column, d = 64
])
def test_selection_column_past_the_slabs(n_ctx, c_cap, budget, max_comm, d, mode):
    """Capacities just past a whole number of slabs of 4096 communities take
    one column of 1024 more per selection block instead of another slab; the
    community counts here reach into that column."""
    w = small_per_head(n_ctx=n_ctx, budget=budget, max_comm=max_comm, mean_size=4, min_size=2, n_kv_heads=2,
                       n_q_heads=4, head_dim=d, key_scale=1.0 / np.sqrt(d), mode=mode, steps=3)
    layer, orc = PY.make_pair(w, 41, w.steps)
    n_comm = synth.graph_n_comm(w, layer.slices)
    assert layer.idx.c_cap == c_cap, layer.idx.c_cap
    assert max(n_comm) > (c_cap // 4096) * 4096, n_comm
    PY.log(f"c_cap {c_cap} n_comm {min(n_comm)}..{max(n_comm)} budget {budget} max_comm {max_comm} d {d} {mode}")
    PY.run_steps(w, 41, w.steps, pair=(layer, orc))


@pytest.mark.parametrize("mode,n_ctx,mean_size", [(synth.PER_HEAD, 3000, 16), (synth.GROUP, 3000, 16),
                                                  (synth.PER_HEAD, 18000, 4)])
def test_zero_query_ties_break_by_id(mode, n_ctx, mean_size):
    """A zero query scores every non-empty community exactly 0, so the
    screening range is empty and the selection computes every exact score:
    the budget then takes the lowest ids, attention is uniform over the
    attended set, and the edges are its lowest non-sink positions.  Every
    decision is an exact tie broken the one documented way, so nothing may
    differ from the oracle, not even inside the tie window.  The last case
    has a community count past one slab of 4096."""
    w = small_per_head(mode=mode, n_ctx=n_ctx, mean_size=mean_size, min_size=2, n_kv_heads=2, n_q_heads=4, steps=3)
    PY.log(f"zero query {mode} n_ctx={n_ctx}")
    st = PY.run_steps(w, 42, w.steps, q_fn=lambda t, q: torch.zeros_like(q))
    assert st.near_sel == 0 and st.near_edges == 0, (st.near_sel, st.near_edges)


@pytest.mark.parametrize("mode", [synth.PER_HEAD, synth.GROUP])
def test_peaked_softmax(mode):
    """Keys scaled 4x: the logits span hundreds, so all but a few tokens'
    probabilities underflow float32.  The running (max, sum) rescaling and the
    split-K combine must stay finite and exact to the tolerance, and the group
    edge weights (sums of probabilities) meet many exact zeros, whose order is
    the position tie-break."""
    w = small_per_head(mode=mode, n_ctx=3000, key_scale=4.0, steps=3)
    PY.log(f"peaked softmax {mode}")
    st = PY.run_steps(w, 43, w.steps)
    PY.log(f"  near-tie selections {st.near_sel}, edges {st.near_edges}, max abs {st.max_abs:.2e}")


def test_largest_kappa():
    """kappa at its maximum (32) with a budget of many communities."""
    w = small_per_head(n_ctx=9000, budget=1500, kappa=32, steps=4)
    PY.log("kappa 32")
    PY.run_steps(w, 34, w.steps)


@pytest.mark.parametrize("dtype,d", [("f32", 128), ("bf16", 64), ("f32", 64)])
def test_dtypes_and_head_dims(dtype, d):
    w = small_group(dtype=dtype, head_dim=d, key_scale=1.0 / np.sqrt(d), batch=2, n_ctx=3000, min_ctx=0, steps=3)
    PY.log(f"{dtype} d={d}")
    PY.run_steps(w, 9, w.steps)


@pytest.mark.parametrize("page_size", [1, 64])
def test_page_sizes(page_size):
    w = small_per_head(n_ctx=2500, steps=3)
    PY.log(f"page size {page_size}")
    PY.run_steps(w, 10, w.steps, layer_kw=dict(page_size=page_size))


def test_group_of_two_and_eight():
    for hq, hkv in ((16, 8), (32, 4)):
        w = small_group(n_q_heads=hq, n_kv_heads=hkv, batch=2, n_ctx=3000, min_ctx=0, steps=2)
        PY.log(f"group {hq // hkv}")
        PY.run_steps(w, 11, w.steps)


def test_empty_communities_never_selected():
    w = small_per_head(n_ctx=3000, n_kv_heads=2, n_q_heads=8, steps=3)
    sl = synth.gen_layer(w, 12)
    for row in sl:
        for s in row:  # spread ids over twice the range: every odd id is empty
            lab = s.part.labels
            lab[lab >= 0] *= 2
            s.part.n_comm = 2 * s.part.n_comm
            s.part.centers = np.repeat(s.part.centers, 2, axis=0)
    PY.log("empty communities")
    layer, orc = PY.make_pair(w, 12, 3, slices=sl)
    PY.run_steps(w, 12, 3, pair=(layer, orc))
    sel = layer.dec.buf.sel.cpu().numpy()
    for g in range(w.n_graphs):
        assert (sel[g, :layer.dec.buf.sel_n[g].item()] % 2 == 0).all()


def test_tail_full_sets_status():
    w = small_per_head(n_ctx=2000, n_kv_heads=1, n_q_heads=4, steps=3)
    PY.log("tail full")
    layer = runner.load_layer(w, 13, extra=4, tail_cap=1)
    dec = layer.dec
    for t in range(2):
        inp = synth.gen_step(w, 13, t, layer.slices)
        dec.step(inp.q.cuda(), inp.k_new.cuda(), inp.v_new.cuda())
    torch.cuda.synchronize()
    assert int(layer.idx.status.item()) & ckv.CKV_ST_TAIL_FULL
    assert (layer.idx.tail_len.cpu().numpy() == 1).all()
    assert layer.kv.seq_len.item() == 2002
    lab = layer.idx.label.cpu().numpy()
    assert (lab[:, 2000] >= 0).all() and (lab[:, 2001] == -1).all()


def test_bad_label_sets_status():
    w = small_per_head(n_ctx=1000, n_kv_heads=1, n_q_heads=4, steps=1)
    sl = synth.gen_layer(w, 14)
    sl[0][0].part.labels[10] = sl[0][0].part.n_comm + 3
    PY.log("bad label")
    layer = runner.load_layer(w, 14, extra=2, slices=sl)
    torch.cuda.synchronize()
    assert int(layer.idx.status.item()) & ckv.CKV_ST_BAD_LABEL
    assert (layer.idx.label[:, 10].cpu().numpy() == -1).all()


def test_deterministic_rerun():
    w = small_group(batch=2, n_ctx=4000, min_ctx=0, steps=4)
    outs = []
    for rep in range(2):
        PY.log(f"determinism rep {rep}")
        layer = runner.load_layer(w, 15, extra=5)
        rec = []
        for t in range(4):
            inp = synth.gen_step(w, 15, t, layer.slices)
            layer.dec.step(inp.q.cuda(), inp.k_new.cuda(), inp.v_new.cuda())
            b = layer.dec.buf
            n = b.tok_n.cpu()
            valid = [b.logits[g, :, :n[g]].cpu().clone() for g in range(n.numel())]
            valid += [b.tok_list[g, :n[g]].cpu().clone() for g in range(n.numel())]
            rec.append([x.cpu().clone() for x in (b.out, b.ml, b.edges, b.assign, b.tok_n)] + valid)
        rec.append([layer.idx.cent.cpu().clone(), layer.idx.csum.cpu().clone()])
        outs.append(rec)
    for a, b in zip(outs[0], outs[1]):
        for x, y in zip(a, b):
            assert torch.equal(x, y)


def test_checkpoint_resume_bit_identical():
    w = small_per_head(n_ctx=3000, n_kv_heads=2, n_q_heads=8, steps=6)
    PY.log("checkpoint/resume")
    ref = runner.load_layer(w, 16, extra=7)
    for t in range(6):
        inp = synth.gen_step(w, 16, t, ref.slices)
        ref.dec.step(inp.q.cuda(), inp.k_new.cuda(), inp.v_new.cuda())
    run = runner.load_layer(w, 16, extra=7)
    for t in range(3):
        inp = synth.gen_step(w, 16, t, run.slices)
        run.dec.step(inp.q.cuda(), inp.k_new.cuda(), inp.v_new.cuda())
    saved = (run.idx.state_dict(), run.kv.kv.clone(), run.kv.seq_len.clone())
    res = runner.load_layer(w, 16, extra=7)
    res.idx.load_state_dict(saved[0])
    res.kv.kv.copy_(saved[1])
    res.kv.seq_len.copy_(saved[2])
    for t in range(3, 6):
        inp = synth.gen_step(w, 16, t, res.slices)
        res.dec.step(inp.q.cuda(), inp.k_new.cuda(), inp.v_new.cuda())
    torch.cuda.synchronize()
    assert torch.equal(ref.dec.buf.out, res.dec.buf.out)
    for k in ckv.CommunityIndex.STATE:
        assert torch.equal(getattr(ref.idx, k), getattr(res.idx, k)), k


@pytest.mark.gpu
@pytest.mark.parametrize("windows", [2, 3])
def test_windowed_steps_match_oracle(windows):
    PY.log(f"windowed steps, {windows} windows")
    st = PY.run_steps(small_per_head(n_ctx=6000, steps=5), 21, 5, windows=windows)
    assert st.graphs > 0
    st = PY.run_steps(small_group(batch=3, n_ctx=5000, min_ctx=2000, steps=4), 22, 4, windows=windows)
    assert st.graphs > 0


def cached_rows(store):
    """K/V of every cached position (slots past seq_len hold no data)."""
    pt, lens, ps = store.page_table.cpu(), store.seq_len.cpu(), store.kv.shape[2]
    kv = store.kv.cpu()
    out = []
    for b in range(lens.numel()):
        pos = torch.arange(int(lens[b]))
        out.append(kv[pt[b, pos // ps].long(), :, pos % ps])
    return torch.cat(out)


@pytest.mark.gpu
def test_windowed_equals_one_window():
    w = small_per_head(n_ctx=5000, steps=6)
    PY.log("windows 1 / 4 / 5 bit-identical")
    runs = []
    for windows in (1, 4, 5):
        layer = runner.load_layer(w, 23, extra=7)
        layer.dec.set_windows(windows)
        rec = []
        for t in range(6):
            inp = synth.gen_step(w, 23, t, layer.slices)
            layer.dec.step(inp.q.cuda(), inp.k_new.cuda(), inp.v_new.cuda())
            b = layer.dec.buf
            n = b.tok_n.cpu()
            rec += [x.cpu().clone() for x in (b.out, b.ml, b.edges, b.assign, b.tok_n, b.sel_n, b.top)]
            rec += [b.tok_list[g, :n[g]].cpu().clone() for g in range(n.numel())]
            rec += [b.logits[g, :, :n[g]].cpu().clone() for g in range(n.numel())]
        rec += [getattr(layer.idx, k).cpu().clone() for k in ckv.CommunityIndex.STATE]
        rec += [layer.kv.seq_len.cpu().clone(), cached_rows(layer.kv)]
        runs.append(rec)
    for other in runs[1:]:
        for x, y in zip(runs[0], other):
            assert torch.equal(x, y)


@pytest.mark.parametrize("case", ["per_head", "group", "per_head_mid", "per_head_long", "group_windows",
                                  "per_head_windows", "tiny_f32", "per_head_empty"])
def test_deferred_combine_equals_complete(case):
    """A gather whose combine runs in the assign kernel gives the same bits as
    a complete gather followed by the assign: outputs, softmax state, edges,
    assignments and the whole index.  The mid case has more spans per graph
    than the assign preloads (and than a wave has lanes), the long case more
    than the combine stages in LDS (256 spans of 256 tokens); the empty case
    attends nothing (no sinks, no community fits the budget)."""
    if case.startswith("group"):
        w = small_group(batch=2, n_ctx=6000, min_ctx=2000, steps=5)
    elif case == "per_head_mid":
        w = small_per_head(n_ctx=24000, budget=20000, n_kv_heads=2, n_q_heads=4, steps=3)
    elif case == "per_head_long":
        w = small_per_head(n_ctx=80000, budget=70000, n_kv_heads=1, n_q_heads=2, steps=2)
    elif case == "tiny_f32":
        w = synth.preset("tiny").replace(steps=6)
    elif case == "per_head_empty":
        w = small_per_head(n_ctx=3000, n_sinks=0, budget=1, min_size=2, steps=3)
    else:
        w = small_per_head(n_ctx=7000, steps=5)
    windows = 3 if case.endswith("windows") else 1
    PY.log(f"deferred combine vs complete gather: {case}")
    runs = []
    for defer in (False, True):
        layer = runner.load_layer(w, 29, extra=w.steps + 1)
        layer.dec.defer = defer
        layer.dec.set_windows(windows)
        rec = []
        for t in range(w.steps):
            inp = synth.gen_step(w, 29, t, layer.slices)
            layer.dec.step(inp.q.cuda(), inp.k_new.cuda(), inp.v_new.cuda())
            b = layer.dec.buf
            n = b.tok_n.cpu()
            rec += [x.cpu().clone() for x in (b.out, b.ml, b.edges, b.assign, b.tok_n)]
            rec += [b.logits[g, :, :n[g]].cpu().clone() for g in range(n.numel())]
        rec += [getattr(layer.idx, k).cpu().clone() for k in ckv.CommunityIndex.STATE]
        rec += [layer.kv.seq_len.cpu().clone(), cached_rows(layer.kv)]
        assert int(layer.idx.status.item()) == 0
        runs.append(rec)
    if case == "per_head_mid":
        assert int(n.max()) > 64 * 256
    if case == "per_head_long":
        assert int(n.max()) > 256 * 256, "the long case must exceed the staged span count"
    if case == "per_head_empty":
        assert int(n.max()) == 0
    for x, y in zip(*runs):
        assert torch.equal(x, y)


def test_nothing_attended():
    """No sinks and no community small enough for the budget: every token list
    is empty; the output is zero and each new token joins the best community."""
    w = small_per_head(n_ctx=3000, n_sinks=0, budget=1, min_size=2, steps=3)
    PY.log("empty token lists")
    PY.run_steps(w, 31, w.steps)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_read_rows_checksum(dtype, d):
    """The read-ceiling kernel reads every byte of the rows it is given: its
    per-block XOR of the rows' 32-bit words equals the host's, including a
    ragged last block and row ids past the store (clamped to its last row)."""
    w = small_per_head(dtype=dtype, head_dim=d, key_scale=1.0 / np.sqrt(d), n_ctx=3000, steps=1)
    PY.log(f"read rows {dtype} d={d}")
    kv = runner.load_layer(w, 41, extra=2).kv
    n_rows = kv.n_pages * kv.n_kv_heads * kv.page_size
    n = 256 * 7 + 77
    rows = torch.randint(0, n_rows, (n,), generator=torch.Generator().manual_seed(5), dtype=torch.int32)
    rows[:3] = torch.tensor([n_rows - 1, n_rows + 5, 2**31 - 1], dtype=torch.int32)
    part = torch.zeros(((n + 255) // 256,), dtype=torch.int32, device="cuda")
    ckv.ckv_read_rows(kv, rows.cuda(), part)
    torch.cuda.synchronize()
    words = kv.kv.view(torch.int32).reshape(n_rows, -1).cpu().numpy()
    r = np.minimum(rows.numpy().astype(np.int64), n_rows - 1)
    ref = np.array([np.bitwise_xor.reduce(words[r[i:i + 256]].ravel()) for i in range(0, n, 256)], dtype=np.int32)
    np.testing.assert_array_equal(part.cpu().numpy(), ref)


def test_dense_baseline_matches_oracle():
    w = synth.preset("qwen3_8b_32k").replace(n_ctx=20000, batch=2, min_ctx=9000)
    PY.log("dense baseline")
    layer, orc = PY.make_pair(w, 17, 1)
    inp = synth.gen_step(w, 17, 0, layer.slices)
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    layer.dec.dense(inp.q.cuda(), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b in range(w.batch):
        for kh in range(w.n_kv_heads):
            ref = orc.dense(inp.q.float().numpy(), b, kh)
            g = got[b, kh * 4:(kh + 1) * 4]
            assert np.all(np.abs(g - ref) <= PY.ATOL + PY.RTOL * np.abs(ref))


@pytest.mark.gpu
@pytest.mark.parametrize("group", [False, True])
def test_attention_mass_recall_matches_oracle(group):
    """The share of dense attention mass the attended tokens carry, from the
    kernels' (max, sum) outputs, against the oracle's definition."""
    w = small_group(batch=2, n_ctx=5000, min_ctx=2000, steps=3) if group else small_per_head(n_ctx=6000, steps=3)
    PY.log(f"recall group={group}")
    layer, orc = PY.make_pair(w, 31, 3)
    dec, buf = layer.dec, layer.dec.buf
    dec.defer = False  # ml is read before the update
    dml = torch.empty((w.batch, w.n_q_heads, 2), dtype=torch.float32, device="cuda")
    dout = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    for t in range(3):
        inp = synth.gen_step(w, 31, t, layer.slices)
        q = inp.q.cuda()
        dec.retrieve(q)
        dec.attend(q)
        dec.dense(q, dout, ml=dml)
        rec = dec.recall(dml).cpu().numpy()
        tl, tn = buf.tok_list.cpu().numpy(), buf.tok_n.cpu().numpy()
        qn = inp.q.float().numpy()
        for g in orc.graph_ids:
            ref = orc.recall(g, qn, np.sort(tl[g, :tn[g]]))
            np.testing.assert_allclose(rec[g], ref, rtol=1e-4, atol=1e-7, err_msg=f"step {t} graph {g}")
            assert np.all(rec[g] <= 1 + 1e-5) and np.all(rec[g] > 0)
        dec.update(inp.k_new.cuda(), inp.v_new.cuda())
        torch.cuda.synchronize()
        orc.append(inp.k_new.float().numpy(), inp.v_new.float().numpy())


# ---------------------------------------------------------------------------
# Centroid budget (Table 6): the step also attends the centroids of the
# next-ranked communities after the selection, each as one softmax term.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode", [synth.PER_HEAD, synth.GROUP])
@pytest.mark.parametrize("cent_budget,defer", [(4, True), (64, False), (256, True)])
def test_centroid_budget(mode, cent_budget, defer):
    """The centroid communities (a tie-consistent continuation of the ranking
    past the selection), the attention output over tokens and centroid terms,
    the softmax state, the edges and the value sums, every step; complete and
    deferred gathers, per-head and query-group (matrix-core) gathers.  The
    queries are scaled by 0.3, which flattens the softmax so that the centroid
    terms move every graph's output by many times the output tolerance (the
    harness counts the graphs where they do)."""
    w = small_per_head(mode=mode, n_ctx=9000, budget=600, steps=4, cent_budget=cent_budget)
    PY.log(f"centroid budget {cent_budget} {mode} defer={defer}")
    st = PY.run_steps(w, 21, w.steps, defer=defer, q_fn=lambda t, q: q * 0.3)
    PY.log(f"  centroid terms {st.cent_terms}, near-tie sets {st.near_cent}, visible in {st.cent_visible} "
           f"of {st.graphs} graphs, max abs {st.max_abs:.2e}")
    assert st.cent_terms >= st.graphs * cent_budget
    assert st.cent_visible >= st.graphs // 2, (st.cent_visible, st.graphs)


@pytest.mark.parametrize("mode", [synth.PER_HEAD, synth.GROUP])
def test_centroid_terms_only(mode):
    """No sinks and a zero budget: the token list is empty and the centroid
    terms are the whole attention (complete and deferred gathers)."""
    for defer in (False, True):
        w = small_per_head(mode=mode, n_ctx=2000, budget=0, n_sinks=0, steps=2, cent_budget=16)
        PY.log(f"centroid terms only {mode} defer={defer}")
        st = PY.run_steps(w, 22, w.steps, defer=defer)
        assert st.cent_terms == st.graphs * 16


def test_centroid_budget_past_the_communities():
    """A budget larger than the communities the selection leaves: every one of
    them is attended as a centroid term."""
    w = small_per_head(n_ctx=1500, budget=300, steps=3, cent_budget=256)
    PY.log("centroid budget past the communities")
    PY.run_steps(w, 23, w.steps)


def test_centroid_budget_long_lists_and_windows():
    """Token lists of more spans than the assign kernel preloads (its
    deferred combine reads the centroid record after 36 span records), and the
    windowed multi-stream step."""
    w = small_per_head(n_ctx=14000, budget=9000, n_kv_heads=2, n_q_heads=8, steps=2, cent_budget=64)
    PY.log("centroid budget, long lists")
    PY.run_steps(w, 24, w.steps)
    w = small_group(steps=3, cent_budget=16)
    PY.log("centroid budget, two windows")
    PY.run_steps(w, 25, w.steps, windows=2)


@pytest.mark.parametrize("n_ctx,mean_size", [(3000, 16), (40000, 8)])
def test_centroid_budget_zero_query(n_ctx, mean_size):
    """A zero query ties every community at score 0: the centroid communities
    are the lowest ids past the selection, decided without any tie window.
    The second case leaves more than 2048 outsiders within the screening
    range, so the centroid selection computes every exact score."""
    w = small_per_head(n_ctx=n_ctx, mean_size=mean_size, min_size=2, n_kv_heads=2, n_q_heads=4, steps=2,
                       cent_budget=256)
    PY.log(f"centroid budget, zero query, n_ctx={n_ctx}")
    st = PY.run_steps(w, 26, w.steps, q_fn=lambda t, q: torch.zeros_like(q))
    assert st.near_sel == 0 and st.near_cent == 0 and st.near_edges == 0


@pytest.mark.parametrize("budget", [5000, 1 << 20])
def test_large_communities(budget):
    """Communities of 2500 to 9000 members, more than the 2048 the index
    build sorts in LDS: the build lists them by its ordered pass over the
    labels.  The CSR (ascending members), the key sums and the centroids are
    checked bit-exact after the build, then the steps as usual (the full
    budget takes every community: equal to dense attention)."""
    w = small_per_head(n_ctx=30000, mean_size=5000, min_size=2500, max_size=9000, n_kv_heads=2, n_q_heads=4,
                       steps=2, budget=budget)
    layer, orc = PY.make_pair(w, 61, w.steps)
    sizes = [int(st.counts.max()) for st in orc.g.values()]
    assert min(sizes) > 2048, sizes
    PY.log(f"large communities: largest per graph {sizes}, budget {budget}")
    PY.run_steps(w, 61, w.steps, pair=(layer, orc), check_dense=budget > w.n_ctx)
