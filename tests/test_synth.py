"""The seeded workload generator: determinism and the planted structure."""
import numpy as np
import torch

from community_kv_retrieval_amd import synth


def test_same_seed_same_tensors():
    w = synth.preset("qwen3_8b_32k").replace(n_ctx=4096, n_kv_heads=2, n_q_heads=8)
    a = synth.gen_layer(w, 5)
    b = synth.gen_layer(w, 5)
    for ra, rb in zip(a, b):
        for sa, sb in zip(ra, rb):
            assert torch.equal(sa.k, sb.k) and torch.equal(sa.v, sb.v)
            np.testing.assert_array_equal(sa.part.labels, sb.part.labels)
    sa = synth.gen_step(w, 5, 3, a)
    sb = synth.gen_step(w, 5, 3, b)
    assert torch.equal(sa.q, sb.q) and torch.equal(sa.k_new, sb.k_new)
    c = synth.gen_layer(w, 6)
    assert not torch.equal(a[0][0].k, c[0][0].k)


def test_geometric_partition_shape():
    w = synth.preset("llama31_8b_128k")
    p = synth.gen_partition(w, 3, 0, 0, 1, w.n_ctx)
    assert (p.labels[:4] == -1).all() and (p.labels[4:] >= 0).all()
    sizes = np.bincount(p.labels[4:], minlength=p.n_comm)
    assert sizes.sum() == w.n_ctx - 4
    assert sizes[:-1].min() >= 4 and sizes.max() <= 64 and sizes[-1] >= 1
    assert 15.0 < sizes.mean() < 17.5           # clamped geometric, mean ~16.1
    assert 7300 < p.n_comm < 8900                # ~8140 communities at 128K
    # members are scattered over the context, not contiguous runs
    pos = np.nonzero(p.labels == 0)[0]
    assert pos.max() - pos.min() > 1000


def test_iid_partition_and_fp32_storage():
    w = synth.preset("tiny")
    sl = synth.gen_layer(w, 1)
    s = sl[0][0]
    assert s.k.dtype == torch.float32 and s.k.shape == (1024, 64)
    assert set(np.unique(s.part.labels[4:])) <= set(range(32))
    # keys of one community sit near its centre (noise std 0.3 per dim)
    lab = s.part.labels
    k = s.k.numpy()
    c = int(lab[10])
    dev = k[lab == c] - s.part.centers[c]
    assert abs(dev.std() - 0.3) < 0.03


def test_bf16_keys_are_scaled_mixture():
    w = synth.preset("qwen3_8b_32k").replace(n_ctx=8192, n_kv_heads=1, n_q_heads=4)
    s = synth.gen_layer(w, 2)[0][0]
    assert s.k.dtype == torch.bfloat16
    k = s.k.float().numpy()
    lab = s.part.labels
    dev = k[lab == 3] * np.sqrt(128) - s.part.centers[3]
    assert abs(dev.std() - 0.25) < 0.03


def test_step_queries_follow_targets():
    w = synth.preset("qwen3_8b_32k").replace(n_ctx=4096)
    sl = synth.gen_layer(w, 4, with_kv=False)
    inp = synth.gen_step(w, 4, 0, sl)
    assert inp.q.shape == (1, 32, 128) and inp.k_new.shape == (1, 8, 128)
    q = inp.q.float().numpy()[0]
    for h in range(32):
        c = inp.target[0, h]
        assert np.abs(q[h] - sl[0][h // 4].part.centers[c]).std() < 0.3
    wg = w.replace(mode=synth.GROUP)
    ig = synth.gen_step(wg, 4, 0, sl)
    assert (ig.target[0].reshape(8, 4) == ig.target[0].reshape(8, 4)[:, :1]).all()


def test_mixed_lengths_in_range():
    w = synth.preset("qwen3_8b_stream_36l")
    lens = synth.seq_lengths(w, 9)
    assert len(lens) == 8 and min(lens) >= 16384 and max(lens) <= 131072
    assert len(set(lens)) > 1
