"""The C ABI on the host: the library loads, exports every symbol the header
declares, sizes workspaces, and rejects bad arguments before any device call
(so none of these tests needs a GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

from community_kv_retrieval_amd import ckv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ckv.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ckv_[a-z_]+)\s*\(", src)))


def test_header_declares_the_four_step_calls():
    names = _declared()
    for n in ("ckv_score_centroids", "ckv_select_communities", "ckv_gather_attend", "ckv_assign_update"):
        assert n in names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", ckv._LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (ckv_[a-z_]+)\b", out))
    missing = [n for n in _declared() if n not in exported]
    assert not missing, missing
    assert set(ckv.EXPORTS) == set(_declared())


def test_abi_version_and_status_strings():
    assert ckv.LIB.ckv_abi_version() == 11
    for code in (0, -1, -2, -3, -4):
        assert ckv.ckv_status_str(code) != "unknown status"
    assert ckv.ckv_status_str(7) == "unknown status"


FAKE = 0x10000  # never dereferenced: validation fails or succeeds before any device call
BIG = 1 << 40  # a workspace size large enough for any shape here


def _kv(**kw):
    d = dict(kv=FAKE, page_table=FAKE, seq_len=FAKE, batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128,
             page_size=16, max_pages=8200, n_pages=8200, dtype=ckv.CKV_DTYPE_BF16)
    d.update(kw)
    return ckv.CkvKV(**d)


def _idx(**kw):
    d = dict(mode=ckv.CKV_MODE_PER_HEAD, n_graphs=32, c_cap=8192, l_cap=131200, tail_cap=256, n_sinks=4)
    for f in ("n_comm", "size", "offs", "toks", "label", "tail_pos", "tail_comm", "tail_len", "csum", "cent",
              "cq", "cscale", "status"):
        d[f] = FAKE
    d.update(kw)
    return ckv.CkvIndex(**d)


def _ws(kv, idx, t_cap):
    return ckv.LIB.ckv_workspace_bytes(ctypes.byref(kv), ctypes.byref(idx) if idx is not None else None, t_cap)


def test_workspace_bytes():
    kv, idx = _kv(), _idx()
    a = _ws(kv, idx, 4100)
    dense = _ws(kv, None, 0)
    assert 0 < dense < a
    # partials of ceil(4100 / 256) = 17 gather blocks x 32 graphs, each 130 floats padded to 160
    # (whole 128-byte lines), the build cursor and the dense region
    assert a >= dense + 4 * 32 * 17 * 160 + 4 * 32 * 8192
    assert _ws(kv, idx, 8200) > a
    assert _ws(_kv(head_dim=96), idx, 4100) == 0
    assert _ws(kv, _idx(n_graphs=31), 4100) == 0
    assert _ws(kv, idx, -1) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), ckv.CKV_E_UNSUPPORTED),
    (dict(dtype=7), ckv.CKV_E_UNSUPPORTED),
    (dict(n_kv_heads=3), ckv.CKV_E_INVALID),          # 32 % 3 != 0
    (dict(n_q_heads=48, n_kv_heads=3), ckv.CKV_E_UNSUPPORTED),  # group of 16
    (dict(page_size=12), ckv.CKV_E_INVALID),
    (dict(kv=None), ckv.CKV_E_INVALID),
    (dict(seq_len=None), ckv.CKV_E_INVALID),
    (dict(batch=0), ckv.CKV_E_INVALID),
])
def test_kv_validation(kw, code):
    kv, idx = _kv(**kw), _idx()
    r = ckv.LIB.ckv_score_centroids(ctypes.byref(kv), ctypes.byref(idx), FAKE, FAKE, FAKE, BIG, None)
    assert r == code


@pytest.mark.parametrize("kw", [dict(n_graphs=8), dict(c_cap=1000), dict(c_cap=32768), dict(tail_cap=0),
                                dict(tail_cap=5000), dict(n_sinks=-1), dict(mode=3), dict(cent=None),
                                dict(status=None), dict(csum=None), dict(cq=None), dict(cscale=None)])
def test_index_validation(kw):
    kv, idx = _kv(), _idx(**kw)
    assert ckv.LIB.ckv_score_centroids(ctypes.byref(kv), ctypes.byref(idx), FAKE, FAKE, FAKE, BIG, None) == ckv.CKV_E_INVALID


@pytest.mark.parametrize("kw", [dict(cent_budget=-1), dict(cent_budget=257),
                                dict(cent_budget=4),  # arrays missing
                                dict(cent_budget=4, cent_sel=FAKE, cent_n=FAKE),  # no value sums
                                dict(cent_budget=4, cent_sel=FAKE, vsum=FAKE),
                                dict(cent_budget=4, cent_n=FAKE, vsum=FAKE)])
def test_centroid_budget_validation(kw):
    kv, idx = _kv(), _idx(**kw)
    for f in (ckv.LIB.ckv_score_centroids,):
        assert f(ctypes.byref(kv), ctypes.byref(idx), FAKE, FAKE, FAKE, BIG, None) == ckv.CKV_E_INVALID
    assert _ws(kv, idx, 4100) == 0


@pytest.mark.parametrize("budget,slots", [(1, 1), (16, 1), (17, 2), (256, 16)])
def test_centroid_budget_adds_record_slots(budget, slots):
    """With a centroid budget every graph and head has one more partial record
    per 16 centroid terms, after its spans (17 spans for t_cap 4100)."""
    kv = _kv()
    off = _idx()
    on = _idx(cent_budget=budget, cent_sel=FAKE, cent_n=FAKE, vsum=FAKE)
    assert _ws(kv, on, 4100) - _ws(kv, off, 4100) == 4 * 32 * 160 * slots
    assert ckv.CKV_MAX_CENT == 256


@pytest.mark.parametrize("first,count", [(0, -1), (-1, 4), (1, 0), (30, 3), (32, 1)])
def test_window_validation(first, count):
    kv, idx = _kv(), _idx(win_first=first, win_count=count)
    for f in (ckv.LIB.ckv_score_centroids,):
        assert f(ctypes.byref(kv), ctypes.byref(idx), FAKE, FAKE, FAKE, BIG, None) == ckv.CKV_E_INVALID


def test_window_view_binding():
    idx = object.__new__(ckv.CommunityIndex)
    idx.n_graphs = 32
    idx.desc = ckv.CkvIndex(0, 32, 256, 1000, 16, 4)
    v = idx.window(8, 8)
    assert (v.desc.win_first, v.desc.win_count) == (8, 8)
    assert (idx.desc.win_first, idx.desc.win_count) == (0, 0)
    for bad in ((0, 0), (-1, 2), (30, 3)):
        with pytest.raises(ValueError):
            idx.window(*bad)


def test_select_validation():
    kv, idx = _kv(), _idx()
    f = ckv.LIB.ckv_select_communities
    args = lambda budget, mc, tcap, sel=FAKE, q=FAKE: (ctypes.byref(kv), ctypes.byref(idx), q, FAKE, budget, mc,
                                                       tcap, sel, FAKE, FAKE, FAKE, FAKE, FAKE, BIG, None)
    assert f(*args(4096, 0, 4099)) == ckv.CKV_E_INVALID   # t_cap below sinks + budget
    assert f(*args(-1, 0, 4100)) == ckv.CKV_E_INVALID
    assert f(*args(4096, -2, 4100)) == ckv.CKV_E_INVALID
    assert f(*args(4096, 0, 4100, sel=None)) == ckv.CKV_E_INVALID
    assert f(*args(4096, 0, 4100, q=None)) == ckv.CKV_E_INVALID


def test_score_select_need_the_candidate_workspace():
    """Scoring leaves the selection's candidates in the workspace: both calls
    refuse a workspace smaller than ckv_workspace_bytes(kv, idx, 0)."""
    kv, idx = _kv(), _idx()
    need = _ws(kv, idx, 0)
    score = lambda ws, nb: ckv.LIB.ckv_score_centroids(ctypes.byref(kv), ctypes.byref(idx), FAKE, FAKE, ws, nb, None)
    sel = lambda ws, nb: ckv.LIB.ckv_select_communities(ctypes.byref(kv), ctypes.byref(idx), FAKE, FAKE, 4096, 0,
                                                        4100, FAKE, FAKE, FAKE, FAKE, FAKE, ws, nb, None)
    for f in (score, sel):
        assert f(None, need) == ckv.CKV_E_WORKSPACE
        assert f(FAKE, need - 1) == ckv.CKV_E_WORKSPACE
    # 32 graphs x 33 tiles x 64 candidates of 24 bytes, one left-out maximum per 16
    assert need >= _ws(kv, None, 0) + 32 * 8192 // 256 * 64 * 24


def test_gather_assign_dense_workspace_checks():
    kv, idx = _kv(), _idx()
    need = _ws(kv, idx, 4100)
    r = ckv.LIB.ckv_gather_attend(ctypes.byref(kv), ctypes.byref(idx), FAKE, FAKE, FAKE, 4100, 1.0, FAKE, FAKE, FAKE,
                                  FAKE, need - 1, None)
    assert r == ckv.CKV_E_WORKSPACE
    r = ckv.LIB.ckv_gather_attend(ctypes.byref(kv), ctypes.byref(idx), FAKE, FAKE, FAKE, 4100, 1.0, FAKE, None, FAKE,
                                  FAKE, need, None)
    assert r == ckv.CKV_E_INVALID
    g = lambda out, ml: ckv.LIB.ckv_gather_attend(ctypes.byref(kv), ctypes.byref(idx), FAKE, FAKE, FAKE, 4100, 1.0,
                                                 out, FAKE, ml, FAKE, need, None)
    assert g(FAKE, None) == ckv.CKV_E_INVALID   # out and ml: both (complete) or neither (deferred)
    assert g(None, FAKE) == ckv.CKV_E_INVALID
    a = lambda kappa, ws, nbytes, ml=FAKE, out=None: ckv.LIB.ckv_assign_update(
        ctypes.byref(kv), ctypes.byref(idx), FAKE, FAKE, FAKE, ml, 4100, FAKE, kappa, FAKE, FAKE, FAKE, FAKE, out,
        ws, nbytes, None)
    assert a(8, FAKE, need, ml=None) == ckv.CKV_E_INVALID   # complete gather: its ml is read
    assert a(0, FAKE, need, ml=None, out=FAKE) == ckv.CKV_E_INVALID
    assert a(0, FAKE, need) == ckv.CKV_E_INVALID
    assert a(33, FAKE, need) == ckv.CKV_E_INVALID
    assert a(8, None, need) == ckv.CKV_E_WORKSPACE
    assert a(8, FAKE, need - 1) == ckv.CKV_E_WORKSPACE
    d = ckv.LIB.ckv_dense_attend(ctypes.byref(kv), FAKE, 1.0, FAKE, None, FAKE, _ws(kv, None, 0) - 1, None)
    assert d == ckv.CKV_E_WORKSPACE


def test_attention_recall_validation():
    kv, idx = _kv(), _idx()
    f = ckv.LIB.ckv_attention_recall
    for args in ((None, FAKE, FAKE), (FAKE, None, FAKE), (FAKE, FAKE, None)):
        assert f(ctypes.byref(kv), ctypes.byref(idx), *args, None) == ckv.CKV_E_INVALID
    assert f(ctypes.byref(kv), ctypes.byref(_idx(n_graphs=31)), FAKE, FAKE, FAKE, None) == ckv.CKV_E_INVALID
    assert f(ctypes.byref(_kv(head_dim=96)), ctypes.byref(idx), FAKE, FAKE, FAKE, None) == ckv.CKV_E_UNSUPPORTED
    assert f(None, ctypes.byref(idx), FAKE, FAKE, FAKE, None) == ckv.CKV_E_INVALID


def test_gather_noalloc_validation():
    """The no-allocation gather checks its scratch need on the host: too large a
    shape is CKV_E_WORKSPACE before any device call; out and ml are required."""
    f = ckv.LIB.ckv_gather_attend_noalloc
    kv, idx = _kv(), _idx()
    args = lambda t_cap, out=FAKE, ml=FAKE: (ctypes.byref(kv), ctypes.byref(idx), FAKE, FAKE, FAKE, t_cap, 1.0, out,
                                             FAKE, ml, None)
    # 32 graphs x 1 head x ceil(t_cap / 256) spans x 160 floats: 4 MiB holds about 204 spans
    assert f(*args(300_000)) == ckv.CKV_E_WORKSPACE
    assert f(*args(4100, out=None)) == ckv.CKV_E_INVALID
    assert f(*args(4100, ml=None)) == ckv.CKV_E_INVALID
    assert f(*args(0)) == ckv.CKV_E_INVALID
    gidx = _idx(mode=ckv.CKV_MODE_QUERY_GROUP, n_graphs=64)
    gkv = _kv(batch=8)
    big = (ctypes.byref(gkv), ctypes.byref(gidx), FAKE, FAKE, FAKE, 4 * 4100, 1.0, FAKE, FAKE, FAKE, None)
    assert f(*big) == ckv.CKV_E_WORKSPACE  # 64 graphs x 4 heads x 65 spans: 10.6 MB


def test_read_rows_validation():
    kv = _kv()
    f = lambda rows, n, part: ckv.LIB.ckv_read_rows(ctypes.byref(kv), rows, n, part, None)
    assert f(FAKE, -1, FAKE) == ckv.CKV_E_INVALID
    assert f(None, 4, FAKE) == ckv.CKV_E_INVALID
    assert f(FAKE, 4, None) == ckv.CKV_E_INVALID
    assert f(None, 0, None) == ckv.CKV_OK  # nothing to read, nothing launched


def test_kv_write_and_build_validation():
    kv, idx = _kv(), _idx()
    w = lambda b, kh, pos0, n, k=FAKE: ckv.LIB.ckv_kv_write(ctypes.byref(kv), b, kh, pos0, n, k, FAKE, None)
    assert w(1, 0, 0, 4) == ckv.CKV_E_INVALID          # batch row out of range
    assert w(0, 8, 0, 4) == ckv.CKV_E_INVALID          # kv head out of range
    assert w(0, 0, 8200 * 16 - 2, 4) == ckv.CKV_E_INVALID  # past the page table
    assert w(0, 0, 0, 4, k=None) == ckv.CKV_E_INVALID
    assert w(0, 0, 0, 0) == ckv.CKV_OK                 # nothing to do, nothing launched
    b = ckv.LIB.ckv_index_build(ctypes.byref(kv), ctypes.byref(idx), None, FAKE, 1 << 40, None)
    assert b == ckv.CKV_E_INVALID
    b = ckv.LIB.ckv_index_build(ctypes.byref(kv), ctypes.byref(idx), FAKE, FAKE, 16, None)
    assert b == ckv.CKV_E_WORKSPACE


def test_binding_rejects_wrong_tensors():
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-only check")
    store = object.__new__(ckv.KVStore)
    store.batch, store.n_q_heads, store.n_kv_heads, store.head_dim, store.dtype = 1, 4, 1, 64, torch.float32
    with pytest.raises(ValueError):
        ckv._need(torch.zeros(3, 64), "q", torch.float32, (1, 4, 64))


def test_time_next_launch_arming():
    f = ckv.LIB.ckv_time_next_launch
    assert f(FAKE, None) == ckv.CKV_E_INVALID
    assert f(None, FAKE) == ckv.CKV_E_INVALID
    assert f(None, None) == ckv.CKV_OK
    # armed events are only consumed by a launch; validation failures launch nothing
    assert f(FAKE, FAKE) == ckv.CKV_OK
    kv, idx = _kv(head_dim=96), _idx()
    assert ckv.LIB.ckv_score_centroids(ctypes.byref(kv), ctypes.byref(idx), FAKE, FAKE, FAKE, BIG, None) == \
        ckv.CKV_E_UNSUPPORTED
    assert f(None, None) == ckv.CKV_OK


def test_prefill_workspace_and_validation():
    kv = _kv()
    wsb = lambda mode, n, k=kv: ckv.LIB.ckv_prefill_workspace_bytes(ctypes.byref(k), mode, n)
    assert wsb(ckv.CKV_MODE_PER_HEAD, 4096) == 4 * 32 * 4096
    assert wsb(ckv.CKV_MODE_QUERY_GROUP, 100) == 12800  # 4 * 32 * 100 rounded to 256
    assert wsb(ckv.CKV_MODE_PER_HEAD, 0) == 0 and wsb(7, 10) == 0
    need = wsb(ckv.CKV_MODE_QUERY_GROUP, 4096)
    f = ckv.LIB.ckv_prefill_topk

    def call(mode=ckv.CKV_MODE_PER_HEAD, b=0, q=FAKE, n=4096, sinks=4, kappa=8, scale=1.0, edges=FAKE,
             ws=FAKE, nbytes=need, k=kv):
        return f(ctypes.byref(k), mode, b, q, n, sinks, kappa, scale, edges, None, ws, nbytes, None)
    assert call(b=1) == ckv.CKV_E_INVALID                       # sequence out of range
    assert call(n=0) == ckv.CKV_E_INVALID
    assert call(n=8200 * 16 + 1) == ckv.CKV_E_INVALID           # past the page table
    assert call(kappa=0) == ckv.CKV_E_INVALID and call(kappa=33) == ckv.CKV_E_INVALID
    assert call(sinks=-1) == ckv.CKV_E_INVALID and call(scale=0.0) == ckv.CKV_E_INVALID
    assert call(q=None) == ckv.CKV_E_INVALID and call(edges=None) == ckv.CKV_E_INVALID
    assert call(mode=5) == ckv.CKV_E_INVALID
    assert call(ws=None) == ckv.CKV_E_WORKSPACE and call(nbytes=need - 1) == ckv.CKV_E_WORKSPACE
    assert call(k=_kv(dtype=ckv.CKV_DTYPE_F32)) == ckv.CKV_E_UNSUPPORTED   # matrix cores: bf16 only
    assert call(mode=ckv.CKV_MODE_QUERY_GROUP, kappa=17) == ckv.CKV_E_UNSUPPORTED
    assert call(mode=ckv.CKV_MODE_QUERY_GROUP, k=_kv(n_kv_heads=4)) == ckv.CKV_E_UNSUPPORTED  # 8 heads per group
