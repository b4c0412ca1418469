"""ctypes binding of libckv.so (the C ABI in include/ckv.h).

Every function here only marshals arguments: torch tensors supply device
memory and the current HIP stream, and each call goes straight to the
library's entry point of the same name.  There is no fallback: importing this
module raises if the library has not been built, and every call raises
CkvError when the library rejects its arguments.

The helper classes (KVStore, CommunityIndex, DecodeBuffers, Decoder) only
allocate the device buffers the entry points expect, with the shapes the
header documents.
"""
from __future__ import annotations

import copy
import ctypes
import math
import os
from ctypes import POINTER, c_float, c_int32, c_size_t, c_void_p
from typing import List, Optional, Sequence

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libckv.so")

CKV_OK, CKV_E_INVALID, CKV_E_UNSUPPORTED, CKV_E_WORKSPACE, CKV_E_HIP = 0, -1, -2, -3, -4
CKV_ST_TAIL_FULL, CKV_ST_CAPACITY, CKV_ST_BAD_LABEL = 1, 2, 4
CKV_DTYPE_F32, CKV_DTYPE_BF16 = 0, 1
CKV_MODE_PER_HEAD, CKV_MODE_QUERY_GROUP = 0, 1
CKV_MAX_KAPPA, CKV_MAX_C_CAP, CKV_MAX_CENT = 32, 16384, 256
CKV_NOALLOC_SCRATCH_BYTES = 4 << 20

EXPORTS = ("ckv_workspace_bytes", "ckv_kv_write", "ckv_index_build", "ckv_score_centroids",
           "ckv_select_communities", "ckv_gather_attend", "ckv_gather_attend_noalloc", "ckv_assign_update",
           "ckv_dense_attend",
           "ckv_attention_recall", "ckv_prefill_workspace_bytes", "ckv_prefill_topk", "ckv_read_rows",
           "ckv_leiden_partition", "ckv_partition_quality", "ckv_extend_partition",
           "ckv_time_next_launch", "ckv_status_str", "ckv_abi_version")


class CkvError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {code} ({ckv_status_str(code)})")
        self.code = code


class CkvKV(ctypes.Structure):
    _fields_ = [("kv", c_void_p), ("page_table", c_void_p), ("seq_len", c_void_p),
                ("batch", c_int32), ("n_q_heads", c_int32), ("n_kv_heads", c_int32),
                ("head_dim", c_int32), ("page_size", c_int32), ("max_pages", c_int32),
                ("n_pages", c_int32), ("dtype", c_int32)]


class CkvIndex(ctypes.Structure):
    _fields_ = [("mode", c_int32), ("n_graphs", c_int32), ("c_cap", c_int32), ("l_cap", c_int32),
                ("tail_cap", c_int32), ("n_sinks", c_int32),
                ("n_comm", c_void_p), ("size", c_void_p), ("offs", c_void_p), ("toks", c_void_p),
                ("label", c_void_p), ("tail_pos", c_void_p), ("tail_comm", c_void_p),
                ("tail_len", c_void_p), ("csum", c_void_p), ("cent", c_void_p), ("cq", c_void_p),
                ("cscale", c_void_p), ("status", c_void_p), ("win_first", c_int32), ("win_count", c_int32),
                ("cent_budget", c_int32), ("cent_sel", c_void_p), ("cent_n", c_void_p), ("vsum", c_void_p)]


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m community_kv_retrieval_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    KVP, IXP = POINTER(CkvKV), POINTER(CkvIndex)
    sig = {
        "ckv_workspace_bytes": (c_size_t, [KVP, IXP, c_int32]),
        "ckv_kv_write": (c_int32, [KVP, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p]),
        "ckv_index_build": (c_int32, [KVP, IXP, c_void_p, c_void_p, c_size_t, c_void_p]),
        "ckv_score_centroids": (c_int32, [KVP, IXP, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
        "ckv_select_communities": (c_int32, [KVP, IXP, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_void_p,
                                             c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                             c_void_p]),
        "ckv_gather_attend": (c_int32, [KVP, IXP, c_void_p, c_void_p, c_void_p, c_int32, c_float, c_void_p,
                                        c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
        "ckv_gather_attend_noalloc": (c_int32, [KVP, IXP, c_void_p, c_void_p, c_void_p, c_int32, c_float,
                                                c_void_p, c_void_p, c_void_p, c_void_p]),
        "ckv_assign_update": (c_int32, [KVP, IXP, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_void_p,
                                        c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                        c_size_t, c_void_p]),
        "ckv_dense_attend": (c_int32, [KVP, c_void_p, c_float, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
        "ckv_attention_recall": (c_int32, [KVP, IXP, c_void_p, c_void_p, c_void_p, c_void_p]),
        "ckv_prefill_workspace_bytes": (c_size_t, [KVP, c_int32, c_int32]),
        "ckv_prefill_topk": (c_int32, [KVP, c_int32, c_int32, c_void_p, c_int32, c_int32, c_int32, c_float,
                                       c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
        "ckv_read_rows": (c_int32, [KVP, c_void_p, c_int32, c_void_p, c_void_p]),
        "ckv_leiden_partition": (c_int32, [c_int32, c_void_p, c_int32, c_void_p, ctypes.c_int64, c_int32,
                                           ctypes.c_int64, ctypes.c_int64, c_int32, c_void_p, c_void_p, c_void_p]),
        "ckv_partition_quality": (c_int32, [c_int32, c_void_p, c_int32, c_void_p, ctypes.c_int64, c_int32,
                                            ctypes.c_int64, ctypes.c_int64, c_int32, c_void_p, c_void_p]),
        "ckv_extend_partition": (c_int32, [c_int32, c_void_p, c_void_p, c_void_p, ctypes.c_int64, c_int32,
                                           c_void_p, c_void_p]),
        "ckv_time_next_launch": (c_int32, [c_void_p, c_void_p]),
        "ckv_status_str": (ctypes.c_char_p, [c_int32]),
        "ckv_abi_version": (c_int32, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    return lib


LIB = _load()


def ckv_status_str(code: int) -> str:
    return LIB.ckv_status_str(code).decode()


def _check(fn: str, code: int):
    if code != CKV_OK:
        raise CkvError(fn, code)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else c_void_p(t.data_ptr())


def _stream(stream) -> c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape: Sequence[int]):
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: expected contiguous device {dtype} {tuple(shape)}, got {t.dtype} "
                         f"{tuple(t.shape)} (contiguous={t.is_contiguous()}, device={t.device})")


# ---------------------------------------------------------------------------
# Device buffers the entry points work on
# ---------------------------------------------------------------------------

class KVStore:
    """Paged K/V pool of one layer: [n_pages][n_kv_heads][page_size][2][head_dim]."""

    def __init__(self, batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, dtype: torch.dtype,
                 capacity: int, page_size: int = 16, device="cuda", shuffle_pages: bool = True,
                 seed: int = 0, seq_len: Optional[Sequence[int]] = None):
        self.batch, self.n_q_heads, self.n_kv_heads, self.head_dim = batch, n_q_heads, n_kv_heads, head_dim
        self.dtype, self.page_size, self.capacity = dtype, page_size, capacity
        self.max_pages = math.ceil(capacity / page_size)
        self.n_pages = batch * self.max_pages
        self.kv = torch.empty((self.n_pages, n_kv_heads, page_size, 2, head_dim), dtype=dtype, device=device)
        ids = torch.arange(self.n_pages, dtype=torch.int32)
        if shuffle_pages:
            g = torch.Generator().manual_seed(seed)
            ids = ids[torch.randperm(self.n_pages, generator=g)]
        self.page_table = ids.view(batch, self.max_pages).contiguous().to(device)
        lens = [0] * batch if seq_len is None else list(seq_len)
        self.seq_len = torch.tensor(lens, dtype=torch.int32, device=device)
        self.desc = CkvKV(self.kv.data_ptr(), self.page_table.data_ptr(), self.seq_len.data_ptr(), batch,
                          n_q_heads, n_kv_heads, head_dim, page_size, self.max_pages, self.n_pages,
                          CKV_DTYPE_F32 if dtype == torch.float32 else CKV_DTYPE_BF16)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


class CommunityIndex:
    """Community state of every graph of one layer (ckv_index)."""

    def __init__(self, kv: KVStore, mode: int, n_comm: Sequence[int], l_cap: int, tail_cap: int,
                 n_sinks: int, c_cap: Optional[int] = None, device="cuda", cent_budget: int = 0):
        G = kv.batch * (kv.n_q_heads if mode == CKV_MODE_PER_HEAD else kv.n_kv_heads)
        if c_cap is None:
            c_cap = max(256, 256 * math.ceil(max(n_comm) / 256))
        D = kv.head_dim
        i32 = dict(dtype=torch.int32, device=device)
        self.mode, self.n_graphs, self.c_cap, self.l_cap = mode, G, c_cap, l_cap
        self.tail_cap, self.n_sinks = tail_cap, n_sinks
        self.n_comm = torch.tensor(list(n_comm), **i32)
        self.size = torch.zeros((G, c_cap), **i32)
        self.offs = torch.zeros((G, c_cap + 4), **i32)  # rows padded to 16 bytes
        self.toks = torch.zeros((G, l_cap), **i32)
        self.label = torch.full((G, l_cap), -1, **i32)
        self.tail_pos = torch.zeros((G, tail_cap), **i32)
        self.tail_comm = torch.zeros((G, tail_cap), **i32)
        self.tail_len = torch.zeros((G,), **i32)
        self.csum = torch.zeros((G, c_cap, D), dtype=torch.float64, device=device)
        self.cent = torch.zeros((G, c_cap, D), dtype=torch.float32, device=device)
        self.cq = torch.zeros((G, c_cap // 256, D, 256), dtype=torch.int8, device=device)  # tile-major
        self.cscale = torch.zeros((G, c_cap), dtype=torch.float32, device=device)
        self.status = torch.zeros((1,), **i32)
        # centroid budget (Table 6): the chosen communities per graph and the value sums
        self.cent_budget = cent_budget
        nb = max(cent_budget, 1)
        self.cent_sel = torch.zeros((G, nb), **i32) if cent_budget > 0 else None
        self.cent_n = torch.zeros((G,), **i32) if cent_budget > 0 else None
        self.vsum = torch.zeros((G, c_cap, D), dtype=torch.float64, device=device) if cent_budget > 0 else None
        self.desc = CkvIndex(mode, G, c_cap, l_cap, tail_cap, n_sinks, *[
            t.data_ptr() for t in (self.n_comm, self.size, self.offs, self.toks, self.label, self.tail_pos,
                                   self.tail_comm, self.tail_len, self.csum, self.cent, self.cq, self.cscale,
                                   self.status)], 0, 0, cent_budget, _ptr(self.cent_sel), _ptr(self.cent_n),
            _ptr(self.vsum))

    def heads_per_graph(self, kv: KVStore) -> int:
        return 1 if self.mode == CKV_MODE_PER_HEAD else kv.group

    def window(self, first: int, count: int) -> "CommunityIndex":
        """The same index (shared state), with the four step calls restricted to
        graphs first .. first + count - 1."""
        if not (0 <= first and 0 < count and first + count <= self.n_graphs):
            raise ValueError(f"window [{first}, {first + count}) outside the {self.n_graphs} graphs")
        v = copy.copy(self)
        v.desc = CkvIndex.from_buffer_copy(self.desc)
        v.desc.win_first, v.desc.win_count = first, count
        return v

    STATE = ("size", "offs", "toks", "label", "tail_pos", "tail_comm", "tail_len", "csum", "cent", "cq", "cscale",
             "status")

    def _state_keys(self):
        return self.STATE + ("n_comm",) + (("vsum", "cent_sel", "cent_n") if self.cent_budget > 0 else ())

    def state_dict(self):
        return {k: getattr(self, k).clone() for k in self._state_keys()}

    def load_state_dict(self, sd):
        for k in self._state_keys():
            getattr(self, k).copy_(sd[k])


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def ckv_workspace_bytes(kv: KVStore, idx: Optional[CommunityIndex], t_cap: int) -> int:
    return int(LIB.ckv_workspace_bytes(ctypes.byref(kv.desc), ctypes.byref(idx.desc) if idx else None, t_cap))


def ckv_kv_write(kv: KVStore, b: int, kv_head: int, pos0: int, k: torch.Tensor, v: torch.Tensor, stream=None):
    n = k.shape[0]
    _need(k, "k", kv.dtype, (n, kv.head_dim))
    _need(v, "v", kv.dtype, (n, kv.head_dim))
    _check("ckv_kv_write", LIB.ckv_kv_write(ctypes.byref(kv.desc), b, kv_head, pos0, n, _ptr(k), _ptr(v),
                                            _stream(stream)))


def ckv_index_build(kv: KVStore, idx: CommunityIndex, labels_in: torch.Tensor, ws: torch.Tensor, stream=None):
    _need(labels_in, "labels_in", torch.int32, (idx.n_graphs, idx.l_cap))
    _check("ckv_index_build", LIB.ckv_index_build(ctypes.byref(kv.desc), ctypes.byref(idx.desc), _ptr(labels_in),
                                                  _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def ckv_score_centroids(kv: KVStore, idx: CommunityIndex, q: torch.Tensor, scores: torch.Tensor,
                        ws: torch.Tensor, stream=None):
    """ws: the workspace the following ckv_select_communities reads the candidates from."""
    _need(q, "q", kv.dtype, (kv.batch, kv.n_q_heads, kv.head_dim))
    _need(scores, "scores", torch.float32, (idx.n_graphs, idx.c_cap))
    _check("ckv_score_centroids", LIB.ckv_score_centroids(ctypes.byref(kv.desc), ctypes.byref(idx.desc), _ptr(q),
                                                          _ptr(scores), _ptr(ws), ws.numel() * ws.element_size(),
                                                          _stream(stream)))


def ckv_select_communities(kv: KVStore, idx: CommunityIndex, q: torch.Tensor, scores: torch.Tensor, budget: int,
                           max_comm: int, sel: torch.Tensor, sel_n: torch.Tensor, top: torch.Tensor,
                           tok_list: torch.Tensor, tok_n: torch.Tensor, ws: torch.Tensor, stream=None):
    G = idx.n_graphs
    _need(q, "q", kv.dtype, (kv.batch, kv.n_q_heads, kv.head_dim))
    _need(scores, "scores", torch.float32, (G, idx.c_cap))
    _need(sel, "sel", torch.int32, (G, idx.c_cap))
    for name, t in (("sel_n", sel_n), ("top", top), ("tok_n", tok_n)):
        _need(t, name, torch.int32, (G,))
    t_cap = tok_list.shape[1]
    _need(tok_list, "tok_list", torch.int32, (G, t_cap))
    _check("ckv_select_communities", LIB.ckv_select_communities(
        ctypes.byref(kv.desc), ctypes.byref(idx.desc), _ptr(q), _ptr(scores), budget, max_comm, t_cap, _ptr(sel),
        _ptr(sel_n), _ptr(top), _ptr(tok_list), _ptr(tok_n), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))


def ckv_gather_attend(kv: KVStore, idx: CommunityIndex, q: torch.Tensor, tok_list: torch.Tensor,
                      tok_n: torch.Tensor, sm_scale: float, out: Optional[torch.Tensor], logits: torch.Tensor,
                      ml: Optional[torch.Tensor], ws: torch.Tensor, stream=None):
    """out = ml = None defers the combine to the next ckv_assign_update(out=...)."""
    G, nh, t_cap = idx.n_graphs, idx.heads_per_graph(kv), tok_list.shape[1]
    _need(q, "q", kv.dtype, (kv.batch, kv.n_q_heads, kv.head_dim))
    _need(tok_list, "tok_list", torch.int32, (G, t_cap))
    _need(tok_n, "tok_n", torch.int32, (G,))
    if out is not None:
        _need(out, "out", torch.float32, (kv.batch, kv.n_q_heads, kv.head_dim))
    _need(logits, "logits", torch.float32, (G, nh, t_cap))
    if ml is not None:
        _need(ml, "ml", torch.float32, (G, nh, 2))
    _check("ckv_gather_attend", LIB.ckv_gather_attend(
        ctypes.byref(kv.desc), ctypes.byref(idx.desc), _ptr(q), _ptr(tok_list), _ptr(tok_n), t_cap,
        float(sm_scale), _ptr(out), _ptr(logits), _ptr(ml), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))


def ckv_gather_attend_noalloc(kv: KVStore, idx: CommunityIndex, q: torch.Tensor, tok_list: torch.Tensor,
                              tok_n: torch.Tensor, sm_scale: float, out: torch.Tensor, logits: torch.Tensor,
                              ml: torch.Tensor, stream=None):
    """ckv_gather_attend (complete) with the library's static scratch instead of a workspace."""
    G, nh, t_cap = idx.n_graphs, idx.heads_per_graph(kv), tok_list.shape[1]
    _need(q, "q", kv.dtype, (kv.batch, kv.n_q_heads, kv.head_dim))
    _need(tok_list, "tok_list", torch.int32, (G, t_cap))
    _need(tok_n, "tok_n", torch.int32, (G,))
    _need(out, "out", torch.float32, (kv.batch, kv.n_q_heads, kv.head_dim))
    _need(logits, "logits", torch.float32, (G, nh, t_cap))
    _need(ml, "ml", torch.float32, (G, nh, 2))
    _check("ckv_gather_attend_noalloc", LIB.ckv_gather_attend_noalloc(
        ctypes.byref(kv.desc), ctypes.byref(idx.desc), _ptr(q), _ptr(tok_list), _ptr(tok_n), t_cap,
        float(sm_scale), _ptr(out), _ptr(logits), _ptr(ml), _stream(stream)))


def ckv_assign_update(kv: KVStore, idx: CommunityIndex, tok_list: torch.Tensor, tok_n: torch.Tensor,
                      logits: torch.Tensor, ml: Optional[torch.Tensor], top: torch.Tensor, kappa: int,
                      k_new: torch.Tensor, v_new: torch.Tensor, edges: torch.Tensor, assign: torch.Tensor,
                      ws: torch.Tensor, stream=None, out: Optional[torch.Tensor] = None):
    """out given: complete a deferred gather first (writes out and, if given, ml)."""
    G, nh, t_cap = idx.n_graphs, idx.heads_per_graph(kv), tok_list.shape[1]
    _need(tok_list, "tok_list", torch.int32, (G, t_cap))
    _need(logits, "logits", torch.float32, (G, nh, t_cap))
    if ml is not None:
        _need(ml, "ml", torch.float32, (G, nh, 2))
    if out is not None:
        _need(out, "out", torch.float32, (kv.batch, kv.n_q_heads, kv.head_dim))
    for name, t in (("tok_n", tok_n), ("top", top), ("assign", assign)):
        _need(t, name, torch.int32, (G,))
    _need(k_new, "k_new", kv.dtype, (kv.batch, kv.n_kv_heads, kv.head_dim))
    _need(v_new, "v_new", kv.dtype, (kv.batch, kv.n_kv_heads, kv.head_dim))
    _need(edges, "edges", torch.int32, (G, kappa))
    _check("ckv_assign_update", LIB.ckv_assign_update(
        ctypes.byref(kv.desc), ctypes.byref(idx.desc), _ptr(tok_list), _ptr(tok_n), _ptr(logits), _ptr(ml),
        t_cap, _ptr(top), kappa, _ptr(k_new), _ptr(v_new), _ptr(edges), _ptr(assign), _ptr(out), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))


def prefill_workspace(kv: KVStore, mode: int, n: int, device="cuda") -> torch.Tensor:
    nbytes = int(LIB.ckv_prefill_workspace_bytes(ctypes.byref(kv.desc), mode, n))
    if nbytes == 0:
        raise ValueError(f"ckv_prefill_workspace_bytes: bad arguments (mode {mode}, n {n})")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def ckv_prefill_topk(kv: KVStore, mode: int, b: int, q: torch.Tensor, n_sinks: int, kappa: int, sm_scale: float,
                     edges: torch.Tensor, weights: Optional[torch.Tensor], ws: torch.Tensor, stream=None):
    """Prefill graph of sequence b: q [n][n_q_heads][head_dim], keys = the store's
    positions 0..n-1; edges [graphs][n][kappa] int32, weights (optional) float32."""
    n = q.shape[0]
    graphs = kv.n_q_heads if mode == CKV_MODE_PER_HEAD else kv.n_kv_heads
    _need(q, "q", kv.dtype, (n, kv.n_q_heads, kv.head_dim))
    _need(edges, "edges", torch.int32, (graphs, n, kappa))
    if weights is not None:
        _need(weights, "weights", torch.float32, (graphs, n, kappa))
    _check("ckv_prefill_topk", LIB.ckv_prefill_topk(
        ctypes.byref(kv.desc), mode, b, _ptr(q), n, n_sinks, kappa, float(sm_scale), _ptr(edges), _ptr(weights),
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def ckv_dense_attend(kv: KVStore, q: torch.Tensor, sm_scale: float, out: torch.Tensor, ws: torch.Tensor,
                     stream=None, ml: Optional[torch.Tensor] = None):
    _need(q, "q", kv.dtype, (kv.batch, kv.n_q_heads, kv.head_dim))
    _need(out, "out", torch.float32, (kv.batch, kv.n_q_heads, kv.head_dim))
    if ml is not None:
        _need(ml, "ml", torch.float32, (kv.batch, kv.n_q_heads, 2))
    _check("ckv_dense_attend", LIB.ckv_dense_attend(ctypes.byref(kv.desc), _ptr(q), float(sm_scale), _ptr(out),
                                                    _ptr(ml), _ptr(ws), ws.numel() * ws.element_size(),
                                                    _stream(stream)))


def ckv_attention_recall(kv: KVStore, idx: CommunityIndex, ml: torch.Tensor, dense_ml: torch.Tensor,
                         recall: torch.Tensor, stream=None):
    """recall[G][hpg]: the share of each head's dense softmax mass (dense_ml
    from ckv_dense_attend) that its graph's attended tokens (ml from the
    gather) carry."""
    G, nh = idx.n_graphs, idx.heads_per_graph(kv)
    _need(ml, "ml", torch.float32, (G, nh, 2))
    _need(dense_ml, "dense_ml", torch.float32, (kv.batch, kv.n_q_heads, 2))
    _need(recall, "recall", torch.float32, (G, nh))
    _check("ckv_attention_recall", LIB.ckv_attention_recall(ctypes.byref(kv.desc), ctypes.byref(idx.desc),
                                                            _ptr(ml), _ptr(dense_ml), _ptr(recall),
                                                            _stream(stream)))


def ckv_read_rows(kv: KVStore, rows: torch.Tensor, part: torch.Tensor, stream=None):
    """The gather's loads over the given pool rows (a read-ceiling measurement);
    part[ceil(n/256)] gets per-block XOR checksums of the rows' 32-bit words."""
    n = rows.numel()
    _need(rows, "rows", torch.int32, (n,))
    _need(part, "part", torch.int32, ((n + 255) // 256,))
    _check("ckv_read_rows", LIB.ckv_read_rows(ctypes.byref(kv.desc), _ptr(rows), n, _ptr(part), _stream(stream)))


def _host_i32(a, name: str, shape) -> "np.ndarray":
    import numpy as np
    if not (isinstance(a, np.ndarray) and a.dtype == np.int32 and a.flags.c_contiguous and a.shape == tuple(shape)):
        raise ValueError(f"{name}: expected a C-contiguous int32 host array of shape {tuple(shape)}")
    return a


def ckv_leiden_partition(n_tokens, n_sinks: int, edges, gamma=(1, 1), n_threads: int = 0):
    """Leiden partition of every graph's token graph (host call).

    n_tokens: int32 [G]; edges: int32 [G][row_stride][kappa] host array.
    Returns (labels int32 [G][row_stride], n_comm int32 [G], quality float64 [G])."""
    import numpy as np
    G, stride, kappa = edges.shape if edges.ndim == 3 else (0, 0, 0)
    _host_i32(edges, "edges", (G, stride, kappa))
    _host_i32(n_tokens, "n_tokens", (G,))
    labels = np.empty((G, stride), dtype=np.int32)
    n_comm = np.empty((G,), dtype=np.int32)
    quality = np.empty((G,), dtype=np.float64)
    _check("ckv_leiden_partition", LIB.ckv_leiden_partition(
        G, n_tokens.ctypes.data, n_sinks, edges.ctypes.data, stride, kappa, int(gamma[0]), int(gamma[1]),
        n_threads, labels.ctypes.data, n_comm.ctypes.data, quality.ctypes.data))
    return labels, n_comm, quality


def ckv_partition_quality(n_tokens, n_sinks: int, edges, labels, gamma=(1, 1), n_threads: int = 0):
    """Modularity of given labels on every graph's token graph (host call)."""
    import numpy as np
    G, stride, kappa = edges.shape if edges.ndim == 3 else (0, 0, 0)
    _host_i32(edges, "edges", (G, stride, kappa))
    _host_i32(n_tokens, "n_tokens", (G,))
    _host_i32(labels, "labels", (G, stride))
    quality = np.empty((G,), dtype=np.float64)
    _check("ckv_partition_quality", LIB.ckv_partition_quality(
        G, n_tokens.ctypes.data, n_sinks, edges.ctypes.data, stride, kappa, int(gamma[0]), int(gamma[1]),
        n_threads, labels.ctypes.data, quality.ctypes.data))
    return quality


def ckv_extend_partition(first, n_tokens, edges, labels, n_comm):
    """Tokens first[g] .. n_tokens[g]-1 join the partition by the vote of
    their edges (host call; labels [G][row_stride] and n_comm [G] int32 are
    updated in place)."""
    import numpy as np
    G, stride, kappa = edges.shape if edges.ndim == 3 else (0, 0, 0)
    _host_i32(edges, "edges", (G, stride, kappa))
    _host_i32(first, "first", (G,))
    _host_i32(n_tokens, "n_tokens", (G,))
    _host_i32(labels, "labels", (G, stride))
    _host_i32(n_comm, "n_comm", (G,))
    _check("ckv_extend_partition", LIB.ckv_extend_partition(
        G, first.ctypes.data, n_tokens.ctypes.data, edges.ctypes.data, stride, kappa, labels.ctypes.data,
        n_comm.ctypes.data))
    return labels, n_comm


def ckv_time_next_launch(start: Optional["torch.cuda.Event"], stop: Optional["torch.cuda.Event"]):
    """Arms the next step kernel of this thread to stamp `start`/`stop` from its own dispatch.

    Both events must already exist on the device (torch creates an event on its
    first record()).  Once the kernel has run, start.elapsed_time(stop) is its
    execution time in ms.  None, None disarms.
    """
    ev = lambda e: None if e is None else c_void_p(e.cuda_event)
    _check("ckv_time_next_launch", LIB.ckv_time_next_launch(ev(start), ev(stop)))


# ---------------------------------------------------------------------------
# One decode step = the four calls in order
# ---------------------------------------------------------------------------

class DecodeBuffers:
    """Per-step outputs of the four calls, sized for one layer."""

    def __init__(self, kv: KVStore, idx: CommunityIndex, budget: int, kappa: int, device="cuda"):
        G, nh = idx.n_graphs, idx.heads_per_graph(kv)
        self.t_cap = max(1, idx.n_sinks + min(budget, idx.l_cap))  # the calls take t_cap >= 1
        i32 = dict(dtype=torch.int32, device=device)
        self.scores = torch.empty((G, idx.c_cap), dtype=torch.float32, device=device)
        self.sel = torch.empty((G, idx.c_cap), **i32)
        self.sel_n = torch.empty((G,), **i32)
        self.top = torch.empty((G,), **i32)
        self.tok_list = torch.empty((G, self.t_cap), **i32)
        self.tok_n = torch.empty((G,), **i32)
        self.out = torch.empty((kv.batch, kv.n_q_heads, kv.head_dim), dtype=torch.float32, device=device)
        self.logits = torch.empty((G, nh, self.t_cap), dtype=torch.float32, device=device)
        self.ml = torch.empty((G, nh, 2), dtype=torch.float32, device=device)
        self.edges = torch.empty((G, kappa), **i32)
        self.assign = torch.empty((G,), **i32)
        self.ws = torch.zeros((ckv_workspace_bytes(kv, idx, self.t_cap),), dtype=torch.uint8, device=device)


class EdgeTable:
    """The token graph of one layer as edge rows: e[g][i][0..kappa) = token i's
    edges in graph g (-1 = none), prompt rows from ckv_prefill_topk, decoded
    rows from each step's ckv_assign_update (Figure 1, panels (1) and (3)).
    Device memory; ckv_leiden_partition reads a host copy of it."""

    def __init__(self, kv: KVStore, mode: int, cap: int, kappa: int, device="cuda"):
        self.mode, self.kappa, self.cap = mode, kappa, cap
        per = kv.n_q_heads if mode == CKV_MODE_PER_HEAD else kv.n_kv_heads
        self.per_seq = per
        self.n_graphs = kv.batch * per
        self.e = torch.full((self.n_graphs, cap, kappa), -1, dtype=torch.int32, device=device)
        # sequence of every graph, to find the row a step's new token takes
        self._gidx = torch.arange(self.n_graphs, device=device)
        self.graph_seq = self._gidx // per

    def pinned(self) -> torch.Tensor:
        """A pinned host buffer shaped like the table (allocated once)."""
        if getattr(self, "_pinned", None) is None:
            self._pinned = torch.empty((self.n_graphs, self.cap, self.kappa), dtype=torch.int32, pin_memory=True)
        return self._pinned

    def put_prefill(self, b: int, edges: torch.Tensor):
        """Rows 0..n-1 of sequence b's graphs from ckv_prefill_topk's edges
        [graphs of the sequence][n][kappa]."""
        _need(edges, "edges", torch.int32, (self.per_seq, edges.shape[1], self.kappa))
        self.e[b * self.per_seq:(b + 1) * self.per_seq, :edges.shape[1]] = edges

    def put_step(self, edges: torch.Tensor, pos: torch.Tensor):
        """Row pos[seq of g] of every graph g from a step's edges [G][kappa];
        pos: the sequences' lengths before the step (the new tokens' positions)."""
        rows = pos.long()[self.graph_seq]
        # a sequence at the table's capacity stores no new token (the step
        # reports it in the index status): its row is left as it was
        ok = rows < self.cap
        rows = rows.clamp(max=self.cap - 1)
        self.e[self._gidx, rows] = torch.where(ok[:, None], edges, self.e[self._gidx, rows])


class PendingRefresh:
    """A partition being computed on host threads (Decoder.refresh_async)."""

    def __init__(self, n_tok, rows: int, gamma):
        self.n_tok, self.rows, self.gamma = n_tok, rows, gamma
        self.thread = None
        self.result = None
        self.error: Optional[BaseException] = None
        self.snapshot_ms = 0.0

    def done(self) -> bool:
        return self.thread is not None and not self.thread.is_alive()


class Decoder:
    """Runs CommunityKV decode steps for one layer.

    With defer set (the default) the gather leaves its per-span softmax states
    in the workspace and the assign call combines them into out and ml, so the
    combine overlaps the assignment instead of ending the gather; the results
    are bit-identical to a complete gather's.

    With windows > 1 a step splits the graphs into that many windows, each run
    on a stream of its own, window w scoring after window w - 1 has scored: the
    later windows' bandwidth-bound scoring and gathering then overlap the
    earlier windows' latency-bound selection and assignment.  The results are
    the same as with one window (every graph's work is unchanged).
    """

    def __init__(self, kv: KVStore, idx: CommunityIndex, budget: int, max_comm: int, kappa: int,
                 sm_scale: float, device="cuda", windows: int = 1, defer: bool = True):
        self.kv, self.idx = kv, idx
        self.budget, self.max_comm, self.kappa, self.sm_scale = budget, max_comm, kappa, sm_scale
        self.defer = defer
        self.device = device
        self.buf = DecodeBuffers(kv, idx, budget, kappa, device)
        self.set_windows(windows)
        # when set, every step records its edges in the table (the graph a
        # refresh partitions)
        self.edge_table: Optional[EdgeTable] = None

    def refresh_async(self, table: "EdgeTable", gamma=(1, 1), n_threads: int = 0) -> PendingRefresh:
        """Start a refresh beside the decode steps (Figure 4 runs the
        partitioning beside the model): the edge rows of the tokens cached now
        are copied to pinned host memory on a stream of their own and a host
        thread partitions them with ckv_leiden_partition, while steps go on.
        refresh_apply() then places the tokens decoded meanwhile by the vote
        of their edges (ckv_extend_partition) and rebuilds the index."""
        import threading
        import time

        import numpy as np
        idx = self.idx
        if table.mode != idx.mode or table.n_graphs != idx.n_graphs or table.cap != idx.l_cap:
            raise ValueError("edge table does not match the index")
        if getattr(table, "_pending", None) is not None:
            raise RuntimeError("a refresh of this edge table is still pending: refresh_apply it first")
        torch.cuda.current_stream().synchronize()   # the steps queued so far
        t0 = time.perf_counter()
        lens = self.kv.seq_len.cpu().numpy()
        n_tok = lens[table.graph_seq.cpu().numpy()].astype(np.int32)
        rows = int(n_tok.max(initial=0))
        host = table.pinned()          # rows >= n_tok[g] are not read
        ready = torch.cuda.Event()
        ready.record()
        side = torch.cuda.Stream()
        with torch.cuda.stream(side):
            side.wait_event(ready)
            host.copy_(table.e, non_blocking=True)   # contiguous both sides: one DMA, no staging
            copied = torch.cuda.Event()
            copied.record(side)
        pend = PendingRefresh(n_tok, rows, gamma)

        def work():
            try:
                copied.synchronize()
                pend.result = ckv_leiden_partition(n_tok, idx.n_sinks, host.numpy(), gamma, n_threads)
            except BaseException as e:  # handed to refresh_apply
                pend.error = e

        pend.thread = threading.Thread(target=work, name="ckv-leiden", daemon=True)
        table._pending = pend   # the pinned snapshot is in use until refresh_apply
        pend.thread.start()
        pend.snapshot_ms = (time.perf_counter() - t0) * 1e3
        return pend

    def refresh_apply(self, pend: PendingRefresh, table: "EdgeTable", c_cap: Optional[int] = None,
                      timings: Optional[dict] = None):
        """Finish a refresh_async: wait for the partition, let every token
        decoded since the snapshot join it by the vote of its edges, and
        rebuild the index from the result (replaces self.idx and the step
        buffers).  Returns the modularity [G] of the snapshot's partition.
        timings receives the ms spent waiting, placing the new tokens and
        building."""
        import time

        import numpy as np
        t0 = time.perf_counter()
        pend.thread.join()
        t1 = time.perf_counter()
        if getattr(table, "_pending", None) is pend:
            table._pending = None
        if pend.error is not None:
            raise pend.error
        labels0, n_comm, quality = pend.result
        idx = self.idx
        torch.cuda.current_stream().synchronize()   # the steps queued so far (their edge rows)
        t_drain = time.perf_counter()
        lens = self.kv.seq_len.cpu().numpy()
        n_now = lens[table.graph_seq.cpu().numpy()].astype(np.int32)
        rows = int(n_now.max(initial=0))
        lo = int(pend.n_tok.min(initial=0))
        host = table.pinned().numpy()   # rows below the snapshot's lengths hold the snapshot already
        host[:, lo:rows] = table.e[:, lo:rows].contiguous().cpu().numpy()
        ckv_extend_partition(pend.n_tok, n_now, host, labels0, n_comm)   # labels0: [G][cap]
        t2 = time.perf_counter()
        self._rebuild(labels0, n_comm, c_cap)
        if timings is not None:
            torch.cuda.synchronize()
            t3 = time.perf_counter()
            timings.update(wait=(t1 - t0) * 1e3, drain=(t_drain - t1) * 1e3, place=(t2 - t_drain) * 1e3,
                           build=(t3 - t2) * 1e3, snapshot=pend.snapshot_ms)
        return quality

    def _rebuild(self, labels, n_comm, c_cap: Optional[int]):
        """New index with n_comm communities per graph, built from labels
        [G][l_cap] (host int32) by ckv_index_build."""
        idx = self.idx
        if int(n_comm.max(initial=0)) > CKV_MAX_C_CAP:
            raise ValueError(f"{int(n_comm.max())} communities exceed the index's limit {CKV_MAX_C_CAP}")
        new = CommunityIndex(self.kv, idx.mode, [max(1, int(c)) for c in n_comm], idx.l_cap, idx.tail_cap,
                             idx.n_sinks, c_cap=c_cap, device=self.device, cent_budget=idx.cent_budget)
        new.n_comm.copy_(torch.from_numpy(n_comm))
        self.idx = new
        self.buf = DecodeBuffers(self.kv, new, self.budget, self.kappa, self.device)
        self.set_windows(self.windows)
        self.build(torch.from_numpy(labels).to(self.device))

    def refresh(self, table: "EdgeTable", gamma=(1, 1), n_threads: int = 0, c_cap: Optional[int] = None,
                timings: Optional[dict] = None):
        """Re-partition every graph's token graph (prompt and decoded rows of
        `table`) with ckv_leiden_partition and rebuild the index from the new
        labels with ckv_index_build ("Refresh" in Tables 8 and 9, against the
        incremental assignment of every step).  Replaces self.idx and the step
        buffers; returns the partitions' modularity [G] (float64, host).
        timings (a dict) receives the wall-clock ms of the three phases:
        copy (edge rows to the host), partition (the library's Leiden) and
        build (new index and ckv_index_build, synchronised)."""
        import time

        import numpy as np
        t0 = time.perf_counter()
        idx = self.idx
        if table.mode != idx.mode or table.n_graphs != idx.n_graphs or table.cap != idx.l_cap:
            raise ValueError("edge table does not match the index")
        lens = self.kv.seq_len.cpu().numpy()
        n_tok = lens[table.graph_seq.cpu().numpy()].astype(np.int32)
        edges = table.e.cpu().numpy()
        t1 = time.perf_counter()
        labels, n_comm, quality = ckv_leiden_partition(n_tok, idx.n_sinks, edges, gamma, n_threads)
        t2 = time.perf_counter()
        self._rebuild(labels, n_comm, c_cap)
        if timings is not None:
            torch.cuda.synchronize()
            t3 = time.perf_counter()
            timings.update(copy=(t1 - t0) * 1e3, partition=(t2 - t1) * 1e3, build=(t3 - t2) * 1e3)
        return quality

    def set_windows(self, windows: int):
        G = self.idx.n_graphs
        windows = max(1, min(int(windows), G))
        self.windows = windows
        self._views, self._streams = [], []
        if windows > 1:
            bounds = [G * w // windows for w in range(windows + 1)]
            self._views = [self.idx.window(bounds[w], bounds[w + 1] - bounds[w]) for w in range(windows)]
            self._streams = [torch.cuda.Stream() for _ in range(windows)]

    def build(self, labels_in: torch.Tensor, stream=None):
        ckv_index_build(self.kv, self.idx, labels_in, self.buf.ws, stream)

    def retrieve(self, q: torch.Tensor, stream=None):
        b = self.buf
        ckv_score_centroids(self.kv, self.idx, q, b.scores, b.ws, stream)
        ckv_select_communities(self.kv, self.idx, q, b.scores, self.budget, self.max_comm, b.sel, b.sel_n, b.top,
                               b.tok_list, b.tok_n, b.ws, stream)

    def attend(self, q: torch.Tensor, stream=None):
        """With defer set, out and ml are written by the following update()."""
        b = self.buf
        out, ml = (None, None) if self.defer else (b.out, b.ml)
        ckv_gather_attend(self.kv, self.idx, q, b.tok_list, b.tok_n, self.sm_scale, out, b.logits, ml, b.ws,
                          stream)

    def update(self, k_new: torch.Tensor, v_new: torch.Tensor, stream=None):
        b = self.buf
        pos = self.kv.seq_len.clone() if self.edge_table is not None else None
        ckv_assign_update(self.kv, self.idx, b.tok_list, b.tok_n, b.logits, b.ml, b.top, self.kappa, k_new, v_new,
                          b.edges, b.assign, b.ws, stream, out=b.out if self.defer else None)
        if self.edge_table is not None:
            self.edge_table.put_step(b.edges, pos)

    def step(self, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, stream=None):
        if self.windows == 1:
            self.retrieve(q, stream)
            self.attend(q, stream)
            self.update(k_new, v_new, stream)
            return self.buf.out
        b, kv = self.buf, self.kv
        cur = torch.cuda.current_stream() if stream is None else stream
        pos = None
        if self.edge_table is not None:
            with torch.cuda.stream(cur):
                pos = kv.seq_len.clone()   # the new tokens' positions, before any window appends
        start = torch.cuda.Event()
        start.record(cur)
        prev = None
        for view, s in zip(self._views, self._streams):
            s.wait_event(start)
            if prev is not None:
                s.wait_event(prev)
            for t in (q, k_new, v_new):
                t.record_stream(s)
            ckv_score_centroids(kv, view, q, b.scores, b.ws, s)
            prev = torch.cuda.Event()
            prev.record(s)
            ckv_select_communities(kv, view, q, b.scores, self.budget, self.max_comm, b.sel, b.sel_n, b.top,
                                   b.tok_list, b.tok_n, b.ws, s)
            out, ml = (None, None) if self.defer else (b.out, b.ml)
            ckv_gather_attend(kv, view, q, b.tok_list, b.tok_n, self.sm_scale, out, b.logits, ml, b.ws, s)
            ckv_assign_update(kv, view, b.tok_list, b.tok_n, b.logits, b.ml, b.top, self.kappa, k_new, v_new,
                              b.edges, b.assign, b.ws, s, out=b.out if self.defer else None)
            done = torch.cuda.Event()
            done.record(s)
            cur.wait_event(done)
        if pos is not None:
            with torch.cuda.stream(cur):
                self.edge_table.put_step(b.edges, pos)
        return b.out

    def dense(self, q: torch.Tensor, out: torch.Tensor, stream=None, ml: Optional[torch.Tensor] = None):
        ckv_dense_attend(self.kv, q, self.sm_scale, out, self.buf.ws, stream, ml=ml)
        return out

    def recall(self, dense_ml: torch.Tensor, recall: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
        """Attention-mass recall of the last gather, per graph and head
        (ckv_attention_recall), from dense_ml of dense(..., ml=).  Needs a
        complete gather's ml: with defer set, call it after update()."""
        if recall is None:
            recall = torch.empty((self.idx.n_graphs, self.idx.heads_per_graph(self.kv)), dtype=torch.float32,
                                 device=dense_ml.device)
        ckv_attention_recall(self.kv, self.idx, self.buf.ml, dense_ml, recall, stream)
        return recall
