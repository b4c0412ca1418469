"""The screening bound the GPU parity runner checks every step, pinned on the CPU.

The scoring kernel streams an int8 copy of the centroid table (per community
scale = max |centroid| / 127, code = round(centroid / scale)); the selection
treats every exact score as lying within cscale * |qbar|_1 * (1/2 + 127 (D + 4)
2^-24) plus a few float32 roundings of the screening score.  Here a plain numpy
screening score, built from that definition, must satisfy the runner's check
against the oracle's exact scores, and planted mistakes must fail it, so the
check is not vacuous.
"""
import numpy as np
import pytest

from oracle import ckv_oracle as O
from tests import parity as PY


def _screening(cent32, q_heads, counts, drop_scale=False, drop_head=False):
    scale = (np.abs(cent32).max(axis=1).astype(np.float32) / np.float32(PY.SCREEN_MAX)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        code = np.clip(np.rint(cent32 / scale[:, None]), -PY.SCREEN_MAX, PY.SCREEN_MAX)
    code = np.where(scale[:, None] > 0, code, 0).astype(np.float32)
    heads = q_heads[:1] if drop_head else q_heads
    qbar = heads.astype(np.float64).sum(axis=0).astype(np.float32)
    dot = (code * qbar[None, :]).astype(np.float32).sum(axis=1, dtype=np.float32)
    s = dot if drop_scale else (scale * dot).astype(np.float32)
    s = np.where(counts > 0, s, -np.inf).astype(np.float32)
    return s, scale


def _case(seed, D, n_heads, C=1500, c_cap=1792):
    r = np.random.default_rng(seed)
    cent = (r.standard_normal((C, D)) * r.uniform(0.01, 3.0, size=(C, 1))).astype(np.float32)
    cent[5] = 0.0  # a zero column: scale 0
    counts = r.integers(0, 40, size=C)
    counts[5] = 3
    q_heads = r.standard_normal((n_heads, D)).astype(np.float32)
    exact = O.score_communities(O.aggregate_query(q_heads), cent, counts)
    return cent, counts, q_heads, exact, c_cap


def _pad(s, scale, c_cap):
    sp = np.full(c_cap, -np.inf, np.float32)
    sp[:s.size] = s
    cp = np.zeros(c_cap, np.float32)
    cp[:scale.size] = scale
    return sp, cp


@pytest.mark.parametrize("seed,D,n_heads", [(1, 128, 1), (2, 64, 1), (3, 128, 4), (4, 64, 8)])
def test_plain_screening_meets_the_bound(seed, D, n_heads):
    cent, counts, q_heads, exact, c_cap = _case(seed, D, n_heads)
    s, scale = _screening(cent, q_heads, counts)
    sp, cp = _pad(s, scale, c_cap)
    PY._check_screening(sp, cp, q_heads, exact, counts, "plain")


def test_bound_is_not_vacuous():
    cent, counts, q_heads, exact, c_cap = _case(7, 128, 4)
    s, scale = _screening(cent, q_heads, counts)
    live = np.nonzero(counts > 0)[0]
    # a score moved just past its bound
    qbar = q_heads.astype(np.float64).sum(axis=0).astype(np.float32).astype(np.float64)
    c = int(live[live != 5][0])
    e = float(scale[c]) * np.abs(qbar).sum() * PY.screen_factor(128) + abs(float(s[c])) * 2.0 ** -21
    moved = s.copy()
    moved[c] = np.float32(float(exact[c]) + 1.5 * e)
    with pytest.raises(AssertionError, match="beyond its bound"):
        PY._check_screening(*_pad(moved, scale, c_cap), q_heads, exact, counts, "moved")
    # the scale left out, one head of a group left out
    for kw in (dict(drop_scale=True), dict(drop_head=True)):
        bad, _ = _screening(cent, q_heads, counts, **kw)
        with pytest.raises(AssertionError, match="beyond its bound"):
            PY._check_screening(*_pad(bad, scale, c_cap), q_heads, exact, counts, str(kw))
    # an empty community or an id past the count not scored -inf
    dead = s.copy()
    dead[int(np.nonzero(counts == 0)[0][0])] = 0.0
    with pytest.raises(AssertionError, match="not -inf"):
        PY._check_screening(*_pad(dead, scale, c_cap), q_heads, exact, counts, "dead")
    sp, cp = _pad(s, scale, c_cap)
    sp[-1] = 0.0
    with pytest.raises(AssertionError, match="not -inf"):
        PY._check_screening(sp, cp, q_heads, exact, counts, "past the count")
