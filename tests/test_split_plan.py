"""Pins of the split-KV partition model (oracle.split_plan).

The pages fix no partition, only that variable lengths are balanced by
splitting work; so the model is pinned by invariants that any valid plan
must satisfy plus the balance bound its own definition promises:

* every page of every request is covered exactly once, in order, by
  contiguous pieces;
* the closed-form split count equals the number of pieces produced;
* the per-part first_split index equals the piece's rank within its request,
  and split_offsets give disjoint, dense partial slots (<= 2(P-1) in total);
* no part carries more than quota + overhead units of work;
* the plan is deterministic.
"""
import numpy as np
import pytest
import torch

from oracle import fixed_cost_pages, num_pages, plan_pieces, rows_per_tile, split_plan
from workloads import WORKLOADS, draw_seqlens


def _check_plan(seqlens, s_q, h_q, P):
    tm, so = split_plan(seqlens, s_q, h_q, P)
    tm2, so2 = split_plan(seqlens, s_q, h_q, P)
    assert np.array_equal(tm, tm2) and np.array_equal(so, so2)
    B = len(seqlens)
    n = [num_pages(int(L)) for L in seqlens]
    pieces = plan_pieces(tm, seqlens)
    seen = {b: [] for b in range(B)}
    c = fixed_cost_pages(rows_per_tile(s_q, h_q))
    cost = [x + c if x > 0 else 0 for x in n]
    C = sum(cost)
    q = max(1, -(-C // P)) if C else 1
    for p, plist in enumerate(pieces):
        units = 0
        for i, (b, lo, hi) in enumerate(plist):
            seen[b].append((lo, hi, p, i))
            units += hi - lo
        # each part holds at most one quota of pages plus the overhead units
        assert units <= q + c, (p, units, q)
        # parts are consecutive in (request, page) order
        if p + 1 < P:
            assert tuple(tm[p, 2:4]) == tuple(tm[p + 1, 0:2])
    for b in range(B):
        segs = seen[b]
        cov = []
        for lo, hi, _, _ in segs:
            cov.extend(range(lo, hi))
        assert cov == list(range(n[b])), (b, segs)
        nsplit = len(segs) if n[b] > 0 else 1
        slots = int(so[b + 1] - so[b])
        assert slots == (nsplit if nsplit >= 2 else 0)
        # piece rank == first_split for the part that begins inside request b
        for rank, (lo, hi, p, i) in enumerate(segs):
            if i == 0 and tm[p, 0] == b and tm[p, 1] > 0:
                assert tm[p, 4] == rank, (b, p, rank, tm[p])
            if lo == 0:
                assert rank == 0
    assert int(so[-1]) <= max(0, 2 * (P - 1))
    assert np.all(np.diff(so) >= 0)
    return tm, so


@pytest.mark.parametrize("P", [1, 2, 3, 7, 64, 256])
@pytest.mark.parametrize("seqlens", [
    [65, 130], [1], [0, 5, 0], [4096] * 8, [64, 64, 64], [1, 2, 3, 5000, 7, 63, 64, 65],
    [0, 0, 0],
])
@pytest.mark.parametrize("s_q,h_q", [(1, 16), (1, 128), (2, 128)])
def test_plan_invariants(seqlens, P, s_q, h_q):
    _check_plan(seqlens, s_q, h_q, P)


@pytest.mark.parametrize("key", ["tiny", "membound", "ridge", "ragged", "long", "draft"])
def test_plan_invariants_workloads(key):
    w = WORKLOADS[key]
    gen = torch.Generator().manual_seed(w.seed)
    sl = [int(x) for x in draw_seqlens(w.seqlen_kind, w.batch, gen)]
    P = 256 if w.rows <= 128 else 128
    _check_plan(sl, w.s_q, w.h_q, P)


def test_plan_balance_random():
    g = np.random.default_rng(0)
    for _ in range(30):
        B = int(g.integers(1, 40))
        sl = [int(x) for x in g.integers(0, 3000, size=B)]
        P = int(g.integers(1, 300))
        _check_plan(sl, 1, int(g.choice([16, 32, 64, 128])), P)


def test_plan_known_small():
    # two requests of 2 and 3 pages, overhead 1 each -> costs 3 and 4, C = 7.
    tm, so = split_plan([65, 130], 1, 16, 256)
    # q = 1: every unit boundary is a part boundary; pages become single pieces
    pieces = [p for p in plan_pieces(tm, [65, 130]) if p]
    assert pieces == [[(0, 0, 1)], [(0, 1, 2)], [(1, 0, 1)], [(1, 1, 2)], [(1, 2, 3)]]
    assert list(so) == [0, 2, 5]
    tm, so = split_plan([65, 130], 1, 16, 1)
    assert list(tm[0, :5]) == [0, 0, 2, 0, 0]
    assert list(so) == [0, 0, 0]
