"""Host logic of the verify-cost price table: the timing trees and the price lookup."""
import itertools

import pytest

from hybrid_deltanet_tree_amd import price_table as pt


def _depths(parent):
    d = []
    for p in parent:
        d.append(0 if p < 0 else d[p] + 1)
    return d


@pytest.mark.parametrize("n", [1, 2, 3, 4, 8, 12, 13, 16, 24, 32, 64])
def test_timing_trees_are_valid_trees(n):
    parent = pt.tree_of(n)
    assert len(parent) == n and parent[0] == -1
    assert all(0 <= p < i for i, p in enumerate(parent) if i > 0)  # parent order
    assert max(_depths(parent)) <= min(n - 1, 12)
    assert parent[:min(n, 12)] == [-1] + list(range(min(n, 12) - 1))  # the chain


@pytest.mark.parametrize("n", [1, 5, 16, 24, 32])
def test_deepest_path_brute_force(n):
    parent = pt.tree_of(n)
    d = _depths(parent)
    path = pt.deepest_path(parent)
    want = min((i for i in range(n) if d[i] == max(d)))
    assert path[-1] == want and path[0] == 0 and len(path) == d[want] + 1
    assert all(parent[b] == a for a, b in zip(path, path[1:]))


def _table():
    # verify_ms = 0.01 n + 1e-5 L + s: linear in context, so lookups are exact
    return {"entries": [dict(n_nodes=n, context=L, slots=s, verify_ms=0.01 * n + 1e-5 * L + s)
                        for n, L, s in itertools.product((4, 16, 32), (1000, 3000, 9000), (1, 4))]}


def test_lookup_exact_points_and_interpolation():
    t = _table()
    for n, L, s in itertools.product((4, 16, 32), (1000, 3000, 9000), (1, 4)):
        assert pt.lookup(t, n, L, s) == pytest.approx(0.01 * n + 1e-5 * L + s)
    assert pt.lookup(t, 16, 2000, 1) == pytest.approx(0.16 + 0.02 + 1)
    assert pt.lookup(t, 16, 6000, 4) == pytest.approx(0.16 + 0.06 + 4)


def test_lookup_rounds_up_and_clamps():
    t = _table()
    assert pt.lookup(t, 5, 3000, 1) == pt.lookup(t, 16, 3000, 1)   # next measured tree size
    assert pt.lookup(t, 4, 3000, 2) == pt.lookup(t, 4, 3000, 4)    # next measured slot count
    assert pt.lookup(t, 4, 10, 1) == pt.lookup(t, 4, 1000, 1)      # below the first context
    assert pt.lookup(t, 4, 12000, 1) == pytest.approx(0.04 + 0.12 + 1)  # linear beyond
    with pytest.raises(KeyError):
        pt.lookup(t, 33, 3000, 1)
    with pytest.raises(KeyError):
        pt.lookup(t, 4, 3000, 5)


def test_shipped_price_file():
    # the MI355X price file of the 64-layer bf16 stack: a full grid, positive prices that
    # grow with the context (measurement noise aside)
    t = pt.load()
    rows = t["entries"]
    grid = {(r["n_nodes"], r["context"], r["slots"]) for r in rows}
    ns = sorted({r["n_nodes"] for r in rows})
    Ls = sorted({r["context"] for r in rows})
    ss = sorted({r["slots"] for r in rows})
    assert len(grid) == len(rows) == len(ns) * len(Ls) * len(ss)
    assert ns[0] == 1 and ns[-1] >= 32 and Ls[-1] >= 262144 and ss == [1, 2, 4]
    for r in rows:
        assert 0 < r["verify_p10_ms"] <= r["verify_ms"] <= r["verify_p90_ms"]
        assert 0 < r["commit_ms"] < r["verify_ms"]
    for n in ns:
        for s in ss:
            v = [pt.lookup(t, n, L, s) for L in Ls]
            assert all(b >= 0.98 * a for a, b in zip(v, v[1:])), (n, s, v)
