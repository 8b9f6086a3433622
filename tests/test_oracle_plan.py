"""Pins of the oracle's zigzag plan (CPU only).

The plan is integer work, so it is pinned exactly: against the cases the
rank-share workloads state (tests/golden/zigzag_plans.txt), against the
closed form of the zigzag rule, and against the invariants the partition must
satisfy (exact cover of the sequence, equal causal work per rank, identity at
D = 1).
"""
import pytest
import torch

from oracle import tsp_oracle as O


def test_golden_cases(golden):
    for S, D, r, C, c0, c1, s0, s1 in (map(int, row) for row in golden("zigzag_plans.txt")):
        p = O.zigzag_plan(S, D, r)
        assert p.chunk_len == C
        assert p.chunk_ids == [c0, c1]
        assert p.chunk_starts == [s0, s1]
        assert p.local_to_global[0].item() == s0
        assert p.local_to_global[C - 1].item() == s0 + C - 1
        assert p.local_to_global[C].item() == s1
        assert p.local_to_global[-1].item() == s1 + C - 1


GRID = [(2, 1), (4, 1), (8, 2), (24, 3), (64, 4), (2048, 4), (96, 6), (256, 8), (1024, 16)]


@pytest.mark.parametrize("S,D", GRID)
def test_exact_cover(S, D):
    seen = torch.zeros(S, dtype=torch.int64)
    for r in range(D):
        p = O.zigzag_plan(S, D, r)
        assert p.local_to_global.numel() == S // D
        seen.index_add_(0, p.local_to_global, torch.ones(S // D, dtype=torch.int64))
    assert torch.equal(seen, torch.ones(S, dtype=torch.int64))


@pytest.mark.parametrize("S,D", GRID)
def test_closed_form_and_ascending(S, D):
    C = S // (2 * D)
    for r in range(D):
        p = O.zigzag_plan(S, D, r)
        assert p.chunk_ids == [r, 2 * D - 1 - r]
        l2g = p.local_to_global
        assert bool((l2g[1:] > l2g[:-1]).all())
        i = torch.arange(S // D)
        expect = torch.where(i < C, r * C + i, (2 * D - 1 - r) * C + (i - C))
        assert torch.equal(l2g, expect)


@pytest.mark.parametrize("S,D", GRID)
def test_equal_causal_work(S, D):
    # number of (query, key) pairs with key <= query, per rank: 2D*C^2 + C
    C = S // (2 * D)
    for r in range(D):
        p = O.zigzag_plan(S, D, r)
        assert int((p.local_to_global + 1).sum()) == 2 * D * C * C + C


def test_identity_at_D1():
    p = O.zigzag_plan(64, 1, 0)
    assert torch.equal(p.local_to_global, torch.arange(64))
    assert p.ring == [0]


@pytest.mark.parametrize("D", [1, 2, 3, 4, 8, 16])
def test_ring_order(D):
    for r in range(D):
        ring = O.zigzag_plan(2 * D * 4, D, r).ring
        assert ring[0] == r
        assert sorted(ring) == list(range(D))
        assert all(ring[(k + 1) % D] == (ring[k] + 1) % D for k in range(D))


@pytest.mark.parametrize("S,D,r", [(30, 4, 0), (16, 0, 0), (16, 2, 2), (16, 2, -1), (0, 2, 0)])
def test_rejects_bad_arguments(S, D, r):
    with pytest.raises(ValueError):
        O.zigzag_plan(S, D, r)
