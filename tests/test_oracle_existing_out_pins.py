"""Pins for the oracle's existing_out (gmm's existing_out on the tpu-inference
wheel diff pages, megablox/gmm.py: each output tile starts from it, only the
rows of the tile's group are stored over it, and no zero fill follows), CPU
only.

The pins tie it to facts other than its own code: an all-zero existing_out
gives the zero-filled result bit for bit; active rows do not depend on it
(checked against per-segment torch products); every other row is the
existing row's exact value (checked row by row against the group bounds
computed here); and the use the argument exists for -- merging expert shards
into one output -- reproduces the unsharded result exactly.  The last test
plants a mistake (existing rows dropped to zero) and checks that the pins
reject it."""
import numpy as np
import torch

import oracle


def _case(seed, sizes, extra, K, N, Ga=None, s=0):
    g = torch.Generator().manual_seed(seed)
    M = sum(sizes) + extra
    Ga = len(sizes) - s if Ga is None else Ga
    lhs = torch.randn(M, K, generator=g)
    rhs = torch.randn(Ga, N, K, generator=g)
    existing = torch.randn(M, N, generator=g) * 5
    return lhs, rhs, torch.tensor(sizes, dtype=torch.int32), existing


def _bounds(sizes, s, Ga):
    o = np.concatenate([[0], np.cumsum(sizes)]).astype(int)
    return o[s], o[s + Ga]


def test_zero_existing_out_is_the_zero_filled_result():
    sizes = [3, 0, 6, 2]
    lhs, rhs, gs, _ = _case(1, sizes, 4, 16, 8, Ga=2, s=1)
    base = oracle.gmm_reference(lhs, rhs, gs, group_offset=1)
    got = oracle.gmm_reference(lhs, rhs, gs, group_offset=1, existing_out=torch.zeros(lhs.shape[0], 8))
    assert np.array_equal(got, base)


def test_active_rows_do_not_depend_on_existing_out():
    sizes = [4, 5, 0, 3, 2]
    s, Ga = 1, 3
    lhs, rhs, gs, existing = _case(2, sizes, 3, 24, 12, Ga=Ga, s=s)
    got = oracle.gmm_reference(lhs, rhs, gs, group_offset=s, existing_out=existing)
    lo, hi = _bounds(sizes, s, Ga)
    o = np.concatenate([[0], np.cumsum(sizes)]).astype(int)
    for h in range(Ga):
        a, b = o[s + h], o[s + h + 1]
        want = (lhs[a:b].double() @ rhs[h].double().t()).numpy()
        np.testing.assert_allclose(got[a:b], want, rtol=1e-12, atol=1e-12)
    assert hi - lo == 8


def test_rows_outside_the_active_groups_are_existing_rows_exactly():
    sizes = [2, 7, 0, 4, 3]
    s, Ga = 1, 2
    lhs, rhs, gs, existing = _case(3, sizes, 5, 16, 8, Ga=Ga, s=s)
    got = oracle.gmm_reference(lhs, rhs, gs, group_offset=s, existing_out=existing)
    lo, hi = _bounds(sizes, s, Ga)
    ex = existing.double().numpy()
    for r in range(lhs.shape[0]):
        if not lo <= r < hi:
            assert np.array_equal(got[r], ex[r]), r


def test_selected_rows_take_their_own_existing_rows():
    sizes = [3, 3, 3]
    lhs, rhs, gs, existing = _case(4, sizes, 2, 16, 8, Ga=1, s=1)
    full = oracle.gmm_reference(lhs, rhs, gs, group_offset=1, existing_out=existing)
    rows = [10, 0, 4, 7, 2]
    part = oracle.gmm_reference(lhs, rhs, gs, group_offset=1, existing_out=existing, rows=rows)
    assert np.array_equal(part, full[rows])


def test_merging_expert_shards_reproduces_the_full_result():
    """Two shards of the experts, each with its slice of the weights: the
    first writes zeros outside its rows, the second is given that output as
    existing_out (float64, so nothing is rounded in between)."""
    sizes = [5, 0, 3, 6, 2, 4]
    lhs, rhs, gs, _ = _case(5, sizes, 3, 32, 16)
    full = oracle.gmm_reference(lhs, rhs, gs)
    a = oracle.gmm_reference(lhs, rhs[:3].contiguous(), gs, group_offset=0)
    merged = oracle.gmm_reference(lhs, rhs[3:].contiguous(), gs, group_offset=3,
                                  existing_out=torch.from_numpy(a))
    assert np.array_equal(merged, full)


def test_planted_existing_rows_dropped_is_caught():
    sizes = [2, 7, 0, 4, 3]
    s, Ga = 1, 2
    lhs, rhs, gs, existing = _case(3, sizes, 5, 16, 8, Ga=Ga, s=s)
    got = oracle.gmm_reference(lhs, rhs, gs, group_offset=s, existing_out=existing)
    mutant = oracle.gmm_reference(lhs, rhs, gs, group_offset=s)  # the zero fill in place of existing rows
    lo, hi = _bounds(sizes, s, Ga)
    ex = existing.double().numpy()
    assert np.array_equal(got[:lo], ex[:lo]) and np.array_equal(got[hi:], ex[hi:])
    assert not (np.array_equal(mutant[:lo], ex[:lo]) and np.array_equal(mutant[hi:], ex[hi:]))
