"""Pins for the oracle's transposed grouped matmul (tgmm, the weight gradient
of gmm), CPU only.

tgmm is tied to things other than its own loop: a library matmul for one
group, the gradient of the (separately pinned) gmm oracle's forward taken by
exact finite differences, a pure-Python triple loop, and the identities the
operation must satisfy (operand swap, empty groups, shard offset, rows
outside the active groups).  The last tests plant plausible mistakes (a
group boundary off by one, a transposed output, an offset not applied) and
check that the pins reject them."""
import numpy as np
import pytest
import torch

import oracle


def _int_tensor(g, shape, lim=3):
    # small integers: every product and sum below is exact in float64
    return torch.randint(-lim, lim + 1, shape, generator=g).to(torch.float32)


def _segments(sizes):
    o = np.concatenate([[0], np.cumsum(sizes)]).astype(int)
    return o


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_tgmm_single_group_is_dense_matmul(dtype):
    g = torch.Generator().manual_seed(11)
    lhs = torch.randn(37, 12, generator=g).to(dtype)
    rhs = torch.randn(37, 9, generator=g).to(dtype)
    got = oracle.tgmm_reference(lhs, rhs, torch.tensor([37], dtype=torch.int32))
    want = torch.mm(lhs.double().t(), rhs.double()).numpy()
    np.testing.assert_allclose(got[0], want, rtol=1e-12, atol=1e-12)


def test_tgmm_is_the_weight_gradient_of_gmm():
    """For the NN forward out = gmm(lhs, W, transpose_rhs=True), W [Ga,K,N],
    L(W) = sum(out * dout) is linear in W and dL/dW[h,k,n] = tgmm(lhs, dout)[h,k,n].
    With integer data, L(W + e_hkn) - L(W) equals that entry exactly."""
    g = torch.Generator().manual_seed(5)
    sizes = [3, 0, 5, 4, 2]  # group 1 empty; rows 14..15 belong to no group
    s, Ga = 1, 3             # active groups 1, 2, 3
    M, K, N = 16, 4, 3
    lhs = _int_tensor(g, (M, K))
    dout = _int_tensor(g, (M, N))
    W = _int_tensor(g, (Ga, K, N))
    gs = torch.tensor(sizes, dtype=torch.int32)

    def loss(w):
        out = oracle.gmm_reference(lhs, w, gs, group_offset=s, transpose_rhs=True)
        return float((out * dout.double().numpy()).sum())

    base = loss(W)
    grad = np.zeros((Ga, K, N))
    for h in range(Ga):
        for k in range(K):
            for n in range(N):
                w2 = W.clone()
                w2[h, k, n] += 1.0
                grad[h, k, n] = loss(w2) - base
    got = oracle.tgmm_reference(lhs, dout, gs, group_offset=s, num_active=Ga)
    assert np.array_equal(got, grad)
    assert np.array_equal(got[0], np.zeros((K, N)))  # the empty group


def test_tgmm_matches_python_loops():
    g = torch.Generator().manual_seed(9)
    sizes = [2, 4, 0, 3]
    M, K, N = 11, 3, 5
    lhs = torch.randn(M, K, generator=g)
    rhs = torch.randn(M, N, generator=g)
    got = oracle.tgmm_reference(lhs, rhs, torch.tensor(sizes, dtype=torch.int32))
    L, R = lhs.double().tolist(), rhs.double().tolist()
    o = _segments(sizes)
    for h in range(len(sizes)):
        for k in range(K):
            for n in range(N):
                t = 0.0
                for r in range(o[h], o[h + 1]):
                    t += L[r][k] * R[r][n]
                assert got[h, k, n] == t


def test_tgmm_operand_swap_is_transpose_bit_exact():
    g = torch.Generator().manual_seed(3)
    sizes = [6, 0, 9, 5]
    lhs = torch.randn(22, 7, generator=g).to(torch.bfloat16)
    rhs = torch.randn(22, 4, generator=g).to(torch.bfloat16)
    gs = torch.tensor(sizes, dtype=torch.int32)
    a = oracle.tgmm_reference(lhs, rhs, gs)
    b = oracle.tgmm_reference(rhs, lhs, gs)
    assert np.array_equal(a, b.transpose(0, 2, 1))


def test_tgmm_shard_offset_and_foreign_rows():
    g = torch.Generator().manual_seed(4)
    sizes = [4, 0, 7, 3, 5]
    M = sum(sizes) + 3
    lhs = torch.randn(M, 6, generator=g)
    rhs = torch.randn(M, 5, generator=g)
    gs = torch.tensor(sizes, dtype=torch.int32)
    full = oracle.tgmm_reference(lhs, rhs, gs)
    assert np.array_equal(full[1], np.zeros((6, 5)))
    s, Ga = 1, 3
    shard = oracle.tgmm_reference(lhs, rhs, gs, group_offset=s, num_active=Ga)
    assert np.array_equal(shard, full[s:s + Ga])
    # rows of inactive groups and rows past the groups do not contribute
    o = _segments(sizes)
    lhs2, rhs2 = lhs.clone(), rhs.clone()
    lhs2[:o[s]] = 99.0
    rhs2[o[s + Ga]:] = -7.0
    assert np.array_equal(oracle.tgmm_reference(lhs2, rhs2, gs, group_offset=s, num_active=Ga), shard)


def test_tgmm_selection_matches_full():
    g = torch.Generator().manual_seed(8)
    sizes = [5, 3, 0, 8]
    lhs = torch.randn(16, 9, generator=g)
    rhs = torch.randn(16, 4, generator=g)
    gs = torch.tensor(sizes, dtype=torch.int32)
    full = oracle.tgmm_reference(lhs, rhs, gs)
    sel = [(3, 8), (0, 0), (2, 4), (1, 5)]
    part = oracle.tgmm_reference(lhs, rhs, gs, select=sel)
    for i, (h, k) in enumerate(sel):
        assert np.array_equal(part[i], full[h, k])


def test_tgmm_invalid_data_is_rejected():
    lhs = torch.zeros(4, 2)
    rhs = torch.zeros(4, 2)
    with pytest.raises(oracle.OracleError):
        oracle.tgmm_reference(lhs, rhs, torch.tensor([3, 2], dtype=torch.int32))  # sum > M
    with pytest.raises(oracle.OracleError):
        oracle.tgmm_reference(lhs, rhs, torch.tensor([-1, 2], dtype=torch.int32))
    with pytest.raises(oracle.OracleError):
        oracle.tgmm_reference(lhs, rhs, torch.tensor([1, 2], dtype=torch.int32), group_offset=1, num_active=2)


# ------------------------------------------------------ planted mistakes

def _grad_case():
    g = torch.Generator().manual_seed(21)
    sizes = [3, 0, 5, 4]
    lhs = _int_tensor(g, (12, 4))
    dout = _int_tensor(g, (12, 4))  # K == N, so a transposed output still fits
    return sizes, lhs, dout


def _segment_grads(sizes, lhs, dout):
    o = _segments(sizes)
    return np.stack([(lhs[o[h]:o[h + 1]].double().t() @ dout[o[h]:o[h + 1]].double()).numpy()
                     for h in range(len(sizes))])


def test_planted_boundary_off_by_one_is_caught():
    sizes, lhs, dout = _grad_case()
    want = _segment_grads(sizes, lhs, dout)
    shifted = list(sizes)
    shifted[2] += 1
    shifted[3] -= 1
    mutant = oracle.tgmm_reference(lhs, dout, torch.tensor(shifted, dtype=torch.int32))
    assert not np.array_equal(mutant, want)
    assert np.array_equal(oracle.tgmm_reference(lhs, dout, torch.tensor(sizes, dtype=torch.int32)), want)


def test_planted_transposed_output_is_caught():
    sizes, lhs, dout = _grad_case()
    want = _segment_grads(sizes, lhs, dout)
    mutant = oracle.tgmm_reference(lhs, dout, torch.tensor(sizes, dtype=torch.int32)).transpose(0, 2, 1)
    assert not np.array_equal(mutant, want)


def test_planted_offset_not_applied_is_caught():
    sizes, lhs, dout = _grad_case()
    want = _segment_grads(sizes, lhs, dout)[2:4]
    # indexing the output by the absolute group instead of g - s gives groups 0, 1
    mutant = oracle.tgmm_reference(lhs, dout, torch.tensor(sizes, dtype=torch.int32))[0:2]
    assert not np.array_equal(mutant, want)
    got = oracle.tgmm_reference(lhs, dout, torch.tensor(sizes, dtype=torch.int32), group_offset=2, num_active=2)
    assert np.array_equal(got, want)
