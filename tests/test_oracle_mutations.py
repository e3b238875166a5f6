"""Planted mistakes (CPU only): each test computes what an oracle with one
plausible bug would return -- by running the real oracle on inputs that
reproduce the bug's effect -- and checks that the pins' own comparisons
reject it.  This shows the pins in test_oracle_pins.py are sensitive to:
a dropped bias, a row mapped to the neighbouring group, a transposed
operand, a wrong quantisation-block index, a per-token scale taken from the
wrong row, a sign error, and a group offset that is not subtracted."""
import numpy as np
import torch

import oracle
from test_oracle_pins import _rand_case, _torch_blocks, _torch_segments


def _close(a, b):
    return np.allclose(a, b, rtol=1e-11, atol=1e-11)


def _scaled_case():
    sizes = [6, 0, 9, 4]
    M, K, N, nb = 21, 64, 12, 4
    g = torch.Generator().manual_seed(8)
    lhs = torch.randn(M, K, generator=g)
    rhs = torch.randn(4, N, K, generator=g)
    rs = torch.rand(4, nb, 1, N, generator=g) + 0.5
    ls = torch.rand(M, nb, generator=g) + 0.25
    bias = torch.randn(4, 1, N, generator=g)
    return sizes, lhs, rhs, rs, ls, bias, nb


def test_dropped_bias_is_caught():
    sizes, lhs, rhs, rs, ls, bias, nb = _scaled_case()
    gs = torch.tensor(sizes, dtype=torch.int32)
    want = _torch_blocks(lhs, rhs, sizes, rs, ls, bias, nb)
    assert _close(oracle.gmm_reference(lhs, rhs, gs, rhs_scale=rs, lhs_scale=ls, rhs_bias=bias), want)
    mutant = oracle.gmm_reference(lhs, rhs, gs, rhs_scale=rs, lhs_scale=ls)
    assert not _close(mutant, want)


def test_wrong_block_index_is_caught():
    sizes, lhs, rhs, rs, ls, bias, nb = _scaled_case()
    gs = torch.tensor(sizes, dtype=torch.int32)
    want = _torch_blocks(lhs, rhs, sizes, rs, ls, bias, nb)
    mutant = oracle.gmm_reference(lhs, rhs, gs, rhs_scale=rs.flip(1).contiguous(), lhs_scale=ls, rhs_bias=bias)
    assert not _close(mutant, want)


def test_token_scale_from_wrong_row_is_caught():
    sizes, lhs, rhs, rs, ls, bias, nb = _scaled_case()
    gs = torch.tensor(sizes, dtype=torch.int32)
    want = _torch_blocks(lhs, rhs, sizes, rs, ls, bias, nb)
    mutant = oracle.gmm_reference(lhs, rhs, gs, rhs_scale=rs, lhs_scale=ls.roll(1, 0).contiguous(),
                                  rhs_bias=bias)
    assert not _close(mutant, want)


def test_row_mapped_to_neighbouring_group_is_caught():
    # the bias probe: rhs = 0, bias[g] = g + 1 reads back each row's group
    sizes = [2, 0, 5, 1, 0, 3]
    M = sum(sizes) + 2
    lhs, _, _ = _rand_case(7, M, 16, 8, sizes)
    rhs = torch.zeros(len(sizes), 8, 16)
    bias = (torch.arange(len(sizes), dtype=torch.float32) + 1)[:, None, None].expand(-1, 1, 8).contiguous()
    row_group = np.repeat(np.arange(len(sizes)), sizes)
    want = np.repeat((row_group + 1)[:, None], 8, axis=1)
    shifted = list(sizes)
    shifted[0] += 1
    shifted[2] -= 1  # group boundaries off by one row
    mutant = oracle.gmm_reference(lhs, rhs, torch.tensor(shifted, dtype=torch.int32), rhs_bias=bias)
    assert not np.array_equal(mutant[:sum(sizes)], want)


def test_transposed_operand_is_caught():
    sizes = [5, 0, 7, 4]
    M = sum(sizes)
    lhs, rhs, gs = _rand_case(3, M, 24, 24, sizes)  # square N = K, so a transposed weight still fits
    want = _torch_segments(lhs, rhs, sizes)
    mutant = oracle.gmm_reference(lhs, rhs.transpose(1, 2).contiguous(), gs)
    assert not _close(mutant, want)


def test_sign_error_is_caught():
    sizes = [5, 0, 7, 4]
    lhs, rhs, gs = _rand_case(3, sum(sizes), 24, 16, sizes)
    want = _torch_segments(lhs, rhs, sizes)
    assert not _close(-oracle.gmm_reference(lhs, rhs, gs), want)


def test_group_offset_not_subtracted_is_caught():
    # the shard run must index its local weights by g - s; indexing the full
    # weight tensor by the local slot instead gives other groups' weights
    sizes = [3, 0, 8, 2, 5]
    M = sum(sizes)
    lhs, rhs, gs = _rand_case(6, M, 24, 16, sizes)
    full = oracle.gmm_reference(lhs, rhs, gs)
    s, ga = 2, 3
    o = np.concatenate([[0], np.cumsum(sizes)])
    mutant = oracle.gmm_reference(lhs, rhs[:ga].contiguous(), gs, group_offset=s)
    assert not np.array_equal(mutant[o[s]:o[s + ga]], full[o[s]:o[s + ga]])
