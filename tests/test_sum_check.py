"""The full-size tests' every-element sum check (parity.sum_check), on the CPU.

A correct output (the oracle's exact values rounded once to bf16, as a
kernel stores them) passes the row and per-group column sums at the
tolerance the full-size tests use; outputs with one planted mistake of the
kinds a tiled kernel makes -- a 256 x 256 tile stored one tile to the right,
a tile computed with the next group's weight, a 32-row block left unwritten
-- fail it."""
import numpy as np
import torch

import oracle
from parity import BF16_SUM_SD, sum_check


def _case():
    g = torch.Generator().manual_seed(5)
    sizes = [700, 0, 333, 900, 67]
    M, K, N = sum(sizes), 384, 768
    lhs = (torch.randn(M, K, generator=g) * 0.02).to(torch.bfloat16)
    rhs = (torch.randn(len(sizes), N, K, generator=g) * 0.02).to(torch.bfloat16)
    return sizes, lhs, rhs


def _sums(out, sizes):
    x = out.double()
    o = np.concatenate([[0], np.cumsum(sizes)])
    cols = np.stack([x[o[g]:o[g + 1]].sum(0).numpy() for g in range(len(sizes))])
    col_ss = np.stack([x[o[g]:o[g + 1]].square().sum(0).sqrt().numpy() for g in range(len(sizes))])
    col_abs = np.stack([x[o[g]:o[g + 1]].abs().sum(0).numpy() for g in range(len(sizes))])
    return (x.sum(1).numpy(), x.square().sum(1).sqrt().numpy(), x.abs().sum(1).numpy(), cols, col_ss, col_abs)


def _want(sizes, lhs, rhs):
    gs = torch.tensor(sizes, dtype=torch.int32)
    w_red = rhs.double().sum(1, keepdim=True).float()
    want_row = oracle.gmm_reference(lhs, w_red, gs)[:, 0]
    o = np.concatenate([[0], np.cumsum(sizes)])
    lhs_red = torch.stack([lhs[o[g]:o[g + 1]].double().sum(0) for g in range(len(sizes))]).float()
    want_col = oracle.gmm_reference(lhs_red, rhs, torch.ones(len(sizes), dtype=torch.int32))
    return want_row, want_col


def _passes(out, sizes, want_row, want_col):
    row, row_ss, row_abs, col, col_ss, col_abs = _sums(out, sizes)
    try:
        sum_check(row, want_row, BF16_SUM_SD * row_ss, row_abs, "rows")
        sum_check(col, want_col, BF16_SUM_SD * col_ss, col_abs, "columns")
        return True
    except AssertionError:
        return False


def test_sum_check_passes_a_correct_output_and_fails_planted_mistakes():
    sizes, lhs, rhs = _case()
    gs = torch.tensor(sizes, dtype=torch.int32)
    exact = oracle.gmm_reference(lhs, rhs, gs)
    out = oracle.round_to(exact, torch.bfloat16)
    want_row, want_col = _want(sizes, lhs, rhs)
    assert _passes(out, sizes, want_row, want_col)

    # a tile stored one tile to the right (rows 256..511 of group 0)
    bad = out.clone()
    bad[256:512, 256:512] = out[256:512, 0:256]
    assert not _passes(bad, sizes, want_row, want_col)

    # a tile computed with the next group's weight (rows of group 2, columns 0..255)
    o = np.concatenate([[0], np.cumsum(sizes)])
    wrong = oracle.gmm_reference(lhs[o[2]:o[3]], rhs[3:4], torch.tensor([sizes[2]], dtype=torch.int32))
    bad = out.clone()
    bad[o[2]:o[2] + 256, 0:256] = oracle.round_to(wrong[:256, 0:256], torch.bfloat16)
    assert not _passes(bad, sizes, want_row, want_col)

    # a 32-row block of one tile left unwritten (zeros)
    bad = out.clone()
    bad[o[3] + 64:o[3] + 96, 512:768] = 0
    assert not _passes(bad, sizes, want_row, want_col)
