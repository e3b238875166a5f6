"""Full-size parity: every workload at its full shape, launched as the
benchmark launches it (automatic tile choice, caller-allocated output),
against the oracle.

- tiny_fp32 and decode_fp8w (small enough): every active row, every element.
- moe_fwd_bf16, moe_dlhs_bf16, w8a8_fp8: sampled rows -- each active group's
  first and last row, both sides of every 256- and 32-row tile boundary (up
  to a few thousand rows), random rows per group and overall.
- Always: rows outside the active groups are all-zero bits (checked on the
  device over all M rows) and no device data flag is raised.
- moe_fwd_bf16, moe_dlhs_bf16, w8a8_fp8 and the weight gradient tgmm_bf16:
  every element, through row and per-group column sums against the oracle
  on reduced operands (see below).

Tolerances are those of tests/parity.py (float32: max error 1e-4 of the
largest reference value; bfloat16: relative Frobenius error 2e-2, globally
and per row)."""
import numpy as np
import pytest
import torch

import workloads
from parity import BF16_SUM_SD, active_range, assert_zero_rows, compare, reference, sample_rows, sum_check

pytestmark = pytest.mark.gpu

EVERY_ROW = {"tiny_fp32", "decode_fp8w"}


@pytest.mark.parametrize("name", list(workloads.FULL))
def test_full_size_against_oracle(name):
    import moe_grouped_matrix_amd as gmm_amd
    gmm_amd.set_tile_policy(0)
    case = workloads.FULL[name](device="cuda")
    print(f"full case {name}: M={case.M} K={case.K} N={case.N} G={case.group_sizes.numel()} "
          f"Ga={case.num_active} offset={case.group_offset} active_rows={case.active_rows()}", flush=True)
    out = torch.empty((case.M, case.N), dtype=case.out_dtype, device="cuda")
    off = (torch.tensor([case.group_offset], dtype=torch.int32, device="cuda")
           if case.group_offset else None)
    gmm_amd.gmm(case.lhs, case.rhs, case.group_sizes, rhs_scale=case.rhs_scale, rhs_bias=case.rhs_bias,
                lhs_scale=case.lhs_scale, group_offset=off, transpose_rhs=case.transpose_rhs, out=out)
    torch.cuda.synchronize()
    assert gmm_amd.device_flags() == 0

    lo, hi = active_range(case)
    assert_zero_rows(out, lo, hi)
    if name in EVERY_ROW:
        rows = list(range(lo, hi))
    else:
        rows = sample_rows(case, tm_list=(256, 32), per_group=4, extra=64, seed=7)
    ref = reference(case, rows=rows)
    got = out[torch.tensor(rows, dtype=torch.long, device="cuda")].cpu()
    rel = compare(got, ref, case.out_dtype, f"{name} ({len(rows)} rows)")
    print(f"full case {name}: {len(rows)} rows compared, error {rel:.3e}", flush=True)


# ---------------------------------------------------------------------------
# Every element at full size, through sums.  The sampled rows above leave
# most of the full-size outputs unread; these identities read all of them:
#   sum_n out[r, n]             = lhs[r, :] . (sum_n W_g[:, n])      (every row r)
#   sum_{r in g} out[r, n]      = (sum_{r in g} lhs[r, :]) . W_g[:, n]  (every group g, column n)
# and for tgmm, out[h] = lhs_g^T rhs_g:
#   sum_n out[h, k, n]          = sum_{r in g} lhs[r, k] (sum_n rhs[r, n])
#   sum_k out[h, k, n]          = sum_{r in g} (sum_k lhs[r, k]) rhs[r, n]
# The right-hand sides come from the oracle on operands reduced in float64
# (rounded once to float32 to pass them in: a relative 2^-24 per entry).  A
# tile stored in the wrong place, skipped or summed over the wrong rows
# moves a sum by about the root of the sum of squares of the tile's values;
# the tolerance is a few of the rounding errors' standard deviation: the
# output rounding (bf16 round to nearest: within half a unit in the last
# place, at most 2^-8 of the value, about uniform, so a sum's spread is at
# most 2^-8/sqrt(3) of the root of the sum of squares; f32 outputs: the
# per-element tolerance of tests/parity.py, 1e-4 of the largest value, over
# the root of the count) with a factor of 8, plus 1e-5 of the sum of
# magnitudes for the float32 accumulation (parity.sum_check;
# tests/test_sum_check.py shows on the CPU that a misplaced tile fails it).

SUM_CASES = ["moe_fwd_bf16", "moe_dlhs_bf16"]


def _segments(sizes):
    o = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    return o


@pytest.mark.parametrize("name", SUM_CASES)
def test_full_size_every_element_by_sums(name):
    import oracle
    import moe_grouped_matrix_amd as gmm_amd
    gmm_amd.set_tile_policy(0)
    case = workloads.FULL[name](device="cuda")
    assert case.group_offset == 0 and case.rhs_scale is None and case.lhs_scale is None and case.rhs_bias is None
    print(f"sums case {name}: M={case.M} K={case.K} N={case.N}", flush=True)
    out = torch.empty((case.M, case.N), dtype=case.out_dtype, device="cuda")
    gmm_amd.gmm(case.lhs, case.rhs, case.group_sizes, transpose_rhs=case.transpose_rhs, out=out)
    torch.cuda.synchronize()
    assert gmm_amd.device_flags() == 0
    sizes = case.sizes_list()
    o = _segments(sizes)
    M, N = case.M, case.N
    # the device's sums, in float64, 32768 rows at a time
    row_sum, row_ss, row_abs = [], [], []
    for i in range(0, M, 32768):
        x = out[i:i + 32768].double()
        row_sum.append(x.sum(1).cpu())
        row_ss.append(x.square().sum(1).sqrt().cpu())
        row_abs.append(x.abs().sum(1).cpu())
    row_sum, row_ss, row_abs = (torch.cat(v).numpy() for v in (row_sum, row_ss, row_abs))
    col_sum = np.zeros((len(sizes), N))
    col_ss = np.zeros((len(sizes), N))
    col_abs = np.zeros((len(sizes), N))
    for g in range(len(sizes)):
        if sizes[g]:
            x = out[o[g]:o[g + 1]].double()
            col_sum[g], col_ss[g], col_abs[g] = (x.sum(0).cpu().numpy(), x.square().sum(0).sqrt().cpu().numpy(),
                                                 x.abs().sum(0).cpu().numpy())
    # the oracle's sums through the reduced operands
    lhs, rhs, gs = case.lhs.cpu(), case.rhs.cpu(), case.group_sizes.cpu()
    w_red = rhs.double().sum(dim=2 if case.transpose_rhs else 1, keepdim=True).float()
    want_row = oracle.gmm_reference(lhs, w_red, gs, transpose_rhs=case.transpose_rhs)[:, 0]
    lhs_red = torch.zeros(len(sizes), case.K, dtype=torch.float64)
    for g in range(len(sizes)):
        lhs_red[g] = lhs[o[g]:o[g + 1]].double().sum(0)
    want_col = oracle.gmm_reference(lhs_red.float(), rhs, torch.ones(len(sizes), dtype=torch.int32),
                                    transpose_rhs=case.transpose_rhs)
    rows_active = np.zeros(M, dtype=bool)
    rows_active[o[0]:o[-1]] = True
    assert np.all(row_sum[~rows_active] == 0)
    sd = BF16_SUM_SD if case.out_dtype == torch.bfloat16 else 0.0
    r1 = sum_check(row_sum[rows_active], want_row[rows_active], sd * row_ss[rows_active], row_abs[rows_active],
                     f"{name} row sums")
    r2 = sum_check(col_sum, want_col, sd * col_ss, col_abs, f"{name} per-group column sums")
    print(f"sums case {name}: {rows_active.sum()} row sums and {len(sizes)}x{N} column sums within "
          f"{max(r1, r2):.3f} of the tolerance", flush=True)


def test_full_size_tgmm_every_element_by_sums():
    import oracle
    import moe_grouped_matrix_amd as gmm_amd
    case = workloads.tgmm_bf16(device="cuda")
    sizes = case.sizes_list()
    Ga, K, N = case.num_active, case.K, case.N
    print(f"tgmm sums case: M={case.M} K={K} N={N} Ga={Ga}", flush=True)
    out = torch.empty((Ga, K, N), dtype=torch.float32, device="cuda")
    gmm_amd.tgmm(case.lhs, case.rhs, case.group_sizes, num_active=Ga, out=out)
    torch.cuda.synchronize()
    assert gmm_amd.device_flags() == 0
    x = out.double()
    row_sum, col_sum = x.sum(2).cpu().numpy(), x.sum(1).cpu().numpy()
    # per-element float32 tolerance of tests/parity.py: 1e-4 of the group's largest value
    amax = x.abs().amax(dim=(1, 2)).cpu().numpy()
    row_abs, col_abs = x.abs().sum(2).cpu().numpy(), x.abs().sum(1).cpu().numpy()
    del x
    lhs, rhs, gs = case.lhs.cpu(), case.rhs.cpu(), case.group_sizes.cpu()
    rhs_red = rhs.double().sum(1, keepdim=True).float()   # [M, 1]
    lhs_red = lhs.double().sum(1, keepdim=True).float()   # [M, 1]
    want_row = oracle.tgmm_reference(lhs, rhs_red, gs, num_active=Ga)[:, :, 0]   # [Ga, K]
    want_col = oracle.tgmm_reference(lhs_red, rhs, gs, num_active=Ga)[:, 0, :]   # [Ga, N]
    r1 = sum_check(row_sum, want_row, 1e-4 * amax[:, None] * np.sqrt(N) / 8, row_abs, "tgmm row sums")
    r2 = sum_check(col_sum, want_col, 1e-4 * amax[:, None] * np.sqrt(K) / 8, col_abs, "tgmm column sums")
    print(f"tgmm sums case: {Ga}x{K} row sums and {Ga}x{N} column sums within {max(r1, r2):.3f} of the tolerance",
          flush=True)


def test_full_size_w8a8_every_element_by_sums():
    """The block-scaled W8A8 product (both scales, bf16 out) at full size,
    every element through the same sums; the scales go into the reduced
    operands:
      sum_n out[r, n] = sum_b ls[r, b] sum_{k in b} x[r, k] (sum_n rs[g, b, n] w_g[n, k])
      sum_{r in g} out[r, n] = sum_b rs[g, b, n] sum_{k in b} (sum_{r in g} ls[r, b] x[r, k]) w_g[n, k]"""
    import oracle
    import moe_grouped_matrix_amd as gmm_amd
    gmm_amd.set_tile_policy(0)
    case = workloads.FULL["w8a8_fp8"](device="cuda")
    assert case.group_offset == 0 and not case.transpose_rhs and case.rhs_bias is None
    print(f"sums case w8a8_fp8: M={case.M} K={case.K} N={case.N}", flush=True)
    out = torch.empty((case.M, case.N), dtype=case.out_dtype, device="cuda")
    gmm_amd.gmm(case.lhs, case.rhs, case.group_sizes, rhs_scale=case.rhs_scale, lhs_scale=case.lhs_scale, out=out)
    torch.cuda.synchronize()
    assert gmm_amd.device_flags() == 0
    sizes = case.sizes_list()
    o = _segments(sizes)
    M, K, N, G = case.M, case.K, case.N, len(sizes)
    row_sum, row_ss, row_abs = [], [], []
    for i in range(0, M, 32768):
        x = out[i:i + 32768].double()
        row_sum.append(x.sum(1).cpu())
        row_ss.append(x.square().sum(1).sqrt().cpu())
        row_abs.append(x.abs().sum(1).cpu())
    row_sum, row_ss, row_abs = (torch.cat(v).numpy() for v in (row_sum, row_ss, row_abs))
    col = [np.zeros((G, N)) for _ in range(3)]
    for g in range(G):
        if sizes[g]:
            x = out[o[g]:o[g + 1]].double()
            col[0][g], col[1][g], col[2][g] = (x.sum(0).cpu().numpy(), x.square().sum(0).sqrt().cpu().numpy(),
                                               x.abs().sum(0).cpu().numpy())
    lhs, rhs, gs = case.lhs.cpu(), case.rhs.cpu(), case.group_sizes.cpu()
    ls, rs = case.lhs_scale.cpu(), case.rhs_scale.cpu()      # [M, nb], [G, nb, 1, N]
    nb = ls.shape[1]
    blk = K // nb
    # w_red[g, k] = sum_n rs[g, b(k), n] w_g[n, k] (e4m3 decoded exactly; float64, then float32)
    w_red = torch.empty(G, 1, K)
    for g in range(G):
        rs_k = rs[g, :, 0, :].double().repeat_interleave(blk, dim=0)   # [K, N]: rs[g, b(k), n]
        w_red[g, 0] = (rhs[g].float().double() * rs_k.t()).sum(0).float()
    want_row = oracle.gmm_reference(lhs, w_red, gs, lhs_scale=ls)[:, 0]
    # lhs_red[g, k] = sum_{r in g} ls[r, b(k)] x[r, k]
    lhs_red = torch.zeros(G, K)
    for g in range(G):
        if sizes[g]:
            xs = lhs[o[g]:o[g + 1]].float().double() * ls[o[g]:o[g + 1]].double().repeat_interleave(blk, dim=1)
            lhs_red[g] = xs.sum(0).float()
    want_col = oracle.gmm_reference(lhs_red, rhs, torch.ones(G, dtype=torch.int32), rhs_scale=rs)
    active = np.zeros(M, dtype=bool)
    active[o[0]:o[-1]] = True
    assert np.all(row_sum[~active] == 0)
    r1 = sum_check(row_sum[active], want_row[active], BF16_SUM_SD * row_ss[active], row_abs[active], "w8a8 row sums")
    r2 = sum_check(col[0], want_col, BF16_SUM_SD * col[1], col[2], "w8a8 per-group column sums")
    print(f"sums case w8a8_fp8: {active.sum()} row sums and {G}x{N} column sums within {max(r1, r2):.3f} of the "
          f"tolerance", flush=True)
