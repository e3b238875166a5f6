"""Helpers shared by the GPU parity tests: run a case through the HIP path,
compute the oracle's rows, and compare to the stated tolerances.

Tolerances (against the oracle's float64 value before rounding, on the same
quantised inputs):
  float32 output: max |out - ref| <= 1e-4 * max |ref|
  bfloat16 output: ||out - ref||_F / ||ref||_F <= 2e-2, and the same bound on
  every row on its own (a single misplaced row barely moves the global norm).
Rows outside the active groups must be all-zero bits."""
import numpy as np
import torch

import oracle

F32_TOL = 1e-4
BF16_TOL = 2e-2


def run_gpu(case, **kw):
    import moe_grouped_matrix_amd as gmm_amd
    out = gmm_amd.gmm(case.lhs, case.rhs, case.group_sizes, out_dtype=case.out_dtype,
                      rhs_scale=case.rhs_scale, rhs_bias=case.rhs_bias, lhs_scale=case.lhs_scale,
                      group_offset=case.group_offset if case.group_offset else None,
                      transpose_rhs=case.transpose_rhs, **kw)
    torch.cuda.synchronize()
    return out


def reference(case, rows=None, return_row_group=False):
    return oracle.gmm_reference(case.lhs, case.rhs, case.group_sizes,
                                group_offset=case.group_offset, transpose_rhs=case.transpose_rhs,
                                rhs_scale=case.rhs_scale, rhs_bias=case.rhs_bias,
                                lhs_scale=case.lhs_scale, rows=rows,
                                return_row_group=return_row_group)


def active_range(case):
    s = case.sizes_list()
    o = np.concatenate([[0], np.cumsum(s)])
    return int(o[case.group_offset]), int(o[case.group_offset + case.num_active])


def compare(out_rows: torch.Tensor, ref: np.ndarray, out_dtype, what=""):
    """out_rows: GPU rows (CPU tensor) matching ref rows (float64)."""
    got = out_rows.to(torch.float64).numpy()
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    if out_dtype == torch.float32:
        scale = np.abs(ref).max()
        err = np.abs(got - ref).max()
        assert err <= F32_TOL * max(scale, 1e-30), f"{what}: max err {err} vs {F32_TOL} * {scale}"
        return err / max(scale, 1e-30)
    num = np.linalg.norm(got - ref)
    den = np.linalg.norm(ref)
    rel = num / den if den > 0 else num
    assert rel <= BF16_TOL, f"{what}: relative Frobenius error {rel}"
    rn = np.linalg.norm(got - ref, axis=1)
    rd = np.linalg.norm(ref, axis=1)
    nz = rd > 0
    if nz.any():
        worst = (rn[nz] / rd[nz]).max()
        assert worst <= BF16_TOL, f"{what}: worst row relative error {worst}"
    assert np.all(got[~nz] == 0) or np.all(rn[~nz] == 0), f"{what}: rows with zero reference are not zero"
    return rel


def assert_zero_rows(out: torch.Tensor, lo: int, hi: int):
    """Rows outside [lo, hi) are all-zero bits (checked on the device)."""
    bits = out.view(torch.int16) if out.dtype == torch.bfloat16 else out.view(torch.int32)
    assert int((bits[:lo] != 0).sum()) == 0, "rows before the active groups are not zero"
    assert int((bits[hi:] != 0).sum()) == 0, "rows after the active groups are not zero"


def sample_rows(case, tm_list=(32, 256), per_group=3, extra=64, seed=0):
    """Rows to check at full size: each active group's first and last row,
    rows on both sides of every m-tile boundary for the tile heights in
    tm_list, random rows per group, and random rows overall."""
    rng = np.random.default_rng(seed)
    s = case.sizes_list()
    o = np.concatenate([[0], np.cumsum(s)])
    rows = set()
    for g in range(case.group_offset, case.group_offset + case.num_active):
        a, b = int(o[g]), int(o[g + 1])
        if a == b:
            continue
        rows.update([a, b - 1])
        for tm in tm_list:
            for r0 in range(a + tm, b, tm):
                if len(rows) > 4000:
                    break
                rows.update([r0 - 1, r0])
        rows.update(int(x) for x in rng.integers(a, b, size=per_group))
    rows.update(int(x) for x in rng.integers(0, case.M, size=extra))
    return sorted(rows)


# Sums of many output elements against exact sums (the every-element checks
# of the full-size tests).  A bf16 output is the nearest bf16 of its float32
# value: within half a unit in the last place, at most 2^-8 of the value and
# about uniform, so a sum of such errors spreads by at most 2^-8/sqrt(3) of
# the root of the sum of the values' squares.
BF16_SUM_SD = 2.0 ** -8 / np.sqrt(3.0)


def sum_check(got, want, spread, mag, what):
    """Assert |got - want| <= 8 spread + 1e-5 mag elementwise (spread: the
    sums' rounding spread; mag: the sum of the summed values' magnitudes,
    for the float32 accumulation); returns the largest ratio to that
    tolerance."""
    got, want, spread, mag = (np.asarray(x, dtype=np.float64) for x in (got, want, spread, mag))
    tol = 8.0 * spread + 1e-5 * mag + 1e-30
    ratio = np.abs(got - want) / tol
    bad = ratio > 1.0
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} sums off, worst {ratio.max():.2f}x the tolerance"
    return float(ratio.max())
