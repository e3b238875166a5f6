"""Full-size parity: every workload at its full shape, launched as the
benchmark launches it (automatic tile choice, caller-allocated output),
against the oracle.

- tiny_fp32 and decode_fp8w (small enough): every active row, every element.
- moe_fwd_bf16, moe_dlhs_bf16, w8a8_fp8: sampled rows -- each active group's
  first and last row, both sides of every 256- and 32-row tile boundary (up
  to a few thousand rows), random rows per group and overall.
- Always: rows outside the active groups are all-zero bits (checked on the
  device over all M rows) and no device data flag is raised.

Tolerances are those of tests/parity.py (float32: max error 1e-4 of the
largest reference value; bfloat16: relative Frobenius error 2e-2, globally
and per row)."""
import numpy as np
import pytest
import torch

import workloads
from parity import active_range, assert_zero_rows, compare, reference, sample_rows

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
