"""GPU parity of the block-scale widening (gmm_widen_scales_run,
widen_block_scale_f32 of the metrale gemm_quant.rs page) against the
oracle, through the C ABI, bit for bit: every E8M0 byte (e = 0 -> 2^-127,
e = 255 -> 0.0 as the page states), every non-NaN bf16 code, f32 values
including -0, infinity and subnormals, shapes with ragged element counts;
then E8M0 block scales widened on the device feeding the W8A8 gmm, against
the oracle's gmm with the oracle's widened scales."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import compare

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.cpu().view(torch.int32)


def test_widen_every_e8m0_byte():
    import moe_grouped_matrix_amd as m
    codes = torch.arange(256, dtype=torch.uint8)
    print("widen e8m0", flush=True)
    got = m.widen_scales(codes.view(torch.float8_e8m0fnu).cuda())
    torch.cuda.synchronize()
    want = oracle.widen_scales_reference(codes, oracle.SCALE_E8M0)
    assert torch.equal(_bits(got), want.view(torch.int32))


def test_widen_every_bf16_code_and_f32():
    import moe_grouped_matrix_amd as m
    codes = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    print("widen bf16 / f32", flush=True)
    got = m.widen_scales(codes.cuda()).cpu()
    want = oracle.widen_scales_reference(codes, oracle.SCALE_BF16)
    ok = ~torch.isnan(want)
    assert torch.equal(got.view(torch.int32)[ok], want.view(torch.int32)[ok])
    g = torch.Generator().manual_seed(2)
    x = torch.randn(3, 7, 1, 11, generator=g)
    x.view(-1)[:4] = torch.tensor([0.0, -0.0, float("inf"), 1e-40])
    got = m.widen_scales(x.cuda())
    torch.cuda.synchronize()
    assert got.shape == x.shape and torch.equal(_bits(got), x.view(torch.int32))


def test_e8m0_scales_feed_the_w8a8_gmm():
    import moe_grouped_matrix_amd as m
    g = torch.Generator().manual_seed(4)
    sizes = [120, 0, 300, 45]
    M, K, N, nb = sum(sizes) + 3, 512, 200, 4
    lhs = (torch.randn(M, K, generator=g) * 8).to(torch.float8_e4m3fn)
    rhs = (torch.randn(len(sizes), N, K, generator=g) * 8).to(torch.float8_e4m3fn)
    rs8 = torch.randint(120, 135, (len(sizes), nb, 1, N), generator=g).to(torch.uint8)
    ls8 = torch.randint(122, 133, (M, nb), generator=g).to(torch.uint8)
    gs = torch.tensor(sizes, dtype=torch.int32)
    print("e8m0 scales + w8a8 gmm", flush=True)
    rs = m.widen_scales(rs8.view(torch.float8_e8m0fnu).cuda())
    ls = m.widen_scales(ls8.view(torch.float8_e8m0fnu).cuda())
    out = m.gmm(lhs.cuda(), rhs.cuda(), gs.cuda(), rhs_scale=rs, lhs_scale=ls, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rs_ref = oracle.widen_scales_reference(rs8, oracle.SCALE_E8M0)
    ls_ref = oracle.widen_scales_reference(ls8, oracle.SCALE_E8M0)
    assert torch.equal(rs.cpu(), rs_ref) and torch.equal(ls.cpu(), ls_ref)
    ref = oracle.gmm_reference(lhs, rhs, gs, rhs_scale=rs_ref, lhs_scale=ls_ref)
    hi = sum(sizes)
    compare(out.cpu()[:hi], ref[:hi], torch.bfloat16, "e8m0-scaled w8a8")


def test_widen_rejects_invalid_arguments():
    import moe_grouped_matrix_amd as m
    with pytest.raises(m.GmmInvalid):
        m.widen_scales(torch.zeros(8, dtype=torch.float8_e4m3fn, device="cuda"))
    with pytest.raises(m.GmmInvalid):
        m.widen_scales(torch.zeros(8, device="cuda"), out=torch.zeros(7, device="cuda"))
    with pytest.raises(m.GmmInvalid):
        m.widen_scales(torch.zeros(8, device="cuda"), out=torch.zeros(8, dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
