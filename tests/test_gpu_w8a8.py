"""The block-scaled fp8 x fp8 (W8A8) kernel against the oracle.

The kernel takes problems with both block scales, scale blocks of one K step
of 128, K >= 384 and N a multiple of 4 (the big tile policy, or the auto
policy on large groups).  Covered here: the four one-byte format pairs,
f32 and bf16 output, no bias / bf16 bias / f32 bias, empty groups, partial
m-tiles, an N tail of 8 columns, the minimum of three K steps and more, and
grids capped so that each workgroup runs several tiles back to back (its
load pipeline crosses from one tile into the next).

Small-integer operands with power-of-two scales keep every sum exact in
fp32, so those results must match the oracle bit for bit; normal operands
with arbitrary f32 scales must meet the tolerances of tests/parity.py."""
import math

import numpy as np
import pytest
import torch

import oracle
from parity import compare

pytestmark = pytest.mark.gpu

FP8 = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
PAIRS = [("e4m3", "e4m3"), ("e5m2", "e5m2"), ("e4m3", "e5m2"), ("e5m2", "e4m3")]


@pytest.fixture
def gm():
    import moe_grouped_matrix_amd as m
    m.set_tile_policy(2)
    yield m
    m.set_grid_limit(0)
    m.set_tile_policy(0)


def _run(gm, lhs, rhs, sizes, ls, rs, bias, out_dtype):
    out = gm.gmm(lhs.cuda(), rhs.cuda(), torch.tensor(sizes, dtype=torch.int32).cuda(), out_dtype=out_dtype,
                 rhs_scale=rs.cuda(), lhs_scale=ls.cuda(), rhs_bias=None if bias is None else bias.cuda())
    torch.cuda.synchronize()
    return out.cpu()


def _ref(lhs, rhs, sizes, ls, rs, bias):
    return oracle.gmm_reference(lhs, rhs, torch.tensor(sizes, dtype=torch.int32), rhs_scale=rs, lhs_scale=ls,
                                rhs_bias=bias)


@pytest.mark.parametrize("K", [384, 640])
@pytest.mark.parametrize("fa,fb", PAIRS, ids=[f"{a}x{b}" for a, b in PAIRS])
def test_exact_inputs_are_bit_exact(gm, fa, fb, K):
    g = torch.Generator().manual_seed(21 + K)
    sizes = [300, 0, 129, 40, 512, 3]
    M, N = sum(sizes) + 5, 264
    nb = K // 128
    lhs = torch.randint(-3, 4, (M, K), generator=g).to(torch.float32).to(FP8[fa])
    rhs = torch.randint(-3, 4, (len(sizes), N, K), generator=g).to(torch.float32).to(FP8[fb])
    ls = 2.0 ** torch.randint(-2, 3, (M, nb), generator=g).to(torch.float32)
    rs = 2.0 ** torch.randint(-3, 4, (len(sizes), nb, 1, N), generator=g).to(torch.float32)
    biases = {"none": None,
              "bf16": torch.randint(-8, 9, (len(sizes), 1, N), generator=g).to(torch.bfloat16),
              "f32": torch.randint(-8, 9, (len(sizes), 1, N), generator=g).to(torch.float32)}
    tiles = sum(math.ceil(s / 256) for s in sizes) * math.ceil(N / 128)
    for limit in (0, 8, 5):
        gm.set_grid_limit(limit)
        for bname, bias in biases.items():
            want = _ref(lhs, rhs, sizes, ls, rs, bias)
            for out_dtype in (torch.float32, torch.bfloat16):
                print(f"w8a8 {fa}x{fb} K={K} grid {limit or 'full'} ({tiles} tiles) bias {bname} out {out_dtype}",
                      flush=True)
                out = _run(gm, lhs, rhs, sizes, ls, rs, bias, out_dtype)
                iv = torch.int16 if out_dtype == torch.bfloat16 else torch.int32
                assert torch.equal(out.view(iv), oracle.round_to(want, out_dtype).view(iv)), (limit, bname, out_dtype)
    assert gm.device_flags() == 0


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_normal_inputs_within_tolerance(gm, out_dtype):
    """Quantised normal operands, f32 scales drawn from [0.5, 1.5), a bf16
    bias; router-like group sizes (an empty group, a tail of one row)."""
    g = torch.Generator().manual_seed(22)
    sizes = [700, 1, 0, 333, 1290, 256, 77]
    M, K, N = sum(sizes) + 9, 1408, 712
    nb = K // 128
    lhs = (torch.randn(M, K, generator=g) * 60).to(torch.float8_e4m3fn)
    rhs = (torch.randn(len(sizes), N, K, generator=g) * 60).to(torch.float8_e4m3fn)
    ls = torch.rand(M, nb, generator=g) + 0.5
    rs = torch.rand(len(sizes), nb, 1, N, generator=g) + 0.5
    bias = (torch.randn(len(sizes), 1, N, generator=g) * 1e4).to(torch.bfloat16)
    want = _ref(lhs, rhs, sizes, ls, rs, bias)
    o = sum(sizes)
    for limit in (0, 16):
        gm.set_grid_limit(limit)
        print(f"w8a8 normal {M}x{K}x{N} grid {limit or 'full'} out {out_dtype}", flush=True)
        out = _run(gm, lhs, rhs, sizes, ls, rs, bias, out_dtype)
        compare(out[:o], want[:o], out_dtype, f"w8a8 normal grid {limit}")
        bits = out[o:].view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32)
        assert int((bits != 0).sum()) == 0
    assert gm.device_flags() == 0
