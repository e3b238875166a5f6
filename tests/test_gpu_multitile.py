"""Every kernel family with many output tiles per workgroup, compared with
the oracle on every element.

In production each workgroup of the persistent kernels runs tens of tiles
back to back, and the big, tgmm, W8A8 and weight-streaming kernels carry
their direct-to-LDS operand ring (and the next tile's bias row) from one
tile into the next with constant wait counts.  The other small-size tests
run about one tile per workgroup; here gmm_set_grid_limit caps the grid so
that each workgroup runs at least four, on a grid that is a multiple of 8
(the XCD-grouped tile order and tgmm's eight work queues) and on one that is
not (plain order, one queue).  Results may only differ from the default
grid in the order of fp32 additions, and must meet the tolerances of
tests/parity.py (float32: max error 1e-4 of the largest reference value;
bfloat16: relative Frobenius error 2e-2, globally and per row); the
small-integer cases are bit-exact."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import active_range, assert_zero_rows, compare, reference, run_gpu

pytestmark = pytest.mark.gpu

LIMITS = (8, 5)


@pytest.fixture
def gm():
    import moe_grouped_matrix_amd as m
    yield m
    m.set_grid_limit(0)
    m.set_tile_policy(0)


def m_tiles(sizes, s, ga, bm):
    return sum(math.ceil(x / bm) for x in sizes[s:s + ga])


# (SMALL workload, tile policy, kernel family, output tile (rows, columns))
FAMILIES = [
    ("moe_fwd_bf16", 2, "big kernel, NT", (256, 256)),
    ("moe_dlhs_bf16", 2, "big kernel, NN in place", (256, 256)),
    ("w8a8_fp8", 2, "W8A8 ring kernel", (256, 128)),
    ("decode_fp8w", 1, "weight-streaming kernel", (64, 256)),
    ("decode_fp8w", 2, "general kernel, big scaled tiles", (256, 128)),
    ("tiny_fp32", 0, "general kernel, f32", (64, 64)),
]


@pytest.mark.parametrize("name,policy,family,tile", FAMILIES,
                         ids=["big_nt", "big_nn", "w8a8", "stream", "general_big_scaled", "general_f32"])
def test_many_tiles_per_workgroup(gm, name, policy, family, tile):
    case = workloads.SMALL[name]().to("cuda")
    sizes = case.sizes_list()
    items = m_tiles(sizes, case.group_offset, case.num_active, tile[0]) * math.ceil(case.N / tile[1])
    ref = reference(case)
    lo, hi = active_range(case)
    gm.set_tile_policy(policy)
    for limit in LIMITS:
        gm.set_grid_limit(limit)
        per_wg = items / limit
        print(f"{family}: {name} policy {policy} grid {limit}: {items} tiles, {per_wg:.1f} per workgroup",
              flush=True)
        out = run_gpu(case)
        assert_zero_rows(out, lo, hi)
        compare(out.cpu()[lo:hi], ref[lo:hi], case.out_dtype, f"{name} grid {limit}")
        assert gm.device_flags() == 0
    assert items / min(LIMITS) >= 4, f"{family}: only {items} tiles"


@pytest.mark.parametrize("T", [False, True], ids=["nt", "nn"])
def test_big_kernel_bias_rows_carried_across_tiles(gm, T):
    """The big kernel loads a tile's bias row with its first K step, into
    the slot the previous tile is not using.  Small integers (sums exact in
    fp32) and a grid of 3 or 2 workgroups over 14 tiles, full and half
    tiles, N tails: bit-exact against the oracle, for each output type."""
    g = torch.Generator().manual_seed(11)
    sizes = [300, 0, 129, 40, 512, 3]
    M, K, N = sum(sizes) + 5, 192, 392
    lhs = torch.randint(-3, 4, (M, K), generator=g).to(torch.bfloat16)
    rhs = torch.randint(-3, 4, (len(sizes), K, N) if T else (len(sizes), N, K), generator=g).to(torch.bfloat16)
    bias = torch.randint(-8, 9, (len(sizes), 1, N), generator=g).to(torch.bfloat16)
    items = m_tiles(sizes, 0, len(sizes), 256) * math.ceil(N / 256)
    gm.set_tile_policy(2)
    for limit in (3, 2):
        gm.set_grid_limit(limit)
        for out_dtype in (torch.float32, torch.bfloat16):
            print(f"big kernel bias nn={T} grid {limit}: {items} tiles, {items / limit:.1f} per workgroup, "
                  f"out {out_dtype}", flush=True)
            case = workloads.Case("bias", lhs.cuda(), rhs.cuda(), torch.tensor(sizes, dtype=torch.int32).cuda(),
                                  transpose_rhs=T, rhs_bias=bias.cuda(), out_dtype=out_dtype)
            out = run_gpu(case).cpu()
            want = oracle.round_to(reference(case), out_dtype)
            iv = torch.int16 if out_dtype == torch.bfloat16 else torch.int32
            assert torch.equal(out.view(iv), want.view(iv)), (T, limit, out_dtype)
    assert items / 3 >= 4
    assert gm.device_flags() == 0


def test_tgmm_many_tiles_per_workgroup(gm):
    """The weight gradient with 18 groups (so eight work queues on a grid
    that is a multiple of 8, one queue otherwise), 6 output tiles per group,
    contraction tails, empty groups: every element against the oracle, on
    two calls in a row per grid (the queues' counters must come back to
    zero)."""
    g = torch.Generator().manual_seed(12)
    sizes = [700, 0, 33, 250, 1, 96, 512, 0, 64, 300, 17, 129, 0, 480, 5, 222, 40, 610]
    M, K, N = sum(sizes) + 9, 512, 520
    lhs = torch.randn(M, K, generator=g).to(torch.bfloat16)
    rhs = torch.randn(M, N, generator=g).to(torch.bfloat16)
    gs = torch.tensor(sizes, dtype=torch.int32)
    ref = oracle.tgmm_reference(lhs, rhs, gs)
    Ga = len(sizes)
    items = Ga * math.ceil(K / 256) * math.ceil(N / 256)
    for limit in LIMITS:
        gm.set_grid_limit(limit)
        for call in range(2):
            print(f"tgmm grid {limit} call {call}: {items} tiles, {items / limit:.1f} per workgroup", flush=True)
            out = gm.tgmm(lhs.cuda(), rhs.cuda(), gs.cuda()).cpu()
            compare(out.reshape(Ga * K, N), ref.reshape(Ga * K, N), torch.float32, f"tgmm grid {limit}")
            for h in range(Ga):
                if sizes[h] == 0:
                    assert torch.all(out[h].view(torch.int32) == 0)
    assert items / min(LIMITS) >= 4
    assert gm.device_flags() == 0


def test_grid_limit_rejects_negative(gm):
    with pytest.raises(gm.GmmInvalid):
        gm.set_grid_limit(-1)
