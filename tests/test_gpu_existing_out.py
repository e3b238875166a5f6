"""GPU parity of gmm with an existing output (gmm_run_existing_out, gmm's
existing_out on the tpu-inference wheel diff pages) against the oracle,
through the C ABI.

For every kernel family (the small-tile kernel for f32 and fp8 x fp8, the
big kernel for bf16 in both weight layouts, the weight-streaming kernel for
bf16 x e4m3): rows outside the active groups (before the first active group,
and from the end of the last on, past the sum of the sizes included) must be
the existing rows bit for bit, in place (existing_out is out) and copied (a
separate buffer, which must stay unchanged); the active rows must match the
oracle to the usual tolerances.  Merging two expert shards in place gives
the unsharded call's output bit for bit (each row is computed the same way
in both).  Invalid existing outputs are rejected before anything is
queued."""
import pytest
import torch

import oracle
from parity import compare

pytestmark = pytest.mark.gpu

PATHS = [
    # (lhs dtype, rhs dtype, transpose_rhs, K, tile policy, out dtype)
    (torch.float32, torch.float32, False, 64, 1, torch.float32),
    (torch.bfloat16, torch.bfloat16, False, 256, 2, torch.bfloat16),
    (torch.bfloat16, torch.bfloat16, True, 256, 2, torch.float32),
    (torch.bfloat16, torch.float8_e4m3fn, False, 768, 1, torch.bfloat16),
    (torch.float8_e4m3fn, torch.float8_e4m3fn, False, 256, 0, torch.bfloat16),
]
PATH_IDS = ["f32_small", "bf16_big_nt", "bf16_big_nn_f32out", "bf16xe4m3_stream", "e4m3xe4m3"]


@pytest.fixture
def policy():
    import moe_grouped_matrix_amd as m
    yield m.set_tile_policy
    m.set_tile_policy(0)


def _inputs(ld, rd, T, K, N, sizes, extra, s, Ga, seed):
    g = torch.Generator().manual_seed(seed)
    M = sum(sizes) + extra
    lhs = torch.randn(M, K, generator=g).to(ld)
    rhs = (torch.randn(Ga, K, N, generator=g) if T else torch.randn(Ga, N, K, generator=g)).to(rd)
    gs = torch.tensor(sizes, dtype=torch.int32)
    return lhs, rhs, gs


def _bounds(sizes, s, Ga):
    o = [0]
    for v in sizes:
        o.append(o[-1] + v)
    return o[s], o[s + Ga]


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("mode", ["in_place", "copy"])
def test_existing_rows_kept_and_active_rows_match(path, mode, policy):
    import moe_grouped_matrix_amd as m
    ld, rd, T, K, pol, od = path
    policy(pol)
    sizes = [40, 0, 300, 7, 0, 129, 64, 33]
    s, Ga, N = 1, 6, 136
    lhs, rhs, gs = _inputs(ld, rd, T, K, N, sizes, 19, s, Ga, seed=K + pol)
    M = lhs.shape[0]
    existing = (torch.randn(M, N, generator=torch.Generator().manual_seed(7)) * 3).to(od)
    print(f"existing_out {mode} lhs={ld} rhs={rd} T={T} K={K} policy={pol} out={od}", flush=True)
    dev_ex = existing.cuda()
    if mode == "in_place":
        out = m.gmm(lhs.cuda(), rhs.cuda(), gs.cuda(), group_offset=s, transpose_rhs=T, existing_out=dev_ex)
        assert out.data_ptr() == dev_ex.data_ptr()
    else:
        out = torch.full((M, N), float("nan"), dtype=od, device="cuda")
        m.gmm(lhs.cuda(), rhs.cuda(), gs.cuda(), group_offset=s, transpose_rhs=T, existing_out=dev_ex, out=out)
    torch.cuda.synchronize()
    assert m.device_flags() == 0
    got = out.cpu()
    lo, hi = _bounds(sizes, s, Ga)
    assert torch.equal(got[:lo], existing[:lo]) and torch.equal(got[hi:], existing[hi:])
    if mode == "copy":
        assert torch.equal(dev_ex.cpu(), existing)
    ref = oracle.gmm_reference(lhs, rhs, gs, group_offset=s, transpose_rhs=T, existing_out=existing)
    compare(got[lo:hi], ref[lo:hi], od, f"existing_out {mode} active rows")


@pytest.mark.parametrize("pol", [1, 2], ids=["small", "big"])
def test_merging_expert_shards_in_place_is_the_full_call(pol, policy):
    import moe_grouped_matrix_amd as m
    policy(pol)
    sizes = [300, 0, 129, 64, 400, 33, 0, 257]
    a = 4
    lhs, rhs, gs = _inputs(torch.bfloat16, torch.bfloat16, False, 256, 264, sizes, 11, 0, len(sizes), seed=3)
    lhs, rhs, gs = lhs.cuda(), rhs.cuda(), gs.cuda()
    print(f"shard merge policy={pol}", flush=True)
    full = m.gmm(lhs, rhs, gs, out_dtype=torch.bfloat16)
    out = m.gmm(lhs, rhs[:a].contiguous(), gs, out_dtype=torch.bfloat16)
    m.gmm(lhs, rhs[a:].contiguous(), gs, group_offset=a, existing_out=out)
    torch.cuda.synchronize()
    assert m.device_flags() == 0
    assert torch.equal(out.cpu().view(torch.int16), full.cpu().view(torch.int16))


def test_invalid_existing_outputs_are_rejected():
    import moe_grouped_matrix_amd as m
    lhs = torch.randn(64, 64, device="cuda")
    rhs = torch.randn(2, 24, 64, device="cuda")
    gs = torch.tensor([30, 20], dtype=torch.int32, device="cuda")
    out = torch.zeros(64, 24, device="cuda")
    with pytest.raises(m.GmmInvalid):
        m.gmm(lhs, rhs, gs, existing_out=torch.zeros(64, 24, dtype=torch.bfloat16, device="cuda"), out=out)
    with pytest.raises(m.GmmInvalid):
        m.gmm(lhs, rhs, gs, existing_out=torch.zeros(63, 24, device="cuda"), out=out)
    big = torch.zeros(65 * 24, device="cuda")
    with pytest.raises(m.GmmInvalid):  # overlaps out without being out
        m.gmm(lhs, rhs, gs, existing_out=big[24:].view(64, 24), out=big[:64 * 24].view(64, 24))
    torch.cuda.synchronize()
