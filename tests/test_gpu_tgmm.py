"""GPU parity of the transposed grouped matmul (the weight gradient of gmm)
against the oracle, through the C ABI (gmm_tgmm_run).

Small cases compare every element: contraction tails (group sizes that are
not multiples of the 32-row step), groups shorter than the kernel's five
steps, empty groups (all-zero bits), K and N tails past the 256-column tiles
(down to 8 columns), a group offset, f32 and bf16 outputs, rows outside the
active groups (ignored), invalid device sizes (clamped and flagged), and
both tile schedules (dynamic: one work queue, and one per XCD over two
calls in a row; gang: every tile shape, bit-exact on small integers).  The
full-size case (the forward workload's shapes) runs in the benchmark's
launch configuration and compares sampled output rows.

Tolerances are those of tests/parity.py (float32: max error 1e-4 of the
largest reference value; bfloat16: relative Frobenius error 2e-2, globally
and per row), and the float32 bound also per group."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import compare

pytestmark = pytest.mark.gpu

CASES = [
    # (group sizes, extra rows past the groups, K, N, out dtype, group offset, active groups)
    ([70, 0, 33, 200, 5, 1, 130], 7, 264, 136, torch.float32, 0, None),
    ([300, 0, 650, 17], 0, 512, 520, torch.bfloat16, 1, 3),
    ([1000, 2000, 0, 777], 3, 256, 256, torch.float32, 0, None),
    ([0, 0, 0], 4, 128, 64, torch.float32, 0, None),
    ([4100, 96, 2500], 0, 1408, 704, torch.float32, 0, None),
]
IDS = ["tails_tiny_groups", "offset_bf16out", "exact_tiles", "all_empty", "model_shapes"]


def _case(sizes, extra, K, N, seed):
    g = torch.Generator().manual_seed(seed)
    M = sum(sizes) + extra
    lhs = torch.randn(M, K, generator=g).to(torch.bfloat16)
    rhs = torch.randn(M, N, generator=g).to(torch.bfloat16)
    return lhs, rhs, torch.tensor(sizes, dtype=torch.int32)


def _check(out, ref, sizes, s, out_dtype, what):
    Ga, K, N = ref.shape
    compare(out.reshape(Ga * K, N), ref.reshape(Ga * K, N), out_dtype, what)
    for h in range(Ga):
        if sizes[s + h] == 0:
            assert torch.all(out[h].view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32) == 0), \
                f"{what}: empty group {h} not all-zero bits"
        elif out_dtype == torch.float32:
            scale = np.abs(ref[h]).max()
            err = np.abs(out[h].double().numpy() - ref[h]).max()
            assert err <= 1e-4 * max(scale, 1e-30), f"{what}: group {h} max err {err} vs {scale}"


@pytest.mark.parametrize("sizes,extra,K,N,out_dtype,s,ga", CASES, ids=IDS)
def test_tgmm_against_oracle(sizes, extra, K, N, out_dtype, s, ga):
    import moe_grouped_matrix_amd as m
    lhs, rhs, gs = _case(sizes, extra, K, N, seed=len(sizes) * 1000 + K)
    Ga = len(sizes) - s if ga is None else ga
    print(f"tgmm case sizes={sizes} K={K} N={N} out={out_dtype} s={s} Ga={Ga}", flush=True)
    out = m.tgmm(lhs.cuda(), rhs.cuda(), gs.cuda(), num_active=Ga, group_offset=s, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert m.device_flags() == 0
    ref = oracle.tgmm_reference(lhs, rhs, gs, group_offset=s, num_active=Ga)
    _check(out.cpu(), ref, sizes, s, out_dtype, f"tgmm {sizes} K={K} N={N}")


def test_tgmm_work_queues_back_to_back():
    """Enough groups for one work queue per XCD (20 and 17 groups over 40 and
    34 tiles, so 40 and 32 workgroups): two calls in a row on the same handle,
    the second smaller, check that the tiles are all handed out and that the
    last workgroup of every queue leaves its counters at zero for the next
    call."""
    import moe_grouped_matrix_amd as m
    rng = np.random.default_rng(7)
    for n_groups, K, N in ((20, 256, 264), (17, 200, 264)):
        sizes = [int(v) for v in rng.integers(0, 300, n_groups)]
        sizes[3] = 0
        sizes[11] = 0
        lhs, rhs, gs = _case(sizes, 5, K, N, seed=n_groups)
        print(f"tgmm queues case groups={n_groups} K={K} N={N}", flush=True)
        out = m.tgmm(lhs.cuda(), rhs.cuda(), gs.cuda(), out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert m.device_flags() == 0
        ref = oracle.tgmm_reference(lhs, rhs, gs)
        _check(out.cpu(), ref, sizes, 0, torch.float32, f"tgmm queues {n_groups} groups")


# (K, N, grid limit, tiles per group T, workgroups per XCD queue W): shapes
# and grids on which the gang schedule runs (at least 16 groups, a grid that
# is a multiple of 8, 3/4 W <= T <= W), covering each tile shape: full tiles
# (one with more than 128 but fewer than 256 valid rows), the L tile with its
# skipped quadrant, tall and wide tiles with partial extents, and a queue with
# an idle workgroup (T < W)
GANG = [
    (384, 384, 32, 3, 4),      # full + tall + wide, one idle workgroup per queue
    (448, 384, 32, 4, 4),      # a partial full tile (192 rows), two tall tiles
    (640, 1408, 128, 15, 16),  # L tile, one tall, three wide; one idle workgroup
    (1408, 1408, 0, 32, 32),   # the model's shape: 25 full, L, 3 tall, 3 wide
]
GANG_SIZES = [0, 37, 300, 5, 128, 77, 0, 250, 33, 96, 1, 160, 64, 200, 31, 400, 17, 90]


@pytest.mark.parametrize("K,N,limit,T,W", GANG, ids=[f"{k}x{n}" for k, n, *_ in GANG])
def test_tgmm_gang_schedule_bit_exact(K, N, limit, T, W):
    """Small-integer operands (every sum exact in fp32): the gang schedule's
    output must equal the oracle bit for bit, f32 and bf16 (rounded once),
    on every element; empty groups all-zero bits; two calls in a row."""
    import moe_grouped_matrix_amd as m
    g = torch.Generator().manual_seed(K + N)
    sizes = GANG_SIZES
    M = sum(sizes) + 11
    lhs = torch.randint(-3, 4, (M, K), generator=g).to(torch.bfloat16)
    rhs = torch.randint(-3, 4, (M, N), generator=g).to(torch.bfloat16)
    gs = torch.tensor(sizes, dtype=torch.int32)
    ref = oracle.tgmm_reference(lhs, rhs, gs)
    m.set_grid_limit(limit)
    try:
        for out_dtype in (torch.float32, torch.bfloat16):
            for call in range(2):
                print(f"tgmm gang K={K} N={N} grid {limit or 'full'}: T={T} of W={W}, out {out_dtype}, call {call}",
                      flush=True)
                out = m.tgmm(lhs.cuda(), rhs.cuda(), gs.cuda(), out_dtype=out_dtype).cpu()
                iv = torch.int16 if out_dtype == torch.bfloat16 else torch.int32
                want = oracle.round_to(ref, out_dtype)
                bad = (out.view(iv) != want.view(iv)).nonzero()
                assert bad.numel() == 0, f"{bad.shape[0]} elements differ, first {bad[:4].tolist()}"
        assert m.device_flags() == 0
    finally:
        m.set_grid_limit(0)


def test_tgmm_gang_schedule_with_group_offset():
    """The gang schedule over a shard: 20 groups, offset s = 2 (a device
    scalar), 17 active groups (so still one queue per XCD), K = N = 384 on a
    grid of 32 (T = 3 tiles of W = 4 workgroups per queue), and then an
    offset past G - Ga, which is flagged and keeps the G - s groups there
    are (15: one queue, the dynamic schedule); the output groups it drops
    are zero."""
    import moe_grouped_matrix_amd as m
    g = torch.Generator().manual_seed(77)
    sizes = GANG_SIZES + [45, 12]
    K = N = 384
    M = sum(sizes) + 3
    lhs = torch.randint(-3, 4, (M, K), generator=g).to(torch.bfloat16)
    rhs = torch.randint(-3, 4, (M, N), generator=g).to(torch.bfloat16)
    gs = torch.tensor(sizes, dtype=torch.int32)
    Ga = 17
    m.set_grid_limit(32)
    try:
        s = torch.tensor([2], dtype=torch.int32, device="cuda")
        print(f"tgmm gang offset 2, Ga={Ga} of G={len(sizes)}", flush=True)
        out = m.tgmm(lhs.cuda(), rhs.cuda(), gs.cuda(), num_active=Ga, group_offset=s).cpu()
        want = oracle.round_to(oracle.tgmm_reference(lhs, rhs, gs, group_offset=2, num_active=Ga), torch.float32)
        assert torch.equal(out.view(torch.int32), want.view(torch.int32))
        assert m.device_flags() == 0
        # offset 5 > G - Ga = 3: flagged; groups 5 .. 19 are output groups 0 .. 14, 15 and 16 are zero
        s = torch.tensor([5], dtype=torch.int32, device="cuda")
        print("tgmm gang offset 5 (clamped)", flush=True)
        out = m.tgmm(lhs.cuda(), rhs.cuda(), gs.cuda(), num_active=Ga, group_offset=s).cpu()
        assert m.device_flags() != 0
        kept = len(sizes) - 5
        want = oracle.round_to(oracle.tgmm_reference(lhs, rhs, gs, group_offset=5, num_active=kept), torch.float32)
        assert torch.equal(out[:kept].view(torch.int32), want.view(torch.int32))
        assert torch.all(out[kept:].view(torch.int32) == 0)
    finally:
        m.set_grid_limit(0)


def test_tgmm_invalid_sizes_are_clamped_and_flagged():
    import moe_grouped_matrix_amd as m
    sizes = [40, -3, 25]
    lhs, rhs, _ = _case([40, 0, 25], 0, 64, 48, seed=5)
    gs = torch.tensor(sizes, dtype=torch.int32)
    out = m.tgmm(lhs.cuda(), rhs.cuda(), gs.cuda(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert m.device_flags() & m.FLAG_NEGATIVE_SIZE
    ref = oracle.tgmm_reference(lhs, rhs, torch.tensor([40, 0, 25], dtype=torch.int32))
    _check(out.cpu(), ref, [40, 0, 25], 0, torch.float32, "tgmm clamped sizes")


def test_tgmm_full_size_sampled():
    """The forward workload's shapes (262144 rows, 128 groups, K = N = 1408,
    f32 out) in the benchmark's launch configuration; output rows sampled at
    the k-tile boundaries and at random, for the largest, smallest and a
    spread of other groups."""
    import moe_grouped_matrix_amd as m
    case = workloads.tgmm_bf16(device="cuda")
    sizes = case.sizes_list()
    print(f"tgmm full case M={case.M} K={case.K} N={case.N} Ga={case.num_active} "
          f"sizes {min(sizes)}..{max(sizes)}", flush=True)
    out = torch.empty((case.num_active, case.K, case.N), dtype=case.out_dtype, device="cuda")
    m.tgmm(case.lhs, case.rhs, case.group_sizes, num_active=case.num_active, out=out)
    torch.cuda.synchronize()
    assert m.device_flags() == 0
    order = np.argsort(sizes)
    groups = sorted({int(order[0]), int(order[-1]), int(order[len(order) // 2])} |
                    set(int(x) for x in np.random.default_rng(3).choice(len(sizes), 6, replace=False)))
    ks = [0, 1, 127, 128, 255, 256, 1023, 1024, 1279, 1280, 1407]
    rng = np.random.default_rng(4)
    sel = [(h, k) for h in groups for k in ks] + [(int(h), int(k)) for h, k in
                                                  zip(rng.integers(0, case.num_active, 24),
                                                      rng.integers(0, case.K, 24))]
    ref = oracle.tgmm_reference(case.lhs.cpu(), case.rhs.cpu(), case.group_sizes.cpu(),
                                num_active=case.num_active, select=sel)
    idx_h = torch.tensor([h for h, _ in sel], device="cuda")
    idx_k = torch.tensor([k for _, k in sel], device="cuda")
    got = out[idx_h, idx_k].cpu()
    rel = compare(got, ref, case.out_dtype, f"tgmm full ({len(sel)} rows)")
    print(f"tgmm full: {len(sel)} rows compared, error {rel:.3e}", flush=True)
