"""Seeded random problems across the space gmm_run accepts, every element
against the oracle.

Each trial draws a dtype path (f32, bf16, the one-byte pairs and packed
four-bit operands on either side; NT, and the in-place NN layout where it
is accepted), K and N on and off the tile
multiples, a group count and offset, group sizes mixing empty groups, tile
edges (one either side of 32, 64, 128 and 256 rows) and free sizes, spare
rows past the last group, optional block scales on either side (any block
that divides K into multiples of the instruction's K step), an optional
bf16 or f32 bias, f32 or bf16 output, sometimes an existing output whose
rows outside the active groups must survive bit for bit, the tile family
and sometimes a small grid so that each workgroup runs several tiles.  The
kernel the library picks (general, big, weight-streaming, W8A8) follows
from the draw, so the trials cross the dispatcher's boundaries rather than
one kernel's.

The bar is the parity bar of the other tests: f32 output within 1e-4 of the
largest reference magnitude, bf16 output within 2e-2 relative Frobenius
error overall and per row, rows outside the active groups zero (or the
existing output's bits).  The same for the transposed product (tgmm): group
counts, offsets, K and N on and off the tile multiples, f32 or bf16 output,
the grid (the single-queue and per-XCD schedules) and the allocation-free
entry point."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import compare

pytestmark = pytest.mark.gpu

# (lhs, rhs, NN accepted, K step of the path): a dtype, or the name of a
# packed four-bit format (two elements to a byte, even ones in the low nibble)
PATHS = [
    (torch.float32, torch.float32, True, 32),
    (torch.bfloat16, torch.bfloat16, True, 64),
    (torch.bfloat16, torch.float8_e4m3fn, False, 64),
    (torch.bfloat16, torch.float8_e5m2, False, 64),
    (torch.bfloat16, torch.int8, False, 64),
    (torch.float8_e4m3fn, torch.float8_e4m3fn, False, 128),
    (torch.float8_e5m2, torch.float8_e4m3fn, False, 128),
    (torch.int8, torch.int8, False, 128),
    (torch.bfloat16, "int4", False, 64),
    (torch.bfloat16, "uint4", False, 64),
    (torch.bfloat16, "fp4_e2m1", False, 64),
    ("int4", torch.int8, False, 128),
    (torch.int8, "uint4", False, 128),
    ("fp4_e2m1", torch.float8_e4m3fn, False, 128),
    (torch.float8_e5m2, "fp4_e2m1", False, 128),
    ("fp4_e2m1", "fp4_e2m1", False, 128),
]
EDGES = [1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]
MAC_BUDGET = 3e8  # M*K*N per trial: the oracle takes well under a second
TRIALS = 160


def _values(rng, shape, dtype, gen):
    if isinstance(dtype, str):  # packed bytes: every nibble value
        return torch.randint(0, 256, (*shape[:-1], shape[-1] // 2), generator=gen).to(torch.uint8)
    if dtype == torch.int8:
        return torch.randint(-127, 128, shape, generator=gen, dtype=torch.int32).to(torch.int8)
    x = torch.randn(shape, generator=gen)
    if dtype in (torch.float8_e4m3fn, torch.float8_e5m2):
        return (x * float(rng.choice([1.0, 8.0, 32.0]))).clamp(-448.0, 448.0).to(dtype)
    return x.to(dtype)


def _sizes(rng, G):
    out = []
    for _ in range(G):
        u = rng.random()
        if u < 0.15:
            out.append(0)
        elif u < 0.6:
            out.append(int(rng.choice(EDGES)))
        else:
            out.append(int(rng.integers(1, 600)))
    return out


def _draw(trial):
    rng = np.random.default_rng(7100 + trial)
    gen = torch.Generator().manual_seed(7100 + trial)
    ld, rd, nn_ok, kg = PATHS[trial % len(PATHS)]
    T = bool(nn_ok and rng.random() < 0.5)
    G = int(rng.integers(1, 13))
    s = int(rng.integers(0, G))
    ga = int(rng.integers(1, G - s + 1)) if rng.random() < 0.9 else 0
    sizes = _sizes(rng, G)
    M = max(1, sum(sizes) + int(rng.integers(0, 20)))
    K = kg * int(rng.integers(1, max(2, 1024 // kg) + 1))
    N = 8 * int(rng.integers(1, 97))
    while M * K * N > MAC_BUDGET and N > 8:
        N = max(8, (N // 2) // 8 * 8)
    while M * K * N > MAC_BUDGET and K > kg:
        K = max(kg, (K // 2) // kg * kg)
    lhs = _values(rng, (M, K), ld, gen)
    rhs = _values(rng, (ga, K, N) if T else (ga, N, K), rd, gen)
    kw = dict(group_offset=s, transpose_rhs=T,
              out_dtype=torch.float32 if rng.random() < 0.5 else torch.bfloat16)
    fmt = dict(lhs_format=ld if isinstance(ld, str) else None, rhs_format=rd if isinstance(rd, str) else None)
    narrow = rd not in (torch.float32, torch.bfloat16)
    if rng.random() < (0.8 if narrow else 0.3):
        steps = K // kg
        divs = [d for d in range(1, steps + 1) if steps % d == 0]
        nb = steps // int(rng.choice(divs))
        if K % 128 == 0 and rng.random() < 0.5:
            nb = K // 128  # blocks of 128: the weight-streaming and W8A8 kernels' form
        kw["rhs_scale"] = (torch.rand((ga, nb, 1, N), generator=gen) + 0.5) * float(2.0 ** rng.integers(-6, 3))
        if ld not in (torch.float32, torch.bfloat16) and rng.random() < 0.7:
            kw["lhs_scale"] = (torch.rand((M, nb), generator=gen) + 0.5) * float(2.0 ** rng.integers(-4, 3))
    if rng.random() < 0.5:
        bdt = torch.bfloat16 if rng.random() < 0.5 else torch.float32
        kw["rhs_bias"] = (torch.randn((ga, 1, N), generator=gen) * 4.0).to(bdt)
    existing = None
    if rng.random() < 0.2:
        existing = torch.randn((M, N), generator=gen).to(kw["out_dtype"])
    policy = int(rng.choice([0, 1, 2]))
    grid = int(rng.choice([0, 0, 0, 5, 16, 40]))
    sz = torch.tensor(sizes, dtype=torch.int32)
    case = workloads.Case(f"sweep{trial}", lhs, rhs, sz, meta=dict(K=K, **fmt), **kw)
    return case, existing, policy, grid


@pytest.mark.parametrize("trial", range(TRIALS))
def test_random_problem_matches_the_oracle(trial):
    import moe_grouped_matrix_amd as m
    case, existing, policy, grid = _draw(trial)
    fmt = {k: v for k, v in case.meta.items() if k != "K"}
    print(f"sweep trial {trial}: lhs {fmt['lhs_format'] or case.lhs.dtype} rhs {fmt['rhs_format'] or case.rhs.dtype} "
          f"nn={case.transpose_rhs} M={case.M} K={case.meta['K']} N={case.N} sizes={case.sizes_list()} s={case.group_offset} "
          f"ga={case.num_active} out={case.out_dtype} rhs_scale={None if case.rhs_scale is None else tuple(case.rhs_scale.shape)} "
          f"lhs_scale={case.lhs_scale is not None} bias={None if case.rhs_bias is None else case.rhs_bias.dtype} "
          f"existing={existing is not None} policy={policy} grid={grid}", flush=True)
    g = case.to("cuda")
    m.set_tile_policy(policy)
    m.set_grid_limit(grid)
    try:
        out = m.gmm(g.lhs, g.rhs, g.group_sizes, out_dtype=case.out_dtype, rhs_scale=g.rhs_scale,
                    rhs_bias=g.rhs_bias, lhs_scale=g.lhs_scale, group_offset=case.group_offset,
                    transpose_rhs=case.transpose_rhs, **fmt,
                    existing_out=None if existing is None else existing.clone().cuda())
        torch.cuda.synchronize()
        assert m.device_flags() == 0
    finally:
        m.set_tile_policy(0)
        m.set_grid_limit(0)
    out = out.cpu()
    s = case.sizes_list()
    o = np.concatenate([[0], np.cumsum(s)])
    lo, hi = int(o[case.group_offset]), int(o[case.group_offset + case.num_active])
    if hi > lo:
        rows = list(range(lo, hi))
        ref = oracle.gmm_reference(case.lhs, case.rhs, case.group_sizes, group_offset=case.group_offset,
                                   transpose_rhs=case.transpose_rhs, rhs_scale=case.rhs_scale,
                                   rhs_bias=case.rhs_bias, lhs_scale=case.lhs_scale, rows=rows, **fmt)
        compare(out[lo:hi], ref, case.out_dtype, what=f"trial {trial}")
    outside = torch.cat([out[:lo], out[hi:]])
    if existing is None:
        bits = outside.view(torch.int16 if out.dtype == torch.bfloat16 else torch.int32)
        assert int((bits != 0).sum()) == 0, "rows outside the active groups are not zero"
    else:
        assert torch.equal(outside, torch.cat([existing[:lo], existing[hi:]])), \
            "rows outside the active groups do not keep the existing output"


# The transposed product (the weight gradient): bf16 operands, f32 or bf16
# out [Ga,K,N]; group counts past 16 with grids that are multiples of 8
# reach the per-XCD schedules, other grids the single queue.
TG_TRIALS = 48


def _draw_tgmm(trial):
    rng = np.random.default_rng(8200 + trial)
    gen = torch.Generator().manual_seed(8200 + trial)
    G = int(rng.integers(1, 41))
    s = int(rng.integers(0, G))
    ga = int(rng.integers(1, G - s + 1)) if rng.random() < 0.9 else 0
    sizes = _sizes(rng, G)
    M = max(1, sum(sizes) + int(rng.integers(0, 20)))
    K = 8 * int(rng.integers(1, 101))
    N = 8 * int(rng.integers(1, 101))
    rows = max(1, sum(sizes[s:s + ga]))
    while rows * K * N > MAC_BUDGET and K > 8:
        K = max(8, (K // 2) // 8 * 8)
    lhs = torch.randn((M, K), generator=gen).to(torch.bfloat16)
    rhs = torch.randn((M, N), generator=gen).to(torch.bfloat16)
    out_dtype = torch.float32 if rng.random() < 0.6 else torch.bfloat16
    grid = int(rng.choice([0, 0, 5, 8, 16, 24, 40]))
    no_alloc = bool(rng.random() < 0.2)
    return lhs, rhs, sizes, s, ga, out_dtype, grid, no_alloc


@pytest.mark.parametrize("trial", range(TG_TRIALS))
def test_random_tgmm_problem_matches_the_oracle(trial):
    import moe_grouped_matrix_amd as m
    lhs, rhs, sizes, s, ga, out_dtype, grid, no_alloc = _draw_tgmm(trial)
    K, N = lhs.shape[1], rhs.shape[1]
    print(f"tgmm sweep trial {trial}: M={lhs.shape[0]} K={K} N={N} sizes={sizes} s={s} ga={ga} "
          f"out={out_dtype} grid={grid} no_alloc={no_alloc}", flush=True)
    gs = torch.tensor(sizes, dtype=torch.int32)
    m.set_grid_limit(grid)
    try:
        out = m.tgmm(lhs.cuda(), rhs.cuda(), gs.cuda(), num_active=ga, group_offset=s, out_dtype=out_dtype,
                     no_alloc=no_alloc)
        torch.cuda.synchronize()
        assert m.device_flags() == 0
    finally:
        m.set_grid_limit(0)
    assert tuple(out.shape) == (ga, K, N)
    if ga == 0:
        return
    out = out.cpu()
    ref = oracle.tgmm_reference(lhs, rhs, gs, group_offset=s, num_active=ga)
    compare(out.reshape(ga * K, N), ref.reshape(ga * K, N), out_dtype, what=f"tgmm trial {trial}")
    iv = torch.int16 if out_dtype == torch.bfloat16 else torch.int32
    for h in range(ga):
        if sizes[s + h] == 0:
            assert int((out[h].view(iv) != 0).sum()) == 0, f"empty group {h} is not all-zero bits"
        elif out_dtype == torch.float32:
            scale = np.abs(ref[h]).max()
            err = np.abs(out[h].double().numpy() - ref[h]).max()
            assert err <= 1e-4 * max(scale, 1e-30), f"group {h}: max err {err} against {scale}"
