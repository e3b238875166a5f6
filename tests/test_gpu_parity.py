"""HIP path against the oracle, element by element, at sizes the oracle
finishes in seconds (several tiles in M, N and K, ragged group boundaries,
empty groups, an N tail), for every dtype path and both tile families.
Also the probes that must hold bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import (active_range, assert_zero_rows, compare, reference, run_gpu)

pytestmark = pytest.mark.gpu

POLICIES = [("auto", 0), ("small", 1), ("big", 2)]


@pytest.fixture(params=POLICIES, ids=[p[0] for p in POLICIES])
def tile_policy(request):
    import moe_grouped_matrix_amd as m
    m.set_tile_policy(request.param[1])
    yield request.param[1]
    m.set_tile_policy(0)


@pytest.mark.parametrize("name", list(workloads.SMALL))
def test_small_workloads_all_elements(name, tile_policy):
    case = workloads.SMALL[name]().to("cuda")
    print(f"case {name} policy {tile_policy} M={case.M} K={case.K} N={case.N} "
          f"G={case.group_sizes.numel()} Ga={case.num_active}", flush=True)
    out = run_gpu(case)
    ref = reference(case)
    lo, hi = active_range(case)
    assert_zero_rows(out, lo, hi)
    compare(out.cpu()[lo:hi], ref[lo:hi], case.out_dtype, name)
    import moe_grouped_matrix_amd as m
    assert m.device_flags() == 0


def _case(lhs, rhs, sizes, **kw):
    return workloads.Case("probe", lhs.cuda(), rhs.cuda(),
                          torch.tensor(sizes, dtype=torch.int32, device="cuda"),
                          **{k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in kw.items()})


PATHS = [
    # (lhs dtype, rhs dtype, transpose_rhs, K granule)
    (torch.float32, torch.float32, False, 32),
    (torch.float32, torch.float32, True, 32),
    (torch.bfloat16, torch.bfloat16, False, 64),
    (torch.bfloat16, torch.bfloat16, True, 64),
    (torch.bfloat16, torch.float8_e4m3fn, False, 64),
    (torch.float8_e4m3fn, torch.float8_e4m3fn, False, 128),
    (torch.bfloat16, torch.float8_e5m2, False, 64),
    (torch.float8_e5m2, torch.float8_e5m2, False, 128),
    (torch.float8_e4m3fn, torch.float8_e5m2, False, 128),
    (torch.float8_e5m2, torch.float8_e4m3fn, False, 128),
    (torch.bfloat16, torch.int8, False, 64),
    (torch.int8, torch.int8, False, 128),
]
PATH_IDS = ["f32_nt", "f32_nn", "bf16_nt", "bf16_nn", "bf16xe4m3_nt", "e4m3xe4m3_nt",
            "bf16xe5m2_nt", "e5m2xe5m2_nt", "e4m3xe5m2_nt", "e5m2xe4m3_nt", "bf16xi8_nt", "i8xi8_nt"]


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_bias_probe_maps_every_row_to_its_group(path, tile_policy):
    """rhs = 0 and bias[g] = g+1 (exact in bf16): every active row must read
    exactly its group's number, every other row 0."""
    ld, rd, T, kg = path
    sizes = [0, 37, 1, 0, 64, 65, 3, 0, 255, 2]
    M, K, N = sum(sizes) + 21, 2 * kg, 136
    Ga = len(sizes) - 2
    lhs = torch.randn(M, K).to(ld)
    rhs = torch.zeros(Ga, K, N) if T else torch.zeros(Ga, N, K)
    bias = (torch.arange(Ga, dtype=torch.float32) + 3)[:, None, None].expand(Ga, 1, N).contiguous()
    for bias_dtype in (torch.float32, torch.bfloat16):
        case = _case(lhs, rhs.to(rd), sizes, group_offset=1, transpose_rhs=T,
                     rhs_bias=bias.to(bias_dtype), out_dtype=torch.float32)
        out = run_gpu(case).cpu()
        ref, rg = reference(case, return_row_group=True)
        assert torch.equal(out, oracle.round_to(ref, torch.float32))
        want = np.where(rg >= 0, rg - 1 + 3, 0).astype(np.float64)
        assert np.array_equal(out[:, 0].numpy(), want)


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_exact_small_integer_inputs_are_bit_exact(path, tile_policy):
    """Small integers make every product and partial sum exact in fp32, so the
    rounded outputs must equal the oracle's bit for bit, whatever the order."""
    ld, rd, T, kg = path
    g = torch.Generator().manual_seed(1)
    sizes = [33, 0, 70, 257, 5]
    M, K, N = sum(sizes) + 7, 4 * kg, 200
    lhs = torch.randint(-3, 4, (M, K), generator=g).to(torch.float32).to(ld)
    shape = (len(sizes), K, N) if T else (len(sizes), N, K)
    rhs = torch.randint(-3, 4, shape, generator=g).to(torch.float32).to(rd)
    for out_dtype in (torch.float32, torch.bfloat16):
        case = _case(lhs, rhs, sizes, transpose_rhs=T, out_dtype=out_dtype)
        out = run_gpu(case).cpu()
        want = oracle.round_to(reference(case), out_dtype)
        assert torch.equal(out.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32),
                           want.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32))


@pytest.mark.parametrize("N", [392, 264])
@pytest.mark.parametrize("T", [False, True], ids=["nt", "nn"])
def test_big_kernel_fewest_k_steps_ragged_n_bias_or_none(N, T):
    """The bf16 big kernel at its fewest K steps for a bf16 K (K = 192: six
    steps of 32, one pass of the middle loop), N tails of 136 columns (full
    tile mode) and 8 columns (half mode), row tiles of at most 128 rows, with
    and without a bias (separate instantiations: without one nothing is
    added), f32 and bf16 output.  Small integers make every sum exact, so the
    output must equal the oracle's bit for bit."""
    import moe_grouped_matrix_amd as m
    g = torch.Generator().manual_seed(7)
    sizes = [300, 0, 129, 40, 512, 3]
    M, K = sum(sizes) + 5, 192
    lhs = torch.randint(-3, 4, (M, K), generator=g).to(torch.bfloat16)
    rhs = torch.randint(-3, 4, (len(sizes), K, N) if T else (len(sizes), N, K), generator=g).to(torch.bfloat16)
    bias = torch.randint(-8, 9, (len(sizes), 1, N), generator=g).to(torch.bfloat16)
    m.set_tile_policy(2)
    try:
        for b in (None, bias):
            for out_dtype in (torch.float32, torch.bfloat16):
                print(f"big kernel K={K} N={N} nn={T} bias={b is not None} out={out_dtype}", flush=True)
                kw = {} if b is None else {"rhs_bias": b}
                case = _case(lhs, rhs, sizes, transpose_rhs=T, out_dtype=out_dtype, **kw)
                out = run_gpu(case).cpu()
                want = oracle.round_to(reference(case), out_dtype)
                iv = torch.int16 if out_dtype == torch.bfloat16 else torch.int32
                assert torch.equal(out.view(iv), want.view(iv)), (N, T, b is not None, out_dtype)
        assert m.device_flags() == 0
    finally:
        m.set_tile_policy(0)


@pytest.mark.parametrize("fmt", ["int4", "uint4", "fp4_e2m1"])
def test_four_bit_weights_are_bit_exact(fmt, tile_policy):
    """bf16 x packed four-bit weights (two to a byte, even elements in the
    low nibble): small-integer activations make every product and sum exact,
    so the outputs equal the oracle's bit for bit -- plain, and with
    power-of-two block scales and a bias; fp4 also as float4_e2m1fn_x2."""
    import moe_grouped_matrix_amd as m
    g = torch.Generator().manual_seed(7)
    sizes = [33, 0, 70, 257, 5]
    M, K, N, nb = sum(sizes) + 7, 256, 200, 2
    lhs = torch.randint(-3, 4, (M, K), generator=g).to(torch.bfloat16)
    packed = torch.randint(0, 256, (len(sizes), N, K // 2), generator=g).to(torch.uint8)
    rs = 2.0 ** torch.randint(-3, 4, (len(sizes), nb, 1, N), generator=g).to(torch.float32)
    bias = torch.randint(-8, 9, (len(sizes), 1, N), generator=g).to(torch.bfloat16)
    gs = torch.tensor(sizes, dtype=torch.int32)
    print(f"four-bit {fmt} policy {tile_policy}", flush=True)
    for out_dtype, kw in ((torch.float32, {}), (torch.bfloat16, {}),
                          (torch.float32, dict(rhs_scale=rs, rhs_bias=bias))):
        out = m.gmm(lhs.cuda(), packed.cuda(), gs.cuda(), rhs_format=fmt, out_dtype=out_dtype,
                    **{k: v.cuda() for k, v in kw.items()}).cpu()
        want = oracle.round_to(oracle.gmm_reference(lhs, packed, gs, rhs_format=fmt, **kw), out_dtype)
        iv = torch.int16 if out_dtype == torch.bfloat16 else torch.int32
        assert torch.equal(out.view(iv), want.view(iv)), (fmt, out_dtype, list(kw))
    if fmt == "fp4_e2m1":
        out = m.gmm(lhs.cuda(), packed.view(torch.float4_e2m1fn_x2).cuda(), gs.cuda(), rhs_format=fmt).cpu()
        assert torch.equal(out, oracle.round_to(oracle.gmm_reference(lhs, packed, gs, rhs_format=fmt),
                                                torch.float32))
    assert m.device_flags() == 0


FOUR_BIT_PAIRS = [
    # (lhs, rhs): a packed four-bit format name or a one-byte dtype
    ("int4", "int4"), ("int4", "uint4"), ("int4", torch.int8), ("uint4", "int4"), ("uint4", "uint4"),
    ("uint4", torch.int8), (torch.int8, "int4"), (torch.int8, "uint4"),
    ("fp4_e2m1", "fp4_e2m1"), ("fp4_e2m1", torch.float8_e4m3fn), ("fp4_e2m1", torch.float8_e5m2),
    (torch.float8_e4m3fn, "fp4_e2m1"), (torch.float8_e5m2, "fp4_e2m1"),
]


def _pair_id(p):
    return "x".join(k if isinstance(k, str) else str(k).split(".")[-1] for k in p)


def _operand(kind, shape, g):
    """(tensor, packed format or None): packed bytes with every nibble
    value, or small integers in a one-byte type."""
    if isinstance(kind, str):
        return torch.randint(0, 256, (*shape[:-1], shape[-1] // 2), generator=g).to(torch.uint8), kind
    lo, hi = (-8, 8) if kind == torch.int8 else (-6, 7)
    return torch.randint(lo, hi, shape, generator=g).to(torch.float32).to(kind), None


@pytest.mark.parametrize("pair", FOUR_BIT_PAIRS, ids=[_pair_id(p) for p in FOUR_BIT_PAIRS])
def test_four_bit_activations_are_bit_exact(pair, tile_policy):
    """Four-bit activations (the Megablox gmm's dtype list holds for lhs as
    for rhs): int4 / uint4 on the int8 matrix instruction, fp4 e2m1 on the
    f8f6f4 one, each with the other four-bit and one-byte types.  Every
    product and partial sum is exact in fp32 (block partials below 2^15,
    power-of-two scales 2^-3 .. 2^3), so the outputs equal the oracle's bit
    for bit: plain (f32 and bf16 out) and with both block scales and a
    bias."""
    import moe_grouped_matrix_amd as m
    g = torch.Generator().manual_seed(8)
    sizes = [33, 0, 70, 257, 5]
    M, K, N, nb = sum(sizes) + 7, 256, 200, 2
    lhs, lf = _operand(pair[0], (M, K), g)
    rhs, rf = _operand(pair[1], (len(sizes), N, K), g)
    rs = 2.0 ** torch.randint(-2, 3, (len(sizes), nb, 1, N), generator=g).to(torch.float32)
    ls = 2.0 ** torch.randint(-1, 2, (M, nb), generator=g).to(torch.float32)
    bias = torch.randint(-8, 9, (len(sizes), 1, N), generator=g).to(torch.bfloat16)
    gs = torch.tensor(sizes, dtype=torch.int32)
    print(f"four-bit activations {_pair_id(pair)} policy {tile_policy}", flush=True)
    for out_dtype, kw in ((torch.float32, {}), (torch.bfloat16, {}),
                          (torch.float32, dict(rhs_scale=rs, lhs_scale=ls, rhs_bias=bias))):
        out = m.gmm(lhs.cuda(), rhs.cuda(), gs.cuda(), lhs_format=lf, rhs_format=rf, out_dtype=out_dtype,
                    **{k: v.cuda() for k, v in kw.items()}).cpu()
        want = oracle.round_to(oracle.gmm_reference(lhs, rhs, gs, lhs_format=lf, rhs_format=rf, **kw), out_dtype)
        iv = torch.int16 if out_dtype == torch.bfloat16 else torch.int32
        assert torch.equal(out.view(iv), want.view(iv)), (_pair_id(pair), out_dtype, list(kw))
    assert m.device_flags() == 0


def test_four_bit_activations_need_a_matching_family():
    """A four-bit activation with a weight outside its family (int4 with an
    fp8 weight, fp4 with a bf16 weight) is a valid problem this library does
    not run."""
    import moe_grouped_matrix_amd as m
    gs = torch.tensor([4], dtype=torch.int32, device="cuda")
    lhs = torch.zeros(4, 64, dtype=torch.uint8, device="cuda")
    for fmt, rhs in (("int4", torch.zeros(1, 8, 128, dtype=torch.float8_e4m3fn, device="cuda")),
                     ("fp4_e2m1", torch.zeros(1, 8, 128, dtype=torch.bfloat16, device="cuda"))):
        with pytest.raises(m.GmmUnsupported):
            m.gmm(lhs, rhs, gs, lhs_format=fmt)


MX_PAIRS = [(torch.float8_e4m3fn, torch.float8_e4m3fn), (torch.float8_e5m2, torch.float8_e4m3fn),
            (torch.float8_e4m3fn, torch.float8_e5m2), (torch.float8_e5m2, torch.float8_e5m2),
            ("fp4_e2m1", "fp4_e2m1"), ("fp4_e2m1", torch.float8_e4m3fn), (torch.float8_e4m3fn, "fp4_e2m1"),
            ("fp4_e2m1", torch.float8_e5m2), (torch.float8_e5m2, "fp4_e2m1")]


@pytest.mark.parametrize("pair", MX_PAIRS, ids=[_pair_id(p) for p in MX_PAIRS])
def test_e8m0_block_scales_on_the_scaled_instruction_are_bit_exact(pair, tile_policy):
    """E8M0 block scales of 32 K elements (the microscaling block; the
    metrale gemm_quant.rs page's E8M0 scale bytes) applied by gfx950's
    scaled f8f6f4 instruction, per row and per column, for every pair of
    e4m3fn, e5m2 and fp4 e2m1 operands.  Small-integer (fp8) or fp4 operands and scales 2^-2 .. 2^2 keep
    every sum exact in fp32: bit-exact against the oracle, which multiplies
    by 2^(e-127) block by block."""
    import moe_grouped_matrix_amd as m
    g = torch.Generator().manual_seed(10)
    sizes = [33, 0, 70, 257, 5]
    M, K, N = sum(sizes) + 7, 256, 200
    nb = K // 32
    lhs, lf = _operand(pair[0], (M, K), g)
    rhs, rf = _operand(pair[1], (len(sizes), N, K), g)
    er = torch.randint(125, 130, (len(sizes), nb, 1, N), generator=g).to(torch.uint8).view(torch.float8_e8m0fnu)
    el = torch.randint(126, 130, (M, nb), generator=g).to(torch.uint8).view(torch.float8_e8m0fnu)
    bias = torch.randint(-8, 9, (len(sizes), 1, N), generator=g).to(torch.bfloat16)
    gs = torch.tensor(sizes, dtype=torch.int32)
    print(f"E8M0 scales {_pair_id(pair)} policy {tile_policy}", flush=True)
    for out_dtype, kw in ((torch.float32, dict(rhs_scale=er)), (torch.float32, dict(lhs_scale=el)),
                          (torch.float32, dict(rhs_scale=er, lhs_scale=el, rhs_bias=bias)),
                          (torch.bfloat16, dict(rhs_scale=er, lhs_scale=el))):
        out = m.gmm(lhs.cuda(), rhs.cuda(), gs.cuda(), lhs_format=lf, rhs_format=rf, out_dtype=out_dtype,
                    **{k: v.cuda() for k, v in kw.items()}).cpu()
        want = oracle.round_to(oracle.gmm_reference(lhs, rhs, gs, lhs_format=lf, rhs_format=rf, **kw), out_dtype)
        iv = torch.int16 if out_dtype == torch.bfloat16 else torch.int32
        assert torch.equal(out.view(iv), want.view(iv)), (_pair_id(pair), out_dtype, list(kw))
    assert m.device_flags() == 0


def test_e8m0_block_scales_limits():
    """E8M0 scales need f8f6f4 operands (e4m3fn, e5m2, fp4 e2m1), blocks
    of 32, and E8M0 on both sides."""
    import moe_grouped_matrix_amd as m
    gs = torch.tensor([4], dtype=torch.int32, device="cuda")
    e8 = lambda *sh: torch.full(sh, 127, dtype=torch.uint8, device="cuda").view(torch.float8_e8m0fnu)  # noqa: E731
    lhs8 = torch.zeros(4, 128, dtype=torch.float8_e4m3fn, device="cuda")
    rhs8 = torch.zeros(1, 8, 128, dtype=torch.float8_e4m3fn, device="cuda")
    with pytest.raises(m.GmmUnsupported):
        m.gmm(lhs8, rhs8, gs, rhs_scale=e8(1, 2, 1, 8))  # blocks of 64
    with pytest.raises(m.GmmInvalid):
        m.gmm(lhs8, rhs8, gs, rhs_scale=e8(1, 4, 1, 8),
              lhs_scale=torch.ones(4, 4, dtype=torch.float32, device="cuda"))
    with pytest.raises(m.GmmUnsupported):
        m.gmm(torch.zeros(4, 128, dtype=torch.bfloat16, device="cuda"), rhs8, gs, rhs_scale=e8(1, 4, 1, 8))


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_scaled_exact_inputs_are_bit_exact(path, tile_policy):
    """Power-of-two block scales, per-row scales and a bias keep the integer
    arithmetic exact: bit-exact against the oracle."""
    ld, rd, T, kg = path
    g = torch.Generator().manual_seed(2)
    sizes = [40, 0, 90, 3]
    nb = 3
    M, K, N = sum(sizes) + 5, nb * (128 if kg == 128 else 2 * kg), 72
    lhs = torch.randint(-3, 4, (M, K), generator=g).to(torch.float32).to(ld)
    shape = (len(sizes), K, N) if T else (len(sizes), N, K)
    rhs = torch.randint(-3, 4, shape, generator=g).to(torch.float32).to(rd)
    rs = 2.0 ** torch.randint(-3, 4, (len(sizes), nb, 1, N), generator=g).to(torch.float32)
    ls = 2.0 ** torch.randint(-2, 3, (M, nb), generator=g).to(torch.float32)
    bias = torch.randint(-8, 9, (len(sizes), 1, N), generator=g).to(torch.bfloat16)
    for kw in (dict(rhs_scale=rs), dict(rhs_scale=rs, rhs_bias=bias), dict(lhs_scale=ls),
               dict(rhs_scale=rs, lhs_scale=ls, rhs_bias=bias)):
        print(f"scaled {list(kw)} nn={T} policy {tile_policy}", flush=True)
        case = _case(lhs, rhs, sizes, transpose_rhs=T, out_dtype=torch.float32, **kw)
        out = run_gpu(case).cpu()
        assert torch.equal(out, oracle.round_to(reference(case), torch.float32)), list(kw)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_transpose_identity(dtype, tile_policy):
    """gmm(L, W, transpose_rhs) == gmm(L, W^T) on the explicitly transposed
    weight: the NN path stages the same operands, so the bits agree."""
    g = torch.Generator().manual_seed(3)
    sizes = [100, 0, 300, 17]
    M, K, N = 430, 192, 264
    lhs = torch.randn(M, K, generator=g).to(dtype)
    w = torch.randn(len(sizes), K, N, generator=g).to(dtype)
    nn = run_gpu(_case(lhs, w, sizes, transpose_rhs=True, out_dtype=torch.float32))
    nt = run_gpu(_case(lhs, w.transpose(1, 2).contiguous(), sizes, out_dtype=torch.float32))
    assert torch.equal(nn, nt)


def test_identity_probe_power_of_two():
    """W_g = 2^j_g * I reproduces the rows times 2^j_g exactly (NT and NN)."""
    sizes = [20, 0, 45, 7]
    M, K = 80, 128
    lhs = torch.randn(M, K).to(torch.bfloat16)
    eye = torch.eye(K)
    w = torch.stack([eye * 2.0 ** j for j in (-2, 5, 0, 3)]).to(torch.bfloat16)
    for T in (False, True):
        out = run_gpu(_case(lhs, w, sizes, transpose_rhs=T, out_dtype=torch.bfloat16)).cpu()
        o = np.concatenate([[0], np.cumsum(sizes)])
        for gi, j in enumerate((-2, 5, 0, 3)):
            a, b = o[gi], o[gi + 1]
            assert torch.equal(out[a:b].float(), lhs[a:b].float() * 2.0 ** j)
        assert torch.all(out[o[-1]:] == 0)


def test_brute_force_tiny_compositions():
    """Many small compositions of rows into groups, including zero groups and
    sizes one either side of the tile heights, for both tile families."""
    import moe_grouped_matrix_amd as m
    rng = np.random.default_rng(4)
    K, N = 64, 64
    for policy in (1, 2):
        m.set_tile_policy(policy)
        try:
            for trial in range(40):
                G = int(rng.integers(1, 6))
                sizes = [int(x) for x in rng.choice([0, 1, 2, 31, 32, 33, 63, 255, 256, 257], size=G)]
                M = sum(sizes) + int(rng.integers(0, 3))
                if M == 0:
                    continue
                s = int(rng.integers(0, G))
                ga = int(rng.integers(0, G - s + 1))
                lhs = torch.randn(M, K).to(torch.bfloat16)
                rhs = torch.randn(max(ga, 0), N, K).to(torch.bfloat16)
                case = _case(lhs, rhs, sizes, group_offset=s, out_dtype=torch.float32)
                print(f"brute policy={policy} sizes={sizes} s={s} ga={ga}", flush=True)
                out = run_gpu(case).cpu()
                ref = reference(case)
                assert np.allclose(out.numpy(), ref, rtol=1e-5, atol=1e-4)
                lo, hi = active_range(case)
                assert_zero_rows(out, lo, hi)
        finally:
            m.set_tile_policy(0)


def test_no_active_group_writes_zeros_everywhere():
    sizes = [10, 20, 5]
    lhs = torch.randn(40, 64).to(torch.bfloat16)
    for s in range(4):
        case = _case(lhs, torch.zeros(0, 32, 64).to(torch.bfloat16), sizes, group_offset=s,
                     out_dtype=torch.bfloat16)
        out = torch.full((40, 32), 7.0, dtype=torch.bfloat16, device="cuda")
        import moe_grouped_matrix_amd as m
        m.gmm(case.lhs, case.rhs, case.group_sizes, group_offset=s, out=out)
        torch.cuda.synchronize()
        assert int((out.view(torch.int16) != 0).sum()) == 0


def test_zero_row_problems():
    """M = 0: gmm returns an empty output without a launch; tgmm writes every
    group of its output as zeros (all groups are empty) over a pre-filled
    buffer, and no data error is flagged."""
    import moe_grouped_matrix_amd as m
    lhs = torch.zeros(0, 64, dtype=torch.bfloat16, device="cuda")
    w = torch.randn(2, 32, 64).to(torch.bfloat16).cuda()
    gs = torch.zeros(2, dtype=torch.int32, device="cuda")
    out = m.gmm(lhs, w, gs, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (0, 32)
    rhs = torch.zeros(0, 40, dtype=torch.bfloat16, device="cuda")
    gs3 = torch.zeros(3, dtype=torch.int32, device="cuda")
    for od in (torch.float32, torch.bfloat16):
        dw = torch.full((3, 64, 40), 7.0, dtype=od, device="cuda")
        m.tgmm(lhs, rhs, gs3, out=dw)
        torch.cuda.synchronize()
        assert int((dw.view(torch.int16) != 0).sum()) == 0
    assert m.device_flags() == 0


def test_single_group_is_dense_matmul():
    g = torch.Generator().manual_seed(5)
    lhs = torch.randn(300, 256, generator=g).to(torch.bfloat16)
    w = torch.randn(1, 136, 256, generator=g).to(torch.bfloat16)
    out = run_gpu(_case(lhs, w, [300], out_dtype=torch.float32)).cpu().double()
    want = lhs.double() @ w[0].double().t()
    assert (out - want).abs().max() <= 1e-4 * want.abs().max()


def test_invalid_device_data_is_flagged_and_in_bounds():
    import moe_grouped_matrix_amd as m
    m.device_flags()
    lhs = torch.randn(64, 64).to(torch.bfloat16).cuda()
    rhs = torch.randn(3, 32, 64).to(torch.bfloat16).cuda()
    for sizes, off, flag in (([10, -5, 20], None, m.FLAG_NEGATIVE_SIZE),
                             ([40, 40, 40], None, m.FLAG_SIZES_EXCEED_M)):
        gs = torch.tensor(sizes, dtype=torch.int32, device="cuda")
        out = m.gmm(lhs, rhs, gs, group_offset=off)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
        assert m.device_flags() & flag
    gs = torch.tensor([10, 10, 10, 10], dtype=torch.int32, device="cuda")
    m.gmm(lhs, rhs, gs, group_offset=2)
    assert m.device_flags() & m.FLAG_BAD_OFFSET


def test_host_validation_errors():
    import moe_grouped_matrix_amd as m
    lhs = torch.randn(16, 64).to(torch.bfloat16).cuda()
    rhs = torch.randn(2, 32, 64).to(torch.bfloat16).cuda()
    gs = torch.tensor([8, 8], dtype=torch.int32, device="cuda")
    with pytest.raises(m.GmmInvalid):
        m.gmm(lhs, rhs[:, :, :32].contiguous(), gs)
    with pytest.raises(m.GmmInvalid):
        m.gmm(lhs, rhs, gs.to(torch.float32))
    with pytest.raises(m.GmmInvalid):
        m.gmm(lhs, rhs, gs, rhs_bias=torch.zeros(2, 1, 31, device="cuda"))
    with pytest.raises(m.GmmUnsupported):
        m.gmm(lhs[:, :48].contiguous(), rhs[:, :, :48].contiguous(), gs)
    with pytest.raises(m.GmmUnsupported):
        m.gmm(lhs, rhs.to(torch.float8_e4m3fn).transpose(1, 2).contiguous(), gs, transpose_rhs=True)
    with pytest.raises(m.GmmUnsupported):
        m.gmm(lhs.float(), rhs, gs)


STREAM_CASES = [
    # (tokens, K, N, out dtype, bias: None | bf16 | f32, scaled, rhs_scale block)
    (48, 768, 328, torch.bfloat16, "bf16", True),
    (48, 896, 640, torch.float32, "f32", True),
    (48, 1024, 192, torch.bfloat16, None, False),
    (48, 768, 256, torch.bfloat16, "bf16", "blk256"),
    (48, 384, 136, torch.bfloat16, "bf16", True),
    (600, 1152, 264, torch.float32, "bf16", True),
]


@pytest.mark.parametrize("wdtype,out_dtype", [(torch.float8_e5m2, torch.bfloat16),
                                              (torch.float8_e5m2, torch.float32),
                                              (torch.int8, torch.bfloat16)],
                         ids=["e5m2_bf16out", "e5m2_f32out", "int8_bf16out"])
def test_weight_streaming_kernel_other_weight_formats(wdtype, out_dtype):
    """The weight-streaming kernel with e5m2 or int8 weights (the decode
    recipe's weights re-encoded -- int8 rounded and clamped to +-127 --
    with their block scales and bias): every element against the oracle of
    the same bytes."""
    import moe_grouped_matrix_amd as m
    m.set_tile_policy(0)
    case = workloads.decode_fp8_weight(tokens=48, experts=24, K=768, N=328, forced_empty=8,
                                       group_offset=4, num_active=14, device="cuda")
    w = case.rhs.float()
    case.rhs = w.round().clamp(-127, 127).to(torch.int8) if wdtype == torch.int8 else w.to(wdtype)
    case.out_dtype = out_dtype
    print(f"stream {wdtype} M={case.M} active_rows={case.active_rows()} out={out_dtype}", flush=True)
    out = run_gpu(case)
    lo, hi = active_range(case)
    assert_zero_rows(out, lo, hi)
    compare(out.cpu()[lo:hi], reference(case)[lo:hi], out_dtype, f"stream {wdtype}")
    assert m.device_flags() == 0


@pytest.mark.parametrize("fmt", ["int4", "uint4", "fp4_e2m1"])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_weight_streaming_kernel_four_bit_weights_bit_exact(fmt, out_dtype):
    """The weight-streaming kernel with packed four-bit weights (two to a
    byte, the even element in the low nibble; every nibble value), on the
    decode recipe's group sizes and offset: small-integer activations,
    power-of-two block scales and an integer bias keep every product, block
    sum and fold exact, so the outputs equal the oracle's bit for bit -- on
    the full grid and on five workgroups (several tiles each)."""
    import moe_grouped_matrix_amd as m
    g = torch.Generator().manual_seed(11)
    base = workloads.decode_fp8_weight(tokens=48, experts=24, K=768, N=328, forced_empty=8,
                                       group_offset=4, num_active=14)
    sizes, s, Ga = base.group_sizes, base.group_offset, base.num_active
    M, K, N = base.M, 768, 328
    lhs = torch.randint(-3, 4, (M, K), generator=g).to(torch.bfloat16)
    packed = torch.randint(0, 256, (Ga, N, K // 2), generator=g).to(torch.uint8)
    rs = 2.0 ** torch.randint(-3, 4, (Ga, K // 128, 1, N), generator=g).to(torch.float32)
    bias = torch.randint(-8, 9, (Ga, 1, N), generator=g).to(torch.bfloat16)
    want = oracle.round_to(oracle.gmm_reference(lhs, packed, sizes, rhs_format=fmt, rhs_scale=rs, rhs_bias=bias,
                                                group_offset=s), out_dtype)
    iv = torch.int16 if out_dtype == torch.bfloat16 else torch.int32
    m.set_tile_policy(0)
    for grid in (0, 5):
        print(f"stream four-bit {fmt} out={out_dtype} grid={grid}", flush=True)
        m.set_grid_limit(grid)
        try:
            out = m.gmm(lhs.cuda(), packed.cuda(), sizes.cuda(), rhs_format=fmt, out_dtype=out_dtype,
                        rhs_scale=rs.cuda(), rhs_bias=bias.cuda(), group_offset=s)
            torch.cuda.synchronize()
        finally:
            m.set_grid_limit(0)
        assert torch.equal(out.cpu().view(iv), want.view(iv)), (fmt, out_dtype, grid)
    assert m.device_flags() == 0


def test_weight_streaming_kernel_mostly_inactive_rows():
    """An expert shard of a decode batch: 2 of 24 experts active, so almost
    all of the 2048 output rows lie outside the active groups and are zeroed
    by workgroups that have no tile."""
    import moe_grouped_matrix_amd as m
    m.set_tile_policy(0)
    case = workloads.decode_fp8_weight(tokens=256, experts=24, K=768, N=328, forced_empty=8,
                                       group_offset=5, num_active=2, device="cuda")
    print(f"stream shard M={case.M} active_rows={case.active_rows()}", flush=True)
    out = run_gpu(case)
    lo, hi = active_range(case)
    assert_zero_rows(out, lo, hi)
    compare(out.cpu()[lo:hi], reference(case)[lo:hi], case.out_dtype, "stream shard")
    assert m.device_flags() == 0


@pytest.mark.parametrize("tokens,K,N,out_dtype,bias,scaled", STREAM_CASES,
                         ids=["bf16out_bias", "f32out_f32bias", "noscale_nobias", "blk256", "k384_n136",
                              "rows_over_64"])
def test_weight_streaming_kernel(tokens, K, N, out_dtype, bias, scaled):
    """bf16 x e4m3 with few rows per group and K >= 384 runs the weight-streaming
    kernel: every element against the oracle, with empty groups, a group
    offset, N tails (N not a multiple of the 256-column tile, down to 8
    columns past one), the fewest K stages the kernel takes (three,
    K = 384), groups of more than one 64-row tile, rows outside the active
    groups, f32 and bf16 outputs and biases, and no scale.  Scale blocks of
    two K stages run on the general kernel, against the same oracle."""
    import moe_grouped_matrix_amd as m
    m.set_tile_policy(0)
    case = workloads.decode_fp8_weight(tokens=tokens, experts=24, K=K, N=N, forced_empty=8,
                                       group_offset=4, num_active=14, device="cuda")
    if bias is None:
        case.rhs_bias = None
    elif bias == "f32":
        case.rhs_bias = case.rhs_bias.float().contiguous()
    if scaled is False:
        case.rhs_scale = None
    elif scaled == "blk256":
        # per-256-K blocks: pairs of 128-K block scales merged (any positive values)
        case.rhs_scale = case.rhs_scale[:, ::2].contiguous() * 1.5
    case.out_dtype = out_dtype
    print(f"stream case tokens={tokens} K={K} N={N} out={out_dtype} bias={bias} scaled={scaled} M={case.M} "
          f"Ga={case.num_active} active_rows={case.active_rows()}", flush=True)
    out = run_gpu(case)
    lo, hi = active_range(case)
    assert_zero_rows(out, lo, hi)
    ref = reference(case)
    compare(out.cpu()[lo:hi], ref[lo:hi], out_dtype, f"stream K={K} N={N}")
    assert m.device_flags() == 0


def _fake(shape, dtype, addr=1 << 20):
    """A tensor view that is never dereferenced: the host rejects the call
    before anything is queued."""
    import moe_grouped_matrix_amd._binding as b
    v = b.GmmTensor()
    v.data = addr
    v.dtype = dtype
    v.ndim = len(shape)
    for i, s in enumerate(shape):
        v.shape[i] = s
    return v


def test_output_tile_beyond_32bit_offsets_is_unsupported():
    """The epilogues address a 256-row output tile (tgmm: up to 384 rows)
    with 32-bit byte offsets: gmm_run and gmm_tgmm_run reject an N whose
    output tile reaches 2 GiB (checked on the host; nothing is launched)."""
    import ctypes

    import moe_grouped_matrix_amd._binding as b
    lib, h = b.load(), b.handle(0)
    K = 64
    for out_dtype, N in ((b.GMM_F32, 2_097_152), (b.GMM_BF16, 4_194_304)):
        lhs, rhs = _fake((1, K), b.GMM_BF16), _fake((1, N, K), b.GMM_BF16)
        gs, out = _fake((1,), b.GMM_I32), _fake((1, N), out_dtype)
        st = lib.gmm_run(h, ctypes.byref(lhs), ctypes.byref(rhs), ctypes.byref(gs), None, None, None, None, 0,
                         ctypes.byref(out), None)
        assert st == b.GMM_E_UNSUPPORTED and b"output tile" in lib.gmm_last_error(h), (out_dtype, N)
        tl, tr, tout = _fake((16, K), b.GMM_BF16), _fake((16, N), b.GMM_BF16), _fake((1, K, N), out_dtype)
        st = lib.gmm_tgmm_run(h, ctypes.byref(tl), ctypes.byref(tr), ctypes.byref(gs), None, ctypes.byref(tout),
                              None)
        assert st == b.GMM_E_UNSUPPORTED and b"output tile" in lib.gmm_last_error(h), (out_dtype, N)
    # tgmm's 384-row tiles: an f32 N that a 256-row tile would allow
    N = 1_500_000
    tl, tr, tout = _fake((16, K), b.GMM_BF16), _fake((16, N), b.GMM_BF16), _fake((1, K, N), b.GMM_F32)
    st = lib.gmm_tgmm_run(h, ctypes.byref(tl), ctypes.byref(tr), ctypes.byref(gs), None, ctypes.byref(tout), None)
    assert st == b.GMM_E_UNSUPPORTED and b"384-row output tile" in lib.gmm_last_error(h)
    # one column less than the limit passes the check (and then fails on the
    # overlap of the fake tensors, still before anything is queued)
    lhs, rhs = _fake((1, K), b.GMM_BF16), _fake((1, 4_194_296, K), b.GMM_BF16)
    gs, out = _fake((1,), b.GMM_I32), _fake((1, 4_194_296), b.GMM_BF16)
    st = lib.gmm_run(h, ctypes.byref(lhs), ctypes.byref(rhs), ctypes.byref(gs), None, None, None, None, 0,
                     ctypes.byref(out), None)
    assert st == b.GMM_E_INVALID and b"overlap" in lib.gmm_last_error(h)
