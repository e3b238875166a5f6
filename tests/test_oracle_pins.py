"""Pins for the CPU oracle (no GPU).

Each test ties the oracle to something other than itself: hand-worked
fixtures under tests/golden/, library routines (torch matmul in float64,
torch's float8 / bfloat16 conversions), exact rational arithmetic, and the
identities the grouped matmul must satisfy.  A dropped term, a wrong sign,
a transposed operand, a wrong group or block index in the oracle fails at
least one of them.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import worklist

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- decoders

def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                yield line


def test_e4m3_golden_values():
    n = 0
    for line in _golden_lines("e4m3fn_values.txt"):
        code, value = line.split()
        got = oracle.decode_e4m3fn(int(code, 16))
        if value == "nan":
            assert math.isnan(got)
        else:
            assert got == float(value) and math.copysign(1, got) == math.copysign(1, float(value))
        n += 1
    assert n == 12


def test_e4m3_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64)
    for c in range(256):
        got = oracle.decode_e4m3fn(c)
        if math.isnan(ref[c].item()):
            assert math.isnan(got), c
        else:
            assert got == ref[c].item(), c


def test_bf16_all_codes_match_torch():
    codes = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    ref = codes.view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.decode_bf16(c) for c in range(0, 65536, 7)])
    want = ref[::7]
    both_nan = np.isnan(got) & np.isnan(want)
    assert np.all((got == want) | both_nan)


def _exact_bf16(x: Fraction) -> Fraction:
    """Nearest bf16 to a rational, ties to even, by exhaustive neighbours."""
    if x == 0:
        return Fraction(0)
    sgn = -1 if x < 0 else 1
    a = abs(x)
    e = math.floor(math.log2(a))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    q = Fraction(2) ** (e - 7)
    lo = (a // q) * q
    hi = lo + q
    if a - lo < hi - a:
        r = lo
    elif hi - a < a - lo:
        r = hi
    else:
        r = lo if (lo / q) % 2 == 0 else hi
    return sgn * r


def test_bf16_rounding_single_step():
    rng = np.random.default_rng(5)
    xs = list(rng.normal(size=2000) * 10.0 ** rng.integers(-30, 30, size=2000))
    # doubles that would round twice through float32 onto a bf16 tie
    xs += [1 + 2 ** -8 + 2 ** -30, -(1 + 2 ** -8 + 2 ** -30), 3 * (1 + 2 ** -8 + 2 ** -29),
           2 ** -130 * (1 + 2 ** -9), 1 + 2 ** -8, 1 + 3 * 2 ** -8]
    for x in xs:
        bits = oracle.round_bf16_bits(float(x))
        got = Fraction(torch.tensor([bits], dtype=torch.int32).to(torch.int16)
                       .view(torch.bfloat16).to(torch.float64).item())
        assert got == _exact_bf16(Fraction(float(x))), x


def test_bf16_rounding_matches_torch_on_float32_inputs():
    x = torch.randn(100000, generator=torch.Generator().manual_seed(3)) * 1e3
    ref = x.to(torch.bfloat16)
    got = oracle.round_to(x.to(torch.float64).numpy(), torch.bfloat16)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


# ---------------------------------------------------------------- fixtures

def _parse_matrix(text):
    rows = [r.split() for r in text.split(";")]
    return [[float(v) for v in r] for r in rows]


def _parse_cases(name):
    cases, cur = [], None
    for line in _golden_lines(name):
        key, _, rest = line.partition(" ")
        if key == "case":
            cur = {"name": rest}
        elif key == "end":
            cases.append(cur)
            cur = None
        else:
            cur[key] = rest
    return cases


@pytest.mark.parametrize("case", _parse_cases("gmm_handworked.txt"), ids=lambda c: c["name"])
def test_handworked_gmm(case):
    sizes = torch.tensor([int(v) for v in case["group_sizes"].split()], dtype=torch.int32)
    lhs = torch.tensor(_parse_matrix(case["lhs"]), dtype=torch.float32)
    rhs = torch.tensor([_parse_matrix(g) for g in case["rhs"].split("|")], dtype=torch.float32)
    kw = dict(group_offset=int(case["group_offset"]), transpose_rhs=bool(int(case["transpose_rhs"])))
    if "rhs_scale" in case:
        sc = torch.tensor([[float(v) for v in g.split()] for g in case["rhs_scale"].split("|")])
        kw["rhs_scale"] = sc[:, :, None, None].contiguous()  # [Ga, nb, 1, N=1]
    if "rhs_bias" in case:
        b = torch.tensor([[float(v) for v in g.split()] for g in case["rhs_bias"].split("|")])
        kw["rhs_bias"] = b[:, None, :].contiguous()
    if "lhs_scale" in case:
        kw["lhs_scale"] = torch.tensor(_parse_matrix(case["lhs_scale"]), dtype=torch.float32)
    got = oracle.gmm_reference(lhs, rhs, sizes, **kw)
    want = np.array(_parse_matrix(case["expect"]))
    assert np.array_equal(got, want), (got, want)


@pytest.mark.parametrize("case", _parse_cases("megablox_metadata_handworked.txt"),
                         ids=lambda c: c["name"])
def test_handworked_megablox_metadata(case):
    ints = lambda k: [int(v) for v in case[k].split()]  # noqa: E731
    o, gids, mids, nt = worklist.megablox_metadata(
        ints("group_sizes"), int(case["m"]), int(case["tm"]), int(case["start_group"]),
        int(case["num_groups"]))
    assert o == ints("offsets")
    assert gids == ints("group_ids")
    assert mids == ints("m_tile_ids")
    assert nt == int(case["num_tiles"])


# ---------------------------------------------------------------- identities

def _rand_case(seed, M, K, N, sizes, dtype=torch.float32, Ga=None, s=0, T=False):
    g = torch.Generator().manual_seed(seed)
    G = len(sizes)
    Ga = G - s if Ga is None else Ga
    lhs = torch.randn(M, K, generator=g).to(dtype)
    rhs = torch.randn(Ga, K, N, generator=g) if T else torch.randn(Ga, N, K, generator=g)
    return lhs, rhs.to(dtype), torch.tensor(sizes, dtype=torch.int32)


def _torch_segments(lhs, rhs, sizes, s=0, T=False):
    """Per-segment dense products with torch in float64."""
    M = lhs.shape[0]
    Ga = rhs.shape[0]
    N = rhs.shape[2] if T else rhs.shape[1]
    out = torch.zeros(M, N, dtype=torch.float64)
    o = np.concatenate([[0], np.cumsum(sizes)])
    for h in range(Ga):
        g = s + h
        w = rhs[h].to(torch.float64)
        w = w if T else w.t()
        out[o[g]:o[g + 1]] = lhs[o[g]:o[g + 1]].to(torch.float64) @ w
    return out.numpy()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_single_group_is_dense_matmul(dtype):
    lhs, rhs, sizes = _rand_case(1, 37, 48, 20, [37], dtype)
    got = oracle.gmm_reference(lhs, rhs, sizes)
    want = (lhs.to(torch.float64) @ rhs[0].to(torch.float64).t()).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_single_group_e4m3_is_dense_matmul():
    g = torch.Generator().manual_seed(2)
    lhs = (torch.randn(16, 64, generator=g) * 4).to(torch.float8_e4m3fn)
    rhs = (torch.randn(1, 24, 64, generator=g) * 4).to(torch.float8_e4m3fn)
    got = oracle.gmm_reference(lhs, rhs, torch.tensor([16], dtype=torch.int32))
    want = (lhs.to(torch.float64) @ rhs[0].to(torch.float64).t()).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("T", [False, True])
def test_segments_match_torch(T):
    sizes = [5, 0, 17, 1, 0, 0, 9, 3]
    M = sum(sizes) + 6
    lhs, rhs, gs = _rand_case(3, M, 32, 24, sizes, T=T)
    got = oracle.gmm_reference(lhs, rhs, gs, transpose_rhs=T)
    np.testing.assert_allclose(got, _torch_segments(lhs, rhs, sizes, T=T), rtol=1e-12, atol=1e-12)
    assert np.all(got[sum(sizes):] == 0)


def test_transpose_identity_bit_exact():
    sizes = [4, 7, 0, 5]
    lhs, rhs, gs = _rand_case(4, 20, 40, 12, sizes)
    nt = oracle.gmm_reference(lhs, rhs, gs, transpose_rhs=False)
    nn = oracle.gmm_reference(lhs, rhs.transpose(1, 2).contiguous(), gs, transpose_rhs=True)
    assert np.array_equal(nt, nn)


def test_empty_groups_emit_nothing():
    base = [3, 6, 2]
    lhs, rhs, gs = _rand_case(5, 11, 16, 8, base)
    ref = oracle.gmm_reference(lhs, rhs, gs)
    g = torch.Generator().manual_seed(9)
    for pos in [(0,), (1,), (3,), (1, 1), (0, 2, 3)]:
        sizes = list(base)
        ws = list(rhs)
        for p in sorted(pos, reverse=True):
            sizes.insert(p, 0)
            ws.insert(p, torch.randn(8, 16, generator=g) * 100)
        got = oracle.gmm_reference(lhs, torch.stack(ws), torch.tensor(sizes, dtype=torch.int32))
        assert np.array_equal(got, ref), pos


def test_group_offset_shard_identity():
    sizes = [3, 0, 8, 2, 5, 0, 4]
    M = sum(sizes) + 3
    lhs, rhs, gs = _rand_case(6, M, 24, 16, sizes)
    full = oracle.gmm_reference(lhs, rhs, gs)
    o = np.concatenate([[0], np.cumsum(sizes)])
    for s in range(len(sizes)):
        for ga in range(0, len(sizes) - s + 1):
            got = oracle.gmm_reference(lhs, rhs[s:s + ga].contiguous() if ga else rhs[:0],
                                       gs, group_offset=s)
            lo, hi = o[s], o[s + ga]
            assert np.array_equal(got[lo:hi], full[lo:hi])
            assert np.all(got[:lo] == 0) and np.all(got[hi:] == 0)


def test_bias_probe_maps_rows_to_groups():
    sizes = [2, 0, 5, 1, 0, 3]
    M = sum(sizes) + 2
    lhs, _, gs = _rand_case(7, M, 16, 8, sizes)
    rhs = torch.zeros(len(sizes), 8, 16)
    bias = (torch.arange(len(sizes), dtype=torch.float32) + 1)[:, None, None].expand(-1, 1, 8)
    got, rg = oracle.gmm_reference(lhs, rhs, gs, rhs_bias=bias.contiguous(), return_row_group=True)
    row_group = np.repeat(np.arange(len(sizes)), sizes)
    assert np.array_equal(rg[:sum(sizes)], row_group) and np.all(rg[sum(sizes):] == -1)
    assert np.array_equal(got[:sum(sizes)], np.repeat((row_group + 1)[:, None], 8, axis=1))
    assert np.all(got[sum(sizes):] == 0)


def _torch_blocks(lhs, rhs, sizes, rs=None, ls=None, bias=None, nb=1):
    """Per-segment, per-block products with torch float64 matmuls."""
    M, K = lhs.shape
    N = rhs.shape[1]
    blk = K // nb
    out = torch.zeros(M, N, dtype=torch.float64)
    o = np.concatenate([[0], np.cumsum(sizes)])
    L = lhs.to(torch.float64)
    for g in range(len(sizes)):
        a, b = o[g], o[g + 1]
        if a == b:
            continue
        acc = torch.zeros(b - a, N, dtype=torch.float64)
        for j in range(nb):
            part = L[a:b, j * blk:(j + 1) * blk] @ rhs[g, :, j * blk:(j + 1) * blk].to(torch.float64).t()
            if rs is not None:
                part = part * rs[g, j, 0, :].to(torch.float64)[None, :]
            if ls is not None:
                part = part * ls[a:b, j].to(torch.float64)[:, None]
            acc += part
        if bias is not None:
            acc += bias[g, 0, :].to(torch.float64)[None, :]
        out[a:b] = acc
    return out.numpy()


def test_block_scales_and_bias_match_blockwise_torch():
    sizes = [6, 0, 9, 4]
    M, K, N, nb = 21, 64, 12, 4
    g = torch.Generator().manual_seed(8)
    lhs = torch.randn(M, K, generator=g)
    rhs = torch.randn(4, N, K, generator=g)
    rs = torch.rand(4, nb, 1, N, generator=g) + 0.5
    ls = torch.rand(M, nb, generator=g) + 0.25
    bias = torch.randn(4, 1, N, generator=g)
    gs = torch.tensor(sizes, dtype=torch.int32)
    got = oracle.gmm_reference(lhs, rhs, gs, rhs_scale=rs, lhs_scale=ls, rhs_bias=bias)
    want = _torch_blocks(lhs, rhs, sizes, rs, ls, bias, nb)
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-11)
    # the scales really are per block: a one-hot block scale picks one K slice
    for j in range(nb):
        one_hot = torch.zeros(4, nb, 1, N)
        one_hot[:, j] = 1
        got = oracle.gmm_reference(lhs, rhs, gs, rhs_scale=one_hot)
        sl = slice(j * K // nb, (j + 1) * K // nb)
        want = _torch_segments(lhs[:, sl].contiguous(), rhs[:, :, sl].contiguous(), sizes)
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_unit_and_power_of_two_scales_are_exact():
    sizes = [5, 3]
    lhs, rhs, gs = _rand_case(10, 8, 32, 8, sizes)
    plain = oracle.gmm_reference(lhs, rhs, gs)
    ones = oracle.gmm_reference(lhs, rhs, gs, rhs_scale=torch.ones(2, 2, 1, 8))
    # with two blocks the sums split differently; equal to the last ulp only
    np.testing.assert_allclose(ones, plain, rtol=1e-13, atol=1e-13)
    one_block = oracle.gmm_reference(lhs, rhs, gs, rhs_scale=torch.ones(2, 1, 1, 8))
    assert np.array_equal(one_block, plain)
    four = oracle.gmm_reference(lhs, rhs, gs, rhs_scale=torch.full((2, 1, 1, 8), 4.0))
    assert np.array_equal(four, 4 * plain)


def test_brute_force_all_compositions():
    """Every composition of M=6 rows into G=3 groups (zeros allowed), plus an
    unassigned tail, against per-segment torch products."""
    K, N = 8, 5
    for total in (6, 4):
        for sizes in itertools.product(range(total + 1), repeat=3):
            if sum(sizes) != total:
                continue
            lhs, rhs, gs = _rand_case(sum(sizes) * 7 + 1, 6, K, N, list(sizes))
            got = oracle.gmm_reference(lhs, rhs, gs)
            np.testing.assert_allclose(got, _torch_segments(lhs, rhs, list(sizes)), rtol=1e-12,
                                       atol=1e-12)


def test_invalid_device_data_is_rejected():
    lhs, rhs, _ = _rand_case(11, 6, 8, 4, [3, 3])
    with pytest.raises(oracle.OracleError):
        oracle.gmm_reference(lhs, rhs, torch.tensor([4, -1], dtype=torch.int32))
    with pytest.raises(oracle.OracleError):
        oracle.gmm_reference(lhs, rhs, torch.tensor([4, 3], dtype=torch.int32))
    with pytest.raises(oracle.OracleError):
        oracle.gmm_reference(lhs, rhs, torch.tensor([3, 3], dtype=torch.int32), group_offset=1)


def test_row_sampling_matches_full():
    sizes = [4, 0, 9, 2]
    lhs, rhs, gs = _rand_case(12, 17, 16, 8, sizes)
    full = oracle.gmm_reference(lhs, rhs, gs)
    rows = [16, 0, 5, 5, 14, 3]
    assert np.array_equal(oracle.gmm_reference(lhs, rhs, gs, rows=rows), full[rows])


# ---------------------------------------------------------------- tile metadata

def _covered_rows_megablox(sizes, m, tm, s, ga):
    o, gids, mids, nt = worklist.megablox_metadata(sizes, m, tm, s, ga)
    cover = {}
    for i in range(nt):
        g, t = gids[i], mids[i]
        for r in range(t * tm, (t + 1) * tm):
            if o[g] <= r < o[g + 1]:  # the store mask of the Megablox kernel
                assert r not in cover
                cover[r] = g
    return cover


def _covered_rows_aligned(sizes, tm, s, ga):
    cover = {}
    for g, r0, n in worklist.tile_worklist(sizes, s, ga, tm):
        for r in range(r0, r0 + n):
            assert r not in cover
            cover[r] = g
    return cover


def test_megablox_invariants_and_aligned_tiles_agree():
    rng = np.random.default_rng(13)
    for trial in range(300):
        G = int(rng.integers(1, 9))
        tm = int(rng.choice([1, 2, 4, 8, 16]))
        tiles_m = int(rng.integers(1, 6))
        m = tm * tiles_m
        cuts = np.sort(rng.integers(0, m + 1, size=G - 1))
        sizes = np.diff(np.concatenate([[0], cuts, [m]])).astype(int).tolist()
        o, gids, mids, nt = worklist.megablox_metadata(sizes, m, tm, 0, G)
        assert o[0] == 0 and o[G] == m
        assert tiles_m <= nt <= tiles_m + G - 1
        assert all(a <= b for a, b in zip(mids[:nt], mids[1:nt]))
        s = int(rng.integers(0, G))
        ga = int(rng.integers(0, G - s + 1))
        mb = _covered_rows_megablox(sizes, m, tm, s, ga) if ga else {}
        al = _covered_rows_aligned(sizes, tm, s, ga)
        assert mb == al
        assert set(al) == set(range(o[s], o[s + ga]))
        want_tiles = sum(-(-sizes[g] // tm) for g in range(s, s + ga))
        assert len(worklist.tile_worklist(sizes, s, ga, tm)) == want_tiles
