"""Pins for the oracle's activation quantiser (per_token_group_quant_fp8 of
the metrale gemm_quant.rs page: bf16 [M,K] -> e4m3fn [M,K] and an f32 scale
per 128-element block of each row), CPU only.

The e4m3fn rounding is tied to the format itself: every finite code round
trips; every rounded value is the nearest finite e4m3fn value by brute force
over all 256 codes, ties to the even mantissa; and it agrees with torch's
float8_e4m3fn conversion on in-range values (a library routine).  The block
arithmetic is tied to an independent numpy-float32 evaluation of the
definition with a brute-force nearest-code search; the largest element of
every block lands on +-448; an all-zero block has scale 1; the dequantised
values lie within half an e4m3 step of the inputs.  The last tests plant
plausible mistakes (the 240 maximum of the other e4m3 variant, truncation
instead of rounding, one scale per row instead of per block) and check that
the pins reject them."""
import numpy as np
import pytest
import torch

import oracle

FINITE = [c for c in range(256) if c & 0x7F != 0x7F]
VALUES = np.array([oracle.decode_e4m3fn(c) for c in FINITE])


def _nearest_code(v: float) -> int:
    """Brute force: the finite code whose value is nearest to v; on a tie the
    one with an even mantissa; the sign of v decides between +0 and -0."""
    d = np.abs(VALUES - v)
    best = np.flatnonzero(d == d.min())
    cands = [FINITE[i] for i in best]
    if len(cands) > 1:
        cands = [c for c in cands if c & 1 == 0] or cands
    if VALUES[FINITE.index(cands[0])] == 0.0:
        return 0x80 if np.signbit(v) else 0x00
    return cands[0]


def test_every_finite_code_round_trips():
    for c in FINITE:
        assert oracle.round_e4m3fn_code(oracle.decode_e4m3fn(c)) == c, hex(c)


def test_rounding_is_nearest_with_ties_to_even():
    rng = np.random.default_rng(1)
    pos = np.sort(np.unique(VALUES[VALUES >= 0]))
    mids = (pos[1:] + pos[:-1]) / 2  # exact ties
    vals = np.concatenate([rng.uniform(-448, 448, 3000), rng.uniform(-0.02, 0.02, 2000),
                           mids, -mids, mids * (1 + 1e-9), mids * (1 - 1e-9), [0.0, -0.0, 448.0, -448.0]])
    for v in vals:
        assert oracle.round_e4m3fn_code(float(v)) == _nearest_code(float(v)), v


def test_rounding_matches_torch_float8_in_range():
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.uniform(-448, 448, 5000), rng.normal(0, 0.05, 5000)]).astype(np.float32)
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.round_e4m3fn_code(float(x)) for x in v], dtype=np.uint8)
    assert np.array_equal(got, want)


def _numpy_quant(x: torch.Tensor, blk: int):
    """The definition in numpy float32, with the brute-force nearest code."""
    xf = x.float().numpy()
    M, K = xf.shape
    q = np.zeros((M, K), dtype=np.uint8)
    sc = np.zeros((M, K // blk), dtype=np.float32)
    for r in range(M):
        for b in range(K // blk):
            blkv = xf[r, b * blk:(b + 1) * blk]
            amax = np.float32(np.abs(blkv).max())
            s = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
            sc[r, b] = s
            t = np.clip(blkv / s, np.float32(-448), np.float32(448))
            q[r, b * blk:(b + 1) * blk] = [_nearest_code(float(v)) for v in t]
    return q, sc


def _input(seed, M, K, sigma=0.02):
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn(M, K, generator=g) * sigma).to(torch.bfloat16)
    x[1, :64] = 0.0                      # an all-zero block when blk <= 64
    x[2, 5] = -0.0
    x[3, 7] = torch.tensor(3.0e-38)      # tiny values next to large ones
    return x


@pytest.mark.parametrize("blk", [32, 64])
def test_blocks_follow_the_definition_bit_for_bit(blk):
    x = _input(3, 5, 128)
    q, s = oracle.quant_fp8_reference(x, blk)
    wq, ws = _numpy_quant(x, blk)
    assert np.array_equal(q.view(torch.uint8).numpy(), wq)
    assert np.array_equal(s.numpy().view(np.uint32), ws.view(np.uint32))


def test_largest_element_of_every_block_lands_on_448():
    x = _input(4, 16, 512)
    q, s = oracle.quant_fp8_reference(x, 128)
    xb = x.float().view(16, 4, 128)
    qb = q.view(torch.uint8).view(16, 4, 128)
    for r in range(16):
        for b in range(4):
            i = int(xb[r, b].abs().argmax())
            if xb[r, b, i] != 0:
                assert int(qb[r, b, i]) in (0x7E, 0xFE)
                assert s[r, b] == np.float32(np.float32(xb[r, b, i].abs()) / np.float32(448))


def test_all_zero_block_has_scale_one_and_zero_codes():
    x = torch.zeros(2, 256, dtype=torch.bfloat16)
    x[1, 128:] = 1.0
    q, s = oracle.quant_fp8_reference(x, 128)
    assert s[0, 0] == 1.0 and s[0, 1] == 1.0 and s[1, 0] == 1.0
    assert torch.all(q.view(torch.uint8)[0] == 0) and torch.all(q.view(torch.uint8)[1, :128] == 0)


def test_dequantised_values_within_half_a_step():
    x = _input(5, 32, 384, sigma=1.0)
    q, s = oracle.quant_fp8_reference(x, 128)
    deq = q.float().view(32, 3, 128) * s[:, :, None]
    err = (deq - x.float().view(32, 3, 128)).abs()
    # half a step: 2^-4 of the value in the normal range, 2^-10 * scale below
    # 2^-6 * scale (the subnormal spacing 2^-9 halved); slack for the
    # binary32 division before rounding
    bound = torch.maximum(x.float().view(32, 3, 128).abs() * 2.0 ** -4, s[:, :, None] * 2.0 ** -10)
    assert torch.all(err <= bound * (1 + 1e-6))


# ------------------------------------------------------ planted mistakes

def test_planted_wrong_format_maximum_is_caught():
    x = _input(6, 4, 128)
    q, s = oracle.quant_fp8_reference(x, 128)
    amax = x.float().abs().amax(dim=1)
    mutant_scale = amax / 240.0  # the largest value of the other (fnuz) e4m3 variant
    assert not torch.equal(mutant_scale, s[:, 0])
    # with that scale the largest element would code 240, not 448
    assert oracle.round_e4m3fn_code(240.0) not in (0x7E, 0xFE)


def test_planted_truncation_is_caught():
    # between 256 and 512 the e4m3 step is 32: 310 lies between 288 and 320,
    # nearer 320; truncation toward zero would give 288
    truncated = oracle.round_e4m3fn_code(288.0)
    assert oracle.round_e4m3fn_code(310.0) == oracle.round_e4m3fn_code(320.0) != truncated
    assert _nearest_code(310.0) != truncated  # the brute-force pin rejects the truncated code


def test_planted_one_scale_per_row_is_caught():
    x = _input(7, 4, 256)
    x[:, 128:] *= 50  # the second block's amax dominates the row
    q, s = oracle.quant_fp8_reference(x, 128)
    row_q, row_s = oracle.quant_fp8_reference(x, 256)
    assert not torch.equal(row_q.view(torch.uint8), q.view(torch.uint8))
    # the per-block pin sees it: the first block's largest element is not 448
    first = row_q.view(torch.uint8)[:, :128]
    i = x[:, :128].float().abs().argmax(dim=1)
    assert not all(int(first[r, i[r]]) in (0x7E, 0xFE) for r in range(4))


def test_oracle_agrees_with_the_input_generators_quantiser():
    """The workloads module quantises the W8A8 test inputs with torch by the
    same reading; the two must give the same codes and scales."""
    import workloads
    x = _input(8, 8, 384, sigma=0.3)
    q, s = oracle.quant_fp8_reference(x, 128)
    wq, ws = workloads.quantize_e4m3_blocks(x.float(), 128)
    assert torch.equal(q.view(torch.uint8), wq.view(torch.uint8).reshape(q.shape))
    assert torch.equal(s, ws.reshape(s.shape))
