"""Pins for the oracle's block-scale widening (widen_block_scale_f32 of the
metrale gemm_quant.rs page: bf16, f32 or E8M0 scales to f32), CPU only.

The E8M0 rule is tied to what the page states: the bit pattern e << 23,
2^-127 for e = 0 and 0.0 for e = 255 (tests/golden/e8m0_widen_values.txt
holds those cases), checked for every byte; bf16 widening is tied to
torch's bf16 -> f32 conversion over all 65536 codes; f32 is passed through
bit for bit.  The last tests plant plausible mistakes (255 as the OCP NaN,
e = 0 flushed to zero, the exponent bias off by one) and check that the
pins reject them."""
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e8m0_widen_values.txt")


def _golden():
    rows = []
    with open(GOLDEN) as fh:
        for ln in fh:
            ln = ln.strip()
            if ln and not ln.startswith("#"):
                e, bits = ln.split()
                rows.append((int(e), int(bits, 16)))
    return rows


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int32).numpy().view(np.uint32)


def test_e8m0_cases_stated_on_the_page():
    rows = _golden()
    got = oracle.widen_scales_reference(torch.tensor([e for e, _ in rows], dtype=torch.uint8),
                                        oracle.SCALE_E8M0)
    assert list(_bits(got)) == [b for _, b in rows]


def test_e8m0_every_byte_is_its_bit_pattern():
    e = torch.arange(256, dtype=torch.uint8)
    got = _bits(oracle.widen_scales_reference(e, oracle.SCALE_E8M0))
    for v in range(1, 255):
        assert got[v] == v << 23, v
    assert got[0] == 0x00400000 and got[255] == 0


def test_bf16_scales_widen_exactly():
    """Every bf16 code (NaN codes compare as NaN: their payload is not a
    scale)."""
    codes = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    got = oracle.widen_scales_reference(codes, oracle.SCALE_BF16)
    want = codes.to(torch.float32)
    nan = torch.isnan(want)
    assert torch.equal(torch.isnan(got), nan)
    assert np.array_equal(_bits(got)[~nan.numpy()], _bits(want)[~nan.numpy()])


def test_f32_scales_pass_through_bit_for_bit():
    g = torch.Generator().manual_seed(1)
    x = torch.randn(4096, generator=g)
    x[:4] = torch.tensor([0.0, -0.0, float("inf"), 1e-40])
    got = oracle.widen_scales_reference(x, oracle.SCALE_F32)
    assert np.array_equal(_bits(got), _bits(x))


def test_planted_mistakes_are_caught():
    rows = dict(_golden())
    # 255 read as the OCP NaN, e = 0 flushed to zero, and a bias of 128
    nan_bits = int(np.float32(np.nan).view(np.uint32))
    assert rows[255] != nan_bits
    assert rows[0] != 0
    assert rows[128] != (128 - 1) << 23 and rows[128] == 128 << 23


def test_gmm_with_e8m0_block_scales_equals_the_powers_of_two():
    """gmm's block scales may come as E8M0 bytes (microscaling): the oracle
    multiplies by 2^(e-127), the same products as f32 scales built here
    with ldexp; byte 255 (NaN in that encoding) is rejected."""
    import numpy as np
    import torch

    import oracle
    g = torch.Generator().manual_seed(9)
    sizes = [6, 0, 9]
    M, N, K, nb = sum(sizes) + 2, 12, 128, 4
    lhs = torch.randint(-3, 4, (M, K), generator=g).to(torch.float8_e4m3fn)
    rhs = torch.randint(-3, 4, (len(sizes), N, K), generator=g).to(torch.float8_e4m3fn)
    er = torch.randint(1, 255, (len(sizes), nb, 1, N), generator=g).to(torch.uint8)
    el = torch.randint(1, 255, (M, nb), generator=g).to(torch.uint8)
    gs = torch.tensor(sizes, dtype=torch.int32)
    got = oracle.gmm_reference(lhs, rhs, gs, rhs_scale=er.view(torch.float8_e8m0fnu),
                               lhs_scale=el.view(torch.float8_e8m0fnu))
    f = lambda e: torch.from_numpy(np.ldexp(1.0, e.numpy().astype(np.int64) - 127)).to(torch.float32)  # noqa: E731
    want = oracle.gmm_reference(lhs, rhs, gs, rhs_scale=f(er), lhs_scale=f(el))
    assert np.array_equal(got, want)
    er[0, 0, 0, 0] = 255
    with pytest.raises(oracle.OracleError):
        oracle.gmm_reference(lhs, rhs, gs, rhs_scale=er.view(torch.float8_e8m0fnu))
