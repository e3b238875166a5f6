"""Pins for the oracle's e5m2 operands (float8_e5m2 is one of the dtypes the
Megablox gmm accepts, assert_is_supported_dtype on the tpu-inference wheel
diff page), CPU only.

The decoder is tied to the OCP 8-bit floating point definition (values
computed here from the fields: 1.0, the largest finite value 57344, the
smallest normal and subnormal, infinities, NaN) and to torch's float8_e5m2
conversion on all 256 codes (a library routine).  gmm with e5m2 on either
side is tied to torch float64 matmuls of the decoded operands.  The last test
plants a plausible mistake (e5m2 bytes read as e4m3fn) and checks that the
pins reject it."""
import math

import numpy as np
import pytest
import torch

import oracle


def _closed_form(code: int) -> float:
    s, e, m = code >> 7, (code >> 2) & 31, code & 3
    if e == 31:
        return math.nan if m else (-math.inf if s else math.inf)
    v = (m / 4.0) * 2.0 ** -14 if e == 0 else (1 + m / 4.0) * 2.0 ** (e - 15)
    return -v if s else v


def test_e5m2_named_values():
    assert oracle.decode_e5m2(0x3C) == 1.0
    assert oracle.decode_e5m2(0x7B) == 57344.0          # largest finite
    assert oracle.decode_e5m2(0x04) == 2.0 ** -14       # smallest normal
    assert oracle.decode_e5m2(0x01) == 2.0 ** -16       # smallest subnormal
    assert oracle.decode_e5m2(0x7C) == math.inf and oracle.decode_e5m2(0xFC) == -math.inf
    assert math.isnan(oracle.decode_e5m2(0x7D)) and math.isnan(oracle.decode_e5m2(0xFF))
    assert math.copysign(1.0, oracle.decode_e5m2(0x80)) == -1.0 and oracle.decode_e5m2(0x80) == 0.0


def test_e5m2_all_codes_match_closed_form_and_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).to(torch.float64)
    for c in range(256):
        got, cf, tv = oracle.decode_e5m2(c), _closed_form(c), ref[c].item()
        if math.isnan(cf):
            assert math.isnan(got) and math.isnan(tv), c
        else:
            assert got == cf == tv, c


def _case(ld, rd, seed):
    g = torch.Generator().manual_seed(seed)
    lhs = (torch.randn(40, 256, generator=g) * 4).to(ld)
    rhs = (torch.randn(1, 24, 256, generator=g) * 4).to(rd)
    return lhs, rhs


@pytest.mark.parametrize("ld,rd", [(torch.float8_e5m2, torch.float8_e5m2),
                                   (torch.float8_e4m3fn, torch.float8_e5m2),
                                   (torch.float8_e5m2, torch.float8_e4m3fn),
                                   (torch.bfloat16, torch.float8_e5m2)])
def test_gmm_with_e5m2_is_the_dense_product(ld, rd):
    lhs, rhs = _case(ld, rd, 3)
    got = oracle.gmm_reference(lhs, rhs, torch.tensor([40], dtype=torch.int32))
    want = (lhs.to(torch.float64) @ rhs[0].to(torch.float64).t()).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_planted_e5m2_read_as_e4m3_is_caught():
    lhs, rhs = _case(torch.float8_e5m2, torch.float8_e5m2, 4)
    want = (lhs.to(torch.float64) @ rhs[0].to(torch.float64).t()).numpy()
    gs = torch.tensor([40], dtype=torch.int32)
    assert np.allclose(oracle.gmm_reference(lhs, rhs, gs), want, rtol=1e-12, atol=1e-12)
    mutant = oracle.gmm_reference(lhs.view(torch.uint8).view(torch.float8_e4m3fn),
                                  rhs.view(torch.uint8).view(torch.float8_e4m3fn), gs)
    assert not np.allclose(np.nan_to_num(mutant), want, rtol=1e-6, atol=1e-6)
