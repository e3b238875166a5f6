"""Pins for the oracle's four-bit weights (int4, uint4 and fp4 e2m1 are on
the Megablox gmm's dtype list, assert_is_supported_dtype on the
tpu-inference wheel diff page), CPU only.

e2m1 is tied to the OCP microscaling formats definition (the eight
magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 with a sign bit); int4 and uint4 to
two's complement and plain binary.  The packing (element i in the low nibble
of byte i/2 when i is even) is tied to a one-hot product that reads the
weights back in order, and gmm with packed weights to torch float64 products
of weights unpacked here with numpy bit operations.  The last test plants a
mistake (the two nibbles of a byte swapped) and checks that the pins reject
it."""
import numpy as np
import pytest
import torch

import oracle

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _unpack(packed: torch.Tensor, fmt: str) -> torch.Tensor:
    b = packed.view(torch.uint8).numpy().astype(np.int64)
    nib = np.stack([b & 15, b >> 4], axis=-1).reshape(*b.shape[:-1], 2 * b.shape[-1])
    if fmt == "int4":
        v = np.where(nib >= 8, nib - 16, nib).astype(np.float64)
    elif fmt == "uint4":
        v = nib.astype(np.float64)
    else:
        mag = np.array(E2M1)[nib & 7]
        v = np.where(nib >= 8, -mag, mag)
    return torch.from_numpy(v)


def test_e2m1_values_follow_the_definition():
    for n in range(16):
        want = E2M1[n & 7] * (-1 if n & 8 else 1)
        assert oracle.decode_e2m1(n) == want, n
    assert np.signbit(oracle.decode_e2m1(8))


@pytest.mark.parametrize("fmt", ["int4", "uint4", "fp4_e2m1"])
def test_one_hot_rows_read_the_packed_weights_in_order(fmt):
    g = torch.Generator().manual_seed(1)
    N, K = 6, 32
    packed = torch.randint(0, 256, (1, N, K // 2), generator=g).to(torch.uint8)
    lhs = torch.eye(K)  # row k picks weight column k
    got = oracle.gmm_reference(lhs, packed, torch.tensor([K], dtype=torch.int32), rhs_format=fmt)
    want = _unpack(packed, fmt)[0].t().numpy()  # [K, N]
    assert np.array_equal(got, want)
    # and the low nibble of byte 0 is element 0
    b0 = int(packed[0, 0, 0])
    lo = b0 & 15
    want0 = {"int4": lo - 16 if lo >= 8 else lo, "uint4": lo,
             "fp4_e2m1": oracle.decode_e2m1(lo)}[fmt]
    assert got[0, 0] == want0


@pytest.mark.parametrize("fmt", ["int4", "uint4", "fp4_e2m1"])
def test_packed_weights_equal_the_float64_product(fmt):
    g = torch.Generator().manual_seed(2)
    sizes = [9, 0, 14, 5]
    M, N, K = sum(sizes) + 3, 20, 128
    lhs = torch.randn(M, K, generator=g).to(torch.bfloat16)
    packed = torch.randint(0, 256, (len(sizes), N, K // 2), generator=g).to(torch.uint8)
    got = oracle.gmm_reference(lhs, packed, torch.tensor(sizes, dtype=torch.int32), rhs_format=fmt)
    w = _unpack(packed, fmt)
    o = np.concatenate([[0], np.cumsum(sizes)]).astype(int)
    want = np.zeros((M, N))
    for h in range(len(sizes)):
        want[o[h]:o[h + 1]] = (lhs[o[h]:o[h + 1]].double() @ w[h].t()).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_float4_tensor_is_accepted_as_packed_bytes():
    g = torch.Generator().manual_seed(3)
    packed = torch.randint(0, 256, (1, 4, 16), generator=g).to(torch.uint8)
    lhs = torch.randn(5, 32, generator=g)
    a = oracle.gmm_reference(lhs, packed, torch.tensor([5], dtype=torch.int32), rhs_format="fp4_e2m1")
    b = oracle.gmm_reference(lhs, packed.view(torch.float4_e2m1fn_x2), torch.tensor([5], dtype=torch.int32),
                             rhs_format="fp4_e2m1")
    assert np.array_equal(a, b)


def test_planted_swapped_nibbles_are_caught():
    g = torch.Generator().manual_seed(4)
    packed = torch.randint(0, 256, (1, 3, 8), generator=g).to(torch.uint8)
    lhs = torch.eye(16)
    good = oracle.gmm_reference(lhs, packed, torch.tensor([16], dtype=torch.int32), rhs_format="uint4")
    swapped = ((packed >> 4) | (packed << 4)).to(torch.uint8)
    mutant = oracle.gmm_reference(lhs, swapped, torch.tensor([16], dtype=torch.int32), rhs_format="uint4")
    want = _unpack(packed, "uint4")[0].t().numpy()
    assert np.array_equal(good, want) and not np.array_equal(mutant, want)
