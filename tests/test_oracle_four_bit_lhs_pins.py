"""Pins for the oracle's four-bit activations, CPU only.

The Megablox gmm's dtype list (assert_is_supported_dtype on the
tpu-inference wheel diff page) holds for lhs as well as rhs (_validate_args
checks both), so int4, uint4 and fp4 e2m1 activations are part of the
operation.  They use the packing of the four-bit weights: two elements to a
byte, element i in the low nibble of byte i/2 when i is even.

Pinned here, each against something other than the oracle: a one-hot weight
that reads every packed activation back in order (against numpy bit
operations); the full table of fp4 e2m1 x e2m1 products (against the OCP
microscaling magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 with a sign, multiplied
here); int4 / uint4 x int8 and x int4 against torch's int64 matmul, bit for
bit; fp4 x e4m3 and fp4 x fp4 with block scales against torch float64
products of operands unpacked here; and two planted mistakes (nibbles of a
byte swapped, int4 read as unsigned) that the pins reject."""
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


def _segments(sizes):
    return np.concatenate([[0], np.cumsum(sizes)]).astype(int)


@pytest.mark.parametrize("fmt", ["int4", "uint4", "fp4_e2m1"])
def test_one_hot_weights_read_the_packed_activations_in_order(fmt):
    g = torch.Generator().manual_seed(1)
    M, K = 7, 64
    packed = torch.randint(0, 256, (M, K // 2), generator=g).to(torch.uint8)
    eye = torch.eye(K).to(torch.bfloat16)[None]  # weight [1, N=K, K]: column n picks element n
    got = oracle.gmm_reference(packed, eye, torch.tensor([M], dtype=torch.int32), lhs_format=fmt)
    assert np.array_equal(got, _unpack(packed, fmt).numpy())
    lo = int(packed[0, 0]) & 15
    want0 = {"int4": lo - 16 if lo >= 8 else lo, "uint4": lo, "fp4_e2m1": oracle.decode_e2m1(lo)}[fmt]
    assert got[0, 0] == want0


def test_fp4_times_fp4_product_table():
    """Row a holds code a at element 0 (zeros elsewhere), weight column b
    code b at element 0: out[a, b] is the product of the two e2m1 values."""
    K = 32
    lhs = torch.zeros(16, K // 2, dtype=torch.uint8)
    rhs = torch.zeros(1, 16, K // 2, dtype=torch.uint8)
    lhs[:, 0] = torch.arange(16, dtype=torch.uint8)
    rhs[0, :, 0] = torch.arange(16, dtype=torch.uint8)
    got = oracle.gmm_reference(lhs, rhs, torch.tensor([16], dtype=torch.int32), lhs_format="fp4_e2m1",
                               rhs_format="fp4_e2m1")
    val = [E2M1[c & 7] * (-1.0 if c & 8 else 1.0) for c in range(16)]
    want = np.array([[val[a] * val[b] for b in range(16)] for a in range(16)])
    assert np.array_equal(got, want)
    assert got[1, 7] == 3.0 and got[15, 15] == 36.0 and got[9, 6] == -2.0


@pytest.mark.parametrize("lfmt", ["int4", "uint4"])
@pytest.mark.parametrize("rfmt", ["int8", "int4", "uint4"])
def test_integer_four_bit_products_equal_int64_matmul(lfmt, rfmt):
    g = torch.Generator().manual_seed(2)
    sizes = [11, 0, 29, 6]
    M, N, K = sum(sizes) + 4, 24, 256
    lhs = torch.randint(0, 256, (M, K // 2), generator=g).to(torch.uint8)
    if rfmt == "int8":
        rhs = torch.randint(-128, 128, (len(sizes), N, K), generator=g).to(torch.int8)
        w = rhs.to(torch.int64)
        kw = {}
    else:
        rhs = torch.randint(0, 256, (len(sizes), N, K // 2), generator=g).to(torch.uint8)
        w = _unpack(rhs, rfmt).to(torch.int64)
        kw = {"rhs_format": rfmt}
    got = oracle.gmm_reference(lhs, rhs, torch.tensor(sizes, dtype=torch.int32), lhs_format=lfmt, **kw)
    a = _unpack(lhs, lfmt).to(torch.int64)
    o = _segments(sizes)
    want = np.zeros((M, N), dtype=np.int64)
    for h in range(len(sizes)):
        want[o[h]:o[h + 1]] = (a[o[h]:o[h + 1]] @ w[h].t()).numpy()
    assert np.array_equal(got, want.astype(np.float64))


@pytest.mark.parametrize("rfmt", ["e4m3", "e5m2", "fp4_e2m1"])
def test_fp4_activations_with_block_scales_equal_the_float64_product(rfmt):
    g = torch.Generator().manual_seed(3)
    sizes = [13, 0, 21]
    M, N, K, nb = sum(sizes) + 2, 16, 256, 2
    lhs = torch.randint(0, 256, (M, K // 2), generator=g).to(torch.uint8)
    if rfmt == "fp4_e2m1":
        rhs = torch.randint(0, 256, (len(sizes), N, K // 2), generator=g).to(torch.uint8)
        w = _unpack(rhs, rfmt)
        kw = {"rhs_format": rfmt}
    else:
        dt = torch.float8_e4m3fn if rfmt == "e4m3" else torch.float8_e5m2
        rhs = (torch.randn(len(sizes), N, K, generator=g) * 4).to(dt)
        w = rhs.double()
        kw = {}
    rs = torch.rand(len(sizes), nb, 1, N, generator=g) + 0.5
    ls = torch.rand(M, nb, generator=g) + 0.5
    got = oracle.gmm_reference(lhs, rhs, torch.tensor(sizes, dtype=torch.int32), lhs_format="fp4_e2m1",
                               rhs_scale=rs, lhs_scale=ls, **kw)
    a = _unpack(lhs, "fp4_e2m1")
    o = _segments(sizes)
    blk = K // nb
    want = np.zeros((M, N))
    for h in range(len(sizes)):
        for b in range(nb):
            part = a[o[h]:o[h + 1], b * blk:(b + 1) * blk] @ w[h][:, b * blk:(b + 1) * blk].t()
            want[o[h]:o[h + 1]] += (part * rs[h, b, 0].double()[None, :] * ls[o[h]:o[h + 1], b].double()[:, None]).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_planted_mistakes_are_caught():
    """Swapping the nibbles of each activation byte, or reading int4 as
    uint4, changes the one-hot read-back the pins compare against."""
    g = torch.Generator().manual_seed(4)
    M, K = 5, 32
    packed = torch.randint(0, 256, (M, K // 2), generator=g).to(torch.uint8)
    packed[0, 0] = 0x9F  # a negative int4 (0xF = -1) and a high nibble that differs
    eye = torch.eye(K).to(torch.bfloat16)[None]
    gs = torch.tensor([M], dtype=torch.int32)
    want = _unpack(packed, "int4").numpy()
    assert np.array_equal(oracle.gmm_reference(packed, eye, gs, lhs_format="int4"), want)
    swapped = ((packed >> 4) | (packed << 4)).to(torch.uint8)
    assert not np.array_equal(oracle.gmm_reference(swapped, eye, gs, lhs_format="int4"), want)
    assert not np.array_equal(oracle.gmm_reference(packed, eye, gs, lhs_format="uint4"), want)
