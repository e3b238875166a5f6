"""Pins for the oracle's int8 operands (int8 is one of the dtypes the
Megablox gmm accepts, assert_is_supported_dtype on the tpu-inference wheel
diff page), CPU only.

int8 x int8 products are exact integers, so the oracle must equal torch's
int64 matmul of the same values bit for bit (a library routine), with and
without power-of-two block scales; bf16 x int8 must equal torch's float64
product of the decoded values; every byte decodes to its two's-complement
value.  The last test plants a mistake (bytes read as unsigned) and checks
that the pins reject it."""
import numpy as np
import torch

import oracle


def _segments_int(lhs, rhs, sizes):
    o = np.concatenate([[0], np.cumsum(sizes)]).astype(int)
    out = torch.zeros(lhs.shape[0], rhs.shape[1], dtype=torch.int64)
    for h in range(len(sizes)):
        out[o[h]:o[h + 1]] = lhs[o[h]:o[h + 1]].to(torch.int64) @ rhs[h].to(torch.int64).t()
    return out.numpy().astype(np.float64)


def _ints(seed, M, K, N, G):
    g = torch.Generator().manual_seed(seed)
    lhs = torch.randint(-128, 128, (M, K), generator=g).to(torch.int8)
    rhs = torch.randint(-128, 128, (G, N, K), generator=g).to(torch.int8)
    return lhs, rhs


def test_every_int8_value_decodes():
    vals = torch.arange(-128, 128, dtype=torch.int16).to(torch.int8)
    lhs = vals.view(256, 1)
    rhs = torch.ones(1, 1, 1, dtype=torch.int8)
    got = oracle.gmm_reference(lhs, rhs, torch.tensor([256], dtype=torch.int32))
    assert np.array_equal(got[:, 0], np.arange(-128, 128, dtype=np.float64))


def test_int8_products_equal_integer_matmul():
    sizes = [7, 0, 19, 12]
    lhs, rhs = _ints(1, sum(sizes) + 3, 256, 24, len(sizes))
    got = oracle.gmm_reference(lhs, rhs, torch.tensor(sizes, dtype=torch.int32))
    want = _segments_int(lhs, rhs, sizes)
    assert np.array_equal(got[:sum(sizes)], want[:sum(sizes)])
    assert np.all(got[sum(sizes):] == 0)


def test_int8_with_power_of_two_block_scales_is_exact():
    sizes = [9, 14]
    nb = 2
    lhs, rhs = _ints(2, sum(sizes), 256, 16, len(sizes))
    g = torch.Generator().manual_seed(3)
    rs = 2.0 ** torch.randint(-4, 4, (len(sizes), nb, 1, 16), generator=g).float()
    got = oracle.gmm_reference(lhs, rhs, torch.tensor(sizes, dtype=torch.int32), rhs_scale=rs)
    o = [0, 9, 23]
    want = np.zeros((23, 16))
    for h in range(2):
        for b in range(nb):
            part = lhs[o[h]:o[h + 1], b * 128:(b + 1) * 128].to(torch.int64) @ \
                rhs[h, :, b * 128:(b + 1) * 128].to(torch.int64).t()
            want[o[h]:o[h + 1]] += part.numpy() * rs[h, b, 0].numpy()
    assert np.array_equal(got, want)


def test_bf16_times_int8_is_the_float64_product():
    g = torch.Generator().manual_seed(4)
    lhs = torch.randn(30, 128, generator=g).to(torch.bfloat16)
    rhs = torch.randint(-128, 128, (1, 20, 128), generator=g).to(torch.int8)
    got = oracle.gmm_reference(lhs, rhs, torch.tensor([30], dtype=torch.int32))
    want = (lhs.double() @ rhs[0].double().t()).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_planted_unsigned_read_is_caught():
    sizes = [10]
    lhs, rhs = _ints(5, 10, 128, 8, 1)
    want = _segments_int(lhs, rhs, sizes)
    mutant = _segments_int(lhs.view(torch.uint8).to(torch.int16), rhs.view(torch.uint8).to(torch.int16), sizes)
    assert not np.array_equal(mutant, want)
    assert np.array_equal(oracle.gmm_reference(lhs, rhs, torch.tensor(sizes, dtype=torch.int32)), want)
