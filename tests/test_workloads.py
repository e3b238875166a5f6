"""The seeded generators produce the stated shapes and structure (no GPU)."""
import numpy as np
import torch

import workloads


def test_router_sizes_full_shape_is_deterministic():
    a = workloads.router_group_sizes(1002, 32768, 128, 8)
    b = workloads.router_group_sizes(1002, 32768, 128, 8)
    assert np.array_equal(a, b)
    assert a.dtype == np.int32 and a.shape == (128,)
    assert a.sum() == 32768 * 8
    assert a.max() <= 32768          # a token picks an expert at most once
    assert a.max() > 8 * a.min()     # Zipf skew


def test_decode_sizes_have_forced_empty_experts():
    s = workloads.router_group_sizes(1004, 256, 128, 8, forced_empty=51)
    assert s.sum() == 2048
    assert (s == 0).sum() >= 51


def test_tiny_fp32_structure():
    c = workloads.tiny_fp32()
    s = c.sizes_list()
    assert s[1] == 0 and sum(s) == 480 and c.M == 512
    assert c.lhs.dtype == torch.float32 and tuple(c.rhs.shape) == (4, 384, 256)


def test_small_cases_shapes():
    for name, make in workloads.SMALL.items():
        c = make()
        assert c.lhs.shape[0] == c.M
        assert c.active_rows() <= c.M
        if c.transpose_rhs:
            assert c.rhs.shape[1] == c.K
        else:
            assert c.rhs.shape[2] == c.K
        if c.rhs_scale is not None:
            assert tuple(c.rhs_scale.shape) == (c.num_active, c.K // 128, 1, c.N)
        if c.lhs_scale is not None:
            assert tuple(c.lhs_scale.shape) == (c.M, c.K // 128)


def test_quantizer_roundtrip_error_is_small():
    x = workloads.normal((64, 256), 1.0, 3)
    q, sc = workloads.quantize_e4m3_blocks(x)
    back = q.to(torch.float32).reshape(64, 2, 128) * sc[:, :, None]
    err = (back.reshape(64, 256) - x).abs().max() / x.abs().max()
    assert err < 0.07  # e4m3 keeps 3 mantissa bits
    assert q.to(torch.float32).abs().max() <= 448
