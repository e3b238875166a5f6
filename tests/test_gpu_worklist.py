"""The device-built group offsets and m-tile table are bit-exact against the
oracle's plain integer loops; invalid device data is clamped and flagged."""
import numpy as np
import pytest
import torch

from oracle import worklist

pytestmark = pytest.mark.gpu


def _check(sizes, s, ga, tm, M):
    import moe_grouped_matrix_amd as m
    gs = torch.tensor(sizes, dtype=torch.int32, device="cuda")
    print(f"worklist G={len(sizes)} s={s} ga={ga} tm={tm} M={M}", flush=True)
    tiles, info = m.debug_worklist(gs, ga, M, tm, group_offset=s if s else None)
    want = worklist.tile_worklist(sizes, s, ga, tm)
    assert int(info[0]) == len(want)
    assert [tuple(t) for t in tiles.tolist()] == want
    o = worklist.group_offsets(sizes)
    assert int(info[1]) == o[s] and int(info[2]) == o[s + ga]
    assert int(info[3]) == 0


def test_worklist_edge_cases():
    _check([5], 0, 1, 4, 5)
    _check([0], 0, 1, 4, 3)
    _check([0, 0, 0], 1, 2, 16, 10)
    _check([3, 0, 5], 0, 3, 4, 8)
    _check([3, 0, 5], 2, 1, 4, 8)
    _check([3, 0, 5], 1, 0, 4, 8)
    _check([32, 32, 1, 31, 33], 0, 5, 32, 200)
    _check([0] * 1023 + [7], 0, 1024, 4, 7)
    _check([1] * 1024, 100, 900, 256, 1024)


def test_worklist_random():
    rng = np.random.default_rng(0)
    for _ in range(60):
        G = int(rng.integers(1, 1025))
        sizes = rng.integers(0, 300, size=G)
        sizes[rng.random(G) < 0.3] = 0
        sizes = sizes.astype(int).tolist()
        s = int(rng.integers(0, G))
        ga = int(rng.integers(0, G - s + 1))
        tm = int(rng.choice([1, 16, 32, 64, 256, 257]))
        M = sum(sizes) + int(rng.integers(0, 50))
        _check(sizes, s, ga, tm, M)


def test_invalid_device_data_is_clamped_and_flagged():
    import moe_grouped_matrix_amd as m
    gs = torch.tensor([4, -3, 5], dtype=torch.int32, device="cuda")
    tiles, info = m.debug_worklist(gs, 3, 20, 4)
    assert int(info[3]) & m.FLAG_NEGATIVE_SIZE
    assert [tuple(t) for t in tiles.tolist()] == worklist.tile_worklist([4, 0, 5], 0, 3, 4)
    gs = torch.tensor([4, 6, 5], dtype=torch.int32, device="cuda")
    tiles, info = m.debug_worklist(gs, 3, 8, 4)
    assert int(info[3]) & m.FLAG_SIZES_EXCEED_M
    assert [tuple(t) for t in tiles.tolist()] == [(0, 0, 4), (1, 4, 4)]
    tiles, info = m.debug_worklist(gs, 2, 100, 4, group_offset=2)
    assert int(info[3]) & m.FLAG_BAD_OFFSET
    assert [tuple(t) for t in tiles.tolist()] == worklist.tile_worklist([4, 6, 5], 2, 1, 4)
    m.device_flags()  # clear what the calls above reported
