"""Tile metadata, written out in plain integer loops (oracle side).

TEST INFRASTRUCTURE ONLY; shares no code with the HIP path.

Two definitions live here:

* ``megablox_metadata`` -- the tile metadata of the Megablox gmm
  (tpu-inference 0.13.2 wheel diff page, megablox/gmm.py,
  make_group_metadata): group offsets as a cumulative sum; each group's
  start rounded down and end rounded up to the m-tile size; empty groups get
  no tile (or one, when empty groups are visited); group ids repeated by tile
  count; m-tile ids repeated by visit count, where a tile is visited once by
  the group owning its first row plus once per group that starts inside it;
  the metadata of the active shard rotated to the front; the tile count of the
  active groups.  It is used only to pin ``tile_worklist`` to the pages.

* ``tile_worklist`` -- the group-aligned m-tiles the GPU path schedules: every
  active non-empty group g is cut into ceil(size_g / tm) tiles that start at
  the group's first row, so no tile holds rows of two groups.  On the pages a
  tile can straddle a group boundary and is then visited once per group with
  a row mask; both schemes compute each active row exactly once with its own
  group's weight, which ``tests/test_oracle_pins.py`` checks.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple


def group_offsets(group_sizes: Sequence[int]) -> List[int]:
    """o[0] = 0, o[g+1] = o[g] + size_g (make_group_metadata, first step)."""
    o = [0]
    for s in group_sizes:
        o.append(o[-1] + int(s))
    return o


def tile_worklist(group_sizes: Sequence[int], group_offset: int, num_active: int,
                  tm: int) -> List[Tuple[int, int, int]]:
    """Group-aligned m-tiles as (group, first_row, rows), groups ascending.

    Only groups group_offset .. group_offset+num_active-1 contribute; empty
    groups contribute nothing."""
    o = group_offsets(group_sizes)
    tiles = []
    for g in range(group_offset, group_offset + num_active):
        size = o[g + 1] - o[g]
        j = 0
        while j * tm < size:
            tiles.append((g, o[g] + j * tm, min(tm, size - j * tm)))
            j += 1
    return tiles


def megablox_metadata(group_sizes: Sequence[int], m: int, tm: int, start_group: int,
                      num_nonzero_groups: int, visit_empty_groups: bool = False):
    """(group_offsets, group_ids, m_tile_ids, num_tiles) as the Megablox
    make_group_metadata defines them, for m divisible by tm.

    The histogram of partial-tile starts is read as a plain count of the
    groups that are non-empty (or visited when empty) and start strictly
    inside tile t."""
    G = len(group_sizes)
    if m % tm:
        raise ValueError("m must be divisible by tm")
    tiles_m = m // tm
    o = group_offsets(group_sizes)
    ends = o[1:]
    starts = o[:-1]
    group_tiles = []
    for g in range(G):
        if group_sizes[g] == 0:
            group_tiles.append(1 if visit_empty_groups else 0)
        else:
            rounded_end = (ends[g] + tm - 1) // tm * tm
            rounded_start = starts[g] // tm * tm
            group_tiles.append((rounded_end - rounded_start) // tm)
    length = tiles_m + G - 1
    group_ids = []
    for g in range(G):
        group_ids.extend([g] * group_tiles[g])
    group_ids = (group_ids + [G - 1] * length)[:length]
    visits = [1] * tiles_m
    for g in range(G):
        if group_sizes[g] == 0:
            counted = visit_empty_groups
        else:
            counted = starts[g] % tm != 0
        if counted and starts[g] // tm < tiles_m:
            visits[starts[g] // tm] += 1
    m_tile_ids = []
    for t in range(tiles_m):
        m_tile_ids.extend([t] * visits[t])
    m_tile_ids = (m_tile_ids + [tiles_m - 1] * length)[:length]
    first = sum(1 for gid in group_ids if gid < start_group)
    group_ids = group_ids[first:] + group_ids[:first]
    m_tile_ids = m_tile_ids[first:] + m_tile_ids[:first]
    end_group = start_group + num_nonzero_groups - 1
    num_tiles = sum(group_tiles[g] for g in range(G) if start_group <= g <= end_group)
    return o, group_ids, m_tile_ids, num_tiles
