"""The transposed product's gang schedule hands out groups at its meets
(tg_gang_meet in gmm_tgmm.hpp).  This CPU model runs the same word
arithmetic under random interleavings of the workgroups' atomic steps:

  - one 64-bit word per queue: arrivals in bits 0..23, and at meet m the
    leader's published list index added into the 20-bit field at bit
    24 + 20 (m % 2);
  - a grid-wide counter from which each queue's leader takes the list item
    after next (the queue's first two items are x and 2 Q - 1 - x);
  - every workgroup adds its arrival (the leader with its index), waits
    until T (m + 1) arrivals are in, and reads the index as the growth of
    the field since the value it saw two meets earlier.

It checks that every workgroup of a queue derives the same sequence of
groups, that the queues together take every group exactly once, and that
the fields never carry into each other, up to the 1024-group maximum.  (A
model of the protocol, not of the kernel's timing: the device code polls
with bounded waits; here a step that would poll just yields.)"""
import random

import pytest

Q = 8
ARR_BITS, FIELD_BITS, FIELD0 = 24, 20, 24


def _simulate(ga: int, T: int, seed: int):
    rng = random.Random(seed)
    words = [0] * Q
    grid_next = [0]
    # per workgroup state: queue, rank, items, meet number, seen fields, phase
    wgs = []
    for x in range(Q):
        for j in range(T):
            wgs.append({"x": x, "j": j, "items": [x, 2 * Q - 1 - x], "m": 0, "seen": [0, 0], "phase": "arrive",
                        "done": False, "after": None})

    def has_successor(wg):
        return wg["items"][-1] < ga

    # a workgroup meets before its (m+1)-th group's loads, only while its
    # current group has a successor; the item after next comes out of meet m
    steps = 0
    while not all(w["done"] for w in wgs):
        steps += 1
        assert steps < 10_000_000, "the model did not finish"
        wg = rng.choice([w for w in wgs if not w["done"]])
        m = wg["m"]
        cur_index = m  # the workgroup is in its m-th group, items[m]
        if cur_index >= len(wg["items"]) or wg["items"][cur_index] >= ga:
            wg["done"] = True
            continue
        if wg["items"][cur_index + 1] >= ga:  # no successor: no meet, this is the last group
            wg["done"] = True
            continue
        sh = FIELD0 + FIELD_BITS * (m & 1)
        x = wg["x"]
        if wg["phase"] == "arrive":
            add = 1
            if wg["j"] == 0:
                mine = 2 * Q + grid_next[0]
                grid_next[0] += 1
                add += mine << sh
            words[x] += add
            assert words[x] < (1 << 64)
            wg["phase"] = "poll"
        else:
            v = words[x]
            if (v & ((1 << ARR_BITS) - 1)) < T * (m + 1):
                continue  # not all arrived: poll again later
            f = (v >> sh) & ((1 << FIELD_BITS) - 1)
            assert f != wg["seen"][m & 1], "all arrived but the leader's index is not in the field"
            idx = f - wg["seen"][m & 1]
            wg["seen"][m & 1] = f
            wg["items"].append(idx)
            wg["m"] += 1
            wg["phase"] = "arrive"
    # the fields never overflowed into each other or past 64 bits
    for x in range(Q):
        v = words[x]
        f0 = (v >> FIELD0) & ((1 << FIELD_BITS) - 1)
        f1 = (v >> (FIELD0 + FIELD_BITS)) & ((1 << FIELD_BITS) - 1)
        assert v == (v & ((1 << ARR_BITS) - 1)) + (f0 << FIELD0) + (f1 << (FIELD0 + FIELD_BITS))
    return wgs


@pytest.mark.parametrize("ga,T,seed", [(16, 4, 1), (17, 3, 2), (40, 5, 3), (128, 4, 4), (300, 2, 5),
                                       (1024, 2, 6)])
def test_gang_meets_hand_every_group_to_exactly_one_queue(ga, T, seed):
    wgs = _simulate(ga, T, seed)
    taken = {}
    for x in range(Q):
        seqs = {tuple(i for i in w["items"] if i < ga) for w in wgs if w["x"] == x}
        assert len(seqs) == 1, f"queue {x}: its workgroups disagree on the groups"
        for i in seqs.pop():
            assert i not in taken, f"group {i} taken by queues {taken[i]} and {x}"
            taken[i] = x
    assert sorted(taken) == list(range(ga))
