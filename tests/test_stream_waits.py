"""The weight-streaming kernel's constant vmcnt waits (gmm_stream.hpp), on
the CPU.

A wave's memory operations complete in the order they were issued, and
`s_waitcnt vmcnt(n)` returns once at most n of them are outstanding: after
the wait every operation but the n newest has completed.  A wait for a
stage is therefore exact when n equals the number of operations issued
after that stage's last load: with fewer it also waits for newer loads
(draining the pipeline), with more the stage may still be in flight.

This model replays one wave's issue order through the kernel's schedule --
the prologue's first S-1 stages and its E range-dropped stores, then for
each tile and stage kt the loads of stage kt+S-1 (or of the next tile's),
the epilogue's E stores in a tile's last stage, and the wait before the
next stage's fragments are read, with the kernel's constants: (S-2) stages
of loads, plus E where the wait is WITH_E (a tile's stage 0 and its last
stage).  It checks that every wait is exact, for waves 0-1 (one load per
stage more: the scales, the bias) and the others, with one-byte weights (6
and 7 loads per stage) and four-bit ones (4 and 5), bf16 and f32 output
(E = 4, 8), and tiles of 3 to 11 stages."""
import pytest

S = 3


def _replay(KT: int, tiles: int, ops: int, E: int, with_e_rule):
    issued = []
    waits = []

    def load(tile, stage):
        issued.extend([("L", tile, stage)] * ops)

    def wait(n, need):
        last = max(i for i, op in enumerate(issued) if op == need)
        waits.append((need, n, len(issued) - 1 - last))

    for st in range(S - 1):
        load(0, st)
    issued.extend([("E", -1)] * E)
    wait((S - 2) * ops + E, ("L", 0, 0))
    for t in range(tiles):
        for kt in range(KT):
            nxt = kt >= KT - S + 1
            kd = kt + S - 1 - KT if nxt else kt + S - 1
            load(t + 1 if nxt else t, kd)
            if kt == KT - 1:
                issued.extend([("E", t)] * E)
            need = ("L", t, kt + 1) if kt + 1 < KT else ("L", t + 1, 0)
            wait((S - 2) * ops + (E if with_e_rule(kt, KT) else 0), need)
    return waits


def _kernel_rule(kt, KT):
    # the kernel's tile loop: kstage(WE, ...) at kt = 0 and kt = KT - 1
    return kt == 0 or kt == KT - 1


@pytest.mark.parametrize("KT", [3, 4, 5, 8, 11])
@pytest.mark.parametrize("ops", [4, 5, 6, 7])
@pytest.mark.parametrize("E", [4, 8])
def test_every_stream_wait_is_exact(KT, ops, E):
    waits = _replay(KT, tiles=4, ops=ops, E=E, with_e_rule=_kernel_rule)
    assert len(waits) == 1 + 4 * KT
    for need, n, newer in waits:
        assert n == newer, f"wait for {need}: vmcnt({n}) but {newer} operations were issued after it"


@pytest.mark.parametrize("rule", [lambda kt, KT: False, lambda kt, KT: kt == KT - 1, lambda kt, KT: kt <= 1])
def test_a_wrong_store_allowance_is_caught(rule):
    """The model is not vacuous: leaving the stores out of a tile boundary's
    waits, or counting them one stage too long, makes some wait inexact."""
    waits = _replay(5, tiles=3, ops=7, E=8, with_e_rule=rule)
    assert any(n != newer for _, n, newer in waits)
