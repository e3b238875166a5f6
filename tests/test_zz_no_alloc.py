"""gmm_tgmm_run_noalloc, the transposed product for callers that cannot
allocate, against gmm_tgmm_run through the C ABI.

Both entry points run the same kernel; only the home of the work-queue
counters differs (the library's static device scratch, cleared by the call,
against a per-stream block of the handle).  Each output tile is summed by one
workgroup in a fixed order whichever workgroup takes it, so the outputs must
agree bit for bit, and both must meet the float32 / bfloat16 tolerances of
tests/parity.py against the oracle.  Three calls in a row on a stream no
tgmm call has used, each smaller than the one before (the gang schedule at
the model's K = N = 1408, whose workgroups meet on the counters; the
dynamic schedule over eight work queues; one work queue, fewer rows and
columns, a bf16 output), queued back to back before one synchronisation:
the scratch keeps each call's state until the next clears it."""
import pytest
import torch

import oracle
from parity import compare

pytestmark = pytest.mark.gpu

CASES = [
    # (group sizes, rows past the groups, K, N, out dtype)
    # the model's K = N = 1408 over 16 groups: the gang schedule (32 tiles per
    # group, one per workgroup of an XCD, meeting on the scratch counters)
    ([50, 0, 33, 64, 1, 96, 20, 0, 64, 30, 17, 129, 0, 48, 5, 22], 4, 1408, 1408, torch.float32),
    # the dynamic schedule (its tiles handed out through the same counters)
    ([700, 0, 33, 250, 1, 96, 512, 0, 64, 300, 17, 129, 0, 480, 5, 222, 40, 610], 9, 512, 520, torch.float32),
    ([40, 0, 300, 7], 3, 256, 136, torch.bfloat16),
]


def _inputs(sizes, extra, K, N, seed):
    g = torch.Generator().manual_seed(seed)
    M = sum(sizes) + extra
    lhs = torch.randn(M, K, generator=g).to(torch.bfloat16)
    rhs = torch.randn(M, N, generator=g).to(torch.bfloat16)
    return lhs, rhs, torch.tensor(sizes, dtype=torch.int32)


def test_noalloc_tgmm_equals_tgmm_run_on_two_calls_in_a_row():
    import moe_grouped_matrix_amd as m
    m.set_grid_limit(0)
    stream = torch.cuda.Stream()
    ins, outs = [], []
    for i, (sizes, extra, K, N, od) in enumerate(CASES):
        lhs, rhs, gs = _inputs(sizes, extra, K, N, 20 + i)
        ins.append((lhs, rhs, gs))
        outs.append(torch.full((len(sizes), K, N), float("nan"), dtype=od, device="cuda"))
    dev = [(a.cuda(), b.cuda(), c.cuda()) for a, b, c in ins]
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for i, (lhs, rhs, gs) in enumerate(dev):
            print(f"no-alloc tgmm call {i}: G={gs.numel()} K={lhs.shape[1]} N={rhs.shape[1]}", flush=True)
            m.tgmm(lhs, rhs, gs, out=outs[i], no_alloc=True, stream=stream)
    stream.synchronize()
    for i, ((lhs, rhs, gs), (sizes, extra, K, N, od)) in enumerate(zip(dev, CASES)):
        want = m.tgmm(lhs, rhs, gs, out_dtype=od)
        torch.cuda.synchronize()
        iv = torch.int16 if od == torch.bfloat16 else torch.int32
        assert torch.equal(outs[i].view(iv), want.view(iv)), f"call {i}: no-alloc result differs"
        ref = oracle.tgmm_reference(*ins[i])
        Ga = len(sizes)
        compare(outs[i].cpu().reshape(Ga * K, N), ref.reshape(Ga * K, N), od, f"no-alloc call {i}")
        for h in range(Ga):
            if sizes[h] == 0:
                assert torch.all(outs[i][h].view(iv) == 0), f"call {i}: empty group {h} not zero"
    assert m.device_flags() == 0


def test_noalloc_tgmm_validates_like_tgmm_run():
    import moe_grouped_matrix_amd as m
    lhs = torch.zeros(8, 64, dtype=torch.bfloat16, device="cuda")
    rhs = torch.zeros(8, 60, dtype=torch.bfloat16, device="cuda")  # N % 8 != 0
    gs = torch.tensor([8], dtype=torch.int32, device="cuda")
    with pytest.raises(m.GmmUnsupported):
        m.tgmm(lhs, rhs, gs, no_alloc=True)
