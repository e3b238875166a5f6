"""GPU parity of the activation quantiser (gmm_quant_fp8_run) against the
oracle, through the C ABI: codes and scales must be identical bit for bit
(the quantised code is an integer decision both sides take in binary32).

Small cases compare every element: ragged row counts, one-block rows, an
all-zero block, -0, values that land exactly on rounding ties between e4m3
values (even-mantissa rule), the subnormal e4m3 range, values that clamp at
448, bf16 extremes, and block scales far from 1 on both sides of the
kernel's switch between division and reciprocal.  The full-size case
quantises the forward workload's activations ([262144,1408] bf16) in the
benchmark's launch configuration and compares every element.  The end-to-end
case feeds the device's codes and scales to the W8A8 gmm and checks it
against the oracle's gmm of the same bytes."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import compare

pytestmark = pytest.mark.gpu


def _check(x, q, s, what):
    wq, ws = oracle.quant_fp8_reference(x.cpu())
    gq = q.cpu().view(torch.uint8)
    bad = (gq != wq.view(torch.uint8)).nonzero()
    assert bad.numel() == 0, f"{what}: {bad.shape[0]} codes differ, first at {bad[0].tolist()}: " \
                             f"x={x.cpu()[tuple(bad[0])].item()} got {int(gq[tuple(bad[0])])} " \
                             f"want {int(wq.view(torch.uint8)[tuple(bad[0])])}"
    assert torch.equal(s.cpu().view(torch.int32), ws.view(torch.int32)), f"{what}: scales differ"


def _adversarial(M, K, seed):
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn(M, K, generator=g) * 0.02).to(torch.bfloat16)
    nb = K // 128
    if M > 4 and nb > 1:
        x[0, :128] = 0.0                                   # all-zero block: scale 1
        x[1, 128:256] = -0.0
        # scale exactly 1 (amax 448), then exact e4m3 ties and neighbours
        pos = np.unique([oracle.decode_e4m3fn(c) for c in range(0x7F)])
        mids = (pos[1:] + pos[:-1]) / 2
        row = np.resize(np.concatenate([mids[:60], -mids[60:120]]), 128).astype(np.float32)
        row[0] = 448.0
        x[2, :128] = torch.from_numpy(row).to(torch.bfloat16)
        # subnormal e4m3 range under scale 1
        sub = np.resize(np.arange(1, 64) * 2.0 ** -12, 128).astype(np.float32)
        sub[0] = 448.0
        x[3, 128:256] = torch.from_numpy(sub * np.where(np.arange(128) % 2, -1, 1)).to(torch.bfloat16)
        # bf16 extremes in one block
        x[4, :128] = torch.tensor([3.0e38, -1.0e-38, 1.0, -2.0] * 32).to(torch.bfloat16)
    if M > 10 and nb > 2:
        # scales far from 1, on both sides of 2^-92 (below it the kernel
        # divides; above, it multiplies by the reciprocal and corrects)
        for i, mag in enumerate([1.0e-30, 2.0 ** -80, 2.0 ** -83, 1.0e20, 3.0]):
            x[5 + i, 256:384] = (torch.randn(128, generator=g) * mag).to(torch.bfloat16)
    return x


@pytest.mark.parametrize("M,K", [(37, 384), (1, 128), (5, 1408), (1000, 256)])
def test_quant_every_element(M, K):
    import moe_grouped_matrix_amd as m
    x = _adversarial(M, K, seed=M + K)
    print(f"quant case M={M} K={K}", flush=True)
    q, s = m.quant_fp8(x.cuda())
    torch.cuda.synchronize()
    _check(x, q, s, f"quant M={M} K={K}")


def test_quant_full_size_every_element():
    """The benchmark's workload (the forward activations, [262144,1408] bf16)
    in its launch configuration; the oracle quantises all of it in about a
    second, so every code and scale is compared."""
    import moe_grouped_matrix_amd as m
    case = workloads.quant_fp8_act(device="cuda")
    x = case.x
    print(f"quant full M={x.shape[0]} K={x.shape[1]}", flush=True)
    q, s = m.quant_fp8(x)
    torch.cuda.synchronize()
    _check(x, q, s, "quant full")


def test_quant_then_w8a8_gmm_end_to_end():
    """Activations quantised on the device feed the fp8 x fp8 gmm with their
    per-token scales; the oracle computes the gmm from the same bytes."""
    import moe_grouped_matrix_amd as m
    g = torch.Generator().manual_seed(11)
    sizes = [100, 0, 260, 37, 140]
    M, K, N = sum(sizes) + 9, 512, 136
    x = (torch.randn(M, K, generator=g) * 0.02).to(torch.bfloat16)
    w = torch.randn(len(sizes), N, K, generator=g) * 0.02
    wq, ws = workloads.quantize_e4m3_blocks(w, 128)            # weight inputs, as the W8A8 workload
    rs = ws.permute(0, 2, 1).unsqueeze(2).contiguous()
    gs = torch.tensor(sizes, dtype=torch.int32)
    print("quant + w8a8 gmm", flush=True)
    q, s = m.quant_fp8(x.cuda())
    out = m.gmm(q, wq.cuda(), gs.cuda(), rhs_scale=rs.cuda(), lhs_scale=s, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    _check(x, q, s, "quant for w8a8")
    ref = oracle.gmm_reference(q.cpu(), wq, gs, rhs_scale=rs, lhs_scale=s.cpu())
    hi = sum(sizes)
    compare(out.cpu()[:hi], ref[:hi], torch.bfloat16, "quant + w8a8 gmm")
    assert torch.all(out.cpu()[hi:].view(torch.int16) == 0)


def test_quant_rejects_invalid_arguments():
    import moe_grouped_matrix_amd as m
    with pytest.raises(m.GmmInvalid):
        m.quant_fp8(torch.zeros(4, 100, dtype=torch.bfloat16, device="cuda"))   # K % 128
    with pytest.raises(m.GmmInvalid):
        m.quant_fp8(torch.zeros(4, 128, dtype=torch.float32, device="cuda"))    # not bf16
    x = torch.zeros(4, 256, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(m.GmmInvalid):
        m.quant_fp8(x, scale=torch.zeros(4, 3, device="cuda"))
    torch.cuda.synchronize()
