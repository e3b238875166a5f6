"""Counted memory operations survive compilation (CPU only: hipcc cross-compiles
gfx950 assembly, nothing runs).

The big kernel's K loop waits on constant vmcnt values that count every
direct-to-LDS load and every output store a wave has issued.  A tile with
half the rows pads its epilogue with range-dropped stores up to the full
tile's count.  If the compiler merged or deleted any of those stores, the
waits after a half tile would be short by that many operations and the next
stages could read LDS before their loads land.  This test compiles the
kernels to assembly and checks that each big-kernel instantiation still has
both epilogues' stores: E for a full tile and E (real plus padding) for a half
tile; likewise the tgmm kernel's four tile shapes, the W8A8 and
weight-streaming kernels' loads and stores, and that the loop kernels do not
spill."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "moe_grouped_matrix_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

# epilogue stores per tile: FM * FN * ST_BLOCK with FM = 4, FN = 2 and four
# 16-byte stores per 32-row block for f32 output, two for bf16
E_FULL = {"true": 32, "false": 16}


def _compile(tmp_path_factory, source):
    """gfx950 assembly of one translation unit, with the library's flags."""
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    from moe_grouped_matrix_amd import build
    out = tmp_path_factory.mktemp("isa") / (source + ".s")
    flags = [f for f in build.HIPCC_FLAGS if f != "-fPIC"] + build.EXTRA_FLAGS.get(source, [])
    cmd = [HIPCC] + flags + ["-I" + os.path.join(ROOT, "include"), "-S", "--cuda-device-only",
                             os.path.join(CSRC, source), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text()


@pytest.fixture(scope="module")
def kernel_asm(tmp_path_factory):
    return _compile(tmp_path_factory, "gmm_kernels.hip")


@pytest.fixture(scope="module")
def w8a8_asm(tmp_path_factory):
    return _compile(tmp_path_factory, "gmm_w8a8.hip")


@pytest.fixture(scope="module")
def stream_asm(tmp_path_factory):
    return _compile(tmp_path_factory, "gmm_stream.hip")


def _functions(asm, pattern):
    for name in re.findall(r"^(" + pattern + r"\S*):", asm, re.M):
        start = asm.index(name + ":")
        end = asm.index(".Lfunc_end", start)
        body = [ln.strip() for ln in asm[start:end].split("\n")]
        yield name, [ln for ln in body if ln and not ln.startswith(";")]


def test_big_kernel_keeps_every_counted_store(kernel_asm):
    seen = 0
    for name, lines in _functions(kernel_asm, r"_ZN4gmmk14gmm_big_kernel"):
        m = re.search(r"BigCfgILb([01])ELb([01])E", name)
        out_f32 = "true" if m.group(2) == "1" else "false"
        stores = sum(1 for ln in lines if ln.startswith("buffer_store"))
        assert stores == 2 * E_FULL[out_f32], (name, stores)
        seen += 1
    assert seen == 8  # NT / NN x bf16 / f32 output x with / without bias


def test_tgmm_kernel_keeps_every_counted_store(kernel_asm):
    seen = 0
    for name, lines in _functions(kernel_asm, r"_ZN4gmmk15gmm_tgmm_kernel"):
        out_f32 = "true" if "TgCfgILb1E" in name else "false"
        stores = sum(1 for ln in lines if ln.startswith("buffer_store"))
        # full, half, tall and wide tiles each pad to the full tile's count
        assert stores == 4 * E_FULL[out_f32], (name, stores)
        seen += 1
    assert seen == 2  # bf16 / f32 output


def test_stream_kernel_keeps_every_counted_operation(stream_asm):
    """The weight-streaming kernel's waits count 8 direct-to-LDS loads per
    stage in the code (4 weight and 2 lhs per wave, the scale load of wave 0
    and the bias load of wave 1: two stages in the prologue and one in each
    of the K loop's four variants; four-bit weights: 2 weight loads, so 6) and E = 4 (bf16 output) or 8 (f32) stores
    per wave and tile: the prologue's E range-dropped stores and the
    epilogue of each of the three loop variants that can end a tile.  Where
    a stage is a tile's stage 0, wave 0's scale load and wave 1's bias load
    have the same form (offset 0) and may be one instruction with the
    resource chosen per wave -- still one load in each of those waves -- so
    up to two loads fewer appear in the code."""
    seen = 0
    for name, lines in _functions(stream_asm, r"_ZN4gmmk17gmm_stream_kernel"):
        m = re.search(r"StreamCfgILb([01])ELi([0-9])E", name)
        out_f32, fb = m.group(1) == "1", int(m.group(2))
        per_stage = 6 if fb >= 3 else 8
        loads = sum(1 for ln in lines if ln.startswith("buffer_load") and ln.endswith(" lds"))
        stores = sum(1 for ln in lines if ln.startswith("buffer_store"))
        assert 6 * per_stage - 2 <= loads <= 6 * per_stage, (name, loads)
        assert stores == 4 * (8 if out_f32 else 4), (name, stores)
        seen += 1
    assert seen == 12  # e4m3fn / e5m2 / int8 / int4 / uint4 / fp4 weights x bf16 / f32 output


def test_loop_kernels_do_not_spill(kernel_asm, w8a8_asm, stream_asm):
    # a spill reload is a vector memory load: its wait would drain every
    # direct-to-LDS load queued behind the K loop's constant counts
    seen = 0
    for asm, pattern in ((kernel_asm, r"_ZN4gmmk15gmm_tgmm_kernel"), (stream_asm, r"_ZN4gmmk17gmm_stream_kernel"),
                         (w8a8_asm, r"_ZN4gmmk15gmm_w8a8_kernel")):
        for name, lines in _functions(asm, pattern):
            assert not any(ln.startswith("scratch_") for ln in lines), name
            seen += 1
    assert seen == 2 + 12 + 8


def test_w8a8_kernel_keeps_every_counted_operation(w8a8_asm):
    """The W8A8 kernel's waits count 14 direct-to-LDS loads per wave and K
    step (three steps' worth in the prologue, one in the loop) and the
    epilogue's stores: 16 for bf16 output (16 bytes per lane after the
    permlane16 swap), 32 for f32."""
    seen = 0
    for name, lines in _functions(w8a8_asm, r"_ZN4gmmk15gmm_w8a8_kernel"):
        out_f32 = re.search(r"W8CfgILi[01]ELi[01]ELb([01])E", name).group(1) == "1"
        loads = sum(1 for ln in lines if ln.startswith("buffer_load") and ln.endswith(" lds"))
        stores = sum(1 for ln in lines if ln.startswith("buffer_store"))
        assert loads == 4 * 14, (name, loads)
        assert stores == (32 if out_f32 else 16), (name, stores)
        seen += 1
    assert seen == 8  # e4m3 / e5m2 on either side x bf16 / f32 output
