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
tile."""
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


@pytest.fixture(scope="module")
def kernel_asm(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "kernels.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-Wno-unused-command-line-argument", "-I" + os.path.join(ROOT, "include"),
           "-S", "--cuda-device-only", os.path.join(CSRC, "gmm_kernels.hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text()


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
        assert stores == 2 * E_FULL[out_f32], (name, stores)
        seen += 1
    assert seen == 2  # bf16 / f32 output


def test_loop_kernels_do_not_spill(kernel_asm):
    # a spill reload is a vector memory load: its wait would drain every
    # direct-to-LDS load queued behind the K loop's constant counts
    for pattern in (r"_ZN4gmmk15gmm_tgmm_kernel", r"_ZN4gmmk17gmm_stream_kernel", r"_ZN4gmmk15gmm_w8a8_kernel"):
        for name, lines in _functions(kernel_asm, pattern):
            assert not any(ln.startswith("scratch_") for ln in lines), name
