"""Build libgmm.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Run ``python -m moe_grouped_matrix_amd.build`` or call ``build()``; the
library is written next to this file."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgmm.so")
SOURCES = [os.path.join(CSRC, n) for n in
           ("gmm_kernels.hip", "gmm_w8a8.hip", "gmm_stream.hip", "gmm_quant.hip", "gmm_api.cpp")]

# Packed fp32 VALU instructions are kept out of the generated code.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wno-unused-command-line-argument"]

# Per-source additions: the block-scaled fp8 kernel and the weight-streaming
# kernel keep their MFMA results in ordinary VGPRs, where their scale folds
# read them.
EXTRA_FLAGS = {"gmm_w8a8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "gmm_stream.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link."""
    tag = ".tmp%d" % os.getpid()
    inc = "-I" + os.path.join(HERE, "..", "include")
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(CSRC, os.path.basename(src) + tag + ".o")
        cmd = [hipcc()] + HIPCC_FLAGS + EXTRA_FLAGS.get(os.path.basename(src), []) + [inc, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    errors = []
    for cmd, pr in procs:
        out, err = pr.communicate()
        if pr.returncode != 0:
            errors.append(" ".join(cmd) + "\n" + out + err)
    try:
        if errors:
            raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
        tmp = LIB + tag
        _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
        os.replace(tmp, LIB)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
