"""The C ABI library loads and exports every function include/gmm.h
declares; the product package does not touch the oracle (no GPU)."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gmm.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:gmm_status|const char\*)\s+(gmm_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib_path():
    from moe_grouped_matrix_amd import _binding, build
    if not os.path.exists(_binding.LIB_PATH):
        build.build()
    return _binding.LIB_PATH


def test_header_declares_the_entry_points():
    assert _declared() == sorted(["gmm_create", "gmm_destroy", "gmm_last_error", "gmm_run", "gmm_run_existing_out",
                                  "gmm_tgmm_run", "gmm_tgmm_run_noalloc", "gmm_quant_fp8_run", "gmm_widen_scales_run",
                                  "gmm_device_flags", "gmm_set_tile_policy", "gmm_set_grid_limit",
                                  "gmm_debug_worklist"])


def test_library_exports_every_declared_symbol(lib_path):
    import moe_grouped_matrix_amd as m
    lib = m.load(lib_path)
    for name in _declared():
        assert hasattr(lib, name), name
    syms = subprocess.run(["nm", "-D", "--defined-only", lib_path], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (gmm_\w+)$", syms, flags=re.M))
    assert set(_declared()) <= exported
    assert sorted(m.EXPORTED) == _declared()


def test_library_has_no_undefined_internal_symbols(lib_path):
    """Every kernel launched from the host has its launch stub in the library
    (a kernel the host compiler silently failed to instantiate would show up
    here as an undefined symbol and only fail at load time on a GPU machine)."""
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib_path], capture_output=True, text=True).stdout
    assert "gmmk" not in syms, [l for l in syms.splitlines() if "gmmk" in l]


def test_product_package_never_references_the_oracle():
    pkg = os.path.join(ROOT, "moe_grouped_matrix_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f


def test_missing_library_fails_loudly(tmp_path):
    from moe_grouped_matrix_amd import _binding
    saved = _binding._lib
    _binding._lib = None
    try:
        with pytest.raises(ImportError):
            _binding.load(str(tmp_path / "nope.so"))
    finally:
        _binding._lib = saved
