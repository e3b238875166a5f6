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


def test_binding_constants_match_the_header():
    """The binding's status codes and device-flag bits are the values the
    header defines (the kernels' own flag constants are checked against the
    header by the library's build: gmm_api.cpp static_asserts them)."""
    from moe_grouped_matrix_amd import _binding as b
    text = open(HEADER).read()
    flags = {k: int(v, 16) for k, v in re.findall(r"#define (GMM_FLAG_\w+) (0x[0-9a-fA-F]+)u", text)}
    assert flags == {"GMM_FLAG_NEGATIVE_SIZE": b.FLAG_NEGATIVE_SIZE, "GMM_FLAG_SIZES_EXCEED_M": b.FLAG_SIZES_EXCEED_M,
                     "GMM_FLAG_BAD_OFFSET": b.FLAG_BAD_OFFSET, "GMM_FLAG_SCHEDULE_TIMEOUT": b.FLAG_SCHEDULE_TIMEOUT}
    status = {k: int(v) for k, v in re.findall(r"^\s*(GMM_(?:OK|E_\w+)) = (-?\d+)", text, flags=re.M)}
    assert status == {"GMM_OK": b.GMM_OK, "GMM_E_INVALID": b.GMM_E_INVALID, "GMM_E_UNSUPPORTED": b.GMM_E_UNSUPPORTED,
                      "GMM_E_HIP": b.GMM_E_HIP, "GMM_E_DEVICE_DATA": b.GMM_E_DEVICE_DATA}


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
    here as an undefined symbol and only fail at load time on a machine with a GPU)."""
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
