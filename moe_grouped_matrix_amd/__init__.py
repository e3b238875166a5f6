"""Grouped matrix multiplication (gmm) for AMD MI355X (gfx950).

The computation runs in hand-written HIP kernels behind the C ABI of
libgmm.so (include/gmm.h); this package is the thin Python binding over it.
Build the library with ``moe_grouped_matrix_amd.build.build()``."""
from ._binding import (EXPORTED, FLAG_BAD_OFFSET, FLAG_NEGATIVE_SIZE, FLAG_SCHEDULE_TIMEOUT,  # noqa: F401
                       FLAG_SIZES_EXCEED_M,
                       LIB_PATH, GmmDeviceDataError, GmmError, GmmInvalid, GmmUnsupported,
                       debug_worklist, device_flags, gmm, handle, load, quant_fp8, set_grid_limit,
                       set_tile_policy, tgmm, widen_scales)

__all__ = ["gmm", "tgmm", "quant_fp8", "widen_scales", "device_flags", "debug_worklist", "set_tile_policy",
           "set_grid_limit", "load", "handle", "GmmError", "GmmInvalid", "GmmUnsupported", "GmmDeviceDataError",
           "LIB_PATH"]
