"""ctypes binding of libgmm.so (the C ABI in include/gmm.h).

Argument marshalling only: torch provides device memory and the current
stream; every step of the computation runs in the library's HIP kernels.
There is no fallback: when libgmm.so is missing or cannot be loaded, every
call raises."""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Union

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgmm.so")

GMM_F32, GMM_BF16, GMM_F8E4M3FN, GMM_I32, GMM_F8E5M2, GMM_E8M0, GMM_I8 = 0, 1, 2, 3, 4, 5, 6
GMM_I4, GMM_U4, GMM_F4E2M1 = 7, 8, 9
# four-bit weights: packed bytes (uint8, or float4_e2m1fn_x2) named by format
PACKED_FORMATS = {"int4": GMM_I4, "uint4": GMM_U4, "fp4_e2m1": GMM_F4E2M1}
GMM_OK, GMM_E_INVALID, GMM_E_UNSUPPORTED, GMM_E_HIP, GMM_E_DEVICE_DATA = 0, -1, -2, -3, -4
FLAG_NEGATIVE_SIZE, FLAG_SIZES_EXCEED_M, FLAG_BAD_OFFSET = 0x1, 0x2, 0x4
FLAG_SCHEDULE_TIMEOUT = 0x8  # not a data error: a tgmm call's workgroups could not all run at once

EXPORTED = ("gmm_create", "gmm_destroy", "gmm_last_error", "gmm_run", "gmm_run_existing_out", "gmm_tgmm_run",
            "gmm_tgmm_run_noalloc",
            "gmm_quant_fp8_run", "gmm_widen_scales_run", "gmm_device_flags", "gmm_set_tile_policy",
            "gmm_set_grid_limit", "gmm_debug_worklist")

_DTYPE = {torch.float32: GMM_F32, torch.bfloat16: GMM_BF16,
          torch.float8_e4m3fn: GMM_F8E4M3FN, torch.float8_e5m2: GMM_F8E5M2, torch.int32: GMM_I32,
          torch.float8_e8m0fnu: GMM_E8M0, torch.int8: GMM_I8}


class GmmError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"gmm status {status}: {msg}")
        self.status = status


class GmmInvalid(GmmError, ValueError):
    pass


class GmmUnsupported(GmmError):
    pass


class GmmDeviceDataError(GmmError):
    pass


class GmmTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4)]


_lib = None
_lock = threading.Lock()
_handles = {}


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libgmm.so (raises when it is not built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise ImportError(f"{path} is not built; run moe_grouped_matrix_amd.build.build()")
            lib = ctypes.CDLL(path)
            vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
            tp = ctypes.POINTER(GmmTensor)
            lib.gmm_create.argtypes = [ctypes.POINTER(vp), ctypes.c_int]
            lib.gmm_create.restype = ctypes.c_int
            lib.gmm_destroy.argtypes = [vp]
            lib.gmm_destroy.restype = ctypes.c_int
            lib.gmm_last_error.argtypes = [vp]
            lib.gmm_last_error.restype = ctypes.c_char_p
            lib.gmm_run.argtypes = [vp, tp, tp, tp, tp, tp, tp, vp, ctypes.c_int, tp, vp]
            lib.gmm_run.restype = ctypes.c_int
            lib.gmm_run_existing_out.argtypes = [vp, tp, tp, tp, tp, tp, tp, vp, ctypes.c_int, tp, tp, vp]
            lib.gmm_run_existing_out.restype = ctypes.c_int
            lib.gmm_widen_scales_run.argtypes = [vp, tp, tp, vp]
            lib.gmm_widen_scales_run.restype = ctypes.c_int
            lib.gmm_quant_fp8_run.argtypes = [vp, tp, tp, tp, vp]
            lib.gmm_quant_fp8_run.restype = ctypes.c_int
            lib.gmm_tgmm_run.argtypes = [vp, tp, tp, tp, vp, tp, vp]
            lib.gmm_tgmm_run.restype = ctypes.c_int
            lib.gmm_tgmm_run_noalloc.argtypes = [vp, tp, tp, tp, vp, tp, vp]
            lib.gmm_tgmm_run_noalloc.restype = ctypes.c_int
            lib.gmm_device_flags.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_uint32)]
            lib.gmm_device_flags.restype = ctypes.c_int
            lib.gmm_set_tile_policy.argtypes = [vp, ctypes.c_int]
            lib.gmm_set_tile_policy.restype = ctypes.c_int
            lib.gmm_set_grid_limit.argtypes = [vp, ctypes.c_int]
            lib.gmm_set_grid_limit.restype = ctypes.c_int
            lib.gmm_debug_worklist.argtypes = [vp, tp, vp, i64, i64, i32, vp, i64, vp, vp]
            lib.gmm_debug_worklist.restype = ctypes.c_int
            _lib = lib
    return _lib


def _raise(status: int, handle) -> None:
    if status == GMM_OK:
        return
    msg = load().gmm_last_error(handle).decode() if handle else ""
    cls = {GMM_E_INVALID: GmmInvalid, GMM_E_UNSUPPORTED: GmmUnsupported,
           GMM_E_DEVICE_DATA: GmmDeviceDataError}.get(status, GmmError)
    raise cls(status, msg)


def handle(device: Union[int, torch.device, None] = None):
    """The library handle of a CUDA/HIP device (created once per device)."""
    lib = load()
    if device is None:
        device = torch.cuda.current_device()
    if isinstance(device, torch.device):
        device = device.index if device.index is not None else torch.cuda.current_device()
    with _lock:
        h = _handles.get(device)
        if h is None:
            hp = ctypes.c_void_p()
            st = lib.gmm_create(ctypes.byref(hp), int(device))
            if st != GMM_OK:
                raise GmmError(st, f"gmm_create failed on device {device}")
            h = hp.value
            _handles[device] = h
    return h


def _view(t: Optional[torch.Tensor], name: str):
    if t is None:
        return None
    if not t.is_cuda:
        raise GmmInvalid(GMM_E_INVALID, f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise GmmInvalid(GMM_E_INVALID, f"{name} must be contiguous")
    if t.dtype not in _DTYPE:
        raise GmmInvalid(GMM_E_INVALID, f"{name}: unsupported dtype {t.dtype}")
    if t.dim() > 4:
        raise GmmInvalid(GMM_E_INVALID, f"{name}: more than 4 dimensions")
    v = GmmTensor()
    v.data = t.data_ptr() if t.numel() else None
    v.dtype = _DTYPE[t.dtype]
    v.ndim = t.dim()
    for i, s in enumerate(t.shape):
        v.shape[i] = s
    return v


def _view_packed(t: torch.Tensor, fmt: str, name: str):
    """A four-bit tensor: bytes [..., K/2] (uint8 or float4_e2m1fn_x2) seen
    by the C ABI as [..., K] elements of the named format."""
    if fmt not in PACKED_FORMATS:
        raise GmmInvalid(GMM_E_INVALID, f"{name}: unknown four-bit format {fmt!r}")
    if t.dtype not in (torch.uint8, torch.float4_e2m1fn_x2):
        raise GmmInvalid(GMM_E_INVALID, f"{name}: four-bit data comes as uint8 or float4_e2m1fn_x2 bytes")
    if not t.is_cuda or not t.is_contiguous() or t.dim() < 1 or t.dim() > 4:
        raise GmmInvalid(GMM_E_INVALID, f"{name} must be a contiguous device tensor of rank 1 to 4")
    v = GmmTensor()
    v.data = t.data_ptr() if t.numel() else None
    v.dtype = PACKED_FORMATS[fmt]
    v.ndim = t.dim()
    for i, s in enumerate(t.shape):
        v.shape[i] = s
    v.shape[t.dim() - 1] = 2 * t.shape[-1]
    return v


def _ref(v):
    return ctypes.byref(v) if v is not None else None


def _offset_ptr(group_offset, device) -> tuple:
    """(pointer, keep-alive) for the group offset argument."""
    if group_offset is None:
        return None, None
    if isinstance(group_offset, torch.Tensor):
        if group_offset.dtype != torch.int32 or group_offset.numel() != 1 or not group_offset.is_cuda:
            raise GmmInvalid(GMM_E_INVALID, "group_offset must be a one-element int32 device tensor")
        t = group_offset.reshape(1)
        if t.data_ptr() % 16:
            t = t.clone()
        return t.data_ptr(), t
    t = torch.tensor([int(group_offset)], dtype=torch.int32, device=device)
    return t.data_ptr(), t


def gmm(lhs: torch.Tensor, rhs: torch.Tensor, group_sizes: torch.Tensor, *,
        out_dtype: torch.dtype = torch.float32,
        rhs_scale: Optional[torch.Tensor] = None,
        rhs_bias: Optional[torch.Tensor] = None,
        lhs_scale: Optional[torch.Tensor] = None,
        group_offset=None,
        transpose_rhs: bool = False,
        existing_out: Optional[torch.Tensor] = None,
        rhs_format: Optional[str] = None,
        lhs_format: Optional[str] = None,
        out: Optional[torch.Tensor] = None,
        stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Grouped matmul on the GPU through libgmm.so.

    lhs [M,K]; rhs [Ga,N,K] (transpose_rhs False) or [Ga,K,N] (True);
    group_sizes int32 [G] on the device; rhs_scale f32 [Ga,nb,1,N];
    rhs_bias [Ga,1,N]; lhs_scale f32 [M,nb]; group_offset an int or a
    one-element int32 device tensor.  Returns out [M,N] of out_dtype (the
    float32 default follows the Megablox gmm).  With existing_out [M,N] the
    rows outside the active groups are its rows instead of zeros
    (gmm_run_existing_out); without out the result is written into
    existing_out itself.  rhs_format "int4", "uint4" or "fp4_e2m1" takes rhs
    as packed bytes [Ga,N,K/2] (uint8 or float4_e2m1fn_x2), two weights to a
    byte, even elements in the low nibble; lhs_format the same for packed
    four-bit activations, lhs bytes [M,K/2].  Four-bit pairs: a bf16 lhs
    with any four-bit weight (widened to bf16); int4 / uint4 / int8 with
    int4 / uint4 / int8 (int8 products); fp4 e2m1 / e4m3fn / e5m2 with
    fp4 e2m1 / e4m3fn / e5m2 (the f8f6f4 products)."""
    lib = load()
    dev = lhs.device
    h = handle(dev)
    M = lhs.shape[0] if lhs.dim() >= 1 else 0
    N = rhs.shape[2] if transpose_rhs else (rhs.shape[1] if rhs.dim() == 3 else 0)
    if out is None:
        out = existing_out if existing_out is not None else torch.empty((M, N), dtype=out_dtype, device=dev)
    packed = {"lhs": lhs_format, "rhs": rhs_format}
    views = [_view(t, n) if packed.get(n) is None else _view_packed(t, packed[n], n)
             for t, n in ((lhs, "lhs"), (rhs, "rhs"), (group_sizes, "group_sizes"),
                          (rhs_scale, "rhs_scale"), (rhs_bias, "rhs_bias"),
                          (lhs_scale, "lhs_scale"), (out, "out"))]
    off_ptr, keep = _offset_ptr(group_offset, dev)
    st = stream if stream is not None else torch.cuda.current_stream(dev)
    if existing_out is None:
        status = lib.gmm_run(h, *[_ref(v) for v in views[:6]], off_ptr, int(bool(transpose_rhs)),
                             _ref(views[6]), ctypes.c_void_p(st.cuda_stream))
    else:
        ex = _view(existing_out, "existing_out")
        status = lib.gmm_run_existing_out(h, *[_ref(v) for v in views[:6]], off_ptr, int(bool(transpose_rhs)),
                                          _ref(ex), _ref(views[6]), ctypes.c_void_p(st.cuda_stream))
    if keep is not None and status == GMM_OK:
        keep.record_stream(st)
    _raise(status, h)
    return out


def widen_scales(src: torch.Tensor, *, out: Optional[torch.Tensor] = None,
                 stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Block scales to float32 through libgmm.so (gmm_widen_scales_run):
    src bfloat16, float32 or float8_e8m0fnu (an E8M0 byte e becomes
    2^(e-127); e = 0 gives 2^-127 and e = 255 gives 0.0, as the metrale
    gemm_quant.rs page states, where torch's own conversion gives NaN)."""
    lib = load()
    dev = src.device
    h = handle(dev)
    if out is None:
        out = torch.empty(src.shape, dtype=torch.float32, device=dev)
    views = [_view(src, "src"), _view(out, "out")]
    st = stream if stream is not None else torch.cuda.current_stream(dev)
    _raise(lib.gmm_widen_scales_run(h, *[_ref(v) for v in views], ctypes.c_void_p(st.cuda_stream)), h)
    return out


def quant_fp8(x: torch.Tensor, *, q: Optional[torch.Tensor] = None, scale: Optional[torch.Tensor] = None,
              stream: Optional[torch.cuda.Stream] = None):
    """Per-token activation quantiser through libgmm.so (gmm_quant_fp8_run):
    x bf16 [M,K] (K % 128 == 0) -> (q float8_e4m3fn [M,K], scale float32
    [M,K/128]), x ~ q * scale per 128-element block; the pair gmm() takes as
    lhs and lhs_scale for fp8 x fp8 products."""
    lib = load()
    dev = x.device
    h = handle(dev)
    M, K = (x.shape[0], x.shape[1]) if x.dim() == 2 else (0, 0)
    if q is None:
        q = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=dev)
    if scale is None:
        scale = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
    views = [_view(t, n) for t, n in ((x, "x"), (q, "q"), (scale, "scale"))]
    st = stream if stream is not None else torch.cuda.current_stream(dev)
    _raise(lib.gmm_quant_fp8_run(h, *[_ref(v) for v in views], ctypes.c_void_p(st.cuda_stream)), h)
    return q, scale


def tgmm(lhs: torch.Tensor, rhs: torch.Tensor, group_sizes: torch.Tensor, *,
         num_active: Optional[int] = None,
         out_dtype: torch.dtype = torch.float32,
         group_offset=None,
         out: Optional[torch.Tensor] = None,
         no_alloc: bool = False,
         stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Transposed grouped matmul (the weight gradient of gmm) through
    libgmm.so: out[h] = lhs_g^T . rhs_g over the rows of group g = s + h,
    zero for an empty group.

    lhs [M,K] and rhs [M,N] bf16; group_sizes int32 [G] on the device;
    num_active Ga defaults to G minus an integer group_offset (or to G when
    the offset is a device tensor).  Returns out [Ga,K,N] of out_dtype.
    no_alloc=True calls gmm_tgmm_run_noalloc (the library's static scratch
    instead of a per-stream counter block; calls on one GPU must not
    overlap); pass `out` (and a tensor group_offset) to keep the call free of
    torch allocations too."""
    lib = load()
    dev = lhs.device
    h = handle(dev)
    if out is None:
        if num_active is None:
            s = int(group_offset) if isinstance(group_offset, int) else 0
            num_active = group_sizes.numel() - s
        out = torch.empty((num_active, lhs.shape[1], rhs.shape[1]), dtype=out_dtype, device=dev)
    views = [_view(t, n) for t, n in ((lhs, "lhs"), (rhs, "rhs"), (group_sizes, "group_sizes"), (out, "out"))]
    off_ptr, keep = _offset_ptr(group_offset, dev)
    st = stream if stream is not None else torch.cuda.current_stream(dev)
    fn = lib.gmm_tgmm_run_noalloc if no_alloc else lib.gmm_tgmm_run
    status = fn(h, *[_ref(v) for v in views[:3]], off_ptr, _ref(views[3]), ctypes.c_void_p(st.cuda_stream))
    if keep is not None and status == GMM_OK:
        keep.record_stream(st)
    _raise(status, h)
    return out


def device_flags(device=None, stream: Optional[torch.cuda.Stream] = None) -> int:
    """Synchronise the stream and return (and clear) the data-error flags."""
    lib = load()
    h = handle(device)
    st = stream if stream is not None else torch.cuda.current_stream()
    v = ctypes.c_uint32(0)
    status = lib.gmm_device_flags(h, ctypes.c_void_p(st.cuda_stream), ctypes.byref(v))
    if status not in (GMM_OK, GMM_E_DEVICE_DATA):
        _raise(status, h)
    return int(v.value)


def set_tile_policy(policy: int, device=None) -> None:
    """0 = shape-based tile choice, 1 = small tiles, 2 = big tiles."""
    lib = load()
    h = handle(device)
    _raise(lib.gmm_set_tile_policy(h, int(policy)), h)


def set_grid_limit(limit: int, device=None) -> None:
    """At most `limit` workgroups per gmm / tgmm launch (0 = the kernel's
    own choice); a test hook that makes each workgroup run many tiles."""
    lib = load()
    h = handle(device)
    _raise(lib.gmm_set_grid_limit(h, int(limit)), h)


def debug_worklist(group_sizes: torch.Tensor, num_active: int, M: int, tm: int,
                   group_offset=None, capacity: Optional[int] = None):
    """Group-aligned m-tiles as the kernels' device code builds them.

    Returns (tiles [n,3] int32 on the CPU: group, first_row, rows;
    info [4]: tile count, first active row, end of the active rows, flags)."""
    lib = load()
    dev = group_sizes.device
    h = handle(dev)
    if capacity is None:
        capacity = (M + tm - 1) // tm + group_sizes.numel() + 1
    tiles = torch.full((max(capacity, 1), 3), -1, dtype=torch.int32, device=dev)
    count = torch.zeros(4, dtype=torch.int32, device=dev)
    off_ptr, keep = _offset_ptr(group_offset, dev)
    st = torch.cuda.current_stream(dev)
    status = lib.gmm_debug_worklist(h, ctypes.byref(_view(group_sizes, "group_sizes")), off_ptr,
                                    int(num_active), int(M), int(tm), tiles.data_ptr(), int(capacity),
                                    count.data_ptr(), ctypes.c_void_p(st.cuda_stream))
    _raise(status, h)
    info = count.cpu()
    n = min(int(info[0]), capacity)
    return tiles[:n].cpu(), info
