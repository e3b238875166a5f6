"""Plain CPU oracle for the grouped matmul (gmm).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg use this package; the product library never imports, loads
or calls it, and it shares no code with the HIP path.

The arithmetic lives in ``gmm_oracle.c`` (plain loops, fp64, k ascending);
this module builds it with gcc, marshals torch CPU tensors into it, and holds
the two tile-metadata definitions in ``worklist.py``.  ``tgmm_reference`` is
the weight-gradient product (lhs_g^T . rhs_g per group).  Citations refer to the
tpu-inference 0.13.2 wheel diff page (megablox/gmm.py), the metrale
gemm_quant.rs page and the MaxText PR page "Megablox: transposed-RHS gmm_v2
kernel for the backward dlhs".

Parity pins: every function here is checked by ``tests/test_oracle_pins.py``
against closed forms, library routines and hand-worked fixtures.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np
import torch

from .worklist import group_offsets, megablox_metadata, tile_worklist  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gmm_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16, E4M3FN, E5M2, I8, I4, U4, F4E2M1 = 0, 1, 2, 3, 4, 5, 6, 7
# four-bit operands: packed bytes (uint8, or float4_e2m1fn_x2) named by format
PACKED_FORMATS = {"int4": I4, "uint4": U4, "fp4_e2m1": F4E2M1}
_DTYPE_CODE = {torch.float32: F32, torch.bfloat16: BF16, torch.float8_e4m3fn: E4M3FN, torch.float8_e5m2: E5M2,
               torch.int8: I8}

OK, E_ARG, E_DATA, E_NOMEM = 0, -1, -4, -5


class OracleError(ValueError):
    pass


def build(force: bool = True) -> str:
    """Compile gmm_oracle.c into liboracle.so with gcc (no fast-math: the
    k-ascending fp64 summation order is kept)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def set_threads(n: int) -> int:
    """Threads the oracle's parallel loops use from now on (n <= 0: keep);
    returns the count in force.  Results do not depend on it."""
    return int(_load().oracle_set_threads(int(n)))


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_decode_bf16.restype = ctypes.c_double
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_threads.restype = ctypes.c_int
        lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
        lib.oracle_decode_e4m3fn.restype = ctypes.c_double
        lib.oracle_decode_e4m3fn.argtypes = [ctypes.c_uint8]
        lib.oracle_decode_e5m2.restype = ctypes.c_double
        lib.oracle_decode_e5m2.argtypes = [ctypes.c_uint8]
        lib.oracle_decode_e2m1.restype = ctypes.c_double
        lib.oracle_decode_e2m1.argtypes = [ctypes.c_uint8]
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.oracle_round_bf16.restype = ctypes.c_uint16
        lib.oracle_round_bf16.argtypes = [ctypes.c_double]
        lib.oracle_round_bf16_array.restype = None
        lib.oracle_round_bf16_array.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        lib.oracle_round_e4m3fn.restype = ctypes.c_uint8
        lib.oracle_round_e4m3fn.argtypes = [ctypes.c_double]
        lib.oracle_widen_scales.restype = ctypes.c_int
        lib.oracle_widen_scales.argtypes = [vp, ctypes.c_int, i64, vp]
        lib.oracle_quant_fp8.restype = ctypes.c_int
        lib.oracle_quant_fp8.argtypes = [vp, i64, i64, i64, vp, vp]
        lib.oracle_tgmm.restype = ctypes.c_int
        lib.oracle_tgmm.argtypes = [vp, i32, i64, i64,
                                    vp, i32, i64,
                                    vp, i64, i64, i64,
                                    vp, vp, i64, vp]
        lib.oracle_gmm.restype = ctypes.c_int
        lib.oracle_gmm.argtypes = [vp, i32, i64, i64,
                                   vp, i32, i64, i64, i32,
                                   vp, i64, i64,
                                   vp, vp, i32,
                                   vp, i64,
                                   vp, i64,
                                   vp, vp]
        _lib = lib
    return _lib


def decode_bf16(bits: int) -> float:
    return _load().oracle_decode_bf16(bits & 0xFFFF)


def round_bf16_bits(x: float) -> int:
    return _load().oracle_round_bf16(float(x))


def decode_e4m3fn(code: int) -> float:
    return _load().oracle_decode_e4m3fn(code & 0xFF)


def decode_e5m2(code: int) -> float:
    return _load().oracle_decode_e5m2(code & 0xFF)


def decode_e2m1(nibble: int) -> float:
    return _load().oracle_decode_e2m1(nibble & 0xF)


def round_e4m3fn_code(x: float) -> int:
    """e4m3fn code nearest to x, |x| <= 448, ties to the even mantissa."""
    return _load().oracle_round_e4m3fn(float(x))


SCALE_BF16, SCALE_F32, SCALE_E8M0 = 0, 1, 2


def widen_scales_reference(src: torch.Tensor, dtype: int) -> torch.Tensor:
    """widen_block_scale_f32 (metrale gemm_quant.rs page): src [total] as bf16
    (dtype 0), f32 (1) or E8M0 bytes (2, a uint8 tensor) -> f32 [total]; E8M0
    e is 2^(e-127), with e = 0 -> 2^-127 and e = 255 -> 0.0 as the page
    states."""
    lib = _load()
    src = _cpu(src).contiguous()
    want = {SCALE_BF16: torch.bfloat16, SCALE_F32: torch.float32, SCALE_E8M0: torch.uint8}.get(dtype)
    if want is None or src.dtype != want:
        raise OracleError("source dtype does not match the dtype code")
    out = torch.empty(src.numel(), dtype=torch.float32)
    if lib.oracle_widen_scales(src.data_ptr(), dtype, src.numel(), out.data_ptr()) != OK:
        raise OracleError("invalid arguments")
    return out.view(src.shape)


def _e8m0_to_f32(t: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if t is None or t.dtype != torch.float8_e8m0fnu:
        return t
    b = t.view(torch.uint8)
    if bool((b == 255).any()):
        raise OracleError("E8M0 scale byte 255 (NaN) in a gmm block scale")
    return widen_scales_reference(b.reshape(-1), SCALE_E8M0).view(t.shape)


def quant_fp8_reference(x: torch.Tensor, blk: int = 128):
    """Per-token activation quantisation (per_token_group_quant_fp8, metrale
    gemm_quant.rs page): x bf16 [M,K] -> (q float8_e4m3fn [M,K], scale f32
    [M,K/blk]) with scale = amax/448 per block of blk (1 for an all-zero
    block) and q the nearest e4m3fn value to clamp(x/scale, +-448), both in
    binary32 (see oracle_quant_fp8 in gmm_oracle.c)."""
    lib = _load()
    x = _cpu(x)
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise OracleError("x must be a bf16 2-tensor")
    M, K = x.shape
    if blk <= 0 or K % blk:
        raise OracleError("K must be a multiple of the block")
    q = torch.empty(M, K, dtype=torch.uint8)
    scale = torch.empty(M, K // blk, dtype=torch.float32)
    rc = lib.oracle_quant_fp8(x.view(torch.int16).data_ptr(), M, K, blk, q.data_ptr(), scale.data_ptr())
    if rc != OK:
        raise OracleError("invalid arguments")
    return q.view(torch.float8_e4m3fn), scale


def _cpu(t: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if t is None:
        return None
    return t.detach().to("cpu").contiguous()


def _code(t: torch.Tensor, name: str) -> int:
    if t.dtype not in _DTYPE_CODE:
        raise OracleError(f"{name}: unsupported dtype {t.dtype}")
    return _DTYPE_CODE[t.dtype]


def gmm_reference(lhs: torch.Tensor, rhs: torch.Tensor, group_sizes: torch.Tensor, *,
                  group_offset: int = 0, transpose_rhs: bool = False,
                  rhs_scale: Optional[torch.Tensor] = None,
                  rhs_bias: Optional[torch.Tensor] = None,
                  lhs_scale: Optional[torch.Tensor] = None,
                  existing_out: Optional[torch.Tensor] = None,
                  rhs_format: Optional[str] = None,
                  lhs_format: Optional[str] = None,
                  rows: Optional[Sequence[int]] = None,
                  return_row_group: bool = False):
    """Reference rows of gmm(lhs, rhs, group_sizes, ...) in float64.

    lhs [M,K]; rhs [Ga,N,K] (transpose_rhs False) or [Ga,K,N] (True);
    group_sizes [G] int32; rhs_scale f32 [Ga,nb,1,N]; rhs_bias [Ga,1,N];
    lhs_scale f32 [M,nb].  ``rows`` selects output rows (all when None).
    rhs_format "int4", "uint4" or "fp4_e2m1": rhs holds packed bytes (uint8
    or float4_e2m1fn_x2) [Ga,N,K/2], two elements to a byte, even elements
    in the low nibble (only the [Ga,N,K] layout).  lhs_format the same for
    packed four-bit activations: lhs bytes [M,K/2] hold the [M,K] elements.
    Returns a float64 numpy array [len(rows), N] (and the group of each row,
    -1 for none, when return_row_group).

    existing_out [M,N] (gmm's existing_out, tpu-inference wheel diff page,
    megablox/gmm.py): every output tile starts as existing_out and only the
    rows of its group are stored over it, and no zero fill follows, so a row
    of no active group is existing_out's row (its exact value) instead of
    zero."""
    lib = _load()
    lhs, rhs, gs = _cpu(lhs), _cpu(rhs), _cpu(group_sizes)
    rhs_scale, rhs_bias, lhs_scale = _cpu(rhs_scale), _cpu(rhs_bias), _cpu(lhs_scale)
    # E8M0 block scales (the microscaling scale byte) are the power of two
    # the page's widening gives, 2^(e-127); byte 255 (the encoding's NaN,
    # 0.0 in the page's widening) is outside the operation
    rhs_scale, lhs_scale = _e8m0_to_f32(rhs_scale), _e8m0_to_f32(lhs_scale)
    if lhs.dim() != 2 or rhs.dim() != 3 or gs.dim() != 1 or gs.dtype != torch.int32:
        raise OracleError("bad ranks / group_sizes dtype")
    M, K = lhs.shape
    lhs_code = None
    if lhs_format is not None:
        if lhs_format not in PACKED_FORMATS or lhs.element_size() != 1:
            raise OracleError("packed four-bit lhs: a known format, bytes, [M,K/2]")
        lhs_code = PACKED_FORMATS[lhs_format]
        K = 2 * lhs.shape[1]
    Ga = rhs.shape[0]
    N = rhs.shape[2] if transpose_rhs else rhs.shape[1]
    Kr = rhs.shape[1] if transpose_rhs else rhs.shape[2]
    rhs_code = None
    if rhs_format is not None:
        if rhs_format not in PACKED_FORMATS or transpose_rhs or rhs.element_size() != 1:
            raise OracleError("packed four-bit rhs: a known format, bytes, [Ga,N,K/2]")
        rhs_code = PACKED_FORMATS[rhs_format]
        Kr = 2 * rhs.shape[2]
    if Kr != K:
        raise OracleError("lhs / rhs contraction sizes differ")
    nb = 1
    if rhs_scale is not None:
        if rhs_scale.dtype != torch.float32 or tuple(rhs_scale.shape[::2]) != (Ga, 1) \
                or rhs_scale.shape[3] != N:
            raise OracleError("rhs_scale must be f32 [Ga,nb,1,N]")
        nb = rhs_scale.shape[1]
    if lhs_scale is not None:
        if lhs_scale.dtype != torch.float32 or lhs_scale.dim() != 2 or lhs_scale.shape[0] != M:
            raise OracleError("lhs_scale must be f32 [M,nb]")
        if rhs_scale is not None and lhs_scale.shape[1] != nb:
            raise OracleError("lhs_scale and rhs_scale disagree on nb")
        nb = lhs_scale.shape[1]
    if rhs_bias is not None and tuple(rhs_bias.shape) != (Ga, 1, N):
        raise OracleError("rhs_bias must be [Ga,1,N]")
    if existing_out is not None:
        existing_out = _cpu(existing_out)
        if tuple(existing_out.shape) != (M, N):
            raise OracleError("existing_out must be [M,N]")
    if rows is None:
        rows_arr = None
        n_rows = M
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n_rows = rows_arr.shape[0]
    out = np.zeros((n_rows, N), dtype=np.float64)
    rg = np.zeros((n_rows,), dtype=np.int64)
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    rc = lib.oracle_gmm(
        ptr(lhs), _code(lhs, "lhs") if lhs_code is None else lhs_code, M, K,
        ptr(rhs), _code(rhs, "rhs") if rhs_code is None else rhs_code, Ga, N, int(bool(transpose_rhs)),
        ptr(gs), gs.shape[0], int(group_offset),
        ptr(rhs_scale), ptr(rhs_bias), _code(rhs_bias, "rhs_bias") if rhs_bias is not None else 0,
        ptr(lhs_scale), nb,
        None if rows_arr is None else rows_arr.ctypes.data, n_rows,
        out.ctypes.data, rg.ctypes.data)
    if rc != OK:
        raise OracleError({E_ARG: "invalid arguments", E_DATA: "invalid group sizes / offset",
                           E_NOMEM: "out of memory"}.get(rc, str(rc)))
    if existing_out is not None:
        ex = existing_out.double().numpy()
        ex = ex if rows_arr is None else ex[rows_arr]
        out[rg < 0] = ex[rg < 0]
    return (out, rg) if return_row_group else out


def tgmm_reference(lhs: torch.Tensor, rhs: torch.Tensor, group_sizes: torch.Tensor, *,
                   group_offset: int = 0, num_active: Optional[int] = None,
                   select: Optional[Sequence[Sequence[int]]] = None) -> np.ndarray:
    """Reference values of tgmm(lhs, rhs, group_sizes) in float64: for active
    group h (group group_offset + h), lhs_g^T . rhs_g over the group's rows,
    zero for an empty group -- the weight gradient of gmm (gmm_oracle.c,
    oracle_tgmm).

    lhs [M,K], rhs [M,N]; group_sizes [G] int32; num_active defaults to
    G - group_offset.  ``select`` is a list of (h, k) pairs (output rows);
    when None every row.  Returns float64 [Ga,K,N], or [len(select),N]."""
    lib = _load()
    lhs, rhs, gs = _cpu(lhs), _cpu(rhs), _cpu(group_sizes)
    if lhs.dim() != 2 or rhs.dim() != 2 or gs.dim() != 1 or gs.dtype != torch.int32:
        raise OracleError("bad ranks / group_sizes dtype")
    M, K = lhs.shape
    if rhs.shape[0] != M:
        raise OracleError("lhs and rhs must have the same rows")
    N = rhs.shape[1]
    G = gs.shape[0]
    Ga = G - int(group_offset) if num_active is None else int(num_active)
    if select is None:
        sh = sk = None
        out = np.zeros((Ga, K, N), dtype=np.float64)
        n_sel = Ga * K
    else:
        sel = np.ascontiguousarray(np.asarray(select, dtype=np.int64).reshape(-1, 2))
        sh = np.ascontiguousarray(sel[:, 0])
        sk = np.ascontiguousarray(sel[:, 1])
        n_sel = sel.shape[0]
        out = np.zeros((n_sel, N), dtype=np.float64)
    rc = lib.oracle_tgmm(lhs.data_ptr(), _code(lhs, "lhs"), M, K,
                         rhs.data_ptr(), _code(rhs, "rhs"), N,
                         gs.data_ptr(), G, int(group_offset), Ga,
                         None if sh is None else sh.ctypes.data, None if sk is None else sk.ctypes.data,
                         n_sel, out.ctypes.data)
    if rc != OK:
        raise OracleError({E_ARG: "invalid arguments", E_DATA: "invalid group sizes / offset",
                           E_NOMEM: "out of memory"}.get(rc, str(rc)))
    return out


def round_to(ref: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """Round float64 reference values once to the output dtype, to nearest
    with ties to even (float32: C's double->float conversion; bfloat16:
    oracle_round_bf16, which never rounds twice through float32)."""
    ref = np.ascontiguousarray(ref, dtype=np.float64)
    if dtype == torch.float32:
        return torch.from_numpy(ref.astype(np.float32))
    if dtype != torch.bfloat16:
        raise OracleError(f"unsupported output dtype {dtype}")
    bits = np.empty(ref.shape, dtype=np.uint16)
    _load().oracle_round_bf16_array(ref.ctypes.data, ref.size, bits.ctypes.data)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
