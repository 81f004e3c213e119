"""Python view of the CPU oracle (liboracle.so, plain C in oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module; the product package never does. It shares no code with the HIP library.

Arrays are numpy; everything is computed by the C functions one element at a time. See oracle.h for
the sources (cited by page title and section) and the arithmetic conventions.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

E2M1, E4M3 = 0, 1
SCALE_E8M0_FLOOR, SCALE_E8M0_CEIL, SCALE_NV, SCALE_NV_4OVER6, SCALE_F32 = 0, 1, 2, 3, 4
SCALE_NV_GIVEN, SCALE_NV_4OVER6_GIVEN = 5, 6  # NVFP4 with the caller's tensor scale
NV_MODES = (SCALE_NV, SCALE_NV_4OVER6, SCALE_NV_GIVEN, SCALE_NV_4OVER6_GIVEN)
ROUND_RNE, ROUND_SR = 0, 1
IN_F32, IN_BF16 = 0, 1

_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int
_U64 = ctypes.c_uint64


def lib() -> ctypes.CDLL:
    """Load liboracle.so, building it with gcc first if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        _build.build()
    L = ctypes.CDLL(_build.LIB)
    L.orc_e2m1_rne.argtypes = [ctypes.c_float]
    L.orc_e2m1_rne.restype = ctypes.c_uint8
    L.orc_e2m1_value.argtypes = [ctypes.c_uint8]
    L.orc_e2m1_value.restype = ctypes.c_float
    L.orc_e4m3_rne.argtypes = [ctypes.c_float]
    L.orc_e4m3_rne.restype = ctypes.c_uint8
    L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
    L.orc_e4m3_value.restype = ctypes.c_float
    L.orc_e8m0_value.argtypes = [ctypes.c_uint8]
    L.orc_e8m0_value.restype = ctypes.c_float
    L.orc_e8m0_scale_exp.argtypes = [ctypes.c_float, _INT, _INT]
    L.orc_e8m0_scale_exp.restype = _INT
    L.orc_sr_u16.argtypes = [_U64, _U64]
    L.orc_sr_u16.restype = ctypes.c_uint32
    L.orc_fwht.argtypes = [_P, _I64, _INT]
    L.orc_fwht.restype = _INT
    L.orc_quantize.argtypes = [_P, _INT, _I64, _I64, _INT, _INT, _INT, _INT, _INT, _INT, _U64,
                               _P, _P, _P]
    L.orc_quantize.restype = _INT
    L.orc_dequantize.argtypes = [_P, _P, _P, _I64, _I64, _INT, _INT, _INT, _INT, _INT, _P]
    L.orc_dequantize.restype = _INT
    L.orc_operand_f64.argtypes = [_P, _P, _P, _I64, _I64, _INT, _INT, _INT, _INT, _INT, _P]
    L.orc_operand_f64.restype = _INT
    L.orc_nv_to_mx8.argtypes = [_P, _P, _I64, _I64, _INT, _P, _P]
    L.orc_nv_to_mx8.restype = _INT
    L.orc_gemm_f64.argtypes = [_P, _P, _I64, _I64, _I64, _P, _P]
    L.orc_gemm_f64.restype = None
    L.orc_gemm_f64_sampled.argtypes = [_P, _P, _I64, _P, _P, _I64, _P, _P]
    L.orc_gemm_f64_sampled.restype = None
    L.orc_encode_array.argtypes = [_P, _I64, _INT, _INT, _U64, _U64, _P]
    L.orc_encode_array.restype = None
    L.orc_decode_array.argtypes = [_P, _I64, _INT, _P]
    L.orc_decode_array.restype = None
    L.orc_sr_u16_array.argtypes = [_U64, _P, _I64, _P]
    L.orc_sr_u16_array.restype = None
    L.orc_philox_array.argtypes = [_P, _P, _I64, _P]
    L.orc_philox_array.restype = None
    L.orc_bf16_array.argtypes = [_P, _I64, _P]
    L.orc_bf16_array.restype = None
    L.orc_sr_with_u_array.argtypes = [_P, _P, _I64, _INT, _P]
    L.orc_sr_with_u_array.restype = None
    _lib = L
    return L


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---- element formats ---------------------------------------------------------------------------
def encode(v, elem=E2M1, round_mode=ROUND_RNE, seed=0, idx0=0) -> np.ndarray:
    """Codes of the fp32 values v (element i uses SR index idx0 + i)."""
    v = _c(v, np.float32).ravel()
    out = np.empty(v.size, dtype=np.uint8)
    lib().orc_encode_array(_ptr(v), v.size, elem, round_mode, seed, idx0, _ptr(out))
    return out


def sr_with_u(v, u16, elem=E2M1) -> np.ndarray:
    """Stochastic rounding of v[i] with the given 16-bit uniforms u16[i]."""
    v = _c(v, np.float32).ravel()
    u16 = _c(u16, np.uint32).ravel()
    out = np.empty(v.size, dtype=np.uint8)
    lib().orc_sr_with_u_array(_ptr(v), _ptr(u16), v.size, elem, _ptr(out))
    return out


def decode(q, elem=E2M1) -> np.ndarray:
    q = _c(q, np.uint8).ravel()
    out = np.empty(q.size, dtype=np.float32)
    lib().orc_decode_array(_ptr(q), q.size, elem, _ptr(out))
    return out


def e8m0_value(code: int) -> float:
    return lib().orc_e8m0_value(code)


def e8m0_scale_exp(amax: float, elem=E2M1, rule=SCALE_E8M0_FLOOR) -> int:
    return lib().orc_e8m0_scale_exp(amax, elem, rule)


def bf16_rne(v) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    v = _c(v, np.float32)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().orc_bf16_array(_ptr(v), v.size, _ptr(out))
    return out


# ---- random bits --------------------------------------------------------------------------------
def philox(ctr, key) -> np.ndarray:
    """Philox4x32-10 on rows of ctr [n, 4] and key [n, 2] (uint32)."""
    ctr = _c(ctr, np.uint32).reshape(-1, 4)
    key = _c(key, np.uint32).reshape(-1, 2)
    out = np.empty_like(ctr)
    lib().orc_philox_array(_ptr(ctr), _ptr(key), ctr.shape[0], _ptr(out))
    return out


def sr_u16(seed: int, idx) -> np.ndarray:
    idx = _c(idx, np.uint64).ravel()
    out = np.empty(idx.size, dtype=np.uint32)
    lib().orc_sr_u16_array(seed, _ptr(idx), idx.size, _ptr(out))
    return out


# ---- rotation -----------------------------------------------------------------------------------
def fwht(x, n: int) -> np.ndarray:
    """Blockwise H_n / sqrt(n) along the last axis, fp32, in the butterfly stage order."""
    y = np.array(x, dtype=np.float32, copy=True, order="C")
    rc = lib().orc_fwht(_ptr(y), y.size, n)
    if rc:
        raise ValueError(f"orc_fwht rejected n={n} for shape {y.shape}")
    return y


# ---- quantize / dequantize ---------------------------------------------------------------------
def scales_shape(rows, cols, block):
    return (rows // block[0], cols // block[1])


def quantize(x, *, elem=E2M1, block=(1, 32), scale_mode=SCALE_E8M0_FLOOR, round_mode=ROUND_RNE,
             hadamard_n=0, seed=0, tensor_scale=None):
    """Quantize a 2-D array along its last (contiguous) axis.

    x: float32 array, or uint16 array holding bf16 bit patterns. tensor_scale: the given g of the
    SCALE_NV*_GIVEN modes.
    Returns (codes uint8, scales uint8 or float32, tensor_scale float32 or None)."""
    x = np.asarray(x)
    if x.ndim != 2:
        raise ValueError("x must be 2-D")
    rows, cols = x.shape
    if x.dtype == np.uint16:
        xd, dt = _c(x, np.uint16), IN_BF16
    else:
        xd, dt = _c(x, np.float32), IN_F32
    codes = np.zeros((rows, cols // 2) if elem == E2M1 else (rows, cols), dtype=np.uint8)
    sdt = np.float32 if scale_mode == SCALE_F32 else np.uint8
    scales = np.zeros(scales_shape(rows, cols, block), dtype=sdt)
    ts = np.zeros(1, dtype=np.float32)
    if scale_mode in (SCALE_NV_GIVEN, SCALE_NV_4OVER6_GIVEN):
        if tensor_scale is None:
            raise ValueError("the _GIVEN modes need tensor_scale")
        ts[0] = np.float32(tensor_scale)
    rc = lib().orc_quantize(_ptr(xd), dt, rows, cols, elem, block[0], block[1], scale_mode,
                            round_mode, hadamard_n, seed, _ptr(codes), _ptr(scales), _ptr(ts))
    if rc:
        raise ValueError(f"orc_quantize rejected the arguments (code {rc})")
    nv = scale_mode in NV_MODES
    return codes, scales, (ts if nv else None)


def dequantize(codes, scales, tensor_scale, rows, cols, *, elem=E2M1, block=(1, 32),
               scale_mode=SCALE_E8M0_FLOOR, hadamard_n=0) -> np.ndarray:
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.float32 if scale_mode == SCALE_F32 else np.uint8)
    ts = None if tensor_scale is None else _c(tensor_scale, np.float32)
    y = np.empty((rows, cols), dtype=np.float32)
    rc = lib().orc_dequantize(_ptr(codes), _ptr(scales), _ptr(ts), rows, cols, elem, block[0],
                              block[1], scale_mode, hadamard_n, _ptr(y))
    if rc:
        raise ValueError(f"orc_dequantize rejected the arguments (code {rc})")
    return y


def operand_f64(codes, scales, tensor_scale, rows, K, *, elem=E2M1, block=(1, 32),
                scale_mode=SCALE_E8M0_FLOOR, nv_exact=False) -> np.ndarray:
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.float32 if scale_mode == SCALE_F32 else np.uint8)
    ts = None if tensor_scale is None else _c(tensor_scale, np.float32)
    out = np.empty((rows, K), dtype=np.float64)
    rc = lib().orc_operand_f64(_ptr(codes), _ptr(scales), _ptr(ts), rows, K, elem, block[0],
                               block[1], scale_mode, int(nv_exact), _ptr(out))
    if rc:
        raise ValueError(f"orc_operand_f64 rejected the arguments (code {rc})")
    return out


def nv_to_mx8(codes, scales, rows, K, block_cols=16):
    """The FP8 re-expression of an NVFP4 operand: (E4M3 codes [rows, K], E8M0 codes [rows, K/32])."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    f8 = np.empty((rows, K), dtype=np.uint8)
    e8 = np.empty((rows, K // 32), dtype=np.uint8)
    rc = lib().orc_nv_to_mx8(_ptr(codes), _ptr(scales), rows, K, block_cols, _ptr(f8), _ptr(e8))
    if rc:
        raise ValueError(f"orc_nv_to_mx8 rejected the arguments (code {rc})")
    return f8, e8


def gemm_f64(a, b):
    """C = a @ b.T in fp64 plus the per-output sum of |products|."""
    a = _c(a, np.float64)
    b = _c(b, np.float64)
    M, K = a.shape
    N = b.shape[0]
    c = np.empty((M, N), dtype=np.float64)
    s = np.empty((M, N), dtype=np.float64)
    lib().orc_gemm_f64(_ptr(a), _ptr(b), M, N, K, _ptr(c), _ptr(s))
    return c, s


def gemm_f64_sampled(a, b, ms, ns):
    a = _c(a, np.float64)
    b = _c(b, np.float64)
    ms = _c(ms, np.int64)
    ns = _c(ns, np.int64)
    c = np.empty(ms.size, dtype=np.float64)
    s = np.empty(ms.size, dtype=np.float64)
    lib().orc_gemm_f64_sampled(_ptr(a), _ptr(b), a.shape[1], _ptr(ms), _ptr(ns), ms.size,
                               _ptr(c), _ptr(s))
    return c, s
