"""Python binding of libbgf.so (the C ABI in include/fp4.h).

Argument marshalling only: every step of quantize / dequantize / rotate / GEMM runs in the HIP
kernels behind the C ABI. torch supplies device memory and the current stream. If the library is
missing this module raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, replace

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbgf.so")

# enums of include/fp4.h
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_ALIGNMENT, ERR_WORKSPACE, ERR_HIP, ERR_INTERNAL = range(7)
DT_F32, DT_BF16 = 0, 1
E2M1, E4M3 = 0, 1
SCALE_E8M0_FLOOR, SCALE_E8M0_CEIL, SCALE_NV, SCALE_NV_4OVER6, SCALE_F32 = range(5)
SCALE_NV_GIVEN, SCALE_NV_4OVER6_GIVEN = 5, 6  # NVFP4 with the caller's (delayed) tensor scale
NV_MODES = (SCALE_NV, SCALE_NV_4OVER6, SCALE_NV_GIVEN, SCALE_NV_4OVER6_GIVEN)
ROUND_RNE, ROUND_SR = 0, 1


class Fp4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


class QParams(ctypes.Structure):
    _fields_ = [("elem", ctypes.c_int32), ("block_rows", ctypes.c_int32),
                ("block_cols", ctypes.c_int32), ("scale_mode", ctypes.c_int32),
                ("round_mode", ctypes.c_int32), ("hadamard_n", ctypes.c_int32),
                ("seed", ctypes.c_uint64)]


class QTensorC(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("tensor_scale", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("p", QParams)]


class QuantItemC(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("ldx", ctypes.c_int64), ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("tensor_scale", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libbgf.so. Raises if it has not been built: there is no other implementation."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python bit_gemm_fwht_amd/build.py` "
                          "(hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    QP = ctypes.POINTER(QParams)
    QT = ctypes.POINTER(QTensorC)
    L.fp4_abi_version.restype = ctypes.c_int
    L.fp4_status_string.argtypes = [ctypes.c_int]
    L.fp4_status_string.restype = ctypes.c_char_p
    for name in ("fp4_codes_bytes", "fp4_scales_bytes", "fp4_workspace_bytes"):
        getattr(L, name).argtypes = [I64, I64, QP]
        getattr(L, name).restype = I64
    L.fp4_quantize.argtypes = [P, I32, I64, I64, I64, QP, P, P, P, P, I64, P]
    L.fp4_quantize.restype = ctypes.c_int
    L.fp4_quantize_colwise.argtypes = [P, I32, I64, I64, I64, QP, P, P, P, P, I64, P]
    L.fp4_quantize_colwise.restype = ctypes.c_int
    L.fp4_quantize_batch.argtypes = [I32, ctypes.POINTER(QuantItemC), I32, QP, P]
    L.fp4_quantize_batch.restype = ctypes.c_int
    L.fp4_quantize_colwise.restype = ctypes.c_int
    L.fp4_dequantize.argtypes = [P, P, P, I64, I64, QP, P, I32, I64, P]
    L.fp4_dequantize.restype = ctypes.c_int
    L.fp4_hadamard.argtypes = [P, I32, I64, I64, I64, I32, P, P]
    L.fp4_hadamard.restype = ctypes.c_int
    L.fp4_gemm_workspace_bytes.argtypes = [QT, QT]
    L.fp4_gemm_workspace_bytes.restype = I64
    L.fp4_gemm.argtypes = [QT, QT, P, I32, I64, QP, QT, P, I64, P]
    L.fp4_gemm.restype = ctypes.c_int
    L.fp4_quantize_noalloc.argtypes = [P, I32, I64, I64, I64, QP, P, P, P, P]
    L.fp4_quantize_noalloc.restype = ctypes.c_int
    L.fp4_gemm_quantize_a_workspace_bytes.argtypes = [I64, QT]
    L.fp4_gemm_quantize_a_workspace_bytes.restype = I64
    L.fp4_gemm_quantize_a.argtypes = [P, I32, I64, I64, QP, QT, QT, P, I32, I64, P, I64, P]
    L.fp4_gemm_quantize_a.restype = ctypes.c_int
    L.fp4_transpose_2d.argtypes = [P, P, I64, I64, QP, P, P, P]
    L.fp4_transpose_2d.restype = ctypes.c_int
    L.fp4_nvfp4_to_mxfp8.argtypes = [P, P, I64, I64, P, P, P]
    L.fp4_nvfp4_to_mxfp8.restype = ctypes.c_int
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().fp4_status_string(status).decode()


def _check(status: int, what: str) -> None:
    if status != OK:
        raise Fp4Error(status, what)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DT_F32
    if t.dtype == torch.bfloat16:
        return DT_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: float32 or bfloat16")


def _stream_ptr(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


@dataclass(frozen=True)
class Params:
    elem: int = E2M1
    block: tuple = (1, 32)
    scale_mode: int = SCALE_E8M0_FLOOR
    round_mode: int = ROUND_RNE
    hadamard_n: int = 0
    seed: int = 0

    def c(self) -> QParams:
        return QParams(self.elem, self.block[0], self.block[1], self.scale_mode, self.round_mode,
                       self.hadamard_n, self.seed)


MXFP4 = Params()


@dataclass
class QTensor:
    """A quantized [rows, cols] tensor: codes, scales and (NVFP4) the fp32 tensor scale."""
    codes: torch.Tensor
    scales: torch.Tensor
    tensor_scale: torch.Tensor | None
    rows: int
    cols: int
    params: Params

    def c(self) -> QTensorC:
        ts = self.tensor_scale.data_ptr() if self.tensor_scale is not None else None
        return QTensorC(self.codes.data_ptr(), self.scales.data_ptr(), ts, self.rows, self.cols,
                        self.params.c())


def buffer_sizes(rows: int, cols: int, params: Params) -> tuple[int, int, int]:
    p = params.c()
    L = lib()
    cb = L.fp4_codes_bytes(rows, cols, ctypes.byref(p))
    sb = L.fp4_scales_bytes(rows, cols, ctypes.byref(p))
    wb = L.fp4_workspace_bytes(rows, cols, ctypes.byref(p))
    if cb < 0 or sb < 0 or wb < 0:
        # the size queries return -1 for anything fp4_quantize would reject, invalid or unsupported
        raise Fp4Error(ERR_INVALID_ARG, f"quantize params {params} for shape ({rows}, {cols}) are rejected "
                       "(invalid, or not supported: e.g. 1D groups need cols % 32 == 0)")
    return cb, sb, wb


def empty_qtensor(rows: int, cols: int, params: Params, device) -> QTensor:
    cb, sb, _ = buffer_sizes(rows, cols, params)
    codes = torch.empty(max(cb, 1), dtype=torch.uint8, device=device)
    scales = torch.empty(max(sb, 1), dtype=torch.uint8, device=device)
    nv = params.scale_mode in NV_MODES
    ts = torch.empty(1, dtype=torch.float32, device=device) if nv else None
    return QTensor(codes, scales, ts, rows, cols, params)


def _set_given_scale(q: QTensor, params: Params, tensor_scale) -> None:
    """The _GIVEN NVFP4 modes read g from the output's tensor-scale buffer."""
    if params.scale_mode in (SCALE_NV_GIVEN, SCALE_NV_4OVER6_GIVEN):
        if tensor_scale is None:
            raise ValueError("the _GIVEN scale modes need tensor_scale (the fp32 g)")
        if isinstance(tensor_scale, torch.Tensor):
            if tensor_scale.data_ptr() != q.tensor_scale.data_ptr():  # else g is in place already
                q.tensor_scale.copy_(tensor_scale.reshape(1))
        else:
            q.tensor_scale.fill_(float(tensor_scale))


def _on(dev, *ts) -> None:
    """Every buffer handed to the library must be device memory of the device the call runs on."""
    for t in ts:
        if t is not None and (not t.is_cuda or t.device != dev):
            raise ValueError(f"a buffer on {t.device} was passed to a call that runs on {dev}")


def _check_q(q: QTensor, rows: int, cols: int, params: Params, dev, what: str) -> None:
    """q's buffers hold at least what a rows x cols tensor quantized with params takes."""
    cb, sb, _ = buffer_sizes(rows, cols, params)
    for t, need, name in ((q.codes, cb, "codes"), (q.scales, sb, "scales")):
        if not t.is_contiguous() or t.numel() * t.element_size() < need:
            raise ValueError(f"{what}.{name} must be contiguous and hold at least {need} bytes")
        _on(dev, t)
    if params.scale_mode in NV_MODES:
        if q.tensor_scale is None or q.tensor_scale.dtype != torch.float32 or q.tensor_scale.numel() < 1:
            raise ValueError(f"{what} needs a one-element float32 tensor_scale buffer")
        _on(dev, q.tensor_scale)


def _ws_bytes(ws: torch.Tensor | None, need: int, dev) -> int:
    if ws is None:
        return 0
    _on(dev, ws)
    nb = ws.numel() * ws.element_size()
    if not ws.is_contiguous() or nb < need:
        raise ValueError(f"workspace must be contiguous and hold at least {need} bytes")
    return nb


def quantize(x: torch.Tensor, params: Params = MXFP4, out: QTensor | None = None,
             workspace: torch.Tensor | None = None, tensor_scale=None) -> QTensor:
    """Quantize a 2-D float32 / bfloat16 CUDA tensor along its last axis. tensor_scale: g for the
    _GIVEN NVFP4 modes (a float or a one-element device tensor)."""
    if x.dim() != 2 or not x.is_cuda:
        raise ValueError("x must be a 2-D CUDA tensor")
    if x.stride(1) != 1:
        raise ValueError("x must be contiguous along its last axis")
    rows, cols = x.shape
    if out is not None:
        _check_q(out, rows, cols, params, x.device, "out")
    q = out if out is not None else empty_qtensor(rows, cols, params, x.device)
    _set_given_scale(q, params, tensor_scale)
    _, _, wb = buffer_sizes(rows, cols, params)
    if wb and workspace is None:
        workspace = torch.empty(wb, dtype=torch.uint8, device=x.device)
    wsb = _ws_bytes(workspace, wb, x.device)
    p = params.c()
    ts = q.tensor_scale.data_ptr() if q.tensor_scale is not None else None
    st = lib().fp4_quantize(x.data_ptr(), _dtype_code(x), rows, cols, x.stride(0), ctypes.byref(p),
                            q.codes.data_ptr(), q.scales.data_ptr(), ts,
                            workspace.data_ptr() if workspace is not None else None, wsb,
                            _stream_ptr(x.device))
    _check(st, "fp4_quantize")
    q.rows, q.cols, q.params = rows, cols, params  # a reused out now describes this tensor
    return q


def quantize_noalloc(x: torch.Tensor, params: Params, out: QTensor, tensor_scale=None) -> QTensor:
    """fp4_quantize_noalloc: quantize into the preallocated `out` with no device allocation at all (the
    tensor-amax scratch is the library's static per-GPU array; overlapping calls on one GPU race)."""
    if x.dim() != 2 or not x.is_cuda or x.stride(1) != 1:
        raise ValueError("x must be a 2-D CUDA tensor, contiguous along its last axis")
    rows, cols = x.shape
    _check_q(out, rows, cols, params, x.device, "out")
    _set_given_scale(out, params, tensor_scale)
    p = params.c()
    ts = out.tensor_scale.data_ptr() if out.tensor_scale is not None else None
    st = lib().fp4_quantize_noalloc(x.data_ptr(), _dtype_code(x), rows, cols, x.stride(0), ctypes.byref(p),
                                    out.codes.data_ptr(), out.scales.data_ptr(), ts, _stream_ptr(x.device))
    _check(st, "fp4_quantize_noalloc")
    out.rows, out.cols, out.params = rows, cols, params
    return out


def quantize_batch(xs, params: Params = MXFP4, outs=None, tensor_scales=None) -> list:
    """Quantize up to four 2-D CUDA tensors of one dtype with the same params in one launch (the
    same codes and scales as quantize() of each). tensor_scales: per-tensor g for the _GIVEN
    NVFP4 modes."""
    n = len(xs)
    if n == 0:
        return []
    outs = list(outs) if outs is not None else [None] * n
    tss = list(tensor_scales) if tensor_scales is not None else [None] * n
    items = (QuantItemC * n)()
    qs = []
    for i, x in enumerate(xs):
        if x.dim() != 2 or not x.is_cuda or x.stride(1) != 1:
            raise ValueError("each x must be a 2-D CUDA tensor, contiguous along its last axis")
        if x.dtype != xs[0].dtype:
            raise ValueError("all tensors of a batch share one dtype")
        _on(xs[0].device, x)
        rows, cols = x.shape
        if outs[i] is not None:
            _check_q(outs[i], rows, cols, params, x.device, f"outs[{i}]")
        q = outs[i] if outs[i] is not None else empty_qtensor(rows, cols, params, x.device)
        _set_given_scale(q, params, tss[i])
        ts = q.tensor_scale.data_ptr() if q.tensor_scale is not None else None
        items[i] = QuantItemC(x.data_ptr(), rows, cols, x.stride(0), q.codes.data_ptr(), q.scales.data_ptr(), ts)
        qs.append(q)
    p = params.c()
    st = lib().fp4_quantize_batch(n, items, _dtype_code(xs[0]), ctypes.byref(p), _stream_ptr(xs[0].device))
    _check(st, "fp4_quantize_batch")
    for q, x in zip(qs, xs):
        q.rows, q.cols, q.params = x.shape[0], x.shape[1], params
    return qs


def quantize_colwise(x: torch.Tensor, params: Params = MXFP4, out: QTensor | None = None,
                     workspace: torch.Tensor | None = None, tensor_scale=None) -> QTensor:
    """Quantize x^T (shape [cols, rows]) along its last axis, i.e. x along its first axis, without
    forming the transpose. Returns the QTensor of the cols x rows tensor."""
    if x.dim() != 2 or not x.is_cuda:
        raise ValueError("x must be a 2-D CUDA tensor")
    if x.stride(1) != 1:
        raise ValueError("x must be contiguous along its last axis")
    rows, cols = x.shape
    if out is not None:
        _check_q(out, cols, rows, params, x.device, "out")
    q = out if out is not None else empty_qtensor(cols, rows, params, x.device)
    _set_given_scale(q, params, tensor_scale)
    _, _, wb = buffer_sizes(cols, rows, params)
    if wb and workspace is None:
        workspace = torch.empty(wb, dtype=torch.uint8, device=x.device)
    wsb = _ws_bytes(workspace, wb, x.device)
    p = params.c()
    ts = q.tensor_scale.data_ptr() if q.tensor_scale is not None else None
    st = lib().fp4_quantize_colwise(x.data_ptr(), _dtype_code(x), rows, cols, x.stride(0),
                                    ctypes.byref(p), q.codes.data_ptr(), q.scales.data_ptr(), ts,
                                    workspace.data_ptr() if workspace is not None else None, wsb,
                                    _stream_ptr(x.device))
    _check(st, "fp4_quantize_colwise")
    q.rows, q.cols, q.params = cols, rows, params
    return q


def dequantize(q: QTensor, dtype=torch.float32, out: torch.Tensor | None = None) -> torch.Tensor:
    """Decode q to float32 / bfloat16 [rows, cols] (out: any row pitch >= cols)."""
    dev = q.codes.device
    _check_q(q, q.rows, q.cols, q.params, dev, "q")
    if out is not None:
        _on(dev, out)
        if out.dim() != 2 or tuple(out.shape) != (q.rows, q.cols) or out.stride(1) != 1 or out.stride(0) < q.cols:
            raise ValueError(f"out must be a row-major [{q.rows}, {q.cols}] tensor")
    y = out if out is not None else torch.empty(q.rows, q.cols, dtype=dtype, device=dev)
    p = q.params.c()
    ts = q.tensor_scale.data_ptr() if q.tensor_scale is not None else None
    st = lib().fp4_dequantize(q.codes.data_ptr(), q.scales.data_ptr(), ts, q.rows, q.cols,
                              ctypes.byref(p), y.data_ptr(), _dtype_code(y), y.stride(0),
                              _stream_ptr(y.device))
    _check(st, "fp4_dequantize")
    return y


def hadamard(x: torch.Tensor, n: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """Blockwise H_n / sqrt(n) along the last axis (fp32 result, contiguous)."""
    if x.dim() != 2 or not x.is_cuda or x.stride(1) != 1:
        raise ValueError("x must be a 2-D CUDA tensor, contiguous along its last axis")
    rows, cols = x.shape
    if out is not None:
        _on(x.device, out)
        if out.dtype != torch.float32 or tuple(out.shape) != (rows, cols) or not out.is_contiguous():
            raise ValueError(f"out must be a contiguous float32 [{rows}, {cols}] tensor")
    y = out if out is not None else torch.empty(rows, cols, dtype=torch.float32, device=x.device)
    st = lib().fp4_hadamard(x.data_ptr(), _dtype_code(x), rows, cols, x.stride(0), n, y.data_ptr(),
                            _stream_ptr(x.device))
    _check(st, "fp4_hadamard")
    return y


def gemm_workspace_bytes(a: QTensor, b: QTensor) -> int:
    ac, bc = a.c(), b.c()
    n = lib().fp4_gemm_workspace_bytes(ctypes.byref(ac), ctypes.byref(bc))
    if n < 0:
        raise Fp4Error(ERR_UNSUPPORTED, "fp4_gemm_workspace_bytes")
    return n


def gemm(a: QTensor, b: QTensor, out_dtype=torch.bfloat16, out: torch.Tensor | None = None,
         workspace: torch.Tensor | None = None, out_q: Params | None = None,
         q_out: QTensor | None = None, keep_c: bool = True, use_workspace: bool = True):
    """C [M, N] = A [M, K] * B [N, K]^T on quantized operands (fp32 accumulation).

    With out_q (MX groups of 32 along N, E8M0 floor / ceil, RNE or SR, optionally rotated along N
    with out_q.hadamard_n <= 128), C is also quantized in the epilogue and (C, C_q) is returned;
    keep_c=False skips writing C and returns (None, C_q). out may be a column block of a wider
    row-major buffer (its row pitch is passed as ldc). use_workspace=False passes no workspace: NVFP4
    operands (M, N >= 256, K % 128 == 0) then take the route that re-expresses them as FP8 in LDS."""
    dev = a.codes.device
    if out is not None:
        if out.dim() != 2 or tuple(out.shape) != (a.rows, b.rows) or out.device != dev:
            raise ValueError(f"out must be a [{a.rows}, {b.rows}] tensor on {dev}")
        if out.stride(1) != 1 or out.stride(0) < b.rows:
            raise ValueError("out must be row-major: unit column stride, row pitch >= N")
    _check_q(a, a.rows, a.cols, a.params, dev, "a")
    _check_q(b, b.rows, b.cols, b.params, dev, "b")
    c = None
    if out_q is None or keep_c:
        c = out if out is not None else torch.empty(a.rows, b.rows, dtype=out_dtype, device=dev)
    wb = gemm_workspace_bytes(a, b) if use_workspace else 0
    if not use_workspace:
        workspace = None
    if wb and workspace is None:
        workspace = torch.empty(wb, dtype=torch.uint8, device=dev)
    ac, bc = a.c(), b.c()
    qp = qc = None
    if out_q is not None:
        if q_out is None:
            q_out = empty_qtensor(a.rows, b.rows, out_q, dev)
        else:
            _check_q(q_out, a.rows, b.rows, out_q, dev, "q_out")
        qp = out_q.c()
        qc = q_out.c()
    st = lib().fp4_gemm(ctypes.byref(ac), ctypes.byref(bc), c.data_ptr() if c is not None else None,
                        _dtype_code(c) if c is not None else 0, c.stride(0) if c is not None else 0,
                        ctypes.byref(qp) if qp is not None else None,
                        ctypes.byref(qc) if qc is not None else None,
                        workspace.data_ptr() if workspace is not None else None,
                        _ws_bytes(workspace, wb, dev), _stream_ptr(dev))
    _check(st, "fp4_gemm")
    if out_q is not None:
        q_out.rows, q_out.cols, q_out.params, q_out.tensor_scale = a.rows, b.rows, out_q, None
        return c, q_out
    return c


def transpose_2d(q: QTensor, out: QTensor | None = None) -> QTensor:
    """The quantized transpose [cols, rows] of a tensor quantized with 32 x 32 blocks (a re-layout:
    the same codes and scales fp4_quantize gives the transposed tensor)."""
    dev = q.codes.device
    _check_q(q, q.rows, q.cols, q.params, dev, "q")
    if out is not None:
        _check_q(out, q.cols, q.rows, q.params, dev, "out")
    t = out if out is not None else empty_qtensor(q.cols, q.rows, q.params, dev)
    p = q.params.c()
    st = lib().fp4_transpose_2d(q.codes.data_ptr(), q.scales.data_ptr(), q.rows, q.cols, ctypes.byref(p),
                                t.codes.data_ptr(), t.scales.data_ptr(), _stream_ptr(dev))
    _check(st, "fp4_transpose_2d")
    t.rows, t.cols, t.params = q.cols, q.rows, q.params
    return t


def nvfp4_to_mxfp8(q: QTensor) -> QTensor:
    """The FP8 re-expression of an NVFP4 tensor (E4M3 elements, one E8M0 scale per 32 along the
    rows), the operand form the GEMM multiplies NVFP4 operands in. The result's tensor_scale is q's
    (it still multiplies the product)."""
    if q.params.scale_mode not in NV_MODES:
        raise ValueError("nvfp4_to_mxfp8 takes an NVFP4 tensor")
    dev = q.codes.device
    _check_q(q, q.rows, q.cols, q.params, dev, "q")
    p8 = Params(elem=E4M3, block=(1, 32), scale_mode=SCALE_E8M0_FLOOR)
    cb, sb, _ = buffer_sizes(q.rows, q.cols, p8)
    codes = torch.empty(cb, dtype=torch.uint8, device=dev)
    scales = torch.empty(sb, dtype=torch.uint8, device=dev)
    st = lib().fp4_nvfp4_to_mxfp8(q.codes.data_ptr(), q.scales.data_ptr(), q.rows, q.cols, codes.data_ptr(),
                                  scales.data_ptr(), _stream_ptr(dev))
    _check(st, "fp4_nvfp4_to_mxfp8")
    return QTensor(codes, scales, q.tensor_scale, q.rows, q.cols, p8)


def gemm_quantize_a(x: torch.Tensor, params: Params, b: QTensor, out_dtype=torch.bfloat16,
                    out: torch.Tensor | None = None, a_out: QTensor | None = None,
                    workspace: torch.Tensor | None = None):
    """C = quantize(x) * B^T with x's rotation and MXFP4 quantization fused into the GEMM launch.
    Returns (C, A_q), A_q the quantized x (the same codes and scales quantize() gives)."""
    if x.dim() != 2 or not x.is_cuda or x.stride(1) != 1:
        raise ValueError("x must be a 2-D CUDA tensor, contiguous along its last axis")
    dev = x.device
    M, K = x.shape
    if K != b.cols:
        raise ValueError(f"x has {K} columns, B has {b.cols}")
    _check_q(b, b.rows, b.cols, b.params, dev, "b")
    if a_out is not None:
        _check_q(a_out, M, K, params, dev, "a_out")
    aq = a_out if a_out is not None else empty_qtensor(M, K, params, dev)
    if out is not None:
        if out.dim() != 2 or tuple(out.shape) != (M, b.rows) or out.device != dev or out.stride(1) != 1 \
                or out.stride(0) < b.rows:
            raise ValueError(f"out must be a row-major [{M}, {b.rows}] tensor on {dev}")
    c = out if out is not None else torch.empty(M, b.rows, dtype=out_dtype, device=dev)
    bc = b.c()
    wb = lib().fp4_gemm_quantize_a_workspace_bytes(M, ctypes.byref(bc))
    if wb < 0:
        raise Fp4Error(ERR_INVALID_ARG, "fp4_gemm_quantize_a_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(wb, dtype=torch.uint8, device=dev)
    wsb = _ws_bytes(workspace, wb, dev)
    p = params.c()
    ac = aq.c()
    st = lib().fp4_gemm_quantize_a(x.data_ptr(), _dtype_code(x), M, x.stride(0), ctypes.byref(p), ctypes.byref(ac),
                                   ctypes.byref(bc), c.data_ptr(), _dtype_code(c), c.stride(0),
                                   workspace.data_ptr(), wsb, _stream_ptr(dev))
    _check(st, "fp4_gemm_quantize_a")
    aq.rows, aq.cols, aq.params, aq.tensor_scale = M, K, params, None
    return c, aq


def upload_qtensor(codes, scales, tensor_scale, rows, cols, params: Params, device) -> QTensor:
    """Wrap host arrays (numpy) of an already-quantized tensor as a device QTensor."""
    import numpy as np
    ct = torch.from_numpy(np.ascontiguousarray(codes).reshape(-1).view(np.uint8)).to(device)
    st = torch.from_numpy(np.ascontiguousarray(scales).reshape(-1).view(np.uint8)).to(device)
    ts = None
    if tensor_scale is not None:
        ts = torch.from_numpy(np.ascontiguousarray(tensor_scale, dtype=np.float32).reshape(1)).to(device)
    return QTensor(ct, st, ts, rows, cols, params)


def with_params(q: QTensor, **kw) -> QTensor:
    return QTensor(q.codes, q.scales, q.tensor_scale, q.rows, q.cols, replace(q.params, **kw))
