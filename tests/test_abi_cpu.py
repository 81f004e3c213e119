"""CPU checks of the C ABI library: it loads without a GPU, exports every entry point the header
declares, and rejects bad arguments on the host before touching the device. Also checks that the
oracle and the HIP path share no code."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def fp4():
    from bit_gemm_fwht_amd import fp4 as m
    if not os.path.exists(m.LIB_PATH):
        from bit_gemm_fwht_amd import build
        build.build()
    m.lib()
    return m


def _declared():
    src = open(os.path.join(ROOT, "include", "fp4.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fp4_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(fp4):
    names = _declared()
    assert {"fp4_quantize", "fp4_dequantize", "fp4_gemm", "fp4_hadamard"} <= set(names)
    L = fp4.lib()
    for n in names:
        assert hasattr(L, n), n
    assert L.fp4_abi_version() == 1


def test_status_strings(fp4):
    for s in range(7):
        assert fp4.status_string(s)


def P(fp4, **kw):
    base = dict(elem=0, block_rows=1, block_cols=32, scale_mode=0, round_mode=0, hadamard_n=0, seed=0)
    base.update(kw)
    return fp4.QParams(**base)


def test_size_queries(fp4):
    L = fp4.lib()
    p = P(fp4)
    assert L.fp4_codes_bytes(4096, 4096, ctypes.byref(p)) == 4096 * 2048
    assert L.fp4_scales_bytes(4096, 4096, ctypes.byref(p)) == 4096 * 128
    assert L.fp4_workspace_bytes(4096, 4096, ctypes.byref(p)) == 0
    nv = P(fp4, block_cols=16, scale_mode=3)
    assert L.fp4_scales_bytes(64, 256, ctypes.byref(nv)) == 64 * 16
    assert L.fp4_workspace_bytes(64, 256, ctypes.byref(nv)) == 256
    p2d = P(fp4, block_rows=32, scale_mode=1)
    assert L.fp4_scales_bytes(4096, 4096, ctypes.byref(p2d)) == 128 * 128
    f8 = P(fp4, elem=1)
    assert L.fp4_codes_bytes(8, 64, ctypes.byref(f8)) == 8 * 64
    f32s = P(fp4, block_rows=256, block_cols=784, scale_mode=4)
    assert L.fp4_scales_bytes(256, 784, ctypes.byref(f32s)) == 4
    # rejected shapes
    assert L.fp4_codes_bytes(4, 33, ctypes.byref(p)) == -1            # cols % 32
    assert L.fp4_codes_bytes(4, 64, ctypes.byref(P(fp4, hadamard_n=48))) == -1
    assert L.fp4_codes_bytes(4, 64, ctypes.byref(P(fp4, block_rows=32))) == -1  # rows % 32
    assert L.fp4_codes_bytes(0, 64, ctypes.byref(p)) == -1


def _quant(fp4, p, rows=64, cols=256, x=0x1000, codes=0x2000, scales=0x3000, ts=None, ws=None,
           wsb=0, ldx=None, dtype=1):
    return fp4.lib().fp4_quantize(x, dtype, rows, cols, ldx or cols, ctypes.byref(p), codes, scales,
                                  ts, ws, wsb, None)


def test_quantize_validation_without_device(fp4):
    """Every one of these returns before any HIP call (the pointers are never touched)."""
    E = fp4
    assert _quant(fp4, P(fp4), x=None) == E.ERR_INVALID_ARG
    assert _quant(fp4, P(fp4), codes=None) == E.ERR_INVALID_ARG
    assert _quant(fp4, P(fp4), cols=250) == E.ERR_INVALID_ARG
    assert _quant(fp4, P(fp4, elem=7)) == E.ERR_INVALID_ARG
    assert _quant(fp4, P(fp4, scale_mode=9)) == E.ERR_INVALID_ARG
    assert _quant(fp4, P(fp4, round_mode=3)) == E.ERR_INVALID_ARG
    assert _quant(fp4, P(fp4, hadamard_n=512)) == E.ERR_INVALID_ARG
    assert _quant(fp4, P(fp4, hadamard_n=128), cols=320) == E.ERR_INVALID_ARG
    assert _quant(fp4, P(fp4, block_cols=64)) == E.ERR_UNSUPPORTED
    assert _quant(fp4, P(fp4, scale_mode=3, round_mode=1, block_cols=16), ts=0x4000, ws=0x5000,
                  wsb=256) == E.ERR_UNSUPPORTED                       # SR with 4/6
    assert _quant(fp4, P(fp4, scale_mode=2)) == E.ERR_UNSUPPORTED        # NV needs 16-blocks
    assert _quant(fp4, P(fp4, scale_mode=2, block_cols=16)) == E.ERR_INVALID_ARG  # no tensor_scale
    assert _quant(fp4, P(fp4, scale_mode=2, block_cols=16), ts=0x4000) == E.ERR_WORKSPACE
    assert _quant(fp4, P(fp4, scale_mode=2, block_cols=16), ts=0x4000, ws=0x5000, wsb=8) == E.ERR_WORKSPACE
    assert _quant(fp4, P(fp4, block_rows=32, scale_mode=4)) == E.ERR_UNSUPPORTED  # 2D needs E8M0
    assert _quant(fp4, P(fp4, block_rows=64, block_cols=256, hadamard_n=16)) == E.ERR_UNSUPPORTED
    assert _quant(fp4, P(fp4), x=0x1004) == E.ERR_ALIGNMENT
    assert _quant(fp4, P(fp4), codes=0x2008) == E.ERR_ALIGNMENT
    assert _quant(fp4, P(fp4), ldx=260) == E.ERR_ALIGNMENT             # pitch not 16-B aligned
    assert _quant(fp4, P(fp4), ldx=100) == E.ERR_INVALID_ARG           # ldx < cols
    assert _quant(fp4, P(fp4), rows=0) == E.ERR_INVALID_ARG            # empty tensors are rejected
    assert _quant(fp4, P(fp4), cols=0) == E.ERR_INVALID_ARG
    assert _quant(fp4, P(fp4), rows=-1) == E.ERR_INVALID_ARG
    assert _quant(fp4, P(fp4), ldx=1 << 24) == E.ERR_UNSUPPORTED       # 64-row tile span >= 2 GiB
    assert _quant(fp4, P(fp4, block_rows=32), ldx=1 << 24) == E.ERR_UNSUPPORTED
    assert fp4.lib().fp4_hadamard(0x1000, 1, 64, 256, 1 << 24, 128, 0x2000, None) == E.ERR_UNSUPPORTED
    assert _quant(fp4, P(fp4), codes=0x1000) == E.ERR_INVALID_ARG      # aliasing


def test_quantize_batch_validation_without_device(fp4):
    """Batched quantize: every rejection happens on the host, before any HIP call."""
    E = fp4
    L = fp4.lib()

    def items(*specs):
        arr = (fp4.QuantItemC * max(len(specs), 1))()
        for i, sp in enumerate(specs):
            base = dict(x=0x10000 * (i + 1), rows=64, cols=256, ldx=256, codes=0x100000 * (i + 1),
                        scales=0x1000000 * (i + 1), tensor_scale=None)
            base.update(sp)
            arr[i] = fp4.QuantItemC(**base)
        return arr

    def run(arr, n, p, dtype=1):
        return L.fp4_quantize_batch(n, arr, dtype, ctypes.byref(p), None)

    two = items({}, {"rows": 96})
    assert run(two, 0, P(fp4)) == E.ERR_INVALID_ARG                       # empty batch
    five = items({}, {}, {}, {}, {})
    assert run(five, 5, P(fp4)) == E.ERR_INVALID_ARG                      # more than four
    assert run(two, 2, P(fp4), dtype=7) == E.ERR_INVALID_ARG
    assert run(two, 2, P(fp4, block_cols=16, scale_mode=2)) == E.ERR_UNSUPPORTED   # NV needs an amax pass
    assert run(two, 2, P(fp4, block_cols=16, scale_mode=5)) == E.ERR_INVALID_ARG   # given g missing
    assert run(two, 2, P(fp4, block_cols=256)) == E.ERR_UNSUPPORTED        # per-row blocks
    assert run(items({}, {"cols": 250, "ldx": 250}), 2, P(fp4)) == E.ERR_INVALID_ARG
    assert run(items({}, {"x": None}), 2, P(fp4)) == E.ERR_INVALID_ARG
    assert run(items({}, {"ldx": 100}), 2, P(fp4)) == E.ERR_INVALID_ARG
    assert run(items({}, {"codes": 0x100008}), 2, P(fp4)) == E.ERR_ALIGNMENT
    assert run(items({}, {"codes": 0x10000}), 2, P(fp4)) == E.ERR_INVALID_ARG    # output = other input
    assert run(items({}, {"scales": 0x100000}), 2, P(fp4)) == E.ERR_INVALID_ARG  # outputs alias
    assert run(items({}, {"rows": 48}), 2, P(fp4, block_rows=32)) == E.ERR_INVALID_ARG  # 2D: rows % 32


def test_gemm_validation_without_device(fp4):
    E = fp4
    L = fp4.lib()

    def qt(rows, cols, **kw):
        return fp4.QTensorC(0x10000, 0x20000, None, rows, cols, P(fp4, **kw))

    a, b = qt(256, 256), qt(128, 256)
    c = 0x30000
    assert L.fp4_gemm(ctypes.byref(a), None, c, 0, 128, None, None, None, 0, None) == E.ERR_INVALID_ARG
    bk = qt(128, 384)
    assert L.fp4_gemm(ctypes.byref(a), ctypes.byref(bk), c, 0, 128, None, None, None, 0, None) == E.ERR_INVALID_ARG
    # K % 128 != 0 runs on the 128 x 128 kernel; NVFP4 there needs the workspace (the in-LDS
    # re-expression takes K % 128 == 0)
    an96 = fp4.QTensorC(0x10000, 0x20000, 0x40000, 256, 96, P(fp4, block_cols=16, scale_mode=2))
    bn96 = fp4.QTensorC(0x50000, 0x60000, 0x70000, 256, 96, P(fp4, block_cols=16, scale_mode=2))
    assert L.fp4_gemm(ctypes.byref(an96), ctypes.byref(bn96), c, 0, 256, None, None, None, 0, None) == E.ERR_WORKSPACE
    b8 = qt(128, 256, elem=1)
    assert L.fp4_gemm(ctypes.byref(a), ctypes.byref(b8), c, 0, 128, None, None, None, 0, None) == E.ERR_UNSUPPORTED
    a0 = qt(0, 256)
    assert L.fp4_gemm(ctypes.byref(a0), ctypes.byref(b), c, 0, 128, None, None, None, 0, None) == E.ERR_INVALID_ARG
    brot = qt(128, 256, hadamard_n=128)
    assert L.fp4_gemm(ctypes.byref(a), ctypes.byref(brot), c, 0, 128, None, None, None, 0, None) == E.ERR_INVALID_ARG
    assert L.fp4_gemm(ctypes.byref(a), ctypes.byref(b), c, 0, 64, None, None, None, 0, None) == E.ERR_INVALID_ARG
    assert L.fp4_gemm(ctypes.byref(a), ctypes.byref(b), 0x30004, 0, 128, None, None, None, 0, None) == E.ERR_ALIGNMENT
    an = fp4.QTensorC(0x10000, 0x20000, 0x40000, 256, 256, P(fp4, block_cols=16, scale_mode=3))
    bn = fp4.QTensorC(0x50000, 0x60000, 0x70000, 128, 256, P(fp4, block_cols=16, scale_mode=2))
    assert L.fp4_gemm_workspace_bytes(ctypes.byref(an), ctypes.byref(bn)) > 0
    assert L.fp4_gemm(ctypes.byref(an), ctypes.byref(bn), c, 0, 128, None, None, None, 0, None) == E.ERR_WORKSPACE
    # fused output quantization: argument checks (nothing is launched on any error)
    def run(oq, cq, cptr=c, bb=b):
        return L.fp4_gemm(ctypes.byref(a), ctypes.byref(bb), cptr, 0, 128,
                          ctypes.byref(oq) if oq is not None else None,
                          ctypes.byref(cq) if cq is not None else None, None, 0, None)
    cq = fp4.QTensorC(0x80000, 0x90000, None, 0, 0, P(fp4))
    assert run(None, None, cptr=None) == E.ERR_INVALID_ARG            # no output at all
    assert run(P(fp4), None) == E.ERR_INVALID_ARG                     # out_q without C_q
    assert run(None, cq) == E.ERR_INVALID_ARG                         # C_q without out_q
    assert run(P(fp4, block_cols=16), cq) == E.ERR_UNSUPPORTED         # only MX groups of 32
    assert run(P(fp4, block_cols=16, scale_mode=2), cq) == E.ERR_UNSUPPORTED
    assert run(P(fp4, hadamard_n=256), cq) == E.ERR_UNSUPPORTED        # rotation of C: n <= 128
    assert run(P(fp4, hadamard_n=48), cq) == E.ERR_INVALID_ARG
    b160 = qt(160, 256)
    assert run(P(fp4, hadamard_n=64), cq, bb=b160) == E.ERR_INVALID_ARG  # N % n != 0
    assert run(P(fp4, round_mode=5), cq) == E.ERR_INVALID_ARG
    b100 = qt(100, 256)
    assert run(P(fp4), cq, bb=b100) == E.ERR_INVALID_ARG               # N % 32 != 0
    cq_mis = fp4.QTensorC(0x80004, 0x90000, None, 0, 0, P(fp4))
    assert run(P(fp4), cq_mis) == E.ERR_ALIGNMENT


def test_oracle_and_hip_path_share_no_code():
    prod = os.path.join(ROOT, "bit_gemm_fwht_amd")
    orc = os.path.join(ROOT, "oracle")
    for d, banned in ((orc, ("bit_gemm_fwht_amd", "csrc", "fp4.h", "device.h")),
                      (prod, ("oracle", "liboracle"))):
        for dirpath, _, files in os.walk(d):
            for f in files:
                if not f.endswith((".c", ".h", ".cpp", ".hip", ".py")):
                    continue
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                for line in text.splitlines():
                    s = line.strip()
                    if s.startswith(("#include", "import ", "from ")):
                        for b in banned:
                            assert b not in s, f"{f}: {s}"


def _quant_cw(fp4, p, rows=256, cols=64, x=0x1000, codes=0x2000, scales=0x3000, ts=None, ws=None,
              wsb=0, ldx=None, dtype=1):
    return fp4.lib().fp4_quantize_colwise(x, dtype, rows, cols, ldx or cols, ctypes.byref(p), codes,
                                          scales, ts, ws, wsb, None)


def test_quantize_colwise_validation_without_device(fp4):
    """The column-wise call checks the transposed shape (cols x rows, groups along x's rows)."""
    E = fp4
    assert _quant_cw(fp4, P(fp4), x=None) == E.ERR_INVALID_ARG
    assert _quant_cw(fp4, P(fp4), rows=250) == E.ERR_INVALID_ARG          # T has 250 columns
    assert _quant_cw(fp4, P(fp4, hadamard_n=128), rows=320) == E.ERR_INVALID_ARG
    assert _quant_cw(fp4, P(fp4, block_rows=32)) == E.ERR_UNSUPPORTED      # 2D tiles
    assert _quant_cw(fp4, P(fp4, block_cols=256)) == E.ERR_UNSUPPORTED     # per-row of T
    assert _quant_cw(fp4, P(fp4, scale_mode=2, block_cols=16)) == E.ERR_INVALID_ARG  # no tensor_scale
    assert _quant_cw(fp4, P(fp4, scale_mode=2, block_cols=16), ts=0x4000) == E.ERR_WORKSPACE
    assert _quant_cw(fp4, P(fp4), x=0x1004) == E.ERR_ALIGNMENT
    assert _quant_cw(fp4, P(fp4), ldx=66) == E.ERR_ALIGNMENT
    assert _quant_cw(fp4, P(fp4), ldx=32) == E.ERR_INVALID_ARG            # ldx < cols
    assert _quant_cw(fp4, P(fp4), codes=0x1000) == E.ERR_INVALID_ARG      # aliasing


def test_nv_given_validation_without_device(fp4):
    """The _GIVEN NVFP4 modes need no workspace (no amax pass) but do need tensor_scale."""
    E = fp4
    L = fp4.lib()
    p = P(fp4, scale_mode=5, block_cols=16)
    assert L.fp4_workspace_bytes(64, 256, ctypes.byref(p)) == 0
    assert L.fp4_workspace_bytes(64, 256, ctypes.byref(P(fp4, scale_mode=2, block_cols=16))) == 256
    assert _quant(fp4, p) == E.ERR_INVALID_ARG                          # no tensor_scale
    assert _quant(fp4, P(fp4, scale_mode=6, block_cols=32), ts=0x4000) == E.ERR_UNSUPPORTED
    assert _quant(fp4, P(fp4, scale_mode=6, block_cols=16, round_mode=1), ts=0x4000) == E.ERR_UNSUPPORTED
    assert _quant(fp4, P(fp4, scale_mode=7, block_cols=16), ts=0x4000) == E.ERR_INVALID_ARG


def test_binding_refuses_an_output_that_is_not_row_major(fp4):
    """The binding passes out.stride(0) as ldc, so it accepts any row pitch >= N but refuses an out
    whose columns are not contiguous, or of the wrong shape (checked before anything is launched)."""
    import torch
    p = fp4.Params()
    a = fp4.QTensor(torch.zeros(64 * 128, dtype=torch.uint8), torch.zeros(64 * 8, dtype=torch.uint8),
                    None, 64, 256, p)
    b = fp4.QTensor(torch.zeros(96 * 128, dtype=torch.uint8), torch.zeros(96 * 8, dtype=torch.uint8),
                    None, 96, 256, p)
    with pytest.raises(ValueError, match="row-major"):
        fp4.gemm(a, b, out=torch.empty(96, 64, dtype=torch.bfloat16).t())
    with pytest.raises(ValueError):
        fp4.gemm(a, b, out=torch.empty(64, 95, dtype=torch.bfloat16))


def test_binding_refuses_host_and_undersized_buffers(fp4):
    """A host pointer handed to a kernel would fault the GPU: the binding refuses host tensors and
    operand buffers smaller than the size queries state, before anything is launched."""
    import torch
    p = fp4.Params()
    a = fp4.QTensor(torch.zeros(64 * 128, dtype=torch.uint8), torch.zeros(64 * 8, dtype=torch.uint8),
                    None, 64, 256, p)
    with pytest.raises(ValueError, match="buffer on cpu"):
        fp4.gemm(a, a)
    with pytest.raises(ValueError, match="buffer on cpu"):
        fp4.dequantize(a)
    with pytest.raises(ValueError, match="CUDA"):
        fp4.hadamard(torch.zeros(4, 256), 128)
    with pytest.raises(ValueError, match="CUDA"):
        fp4.quantize(torch.zeros(4, 256), p)
    short = fp4.QTensor(torch.zeros(64 * 128 - 1, dtype=torch.uint8), a.scales, None, 64, 256, p)
    with pytest.raises(ValueError, match="at least 8192 bytes"):
        fp4._check_q(short, 64, 256, p, torch.device("cpu"), "q")


def test_nvfp4_to_mxfp8_rejects_bad_arguments(fp4):
    """Host-side checks of the re-expression entry point (nothing reaches the device)."""
    L = fp4.lib()
    E = fp4
    good = dict(codes=0x10000, scales=0x20000, rows=8, cols=64, oc=0x30000, os=0x40000)

    def call(**kw):
        a = dict(good, **kw)
        return L.fp4_nvfp4_to_mxfp8(a["codes"], a["scales"], a["rows"], a["cols"], a["oc"], a["os"], None)

    assert call(codes=None) == E.ERR_INVALID_ARG
    assert call(os=None) == E.ERR_INVALID_ARG
    assert call(rows=0) == E.ERR_INVALID_ARG
    assert call(cols=48) == E.ERR_INVALID_ARG        # cols % 32
    assert call(codes=0x10008) == E.ERR_ALIGNMENT     # codes need 16 bytes
    assert call(scales=0x20001) == E.ERR_ALIGNMENT    # scales need 2 bytes
    assert call(oc=0x30004) == E.ERR_ALIGNMENT
    assert call(oc=0x10000) == E.ERR_INVALID_ARG      # output aliases an input
    assert call(os=0x30000) == E.ERR_INVALID_ARG      # outputs alias each other


def test_transpose_2d_rejects_bad_arguments(fp4):
    L = fp4.lib()
    p2d = P(fp4, block_rows=32, block_cols=32, scale_mode=1)
    g = dict(codes=0x10000, scales=0x20000, rows=64, cols=96, oc=0x30000, os=0x40000, p=p2d)

    def call(**kw):
        a = dict(g, **kw)
        return L.fp4_transpose_2d(a["codes"], a["scales"], a["rows"], a["cols"], ctypes.byref(a["p"]), a["oc"],
                                  a["os"], None)

    assert call(p=P(fp4)) == fp4.ERR_UNSUPPORTED                          # 1 x 32 groups: not a 2D tensor
    assert call(p=P(fp4, block_rows=32, scale_mode=1, hadamard_n=32)) == fp4.ERR_UNSUPPORTED  # rotated
    assert call(rows=48) == fp4.ERR_INVALID_ARG                          # rows % 32
    assert call(codes=None) == fp4.ERR_INVALID_ARG
    assert call(oc=0x10000) == fp4.ERR_INVALID_ARG                       # aliases the input
    assert call(codes=0x10008) == fp4.ERR_ALIGNMENT
    assert call(oc=0x30008) == fp4.ERR_ALIGNMENT
