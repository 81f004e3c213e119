"""Seeded random sweep over shapes and modes (GPU parity through the C ABI, against the oracle).

Each case draws its own shape and mode combination from a fixed seed, so the set is the same on
every run: quantize cases must match the oracle's codes, scales and tensor scale byte for byte;
GEMM cases must meet the same per-output bound as the fixed parity tests. The draws favour ragged
sizes (row counts that are not multiples of the tile heights, widths that are not multiples of the
stage depths) and every element / scale / rounding / rotation combination the library accepts."""
import numpy as np
import pytest
import torch

from bit_gemm_fwht_amd import fp4
from bit_gemm_fwht_amd import workloads as wl
from test_gpu_parity import (CEIL, E2M1, E4M3, F32, FLOOR, NV, NV46, RNE, SR, P, _check_quant, _gemm_check,
                             _orc_quant, _to_dev)

DEV = "cuda:0"

pytestmark = pytest.mark.gpu

N_QUANT, N_GEMM, N_EXTRA, N_TILES = 40, 24, 16, 24


def _quant_case(seed):
    rng = np.random.default_rng(1000 + seed)
    mode = rng.choice(["mx", "mx16", "2d", "nv", "nv46", "f32", "f32_16"])
    elem = E4M3 if (mode in ("mx", "mx16", "2d", "f32") and rng.random() < 0.35) else E2M1
    rnd = SR if (mode not in ("nv46",) and rng.random() < 0.4) else RNE
    block = {"mx": (1, 32), "mx16": (1, 16), "2d": (32, 32), "nv": (1, 16), "nv46": (1, 16),
             "f32": (1, 32), "f32_16": (1, 16)}[mode]
    scale = {"mx": FLOOR, "mx16": CEIL, "2d": CEIL, "nv": NV, "nv46": NV46, "f32": F32, "f32_16": F32}[mode]
    if mode == "mx" and rng.random() < 0.5:
        scale = CEIL
    cols = int(rng.choice([32, 64, 96, 128, 160, 256, 384, 512, 1024]))
    hns = [h for h in (0, 16, 32, 64, 128, 256) if h == 0 or cols % h == 0]
    hn = int(rng.choice(hns))
    rows = int(rng.integers(1, 9)) * 32 if mode == "2d" else int(rng.integers(1, 300))
    dtype = "bf16" if rng.random() < 0.6 else "f32"
    return rows, cols, dtype, P(elem=elem, block=block, scale_mode=scale, round_mode=rnd, hadamard_n=hn,
                                seed=int(rng.integers(0, 2**40)))


@pytest.mark.parametrize("seed", range(N_QUANT))
def test_random_quantize(orc, seed):
    rows, cols, dtype, params = _quant_case(seed)
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, cols)) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32)
    x[rng.random((rows, cols)) < 0.01] *= 40.0  # sparse outliers
    x[rng.random((rows, cols)) < 0.01] = 0.0
    if dtype == "bf16":
        x = wl.f32_to_bf16_bits(x)
    _check_quant(orc, x, params)


def _gemm_case(seed):
    rng = np.random.default_rng(2000 + seed)
    kind = rng.choice(["mxfp4", "mxfp4_2d", "mxfp8", "nvfp4"])
    big = rng.random() < 0.5  # shapes that take the 256 x 256 kernel
    K = int(rng.choice([256, 512, 768, 1024])) if big else int(rng.choice([128, 384, 640]))
    if big:
        M, N = int(rng.integers(256, 700)), int(rng.integers(8, 22)) * 32
    else:
        M, N = int(rng.integers(1, 300)), int(rng.integers(1, 12)) * 32
    if kind == "mxfp4":
        pa, pb = P(), P(scale_mode=CEIL)
    elif kind == "mxfp4_2d":
        pa, pb = P(scale_mode=CEIL), P(block=(32, 32), scale_mode=CEIL)
    elif kind == "mxfp8":
        pa, pb = P(elem=E4M3), P(elem=E4M3, scale_mode=CEIL)
    else:
        pa, pb = P(block=(1, 16), scale_mode=NV46), P(block=(1, 16), scale_mode=NV)
    c_dtype = torch.bfloat16 if rng.random() < 0.5 else torch.float32
    return M, N, K, pa, pb, c_dtype


@pytest.mark.parametrize("seed", range(N_GEMM))
def test_random_gemm(orc, seed):
    M, N, K, pa, pb, c_dtype = _gemm_case(seed)
    rng = np.random.default_rng(seed)
    A = (rng.standard_normal((M, K)) * 10.0 ** rng.uniform(-2, 2)).astype(np.float32)
    B = (rng.standard_normal((N, K)) * 10.0 ** rng.uniform(-3, 1)).astype(np.float32)
    _gemm_check(orc, A, B, pa, pb, c_dtype=c_dtype)


def _tile_case(seed):
    """Shapes around the tile-size choices: M or N below 256, the 128 / 256 boundaries, grids of
    256 x 256 tiles on either side of half the CU count, ragged edges, K from one stage to many, with
    the plain output or the fused output quantize."""
    rng = np.random.default_rng(3000 + seed)
    kind = rng.choice(["mxfp4", "mxfp4_2d", "mxfp8", "nvfp4"])
    M = int(rng.choice([int(rng.integers(1, 129)), int(rng.integers(120, 264)), int(rng.integers(250, 1400)),
                        int(rng.integers(2600, 4200))]))
    N = 32 * int(rng.choice([int(rng.integers(1, 9)), int(rng.integers(7, 10)), int(rng.integers(8, 45)),
                             int(rng.integers(80, 131))]))
    K = int(rng.choice([256, 512, 768, 1024, 2048, 4096]))
    if kind == "mxfp4":
        pa, pb = P(scale_mode=CEIL), P()
    elif kind == "mxfp4_2d":
        pa, pb = P(), P(block=(32, 32), scale_mode=CEIL)
    elif kind == "mxfp8":
        pa, pb = P(elem=E4M3), P(elem=E4M3, scale_mode=CEIL)
        K = int(rng.choice([128, 384, 640, 1024, 2048]))
    else:
        pa, pb = P(block=(1, 16), scale_mode=NV46), P(block=(1, 16), scale_mode=NV)
        K = int(rng.choice([128, 384, 640, 1024, 2048]))
    c_dtype = torch.bfloat16 if rng.random() < 0.5 else torch.float32
    out_q = None
    if rng.random() < 0.35:
        hn = int(rng.choice([h for h in (0, 32, 128) if N % max(h, 32) == 0]))
        out_q = P(elem=E2M1 if rng.random() < 0.7 else E4M3, scale_mode=FLOOR if rng.random() < 0.5 else CEIL,
                  round_mode=SR if rng.random() < 0.4 else RNE, hadamard_n=hn, seed=int(rng.integers(0, 2**40)))
    return M, N, K, pa, pb, c_dtype, out_q


@pytest.mark.parametrize("seed", range(N_TILES))
def test_random_gemm_tile_choices(orc, seed):
    """C within the GEMM bound on 4096 sampled outputs; with the fused output quantize, C_q equal to
    the oracle's quantization of the same call's fp32 C, byte for byte."""
    M, N, K, pa, pb, c_dtype, out_q = _tile_case(seed)
    rng = np.random.default_rng(seed)
    A = (rng.standard_normal((M, K)) * 10.0 ** rng.uniform(-1, 1)).astype(np.float32)
    B = (rng.standard_normal((N, K)) * 10.0 ** rng.uniform(-2, 0)).astype(np.float32)
    ms, ns = rng.integers(0, M, 4096), rng.integers(0, N, 4096)
    _gemm_check(orc, A, B, pa, pb, c_dtype=c_dtype, sample=(ms, ns))
    if out_q is not None:
        qa, qb = fp4.quantize(_to_dev(A), pa), fp4.quantize(_to_dev(B), pb)
        c, cq = fp4.gemm(qa, qb, out_dtype=torch.float32, out_q=out_q)
        torch.cuda.synchronize()
        oc, os_, _ = _orc_quant(orc, c.cpu().numpy(), out_q)
        assert np.array_equal(cq.codes.cpu().numpy(), oc.reshape(-1)), f"C_q codes ({M}, {N}, {K})"
        assert np.array_equal(cq.scales.cpu().numpy(), os_.reshape(-1).view(np.uint8)), f"C_q scales ({M}, {N}, {K})"


def _input(rng, rows, cols, dtype):
    x = (rng.standard_normal((rows, cols)) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32)
    x[rng.random((rows, cols)) < 0.01] *= 40.0
    return wl.f32_to_bf16_bits(x) if dtype == "bf16" else x


def _same(q, oc, os_, what):
    assert np.array_equal(q.codes.cpu().numpy(), oc.reshape(-1)), f"{what}: codes differ from the oracle"
    assert np.array_equal(q.scales.cpu().numpy(), os_.reshape(-1).view(np.uint8)), f"{what}: scales differ"


@pytest.mark.parametrize("seed", range(N_EXTRA))
def test_random_strided_colwise_batch(orc, seed):
    """A 1D mode from the quantize draw, applied three more ways: with a row pitch wider than the
    row, column-wise (x^T without forming it), and in a batch with a second tensor."""
    rows, cols, dtype, params = _quant_case(100 + seed)
    if params.block[0] != 1:
        params = P(elem=params.elem, block=(1, 32), scale_mode=CEIL, round_mode=params.round_mode,
                   hadamard_n=params.hadamard_n, seed=params.seed)
    rng = np.random.default_rng(500 + seed)
    x = _input(rng, rows, cols, dtype)
    oc, os_, ot = _orc_quant(orc, x, params)
    # strided rows: x is the left part of a wider buffer
    xd = _to_dev(x)
    wide = torch.zeros(rows, cols + 32 * int(rng.integers(1, 4)), dtype=xd.dtype, device=DEV)
    wide[:, :cols] = xd
    q = fp4.quantize(wide[:, :cols], params)
    torch.cuda.synchronize()
    _same(q, oc, os_, "strided")
    # column-wise: quantize y^T for y = xc^T, xc the first r8 rows of x (y's row count, cols, a
    # multiple of 32; its row pitch, r8 elements, a multiple of 16 bytes)
    r8 = rows // 8 * 8
    if cols % 32 == 0 and r8 >= 8:
        xc = np.ascontiguousarray(x[:r8])
        occ, osc, _ = _orc_quant(orc, xc, params)
        qc = fp4.quantize_colwise(_to_dev(np.ascontiguousarray(xc.T)), params)
        torch.cuda.synchronize()
        _same(qc, occ, osc, "colwise")
    # batched with a second tensor of another shape (modes without a tensor-wide amax)
    if params.scale_mode not in (NV, NV46):
        rows2 = int(rng.integers(1, 200))
        x2 = _input(rng, rows2, cols, dtype)
        oc2, os2, _ = _orc_quant(orc, x2, params)
        q1, q2 = fp4.quantize_batch([_to_dev(x), _to_dev(x2)], params)
        torch.cuda.synchronize()
        _same(q1, oc, os_, "batch item 0")
        _same(q2, oc2, os2, "batch item 1")


@pytest.mark.parametrize("seed", range(N_EXTRA))
def test_random_fused_output_quantize(orc, seed):
    """Random GEMM shape and operand kind with a random fused output quantize (element, scale
    rule, rounding, rotation along N): codes and scales equal the oracle's quantization of the
    fp32 C the same call stores."""
    M, N, K, pa, pb, _ = _gemm_case(300 + seed)
    rng = np.random.default_rng(700 + seed)
    hns = [h for h in (0, 16, 32, 64, 128) if h == 0 or N % h == 0]
    oq = P(elem=E4M3 if rng.random() < 0.3 else E2M1, scale_mode=CEIL if rng.random() < 0.5 else FLOOR,
           round_mode=SR if rng.random() < 0.4 else RNE, hadamard_n=int(rng.choice(hns)),
           seed=int(rng.integers(0, 2**40)))
    A = (rng.standard_normal((M, K))).astype(np.float32)
    B = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    ca, sa, ta = _orc_quant(orc, A, pa)
    cb, sb, tb = _orc_quant(orc, B, pb)
    qa = fp4.upload_qtensor(ca, sa, ta, M, K, pa, DEV)
    qb = fp4.upload_qtensor(cb, sb, tb, N, K, pb, DEV)
    c, cq = fp4.gemm(qa, qb, out_dtype=torch.float32, out_q=oq)
    torch.cuda.synchronize()
    oc, os_, _ = _orc_quant(orc, c.cpu().numpy(), oq)
    _same(cq, oc, os_, f"fused out_q {oq}")
