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
from test_gpu_parity import (CEIL, E2M1, E4M3, F32, FLOOR, NV, NV46, RNE, SR, P, _check_quant, _gemm_check)

pytestmark = pytest.mark.gpu

N_QUANT, N_GEMM = 24, 16


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
