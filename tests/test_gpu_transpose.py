"""A tensor quantized with 32 x 32 blocks, re-laid out as the quantized form of its transpose
(fp4_transpose_2d), equals the oracle's quantization of the transposed tensor byte for byte, and the
GEMM that contracts the weight along its other axis (Y = X W, W as stored) runs on it."""
import numpy as np
import pytest
import torch

from bit_gemm_fwht_amd import fp4
from bit_gemm_fwht_amd import workloads as wl
from test_gpu_parity import CEIL, E4M3, FLOOR, P, _gemm_tol, _orc_quant, _to_dev, report_ratio

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("rows,cols", [(64, 64), (96, 160), (256, 512), (32, 32), (160, 288), (416, 96), (4096, 4096)])
@pytest.mark.parametrize("elem,sm", [(fp4.E2M1, CEIL), (fp4.E2M1, FLOOR), (E4M3, CEIL)])
def test_transpose_equals_quantize_of_transpose(orc, rows, cols, elem, sm):
    rng = np.random.default_rng(rows + cols + elem)
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    w.reshape(-1)[rng.choice(w.size, size=max(w.size // 500, 1), replace=False)] *= 30  # a few outliers
    w[:32, :32] = 0.0  # an all-zero tile
    p = P(elem=elem, block=(32, 32), scale_mode=sm)
    q = fp4.quantize(_to_dev(wl.f32_to_bf16_bits(w)), p)
    t = fp4.transpose_2d(q)
    torch.cuda.synchronize()
    oc, os_, _ = _orc_quant(orc, np.ascontiguousarray(wl.f32_to_bf16_bits(w).T), p)
    assert (t.rows, t.cols) == (cols, rows)
    assert np.array_equal(t.codes.cpu().numpy(), oc.reshape(-1)), "codes differ from the oracle's quantize of W^T"
    assert np.array_equal(t.scales.cpu().numpy(), os_.reshape(-1)), "scales differ"
    back = fp4.transpose_2d(t)  # and back again: the original codes
    torch.cuda.synchronize()
    assert torch.equal(back.codes, q.codes) and torch.equal(back.scales, q.scales)


def _forward_check(orc, X, W, px, pw, c_dtype, sample=None):
    """Y = X W with W [K, N] quantized 2D as stored, fed to the GEMM through its transpose."""
    M, K = X.shape
    N = W.shape[1]
    qx = fp4.quantize(_to_dev(X), px)
    qw = fp4.quantize(_to_dev(W), pw)
    qwt = fp4.transpose_2d(qw)
    y = fp4.gemm(qx, qwt, out_dtype=c_dtype)
    torch.cuda.synchronize()
    ox = _orc_quant(orc, X, px)
    owt = _orc_quant(orc, np.ascontiguousarray(W.T), pw)
    if sample is None:
        ms, ns = np.repeat(np.arange(M), N), np.tile(np.arange(N), M)
    else:
        rng = np.random.default_rng(1)
        ms, ns = rng.integers(0, M, sample), rng.integers(0, N, sample)
    ur, im = np.unique(ms, return_inverse=True)
    un, inn = np.unique(ns, return_inverse=True)
    a64 = orc.operand_f64(ox[0][ur], ox[1][ur], None, len(ur), K, elem=px.elem, block=px.block,
                          scale_mode=px.scale_mode)
    b64 = orc.operand_f64(owt[0][un], np.ascontiguousarray(owt[1][un // 32]), None, len(un), K,
                          elem=pw.elem, block=(1, 32), scale_mode=pw.scale_mode)
    ref, sabs = orc.gemm_f64_sampled(a64, b64, im, inn)
    got = y[torch.from_numpy(ms).to(DEV), torch.from_numpy(ns).to(DEV)].float().cpu().numpy().astype(np.float64)
    tol = _gemm_tol(ref, sabs, a64, b64, im, inn, px, K, c_dtype)
    err = np.abs(got - ref)
    report_ratio(err, ref, sabs, c_dtype, f"{M}x{N}x{K} forward through the 2D transpose")
    assert np.all(err <= tol), f"{np.sum(err > tol)} outputs exceed the bound"


@pytest.mark.parametrize("M,K,N", [(200, 256, 96), (512, 384, 640), (64, 128, 32)])
def test_forward_gemm_on_the_transposed_weight(orc, M, K, N):
    rng = np.random.default_rng(M + K + N)
    X = rng.standard_normal((M, K)).astype(np.float32)
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    for c_dtype in (torch.float32, torch.bfloat16):
        _forward_check(orc, X, W, P(scale_mode=CEIL), P(block=(32, 32), scale_mode=CEIL), c_dtype)


def test_forward_gemm_on_the_transposed_weight_full_size(orc):
    """At the backward workload's shapes: W 4096 x 4096 (2D, truncation-free, no rotation) quantized
    once; Y = X W for X 8192 x 4096 through its transpose, 4096 sampled outputs."""
    x, w = wl.forward_2d(0)
    _forward_check(orc, x, w, P(scale_mode=CEIL), P(block=(32, 32), scale_mode=CEIL), torch.bfloat16, sample=4096)
