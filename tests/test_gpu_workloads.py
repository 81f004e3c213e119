"""Parity at the full sizes of the large workloads, in the configuration bench.py times:
quantization compared element for element with the oracle (codes and scales bit-exact), GEMM
outputs compared on a seeded sample of 4096 positions (the oracle computes each one on its own)."""
import numpy as np
import pytest
import torch

from bit_gemm_fwht_amd import fp4
from bit_gemm_fwht_amd import workloads as wl
from test_gpu_parity import CEIL, E4M3, NV46, SR, P, _gemm_tol, _orc_quant, _to_dev, report_ratio

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _quant_both(orc, x, params):
    q = fp4.quantize(_to_dev(x), params)
    torch.cuda.synchronize()
    oc, os_, ots = _orc_quant(orc, x, params)
    assert np.array_equal(q.codes.cpu().numpy(), oc.reshape(-1)), "codes differ from the oracle"
    assert np.array_equal(q.scales.cpu().numpy(), os_.reshape(-1).view(np.uint8)), "scales differ"
    if ots is not None:
        assert q.tensor_scale.cpu().numpy().view(np.uint32)[0] == ots.view(np.uint32)[0]
    return q, (oc, os_, ots)


def _sampled_gemm(orc, qa, qb, oa, ob, pa, pb, c_dtype, n=4096, seed=0):
    c = fp4.gemm(qa, qb, out_dtype=c_dtype)
    torch.cuda.synchronize()
    M, N, K = qa.rows, qb.rows, qa.cols
    rng = np.random.default_rng(seed)
    ms = rng.integers(0, M, n)
    ns = rng.integers(0, N, n)
    ms[:4] = [0, M - 1, 0, M - 1]
    ns[:4] = [0, N - 1, N - 1, 0]
    got = c[torch.from_numpy(ms).to(DEV), torch.from_numpy(ns).to(DEV)].float().cpu().numpy().astype(np.float64)
    ur, im = np.unique(ms, return_inverse=True)
    un, inn = np.unique(ns, return_inverse=True)
    kw_a = dict(elem=pa.elem, block=pa.block, scale_mode=pa.scale_mode)
    a64 = orc.operand_f64(oa[0][ur], oa[1][ur], oa[2], len(ur), K, **kw_a)
    if pb.block[0] == 1:
        b64 = orc.operand_f64(ob[0][un], ob[1][un], ob[2], len(un), K, elem=pb.elem, block=pb.block,
                              scale_mode=pb.scale_mode)
    else:
        b64 = orc.operand_f64(ob[0][un], np.ascontiguousarray(ob[1][un // 32]), ob[2], len(un), K,
                              elem=pb.elem, block=(1, 32), scale_mode=pb.scale_mode)
    ref, sabs = orc.gemm_f64_sampled(a64, b64, im, inn)
    tol = _gemm_tol(ref, sabs, a64, b64, im, inn, pa, K, c_dtype)
    err = np.abs(got - ref)
    report_ratio(err, ref, sabs, c_dtype, f"{M}x{N}x{K} {pa.elem}/{pa.scale_mode} sampled {n}")
    assert np.all(err <= tol), f"{np.sum(err > tol)} of {n} sampled outputs exceed the bound"


def test_llama7b_forward_linear(orc):
    """X 4096x4096, W 11008x4096 (bf16), H_128 + MXFP4; 4096x11008x4096 GEMM to bf16. The operands
    are quantized as the benchmark does it, X and W in one batched launch."""
    x, w, _ = wl.llama_linear(0)
    p = P(hadamard_n=128)
    qx, qw = fp4.quantize_batch([_to_dev(x), _to_dev(w)], p)
    torch.cuda.synchronize()
    ox, ow = _orc_quant(orc, x, p), _orc_quant(orc, w, p)
    for q, o in ((qx, ox), (qw, ow)):
        assert np.array_equal(q.codes.cpu().numpy(), o[0].reshape(-1)), "codes differ from the oracle"
        assert np.array_equal(q.scales.cpu().numpy(), o[1].reshape(-1).view(np.uint8)), "scales differ"
    _sampled_gemm(orc, qx, qw, ox, ow, p, p, torch.bfloat16)


def test_backward_2d_scales(orc):
    """W 4096x4096 2D 32x32 truncation-free RNE, dY 8192x4096 group-32 truncation-free SR (seed 7),
    both rotated by H_128; dX = dY W^T in MXFP4, and the MXFP8 variant."""
    w, dy = wl.backward_2d(0)
    pw = P(block=(32, 32), scale_mode=CEIL, hadamard_n=128)
    pd = P(scale_mode=CEIL, round_mode=SR, hadamard_n=128, seed=7)
    qw, ow = _quant_both(orc, w, pw)
    qd, od = _quant_both(orc, dy, pd)
    _sampled_gemm(orc, qd, qw, od, ow, pd, pw, torch.bfloat16)
    pw8 = P(elem=E4M3, scale_mode=CEIL, hadamard_n=128)
    pd8 = P(elem=E4M3, scale_mode=CEIL, round_mode=SR, hadamard_n=128, seed=7)
    qw8, ow8 = _quant_both(orc, w, pw8)
    qd8, od8 = _quant_both(orc, dy, pd8)
    _sampled_gemm(orc, qd8, qw8, od8, ow8, pd8, pw8, torch.bfloat16)


def test_nvfp4_4over6(orc):
    """X 8192x8192 Laplace with 0.1% x30 outliers and W 8192x8192 N(0, 0.02^2), NVFP4 with the
    4/6 choice; the 8192^3 GEMM through the FP8 re-expression."""
    x, w = wl.nvfp4_4over6(0)
    p = P(block=(1, 16), scale_mode=NV46)
    qx, ox = _quant_both(orc, x, p)
    qw, ow = _quant_both(orc, w, p)
    _sampled_gemm(orc, qx, qw, ox, ow, p, p, torch.bfloat16)


def test_nvfp4_4over6_given_scale(orc):
    """The delayed-scale workload: with g handed in as each tensor's own RN(amax / 2688), the
    _GIVEN mode's codes and scales equal the oracle's plain NVFP4 + 4/6 quantization (one pass)."""
    x, _ = wl.nvfp4_4over6(0)
    amax = np.float32(np.abs(wl.bf16_bits_to_f32(x)).max())
    g = float(amax / np.float32(2688.0))
    q = fp4.quantize(_to_dev(x), P(block=(1, 16), scale_mode=fp4.SCALE_NV_4OVER6_GIVEN), tensor_scale=g)
    torch.cuda.synchronize()
    oc, os_, ots = _orc_quant(orc, x, P(block=(1, 16), scale_mode=NV46))
    assert np.array_equal(q.codes.cpu().numpy(), oc.reshape(-1)), "codes differ from the oracle"
    assert np.array_equal(q.scales.cpu().numpy(), os_.reshape(-1).view(np.uint8)), "scales differ"
    assert q.tensor_scale.cpu().numpy().view(np.uint32)[0] == ots.view(np.uint32)[0]


def test_llama7b_fused_output_quantize(orc):
    """The headline GEMM with the fused H_128 MXFP4 output quantize: sampled rows of C_q equal the
    oracle's quantization of the same rows of the fp32 C the call stores."""
    x, w, _ = wl.llama_linear(0)
    p = P(hadamard_n=128)
    qx, qw = fp4.quantize_batch([_to_dev(x), _to_dev(w)], p)
    oq = P(hadamard_n=128)
    c, cq = fp4.gemm(qx, qw, out_dtype=torch.float32, out_q=oq)
    torch.cuda.synchronize()
    M, N = c.shape
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(5).integers(0, M, 62)]))
    c_rows = c[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    oc, os_, _ = _orc_quant(orc, c_rows, oq)
    codes = cq.codes.view(M, N // 2)[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    scales = cq.scales.view(M, N // 32)[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    assert np.array_equal(codes, oc.reshape(len(rows), N // 2)), "C_q codes differ from the oracle"
    assert np.array_equal(scales, os_.reshape(len(rows), N // 32).view(np.uint8)), "C_q scales differ"


def test_backward_dw_colwise(orc):
    """dW = dY^T X over 8192 tokens: dY and X (as stored, [tokens, 4096]) quantized column-wise
    (H_128 along tokens, E8M0 ceil; dY SR) equal the oracle's quantization of the transposes; the
    4096x4096x8192 GEMM on sampled outputs."""
    dy, x = wl.backward_dw(0)
    pd = P(scale_mode=CEIL, round_mode=SR, hadamard_n=128, seed=7)
    px = P(scale_mode=CEIL, hadamard_n=128)
    qs, os_ = [], []
    for t, p in ((dy, pd), (x, px)):
        q = fp4.quantize_colwise(_to_dev(t), p)
        torch.cuda.synchronize()
        o = _orc_quant(orc, np.ascontiguousarray(t.T), p)
        assert np.array_equal(q.codes.cpu().numpy(), o[0].reshape(-1)), "codes differ from the oracle"
        assert np.array_equal(q.scales.cpu().numpy(), o[1].reshape(-1).view(np.uint8)), "scales differ"
        qs.append(q)
        os_.append(o)
    _sampled_gemm(orc, qs[0], qs[1], os_[0], os_[1], pd, px, torch.bfloat16)
