"""The GEMM with A's rotation + MXFP4 quantization fused into its launch (fp4_gemm_quantize_a):
A's codes and scales equal the oracle's quantize byte for byte, C equals fp4_gemm on those codes bit
for bit (the same tile arithmetic) and meets the bound against the oracle's fp64 product; shapes off
the 256 x 256 tile path take the two-launch route with the same results."""
import ctypes

import numpy as np
import pytest
import torch

from bit_gemm_fwht_amd import fp4
from bit_gemm_fwht_amd import workloads as wl
from test_gpu_parity import CEIL, FLOOR, RNE, SR, P, _gemm_tol, _orc_quant, _to_dev, report_ratio

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _check(orc, A, B, pa, pb, c_dtype, sample=None):
    M, K = A.shape
    N = B.shape[0]
    qb = fp4.quantize(_to_dev(B), pb)
    bc = qb.c()
    ws = torch.full((fp4.lib().fp4_gemm_quantize_a_workspace_bytes(M, ctypes.byref(bc)),), 0xFF, dtype=torch.uint8,
                    device=DEV)  # stale counters: the call must clear them
    c, qa = fp4.gemm_quantize_a(_to_dev(A), pa, qb, out_dtype=c_dtype, workspace=ws)
    ref_c = fp4.gemm(qa, qb, out_dtype=c_dtype)  # the plain GEMM on the codes the fused call wrote
    torch.cuda.synchronize()
    if M >= 256 and N >= 256 and K % 256 == 0:  # the one-launch path: counter, then the status word
        assert ws[4:8].cpu().numpy().view(np.uint32)[0] == 0, "the hand-over wait gave up"
    oc, os_, _ = _orc_quant(orc, A, pa)
    assert np.array_equal(qa.codes.cpu().numpy(), oc.reshape(-1)), "A codes differ from the oracle"
    assert np.array_equal(qa.scales.cpu().numpy(), os_.reshape(-1)), "A scales differ from the oracle"
    assert torch.equal(c.view(torch.int16) if c_dtype == torch.bfloat16 else c.view(torch.int32),
                       ref_c.view(torch.int16) if c_dtype == torch.bfloat16 else ref_c.view(torch.int32))
    ob = _orc_quant(orc, B, pb)
    if sample is None:
        ms, ns = np.repeat(np.arange(M), N), np.tile(np.arange(N), M)
    else:
        rng = np.random.default_rng(3)
        ms, ns = rng.integers(0, M, sample), rng.integers(0, N, sample)
    ur, im = np.unique(ms, return_inverse=True)
    un, inn = np.unique(ns, return_inverse=True)
    a64 = orc.operand_f64(oc[ur], os_[ur], None, len(ur), K, elem=pa.elem, block=pa.block, scale_mode=pa.scale_mode)
    if pb.block[0] == 1:
        b64 = orc.operand_f64(ob[0][un], ob[1][un], None, len(un), K, elem=pb.elem, block=pb.block,
                              scale_mode=pb.scale_mode)
    else:
        b64 = orc.operand_f64(ob[0][un], np.ascontiguousarray(ob[1][un // 32]), None, len(un), K, elem=pb.elem,
                              block=(1, 32), scale_mode=pb.scale_mode)
    ref, sabs = orc.gemm_f64_sampled(a64, b64, im, inn)
    got = c[torch.from_numpy(ms).to(DEV), torch.from_numpy(ns).to(DEV)].float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    report_ratio(err, ref, sabs, c_dtype, f"{M}x{N}x{K} fused A quantize")
    tol = _gemm_tol(ref, sabs, a64, b64, im, inn, pa, K, c_dtype)
    assert np.all(err <= tol), f"{np.sum(err > tol)} outputs exceed the bound"


CASES = [
    # M, N, K, A dtype, pa, pb, C dtype
    (256, 256, 256, "bf16", P(hadamard_n=128), P(hadamard_n=128), torch.float32),
    (512, 768, 1024, "bf16", P(hadamard_n=128), P(hadamard_n=128), torch.bfloat16),
    (300, 520, 512, "f32", P(scale_mode=CEIL, round_mode=SR, seed=9), P(scale_mode=CEIL), torch.float32),
    (768, 512, 512, "bf16", P(hadamard_n=32, scale_mode=CEIL), P(block=(32, 32), scale_mode=CEIL, hadamard_n=32),
     torch.bfloat16),
    (1280, 256, 768, "f32", P(hadamard_n=64), P(hadamard_n=64), torch.float32),
    (128, 256, 256, "bf16", P(hadamard_n=128), P(hadamard_n=128), torch.float32),   # two-launch route: M < 256
    (512, 512, 384, "bf16", P(hadamard_n=128), P(hadamard_n=128), torch.bfloat16),  # two-launch route: K % 256
    (300, 288, 224, "f32", P(hadamard_n=32), P(hadamard_n=32), torch.float32),      # two-launch route: K % 128
    (64, 96, 96, "bf16", P(scale_mode=CEIL), P(block=(32, 32), scale_mode=CEIL), torch.bfloat16),
]


@pytest.mark.parametrize("M,N,K,dt,pa,pb,c_dtype", CASES)
def test_fused_quantize_a(orc, M, N, K, dt, pa, pb, c_dtype):
    rng = np.random.default_rng(M + N + K)
    A = rng.standard_normal((M, K)).astype(np.float32)
    A[:, rng.choice(K, size=max(K // 100, 1), replace=False)] *= 20  # outlier channels
    B = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    if dt == "bf16":
        A, B = wl.f32_to_bf16_bits(A), wl.f32_to_bf16_bits(B)
    _check(orc, A, B, pa, pb, c_dtype)


def test_fused_quantize_a_llama7b_forward_linear(orc):
    """The headline shapes: X 4096 x 4096 bf16 rotated and quantized inside the 4096 x 11008 x 4096
    GEMM launch; W quantized by its own launch; 4096 sampled outputs."""
    x, w, _ = wl.llama_linear(0)
    p = P(hadamard_n=128)
    _check(orc, x, w, p, p, torch.bfloat16, sample=4096)
