"""The library keeps no state between calls: quantize + GEMM sequences issued on two streams at
once (one NVFP4 with the 4/6 choice and its tensor-amax workspace, one rotated MXFP4) give the
same codes, scales, tensor scales and C, bit for bit, as the same calls run one after the other.
Serial results are themselves checked against the oracle by the parity tests."""
import numpy as np
import pytest
import torch

from bit_gemm_fwht_amd import fp4
from bit_gemm_fwht_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _bf16(rng, rows, cols, scale):
    x = (rng.standard_normal((rows, cols)) * scale).astype(np.float32)
    return torch.from_numpy(wl.f32_to_bf16_bits(x).view(np.int16)).to(DEV).view(torch.bfloat16)


def _work(x, w, p):
    qx = fp4.quantize(x, p)
    qw = fp4.quantize(w, p)
    c = fp4.gemm(qx, qw, out_dtype=torch.float32)
    return qx, qw, c


def _same(a, b):
    for qa, qb in zip(a[:2], b[:2]):
        assert torch.equal(qa.codes, qb.codes)
        assert torch.equal(qa.scales, qb.scales)
        if qa.tensor_scale is not None:
            assert torch.equal(qa.tensor_scale, qb.tensor_scale)
    assert torch.equal(a[2], b[2])


@pytest.mark.parametrize("shape", [(384, 256, 512), (512, 768, 1024)])
def test_two_streams_match_serial(shape):
    M, N, K = shape
    rng = np.random.default_rng(11)
    x1, w1 = _bf16(rng, M, K, 1.0), _bf16(rng, N, K, 0.02)
    x2, w2 = _bf16(rng, M, K, 3.0), _bf16(rng, N, K, 0.05)
    p_nv = fp4.Params(block=(1, 16), scale_mode=fp4.SCALE_NV_4OVER6)
    p_mx = fp4.Params(hadamard_n=128)
    r1, r2 = _work(x1, w1, p_nv), _work(x2, w2, p_mx)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(device=DEV), torch.cuda.Stream(device=DEV)
    for _ in range(4):
        with torch.cuda.stream(s1):
            a = _work(x1, w1, p_nv)
        with torch.cuda.stream(s2):
            b = _work(x2, w2, p_mx)
        torch.cuda.synchronize()
        _same(a, r1)
        _same(b, r2)
