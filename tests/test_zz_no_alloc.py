"""fp4_quantize_noalloc (no workspace argument: the tensor-amax word lives in the library's static
per-GPU array) against fp4_quantize with a caller workspace and against the oracle, through the C
ABI: two calls in a row, the second on a smaller tensor, for the modes that use the scratch (NVFP4,
4/6, per-tensor fp32 scale) and one that does not (MXFP4)."""
import ctypes

import numpy as np
import pytest
import torch

from bit_gemm_fwht_amd import fp4
from bit_gemm_fwht_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bufs(rows, cols, params):
    cb, sb, wb = fp4.buffer_sizes(rows, cols, params)
    return (torch.full((cb,), 0xAA, dtype=torch.uint8, device=DEV),
            torch.full((max(sb, 1),), 0xAA, dtype=torch.uint8, device=DEV),
            torch.full((1,), -1.0, dtype=torch.float32, device=DEV), wb)


def _noalloc(x, params):
    rows, cols = x.shape
    codes, scales, ts, _ = _bufs(rows, cols, params)
    p = params.c()
    st = fp4.lib().fp4_quantize_noalloc(x.data_ptr(), fp4.DT_BF16, rows, cols, x.stride(0), ctypes.byref(p),
                                        codes.data_ptr(), scales.data_ptr(), ts.data_ptr(),
                                        torch.cuda.current_stream().cuda_stream)
    assert st == fp4.OK, fp4.status_string(st)
    return codes, scales, ts


def _with_workspace(x, params):
    rows, cols = x.shape
    codes, scales, ts, wb = _bufs(rows, cols, params)
    ws = torch.full((max(wb, 1),), 0x55, dtype=torch.uint8, device=DEV)
    p = params.c()
    st = fp4.lib().fp4_quantize(x.data_ptr(), fp4.DT_BF16, rows, cols, x.stride(0), ctypes.byref(p),
                                codes.data_ptr(), scales.data_ptr(), ts.data_ptr(), ws.data_ptr(), wb,
                                torch.cuda.current_stream().cuda_stream)
    assert st == fp4.OK, fp4.status_string(st)
    return codes, scales, ts


MODES = [
    fp4.Params(block=(1, 16), scale_mode=fp4.SCALE_NV_4OVER6),
    fp4.Params(block=(1, 16), scale_mode=fp4.SCALE_NV, hadamard_n=64),
    fp4.Params(hadamard_n=128),
]


@pytest.mark.parametrize("params", MODES, ids=["nvfp4_4over6", "nvfp4_h64", "mxfp4_h128"])
def test_noalloc_matches_quantize(orc, params):
    big, _ = wl.nvfp4_4over6(3, m=320, n=16, k=1024)
    small = big[:96, :512].copy() * np.uint16(1)  # a smaller tensor with a smaller amax
    small = np.ascontiguousarray(small)
    for host in (big, small):  # the second call reuses the scratch the first one left behind
        x = torch.from_numpy(host.view(np.int16)).to(DEV).view(torch.bfloat16)
        got = _noalloc(x, params)
        ref = _with_workspace(x, params)
        torch.cuda.synchronize()
        for g, r in zip(got, ref):
            assert torch.equal(g, r)
        oc, os_, ots = orc.quantize(host, elem=params.elem, block=params.block, scale_mode=params.scale_mode,
                                    round_mode=params.round_mode, hadamard_n=params.hadamard_n, seed=params.seed)
        assert np.array_equal(got[0].cpu().numpy(), oc.reshape(-1))
        assert np.array_equal(got[1].cpu().numpy()[:os_.size], os_.reshape(-1).view(np.uint8))
        if ots is not None:
            assert got[2].cpu().numpy().view(np.uint32)[0] == ots.view(np.uint32)[0]


def test_noalloc_per_tensor_scale(orc):
    """Per-tensor fp32 scale (the tensor amax through the scratch word), larger tensor first."""
    for rows, cols, seed in ((256, 512, 0), (64, 128, 1)):
        host = (np.random.default_rng(seed).standard_normal((rows, cols)) * (4.0 - 3 * seed)).astype(np.float32)
        hb = wl.f32_to_bf16_bits(host)
        x = torch.from_numpy(hb.view(np.int16)).to(DEV).view(torch.bfloat16)
        params = fp4.Params(block=(rows, cols), scale_mode=fp4.SCALE_F32)
        got = _noalloc(x, params)
        ref = _with_workspace(x, params)
        torch.cuda.synchronize()
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1][:4], ref[1][:4])
        oc, os_, _ = orc.quantize(hb, block=(rows, cols), scale_mode=fp4.SCALE_F32)
        assert np.array_equal(got[0].cpu().numpy(), oc.reshape(-1))
        assert got[1][:4].cpu().numpy().view(np.float32)[0] == os_.reshape(-1)[0]
