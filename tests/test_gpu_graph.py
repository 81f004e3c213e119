"""The library's launches captured into a HIP graph (torch.cuda.CUDAGraph): quantize in the modes
whose launches clear or reduce on the device (per-tensor fp32 scale: amax clear + atomic max; NVFP4
with its tensor amax; MXFP4 with H_128 and SR) and the block-scaled GEMM, replayed several times
with eager work and synchronizations in between; every replay equals the eager result. The
library allocates nothing and clears with fill kernels, never hipMemsetAsync, so that a captured
clear replays correctly."""
import numpy as np
import pytest
import torch

from bit_gemm_fwht_amd import fp4

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(seed):
    g = torch.Generator().manual_seed(seed)
    a = (torch.randn(512, 1024, generator=g) * 3).to(DEV)
    b = torch.randn(768, 1024, generator=g).to(torch.bfloat16).to(DEV)
    return a, b


def test_graph_replays_equal_eager():
    a, b = _inputs(0)
    pt = fp4.Params(block=(512, 1024), scale_mode=fp4.SCALE_F32)
    pn = fp4.Params(block=(1, 16), scale_mode=fp4.SCALE_NV_4OVER6)
    pm = fp4.Params(hadamard_n=128, scale_mode=fp4.SCALE_E8M0_CEIL, round_mode=fp4.ROUND_SR, seed=11)
    px = fp4.Params(hadamard_n=128)
    qt = fp4.empty_qtensor(512, 1024, pt, DEV)
    wt = torch.empty(max(fp4.buffer_sizes(512, 1024, pt)[2], 1), dtype=torch.uint8, device=DEV)
    qn = fp4.empty_qtensor(768, 1024, pn, DEV)
    wn = torch.empty(max(fp4.buffer_sizes(768, 1024, pn)[2], 1), dtype=torch.uint8, device=DEV)
    qm = fp4.empty_qtensor(512, 1024, pm, DEV)
    qa = fp4.empty_qtensor(512, 1024, px, DEV)
    qb = fp4.empty_qtensor(768, 1024, px, DEV)
    c = torch.empty(512, 768, dtype=torch.bfloat16, device=DEV)

    def step():
        fp4.quantize(a, pt, out=qt, workspace=wt)
        fp4.quantize(b, pn, out=qn, workspace=wn)
        fp4.quantize(a, pm, out=qm)
        fp4.quantize(a, px, out=qa)
        fp4.quantize(b, px, out=qb)
        fp4.gemm(qa, qb, out=c)

    def snapshot():
        torch.cuda.synchronize()
        return [t.clone() for t in (qt.codes, qt.scales, qn.codes, qn.scales, qn.tensor_scale, qm.codes, qm.scales,
                                    qa.codes, qa.scales, qb.codes, qb.scales, c)]

    step()
    ref = snapshot()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        # eager work between replays: overwrite every output, then replay
        for t in (qt.codes, qn.codes, qm.codes, qa.codes, qb.codes):
            t.fill_(0x5A)
        c.fill_(7.0)
        fp4.quantize(b, px, out=qb)  # an eager launch of the same library between replays
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        for i, (x, y) in enumerate(zip(ref, got)):
            assert torch.equal(x, y), f"replay {rep}: output {i} differs from the eager result"
