"""Exhaustive sweeps of the hardware converts the library relies on, through its entry points:

- E2M1 round-to-nearest-even (fp4_quantize, the scaled FP4 convert): every fp32 bit pattern with
  |v| < 8, both signs (subnormals, zeros and the saturating range [6, 8) included), 31 to a group
  beside a 4.0 that fixes the group's floor-rule scale to 2^0, against the oracle's quantize.
- E4M3 round-to-nearest-even (the scaled FP8 convert): every pattern with |v| < 512 beside a 256.0
  (scale 2^0 for E4M3's floor rule; (448, 512) saturates), against the oracle.
- stochastic rounding to E2M1 and to E4M3 over the same two sweeps, with the same group scale pins,
  against the oracle's rule fed the same Philox uniforms (element index within the launch).
- fp32 -> bf16 (the hardware packed convert every bf16 output uses): dequantize with fp32 block
  scales d and unit codes returns bf16(1.0 * d) = bf16(d) for every fp32 pattern d, against torch's
  cast of d (the cast the oracle's bf16 rounding is pinned to).
The element grid and its rounding come from the caveduck.io post's "FP4라는 무리수" (the 15 values)
and OCP E4M3FN; these sweeps replace probes of the instructions with tests of the product path."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from bit_gemm_fwht_amd import fp4

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
ROWS = 1 << 22  # groups per chunk (4M x 32 fp32 = 512 MiB)


def _patterns(start, count, npos):
    """count consecutive sweep indices from start as fp32 bit patterns: [0, npos) are the positive
    patterns 0 .. npos-1, [npos, 2 npos) the same with the sign bit; past 2 npos zeros."""
    i = np.arange(start, start + count, dtype=np.uint64)
    p = np.where(i < npos, i, (i - npos) | np.uint64(0x80000000))
    p = np.where(i < 2 * npos, p, 0)
    return p.astype(np.uint32)


def _oracle_quantize(orc, x, elem, threads=16):
    """The oracle's quantize of [rows, 32] (1 x 32 groups, E8M0 floor, RNE) on row slices in
    parallel (the C oracle releases the interpreter lock)."""
    rows = x.shape[0]
    step = -(-rows // threads)
    with ThreadPoolExecutor(max_workers=threads) as ex:
        parts = list(ex.map(lambda lo: orc.quantize(x[lo:lo + step], elem=elem), range(0, rows, step)))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def _oracle_sr_codes(orc, x, elem, seed, threads=16):
    """The oracle's stochastic rounding of x (a [rows, 32] chunk whose group scales are all 2^0, so
    the elements are the values rounded) with element i of the chunk keyed by index i, packed as
    the library packs codes; row slices in parallel, each with its own first index."""
    flat = x.reshape(-1)
    step = -(-flat.size // threads) // 32 * 32 + 32
    with ThreadPoolExecutor(max_workers=threads) as ex:
        parts = list(ex.map(lambda lo: orc.encode(flat[lo:lo + step], elem=elem, round_mode=orc.ROUND_SR,
                                                   seed=seed, idx0=lo), range(0, flat.size, step)))
    c = np.concatenate(parts)
    return (c[0::2] | (c[1::2] << 4)).astype(np.uint8) if elem == fp4.E2M1 else c


def _sweep(orc, elem, pin, npos, sr_seed=None):
    total = 2 * npos
    groups = -(-total // 31)
    p = fp4.Params(elem=elem) if sr_seed is None else fp4.Params(elem=elem, round_mode=fp4.ROUND_SR, seed=sr_seed)
    done = 0
    for g0 in range(0, groups, ROWS):
        rows = min(ROWS, groups - g0)
        x = np.empty((rows, 32), dtype=np.float32)
        x[:, 0] = pin
        x[:, 1:] = _patterns(g0 * 31, rows * 31, npos).view(np.float32).reshape(rows, 31)
        q = fp4.quantize(torch.from_numpy(x).to(DEV), p)
        torch.cuda.synchronize()
        codes, scales = q.codes.cpu().numpy(), q.scales.cpu().numpy()
        assert np.all(scales == 127), "the pinned group max must give the scale 2^0"
        if sr_seed is None:
            oc, os_ = _oracle_quantize(orc, x, elem)
            assert np.array_equal(scales, os_.reshape(-1))
        else:
            oc = _oracle_sr_codes(orc, x, elem, sr_seed)
        bad = np.nonzero(codes != oc.reshape(-1))[0]
        assert bad.size == 0, f"{bad.size} code bytes differ in groups {g0}..{g0 + rows}, first byte {bad[0]}"
        done += rows
    assert done == groups


@pytest.mark.timeout(900)
def test_e2m1_rne_every_fp32_below_8(orc):
    _sweep(orc, fp4.E2M1, 4.0, 0x41000000)  # 0x41000000 = 8.0


@pytest.mark.timeout(900)
def test_e4m3_rne_every_fp32_below_512(orc):
    _sweep(orc, fp4.E4M3, 256.0, 0x44000000)  # 0x44000000 = 512.0


@pytest.mark.timeout(900)
def test_e2m1_sr_every_fp32_below_8(orc):
    """Stochastic rounding to E2M1 (Philox4x32-10 16-bit uniforms keyed by element index) on every
    fp32 pattern with |v| < 8, against the oracle's rule with the same uniforms."""
    _sweep(orc, fp4.E2M1, 4.0, 0x41000000, sr_seed=0x5EED)


@pytest.mark.timeout(900)
def test_e4m3_sr_every_fp32_below_512(orc):
    _sweep(orc, fp4.E4M3, 256.0, 0x44000000, sr_seed=0x5EED)


@pytest.mark.timeout(900)
def test_bf16_convert_every_fp32_pattern():
    R = 1 << 23  # rows of 32 per chunk: two fp32-scaled blocks of 16 per row, 2^24 scales
    p = fp4.Params(block=(1, 16), scale_mode=fp4.SCALE_F32)
    codes = torch.full((R * 16,), 0x22, dtype=torch.uint8, device=DEV)  # every element 1.0
    y = torch.empty(R, 32, dtype=torch.bfloat16, device=DEV)
    checked = 0
    for c0 in range(0, 1 << 32, 2 * R):
        d = torch.arange(c0, c0 + 2 * R, dtype=torch.int64, device=DEV).to(torch.int32).view(torch.float32)
        q = fp4.QTensor(codes, d.view(torch.uint8), None, R, 32, p)
        fp4.dequantize(q, out=y)
        got = y.view(R * 2, 16)
        ref = d.to(torch.bfloat16)
        nan = torch.isnan(d)
        g0 = got[:, 0]
        same = (g0.view(torch.int16) == ref.view(torch.int16)) | nan
        assert bool(same.all()), f"chunk {c0:#x}: {int((~same).sum())} patterns convert differently"
        assert bool(torch.isnan(g0[nan]).all())
        assert bool((got.view(torch.int16) == got[:, :1].view(torch.int16)).logical_or(nan[:, None]).all())
        checked += 2 * R
    assert checked == 1 << 32
