"""How often the reciprocal reading of "divide by the scale" changes a code.

Where a block scale d is not a power of two (fp32 scales, NVFP4's E4M3 x fp32 scales), the
quantizer here computes each element as RN(x * RN(1/d)) before the rounding to the element format,
where a literal reading of the caveduck.io post ("FP4라는 무리수": divide the values by the scale,
then round to the grid) would compute RN(x / d). The two can differ by one fp32 ulp, which changes
the code only when x/d lies within an ulp of a rounding boundary of the grid. These tests re-derive
the scales and codes in numpy both ways, pin the re-derivation to the oracle (the reciprocal form
reproduces the oracle's codes exactly), and count the codes that the literal division would change
on the small MXFP4 check (A's per-tensor fp32 scale), the MNIST-MLP study's fp32-scale variants and
a row sample of the NVFP4 + 4/6 tensors (the 4/6 choice re-decided with the divided values).
"""
import numpy as np
import pytest

import oracle as orc
from bit_gemm_fwht_amd import workloads as wl

F32 = np.float32
FLT_MAX = np.finfo(np.float32).max


def unpack(codes):
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)
    out = np.empty(c.size * 2, dtype=np.uint8)
    out[0::2] = c & 0xF
    out[1::2] = c >> 4
    return out


def recip(d):
    """RN(1/d) with 0 -> 0 and an overflowing reciprocal -> FLT_MAX (the quantizer's rule)."""
    d = np.asarray(d, dtype=F32)
    with np.errstate(divide="ignore"):
        r = np.where(d == 0, F32(0), F32(1) / np.where(d == 0, F32(1), d)).astype(F32)
    return np.where(np.isinf(r), FLT_MAX, r).astype(F32)


def divide(x, d):
    d = np.asarray(d, dtype=F32)
    return np.where(d == 0, F32(0), x / np.where(d == 0, F32(1), d)).astype(F32)


def per_element(scales, rows, cols, block):
    br, bc = block
    s = np.asarray(scales, dtype=F32).reshape(rows // br if br <= rows else 1, -1)
    return np.repeat(np.repeat(s, br, axis=0)[:rows], bc, axis=1)[:, :cols]


def f32_case(x, block):
    """(elements, codes changed by the literal division) for the fp32-scale mode."""
    rows, cols = x.shape
    codes, scales, _ = orc.quantize(x, block=block, scale_mode=orc.SCALE_F32)
    d = per_element(scales, rows, cols, block)
    mine = orc.encode((x * recip(d)).astype(F32))
    assert np.array_equal(mine, unpack(codes)), "the reciprocal re-derivation must reproduce the oracle"
    lit = orc.encode(divide(x, d))
    return x.size, int((lit != mine).sum())


def sse16(x, q, d):
    """The fixed-order fp32 SSE of each 16-block: pairwise sums of RN(RN(x - RN(val(q) d))^2)."""
    e = (x - (orc.decode(q).reshape(x.shape) * d).astype(F32)).astype(F32)
    t = (e * e).astype(F32).reshape(-1, 16)
    while t.shape[1] > 1:
        t = (t[:, 0::2] + t[:, 1::2]).astype(F32)
    return t[:, 0]


def nv46_case(x, g):
    """NVFP4 with the 4/6 choice and the given tensor scale g, re-derived both ways."""
    rows, cols = x.shape
    codes, scales, _ = orc.quantize(x, block=(1, 16), scale_mode=orc.SCALE_NV_4OVER6_GIVEN, tensor_scale=g)
    xb = x.reshape(-1, 16)
    amax = np.abs(xb).max(axis=1).astype(F32)
    g = F32(g)
    out = {}
    for name, div in (("recip", False), ("divide", True)):
        cand = []
        for m in (F32(6), F32(4)):
            s = orc.encode((amax / F32(m * g)).astype(F32), elem=orc.E4M3)
            d = (orc.decode(s, elem=orc.E4M3) * g).astype(F32)
            de = np.repeat(d, 16).reshape(xb.shape)
            v = divide(xb, de) if div else (xb * recip(de)).astype(F32)
            q = orc.encode(v).reshape(xb.shape)
            cand.append((s, q, sse16(xb, q, de)))
        four = cand[1][2] < cand[0][2]
        out[name] = (np.where(four, cand[1][0], cand[0][0]), np.where(four[:, None], cand[1][1], cand[0][1]), four)
    s_r, q_r, four_r = out["recip"]
    assert np.array_equal(q_r.reshape(-1), unpack(codes)), "re-derived codes must equal the oracle's"
    assert np.array_equal(s_r, np.asarray(scales).reshape(-1)), "re-derived block scales must equal the oracle's"
    s_d, q_d, four_d = out["divide"]
    return x.size, int((q_d != q_r).sum()), int((four_d != four_r).sum()), four_r.size


def test_tiny_per_tensor_fp32_scale():
    a, _ = wl.tiny_mxfp4(0)
    n, changed = f32_case(a, (256, 256))
    print(f"\nsmall MXFP4 check, A per-tensor fp32 scale: {changed} of {n} codes change")
    assert changed <= n // 1000


@pytest.mark.parametrize("outlier", [False, True], ids=["clean", "outlier"])
def test_mnist_fp32_scales(outlier):
    layers = wl.mnist_mlp(0, outlier=outlier)
    tot = ch = 0
    for name, w in layers.items():
        for gran in ("per_tensor", "per_row", "group32"):
            x = w.reshape(1, -1) if gran == "group32" else w
            block = {"per_tensor": x.shape, "per_row": (1, x.shape[1]), "group32": (1, 32)}[gran]
            n, c = f32_case(np.ascontiguousarray(x), block)
            print(f"\nMNIST-MLP {'outlier' if outlier else 'clean'} {name} {gran}: {c} of {n} codes change")
            tot += n
            ch += c
    assert ch <= tot // 1000


def test_nvfp4_4over6_row_sample():
    xb, wb = wl.nvfp4_4over6(0)
    for name, bits in (("X", xb), ("W", wb)):
        full = wl.bf16_bits_to_f32(bits)
        amax = F32(np.abs(full).max())
        g = F32(amax / F32(2688.0))
        sample = np.ascontiguousarray(full[:256])  # 256 of the 8192 rows
        n, changed, flips, blocks = nv46_case(sample, g)
        print(f"\nNVFP4 + 4/6 {name}, rows 0-255: {changed} of {n} codes change, "
              f"the 4/6 choice flips in {flips} of {blocks} blocks")
        assert changed <= n // 1000
