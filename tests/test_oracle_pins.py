"""Pins for the CPU oracle: it is checked against what the pages and the mathematics fix, never
against itself. CPU only.

Each test names the passage it pins (page title and section).
"""
import json
import os
import shutil
import subprocess
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg
import torch

from bit_gemm_fwht_amd import workloads as wl

HERE = os.path.dirname(os.path.abspath(__file__))
GOLD = os.path.join(HERE, "golden")


def _grid():
    vals = []
    for line in open(os.path.join(GOLD, "e2m1_grid.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            vals.append(float(line))
    return np.array(vals)


def _unpack(codes, rows, cols):
    lo = codes & 0xF
    hi = codes >> 4
    out = np.empty((rows, cols), dtype=np.uint8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


# ---------------------------------------------------------------------------------------------
# E2M1 grid and encoder (caveduck.io "low-bit quantization": grid equation; round-to-nearest)
# ---------------------------------------------------------------------------------------------
def test_e2m1_decode_matches_printed_grid(orc):
    grid = _grid()
    dec = orc.decode(np.arange(16, dtype=np.uint8))
    assert np.array_equal(dec[:8], grid)
    assert np.array_equal(dec[8:], -grid)
    assert np.signbit(dec[8]) and dec[8] == 0
    assert len(set(dec.tolist())) == 15  # +0 and -0 compare equal: 15 distinct values


def _nearest_bruteforce(v, grid):
    """Nearest grid magnitude by exact rational distances; ties to the even code; |v| > 6 -> 6."""
    out = []
    for x in v:
        a = abs(Fraction(float(x)))
        best, bd = 0, None
        for i, g in enumerate(grid):
            d = abs(a - Fraction(g))
            if bd is None or d < bd or (d == bd and i % 2 == 0):
                best, bd = i, d
        out.append(best | (8 if np.signbit(x) else 0))
    return np.array(out, dtype=np.uint8)


def _e2m1_probe_values():
    grid = _grid()
    pts = []
    # dense windows of fp32 neighbours around every midpoint and every grid point
    centers = list(grid) + [(a + b) / 2 for a, b in zip(grid[:-1], grid[1:])] + [7.0, 8.0]
    for c in centers:
        u = np.float32(c).view(np.uint32).astype(np.int64)
        w = np.arange(u - 40, u + 41, dtype=np.int64)
        w = w[w >= 0]
        pts.append(w.astype(np.uint32).view(np.float32))
    pts.append(np.array([0.0, 1e-45, 1e-40, 1e-20], dtype=np.float32))
    v = np.concatenate(pts)
    return np.concatenate([v, -v])


def test_e2m1_rne_equals_bruteforce_nearest(orc):
    grid = _grid()
    v = _e2m1_probe_values()
    assert np.array_equal(orc.encode(v), _nearest_bruteforce(v, grid))


def test_e2m1_rne_all_bf16_patterns(orc):
    """Every bf16 value (as fp32), brute force in float64: distances to the grid are exact here
    because all bf16 values below 8 have at most 8 significant bits."""
    grid = _grid()
    v = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    v = v[np.isfinite(v)]
    a = np.abs(v.astype(np.float64))
    d = np.abs(a[:, None] - grid[None, :])
    best = np.argmin(d, axis=1)
    # ties: argmin takes the lower index; move to the even index when tied with the next one
    nxt = np.minimum(best + 1, 7)
    tie = (d[np.arange(len(a)), nxt] == d[np.arange(len(a)), best]) & (nxt != best) & (best % 2 == 1)
    best = np.where(tie, nxt, best)
    best = np.where(a > 6, 7, best)
    ref = (best | np.where(np.signbit(v), 8, 0)).astype(np.uint8)
    assert np.array_equal(orc.encode(v), ref)


def test_e2m1_random_fp32_against_threshold_table(orc):
    """Random fp32 (all exponents) against the midpoint-threshold form of the same rule."""
    rng = np.random.default_rng(1)
    u = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    v = u.view(np.float32)
    v = v[np.isfinite(v)]
    a = np.abs(v)
    m = np.select([a <= 0.25, a < 0.75, a <= 1.25, a < 1.75, a <= 2.5, a < 3.5, a <= 5.0],
                  [0, 1, 2, 3, 4, 5, 6], 7).astype(np.uint8)
    ref = m | np.where(np.signbit(v), 8, 0).astype(np.uint8)
    assert np.array_equal(orc.encode(v), ref)


def test_hand_vectors(orc):
    hv = json.load(open(os.path.join(GOLD, "hand_vectors.json")))
    mp = hv["midpoints"]
    assert orc.encode(np.array(mp["v"], dtype=np.float32)).tolist() == mp["codes"]
    for blk in hv["blocks"]:
        x = np.zeros((1, 32), dtype=np.float32)
        x[0, : len(blk["x"])] = blk["x"]
        if blk["x"] == [0.0, -0.0]:
            x[0, 1] = -0.0
        rule = orc.SCALE_E8M0_FLOOR if blk["rule"] == "floor" else orc.SCALE_E8M0_CEIL
        codes, scales, _ = orc.quantize(x, block=(1, 32), scale_mode=rule)
        assert int(scales[0, 0]) - 127 == blk["k"], blk["what"]
        q = _unpack(codes, 1, 32)[0, : len(blk["codes"])]
        assert q.tolist() == blk["codes"], blk["what"]
        if "dequant" in blk:
            y = orc.dequantize(codes, scales, None, 1, 32, scale_mode=rule)
            assert y[0, : len(blk["dequant"])].tolist() == blk["dequant"]


# ---------------------------------------------------------------------------------------------
# E4M3 (the MXFP8 elements and the NVFP4 block scales) and E8M0: library routines
# ---------------------------------------------------------------------------------------------
def test_e4m3_decode_matches_torch(orc):
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(orc.decode(codes, orc.E4M3), ref)


def test_e4m3_rne_matches_torch_in_range(orc):
    rng = np.random.default_rng(2)
    v = np.concatenate([
        (np.arange(65536, dtype=np.uint32) << 16).view(np.float32),
        rng.standard_normal(100_000).astype(np.float32) * np.float32(50),
        rng.standard_normal(100_000).astype(np.float32) * np.float32(0.01),
    ])
    v = v[np.isfinite(v) & (np.abs(v) < 448)]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.encode(v, orc.E4M3), ref)


def test_e4m3_saturates(orc):
    v = np.array([448.0, 449.0, 464.0, 1e6, -500.0, np.float32(3e38)], dtype=np.float32)
    assert orc.encode(v, orc.E4M3).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7E]


def test_bf16_rne_matches_torch(orc):
    """fp32 -> bf16 (round to nearest even) against torch's CPU cast: every fp32 high half (sign,
    exponent, top mantissa bits, so every binade incl. subnormals, +-0 and values near FLT_MAX) with
    the low halves that decide the rounding (0, 1, just below / at / just above the tie, all ones),
    plus 2^22 random fp32 patterns. NaN inputs are checked to stay NaN (payloads are free)."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000], dtype=np.uint32)
    rng = np.random.default_rng(21)
    u = np.concatenate([(hi[:, None] | lows[None, :]).ravel(),
                        rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)])
    v = u.view(np.float32)
    got = orc.bf16_rne(v)
    ref = torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(v)
    assert np.array_equal(got[~nan], ref[~nan])
    g32 = (got[nan].astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.isnan(g32))
    # ties go to the even bf16 mantissa; values past the largest bf16 round to infinity
    assert orc.bf16_rne(np.float32([1.0 + 2.0**-8]))[0] == 0x3F80
    assert orc.bf16_rne(np.float32([1.0 + 3 * 2.0**-8]))[0] == 0x3F82
    assert orc.bf16_rne(np.float32([3.4028235e38]))[0] == 0x7F80


def test_e8m0_decode_matches_torch(orc):
    codes = np.arange(255, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).float().numpy()
    got = np.array([orc.e8m0_value(int(c)) for c in codes], dtype=np.float32)
    assert np.array_equal(got, ref)


def _amax_samples():
    rng = np.random.default_rng(3)
    v = (np.arange(1, 0x7F80, dtype=np.uint32) << 16).view(np.float32)  # all positive bf16
    w = rng.integers(1, 0x7F800000, size=50_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    return np.concatenate([v, w, np.float32([6.0, 6.0000005, 448.0, 3.0, 3.5, 1e-45])])


@pytest.mark.parametrize("elem,maxval,lo_floor", [(0, 6.0, 4.0), (1, 448.0, 256.0)])
def test_e8m0_scale_rules(orc, elem, maxval, lo_floor):
    """Floor rule (tiny MXFP4 check: 2^(floor(log2 amax) - 2)): amax / 2^k lies in [4, 8) for E2M1
    ([256, 512) for E4M3). Truncation-free rule (the 2D-scaling abstract; 2^ceil(log2(amax/6))):
    maxval * 2^k >= amax and maxval * 2^(k-1) < amax."""
    for amax in _amax_samples():
        a = Fraction(float(amax))
        kf = orc.e8m0_scale_exp(float(amax), elem, orc.SCALE_E8M0_FLOOR)
        kc = orc.e8m0_scale_exp(float(amax), elem, orc.SCALE_E8M0_CEIL)
        if -127 < kf < 127:
            r = a / Fraction(2) ** kf
            assert Fraction(lo_floor) <= r < 2 * Fraction(lo_floor), (amax, kf)
        if -127 < kc < 127:
            assert Fraction(maxval) * Fraction(2) ** kc >= a, (amax, kc)
            assert Fraction(maxval) * Fraction(2) ** (kc - 1) < a, (amax, kc)
    assert orc.e8m0_scale_exp(0.0, elem, orc.SCALE_E8M0_FLOOR) == -127
    assert orc.e8m0_scale_exp(1e-45, elem, orc.SCALE_E8M0_FLOOR) == -127


# ---------------------------------------------------------------------------------------------
# Hadamard rotation (caveduck.io post §7; Quartet notes "Hadamard rotation")
# ---------------------------------------------------------------------------------------------
def _c_n_exact(n):
    """RN_fp32(1/sqrt(n)) by exact rational arithmetic."""
    # candidates around the float64 estimate; pick the fp32 nearest to 1/sqrt(n): compare squares
    est = np.float32(1.0 / np.sqrt(n))
    u = int(est.view(np.uint32))
    cands = [np.array([u + d], dtype=np.uint32).view(np.float32)[0] for d in (-2, -1, 0, 1, 2)]
    target = Fraction(1, n)  # compare c^2 with 1/n, monotone in c > 0

    def err(c):
        # |c - 1/sqrt(n)| ordering equals |c^2 - 1/n| ordering only approximately; use exact
        # bracketing: the nearest float is the one whose midpoint interval contains 1/sqrt(n)
        return abs(Fraction(float(c)) ** 2 - target)

    best = min(cands, key=err)
    # verify by midpoints: (best - half ulp)^2 < 1/n < (best + half ulp)^2
    b = Fraction(float(best))
    ulp = Fraction(float(np.nextafter(best, np.float32(1)))) - b
    assert (b - ulp / 2) ** 2 < target < (b + ulp / 2) ** 2
    return best


@pytest.mark.parametrize("n", [2, 4, 8, 16, 32, 64, 128, 256])
def test_fwht_constant_and_unit_vectors(orc, n):
    c = _c_n_exact(n)
    e = np.zeros((1, n), dtype=np.float32)
    e[0, 0] = 1.0
    y = orc.fwht(e, n)
    assert np.all(np.abs(y) == c)  # an outlier spreads to +-1/sqrt(n) on every coordinate
    H = scipy.linalg.hadamard(n)
    for j in [0, n // 2, n - 1]:
        e = np.zeros((1, n), dtype=np.float32)
        e[0, j] = 1.0
        y = orc.fwht(e, n)[0]
        assert np.array_equal(np.sign(y), H[:, j].astype(np.float32))


@pytest.mark.parametrize("n", [2, 4, 8, 16, 32, 64])
def test_fwht_against_explicit_hadamard(orc, n):
    H = scipy.linalg.hadamard(n).astype(np.float64)
    assert np.array_equal(H @ H.T, n * np.eye(n))
    rng = np.random.default_rng(n)
    x = rng.standard_normal((500, n)).astype(np.float32)
    x[::7, 0] *= 50  # outliers
    y = orc.fwht(x, n).astype(np.float64)
    ref = (x.astype(np.float64) @ H.T) / np.sqrt(n)
    # each stage's rounding reaches an output with coefficient +-1; the stage values are bounded
    # by the l1 norm of the chunk. Bound: log2(n) * 2^-24 * ||x||_1 / sqrt(n) + 2 * 2^-24 |y|.
    l1 = np.abs(x.astype(np.float64)).sum(axis=1, keepdims=True)
    bound = np.log2(n) * 2.0**-24 * l1 / np.sqrt(n) + 2 * 2.0**-24 * np.abs(ref)
    assert np.all(np.abs(y - ref) <= bound)


@pytest.mark.parametrize("n", [16, 128, 256])
def test_fwht_orthogonal(orc, n):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((64, 4 * n)).astype(np.float32)
    y = orc.fwht(x, n)
    nx = np.linalg.norm(x.astype(np.float64).reshape(-1, n), axis=1)
    ny = np.linalg.norm(y.astype(np.float64).reshape(-1, n), axis=1)
    assert np.max(np.abs(ny / nx - 1)) < 1e-6
    z = orc.fwht(y, n)  # H/sqrt(n) is symmetric and orthogonal: its own inverse
    assert np.max(np.abs(z - x)) < 1e-5 * np.max(np.abs(x))


def test_rotation_invariance(orc):
    """(x H)(H^T W) = x W (Quartet notes; caveduck.io post §7), blockwise along K."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((8, 256)).astype(np.float32)
    w = rng.standard_normal((16, 256)).astype(np.float32)
    xr = orc.fwht(x, 128).astype(np.float64)
    wr = orc.fwht(w, 128).astype(np.float64)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.allclose(xr @ wr.T, ref, rtol=0, atol=1e-4)


def test_rotation_spreads_outlier_kurtosis():
    """Shape check for the kurtosis drop of §7 (13,717 -> 54 on the trained fc2; values unpinned):
    a 50x outlier in N(0, 0.05^2) weights, rotated with H_256, loses orders of magnitude."""
    import oracle as orc
    w = wl.mnist_mlp(0)["fc2"].copy()
    wl.set_outlier(w)

    def kurt(a):
        a = a.astype(np.float64).ravel()
        a = a - a.mean()
        return float(np.mean(a**4) / np.mean(a**2) ** 2)

    k0 = kurt(w)
    k1 = kurt(orc.fwht(w, 256))
    assert k0 > 1000 and k1 < k0 / 100


# ---------------------------------------------------------------------------------------------
# Outliers, groups, effective bits (caveduck.io post §1-§3)
# ---------------------------------------------------------------------------------------------
def test_per_tensor_outlier_collapse(orc):
    """§1: with S = amax/6 and one 50x outlier, every other |w| <= amax/50 maps below 0.25, so
    exactly one non-zero code remains, and the MSE is the energy of the rest."""
    a, _ = wl.tiny_mxfp4(0)
    codes, scales, _ = orc.quantize(a, block=a.shape, scale_mode=orc.SCALE_F32)
    q = _unpack(codes, *a.shape)
    assert np.count_nonzero(q & 7) == 1
    y = orc.dequantize(codes, scales, None, *a.shape, block=a.shape, scale_mode=orc.SCALE_F32)
    o = np.unravel_index(np.argmax(np.abs(a)), a.shape)
    rest = a.astype(np.float64).copy()
    rest[o] = 0
    mse = np.mean((y.astype(np.float64) - a) ** 2)
    expect = np.sum(rest**2) / a.size + (float(y[o]) - float(a[o])) ** 2 / a.size
    assert abs(mse - expect) <= 1e-6 * expect
    fc1 = wl.mnist_mlp(0, outlier=True)["fc1"]
    c1, _, _ = orc.quantize(fc1, block=fc1.shape, scale_mode=orc.SCALE_F32)
    assert np.count_nonzero(_unpack(c1, *fc1.shape) & 7) == 1


def test_group_containment(orc):
    """§2: with 32-element groups the outlier's damage stays in its group: every other group has
    identical codes and scales, and its 31 neighbours become +-0 (|w|/d < 8/50 < 0.25)."""
    clean = wl.mnist_mlp(0)["fc1"].reshape(1, -1)
    dirty = wl.mnist_mlp(0, outlier=True)["fc1"].reshape(1, -1)
    o = int(np.argmax(np.abs(dirty)))
    g = o // 32
    c0, s0, _ = orc.quantize(clean, block=(1, 32))
    c1, s1, _ = orc.quantize(dirty, block=(1, 32))
    q0 = _unpack(c0, 1, clean.size)[0].reshape(-1, 32)
    q1 = _unpack(c1, 1, clean.size)[0].reshape(-1, 32)
    keep = np.arange(q0.shape[0]) != g
    assert np.array_equal(q0[keep], q1[keep])
    assert np.array_equal(s0[0, keep], s1[0, keep])
    nb = np.delete(q1[g], o % 32)
    assert np.all((nb & 7) == 0)


def test_effective_bits(orc):
    """§3: MXFP4 costs 4 + 8/32 = 4.25 bits per element; fc1 (200,704 weights) has 6,272 groups."""
    fc1 = wl.mnist_mlp(0)["fc1"].reshape(1, -1)
    codes, scales, _ = orc.quantize(fc1, block=(1, 32))
    assert scales.size == 6272
    assert (codes.nbytes + scales.nbytes) * 8 == 4.25 * fc1.size
    c2, s2, ts = orc.quantize(fc1, block=(1, 16), scale_mode=orc.SCALE_NV)
    assert (c2.nbytes + s2.nbytes + ts.nbytes) * 8 == 4.5 * fc1.size + 32


def test_mse_table_shapes(orc):
    """Shapes of tables T1/T2 of §1 and §3 on random stand-ins for the trained MLP (the printed
    values themselves are unpinned: the trained weights are not available)."""
    def mse(x, block, mode):
        c, s, t = orc.quantize(x, block=block, scale_mode=mode)
        y = orc.dequantize(c, s, t, *x.shape, block=block, scale_mode=mode)
        return float(np.mean((y.astype(np.float64) - x) ** 2))

    clean = wl.mnist_mlp(0)["fc1"]
    dirty = wl.mnist_mlp(0, outlier=True)["fc1"]
    flat_c, flat_d = clean.reshape(1, -1), dirty.reshape(1, -1)
    pt = mse(dirty, dirty.shape, orc.SCALE_F32) / mse(clean, clean.shape, orc.SCALE_F32)
    pr = mse(dirty, (1, 784), orc.SCALE_F32) / mse(clean, (1, 784), orc.SCALE_F32)
    pg = mse(flat_d, (1, 32), orc.SCALE_F32) / mse(flat_c, (1, 32), orc.SCALE_F32)
    assert pt > 10 and pr < 1.5 and pg < 1.2
    ratio = mse(flat_c, (1, 32), orc.SCALE_E8M0_FLOOR) / mse(flat_c, (1, 32), orc.SCALE_F32)
    assert 1.0 <= ratio <= 1.6


# ---------------------------------------------------------------------------------------------
# 2D blocks (transposition invariance), truncation-free scaling (2D-scaling abstract)
# ---------------------------------------------------------------------------------------------
def test_2d_scales_transposition_invariant(orc):
    w, _ = wl.backward_2d(0, m=32, n=256, k=512)
    wf = wl.bf16_bits_to_f32(w).reshape(256, 512)
    for mode in (orc.SCALE_E8M0_FLOOR, orc.SCALE_E8M0_CEIL):
        c, s, _ = orc.quantize(wf, block=(32, 32), scale_mode=mode)
        ct, st, _ = orc.quantize(np.ascontiguousarray(wf.T), block=(32, 32), scale_mode=mode)
        assert np.array_equal(s.T, st)
        assert np.array_equal(_unpack(c, 256, 512).T, _unpack(ct, 512, 256))
    # 1D groups are not transposition invariant (the instability the abstract names)
    c, s, _ = orc.quantize(wf, block=(1, 32))
    ct, st, _ = orc.quantize(np.ascontiguousarray(wf.T), block=(1, 32))
    assert not np.array_equal(_unpack(c, 256, 512).T, _unpack(ct, 512, 256))


@pytest.mark.parametrize("elem,maxval", [(0, 6.0), (1, 448.0)])
def test_truncation_free_never_saturates(orc, elem, maxval):
    w, dy = wl.backward_2d(0, m=64, n=64, k=256)
    x = wl.bf16_bits_to_f32(dy).reshape(64, 256)
    for rnd in (orc.ROUND_RNE, orc.ROUND_SR):
        c, s, _ = orc.quantize(x, elem=elem, block=(1, 32), scale_mode=orc.SCALE_E8M0_CEIL,
                               round_mode=rnd, seed=7)
        d = np.repeat(np.array([[orc.e8m0_value(int(v)) for v in row] for row in s]), 32, axis=1)
        v = x / d
        assert np.all(np.abs(v) <= maxval)


# ---------------------------------------------------------------------------------------------
# Stochastic rounding and Philox
# ---------------------------------------------------------------------------------------------
def test_philox_against_rocrand():
    """Philox4x32-10 (Salmon et al., SC'11) against rocRAND's open-source header implementation."""
    import oracle as orc
    hdr = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"
    if not os.path.exists(hdr) or shutil.which("g++") is None:
        pytest.skip("rocRAND header or g++ missing: Philox parity unpinned")
    exe = os.path.join(HERE, "_philox_pin.bin")
    subprocess.run(["g++", "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    os.path.join(HERE, "philox_rocrand_pin.cpp"), "-o", exe], check=True)
    try:
        rng = np.random.default_rng(5)
        ctr = rng.integers(0, 2**32, size=(2000, 4), dtype=np.uint64).astype(np.uint32)
        key = rng.integers(0, 2**32, size=(2000, 2), dtype=np.uint64).astype(np.uint32)
        ctr[0] = 0
        key[0] = 0
        ctr[1] = 0xFFFFFFFF
        key[1] = 0xFFFFFFFF
        inp = "\n".join(" ".join(str(int(v)) for v in list(c) + list(k)) for c, k in zip(ctr, key))
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
        ref = np.array([[int(t) for t in line.split()] for line in out.strip().splitlines()],
                       dtype=np.uint32)
    finally:
        os.remove(exe)
    assert np.array_equal(orc.philox(ctr, key), ref)


def test_sr_bits_layout(orc):
    """8 elements per Philox call: element idx takes half (idx & 1) of word (idx >> 1) & 3 of the
    block for counter idx >> 3 under key = seed."""
    seed = 0x123456789ABCDEF
    idx = np.arange(64, dtype=np.uint64) + np.uint64(2**40)
    u = orc.sr_u16(seed, idx)
    for i, ix in enumerate(idx.tolist()):
        g = ix >> 3
        blk = orc.philox(np.array([[g & 0xFFFFFFFF, g >> 32, 0, 0]]),
                         np.array([[seed & 0xFFFFFFFF, seed >> 32]]))[0]
        w = int(blk[(ix >> 1) & 3])
        assert u[i] == ((w >> 16) if ix & 1 else (w & 0xFFFF))


@pytest.mark.parametrize("elem", [0, 1])
def test_sr_exact_expectation(orc, elem):
    """Enumerating all 2^16 uniforms: P(up) = ceil(p 2^16) / 2^16, so the bias is at most 2^-16 of
    the local gap, and zero when p 2^16 is an integer; every result is one of the two neighbours."""
    grid = np.unique(np.abs(orc.decode(np.arange(256 if elem else 16, dtype=np.uint8), elem)))
    grid = grid[np.isfinite(grid)]
    rng = np.random.default_rng(9)
    vmax = 6.0 if elem == 0 else 448.0
    vs = np.concatenate([rng.uniform(-vmax, vmax, 40).astype(np.float32), np.float32([0.3, 2.5, -5.5])])
    u = np.arange(65536, dtype=np.uint32)
    for v in vs:
        a = abs(float(v))
        lo = grid[grid <= a].max()
        hi = grid[grid > a].min()
        codes = orc.sr_with_u(np.full(u.size, v, dtype=np.float32), u, elem)
        vals = np.abs(orc.decode(codes, elem).astype(np.float64))
        assert set(np.unique(vals)) <= {float(lo), float(hi)}
        p = Fraction(a) - Fraction(float(lo))
        p /= Fraction(float(hi)) - Fraction(float(lo))
        n_up = int(np.count_nonzero(vals == hi))
        assert n_up == -(-p * 65536 // 1)  # ceil(p * 2^16)


def test_sr_unbiased_over_seeds(orc):
    """Mean over 10^4 seeds is within 5 sigma of the input for every element."""
    rng = np.random.default_rng(4)
    x = rng.uniform(-5.9, 5.9, size=(1, 32)).astype(np.float32)
    x[0, 0] = 0.1
    x[0, 1] = 5.5
    acc = np.zeros(32)
    acc2 = np.zeros(32)
    n = 10_000
    for seed in range(n):
        c, s, _ = orc.quantize(x, block=(1, 32), scale_mode=orc.SCALE_E8M0_CEIL,
                               round_mode=orc.ROUND_SR, seed=seed)
        y = orc.dequantize(c, s, None, 1, 32, scale_mode=orc.SCALE_E8M0_CEIL)[0].astype(np.float64)
        acc += y
        acc2 += y * y
    mean = acc / n
    sd = np.sqrt(np.maximum(acc2 / n - mean**2, 0)) / np.sqrt(n)
    assert np.all(np.abs(mean - x[0]) <= 5 * sd + 1e-12)


# ---------------------------------------------------------------------------------------------
# NVFP4 and 4/6 (Four Over Six summary: methodology)
# ---------------------------------------------------------------------------------------------
def test_4over6_never_worse_than_plain_nvfp4(orc):
    x, _ = wl.nvfp4_4over6(0, m=64, n=16, k=512)
    xf = wl.bf16_bits_to_f32(x).reshape(64, 512)
    out = {}
    for mode in (orc.SCALE_NV, orc.SCALE_NV_4OVER6):
        c, s, t = orc.quantize(xf, block=(1, 16), scale_mode=mode)
        y = orc.dequantize(c, s, t, 64, 512, block=(1, 16), scale_mode=mode)
        out[mode] = (((y.astype(np.float64) - xf) ** 2).reshape(-1, 16).sum(axis=1), s, t)
    sse6, s6, t6 = out[orc.SCALE_NV]
    sse46, s46, t46 = out[orc.SCALE_NV_4OVER6]
    assert t6[0] == t46[0]
    assert np.all(sse46 <= sse6 * (1 + 1e-5) + 1e-30)
    changed = (s6 != s46).ravel()
    assert 0 < changed.mean() < 1          # both candidates are taken somewhere
    assert np.all(sse46[changed] < sse6[changed] * (1 + 1e-5))


def test_nvfp4_scales(orc):
    """g = amax_t / (6 * 448); block scale E4M3(amax_b / (6 g)) maps the block max near 6."""
    x, _ = wl.nvfp4_4over6(0, m=32, n=16, k=256)
    xf = wl.bf16_bits_to_f32(x).reshape(32, 256)
    c, s, t = orc.quantize(xf, block=(1, 16), scale_mode=orc.SCALE_NV)
    amax_t = np.float32(np.abs(xf).max())
    assert t[0] == np.float32(amax_t / np.float32(2688))
    amax_b = np.abs(xf).reshape(-1, 16).max(axis=1)
    tt = (amax_b.astype(np.float32) / (np.float32(6) * t[0])).astype(np.float32)
    ref = torch.from_numpy(np.minimum(tt, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(s.ravel(), ref)


def test_nvfp4_fp8_rescale_is_exact_when_scales_are_powers_of_two(orc):
    """The FP8 re-expression of NVFP4 operands is lossless when both 16-block scales of a 32-group
    are equal powers of two (E4M3 then holds every value val(q) * s * 2^-E exactly)."""
    rng = np.random.default_rng(8)
    rows, K = 8, 128
    codes = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    e = rng.integers(-6, 8, size=(rows, K // 32))
    svals = np.repeat(2.0 ** e, 2, axis=1).astype(np.float32)
    scales = torch.from_numpy(svals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ts = np.float32([0.75])
    a = orc.operand_f64(codes, scales, ts, rows, K, block=(1, 16), scale_mode=orc.SCALE_NV)
    b = orc.operand_f64(codes, scales, ts, rows, K, block=(1, 16), scale_mode=orc.SCALE_NV,
                        nv_exact=True)
    assert np.array_equal(a, b)


def _e2m1_exact(code):
    """E2M1 value of a code as an exact fraction, from the grid the page prints."""
    mag = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
           Fraction(4), Fraction(6)][code & 7]
    return -mag if code & 8 else mag


def _e4m3_exact(code):
    """E4M3FN value (finite codes) as an exact fraction: bias 7, subnormal step 2^-9."""
    e, m = (code >> 3) & 15, code & 7
    v = Fraction(m, 512) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)
    return -v if code & 0x80 else v


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_nvfp4_fp8_rescale_rule(orc, seed):
    """The re-expression NVFP4 -> E4M3 elements under one power-of-two scale per 32-wide K group,
    checked in exact arithmetic: per group, 448 * 2^E >= 6 S > 448 * 2^(E-1) (E is the smallest
    such exponent; S the group's larger block scale), E = -127 for S = 0, and every element is the
    E4M3 nearest-even rounding (torch's float8_e4m3fn cast) of the exact val(q) * s_blk * 2^-E.
    Scale codes cover E4M3 subnormals, zero and the largest code; an E one too large or too small,
    a swapped block scale or another rounding fails here."""
    rng = np.random.default_rng(100 + seed)
    rows, K = 24, 256
    codes = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, size=(rows, K // 16), dtype=np.uint8)  # 0x00 .. 0x7E
    scales[0, :4] = 0                      # two all-zero groups
    scales[1, :2] = [1, 2]                 # subnormal block scales
    scales[2, :2] = [0x7E, 0x7E]           # the largest scale
    scales[3, :2] = [0x08, 0x01]           # 2^-6 next to the smallest subnormal
    f8, e8 = orc.nv_to_mx8(codes, scales, rows, K)
    nib = np.empty((rows, K), dtype=np.uint8)
    nib[:, 0::2] = codes & 0xF
    nib[:, 1::2] = codes >> 4
    two = Fraction(2)
    for r in range(rows):
        for g in range(K // 32):
            s = [_e4m3_exact(int(scales[r, 2 * g])), _e4m3_exact(int(scales[r, 2 * g + 1]))]
            S = max(s)
            E = int(e8[r, g]) - 127
            if S == 0:
                assert E == -127
            else:
                assert 448 * two ** E >= 6 * S > 448 * two ** (E - 1), (r, g, E, S)
            args = []
            for j in range(32):
                t = _e2m1_exact(int(nib[r, 32 * g + j])) * s[j // 16] * two ** (-E)
                assert abs(t) <= 448
                tf = np.float32(float(t))
                assert Fraction(float(tf)) == t  # the argument is exact in fp32
                if t == 0 and nib[r, 32 * g + j] & 8:
                    tf = np.float32(-0.0)
                args.append(tf)
            ref = torch.from_numpy(np.array(args, dtype=np.float32)).to(torch.float8_e4m3fn)
            ref = ref.view(torch.uint8).numpy()
            assert np.array_equal(f8[r, 32 * g:32 * g + 32], ref), (r, g)
    # the GEMM reference multiplies exactly these values
    ts = np.float32([0.375])
    a = orc.operand_f64(codes, scales, ts, rows, K, block=(1, 16), scale_mode=orc.SCALE_NV)
    e4 = torch.from_numpy(f8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(a, e4 * np.repeat(2.0 ** (e8.astype(np.float64) - 127), 32, axis=1) * 0.375)


# ---------------------------------------------------------------------------------------------
# Dequantize and the GEMM reference
# ---------------------------------------------------------------------------------------------
def test_dequantize_round_trip_of_grid_values(orc):
    """Values already on the grid times a power of two come back exactly."""
    rng = np.random.default_rng(6)
    grid = _grid()
    q = rng.integers(0, 8, size=(16, 64))
    sign = np.where(rng.random((16, 64)) < 0.5, -1.0, 1.0)
    k = rng.integers(-20, 20, size=(16, 2))
    x = (sign * grid[q] * np.repeat(2.0 ** k, 32, axis=1)).astype(np.float32)
    x[:, ::32] = np.repeat(6.0 * 2.0 ** k, 1, axis=1)  # block max 6 * 2^k so that the floor rule gives k
    c, s, _ = orc.quantize(x, block=(1, 32))
    assert np.array_equal(s.astype(np.int64) - 127, k)
    y = orc.dequantize(c, s, None, 16, 64)
    assert np.array_equal(y, x)


def test_gemm_reference_against_numpy(orc):
    a, b = wl.tiny_mxfp4(0)
    ca, sa, _ = orc.quantize(a, block=(1, 32))
    cb, sb, _ = orc.quantize(b, block=(1, 32))
    A = orc.operand_f64(ca, sa, None, 256, 256)
    B = orc.operand_f64(cb, sb, None, 256, 256)
    assert np.array_equal(A, orc.dequantize(ca, sa, None, 256, 256).astype(np.float64))
    c, s = orc.gemm_f64(A, B)
    assert np.allclose(c, A @ B.T, rtol=1e-13, atol=1e-9)
    assert np.allclose(s, np.abs(A) @ np.abs(B).T, rtol=1e-13)
    ms = np.array([0, 5, 255])
    ns = np.array([3, 0, 255])
    c2, s2 = orc.gemm_f64_sampled(A, B, ms, ns)
    assert np.array_equal(c2, c[ms, ns]) and np.array_equal(s2, s[ms, ns])


def test_nvfp4_given_tensor_scale(orc):
    """Delayed NVFP4 scaling (the caller's tensor scale g): with g equal to the tensor's own
    amax / 2688 it reduces to plain NVFP4 (and 4/6), byte for byte; with g far below that every
    block scale saturates to the largest E4M3 value (code 0x7E) and the block's largest elements to
    +-6; 4/6 is never worse than its 6-only counterpart per block."""
    rng = np.random.default_rng(17)
    x = (rng.laplace(size=(16, 128)) * 3).astype(np.float32)
    for plain, given in ((orc.SCALE_NV, orc.SCALE_NV_GIVEN), (orc.SCALE_NV_4OVER6, orc.SCALE_NV_4OVER6_GIVEN)):
        c0, s0, t0 = orc.quantize(x, block=(1, 16), scale_mode=plain)
        c1, s1, t1 = orc.quantize(x, block=(1, 16), scale_mode=given, tensor_scale=t0[0])
        assert np.array_equal(c0, c1) and np.array_equal(s0, s1) and t1[0] == t0[0]
    amax_b = np.abs(x).reshape(16, 8, 16).max(axis=-1)
    g_small = float(amax_b.min()) / (6 * 448 * 100)
    c, s, _ = orc.quantize(x, block=(1, 16), scale_mode=orc.SCALE_NV_GIVEN, tensor_scale=g_small)
    assert np.all(s == 0x7E)
    mag = np.stack([c & 0xF, c >> 4], axis=-1).reshape(16, 8, 16) & 7
    arg = np.abs(x).reshape(16, 8, 16).argmax(axis=-1)
    assert np.all(np.take_along_axis(mag, arg[..., None], -1) == 7)
    g = float(np.abs(x).max()) / 2688 * 0.37
    c6, s6, _ = orc.quantize(x, block=(1, 16), scale_mode=orc.SCALE_NV_GIVEN, tensor_scale=g)
    c46, s46, _ = orc.quantize(x, block=(1, 16), scale_mode=orc.SCALE_NV_4OVER6_GIVEN, tensor_scale=g)
    gt = np.array([g], np.float32)
    y6 = orc.dequantize(c6, s6, gt, 16, 128, block=(1, 16), scale_mode=orc.SCALE_NV_GIVEN)
    y46 = orc.dequantize(c46, s46, gt, 16, 128, block=(1, 16), scale_mode=orc.SCALE_NV_4OVER6_GIVEN)
    e6 = ((y6.astype(np.float64) - x) ** 2).reshape(16, 8, 16).sum(-1)
    e46 = ((y46.astype(np.float64) - x) ** 2).reshape(16, 8, 16).sum(-1)
    assert np.all(e46 <= e6 * (1 + 1e-6) + 1e-30)
