"""GPU parity: the HIP path (called through the C ABI) against the CPU oracle on the same seeded
inputs. Codes, scales and tensor scales must be bit-identical (stochastic rounding included);
dequantized values and rotations bit-identical; GEMM outputs within
|C - C_ref| <= 1e-5 * sum_k |a_k b_k| (+ half a bf16 ulp of C_ref for bf16 outputs)."""
import numpy as np
import pytest
import torch

from bit_gemm_fwht_amd import fp4
from bit_gemm_fwht_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _to_dev(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def _gpu_quant(x: np.ndarray, params: fp4.Params):
    xt = _to_dev(x)
    q = fp4.quantize(xt, params)
    torch.cuda.synchronize()
    codes = q.codes.cpu().numpy()
    scales = q.scales.cpu().numpy()
    ts = q.tensor_scale.cpu().numpy() if q.tensor_scale is not None else None
    return q, codes, scales, ts


def _orc_quant(orc, x, params: fp4.Params):
    return orc.quantize(x, elem=params.elem, block=params.block, scale_mode=params.scale_mode,
                        round_mode=params.round_mode, hadamard_n=params.hadamard_n, seed=params.seed)


def _check_quant(orc, x, params, check_dequant=True):
    q, gc, gs, gts = _gpu_quant(x, params)
    oc, os_, ots = _orc_quant(orc, x, params)
    oc = oc.reshape(-1)
    os_ = os_.reshape(-1).view(np.uint8)
    assert gc.shape == oc.shape and gs.shape == os_.shape
    bad = np.nonzero(gc != oc)[0]
    assert bad.size == 0, f"{bad.size} code bytes differ, first at {bad[:8]}: gpu {gc[bad[:8]]} oracle {oc[bad[:8]]}"
    bad = np.nonzero(gs != os_)[0]
    assert bad.size == 0, f"{bad.size} scale bytes differ, first at {bad[:8]}: gpu {gs[bad[:8]]} oracle {os_[bad[:8]]}"
    if ots is not None:
        assert gts.view(np.uint32)[0] == ots.view(np.uint32)[0]
    if check_dequant:
        rows, cols = x.shape
        oc2, os2, ots2 = _orc_quant(orc, x, params)
        ref = orc.dequantize(oc2, os2, ots2, rows, cols, elem=params.elem, block=params.block,
                             scale_mode=params.scale_mode, hadamard_n=params.hadamard_n)
        for dt in (torch.float32, torch.bfloat16):
            y = fp4.dequantize(q, dtype=dt)
            torch.cuda.synchronize()
            if dt == torch.float32:
                got = y.cpu().numpy()
                bad = np.nonzero(got.view(np.uint32) != ref.view(np.uint32))
                assert bad[0].size == 0, f"dequant differs at {bad[0][:4]}, {bad[1][:4]}"
            else:
                got = y.view(torch.int16).cpu().numpy().view(np.uint16)
                assert np.array_equal(got, orc.bf16_rne(ref))
    return q


def _mix(rows, cols, seed, dtype="bf16", scale=1.0):
    """N(0, scale^2) with a few outliers, exact midpoints, zeros and tiny values mixed in."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, cols)) * scale).astype(np.float32)
    flat = x.reshape(-1)
    n = flat.size
    idx = rng.choice(n, size=max(n // 50, 1), replace=False)
    flat[idx[: len(idx) // 4]] *= 40
    flat[idx[len(idx) // 4: len(idx) // 2]] = 0.0
    flat[idx[len(idx) // 2: 3 * len(idx) // 4]] = -0.0
    flat[idx[3 * len(idx) // 4:]] = rng.choice(np.float32([0.25, 0.75, 1.25, 2.5, 3.5, 5.0, 1e-39, -1e-42]),
                                               size=len(idx) - 3 * len(idx) // 4)
    if dtype == "bf16":
        return wl.f32_to_bf16_bits(x)
    return x


P = fp4.Params
E2M1, E4M3 = fp4.E2M1, fp4.E4M3
FLOOR, CEIL, NV, NV46, F32 = (fp4.SCALE_E8M0_FLOOR, fp4.SCALE_E8M0_CEIL, fp4.SCALE_NV,
                              fp4.SCALE_NV_4OVER6, fp4.SCALE_F32)
RNE, SR = fp4.ROUND_RNE, fp4.ROUND_SR


# ---------------------------------------------------------------------------------------------
# quantize / dequantize parity
# ---------------------------------------------------------------------------------------------
def test_tiny_mxfp4_check(orc):
    """Tiny MXFP4 check: A, B 256x256 N(0,1) with a 50x outlier in A; group 32, E8M0 floor, RNE."""
    a, b = wl.tiny_mxfp4(0)
    _check_quant(orc, a, P())
    _check_quant(orc, b, P())
    # per-tensor S = amax / 6 on A: the outlier collapse
    q = _check_quant(orc, a, P(block=a.shape, scale_mode=F32))
    codes = q.codes.cpu().numpy()
    nz = np.count_nonzero(codes & 0x7) + np.count_nonzero((codes >> 4) & 0x7)
    assert nz == 1


SEG_CASES = []
for dt in ("bf16", "f32"):
    for hn in (0, 16, 32, 64, 128, 256):
        for elem in (E2M1, E4M3):
            for sm in (FLOOR, CEIL):
                for rnd in (RNE, SR):
                    SEG_CASES.append((dt, hn, elem, sm, rnd))


@pytest.mark.parametrize("dt,hn,elem,sm,rnd", SEG_CASES)
def test_group32_parity(orc, dt, hn, elem, sm, rnd):
    # 37 rows x 512 columns = 592 lanes: three workgroups, the last one ragged
    x = _mix(37, 512, seed=hn + 7 * elem + 13 * sm + 29 * rnd, dtype=dt)
    _check_quant(orc, x, P(elem=elem, scale_mode=sm, round_mode=rnd, hadamard_n=hn, seed=12345))


@pytest.mark.parametrize("elem,sm,rnd,hn", [(E2M1, FLOOR, RNE, 0), (E2M1, CEIL, SR, 128),
                                            (E4M3, FLOOR, RNE, 64), (E2M1, F32, RNE, 0),
                                            (E2M1, F32, SR, 32), (E4M3, F32, RNE, 256)])
def test_group16_and_f32_scales(orc, elem, sm, rnd, hn):
    x = _mix(40, 768, seed=3, dtype="bf16")
    _check_quant(orc, x, P(elem=elem, block=(1, 16), scale_mode=sm, round_mode=rnd, hadamard_n=hn, seed=9))
    _check_quant(orc, x, P(elem=elem, block=(1, 32), scale_mode=sm, round_mode=rnd, hadamard_n=hn, seed=9))


@pytest.mark.parametrize("cols", [512, 288])
@pytest.mark.parametrize("elem,sm,rnd,hn", [(E2M1, FLOOR, RNE, 0), (E2M1, CEIL, RNE, 32),
                                            (E2M1, CEIL, SR, 0), (E4M3, CEIL, SR, 32),
                                            (E2M1, CEIL, RNE, 128)])
def test_2d_parity(orc, cols, elem, sm, rnd, hn):
    if cols % max(hn, 1):
        pytest.skip("rotation size does not divide the width")
    x = _mix(96, cols, seed=5, dtype="bf16", scale=0.02)
    _check_quant(orc, x, P(elem=elem, block=(32, 32), scale_mode=sm, round_mode=rnd, hadamard_n=hn, seed=7))


@pytest.mark.parametrize("sm,rnd,hn", [(NV, RNE, 0), (NV46, RNE, 0), (NV, SR, 0), (NV46, RNE, 128),
                                        (NV, RNE, 64)])
def test_nvfp4_parity(orc, sm, rnd, hn):
    x, _ = wl.nvfp4_4over6(0, m=48, n=16, k=1024)
    _check_quant(orc, x, P(block=(1, 16), scale_mode=sm, round_mode=rnd, hadamard_n=hn, seed=3))


@pytest.mark.parametrize("outlier", [False, True])
@pytest.mark.parametrize("elem,sm,rnd", [(E2M1, F32, RNE), (E2M1, FLOOR, RNE), (E2M1, CEIL, SR),
                                         (E4M3, FLOOR, RNE), (E4M3, F32, SR)])
def test_mnist_mlp_granularities(orc, outlier, elem, sm, rnd):
    """MNIST-MLP-shaped weights: per-tensor, per-row and flattened group-32 scales."""
    w = wl.mnist_mlp(0, outlier=outlier)
    for name, x in w.items():
        rows, cols = x.shape
        _check_quant(orc, x, P(elem=elem, block=(rows, cols), scale_mode=sm, round_mode=rnd, seed=1))
        _check_quant(orc, x, P(elem=elem, block=(1, cols), scale_mode=sm, round_mode=rnd, seed=1))
        flat = x.reshape(1, -1)
        _check_quant(orc, flat, P(elem=elem, block=(1, 32), scale_mode=sm, round_mode=rnd, seed=1))


def test_degenerate_inputs(orc):
    z = np.zeros((32, 256), dtype=np.float32)
    z[1, ::2] = -0.0
    for params in (P(), P(scale_mode=CEIL, round_mode=SR), P(block=(1, 16), scale_mode=NV46),
                   P(block=(32, 32)), P(elem=E4M3), P(block=(32, 256), scale_mode=F32),
                   P(hadamard_n=256)):
        _check_quant(orc, z, params)
    tiny = np.full((32, 256), 1e-40, dtype=np.float32)
    tiny[:, ::3] = -3e-39
    tiny[:, 1::7] = 1e-45
    for params in (P(), P(scale_mode=CEIL), P(elem=E4M3), P(scale_mode=CEIL, round_mode=SR),
                   P(block=(1, 16), scale_mode=NV)):
        _check_quant(orc, tiny, params)
    big = np.full((32, 256), 3e38, dtype=np.float32)
    big[:, ::2] = -1.7e38
    for params in (P(), P(scale_mode=CEIL), P(elem=E4M3, scale_mode=CEIL)):
        _check_quant(orc, big, params)
    one = _mix(1, 32, seed=1, dtype="f32")
    _check_quant(orc, one, P())


def test_hadamard_parity(orc):
    for hn in (16, 32, 64, 128, 256):
        x = _mix(19, 1024, seed=hn, dtype="f32")
        y = fp4.hadamard(_to_dev(x), hn)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint32), orc.fwht(x, hn).view(np.uint32))
        xb = _mix(19, 1024, seed=hn, dtype="bf16")
        y = fp4.hadamard(_to_dev(xb), hn)
        ref = orc.fwht(wl.bf16_bits_to_f32(xb).reshape(19, 1024), hn)
        assert np.array_equal(y.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_sr_seed_reproducible_and_distinct():
    x = _to_dev(_mix(64, 512, seed=2, dtype="bf16"))
    p = P(scale_mode=CEIL, round_mode=SR, seed=7)
    a = fp4.quantize(x, p).codes.cpu().numpy()
    b = fp4.quantize(x, p).codes.cpu().numpy()
    c = fp4.quantize(x, P(scale_mode=CEIL, round_mode=SR, seed=8)).codes.cpu().numpy()
    assert np.array_equal(a, b) and not np.array_equal(a, c)


# ---------------------------------------------------------------------------------------------
# GEMM parity
# ---------------------------------------------------------------------------------------------
def fp8_alignment_term(a64, b64, im, inn, K, chunk=2048):
    """The FP8 matrix core's alignment loss bound for outputs (im[i], inn[i]): per aligned block of 8
    consecutive K products, with e = floor(log2 max |a_k b_k|) over the block, each product is
    truncated toward zero to a multiple of 2^(e - 13) (test_fp8_matrix_core_alignment_model pins
    this on crafted operands), so the block loses at most sum_k min(|a_k b_k|, 2^(e - 13))."""
    out = np.empty(len(im))
    for lo in range(0, len(im), chunk):
        p = np.abs(a64[im[lo:lo + chunk]] * b64[inn[lo:lo + chunk]]).reshape(-1, K // 8, 8)
        pm = p.max(axis=-1, keepdims=True)
        e = np.floor(np.log2(np.where(pm > 0, pm, 1.0)))
        unit = np.where(pm > 0, 2.0 ** (e - 13), 0.0)
        out[lo:lo + chunk] = np.minimum(p, unit).sum(axis=(-1, -2))
    return out


def _gemm_tol(ref, sabs, a64, b64, im, inn, params_a, K, c_dtype):
    """Per-output bound for outputs (im[i], inn[i]): 1e-5 * sum |a_k b_k|, plus half a bf16 ulp for
    bf16 outputs, plus, for operands multiplied on the FP8 matrix core (MXFP8, NVFP4 through its
    FP8 re-expression), the alignment loss of that matrix core (fp8_alignment_term). FP4 products
    of one 32-group span less than 2^8 and are summed exactly, so MXFP4 takes no such term."""
    tol = 1e-5 * sabs
    if params_a.elem == E4M3 or params_a.scale_mode in fp4.NV_MODES:
        tol = tol + fp8_alignment_term(a64, b64, im, inn, K)
    if c_dtype == torch.bfloat16:
        tol = tol + np.abs(ref) * 2.0**-8 + 1e-38  # half a bf16 ulp is at most 2^-8 |ref|
    return tol


def _gemm_check(orc, A, B, params_a, params_b, c_dtype=torch.float32, sample=None):
    """Quantize on the oracle, upload, multiply on the GPU, compare with the fp64 reference."""
    M, K = A.shape
    N = B.shape[0]
    ca, sa, ta = _orc_quant(orc, A, params_a)
    cb, sb, tb = _orc_quant(orc, B, params_b)
    qa = fp4.upload_qtensor(ca, sa, ta, M, K, params_a, DEV)
    qb = fp4.upload_qtensor(cb, sb, tb, N, K, params_b, DEV)
    c = fp4.gemm(qa, qb, out_dtype=c_dtype)
    torch.cuda.synchronize()
    got = c.float().cpu().numpy().astype(np.float64)
    kw_a = dict(elem=params_a.elem, block=params_a.block, scale_mode=params_a.scale_mode)
    kw_b = dict(elem=params_b.elem, block=params_b.block, scale_mode=params_b.scale_mode)
    if sample is None:
        a64 = orc.operand_f64(ca, sa, ta, M, K, **kw_a)
        b64 = orc.operand_f64(cb, sb, tb, N, K, **kw_b)
        ref, sabs = orc.gemm_f64(a64, b64)
        g = got
    else:
        ms, ns = sample
        ur, inv_m = np.unique(ms, return_inverse=True)
        un, inv_n = np.unique(ns, return_inverse=True)
        ca_r = ca[ur]
        sa_r = sa[ur] if params_a.block[0] == 1 else None
        cb_r = cb[un]
        sb_r = sb[un] if params_b.block[0] == 1 else sb[un // 32]
        a64 = orc.operand_f64(ca_r, sa_r, ta, len(ur), K, **kw_a)
        if params_b.block[0] == 1:
            b64 = orc.operand_f64(cb_r, sb_r, tb, len(un), K, **kw_b)
        else:  # 2D scales: expand the sampled rows' tile scales to per-row groups
            kw1 = dict(kw_b, block=(1, 32))
            b64 = orc.operand_f64(cb_r, np.ascontiguousarray(sb_r), tb, len(un), K, **kw1)
        ref, sabs = orc.gemm_f64_sampled(a64, b64, inv_m, inv_n)
        g = got[ms, ns]
    if sample is None:
        im, inn = np.repeat(np.arange(M), N), np.tile(np.arange(N), M)
        tol = _gemm_tol(ref.reshape(-1), sabs.reshape(-1), a64, b64, im, inn, params_a, K,
                        c_dtype).reshape(M, N)
    else:
        tol = _gemm_tol(ref, sabs, a64, b64, inv_m, inv_n, params_a, K, c_dtype)
    err = np.abs(g - ref)
    report_ratio(err, ref, sabs, c_dtype, f"{M}x{N}x{K} {params_a.elem}/{params_a.scale_mode}")
    worst = np.argmax(err - tol)
    assert np.all(err <= tol), f"max excess at {worst}: err {err.flat[worst]} tol {tol.flat[worst]} ref {ref.flat[worst]}"
    return c


def report_ratio(err, ref, sabs, c_dtype, what):
    """Print max |C - C_ref| / (1e-5 sum |a b|) (after taking off half a bf16 ulp of C_ref for bf16
    outputs): below 1 the stated bound holds without the FP8 matrix-core term."""
    e = np.asarray(err, dtype=np.float64)
    if c_dtype == torch.bfloat16:
        e = np.maximum(e - np.abs(ref) * 2.0**-8, 0.0)
    s = 1e-5 * np.asarray(sabs, dtype=np.float64)
    r = np.where(s > 0, e / np.where(s > 0, s, 1.0), np.where(e > 0, np.inf, 0.0))
    print(f"GEMM-ERR-RATIO {what} {'bf16' if c_dtype == torch.bfloat16 else 'f32'} {float(r.max()):.4g}")
    return float(r.max())


def test_gemm_tiny_mxfp4(orc):
    a, b = wl.tiny_mxfp4(0)
    _gemm_check(orc, a, b, P(), P())
    _gemm_check(orc, a, b, P(), P(), c_dtype=torch.bfloat16)


@pytest.mark.parametrize("M,N,K", [(200, 136, 384), (1, 1, 128), (129, 257, 256), (64, 300, 512),
                                   (256, 256, 128), (300, 520, 384), (512, 768, 1024),
                                   (257, 511, 640)])
@pytest.mark.parametrize("kind", ["mxfp4", "mxfp4_2d", "mxfp8", "nvfp4"])
def test_gemm_shapes(orc, M, N, K, kind):
    rng = np.random.default_rng(M + N + K)
    A = rng.standard_normal((M, K)).astype(np.float32)
    B = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    if kind == "mxfp4":
        pa, pb = P(), P(scale_mode=CEIL)
    elif kind == "mxfp4_2d":
        if N % 32:
            pytest.skip("2D tiles need N % 32 == 0")
        pa, pb = P(), P(block=(32, 32), scale_mode=CEIL)
    elif kind == "mxfp8":
        pa, pb = P(elem=E4M3), P(elem=E4M3, scale_mode=CEIL)
    else:
        pa, pb = P(block=(1, 16), scale_mode=NV46), P(block=(1, 16), scale_mode=NV)
    _gemm_check(orc, A, B, pa, pb)
    _gemm_check(orc, A, B, pa, pb, c_dtype=torch.bfloat16)


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (200, 136, 96), (129, 256, 160), (300, 520, 224),
                                   (257, 320, 4192)])
@pytest.mark.parametrize("kind", ["mxfp4", "mxfp4_2d", "mxfp8", "nvfp4"])
def test_gemm_k_not_a_multiple_of_128(orc, M, N, K, kind):
    """K % 32 == 0 but K % 128 != 0: the last 128-deep step of the 128 x 128 kernel reads past K,
    where the pieces of A and B are zero and the scale bytes of the missing groups code 0, so C is
    the product over the real K (the same bound as every other shape)."""
    rng = np.random.default_rng(M + 5 * N + K)
    A = rng.standard_normal((M, K)).astype(np.float32)
    B = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    if kind == "mxfp4":
        pa, pb = P(), P(scale_mode=CEIL)
    elif kind == "mxfp4_2d":
        if N % 32:
            pytest.skip("2D tiles need N % 32 == 0")
        pa, pb = P(), P(block=(32, 32), scale_mode=CEIL)
    elif kind == "mxfp8":
        pa, pb = P(elem=E4M3), P(elem=E4M3, scale_mode=CEIL)
    else:
        pa, pb = P(block=(1, 16), scale_mode=NV46), P(block=(1, 16), scale_mode=NV)
    _gemm_check(orc, A, B, pa, pb)
    _gemm_check(orc, A, B, pa, pb, c_dtype=torch.bfloat16)


@pytest.mark.parametrize("kind", ["mxfp4", "mxfp4_2d", "mxfp8", "nvfp4"])
@pytest.mark.parametrize("c_dtype", [torch.float32, torch.bfloat16])
def test_gemm_128_tiles_equal_256_tiles(orc, kind, c_dtype):
    """A product whose 256 x 256 tile grid would fill at most half the CUs runs on 128 x 128 tiles of
    the same kernel (two workgroups per CU). Both accumulate every output over K in the same order,
    so C from the 4096-row product (144 tiles of 256 x 256) and C from its first 512 rows alone
    (18 such tiles, hence 128 x 128 tiles) agree bit for bit, and so does C from its first 200 rows
    (M below 256); the 512-row launch also meets the bound against the oracle."""
    M, N, K = 4096, 2304, 512
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert 2 * 144 > cus >= 2 * 18, f"{cus} CUs: the two launches would not take different tile sizes"
    rng = np.random.default_rng(41)
    A = rng.standard_normal((M, K)).astype(np.float32)
    B = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    if kind == "mxfp4":
        pa, pb = P(), P(scale_mode=CEIL)
    elif kind == "mxfp4_2d":
        pa, pb = P(), P(block=(32, 32), scale_mode=CEIL)
    elif kind == "mxfp8":
        pa, pb = P(elem=E4M3), P(elem=E4M3, scale_mode=CEIL)
    else:
        pa, pb = P(block=(1, 16), scale_mode=NV46), P(block=(1, 16), scale_mode=NV)
    qa = fp4.quantize(_to_dev(A), pa)
    qb = fp4.quantize(_to_dev(B), pb)
    c_full = fp4.gemm(qa, qb, out_dtype=c_dtype)
    iv = torch.int16 if c_dtype == torch.bfloat16 else torch.int32
    for rows in (512, 200):  # 18 tiles of 256 x 256; M below 256 (both on 128 x 128 tiles)
        cb = fp4.buffer_sizes(rows, K, pa)
        qa_top = fp4.QTensor(qa.codes[:cb[0]], qa.scales[:cb[1]], qa.tensor_scale, rows, K, pa)
        c_top = fp4.gemm(qa_top, qb, out_dtype=c_dtype)
        torch.cuda.synchronize()
        assert torch.equal(c_top.view(iv), c_full[:rows].view(iv)), f"first {rows} rows differ"
    rows = 512
    _gemm_check(orc, A[:rows], B, pa, pb, c_dtype=c_dtype, sample=(np.random.default_rng(5).integers(0, rows, 4096),
                                                                   np.random.default_rng(6).integers(0, N, 4096)))


@pytest.mark.parametrize("kind", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("oq_args", [dict(), dict(scale_mode=CEIL, round_mode=SR, seed=3, hadamard_n=128),
                                     dict(elem=E4M3, hadamard_n=32)], ids=["e2m1", "e2m1_sr_h128", "e4m3_h32"])
def test_fused_output_quantize_128_tiles_equal_256_tiles(kind, oq_args):
    """The fused output quantize on 128 x 128 tiles (the first 512 or 200 rows of A alone) writes
    the same C and C_q bytes as on 256 x 256 tiles (the 4096-row product): the quantization of a
    row of C depends on that row only, stochastic rounding included (keyed by m * N + n)."""
    M, N, K = 4096, 2304, 512
    rng = np.random.default_rng(43)
    A = rng.standard_normal((M, K)).astype(np.float32)
    B = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    if kind == "mxfp4":
        pa, pb = P(), P(scale_mode=CEIL)
    else:
        pa, pb = P(block=(1, 16), scale_mode=NV46), P(block=(1, 16), scale_mode=NV)
    oq = P(**oq_args)
    qa = fp4.quantize(_to_dev(A), pa)
    qb = fp4.quantize(_to_dev(B), pb)
    c_full, q_full = fp4.gemm(qa, qb, out_dtype=torch.float32, out_q=oq)
    for rows in (512, 200):
        cb = fp4.buffer_sizes(rows, K, pa)
        qa_top = fp4.QTensor(qa.codes[:cb[0]], qa.scales[:cb[1]], qa.tensor_scale, rows, K, pa)
        c_top, q_top = fp4.gemm(qa_top, qb, out_dtype=torch.float32, out_q=oq)
        torch.cuda.synchronize()
        qc, qs = fp4.buffer_sizes(rows, N, oq)[:2]
        assert torch.equal(c_top.view(torch.int32), c_full[:rows].view(torch.int32)), f"C, first {rows} rows"
        assert torch.equal(q_top.codes, q_full.codes[:qc]), f"C_q codes, first {rows} rows"
        assert torch.equal(q_top.scales, q_full.scales[:qs]), f"C_q scales, first {rows} rows"


def test_nvfp4_gemm_without_workspace_needs_k_multiple_of_128():
    """The in-LDS re-expression runs 128-deep stages: with K % 128 != 0 an NVFP4 product needs the
    workspace, and the call says so before it launches anything."""
    M, N, K = 256, 256, 160
    rng = np.random.default_rng(11)
    pa = P(block=(1, 16), scale_mode=NV46)
    qa = fp4.quantize(_to_dev(rng.standard_normal((M, K)).astype(np.float32)), pa)
    qb = fp4.quantize(_to_dev(rng.standard_normal((N, K)).astype(np.float32)), pa)
    with pytest.raises(fp4.Fp4Error) as ei:
        fp4.gemm(qa, qb, use_workspace=False)
    assert ei.value.status == fp4.ERR_WORKSPACE


OUTQ_CASES = [(E2M1, FLOOR, RNE), (E2M1, CEIL, SR), (E4M3, FLOOR, RNE), (E4M3, CEIL, SR)]


@pytest.mark.parametrize("M,N,K", [(200, 160, 384), (64, 96, 128), (512, 768, 1024), (300, 544, 512)])
@pytest.mark.parametrize("kind", ["mxfp4", "mxfp8", "nvfp4"])
def test_gemm_fused_output_quantize(orc, M, N, K, kind):
    """The epilogue's MX quantization of C along N equals the oracle's quantization of the very fp32
    C the same call stores (bit-exact codes and scales, SR included); C itself meets the GEMM bound;
    skipping C or storing it as bf16 leaves the quantized output unchanged."""
    rng = np.random.default_rng(M * 7 + N + K)
    A = rng.standard_normal((M, K)).astype(np.float32)
    B = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    if kind == "mxfp4":
        pa, pb = P(), P(scale_mode=CEIL)
    elif kind == "mxfp8":
        pa, pb = P(elem=E4M3), P(elem=E4M3)
    else:
        pa, pb = P(block=(1, 16), scale_mode=NV46), P(block=(1, 16), scale_mode=NV)
    ca, sa, ta = _orc_quant(orc, A, pa)
    cb, sb, tb = _orc_quant(orc, B, pb)
    qa = fp4.upload_qtensor(ca, sa, ta, M, K, pa, DEV)
    qb = fp4.upload_qtensor(cb, sb, tb, N, K, pb, DEV)
    _gemm_check(orc, A, B, pa, pb)  # the fp32 C of the plain call meets the GEMM bound
    for elem, sm, rnd in OUTQ_CASES:
        oq = P(elem=elem, scale_mode=sm, round_mode=rnd, seed=7)
        c, cq = fp4.gemm(qa, qb, out_dtype=torch.float32, out_q=oq)
        torch.cuda.synchronize()
        c_host = c.cpu().numpy()
        oc, os_, _ = _orc_quant(orc, c_host, oq)
        gc, gs = cq.codes.cpu().numpy(), cq.scales.cpu().numpy()
        oc, os_ = oc.reshape(-1), os_.reshape(-1).view(np.uint8)
        bad = np.nonzero(gc != oc)[0]
        assert bad.size == 0, f"{(elem, sm, rnd)}: {bad.size} code bytes differ, first at {bad[:8]}"
        bad = np.nonzero(gs != os_)[0]
        assert bad.size == 0, f"{(elem, sm, rnd)}: {bad.size} scale bytes differ, first at {bad[:8]}"
        # the plain call's C is the same fp32 C
        c_plain = fp4.gemm(qa, qb, out_dtype=torch.float32)
        assert torch.equal(c_plain.view(torch.int32), c.view(torch.int32))
        # without C, and with bf16 C: the same codes and scales
        for kw in (dict(keep_c=False), dict(out_dtype=torch.bfloat16)):
            c2, cq2 = fp4.gemm(qa, qb, out_q=oq, **kw)
            torch.cuda.synchronize()
            assert (c2 is None) == ("keep_c" in kw)
            assert torch.equal(cq2.codes, cq.codes) and torch.equal(cq2.scales, cq.scales)


@pytest.mark.parametrize("M,N,K,kind,hns", [
    (200, 160, 384, "mxfp4", (16, 32)),     # small kernel, ragged M
    (64, 128, 128, "mxfp8", (64, 128)),     # small kernel: a 128-chunk spans both wave columns
    (512, 768, 1024, "mxfp4", (64, 128)),   # 256 x 256 kernel
    (300, 640, 512, "nvfp4", (32, 128)),    # 256 x 256 kernel, ragged M, last tile half empty
])
def test_gemm_fused_output_quantize_rotated(orc, M, N, K, kind, hns):
    """Epilogue rotation along N before the output quantize: the codes and scales equal the
    oracle's quantization, with the same n, of the very fp32 C the call stores (rotation stages in
    the oracle's order, so bit-exact); C itself is stored unrotated."""
    rng = np.random.default_rng(M + 3 * N + K)
    A = rng.standard_normal((M, K)).astype(np.float32)
    B = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    if kind == "mxfp4":
        pa, pb = P(), P(scale_mode=CEIL)
    elif kind == "mxfp8":
        pa, pb = P(elem=E4M3), P(elem=E4M3)
    else:
        pa, pb = P(block=(1, 16), scale_mode=NV46), P(block=(1, 16), scale_mode=NV)
    ca, sa, ta = _orc_quant(orc, A, pa)
    cb, sb, tb = _orc_quant(orc, B, pb)
    qa = fp4.upload_qtensor(ca, sa, ta, M, K, pa, DEV)
    qb = fp4.upload_qtensor(cb, sb, tb, N, K, pb, DEV)
    c_plain = fp4.gemm(qa, qb, out_dtype=torch.float32)
    for hn in hns:
        for elem, sm, rnd in ((E2M1, FLOOR, RNE), (E2M1, CEIL, SR), (E4M3, CEIL, RNE)):
            oq = P(elem=elem, scale_mode=sm, round_mode=rnd, seed=5, hadamard_n=hn)
            c, cq = fp4.gemm(qa, qb, out_dtype=torch.float32, out_q=oq)
            torch.cuda.synchronize()
            assert torch.equal(c_plain.view(torch.int32), c.view(torch.int32))
            oc, os_, _ = _orc_quant(orc, c.cpu().numpy(), oq)
            gc, gs = cq.codes.cpu().numpy(), cq.scales.cpu().numpy()
            oc, os_ = oc.reshape(-1), os_.reshape(-1).view(np.uint8)
            bad = np.nonzero(gc != oc)[0]
            assert bad.size == 0, f"{(hn, elem, sm, rnd)}: {bad.size} code bytes differ, first at {bad[:8]}"
            bad = np.nonzero(gs != os_)[0]
            assert bad.size == 0, f"{(hn, elem, sm, rnd)}: {bad.size} scale bytes differ, first at {bad[:8]}"
            _, cq2 = fp4.gemm(qa, qb, out_q=oq, keep_c=False)
            torch.cuda.synchronize()
            assert torch.equal(cq2.codes, cq.codes) and torch.equal(cq2.scales, cq.scales)


@pytest.mark.parametrize("rows,cols,hn", [(107, 128, 32), (107, 128, 64), (86, 32, 0), (3, 256, 128)])
def test_tensor_amax_ignores_memory_past_the_tensor(orc, rows, cols, hn):
    """Regression: the last workgroup's trailing waves (segment count not a multiple of 256) must
    read nothing past the tensor. The tensor is the head of a larger buffer whose tail holds 1e30,
    so any read past its end would show up in the NVFP4 tensor scale and the codes."""
    rng = np.random.default_rng(rows + cols + hn)
    x = (rng.standard_normal((rows, cols)) * 3).astype(np.float32)
    big = torch.full((rows + 256, cols), 1e30, dtype=torch.float32, device=DEV)
    big[:rows] = torch.from_numpy(x).to(DEV)
    for sm in (NV, NV46):
        p = P(block=(1, 16), scale_mode=sm, hadamard_n=hn)
        q = fp4.quantize(big[:rows], p)
        torch.cuda.synchronize()
        oc, os_, ot = _orc_quant(orc, x, p)
        assert q.tensor_scale.cpu().numpy().view(np.uint32)[0] == ot.view(np.uint32)[0]
        assert np.array_equal(q.codes.cpu().numpy(), oc.reshape(-1))
        assert np.array_equal(q.scales.cpu().numpy(), os_.reshape(-1).view(np.uint8))


BATCH_CASES = [
    # dtype, shapes, params
    ("bf16", [(4096 // 16, 4096 // 8), (11008 // 43, 4096 // 8)], dict(hadamard_n=128)),
    ("f32", [(96, 256), (40, 64), (200, 160)], dict(scale_mode=CEIL, round_mode=SR, seed=9, hadamard_n=32)),
    ("bf16", [(64, 512), (128, 256)], dict(block=(32, 32), scale_mode=CEIL, hadamard_n=64)),
    ("bf16", [(33, 128), (64, 96), (8, 32), (130, 256)], dict(elem=E4M3, round_mode=SR, seed=2)),
    ("f32", [(64, 128), (96, 64)], dict(block=(1, 16), scale_mode=fp4.SCALE_NV_4OVER6_GIVEN)),
    ("bf16", [(64, 256), (32, 64)], dict(block=(1, 16), scale_mode=F32, hadamard_n=16)),
]


@pytest.mark.parametrize("dt,shapes,kw", BATCH_CASES)
def test_quantize_batch_parity(orc, dt, shapes, kw):
    """One launch over several tensors gives, for each, the codes and scales of its own
    fp4_quantize call, and those equal the oracle's."""
    rng = np.random.default_rng(len(shapes) * 100 + shapes[0][0])
    params = P(**kw)
    given = params.scale_mode == fp4.SCALE_NV_4OVER6_GIVEN
    xs, gs = [], []
    for r, c in shapes:
        x = (rng.standard_normal((r, c)) * rng.uniform(0.01, 100)).astype(np.float32)
        gs.append(float(np.abs(x).max()) / 2688 * 0.8 if given else None)
        xs.append(wl.f32_to_bf16_bits(x) if dt == "bf16" else x)
    xt = [_to_dev(x) for x in xs]
    qs = fp4.quantize_batch(xt, params, tensor_scales=gs if given else None)
    torch.cuda.synchronize()
    for i, (x, q) in enumerate(zip(xs, qs)):
        one = fp4.quantize(xt[i], params, tensor_scale=gs[i])
        torch.cuda.synchronize()
        assert torch.equal(q.codes, one.codes) and torch.equal(q.scales, one.scales), f"item {i}"
        oc, os_, _ = orc.quantize(x, elem=params.elem, block=params.block, scale_mode=params.scale_mode,
                                  round_mode=params.round_mode, hadamard_n=params.hadamard_n, seed=params.seed,
                                  tensor_scale=gs[i])
        assert np.array_equal(q.codes.cpu().numpy(), oc.reshape(-1)), f"item {i} codes"
        assert np.array_equal(q.scales.cpu().numpy(), os_.reshape(-1).view(np.uint8)), f"item {i} scales"


CW_CASES = [
    # dtype, rows, cols, params
    ("bf16", 256, 64, dict()),
    ("bf16", 384, 200, dict(hadamard_n=128)),
    ("f32", 96, 48, dict(hadamard_n=32, scale_mode=CEIL, round_mode=SR, seed=7)),
    ("bf16", 512, 72, dict(hadamard_n=256, round_mode=SR, scale_mode=CEIL, seed=3)),
    ("bf16", 256, 104, dict(elem=E4M3, hadamard_n=64)),
    ("f32", 128, 40, dict(block=(1, 16), scale_mode=NV46)),
    ("bf16", 256, 64, dict(block=(1, 16), scale_mode=NV, hadamard_n=128)),
    ("bf16", 160, 40, dict(block=(1, 16), scale_mode=F32, round_mode=SR, seed=11)),
    ("f32", 64, 132, dict(scale_mode=F32, hadamard_n=16)),
]


@pytest.mark.parametrize("dt,rows,cols,kw", CW_CASES)
def test_quantize_colwise_parity(orc, dt, rows, cols, kw):
    """Column-wise quantization of x equals the oracle's quantization of x^T, bit for bit (also
    with a row pitch wider than the row)."""
    rng = np.random.default_rng(rows * 31 + cols)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x[rng.integers(rows), rng.integers(cols)] *= 40.0
    params = P(**kw)
    xt = np.ascontiguousarray(x.T)
    if dt == "bf16":
        xb = wl.f32_to_bf16_bits(x)
        xt_in = np.ascontiguousarray(xb.T)
        dev = _to_dev(xb)
    else:
        xt_in = xt
        dev = _to_dev(x)
    oc, os_, ots = _orc_quant(orc, xt_in, params)
    for pitch in (0, 24):
        if pitch:
            wide = torch.zeros(rows, cols + pitch, dtype=dev.dtype, device=DEV)
            wide[:, :cols] = dev
            src = wide[:, :cols]
        else:
            src = dev
        q = fp4.quantize_colwise(src, params)
        torch.cuda.synchronize()
        assert q.rows == cols and q.cols == rows
        gc, gs = q.codes.cpu().numpy(), q.scales.cpu().numpy()
        bad = np.nonzero(gc != oc.reshape(-1))[0]
        assert bad.size == 0, f"pitch {pitch}: {bad.size} code bytes differ, first at {bad[:8]}"
        bad = np.nonzero(gs != os_.reshape(-1).view(np.uint8))[0]
        assert bad.size == 0, f"pitch {pitch}: {bad.size} scale bytes differ, first at {bad[:8]}"
        if ots is not None:
            assert q.tensor_scale.cpu().numpy().view(np.uint32)[0] == ots.view(np.uint32)[0]


def test_weight_gradient_gemm_colwise(orc):
    """dW = dY^T X for a backward step: both operands quantized column-wise (the contraction runs
    over the 512 tokens), then the block-scaled GEMM; checked against the fp64 product of the
    oracle's quantization of dY^T and X^T."""
    rng = np.random.default_rng(5)
    T, N, K = 512, 288, 320  # tokens, output features, input features
    dy = (rng.standard_t(3, (T, N)) * 1e-3).astype(np.float32)
    xx = rng.standard_normal((T, K)).astype(np.float32)
    pa = P(hadamard_n=128, scale_mode=CEIL, round_mode=SR, seed=7)
    pb = P(hadamard_n=128)
    qa = fp4.quantize_colwise(_to_dev(wl.f32_to_bf16_bits(dy)), pa)
    qb = fp4.quantize_colwise(_to_dev(wl.f32_to_bf16_bits(xx)), pb)
    dw = fp4.gemm(qa, qb, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ca, sa, _ = _orc_quant(orc, np.ascontiguousarray(wl.f32_to_bf16_bits(dy).T), pa)
    cb, sb, _ = _orc_quant(orc, np.ascontiguousarray(wl.f32_to_bf16_bits(xx).T), pb)
    assert np.array_equal(qa.codes.cpu().numpy(), ca.reshape(-1))
    assert np.array_equal(qb.codes.cpu().numpy(), cb.reshape(-1))
    a64 = orc.operand_f64(ca, sa, None, N, T)
    b64 = orc.operand_f64(cb, sb, None, K, T)
    ref, sabs = orc.gemm_f64(a64, b64)
    err = np.abs(dw.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= 1e-5 * sabs + 1e-30)


NVG, NV46G = fp4.SCALE_NV_GIVEN, fp4.SCALE_NV_4OVER6_GIVEN


@pytest.mark.parametrize("mode", [NVG, NV46G])
@pytest.mark.parametrize("gfac", [1.0, 0.25, 3.0])
@pytest.mark.parametrize("hn,rnd", [(0, RNE), (128, RNE), (0, SR)])
def test_nvfp4_given_tensor_scale_parity(orc, mode, gfac, hn, rnd):
    """Delayed NVFP4 scaling: codes and scales bit-exact against the oracle for the caller's g
    (the tensor's own amax-derived g times gfac: below 1 some blocks saturate), row-wise and
    column-wise, and the GEMM on such operands within the bound."""
    if mode == NV46G and rnd == SR:
        pytest.skip("SR is not combined with 4/6")
    rng = np.random.default_rng(int(gfac * 10) + hn)
    x = (rng.laplace(size=(256, 256)) * 2).astype(np.float32)
    xb = wl.f32_to_bf16_bits(x)
    g0 = float(np.abs(wl.bf16_bits_to_f32(xb)).max()) / 2688.0
    g = float(np.float32(g0 * gfac))
    params = P(block=(1, 16), scale_mode=mode, round_mode=rnd, hadamard_n=hn, seed=5)
    q = fp4.quantize(_to_dev(xb), params, tensor_scale=g)
    torch.cuda.synchronize()
    oc, os_, ots = orc.quantize(xb, block=(1, 16), scale_mode=mode, round_mode=rnd, hadamard_n=hn,
                                seed=5, tensor_scale=g)
    assert np.array_equal(q.codes.cpu().numpy(), oc.reshape(-1))
    assert np.array_equal(q.scales.cpu().numpy(), os_.reshape(-1))
    assert q.tensor_scale.cpu().numpy()[0] == np.float32(g)
    qt = fp4.quantize_colwise(_to_dev(xb), params, tensor_scale=g)
    torch.cuda.synchronize()
    oct_, ost, _ = orc.quantize(np.ascontiguousarray(xb.T), block=(1, 16), scale_mode=mode,
                                round_mode=rnd, hadamard_n=hn, seed=5, tensor_scale=g)
    assert np.array_equal(qt.codes.cpu().numpy(), oct_.reshape(-1))
    assert np.array_equal(qt.scales.cpu().numpy(), ost.reshape(-1))
    if rnd == RNE:
        w = (rng.standard_normal((160, 256)) * 0.02).astype(np.float32)
        pw = P(block=(1, 16), scale_mode=mode, hadamard_n=hn)
        gw = float(np.abs(w).max()) / 2688.0 * 0.5
        cb, sb, tb = orc.quantize(w, block=(1, 16), scale_mode=mode, hadamard_n=hn, tensor_scale=gw)
        qb = fp4.upload_qtensor(cb, sb, tb, 160, 256, pw, DEV)
        qa = fp4.upload_qtensor(oc, os_, ots, 256, 256, params, DEV)
        c = fp4.gemm(qa, qb, out_dtype=torch.float32)
        torch.cuda.synchronize()
        a64 = orc.operand_f64(oc, os_, ots, 256, 256, block=(1, 16), scale_mode=mode)
        b64 = orc.operand_f64(cb, sb, tb, 160, 256, block=(1, 16), scale_mode=mode)
        ref, sabs = orc.gemm_f64(a64, b64)
        im, inn = np.repeat(np.arange(256), 160), np.tile(np.arange(160), 256)
        tol = _gemm_tol(ref.reshape(-1), sabs.reshape(-1), a64, b64, im, inn, params, 256,
                        torch.float32).reshape(256, 160)
        assert np.all(np.abs(c.cpu().numpy() - ref) <= tol)


# (4096, 2304, 256): 144 tiles of 256 x 256 (more than half the CUs fill: the 256 x 256 kernel);
# (512, 768, 1024) and (300, 544, 640) NVFP4: 128 x 128 tiles; the others the register-staged kernel
@pytest.mark.parametrize("M,N,K", [(4096, 2304, 256), (512, 768, 1024), (300, 544, 640), (200, 160, 384)])
@pytest.mark.parametrize("kind", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("c_dtype", [torch.bfloat16, torch.float32])
def test_gemm_into_a_column_block(M, N, K, kind, c_dtype):
    """C written into a column block of a wider buffer (row pitch ldc > N; block start 16-byte
    aligned, pitch a multiple of 16 bytes or not): the block holds exactly the contiguous call's C
    (itself checked against the oracle above) and no element outside it changes; a block start
    that is not 16-byte aligned is refused."""
    rng = np.random.default_rng(M + 3 * N + K)
    a = torch.from_numpy(wl.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32)).view(np.int16))
    b = torch.from_numpy(wl.f32_to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32)).view(np.int16))
    a, b = a.to(DEV).view(torch.bfloat16), b.to(DEV).view(torch.bfloat16)
    if kind == "mxfp4":
        pa, pb = P(hadamard_n=128), P(hadamard_n=128, scale_mode=CEIL)
    else:
        pa, pb = P(block=(1, 16), scale_mode=NV46), P(block=(1, 16), scale_mode=NV)
    qa, qb = fp4.quantize(a, pa), fp4.quantize(b, pb)
    ref = fp4.gemm(qa, qb, out_dtype=c_dtype)
    ibits = torch.int16 if c_dtype == torch.bfloat16 else torch.int32
    for col0, pad in ((0, 64), (16, 48), (0, 3), (16, 1)):
        wide = torch.full((M, col0 + N + pad), -7.25, dtype=c_dtype, device=DEV)
        got = fp4.gemm(qa, qb, out=wide[:, col0:col0 + N])
        torch.cuda.synchronize()
        assert got.data_ptr() == wide[:, col0:].data_ptr()
        assert torch.equal(wide[:, col0:col0 + N].contiguous().view(ibits), ref.view(ibits)), (col0, pad)
        outside = torch.cat([wide[:, :col0].reshape(-1), wide[:, col0 + N:].reshape(-1)])
        assert bool((outside == -7.25).all()), f"elements outside the block changed ({col0}, {pad})"
    wide = torch.zeros((M, N + 8), dtype=c_dtype, device=DEV)
    with pytest.raises(fp4.Fp4Error):
        fp4.gemm(qa, qb, out=wide[:, 1:N + 1])


def test_reused_outputs_describe_what_was_written(orc):
    """An output QTensor allocated for other params (same buffer sizes) and reused: after the call
    it carries the params and shape of what was written, and those codes equal the oracle's."""
    rng = np.random.default_rng(21)
    x = rng.standard_normal((96, 256)).astype(np.float32)
    p_old, p_new = P(scale_mode=CEIL), P(hadamard_n=64, round_mode=SR, seed=5)
    q = fp4.empty_qtensor(96, 256, p_old, DEV)
    got = fp4.quantize(_to_dev(x), p_new, out=q)
    torch.cuda.synchronize()
    assert got is q and q.params == p_new and (q.rows, q.cols) == (96, 256)
    oc, os_, _ = _orc_quant(orc, x, p_new)
    assert np.array_equal(q.codes.cpu().numpy(), oc.reshape(-1))
    assert np.array_equal(q.scales.cpu().numpy(), os_.reshape(-1).view(np.uint8))
    # the fused output quantize fills a C_q allocated for another rule
    w = (rng.standard_normal((64, 256)) * 0.05).astype(np.float32)
    qa, qb = fp4.quantize(_to_dev(x), P()), fp4.quantize(_to_dev(w), P())
    oq = P(scale_mode=CEIL)
    cq = fp4.empty_qtensor(96, 64, P(), DEV)
    c, cq2 = fp4.gemm(qa, qb, out_dtype=torch.float32, out_q=oq, q_out=cq)
    torch.cuda.synchronize()
    assert cq2 is cq and cq.params == oq and (cq.rows, cq.cols) == (96, 64)
    oc, os_, _ = _orc_quant(orc, c.cpu().numpy(), oq)
    assert np.array_equal(cq.codes.cpu().numpy(), oc.reshape(-1))


def _nv_quotient_edge_input(g, seed):
    """fp32 [64, 512] whose 16-blocks have maxima spread over fp32's range (zeros included) and,
    in half the rows, maxima placed at and one ulp around RN(mid * c) for E4M3 rounding midpoints
    mid and c = RN(6 g), where the block-scale quotient amax / c lands on or next to a tie."""
    rng = np.random.default_rng(seed)
    x = rng.uniform(-1.0, 1.0, size=(64, 512)).astype(np.float32)
    blocks = x.reshape(-1, 16)
    nb = blocks.shape[0]
    mag = np.float32(2.0) ** rng.integers(-126, 120, size=nb).astype(np.float32)
    blocks *= mag[:, None]
    blocks[rng.choice(nb, size=nb // 16, replace=False)] = 0.0
    c = np.float32(np.float32(6.0) * np.float32(g))
    # E4M3 rounding midpoints between consecutive normal codes (1 + (2m + 1)/16) * 2^e
    mids = np.array([(1 + (2 * m + 1) / 16) * 2.0 ** e for e in range(-6, 9) for m in range(8)], dtype=np.float32)
    half = nb // 2
    with np.errstate(over="ignore", under="ignore"):
        target = (mids[rng.integers(0, mids.size, size=half)] * c).astype(np.float32)
    step = rng.integers(-1, 2, size=half)
    target = np.where(step < 0, np.nextafter(target, np.float32(0)),
                      np.where(step > 0, np.nextafter(target, np.float32(np.inf)), target)).astype(np.float32)
    ok = np.isfinite(target) & (target > 0)
    tb = (rng.uniform(-0.5, 0.5, size=(int(ok.sum()), 16)) * target[ok][:, None].astype(np.float64)).astype(np.float32)
    tb[:, 3] = target[ok]
    blocks[half:][ok] = tb
    assert np.isfinite(x).all()
    return x


@pytest.mark.parametrize("mode", [NVG, NV46G])
@pytest.mark.parametrize("g", [2.0 ** -130, 2.0 ** -102, 2.0 ** -98, 1e-20, 3.1e-3, 1.0, 3.3e4, 2.0 ** 97, 2.0 ** 99, 2.0 ** 110])
def test_nvfp4_block_scale_quotient_edges(orc, mode, g):
    """The block-scale quotient amax / RN(M g) is computed from RN(1/RN(M g)) with two Markstein
    corrections where divisor and block max lie in [2^-100, 2^100], and by division elsewhere:
    codes and scales stay byte-exact against the oracle for tensor scales on both sides of those
    bounds, block maxima across fp32's range, and maxima that put the quotient on or one ulp from an
    E4M3 rounding midpoint."""
    x = _nv_quotient_edge_input(g, seed=int(abs(np.log2(g))) + (mode == NV46G))
    params = P(block=(1, 16), scale_mode=mode)
    q = fp4.quantize(_to_dev(x), params, tensor_scale=float(np.float32(g)))
    torch.cuda.synchronize()
    oc, os_, _ = orc.quantize(x, block=(1, 16), scale_mode=mode, tensor_scale=float(np.float32(g)))
    gc, gs = q.codes.cpu().numpy(), q.scales.cpu().numpy()
    bad = np.nonzero(gs != os_.reshape(-1).view(np.uint8))[0]
    assert bad.size == 0, f"{bad.size} scale bytes differ, first at {bad[:8]}"
    bad = np.nonzero(gc != oc.reshape(-1))[0]
    assert bad.size == 0, f"{bad.size} code bytes differ, first at {bad[:8]}"
