"""CPU checks of the benchmark's host logic and of the synthetic workload recipes: one GPU only,
every workload's quantization is accepted by the library's size queries, the traffic summary is
read only when its recorded kernel hash matches, and the generators draw the stated shapes,
outlier counts and distributions."""
import hashlib
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from bit_gemm_fwht_amd import workloads as wl  # noqa: E402


@pytest.fixture(scope="module")
def fp4():
    from bit_gemm_fwht_amd import fp4 as m
    if not os.path.exists(m.LIB_PATH):
        from bit_gemm_fwht_amd import build
        build.build()
    m.lib()
    return m


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("name", sorted(bench.WORKLOADS))
def test_workload_quantization_is_valid(fp4, name):
    wk = bench.WORKLOADS[name]
    for side, rows in (("a", wk["M"]), ("b", wk["N"])):  # B as the GEMM takes it ([N, K])
        p = bench.params_of(fp4, wk[side])
        codes, scales, _ = fp4.buffer_sizes(rows, wk["K"], p)
        per = 1 if p.elem == fp4.E4M3 else 0.5
        assert codes == int(rows * wk["K"] * per)
        assert scales > 0
    assert wk["fp8"] == (bench.params_of(fp4, wk["a"]).elem == fp4.E4M3 or name.startswith("nvfp4"))


def test_traffic_summary_is_read_only_for_the_current_kernel(tmp_path, monkeypatch):
    src = hashlib.sha256(open(bench.GEMM_SRC, "rb").read()).hexdigest()
    f = tmp_path / "summary.md"
    f.write_text(f"kernel source sha256: {src}\ncalibrated bytes per launch: 123456789\n")
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(f))
    assert bench.measured_traffic() == 123456789
    f.write_text(f"kernel source sha256: {'0' * 64}\ncalibrated bytes per launch: 123456789\n")
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(tmp_path / "missing.md"))
    assert bench.measured_traffic() is None


def test_committed_traffic_summary_format():
    text = open(bench.TRAFFIC_SUMMARY).read()
    assert "kernel source sha256:" in text and "calibrated bytes per launch:" in text
    assert "rocprofv3" in text  # the command that produced it


def test_llama_linear_recipe():
    x, w, ch = wl.llama_linear(0, m=512, n=384, k=4096)
    assert x.shape == (512, 4096) and w.shape == (384, 4096) and x.dtype == np.uint16
    assert len(ch) == 41 and len(np.unique(ch)) == 41  # 1 % of 4096 channels
    xf, wf = wl.bf16_bits_to_f32(x), wl.bf16_bits_to_f32(w)
    others = np.setdiff1d(np.arange(4096), ch)
    s_out, s_in = xf[:, ch].std(), xf[:, others].std()
    assert 18.0 < s_out / s_in < 22.0
    assert abs(wf.std() - 0.02) < 0.0005 and abs(wf.mean()) < 0.0005
    # seeded: the same draw twice
    x2, _, ch2 = wl.llama_linear(0, m=512, n=384, k=4096)
    assert np.array_equal(x, x2) and np.array_equal(ch, ch2)


def test_backward_2d_recipe():
    w, dy = wl.backward_2d(0, m=1024, n=512, k=4096)
    assert w.shape == (512, 4096) and dy.shape == (1024, 4096)
    d = wl.bf16_bits_to_f32(dy).astype(np.float64) / 1e-3
    # Student-t(3): median |t| = 0.765, heavy tails (kurtosis far above the normal's 3)
    assert abs(np.median(np.abs(d)) - 0.765) < 0.02
    assert np.mean(np.abs(d) > 10) > 1e-3


def test_nvfp4_4over6_recipe():
    x, w = wl.nvfp4_4over6(0, m=1024, n=256, k=1024)
    assert x.shape == (1024, 1024) and w.shape == (256, 1024)
    xf = np.abs(wl.bf16_bits_to_f32(x).astype(np.float64))
    # Laplace(0, 1) with 0.1 % of entries (1049 of 1024^2) scaled x30: an unscaled draw exceeds 30
    # with probability e^-30, a scaled one with probability e^-1, so about 1049 / e = 386 do
    assert 300 < np.sum(xf > 30.0) < 480
    assert abs(np.median(xf) - np.log(2.0)) < 0.02


def test_backward_dw_recipe():
    dy, x = wl.backward_dw(0, t=1024, d_out=256, d_in=512)
    assert dy.shape == (1024, 256) and x.shape == (1024, 512)
    d = wl.bf16_bits_to_f32(dy).astype(np.float64) / 1e-3
    assert abs(np.median(np.abs(d)) - 0.765) < 0.03  # Student-t(3)
    xf = wl.bf16_bits_to_f32(x)
    s = xf.std(axis=0)
    assert np.sum(s > 10) == 5  # 1 % of 512 channels (rounded) scaled x20


def test_given_scale_is_the_tensors_own_nvfp4_scale():
    """The delayed tensor scale the benchmark hands the _GIVEN modes is RN(amax / 2688), the scale
    the plain NVFP4 mode computes, so both modes give the same codes."""
    import oracle as orc
    rng = np.random.default_rng(3)
    x = wl.f32_to_bf16_bits(rng.laplace(size=(64, 256)).astype(np.float32))
    g = bench.given_scale(x)
    _, _, ts = orc.quantize(x, block=(1, 16), scale_mode=orc.SCALE_NV_4OVER6)
    assert np.float32(g) == ts.reshape(-1)[0]
    c1, s1, _ = orc.quantize(x, block=(1, 16), scale_mode=orc.SCALE_NV_4OVER6)
    c2, s2, _ = orc.quantize(x, block=(1, 16), scale_mode=orc.SCALE_NV_4OVER6_GIVEN, tensor_scale=g)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_cpu_baseline_slices_cover_the_rows():
    for n, parts, align in ((1536, 16, 32), (4128, 8, 32), (64, 16, 32), (1, 4, 1), (1000, 3, 1)):
        s = bench._slices(n, parts, align)
        assert s[0][0] == 0 and s[-1][1] == n and len(s) <= parts
        assert all(a[1] == b[0] for a, b in zip(s, s[1:]))
        assert all(lo % align == 0 for lo, _ in s)
    assert 1 <= bench.host_threads() <= 16
    assert isinstance(bench.cpu_model(), str)


def test_small_workloads_are_selectable():
    assert set(bench.SMALL_WORKLOADS) == {"tiny_mxfp4", "mnist_mlp"}
    for name in bench.SMALL_WORKLOADS:
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--workload", name],
                           capture_output=True, text=True, timeout=120)
        assert r.returncode == 2 and "one GPU" in r.stderr  # parsed, then refused before any GPU work


@pytest.mark.parametrize("name", sorted(bench.WORKLOADS))
def test_workload_inputs_have_the_stated_shapes(name, monkeypatch):
    """inputs_of returns A [M, K] and B as the step takes it ([N, K], or [K, N] when B is re-laid out
    from its stored orientation, or [tokens, features] for the column-wise workload); generators are
    replaced by shape-only stand-ins so that nothing large is drawn."""
    wk = bench.WORKLOADS[name]
    calls = {}

    def fake(tag):
        def f(seed, **kw):
            calls[tag] = True
            return tag
        return f

    import bit_gemm_fwht_amd.workloads as wlm
    for tag in ("llama_linear", "backward_2d", "nvfp4_4over6", "backward_dw", "forward_2d"):
        monkeypatch.setattr(wlm, tag, fake(tag))
    want = {"llama7b": "llama_linear", "backward_2d": "backward_2d", "nvfp4": "nvfp4_4over6",
            "backward_dw": "backward_dw", "forward_2d": "forward_2d"}
    try:
        bench.inputs_of(name)
    except (TypeError, ValueError):
        pass  # unpacking the stand-in fails after the generator was chosen
    tag = next(v for k, v in want.items() if name.startswith(k))
    assert calls == {tag: True}, (name, calls)


def test_event_stride_leaves_enough_samples():
    import bench
    for steps, stride in ((1, 1), (20, 1), (31, 1), (32, 2), (50, 3), (128, 8), (200, 8), (5000, 8)):
        assert bench.event_stride(steps) == stride
        assert len(range(0, steps, stride)) >= min(steps, 16)


@pytest.mark.parametrize("argv", [["--shard", "3"], ["--shard", "0"], ["--shard", "8", "--workload", "backward_dw_colwise"],
                                  ["--shard", "4", "--workload", "llama7b_fused_out_q"],  # 2752 % 128 (C's H_128)
                                  ["--shard", "8", "--workload", "forward_2d_transposed"]])
def test_shard_must_be_a_column_split_into_multiples_of_32(argv):
    """--shard S takes the first N/S rows of B: S must divide N into multiples of 32, and the workloads
    whose B is not a plain [N, K] row block refuse it (before any GPU work)."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode != 0 and "--shard" in (r.stderr + r.stdout)
