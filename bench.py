"""Benchmark of the quantize + block-scaled GEMM hot path on one MI355X.

Default workload (the headline): one step = the whole path over one batch of a Llama-7B-shaped
forward linear:
  X bf16 [4096, 4096] (N(0,1), 1% of channels x20) and W bf16 [11008, 4096] (N(0, 0.02^2)),
  both rotated along K by blockwise H_128 / sqrt(128) and quantized to MXFP4 (E2M1 elements,
  one E8M0 floor scale per 32, round to nearest even) in one batched launch, then C = X W^T on the
  MXFP4 operands, fp32 accumulation, bf16 output.
`--workload` selects one of the other full-size workloads instead (same JSON layout):
  backward_2d        dX = dY W^T, 8192 x 4096 x 4096: W 2D 32x32 truncation-free RNE, dY group-32
                     truncation-free with Philox stochastic rounding (seed 7), both H_128; MXFP4
  backward_2d_mxfp8  the same with E4M3 elements (MXFP8, the FP8 matrix cores)
  nvfp4_4over6       8192^3: X Laplace with 0.1% x30 outliers, W N(0, 0.02^2), NVFP4 with the
                     4/6 choice (tensor amax pass + quantize), GEMM through the FP8 re-expression
  nvfp4_4over6_lds   the same with the FP8 re-expression done in LDS inside the GEMM (no pre-pass,
                     no workspace)
and three that measure extensions of the path:
  nvfp4_4over6_given the same with delayed tensor scales (g given, from each tensor's own amax
                     taken once before timing): one quantize pass per tensor, no amax pass
  llama7b_fused_out_q the headline with the fused output quantize: C (bf16) and C_q (MXFP4,
                     H_128 along N, E8M0 floor, RNE) from the GEMM's epilogue
  forward_2d_transposed Y = X W at the backward's shapes (8192 x 4096 x 4096): W [K, N] quantized once
                     with 2D 32x32 truncation-free scales as stored, re-laid out each step as the
                     quantized W^T the GEMM takes (no re-quantization), X group-32 truncation-free
  llama7b_fused_quantize_a the headline with X's rotation + quantize fused into the GEMM launch (one
                     persistent launch: the grid quantizes X, each tile waits for its rows); W keeps
                     its own quantize launch; `gemm` then times X's quantize and the product together
  backward_dw_colwise dW = dY^T X over 8192 tokens (4096 x 4096 x 8192): dY and X as stored
                     [tokens, features], quantized column-wise (along tokens, H_128, E8M0 ceil;
                     dY with Philox SR) without forming the transposes
and the two small, launch-latency-bound workloads (reported in microseconds):
  tiny_mxfp4         A, B fp32 256x256, A's largest entry x50: MXFP4 quantize of both, the 256^3
                     GEMM (fp32 out) and A's per-tensor fp32-scale quantize (the outlier collapse)
  mnist_mlp          MNIST-MLP-shaped fp32 weights (256x784, 128x256, 10x128), clean and with a 50x
                     outlier in fc1: every per-tensor / per-row / group-32 x fp32 / E8M0 floor / E8M0
                     ceil quantization, with the MSE of each (quantize-only)
Inputs are resident in HBM before timing starts; the step cycles over several copies of the inputs
(more than the 256 MB last-level cache) so that every step reads its inputs from HBM. Before the
warm-up steps the step runs untimed for --settle seconds (0.3 s), the time the GPU takes to reach
the steady clocks of sustained work.

Prints one JSON line. `value` is the step's effective throughput in TFLOP/s (GEMM FLOPs over the
whole step time, quantization included); the per-kernel GB/s / TFLOP/s and roofline fractions are
in the extra fields. `roofline` is the dominant kernel (the GEMM): algorithmic FLOPs per launch over
its average launch time from HIP events on the launch stream (created with
hipEventDisableSystemFence, so that recording them does not flush the caches between the kernels
they bracket); its `traffic` is the measured memory
traffic per launch from the committed counter summary (headline workload only), reported only while
the summary's kernel source hash matches the current source. `cpu_baseline` times the CPU oracle on
a bounded sample of the same step, at one thread and at every host thread the process may use (up
to 16), and adds the CPU model and an fp32 torch.matmul on the host as a BLAS reference point.

`--shard S` measures one GPU's share of a column-parallel split over S GPUs (W's first N/S rows, all
of X) at its real shape. `--copy-calibration MIB` instead runs only a plain device-to-device copy of MIB MiB a few times
(the reference kernel whose FETCH_SIZE / WRITE_SIZE counter readings calibrate the GEMM's).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
FP4_PEAK_TFLOPS = 10100.0       # MI355X dense MXFP4 matrix throughput, TFLOP/s
FP8_PEAK_TFLOPS = 5000.0        # MI355X dense FP8 matrix throughput, TFLOP/s
ROOT = os.path.dirname(os.path.abspath(__file__))
GEMM_SRC = os.path.join(ROOT, "bit_gemm_fwht_amd", "csrc", "gemm.hip")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemm_llama7b_forward_linear_traffic.md")
HEADLINE = "llama7b_forward_linear"
# workloads whose B is not a plain [N, K] row block (a stored W [K, N] re-laid out; column-wise operands)
SHARD_EXCLUDED = {"forward_2d_transposed", "backward_dw_colwise"}

# name -> shapes (C = A B^T: A [M, K], B [N, K]), quantization of A and B, CPU-sample fraction
WORKLOADS = {
    "llama7b_forward_linear": dict(
        M=4096, N=11008, K=4096, a=dict(hadamard_n=128), b=dict(hadamard_n=128), batched=True,
        quant="E2M1 + E8M0 per 32 (floor), RNE", fp8=False, f=0.375,
        kernel="k_gemm_big (MXFP4, 256x256 tiles, 32x32x64 scaled MFMA, bf16 out)"),
    "backward_2d": dict(
        M=8192, N=4096, K=4096, a=dict(hadamard_n=128, scale="ceil", sr=True),
        b=dict(hadamard_n=128, block=(32, 32), scale="ceil"), batched=False,
        quant="dY: E2M1 + E8M0 per 32 (ceil), Philox SR; W: E2M1 + E8M0 per 32x32 (ceil), RNE",
        fp8=False, f=0.375, kernel="k_gemm_big (MXFP4, 2D B scales, 256x256 tiles, bf16 out)"),
    "backward_2d_mxfp8": dict(
        M=8192, N=4096, K=4096, a=dict(hadamard_n=128, scale="ceil", sr=True, e4m3=True),
        b=dict(hadamard_n=128, scale="ceil", e4m3=True), batched=False,
        quant="dY: E4M3 + E8M0 per 32 (ceil), Philox SR; W: E4M3 + E8M0 per 32 (ceil), RNE",
        fp8=True, f=0.375, kernel="k_gemm_big (MXFP8, 256x256 tiles, 32x32x64 scaled MFMA, bf16 out)"),
    "nvfp4_4over6": dict(
        M=8192, N=8192, K=8192, a=dict(nv46=True), b=dict(nv46=True), batched=False,
        quant="E2M1 + E4M3 per 16 x fp32 tensor scale, 4/6 choice, RNE", fp8=True, f=0.1875,
        kernel="fp4_gemm call: NVFP4->FP8 re-expression of both operands + k_gemm_big (FP8, bf16 out)"),
    "nvfp4_4over6_lds": dict(
        M=8192, N=8192, K=8192, a=dict(nv46=True), b=dict(nv46=True), batched=False, nv_lds=True,
        quant="E2M1 + E4M3 per 16 x fp32 tensor scale, 4/6 choice, RNE", fp8=True, f=0.1875,
        kernel="k_gemm_nv (NVFP4 operands re-expressed as FP8 in LDS, FP8 scaled MFMA, bf16 out; no workspace)"),
    "nvfp4_4over6_given": dict(
        M=8192, N=8192, K=8192, a=dict(nv46=True, given=True), b=dict(nv46=True, given=True), batched=False,
        quant="E2M1 + E4M3 per 16 x given fp32 tensor scale, 4/6 choice, RNE", fp8=True, f=0.1875,
        kernel="fp4_gemm call: NVFP4->FP8 re-expression of both operands + k_gemm_big (FP8, bf16 out)"),
    "llama7b_fused_out_q": dict(
        M=4096, N=11008, K=4096, a=dict(hadamard_n=128), b=dict(hadamard_n=128), batched=True,
        out_q=dict(hadamard_n=128),
        quant="E2M1 + E8M0 per 32 (floor), RNE; C_q: the same along N after H_128", fp8=False, f=0.375,
        kernel="k_gemm_big (MXFP4, bf16 C + fused H_128 MXFP4 quantize of C along N)"),
    "forward_2d_transposed": dict(
        M=8192, N=4096, K=4096, a=dict(scale="ceil"), b=dict(block=(32, 32), scale="ceil"), batched=False,
        transposed_b=True,
        quant="X: E2M1 + E8M0 per 32 (ceil), RNE; W: E2M1 + E8M0 per 32x32 (ceil), RNE, quantized once as "
              "stored [K, N] and re-laid out as its transpose each step",
        fp8=False, f=0.375, kernel="k_gemm_big (MXFP4, 2D B scales from the transposed weight, bf16 out)"),
    "llama7b_fused_quantize_a": dict(
        M=4096, N=11008, K=4096, a=dict(hadamard_n=128), b=dict(hadamard_n=128), batched=False,
        fused_a=True,
        quant="E2M1 + E8M0 per 32 (floor), RNE; X rotated and quantized inside the GEMM launch", fp8=False,
        f=0.375, kernel="k_gemm_fused_a (X's H_128 + MXFP4 quantize, then the 256x256 MXFP4 tiles, bf16 out)"),
    "backward_dw_colwise": dict(
        M=4096, N=4096, K=8192, a=dict(hadamard_n=128, scale="ceil", sr=True),
        b=dict(hadamard_n=128, scale="ceil"), batched=False, colwise=True,
        quant="column-wise (along tokens): dY E2M1 + E8M0 per 32 (ceil), Philox SR; X the same, RNE",
        fp8=False, f=0.375, kernel="k_gemm_big (MXFP4, 256x256 tiles, bf16 out)"),
}


# the two latency-bound workloads (under 1 MB each), reported in microseconds
SMALL_WORKLOADS = {
    "tiny_mxfp4": "A, B fp32 256x256 ~ N(0,1), A's largest entry x50: MXFP4 quantize of both (E8M0 "
                  "floor, RNE, no rotation), the 256^3 MXFP4 GEMM (fp32 out), and A's per-tensor "
                  "fp32-scale quantize (the outlier collapse)",
    "mnist_mlp": "fp32 weights 256x784, 128x256, 10x128 ~ N(0, 0.05^2), clean and with fc1's largest "
                 "entry x50: every {per-tensor, per-row, group-32 (flattened)} x {fp32 S = amax/6, E8M0 "
                 "floor, E8M0 ceil} quantization to E2M1 (quantize only), with the MSE of each",
}

# The caveduck.io post's figures for the trained MNIST MLP (unstated machine): context only, the
# synthetic weights here are random stand-ins with the same shapes.
PAGE_MSE_CONTEXT = {
    "table1_fc1_mse_clean_to_outlier": {"per_tensor": [5.4e-5, 1.2e-3], "per_channel": [1.7e-5, 2.3e-5],
                                        "group32": [1.2e-5, 1.2e-5]},
    "table2_group32_fp32_vs_pow2_mse": {"fc1": [1.23e-5, 1.58e-5], "fc2": [2.66e-5, 3.62e-5],
                                        "fc3": [6.12e-5, 6.30e-5]},
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(WORKLOADS) + sorted(SMALL_WORKLOADS))
    ap.add_argument("--copies", type=int, default=4, help="input copies cycled through (> LLC)")
    ap.add_argument("--settle", type=float, default=0.3,
                    help="seconds of untimed steps before the warm-up steps (clock ramp-up)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-fraction", type=float, default=None,
                    help="fraction f of A rows and B rows the CPU oracle processes")
    ap.add_argument("--k", type=int, default=0,
                    help="headline workload only: another contraction depth K (a multiple of 256), e.g. a long K "
                         "that amortises the GEMM's first round and epilogue over more main-loop stages")
    ap.add_argument("--shard", type=int, default=1, metavar="S",
                    help="one GPU's share of a column-parallel split over S GPUs: the GEMM over the first "
                         "N/S rows of B (output features), all of A (A's quantize included, as each GPU "
                         "would run it)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration) and exit")
    return ap.parse_args()


def params_of(fp4, spec):
    """fp4.Params for one operand's quantization spec."""
    if spec.get("nv46"):
        return fp4.Params(block=(1, 16),
                          scale_mode=fp4.SCALE_NV_4OVER6_GIVEN if spec.get("given") else fp4.SCALE_NV_4OVER6)
    return fp4.Params(elem=fp4.E4M3 if spec.get("e4m3") else fp4.E2M1, block=spec.get("block", (1, 32)),
                      scale_mode=fp4.SCALE_E8M0_CEIL if spec.get("scale") == "ceil" else fp4.SCALE_E8M0_FLOOR,
                      round_mode=fp4.ROUND_SR if spec.get("sr") else fp4.ROUND_RNE,
                      hadamard_n=spec.get("hadamard_n", 0), seed=7 if spec.get("sr") else 0)


def inputs_of(name, k=0):
    """Host bf16 bit patterns (A, B) of a workload: A [M, K] is the left operand (k: another K for
    the headline workload)."""
    from bit_gemm_fwht_amd import workloads as wl
    if name == "llama7b_forward_linear":
        x, w, _ = wl.llama_linear(0, k=k) if k else wl.llama_linear(0)
        return x, w
    if name.startswith("backward_2d"):
        w, dy = wl.backward_2d(0)
        return dy, w
    if name in ("llama7b_fused_out_q", "llama7b_fused_quantize_a"):
        x, w, _ = wl.llama_linear(0)
        return x, w
    if name == "backward_dw_colwise":
        return wl.backward_dw(0)  # dY [tokens, 4096], X [tokens, 4096]
    if name == "forward_2d_transposed":
        return wl.forward_2d(0)  # X [8192, 4096], W [4096 (K), 4096 (N)]
    return wl.nvfp4_4over6(0)  # nvfp4_4over6, _lds and _given


def given_scale(bits) -> float:
    """The delayed tensor scale of a bf16 tensor taken from its own amax: RN(amax / 2688) in fp32
    (1 for an all-zero tensor)."""
    amax = np.float32(np.abs(workloads_f32(bits)).max())
    return float(amax / np.float32(2688.0)) if amax > 0 else 1.0


def workloads_f32(bits):
    from bit_gemm_fwht_amd import workloads as wl
    return wl.bf16_bits_to_f32(bits)


def measured_traffic():
    """Bytes per GEMM launch from the committed counter summary, or None when it is missing or was
    taken on another version of the kernel source."""
    try:
        text = open(TRAFFIC_SUMMARY).read()
        src = hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()
    except OSError:
        return None
    m_src = re.search(r"kernel source sha256: ([0-9a-f]{64})", text)
    m_b = re.search(r"calibrated bytes per launch: ([0-9]+)", text)
    if not m_src or not m_b or m_src.group(1) != src:
        return None
    return int(m_b.group(1))


def event_stride(steps: int) -> int:
    """Every how many timed steps the per-phase events are recorded: every eighth step where that
    still leaves 16 or more samples, else a smaller stride (every step for 31 steps or fewer)."""
    return max(1, min(8, steps // 16))


class HipTimingEvent:
    """A HIP event for timing, created with hipEventDisableSystemFence: recording it writes a
    timestamp on the stream without the system-scope cache write-back and invalidation that a
    default event (and so torch.cuda.Event) performs, which slows the kernel that follows it and
    adds several microseconds to every interval. Recorded on the stream the library launches on."""

    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            import ctypes
            # the HIP runtime torch has loaded (one runtime per process)
            path = "libamdhip64.so"
            with open("/proc/self/maps") as f:
                for line in f:
                    if "libamdhip64" in line:
                        path = line.split()[-1]
                        break
            h = ctypes.CDLL(path)
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = h
        return cls._hip

    def __init__(self, stream_handle):
        import ctypes
        self._c = ctypes
        self.stream = ctypes.c_void_p(stream_handle)
        self.h = ctypes.c_void_p()
        rc = self._lib().hipEventCreateWithFlags(ctypes.byref(self.h), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self):
        rc = self._lib().hipEventRecord(self.h, self.stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end):
        """Milliseconds from this event to `end` (both recorded and complete)."""
        f = self._c.c_float()
        rc = self._lib().hipEventElapsedTime(self._c.byref(f), self.h, end.h)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return f.value

    def __del__(self):
        if self._hip is not None and self.h:
            self._hip.hipEventDestroy(self.h)


def copy_calibration(mib):
    import torch
    n = mib << 20
    x = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)


def host_threads() -> int:
    """Threads the CPU baseline may use: the host cores this process may run on, capped at the 16
    that one GPU's share of a GPU host provides."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _slices(n, parts, align):
    """[lo, hi) row ranges covering n rows in at most `parts` pieces, cut at multiples of align."""
    step = -(-(-(-n // parts)) // align) * align  # ceil(ceil(n / parts) / align) * align
    return [(lo, min(n, lo + step)) for lo in range(0, n, step)]


def _oracle_step(orc, As, Bs, pa, pb, K, threads, out_q=None, ga=None, gb=None):
    """The oracle's pass over a sample: quantize A and B rows, their fp64 operand values, the fp64
    GEMM of the sampled block (and its output quantize). With threads > 1 the rows are cut into
    slices run on a thread pool (the C oracle releases the interpreter lock while it runs); the SR
    element index and an NVFP4 tensor amax then restart per slice, the work is the same.
    Returns (seconds for the quantize part, seconds for the GEMM part)."""
    from concurrent.futures import ThreadPoolExecutor

    def q(x, p, ts=None):
        return orc.quantize(x, elem=p.elem, block=p.block, scale_mode=p.scale_mode,
                            round_mode=p.round_mode, hadamard_n=p.hadamard_n, seed=p.seed,
                            tensor_scale=ts)

    def operand(x, p, ts):
        rows = x.shape[0]
        c, s, t = q(x, p, ts)
        if p.block[0] == 1:
            return orc.operand_f64(c, s, t, rows, K, elem=p.elem, block=p.block, scale_mode=p.scale_mode)
        srow = np.ascontiguousarray(s.reshape(rows // 32, -1)[np.arange(rows) // 32])  # 2D tiles
        return orc.operand_f64(c, srow, t, rows, K, elem=p.elem, block=(1, 32), scale_mode=p.scale_mode)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        t0 = time.perf_counter()
        fa = [ex.submit(operand, As[lo:hi], pa, ga) for lo, hi in _slices(As.shape[0], threads, 32)]
        fb = [ex.submit(operand, Bs[lo:hi], pb, gb) for lo, hi in _slices(Bs.shape[0], threads, 32)]
        a64 = np.concatenate([f.result() for f in fa])
        b64 = np.concatenate([f.result() for f in fb])
        t1 = time.perf_counter()

        def gemm_rows(lo, hi):
            c, _ = orc.gemm_f64(a64[lo:hi], b64)
            if out_q is not None:
                q(c.astype(np.float32), out_q)
            return c

        parts = [ex.submit(gemm_rows, lo, hi) for lo, hi in _slices(a64.shape[0], threads, 1)]
        for f in parts:
            f.result()
        t2 = time.perf_counter()
    return t1 - t0, t2 - t1


def blas_reference(M, N, K):
    """torch.matmul in fp32 on the host CPU for the same M x N x K (random operands), as a BLAS
    reference point for the GEMM; TFLOP/s and the threads torch uses."""
    import torch
    g = torch.Generator().manual_seed(0)
    a = torch.randn(M, K, generator=g)
    b = torch.randn(N, K, generator=g)
    torch.matmul(a[:64], b[:64].T)  # warm the library up
    t0 = time.perf_counter()
    torch.matmul(a, b.T)
    dt = time.perf_counter() - t0
    return {"TFLOP/s": round(2.0 * M * N * K / dt / 1e12, 4), "threads": torch.get_num_threads(),
            "s": round(dt, 3), "what": f"torch.matmul fp32 on the host CPU, {M}x{N}x{K}"}


def cpu_baseline(wk, a_bits, b_bits, pa, pb, f, out_q=None, ga=None, gb=None):
    """Time the oracle on f*M rows of A, f*N rows of B and the f*M x f*N block of C (and its output
    quantize), at one thread and at all host threads, and scale each to a whole step:
    T = T_quantize / f + T_gemm / f^2. Column-wise operands sample columns of the stored tensors
    (rows of their transposes). Also reports the CPU model and a BLAS fp32 matmul reference."""
    import oracle as orc
    M, N, K = wk["M"], wk["N"], wk["K"]
    sm, sn = max(int(M * f) // 32 * 32, 32), max(int(N * f) // 32 * 32, 32)  # whole 32-row tiles
    if out_q is not None and out_q.hadamard_n:  # C's sampled rows hold whole rotation chunks
        sn = max(sn // out_q.hadamard_n * out_q.hadamard_n, out_q.hadamard_n)
    if wk.get("colwise"):
        As = np.ascontiguousarray(a_bits[:, :sm].T)
        Bs = np.ascontiguousarray(b_bits[:, :sn].T)
    elif wk.get("transposed_b"):  # the oracle quantizes W^T's rows directly
        As = np.ascontiguousarray(a_bits[:sm])
        Bs = np.ascontiguousarray(b_bits[:, :sn].T)
    else:
        As = np.ascontiguousarray(a_bits[:sm])
        Bs = np.ascontiguousarray(b_bits[:sn])
    fm, fn = sm / M, sn / N
    flops = 2.0 * M * N * K
    runs = {}
    nthreads = host_threads()
    for th in sorted({1, nthreads}):
        tq, tg = _oracle_step(orc, As, Bs, pa, pb, K, th, out_q=out_q, ga=ga, gb=gb)
        t_step = tq / ((fm + fn) / 2) + tg / (fm * fn)
        runs[th] = dict(value=round(flops / t_step / 1e12, 6), step_s=round(t_step, 3),
                        tq=round(tq, 2), tg=round(tg, 2))
    best = runs[nthreads]
    return {
        "value": best["value"],
        "unit": "TFLOP/s",
        "cores": nthreads,
        "kind": "oracle",
        "sample": (f"oracle quantize of {sm} A rows + {sn} B rows and the fp64 GEMM of their {sm}x{sn} "
                   f"block over K={K}{' with its output quantize' if out_q is not None else ''}, scaled to a "
                   f"full step as T_q/f + T_gemm/f^2 with f={f}; at {nthreads} threads: {best['tq']} s + "
                   f"{best['tg']} s (row slices on a thread pool), at 1 thread: {runs[1]['tq']} s + {runs[1]['tg']} s"),
        "step_s": best["step_s"],
        "single_thread": {"value": runs[1]["value"], "step_s": runs[1]["step_s"], "cores": 1},
        "cpu_model": cpu_model(),
        "blas_fp32": blas_reference(M, N, K),
    }


def _timed_steps(step, args, nparts):
    """Run step(i, ev) untimed for --settle seconds and --warmup steps, then time --steps steps with
    fence-free HIP events (ev[(nparts + 1) * i + j] before part j of step i, one after the last).
    Returns (wall seconds per step, mean seconds of each part)."""
    import torch
    t_settle = time.perf_counter()
    i = 0
    while time.perf_counter() - t_settle < args.settle:
        for _ in range(20):
            step(i, None)
            i += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i, None)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    per = nparts + 1
    evs = [HipTimingEvent(stream) for _ in range(per * args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[per * i:per * i + per])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    parts = [float(np.mean([evs[per * i + j].elapsed_time(evs[per * i + j + 1]) for i in range(args.steps)])) * 1e-3
             for j in range(nparts)]
    return wall, parts


def _graph_step_time(step, args):
    """The same step captured once into a HIP graph (torch.cuda.CUDAGraph records the library's
    launches on its capture stream) and replayed --steps times back to back: seconds per replay.
    The library allocates nothing and clears with fill kernels, so its launches capture as they are."""
    import torch
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the launch paths on the capture stream
        step(0, None)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step(0, None)
    for _ in range(max(args.warmup, 3)):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / args.steps


def _base_line(args, value, unit, dtype, config, wall):
    return {"metric": "quantize GB/s (% HBM peak); MXFP4 GEMM TFLOP/s (% FP4 MFMA peak)", "value": value,
            "unit": unit, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(wall * 1e3, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": dtype,
            "data": "synthetic (seeded numpy draws of the workload's shapes and distributions)", "config": config}


def run_tiny(args):
    """Tiny MXFP4 check: quantize A and B (MXFP4), the 256^3 GEMM, and A's per-tensor quantize."""
    import torch
    import oracle as orc
    from bit_gemm_fwht_amd import fp4
    from bit_gemm_fwht_amd import workloads as wl
    dev = torch.device("cuda:0")
    a, b = wl.tiny_mxfp4(0)
    at = torch.from_numpy(a).to(dev)
    bt = torch.from_numpy(b).to(dev)
    mx = fp4.Params()
    pt = fp4.Params(block=(256, 256), scale_mode=fp4.SCALE_F32)
    qa, qb, qt = (fp4.empty_qtensor(256, 256, p, dev) for p in (mx, mx, pt))
    ws = torch.empty(fp4.buffer_sizes(256, 256, pt)[2], dtype=torch.uint8, device=dev)
    c = torch.empty(256, 256, dtype=torch.float32, device=dev)

    def step(i, ev):
        if ev: ev[0].record()
        fp4.quantize(at, mx, out=qa)
        fp4.quantize(bt, mx, out=qb)
        if ev: ev[1].record()
        fp4.gemm(qa, qb, out=c)
        if ev: ev[2].record()
        fp4.quantize(at, pt, out=qt, workspace=ws)
        if ev: ev[3].record()

    wall, (tq, tg, tt) = _timed_steps(step, args, 3)
    wall_graph = _graph_step_time(step, args)
    flops = 2.0 * 256**3
    qbytes = 2 * (256 * 256 * 4 + 256 * 128 + 256 * 8) + 256 * 256 * 4 + 256 * 128 + 4
    codes = qt.codes.cpu().numpy()
    nonzero = int(np.count_nonzero(codes & 0x7) + np.count_nonzero((codes >> 4) & 0x7))
    # the oracle over the same step (it is small enough to run whole)
    t0 = time.perf_counter()
    ca, sa, _ = orc.quantize(a)
    cb, sb, _ = orc.quantize(b)
    c64, _ = orc.gemm_f64(orc.operand_f64(ca, sa, None, 256, 256), orc.operand_f64(cb, sb, None, 256, 256))
    orc.quantize(a, block=(256, 256), scale_mode=orc.SCALE_F32)
    t_orc = time.perf_counter() - t0
    err = float(np.abs(c.cpu().numpy().astype(np.float64) - c64).max())
    out = _base_line(args, round(flops / wall / 1e12, 4), "TFLOP/s", "mxfp4",
                     {"workload": "tiny_mxfp4", "M": 256, "N": 256, "K": 256, "input": "fp32",
                      "quant": "E2M1 + E8M0 per 32 (floor), RNE; A also per tensor with fp32 S = amax/6",
                      "output": "fp32"}, wall)
    out.update({
        "latency_us": {"step": round(wall * 1e6, 2), "quantize_a_b": round(tq * 1e6, 2), "gemm": round(tg * 1e6, 2),
                       "per_tensor_quantize_a": round(tt * 1e6, 2),
                       "step_hip_graph_replay": round(wall_graph * 1e6, 2)},
        "roofline": {"bound": "mfma", "achieved": round(flops / tg / 1e12, 3), "peak": FP4_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(flops / tg / 1e12 / FP4_PEAK_TFLOPS, 6), "traffic": None,
                     "note": "33.6 MFLOP on 256 x 256 outputs: four 128x128 tiles, launch-latency bound"},
        "quantize": {"GB/s": round(qbytes / (tq + tt) / 1e9, 2), "frac": round(qbytes / (tq + tt) / 1e9 / HBM_PEAK_GBS, 6),
                     "us": round((tq + tt) * 1e6, 2), "bytes": qbytes},
        "checks": {"per_tensor_nonzero_codes": nonzero, "gemm_max_abs_err_vs_fp64_oracle": err},
        "cpu_baseline": {"value": round(flops / t_orc / 1e12, 8), "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
                         "sample": f"the whole step on the oracle: {t_orc * 1e3:.1f} ms", "cpu_model": cpu_model()},
    })
    print(json.dumps(out), flush=True)


def run_mnist(args):
    """MNIST-MLP-shaped weight quantization: every granularity x scale variant, clean and with the
    50x outlier in fc1, quantize-only; the MSE of each from the GPU's dequantized values (identical to
    the oracle's, which is checked)."""
    import torch
    import oracle as orc
    from bit_gemm_fwht_amd import fp4
    from bit_gemm_fwht_amd import workloads as wl
    dev = torch.device("cuda:0")
    sets = {"clean": wl.mnist_mlp(0, outlier=False), "outlier": wl.mnist_mlp(0, outlier=True)}
    scales = {"fp32": fp4.SCALE_F32, "e8m0_floor": fp4.SCALE_E8M0_FLOOR, "e8m0_ceil": fp4.SCALE_E8M0_CEIL}
    jobs = []  # (set, layer, granularity, scale, host array as quantized, device tensor, params, qtensor, ws)
    for sname, layers in sets.items():
        for lname, w in layers.items():
            for gran in ("per_tensor", "per_row", "group32"):
                x = w.reshape(1, -1) if gran == "group32" else w
                rows, cols = x.shape
                block = {"per_tensor": (rows, cols), "per_row": (1, cols), "group32": (1, 32)}[gran]
                xt = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
                for scn, sm in scales.items():
                    p = fp4.Params(block=block, scale_mode=sm)
                    q = fp4.empty_qtensor(rows, cols, p, dev)
                    wb = fp4.buffer_sizes(rows, cols, p)[2]
                    ws = torch.empty(wb, dtype=torch.uint8, device=dev) if wb else None
                    jobs.append((sname, lname, gran, scn, np.ascontiguousarray(x), xt, p, q, ws))

    def step(i, ev):
        if ev: ev[0].record()
        for j in jobs:
            fp4.quantize(j[5], j[6], out=j[7], workspace=j[8])
        if ev: ev[1].record()

    wall, (tq,) = _timed_steps(step, args, 1)
    wall_graph = _graph_step_time(step, args)
    nbytes = 0
    mse = {}
    t_orc = 0.0
    outlier_at = np.unravel_index(int(np.argmax(np.abs(sets["outlier"]["fc1"]))), sets["outlier"]["fc1"].shape)
    for sname, lname, gran, scn, x, xt, p, q, ws in jobs:
        cb, sb, _ = fp4.buffer_sizes(x.shape[0], x.shape[1], p)
        nbytes += x.size * 4 + cb + sb
        y = fp4.dequantize(q).cpu().numpy().astype(np.float64)
        d2 = (y - x.astype(np.float64)) ** 2
        t0 = time.perf_counter()
        oc, os_, _ = orc.quantize(x, block=p.block, scale_mode=p.scale_mode)
        yo = orc.dequantize(oc, os_, None, x.shape[0], x.shape[1], block=p.block, scale_mode=p.scale_mode)
        t_orc += time.perf_counter() - t0
        entry = {"mse": float(d2.mean()), "oracle_equal": bool(np.array_equal(y, yo.astype(np.float64)))}
        if sname == "outlier" and lname == "fc1":
            keep = np.ones(sets["outlier"]["fc1"].shape, dtype=bool)
            keep[outlier_at] = False
            entry["mse_without_outlier"] = float(d2.reshape(keep.shape)[keep].mean())
        mse.setdefault(sname, {}).setdefault(lname, {}).setdefault(gran, {})[scn] = entry
    out = _base_line(args, round(nbytes / tq / 1e9, 3), "GB/s", "e2m1",
                     {"workload": "mnist_mlp", "tensors": "fc1 256x784, fc2 128x256, fc3 10x128 fp32",
                      "variants": len(jobs), "input": "fp32", "quant": "E2M1; per tensor / per row / per 32 (flattened); "
                      "fp32 S = amax/6, E8M0 floor, E8M0 ceil; RNE"}, wall)
    out.update({
        "latency_us": {"step": round(wall * 1e6, 2), "quantize_all_variants": round(tq * 1e6, 2),
                       "quantize_calls": len(jobs), "step_hip_graph_replay": round(wall_graph * 1e6, 2)},
        "roofline": {"bound": "hbm", "achieved": round(nbytes / tq / 1e9, 3), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(nbytes / tq / 1e9 / HBM_PEAK_GBS, 6), "traffic": None,
                     "note": f"{len(jobs)} quantize calls over 0.94 MB of weights: launch-latency bound"},
        "mse": mse,
        "page_context": PAGE_MSE_CONTEXT,
        "cpu_baseline": {"value": round(nbytes / t_orc / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                         "sample": f"every variant quantized and dequantized on the oracle: {t_orc * 1e3:.1f} ms",
                         "cpu_model": cpu_model()},
    })
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path shards by "
              "rows of X / W with no exchange between GPUs", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    import torch

    from bit_gemm_fwht_amd import fp4

    fp4.lib()  # fail loudly if the HIP library is missing
    if args.workload == "tiny_mxfp4":
        return run_tiny(args)
    if args.workload == "mnist_mlp":
        return run_mnist(args)
    dev = torch.device("cuda:0")
    wk = dict(WORKLOADS[args.workload])
    if args.k:
        if args.workload != HEADLINE or args.k % 256:
            raise SystemExit(f"--k applies to {HEADLINE} only and must be a multiple of 256")
        wk["K"] = args.k
    if args.shard != 1:
        n_s = wk["N"] // args.shard if args.shard > 1 else 0
        unit = max(32, wk.get("out_q", {}).get("hadamard_n", 0))  # C's quantize groups / rotation chunks
        if (args.workload in SHARD_EXCLUDED or n_s == 0 or wk["N"] % args.shard or n_s % unit):
            raise SystemExit(f"--shard {args.shard}: not a column-parallel split of {args.workload} "
                             f"(N = {wk['N']} must split into multiples of {unit}; "
                             f"not for {sorted(SHARD_EXCLUDED)})")
        wk["N"] = n_s
    M, N, K = wk["M"], wk["N"], wk["K"]
    pa, pb = params_of(fp4, wk["a"]), params_of(fp4, wk["b"])
    a_bits, b_bits = inputs_of(args.workload, args.k)
    if args.shard > 1:  # this GPU's rows of B: the first N/S output features
        b_bits = np.ascontiguousarray(b_bits[:N])
    a0 = torch.from_numpy(a_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    b0 = torch.from_numpy(b_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    As = [a0] + [a0.clone() for _ in range(args.copies - 1)]
    Bs = [b0] + [b0.clone() for _ in range(args.copies - 1)]
    qa = [fp4.empty_qtensor(M, K, pa, dev) for _ in range(args.copies)]
    qb = [fp4.empty_qtensor(N, K, pb, dev) for _ in range(args.copies)]
    cs = [torch.empty(M, N, dtype=torch.bfloat16, device=dev) for _ in range(args.copies)]
    transposed_b = bool(wk.get("transposed_b"))
    fused_a = bool(wk.get("fused_a"))
    wsf = None
    if fused_a:
        import ctypes
        bc = qb[0].c()
        wsf = torch.empty(fp4.lib().fp4_gemm_quantize_a_workspace_bytes(M, ctypes.byref(bc)), dtype=torch.uint8,
                          device=dev)
    if transposed_b:  # W [K, N] quantized once as stored (2D tiles); each step re-lays it out as W^T
        qw_stored = [fp4.quantize(Bs[j], pb) for j in range(args.copies)]
        torch.cuda.synchronize()
    colwise = bool(wk.get("colwise"))
    quantize_one = fp4.quantize_colwise if colwise else fp4.quantize
    # delayed tensor scales: g of each tensor from its own amax, set once in the outputs' buffers
    ga = gb = None
    if wk["a"].get("given"):
        ga, gb = given_scale(a_bits), given_scale(b_bits)
        for q in qa:
            q.tensor_scale.fill_(ga)
        for q in qb:
            q.tensor_scale.fill_(gb)
    oq = cq = None
    if wk.get("out_q"):
        oq = fp4.Params(hadamard_n=wk["out_q"]["hadamard_n"])
        cq = [fp4.empty_qtensor(M, N, oq, dev) for _ in range(args.copies)]
    # workspaces allocated once, outside the timed region
    wsa = wsb = wsg = None
    nb = fp4.buffer_sizes(M, K, pa)[2]
    if nb:
        wsa = torch.empty(nb, dtype=torch.uint8, device=dev)
    nb = fp4.buffer_sizes(N, K, pb)[2]
    if nb:
        wsb = torch.empty(nb, dtype=torch.uint8, device=dev)
    nb = fp4.gemm_workspace_bytes(qa[0], qb[0])
    if nb and not wk.get("nv_lds"):
        wsg = torch.empty(nb, dtype=torch.uint8, device=dev)
    use_ws = not wk.get("nv_lds")

    # Timing events on the launch stream, on every `stride`-th step of the timed region: one before
    # the step's quantize, one between its quantize and GEMM, one after its GEMM. An event record
    # costs the stream a few microseconds (measured: 143.2 us per step without events, 146-151 with
    # two on every step, 143.7-144.3 with three on every eighth), so the other steps run without.
    def step(i, ev=None):
        j = i % args.copies
        if ev is not None:
            ev[0].record()
        if wk["batched"]:
            fp4.quantize_batch([As[j], Bs[j]], pa, outs=[qa[j], qb[j]])
        elif transposed_b:
            fp4.transpose_2d(qw_stored[j], out=qb[j])
            quantize_one(As[j], pa, out=qa[j], workspace=wsa)
        elif fused_a:  # only W here: X is rotated and quantized by the GEMM launch itself
            quantize_one(Bs[j], pb, out=qb[j], workspace=wsb)
        else:
            quantize_one(As[j], pa, out=qa[j], workspace=wsa,
                         tensor_scale=qa[j].tensor_scale if ga is not None else None)
            quantize_one(Bs[j], pb, out=qb[j], workspace=wsb,
                         tensor_scale=qb[j].tensor_scale if gb is not None else None)
        if ev is not None:
            ev[1].record()
        if oq is not None:
            fp4.gemm(qa[j], qb[j], out=cs[j], workspace=wsg, out_q=oq, q_out=cq[j])
        elif fused_a:
            fp4.gemm_quantize_a(As[j], pa, qb[j], out=cs[j], a_out=qa[j], workspace=wsf)
        else:
            fp4.gemm(qa[j], qb[j], out=cs[j], workspace=wsg, use_workspace=use_ws)
        if ev is not None:
            ev[2].record()

    # The GPU's clocks ramp up over the first tens of milliseconds of sustained work (a step runs
    # ~15 % slower at first): run the step untimed for --settle seconds before the warm-up steps,
    # so that the timed steps see the steady state a continuously busy GPU runs at.
    t_settle = time.perf_counter()
    i = 0
    while time.perf_counter() - t_settle < args.settle:
        for _ in range(20):
            step(i)
            i += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev).cuda_stream
    stride = event_stride(args.steps)
    sampled = list(range(0, args.steps, stride))
    evs = {i: [HipTimingEvent(stream) for _ in range(3)] for i in sampled}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs.get(i))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tq = np.mean([evs[i][0].elapsed_time(evs[i][1]) for i in sampled]) * 1e-3
    t_g = np.mean([evs[i][1].elapsed_time(evs[i][2]) for i in sampled]) * 1e-3
    ms_per_step = wall / args.steps * 1e3

    flops = 2.0 * M * N * K

    def qbytes(rows, p):  # bf16 in, codes and scales out
        cb, sb, _ = fp4.buffer_sizes(rows, K, p)
        return rows * K * 2 + cb + sb

    bytes_q = qbytes(M, pa) + qbytes(N, pb)
    if fused_a:  # the timed quantize launch is W's alone
        bytes_q = qbytes(N, pb)
    if transposed_b:  # the re-layout reads and writes W's codes and scales once
        cbw, sbw, _ = fp4.buffer_sizes(N, K, pb)
        bytes_q = qbytes(M, pa) + 2 * (cbw + sbw)
    gemm_tflops = flops / t_g / 1e12
    peak = FP8_PEAK_TFLOPS if wk["fp8"] else FP4_PEAK_TFLOPS
    dtype = "nvfp4" if args.workload.startswith("nvfp4") else {False: "mxfp4", True: "mxfp8"}[wk["fp8"]]
    out = {
        "metric": "quantize GB/s (% HBM peak); MXFP4 GEMM TFLOP/s (% FP4 MFMA peak)",
        "value": round(flops / (wall / args.steps) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded numpy draws of the workload's shapes and distributions)",
        "config": {"workload": args.workload, "M": M, "N": N, "K": K, "input": "bf16",
                   "hadamard_n": pa.hadamard_n, "quant": wk["quant"], "output": "bf16",
                   "input_copies": args.copies,
                   **({"shard": f"1/{args.shard} of N (column-parallel; all of A)"} if args.shard > 1 else {})},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / peak, 4),
                     "traffic": (measured_traffic() if args.workload == HEADLINE and not args.k and args.shard == 1
                                 else None),
                     "kernel": wk["kernel"]},
        "quantize": {"GB/s": round(bytes_q / tq / 1e9, 1),
                     "frac": round(bytes_q / tq / 1e9 / HBM_PEAK_GBS, 4),
                     "us": round(tq * 1e6, 2), "bytes": int(bytes_q),
                     "launches": ("one batched k_segment launch for A and B" if wk["batched"]
                                  else "quantize of A + the 2D re-layout of B's codes" if transposed_b
                                  else "W alone (X is quantized inside the GEMM launch)" if fused_a
                                  else "separate launches for A and B")
                     + (", column-wise" if colwise else "") + (", given tensor scales" if ga is not None else "")},
        "gemm": {"TFLOP/s": round(gemm_tflops, 2), "frac": round(gemm_tflops / peak, 4),
                 "us": round(t_g * 1e6, 2), "flops": flops},
        "phase_timing": f"HIP events on the launch stream around quantize and GEMM of {len(sampled)} of the "
                        f"{args.steps} timed steps (every {stride}th)",
    }
    if oq is not None:
        cb, sb, _ = fp4.buffer_sizes(M, N, oq)
        out["gemm"]["fused_out_q"] = f"C (bf16) and C_q ({cb + sb} bytes: MXFP4 along N after H_{oq.hadamard_n})"
    if not args.no_cpu_baseline:
        f = args.cpu_fraction if args.cpu_fraction is not None else wk["f"]
        out["cpu_baseline"] = cpu_baseline(wk, a_bits, b_bits, pa, pb, f, out_q=oq, ga=ga, gb=gb)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
