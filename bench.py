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
and three that measure extensions of the path:
  nvfp4_4over6_given the same with delayed tensor scales (g given, from each tensor's own amax
                     taken once before timing): one quantize pass per tensor, no amax pass
  llama7b_fused_out_q the headline with the fused output quantize: C (bf16) and C_q (MXFP4,
                     H_128 along N, E8M0 floor, RNE) from the GEMM's epilogue
  backward_dw_colwise dW = dY^T X over 8192 tokens (4096 x 4096 x 8192): dY and X as stored
                     [tokens, features], quantized column-wise (along tokens, H_128, E8M0 ceil;
                     dY with Philox SR) without forming the transposes
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
a bounded sample of the same step.

`--copy-calibration MIB` instead runs only a plain device-to-device copy of MIB MiB a few times
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
    "nvfp4_4over6_given": dict(
        M=8192, N=8192, K=8192, a=dict(nv46=True, given=True), b=dict(nv46=True, given=True), batched=False,
        quant="E2M1 + E4M3 per 16 x given fp32 tensor scale, 4/6 choice, RNE", fp8=True, f=0.1875,
        kernel="fp4_gemm call: NVFP4->FP8 re-expression of both operands + k_gemm_big (FP8, bf16 out)"),
    "llama7b_fused_out_q": dict(
        M=4096, N=11008, K=4096, a=dict(hadamard_n=128), b=dict(hadamard_n=128), batched=True,
        out_q=dict(hadamard_n=128),
        quant="E2M1 + E8M0 per 32 (floor), RNE; C_q: the same along N after H_128", fp8=False, f=0.375,
        kernel="k_gemm_big (MXFP4, bf16 C + fused H_128 MXFP4 quantize of C along N)"),
    "backward_dw_colwise": dict(
        M=4096, N=4096, K=8192, a=dict(hadamard_n=128, scale="ceil", sr=True),
        b=dict(hadamard_n=128, scale="ceil"), batched=False, colwise=True,
        quant="column-wise (along tokens): dY E2M1 + E8M0 per 32 (ceil), Philox SR; X the same, RNE",
        fp8=False, f=0.375, kernel="k_gemm_big (MXFP4, 256x256 tiles, bf16 out)"),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(WORKLOADS))
    ap.add_argument("--copies", type=int, default=4, help="input copies cycled through (> LLC)")
    ap.add_argument("--settle", type=float, default=0.3,
                    help="seconds of untimed steps before the warm-up steps (clock ramp-up)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-fraction", type=float, default=None,
                    help="fraction f of A rows and B rows the CPU oracle processes")
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


def inputs_of(name):
    """Host bf16 bit patterns (A, B) of a workload: A [M, K] is the left operand."""
    from bit_gemm_fwht_amd import workloads as wl
    if name == "llama7b_forward_linear":
        x, w, _ = wl.llama_linear(0)
        return x, w
    if name.startswith("backward_2d"):
        w, dy = wl.backward_2d(0)
        return dy, w
    if name == "llama7b_fused_out_q":
        x, w, _ = wl.llama_linear(0)
        return x, w
    if name == "backward_dw_colwise":
        return wl.backward_dw(0)  # dY [tokens, 4096], X [tokens, 4096]
    return wl.nvfp4_4over6(0)


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


def cpu_baseline(wk, a_bits, b_bits, pa, pb, f, out_q=None, ga=None, gb=None):
    """Time the oracle on f*M rows of A, f*N rows of B and the f*M x f*N block of C (and its output
    quantize), and scale to a whole step: T = T_quantize / f + T_gemm / f^2. Column-wise operands
    sample columns of the stored tensors (rows of their transposes)."""
    import oracle as orc
    M, N, K = wk["M"], wk["N"], wk["K"]
    sm, sn = max(int(M * f) // 32 * 32, 32), max(int(N * f) // 32 * 32, 32)  # whole 32-row tiles
    if out_q is not None and out_q.hadamard_n:  # C's sampled rows hold whole rotation chunks
        sn = max(sn // out_q.hadamard_n * out_q.hadamard_n, out_q.hadamard_n)
    if wk.get("colwise"):
        As = np.ascontiguousarray(a_bits[:, :sm].T)
        Bs = np.ascontiguousarray(b_bits[:, :sn].T)
    else:
        As = np.ascontiguousarray(a_bits[:sm])
        Bs = np.ascontiguousarray(b_bits[:sn])

    def q(x, p, ts=None):
        return orc.quantize(x, elem=p.elem, block=p.block, scale_mode=p.scale_mode,
                            round_mode=p.round_mode, hadamard_n=p.hadamard_n, seed=p.seed,
                            tensor_scale=ts)

    t0 = time.perf_counter()
    ca, sa, ta = q(As, pa, ga)
    cb, sb, tb = q(Bs, pb, gb)
    t1 = time.perf_counter()
    a64 = orc.operand_f64(ca, sa, ta, sm, K, elem=pa.elem, block=pa.block, scale_mode=pa.scale_mode)
    if pb.block[0] == 1:
        b64 = orc.operand_f64(cb, sb, tb, sn, K, elem=pb.elem, block=pb.block, scale_mode=pb.scale_mode)
    else:  # 2D tiles: each row takes its tile row's scales
        srow = np.ascontiguousarray(sb.reshape(sn // 32, -1)[np.arange(sn) // 32])
        b64 = orc.operand_f64(cb, srow, tb, sn, K, elem=pb.elem, block=(1, 32), scale_mode=pb.scale_mode)
    c64, _ = orc.gemm_f64(a64, b64)
    if out_q is not None:
        q(c64.astype(np.float32), out_q)
    t2 = time.perf_counter()
    fm, fn = sm / M, sn / N
    t_step = (t1 - t0) / ((fm + fn) / 2) + (t2 - t1) / (fm * fn)
    return {
        "value": round(2.0 * M * N * K / t_step / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"oracle quantize of {sm} A rows + {sn} B rows ({t1 - t0:.2f} s) and the fp64 "
                   f"GEMM of their {sm}x{sn} block over K={K}"
                   f"{' with its output quantize' if out_q is not None else ''} ({t2 - t1:.2f} s), "
                   f"scaled to a full step as T_q/f + T_gemm/f^2 with f={f} (the sampled row fractions)"),
        "step_s": round(t_step, 3),
    }


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
    dev = torch.device("cuda:0")
    wk = WORKLOADS[args.workload]
    M, N, K = wk["M"], wk["N"], wk["K"]
    pa, pb = params_of(fp4, wk["a"]), params_of(fp4, wk["b"])
    a_bits, b_bits = inputs_of(args.workload)
    a0 = torch.from_numpy(a_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    b0 = torch.from_numpy(b_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    As = [a0] + [a0.clone() for _ in range(args.copies - 1)]
    Bs = [b0] + [b0.clone() for _ in range(args.copies - 1)]
    qa = [fp4.empty_qtensor(M, K, pa, dev) for _ in range(args.copies)]
    qb = [fp4.empty_qtensor(N, K, pb, dev) for _ in range(args.copies)]
    cs = [torch.empty(M, N, dtype=torch.bfloat16, device=dev) for _ in range(args.copies)]
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
    if nb:
        wsg = torch.empty(nb, dtype=torch.uint8, device=dev)

    # Timing events on the launch stream: one before each step's quantize and one between its
    # quantize and GEMM; a GEMM ends where the next step's first event is recorded (plus one after
    # the last step), so each step adds two event records, not three.
    def step(i, ev=None):
        j = i % args.copies
        if ev is not None:
            ev[2 * i].record()
        if wk["batched"]:
            fp4.quantize_batch([As[j], Bs[j]], pa, outs=[qa[j], qb[j]])
        else:
            quantize_one(As[j], pa, out=qa[j], workspace=wsa,
                         tensor_scale=qa[j].tensor_scale if ga is not None else None)
            quantize_one(Bs[j], pb, out=qb[j], workspace=wsb,
                         tensor_scale=qb[j].tensor_scale if gb is not None else None)
        if ev is not None:
            ev[2 * i + 1].record()
        if oq is not None:
            fp4.gemm(qa[j], qb[j], out=cs[j], workspace=wsg, out_q=oq, q_out=cq[j])
        else:
            fp4.gemm(qa[j], qb[j], out=cs[j], workspace=wsg)

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
    evs = [HipTimingEvent(stream) for _ in range(2 * args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs)
    evs[-1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tq = np.mean([evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(args.steps)]) * 1e-3
    t_g = np.mean([evs[2 * i + 1].elapsed_time(evs[2 * i + 2]) for i in range(args.steps)]) * 1e-3
    ms_per_step = wall / args.steps * 1e3

    flops = 2.0 * M * N * K

    def qbytes(rows, p):  # bf16 in, codes and scales out
        cb, sb, _ = fp4.buffer_sizes(rows, K, p)
        return rows * K * 2 + cb + sb

    bytes_q = qbytes(M, pa) + qbytes(N, pb)
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
                   "input_copies": args.copies},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / peak, 4),
                     "traffic": measured_traffic() if args.workload == HEADLINE else None,
                     "kernel": wk["kernel"]},
        "quantize": {"GB/s": round(bytes_q / tq / 1e9, 1),
                     "frac": round(bytes_q / tq / 1e9 / HBM_PEAK_GBS, 4),
                     "us": round(tq * 1e6, 2), "bytes": int(bytes_q),
                     "launches": ("one batched k_segment launch for A and B" if wk["batched"]
                                  else "separate launches for A and B")
                     + (", column-wise" if colwise else "") + (", given tensor scales" if ga is not None else "")},
        "gemm": {"TFLOP/s": round(gemm_tflops, 2), "frac": round(gemm_tflops / peak, 4),
                 "us": round(t_g * 1e6, 2), "flops": flops},
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
