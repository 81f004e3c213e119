"""Benchmark of the quantize + MXFP4 GEMM hot path on one MI355X.

One step = the whole path over one batch of a Llama-7B-shaped forward linear:
  X bf16 [4096, 4096] (N(0,1), 1% of channels x20) and W bf16 [11008, 4096] (N(0, 0.02^2)),
  both rotated along K by blockwise H_128 / sqrt(128) and quantized to MXFP4 (E2M1 elements,
  one E8M0 floor scale per 32, round to nearest even) in one batched launch, then C = X W^T on the
  MXFP4 operands, fp32 accumulation, bf16 output.
Inputs are resident in HBM before timing starts; the step cycles over several copies of X and W
(more than the 256 MB last-level cache) so that every step reads its inputs from HBM.

Prints one JSON line. `value` is the step's effective throughput in TFLOP/s (GEMM FLOPs over the
whole step time, quantization included); the per-kernel GB/s / TFLOP/s and roofline fractions are
in the extra fields. `roofline` is the dominant kernel (the GEMM): algorithmic FLOPs per launch over
its average launch time from HIP events on the launch stream; its `traffic` is the measured memory
traffic per launch from the committed counter summary, reported only while the summary's kernel
source hash matches the current source. `cpu_baseline` times the CPU oracle on a bounded sample of
the same step.

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
M, N, K = 4096, 11008, 4096
HN = 128
ROOT = os.path.dirname(os.path.abspath(__file__))
GEMM_SRC = os.path.join(ROOT, "bit_gemm_fwht_amd", "csrc", "gemm.hip")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemm_llama7b_forward_linear_traffic.md")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--copies", type=int, default=4, help="input copies cycled through (> LLC)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-fraction", type=float, default=0.25,
                    help="fraction f of X rows and W rows the CPU oracle processes")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration) and exit")
    return ap.parse_args()


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


def copy_calibration(mib):
    import torch
    n = mib << 20
    x = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)


def cpu_baseline(x_bits, w_bits, f):
    """Time the oracle on f*M rows of X, f*N rows of W and the f*M x f*N block of C, and scale to
    a whole step: T = T_quantize / f + T_gemm / f^2."""
    import oracle as orc
    sm, sn = max(int(M * f), 1), max(int(N * f), 1)
    xs = np.ascontiguousarray(x_bits[:sm])
    ws = np.ascontiguousarray(w_bits[:sn])
    t0 = time.perf_counter()
    ca, sa, _ = orc.quantize(xs, hadamard_n=HN)
    cb, sb, _ = orc.quantize(ws, hadamard_n=HN)
    t1 = time.perf_counter()
    a64 = orc.operand_f64(ca, sa, None, sm, K)
    b64 = orc.operand_f64(cb, sb, None, sn, K)
    orc.gemm_f64(a64, b64)
    t2 = time.perf_counter()
    t_step = (t1 - t0) / f + (t2 - t1) / (f * f)
    return {
        "value": round(2.0 * M * N * K / t_step / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"oracle quantize of {sm} X rows + {sn} W rows ({t1 - t0:.2f} s) and the fp64 "
                   f"GEMM of their {sm}x{sn} block over K={K} ({t2 - t1:.2f} s), scaled to a full "
                   f"step as T_q/f + T_gemm/f^2 with f={f}"),
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
    from bit_gemm_fwht_amd import workloads as wl

    fp4.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    x_bits, w_bits, _ = wl.llama_linear(0, m=M, n=N, k=K)
    x0 = torch.from_numpy(x_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    w0 = torch.from_numpy(w_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    xs = [x0] + [x0.clone() for _ in range(args.copies - 1)]
    ws = [w0] + [w0.clone() for _ in range(args.copies - 1)]
    params = fp4.Params(hadamard_n=HN)
    qx = [fp4.empty_qtensor(M, K, params, dev) for _ in range(args.copies)]
    qw = [fp4.empty_qtensor(N, K, params, dev) for _ in range(args.copies)]
    cs = [torch.empty(M, N, dtype=torch.bfloat16, device=dev) for _ in range(args.copies)]

    # Timing events on the launch stream: one before each step's quantize and one between its
    # quantize and GEMM; a GEMM ends where the next step's first event is recorded (plus one after
    # the last step), so each step adds two event records, not three.
    def step(i, ev=None):
        j = i % args.copies
        if ev is not None:
            ev[2 * i].record()
        fp4.quantize_batch([xs[j], ws[j]], params, outs=[qx[j], qw[j]])
        if ev is not None:
            ev[2 * i + 1].record()
        fp4.gemm(qx[j], qw[j], out=cs[j])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps + 1)]
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
    bytes_q = (M + N) * K * (2 + 0.5 + 1 / 32)  # bf16 in, E2M1 codes and E8M0 scales out
    gemm_tflops = flops / t_g / 1e12
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
        "dtype": "mxfp4",
        "data": "synthetic (seeded numpy draws of the workload's shapes and distributions)",
        "config": {"workload": "llama7b_forward_linear", "M": M, "N": N, "K": K,
                   "input": "bf16", "hadamard_n": HN,
                   "quant": "E2M1 + E8M0 per 32 (floor), RNE", "output": "bf16",
                   "input_copies": args.copies},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": FP4_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / FP4_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(),
                     "kernel": "k_gemm_big (MXFP4, 256x256 tiles, 32x32x64 scaled MFMA, bf16 out)"},
        "quantize_xw": {"GB/s": round(bytes_q / tq / 1e9, 1),
                        "frac": round(bytes_q / tq / 1e9 / HBM_PEAK_GBS, 4),
                        "us": round(tq * 1e6, 2), "bytes": int(bytes_q),
                        "kernel": "k_segment (bf16, FWHT-128, MXFP4; X and W in one launch)"},
        "gemm": {"TFLOP/s": round(gemm_tflops, 2), "frac": round(gemm_tflops / FP4_PEAK_TFLOPS, 4),
                 "us": round(t_g * 1e6, 2), "flops": flops},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x_bits, w_bits, args.cpu_fraction)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
