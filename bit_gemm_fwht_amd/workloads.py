"""Seeded synthetic inputs for the quantize + GEMM path.

This module only draws random numbers and lays them out; it holds none of the quantizer's or the
GEMM's arithmetic. Both the HIP path and the CPU oracle are fed from it.

Shapes and distributions follow the workloads the source pages describe (stand-ins where the pages
used trained weights or datasets that are not available here):
  tiny_mxfp4    A, B fp32 256x256 ~ N(0,1), seed 0, one element of A set to 50 x max|A|
                (the outlier experiment of the caveduck.io post, §1).
  mnist_mlp     fp32 weights 256x784, 128x256, 10x128 ~ N(0, 0.05^2) (the MLP 784->256->128->10
                of the same post; random stand-ins for its trained weights), optional 50x outlier
                in fc1.
  llama_linear  X bf16 4096x4096 ~ N(0,1) with 1% of channels x20; W bf16 [11008, 4096]
                ~ N(0, 0.02^2) (a Llama-7B-shaped forward linear, stored K-contiguous).
  backward_2d   W bf16 4096x4096 ~ N(0, 0.02^2); dY bf16 8192x4096 ~ Student-t(3) x 1e-3.
  nvfp4_4over6  X bf16 8192x8192 ~ Laplace(0,1) with 0.1% of entries x30; W bf16 8192x8192
                ~ N(0, 0.02^2).
  forward_2d    X bf16 8192x4096 ~ Student-t(3), W bf16 4096x4096 ~ N(0, 0.02^2): Y = X W with W
                contracted along its first axis (the 2D-quantized weight reused through its transpose).
  backward_dw   dY bf16 8192x4096 ~ Student-t(3) x 1e-3 and X bf16 8192x4096 ~ N(0,1) with 1% of
                channels x20: the operands of dW = dY^T X (the column-wise quantize).
Every generator takes its own numpy Generator seeded with `seed`, and draws the tensors in the
order listed. bf16 tensors are returned as uint16 bit patterns (round-to-nearest-even of the fp32
draw).
"""
from __future__ import annotations

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest even) and return the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def set_outlier(x: np.ndarray, factor: float = 50.0) -> tuple[int, int]:
    """Set the first row-major argmax of |x| to +factor * max|x| (in place); return its index."""
    flat = x.reshape(-1)
    i = int(np.argmax(np.abs(flat)))
    flat[i] = np.float32(factor) * np.float32(np.abs(flat[i]))
    return np.unravel_index(i, x.shape)


def tiny_mxfp4(seed: int = 0, outlier: bool = True):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((256, 256), dtype=np.float32)
    b = rng.standard_normal((256, 256), dtype=np.float32)
    if outlier:
        set_outlier(a)
    return a, b


def mnist_mlp(seed: int = 0, outlier: bool = False):
    rng = np.random.default_rng(seed)
    shapes = [("fc1", (256, 784)), ("fc2", (128, 256)), ("fc3", (10, 128))]
    out = {}
    for name, shp in shapes:
        out[name] = (rng.standard_normal(shp, dtype=np.float32) * np.float32(0.05)).astype(np.float32)
    if outlier:
        set_outlier(out["fc1"])
    return out


def llama_linear(seed: int = 0, m: int = 4096, n: int = 11008, k: int = 4096):
    """X [m, k] and W [n, k] as bf16 bits; the outlier channel set is drawn after X."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k), dtype=np.float32)
    nch = int(round(0.01 * k))
    ch = rng.choice(k, size=nch, replace=False)
    x[:, ch] *= np.float32(20.0)
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    return f32_to_bf16_bits(x), f32_to_bf16_bits(w), np.sort(ch)


def backward_2d(seed: int = 0, m: int = 8192, n: int = 4096, k: int = 4096):
    """W [n, k] ~ N(0, 0.02^2) and dY [m, k] ~ Student-t(3) * 1e-3, as bf16 bits. dX = dY W^T
    contracts both operands over their contiguous axis (k), the layout the GEMM takes."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    dy = (rng.standard_t(3.0, size=(m, k)) * 1e-3).astype(np.float32)
    return f32_to_bf16_bits(w), f32_to_bf16_bits(dy)


def forward_2d(seed: int = 0, m: int = 8192, k: int = 4096, n: int = 4096):
    """X [m, k] ~ Student-t(3) (activations) and W [k, n] ~ N(0, 0.02^2) as bf16 bits: the forward
    Y = X W of the layer whose weight the backward workload quantizes with 2D blocks, contracting W
    along its first (non-contiguous) axis."""
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3.0, size=(m, k)).astype(np.float32)
    w = rng.standard_normal((k, n), dtype=np.float32) * np.float32(0.02)
    return f32_to_bf16_bits(x), f32_to_bf16_bits(w)


def nvfp4_4over6(seed: int = 0, m: int = 8192, n: int = 8192, k: int = 8192):
    rng = np.random.default_rng(seed)
    x = rng.laplace(0.0, 1.0, size=(m, k)).astype(np.float32)
    nout = int(round(0.001 * m * k))
    idx = rng.choice(m * k, size=nout, replace=False)
    x.reshape(-1)[idx] *= np.float32(30.0)
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    return f32_to_bf16_bits(x), f32_to_bf16_bits(w)


def backward_dw(seed: int = 0, t: int = 8192, d_out: int = 4096, d_in: int = 4096):
    """dY [t, d_out] ~ Student-t(3) * 1e-3 and X [t, d_in] ~ N(0, 1) with 1% of channels x20, as
    bf16 bits: the two operands of the weight gradient dW = dY^T X, which contracts over the token
    axis t (the first axis of both as stored)."""
    rng = np.random.default_rng(seed)
    dy = (rng.standard_t(3.0, size=(t, d_out)) * 1e-3).astype(np.float32)
    x = rng.standard_normal((t, d_in), dtype=np.float32)
    ch = rng.choice(d_in, size=int(round(0.01 * d_in)), replace=False)
    x[:, ch] *= np.float32(20.0)
    return f32_to_bf16_bits(dy), f32_to_bf16_bits(x)


def scaled_down(kind: str, seed: int = 0, **shape):
    """The same distributions at other sizes (parity cases that span a few tiles and a tail)."""
    return {"llama_linear": llama_linear, "backward_2d": backward_2d,
            "nvfp4_4over6": nvfp4_4over6}[kind](seed, **shape)
