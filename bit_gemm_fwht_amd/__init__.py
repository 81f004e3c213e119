"""Block-scaled FP4 / FP8 quantization and GEMM for AMD MI355X (gfx950).

The work is done by hand-written HIP kernels in libbgf.so behind the C ABI of include/fp4.h:
blockwise Walsh-Hadamard rotation, MXFP4 / MXFP8 / NVFP4 / 2D-tile / 4-over-6 quantization with
round-to-nearest-even or Philox stochastic rounding, column-wise quantization (of x^T without
forming it), batched quantization of several tensors in one launch, dequantization, and the block-scaled GEMM on the gfx950 matrix cores. `fp4` is the Python binding (torch supplies memory and streams);
`workloads` draws the seeded synthetic inputs.
"""
from .fp4 import (DT_BF16, DT_F32, E2M1, E4M3, MXFP4, ROUND_RNE, ROUND_SR, SCALE_E8M0_CEIL,
                  SCALE_E8M0_FLOOR, SCALE_F32, SCALE_NV, SCALE_NV_4OVER6, SCALE_NV_GIVEN,
                  SCALE_NV_4OVER6_GIVEN, Fp4Error, Params, QTensor, dequantize, empty_qtensor,
                  gemm, hadamard, quantize, quantize_batch, quantize_colwise)

__all__ = ["DT_BF16", "DT_F32", "E2M1", "E4M3", "MXFP4", "ROUND_RNE", "ROUND_SR",
           "SCALE_E8M0_CEIL", "SCALE_E8M0_FLOOR", "SCALE_F32", "SCALE_NV", "SCALE_NV_4OVER6",
           "SCALE_NV_GIVEN", "SCALE_NV_4OVER6_GIVEN", "Fp4Error", "Params", "QTensor",
           "dequantize", "empty_qtensor", "gemm", "hadamard", "quantize", "quantize_batch",
           "quantize_colwise"]
