// Internal interfaces between the C ABI (fp4_abi.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bgf {

enum { DT_F32 = 0, DT_BF16 = 1 };
enum { ELEM_E2M1 = 0, ELEM_E4M3 = 1 };
enum { SC_E8M0 = 0, SC_NV = 1, SC_F32 = 2 };  // scale classes (floor/ceil and 4/6 are runtime)
enum { RND_RNE = 0, RND_SR = 1 };
enum { PASS_QUANT = 0, PASS_AMAX = 1, PASS_ROTATE = 2 };

struct SegArgs {
    const void* x;
    int64_t rows, cols, ldx;
    int64_t nseg;          // rows * cols / 32
    uint8_t* codes;
    void* scales;
    float* tensor_scale;   // NV: receives g
    uint32_t* ws;          // tensor amax (fp32 bits), NV modes
    float* yrot;           // rotation pass output [rows, cols] fp32
    uint64_t seed;
    int ceil_rule;
    int four_six;
    int nv_given;          // NV: g is read from tensor_scale (no amax pass)
    // column-wise view: rows x cols describe T = x^T, x is [cols, rows] with row pitch ldx
    int colwise;
};

// Several tensors quantized with one mode in one launch: the workgroups of item i are
// [start[i], start[i + 1]) (start[n] = the grid size); one item for every other launch.
constexpr int kMaxBatch = 4;
struct SegBatch {
    SegArgs t[kMaxBatch];
    uint32_t start[kMaxBatch];
    int n;
};

struct RowArgs {
    const void* x;
    int64_t rows, cols, ldx;
    uint8_t* codes;
    void* scales;
    uint32_t* ws;
    uint64_t seed;
    int ceil_rule;
    int per_tensor;
};

struct DeqArgs {
    const uint8_t* codes;
    const void* scales;
    const float* tensor_scale;
    int64_t rows, cols, nseg;
    void* y;
    int64_t ldy;
    int per_tensor;
};

hipError_t launch_segment(const SegArgs& a, int in_dtype, int hn, int elem, int sc, int rnd, int br,
                          int bc, int pass, hipStream_t s);
// PASS_QUANT of n <= kMaxBatch tensors sharing every mode parameter, in one launch
hipError_t launch_segment_batch(const SegArgs* items, int n, int in_dtype, int hn, int elem, int sc, int rnd,
                                int br, int bc, hipStream_t s);
hipError_t launch_zero_u32(uint32_t* p, int n, hipStream_t s);
hipError_t launch_amax_rows(const void* x, int in_dtype, int64_t rows, int64_t cols, int64_t ldx,
                            uint32_t* ws, hipStream_t s);
hipError_t launch_rowblock(const RowArgs& a, int in_dtype, int elem, int sc, int rnd, hipStream_t s);
hipError_t launch_dequant_segment(const DeqArgs& a, int elem, int sc, int br, int bc, int hn,
                                  int out_dtype, hipStream_t s);
hipError_t launch_dequant_rowblock(const DeqArgs& a, int elem, int sc, int out_dtype, hipStream_t s);

// 2D (32 x 32) quantized tensor [rows, cols] -> the quantized form of its transpose [cols, rows]
struct TransposeArgs {
    const uint8_t* codes;
    const uint8_t* scales;
    int64_t rows, cols;
    uint8_t* out_codes;
    uint8_t* out_scales;
};
hipError_t launch_transpose_2d(const TransposeArgs& a, int elem, hipStream_t s);

// GEMM
struct GemmArgs {
    const uint8_t* a;        // [M, K/2] (E2M1) or [M, K] (E4M3)
    const uint8_t* b;        // [N, K/2] or [N, K]
    const uint8_t* sa;       // [M, K/32] E8M0, or [M, K/16] E4M3 (NV)
    const uint8_t* sb;       // [N, K/32], [N/32, K/32] (2D), or [N, K/16] (NV)
    const float* ga;         // NV tensor scales
    const float* gb;
    int64_t M, N, K;
    void* c;
    int64_t ldc;
    int b_2d;
    // fused output quantization along N (MX groups of 32)
    uint8_t* qcodes;
    uint8_t* qscales;
    int q_elem, q_ceil, q_round, q_hn;  // q_hn: rotation of C along N before the quantize (0 = none)
    uint64_t q_seed;
    // NV operands re-expressed as MXFP8 (workspace)
    uint8_t* a8;
    uint8_t* sa8;
    uint8_t* b8;
    uint8_t* sb8;
};

// NVFP4 [rows, cols] -> E4M3 [rows, cols] + E8M0 [rows, cols / 32] (the GEMM's FP8 re-expression)
hipError_t launch_nv_to_fp8(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                            uint8_t* out, uint8_t* out_scales, hipStream_t s);

// MXFP4 GEMM (256 x 256 tile path) whose A operand is rotated (hn along K) and quantized (E8M0,
// E2M1, rnd) from `a` inside the same launch; g.a / g.sa are a's codes / scales outputs. ws: at
// least 2 words (a counter and a status word, cleared by the launch).
hipError_t launch_gemm_fused_a(const GemmArgs& g, const SegArgs& a, int in_dtype, int hn, int rnd, int c_dtype,
                               uint32_t* ws, hipStream_t s);

// kind: 0 MXFP4, 1 MXFP8, 2 NVFP4 (via the FP8 rescale)
hipError_t launch_gemm(const GemmArgs& g, int kind, int c_dtype, int fused_q, hipStream_t s);

}  // namespace bgf
