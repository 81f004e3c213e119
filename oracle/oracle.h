/*
 * Plain, slow CPU oracle for block-scaled FP4 / FP8 quantization, the blockwise Walsh-Hadamard
 * rotation and the block-scaled GEMM.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the benchmark's CPU-baseline
 * leg may load this library. The product path (the HIP library) never links, loads or calls it, and
 * shares no code, header, table or constant with it.
 *
 * Every function computes what the source pages define, one element at a time, in the order the
 * pages give, with IEEE fp32 round-to-nearest-even for each fp32 operation (built with
 * -ffp-contract=off, no fast-math, denormals kept) and exact fp64 sums for the GEMM.
 *
 * Sources (cited by title and section):
 *   [LowBit]  caveduck.io post "low-bit quantization" (lightweighting series #4): the FP4 grid
 *             equation in "FP4라는 무리수", §1 (per-tensor scale, outlier collapse), §2 (group
 *             scales, MXFP4), §3 (2^k scales, effective bits), §7 (Hadamard rotation).
 *   [Quartet] lecture notes "Quartet — Native 4-bit training that actually trains": Hadamard
 *             rotation equation, QuTLASS kernel list (stochastic rounding, online quantization).
 *   [TIBQ]    abstract of "Stable FP4 Training via Transposition-Invariant Block Quantization":
 *             2D block scales, truncation-free scaling, stochastic rounding.
 *   [4over6]  summary page of "Four Over Six: More Accurate NVFP4 Quantization with Adaptive
 *             Block Scaling": methodology steps 1-3 (two candidate scales per block, keep the one
 *             with the lower error).
 *   [Philox]  Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11.
 */
#ifndef BGF_ORACLE_H
#define BGF_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element formats */
#define ORC_ELEM_E2M1 0   /* FP4: 1 sign, 2 exponent, 1 mantissa bit */
#define ORC_ELEM_E4M3 1   /* FP8 (OCP E4M3FN): the MXFP8 variant */
/* scale rules */
#define ORC_SCALE_E8M0_FLOOR 0  /* 2^(floor(log2 amax) - emax_elem) */
#define ORC_SCALE_E8M0_CEIL 1   /* truncation-free: smallest 2^k with maxval * 2^k >= amax */
#define ORC_SCALE_NV 2          /* E4M3 block scale x fp32 tensor scale (NVFP4) */
#define ORC_SCALE_NV_4OVER6 3   /* NVFP4 with the 4/6 choice per block */
#define ORC_SCALE_F32 4         /* fp32 scale S = amax / maxval */
/* NVFP4 with a tensor scale g given by the caller (delayed scaling: g from an earlier amax, the
 * moving-average scale the Quartet notes' open questions point to) instead of this tensor's amax;
 * tensor_scale is then an input */
#define ORC_SCALE_NV_GIVEN 5
#define ORC_SCALE_NV_4OVER6_GIVEN 6
/* rounding */
#define ORC_ROUND_RNE 0
#define ORC_ROUND_SR 1
/* input dtypes */
#define ORC_IN_F32 0
#define ORC_IN_BF16 1

/* ---- number formats ---- */
uint8_t orc_e2m1_rne(float v);                 /* nearest of the 15 values, ties to even code */
uint8_t orc_e2m1_sr(float v, uint32_t u16);    /* stochastic rounding with a 16-bit uniform */
float orc_e2m1_value(uint8_t code);
uint8_t orc_e4m3_rne(float v);                 /* OCP E4M3FN, ties to even, saturating at 448 */
uint8_t orc_e4m3_sr(float v, uint32_t u16);
float orc_e4m3_value(uint8_t code);
float orc_e8m0_value(uint8_t code);            /* 2^(code-127); 255 is NaN */
uint16_t orc_bf16_rne(float v);                /* fp32 -> bf16 bits, round to nearest even */

/* ---- random bits ---- */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
uint32_t orc_sr_u16(uint64_t seed, uint64_t idx);  /* the 16-bit uniform of element idx */

/* ---- rotation ---- */
int orc_fwht(float* x, int64_t len, int n);    /* in place on each n-chunk of x[0..len) */

/* ---- scales ---- */
int orc_e8m0_scale_exp(float amax, int elem, int rule);   /* returns k (E8M0 code = k + 127) */

/* ---- quantize / dequantize ----
 * x: [rows, cols] row-major (fp32 or bf16 bits). Blocks are block_rows x block_cols tiles
 * (1 x 32 MX, 1 x 16 NV, 32 x 32 2D, 1 x cols per row, rows x cols per tensor).
 * codes: E2M1 -> [rows, cols/2] bytes, element 2j in the low nibble of byte j;
 *        E4M3 -> [rows, cols] bytes.
 * scales: [rows/block_rows, cols/block_cols]; u8 E8M0 / E4M3 codes, or fp32 for ORC_SCALE_F32.
 * tensor_scale: NV modes only, receives g (may be NULL otherwise); the _GIVEN modes read g from it.
 * Returns 0, or a negative number for an argument it does not accept. */
int orc_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int elem,
                 int block_rows, int block_cols, int scale_mode, int round_mode, int hadamard_n,
                 uint64_t seed, uint8_t* codes, void* scales, float* tensor_scale);

/* y = RN(val(q) * d), then the same rotation again when hadamard_n > 0 (H/sqrt(n) is its own
 * inverse). y: fp32 [rows, cols]. */
int orc_dequantize(const uint8_t* codes, const void* scales, const float* tensor_scale,
                   int64_t rows, int64_t cols, int elem, int block_rows, int block_cols,
                   int scale_mode, int hadamard_n, float* y);

/* The values the block-scaled matrix core multiplies, in fp64, for a K-quantized operand
 * [rows, K]. MX (E8M0) operands: val(q) * 2^k, exact. NVFP4 operands: each 32-wide K group is
 * re-expressed as E4M3 elements under one power-of-two scale (the FP8 rescale); with_nv_exact = 1
 * returns the exact NVFP4 values val(q) * val(s) * g instead, for the informational gap. */
int orc_operand_f64(const uint8_t* codes, const void* scales, const float* tensor_scale,
                    int64_t rows, int64_t K, int elem, int block_rows, int block_cols,
                    int scale_mode, int with_nv_exact, double* out);

/* The FP8 re-expression of an NVFP4 operand (E2M1 codes [rows, K/2], E4M3 block scales
 * [rows, K/block_cols], block_cols dividing 32): per 32-wide K group, E = the smallest exponent with
 * 448 * 2^E >= 6 S (S the group's largest block scale; E = -127 when S = 0) and elements
 * f = E4M3(val(q) * s_blk * 2^-E), nearest even. out_codes: E4M3 [rows, K]; out_scales: E8M0
 * codes E + 127 [rows, K/32]. */
int orc_nv_to_mx8(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t K,
                  int block_cols, uint8_t* out_codes, uint8_t* out_scales);

/* C[m,n] = sum_k a[m,k] * b[n,k] in fp64 and S[m,n] = sum_k |a[m,k] b[n,k]| (the error scale).
 * Full or at (ms[i], ns[i]) pairs. */
void orc_gemm_f64(const double* a, const double* b, int64_t M, int64_t N, int64_t K,
                  double* c, double* sabs);
void orc_gemm_f64_sampled(const double* a, const double* b, int64_t K, const int64_t* ms,
                          const int64_t* ns, int64_t count, double* c, double* sabs);


/* ---- array helpers (element functions applied one by one) ---- */
void orc_encode_array(const float* v, int64_t n, int elem, int round_mode, uint64_t seed,
                      uint64_t idx0, uint8_t* out);
void orc_decode_array(const uint8_t* q, int64_t n, int elem, float* out);
void orc_sr_u16_array(uint64_t seed, const uint64_t* idx, int64_t n, uint32_t* out);
void orc_philox_array(const uint32_t* ctr, const uint32_t* key, int64_t n, uint32_t* out);
void orc_bf16_array(const float* v, int64_t n, uint16_t* out);
void orc_sr_with_u_array(const float* v, const uint32_t* u16, int64_t n, int elem, uint8_t* out);

#ifdef __cplusplus
}
#endif
#endif
