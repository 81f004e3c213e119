/*
 * fp4.h - C ABI of the MI355X (gfx950) block-scaled FP4 / FP8 quantize + GEMM library
 * (libbgf.so, built from bit_gemm_fwht_amd/csrc).
 *
 * What it computes (sources cited by page title and section):
 *  - the blockwise Hadamard rotation y = x (H_n / sqrt(n)) of the lecture notes "Quartet — Native
 *    4-bit training that actually trains" (section on Hadamard rotation) and of §7 of the
 *    caveduck.io post "low-bit quantization" (rotation to spread outliers, O(n log n));
 *  - block-scaled quantization to FP4 E2M1 (the 15-value grid of that post's section
 *    "FP4라는 무리수") or FP8 E4M3, with one shared scale per block: per tensor (§1), per row or
 *    per 32-element group / MXFP4 (§2), power-of-two E8M0 scales (§3), 32x32 transposition-
 *    invariant 2D blocks with truncation-free scales and stochastic rounding ("Stable FP4 Training
 *    via Transposition-Invariant Block Quantization", abstract), NVFP4 16-element blocks with an
 *    E4M3 block scale and an fp32 tensor scale, and the adaptive 4/6 choice ("Four Over Six: More
 *    Accurate NVFP4 Quantization with Adaptive Block Scaling", methodology);
 *  - the GEMM on the quantized operands, one call, fp32 accumulation (the QuTLASS kernel list
 *    of the Quartet notes: 4-bit GEMM, online quantization of the output).
 *
 * Conventions for every entry point:
 *  - Pointers named x, y, codes, scales, tensor_scale, C and workspace are DEVICE pointers
 *    (memory of the current HIP device); fp4_qparams / fp4_qtensor structs are HOST pointers.
 *  - The caller owns every buffer and keeps it alive until the work queued on `stream` (a
 *    hipStream_t, or NULL for the default stream) has completed. The library allocates nothing,
 *    keeps no pointer after returning and holds no mutable global state beyond write-once facts
 *    per device (its CU count, which kernels have had their LDS limit raised; both thread-safe)
 *    and the allocation-free quantize's scratch below: calls on different streams may run
 *    concurrently.
 *  - All work is queued asynchronously on `stream`; a return of FP4_OK means "queued".
 *  - Every argument is validated on the host before anything is queued. On any error nothing is
 *    queued and the outputs are left untouched. A launch failure returns FP4_ERR_HIP; a device
 *    fault surfaces at the caller's next synchronisation. No C++ exception crosses this ABI.
 *  - Non-finite inputs are outside the contract: kernels do not fault, results are unspecified. So
 *    are finite inputs whose rotation overflows fp32 in an intermediate butterfly stage (max |x|
 *    near 2^128 / n for hadamard_n = n): the overflowed values become inf / NaN, whose payloads and
 *    ordering are not reproduced bit for bit.
 *
 * Layouts:
 *  - x / y: row-major [rows, cols] with leading dimension ld (elements), fp32 or bf16.
 *  - codes: E2M1 -> [rows, cols/2] bytes, element 2j in the low nibble of byte j, bit 3 of a
 *    nibble is the sign; E4M3 -> [rows, cols] bytes. Contiguous.
 *  - scales: row-major [rows/block_rows, cols/block_cols]; one byte per block (E8M0 code k+127,
 *    or an E4M3 code in the NVFP4 modes), or one fp32 per block in FP4_SCALE_F32. Contiguous.
 *  - tensor_scale: one fp32 (NVFP4 modes only), written by fp4_quantize (read by it in the _GIVEN
 *    modes), read by the others.
 *  - The quantization axis is always the contiguous `cols` axis (K for GEMM operands).
 */
#ifndef BGF_FP4_H
#define BGF_FP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP4_ABI_VERSION 1

typedef enum {
    FP4_OK = 0,
    FP4_ERR_INVALID_ARG = 1,  /* null pointer, non-positive size, sizes that do not tile */
    FP4_ERR_UNSUPPORTED = 2,  /* a valid combination this library does not implement */
    FP4_ERR_ALIGNMENT = 3,    /* a device pointer or row pitch not aligned to 16 bytes */
    FP4_ERR_WORKSPACE = 4,    /* workspace missing or smaller than the size query returned */
    FP4_ERR_HIP = 5,          /* the HIP runtime rejected a launch */
    FP4_ERR_INTERNAL = 6
} fp4_status;

enum { FP4_DT_F32 = 0, FP4_DT_BF16 = 1 };
enum { FP4_ELEM_E2M1 = 0, FP4_ELEM_E4M3 = 1 };
enum {
    FP4_SCALE_E8M0_FLOOR = 0, /* 2^(floor(log2 amax) - emax): emax 2 for E2M1 (6 = 1.5*2^2),
                                  8 for E4M3 (448 = 1.75*2^8); values above the grid saturate */
    FP4_SCALE_E8M0_CEIL = 1,  /* truncation-free: the smallest 2^k with maxval * 2^k >= amax */
    FP4_SCALE_NV = 2,         /* NVFP4: s = E4M3(amax_b / (6 g)), g = amax_tensor / (6 * 448) */
    FP4_SCALE_NV_4OVER6 = 3,  /* NVFP4, per block the better of the maps amax->6 and amax->4 */
    FP4_SCALE_F32 = 4,        /* fp32 S = amax / maxval (per tensor / per row / per group) */
    /* NVFP4 (and 4/6) with the tensor scale g GIVEN by the caller in *tensor_scale (an input):
     * delayed scaling, e.g. g from an earlier step's amax, so the quantize is a single pass with no
     * tensor amax; blocks whose amax exceeds 6 * 448 * g get the largest block scale and saturate */
    FP4_SCALE_NV_GIVEN = 5,
    FP4_SCALE_NV_4OVER6_GIVEN = 6
};
enum { FP4_ROUND_RNE = 0, FP4_ROUND_SR = 1 };

/* How a tensor is quantized.
 *  elem        FP4_ELEM_E2M1 or FP4_ELEM_E4M3.
 *  block_rows, block_cols
 *              (1, 32) MX groups; (1, 16) NVFP4 blocks (also allowed for E8M0 / F32 scales);
 *              (32, 32) 2D tiles (E8M0 scales); (1, cols) per row; (rows, cols) per tensor.
 *  scale_mode  FP4_SCALE_*.
 *  round_mode  FP4_ROUND_RNE (ties to even, saturating) or FP4_ROUND_SR (stochastic rounding).
 *  hadamard_n  0 (no rotation) or 16, 32, 64, 128, 256: rotate each contiguous n-chunk of a row
 *              by H_n / sqrt(n) (Sylvester order) before quantizing; n must divide cols.
 *  seed        Philox4x32-10 key for SR. Element (r, c) draws the 16-bit uniform
 *              u = half (idx & 1) of word (idx >> 1) & 3 of Philox(counter = idx >> 3, key = seed),
 *              idx = r * cols + c, and rounds up iff u < p * 2^16 where p is its position between
 *              the two neighbouring grid values. Results are reproducible for a given seed. */
typedef struct fp4_qparams {
    int32_t elem;
    int32_t block_rows;
    int32_t block_cols;
    int32_t scale_mode;
    int32_t round_mode;
    int32_t hadamard_n;
    uint64_t seed;
} fp4_qparams;

/* A quantized tensor as the GEMM reads (A, B) or writes (C_q) it. codes / scales / tensor_scale are
 * device pointers with the layouts above; rows x cols is the logical shape (cols = K for GEMM
 * operands); p describes how it was quantized. */
typedef struct fp4_qtensor {
    void* codes;
    void* scales;
    float* tensor_scale;
    int64_t rows;
    int64_t cols;
    fp4_qparams p;
} fp4_qtensor;

int fp4_abi_version(void);
const char* fp4_status_string(int status);

/* Byte sizes of the codes / scales buffers for a rows x cols tensor quantized with *p, and of the
 * device workspace fp4_quantize needs (0, or 256 for the modes that first take a tensor-wide
 * amax: NVFP4 and per-tensor blocks). Return -1 for arguments fp4_quantize would reject. */
int64_t fp4_codes_bytes(int64_t rows, int64_t cols, const fp4_qparams* p);
int64_t fp4_scales_bytes(int64_t rows, int64_t cols, const fp4_qparams* p);
int64_t fp4_workspace_bytes(int64_t rows, int64_t cols, const fp4_qparams* p);

/* Quantize x [rows, cols] (x_dtype FP4_DT_F32 / FP4_DT_BF16, leading dimension ldx >= cols) into
 * codes / scales (and tensor_scale for NVFP4) as described by *p. Per block: rotate (if
 * hadamard_n), take amax = max |x| over the block, encode the scale, then each element
 * v = x * RN(1/d) (d the decoded scale; exactly x / d for power-of-two scales) is rounded to the
 * element grid. Requirements: cols even for E2M1; blocks tile the tensor; 1D groups and 2D tiles
 * need cols % 32 == 0 (and rows % 32 == 0 for 2D); per-row / per-tensor blocks take no rotation;
 * SR is not combined with 4/6; x and ldx * element size 16-byte aligned; codes 16-byte aligned;
 * a row pitch ldx != cols (and any 2D tiling) needs 64 * ldx * element size < 2^31 (32-bit
 * offsets within a wave's tile), else FP4_ERR_UNSUPPORTED.
 * workspace: device memory of fp4_workspace_bytes() bytes (may be NULL when that is 0). */
int fp4_quantize(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                 const fp4_qparams* p, void* codes, void* scales, float* tensor_scale,
                 void* workspace, int64_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid hipMalloc): fp4_quantize without a workspace argument. The scratch the
 * tensor-wide amax needs (NVFP4 and 4/6 without a given tensor scale, per-tensor blocks) is taken
 * from a static device array of the library, FP4_NOALLOC_SCRATCH_BYTES per GPU, held by each GPU
 * the library runs on until the process ends. This call allocates nothing (no hipMalloc, no
 * allocating library routine); its first call on a device looks up that device's copy of the array.
 * The word it uses is cleared by a kernel before each use. Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (e.g. on two streams) race on it and must be
 * serialised by the caller. Arguments, results and errors as for fp4_quantize; a mode whose
 * workspace exceeds the array returns FP4_ERR_WORKSPACE (none does today: fp4_workspace_bytes is at
 * most 256). */
#define FP4_NOALLOC_SCRATCH_BYTES 256
int fp4_quantize_noalloc(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                         const fp4_qparams* p, void* codes, void* scales, float* tensor_scale, void* stream);

/* One tensor of a batched quantize: x [rows, cols] with leading dimension ldx, its codes, scales
 * and tensor_scale (an input, the tensor scale g, in the _GIVEN NVFP4 modes; else unused). */
typedef struct {
    const void* x;
    int64_t rows, cols, ldx;
    void* codes;
    void* scales;
    float* tensor_scale;
} fp4_quant_item;

/* Batched quantization: the same result as fp4_quantize(items[i].x, x_dtype, ..., p, ...) for each
 * i, in one launch (one ramp and one tail instead of count, e.g. a layer's activations and weights
 * quantized with one recipe). 1 <= count <= 4; every item shares x_dtype and *p (SR keys each item
 * by its own element index, as separate calls with p->seed would). Modes that need a tensor-wide
 * amax first (NVFP4 and 4/6 without a given tensor scale, per-tensor blocks) and per-row blocks
 * return FP4_ERR_UNSUPPORTED; requirements and alignment per item as for fp4_quantize; no output
 * may alias any item's input or another output. No workspace. */
int fp4_quantize_batch(int32_t count, const fp4_quant_item* items, int32_t x_dtype, const fp4_qparams* p,
                       void* stream);

/* Column-wise quantization: quantize T = x^T without forming it. x is [rows, cols] (row pitch ldx);
 * the result is exactly fp4_quantize of the [cols, rows] tensor T with *p: codes, scales and the
 * rotation run along x's rows (T's contiguous axis), e.g. to feed dW = dY^T X, whose contraction
 * runs over the token axis (the backward pass of the Quartet notes' recipe; the transposition-
 * invariant blocks of "Stable FP4 Training via Transposition-Invariant Block Quantization" exist so
 * that a weight quantized once serves both orientations). Sizes and layouts are those of a cols x
 * rows tensor (fp4_codes_bytes(cols, rows, p), ...). Supported: 1D groups (block_rows == 1,
 * block_cols 16 or 32; rows % 32 == 0), every scale, rounding and Hadamard mode fp4_quantize
 * accepts for them; other blocks return FP4_ERR_UNSUPPORTED. Alignment as for fp4_quantize. */
int fp4_quantize_colwise(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                         const fp4_qparams* p, void* codes, void* scales, float* tensor_scale,
                         void* workspace, int64_t ws_bytes, void* stream);

/* y = RN(val(q) * d) for every element (d the decoded block scale: 2^k, the fp32 scale, or
 * RN(E4M3(s) * g) in the NVFP4 modes), then the rotation again when p->hadamard_n > 0 (H/sqrt(n)
 * is its own inverse). y: [rows, cols] fp32 or bf16 (round to nearest even), leading dim ldy. */
int fp4_dequantize(const void* codes, const void* scales, const float* tensor_scale, int64_t rows,
                   int64_t cols, const fp4_qparams* p, void* y, int32_t y_dtype, int64_t ldy,
                   void* stream);

/* The rotation alone: y [rows, cols] = x with each n-chunk of every row multiplied by H_n/sqrt(n),
 * fp32 out (the same arithmetic fp4_quantize applies before it quantizes). */
int fp4_hadamard(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                 int32_t hadamard_n, float* y, void* stream);

/* C [M, N] = A [M, K] * B [N, K]^T on the quantized operands, fp32 accumulation; C fp32 or bf16
 * (round to nearest even) with leading dimension ldc >= N (elements; C itself 16-byte aligned, else
 * FP4_ERR_ALIGNMENT; a pitch that is not a multiple of 16 bytes only narrows the stores), so C may
 * be a column block of a wider row-major buffer. Supported operand pairs:
 * MXFP4 x MXFP4 (E2M1, E8M0 (1, 32) groups; B may use (32, 32) 2D tiles), MXFP8 x MXFP8 (E4M3,
 * E8M0 (1, 32)), and NVFP4 x NVFP4 (E2M1, (1, 16) NV or 4/6 scales: each 32-wide K group is
 * re-expressed as E4M3 elements under one power-of-two scale and multiplied on the FP8 matrix
 * cores, and the product of the two tensor scales is applied in the epilogue).
 * K is a multiple of 32 (every operand layout requires it). Tiles: with K % 256 == 0 (MXFP4) or
 * K % 128 == 0 (MXFP8, NVFP4), 256 x 256 where M, N >= 256 and the grid fills more than half the
 * CUs, else 128 x 128 on the same kernel; any other K
 * runs on a 128 x 128 kernel whose last 128-deep step may lie partly past K (it reads nothing
 * there). Every tiling accumulates each output over K in the same order.
 * Operands must not be rotated differently: a rotation along K cancels in A B^T
 * only when both were rotated with the same n, which the caller ensures.
 * Optional fused output quantization ("online quantization" of the output in the QuTLASS kernel
 * list of the Quartet notes): if out_q is non-NULL, C_q->codes / C_q->scales (device, codes
 * 16-byte aligned) receive the fp32 result -- the value an fp32 C would hold -- quantized along N
 * exactly as fp4_quantize would quantize that fp32 C with *out_q: E2M1 or E4M3 elements, E8M0
 * floor or ceil scales, (1, 32) groups, RNE or SR (element (m, n) keyed by m * N + n), and, with
 * out_q->hadamard_n = n in {16, 32, 64, 128}, each n-chunk of a row of C rotated by H_n / sqrt(n)
 * before it is quantized (an output that feeds the next layer's rotated GEMM; C itself is stored
 * unrotated). Requires N % 32 == 0 and N % n == 0 (n = 256: FP4_ERR_UNSUPPORTED);
 * C_q->rows, cols, p are set to M, N, *out_q and tensor_scale to
 * NULL. C may then be NULL (only the quantized output is written); out_q and C_q are given
 * together or not at all. workspace: fp4_gemm_workspace_bytes() bytes; NVFP4 operands with
 * M, N >= 256 and K % 128 == 0 may instead pass NULL and 0 (the re-expression then happens in LDS,
 * inside the 256 x 256 tiles), other NVFP4 shapes return FP4_ERR_WORKSPACE without it. */
int64_t fp4_gemm_workspace_bytes(const fp4_qtensor* A, const fp4_qtensor* B);
int fp4_gemm(const fp4_qtensor* A, const fp4_qtensor* B, void* C, int32_t c_dtype, int64_t ldc,
             const fp4_qparams* out_q, fp4_qtensor* C_q, void* workspace, int64_t ws_bytes,
             void* stream);

/* The MXFP4 GEMM with A's rotation and quantization fused in ("fused rotation" before the 4-bit GEMM
 * in the QuTLASS kernel list of the Quartet notes): a [M, K] (fp32 or bf16, row pitch lda) is rotated
 * along K by H_n / sqrt(n) (n = pa->hadamard_n, which must equal B's) and quantized with *pa
 * (E2M1, (1, 32) E8M0 floor or ceil, nearest even or stochastic; n in {0, 16, 32, 64, 128}), and
 * C [M, N] = A_q B^T as fp4_gemm computes it (B: MXFP4, (1, 32) or (32, 32) blocks, K = B->cols).
 * A_q->codes / A_q->scales (device, as fp4_quantize writes them) receive A's codes and scales, the
 * same bytes fp4_quantize returns, and the product uses them; A_q->rows, cols, p, tensor_scale are
 * set to M, K, *pa, NULL. On the 256 x 256 tile path (M, N >= 256, K % 256 == 0) one persistent
 * launch first quantizes A with the whole grid (A once, not once per tile), then hands it over with
 * one grid-wide release / acquire and runs the tiles (the workgroups must all be resident: the
 * launch is cooperative, which fails with FP4_ERR_HIP when it cannot be); other shapes run the
 * quantize launch and then fp4_gemm. workspace: fp4_gemm_quantize_a_workspace_bytes(M, B) bytes
 * (256) of device memory: a counter and a status word, cleared by the call; the status word is
 * non-zero afterwards only if the hand-over wait gave up (never with every workgroup resident). Requirements and alignment as for
 * fp4_quantize (a, lda) and fp4_gemm (C, ldc); C is required. */
int64_t fp4_gemm_quantize_a_workspace_bytes(int64_t M, const fp4_qtensor* B);
int fp4_gemm_quantize_a(const void* a, int32_t a_dtype, int64_t M, int64_t lda, const fp4_qparams* pa,
                        fp4_qtensor* A_q, const fp4_qtensor* B, void* C, int32_t c_dtype, int64_t ldc,
                        void* workspace, int64_t ws_bytes, void* stream);

/* The quantized form of the transpose of a tensor quantized with 32 x 32 blocks ((32, 32) E8M0 tiles,
 * E2M1 or E4M3 elements, hadamard_n == 0): codes / scales of T [rows, cols] become out_codes /
 * out_scales of T^T [cols, rows], exactly what fp4_quantize with the same *p returns for T^T (one
 * scale per 32 x 32 tile makes each tile of T^T the same elements, amax and scale as a tile of T:
 * "Stable FP4 Training via Transposition-Invariant Block Quantization", abstract), so a weight
 * quantized once serves GEMMs that contract it along either axis. A pure re-layout (no arithmetic):
 * element (r, c) moves to (c, r) and scale (i, j) to (j, i). With a rotation the codes describe the
 * rotated tensor, whose transpose is rotated along the other axis, so hadamard_n != 0 returns
 * FP4_ERR_UNSUPPORTED. Layouts as everywhere: out_codes [cols, rows/2] (E2M1) or [cols, rows]
 * (E4M3), out_scales [cols/32, rows/32]; codes and out_codes 16-byte aligned (else
 * FP4_ERR_ALIGNMENT); outputs must not alias the inputs. */
int fp4_transpose_2d(const void* codes, const void* scales, int64_t rows, int64_t cols, const fp4_qparams* p,
                     void* out_codes, void* out_scales, void* stream);

/* The FP8 re-expression of an NVFP4 tensor, the operand form the GEMM multiplies NVFP4 x NVFP4 in
 * (the gfx950 scaled matrix instructions take one power-of-two scale per 32 K values): codes
 * (E2M1 [rows, cols/2]) and scales (E4M3 [rows, cols/16], the (1, 16) blocks of the NVFP4 modes of
 * "Four Over Six: More Accurate NVFP4 Quantization with Adaptive Block Scaling", methodology) become
 * out_codes (E4M3 [rows, cols]) and out_scales (E8M0 [rows, cols/32]): per 32-wide group, with S the
 * larger of its two block scales, E is the smallest exponent with 448 * 2^E >= 6 S (E = -127 when
 * S = 0, code E + 127) and each element is E4M3(val(q) * s_blk * 2^-E), nearest even (lossy: the
 * product of a 2-bit element and a 4-bit scale can need 6 significant bits). The fp32 tensor scale
 * is not involved (it multiplies the GEMM's result). Requirements: cols % 32 == 0; codes and
 * out_codes 16-byte aligned, scales 2-byte aligned; outputs must not alias the inputs. */
int fp4_nvfp4_to_mxfp8(const void* codes, const void* scales, int64_t rows, int64_t cols, void* out_codes,
                       void* out_scales, void* stream);

#ifdef __cplusplus
}
#endif
#endif
