/*
 * Plain, slow CPU oracle. TEST INFRASTRUCTURE ONLY: see oracle.h for who may load it, the sources
 * and the arithmetic conventions (fp32 round-to-nearest-even per operation, no contraction, no
 * flush of denormals; exact fp64 sums for the GEMM).
 *
 * Built with: gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off -fno-fast-math (oracle/build.py).
 */
#include "oracle.h"

#include <float.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

static int is_nv_mode(int m) {
    return m == ORC_SCALE_NV || m == ORC_SCALE_NV_4OVER6 || m == ORC_SCALE_NV_GIVEN ||
           m == ORC_SCALE_NV_4OVER6_GIVEN;
}
static int is_4over6_mode(int m) { return m == ORC_SCALE_NV_4OVER6 || m == ORC_SCALE_NV_4OVER6_GIVEN; }
static int is_given_mode(int m) { return m == ORC_SCALE_NV_GIVEN || m == ORC_SCALE_NV_4OVER6_GIVEN; }

/* ------------------------------------------------------------------------------------------------
 * Number formats
 * ----------------------------------------------------------------------------------------------*/

/* [LowBit] "FP4라는 무리수": E2M1 has 1 sign, 2 exponent and 1 mantissa bit and represents exactly
 * +-{0.5, 1, 1.5, 2, 3, 4, 6} and 0, in [-6, 6]. Codes: bit 3 is the sign, bits 0-2 index the
 * magnitudes below in increasing order. */
static const float E2M1_MAG[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

float orc_e2m1_value(uint8_t code) {
    float m = E2M1_MAG[code & 7];
    return (code & 8) ? -m : m;
}

/* Round to the nearest grid value, ties to the even code, saturating at 6 ([LowBit] §1 and §6 name
 * round-to-nearest; the range is [-6, 6]). The sign of v is kept, also on a zero result. The
 * distances are exact in double wherever a decision is close (|v| near a midpoint >= 0.25). */
uint8_t orc_e2m1_rne(float v) {
    uint8_t sign = signbit(v) ? 8 : 0;
    double a = fabs((double)v);
    if (!(a < 6.0)) return sign | 7;
    int best = 0;
    double bd = a;
    for (int i = 1; i < 8; ++i) {
        double d = fabs(a - (double)E2M1_MAG[i]);
        if (d < bd || (d == bd && (i & 1) == 0)) {
            best = i;
            bd = d;
        }
    }
    return (uint8_t)(sign | best);
}

/* Stochastic rounding ([Quartet] QuTLASS kernels; [TIBQ] abstract): between the grid neighbours
 * lo <= |v| < hi, round up with probability p = (|v| - lo) / (hi - lo). With a 16-bit uniform u
 * the rule is "up iff u < p * 2^16"; p and p * 2^16 are exact (|v| - lo is exact and the gap is a
 * power of two). |v| >= 6 saturates. */
uint8_t orc_e2m1_sr(float v, uint32_t u16) {
    uint8_t sign = signbit(v) ? 8 : 0;
    float a = fabsf(v);
    if (!(a < 6.0f)) return sign | 7;
    int lo = 0;
    while (lo < 6 && E2M1_MAG[lo + 1] <= a) ++lo;
    float p = (a - E2M1_MAG[lo]) / (E2M1_MAG[lo + 1] - E2M1_MAG[lo]);
    int up = (float)u16 < p * 65536.0f;
    return (uint8_t)(sign | (lo + up));
}

/* OCP E4M3FN: bias 7, subnormal step 2^-9, largest finite 448 (code 0x7E), 0x7F is NaN. */
float orc_e4m3_value(uint8_t code) {
    int e = (code >> 3) & 15, m = code & 7;
    float v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexpf((float)m, -9);
    else
        v = ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return (code & 0x80) ? -v : v;
}

/* largest magnitude code c in [0, 126] with value(c) <= a, for 0 <= a < 448 */
static int e4m3_floor_code(float a) {
    int lo = 0, hi = 126;
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (orc_e4m3_value((uint8_t)mid) <= a)
            lo = mid;
        else
            hi = mid;
    }
    return lo;
}

/* Nearest E4M3 value, ties to the even code, saturating at 448 (the MXFP8 elements of [TIBQ]). */
uint8_t orc_e4m3_rne(float v) {
    uint8_t sign = signbit(v) ? 0x80 : 0;
    float a = fabsf(v);
    if (!(a < 448.0f)) return sign | 0x7E;
    int lo = e4m3_floor_code(a);
    double dlo = (double)a - orc_e4m3_value((uint8_t)lo);
    double dhi = (double)orc_e4m3_value((uint8_t)(lo + 1)) - (double)a;
    int c = dlo < dhi ? lo : (dhi < dlo ? lo + 1 : ((lo & 1) ? lo + 1 : lo));
    return (uint8_t)(sign | c);
}

uint8_t orc_e4m3_sr(float v, uint32_t u16) {
    uint8_t sign = signbit(v) ? 0x80 : 0;
    float a = fabsf(v);
    if (!(a < 448.0f)) return sign | 0x7E;
    int lo = e4m3_floor_code(a);
    float glo = orc_e4m3_value((uint8_t)lo), ghi = orc_e4m3_value((uint8_t)(lo + 1));
    float p = (a - glo) / (ghi - glo);
    int up = (float)u16 < p * 65536.0f;
    return (uint8_t)(sign | (lo + up));
}

/* [LowBit] §3: the MXFP4 group scale is an 8-bit exponent, 2^k only. Code = k + 127. */
float orc_e8m0_value(uint8_t code) {
    if (code == 255) return NAN;
    return ldexpf(1.0f, (int)code - 127);
}

uint16_t orc_bf16_rne(float v) {
    uint32_t u;
    memcpy(&u, &v, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------------------------------------
 * Random bits: Philox4x32-10 [Philox]. Each round multiplies words 0 and 2 by the two round
 * constants (full 64-bit products), and the new state is (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2),
 * hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)). The key is advanced by the Weyl constants before every round
 * after the first.
 * ----------------------------------------------------------------------------------------------*/
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c0 = n0;
        c1 = n1;
        c2 = n2;
        c3 = n3;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

/* The uniform for element idx (row-major index in the logical tensor): one Philox call serves 8
 * consecutive elements. Counter = (idx / 8 as a 64-bit number, 0, 0), key = the 64-bit seed; word
 * (idx / 2) % 4 is split into a low half (even idx) and a high half (odd idx). */
uint32_t orc_sr_u16(uint64_t seed, uint64_t idx) {
    uint64_t g = idx >> 3;
    uint32_t ctr[4] = {(uint32_t)g, (uint32_t)(g >> 32), 0u, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    orc_philox4x32_10(ctr, key, out);
    uint32_t w = out[(idx >> 1) & 3];
    return (idx & 1) ? (w >> 16) : (w & 0xFFFFu);
}

/* ------------------------------------------------------------------------------------------------
 * Rotation: [LowBit] §7 and [Quartet] "Hadamard rotation": multiply by the orthogonal matrix
 * H_n / sqrt(n) (H_n has +-1 entries), computed in O(n log n). Sylvester (natural) order: stage
 * h = 1, 2, 4, ..., n/2 replaces every pair (x[i], x[i+h]) with i & h == 0 by (x[i] + x[i+h],
 * x[i] - x[i+h]); afterwards every entry is multiplied by c_n = RN(1/sqrt(n)). Blockwise: the
 * transform acts on each contiguous n-chunk.
 * ----------------------------------------------------------------------------------------------*/
static float inv_sqrt_rn(int n) { return (float)(1.0L / sqrtl((long double)n)); }

static int is_pow2(int64_t n) { return n > 0 && (n & (n - 1)) == 0; }

int orc_fwht(float* x, int64_t len, int n) {
    if (!is_pow2(n) || n < 2 || n > 4096 || len % n) return -1;
    float c = inv_sqrt_rn(n);
    for (int64_t base = 0; base < len; base += n) {
        float* v = x + base;
        for (int h = 1; h < n; h <<= 1)
            for (int i = 0; i < n; ++i)
                if (!(i & h)) {
                    float a = v[i], b = v[i + h];
                    v[i] = a + b;
                    v[i + h] = a - b;
                }
        for (int i = 0; i < n; ++i) v[i] = v[i] * c;
    }
    return 0;
}

/* ------------------------------------------------------------------------------------------------
 * Scales
 * ----------------------------------------------------------------------------------------------*/
static float elem_maxval(int elem) { return elem == ORC_ELEM_E2M1 ? 6.0f : 448.0f; }
static int elem_emax(int elem) { return elem == ORC_ELEM_E2M1 ? 2 : 8; }

/* [LowBit] §3 (power-of-two scales). Floor rule: k = floor(log2 amax) - emax, where emax is the
 * exponent of the element format's largest value (6 = 1.5 * 2^2, 448 = 1.75 * 2^8). Ceil rule
 * ([TIBQ] truncation-free scaling): the smallest k with maxval * 2^k >= amax. k is clamped to
 * [-127, 127]; amax = 0 gives -127. */
int orc_e8m0_scale_exp(float amax, int elem, int rule) {
    if (!(amax > 0.0f)) return -127;
    int ex;
    frexp((double)amax, &ex); /* amax = m * 2^ex, m in [0.5, 1) */
    int k;
    if (rule == ORC_SCALE_E8M0_FLOOR) {
        k = (ex - 1) - elem_emax(elem);
    } else {
        k = (ex - 1) - elem_emax(elem) - 1;
        while (ldexp((double)elem_maxval(elem), k) < (double)amax) ++k;
    }
    if (k < -127) k = -127;
    if (k > 127) k = 127;
    return k;
}

/* reciprocal of a scale, with 0 -> 0 and an overflowing reciprocal clamped to FLT_MAX */
static float recip(float d) {
    if (d == 0.0f) return 0.0f;
    float r = 1.0f / d;
    if (isinf(r)) r = FLT_MAX;
    return r;
}

/* Fixed-order fp32 sum of a power-of-two number of terms: ((t0+t1)+(t2+t3))+... */
static float tree_sum(float* t, int n) {
    for (int w = n; w > 1; w >>= 1)
        for (int i = 0; i < w / 2; ++i) t[i] = t[2 * i] + t[2 * i + 1];
    return t[0];
}

/* ------------------------------------------------------------------------------------------------
 * Quantize
 * ----------------------------------------------------------------------------------------------*/
static int check_layout(int64_t rows, int64_t cols, int elem, int br, int bc, int scale_mode,
                        int round_mode, int hadamard_n) {
    if (rows <= 0 || cols <= 0 || br <= 0 || bc <= 0) return -1;
    if (rows % br || cols % bc) return -2;
    if (elem != ORC_ELEM_E2M1 && elem != ORC_ELEM_E4M3) return -3;
    if (elem == ORC_ELEM_E2M1 && (cols & 1)) return -4;
    if (scale_mode < 0 || scale_mode > 6) return -5;
    if (round_mode != ORC_ROUND_RNE && round_mode != ORC_ROUND_SR) return -6;
    if (hadamard_n && (!is_pow2(hadamard_n) || hadamard_n < 2 || cols % hadamard_n)) return -7;
    if (is_nv_mode(scale_mode)) {
        if (elem != ORC_ELEM_E2M1 || br != 1 || !is_pow2(bc) || bc > 64) return -8;
        if (is_4over6_mode(scale_mode) && round_mode == ORC_ROUND_SR) return -9;
    }
    return 0;
}

static float* to_f32(const void* x, int x_dtype, int64_t n) {
    float* f = (float*)malloc((size_t)n * sizeof(float));
    if (!f) return NULL;
    if (x_dtype == ORC_IN_BF16) {
        const uint16_t* h = (const uint16_t*)x;
        for (int64_t i = 0; i < n; ++i) {
            uint32_t u = (uint32_t)h[i] << 16;
            memcpy(&f[i], &u, 4);
        }
    } else {
        memcpy(f, x, (size_t)n * sizeof(float));
    }
    return f;
}

static void put_code(uint8_t* codes, int elem, int64_t cols, int64_t r, int64_t c, uint8_t q) {
    if (elem == ORC_ELEM_E4M3) {
        codes[r * cols + c] = q;
    } else {
        uint8_t* b = &codes[r * (cols / 2) + c / 2];
        if (c & 1)
            *b = (uint8_t)((*b & 0x0F) | (q << 4));
        else
            *b = (uint8_t)((*b & 0xF0) | (q & 0x0F));
    }
}

static uint8_t get_code(const uint8_t* codes, int elem, int64_t cols, int64_t r, int64_t c) {
    if (elem == ORC_ELEM_E4M3) return codes[r * cols + c];
    uint8_t b = codes[r * (cols / 2) + c / 2];
    return (c & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 0x0F);
}

static uint8_t encode_elem(float v, int elem, int round_mode, uint64_t seed, uint64_t idx) {
    if (round_mode == ORC_ROUND_SR) {
        uint32_t u = orc_sr_u16(seed, idx);
        return elem == ORC_ELEM_E2M1 ? orc_e2m1_sr(v, u) : orc_e4m3_sr(v, u);
    }
    return elem == ORC_ELEM_E2M1 ? orc_e2m1_rne(v) : orc_e4m3_rne(v);
}

static float elem_value(uint8_t q, int elem) {
    return elem == ORC_ELEM_E2M1 ? orc_e2m1_value(q) : orc_e4m3_value(q);
}

/* NVFP4 block-scale candidate for target maximum M: t = amax_b / RN(M g), s = E4M3(t) (RNE,
 * saturating), d = RN(val(s) g). */
static uint8_t nv_candidate(float amax_b, float g, float M, float* d) {
    float t = amax_b / (M * g);
    uint8_t s = orc_e4m3_rne(t);
    *d = orc_e4m3_value(s) * g;
    return s;
}

/* block SSE of encoding xs[0..n) with scale d (RNE), summed in the fixed tree order */
static float block_sse(const float* xs, int n, float d) {
    float r = recip(d);
    float t[64];
    for (int i = 0; i < n; ++i) {
        uint8_t q = orc_e2m1_rne(xs[i] * r);
        float deq = orc_e2m1_value(q) * d;
        float err = xs[i] - deq;
        t[i] = err * err;
    }
    return tree_sum(t, n);
}

int orc_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int elem,
                 int block_rows, int block_cols, int scale_mode, int round_mode, int hadamard_n,
                 uint64_t seed, uint8_t* codes, void* scales, float* tensor_scale) {
    int rc = check_layout(rows, cols, elem, block_rows, block_cols, scale_mode, round_mode,
                          hadamard_n);
    if (rc) return rc;
    int64_t n = rows * cols;
    float* xf = to_f32(x, x_dtype, n);
    if (!xf) return -100;
    if (hadamard_n) orc_fwht(xf, n, hadamard_n);

    const int nv = is_nv_mode(scale_mode);
    float g = 1.0f;
    if (is_given_mode(scale_mode)) {
        /* delayed scaling: the caller's g; blocks whose amax exceeds 6 * 448 * g get the largest
         * block scale and their elements saturate */
        if (!tensor_scale) {
            free(xf);
            return -10;
        }
        g = *tensor_scale;
    } else if (nv) {
        /* fp32 tensor scale g = amax_t / (6 * 448), so that the block scales use the E4M3 range */
        float amax_t = 0.0f;
        for (int64_t i = 0; i < n; ++i) amax_t = fmaxf(amax_t, fabsf(xf[i]));
        g = amax_t > 0.0f ? amax_t / 2688.0f : 1.0f;
        if (tensor_scale) *tensor_scale = g;
    }

    const int64_t nbr = rows / block_rows, nbc = cols / block_cols;
    const float maxval = elem_maxval(elem);
    float xs[64];
    for (int64_t I = 0; I < nbr; ++I)
        for (int64_t J = 0; J < nbc; ++J) {
            /* group amax over the block */
            float amax = 0.0f;
            for (int64_t r = I * block_rows; r < (I + 1) * block_rows; ++r)
                for (int64_t c = J * block_cols; c < (J + 1) * block_cols; ++c)
                    amax = fmaxf(amax, fabsf(xf[r * cols + c]));
            /* scale */
            float d;
            int64_t sidx = I * nbc + J;
            if (scale_mode == ORC_SCALE_E8M0_FLOOR || scale_mode == ORC_SCALE_E8M0_CEIL) {
                int k = orc_e8m0_scale_exp(amax, elem, scale_mode);
                ((uint8_t*)scales)[sidx] = (uint8_t)(k + 127);
                d = ldexpf(1.0f, k);
            } else if (scale_mode == ORC_SCALE_F32) {
                d = amax / maxval;
                ((float*)scales)[sidx] = d;
            } else {
                float d6;
                uint8_t s6 = nv_candidate(amax, g, 6.0f, &d6);
                uint8_t s = s6;
                d = d6;
                if (is_4over6_mode(scale_mode)) {
                    /* [4over6] methodology: a second candidate maps the block max to 4 instead of
                     * 6; keep the one with the lower block error (strictly lower, else 6). */
                    float d4;
                    uint8_t s4 = nv_candidate(amax, g, 4.0f, &d4);
                    const float* row = xf + I * cols + J * block_cols;
                    memcpy(xs, row, (size_t)block_cols * sizeof(float));
                    float sse6 = block_sse(xs, block_cols, d6);
                    float sse4 = block_sse(xs, block_cols, d4);
                    if (sse4 < sse6) {
                        s = s4;
                        d = d4;
                    }
                }
                ((uint8_t*)scales)[sidx] = s;
            }
            /* elements: v = RN(x * RN(1/d)) (for power-of-two d this is x / d exactly) */
            float rcp = recip(d);
            for (int64_t r = I * block_rows; r < (I + 1) * block_rows; ++r)
                for (int64_t c = J * block_cols; c < (J + 1) * block_cols; ++c) {
                    float v = xf[r * cols + c] * rcp;
                    uint8_t q = encode_elem(v, elem, round_mode, seed, (uint64_t)(r * cols + c));
                    put_code(codes, elem, cols, r, c, q);
                }
        }
    free(xf);
    return 0;
}

/* decoded scale of block (I, J) */
static float block_scale(const void* scales, const float* tensor_scale, int scale_mode,
                         int64_t sidx) {
    if (scale_mode == ORC_SCALE_E8M0_FLOOR || scale_mode == ORC_SCALE_E8M0_CEIL)
        return orc_e8m0_value(((const uint8_t*)scales)[sidx]);
    if (scale_mode == ORC_SCALE_F32) return ((const float*)scales)[sidx];
    float g = tensor_scale ? *tensor_scale : 1.0f;
    return orc_e4m3_value(((const uint8_t*)scales)[sidx]) * g;
}

int orc_dequantize(const uint8_t* codes, const void* scales, const float* tensor_scale,
                   int64_t rows, int64_t cols, int elem, int block_rows, int block_cols,
                   int scale_mode, int hadamard_n, float* y) {
    int rc = check_layout(rows, cols, elem, block_rows, block_cols, scale_mode, ORC_ROUND_RNE,
                          hadamard_n);
    if (rc) return rc;
    const int64_t nbc = cols / block_cols;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            int64_t sidx = (r / block_rows) * nbc + c / block_cols;
            float d = block_scale(scales, tensor_scale, scale_mode, sidx);
            y[r * cols + c] = elem_value(get_code(codes, elem, cols, r, c), elem) * d;
        }
    if (hadamard_n) orc_fwht(y, rows * cols, hadamard_n);
    return 0;
}

/* ------------------------------------------------------------------------------------------------
 * GEMM operands and the fp64 reference product
 * ----------------------------------------------------------------------------------------------*/
int orc_operand_f64(const uint8_t* codes, const void* scales, const float* tensor_scale,
                    int64_t rows, int64_t K, int elem, int block_rows, int block_cols,
                    int scale_mode, int with_nv_exact, double* out) {
    int rc = check_layout(rows, K, elem, block_rows, block_cols, scale_mode, ORC_ROUND_RNE, 0);
    if (rc) return rc;
    const int64_t nbc = K / block_cols;
    const int nv = is_nv_mode(scale_mode);
    if (!nv || with_nv_exact) {
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t k = 0; k < K; ++k) {
                int64_t sidx = (r / block_rows) * nbc + k / block_cols;
                double q = (double)elem_value(get_code(codes, elem, K, r, k), elem);
                double d;
                if (nv) {
                    d = (double)orc_e4m3_value(((const uint8_t*)scales)[sidx]) *
                        (double)(tensor_scale ? *tensor_scale : 1.0f);
                } else {
                    d = (double)block_scale(scales, tensor_scale, scale_mode, sidx);
                }
                out[r * K + k] = q * d;
            }
        return 0;
    }
    /* NVFP4 on a matrix core that takes one power-of-two scale per 32 K values: the operand is
     * first re-expressed as E4M3 elements with one E8M0 exponent per 32-wide K group
     * (orc_nv_to_mx8); the value the product sees is val(f) * 2^E * g. */
    if (K % 32 || 32 % block_cols) return -10;
    uint8_t* f8 = (uint8_t*)malloc((size_t)(rows * K));
    uint8_t* e8 = (uint8_t*)malloc((size_t)(rows * (K / 32)));
    if (!f8 || !e8) {
        free(f8);
        free(e8);
        return -100;
    }
    rc = orc_nv_to_mx8(codes, scales, rows, K, block_cols, f8, e8);
    if (rc) {
        free(f8);
        free(e8);
        return rc;
    }
    const double g = (double)(tensor_scale ? *tensor_scale : 1.0f);
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < K; ++k) {
            int E = (int)e8[r * (K / 32) + k / 32] - 127;
            out[r * K + k] = (double)orc_e4m3_value(f8[r * K + k]) * ldexp(1.0, E) * g;
        }
    free(f8);
    free(e8);
    return 0;
}

/* The re-expression of an NVFP4 operand (E2M1 codes with one E4M3 scale per block_cols-wide block,
 * block_cols dividing 32) as E4M3 elements with one power-of-two (E8M0) scale per 32-wide K group,
 * the operand form of a matrix core that takes only power-of-two block scales. Per group: S = the
 * largest of its E4M3 block scales; E = the smallest exponent with 448 * 2^E >= 6 S, so that every
 * |val(q) * s_blk| <= 6 S fits below 448 * 2^E (E = -127 when S = 0); each element becomes
 * f = E4M3(val(q) * s_blk * 2^-E), nearest even. val(q) * s_blk is exact in fp32 (2 and 4
 * significant bits) and so is the scaling by 2^-E; the E4M3 rounding is the one lossy step. The
 * tensor scale g is not part of it (it multiplies the whole product). Out: E4M3 codes [rows, K],
 * E8M0 codes E + 127 [rows, K / 32]. */
int orc_nv_to_mx8(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t K,
                  int block_cols, uint8_t* out_codes, uint8_t* out_scales) {
    if (rows <= 0 || K <= 0 || K % 32 || block_cols <= 0 || 32 % block_cols) return -10;
    const int64_t nbc = K / block_cols;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k0 = 0; k0 < K; k0 += 32) {
            float S = 0.0f;
            for (int64_t k = k0; k < k0 + 32; k += block_cols)
                S = fmaxf(S, orc_e4m3_value(scales[r * nbc + k / block_cols]));
            int E = -127;
            if (S > 0.0f) {
                E = -40;
                while (ldexp(448.0, E) < 6.0 * (double)S) ++E;
            }
            out_scales[r * (K / 32) + k0 / 32] = (uint8_t)(E + 127);
            for (int64_t k = k0; k < k0 + 32; ++k) {
                float s_blk = orc_e4m3_value(scales[r * nbc + k / block_cols]);
                float t = orc_e2m1_value(get_code(codes, ORC_ELEM_E2M1, K, r, k)) * s_blk;
                t = ldexpf(t, -E);
                out_codes[r * K + k] = orc_e4m3_rne(t);
            }
        }
    return 0;
}

void orc_gemm_f64(const double* a, const double* b, int64_t M, int64_t N, int64_t K, double* c,
                  double* sabs) {
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0, t = 0.0;
            const double* ar = a + m * K;
            const double* br = b + n * K;
            for (int64_t k = 0; k < K; ++k) {
                double p = ar[k] * br[k];
                s += p;
                t += fabs(p);
            }
            c[m * N + n] = s;
            if (sabs) sabs[m * N + n] = t;
        }
}

void orc_gemm_f64_sampled(const double* a, const double* b, int64_t K, const int64_t* ms,
                          const int64_t* ns, int64_t count, double* c, double* sabs) {
    for (int64_t i = 0; i < count; ++i) {
        const double* ar = a + ms[i] * K;
        const double* br = b + ns[i] * K;
        double s = 0.0, t = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double p = ar[k] * br[k];
            s += p;
            t += fabs(p);
        }
        c[i] = s;
        if (sabs) sabs[i] = t;
    }
}

/* ------------------------------------------------------------------------------------------------
 * Array helpers for the Python wrapper (one element at a time, same functions as above)
 * ----------------------------------------------------------------------------------------------*/
void orc_encode_array(const float* v, int64_t n, int elem, int round_mode, uint64_t seed,
                      uint64_t idx0, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i)
        out[i] = encode_elem(v[i], elem, round_mode, seed, idx0 + (uint64_t)i);
}

void orc_decode_array(const uint8_t* q, int64_t n, int elem, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = elem_value(q[i], elem);
}

void orc_sr_u16_array(uint64_t seed, const uint64_t* idx, int64_t n, uint32_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_sr_u16(seed, idx[i]);
}

void orc_philox_array(const uint32_t* ctr, const uint32_t* key, int64_t n, uint32_t* out) {
    for (int64_t i = 0; i < n; ++i) orc_philox4x32_10(ctr + 4 * i, key + 2 * i, out + 4 * i);
}

void orc_bf16_array(const float* v, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_rne(v[i]);
}

void orc_sr_with_u_array(const float* v, const uint32_t* u16, int64_t n, int elem, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i)
        out[i] = elem == ORC_ELEM_E2M1 ? orc_e2m1_sr(v[i], u16[i]) : orc_e4m3_sr(v[i], u16[i]);
}
