// Device-side building blocks for gfx950 (CDNA4): bf16 unpacking, lane exchange, the
// hardware scaled converts to FP4 / FP8, Philox4x32-10, and the scale rules.
//
// Everything here is computed in fp32 with IEEE round-to-nearest-even per operation; the library
// is compiled with -ffp-contract=off so that no multiply-add is fused unless written as fmaf.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bgf {

typedef short v2s __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------------------------
// bf16 <-> fp32 (bf16 is the top half of an fp32: widening is exact)
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 values to packed bf16 (a in the low half), round to nearest even, with the hardware
// convert (v_cvt_pk_bf16_f32). Every bf16 output of the library (GEMM epilogues, dequantize) goes
// through it; a GPU test sweeps it over every fp32 bit pattern.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float a, float b) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// ---------------------------------------------------------------------------------------------
// Lane exchange through the LDS crossbar (ds_swizzle, bit mode: lane l of each 32-lane half reads
// lane ((l & and) | or) ^ xor of the same half; no LDS memory is touched). It runs on the LDS
// pipeline rather than as a VALU instruction: measured on the rotate + quantize, the butterfly
// stages across lanes cost 2.7 us (H_128) and 4.3 us (H_256) less over the Llama-7B X and W than
// with DPP moves, which take a VALU slot each (two for l ^ 4), next to the butterfly's own.
// ---------------------------------------------------------------------------------------------
// value of lane (lane ^ M), M in {1, 2, 4, 8, 16}
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
    static_assert(M >= 1 && M <= 16 && (M & (M - 1)) == 0, "xor within a 32-lane half");
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (M << 10) | 0x1F));
}

// 1 / sqrt(n) rounded to the nearest fp32, for the Hadamard normalisation
template <int N>
__device__ __forceinline__ float inv_sqrt_n() {
    if constexpr (N == 16) return __uint_as_float(0x3E800000u);   // 0.25
    if constexpr (N == 32) return __uint_as_float(0x3E3504F3u);   // 0.17677669...
    if constexpr (N == 64) return __uint_as_float(0x3E000000u);   // 0.125
    if constexpr (N == 128) return __uint_as_float(0x3DB504F3u);  // 0.08838834...
    if constexpr (N == 256) return __uint_as_float(0x3D800000u);  // 0.0625
    return 1.0f;
}

// ---------------------------------------------------------------------------------------------
// Hardware converts. The scale operand of the gfx950 scaled converts only contributes its
// exponent: the result is the conversion of x / 2^floor(log2 scale), computed exactly, rounded to
// nearest even. FP4 saturates at +-6; FP8 (E4M3) does not saturate, so callers clamp first.
// ---------------------------------------------------------------------------------------------
// two fp32 -> two E2M1 nibbles placed in byte SEL of `old`
template <int SEL>
__device__ __forceinline__ uint32_t cvt_fp4x2(uint32_t old, float a, float b, float scale) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, scale, SEL);
}
// two fp32 -> two E4M3 bytes in the low (HI = false) or high half of `old`
template <bool HI>
__device__ __forceinline__ uint32_t cvt_fp8x2(uint32_t old, float a, float b, float scale) {
    v2s o;
    o[0] = (short)(old & 0xFFFF);
    o[1] = (short)(old >> 16);
    v2s r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, a, b, scale, HI);
    return ((uint32_t)(uint16_t)r[0]) | ((uint32_t)(uint16_t)r[1] << 16);
}
// decode: byte SEL of `src` (two E2M1 nibbles) -> two fp32, exact
template <int SEL>
__device__ __forceinline__ v2f fp4x2_to_f32(uint32_t src) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(src, 1.0f, SEL);
}
// decode: half HI of `src` (two E4M3 bytes) -> two fp32, exact
template <bool HI>
__device__ __forceinline__ v2f fp8x2_to_f32(uint32_t src) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(src, 1.0f, HI);
}

// E4M3 code of t >= 0, nearest even, saturating at 448 (code 0x7E); NaN -> 0x7E
__device__ __forceinline__ uint32_t e4m3_code_sat(float t) {
    if (!(t < 448.0f)) return 0x7Eu;
    return cvt_fp8x2<false>(0u, t, 0.0f, 1.0f) & 0xFFu;
}
// value of a non-negative E4M3 code (0..0x7E)
__device__ __forceinline__ float e4m3_value(uint32_t c) {
    uint32_t e = (c >> 3) & 15u, m = c & 7u;
    if (e == 0) return (float)m * 0.001953125f;  // m * 2^-9, exact
    return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// ---------------------------------------------------------------------------------------------
// Scale rules
// ---------------------------------------------------------------------------------------------
// E8M0 exponent k for a block max: floor rule k = floor(log2 amax) - EMAX; ceil (truncation-free)
// rule: the smallest k with maxval * 2^k >= amax, i.e. one more than the floor rule when the
// mantissa of amax exceeds that of maxval (1.5 for E2M1, 1.75 for E4M3). Clamped to [-127, 127];
// amax = 0 gives -127.
template <int EMAX, uint32_t MAXMANT>
__device__ __forceinline__ int e8m0_exp(float amax, bool ceil_rule) {
    uint32_t u = __float_as_uint(amax);
    if (u == 0u) return -127;
    int e;
    uint32_t mant;
    uint32_t ef = u >> 23;
    if (ef != 0u) {
        e = (int)ef - 127;
        mant = u & 0x7FFFFFu;
    } else {  // subnormal amax
        int p = 31 - __clz(u);
        e = p - 149;
        mant = (u << (23 - p)) & 0x7FFFFFu;
    }
    int k = e - EMAX + ((ceil_rule && mant > MAXMANT) ? 1 : 0);
    return k < -127 ? -127 : (k > 127 ? 127 : k);
}

// 2^k as an fp32 for k in [-126, 127]
__device__ __forceinline__ float pow2f(int k) { return __uint_as_float((uint32_t)(k + 127) << 23); }

// reciprocal of a scale: 0 -> 0, an overflowing reciprocal -> FLT_MAX
__device__ __forceinline__ float scale_recip(float d) {
    if (d == 0.0f) return 0.0f;
    float r = 1.0f / d;
    return (__float_as_uint(r) & 0x7FFFFFFFu) == 0x7F800000u ? 3.40282347e38f : r;
}

// ---------------------------------------------------------------------------------------------
// Philox4x32-10 (Salmon et al., SC'11): 10 rounds of two 32x32->64 multiplies and a key schedule
// advanced by the Weyl constants.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ void philox4x32_10(uint32_t& c0, uint32_t& c1, uint32_t& c2,
                                              uint32_t& c3, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        // three-input xors (0x96 is the truth table of a ^ b ^ c)
        const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
        const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
}

// ---------------------------------------------------------------------------------------------
// Stochastic rounding: between the grid neighbours lo <= |v| < hi, round up iff u < p * 2^16,
// p = (|v| - lo) / (hi - lo) (exact: the gap is a power of two). Saturates at the grid maximum.
// Returns the code (sign bit 3 for E2M1, bit 7 for E4M3).
// ---------------------------------------------------------------------------------------------
// Both are branch-free and select-free: |v| is clamped to the grid maximum (which then rounds to
// the top code and never up), scaled by the grid spacing of its binade (a power of two, exact) to a
// position q in grid steps, and lo's code follows from floor(q) and the binade's exponent field;
// data-dependent branches per range would diverge within a wave on any real tensor.
__device__ __forceinline__ uint32_t e2m1_sr(float v, uint32_t u16) {
    // |v| clamped to 6 (a NaN clamps to 6 as well): the steps below then give code 7 and never
    // round up, so saturation needs no select
    const float a = fminf(fabsf(v), 6.0f);
    const uint32_t ua = __float_as_uint(a);
    // grid spacing 2^(e-1): e = 0 on [0, 2) (0, 0.5, 1, 1.5), 1 on [2, 4) (2, 3), 2 from 4 (4, 6);
    // ue = the exponent field clamped to [127, 129] (e + 127)
    const uint32_t ue = min(max(ua & 0x7F800000u, 0x3F800000u), 0x40800000u);
    const float q = a * __uint_as_float(0x7F800000u - ue);  // |v| / 2^(e-1): position in grid steps, exact
    const float fl = floorf(q);                             // lo's position (exact)
    // up iff u16 < (q - fl) 2^16, i.e. fl + u16 2^-16 < q (both sides exact)
    const uint32_t up = __builtin_fmaf((float)u16, 0x1p-16f, fl) < q ? 1u : 0u;
    // codes: position fl on [0, 2) is code fl; on [2, 4) and [4, 6] code fl + 2 e
    const uint32_t code = (uint32_t)(int)fl + (ue >> 22) - 254u + up;
    return ((__float_as_uint(v) >> 28) & 8u) | code;
}

__device__ __forceinline__ uint32_t e4m3_sr(float v, uint32_t u16) {
    // |v| clamped to 448 (a NaN clamps to 448 as well): code 0x7E, never rounded up
    const float a = fminf(fabsf(v), 448.0f);
    const uint32_t ua = __float_as_uint(a);
    // grid spacing 2^(e-3) with e = max(exponent, -6) (subnormals share 2^-6's spacing 2^-9);
    // ue = that exponent's field
    const uint32_t ue = max(ua & 0x7F800000u, 0x3C800000u);
    const float q = a * __uint_as_float(0x80800000u - ue);  // |v| / 2^(e-3): position in grid steps, exact
    const float fl = floorf(q);                             // lo's position (exact)
    // up iff u16 < (q - fl) 2^16, i.e. fl + u16 2^-16 < q (both sides exact)
    const uint32_t up = __builtin_fmaf((float)u16, 0x1p-16f, fl) < q ? 1u : 0u;
    // code 8 (e + 6) + fl: fl in [8, 16) for normals, [0, 8) below 2^-6
    const uint32_t code = (uint32_t)(int)fl + (ue >> 20) - 968u + up;
    return ((__float_as_uint(v) >> 24) & 0x80u) | code;
}

}  // namespace bgf
