// Per-block quantization steps shared by the quantize kernels and the GEMM's fused output
// quantization: block amax, Philox words for stochastic rounding, and the element encode under a
// power-of-two (E8M0) or general scale. A block is B consecutive values of a lane's 32-element
// segment v, starting at OFF.
#pragma once
#include "device.h"
#include "fp4_internal.h"

namespace bgf {

template <int B, int OFF>
__device__ __forceinline__ float block_amax(const float (&v)[32]) {
    float m = 0.0f;
#pragma unroll
    for (int i = OFF; i < OFF + B; ++i) m = fmaxf(m, fabsf(v[i]));
    return m;
}

// Random source of stochastic rounding for the segment of elements idx0 .. idx0 + 31 (idx0 a
// multiple of 32): u16 for element idx is the low (even idx) / high (odd idx) half of word
// (idx >> 1) & 3 of the Philox4x32-10 call for counter idx >> 3 and key seed. The words are
// generated where they are used, one call per 8 elements, so that only four are live at a time.
struct SrSource {
    uint64_t seed, idx0;
};

// the four words of group g8 (elements 8 g8 .. 8 g8 + 7 of the segment)
__device__ __forceinline__ void philox_group(const SrSource& sr, int g8, uint32_t (&c)[4]) {
    const uint64_t ctr = (sr.idx0 >> 3) + (uint64_t)g8;
    c[0] = (uint32_t)ctr;
    c[1] = (uint32_t)(ctr >> 32);
    c[2] = 0u;
    c[3] = 0u;
    philox4x32_10(c[0], c[1], c[2], c[3], (uint32_t)sr.seed, (uint32_t)(sr.seed >> 32));
}
// u16 of element e (0..7) of a group
__device__ __forceinline__ uint32_t sr_u16(const uint32_t (&c)[4], int e) {
    const uint32_t word = c[e >> 1];
    return (e & 1) ? (word >> 16) : (word & 0xFFFFu);
}

// Blockwise H_n / sqrt(n) along a row for n in {0, 16, 32, 64, 128} chosen at run time (the same
// for every lane of the wave; every lane must take part): a lane holds 32 consecutive values of
// the row, and for n >= 64 the groups of 32 that make up a chunk sit in consecutive lanes (group g
// of a 128-chunk in lane 4 k + g). Stages h = 1, 2, ..., n / 2 in that order -- h < 32 in
// registers, h = 32 and 64 with lanes l ^ 1 and l ^ 2 -- then one multiply by RN(1/sqrt(n)).
__device__ __forceinline__ void fwht_groups(float (&v)[32], int n) {
    if (n == 0) return;
#pragma unroll
    for (int h = 1; h < 32; h <<= 1) {
        if (h < n) {
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                if (!(i & h)) {
                    const float a = v[i], b = v[i + h];
                    v[i] = a + b;
                    v[i + h] = a - b;
                }
            }
        }
    }
    const int lane = __lane_id();
    if (n >= 64) {
        // lower lane: partner + self = a + b; upper lane: partner - self = a - b (one rounding)
        const float sgn = (lane & 1) ? -1.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = __builtin_fmaf(v[i], sgn, lane_xor<1>(v[i]));
    }
    if (n >= 128) {
        const float sgn = (lane & 2) ? -1.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = __builtin_fmaf(v[i], sgn, lane_xor<2>(v[i]));
    }
    const float c = n == 16 ? inv_sqrt_n<16>() : n == 32 ? inv_sqrt_n<32>() : n == 64 ? inv_sqrt_n<64>() : inv_sqrt_n<128>();
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = v[i] * c;
}

// Encode elements [OFF, OFF + B) of v into out (nibbles for E2M1: element j -> nibble j of the
// 16-byte segment; bytes for E4M3). Scale arguments:
//  pow2: the block scale is 2^k (k >= -126 after the caller's adjustment): the hardware convert
//        divides by it exactly (RNE); SR multiplies by rcp = 2^-k exactly.
//  else: elements are v * rcp (RN), converted with scale 1.
template <int ELEM, int RND, int B, int OFF>
__device__ __forceinline__ void encode_block(float (&v)[32], bool pow2, float cvt_scale, float rcp,
                                             float clampv, const SrSource& sr,
                                             uint32_t (&out)[8]) {
    if constexpr (RND == RND_RNE) {
        if (!pow2) {
#pragma unroll
            for (int i = OFF; i < OFF + B; ++i) v[i] = v[i] * rcp;
        }
        if constexpr (ELEM == ELEM_E2M1) {
#pragma unroll
            for (int w = OFF / 8; w < (OFF + B) / 8; ++w) {
                uint32_t r = 0u;
                r = cvt_fp4x2<0>(r, v[8 * w + 0], v[8 * w + 1], cvt_scale);
                r = cvt_fp4x2<1>(r, v[8 * w + 2], v[8 * w + 3], cvt_scale);
                r = cvt_fp4x2<2>(r, v[8 * w + 4], v[8 * w + 5], cvt_scale);
                r = cvt_fp4x2<3>(r, v[8 * w + 6], v[8 * w + 7], cvt_scale);
                out[w] = r;
            }
        } else {
#pragma unroll
            for (int w = OFF / 4; w < (OFF + B) / 4; ++w) {
                // saturate at +-448 (times the scale) before the non-saturating convert
                const float a0 = __builtin_amdgcn_fmed3f(v[4 * w + 0], -clampv, clampv);
                const float a1 = __builtin_amdgcn_fmed3f(v[4 * w + 1], -clampv, clampv);
                const float a2 = __builtin_amdgcn_fmed3f(v[4 * w + 2], -clampv, clampv);
                const float a3 = __builtin_amdgcn_fmed3f(v[4 * w + 3], -clampv, clampv);
                uint32_t r = 0u;
                r = cvt_fp8x2<false>(r, a0, a1, cvt_scale);
                r = cvt_fp8x2<true>(r, a2, a3, cvt_scale);
                out[w] = r;
            }
        }
    } else {
#pragma unroll
        for (int i = OFF; i < OFF + B; ++i) v[i] = v[i] * rcp;
        if constexpr (ELEM == ELEM_E2M1) {
            // word w of out holds the 8 nibbles of group w
#pragma unroll
            for (int w = OFF / 8; w < (OFF + B) / 8; ++w) {
                uint32_t c[4];
                philox_group(sr, w, c);
                uint32_t r = 0u;
#pragma unroll
                for (int j = 0; j < 8; ++j) r |= e2m1_sr(v[8 * w + j], sr_u16(c, j)) << (4 * j);
                out[w] = r;
            }
        } else {
            // words 2 g8 and 2 g8 + 1 of out hold the 8 bytes of group g8
#pragma unroll
            for (int g8 = OFF / 8; g8 < (OFF + B) / 8; ++g8) {
                uint32_t c[4];
                philox_group(sr, g8, c);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int w = 2 * g8 + h;
                    uint32_t r = 0u;
#pragma unroll
                    for (int j = 0; j < 4; ++j) r |= e4m3_sr(v[4 * w + j], sr_u16(c, 4 * h + j)) << (8 * j);
                    out[w] = r;
                }
            }
        }
    }
}

// E8M0 path for one block: returns the scale byte; encodes into out.
template <int ELEM, int RND, int B, int OFF>
__device__ __forceinline__ uint32_t e8m0_block(float (&v)[32], float amax, bool ceil_rule,
                                               const SrSource& sr, uint32_t (&out)[8]) {
    int k = (ELEM == ELEM_E2M1) ? e8m0_exp<2, 0x400000u>(amax, ceil_rule)
                                : e8m0_exp<8, 0x600000u>(amax, ceil_rule);
    const uint32_t sbyte = (uint32_t)(k + 127);
    if (k == -127) {
        // 2^-127 is not a normal fp32: divide by 2^-126 after doubling (exact for such tiny x)
#pragma unroll
        for (int i = OFF; i < OFF + B; ++i) v[i] = v[i] * 2.0f;
        k = -126;
    }
    const float scale = pow2f(k);
    const float rcp = __builtin_amdgcn_ldexpf(1.0f, -k);
    const float clampv = 448.0f * scale;
    encode_block<ELEM, RND, B, OFF>(v, true, scale, rcp, clampv, sr, out);
    return sbyte;
}

}  // namespace bgf
