// Segment loading and the blockwise rotation of a segment, shared by the quantize kernels and the
// GEMM that rotates and quantizes its A operand itself.
//
// Work unit: one lane owns one "segment", 32 consecutive elements of a row (64 B of bf16 or 128 B
// of fp32, loaded with 128-bit loads). A 32-element MX group is then exactly one lane, a
// 16-element NVFP4 block half a lane, and a Hadamard chunk of n elements n/32 adjacent lanes:
//  - n <= 32: all butterfly stages run inside the lane's registers;
//  - n = 64, 128, 256: stages h = 1..16 run in registers, then h = 32, 64, 128 pair lane l with
//    lane l ^ 1, ^ 2, ^ 4 through the LDS crossbar (ds_swizzle).
// Each stage computes partner + (+-1) * self in one fused multiply-add, which equals the
// butterfly's sum / difference exactly, in the same stage order as the definition (h ascending,
// then one multiply by RN(1/sqrt(n))), so rotated values are bit-identical to that order.
#pragma once

#include "device.h"
#include "fp4_internal.h"

namespace bgf {

// 16-byte pieces per 32-element segment, and the LDS slice a wave needs to transpose 64 of them
template <int IN>
struct SegIO {
    static constexpr int P = IN == DT_BF16 ? 4 : 8;
    static constexpr int ESZ = IN == DT_BF16 ? 2 : 4;
};

// Gives every lane of the wave the 32 elements of segment `lane` of a 64-segment wave tile.
// Piece ch = 64 i + lane (16 bytes: piece ch % P of tile segment ch / P) is read from byte offset
// off[i] of the buffer rs (offsets past the buffer's extent, such as -1, read as zeros). The loads
// are wave-wide and 16 bytes per lane, consecutive lanes reading consecutive pieces (whole cache
// lines wherever segments are adjacent in memory); the pieces are then transposed through the
// wave's own LDS slice, piece q of segment s at 16-byte slot P s + (q ^ ((s / G) % P)) with
// G = 16 / P, so that both the writes and the reads of any 16 consecutive lanes touch 16 distinct
// slots of one 256-byte bank sweep. A wave's LDS accesses complete in order, so the read-back needs
// no barrier.
// With RAW, the transposition is skipped: v holds the 32 elements the lane loaded itself, from
// several segments (enough for an order-free reduction such as the tensor amax).
template <int IN, bool RAW = false>
__device__ __forceinline__ void unpack_wave_segments(const u32x4 (&raw)[SegIO<IN>::P], u32x4* lds, float (&v)[32]) {
    constexpr int P = SegIO<IN>::P, G = 16 / P;
    const int lane = __lane_id();
    if constexpr (RAW) {
#pragma unroll
        for (int q = 0; q < P; ++q) {
            if constexpr (IN == DT_BF16) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    v[8 * q + 2 * j] = bf16_lo(raw[q][j]);
                    v[8 * q + 2 * j + 1] = bf16_hi(raw[q][j]);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) v[4 * q + j] = __uint_as_float(raw[q][j]);
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const int ch = 64 * i + lane, sg = ch / P, q = ch % P;
        lds[P * sg + (q ^ ((sg / G) % P))] = raw[i];
    }
#pragma unroll
    for (int q = 0; q < P; ++q) {
        const u32x4 w = lds[P * lane + (q ^ ((lane / G) % P))];
        if constexpr (IN == DT_BF16) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[8 * q + 2 * j] = bf16_lo(w[j]);
                v[8 * q + 2 * j + 1] = bf16_hi(w[j]);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) v[4 * q + j] = __uint_as_float(w[j]);
        }
    }
}

template <int IN, bool RAW = false>
__device__ __forceinline__ void load_wave_segments(__amdgpu_buffer_rsrc_t rs, const int (&off)[SegIO<IN>::P],
                                                   u32x4* lds, float (&v)[32]) {
    constexpr int P = SegIO<IN>::P;
    u32x4 raw[P];
#pragma unroll
    for (int i = 0; i < P; ++i) raw[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, off[i], 0, 2 /* nt */);
    unpack_wave_segments<IN, RAW>(raw, lds, v);
}

// Issues the loads of the wave tile of 64 consecutive segments wbase .. wbase + 63 of a row-major
// [rows, cols] tensor with row pitch ldx (segments past nseg read as zeros) into raw; the values
// arrive asynchronously, so several tiles' loads can be in flight before the first is unpacked.
template <int IN>
__device__ __forceinline__ void issue_wave_segments_1d(const SegArgs& a, int64_t wbase, u32x4 (&raw)[SegIO<IN>::P]) {
    constexpr int P = SegIO<IN>::P, ESZ = SegIO<IN>::ESZ;
    const int lane = __lane_id();
    const int64_t spr = a.cols >> 5;
    const char* const xb = reinterpret_cast<const char*>(a.x);
    int off[P];
    __amdgpu_buffer_rsrc_t rs;
    if (a.ldx == a.cols) {
        // contiguous rows: the tile is one run of bytes; the extent stops at the tensor's end, and
        // is 0 for a tile wholly past it (the last workgroup's trailing waves), so that nothing
        // beyond the tensor is read
        int64_t left = (a.nseg - wbase) * 32 * ESZ;
        left = left < 0 ? 0 : (left < 64 * 32 * ESZ ? left : 64 * 32 * ESZ);
        rs = __builtin_amdgcn_make_buffer_rsrc((void*)(xb + (left > 0 ? wbase * 32 * ESZ : 0)), (short)0, (int)left,
                                               0x00020000);
#pragma unroll
        for (int i = 0; i < P; ++i) off[i] = 16 * (64 * i + lane);
    } else {
        // strided rows: per-piece offsets from the tile's first segment (row pitch below 32 MiB)
        const int64_t r0 = wbase / spr;
        const int64_t base = r0 * a.ldx + (wbase - r0 * spr) * 32;
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const int ch = 64 * i + lane;
            const int64_t sg = wbase + ch / P;
            const int64_t r = sg / spr;
            off[i] = sg < a.nseg ? (int)((r * a.ldx + (sg - r * spr) * 32 - base) * ESZ + 16 * (ch % P)) : -1;
        }
        rs = __builtin_amdgcn_make_buffer_rsrc((void*)(xb + base * ESZ), (short)0, 0x7FFFFFFF, 0x00020000);
    }
#pragma unroll
    for (int i = 0; i < P; ++i) raw[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, off[i], 0, 2 /* nt */);
}

// Loads the wave tile of 64 consecutive segments wbase .. wbase + 63 and gives every lane the 32
// elements of segment wbase + lane.
template <int IN, bool RAW = false>
__device__ __forceinline__ void load_wave_segments_1d(const SegArgs& a, int64_t wbase, u32x4* lds, float (&v)[32]) {
    u32x4 raw[SegIO<IN>::P];
    issue_wave_segments_1d<IN>(a, wbase, raw);
    unpack_wave_segments<IN, RAW>(raw, lds, v);
}

// Blockwise H_n / sqrt(n) on the segment (see the file comment for the lane mapping).
template <int HN>
__device__ __forceinline__ void fwht_segment(float (&v)[32]) {
    if constexpr (HN > 0) {
        constexpr int HIN = HN < 32 ? HN : 32;  // in-register extent
#pragma unroll
        for (int h = 1; h < HIN; h <<= 1) {
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                if (!(i & h)) {
                    const float a = v[i], b = v[i + h];
                    v[i] = a + b;
                    v[i + h] = a - b;
                }
            }
        }
        if constexpr (HN >= 64) {
            const int lane = __lane_id();
#pragma unroll
            for (int m = 1; m < HN / 32; m <<= 1) {
                const float sgn = (lane & m) ? -1.0f : 1.0f;
#pragma unroll
                for (int i = 0; i < 32; ++i) {
                    float partner;
                    if (m == 1) partner = lane_xor<1>(v[i]);
                    else if (m == 2) partner = lane_xor<2>(v[i]);
                    else partner = lane_xor<4>(v[i]);
                    // lower lane: partner + self = a + b; upper lane: partner - self = a - b
                    v[i] = __builtin_fmaf(v[i], sgn, partner);
                }
            }
        }
        const float c = inv_sqrt_n<HN>();
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = v[i] * c;
    }
}

}  // namespace bgf
