// Fused rotate + quantize, dequantize and the rotation alone, for gfx950.
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
// Group amax, scale encode, element rounding (hardware RNE convert, or Philox-driven stochastic
// rounding in software) and nibble packing then happen in registers; each lane stores 16 B of
// codes (32 B for E4M3) and its block scale(s).
//
// 2D (32 x 32) blocks: a workgroup covers 32 rows x 8 segments; the tile max goes through LDS.
// Per-row / per-tensor blocks (any even width, no rotation) use a row-per-workgroup kernel.
#include <float.h>

#include "device.h"
#include "fp4_internal.h"
#include "quant_block.h"
#include "segment.h"

namespace bgf {

constexpr int kThreads = 256;

// Column-wise view: the logical tensor is T = x^T ([rows, cols] of SegArgs describe T; x is
// [cols, rows] with row pitch ldx). A workgroup tile is TCW = 4 * 64 / SEGW consecutive T-rows (x
// columns) by SEGW consecutive segments (32 SEGW x rows). Wave w takes T-rows w * 64 / SEGW ..,
// and lane l of it T-row l / SEGW of those and segment l % SEGW, so the segments of one Hadamard
// chunk (up to SEGW) sit in lanes l ^ 1, l ^ 2, (l ^ 4). The workgroup reads the tile's x rows
// with 16-byte loads (each row piece TCW elements long: whole cache lines), stores them in LDS as
// SEGW blocks of 32 rows (each block skewed by 8 dwords, so that the column reads below hit
// distinct banks), and each lane then reads its column of 32 values. Every thread of the
// workgroup must call it (it holds a barrier).
template <int IN, int SEGW>
__device__ __forceinline__ void load_block_segments_t(const SegArgs& a, int64_t tt, int64_t ts, uint8_t* lds,
                                                      float (&v)[32]) {
    constexpr int P = SegIO<IN>::P, ESZ = SegIO<IN>::ESZ, TCW = 4 * 64 / SEGW, PITCH = TCW * ESZ;
    constexpr int PPR = PITCH / 16, BSTR = 32 * PITCH + 32;
    static_assert(32 * SEGW * PPR == kThreads * P, "tile pieces per thread");
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t x0 = (ts * SEGW * 32) * a.ldx + tt * TCW;  // first element of the tile in x
    const int64_t total = a.cols * a.ldx;                     // elements of x (T-columns are x rows)
    int64_t left = (total - x0) * ESZ;
    left = left < 0 ? 0 : (left > 0x7FFFFFFF ? 0x7FFFFFFF : left);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const char*>(a.x) + (left > 0 ? x0 * ESZ : 0)), (short)0, (int)left, 0x00020000);
    u32x4 raw[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const int ch = kThreads * i + tid, rho = ch / PPR, q = ch % PPR;
        // pieces that start at or past x's last column read zeros; x rows past the end lie past
        // the buffer's extent and read zeros too
        const bool colok = tt * TCW + (16 * q) / ESZ < a.rows;
        raw[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, colok ? (int)(rho * a.ldx * ESZ + 16 * q) : -1, 0, 2 /* nt */);
    }
    __syncthreads();  // the previous tile's column reads are done
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const int ch = kThreads * i + tid, rho = ch / PPR, q = ch % PPR;
        *reinterpret_cast<u32x4*>(lds + (rho / 32) * BSTR + (rho % 32) * PITCH + 16 * q) = raw[i];
    }
    __syncthreads();
    const int j = wv * (64 / SEGW) + lane / SEGW, sg = lane % SEGW;
    const uint8_t* col = lds + sg * BSTR + j * ESZ;
#pragma unroll
    for (int r = 0; r < 32; ++r) {
        if constexpr (IN == DT_BF16)
            v[r] = __uint_as_float((uint32_t)(*reinterpret_cast<const uint16_t*>(col + r * PITCH)) << 16);
        else
            v[r] = *reinterpret_cast<const float*>(col + r * PITCH);
    }
}

// NVFP4 block scales of one tensor scale g: entry s of the table holds d = RN(val(s) g) and its
// reciprocal RN(1/d) (0 for d = 0), so that a block needs no division for its reciprocal. Filled by
// the workgroup's first 128 threads (code 0x7F, E4M3's NaN, is never chosen: the code saturates).
__device__ __forceinline__ void nv_table_fill(float2* tab, float g) {
    if (threadIdx.x < 128) {
        const uint32_t s = threadIdx.x;
        const float d = s < 0x7Fu ? e4m3_value(s) * g : 0.0f;
        tab[s] = make_float2(d, scale_recip(d));
    }
}

// The divisors of one tensor's block-scale quotients: c = RN(M g) for M = 6 and 4, their
// reciprocals RN(1/c), and whether both c lie in [2^-100, 2^100] (then the quotients below need no
// division).
struct NvDiv {
    float c6, y6, c4, y4;
    bool fast;
};
__device__ __forceinline__ NvDiv nv_div(float g) {
    NvDiv n;
    n.c6 = 6.0f * g;
    n.c4 = 4.0f * g;
    n.y6 = 1.0f / n.c6;
    n.y4 = 1.0f / n.c4;
    n.fast = n.c6 >= 0x1p-100f && n.c6 <= 0x1p100f && n.c4 >= 0x1p-100f && n.c4 <= 0x1p100f;
    return n;
}

// RN(a / c) from y = RN(1/c) with two Markstein corrections (Markstein, "Computation of elementary
// functions on the IBM RISC System/6000 processor", 1990): q0 = RN(a y) is within 1.5 ulp of a/c,
// q1 = RN(q0 + RN(a - c q0) y) within one ulp, and with r1 = a - c q1 exact (a fused multiply-add)
// RN(q1 + r1 y) is the correctly rounded quotient. Valid while nothing underflows or overflows:
// c and a (or a = 0) in [2^-100, 2^100], checked by the caller.
__device__ __forceinline__ float div_by_recip(float a, float c, float y) {
    const float q0 = a * y;
    const float r0 = __builtin_fmaf(-c, q0, a);
    const float q1 = __builtin_fmaf(r0, y, q0);
    const float r1 = __builtin_fmaf(-c, q1, a);
    return __builtin_fmaf(r1, y, q1);
}

// NVFP4 candidate: s = E4M3(amax_b / RN(M g)), d = RN(val(s) g), r = RN(1/d); c = RN(M g), y = RN(1/c)
__device__ __forceinline__ uint32_t nv_candidate(float amax, float c, float y, bool fast, const float2* tab,
                                                 float& d, float& r) {
    float t;
    if (fast && (amax == 0.0f || (amax >= 0x1p-100f && amax <= 0x1p100f)))
        t = div_by_recip(amax, c, y);
    else
        t = amax / c;
    const uint32_t s = e4m3_code_sat(t);
    const float2 e = tab[s];
    d = e.x;
    r = e.y;
    return s;
}

// RNE codes of the 16-element block at OFF with scale d (r = its reciprocal), packed as the encode
// does (two words, element j in nibble j % 8 of word j / 8), and the block's SSE of the decoded
// values in the fixed pairwise tree over the 16 squared errors RN(x - RN(q d))^2.
template <int OFF>
__device__ __forceinline__ float nv_codes_sse(const float (&v)[32], float d, float r, uint32_t (&code)[2]) {
    float t[16];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        const int b = OFF + 8 * w;
        uint32_t c = cvt_fp4x2<0>(0u, v[b] * r, v[b + 1] * r, 1.0f);
        c = cvt_fp4x2<1>(c, v[b + 2] * r, v[b + 3] * r, 1.0f);
        c = cvt_fp4x2<2>(c, v[b + 4] * r, v[b + 5] * r, 1.0f);
        c = cvt_fp4x2<3>(c, v[b + 6] * r, v[b + 7] * r, 1.0f);
        code[w] = c;
        const v2f q0 = fp4x2_to_f32<0>(c), q1 = fp4x2_to_f32<1>(c), q2 = fp4x2_to_f32<2>(c), q3 = fp4x2_to_f32<3>(c);
        const float dq[8] = {q0[0], q0[1], q1[0], q1[1], q2[0], q2[1], q3[0], q3[1]};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float e = v[b + j] - dq[j] * d;
            t[8 * w + j] = e * e;
        }
    }
#pragma unroll
    for (int w = 16; w > 1; w >>= 1)
#pragma unroll
        for (int i = 0; i < w / 2; ++i) t[i] = t[2 * i] + t[2 * i + 1];
    return t[0];
}

// NVFP4 path for one 16-element block: returns the E4M3 scale code. With four_six (RNE only) both
// candidates are encoded once; the SSE comparison picks one and its codes are kept as they are.
template <int RND, int OFF>
__device__ __forceinline__ uint32_t nv_block(float (&v)[32], float amax, const NvDiv& nd, const float2* tab,
                                             bool four_six, const SrSource& sr, uint32_t (&out)[8]) {
    float d, r;
    uint32_t s = nv_candidate(amax, nd.c6, nd.y6, nd.fast, tab, d, r);
    if constexpr (RND == RND_RNE) {
        if (four_six) {
            float d4, r4;
            const uint32_t s4 = nv_candidate(amax, nd.c4, nd.y4, nd.fast, tab, d4, r4);
            uint32_t c6[2], c4[2];
            const float e6 = nv_codes_sse<OFF>(v, d, r, c6);
            const float e4 = nv_codes_sse<OFF>(v, d4, r4, c4);
            const bool four = e4 < e6;
            out[OFF / 8] = four ? c4[0] : c6[0];
            out[OFF / 8 + 1] = four ? c4[1] : c6[1];
            return four ? s4 : s;
        }
    }
    encode_block<ELEM_E2M1, RND, 16, OFF>(v, false, 1.0f, r, 448.0f, sr, out);
    return s;
}

// fp32-scale path for one block: writes the scale value.
template <int ELEM, int RND, int B, int OFF>
__device__ __forceinline__ float f32_block(float (&v)[32], float amax, const SrSource& sr,
                                           uint32_t (&out)[8]) {
    const float d = amax / (ELEM == ELEM_E2M1 ? 6.0f : 448.0f);
    encode_block<ELEM, RND, B, OFF>(v, false, 1.0f, scale_recip(d), 448.0f, sr, out);
    return d;
}

// ---------------------------------------------------------------------------------------------
// The segment kernel (1D groups, 2D tiles, amax pass, rotation pass)
// ---------------------------------------------------------------------------------------------
template <int IN, int HN, int ELEM, int SC, int RND, int BR, int BC, int PASS, bool TRX>
__global__ __launch_bounds__(kThreads) void k_segment(SegBatch b) {
    constexpr int P = SegIO<IN>::P, ESZ = SegIO<IN>::ESZ;
    // this workgroup's item of the batch and its workgroup index within the item (uniform)
    int it = 0;
#pragma unroll
    for (int i = 1; i < kMaxBatch; ++i)
        if (i < b.n && blockIdx.x >= b.start[i]) it = i;
    const SegArgs a = it == 0 ? b.t[0] : it == 1 ? b.t[1] : it == 2 ? b.t[2] : b.t[3];
    const uint32_t blk = blockIdx.x - (it == 0 ? b.start[0] : it == 1 ? b.start[1] : it == 2 ? b.start[2] : b.start[3]);
    // column-wise view: workgroup tiles of TCW T-rows x SEGW segments (see load_block_segments_t)
    constexpr int SEGW = HN >= 256 ? 8 : 4, TCW = 4 * 64 / SEGW;
    static_assert(!TRX || (BR == 1 && PASS != PASS_ROTATE), "column-wise view: 1D groups only");
    __shared__ u32x4 stage[kThreads / 64][64 * P + (TRX ? 16 : 0)];
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;  // wave-uniform wv
    const int64_t spr = a.cols >> 5;  // segments per row

    if constexpr (PASS == PASS_AMAX) {
        // tensor amax of the (rotated) input: a grid-stride walk over 256-segment groups, one
        // atomic max per workgroup (non-negative floats order like their bit patterns)
        float m = 0.0f;
        if constexpr (TRX) {
            const int64_t ntt = (a.rows + TCW - 1) / TCW, ntiles = ntt * ((spr + SEGW - 1) / SEGW);
            for (int64_t w = blockIdx.x; w < ntiles; w += gridDim.x) {  // workgroup-uniform
                float v[32];
                load_block_segments_t<IN, SEGW>(a, w % ntt, w / ntt, reinterpret_cast<uint8_t*>(&stage[0][0]), v);
                fwht_segment<HN>(v);
                m = fmaxf(m, block_amax<32, 0>(v));  // lanes outside the tensor hold zeros
            }
        } else {
            for (int64_t g0 = (int64_t)blockIdx.x * kThreads; g0 < a.nseg; g0 += (int64_t)gridDim.x * kThreads) {
                float v[32];
                // without a rotation the max needs no segment order: skip the LDS transposition
                load_wave_segments_1d<IN, HN == 0>(a, g0 + 64 * wv, stage[wv], v);
                fwht_segment<HN>(v);
                m = fmaxf(m, block_amax<32, 0>(v));
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
        __shared__ float red[kThreads / 64];
        if (lane == 0) red[wv] = m;
        __syncthreads();
        if (threadIdx.x == 0) {
            float t = red[0];
#pragma unroll
            for (int i = 1; i < kThreads / 64; ++i) t = fmaxf(t, red[i]);
            atomicMax(a.ws, __float_as_uint(t));
        }
        return;
    }

    // this lane's segment: lane of a 64-segment wave tile. seg = row * spr + sc indexes codes and
    // scales; 32 seg is the row-major index of the segment's first element.
    int64_t seg, row = 0, sc = 0;
    bool valid;
    float v[32];
    if constexpr (TRX) {
        const int64_t ntt = (a.rows + TCW - 1) / TCW;
        const int64_t tt = blk % ntt, ts = blk / ntt;
        const int64_t tr = tt * TCW + wv * (64 / SEGW) + lane / SEGW;
        sc = ts * SEGW + lane % SEGW;
        valid = tr < a.rows && sc < spr;
        seg = tr * spr + sc;
        load_block_segments_t<IN, SEGW>(a, tt, ts, reinterpret_cast<uint8_t*>(&stage[0][0]), v);
    } else if constexpr (BR == 1) {
        const int64_t wbase = (int64_t)blk * kThreads + 64 * wv;
        seg = wbase + lane;
        valid = seg < a.nseg;
        load_wave_segments_1d<IN>(a, wbase, stage[wv], v);
    } else {
        // 2D: a workgroup covers 32 rows x 8 segments, wave wv rows 8 wv .. 8 wv + 7
        const int64_t ngc = (spr + 7) >> 3;
        const int64_t R = blk / (uint32_t)ngc, C = blk - R * ngc;
        row = R * 32 + 8 * wv + (lane >> 3);
        sc = C * 8 + (lane & 7);
        valid = sc < spr;
        // wave tile: rows 8 wv + s / 8 and segment columns C * 8 + s % 8 of the workgroup's rows
        int off[P];
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const int ch = 64 * i + lane, s2 = ch / P;
            const int64_t c2 = C * 8 + (s2 & 7);
            off[i] = c2 < spr ? (int)(((s2 >> 3) * a.ldx + c2 * 32) * ESZ + 16 * (ch % P)) : -1;
        }
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(reinterpret_cast<const char*>(a.x) + (R * 32 + 8 * wv) * a.ldx * ESZ), (short)0, 0x7FFFFFFF, 0x00020000);
        load_wave_segments<IN>(rs, off, stage[wv], v);
        seg = row * spr + sc;
    }
    fwht_segment<HN>(v);

    if constexpr (PASS == PASS_ROTATE) {
        if (valid) {
            float4* y = reinterpret_cast<float4*>(a.yrot + seg * 32);
#pragma unroll
            for (int i = 0; i < 8; ++i) y[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
        }
        return;
    }
    if constexpr (PASS == PASS_QUANT) {
        const SrSource sr{a.seed, (uint64_t)seg * 32u};
        uint32_t out[8];
        if constexpr (BR == 32) {
            // tile max over 32 rows: thread (r, j) of the 32 x 8 layout
            __shared__ float tile[kThreads];
            tile[threadIdx.x] = block_amax<32, 0>(v);
            __syncthreads();
            float m = 0.0f;
#pragma unroll
            for (int r = 0; r < 32; ++r) m = fmaxf(m, tile[r * 8 + (threadIdx.x & 7)]);
            const uint32_t s = e8m0_block<ELEM, RND, 32, 0>(v, m, a.ceil_rule != 0, sr, out);
            if (valid && (threadIdx.x >> 3) == 0)
                reinterpret_cast<uint8_t*>(a.scales)[(row >> 5) * spr + sc] = (uint8_t)s;
        } else if constexpr (SC == SC_E8M0) {
            if constexpr (BC == 32) {
                const uint32_t s = e8m0_block<ELEM, RND, 32, 0>(v, block_amax<32, 0>(v), a.ceil_rule != 0, sr, out);
                if (valid) reinterpret_cast<uint8_t*>(a.scales)[seg] = (uint8_t)s;
            } else {
                const float m0 = block_amax<16, 0>(v), m1 = block_amax<16, 16>(v);
                const uint32_t s0 = e8m0_block<ELEM, RND, 16, 0>(v, m0, a.ceil_rule != 0, sr, out);
                const uint32_t s1 = e8m0_block<ELEM, RND, 16, 16>(v, m1, a.ceil_rule != 0, sr, out);
                if (valid) reinterpret_cast<uint16_t*>(a.scales)[seg] = (uint16_t)(s0 | (s1 << 8));
            }
        } else if constexpr (SC == SC_NV) {
            float g;
            if (a.nv_given) {
                g = *a.tensor_scale;  // the caller's (delayed) tensor scale
            } else {
                const float amax_t = __uint_as_float(*a.ws);
                g = amax_t > 0.0f ? amax_t / 2688.0f : 1.0f;
                if (blk == 0 && threadIdx.x == 0) *a.tensor_scale = g;
            }
            __shared__ float2 nvtab[128];
            nv_table_fill(nvtab, g);
            __syncthreads();
            const float m0 = block_amax<16, 0>(v), m1 = block_amax<16, 16>(v);
            const NvDiv nd = nv_div(g);
            const uint32_t s0 = nv_block<RND, 0>(v, m0, nd, nvtab, a.four_six != 0, sr, out);
            const uint32_t s1 = nv_block<RND, 16>(v, m1, nd, nvtab, a.four_six != 0, sr, out);
            if (valid) reinterpret_cast<uint16_t*>(a.scales)[seg] = (uint16_t)(s0 | (s1 << 8));
        } else {  // SC_F32
            if constexpr (BC == 32) {
                const float d = f32_block<ELEM, RND, 32, 0>(v, block_amax<32, 0>(v), sr, out);
                if (valid) reinterpret_cast<float*>(a.scales)[seg] = d;
            } else {
                const float m0 = block_amax<16, 0>(v), m1 = block_amax<16, 16>(v);
                const float d0 = f32_block<ELEM, RND, 16, 0>(v, m0, sr, out);
                const float d1 = f32_block<ELEM, RND, 16, 16>(v, m1, sr, out);
                if (valid) reinterpret_cast<float2*>(a.scales)[seg] = make_float2(d0, d1);
            }
        }
        if (valid) {
            if constexpr (ELEM == ELEM_E2M1) {
                uint4* dst = reinterpret_cast<uint4*>(a.codes + seg * 16);
                *dst = make_uint4(out[0], out[1], out[2], out[3]);
            } else {
                uint4* dst = reinterpret_cast<uint4*>(a.codes + seg * 32);
                dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
                dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
            }
        }
    }
}

// ---------------------------------------------------------------------------------------------
// Per-row / per-tensor blocks: one workgroup per row, any even width, no rotation
// ---------------------------------------------------------------------------------------------
template <int IN>
__device__ __forceinline__ float load_elem(const void* x, int64_t i) {
    if constexpr (IN == DT_BF16) return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(x)[i] << 16);
    return reinterpret_cast<const float*>(x)[i];
}

template <int IN>
__global__ __launch_bounds__(kThreads) void k_amax_rows(const void* x, int64_t rows, int64_t cols,
                                                        int64_t ldx, uint32_t* ws) {
    __shared__ float red[kThreads];
    float m = 0.0f;
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x)
        for (int64_t c = threadIdx.x; c < cols; c += kThreads) m = fmaxf(m, fabsf(load_elem<IN>(x, r * ldx + c)));
    red[threadIdx.x] = m;
    __syncthreads();
    for (int s = kThreads / 2; s > 0; s >>= 1) {
        if (threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
        __syncthreads();
    }
    if (threadIdx.x == 0) atomicMax(ws, __float_as_uint(red[0]));
}

template <int IN, int ELEM, int SC, int RND>
__global__ __launch_bounds__(kThreads) void k_rowblock(RowArgs a) {
    __shared__ float red[kThreads];
    const int64_t row = blockIdx.x;
    const void* xr = reinterpret_cast<const char*>(a.x) + row * a.ldx * (IN == DT_BF16 ? 2 : 4);
    float amax;
    if (a.per_tensor) {
        amax = __uint_as_float(*a.ws);
    } else {
        float m = 0.0f;
        for (int64_t c = threadIdx.x; c < a.cols; c += kThreads) m = fmaxf(m, fabsf(load_elem<IN>(xr, c)));
        red[threadIdx.x] = m;
        __syncthreads();
        for (int s = kThreads / 2; s > 0; s >>= 1) {
            if (threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
            __syncthreads();
        }
        amax = red[0];
    }
    // scale
    float rcp, cvt_scale = 1.0f, clampv = 448.0f;
    bool pow2 = false;
    float pre = 1.0f;
    const int64_t sidx = a.per_tensor ? 0 : row;
    const bool writer = threadIdx.x == 0 && (!a.per_tensor || row == 0);
    if constexpr (SC == SC_E8M0) {
        int k = (ELEM == ELEM_E2M1) ? e8m0_exp<2, 0x400000u>(amax, a.ceil_rule != 0)
                                    : e8m0_exp<8, 0x600000u>(amax, a.ceil_rule != 0);
        if (writer) reinterpret_cast<uint8_t*>(a.scales)[sidx] = (uint8_t)(k + 127);
        if (k == -127) {
            pre = 2.0f;
            k = -126;
        }
        pow2 = true;
        cvt_scale = pow2f(k);
        rcp = __builtin_amdgcn_ldexpf(1.0f, -k);
        clampv = 448.0f * cvt_scale;
    } else {
        const float d = amax / (ELEM == ELEM_E2M1 ? 6.0f : 448.0f);
        if (writer) reinterpret_cast<float*>(a.scales)[sidx] = d;
        rcp = scale_recip(d);
    }
    // elements, two per step
    for (int64_t p = threadIdx.x; p < a.cols / 2; p += kThreads) {
        float x0 = load_elem<IN>(xr, 2 * p) * pre, x1 = load_elem<IN>(xr, 2 * p + 1) * pre;
        const uint64_t idx = (uint64_t)(row * a.cols + 2 * p);
        uint32_t q0, q1;
        if constexpr (RND == RND_SR) {
            x0 = x0 * rcp;
            x1 = x1 * rcp;
            uint32_t c0 = (uint32_t)(idx >> 3), c1 = (uint32_t)(idx >> 35), c2 = 0u, c3 = 0u;
            philox4x32_10(c0, c1, c2, c3, (uint32_t)a.seed, (uint32_t)(a.seed >> 32));
            const uint32_t words[4] = {c0, c1, c2, c3};
            const uint32_t w = words[(idx >> 1) & 3];  // idx even: this word holds both uniforms
            if constexpr (ELEM == ELEM_E2M1) {
                q0 = e2m1_sr(x0, w & 0xFFFFu);
                q1 = e2m1_sr(x1, w >> 16);
            } else {
                q0 = e4m3_sr(x0, w & 0xFFFFu);
                q1 = e4m3_sr(x1, w >> 16);
            }
        } else {
            if (!pow2) {
                x0 = x0 * rcp;
                x1 = x1 * rcp;
            }
            if constexpr (ELEM == ELEM_E2M1) {
                const uint32_t r = cvt_fp4x2<0>(0u, x0, x1, cvt_scale);
                q0 = r & 0xFu;
                q1 = (r >> 4) & 0xFu;
            } else {
                const uint32_t r = cvt_fp8x2<false>(0u, __builtin_amdgcn_fmed3f(x0, -clampv, clampv),
                                                    __builtin_amdgcn_fmed3f(x1, -clampv, clampv), cvt_scale);
                q0 = r & 0xFFu;
                q1 = (r >> 8) & 0xFFu;
            }
        }
        if constexpr (ELEM == ELEM_E2M1) {
            a.codes[row * (a.cols / 2) + p] = (uint8_t)(q0 | (q1 << 4));
        } else {
            a.codes[row * a.cols + 2 * p] = (uint8_t)q0;
            a.codes[row * a.cols + 2 * p + 1] = (uint8_t)q1;
        }
    }
}

__global__ void k_zero_u32(uint32_t* p, int n) {
    if ((int)threadIdx.x < n) p[threadIdx.x] = 0u;
}

// ---------------------------------------------------------------------------------------------
// Dequantize
// ---------------------------------------------------------------------------------------------
template <int ELEM, int SC, int HN, int BR, int BC, int OUT>
__global__ __launch_bounds__(kThreads) void k_dequant_segment(DeqArgs a) {
    const int64_t seg = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const bool valid = seg < a.nseg;
    const int64_t spr = a.cols >> 5;
    const int64_t row = valid ? seg / spr : 0;
    const int64_t sc = valid ? seg - row * spr : 0;
    float v[32];
    if (valid) {
        // block scales of this segment
        float d0, d1;
        if constexpr (SC == SC_F32) {
            const float* s = reinterpret_cast<const float*>(a.scales);
            if constexpr (BC == 32) d0 = d1 = s[(row / BR) * spr + sc];
            else { d0 = s[2 * seg]; d1 = s[2 * seg + 1]; }
        } else {
            const uint8_t* s = reinterpret_cast<const uint8_t*>(a.scales);
            uint32_t b0, b1;
            if constexpr (BC == 32) b0 = b1 = s[(row / BR) * spr + sc];
            else { b0 = s[2 * seg]; b1 = s[2 * seg + 1]; }
            if constexpr (SC == SC_E8M0) {
                d0 = __builtin_amdgcn_ldexpf(1.0f, (int)b0 - 127);
                d1 = __builtin_amdgcn_ldexpf(1.0f, (int)b1 - 127);
            } else {
                const float g = *a.tensor_scale;
                d0 = e4m3_value(b0 & 0x7Fu) * g;
                d1 = e4m3_value(b1 & 0x7Fu) * g;
            }
        }
        if constexpr (ELEM == ELEM_E2M1) {
            const uint4 q = *reinterpret_cast<const uint4*>(a.codes + seg * 16);
            const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const v2f p0 = fp4x2_to_f32<0>(qw[w]), p1 = fp4x2_to_f32<1>(qw[w]);
                const v2f p2 = fp4x2_to_f32<2>(qw[w]), p3 = fp4x2_to_f32<3>(qw[w]);
                const float d = (w < 2) ? d0 : d1;
                v[8 * w + 0] = p0[0] * d;
                v[8 * w + 1] = p0[1] * d;
                v[8 * w + 2] = p1[0] * d;
                v[8 * w + 3] = p1[1] * d;
                v[8 * w + 4] = p2[0] * d;
                v[8 * w + 5] = p2[1] * d;
                v[8 * w + 6] = p3[0] * d;
                v[8 * w + 7] = p3[1] * d;
            }
        } else {
            const uint4* src = reinterpret_cast<const uint4*>(a.codes + seg * 32);
            const uint4 q0 = src[0], q1 = src[1];
            const uint32_t qw[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const v2f p0 = fp8x2_to_f32<false>(qw[w]), p1 = fp8x2_to_f32<true>(qw[w]);
                const float d = (w < 4) ? d0 : d1;
                v[4 * w + 0] = p0[0] * d;
                v[4 * w + 1] = p0[1] * d;
                v[4 * w + 2] = p1[0] * d;
                v[4 * w + 3] = p1[1] * d;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = 0.0f;
    }
    fwht_segment<HN>(v);
    if (!valid) return;
    char* base = reinterpret_cast<char*>(a.y) + (row * a.ldy + sc * 32) * (OUT == DT_BF16 ? 2 : 4);
    if constexpr (OUT == DT_F32) {
        float4* y = reinterpret_cast<float4*>(base);
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
    } else {
        // the hardware packed convert (round to nearest even), the one the GEMM epilogue uses
        uint4* y = reinterpret_cast<uint4*>(base);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t w[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) w[j] = pack_bf16x2_rne(v[8 * i + 2 * j], v[8 * i + 2 * j + 1]);
            y[i] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
}

// per-row / per-tensor layouts (any even width): element-wise
template <int ELEM, int SC, int OUT>
__global__ __launch_bounds__(kThreads) void k_dequant_rowblock(DeqArgs a) {
    const int64_t row = blockIdx.x;
    const int64_t sidx = a.per_tensor ? 0 : row;
    float d;
    if constexpr (SC == SC_F32) d = reinterpret_cast<const float*>(a.scales)[sidx];
    else d = __builtin_amdgcn_ldexpf(1.0f, (int)reinterpret_cast<const uint8_t*>(a.scales)[sidx] - 127);
    for (int64_t c = threadIdx.x; c < a.cols; c += kThreads) {
        float q;
        if constexpr (ELEM == ELEM_E2M1) {
            const uint32_t b = a.codes[row * (a.cols / 2) + c / 2];
            const uint32_t nib = (c & 1) ? (b >> 4) : (b & 0xFu);
            q = fp4x2_to_f32<0>(nib)[0];
        } else {
            q = fp8x2_to_f32<false>((uint32_t)a.codes[row * a.cols + c])[0];
        }
        const float y = q * d;
        if constexpr (OUT == DT_F32) reinterpret_cast<float*>(a.y)[row * a.ldy + c] = y;
        else reinterpret_cast<uint16_t*>(a.y)[row * a.ldy + c] = (uint16_t)pack_bf16x2_rne(y, 0.0f);
    }
}

// ---------------------------------------------------------------------------------------------
// Host-side launchers (dispatch over the compile-time variants)
// ---------------------------------------------------------------------------------------------
#define BGF_LAUNCH(kern, grid, ...)                                                        \
    do {                                                                                   \
        hipLaunchKernelGGL((kern), dim3(grid), dim3(kThreads), 0, stream, __VA_ARGS__);    \
        return hipGetLastError();                                                          \
    } while (0)

// workgroups of one item of a launch (the amax pass walks the tensor with at most 512 of them)
template <int HN, int BR>
static int64_t seg_grid(const SegArgs& a, int pass) {
    int64_t grid;
    if (a.colwise) {
        constexpr int SEGW = HN >= 256 ? 8 : 4, TCW = 4 * 64 / SEGW;
        grid = ((a.rows + TCW - 1) / TCW) * (((a.cols >> 5) + SEGW - 1) / SEGW);
    } else if (BR == 1 || pass != PASS_QUANT) {
        grid = (a.nseg + kThreads - 1) / kThreads;
    } else {
        grid = (a.rows / 32) * (((a.cols >> 5) + 7) >> 3);
    }
    if (pass == PASS_AMAX && grid > 512) grid = 512;  // two workgroups per CU: measured fastest
    return grid;
}

template <int IN, int HN, int ELEM, int SC, int RND, int BR, int BC>
static hipError_t launch_seg_q(SegBatch b, int pass, hipStream_t stream) {
    // amax and rotation passes, and column-wise views, take one item
    if ((pass != PASS_QUANT || b.t[0].colwise) && b.n != 1) return hipErrorInvalidValue;
    int64_t grid = 0;
    for (int i = 0; i < b.n; ++i) {
        b.start[i] = (uint32_t)grid;
        grid += seg_grid<HN, BR>(b.t[i], pass);
    }
    if (grid <= 0 || grid >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    if (b.t[0].colwise) {
        if constexpr (BR == 1) {
            if (pass == PASS_AMAX) BGF_LAUNCH((k_segment<IN, HN, ELEM, SC, RND, 1, 32, PASS_AMAX, true>), grid, b);
            BGF_LAUNCH((k_segment<IN, HN, ELEM, SC, RND, 1, BC, PASS_QUANT, true>), grid, b);
        }
        return hipErrorInvalidValue;
    }
    if (pass == PASS_AMAX) BGF_LAUNCH((k_segment<IN, HN, ELEM, SC, RND, 1, 32, PASS_AMAX, false>), grid, b);
    if (pass == PASS_ROTATE) BGF_LAUNCH((k_segment<IN, HN, ELEM, SC, RND, 1, 32, PASS_ROTATE, false>), grid, b);
    BGF_LAUNCH((k_segment<IN, HN, ELEM, SC, RND, BR, BC, PASS_QUANT, false>), grid, b);
}

template <int IN, int HN>
static hipError_t dispatch_seg_hn(const SegBatch& a, int elem, int sc, int rnd, int br, int bc,
                                  int pass, hipStream_t s) {
    if (pass != PASS_QUANT) return launch_seg_q<IN, HN, ELEM_E2M1, SC_E8M0, RND_RNE, 1, 32>(a, pass, s);
#define BGF_RB(E, S, R)                                                                    \
    do {                                                                                   \
        if (br == 32) return launch_seg_q<IN, HN, E, S, R, 32, 32>(a, pass, s);            \
        if (bc == 32) return launch_seg_q<IN, HN, E, S, R, 1, 32>(a, pass, s);             \
        return launch_seg_q<IN, HN, E, S, R, 1, 16>(a, pass, s);                           \
    } while (0)
    if (sc == SC_NV) {
        if (rnd == RND_SR) return launch_seg_q<IN, HN, ELEM_E2M1, SC_NV, RND_SR, 1, 16>(a, pass, s);
        return launch_seg_q<IN, HN, ELEM_E2M1, SC_NV, RND_RNE, 1, 16>(a, pass, s);
    }
    if (elem == ELEM_E2M1) {
        if (sc == SC_E8M0) {
            if (rnd == RND_SR) BGF_RB(ELEM_E2M1, SC_E8M0, RND_SR);
            BGF_RB(ELEM_E2M1, SC_E8M0, RND_RNE);
        }
        if (rnd == RND_SR) {
            if (bc == 32) return launch_seg_q<IN, HN, ELEM_E2M1, SC_F32, RND_SR, 1, 32>(a, pass, s);
            return launch_seg_q<IN, HN, ELEM_E2M1, SC_F32, RND_SR, 1, 16>(a, pass, s);
        }
        if (bc == 32) return launch_seg_q<IN, HN, ELEM_E2M1, SC_F32, RND_RNE, 1, 32>(a, pass, s);
        return launch_seg_q<IN, HN, ELEM_E2M1, SC_F32, RND_RNE, 1, 16>(a, pass, s);
    }
    // E4M3 elements: E8M0 or fp32 scales
    if (sc == SC_F32) {
        if (rnd == RND_SR) {
            if (bc == 32) return launch_seg_q<IN, HN, ELEM_E4M3, SC_F32, RND_SR, 1, 32>(a, pass, s);
            return launch_seg_q<IN, HN, ELEM_E4M3, SC_F32, RND_SR, 1, 16>(a, pass, s);
        }
        if (bc == 32) return launch_seg_q<IN, HN, ELEM_E4M3, SC_F32, RND_RNE, 1, 32>(a, pass, s);
        return launch_seg_q<IN, HN, ELEM_E4M3, SC_F32, RND_RNE, 1, 16>(a, pass, s);
    }
    if (rnd == RND_SR) BGF_RB(ELEM_E4M3, SC_E8M0, RND_SR);
    BGF_RB(ELEM_E4M3, SC_E8M0, RND_RNE);
#undef BGF_RB
}

static hipError_t launch_batch(const SegBatch& a, int in_dtype, int hn, int elem, int sc, int rnd, int br,
                               int bc, int pass, hipStream_t s) {
#define BGF_HN(IN)                                                                         \
    switch (hn) {                                                                          \
        case 0: return dispatch_seg_hn<IN, 0>(a, elem, sc, rnd, br, bc, pass, s);          \
        case 16: return dispatch_seg_hn<IN, 16>(a, elem, sc, rnd, br, bc, pass, s);        \
        case 32: return dispatch_seg_hn<IN, 32>(a, elem, sc, rnd, br, bc, pass, s);        \
        case 64: return dispatch_seg_hn<IN, 64>(a, elem, sc, rnd, br, bc, pass, s);        \
        case 128: return dispatch_seg_hn<IN, 128>(a, elem, sc, rnd, br, bc, pass, s);      \
        case 256: return dispatch_seg_hn<IN, 256>(a, elem, sc, rnd, br, bc, pass, s);      \
        default: return hipErrorInvalidValue;                                              \
    }
    if (in_dtype == DT_BF16) { BGF_HN(DT_BF16) }
    BGF_HN(DT_F32)
#undef BGF_HN
}

hipError_t launch_segment(const SegArgs& a, int in_dtype, int hn, int elem, int sc, int rnd, int br,
                          int bc, int pass, hipStream_t s) {
    SegBatch b{};
    b.t[0] = a;
    b.n = 1;
    return launch_batch(b, in_dtype, hn, elem, sc, rnd, br, bc, pass, s);
}

hipError_t launch_segment_batch(const SegArgs* items, int n, int in_dtype, int hn, int elem, int sc, int rnd,
                                int br, int bc, hipStream_t s) {
    if (n < 1 || n > kMaxBatch) return hipErrorInvalidValue;
    SegBatch b{};
    for (int i = 0; i < n; ++i) b.t[i] = items[i];
    b.n = n;
    return launch_batch(b, in_dtype, hn, elem, sc, rnd, br, bc, PASS_QUANT, s);
}

hipError_t launch_zero_u32(uint32_t* p, int n, hipStream_t stream) {
    hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(64), 0, stream, p, n);
    return hipGetLastError();
}

hipError_t launch_amax_rows(const void* x, int in_dtype, int64_t rows, int64_t cols, int64_t ldx,
                            uint32_t* ws, hipStream_t stream) {
    // one atomic max per workgroup on one word: more than ~512 workgroups only add contention
    const int64_t grid = rows < 512 ? rows : 512;
    if (in_dtype == DT_BF16) BGF_LAUNCH(k_amax_rows<DT_BF16>, grid, x, rows, cols, ldx, ws);
    BGF_LAUNCH(k_amax_rows<DT_F32>, grid, x, rows, cols, ldx, ws);
}

hipError_t launch_rowblock(const RowArgs& a, int in_dtype, int elem, int sc, int rnd,
                           hipStream_t stream) {
#define BGF_RBK(IN)                                                                        \
    do {                                                                                   \
        if (elem == ELEM_E2M1) {                                                           \
            if (sc == SC_E8M0) {                                                           \
                if (rnd == RND_SR) BGF_LAUNCH((k_rowblock<IN, ELEM_E2M1, SC_E8M0, RND_SR>), a.rows, a); \
                BGF_LAUNCH((k_rowblock<IN, ELEM_E2M1, SC_E8M0, RND_RNE>), a.rows, a);     \
            }                                                                              \
            if (rnd == RND_SR) BGF_LAUNCH((k_rowblock<IN, ELEM_E2M1, SC_F32, RND_SR>), a.rows, a); \
            BGF_LAUNCH((k_rowblock<IN, ELEM_E2M1, SC_F32, RND_RNE>), a.rows, a);          \
        }                                                                                  \
        if (sc == SC_E8M0) {                                                               \
            if (rnd == RND_SR) BGF_LAUNCH((k_rowblock<IN, ELEM_E4M3, SC_E8M0, RND_SR>), a.rows, a); \
            BGF_LAUNCH((k_rowblock<IN, ELEM_E4M3, SC_E8M0, RND_RNE>), a.rows, a);         \
        }                                                                                  \
        if (rnd == RND_SR) BGF_LAUNCH((k_rowblock<IN, ELEM_E4M3, SC_F32, RND_SR>), a.rows, a); \
        BGF_LAUNCH((k_rowblock<IN, ELEM_E4M3, SC_F32, RND_RNE>), a.rows, a);              \
    } while (0)
    if (in_dtype == DT_BF16) BGF_RBK(DT_BF16);
    BGF_RBK(DT_F32);
#undef BGF_RBK
}

template <int ELEM, int SC, int BR, int BC, int OUT>
static hipError_t dq_hn(const DeqArgs& a, int hn, hipStream_t stream) {
    const int64_t grid = (a.nseg + kThreads - 1) / kThreads;
    switch (hn) {
        case 0: BGF_LAUNCH((k_dequant_segment<ELEM, SC, 0, BR, BC, OUT>), grid, a);
        case 16: BGF_LAUNCH((k_dequant_segment<ELEM, SC, 16, BR, BC, OUT>), grid, a);
        case 32: BGF_LAUNCH((k_dequant_segment<ELEM, SC, 32, BR, BC, OUT>), grid, a);
        case 64: BGF_LAUNCH((k_dequant_segment<ELEM, SC, 64, BR, BC, OUT>), grid, a);
        case 128: BGF_LAUNCH((k_dequant_segment<ELEM, SC, 128, BR, BC, OUT>), grid, a);
        case 256: BGF_LAUNCH((k_dequant_segment<ELEM, SC, 256, BR, BC, OUT>), grid, a);
        default: return hipErrorInvalidValue;
    }
}

template <int OUT>
static hipError_t dq_out(const DeqArgs& a, int elem, int sc, int br, int bc, int hn, hipStream_t s) {
    if (sc == SC_NV) return dq_hn<ELEM_E2M1, SC_NV, 1, 16, OUT>(a, hn, s);
    if (elem == ELEM_E2M1) {
        if (sc == SC_F32) {
            if (bc == 32) return dq_hn<ELEM_E2M1, SC_F32, 1, 32, OUT>(a, hn, s);
            return dq_hn<ELEM_E2M1, SC_F32, 1, 16, OUT>(a, hn, s);
        }
        if (br == 32) return dq_hn<ELEM_E2M1, SC_E8M0, 32, 32, OUT>(a, hn, s);
        if (bc == 32) return dq_hn<ELEM_E2M1, SC_E8M0, 1, 32, OUT>(a, hn, s);
        return dq_hn<ELEM_E2M1, SC_E8M0, 1, 16, OUT>(a, hn, s);
    }
    if (sc == SC_F32) {
        if (bc == 32) return dq_hn<ELEM_E4M3, SC_F32, 1, 32, OUT>(a, hn, s);
        return dq_hn<ELEM_E4M3, SC_F32, 1, 16, OUT>(a, hn, s);
    }
    if (br == 32) return dq_hn<ELEM_E4M3, SC_E8M0, 32, 32, OUT>(a, hn, s);
    if (bc == 32) return dq_hn<ELEM_E4M3, SC_E8M0, 1, 32, OUT>(a, hn, s);
    return dq_hn<ELEM_E4M3, SC_E8M0, 1, 16, OUT>(a, hn, s);
}

hipError_t launch_dequant_segment(const DeqArgs& a, int elem, int sc, int br, int bc, int hn,
                                  int out_dtype, hipStream_t s) {
    if (out_dtype == DT_BF16) return dq_out<DT_BF16>(a, elem, sc, br, bc, hn, s);
    return dq_out<DT_F32>(a, elem, sc, br, bc, hn, s);
}

hipError_t launch_dequant_rowblock(const DeqArgs& a, int elem, int sc, int out_dtype,
                                   hipStream_t stream) {
    const int64_t grid = a.rows;
#define BGF_DQR(OUT)                                                                       \
    do {                                                                                   \
        if (elem == ELEM_E2M1) {                                                           \
            if (sc == SC_F32) BGF_LAUNCH((k_dequant_rowblock<ELEM_E2M1, SC_F32, OUT>), grid, a); \
            BGF_LAUNCH((k_dequant_rowblock<ELEM_E2M1, SC_E8M0, OUT>), grid, a);           \
        }                                                                                  \
        if (sc == SC_F32) BGF_LAUNCH((k_dequant_rowblock<ELEM_E4M3, SC_F32, OUT>), grid, a); \
        BGF_LAUNCH((k_dequant_rowblock<ELEM_E4M3, SC_E8M0, OUT>), grid, a);               \
    } while (0)
    if (out_dtype == DT_BF16) BGF_DQR(DT_BF16);
    BGF_DQR(DT_F32);
#undef BGF_DQR
}

}  // namespace bgf
