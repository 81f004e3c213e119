// Block-scaled GEMM C = A * B^T on gfx950's scaled matrix instructions (V_MFMA_SCALE_F32_*_F8F6F4).
//
// Operands are K-contiguous: A [M, K] and B [N, K] as packed E2M1 (2 per byte) or E4M3 bytes,
// with one E8M0 scale per row and 32-wide K group (B may instead carry one scale per 32 x 32
// tile). The matrix core applies both scales itself, so the main loop is loads + MFMA only.
// Three kernels: k_gemm_big (256 x 256 tiles, 32x32x64 MFMA, operands copied straight into LDS; the
// path for M, N >= 256 and K a multiple of its stage depth), k_gemm_mid (the same with 128 x 128
// tiles, two workgroups per CU, where M or N is below 256 or 256 x 256 tiles would fill at most
// half the CUs; k_gemm_mid_q with the fused output quantize) and k_gemm below (128 x 128 tiles, 16x16x128 MFMA, operands
// staged through registers; every other shape, K any multiple of 32).
//
// Lane layouts of the 16x16x128 scaled MFMA (established with one-hot probes on the hardware):
//  - FP4: lane l supplies row l % 16 and the 32 K values [32 (l / 16), +32) as 16 contiguous
//    bytes; FP8: the same row, K values [16 (l / 16), +16) and [64 + 16 (l / 16), +16) as two
//    16-byte pieces. In both, lane l's scale byte belongs to row l % 16, K group l / 16.
//  - result: lane l holds D[4 (l / 16) + i][l % 16], i = 0..3, for D = opA * opB^T.
// The kernel feeds B tiles as opA and A tiles as opB, so each lane ends up with 4 consecutive
// columns n of one output row m and writes them with one vector store.
//
// Tiling: a 256-thread workgroup computes a 128 x 128 block of C; its 4 waves each own a 64 x 64
// quadrant (4 x 4 MFMA tiles, 64 accumulator registers). Each 128-deep K step stages the A and B
// slabs (64 B or 128 B per row, rows padded by 16 B so that the 16-byte fragment reads of
// consecutive rows fall in different LDS banks) and the scale dwords through LDS; the next step's
// global loads are issued before the current step's MFMAs.
//
// NVFP4 operands (16-element blocks with E4M3 scales and an fp32 tensor scale) are first
// re-expressed as E4M3 elements with one power-of-two scale per 32-wide K group, the form the
// matrix core takes: per group, with S the larger of its two block scales, E is the smallest
// exponent with 448 * 2^E >= 6 S and every element becomes E4M3(val(q) * s_blk * 2^-E) (nearest
// even). The MXFP8 product is then scaled by RN(g_A * g_B) in the epilogue.
#include <atomic>
#include <type_traits>

#include "device.h"
#include "fp4_internal.h"
#include "quant_block.h"
#include "segment.h"

namespace bgf {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 128, NT = 256;

template <bool FP8>
struct Cfg {
    static constexpr int RB = FP8 ? 128 : 64;      // bytes per row per K step
    static constexpr int LD = RB + 16;             // padded LDS row pitch
    static constexpr int CH = RB / 16;             // 16-byte chunks per row
    static constexpr int LOADS = BM * CH / NT;     // 16-byte loads per thread per operand
};

// The four E8M0 scale bytes of K groups 4 kt .. 4 kt + 3 in one row of a scale matrix with kgroups
// columns: one dword load when kgroups % 4 == 0 (the row starts stay 4-byte aligned), else single
// bytes, with groups past the row as code 0 (their elements are zero, so the products are too).
__device__ __forceinline__ uint32_t scale_dword(const uint8_t* row, int64_t kgroups, int kt) {
    const int64_t g0 = 4 * (int64_t)kt;
    if (!(kgroups & 3)) return *reinterpret_cast<const uint32_t*>(row + g0);
    uint32_t v = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (g0 + j < kgroups) v |= (uint32_t)row[g0 + j] << (8 * j);
    return v;
}

// One K step's global loads of the 128 x 128 kernel: LOADS 16-byte pieces of A and of B per
// thread (rows beyond M / N and pieces beyond K read as zero: K % 32 == 0 keeps each piece wholly
// inside or outside a row) and one scale dword (threads < 128: A's rows, else B's).
template <bool FP8, bool B2D>
__device__ __forceinline__ void small_gload(const uint8_t* a, const uint8_t* b, const uint8_t* sa, const uint8_t* sb,
                                            int64_t M, int64_t N, int64_t m0, int64_t n0, int64_t rowbytes,
                                            int64_t kgroups, int kt, int tid, u32x4 (&ra)[Cfg<FP8>::LOADS],
                                            u32x4 (&rb)[Cfg<FP8>::LOADS], uint32_t& rsa, uint32_t& rsb) {
    using C = Cfg<FP8>;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
        const int ch = tid + NT * i, r = ch / C::CH, c = ch % C::CH;
        const int64_t m = m0 + r, n = n0 + r;
        const int64_t off = (int64_t)kt * C::RB + 16 * c;
        const bool kin = off < rowbytes;
        ra[i] = m < M && kin ? *reinterpret_cast<const u32x4*>(a + m * rowbytes + off) : (u32x4){0u, 0u, 0u, 0u};
        rb[i] = n < N && kin ? *reinterpret_cast<const u32x4*>(b + n * rowbytes + off) : (u32x4){0u, 0u, 0u, 0u};
    }
    if (tid < BM) {
        const int64_t m = m0 + tid;
        rsa = m < M ? scale_dword(sa + m * kgroups, kgroups, kt) : 0u;
    } else {
        const int64_t n = n0 + (tid - BM);
        const int64_t srow = B2D ? (n >> 5) : n;
        rsb = n < N ? scale_dword(sb + srow * kgroups, kgroups, kt) : 0u;
    }
}

// ---------------------------------------------------------------------------------------------
// Fused output quantization ("online quantization" of the GEMM output in the QuTLASS kernel list
// of the Quartet lecture notes), in both kernels' epilogues: C, as the fp32 values the plain output
// path would store (accumulator times the NVFP4 tensor-scale product), optionally rotated along N
// by the blockwise H_n / sqrt(n) (n <= 128), quantized along N in MX groups of 32 with the rules of
// the quantize kernels: E8M0 floor or ceil scale from the group amax, E2M1 or E4M3 elements, round
// to nearest even or stochastic rounding keyed by the row-major index m * N + n of C. Codes are
// [M, N/2] (E2M1) or [M, N] (E4M3) bytes, scales [M, N/32]. The C tile is staged in LDS so that
// one lane holds one group and the groups of a row sit in consecutive lanes.
// ---------------------------------------------------------------------------------------------
// FQ: fused output quantize, 0 none, FQ_RNE or FQ_SR (a template argument, so that the nearest-even
// variant carries no stochastic-rounding registers)
constexpr int FQ_NONE = 0, FQ_RNE = 1, FQ_SR = 2;

template <bool FP8, bool B2D, int OUT, bool NVG, int FQ>
__global__ __launch_bounds__(NT) void k_gemm(GemmArgs g) {
    using C = Cfg<FP8>;
    // operand slabs; the fused output quantize reuses them to stage 32 rows of C at a time
    __shared__ __attribute__((aligned(16))) uint8_t sAB[(BM + BN) * C::LD];
    uint8_t* const sA = sAB;
    uint8_t* const sB = sAB + BM * C::LD;
    __shared__ uint32_t sSA[BM], sSB[BN];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
    const int64_t rowbytes = FP8 ? g.K : g.K / 2;
    const int64_t kgroups = g.K / 32;
    const int KT = (int)((g.K + BK - 1) / BK);  // the last step may be partly past K

    u32x4 ra[C::LOADS], rb[C::LOADS];
    uint32_t rsa = 0, rsb = 0;

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};

    const int fr = lane & 15, fg = lane >> 4;
    const uint8_t *const ga = g.a, *const gb = g.b, *const gsa = g.sa, *const gsb = g.sb;
    const int64_t M = g.M, N = g.N;
    small_gload<FP8, B2D>(ga, gb, gsa, gsb, M, N, m0, n0, rowbytes, kgroups, 0, tid, ra, rb, rsa, rsb);
    for (int kt = 0; kt < KT; ++kt) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < C::LOADS; ++i) {
            const int ch = tid + NT * i, r = ch / C::CH, c = ch % C::CH;
            *reinterpret_cast<u32x4*>(sA + r * C::LD + 16 * c) = ra[i];
            *reinterpret_cast<u32x4*>(sB + r * C::LD + 16 * c) = rb[i];
        }
        if (tid < BM) sSA[tid] = rsa;
        else sSB[tid - BM] = rsb;
        __syncthreads();
        if (kt + 1 < KT) small_gload<FP8, B2D>(ga, gb, gsa, gsb, M, N, m0, n0, rowbytes, kgroups, kt + 1, tid, ra, rb, rsa, rsb);

        v8i fa[4], fb[4];
        int sa_[4], sb_[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ra_ = wm * 64 + 16 * i + fr;  // A tile row (output m)
            const int rb_ = wn * 64 + 16 * i + fr;  // B tile row (output n)
            if constexpr (!FP8) {
                const u32x4 xa = *reinterpret_cast<const u32x4*>(sA + ra_ * C::LD + 16 * fg);
                const u32x4 xb = *reinterpret_cast<const u32x4*>(sB + rb_ * C::LD + 16 * fg);
                fa[i] = (v8i){(int)xa[0], (int)xa[1], (int)xa[2], (int)xa[3], 0, 0, 0, 0};
                fb[i] = (v8i){(int)xb[0], (int)xb[1], (int)xb[2], (int)xb[3], 0, 0, 0, 0};
            } else {
                const u32x4 xa0 = *reinterpret_cast<const u32x4*>(sA + ra_ * C::LD + 16 * fg);
                const u32x4 xa1 = *reinterpret_cast<const u32x4*>(sA + ra_ * C::LD + 64 + 16 * fg);
                const u32x4 xb0 = *reinterpret_cast<const u32x4*>(sB + rb_ * C::LD + 16 * fg);
                const u32x4 xb1 = *reinterpret_cast<const u32x4*>(sB + rb_ * C::LD + 64 + 16 * fg);
                fa[i] = (v8i){(int)xa0[0], (int)xa0[1], (int)xa0[2], (int)xa0[3],
                              (int)xa1[0], (int)xa1[1], (int)xa1[2], (int)xa1[3]};
                fb[i] = (v8i){(int)xb0[0], (int)xb0[1], (int)xb0[2], (int)xb0[3],
                              (int)xb1[0], (int)xb1[1], (int)xb1[2], (int)xb1[3]};
            }
            sa_[i] = (int)((sSA[ra_] >> (8 * fg)) & 0xFFu);
            sb_[i] = (int)((sSB[rb_] >> (8 * fg)) & 0xFFu);
        }
#pragma unroll
        for (int in = 0; in < 4; ++in)
#pragma unroll
            for (int im = 0; im < 4; ++im)
                acc[in][im] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    fb[in], fa[im], acc[in][im], FP8 ? 0 : 4, FP8 ? 0 : 4, 0, sb_[in], 0, sa_[im]);
    }

    // epilogue: lane holds C[m][n .. n+3]
    float gscale = 1.0f;
    if constexpr (NVG) gscale = (*g.ga) * (*g.gb);
    if constexpr (FQ != FQ_NONE) {
        // fused output quantization (the rules of the big kernel's epilogue): four rounds of 32
        // rows; the two waves holding a round's rows stage their fp32 values in LDS, then one
        // thread per 32-column group (the four groups of a row in consecutive lanes) reads its
        // group back, rotates it along N if asked and quantizes it
        constexpr int EQ = 528;  // staged row pitch: 128 fp32 + 16 bytes of padding
        static_assert(32 * EQ <= (BM + BN) * C::LD, "staging exceeds the operand slabs");
        for (int rr = 0; rr < 4; ++rr) {
            __syncthreads();  // the slabs are free (main loop / previous round done)
            if (wm == (rr >> 1)) {  // wave-uniform
#pragma unroll
                for (int im = 0; im < 4; ++im) {
                    if ((im >> 1) != (rr & 1)) continue;
                    const int row = 16 * (im & 1) + fr;
#pragma unroll
                    for (int in = 0; in < 4; ++in) {
                        f32x4 v;
#pragma unroll
                        for (int i = 0; i < 4; ++i) v[i] = NVG ? acc[in][im][i] * gscale : acc[in][im][i];
                        *reinterpret_cast<f32x4*>(sAB + row * EQ + 4 * (wn * 64 + 16 * in + 4 * fg)) = v;
                    }
                }
            }
            __syncthreads();
            if (tid < 128) {  // waves 0 and 1, every lane
                const int r = tid >> 2, j = tid & 3;
                const int64_t m = m0 + 32 * rr + r, nb = n0 + 32 * j;
                float v[32];
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const f32x4 x = *reinterpret_cast<const f32x4*>(sAB + r * EQ + 4 * (32 * j + 4 * c));
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[4 * c + i] = x[i];
                }
                fwht_groups(v, g.q_hn);
                uint32_t out[8];
                const float amax = block_amax<32, 0>(v);
                uint32_t sbyte;
                const SrSource sr{g.q_seed, (uint64_t)(m * g.N + nb)};
                if constexpr (FQ == FQ_SR) {
                    sbyte = g.q_elem == ELEM_E2M1 ? e8m0_block<ELEM_E2M1, RND_SR, 32, 0>(v, amax, g.q_ceil != 0, sr, out)
                                                  : e8m0_block<ELEM_E4M3, RND_SR, 32, 0>(v, amax, g.q_ceil != 0, sr, out);
                } else {
                    sbyte = g.q_elem == ELEM_E2M1 ? e8m0_block<ELEM_E2M1, RND_RNE, 32, 0>(v, amax, g.q_ceil != 0, sr, out)
                                                  : e8m0_block<ELEM_E4M3, RND_RNE, 32, 0>(v, amax, g.q_ceil != 0, sr, out);
                }
                if (m < g.M && nb < g.N) {
                    if (g.q_elem == ELEM_E2M1) {
                        *reinterpret_cast<u32x4*>(g.qcodes + m * (g.N / 2) + nb / 2) = (u32x4){out[0], out[1], out[2], out[3]};
                    } else {
                        u32x4* d = reinterpret_cast<u32x4*>(g.qcodes + m * g.N + nb);
                        d[0] = (u32x4){out[0], out[1], out[2], out[3]};
                        d[1] = (u32x4){out[4], out[5], out[6], out[7]};
                    }
                    g.qscales[m * (g.N / 32) + nb / 32] = (uint8_t)sbyte;
                }
            }
        }
        if (!g.c) return;
    }
#pragma unroll
    for (int in = 0; in < 4; ++in)
#pragma unroll
        for (int im = 0; im < 4; ++im) {
            const int64_t m = m0 + wm * 64 + 16 * im + fr;
            const int64_t n = n0 + wn * 64 + 16 * in + 4 * fg;
            if (m >= g.M) continue;
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = NVG ? acc[in][im][i] * gscale : acc[in][im][i];
            if constexpr (OUT == DT_F32) {
                float* cp = reinterpret_cast<float*>(g.c) + m * g.ldc + n;
                if (n + 3 < g.N && ((g.ldc & 3) == 0)) {
                    *reinterpret_cast<f32x4*>(cp) = (f32x4){v[0], v[1], v[2], v[3]};
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (n + i < g.N) cp[i] = v[i];
                }
            } else {
                uint16_t* cp = reinterpret_cast<uint16_t*>(g.c) + m * g.ldc + n;
                const uint32_t w0 = pack_bf16x2_rne(v[0], v[1]);
                const uint32_t w1 = pack_bf16x2_rne(v[2], v[3]);
                if (n + 3 < g.N && ((g.ldc & 3) == 0)) {
                    *reinterpret_cast<u32x2*>(cp) = (u32x2){w0, w1};
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (n + i < g.N) cp[i] = (uint16_t)pack_bf16x2_rne(v[i], 0.0f);
                }
            }
        }
}

// ---------------------------------------------------------------------------------------------
// Large-tile pipelined kernel: 256 x 256 workgroup tile, 8 waves (two per SIMD, so one wave's
// waits are covered by the other's matrix work), each wave a 128 x 64 quadrant of 4 x 2 tiles of
// the 32x32x64 scaled MFMA (lane l: row l % 32, 32 K values of group l / 32 of the instruction's
// 64; result lane l, register i: D[8 (i / 4) + 4 (l / 32) + i % 4][l % 32]).
// A multi-stage LDS ring is filled by direct global->LDS 128-bit loads (no VGPR staging): each
// wave writes 1 KB contiguous blocks, so a row's 16-byte chunks are placed by choosing which
// chunk each lane fetches. The chunk slot is XOR-swizzled with bits of the row so that the
// 16-byte fragment reads of consecutive rows hit distinct LDS banks (for 32 and 64 banks).
// Scales: one dword (4 K groups) per row per 128-deep step, shifted per lane so that a fixed
// OPSEL byte selects the lane's group.
// Workgroups are renumbered so that each of the 8 XCDs (which receive workgroup ids round-robin)
// owns a contiguous run of tiles, walked in groups of 4 tile rows for L2 reuse.
// ---------------------------------------------------------------------------------------------
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// TS = 256: 8 waves of 128 x 64 (one workgroup per CU: two 68 KB stages); TS = 128: 4 waves of
// 64 x 64 (two workgroups per CU: two 34 KB stages each), for grids of 256 x 256 tiles that would
// leave most CUs idle.
template <bool FP8, int TS = 256>
struct Big {
    static constexpr int TM = TS, TN = TS, NW = TS == 256 ? 8 : 4, NTH = 64 * NW;
    static constexpr int WTM = TS == 256 ? 4 : 2, WTN = 2;  // 32x32 tiles per wave (M x N)
    static constexpr int WN = TN / (32 * WTN);        // waves along N
    // One stage covers 128 bytes of every row (full 128-byte cache lines): 256 K values of FP4
    // or 128 of FP8.
    static constexpr int KSTEP = FP8 ? 128 : 256;
    static constexpr int RB = 128;                    // bytes per row per stage
    static constexpr int CPR = RB / 16;               // 16-byte chunks per row
    static constexpr int NKK = KSTEP / 64;            // 64-deep MFMA steps per stage
    static constexpr int SPR = KSTEP / 32;            // scale bytes per row per stage
    static constexpr int NST = 2;                     // pipeline stages
    static constexpr int OPB = TM * RB;               // operand bytes per stage
    static constexpr int SB = TM * SPR;               // scale bytes per operand per stage
    // stage layout: A's scales, B's scales, A's codes, B's codes (scales first, so that the
    // scale reads of a stage reach every tile with one base register and 16-bit offsets)
    static constexpr int OFF_SB = SB, OFF_A = 2 * SB, OFF_B = 2 * SB + OPB;
    static constexpr int STAGE = 2 * OPB + 2 * SB;
    static constexpr int IPW = OPB / 1024 / NW;       // 1 KB code loads per wave per operand
    static constexpr int SPW = 2 * SB / 256 / NW;     // 256 B scale loads per wave (both operands)
    static constexpr int LOADS = 2 * IPW + SPW;       // vector-memory instructions per thread per stage
};

// 16-byte chunk slot of chunk c in row r: c ^ swz(r), distinct over any 8 consecutive rows and over
// any 8 rows of equal parity (conflict-free 16-byte fragment reads for 32 or 64 LDS banks)
__device__ __forceinline__ int chunk_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }


// s_waitcnt with vmcnt = N (gfx9 encoding: vmcnt bits [3:0] and [15:14]); expcnt and lgkmcnt at
// their maximum, i.e. not waited for
template <int N>
__device__ __forceinline__ void wait_vm() {
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier without the memory fence of __syncthreads (which waits for every outstanding
// vector-memory operation, including the next stage's prefetch). The empty asm statements keep
// the compiler from moving LDS or memory accesses across it; the caller waits for what must have
// completed.
__device__ __forceinline__ void barrier_only() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// s_waitcnt lgkmcnt(0): this wave's LDS reads and writes have completed
__device__ __forceinline__ void wait_lgkm0() {
    __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));
}

// ---------------------------------------------------------------------------------------------
// NVFP4 -> MXFP8 re-expression of one 32-wide K group of a row: q holds its 32 E2M1 codes (element
// k in nibble k % 8 of word k / 8), s01 its two E4M3 block scales (byte 0: elements 0-15). With S
// the larger block scale, E is the smallest exponent with 448 * 2^E >= 6 S, and every element
// becomes E4M3(val(q) * s_blk * 2^-E): val(q) * s_blk is exact in fp32 and the scaled convert
// divides it by 2^E exactly before rounding to nearest even. o: 32 E4M3 bytes in element order.
// Returns the E8M0 code E + 127 (E = -127 for S = 0, every element then 0).
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t nv_group_to_fp8(const u32x4 q, uint32_t s01, uint32_t (&o)[8]) {
    const float s0 = e4m3_value(s01 & 0x7Fu), s1 = e4m3_value((s01 >> 8) & 0x7Fu);
    const float S = fmaxf(s0, s1);
    // E = smallest exponent with 448 * 2^E >= 6 S (6 S is exact in fp32)
    const int E = e8m0_exp<8, 0x600000u>(6.0f * S, true);
    const float sc = E > -127 ? pow2f(E) : 1.0f;  // S = 0: every product is 0
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float sb = w < 2 ? s0 : s1;
        const v2f p0 = fp4x2_to_f32<0>(q[w]), p1 = fp4x2_to_f32<1>(q[w]);
        const v2f p2 = fp4x2_to_f32<2>(q[w]), p3 = fp4x2_to_f32<3>(q[w]);
        uint32_t r0 = 0u, r1 = 0u;
        r0 = cvt_fp8x2<false>(r0, p0[0] * sb, p0[1] * sb, sc);
        r0 = cvt_fp8x2<true>(r0, p1[0] * sb, p1[1] * sb, sc);
        r1 = cvt_fp8x2<false>(r1, p2[0] * sb, p2[1] * sb, sc);
        r1 = cvt_fp8x2<true>(r1, p3[0] * sb, p3[1] * sb, sc);
        o[2 * w] = r0;
        o[2 * w + 1] = r1;
    }
    return (uint32_t)(E + 127);
}

// Tile coordinates of work item b (a workgroup index of the one-tile-per-workgroup launch): the
// workgroups of each of the 8 XCDs (which receive ids round-robin) own a contiguous run of tiles,
// walked in groups of 4 tile rows for L2 reuse.
__device__ __forceinline__ void big_tile_coords(int b, int ntm, int ntn, int& tm, int& tn) {
    const int T = ntm * ntn;
    if (T % 8 == 0) b = (b % 8) * (T / 8) + b / 8;
    const int GM = 4;
    const int grp = b / (GM * ntn), first = grp * GM;
    const int gs = (ntm - first) < GM ? (ntm - first) : GM;
    tm = first + (b % (GM * ntn)) % gs;
    tn = (b % (GM * ntn)) / gs;
}

// Epilogue of a TS x TS tile: the accumulators (lane layout of the 32x32x64 MFMA tiles of
// big_tile) to C, and to C_q when FQ; uses the first TS * 528 bytes of `smem`, which
// must be free (no copy into it still in flight). Every thread of the workgroup must call it.
template <bool FP8, int OUT, bool NVG, int FQ, int TS = 256>
__device__ __forceinline__ void big_epilogue(const GemmArgs& g, v16f (&acc)[Big<FP8, TS>::WTN][Big<FP8, TS>::WTM],
                                             int64_t m0, int64_t n0, uint8_t* smem) {
    using C = Big<FP8, TS>;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int fr = lane & 31, fg = lane >> 5;
    // Epilogue, staged through LDS so that every global store writes whole 16-byte pieces of a
    // row and consecutive lanes cover consecutive bytes. Lane (fr, fg) holds, for 4-register group
    // q of tile (im, in), C[m][n .. n+3] with m = wm*128 + 32 im + fr and
    // n = wn*64 + 32 in + 8 q + 4 fg. A pass stages 256 rows x 512 bytes: bf16 output in one pass
    // (all 256 columns), fp32 output in two (pass p holds columns wn*64 + 32 p + [0, 32) of each
    // wave column wn, i.e. four 128-byte runs per row).
    constexpr int EP = 528;                       // staged row pitch (512 B + 16 B of padding)
    static_assert(TS == 128 || 256 * EP <= C::NST * C::STAGE, "staging buffer exceeds the stage buffers");
    constexpr int PASSES = OUT == DT_F32 ? 2 : 1;
    float gscale = 1.0f;
    if constexpr (NVG) gscale = (*g.ga) * (*g.gb);
    // an opaque zero keeps the compiler from computing the output addresses before the main
    // loop, where they would only add register pressure
    int opaque_zero;
    asm volatile("s_mov_b32 %0, 0" : "=s"(opaque_zero));
    const int64_t me0 = m0 + opaque_zero, ne0 = n0 + opaque_zero, ldc = g.ldc + opaque_zero;
    char* const cbase = reinterpret_cast<char*>(g.c) + opaque_zero;
    const int64_t Mx = g.M + opaque_zero, Nx = g.N + opaque_zero;
    if constexpr (TS == 128 && FQ == FQ_NONE) {
        // 128 x 128 tile, plain output: one pass stages all 128 rows (128 fp32 or bf16 values per
        // row), then each row goes out as 16 (bf16) or 32 (fp32) 16-byte pieces
        static_assert(128 * EP <= C::NST * C::STAGE, "staging buffer exceeds the stage buffers");
        constexpr int ESZ = OUT == DT_F32 ? 4 : 2;
        const bool vec_ok = ((reinterpret_cast<uintptr_t>(g.c) & 15) == 0) && ((ldc * ESZ) % 16 == 0);
        barrier_only();  // every wave is done reading the stage buffers
#pragma unroll
        for (int im = 0; im < C::WTM; ++im)
#pragma unroll
            for (int in = 0; in < C::WTN; ++in) {
                const int row = wm * 32 * C::WTM + 32 * im + fr;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float v[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = NVG ? acc[in][im][4 * q + i] * gscale : acc[in][im][4 * q + i];
                    const int col = wn * 32 * C::WTN + 32 * in + 8 * q + 4 * fg;
                    if constexpr (OUT == DT_F32) {
                        *reinterpret_cast<f32x4*>(smem + row * EP + 4 * col) = (f32x4){v[0], v[1], v[2], v[3]};
                    } else {
                        *reinterpret_cast<u32x2*>(smem + row * EP + 2 * col) =
                            (u32x2){pack_bf16x2_rne(v[0], v[1]), pack_bf16x2_rne(v[2], v[3])};
                    }
                }
            }
        wait_lgkm0();
        barrier_only();
        constexpr int EPC = 16 / ESZ;     // elements per 16-byte piece
        constexpr int PPR = C::TN / EPC;  // pieces per row
        const int c16 = tid % PPR;
        const int64_t n = ne0 + EPC * c16;
#pragma unroll 4
        for (int r = tid / PPR; r < C::TM; r += C::NTH / PPR) {
            const int64_t m = me0 + r;
            if (m >= Mx) break;
            const u32x4 val = *reinterpret_cast<const u32x4*>(smem + r * EP + 16 * c16);
            char* cp = cbase + (m * ldc + n) * ESZ;
            if (vec_ok && n + EPC <= Nx) {
                *reinterpret_cast<u32x4*>(cp) = val;
            } else {
#pragma unroll
                for (int i = 0; i < EPC; ++i) {
                    if (n + i < Nx) {
                        if constexpr (OUT == DT_F32)
                            reinterpret_cast<uint32_t*>(cp)[i] = val[i];
                        else
                            reinterpret_cast<uint16_t*>(cp)[i] = (uint16_t)(val[i >> 1] >> (16 * (i & 1)));
                    }
                }
            }
        }
        return;
    }
    if constexpr (FQ != FQ_NONE) {
        // fused output quantization, in passes of 128 columns (two for 256 x 256 tiles, one for
        // 128 x 128): the fp32 values (as an fp32 C would hold them) are staged in LDS, [TS rows][128]
        // per pass (pass p holds tile columns [128 p, 128 p + 128), written by the waves whose 64
        // columns lie there), then one thread per 32-column group reads its group back, rotates it
        // along N if asked (the four groups of a row are in consecutive lanes) and quantizes it with
        // the rules of the quantize kernels
        static_assert(C::WTN == 2, "64 columns per wave");
        static_assert(C::TM * EP <= C::NST * C::STAGE, "staging buffer exceeds the stage buffers");
        for (int p = 0; p < C::TN / 128; ++p) {
            barrier_only();  // every wave is done with the stage buffers / the last pass
            if ((wn >> 1) == p) {  // wave-uniform
#pragma unroll
                for (int in = 0; in < C::WTN; ++in)
#pragma unroll
                    for (int im = 0; im < C::WTM; ++im) {
                        const int row = wm * 32 * C::WTM + 32 * im + fr;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            f32x4 v;
#pragma unroll
                            for (int i = 0; i < 4; ++i) v[i] = NVG ? acc[in][im][4 * q + i] * gscale : acc[in][im][4 * q + i];
                            *reinterpret_cast<f32x4*>(smem + row * EP + 4 * (64 * (wn & 1) + 32 * in + 8 * q + 4 * fg)) = v;
                        }
                    }
            }
            wait_lgkm0();
            barrier_only();
#pragma unroll 1
            for (int t = tid; t < C::TM * 4; t += C::NTH) {  // two sweeps, every lane in both
                const int r = t >> 2, j = t & 3;  // row, staged group
                const int64_t m = me0 + r, nb = ne0 + 128 * p + 32 * j;
                float v[32];
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const f32x4 x = *reinterpret_cast<const f32x4*>(smem + r * EP + 4 * (32 * j + 4 * c));
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[4 * c + i] = x[i];
                }
                fwht_groups(v, g.q_hn);
                uint32_t out[8];
                const float amax = block_amax<32, 0>(v);
                uint32_t sbyte;
                const SrSource sr{g.q_seed, (uint64_t)(m * Nx + nb)};
                if constexpr (FQ == FQ_SR) {
                    sbyte = g.q_elem == ELEM_E2M1 ? e8m0_block<ELEM_E2M1, RND_SR, 32, 0>(v, amax, g.q_ceil != 0, sr, out)
                                                  : e8m0_block<ELEM_E4M3, RND_SR, 32, 0>(v, amax, g.q_ceil != 0, sr, out);
                } else {
                    sbyte = g.q_elem == ELEM_E2M1 ? e8m0_block<ELEM_E2M1, RND_RNE, 32, 0>(v, amax, g.q_ceil != 0, sr, out)
                                                  : e8m0_block<ELEM_E4M3, RND_RNE, 32, 0>(v, amax, g.q_ceil != 0, sr, out);
                }
                if (m < Mx && nb < Nx) {
                    if (g.q_elem == ELEM_E2M1) {
                        *reinterpret_cast<u32x4*>(g.qcodes + m * (Nx / 2) + nb / 2) = (u32x4){out[0], out[1], out[2], out[3]};
                    } else {
                        u32x4* d = reinterpret_cast<u32x4*>(g.qcodes + m * Nx + nb);
                        d[0] = (u32x4){out[0], out[1], out[2], out[3]};
                        d[1] = (u32x4){out[4], out[5], out[6], out[7]};
                    }
                    g.qscales[m * (Nx / 32) + nb / 32] = (uint8_t)sbyte;
                }
            }
            if (g.c) {
                // C from the same staged values: 16-byte output pieces, staged column c of a row
                // is tile column 128 p + c
                constexpr int ESZ = OUT == DT_F32 ? 4 : 2, EPC = 16 / ESZ, PPR = 128 / EPC;
                const bool vec_ok = ((reinterpret_cast<uintptr_t>(g.c) & 15) == 0) && ((ldc * ESZ) % 16 == 0);
#pragma unroll 1
                for (int t = tid; t < C::TM * PPR; t += C::NTH) {
                    const int r = t / PPR, c = (t % PPR) * EPC;
                    const int64_t m = me0 + r, n = ne0 + 128 * p + c;
                    if (m >= Mx) continue;
                    const float* src = reinterpret_cast<const float*>(smem + r * EP) + c;
                    u32x4 val;
                    if constexpr (OUT == DT_F32) {
                        val = *reinterpret_cast<const u32x4*>(src);
                    } else {
                        const f32x4 a = *reinterpret_cast<const f32x4*>(src), b = *reinterpret_cast<const f32x4*>(src + 4);
                        val = (u32x4){pack_bf16x2_rne(a[0], a[1]), pack_bf16x2_rne(a[2], a[3]),
                                      pack_bf16x2_rne(b[0], b[1]), pack_bf16x2_rne(b[2], b[3])};
                    }
                    char* cp = cbase + (m * ldc + n) * ESZ;
                    if (vec_ok && n + EPC <= Nx) {
                        *reinterpret_cast<u32x4*>(cp) = val;
                    } else {
                        for (int i = 0; i < EPC; ++i) {
                            if (n + i < Nx) {
                                if constexpr (OUT == DT_F32)
                                    reinterpret_cast<uint32_t*>(cp)[i] = val[i];
                                else
                                    reinterpret_cast<uint16_t*>(cp)[i] = (uint16_t)(val[i >> 1] >> (16 * (i & 1)));
                            }
                        }
                    }
                }
            }
        }
        return;
    }
    constexpr int ESZ = OUT == DT_F32 ? 4 : 2;
    // 16-byte stores need a 16-byte aligned row start
    const bool vec_ok = ((reinterpret_cast<uintptr_t>(g.c) & 15) == 0) && ((ldc * ESZ) % 16 == 0);
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        barrier_only();  // every wave is done reading the stage buffers / the last pass
#pragma unroll
        for (int im = 0; im < C::WTM; ++im)
#pragma unroll
            for (int inn = 0; inn < (OUT == DT_F32 ? 1 : C::WTN); ++inn) {
                const int in = OUT == DT_F32 ? p : inn;
                const int row = wm * 128 + 32 * im + fr;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float v[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = NVG ? acc[in][im][4 * q + i] * gscale : acc[in][im][4 * q + i];
                    if constexpr (OUT == DT_F32) {
                        const int col = wn * 32 + 8 * q + 4 * fg;
                        *reinterpret_cast<f32x4*>(smem + row * EP + 4 * col) = (f32x4){v[0], v[1], v[2], v[3]};
                    } else {
                        const int col = wn * 64 + 32 * in + 8 * q + 4 * fg;
                        *reinterpret_cast<u32x2*>(smem + row * EP + 2 * col) =
                            (u32x2){pack_bf16x2_rne(v[0], v[1]), pack_bf16x2_rne(v[2], v[3])};
                    }
                }
            }
        wait_lgkm0();
        barrier_only();
        // 32 lanes per row, 16 rows per sweep of the workgroup
        const int c16 = tid & 31;
        const int64_t n = OUT == DT_F32 ? ne0 + (c16 >> 3) * 64 + 32 * p + 4 * (c16 & 7) : ne0 + 8 * c16;
        constexpr int EPC = 16 / ESZ;  // elements per 16-byte piece
#pragma unroll 4
        for (int r = tid >> 5; r < 256; r += C::NTH / 32) {
            const int64_t m = me0 + r;
            if (m >= Mx) break;
            const u32x4 val = *reinterpret_cast<const u32x4*>(smem + r * EP + 16 * c16);
            char* cp = cbase + (m * ldc + n) * ESZ;
            if (vec_ok && n + EPC <= Nx) {
                *reinterpret_cast<u32x4*>(cp) = val;
            } else {
#pragma unroll
                for (int i = 0; i < EPC; ++i) {
                    if (n + i < Nx) {
                        if constexpr (OUT == DT_F32)
                            reinterpret_cast<uint32_t*>(cp)[i] = val[i];
                        else
                            reinterpret_cast<uint16_t*>(cp)[i] = (uint16_t)(val[i >> 1] >> (16 * (i & 1)));
                    }
                }
            }
        }
    }
}

// One TS x TS tile of C (tile row tm, tile column tn) by the whole workgroup (512 threads for
// TS = 256, 256 for TS = 128), LDS `smem` of Big<FP8, TS>::NST stages; every thread must call it.
// Leaves the LDS free (every copy into it has landed) but does not end with a barrier.
template <bool FP8, bool B2D, int OUT, bool NVG, int FQ, int TS = 256>
__device__ __forceinline__ void big_tile(const GemmArgs& g, int tm, int tn, uint8_t* smem) {
    using C = Big<FP8, TS>;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int64_t m0 = (int64_t)tm * C::TM, n0 = (int64_t)tn * C::TN;

    const int64_t rowbytes = FP8 ? g.K : g.K / 2;
    const int64_t kgroups = g.K / 32;
    const int KT = (int)(g.K / C::KSTEP);

    // Direct-to-LDS copies go through buffer resources: base + 32-bit byte offset. The row part of
    // every offset sits in the per-lane (vector) offset, which the range check covers, so rows
    // beyond M or N read as zero (they only feed outputs that are never stored); the scalar offset
    // only adds the K position within a row.
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc((void*)g.a, (short)0, (int)(g.M * rowbytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc((void*)g.b, (short)0, (int)(g.N * rowbytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t rSA = __builtin_amdgcn_make_buffer_rsrc((void*)g.sa, (short)0, (int)(g.M * kgroups), 0x00020000);
    const __amdgpu_buffer_rsrc_t rSB = __builtin_amdgcn_make_buffer_rsrc(
        (void*)g.sb, (short)0, (int)((B2D ? (g.N + 31) / 32 : g.N) * kgroups), 0x00020000);
    // extent 0: every read through it is out of range and returns zeros
    const __amdgpu_buffer_rsrc_t rZ = __builtin_amdgcn_make_buffer_rsrc((void*)g.a, (short)0, 0, 0x00020000);
    // copy i of this wave fills LDS rows r = (wave * IPW + i) * 8 + lane / 8, slot lane % 8, with
    // chunk slot ^ swz(r) = slot ^ (lane / 8) ^ (i & 1) of the row (IPW is even); wave * IPW * 8 is
    // a multiple of 16, so swz(r) = (lane / 8) ^ (i & 1)
    const int r0 = wave * C::IPW * 8 + (lane >> 3);
    // (a literal bound: with the dependent C::IPW here the host pass silently drops the kernel stub)
    static_assert(C::IPW == 4, "four 1 KB copies per wave and operand");
    int voA[4], voB[4];
#pragma unroll
    for (int i = 0; i < C::IPW; ++i) {
        const int c = (lane & 7) ^ ((lane >> 3) & 7) ^ (i & 1);
        voA[i] = (int)((m0 + r0 + 8 * i) * rowbytes + 16 * c);
        voB[i] = (int)((n0 + r0 + 8 * i) * rowbytes + 16 * c);
    }
    // scale dwords: the stage holds SPR bytes of each of A's and B's 256 rows, row-major, as
    // consecutive dwords; waves take them in order, A's first
    int voS[C::SPW];
#pragma unroll
    for (int j = 0; j < C::SPW; ++j) {
        const int d = (wave * C::SPW + j) * 64 + lane;       // dword index over both operands
        const bool isb = (wave * C::SPW + j) * 64 >= C::SB / 4;
        const int dd = isb ? d - C::SB / 4 : d;
        const int r = dd / (C::SPR / 4), part = dd % (C::SPR / 4);
        if (!isb) {
            voS[j] = (int)((m0 + r) * kgroups + 4 * part);
        } else {
            const int64_t n = B2D ? ((n0 + r) >> 5) : (n0 + r);
            voS[j] = (int)(n * kgroups + 4 * part);
        }
    }

    // The copies of a stage are issued in NKK parts, one per 64-deep MFMA step of the previous
    // stage, so that no wave stalls on a full address FIFO with all its copies at once (part p:
    // A and B copies i in [p IPW / NKK, (p + 1) IPW / NKK); the scales with part 0).
    static_assert(C::IPW % C::NKK == 0, "copies per step");
    // Stage KT (one past the last) is a dummy: its copies go through the zero-extent resource, so
    // they read nothing and write zeros into the free stage buffer.
    auto issue_part = [&](int kt, int part) {
        uint8_t* st = smem + (kt % C::NST) * C::STAGE;
        const bool real = kt < KT;
        const int so = real ? kt * C::RB : 0, ss = real ? kt * C::SPR : 0;
        const __amdgpu_buffer_rsrc_t qA = real ? rA : rZ, qB = real ? rB : rZ;
        const __amdgpu_buffer_rsrc_t qSA = real ? rSA : rZ, qSB = real ? rSB : rZ;
        constexpr int IPP = C::IPW / C::NKK;
#pragma unroll
        for (int ii = 0; ii < IPP; ++ii) {
            const int i = part * IPP + ii;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(qA, (lds_ptr_t)(st + C::OFF_A + (wave * C::IPW + i) * 1024), 16,
                                                     voA[i], so, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(qB, (lds_ptr_t)(st + C::OFF_B + (wave * C::IPW + i) * 1024),
                                                     16, voB[i], so, 0, 0);
        }
        if (part != 0) return;
#pragma unroll
        for (int j = 0; j < C::SPW; ++j) {
            if ((wave * C::SPW + j) * 64 >= C::SB / 4)  // wave-uniform
                __builtin_amdgcn_raw_ptr_buffer_load_lds(qSB, (lds_ptr_t)(st + (wave * C::SPW + j) * 256),
                                                         4, voS[j], ss, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(qSA, (lds_ptr_t)(st + (wave * C::SPW + j) * 256),
                                                         4, voS[j], ss, 0, 0);
        }
    };
    auto issue = [&](int kt) {
#pragma unroll
        for (int p = 0; p < C::NKK; ++p) issue_part(kt, p);
    };

    v16f acc[C::WTN][C::WTM];
#pragma unroll
    for (int i = 0; i < C::WTN; ++i)
#pragma unroll
        for (int j = 0; j < C::WTM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // Fragment addresses: rows of tile i of this wave are wm*128 + 32 i + l%32 (A) and
    // wn*64 + 32 i + l%32 (B); their low 4 bits, hence the chunk swizzle, depend on the lane only,
    // so a tile adds the constant 32 * 128 bytes and a K step only changes the chunk term.
    const int fr = lane & 31, fg = lane >> 5;
    const int sw = chunk_swz(fr);
    constexpr int NP = FP8 ? 2 : 1;
    int ch[C::NKK][NP];
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk)
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int c = FP8 ? (4 * kk + 2 * p + fg) : (2 * kk + fg);
            ch[kk][p] = 16 * (c ^ sw);
        }
    const int aRow = C::OFF_A + (wm * 32 * C::WTM + fr) * C::RB, bRow = C::OFF_B + (wn * 32 * C::WTN + fr) * C::RB;
    const int aScl = C::SPR * (wm * 32 * C::WTM + fr), bScl = C::OFF_SB + C::SPR * (wn * 32 * C::WTN + fr);
    const int sshift = 8 * fg;

    issue(0);

    auto frag = [&](const uint8_t* p0, const uint8_t* p1) -> v8i {
        const u32x4 x0 = *reinterpret_cast<const u32x4*>(p0);
        if constexpr (!FP8) {
            return (v8i){(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], 0, 0, 0, 0};
        } else {
            const u32x4 x1 = *reinterpret_cast<const u32x4*>(p1);
            return (v8i){(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                         (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
        }
    };

    // One stage: NKK 64-deep steps. Fragments are double-buffered in registers: the reads for step
    // kk + 1 are issued while the MFMAs of step kk run, interleaved one read per MFMA.
    auto load_frags = [&](const uint8_t* st, int kk, v8i (&fa)[C::WTM], v8i (&fb)[C::WTN]) {
#pragma unroll
        for (int i = 0; i < C::WTM; ++i)
            fa[i] = frag(st + aRow + 32 * C::RB * i + ch[kk][0], st + aRow + 32 * C::RB * i + ch[kk][NP - 1]);
#pragma unroll
        for (int i = 0; i < C::WTN; ++i)
            fb[i] = frag(st + bRow + 32 * C::RB * i + ch[kk][0], st + bRow + 32 * C::RB * i + ch[kk][NP - 1]);
    };
    // one stage's MFMAs, with the copies of stage `next` issued along the way
    auto compute = [&](const uint8_t* st, int next) {
        int sa[C::WTM][C::SPR / 4], sb[C::WTN][C::SPR / 4];
#pragma unroll
        for (int i = 0; i < C::WTM; ++i)
#pragma unroll
            for (int d = 0; d < C::SPR / 4; ++d)
                sa[i][d] = (int)(*reinterpret_cast<const uint32_t*>(st + aScl + C::SPR * 32 * i + 4 * d) >> sshift);
#pragma unroll
        for (int i = 0; i < C::WTN; ++i)
#pragma unroll
            for (int d = 0; d < C::SPR / 4; ++d)
                sb[i][d] = (int)(*reinterpret_cast<const uint32_t*>(st + bScl + C::SPR * 32 * i + 4 * d) >> sshift);
        v8i fa[2][C::WTM], fb[2][C::WTN];
        load_frags(st, 0, fa[0], fb[0]);
#pragma unroll
        for (int kk = 0; kk < C::NKK; ++kk) {
            const int cur = kk & 1, nxt = cur ^ 1;
            issue_part(next, kk);
            if (kk + 1 < C::NKK) load_frags(st, kk + 1, fa[nxt], fb[nxt]);
            // scale byte of group 2 kk + (l / 32): dword kk / 2 after the lane shift, byte 2 (kk % 2)
#pragma unroll
            for (int in = 0; in < C::WTN; ++in)
#pragma unroll
                for (int im = 0; im < C::WTM; ++im) {
                    if ((kk & 1) == 0)
                        acc[in][im] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            fb[cur][in], fa[cur][im], acc[in][im], FP8 ? 0 : 4, FP8 ? 0 : 4, 0,
                            sb[in][kk >> 1], 0, sa[im][kk >> 1]);
                    else
                        acc[in][im] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            fb[cur][in], fa[cur][im], acc[in][im], FP8 ? 0 : 4, FP8 ? 0 : 4, 2,
                            sb[in][kk >> 1], 2, sa[im][kk >> 1]);
                }
            // issue this step's part of the next stage's copies, the next step's reads, then this
            // step's MFMAs; nothing moves across step boundaries
            if (kk == 0) __builtin_amdgcn_sched_group_barrier(0x020, 2 * (C::IPW / C::NKK) + C::SPW, 0);
            else __builtin_amdgcn_sched_group_barrier(0x020, 2 * (C::IPW / C::NKK), 0);
            if (kk + 1 < C::NKK) __builtin_amdgcn_sched_group_barrier(0x100, (C::WTM + C::WTN) * NP, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, C::WTM * C::WTN, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // main loop, unrolled by the stage count so every stage base is a constant
    for (int k0 = 0; k0 < KT; k0 += C::NST) {
#pragma unroll
        for (int s = 0; s < C::NST; ++s) {
            const int kt = k0 + s;
            if (kt < KT) {
                wait_vm<0>();    // this wave's copies of stage kt have landed
                barrier_only();  // ... and everyone's; stage kt-1 is no longer read
                compute(smem + s * C::STAGE, kt + 1);
            }
        }
    }
    wait_vm<0>();  // the dummy stage's zero-fill has landed before the LDS is reused

    big_epilogue<FP8, OUT, NVG, FQ, TS>(g, acc, m0, n0, smem);
}

// ---------------------------------------------------------------------------------------------
// NVFP4 x NVFP4 with the FP8 re-expression done in LDS (no pre-pass, no workspace): per 128-deep K
// stage the workgroup copies the raw E2M1 codes (64 B per row) and E4M3 block scales (8 B per row)
// of its 256 A rows and 256 B rows straight into LDS (two raw stages in a ring, 36 KB each), then
// every thread re-expresses one row's four 32-wide groups (nv_group_to_fp8, the same arithmetic as
// the pre-pass) into a single FP8 stage laid out exactly as the MXFP8 tiles' (66 KB), and the
// FP8 scaled MFMAs run on it as in big_tile. Two barriers per stage: one before the conversion (raw
// stage landed, FP8 stage free), one before the MFMAs (FP8 stage complete); the next raw stage's
// copies are in flight across both.
// ---------------------------------------------------------------------------------------------
struct NvLds {
    static constexpr int ROWS = 512;                 // A's 256 tile rows, then B's 256
    static constexpr int CB = 64;                    // E2M1 code bytes per row per stage
    static constexpr int SBY = 8;                    // E4M3 block scales per row per stage
    static constexpr int RAW_SCALES = 0, RAW_CODES = ROWS * SBY;
    static constexpr int RAW = ROWS * (CB + SBY);    // one raw stage
    static constexpr int FP8 = 2 * RAW;              // the FP8 stage, after the two raw stages
    static constexpr int LDS = FP8 + Big<true>::STAGE;
};

template <int OUT, int FQ>
__device__ __forceinline__ void nv_lds_tile(const GemmArgs& g, int tm, int tn, uint8_t* smem) {
    using C = Big<true>;
    using NL = NvLds;
    static_assert(NL::LDS <= 160 * 1024, "LDS budget");
    static_assert(256 * 528 <= NL::LDS, "epilogue staging");
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int wm = wave >> 2, wn = wave & 3;
    const int64_t m0 = (int64_t)tm * C::TM, n0 = (int64_t)tn * C::TN;
    const int64_t rowbytes = g.K / 2, sgroups = g.K / 16;
    const int KT = (int)(g.K / C::KSTEP);

    // raw copies: wave w moves rows 64 w .. 64 w + 63 of the 512 (A's for w < 4, else B's); rows past
    // M or N lie past the buffers' extents and read as zeros (their scales 0, so their FP8 values 0)
    const bool isB = wave >= 4;
    const int64_t orow0 = (isB ? n0 : m0) + 64 * (wave & 3);
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(isB ? g.b : g.a), (short)0, (int)((isB ? g.N : g.M) * rowbytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(isB ? g.sb : g.sa), (short)0, (int)((isB ? g.N : g.M) * sgroups), 0x00020000);
    // code copy i: rows 16 i + lane / 4 of the wave's 64, LDS slot lane % 4 of the row holding
    // chunk (lane % 4) ^ ((row / 4) % 4), so that a thread's reads of its row's chunks spread over
    // the banks; scale copy j: rows 32 j + lane / 2, dword lane % 2
    int voC[4], voS[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ro = 16 * i + (lane >> 2), q = (lane & 3) ^ ((lane >> 4) & 3);
        voC[i] = (int)((orow0 + ro) * rowbytes + 16 * q);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) voS[j] = (int)((orow0 + 32 * j + (lane >> 1)) * sgroups + 4 * (lane & 1));
    auto issue_raw = [&](int kt) {
        uint8_t* st = smem + (kt & 1) * NL::RAW;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, (lds_ptr_t)(st + NL::RAW_CODES + (64 * wave + 16 * i) * NL::CB),
                                                     16, voC[i], kt * NL::CB, 0, 0);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(st + NL::RAW_SCALES + (64 * wave + 32 * j) * NL::SBY),
                                                     4, voS[j], kt * NL::SBY, 0, 0);
    };
    uint8_t* const fp8 = smem + NL::FP8;
    // conversion: thread t re-expresses row t of the 512 (its four 32-wide groups)
    auto convert = [&](int kt) {
        const uint8_t* raw = smem + (kt & 1) * NL::RAW;
        const int t = tid, row = t & 255;
        const uint2 sc = *reinterpret_cast<const uint2*>(raw + NL::RAW_SCALES + t * NL::SBY);
        uint8_t* dst = fp8 + (t < 256 ? C::OFF_A : C::OFF_B) + row * C::RB;
        const int sw = chunk_swz(row);
        uint32_t e = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u32x4 q = *reinterpret_cast<const u32x4*>(raw + NL::RAW_CODES + t * NL::CB + 16 * (j ^ ((t >> 2) & 3)));
            const uint32_t s01 = ((j < 2 ? sc.x : sc.y) >> (16 * (j & 1))) & 0xFFFFu;
            uint32_t o[8];
            e |= nv_group_to_fp8(q, s01, o) << (8 * j);
            *reinterpret_cast<u32x4*>(dst + 16 * ((2 * j) ^ sw)) = (u32x4){o[0], o[1], o[2], o[3]};
            *reinterpret_cast<u32x4*>(dst + 16 * ((2 * j + 1) ^ sw)) = (u32x4){o[4], o[5], o[6], o[7]};
        }
        *reinterpret_cast<uint32_t*>(fp8 + (t < 256 ? 0 : C::OFF_SB) + row * C::SPR) = e;
    };

    v16f acc[C::WTN][C::WTM];
#pragma unroll
    for (int i = 0; i < C::WTN; ++i)
#pragma unroll
        for (int j = 0; j < C::WTM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // fragments as in big_tile (FP8: two 16-byte pieces per lane and 64-deep step)
    const int fr = lane & 31, fg = lane >> 5;
    const int sw = chunk_swz(fr);
    int ch[C::NKK][2];
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk)
#pragma unroll
        for (int p = 0; p < 2; ++p) ch[kk][p] = 16 * ((4 * kk + 2 * p + fg) ^ sw);
    const int aRow = C::OFF_A + (wm * 128 + fr) * C::RB, bRow = C::OFF_B + (wn * 64 + fr) * C::RB;
    const int aScl = C::SPR * (wm * 128 + fr), bScl = C::OFF_SB + C::SPR * (wn * 64 + fr);
    const int sshift = 8 * fg;
    auto frag = [&](const uint8_t* p0, const uint8_t* p1) -> v8i {
        const u32x4 x0 = *reinterpret_cast<const u32x4*>(p0);
        const u32x4 x1 = *reinterpret_cast<const u32x4*>(p1);
        return (v8i){(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
    };
    auto load_frags = [&](int kk, v8i (&fa)[C::WTM], v8i (&fb)[C::WTN]) {
#pragma unroll
        for (int i = 0; i < C::WTM; ++i)
            fa[i] = frag(fp8 + aRow + 32 * C::RB * i + ch[kk][0], fp8 + aRow + 32 * C::RB * i + ch[kk][1]);
#pragma unroll
        for (int i = 0; i < C::WTN; ++i)
            fb[i] = frag(fp8 + bRow + 32 * C::RB * i + ch[kk][0], fp8 + bRow + 32 * C::RB * i + ch[kk][1]);
    };
    auto compute = [&]() {
        int sa[C::WTM], sb[C::WTN];
#pragma unroll
        for (int i = 0; i < C::WTM; ++i) sa[i] = (int)(*reinterpret_cast<const uint32_t*>(fp8 + aScl + C::SPR * 32 * i) >> sshift);
#pragma unroll
        for (int i = 0; i < C::WTN; ++i) sb[i] = (int)(*reinterpret_cast<const uint32_t*>(fp8 + bScl + C::SPR * 32 * i) >> sshift);
        v8i fa[2][C::WTM], fb[2][C::WTN];
        load_frags(0, fa[0], fb[0]);
#pragma unroll
        for (int kk = 0; kk < C::NKK; ++kk) {
            const int cur = kk & 1, nxt = cur ^ 1;
            if (kk + 1 < C::NKK) load_frags(kk + 1, fa[nxt], fb[nxt]);
#pragma unroll
            for (int in = 0; in < C::WTN; ++in)
#pragma unroll
                for (int im = 0; im < C::WTM; ++im) {
                    if (kk == 0)
                        acc[in][im] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[cur][in], fa[cur][im], acc[in][im],
                                                                                      0, 0, 0, sb[in], 0, sa[im]);
                    else
                        acc[in][im] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[cur][in], fa[cur][im], acc[in][im],
                                                                                      0, 0, 2, sb[in], 2, sa[im]);
                }
        }
    };

    issue_raw(0);
    for (int kt = 0; kt < KT; ++kt) {
        wait_vm<0>();    // this wave's raw copies of stage kt have landed
        barrier_only();  // ... and everyone's; the FP8 stage and raw stage kt + 1 are free
        if (kt + 1 < KT) issue_raw(kt + 1);
        convert(kt);
        wait_lgkm0();
        barrier_only();  // the FP8 stage is complete
        compute();
    }
    wait_vm<0>();
    big_epilogue<true, OUT, true, FQ>(g, acc, m0, n0, smem);
}

template <int OUT, int FQ>
__global__ __launch_bounds__(512) void k_gemm_nv(GemmArgs g) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int ntm = (int)((g.M + 255) / 256), ntn = (int)((g.N + 255) / 256);
    int tm, tn;
    big_tile_coords(blockIdx.x, ntm, ntn, tm, tn);
    nv_lds_tile<OUT, FQ>(g, tm, tn, smem);
}

template <bool FP8, bool B2D, int OUT, bool NVG, int FQ>
__global__ __launch_bounds__(512) void k_gemm_big(GemmArgs g) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int ntm = (int)((g.M + 255) / 256), ntn = (int)((g.N + 255) / 256);
    int tm, tn;
    big_tile_coords(blockIdx.x, ntm, ntn, tm, tn);
    big_tile<FP8, B2D, OUT, NVG, FQ>(g, tm, tn, smem);
}

// 128 x 128 tiles of the same kernel, two workgroups per CU: plain output, and with the fused
// output quantize
template <bool FP8, bool B2D, int OUT, bool NVG>
__global__ __launch_bounds__(256, 2) void k_gemm_mid(GemmArgs g) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int ntm = (int)((g.M + 127) / 128), ntn = (int)((g.N + 127) / 128);
    int tm, tn;
    big_tile_coords(blockIdx.x, ntm, ntn, tm, tn);
    big_tile<FP8, B2D, OUT, NVG, FQ_NONE, 128>(g, tm, tn, smem);
}

template <bool FP8, bool B2D, int OUT, bool NVG, int FQ>
__global__ __launch_bounds__(256, 2) void k_gemm_mid_q(GemmArgs g) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int ntm = (int)((g.M + 127) / 128), ntn = (int)((g.N + 127) / 128);
    int tm, tn;
    big_tile_coords(blockIdx.x, ntm, ntn, tm, tn);
    big_tile<FP8, B2D, OUT, NVG, FQ, 128>(g, tm, tn, smem);
}

// ---------------------------------------------------------------------------------------------
// GEMM with the rotation and MX quantization of A fused in (bf16 / fp32 activations in; the QuTLASS
// kernel list of the Quartet notes: rotation fused before the GEMM, no separate launch). One
// persistent launch, every workgroup resident at once (a cooperative launch guarantees it):
//  1. all workgroups rotate + quantize A [M, K] exactly as the quantize kernels do (one wave per
//     64-segment wave tile, grid-stride), writing the caller's A codes and scales; then each
//     workgroup publishes its part with one agent-scope release (the stores leave the XCD's L2);
//  2. each workgroup waits (one agent-scope acquire, bounded spin) until every workgroup has
//     published, then walks its tiles (b, b + G, ...) in the usual XCD-grouped order with the
//     256 x 256 tile unchanged.
// Measured at 4096 x 11008 x 4096 (X bf16, H_128): this launch takes 150-158 us against 13 us for
// X's own quantize launch plus 111-122 us for the GEMM: the cooperative launch adds ~25 us, and
// phase 1 runs at the GEMM's occupancy (8 waves per CU, against the quantize kernel's many), about
// 2.5 us per wave tile and wave (four tiles' loads in flight per wave measured no faster). The
// separate quantize stays the faster route; this one saves A's extra pass only where a caller needs
// a single launch.
// A is quantized once by the whole grid, not once per tile. The hand-over is grid-wide rather than
// per tile row: an agent-scope acquire invalidates the XCD's L2 and a release writes it back, and
// with one release per wave tile and one acquire per tile (each tile waiting only for its own tile
// row) the 4096 x 11008 x 4096 product ran 3.3x slower; the first round of tiles needs rows of A
// from every tile row anyway.
// ---------------------------------------------------------------------------------------------
struct FusedA {
    SegArgs a;              // A's input and its codes / scales outputs (also g.a / g.sa)
    uint32_t* done;         // workgroups that have published their part of A (cleared before)
    uint32_t* status;       // bit 0 set if the wait gave up (results then invalid)
    int64_t units;          // wave tiles of 64 segments covering A
    int hn;                 // rotation of A along K (0, 16, 32, 64, 128)
};

__global__ void k_fill_u32(uint32_t* p, int n, uint32_t v) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = v;
}

template <int IN, int RND, bool B2D, int OUT>
__global__ __launch_bounds__(512) void k_gemm_fused_a(GemmArgs g, FusedA f) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    constexpr int P = SegIO<IN>::P;
    // phase 1: A's wave tiles, each wave with its own LDS slice for the segment transposition
    u32x4* lds = reinterpret_cast<u32x4*>(smem) + wave * 64 * P;
    const int64_t nw = (int64_t)gridDim.x * 8;
    for (int64_t u = (int64_t)blockIdx.x * 8 + wave; u < f.units; u += nw) {
        const int64_t wbase = u * 64, seg = wbase + lane;
        float v[32];
        load_wave_segments_1d<IN>(f.a, wbase, lds, v);
        fwht_groups(v, f.hn);
        uint32_t out[8];
        const SrSource sr{f.a.seed, (uint64_t)seg * 32u};
        const uint32_t s = e8m0_block<ELEM_E2M1, RND, 32, 0>(v, block_amax<32, 0>(v), f.a.ceil_rule != 0, sr, out);
        if (seg < f.a.nseg) {
            reinterpret_cast<uint8_t*>(f.a.scales)[seg] = (uint8_t)s;
            *reinterpret_cast<u32x4*>(f.a.codes + seg * 16) = (u32x4){out[0], out[1], out[2], out[3]};
        }
    }
    __syncthreads();  // the workgroup's stores are done; every wave is done with its LDS slice
    if (tid == 0) {
        // release: the workgroup's stores reach memory beyond this XCD's L2 before the count
        __hip_atomic_fetch_add(f.done, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        // every workgroup is resident and publishes before it waits, so the count arrives; the
        // bound only keeps a broken launch from spinning for ever
        for (uint32_t spin = 0;
             __hip_atomic_load(f.done, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < gridDim.x; ++spin) {
            if (spin > (1u << 24)) {
                atomicOr(f.status, 1u);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    __syncthreads();
    // phase 2: the tiles of this workgroup
    const int ntm = (int)((g.M + 255) / 256), ntn = (int)((g.N + 255) / 256);
    for (int t = blockIdx.x; t < ntm * ntn; t += gridDim.x) {
        int tm, tn;
        big_tile_coords(t, ntm, ntn, tm, tn);
        big_tile<false, B2D, OUT, false, FQ_NONE>(g, tm, tn, smem);
        __syncthreads();  // the next tile's copies overwrite the epilogue's staging
    }
}

// Raises KERNEL's dynamic LDS limit to `lds` bytes once per device (the attribute belongs to the
// function on the current device), instead of on every launch.
template <auto KERNEL>
static hipError_t allow_lds(size_t lds) {
    static std::atomic<uint64_t> done{0};  // bit d: set on device d
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 64 && ((done.load(std::memory_order_acquire) >> dev) & 1u)) return hipSuccess;
    e = hipFuncSetAttribute((const void*)KERNEL, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e == hipSuccess && dev < 64) done.fetch_or(uint64_t(1) << dev, std::memory_order_acq_rel);
    return e;
}

template <int IN, int RND, bool B2D, int OUT>
static hipError_t launch_fused_a_k(const GemmArgs& g, const FusedA& f, hipStream_t s) {
    using C = Big<false>;
    auto k = k_gemm_fused_a<IN, RND, B2D, OUT>;
    const size_t lds = (size_t)C::NST * C::STAGE;
    hipError_t e = allow_lds<k_gemm_fused_a<IN, RND, B2D, OUT>>(lds);
    if (e != hipSuccess) return e;
    int per_cu = 0, dev = 0, cus = 0;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, C::NTH, lds)) != hipSuccess) return e;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    const int64_t tiles = ((g.M + 255) / 256) * ((g.N + 255) / 256);
    const int64_t resident = (int64_t)per_cu * cus;
    if (resident < 1) return hipErrorInvalidConfiguration;
    const unsigned grid = (unsigned)(tiles < resident ? tiles : resident);
    GemmArgs ga = g;
    FusedA fa = f;
    void* args[] = {&ga, &fa};
    return hipLaunchCooperativeKernel((const void*)k, dim3(grid), dim3(C::NTH), args, (unsigned)lds, s);
}

hipError_t launch_gemm_fused_a(const GemmArgs& g, const SegArgs& a, int in_dtype, int hn, int rnd, int c_dtype,
                               uint32_t* ws, hipStream_t s) {
    FusedA f{};
    f.a = a;
    f.done = ws;
    f.status = ws + 1;
    f.units = (a.nseg + 63) / 64;
    f.hn = hn;
    hipLaunchKernelGGL(k_fill_u32, dim3(1), dim3(256), 0, s, ws, 2, 0u);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
#define BGF_FA(IN, RND)                                                                              \
    do {                                                                                             \
        if (g.b_2d) {                                                                                \
            if (c_dtype == DT_BF16) return launch_fused_a_k<IN, RND, true, DT_BF16>(g, f, s);         \
            return launch_fused_a_k<IN, RND, true, DT_F32>(g, f, s);                                  \
        }                                                                                            \
        if (c_dtype == DT_BF16) return launch_fused_a_k<IN, RND, false, DT_BF16>(g, f, s);            \
        return launch_fused_a_k<IN, RND, false, DT_F32>(g, f, s);                                     \
    } while (0)
    if (in_dtype == DT_BF16) {
        if (rnd == RND_SR) BGF_FA(DT_BF16, RND_SR);
        BGF_FA(DT_BF16, RND_RNE);
    }
    if (rnd == RND_SR) BGF_FA(DT_F32, RND_SR);
    BGF_FA(DT_F32, RND_RNE);
#undef BGF_FA
}

// ---------------------------------------------------------------------------------------------
// NVFP4 -> MXFP8 re-expression: one lane per 32-wide K group of one row.
// ---------------------------------------------------------------------------------------------
// Both operands in one launch: the first ga groups are A's, the next gb B's.
struct NvPair {
    const uint8_t* codes[2];
    const uint8_t* scales[2];
    uint8_t* out[2];
    uint8_t* out_scales[2];
    int64_t groups[2];
};

__global__ __launch_bounds__(256) void k_nv_to_fp8(NvPair pr) {
    int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int op = gi < pr.groups[0] ? 0 : 1;
    if (op == 1) gi -= pr.groups[0];
    if (gi >= pr.groups[op]) return;
    const uint8_t* const codes = op ? pr.codes[1] : pr.codes[0];
    const uint8_t* const scales = op ? pr.scales[1] : pr.scales[0];
    uint8_t* const out = op ? pr.out[1] : pr.out[0];
    uint8_t* const out_scales = op ? pr.out_scales[1] : pr.out_scales[0];
    const u32x4 q = *reinterpret_cast<const u32x4*>(codes + gi * 16);
    const uint32_t s01 = *reinterpret_cast<const uint16_t*>(scales + gi * 2);
    uint32_t o[8];
    out_scales[gi] = (uint8_t)nv_group_to_fp8(q, s01, o);
    u32x4* dst = reinterpret_cast<u32x4*>(out + gi * 32);
    dst[0] = (u32x4){o[0], o[1], o[2], o[3]};
    dst[1] = (u32x4){o[4], o[5], o[6], o[7]};
}

hipError_t launch_nv_to_fp8(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                            uint8_t* out, uint8_t* out_scales, hipStream_t s) {
    const int64_t groups = rows * (cols / 32);
    NvPair pr{{codes, codes}, {scales, scales}, {out, out}, {out_scales, out_scales}, {groups, 0}};
    hipLaunchKernelGGL(k_nv_to_fp8, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, s, pr);
    return hipGetLastError();
}

// Compute units of the current device (looked up once per device).
static hipError_t cu_count(int* n) {
    static std::atomic<int> cus[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 64 && (*n = cus[dev].load(std::memory_order_acquire)) > 0) return hipSuccess;
    e = hipDeviceGetAttribute(n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess && dev < 64) cus[dev].store(*n, std::memory_order_release);
    return e;
}

template <bool FP8, bool B2D, bool NVG, int FQ>
static hipError_t launch_out(const GemmArgs& g, int c_dtype, hipStream_t s) {
    const int64_t rowb = FP8 ? g.K : g.K / 2;
    const bool direct = g.K % Big<FP8>::KSTEP == 0 && g.M * rowb < (1ll << 31) && g.N * rowb < (1ll << 31);
    const int64_t big_tiles = ((g.M + 255) / 256) * ((g.N + 255) / 256);
    // 128 x 128 tiles where 256 x 256 ones would fill at most half the CUs (measured faster there:
    // 64-128 such tiles on 256 CUs; slower from 176 on) and where M or N is below 256 (faster than
    // the register-staged kernel)
    if (direct) {
        int cus = 0;
        const hipError_t e = cu_count(&cus);
        if (e != hipSuccess) return e;
        if (g.M < 256 || g.N < 256 || 2 * big_tiles <= cus) {
            using C = Big<FP8, 128>;
            const unsigned tiles = (unsigned)(((g.M + 127) / 128) * ((g.N + 127) / 128));
            const size_t lds = (size_t)C::NST * C::STAGE;
            hipError_t e2;
            if constexpr (FQ == FQ_NONE) {
                if (c_dtype == DT_BF16) {
                    if ((e2 = allow_lds<k_gemm_mid<FP8, B2D, DT_BF16, NVG>>(lds)) != hipSuccess) return e2;
                    hipLaunchKernelGGL((k_gemm_mid<FP8, B2D, DT_BF16, NVG>), dim3(tiles), dim3(C::NTH), lds, s, g);
                } else {
                    if ((e2 = allow_lds<k_gemm_mid<FP8, B2D, DT_F32, NVG>>(lds)) != hipSuccess) return e2;
                    hipLaunchKernelGGL((k_gemm_mid<FP8, B2D, DT_F32, NVG>), dim3(tiles), dim3(C::NTH), lds, s, g);
                }
            } else {
                if (c_dtype == DT_BF16) {
                    if ((e2 = allow_lds<k_gemm_mid_q<FP8, B2D, DT_BF16, NVG, FQ>>(lds)) != hipSuccess) return e2;
                    hipLaunchKernelGGL((k_gemm_mid_q<FP8, B2D, DT_BF16, NVG, FQ>), dim3(tiles), dim3(C::NTH), lds, s, g);
                } else {
                    if ((e2 = allow_lds<k_gemm_mid_q<FP8, B2D, DT_F32, NVG, FQ>>(lds)) != hipSuccess) return e2;
                    hipLaunchKernelGGL((k_gemm_mid_q<FP8, B2D, DT_F32, NVG, FQ>), dim3(tiles), dim3(C::NTH), lds, s, g);
                }
            }
            return hipGetLastError();
        }
    }
    if (g.M >= 256 && g.N >= 256 && direct) {
        using C = Big<FP8>;
        const unsigned tiles = (unsigned)(((g.M + 255) / 256) * ((g.N + 255) / 256));
        const size_t lds = (size_t)C::NST * C::STAGE;
        if (c_dtype == DT_BF16) {
            hipError_t e = allow_lds<k_gemm_big<FP8, B2D, DT_BF16, NVG, FQ>>(lds);
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL((k_gemm_big<FP8, B2D, DT_BF16, NVG, FQ>), dim3(tiles), dim3(C::NTH), lds, s, g);
        } else {
            hipError_t e = allow_lds<k_gemm_big<FP8, B2D, DT_F32, NVG, FQ>>(lds);
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL((k_gemm_big<FP8, B2D, DT_F32, NVG, FQ>), dim3(tiles), dim3(C::NTH), lds, s, g);
        }
        return hipGetLastError();
    }
    dim3 grid((unsigned)((g.N + BN - 1) / BN), (unsigned)((g.M + BM - 1) / BM));
    if (c_dtype == DT_BF16) hipLaunchKernelGGL((k_gemm<FP8, B2D, DT_BF16, NVG, FQ>), grid, dim3(NT), 0, s, g);
    else hipLaunchKernelGGL((k_gemm<FP8, B2D, DT_F32, NVG, FQ>), grid, dim3(NT), 0, s, g);
    return hipGetLastError();
}

template <int FQ>
static hipError_t launch_kind(const GemmArgs& g, int kind, int c_dtype, hipStream_t s) {
    if (kind == 0) {
        if (g.b_2d) return launch_out<false, true, false, FQ>(g, c_dtype, s);
        return launch_out<false, false, false, FQ>(g, c_dtype, s);
    }
    if (kind == 1) return launch_out<true, false, false, FQ>(g, c_dtype, s);
    // NVFP4 with no workspace: the re-expression in LDS (256 x 256 tiles, K % 128 == 0)
    if (!g.a8 && g.M >= 256 && g.N >= 256 && g.K % Big<true>::KSTEP == 0 && g.M * (g.K / 2) < (1ll << 31) && g.N * (g.K / 2) < (1ll << 31)) {
        const unsigned tiles = (unsigned)(((g.M + 255) / 256) * ((g.N + 255) / 256));
        const size_t lds = (size_t)NvLds::LDS;
        hipError_t e = c_dtype == DT_BF16 ? allow_lds<k_gemm_nv<DT_BF16, FQ>>(lds) : allow_lds<k_gemm_nv<DT_F32, FQ>>(lds);
        if (e != hipSuccess) return e;
        if (c_dtype == DT_BF16) hipLaunchKernelGGL((k_gemm_nv<DT_BF16, FQ>), dim3(tiles), dim3(512), lds, s, g);
        else hipLaunchKernelGGL((k_gemm_nv<DT_F32, FQ>), dim3(tiles), dim3(512), lds, s, g);
        return hipGetLastError();
    }
    if (!g.a8) return hipErrorInvalidValue;
    // NVFP4: re-express both operands into the workspace, then the FP8 product with the tensor scales
    const int64_t ga = g.M * (g.K / 32), gb = g.N * (g.K / 32);
    NvPair pr{{g.a, g.b}, {g.sa, g.sb}, {g.a8, g.b8}, {g.sa8, g.sb8}, {ga, gb}};
    hipLaunchKernelGGL(k_nv_to_fp8, dim3((unsigned)((ga + gb + 255) / 256)), dim3(256), 0, s, pr);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    GemmArgs h = g;
    h.a = g.a8;
    h.b = g.b8;
    h.sa = g.sa8;
    h.sb = g.sb8;
    return launch_out<true, false, true, FQ>(h, c_dtype, s);
}

hipError_t launch_gemm(const GemmArgs& g, int kind, int c_dtype, int fused_q, hipStream_t s) {
    if (fused_q) {
        if (g.q_round == RND_SR) return launch_kind<FQ_SR>(g, kind, c_dtype, s);
        return launch_kind<FQ_RNE>(g, kind, c_dtype, s);
    }
    return launch_kind<FQ_NONE>(g, kind, c_dtype, s);
}

}  // namespace bgf
