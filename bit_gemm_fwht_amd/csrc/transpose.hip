// Re-layout of a tensor quantized with 32 x 32 blocks into the quantized form of its transpose.
//
// With one scale per 32 x 32 tile, the tile of T^T at (j, i) holds exactly the elements of T's tile
// (i, j), so its amax, its scale and every element code are the same: quantizing T^T is a
// transposition of T's codes and of its scale grid, with no arithmetic (the transposition
// invariance of the 2D block scales in "Stable FP4 Training via Transposition-Invariant Block
// Quantization", abstract). A tensor quantized once can then feed a GEMM that contracts it along
// either axis.
//
// E4M3: a 256-thread workgroup moves a 64 x 64 element tile: it reads 64 rows of codes (64 bytes per
// row: whole 16-byte pieces, consecutive threads on consecutive bytes), spreads the elements one
// per LDS byte, and writes 64 rows of the transposed tile the same way; the 2 x 2 scales of the
// tile are transposed by four threads. (E2M1's 4-bit codes have their own kernel below.)
#include "device.h"
#include "fp4_internal.h"

namespace bgf {

constexpr int TT = 64;           // tile edge (elements)
constexpr int TPITCH = TT + 4;   // LDS row pitch in bytes (breaks the column reads across banks)

__global__ __launch_bounds__(256) void k_transpose_2d_e4m3(TransposeArgs a) {
    __shared__ uint8_t tile[TT * TPITCH];
    const int tid = threadIdx.x;
    const int64_t ntc = (a.cols + TT - 1) / TT;
    const int64_t r0 = (int64_t)(blockIdx.x / ntc) * TT, c0 = (int64_t)(blockIdx.x % ntc) * TT;
    constexpr int PPR = TT / 16;  // 16-byte pieces per tile row
    // read: piece p of tile row r (rows and columns past the tensor are skipped; their LDS bytes
    // only feed outputs that are not written)
    for (int t = tid; t < TT * PPR; t += 256) {
        const int r = t / PPR, p = t % PPR;
        const int64_t gr = r0 + r, gc = c0 + (int64_t)p * 16;  // first element of the piece
        if (gr >= a.rows || gc >= a.cols) continue;
        const u32x4 w = *reinterpret_cast<const u32x4*>(a.codes + gr * a.cols + gc);
        uint8_t* dst = tile + r * TPITCH + (gc - c0);
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int b = 0; b < 4; ++b) dst[4 * q + b] = (uint8_t)((w[q] >> (8 * b)) & 0xFFu);
    }
    __syncthreads();
    // write: piece p of output row c (= tile column c), elements r = its rows of the input tile
    for (int t = tid; t < TT * PPR; t += 256) {
        const int c = t / PPR, p = t % PPR;
        const int64_t oc = c0 + c, orr = r0 + (int64_t)p * 16;  // output row, first output column
        if (oc >= a.cols || orr >= a.rows) continue;
        const int rb = p * 16;
        u32x4 w;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t v = 0u;
#pragma unroll
            for (int b = 0; b < 4; ++b) v |= (uint32_t)tile[(rb + 4 * q + b) * TPITCH + c] << (8 * b);
            w[q] = v;
        }
        *reinterpret_cast<u32x4*>(a.out_codes + oc * a.rows + orr) = w;
    }
    // scales: [rows / 32, cols / 32] -> [cols / 32, rows / 32]
    if (tid < 4) {
        const int64_t si = r0 / 32 + (tid >> 1), sj = c0 / 32 + (tid & 1);
        const int64_t sr = a.rows / 32, scn = a.cols / 32;
        if (si < sr && sj < scn) a.out_scales[sj * sr + si] = a.scales[si * scn + sj];
    }
}

// E2M1: a 256-thread workgroup moves a 128 x 128 element tile (8 KB of codes). Each thread reads two
// 16-byte pieces into LDS (rows of 64 bytes, consecutive threads on consecutive bytes), transposes
// one 8 x 8 block of nibbles in registers (eight 32-bit rows; three rounds of masked swaps of
// 4 x 4, 2 x 2 and 1 x 1 sub-blocks), writes the block's eight output rows to a second LDS tile,
// and stores two 16-byte pieces of the transposed tile. The 4 x 4 scales of the tile are transposed
// by sixteen threads. Tensor dimensions are multiples of 32, so every piece and every 8 x 8 block
// lies wholly inside or wholly outside the tensor.
constexpr int T4 = 128;        // tile edge (elements)
constexpr int P4 = T4 / 2 + 16;  // LDS row pitch in bytes (64 bytes of codes + 16 of padding)

__device__ __forceinline__ void swap_blocks(uint32_t& a, uint32_t& b, int sh, uint32_t m) {
    // exchange the bits of a under (m << sh) with the bits of b under m
    const uint32_t t = ((a >> sh) ^ b) & m;
    b ^= t;
    a ^= t << sh;
}

__global__ __launch_bounds__(256) void k_transpose_2d_e2m1(TransposeArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t tin[T4 * P4];
    __shared__ __attribute__((aligned(16))) uint8_t tout[T4 * P4];
    const int tid = threadIdx.x;
    const int64_t ntc = (a.cols + T4 - 1) / T4;
    const int64_t r0 = (int64_t)(blockIdx.x / ntc) * T4, c0 = (int64_t)(blockIdx.x % ntc) * T4;
    const int64_t in_pitch = a.cols / 2, out_pitch = a.rows / 2;
    // read: piece p (32 elements) of tile row r
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int q = tid + 256 * i, r = q >> 2, p = q & 3;
        if (r0 + r < a.rows && c0 + 32 * p < a.cols)
            *reinterpret_cast<u32x4*>(tin + r * P4 + 16 * p) =
                *reinterpret_cast<const u32x4*>(a.codes + (r0 + r) * in_pitch + c0 / 2 + 16 * p);
    }
    __syncthreads();
    // 8 x 8 nibble block (bi, bj): input rows 8 bi .. 8 bi + 7, elements 8 bj .. 8 bj + 7 (one word)
    const int bj = tid & 15, bi = tid >> 4;
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] = *reinterpret_cast<const uint32_t*>(tin + (8 * bi + k) * P4 + 4 * bj);
#pragma unroll
    for (int k = 0; k < 4; ++k) swap_blocks(w[k], w[k + 4], 16, 0x0000FFFFu);
#pragma unroll
    for (int k = 0; k < 8; k += (k & 1) ? 3 : 1) swap_blocks(w[k], w[k + 2], 8, 0x00FF00FFu);  // k = 0, 1, 4, 5
#pragma unroll
    for (int k = 0; k < 8; k += 2) swap_blocks(w[k], w[k + 1], 4, 0x0F0F0F0Fu);
    // w[j] is output row 8 bj + j (input element column), nibble k = input row 8 bi + k
#pragma unroll
    for (int j = 0; j < 8; ++j) *reinterpret_cast<uint32_t*>(tout + (8 * bj + j) * P4 + 4 * bi) = w[j];
    __syncthreads();
    // write: piece p of output row c (= input element column c0 + c)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int q = tid + 256 * i, c = q >> 2, p = q & 3;
        if (c0 + c < a.cols && r0 + 32 * p < a.rows)
            *reinterpret_cast<u32x4*>(a.out_codes + (c0 + c) * out_pitch + r0 / 2 + 16 * p) =
                *reinterpret_cast<const u32x4*>(tout + c * P4 + 16 * p);
    }
    if (tid < 16) {
        const int64_t si = r0 / 32 + (tid >> 2), sj = c0 / 32 + (tid & 3);
        const int64_t sr = a.rows / 32, scn = a.cols / 32;
        if (si < sr && sj < scn) a.out_scales[sj * sr + si] = a.scales[si * scn + sj];
    }
}

hipError_t launch_transpose_2d(const TransposeArgs& a, int elem, hipStream_t s) {
    if (elem == ELEM_E2M1) {
        const int64_t tiles = ((a.rows + T4 - 1) / T4) * ((a.cols + T4 - 1) / T4);
        if (tiles <= 0 || tiles >= (int64_t(1) << 31)) return hipErrorInvalidValue;
        hipLaunchKernelGGL(k_transpose_2d_e2m1, dim3((unsigned)tiles), dim3(256), 0, s, a);
        return hipGetLastError();
    }
    const int64_t tiles = ((a.rows + TT - 1) / TT) * ((a.cols + TT - 1) / TT);
    if (tiles <= 0 || tiles >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_transpose_2d_e4m3, dim3((unsigned)tiles), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace bgf
