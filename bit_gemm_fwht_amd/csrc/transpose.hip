// Re-layout of a tensor quantized with 32 x 32 blocks into the quantized form of its transpose.
//
// With one scale per 32 x 32 tile, the tile of T^T at (j, i) holds exactly the elements of T's tile
// (i, j), so its amax, its scale and every element code are the same: quantizing T^T is a
// transposition of T's codes and of its scale grid, with no arithmetic (the transposition
// invariance of the 2D block scales in "Stable FP4 Training via Transposition-Invariant Block
// Quantization", abstract). A tensor quantized once can then feed a GEMM that contracts it along
// either axis.
//
// A 256-thread workgroup moves a 64 x 64 element tile: it reads 64 rows of codes (32 bytes per row
// for E2M1, 64 for E4M3: whole 16-byte pieces, consecutive threads on consecutive bytes), spreads
// the elements one per LDS byte, and writes 64 rows of the transposed tile the same way; the 2 x 2
// scales of the tile are transposed by four threads.
#include "device.h"
#include "fp4_internal.h"

namespace bgf {

constexpr int TT = 64;           // tile edge (elements)
constexpr int TPITCH = TT + 4;   // LDS row pitch in bytes (breaks the column reads across banks)

template <int ELEM>
__global__ __launch_bounds__(256) void k_transpose_2d(TransposeArgs a) {
    __shared__ uint8_t tile[TT * TPITCH];
    const int tid = threadIdx.x;
    const int64_t ntc = (a.cols + TT - 1) / TT;
    const int64_t r0 = (int64_t)(blockIdx.x / ntc) * TT, c0 = (int64_t)(blockIdx.x % ntc) * TT;
    constexpr int BPR = ELEM == ELEM_E2M1 ? TT / 2 : TT;  // code bytes per tile row
    constexpr int PPR = BPR / 16;                          // 16-byte pieces per tile row
    const int64_t in_pitch = ELEM == ELEM_E2M1 ? a.cols / 2 : a.cols;
    const int64_t out_pitch = ELEM == ELEM_E2M1 ? a.rows / 2 : a.rows;
    // read: piece p of tile row r (rows and columns past the tensor are skipped; their LDS bytes
    // only feed outputs that are not written)
    for (int t = tid; t < TT * PPR; t += 256) {
        const int r = t / PPR, p = t % PPR;
        const int64_t gr = r0 + r;
        const int64_t gc = c0 + (int64_t)p * (ELEM == ELEM_E2M1 ? 32 : 16);  // first element of the piece
        if (gr >= a.rows || gc >= a.cols) continue;
        const u32x4 w = *reinterpret_cast<const u32x4*>(a.codes + gr * in_pitch + (ELEM == ELEM_E2M1 ? gc / 2 : gc));
        uint8_t* dst = tile + r * TPITCH + (gc - c0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const uint32_t byte = (w[q] >> (8 * b)) & 0xFFu;
                if constexpr (ELEM == ELEM_E2M1) {
                    dst[8 * q + 2 * b] = (uint8_t)(byte & 0xFu);
                    dst[8 * q + 2 * b + 1] = (uint8_t)(byte >> 4);
                } else {
                    dst[4 * q + b] = (uint8_t)byte;
                }
            }
        }
    }
    __syncthreads();
    // write: piece p of output row c (= tile column c), elements r = its rows of the input tile
    for (int t = tid; t < TT * PPR; t += 256) {
        const int c = t / PPR, p = t % PPR;
        const int64_t oc = c0 + c;                                            // output row
        const int64_t orr = r0 + (int64_t)p * (ELEM == ELEM_E2M1 ? 32 : 16);  // first output column
        if (oc >= a.cols || orr >= a.rows) continue;
        const int rb = p * (ELEM == ELEM_E2M1 ? 32 : 16);
        u32x4 w;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t v = 0u;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                if constexpr (ELEM == ELEM_E2M1) {
                    const uint32_t lo = tile[(rb + 8 * q + 2 * b) * TPITCH + c];
                    const uint32_t hi = tile[(rb + 8 * q + 2 * b + 1) * TPITCH + c];
                    v |= (lo | (hi << 4)) << (8 * b);
                } else {
                    v |= (uint32_t)tile[(rb + 4 * q + b) * TPITCH + c] << (8 * b);
                }
            }
            w[q] = v;
        }
        *reinterpret_cast<u32x4*>(a.out_codes + oc * out_pitch + (ELEM == ELEM_E2M1 ? orr / 2 : orr)) = w;
    }
    // scales: [rows / 32, cols / 32] -> [cols / 32, rows / 32]
    if (tid < 4) {
        const int64_t si = r0 / 32 + (tid >> 1), sj = c0 / 32 + (tid & 1);
        const int64_t sr = a.rows / 32, scn = a.cols / 32;
        if (si < sr && sj < scn) a.out_scales[sj * sr + si] = a.scales[si * scn + sj];
    }
}

hipError_t launch_transpose_2d(const TransposeArgs& a, int elem, hipStream_t s) {
    const int64_t tiles = ((a.rows + TT - 1) / TT) * ((a.cols + TT - 1) / TT);
    if (tiles <= 0 || tiles >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    if (elem == ELEM_E2M1) hipLaunchKernelGGL(k_transpose_2d<ELEM_E2M1>, dim3((unsigned)tiles), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_transpose_2d<ELEM_E4M3>, dim3((unsigned)tiles), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace bgf
