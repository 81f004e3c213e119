// C ABI of libbgf (declared in include/fp4.h): host-side validation, size queries and dispatch to
// the HIP kernels. Nothing is queued unless every argument has been accepted.
#include "../../include/fp4.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "fp4_internal.h"

namespace {

using namespace bgf;

enum Layout { L_BAD = 0, L_SEG1D, L_SEG2D, L_ROW, L_TENSOR };

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool valid_hn(int n) { return n == 0 || n == 16 || n == 32 || n == 64 || n == 128 || n == 256; }
// The segment kernels address a wave's 64 segments (up to 64 rows of a strided tensor, or the 8
// rows of a 2D tile's slice) with 32-bit byte offsets from the tile's first row.
bool pitch_ok(int64_t ld, int esz) { return 64 * ld * esz < (int64_t(1) << 31); }

bool is_nv(int sm) {
    return sm == FP4_SCALE_NV || sm == FP4_SCALE_NV_4OVER6 || sm == FP4_SCALE_NV_GIVEN ||
           sm == FP4_SCALE_NV_4OVER6_GIVEN;
}
bool is_4over6(int sm) { return sm == FP4_SCALE_NV_4OVER6 || sm == FP4_SCALE_NV_4OVER6_GIVEN; }
bool is_given(int sm) { return sm == FP4_SCALE_NV_GIVEN || sm == FP4_SCALE_NV_4OVER6_GIVEN; }

int scale_class(int sm) {
    if (sm == FP4_SCALE_E8M0_FLOOR || sm == FP4_SCALE_E8M0_CEIL) return SC_E8M0;
    if (is_nv(sm)) return SC_NV;
    return SC_F32;
}

// Classify and validate a (rows, cols, params) triple; returns FP4_OK and the layout.
int check_params(int64_t rows, int64_t cols, const fp4_qparams* p, Layout* lay) {
    *lay = L_BAD;
    if (!p || rows <= 0 || cols <= 0) return FP4_ERR_INVALID_ARG;
    if (p->elem != FP4_ELEM_E2M1 && p->elem != FP4_ELEM_E4M3) return FP4_ERR_INVALID_ARG;
    if (p->scale_mode < FP4_SCALE_E8M0_FLOOR || p->scale_mode > FP4_SCALE_NV_4OVER6_GIVEN) return FP4_ERR_INVALID_ARG;
    if (p->round_mode != FP4_ROUND_RNE && p->round_mode != FP4_ROUND_SR) return FP4_ERR_INVALID_ARG;
    if (p->block_rows <= 0 || p->block_cols <= 0) return FP4_ERR_INVALID_ARG;
    if (rows % p->block_rows || cols % p->block_cols) return FP4_ERR_INVALID_ARG;
    if (p->elem == FP4_ELEM_E2M1 && (cols & 1)) return FP4_ERR_INVALID_ARG;
    if (!valid_hn(p->hadamard_n)) return FP4_ERR_INVALID_ARG;
    if (p->hadamard_n && cols % p->hadamard_n) return FP4_ERR_INVALID_ARG;
    const int br = p->block_rows, bc = p->block_cols;
    if (br == 1 && (bc == 16 || bc == 32) && cols % 32 == 0) *lay = L_SEG1D;
    else if (br == 32 && bc == 32 && cols % 32 == 0) *lay = L_SEG2D;
    else if (br == 1 && bc == cols) *lay = L_ROW;
    else if (br == rows && bc == cols) *lay = L_TENSOR;
    else return FP4_ERR_UNSUPPORTED;
    if (is_nv(p->scale_mode)) {
        if (p->elem != FP4_ELEM_E2M1 || *lay != L_SEG1D || bc != 16) return FP4_ERR_UNSUPPORTED;
        if (is_4over6(p->scale_mode) && p->round_mode == FP4_ROUND_SR) return FP4_ERR_UNSUPPORTED;
    }
    if (*lay == L_SEG2D && scale_class(p->scale_mode) != SC_E8M0) return FP4_ERR_UNSUPPORTED;
    if ((*lay == L_ROW || *lay == L_TENSOR) && p->hadamard_n) return FP4_ERR_UNSUPPORTED;
    return FP4_OK;
}

int64_t codes_bytes(int64_t rows, int64_t cols, const fp4_qparams* p) {
    return p->elem == FP4_ELEM_E2M1 ? rows * (cols / 2) : rows * cols;
}
int64_t scales_bytes(int64_t rows, int64_t cols, const fp4_qparams* p) {
    const int64_t n = (rows / p->block_rows) * (cols / p->block_cols);
    return scale_class(p->scale_mode) == SC_F32 ? 4 * n : n;
}
int64_t ws_bytes_needed(Layout lay, const fp4_qparams* p) {
    return ((is_nv(p->scale_mode) && !is_given(p->scale_mode)) || lay == L_TENSOR) ? 256 : 0;
}

int hip_status(hipError_t e) { return e == hipSuccess ? FP4_OK : FP4_ERR_HIP; }

// Library-owned device scratch of fp4_quantize_noalloc: one copy per GPU, alive until the process
// ends. Host code never passes `scratch` itself to a kernel (in host code the name is a host-side
// stand-in, not a device address): the device address is looked up once per device with that device
// current and kept in scratch_ptr.
__device__ __attribute__((aligned(256))) uint8_t scratch[FP4_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

int scratch_for_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return FP4_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return FP4_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FP4_ERR_HIP;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return FP4_OK;
}

}  // namespace

extern "C" {

int fp4_abi_version(void) { return FP4_ABI_VERSION; }

const char* fp4_status_string(int s) {
    switch (s) {
        case FP4_OK: return "ok";
        case FP4_ERR_INVALID_ARG: return "invalid argument";
        case FP4_ERR_UNSUPPORTED: return "unsupported combination";
        case FP4_ERR_ALIGNMENT: return "misaligned pointer or pitch (16 bytes required)";
        case FP4_ERR_WORKSPACE: return "workspace missing or too small";
        case FP4_ERR_HIP: return "HIP runtime error";
        case FP4_ERR_INTERNAL: return "internal error";
        default: return "unknown status";
    }
}

int64_t fp4_codes_bytes(int64_t rows, int64_t cols, const fp4_qparams* p) {
    Layout lay;
    if (check_params(rows, cols, p, &lay) != FP4_OK) return -1;
    return codes_bytes(rows, cols, p);
}

int64_t fp4_scales_bytes(int64_t rows, int64_t cols, const fp4_qparams* p) {
    Layout lay;
    if (check_params(rows, cols, p, &lay) != FP4_OK) return -1;
    return scales_bytes(rows, cols, p);
}

int64_t fp4_workspace_bytes(int64_t rows, int64_t cols, const fp4_qparams* p) {
    Layout lay;
    if (check_params(rows, cols, p, &lay) != FP4_OK) return -1;
    return ws_bytes_needed(lay, p);
}

int fp4_quantize(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                 const fp4_qparams* p, void* codes, void* scales, float* tensor_scale,
                 void* workspace, int64_t ws_bytes, void* stream) {
    try {
        Layout lay;
        int rc = check_params(rows, cols, p, &lay);
        if (rc != FP4_OK) return rc;
        if (!x || !codes || !scales) return FP4_ERR_INVALID_ARG;
        if (x_dtype != FP4_DT_F32 && x_dtype != FP4_DT_BF16) return FP4_ERR_INVALID_ARG;
        if (ldx < cols) return FP4_ERR_INVALID_ARG;
        if (codes == x || scales == x || codes == scales) return FP4_ERR_INVALID_ARG;
        if (is_nv(p->scale_mode) && !tensor_scale) return FP4_ERR_INVALID_ARG;
        const int esz = x_dtype == FP4_DT_BF16 ? 2 : 4;
        if (lay == L_SEG1D || lay == L_SEG2D) {
            if (!aligned(x, 16) || (ldx * esz) % 16 || !aligned(codes, 16) || !aligned(scales, 8))
                return FP4_ERR_ALIGNMENT;
            if ((ldx != cols || lay == L_SEG2D) && !pitch_ok(ldx, esz)) return FP4_ERR_UNSUPPORTED;
        }
        const int64_t need = ws_bytes_needed(lay, p);
        if (need && (!workspace || ws_bytes < need)) return FP4_ERR_WORKSPACE;
        if (need && !aligned(workspace, 4)) return FP4_ERR_ALIGNMENT;

        hipStream_t s = reinterpret_cast<hipStream_t>(stream);
        const int sc = scale_class(p->scale_mode);
        uint32_t* ws = reinterpret_cast<uint32_t*>(workspace);
        if (lay == L_SEG1D || lay == L_SEG2D) {
            SegArgs a{};
            a.x = x;
            a.rows = rows;
            a.cols = cols;
            a.ldx = ldx;
            a.nseg = rows * (cols / 32);
            a.codes = reinterpret_cast<uint8_t*>(codes);
            a.scales = scales;
            a.tensor_scale = tensor_scale;
            a.ws = ws;
            a.seed = p->seed;
            a.ceil_rule = p->scale_mode == FP4_SCALE_E8M0_CEIL;
            a.four_six = is_4over6(p->scale_mode);
            a.nv_given = is_given(p->scale_mode);
            if (sc == SC_NV && !a.nv_given) {
                if ((rc = hip_status(launch_zero_u32(ws, 1, s))) != FP4_OK) return rc;
                rc = hip_status(launch_segment(a, x_dtype, p->hadamard_n, p->elem, sc, p->round_mode, 1,
                                               32, PASS_AMAX, s));
                if (rc != FP4_OK) return rc;
            }
            return hip_status(launch_segment(a, x_dtype, p->hadamard_n, p->elem, sc, p->round_mode,
                                             p->block_rows, p->block_cols, PASS_QUANT, s));
        }
        RowArgs a{};
        a.x = x;
        a.rows = rows;
        a.cols = cols;
        a.ldx = ldx;
        a.codes = reinterpret_cast<uint8_t*>(codes);
        a.scales = scales;
        a.ws = ws;
        a.seed = p->seed;
        a.ceil_rule = p->scale_mode == FP4_SCALE_E8M0_CEIL;
        a.per_tensor = lay == L_TENSOR;
        if (lay == L_TENSOR) {
            if ((rc = hip_status(launch_zero_u32(ws, 1, s))) != FP4_OK) return rc;
            if ((rc = hip_status(launch_amax_rows(x, x_dtype, rows, cols, ldx, ws, s))) != FP4_OK) return rc;
        }
        return hip_status(launch_rowblock(a, x_dtype, p->elem, sc, p->round_mode, s));
    } catch (...) {
        return FP4_ERR_INTERNAL;
    }
}

int fp4_quantize_noalloc(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                         const fp4_qparams* p, void* codes, void* scales, float* tensor_scale, void* stream) {
    try {
        Layout lay;
        const int rc = check_params(rows, cols, p, &lay);
        if (rc != FP4_OK) return rc;
        const int64_t need = ws_bytes_needed(lay, p);
        if (need > FP4_NOALLOC_SCRATCH_BYTES) return FP4_ERR_WORKSPACE;
        void* ws = nullptr;
        if (need) {
            const int s = scratch_for_current_device(&ws);
            if (s != FP4_OK) return s;
        }
        return fp4_quantize(x, x_dtype, rows, cols, ldx, p, codes, scales, tensor_scale, ws, need, stream);
    } catch (...) {
        return FP4_ERR_INTERNAL;
    }
}

int fp4_quantize_batch(int32_t count, const fp4_quant_item* items, int32_t x_dtype, const fp4_qparams* p,
                       void* stream) {
    try {
        if (count < 1 || count > kMaxBatch || !items || !p) return FP4_ERR_INVALID_ARG;
        if (x_dtype != FP4_DT_F32 && x_dtype != FP4_DT_BF16) return FP4_ERR_INVALID_ARG;
        const int sc = scale_class(p->scale_mode);
        if (sc == SC_NV && !is_given(p->scale_mode)) return FP4_ERR_UNSUPPORTED;
        const int esz = x_dtype == FP4_DT_BF16 ? 2 : 4;
        SegArgs a[kMaxBatch] = {};
        for (int i = 0; i < count; ++i) {
            const fp4_quant_item& t = items[i];
            Layout lay;
            int rc = check_params(t.rows, t.cols, p, &lay);
            if (rc != FP4_OK) return rc;
            if (lay != L_SEG1D && lay != L_SEG2D) return FP4_ERR_UNSUPPORTED;
            if (!t.x || !t.codes || !t.scales) return FP4_ERR_INVALID_ARG;
            if (t.ldx < t.cols) return FP4_ERR_INVALID_ARG;
            if (sc == SC_NV && !t.tensor_scale) return FP4_ERR_INVALID_ARG;
            if (!aligned(t.x, 16) || (t.ldx * esz) % 16 || !aligned(t.codes, 16) || !aligned(t.scales, 8))
                return FP4_ERR_ALIGNMENT;
            if ((t.ldx != t.cols || lay == L_SEG2D) && !pitch_ok(t.ldx, esz)) return FP4_ERR_UNSUPPORTED;
            a[i].x = t.x;
            a[i].rows = t.rows;
            a[i].cols = t.cols;
            a[i].ldx = t.ldx;
            a[i].nseg = t.rows * (t.cols / 32);
            a[i].codes = reinterpret_cast<uint8_t*>(t.codes);
            a[i].scales = t.scales;
            a[i].tensor_scale = t.tensor_scale;
            a[i].seed = p->seed;
            a[i].ceil_rule = p->scale_mode == FP4_SCALE_E8M0_CEIL;
            a[i].four_six = is_4over6(p->scale_mode);
            a[i].nv_given = is_given(p->scale_mode);
        }
        // outputs must not alias each other or any input
        for (int i = 0; i < count; ++i) {
            const void* outs[2] = {items[i].codes, items[i].scales};
            for (const void* o : outs) {
                for (int j = 0; j < count; ++j) {
                    if (o == items[j].x) return FP4_ERR_INVALID_ARG;
                    if (j != i && (o == items[j].codes || o == items[j].scales)) return FP4_ERR_INVALID_ARG;
                }
            }
            if (items[i].codes == items[i].scales) return FP4_ERR_INVALID_ARG;
        }
        return hip_status(launch_segment_batch(a, count, x_dtype, p->hadamard_n, p->elem, sc, p->round_mode,
                                               p->block_rows, p->block_cols, reinterpret_cast<hipStream_t>(stream)));
    } catch (...) {
        return FP4_ERR_INTERNAL;
    }
}

int fp4_quantize_colwise(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                         const fp4_qparams* p, void* codes, void* scales, float* tensor_scale,
                         void* workspace, int64_t ws_bytes, void* stream) {
    try {
        // the quantized tensor is T = x^T: cols x rows, groups along x's rows
        Layout lay;
        int rc = check_params(cols, rows, p, &lay);
        if (rc != FP4_OK) return rc;
        if (lay != L_SEG1D) return FP4_ERR_UNSUPPORTED;
        if (!x || !codes || !scales) return FP4_ERR_INVALID_ARG;
        if (x_dtype != FP4_DT_F32 && x_dtype != FP4_DT_BF16) return FP4_ERR_INVALID_ARG;
        if (ldx < cols) return FP4_ERR_INVALID_ARG;
        if (codes == x || scales == x || codes == scales) return FP4_ERR_INVALID_ARG;
        if (is_nv(p->scale_mode) && !tensor_scale) return FP4_ERR_INVALID_ARG;
        const int esz = x_dtype == FP4_DT_BF16 ? 2 : 4;
        if (!aligned(x, 16) || (ldx * esz) % 16 || !aligned(codes, 16) || !aligned(scales, 8))
            return FP4_ERR_ALIGNMENT;
        // tile offsets are 32-bit: 256 rows of x must span less than 2 GiB
        if (256 * ldx * esz >= (int64_t(1) << 31)) return FP4_ERR_UNSUPPORTED;
        const int64_t need = ws_bytes_needed(lay, p);
        if (need && (!workspace || ws_bytes < need)) return FP4_ERR_WORKSPACE;
        if (need && !aligned(workspace, 4)) return FP4_ERR_ALIGNMENT;

        hipStream_t s = reinterpret_cast<hipStream_t>(stream);
        const int sc = scale_class(p->scale_mode);
        uint32_t* ws = reinterpret_cast<uint32_t*>(workspace);
        SegArgs a{};
        a.x = x;
        a.rows = cols;  // T's shape
        a.cols = rows;
        a.ldx = ldx;
        a.nseg = cols * (rows / 32);
        a.codes = reinterpret_cast<uint8_t*>(codes);
        a.scales = scales;
        a.tensor_scale = tensor_scale;
        a.ws = ws;
        a.seed = p->seed;
        a.ceil_rule = p->scale_mode == FP4_SCALE_E8M0_CEIL;
        a.four_six = is_4over6(p->scale_mode);
        a.nv_given = is_given(p->scale_mode);
        a.colwise = 1;
        if (sc == SC_NV && !a.nv_given) {
            if ((rc = hip_status(launch_zero_u32(ws, 1, s))) != FP4_OK) return rc;
            rc = hip_status(launch_segment(a, x_dtype, p->hadamard_n, p->elem, sc, p->round_mode, 1, 32, PASS_AMAX, s));
            if (rc != FP4_OK) return rc;
        }
        return hip_status(launch_segment(a, x_dtype, p->hadamard_n, p->elem, sc, p->round_mode, 1,
                                         p->block_cols, PASS_QUANT, s));
    } catch (...) {
        return FP4_ERR_INTERNAL;
    }
}

int fp4_dequantize(const void* codes, const void* scales, const float* tensor_scale, int64_t rows,
                   int64_t cols, const fp4_qparams* p, void* y, int32_t y_dtype, int64_t ldy,
                   void* stream) {
    try {
        Layout lay;
        int rc = check_params(rows, cols, p, &lay);
        if (rc != FP4_OK) return rc;
        if (!codes || !scales || !y) return FP4_ERR_INVALID_ARG;
        if (y_dtype != FP4_DT_F32 && y_dtype != FP4_DT_BF16) return FP4_ERR_INVALID_ARG;
        if (ldy < cols) return FP4_ERR_INVALID_ARG;
        if (is_nv(p->scale_mode) && !tensor_scale) return FP4_ERR_INVALID_ARG;
        const int esz = y_dtype == FP4_DT_BF16 ? 2 : 4;
        if (lay == L_SEG1D || lay == L_SEG2D) {
            if (!aligned(y, 16) || (ldy * esz) % 16 || !aligned(codes, 16) || !aligned(scales, 8))
                return FP4_ERR_ALIGNMENT;
        }
        DeqArgs a{};
        a.codes = reinterpret_cast<const uint8_t*>(codes);
        a.scales = scales;
        a.tensor_scale = tensor_scale;
        a.rows = rows;
        a.cols = cols;
        a.nseg = rows * (cols / 32);
        a.y = y;
        a.ldy = ldy;
        a.per_tensor = lay == L_TENSOR;
        hipStream_t s = reinterpret_cast<hipStream_t>(stream);
        const int sc = scale_class(p->scale_mode);
        if (lay == L_SEG1D || lay == L_SEG2D)
            return hip_status(launch_dequant_segment(a, p->elem, sc, p->block_rows, p->block_cols,
                                                     p->hadamard_n, y_dtype, s));
        return hip_status(launch_dequant_rowblock(a, p->elem, sc, y_dtype, s));
    } catch (...) {
        return FP4_ERR_INTERNAL;
    }
}

int fp4_hadamard(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                 int32_t hadamard_n, float* y, void* stream) {
    try {
        if (!x || !y || rows <= 0 || cols <= 0 || ldx < cols) return FP4_ERR_INVALID_ARG;
        if (x_dtype != FP4_DT_F32 && x_dtype != FP4_DT_BF16) return FP4_ERR_INVALID_ARG;
        if (!valid_hn(hadamard_n) || cols % 32 || (hadamard_n && cols % hadamard_n)) return FP4_ERR_INVALID_ARG;
        const int esz = x_dtype == FP4_DT_BF16 ? 2 : 4;
        if (!aligned(x, 16) || (ldx * esz) % 16 || !aligned(y, 16)) return FP4_ERR_ALIGNMENT;
        if (ldx != cols && !pitch_ok(ldx, esz)) return FP4_ERR_UNSUPPORTED;
        SegArgs a{};
        a.x = x;
        a.rows = rows;
        a.cols = cols;
        a.ldx = ldx;
        a.nseg = rows * (cols / 32);
        a.yrot = y;
        return hip_status(launch_segment(a, x_dtype, hadamard_n, FP4_ELEM_E2M1, SC_E8M0, FP4_ROUND_RNE,
                                         1, 32, PASS_ROTATE, reinterpret_cast<hipStream_t>(stream)));
    } catch (...) {
        return FP4_ERR_INTERNAL;
    }
}

// ---------------------------------------------------------------------------------------------
// GEMM
// ---------------------------------------------------------------------------------------------
namespace {

// 0 MXFP4, 1 MXFP8, 2 NVFP4; -1 unsupported
int gemm_kind(const fp4_qtensor* A, const fp4_qtensor* B, int* b2d) {
    const fp4_qparams &pa = A->p, &pb = B->p;
    *b2d = 0;
    if (pa.elem != pb.elem) return -1;
    const bool a_mx = scale_class(pa.scale_mode) == SC_E8M0 && pa.block_rows == 1 && pa.block_cols == 32;
    const bool b_mx = scale_class(pb.scale_mode) == SC_E8M0 && pb.block_rows == 1 && pb.block_cols == 32;
    const bool b_2d = scale_class(pb.scale_mode) == SC_E8M0 && pb.block_rows == 32 && pb.block_cols == 32;
    if (pa.elem == FP4_ELEM_E2M1 && a_mx && (b_mx || b_2d)) {
        *b2d = b_2d;
        return 0;
    }
    if (pa.elem == FP4_ELEM_E4M3 && a_mx && b_mx) return 1;
    const bool a_nv = is_nv(pa.scale_mode) && pa.block_rows == 1 && pa.block_cols == 16;
    const bool b_nv = is_nv(pb.scale_mode) && pb.block_rows == 1 && pb.block_cols == 16;
    if (pa.elem == FP4_ELEM_E2M1 && a_nv && b_nv) return 2;
    return -1;
}

int64_t gemm_ws(const fp4_qtensor* A, const fp4_qtensor* B, int kind) {
    if (kind != 2) return 0;
    auto r = [](int64_t x) { return (x + 255) / 256 * 256; };
    const int64_t K = A->cols;
    return r(A->rows * K) + r(A->rows * K / 32) + r(B->rows * K) + r(B->rows * K / 32);
}

int check_operand(const fp4_qtensor* T) {
    Layout lay;
    int rc = check_params(T->rows, T->cols, &T->p, &lay);
    if (rc != FP4_OK) return rc;
    if (!T->codes || !T->scales) return FP4_ERR_INVALID_ARG;
    if (!aligned(T->codes, 16) || !aligned(T->scales, 4)) return FP4_ERR_ALIGNMENT;
    if (is_nv(T->p.scale_mode) && !T->tensor_scale) return FP4_ERR_INVALID_ARG;
    return FP4_OK;
}

}  // namespace

int64_t fp4_gemm_workspace_bytes(const fp4_qtensor* A, const fp4_qtensor* B) {
    if (!A || !B || check_operand(A) != FP4_OK || check_operand(B) != FP4_OK) return -1;
    int b2d;
    const int kind = gemm_kind(A, B, &b2d);
    if (kind < 0) return -1;
    return gemm_ws(A, B, kind);
}

int fp4_gemm(const fp4_qtensor* A, const fp4_qtensor* B, void* C, int32_t c_dtype, int64_t ldc,
             const fp4_qparams* out_q, fp4_qtensor* C_q, void* workspace, int64_t ws_bytes,
             void* stream) {
    try {
        if (!A || !B) return FP4_ERR_INVALID_ARG;
        int rc;
        if ((rc = check_operand(A)) != FP4_OK) return rc;
        if ((rc = check_operand(B)) != FP4_OK) return rc;
        if (A->cols != B->cols) return FP4_ERR_INVALID_ARG;
        const int64_t M = A->rows, N = B->rows, K = A->cols;
        if (K % 32) return FP4_ERR_INVALID_ARG;  // operand checks already keep K a multiple of 32
        if (A->p.hadamard_n != B->p.hadamard_n) return FP4_ERR_INVALID_ARG;
        int b2d;
        const int kind = gemm_kind(A, B, &b2d);
        if (kind < 0) return FP4_ERR_UNSUPPORTED;
        // fused output quantization: MX groups of 32 along N, E8M0 floor / ceil, optional rotation
        // of C along N (n <= 128) before it
        const bool fq = out_q != nullptr;
        if (fq != (C_q != nullptr)) return FP4_ERR_INVALID_ARG;
        if (fq) {
            if (out_q->elem != FP4_ELEM_E2M1 && out_q->elem != FP4_ELEM_E4M3) return FP4_ERR_INVALID_ARG;
            if (out_q->round_mode != FP4_ROUND_RNE && out_q->round_mode != FP4_ROUND_SR) return FP4_ERR_INVALID_ARG;
            if (out_q->block_rows != 1 || out_q->block_cols != 32) return FP4_ERR_UNSUPPORTED;
            if (out_q->scale_mode != FP4_SCALE_E8M0_FLOOR && out_q->scale_mode != FP4_SCALE_E8M0_CEIL)
                return FP4_ERR_UNSUPPORTED;
            if (!valid_hn(out_q->hadamard_n)) return FP4_ERR_INVALID_ARG;
            if (out_q->hadamard_n > 128) return FP4_ERR_UNSUPPORTED;
            if (N % 32 || (out_q->hadamard_n && N % out_q->hadamard_n)) return FP4_ERR_INVALID_ARG;
            if (!C_q->codes || !C_q->scales) return FP4_ERR_INVALID_ARG;
            if (!aligned(C_q->codes, 16)) return FP4_ERR_ALIGNMENT;
        }
        if (!fq && !C) return FP4_ERR_INVALID_ARG;
        if (C) {
            if (c_dtype != FP4_DT_F32 && c_dtype != FP4_DT_BF16) return FP4_ERR_INVALID_ARG;
            if (ldc < N) return FP4_ERR_INVALID_ARG;
            if (!aligned(C, 16)) return FP4_ERR_ALIGNMENT;
        } else {
            c_dtype = FP4_DT_BF16;  // selects the kernel variant only; nothing is stored
            ldc = N;
        }
        int64_t need = gemm_ws(A, B, kind);
        // NVFP4 without a workspace: the FP8 re-expression happens in LDS (256 x 256 tile shapes)
        const bool nv_in_lds = kind == 2 && !workspace && ws_bytes == 0 && M >= 256 && N >= 256 && K % 128 == 0 &&
                               M * (K / 2) < (int64_t(1) << 31) && N * (K / 2) < (int64_t(1) << 31);
        if (nv_in_lds) need = 0;
        if (need && (!workspace || ws_bytes < need)) return FP4_ERR_WORKSPACE;
        if (need && !aligned(workspace, 256)) return FP4_ERR_ALIGNMENT;

        GemmArgs g{};
        g.a = reinterpret_cast<const uint8_t*>(A->codes);
        g.b = reinterpret_cast<const uint8_t*>(B->codes);
        g.sa = reinterpret_cast<const uint8_t*>(A->scales);
        g.sb = reinterpret_cast<const uint8_t*>(B->scales);
        g.ga = A->tensor_scale;
        g.gb = B->tensor_scale;
        g.M = M;
        g.N = N;
        g.K = K;
        g.c = C;
        g.ldc = ldc;
        g.b_2d = b2d;
        if (fq) {
            g.qcodes = reinterpret_cast<uint8_t*>(C_q->codes);
            g.qscales = reinterpret_cast<uint8_t*>(C_q->scales);
            g.q_elem = out_q->elem == FP4_ELEM_E2M1 ? ELEM_E2M1 : ELEM_E4M3;
            g.q_ceil = out_q->scale_mode == FP4_SCALE_E8M0_CEIL;
            g.q_round = out_q->round_mode == FP4_ROUND_SR ? RND_SR : RND_RNE;
            g.q_seed = out_q->seed;
            g.q_hn = out_q->hadamard_n;
            // describe what was written
            C_q->rows = M;
            C_q->cols = N;
            C_q->tensor_scale = nullptr;
            C_q->p = *out_q;
        }
        if (kind == 2 && !nv_in_lds) {
            auto r = [](int64_t x) { return (x + 255) / 256 * 256; };
            uint8_t* w = reinterpret_cast<uint8_t*>(workspace);
            g.a8 = w;
            w += r(M * K);
            g.sa8 = w;
            w += r(M * K / 32);
            g.b8 = w;
            w += r(N * K);
            g.sb8 = w;
        }
        return hip_status(launch_gemm(g, kind, c_dtype, fq ? 1 : 0, reinterpret_cast<hipStream_t>(stream)));
    } catch (...) {
        return FP4_ERR_INTERNAL;
    }
}

int64_t fp4_gemm_quantize_a_workspace_bytes(int64_t M, const fp4_qtensor* B) {
    if (M <= 0 || !B) return -1;
    return 256;  // a counter and a status word
}

int fp4_gemm_quantize_a(const void* a, int32_t a_dtype, int64_t M, int64_t lda, const fp4_qparams* pa,
                        fp4_qtensor* A_q, const fp4_qtensor* B, void* C, int32_t c_dtype, int64_t ldc,
                        void* workspace, int64_t ws_bytes, void* stream) {
    try {
        if (!a || !pa || !A_q || !B || !C) return FP4_ERR_INVALID_ARG;
        int rc = check_operand(B);
        if (rc != FP4_OK) return rc;
        const int64_t K = B->cols, N = B->rows;
        Layout lay;
        if ((rc = check_params(M, K, pa, &lay)) != FP4_OK) return rc;
        // A: MXFP4 groups along K (E8M0 floor / ceil, nearest even or stochastic), rotated like B
        if (pa->elem != FP4_ELEM_E2M1 || lay != L_SEG1D || pa->block_cols != 32 || scale_class(pa->scale_mode) != SC_E8M0)
            return FP4_ERR_UNSUPPORTED;
        if (pa->hadamard_n > 128) return FP4_ERR_UNSUPPORTED;
        if (pa->hadamard_n != B->p.hadamard_n) return FP4_ERR_INVALID_ARG;
        if (a_dtype != FP4_DT_F32 && a_dtype != FP4_DT_BF16) return FP4_ERR_INVALID_ARG;
        if (c_dtype != FP4_DT_F32 && c_dtype != FP4_DT_BF16) return FP4_ERR_INVALID_ARG;
        if (lda < K || ldc < N) return FP4_ERR_INVALID_ARG;
        if (!A_q->codes || !A_q->scales) return FP4_ERR_INVALID_ARG;
        if (A_q->codes == a || A_q->scales == a || A_q->codes == A_q->scales) return FP4_ERR_INVALID_ARG;
        const int esz = a_dtype == FP4_DT_BF16 ? 2 : 4;
        if (!aligned(a, 16) || (lda * esz) % 16 || !aligned(A_q->codes, 16) || !aligned(A_q->scales, 8) ||
            !aligned(C, 16))
            return FP4_ERR_ALIGNMENT;
        if (lda != K && !pitch_ok(lda, esz)) return FP4_ERR_UNSUPPORTED;
        fp4_qtensor Aq = *A_q;
        Aq.rows = M;
        Aq.cols = K;
        Aq.tensor_scale = nullptr;
        Aq.p = *pa;
        int b2d;
        if (gemm_kind(&Aq, B, &b2d) != 0) return FP4_ERR_UNSUPPORTED;  // B must be MXFP4 (1 x 32 or 2D)
        const int64_t need = fp4_gemm_quantize_a_workspace_bytes(M, B);
        if (!workspace || ws_bytes < need) return FP4_ERR_WORKSPACE;
        if (!aligned(workspace, 4)) return FP4_ERR_ALIGNMENT;

        hipStream_t s = reinterpret_cast<hipStream_t>(stream);
        const bool fused = M >= 256 && N >= 256 && K % 256 == 0 && M * (K / 2) < (int64_t(1) << 31) &&
                           N * (K / 2) < (int64_t(1) << 31);
        // describe what is written into A_q
        A_q->rows = M;
        A_q->cols = K;
        A_q->tensor_scale = nullptr;
        A_q->p = *pa;
        if (!fused) {  // shapes outside the 256 x 256 tile path: the quantize launch, then the GEMM
            rc = fp4_quantize(a, a_dtype, M, K, lda, pa, A_q->codes, A_q->scales, nullptr, nullptr, 0, stream);
            if (rc != FP4_OK) return rc;
            return fp4_gemm(A_q, B, C, c_dtype, ldc, nullptr, nullptr, nullptr, 0, stream);
        }
        SegArgs sa{};
        sa.x = a;
        sa.rows = M;
        sa.cols = K;
        sa.ldx = lda;
        sa.nseg = M * (K / 32);
        sa.codes = reinterpret_cast<uint8_t*>(A_q->codes);
        sa.scales = A_q->scales;
        sa.seed = pa->seed;
        sa.ceil_rule = pa->scale_mode == FP4_SCALE_E8M0_CEIL;
        GemmArgs g{};
        g.a = reinterpret_cast<const uint8_t*>(A_q->codes);
        g.b = reinterpret_cast<const uint8_t*>(B->codes);
        g.sa = reinterpret_cast<const uint8_t*>(A_q->scales);
        g.sb = reinterpret_cast<const uint8_t*>(B->scales);
        g.M = M;
        g.N = N;
        g.K = K;
        g.c = C;
        g.ldc = ldc;
        g.b_2d = b2d;
        return hip_status(launch_gemm_fused_a(g, sa, a_dtype, pa->hadamard_n,
                                              pa->round_mode == FP4_ROUND_SR ? RND_SR : RND_RNE, c_dtype,
                                              reinterpret_cast<uint32_t*>(workspace), s));
    } catch (...) {
        return FP4_ERR_INTERNAL;
    }
}

int fp4_transpose_2d(const void* codes, const void* scales, int64_t rows, int64_t cols, const fp4_qparams* p,
                     void* out_codes, void* out_scales, void* stream) {
    try {
        Layout lay;
        int rc = check_params(rows, cols, p, &lay);
        if (rc != FP4_OK) return rc;
        if (lay != L_SEG2D || p->hadamard_n != 0) return FP4_ERR_UNSUPPORTED;
        if (!codes || !scales || !out_codes || !out_scales) return FP4_ERR_INVALID_ARG;
        const void* ins[2] = {codes, scales};
        for (const void* q : ins)
            if (q == out_codes || q == out_scales) return FP4_ERR_INVALID_ARG;
        if (out_codes == out_scales) return FP4_ERR_INVALID_ARG;
        if (!aligned(codes, 16) || !aligned(out_codes, 16)) return FP4_ERR_ALIGNMENT;
        TransposeArgs t{};
        t.codes = reinterpret_cast<const uint8_t*>(codes);
        t.scales = reinterpret_cast<const uint8_t*>(scales);
        t.rows = rows;
        t.cols = cols;
        t.out_codes = reinterpret_cast<uint8_t*>(out_codes);
        t.out_scales = reinterpret_cast<uint8_t*>(out_scales);
        return hip_status(launch_transpose_2d(t, p->elem == FP4_ELEM_E2M1 ? ELEM_E2M1 : ELEM_E4M3,
                                              reinterpret_cast<hipStream_t>(stream)));
    } catch (...) {
        return FP4_ERR_INTERNAL;
    }
}

int fp4_nvfp4_to_mxfp8(const void* codes, const void* scales, int64_t rows, int64_t cols, void* out_codes,
                       void* out_scales, void* stream) {
    try {
        if (!codes || !scales || !out_codes || !out_scales || rows <= 0 || cols <= 0) return FP4_ERR_INVALID_ARG;
        if (cols % 32) return FP4_ERR_INVALID_ARG;
        if (!aligned(codes, 16) || !aligned(scales, 2) || !aligned(out_codes, 16)) return FP4_ERR_ALIGNMENT;
        const void* ins[2] = {codes, scales};
        for (const void* p : ins)
            if (p == out_codes || p == out_scales) return FP4_ERR_INVALID_ARG;
        if (out_codes == out_scales) return FP4_ERR_INVALID_ARG;
        if (rows * (cols / 32) >= (int64_t(1) << 39)) return FP4_ERR_UNSUPPORTED;  // grid size
        return hip_status(launch_nv_to_fp8(reinterpret_cast<const uint8_t*>(codes),
                                           reinterpret_cast<const uint8_t*>(scales), rows, cols,
                                           reinterpret_cast<uint8_t*>(out_codes),
                                           reinterpret_cast<uint8_t*>(out_scales),
                                           reinterpret_cast<hipStream_t>(stream)));
    } catch (...) {
        return FP4_ERR_INTERNAL;
    }
}

}  // extern "C"
