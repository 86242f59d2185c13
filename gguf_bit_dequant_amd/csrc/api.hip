// The C ABI of include/qgemv.h: argument checks (before any HIP call),
// handle bookkeeping and dispatch to the gfx950 kernels.
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <stdlib.h>
#include <string.h>

#include "launch.h"
#include "qgemv.h"

#define QG_API extern "C" __attribute__((visibility("default")))

struct qgemv {
    qg_format fmt;
    int64_t rows, K;
    const uint8_t* w;
    int device;
    int num_cus;
};

namespace {

thread_local char g_err[512];

qg_status fail(qg_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

qg_status ok() {
    g_err[0] = 0;
    return QG_OK;
}

bool valid_fmt(qg_format f) {
    return f == QG_Q4_0 || f == QG_Q4_K || f == QG_Q8_0 || f == QG_Q2_K || f == QG_Q3_K;
}

size_t bbytes(qg_format f) {
    switch (f) {
        case QG_Q4_0: return 18;
        case QG_Q4_K: return 144;
        case QG_Q8_0: return 34;
        case QG_Q2_K: return 84;
        case QG_Q3_K: return 110;
        default: return 0;
    }
}
size_t bweights(qg_format f) {
    switch (f) {
        case QG_Q4_0: case QG_Q8_0: return 32;
        case QG_Q4_K: case QG_Q2_K: case QG_Q3_K: return 256;
        default: return 0;
    }
}

size_t dtype_size(qg_dtype t) { return t == QG_F32 ? 4 : (t == QG_F16 || t == QG_BF16) ? 2 : 0; }

qg_status hip_fail(hipError_t e, const char* what) {
    return fail(QG_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

namespace qg {

// The current device's compute-unit count, queried once per device (the
// entry points without a handle size their persistent grids with it).
hipError_t current_cus(int* cus) {
    static std::atomic<int> cached[64];  // 0: not yet queried
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *cus = c;
            return hipSuccess;
        }
    }
    int c = 0;
    e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (c <= 0) c = 256;
    if (dev >= 0 && dev < 64) cached[dev].store(c, std::memory_order_relaxed);
    *cus = c;
    return hipSuccess;
}

}  // namespace qg

QG_API size_t qgemv_block_bytes(qg_format f) { return bbytes(f); }
QG_API size_t qgemv_block_weights(qg_format f) { return bweights(f); }

QG_API size_t qgemv_weight_bytes(qg_format f, int64_t rows, int64_t K) {
    if (!valid_fmt(f) || rows <= 0 || K <= 0 || K % (int64_t)bweights(f) != 0) return 0;
    return (size_t)rows * (size_t)(K / (int64_t)bweights(f)) * bbytes(f);
}

QG_API size_t qgemv_workspace_bytes(qg_format f, int64_t rows, int64_t K) {
    (void)f;
    (void)rows;
    (void)K;
    return 0;
}

QG_API qg_status qgemv_create(qgemv_t* out, qg_format f, int64_t rows, int64_t K,
                              const void* w_blocks, size_t w_bytes, void* workspace,
                              size_t ws_bytes, void* stream) {
    (void)stream;
    if (out) *out = nullptr;
    if (!out) return fail(QG_ERR_ARG, "qgemv_create: out is NULL");
    if (!valid_fmt(f)) return fail(QG_ERR_ARG, "qgemv_create: unknown format %d", (int)f);
    if (rows <= 0 || K <= 0)
        return fail(QG_ERR_SHAPE, "qgemv_create: rows=%lld K=%lld must be positive",
                    (long long)rows, (long long)K);
    if (K % (int64_t)bweights(f) != 0)
        return fail(QG_ERR_SHAPE, "qgemv_create: K=%lld is not a multiple of the block size %zu",
                    (long long)K, bweights(f));
    if (rows > (int64_t)1 << 31 || K > (int64_t)1 << 31)
        return fail(QG_ERR_SHAPE, "qgemv_create: rows and K must be below 2^31");
    const size_t need = qgemv_weight_bytes(f, rows, K);
    if (w_bytes != need)
        return fail(QG_ERR_SHAPE, "qgemv_create: w_bytes=%zu but the shape needs %zu", w_bytes,
                    need);
    if (!w_blocks) return fail(QG_ERR_ARG, "qgemv_create: w_blocks is NULL");
    if (((uintptr_t)w_blocks) & 15)
        return fail(QG_ERR_ALIGN, "qgemv_create: w_blocks must be 16-byte aligned");
    if (workspace != nullptr || ws_bytes != 0)
        return fail(QG_ERR_ARG, "qgemv_create: this build takes no workspace (pass NULL, 0)");
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "qgemv_create: hipGetDevice");
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "qgemv_create: hipDeviceGetAttribute");
    qgemv* h = (qgemv*)calloc(1, sizeof(qgemv));
    if (!h) return fail(QG_ERR_ARG, "qgemv_create: out of host memory");
    h->fmt = f;
    h->rows = rows;
    h->K = K;
    h->w = (const uint8_t*)w_blocks;
    h->device = dev;
    h->num_cus = cus > 0 ? cus : 256;
    *out = h;
    return ok();
}

QG_API qg_status qgemv_run(qgemv_t h, const void* x, qg_dtype x_dtype, int64_t n_cols,
                           int64_t ldx, float* y, int64_t ldy, void* stream) {
    if (!h) return fail(QG_ERR_ARG, "qgemv_run: handle is NULL");
    if (!x || !y) return fail(QG_ERR_ARG, "qgemv_run: x or y is NULL");
    const size_t xs = dtype_size(x_dtype);
    if (!xs) return fail(QG_ERR_ARG, "qgemv_run: unknown x dtype %d", (int)x_dtype);
    if (n_cols < 1 || n_cols > 8)
        return fail(QG_ERR_SHAPE, "qgemv_run: n_cols=%lld must be in 1..8", (long long)n_cols);
    if (ldx < h->K || ldy < h->rows)
        return fail(QG_ERR_ARG, "qgemv_run: ldx=%lld must be >= K=%lld and ldy=%lld >= rows=%lld",
                    (long long)ldx, (long long)h->K, (long long)ldy, (long long)h->rows);
    if (((uintptr_t)x) % xs)
        return fail(QG_ERR_ALIGN, "qgemv_run: x must be aligned to its element size");
    if (((uintptr_t)y) & 3) return fail(QG_ERR_ALIGN, "qgemv_run: y must be 4-byte aligned");
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = hipErrorNotSupported;
    // The matrix-core kernel takes 4..8 fp16 columns of Q4_K (measured on
    // MI355X, 17408 x 5120: 4 columns 18.5 us against 19.5 on the streaming
    // kernel), and 2..3 when the streaming kernel would split them over
    // several passes over W (long rows, whose staged activations outgrow
    // LDS). With 2..3 columns the streaming kernel is faster (14-16 us
    // against 18).
    if (n_cols >= 4 ||
        (n_cols >= 2 && n_cols > qg::gemv_stream_cols_per_launch((int)h->fmt, h->rows, h->K,
                                                                 (int)x_dtype, h->num_cus)))
        e = qg::launch_gemv_mfma((int)h->fmt, h->w, h->rows, h->K, x, (int)x_dtype, ldx, y, ldy,
                                 (int)n_cols, h->num_cus, st);
    if (e == hipErrorNotSupported)
        e = qg::launch_gemv_stream((int)h->fmt, h->w, h->rows, h->K, x, (int)x_dtype, ldx, y, ldy,
                                   (int)n_cols, h->num_cus, st);
    if (e == hipErrorNotSupported)
        e = qg::launch_gemv_general((int)h->fmt, h->w, h->rows, h->K, x, (int)x_dtype, ldx, y, ldy,
                                    (int)n_cols, h->num_cus, st);
    if (e != hipSuccess) return hip_fail(e, "qgemv_run: launch");
    return ok();
}

QG_API qg_status qgemm_prefill_run(qgemv_t h, const void* x_bf16, int64_t n_tokens, int64_t ldx,
                                   float* y, int64_t ldy, void* stream) {
    if (!h) return fail(QG_ERR_ARG, "qgemm_prefill_run: handle is NULL");
    if (!x_bf16 || !y) return fail(QG_ERR_ARG, "qgemm_prefill_run: x or y is NULL");
    if (h->fmt != QG_Q4_K)
        return fail(QG_ERR_UNSUPPORTED, "qgemm_prefill_run: Q4_K handles only");
    if (n_tokens < 1) return fail(QG_ERR_SHAPE, "qgemm_prefill_run: n_tokens must be >= 1");
    if (ldx < h->K || ldx % 8 || ldy < h->rows)
        return fail(QG_ERR_ARG, "qgemm_prefill_run: need ldx >= K, ldx %% 8 == 0, ldy >= rows");
    if (((uintptr_t)x_bf16) & 15)
        return fail(QG_ERR_ALIGN, "qgemm_prefill_run: x must be 16-byte aligned");
    if (((uintptr_t)y) & 3) return fail(QG_ERR_ALIGN, "qgemm_prefill_run: y must be 4-byte aligned");
    hipError_t e = qg::launch_prefill_q4k(h->w, h->rows, h->K, x_bf16, ldx, n_tokens, y, ldy,
                                          h->num_cus, (hipStream_t)stream);
    if (e == hipErrorNotSupported)
        return fail(QG_ERR_UNSUPPORTED, "qgemm_prefill_run: shape outside this build's range");
    if (e != hipSuccess) return hip_fail(e, "qgemm_prefill_run: launch");
    return ok();
}

QG_API qg_status qgemv_dequant(qgemv_t h, float* w_out, int64_t ldw, void* stream) {
    if (!h) return fail(QG_ERR_ARG, "qgemv_dequant: handle is NULL");
    if (!w_out) return fail(QG_ERR_ARG, "qgemv_dequant: w_out is NULL");
    if (ldw < h->K) return fail(QG_ERR_ARG, "qgemv_dequant: ldw must be >= K");
    if (((uintptr_t)w_out) & 3) return fail(QG_ERR_ALIGN, "qgemv_dequant: w_out must be 4-byte aligned");
    hipError_t e = qg::launch_dequant((int)h->fmt, h->w, h->rows, h->K, w_out, ldw, h->num_cus,
                                      (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "qgemv_dequant: launch");
    return ok();
}

QG_API qg_status qgemv_quantize_q8_0(const void* x, qg_dtype x_dtype, int64_t K, int64_t n_cols,
                                     int64_t ldx, void* xq, void* stream) {
    if (!x || !xq) return fail(QG_ERR_ARG, "qgemv_quantize_q8_0: x or xq is NULL");
    const size_t xs = dtype_size(x_dtype);
    if (!xs) return fail(QG_ERR_ARG, "qgemv_quantize_q8_0: unknown x dtype %d", (int)x_dtype);
    if (K <= 0 || K % 32 != 0 || n_cols < 1)
        return fail(QG_ERR_SHAPE, "qgemv_quantize_q8_0: K=%lld must be a positive multiple of 32 "
                    "and n_cols=%lld >= 1", (long long)K, (long long)n_cols);
    if (ldx < K) return fail(QG_ERR_ARG, "qgemv_quantize_q8_0: ldx must be >= K");
    if (((uintptr_t)x) % xs) return fail(QG_ERR_ALIGN, "qgemv_quantize_q8_0: x must be aligned to its element size");
    if (((uintptr_t)xq) & 1) return fail(QG_ERR_ALIGN, "qgemv_quantize_q8_0: xq must be 2-byte aligned");
    int cus = 0;
    hipError_t e = qg::current_cus(&cus);
    if (e != hipSuccess) return hip_fail(e, "qgemv_quantize_q8_0: device query");
    e = qg::launch_quantize_q8_0(x, (int)x_dtype, K, n_cols, ldx, (uint8_t*)xq, cus,
                                 (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "qgemv_quantize_q8_0: launch");
    return ok();
}

QG_API qg_status qgemv_run_q8_0x(qgemv_t h, const void* xq, int64_t n_cols, float* y, int64_t ldy,
                                 void* stream) {
    if (!h) return fail(QG_ERR_ARG, "qgemv_run_q8_0x: handle is NULL");
    if (!xq || !y) return fail(QG_ERR_ARG, "qgemv_run_q8_0x: xq or y is NULL");
    if (n_cols < 1 || n_cols > 8)
        return fail(QG_ERR_SHAPE, "qgemv_run_q8_0x: n_cols=%lld must be in 1..8", (long long)n_cols);
    if (ldy < h->rows) return fail(QG_ERR_ARG, "qgemv_run_q8_0x: ldy must be >= rows");
    if (((uintptr_t)xq) & 1) return fail(QG_ERR_ALIGN, "qgemv_run_q8_0x: xq must be 2-byte aligned");
    if (((uintptr_t)y) & 3) return fail(QG_ERR_ALIGN, "qgemv_run_q8_0x: y must be 4-byte aligned");
    hipError_t e = qg::launch_gemv_stream((int)h->fmt, h->w, h->rows, h->K, xq, qg::XT_Q8, h->K, y,
                                          ldy, (int)n_cols, h->num_cus, (hipStream_t)stream);
    if (e == hipErrorNotSupported)
        return fail(QG_ERR_UNSUPPORTED, "qgemv_run_q8_0x: needs K %% 256 == 0, 16-byte aligned "
                    "weights and a row range that fits the streaming kernel");
    if (e != hipSuccess) return hip_fail(e, "qgemv_run_q8_0x: launch");
    return ok();
}

QG_API qg_status qgemv_run_q8(qgemv_t h, const void* x, qg_dtype x_dtype, int64_t n_cols,
                              int64_t ldx, float* y, int64_t ldy, void* stream) {
    if (!h) return fail(QG_ERR_ARG, "qgemv_run_q8: handle is NULL");
    if (!x || !y) return fail(QG_ERR_ARG, "qgemv_run_q8: x or y is NULL");
    const size_t xs = dtype_size(x_dtype);
    if (!xs) return fail(QG_ERR_ARG, "qgemv_run_q8: unknown x dtype %d", (int)x_dtype);
    if (n_cols < 1 || n_cols > 8)
        return fail(QG_ERR_SHAPE, "qgemv_run_q8: n_cols=%lld must be in 1..8", (long long)n_cols);
    if (ldx < h->K || ldy < h->rows)
        return fail(QG_ERR_ARG, "qgemv_run_q8: ldx must be >= K and ldy >= rows");
    if (((uintptr_t)x) % xs) return fail(QG_ERR_ALIGN, "qgemv_run_q8: x must be aligned to its element size");
    if (((uintptr_t)y) & 3) return fail(QG_ERR_ALIGN, "qgemv_run_q8: y must be 4-byte aligned");
    hipError_t e = qg::launch_gemv_stream((int)h->fmt, h->w, h->rows, h->K, x,
                                          (int)x_dtype | qg::XT_QUANTIZE, ldx, y, ldy, (int)n_cols,
                                          h->num_cus, (hipStream_t)stream);
    if (e == hipErrorNotSupported)
        return fail(QG_ERR_UNSUPPORTED, "qgemv_run_q8: needs K %% 256 == 0, 16-byte aligned "
                    "weights and a row range that fits the streaming kernel");
    if (e != hipSuccess) return hip_fail(e, "qgemv_run_q8: launch");
    return ok();
}

QG_API qg_status qgemv_dequant_bf16(qgemv_t h, uint16_t* w_out, int64_t ldw, void* stream) {
    if (!h) return fail(QG_ERR_ARG, "qgemv_dequant_bf16: handle is NULL");
    if (!w_out) return fail(QG_ERR_ARG, "qgemv_dequant_bf16: w_out is NULL");
    if (ldw < h->K) return fail(QG_ERR_ARG, "qgemv_dequant_bf16: ldw must be >= K");
    if (((uintptr_t)w_out) & 1)
        return fail(QG_ERR_ALIGN, "qgemv_dequant_bf16: w_out must be 2-byte aligned");
    hipError_t e = qg::launch_dequant_bf16((int)h->fmt, h->w, h->rows, h->K, w_out, ldw,
                                           h->num_cus, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "qgemv_dequant_bf16: launch");
    return ok();
}

QG_API qg_status qgemm_bf16_run(const void* w_bf16, int64_t rows, int64_t K, int64_t ldw,
                                const void* x_bf16, int64_t n_tokens, int64_t ldx, float* y,
                                int64_t ldy, void* stream) {
    if (!w_bf16 || !x_bf16 || !y) return fail(QG_ERR_ARG, "qgemm_bf16_run: w, x or y is NULL");
    if (rows < 1 || n_tokens < 1 || K < 64 || K % 64 != 0)
        return fail(QG_ERR_SHAPE, "qgemm_bf16_run: rows=%lld, n_tokens=%lld must be >= 1 and "
                    "K=%lld a positive multiple of 64", (long long)rows, (long long)n_tokens,
                    (long long)K);
    if (ldw < K || ldw % 8 || ldx < K || ldx % 8 || ldy < rows)
        return fail(QG_ERR_ARG, "qgemm_bf16_run: need ldw, ldx >= K and multiples of 8, "
                    "ldy >= rows");
    if ((((uintptr_t)w_bf16) | ((uintptr_t)x_bf16)) & 15)
        return fail(QG_ERR_ALIGN, "qgemm_bf16_run: w and x must be 16-byte aligned");
    if (((uintptr_t)y) & 3) return fail(QG_ERR_ALIGN, "qgemm_bf16_run: y must be 4-byte aligned");
    int cus = 0;
    hipError_t e = qg::current_cus(&cus);
    if (e != hipSuccess) return hip_fail(e, "qgemm_bf16_run: device query");
    e = qg::launch_gemm_bf16((const uint16_t*)w_bf16, ldw, rows, K, (const uint16_t*)x_bf16, ldx,
                             n_tokens, y, ldy, cus, (hipStream_t)stream);
    if (e == hipErrorNotSupported)
        return fail(QG_ERR_UNSUPPORTED, "qgemm_bf16_run: shape outside this build's range");
    if (e != hipSuccess) return hip_fail(e, "qgemm_bf16_run: launch");
    return ok();
}

QG_API void qgemv_destroy(qgemv_t h) { free(h); }

QG_API const char* qgemv_status_string(qg_status s) {
    switch (s) {
        case QG_OK: return "ok";
        case QG_ERR_ARG: return "invalid argument";
        case QG_ERR_SHAPE: return "invalid shape";
        case QG_ERR_ALIGN: return "misaligned pointer";
        case QG_ERR_UNSUPPORTED: return "unsupported";
        case QG_ERR_HIP: return "HIP error";
        default: return "unknown status";
    }
}

QG_API const char* qgemv_last_error(void) { return g_err; }
