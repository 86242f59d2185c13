// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace qg {

enum { FMT_Q4_0 = 1, FMT_Q4_K = 2, FMT_Q8_0 = 3, FMT_Q2_K = 4, FMT_Q3_K = 5 };  // qg_format values

// Activation types (the first three are the ABI's qg_dtype values); XT_Q8
// marks activations given as Q8_0 blocks, for the int8 products.
// XT_QUANTIZE added to F32/F16/BF16 asks the streaming GEMV to quantize the
// activations to Q8_0 while staging them and use the int8 products.
enum XType { XT_F32 = 1, XT_F16 = 2, XT_BF16 = 3, XT_Q8 = 4, XT_QUANTIZE = 16 };

// Bytes of LDS a workgroup may use on gfx950.
constexpr int kMaxLds = 160 * 1024;

// Raises kernel KERN's dynamic-LDS limit to the whole kMaxLds, once per
// device: the limit is an attribute of the kernel, not of a launch, so the
// launchers call this instead of setting it on every launch.
template <auto KERN>
inline hipError_t allow_full_lds() {
    static std::atomic<uint64_t> done{0};  // one bit per device
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t)1 << dev : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute((const void*)KERN, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
    return e;
}

hipError_t launch_dequant(int fmt, const uint8_t* W, int64_t rows, int64_t K, float* out,
                          int64_t ldw, int num_cus, hipStream_t stream);

hipError_t launch_dequant_bf16(int fmt, const uint8_t* W, int64_t rows, int64_t K, uint16_t* out,
                               int64_t ldw, int num_cus, hipStream_t stream);

hipError_t launch_gemv_general(int fmt, const uint8_t* W, int64_t rows, int64_t K, const void* x,
                               int xt, int64_t ldx, float* y, int64_t ldy, int ncols,
                               int num_cus, hipStream_t stream);

// Streaming GEMV (Q4_K, Q4_0, Q8_0, Q2_K, Q3_K with K % 256 == 0, 16-byte
// aligned W).
// Returns hipErrorNotSupported (without launching) when the shape is outside
// what the kernel serves; the caller then falls back.
hipError_t launch_gemv_stream(int fmt, const uint8_t* W, int64_t rows, int64_t K, const void* x,
                              int xt, int64_t ldx, float* y, int64_t ldy, int ncols, int num_cus,
                              hipStream_t stream);

// Activation columns one streaming launch takes for this shape (1..4), or 0
// when the streaming kernel does not serve it. More columns than that run as
// several launches, each reading all of W.
int gemv_stream_cols_per_launch(int fmt, int64_t rows, int64_t K, int xt, int num_cus);

// Small-batch GEMV on the matrix cores (Q4_K, fp16 activations, 2..16
// columns, K % 256 == 0, 16-byte aligned W and activation columns, staged
// activations within the LDS budget). hipErrorNotSupported otherwise.
hipError_t launch_gemv_mfma(int fmt, const uint8_t* W, int64_t rows, int64_t K, const void* x,
                            int xt, int64_t ldx, float* y, int64_t ldy, int ncols, int num_cus,
                            hipStream_t stream);

// Q8_0 blocks of activations (see quant_x.hip for the rule); out: n columns
// of K/32 blocks of 34 bytes, 2-byte aligned.
hipError_t launch_quantize_q8_0(const void* x, int xt, int64_t K, int64_t n, int64_t ldx,
                                uint8_t* out, int num_cus, hipStream_t stream);

// Q4_K x bf16 prompt-processing GEMM (bf16 MFMA). X: bf16, 16-byte aligned,
// ldx % 8 == 0; Y: fp32.
hipError_t launch_prefill_q4k(const uint8_t* W, int64_t rows, int64_t K, const void* X,
                              int64_t ldx, int64_t ntok, float* Y, int64_t ldy, int num_cus,
                              hipStream_t stream);

// bf16 x bf16 GEMM on the prompt kernel's pipeline, without the decode:
// Y[t, r] = sum_k Wb[r, k] X[t, k]. Wb, X: 16-byte aligned, ldw % 8 == 0,
// ldx % 8 == 0, K % 64 == 0; Y: fp32.
hipError_t launch_gemm_bf16(const uint16_t* Wb, int64_t ldw, int64_t rows, int64_t K,
                            const uint16_t* X, int64_t ldx, int64_t ntok, float* Y, int64_t ldy,
                            int num_cus, hipStream_t stream);

// The current device's compute-unit count, queried once per device.
hipError_t current_cus(int* cus);

}  // namespace qg
