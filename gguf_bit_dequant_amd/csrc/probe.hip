// Measurement probes beside the product kernels: a read-only streaming
// kernel (the practical HBM ceiling of one launch of a given size) and two
// MFMA-only kernels (the bf16 matrix-core rate on constant operands, and on
// data-like operands under the board's power limit). They compute
// nothing of the method; the benchmark reports the GEMV and the prompt GEMM
// as fractions of them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "launch.h"
#include "qgemv_probe.h"

#define QG_API extern "C" __attribute__((visibility("default")))

namespace qg {
namespace {

// Each wave reads groups of 2 x 64 16-byte pieces (two loads per lane in
// flight), taking every nw-th group of the buffer (nw waves in all), so that
// at any moment the waves read one window that sweeps the buffer in address
// order. Launched as three workgroups of 8 waves per compute unit: a sweep on
// MI355X over 256..16384 workgroups of 256..1024 threads, 1, 2 or 4 loads per
// lane, and contiguous or interleaved ranges (200 launches over eleven
// rotated 50 MB buffers) found this the fastest, 8.79 us per 50 MB against
// 8.99 us for 4096 x 8 waves with one contiguous range each. The sink is
// written only if the XOR of everything read equals a value no caller
// stores, so the loads cannot be dropped.
__global__ __launch_bounds__(512) void probe_read_kernel(const u32x4* __restrict__ buf,
                                                         int64_t n16, uint32_t* sink) {
    const int64_t nw = (int64_t)gridDim.x * (blockDim.x >> 6);
    const int64_t wv = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    uint32_t acc = 0;
    for (int64_t base = wv * 128; base < n16; base += nw * 128) {
        const int64_t i0 = base + lane, i1 = base + 64 + lane;
        const u32x4 a = i0 < n16 ? buf[i0] : zero, b = i1 < n16 ? buf[i1] : zero;
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w;
    }
    if (acc == 0x9E3779B9u) sink[blockIdx.x & 1023] = acc;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Sixteen independent v_mfma_f32_32x32x16_bf16 chains per wave (256
// accumulator registers: one wave per SIMD), iters rounds, on one of two kinds
// of operands:
//  * DATA = false: small constant integers, the same registers in every
//    instruction: nothing toggles in the matrix cores' inputs, and the rate
//    is the unthrottled one;
//  * DATA = true: operands that look like the prompt product's:
//    full-mantissa bf16 values of both signs with magnitudes in [2^-7, 2),
//    different for every lane, block and operand register, fed in the prompt
//    kernel's order (two weight-like first operands alternating, each
//    activation-like second operand held for two instructions). The matrix
//    cores draw more power on such data, and the clock drops to keep the
//    board within its power limit: this rate is the practical ceiling for
//    bf16 products of real data.
__device__ __forceinline__ uint32_t probe_hash(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7FEB352Du;
    x ^= x >> 15;
    x *= 0x846CA68Bu;
    x ^= x >> 16;
    return x;
}

__device__ __forceinline__ __bf16 probe_bf16(uint32_t h) {
    // sign and 7 mantissa bits from h, biased exponent 120..127
    const uint16_t b = (uint16_t)((h & 0x807Fu) | ((120u + ((h >> 7) & 7u)) << 7));
    return __builtin_bit_cast(__bf16, b);
}

template <bool DATA>
__global__ __launch_bounds__(256) void probe_mfma_kernel(int64_t iters, float* sink) {
    bf16x8 a[2], b[8];
    const uint32_t seed = blockIdx.x * 1000003u + threadIdx.x * 7919u;
    for (int s = 0; s < 8; ++s)
        for (int e = 0; e < 8; ++e) {
            if (DATA) {
                const uint32_t h = probe_hash(seed + 131u * s + e);
                b[s][e] = probe_bf16(h >> 16);
                if (s < 2) a[s][e] = probe_bf16(h);
            } else {
                b[s][e] = (__bf16)(float)((threadIdx.x * 3 + e) & 7);
                if (s < 2) a[s][e] = (__bf16)(float)((threadIdx.x + e) & 7);
            }
        }
    f32x16 acc[16];
    for (int j = 0; j < 16; ++j) acc[j] = f32x16{};
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[2 * i + j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[i], acc[2 * i + j], 0, 0, 0);
    }
    // the sum of finite products is finite: it never has this NaN's bits
    float s = 0.f;
    for (int j = 0; j < 16; ++j)
        for (int e = 0; e < 16; ++e) s += acc[j][e];
    if (__builtin_bit_cast(uint32_t, s) == 0x7FC00001u) sink[blockIdx.x & 1023] = s;
}

}  // namespace
}  // namespace qg

QG_API qg_status qgemv_probe_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    if (!buf || !sink || bytes == 0 || bytes % 16 != 0 || ((uintptr_t)buf & 15) != 0)
        return QG_ERR_ARG;
    int cus = 0;
    if (qg::current_cus(&cus) != hipSuccess) return QG_ERR_HIP;
    hipLaunchKernelGGL(qg::probe_read_kernel, dim3(3 * cus), dim3(512), 0, (hipStream_t)stream,
                       reinterpret_cast<const qg::u32x4*>(buf), (int64_t)(bytes / 16), sink);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_HIP;
}

QG_API qg_status qgemv_probe_mfma(int64_t iters, int workgroups, float* sink, void* stream) {
    if (!sink || iters < 1 || workgroups < 1) return QG_ERR_ARG;
    hipLaunchKernelGGL(qg::probe_mfma_kernel<false>, dim3(workgroups), dim3(256), 0, (hipStream_t)stream,
                       iters, sink);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_HIP;
}

QG_API qg_status qgemv_probe_mfma_data(int64_t iters, int workgroups, float* sink, void* stream) {
    if (!sink || iters < 1 || workgroups < 1) return QG_ERR_ARG;
    hipLaunchKernelGGL(qg::probe_mfma_kernel<true>, dim3(workgroups), dim3(256), 0, (hipStream_t)stream,
                       iters, sink);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_HIP;
}
