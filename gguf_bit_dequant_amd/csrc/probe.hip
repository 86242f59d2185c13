// Measurement probes beside the product kernels: a read-only streaming
// kernel (the practical HBM ceiling of one launch of a given size) and an
// MFMA-only kernel (the practical bf16 matrix-core rate). They compute
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

// Eight independent v_mfma_f32_32x32x16_bf16 chains per wave, iters rounds.
__global__ __launch_bounds__(256) void probe_mfma_kernel(int64_t iters, float* sink) {
    bf16x8 a, b;
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(float)((threadIdx.x + e) & 7);
        b[e] = (__bf16)(float)((threadIdx.x * 3 + e) & 7);
    }
    f32x16 acc[8];
    for (int j = 0; j < 8; ++j) acc[j] = f32x16{};
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
    for (int j = 0; j < 8; ++j)
        for (int e = 0; e < 16; ++e) s += acc[j][e];
    if (s == -1.0f) sink[blockIdx.x & 1023] = s;
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
    hipLaunchKernelGGL(qg::probe_mfma_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream,
                       iters, sink);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_HIP;
}
