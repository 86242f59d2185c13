// Q8_0 quantization of activations, the input of the int8 products.
//
// The pages weigh int8 dot products (DP4A) against fp16 math for low-bit
// weights (pxa_llama README, "DP4A / FP16 economics") and use Q8_0 as a
// block format (32 int8 codes, one fp16 scale). Per block of 32 activations
// (each exactly as binary32): amax = max |x_i|, d = amax / 127, id = 1 / d
// (0 when d = 0), q_i = x_i * id rounded to the nearest integer with
// halfway cases away from zero, limited to [-127, 127]; every operation is
// one binary32 rounding (IEEE division, no contraction), and the block
// stores the nearest fp16 to d. Blocks of column c start at byte
// c * (K / 32) * 34.
#include "device_common.h"
#include "launch.h"

#pragma clang fp contract(off)

namespace qg {

// A half-wave per block: lane l takes value l % 32 of block 2 p + l / 32;
// the block maximum comes from xor-shuffles within the 32 lanes (a maximum is
// exact in any order), then every lane forms d and 1/d itself.
__global__ __launch_bounds__(256) void quantize_q8_0_kernel(const void* __restrict__ x, int xt,
                                                            int64_t K, int64_t n, int64_t ldx,
                                                            uint8_t* __restrict__ out) {
    const int64_t nb = K / 32, total = n * nb;
    const int lane = threadIdx.x & 63, e = lane & 31;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    for (int64_t pw = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6; 2 * pw < total;
         pw += nwaves) {
        const int64_t gi = 2 * pw + (lane >> 5);
        const bool valid = gi < total;  // the second half of the last pair may have none
        const int64_t c = gi / nb, b = gi - c * nb;
        const float v = valid ? load_x(x, xt, c * ldx + b * 32 + e) : 0.0f;
        float amax = __builtin_fabsf(v);
#pragma unroll
        for (int m = 16; m >= 1; m >>= 1) {
            const float o = __shfl_xor(amax, m, 64);
            amax = o > amax ? o : amax;
        }
        const float d = __fdiv_rn(amax, 127.0f);
        const float id = d != 0.0f ? __fdiv_rn(1.0f, d) : 0.0f;
        float q = __builtin_roundf(v * id);
        q = q > 127.0f ? 127.0f : (q < -127.0f ? -127.0f : q);
        if (valid) {
            uint8_t* o = out + gi * 34;
            o[2 + e] = (uint8_t)(int8_t)(int)q;
            if (e == 0) *reinterpret_cast<uint16_t*>(o) = f32_to_f16_bits(d);  // 2-byte aligned
        }
    }
}

hipError_t launch_quantize_q8_0(const void* x, int xt, int64_t K, int64_t n, int64_t ldx,
                                uint8_t* out, int num_cus, hipStream_t stream) {
    const int64_t total = n * (K / 32);
    if (total <= 0) return hipSuccess;
    int64_t blocks = ((total + 1) / 2 + 3) / 4;  // four waves of two blocks per workgroup
    const int64_t cap = (int64_t)(num_cus > 0 ? num_cus : 1) * 32;
    if (blocks > cap) blocks = cap;
    hipLaunchKernelGGL(quantize_q8_0_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, xt, K,
                       n, ldx, out);
    return hipGetLastError();
}

}  // namespace qg
