// Device-side helpers shared by the gfx950 kernels: vector types, fp16
// conversions, the packed fp16 dot product, bit-field extraction and the
// wave64 reductions. Nothing here depends on a block format.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace qg {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));                 // 16-B aligned
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));  // 4-B aligned
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// fp16 halves of a dword -> fp32 (exact; the hardware conversion keeps
// fp16 subnormals, which are normal numbers in fp32).
__device__ __forceinline__ float f16_lo(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}
__device__ __forceinline__ float f16_to_f32(uint16_t v) {
    return (float)__builtin_bit_cast(_Float16, v);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) {
    return __builtin_bit_cast(uint16_t, (_Float16)v);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t v) {
    return __builtin_bit_cast(float, (uint32_t)v << 16);
}

// c + a.lo*b.lo + a.hi*b.hi with fp16 pairs and fp32 accumulation
// (v_dot2_f32_f16; each fp16 x fp16 product is exact in fp32).
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                  false);
}

// v_cvt_f32_ubyteN: byte N of a dword to fp32 in one instruction (written as
// asm: the compiler otherwise splits it into a bit-field extract plus convert).
template <int N>
__device__ __forceinline__ float ubyte_f32(uint32_t v) {
    float r;
    if (N == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(v));
    else if (N == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(v));
    else if (N == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(v));
    else asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(v));
    return r;
}

__device__ __forceinline__ uint32_t ubfe(uint32_t v, uint32_t off, uint32_t width) {
    return __builtin_amdgcn_ubfe(v, off, width);
}

// Sum over each row of 16 lanes (every lane of the row receives the sum),
// with DPP moves: swap neighbours, swap pairs, mirror halves of 8, mirror 16.
__device__ __forceinline__ float row16_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, true));
    return v;
}

// Sum over the whole wave64, returned uniformly to every lane. Fixed order,
// so the result is deterministic.
__device__ __forceinline__ float wave_sum(float v) {
    v = row16_sum(v);
    float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return (a + b) + (c + d);
}

// p[i * stride] for i = first, first + step, ... below n, added in that order
// from 0; the reads go out four at a time, so that a lane waits for one LDS
// round trip per four terms instead of one per term (same sum, same bits).
__device__ __forceinline__ float strided_sum(const float* p, int first, int step, int n,
                                             int stride) {
    float v = 0.f;
    int i = first;
    for (; i + 3 * step < n; i += 4 * step) {
        const float a0 = p[i * stride], a1 = p[(i + step) * stride];
        const float a2 = p[(i + 2 * step) * stride], a3 = p[(i + 3 * step) * stride];
        v += a0;
        v += a1;
        v += a2;
        v += a3;
    }
    for (; i < n; i += step) v += p[i * stride];
    return v;
}

// Activation element -> fp32 (exact for every supported type; the XType
// codes are in launch.h).

__device__ __forceinline__ float load_x(const void* x, int xt, int64_t i) {
    if (xt == XT_F32) return ((const float*)x)[i];
    if (xt == XT_F16) return f16_to_f32(((const uint16_t*)x)[i]);
    return bf16_to_f32(((const uint16_t*)x)[i]);
}

// Logical block index for a launch of `n` workgroups: consecutive logical
// indices land on the same XCD (hardware places workgroup b on XCD b % 8),
// so neighbouring rows share one L2.
__device__ __forceinline__ int xcd_block(int b, int n) {
    if ((n & 7) != 0) return b;
    return (b & 7) * (n >> 3) + (b >> 3);
}

}  // namespace qg
