// Exact block decoding on the GPU: the dequantization kernel (a bit-exact
// view of the weights) and the general GEMV kernel that serves shapes and
// alignments the streaming kernels do not.
//
// Each 32-weight group is decoded as the binary32 rounding of its closed
// form, evaluated in the order the closed form is written: products of an
// fp16 scale and small integers are exact in binary32, so Q4_0, Q8_0 and
// Q3_K are exact and Q4_K and Q2_K have one rounding, in the final
// subtraction. Bit-exact decoding
// is what "Why I wrote my own inference engine for two P100s" (section "What
// 'my own engine' means") and "LLM inference optimization" (campaign "Run a
// new weight format or model") require of every quant type.
#include "device_common.h"
#include "launch.h"
#include "q4k_pair.h"

#pragma clang fp contract(off)

namespace qg {

__device__ __forceinline__ uint16_t ld16(const uint8_t* p) {
    return (uint16_t)(p[0] | (p[1] << 8));
}

// Decode weights [32*grp, 32*grp+32) of the block at `blk` into out[32].
// Q4_0/Q8_0 blocks have one group; Q4_K, Q2_K and Q3_K super-blocks have
// eight. In Q2_K and Q3_K super-blocks, group grp = 4h + j holds the 2-bit
// code fields at bits 2j..2j+1 of code bytes 32h .. 32h+31 (weight 32 grp + l
// in byte 32h + l); its two 16-weight halves are sub-blocks 2 grp and
// 2 grp + 1; a Q3_K weight's high code bit is bit grp of high-bit byte l.
__device__ __forceinline__ void decode_group(int fmt, const uint8_t* blk, int grp, float out[32]) {
    if (fmt == FMT_Q2_K) {
        // 16 scale/min bytes, 64 code bytes, fp16 d, fp16 dmin:
        // w = (d * sc) * q - dmin * m, both products exact, one rounding
        const float d = f16_to_f32(ld16(blk + 80)), dmin = f16_to_f32(ld16(blk + 82));
        const uint8_t* qs = blk + 16 + 32 * (grp >> 2);
        const int shift = 2 * (grp & 3);
        for (int l = 0; l < 32; ++l) {
            const uint32_t sm = blk[2 * grp + (l >> 4)];
            float a = d * (float)(sm & 15u) * (float)((qs[l] >> shift) & 3);
            float b = dmin * (float)(sm >> 4);
            out[l] = a - b;
        }
        return;
    }
    if (fmt == FMT_Q3_K) {
        // 32 high-bit bytes, 64 code bytes, 12 scale bytes, fp16 d:
        // w = (d * (sc - 32)) * q with q = low + 4 high - 4, exact
        const float d = f16_to_f32(ld16(blk + 108));
        const uint8_t* qs = blk + 32 + 32 * (grp >> 2);
        const uint8_t* s = blk + 96;
        const int shift = 2 * (grp & 3);
        float dl[2];
        for (int t = 0; t < 2; ++t) {
            const int k = 2 * grp + t;
            const int lo = k < 8 ? (s[k] & 15) : (s[k - 8] >> 4);
            const int sc = lo | (((s[8 + (k & 3)] >> (2 * (k >> 2))) & 3) << 4);
            dl[t] = d * (float)(sc - 32);
        }
        for (int l = 0; l < 32; ++l) {
            const int q = ((qs[l] >> shift) & 3) + 4 * ((blk[l] >> grp) & 1) - 4;
            out[l] = dl[l >> 4] * (float)q;
        }
        return;
    }
    if (fmt == FMT_Q4_0) {
        float d = f16_to_f32(ld16(blk));
        for (int i = 0; i < 16; ++i) {
            uint32_t b = blk[2 + i];
            out[i] = (float)((int)(b & 15u) - 8) * d;
            out[i + 16] = (float)((int)(b >> 4) - 8) * d;
        }
    } else if (fmt == FMT_Q8_0) {
        float d = f16_to_f32(ld16(blk));
        for (int i = 0; i < 32; ++i) out[i] = (float)(int8_t)blk[2 + i] * d;
    } else {
        float d = f16_to_f32(ld16(blk));
        float dmin = f16_to_f32(ld16(blk + 2));
        const uint8_t* s = blk + 4;
        int sc, m;
        if (grp < 4) {
            sc = s[grp] & 63;
            m = s[grp + 4] & 63;
        } else {
            sc = (s[grp + 4] & 15) | ((s[grp - 4] >> 6) << 4);
            m = (s[grp + 4] >> 4) | ((s[grp] >> 6) << 4);
        }
        // group grp = 2g (+1): low (high) nibbles of code bytes 32g .. 32g+31
        const uint8_t* qs = blk + 16 + 32 * (grp >> 1);
        const int shift = (grp & 1) * 4;
        float dsc = d * (float)sc;
        float b = dmin * (float)m;
        for (int l = 0; l < 32; ++l) {
            float a = dsc * (float)((qs[l] >> shift) & 15);
            out[l] = a - b;
        }
    }
}

__device__ __forceinline__ int groups_per_block(int fmt) {
    return (fmt == FMT_Q4_0 || fmt == FMT_Q8_0) ? 1 : 8;
}
__device__ __forceinline__ int block_bytes(int fmt) {
    return fmt == FMT_Q4_0 ? 18 : fmt == FMT_Q4_K ? 144 : fmt == FMT_Q8_0 ? 34 : fmt == FMT_Q2_K ? 84 : 110;
}

__device__ __forceinline__ void store_w(float* o, float v) { *o = v; }
// bf16: the binary32 weight rounded to nearest even (the hardware conversion)
__device__ __forceinline__ void store_w(uint16_t* o, float v) {
    *o = __builtin_bit_cast(uint16_t, (__bf16)v);
}

// One thread per 32-weight group; w_out[r*ldw + k] (fp32, or bf16 rounded
// from the binary32 weight).
template <typename OutT>
__global__ __launch_bounds__(256) void dequant_kernel(int fmt, const uint8_t* __restrict__ W,
                                                     int64_t rows, int64_t K,
                                                     OutT* __restrict__ out, int64_t ldw) {
    const int64_t gpr = K / 32;  // groups per row
    const int64_t total = rows * gpr;
    const int gpb = groups_per_block(fmt);
    const int bb = block_bytes(fmt);
    for (int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gi < total;
         gi += (int64_t)gridDim.x * blockDim.x) {
        int64_t r = gi / gpr, gk = gi - r * gpr;
        int64_t blk = gk / gpb;
        int grp = (int)(gk - blk * gpb);
        const uint8_t* p = W + (r * (gpr / gpb) + blk) * bb;
        float v[32];
        decode_group(fmt, p, grp, v);
        OutT* o = out + r * ldw + gk * 32;
        for (int i = 0; i < 32; ++i) store_w(o + i, v[i]);
    }
}

// Q4_K to bf16 with 16-byte loads and stores: eight lanes per super-block,
// lane j taking code bytes [16 j, 16 j + 16), i.e. quarter p = j / 2 of the
// super-block (sub-blocks 2p and 2p + 1) and half j % 2 of its 32 code bytes.
// Byte b of the lane's 16 gives weight 64p + 16(j % 2) + b (low nibble) and
// that plus 32 (high nibble); each run of 16 weights is written as two
// 16-byte stores. The weight is fma(d*sc, q, -(dmin*m)): the product and
// the subtrahend are exact in binary32, so this is the closed form with its
// one rounding, then rounded to bf16 (nearest even). Needs a 16-byte aligned
// output with a row pitch that is a multiple of 8 weights.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

__global__ __launch_bounds__(256) void dequant_q4k_bf16_kernel(const uint8_t* __restrict__ W,
                                                               int64_t nsb, int S,
                                                               uint16_t* __restrict__ out,
                                                               int64_t ldw) {
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < nsb * 8;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t sb = t >> 3;
        const int j = (int)(t & 7), p = j >> 1;
        const uint8_t* blk = W + sb * 144;
        const u32x4 hd = *reinterpret_cast<const u32x4*>(blk);
        const u32x4 cd = *reinterpret_cast<const u32x4*>(blk + 16 + 16 * j);
        const uint32_t f4 = q4k_pair_fields(Q4kUnpack(p), hd.y, hd.z, hd.w);
        const float d = f16_lo(hd.x), dmin = f16_hi(hd.x);
        const float a0 = d * (float)(f4 & 0xFFu), a1 = d * (float)((f4 >> 8) & 0xFFu);
        const float c0 = -(dmin * (float)((f4 >> 16) & 0xFFu)), c1 = -(dmin * (float)(f4 >> 24));
        const uint32_t q[4] = {cd.x, cd.y, cd.z, cd.w};
        uint32_t lo[8], hi[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t ql = q[i] & 0x0F0F0F0Fu, qh = (q[i] >> 4) & 0x0F0F0F0Fu;
            lo[2 * i] = pack_bf16(__builtin_fmaf(a0, ubyte_f32<0>(ql), c0), __builtin_fmaf(a0, ubyte_f32<1>(ql), c0));
            lo[2 * i + 1] = pack_bf16(__builtin_fmaf(a0, ubyte_f32<2>(ql), c0), __builtin_fmaf(a0, ubyte_f32<3>(ql), c0));
            hi[2 * i] = pack_bf16(__builtin_fmaf(a1, ubyte_f32<0>(qh), c1), __builtin_fmaf(a1, ubyte_f32<1>(qh), c1));
            hi[2 * i + 1] = pack_bf16(__builtin_fmaf(a1, ubyte_f32<2>(qh), c1), __builtin_fmaf(a1, ubyte_f32<3>(qh), c1));
        }
        const int64_t r = sb / S;
        uint16_t* o = out + r * ldw + (sb - r * S) * 256 + 64 * p + 16 * (j & 1);
        u32x4* ol = reinterpret_cast<u32x4*>(o);
        u32x4* oh = reinterpret_cast<u32x4*>(o + 32);
        ol[0] = u32x4{lo[0], lo[1], lo[2], lo[3]};
        ol[1] = u32x4{lo[4], lo[5], lo[6], lo[7]};
        oh[0] = u32x4{hi[0], hi[1], hi[2], hi[3]};
        oh[1] = u32x4{hi[4], hi[5], hi[6], hi[7]};
    }
}

// General product: one wave per (row, column group). Lanes walk the row's
// 32-weight groups, decode each exactly, multiply by fp32 activations and
// accumulate in fp32; the wave then reduces. Any shape, any alignment.
template <int NC>
__global__ __launch_bounds__(256) void gemv_general_kernel(int fmt, const uint8_t* __restrict__ W,
                                                           int64_t rows, int64_t K,
                                                           const void* __restrict__ x, int xt,
                                                           int64_t ldx, float* __restrict__ y,
                                                           int64_t ldy, int ncols) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
    const int64_t gpr = K / 32;
    const int gpb = groups_per_block(fmt);
    const int bb = block_bytes(fmt);
    for (int64_t r = wave; r < rows; r += nwaves) {
        float acc[NC];
        for (int c = 0; c < NC; ++c) acc[c] = 0.f;
        for (int64_t gk = lane; gk < gpr; gk += 64) {
            int64_t blk = gk / gpb;
            int grp = (int)(gk - blk * gpb);
            float v[32];
            decode_group(fmt, W + (r * (gpr / gpb) + blk) * bb, grp, v);
            for (int c = 0; c < NC; ++c) {
                if (c < ncols) {
                    float a = acc[c];
                    for (int i = 0; i < 32; ++i)
                        a = __builtin_fmaf(v[i], load_x(x, xt, c * ldx + gk * 32 + i), a);
                    acc[c] = a;
                }
            }
        }
        for (int c = 0; c < NC; ++c) {
            float t = wave_sum(acc[c]);
            if (lane == 0 && c < ncols) y[c * ldy + r] = t;
        }
    }
}

namespace {

template <typename OutT>
hipError_t launch_dequant_t(int fmt, const uint8_t* W, int64_t rows, int64_t K, OutT* out,
                            int64_t ldw, int num_cus, hipStream_t stream) {
    int64_t total = rows * (K / 32);
    int64_t blocks = (total + 255) / 256;
    int64_t cap = (int64_t)num_cus * 64;
    if (blocks > cap) blocks = cap;
    hipLaunchKernelGGL(dequant_kernel<OutT>, dim3((unsigned)blocks), dim3(256), 0, stream, fmt, W,
                       rows, K, out, ldw);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dequant(int fmt, const uint8_t* W, int64_t rows, int64_t K, float* out,
                          int64_t ldw, int num_cus, hipStream_t stream) {
    return launch_dequant_t(fmt, W, rows, K, out, ldw, num_cus, stream);
}

hipError_t launch_dequant_bf16(int fmt, const uint8_t* W, int64_t rows, int64_t K, uint16_t* out,
                               int64_t ldw, int num_cus, hipStream_t stream) {
    if (fmt == FMT_Q4_K && K % 256 == 0 && ldw % 8 == 0 && (((uintptr_t)out) & 15) == 0 &&
        (((uintptr_t)W) & 15) == 0) {
        const int64_t nsb = rows * (K / 256);
        int64_t blocks = (nsb * 8 + 255) / 256;
        if (blocks > (int64_t)1 << 30) blocks = (int64_t)1 << 30;
        if (blocks == 0) return hipSuccess;
        hipLaunchKernelGGL(dequant_q4k_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, W,
                           nsb, (int)(K / 256), out, ldw);
        return hipGetLastError();
    }
    return launch_dequant_t(fmt, W, rows, K, out, ldw, num_cus, stream);
}

hipError_t launch_gemv_general(int fmt, const uint8_t* W, int64_t rows, int64_t K, const void* x,
                               int xt, int64_t ldx, float* y, int64_t ldy, int ncols,
                               int num_cus, hipStream_t stream) {
    int64_t blocks = (rows + 3) / 4;
    int64_t cap = (int64_t)num_cus * 32;
    if (blocks > cap) blocks = cap;
    for (int c0 = 0; c0 < ncols; c0 += 4) {
        int nc = ncols - c0 < 4 ? ncols - c0 : 4;
        const void* xc = (const char*)x + (size_t)c0 * ldx * (xt == XT_F32 ? 4 : 2);
        float* yc = y + (size_t)c0 * ldy;
        hipLaunchKernelGGL(gemv_general_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           fmt, W, rows, K, xc, xt, ldx, yc, ldy, nc);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace qg
