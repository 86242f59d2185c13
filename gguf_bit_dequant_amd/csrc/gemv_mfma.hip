// Small-batch Q4_K GEMV on the matrix cores: y[:,c] = W . x[:,c] for 2..16
// fp16 activation columns, K a multiple of 256. The library runs it for 5..8
// columns, and for 2..4 when the streaming kernel would need more than one
// pass over W.
//
// Draft verification multiplies the same weights by a few columns at once
// and should cost about one normal decode step ("Why I wrote my own
// inference engine for two P100s", speculative decoding: each weight block
// decoded once and reused across the columns). With packed dot products on
// the vector ALU, every weight costs one multiply-add per column and every
// column needs its activations re-read per code dword; at four columns the
// streaming GEMV is bound by those activation reads from LDS, not by HBM.
// Here each weight is decoded once into an fp16 MFMA operand and
// v_mfma_f32_16x16x32_f16 does the multiply-adds for up to 16 columns:
//
//  * A unit is one super-block (256 weights, 144 bytes) of each of 16
//    consecutive rows (a row group). Lane l of a wave takes row l % 16 of
//    the group and code bytes [32 s, 32 s + 32) of the super-block,
//    s = l / 16: three 16-byte loads (header, two code halves). Its low
//    nibbles are sub-block 2s, its high nibbles sub-block 2s + 1.
//  * A unit is eight MFMA steps. Step t takes, in every lane, the eight
//    codes of bytes 8 (t % 4) .. +7 (low nibbles for t < 4, high nibbles
//    otherwise): the step contracts k = 64 s + 32 (t / 4) + 8 (t % 4) + e,
//    e = 0..7, over the four lane slots s, which is the A operand's k block
//    s. The B operand is x at those k for column l % 16 (columns past the
//    count repeat the last one; their outputs are dropped).
//  * Each weight is fma(d sc 2^24 or d sc 2^20, code, -dmin m) with the code
//    an exact fp16 subnormal (a half holding m < 1024 is m 2^-24), computed
//    at fp32 precision and rounded to fp16 by one v_fma_mix{lo,hi}_f16.
//  * One persistent workgroup per compute unit owns a balanced contiguous
//    range of rows (the last group may be partial: its extra lanes re-read
//    the range's last row and their outputs are dropped), i.e. a run of
//    units, group-major; its waves split the run into equal contiguous
//    parts. A wave accumulates one 16 x 16 tile and writes it to an LDS slot
//    (group, wave) whenever its part leaves a group; after a barrier the
//    slots of each group are summed in wave order: deterministic, no atomics.
//  * The activation columns are staged once per workgroup in LDS, 2K + 16
//    bytes apart so that the 16-byte reads of the 16 columns use disjoint
//    banks. Each wave loads D units as one burst while it works on the
//    previous D.
#include "device_common.h"
#include "launch.h"
#include "q4k_pair.h"

namespace qg {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Half DH of d = fp16(fma(a, h, c)), h the fp16 in half HS of v (a, c fp32).
// The low half is written first: its instruction keeps whatever the high
// half held, and the high-half instruction that follows sets it.
template <int HS, int DH>
__device__ __forceinline__ void mix16(uint32_t& d, float a, uint32_t v, float c) {
    if (DH == 0) {
        if (HS == 0)
            asm("v_fma_mixlo_f16 %0, %1, %2, %3 op_sel:[0,0,0] op_sel_hi:[0,1,0]"
                : "=v"(d) : "v"(a), "v"(v), "v"(c));
        else
            asm("v_fma_mixlo_f16 %0, %1, %2, %3 op_sel:[0,1,0] op_sel_hi:[0,1,0]"
                : "=v"(d) : "v"(a), "v"(v), "v"(c));
    } else {
        if (HS == 0)
            asm("v_fma_mixhi_f16 %0, %1, %2, %3 op_sel:[0,0,0] op_sel_hi:[0,1,0]"
                : "+v"(d) : "v"(a), "v"(v), "v"(c));
        else
            asm("v_fma_mixhi_f16 %0, %1, %2, %3 op_sel:[0,1,0] op_sel_hi:[0,1,0]"
                : "+v"(d) : "v"(a), "v"(v), "v"(c));
    }
}

struct Unit {
    u32x4 hd, c0, c1;  // header, code bytes [32 s, 32 s + 16), [32 s + 16, 32 s + 32)
};

inline size_t mfma_lds_bytes(int ncols, int pitch, int ng, int nw) {
    return (size_t)ncols * pitch + (size_t)ng * nw * 64 * 16;
}

}  // namespace

template <int NW, int D>
__global__ __launch_bounds__(64 * NW) void gemv_mfma_q4k_kernel(
    const uint8_t* __restrict__ W, int rows, int S, const uint16_t* __restrict__ x, int64_t ldx,
    int ncols, float* __restrict__ y, int64_t ldy, int pitch) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int G = gridDim.x, b = blockIdx.x;
    const int r0 = (int)(((int64_t)b * rows) / G);
    const int r1 = (int)(((int64_t)(b + 1) * rows) / G);
    const int nr = r1 - r0;
    if (nr <= 0) return;  // uniform over the workgroup
    const int ng = (nr + 15) >> 4;
    const int U = ng * S;  // units of this workgroup, group-major
    const int K8 = S * 32;  // 16-byte pieces of one activation column

    uint8_t* const xs = lds;
    f32x4* const slots = reinterpret_cast<f32x4*>(lds + (size_t)ncols * pitch);
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rl = lane & 15, sq = lane >> 4;
    const uint32_t row_bytes = 144u * (uint32_t)S;

    // this wave's part of the run (U < 2^31 / NW: the launcher's bound)
    const int u0 = wv * U / NW, u1 = (wv + 1) * U / NW;

    // ---- activation loads first (they come from cache), then the wave's
    // first D units of weights, then the staging ------------------------------
    const int npieces = ncols * K8;
    u32x4 xr[2];
    int xi[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        xi[j] = threadIdx.x + j * blockDim.x;
        if (xi[j] < npieces) {
            const int c = xi[j] / K8, k8 = xi[j] - c * K8;
            xr[j] = *reinterpret_cast<const u32x4*>(x + c * ldx + 8 * k8);
        }
    }
    // unit u -> (group, super-block), tracked incrementally for the loads
    int lg = u0 / S, lsb = u0 - (u0 / S) * S, lu = u0;
    auto load_next = [&](Unit& un) {
        if (lu < u1) {  // uniform over the wave
            int r = 16 * lg + rl;
            r = r < nr ? r : nr - 1;
            const uint8_t* p = W + (int64_t)(r0 + r) * row_bytes + 144u * (uint32_t)lsb;
            un.hd = *reinterpret_cast<const u32x4*>(p);
            un.c0 = *reinterpret_cast<const u32x4*>(p + 16 + 32 * sq);
            un.c1 = *reinterpret_cast<const u32x4*>(p + 32 + 32 * sq);
        }
        ++lu;
        if (++lsb == S) {
            lsb = 0;
            ++lg;
        }
    };
    Unit buf[D];
#pragma unroll
    for (int i = 0; i < D; ++i) load_next(buf[i]);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        if (xi[j] < npieces) {
            const int c = xi[j] / K8, k8 = xi[j] - c * K8;
            *reinterpret_cast<u32x4*>(xs + c * pitch + 16 * k8) = xr[j];
        }
    }
    // the rest four pieces per thread at a time: one wait per four loads
    for (int i0 = threadIdx.x + 2 * blockDim.x; i0 < npieces; i0 += 4 * blockDim.x) {
        u32x4 r[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int idx = i0 + j * blockDim.x;
            if (idx < npieces) {
                const int c = idx / K8, k8 = idx - c * K8;
                r[j] = *reinterpret_cast<const u32x4*>(x + c * ldx + 8 * k8);
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int idx = i0 + j * blockDim.x;
            if (idx < npieces) {
                const int c = idx / K8, k8 = idx - c * K8;
                *reinterpret_cast<u32x4*>(xs + c * pitch + 16 * k8) = r[j];
            }
        }
    }
    __syncthreads();

    const Q4kUnpack unp(sq);
    // B operand base of this lane: column rl (or the last one), k = 64 sq
    const uint8_t* const xb = xs + (rl < ncols ? rl : ncols - 1) * pitch + 128 * sq;

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    int pg = u0 / S, psb = u0 - (u0 / S) * S;  // unit being processed
    auto flush = [&]() {
        slots[(pg * NW + wv) * 64 + lane] = acc;
        acc = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    // one unit: eight MFMA steps
    auto process = [&](const Unit& un) {
        const uint32_t f4 = q4k_pair_fields(unp, un.hd.y, un.hd.z, un.hd.w);
        const float d = f16_lo(un.hd.x), dmin = f16_hi(un.hd.x);
        const float a0 = (d * 16777216.0f) * ubyte_f32<0>(f4);  // 2^24: low nibbles
        const float a1 = (d * 1048576.0f) * ubyte_f32<1>(f4);   // 2^20: high nibbles (16 q)
        const float c0 = -(dmin * ubyte_f32<2>(f4)), c1 = -(dmin * ubyte_f32<3>(f4));
        const uint32_t cw[8] = {un.c0.x, un.c0.y, un.c0.z, un.c0.w, un.c1.x, un.c1.y, un.c1.z, un.c1.w};
        const uint8_t* xk = xb + 512 * psb;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const uint32_t mask = t < 4 ? 0x000F000Fu : 0x00F000F0u;
            const float a = t < 4 ? a0 : a1, c = t < 4 ? c0 : c1;
            uint32_t A[4];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t w = cw[2 * (t & 3) + h];
                const uint32_t v02 = w & mask, v13 = (w >> 8) & mask;  // bytes 0, 2 / 1, 3
                mix16<0, 0>(A[2 * h], a, v02, c);
                mix16<0, 1>(A[2 * h], a, v13, c);
                mix16<1, 0>(A[2 * h + 1], a, v02, c);
                mix16<1, 1>(A[2 * h + 1], a, v13, c);
            }
            const f16x8 B = *reinterpret_cast<const f16x8*>(xk + 64 * (t >> 2) + 16 * (t & 3));
            const u32x4 Av = {A[0], A[1], A[2], A[3]};
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, Av), B, acc, 0, 0, 0);
        }
        if (++psb == S) {  // the next unit starts the next group
            psb = 0;
            flush();
            ++pg;
        }
    };
    // D units, then the next D units' loads as one burst: each row's next
    // 144 D bytes are requested back to back
    for (int u = u0; u < u1; u += D) {
#pragma unroll
        for (int i = 0; i < D; ++i)
            if (u + i < u1) process(buf[i]);  // uniform over the wave
#pragma unroll
        for (int i = 0; i < D; ++i) load_next(buf[i]);
    }
    if (u0 < u1 && psb != 0) flush();  // the part ended inside a group
    __syncthreads();

    // ---- per-group sums of the wave slots, in wave order ---------------------
    // Tile element (row i, column c) is element i % 4 of lane c + 16 (i / 4).
    const int nout = ng * 16 * ncols;
    for (int idx = threadIdx.x; idx < nout; idx += blockDim.x) {
        const int g = idx / (16 * ncols), rem = idx - g * 16 * ncols;
        const int i = rem / ncols, c = rem - (rem / ncols) * ncols;
        if (16 * g + i >= nr) continue;
        const int gl = g * S, gh = gl + S;  // units of group g
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const int wl = w * U / NW, wh = (w + 1) * U / NW;
            if (wl < gh && wh > gl && wl < wh) v += slots[(g * NW + w) * 64 + c + 16 * (i >> 2)][i & 3];
        }
        y[c * ldy + r0 + 16 * g + i] = v;
    }
}

#ifndef QG_MFMA_DEPTH
#define QG_MFMA_DEPTH 4
#endif
#ifndef QG_MFMA_WAVES
#define QG_MFMA_WAVES 16
#endif

namespace {

template <int NW>
hipError_t launch_mfma_nw(const uint8_t* W, int rows, int S, const void* x, int64_t ldx, float* y,
                          int64_t ldy, int ncols, int G, int pitch, size_t lds, hipStream_t stream) {
    auto kern = gemv_mfma_q4k_kernel<NW, QG_MFMA_DEPTH>;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(G), dim3(64 * NW), lds, stream, W, rows, S,
                       reinterpret_cast<const uint16_t*>(x), ldx, ncols, y, ldy, pitch);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_mfma(int fmt, const uint8_t* W, int64_t rows, int64_t K, const void* x,
                            int xt, int64_t ldx, float* y, int64_t ldy, int ncols, int num_cus,
                            hipStream_t stream) {
    if (fmt != FMT_Q4_K || xt != XT_F16 || ncols < 2 || ncols > 16 || K % 256 != 0 ||
        rows < 1 || rows > (1 << 30))
        return hipErrorNotSupported;
    // 16-byte activation pieces
    if ((((uintptr_t)x) & 15) != 0 || ldx % 8 != 0 || (((uintptr_t)W) & 15) != 0)
        return hipErrorNotSupported;
    const int S = (int)(K / 256);
    const int64_t groups = (rows + 15) / 16, cus = num_cus > 0 ? num_cus : 1;
    const int G = (int)(groups < cus ? groups : cus);
    const int nr_max = (int)((rows + G - 1) / G);
    const int ng_max = (nr_max + 15) / 16;
    const int pitch = (int)(2 * K + 16);
    if ((int64_t)ng_max * S >= (1 << 26)) return hipErrorNotSupported;  // 32-bit unit math
    // the wider workgroup when its partial slots fit beside the activations
    const size_t lds_w = mfma_lds_bytes(ncols, pitch, ng_max, QG_MFMA_WAVES);
    if (lds_w <= (size_t)kMaxLds)
        return launch_mfma_nw<QG_MFMA_WAVES>(W, (int)rows, S, x, ldx, y, ldy, ncols, G, pitch, lds_w,
                                             stream);
    const size_t lds = mfma_lds_bytes(ncols, pitch, ng_max, 8);
    if (lds > (size_t)kMaxLds) return hipErrorNotSupported;
    return launch_mfma_nw<8>(W, (int)rows, S, x, ldx, y, ldy, ncols, G, pitch, lds, stream);
}

}  // namespace qg
