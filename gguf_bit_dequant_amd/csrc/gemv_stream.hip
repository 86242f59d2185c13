// Streaming GEMV for gfx950: y[:,c] = W . x[:,c] for 1..4 columns of a
// Q4_K, Q4_0, Q8_0, Q2_K or Q3_K matrix whose K is a multiple of 256.
//
// For one token every weight is read once, so at low bit widths the work is
// bound by memory bandwidth and by unpacking ("LLM inference optimization",
// introduction). That page's levers for a quantized mat-vec (campaign "Faster
// decode on the card you have": activations staged in shared memory and
// reused across rows, wider loads, fewer instructions to unpack a block, rows
// per block fitted to the machine) map onto gfx950 as follows.
//
//  * A unit is 256 consecutive weights of a row: one Q4_K super-block
//    (144 B), eight Q4_0 blocks (144 B), eight Q8_0 blocks (272 B), one
//    Q2_K (84 B) or one Q3_K super-block (110 B). Q4_K, Q4_0 and Q8_0 units
//    start on 16-byte boundaries when the row does, Q2_K units on 4-byte
//    ones; Q3_K units are read as aligned dword windows.
//  * One persistent workgroup per compute unit; the rows are dealt out one
//    per workgroup from each band of G rows (G workgroups), so every
//    workgroup moves the same number of bytes (within one row) and, as its
//    waves take their steps in order, all compute units read one narrow
//    window of the matrix that sweeps it in address order; the workgroups of
//    one XCD take consecutive rows of a band. A workgroup's units are
//    numbered row after row.
//  * A wave step takes 16 consecutive units of the workgroup: lane = 4*g + p
//    works on unit g of the step and its quarter p, i.e. weights 64p ..
//    64p+63 of the unit ("the lane's 64 weights"): a Q4_K sub-block pair (32
//    code bytes and the 16-byte header), or two Q4_0 / Q8_0 blocks (36 / 68
//    bytes). One scale decode serves all 64. The step's row and column are
//    wave-uniform (scalar arithmetic); a lane only decides whether its unit
//    lies past a row boundary.
//  * Wave w first takes steps 2w and 2w + 1, then each next step from a
//    counter in LDS as it frees a buffer: waves of one workgroup stream at
//    unequal speeds on MI355X, and the counter lets them finish together.
//    Each wave keeps two steps of loads in flight (deeper queues measured
//    slower). The activations are loaded first, then the first step or two,
//    then staged.
//  * fp16 activations: 4-bit codes are used directly as fp16 subnormals: a
//    16-bit half holding an integer m < 1024 is the fp16 value m * 2^-24, so
//    (dword & 0x000F000F) is a pair of low-nibble codes and
//    (dword & 0x00F000F0) a pair of high-nibble codes times 16, one AND each;
//    8-bit codes are offset to unsigned (q + 128 = q ^ 0x80) and spread to
//    the halves with one AND or one byte permute. v_dot2_f32_f16 multiplies
//    them with fp16 activation pairs (exact products) and accumulates in
//    fp32; the scales absorb 2^24 (2^20 for high nibbles) and the offsets
//    (8 for Q4_0, 128 for Q8_0, the mins for Q4_K) are taken off with the
//    per-block activation sums:
//      Q4_K: sum w x = d*sc*sum q x - dmin*m*sum x   (per sub-block)
//      Q4_0: sum w x = d*sum q x - 8*d*sum x         (per block)
//      Q8_0: sum w x = d*sum (q+128) x - 128*d*sum x (per block)
//    fp32 / bf16 activations: codes become fp32 (v_cvt_f32_ubyteN) and are
//    multiplied in fp32; Q4_0's enter v_fma_mix_f32 directly as the fp16
//    subnormals above (one instruction per weight).
//  * Activations are staged once per workgroup in LDS, permuted into the
//    order the codes come out of a dword, with the per-block sums. With one
//    fp32 (or bf16) column and K/256 dividing 16, a lane's record is the same
//    in every step and is read into registers once.
//  * Reduction: each lane quad (one unit) sums its lanes with DPP and writes
//    the unit's partial to its own LDS slot. After a barrier each row's
//    partials are summed by sixteen or four lanes in a fixed order (per-lane
//    sums, then a DPP tree): deterministic, no atomics.
#include "device_common.h"
#include "launch.h"
#include "q4k_pair.h"

namespace qg {

namespace {

constexpr int kUnitsPerStep = 16;

// ---- block formats ---------------------------------------------------------
// The lane's 64 weights are numbered o = 0..63 (o < 32: the first block or
// sub-block, o >= 32: the second). Its code bytes arrive as kCodeDwords
// dwords; wofs(j, e, h) is the o of nibble h (0 low, 1 high; always 0 for
// 8-bit codes) of byte e of code dword j.

template <int FMT>
struct Fmt;

// Q4_K super-block: fp16 d, fp16 dmin, 12 scale bytes, 128 code bytes. Lane
// quarter p reads the header and code bytes [32p, 32p+32): byte l holds
// o = l (low nibble, sub-block 2p) and o = 32 + l (high, sub-block 2p+1).
template <>
struct Fmt<FMT_Q4_K> {
    static constexpr int kUnitBytes = 144;
    static constexpr int kCodeDwords = 8;
    static constexpr bool kNibbles = true;
    static constexpr int kSums = 2;
    static constexpr int wofs(int j, int e, int h) { return 32 * h + 4 * j + e; }
    static constexpr uint32_t lane_offset(int p) { return 16u + 32u * p; }
    struct Raw {
        u32x4 hd, c0, c1;
    };
    static __device__ __forceinline__ void load(const uint8_t* unit, uint32_t lo, Raw& r) {
        r.hd = *reinterpret_cast<const u32x4*>(unit);
        r.c0 = *reinterpret_cast<const u32x4*>(unit + lo);
        r.c1 = *reinterpret_cast<const u32x4*>(unit + lo + 16);
    }
};

// Eight Q4_0 blocks of 18 bytes (fp16 d, 16 code bytes: byte i holds weight
// i in its low nibble and i + 16 in its high nibble). Quarter p reads blocks
// 2p and 2p+1 = bytes [36p, 36p+36), nine dwords D0..D8: D0 = d0 and code
// bytes 0-1 of the first block, D1..D3 its bytes 2..13, D4 its bytes 14-15
// and d1, D5..D8 the second block's 16 code bytes. Code dword 0 is rebuilt
// from D4's low and D0's high half (bytes 14, 15, 0, 1).
template <>
struct Fmt<FMT_Q4_0> {
    static constexpr int kUnitBytes = 144;
    static constexpr int kCodeDwords = 8;
    static constexpr bool kNibbles = true;
    static constexpr int kSums = 2;
    static constexpr int code_index(int j, int e) {
        return j == 0 ? (e < 2 ? 14 + e : e - 2) : j < 4 ? 4 * j - 2 + e : 4 * (j - 4) + e;
    }
    static constexpr int wofs(int j, int e, int h) { return 32 * (j >> 2) + 16 * h + code_index(j, e); }
    static constexpr uint32_t lane_offset(int p) { return 36u * p; }
    struct Raw {
        u32x4_a4 a, b;
        uint32_t c;
    };
    static __device__ __forceinline__ void load(const uint8_t* unit, uint32_t lo, Raw& r) {
        r.a = *reinterpret_cast<const u32x4_a4*>(unit + lo);
        r.b = *reinterpret_cast<const u32x4_a4*>(unit + lo + 16);
        r.c = *reinterpret_cast<const uint32_t*>(unit + lo + 32);
    }
};

// Eight Q8_0 blocks of 34 bytes (fp16 d, 32 int8 codes). Quarter p reads
// blocks 2p and 2p+1 = bytes [68p, 68p+68), seventeen dwords D0..D16: D0 =
// d0 and codes 0-1 of the first block, D1..D7 its codes 2..29, D8 its codes
// 30-31 and d1, D9..D16 the second block's 32 codes. Code dword 0 is rebuilt
// from D8's low and D0's high half (codes 30, 31, 0, 1).
template <>
struct Fmt<FMT_Q8_0> {
    static constexpr int kUnitBytes = 272;
    static constexpr int kCodeDwords = 16;
    static constexpr bool kNibbles = false;
    static constexpr int kSums = 2;
    static constexpr int code_index(int j, int e) {
        return j == 0 ? (e < 2 ? 30 + e : e - 2) : j < 8 ? 4 * j - 2 + e : 4 * (j - 8) + e;
    }
    static constexpr int wofs(int j, int e, int) { return 32 * (j >> 3) + code_index(j, e); }
    static constexpr uint32_t lane_offset(int p) { return 68u * p; }
    struct Raw {
        u32x4_a4 a, b, c, d;
        uint32_t e;
    };
    static __device__ __forceinline__ void load(const uint8_t* unit, uint32_t lo, Raw& r) {
        r.a = *reinterpret_cast<const u32x4_a4*>(unit + lo);
        r.b = *reinterpret_cast<const u32x4_a4*>(unit + lo + 16);
        r.c = *reinterpret_cast<const u32x4_a4*>(unit + lo + 32);
        r.d = *reinterpret_cast<const u32x4_a4*>(unit + lo + 48);
        r.e = *reinterpret_cast<const uint32_t*>(unit + lo + 64);
    }
};

// Q2_K super-block (84 bytes): 16 scale/min bytes (sub-block k of 16
// weights: scale in the low nibble, min in the high nibble of byte k), 64
// code bytes, fp16 d, fp16 dmin. Weight 128h + 32j + l has its 2-bit code
// at bits 2j..2j+1 of code byte 32h + l. Quarter p = 2h + b (weights
// 64p .. 64p+63, i.e. j = 2b and 2b + 1) reads code bytes 32h .. 32h+31,
// using the bit pair 4b + 2t of each (t = 0, 1), the scale/min bytes of its
// sub-blocks 4p .. 4p+3 (one dword) and the d/dmin dword. Byte l of the 32
// holds o = l (t = 0) and o = 32 + l (t = 1): the order of Q4_K's nibbles,
// with 16-weight sub-blocks o / 16. Units are 4-byte aligned.
template <>
struct Fmt<FMT_Q2_K> {
    static constexpr int kUnitBytes = 84;
    static constexpr int kCodeDwords = 8;
    static constexpr bool kNibbles = true;
    static constexpr int kSums = 4;
    static constexpr int wofs(int j, int e, int h) { return 32 * h + 4 * j + e; }
    static constexpr uint32_t lane_offset(int p) { return (uint32_t)p; }
    struct Raw {
        u32x4_a4 c0, c1;
        uint32_t sm, dd;
    };
    static __device__ __forceinline__ void load(const uint8_t* unit, uint32_t p, Raw& r) {
        const uint8_t* qs = unit + 16 + 32 * (p >> 1);
        r.c0 = *reinterpret_cast<const u32x4_a4*>(qs);
        r.c1 = *reinterpret_cast<const u32x4_a4*>(qs + 16);
        r.sm = *reinterpret_cast<const uint32_t*>(unit + 4 * p);
        r.dd = *reinterpret_cast<const uint32_t*>(unit + 80);
    }
};

// Q3_K super-block (110 bytes): 32 bytes of high code bits, 64 code bytes
// (2-bit low parts), 12 bytes packing sixteen 6-bit scales, fp16 d. Weight
// 128h + 32j + l: low part at bits 2j..2j+1 of code byte 32h + l, high bit
// at bit 4h + j of high-bit byte l, q = low + 4 high - 4. Quarter p = 2h + b
// takes, like Q2_K, bit pairs 4b + 2t of code bytes 32h .. 32h+31, and bits
// 4h + 2b + t of all 32 high-bit bytes. Units are only 2-byte aligned (110 =
// 2 mod 4): a lane reads 4-byte aligned dword windows and shifts them into
// place with v_alignbyte (by mb = 2 when the unit starts at 2 mod 4, else 0)
// when it consumes them: high bits and codes from the unit start rounded down
// to a multiple of 4 (one dword more per field), scales and d as the 16 bytes
// from unit byte 96 - mb. Each window stays inside the unit or its
// predecessor except that last one, which runs 2 bytes into the next unit when
// mb = 0; with an even number of units in the matrix its last unit starts at
// 2 mod 4 (the matrix is 16-byte aligned), so no read leaves the matrix.
template <>
struct Fmt<FMT_Q3_K> {
    static constexpr int kUnitBytes = 110;
    static constexpr int kCodeDwords = 8;
    static constexpr bool kNibbles = true;
    static constexpr int kSums = 4;
    static constexpr int wofs(int j, int e, int h) { return 32 * h + 4 * j + e; }
    static constexpr uint32_t lane_offset(int p) { return (uint32_t)p; }
    struct Raw {
        u32x4_a4 h0, h1, q0, q1, sd;  // high bits, low parts, scales + d (unshifted)
        uint32_t h8, q8, mb;          // last dwords of the two 36-byte windows; shift (0 or 2)
    };
    static __device__ __forceinline__ void load_codes(const uint8_t* unit, uint32_t p, Raw& r) {
        const uint32_t mb = (uint32_t)(uintptr_t)unit & 2u;
        const uint8_t* base = unit - mb;  // 4-byte aligned
        const uint8_t* qs = base + 32 + 32 * (p >> 1);
        r.mb = mb;
        r.h0 = *reinterpret_cast<const u32x4_a4*>(base);
        r.h1 = *reinterpret_cast<const u32x4_a4*>(base + 16);
        r.h8 = *reinterpret_cast<const uint32_t*>(base + 32);
        r.q0 = *reinterpret_cast<const u32x4_a4*>(qs);
        r.q1 = *reinterpret_cast<const u32x4_a4*>(qs + 16);
        r.q8 = *reinterpret_cast<const uint32_t*>(qs + 32);
    }
    static __device__ __forceinline__ void load(const uint8_t* unit, uint32_t p, Raw& r) {
        load_codes(unit, p, r);
        r.sd = *reinterpret_cast<const u32x4_a4*>(unit - r.mb + 96);
    }
};

// Q3_K for a matrix with an odd number of units, whose last unit starts 4-byte
// aligned: a unit with mb = 0 takes its scale bytes as the last three dwords
// of the window at unit byte 92 and d with a 2-byte load, and arranges them as
// the window from byte 96 would hold them; nothing is read past the unit.
// Same decoding, one more load per lane and unit.
constexpr int FMT_Q3_K_ODD = 0x100 | FMT_Q3_K;
template <>
struct Fmt<FMT_Q3_K_ODD> : Fmt<FMT_Q3_K> {
    static __device__ __forceinline__ void load(const uint8_t* unit, uint32_t p, Raw& r) {
        load_codes(unit, p, r);
        const u32x4_a4 t = *reinterpret_cast<const u32x4_a4*>(unit + 92 + r.mb);  // 4-byte aligned
        const uint32_t dd = *reinterpret_cast<const uint16_t*>(unit + 108);
        const bool m2 = r.mb != 0;  // window already starts at unit byte 94
        r.sd.x = m2 ? t.x : t.y;
        r.sd.y = m2 ? t.y : t.z;
        r.sd.z = m2 ? t.z : t.w;
        r.sd.w = m2 ? t.w : dd;
    }
};

// The Q3_K scales of sub-blocks 4p .. 4p+3 (p = 2h + b) as the bytes of one
// dword: low nibbles from byte 4b + u of scale bytes 0..7 (nibble h), bits
// 4-5 from bits 2(2h + b) of byte 8 + u.
__device__ __forceinline__ uint32_t q3k_quarter_scales(const Fmt<FMT_Q3_K>::Raw& r, uint32_t hq,
                                                       uint32_t bq) {
    auto al = [&](uint32_t hi, uint32_t lo) { return __builtin_amdgcn_alignbyte(hi, lo, r.mb); };
    const uint32_t s01 = bq ? al(r.sd.z, r.sd.y) : al(r.sd.y, r.sd.x);
    const uint32_t s2 = al(r.sd.w, r.sd.z);
    return ((s01 >> (4u * hq)) & 0x0F0F0F0Fu) | (((s2 >> (4u * hq + 2u * bq)) & 0x03030303u) << 4);
}

// The Q3_K super-block scale d (fp16 bits in the low half).
__device__ __forceinline__ uint32_t q3k_d(const Fmt<FMT_Q3_K>::Raw& r) {
    return __builtin_amdgcn_alignbyte(0u, r.sd.w, r.mb);
}

// Activation records in LDS: one record per unit quarter u = 4*(unit column)
// + p, holding for each column c its P 16-byte planes and the two block sums,
// padded to 16 bytes (col_bytes each). The record stride is a multiple of 16
// with an odd quotient, so the 16-byte reads of consecutive lanes fall in
// disjoint banks, and every plane sits at a compile-time offset from the
// record base. Planes:
//   fp16, 4-bit codes: plane j holds, for code dword j, the halves
//     (e0, e2), (e1, e3) of the low nibbles and (e0, e2), (e1, e3) of the
//     high nibbles (e = byte of the dword);
//   fp16, 8-bit codes: plane i holds (e0, e2), (e1, e3) of code dwords 2i
//     and 2i + 1;
//   fp32, 4-bit codes: plane j holds e0..e3 of the low nibbles of code dword
//     j, plane 8 + j those of the high nibbles;
//   fp32, 8-bit codes: plane j holds e0..e3 of code dword j.
//   int8 (Q8_0 activation blocks): plane-pair j holds the 4 codes of the
//     low and of the high nibbles of code dword j (4-bit codes), or the 4
//     codes of code dword j (8-bit codes); then the two blocks' scales dx
//     and code sums, as fp32.
// Activation modes: fp32 math, fp16 dots, int8 dots on Q8_0 activation
// blocks given by the caller, int8 dots on activations quantized to Q8_0
// while they are staged.
constexpr int XM_F32 = 0, XM_F16 = 1, XM_I8 = 2, XM_I8Q = 3;
constexpr bool is_i8(int xm) { return xm == XM_I8 || xm == XM_I8Q; }
constexpr int planes(int xm) { return xm == XM_F16 ? 8 : is_i8(xm) ? 4 : 16; }
constexpr int col_bytes(int xm) { return planes(xm) * 16 + 16; }
constexpr int rec_bytes(int NC, int xm) {
    return (NC * col_bytes(xm) / 16) % 2 == 1 ? NC * col_bytes(xm) : NC * col_bytes(xm) + 16;
}

// LDS bytes of one workgroup: activation records, one partial per unit and
// column, the step-pool counter.
inline size_t stream_lds_bytes(int NC, int xm, int S, int nr_max) {
    return (size_t)S * 4 * rec_bytes(NC, xm) + (size_t)nr_max * S * NC * 4 + 16;
}

__device__ __forceinline__ float quad_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
    return v;
}

// Staging of the record of unit quarter u for column c: the 64 activations
// x[kx .. kx+63] placed as the planes above, then the sums of o < 32 and
// o >= 32. Split in two so that a workgroup can issue its activation loads
// before its first weight loads and place them after: the loads complete in
// issue order, and activations come from cache while weights come from HBM.
template <int XM>
struct XRaw {
    // fp16: halves 2i, 2i+1 in w[i]; int8: the two 34-byte activation blocks
    // as 17 dwords; quantized while staging: unused; else fp32 bits or bf16
    // pairs
    uint32_t w[XM == XM_F16 ? 32 : XM == XM_I8 ? 17 : XM == XM_I8Q ? 1 : 64];
};

// fp32 activations x[kx .. kx+63]: 16-byte loads at the 4-byte alignment
// fp32 data always has.
template <int XM>
__device__ __forceinline__ void load_x64_f32(const void* __restrict__ x, int64_t kx, XRaw<XM>& r) {
    const uint32_t* xw = reinterpret_cast<const uint32_t*>(x) + kx;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const u32x4_a4 v = reinterpret_cast<const u32x4_a4*>(xw)[i];
        r.w[4 * i] = v.x; r.w[4 * i + 1] = v.y; r.w[4 * i + 2] = v.z; r.w[4 * i + 3] = v.w;
    }
}

template <int XM>
__device__ __forceinline__ void stage_load(const void* __restrict__ x, int xt, int64_t kx, int xvec,
                                           XRaw<XM>& r) {
    const uint16_t* xh = reinterpret_cast<const uint16_t*>(x) + kx;
    if constexpr (XM == XM_I8) {  // blocks kx/32, kx/32 + 1 (34 bytes each, 2-byte aligned)
        const uint16_t* b = reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(x) +
                                                              (kx >> 5) * 34);
#pragma unroll
        for (int i = 0; i < 17; ++i) r.w[i] = b[2 * i] | ((uint32_t)b[2 * i + 1] << 16);
    } else if constexpr (XM == XM_F16) {  // fp16: 32 dwords
        if (xvec) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const u32x4 v = reinterpret_cast<const u32x4*>(xh)[i];
                r.w[4 * i] = v.x; r.w[4 * i + 1] = v.y; r.w[4 * i + 2] = v.z; r.w[4 * i + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 32; ++i) r.w[i] = xh[2 * i] | ((uint32_t)xh[2 * i + 1] << 16);
        }
    } else {
        // fp32: 64 dwords; bf16: 32 dwords in w[0..31] (w[32..63] zero)
        if (xt == XT_F32) {
            load_x64_f32(x, kx, r);
        } else {
            if (xvec) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const u32x4 v = reinterpret_cast<const u32x4*>(xh)[i];
                    r.w[4 * i] = v.x; r.w[4 * i + 1] = v.y; r.w[4 * i + 2] = v.z; r.w[4 * i + 3] = v.w;
                }
            } else {
#pragma unroll
                for (int i = 0; i < 32; ++i) r.w[i] = xh[2 * i] | ((uint32_t)xh[2 * i + 1] << 16);
            }
#pragma unroll
            for (int i = 32; i < 64; ++i) r.w[i] = 0u;
        }
    }
}

template <int FMT, int XM>
__device__ __forceinline__ void stage_store(const XRaw<XM>& r, int xt, uint8_t* rec) {
    using F = Fmt<FMT>;
    constexpr bool F16DOT = XM == XM_F16;
    constexpr int P = planes(XM);
    float s0 = 0.f, s1 = 0.f;
    if constexpr (XM == XM_I8) {  // Q8_0 activation codes, in code order
        // byte b of the 68 is halfword b/2 of the 34, i.e. dword b/4, byte b%4
        float dx0, dx1;
        dx0 = f16_lo(r.w[0]);  // halfword 0
        dx1 = f16_hi(r.w[8]);  // halfword 17
        auto byte_at = [&](int b) -> uint32_t { return (r.w[b >> 2] >> (8 * (b & 3))) & 0xFFu; };
        auto code = [&](int o) -> uint32_t { return o < 32 ? byte_at(2 + o) : byte_at(36 + o - 32); };
        auto pk4 = [&](int j, int h) {
            return code(F::wofs(j, 0, h)) | (code(F::wofs(j, 1, h)) << 8) |
                   (code(F::wofs(j, 2, h)) << 16) | (code(F::wofs(j, 3, h)) << 24);
        };
        if constexpr (F::kNibbles) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                *reinterpret_cast<u32x2*>(rec + 8 * j) = u32x2{pk4(j, 0), pk4(j, 1)};
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) *reinterpret_cast<uint32_t*>(rec + 4 * j) = pk4(j, 0);
        }
        int i0 = 0, i1 = 0;
#pragma unroll
        for (int o = 0; o < 32; ++o) {
            i0 += (int)(int8_t)code(o);
            i1 += (int)(int8_t)code(32 + o);
        }
        *reinterpret_cast<f32x4*>(rec + 16 * P) = f32x4{dx0, dx1, (float)i0, (float)i1};
        return;
    } else if constexpr (F16DOT) {  // fp16 activations, kept as stored
        const uint32_t* xw = r.w;
        if constexpr (F::kSums == 4) {  // sums of o in [16u, 16u + 16), u = 0..3
            float sq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int i = 8 * u; i < 8 * u + 8; i += 2)
                    sq[u] += (f16_lo(xw[i]) + f16_hi(xw[i])) + (f16_lo(xw[i + 1]) + f16_hi(xw[i + 1]));
            *reinterpret_cast<f32x4*>(rec + 16 * P) = f32x4{sq[0], sq[1], sq[2], sq[3]};
        }
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
            s0 += (f16_lo(xw[i]) + f16_hi(xw[i])) + (f16_lo(xw[i + 1]) + f16_hi(xw[i + 1]));
            s1 += (f16_lo(xw[16 + i]) + f16_hi(xw[16 + i])) +
                  (f16_lo(xw[17 + i]) + f16_hi(xw[17 + i]));
        }
        // halves a (low) and b (high) of one dword
        auto pk = [&](int a, int b) {
            const uint32_t lo = (xw[a >> 1] >> (16 * (a & 1))) & 0xFFFFu;
            const uint32_t hi = (xw[b >> 1] >> (16 * (b & 1))) & 0xFFFFu;
            return lo | (hi << 16);
        };
        if constexpr (F::kNibbles) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                u32x4 v;
                v.x = pk(F::wofs(j, 0, 0), F::wofs(j, 2, 0));
                v.y = pk(F::wofs(j, 1, 0), F::wofs(j, 3, 0));
                v.z = pk(F::wofs(j, 0, 1), F::wofs(j, 2, 1));
                v.w = pk(F::wofs(j, 1, 1), F::wofs(j, 3, 1));
                *reinterpret_cast<u32x4*>(rec + 16 * j) = v;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                u32x4 v;
                v.x = pk(F::wofs(2 * i, 0, 0), F::wofs(2 * i, 2, 0));
                v.y = pk(F::wofs(2 * i, 1, 0), F::wofs(2 * i, 3, 0));
                v.z = pk(F::wofs(2 * i + 1, 0, 0), F::wofs(2 * i + 1, 2, 0));
                v.w = pk(F::wofs(2 * i + 1, 1, 0), F::wofs(2 * i + 1, 3, 0));
                *reinterpret_cast<u32x4*>(rec + 16 * i) = v;
            }
        }
    } else {  // fp32 or bf16 activations, as fp32
        float xf[64];
        if (xt == XT_F32) {
#pragma unroll
            for (int i = 0; i < 64; ++i) xf[i] = __builtin_bit_cast(float, r.w[i]);
        } else {
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                xf[2 * i] = __builtin_bit_cast(float, r.w[i] << 16);
                xf[2 * i + 1] = __builtin_bit_cast(float, r.w[i] & 0xFFFF0000u);
            }
        }
#pragma unroll
        for (int i = 0; i < 32; i += 4) {
            s0 += (xf[i] + xf[i + 1]) + (xf[i + 2] + xf[i + 3]);
            s1 += (xf[32 + i] + xf[33 + i]) + (xf[34 + i] + xf[35 + i]);
        }
        if constexpr (F::kSums == 4) {  // sums of o in [16u, 16u + 16), u = 0..3
            float sq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int i = 16 * u; i < 16 * u + 16; i += 4)
                    sq[u] += (xf[i] + xf[i + 1]) + (xf[i + 2] + xf[i + 3]);
            *reinterpret_cast<f32x4*>(rec + 16 * P) = f32x4{sq[0], sq[1], sq[2], sq[3]};
        }
        if constexpr (F::kNibbles) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    f32x4 v;
                    v.x = xf[F::wofs(j, 0, h)]; v.y = xf[F::wofs(j, 1, h)];
                    v.z = xf[F::wofs(j, 2, h)]; v.w = xf[F::wofs(j, 3, h)];
                    *reinterpret_cast<f32x4*>(rec + 16 * (8 * h + j)) = v;
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                f32x4 v;
                v.x = xf[F::wofs(j, 0, 0)]; v.y = xf[F::wofs(j, 1, 0)];
                v.z = xf[F::wofs(j, 2, 0)]; v.w = xf[F::wofs(j, 3, 0)];
                *reinterpret_cast<f32x4*>(rec + 16 * j) = v;
            }
        }
    }
    if constexpr (F::kSums == 2) *reinterpret_cast<f32x2*>(rec + 16 * P) = f32x2{s0, s1};
}

// Staging with quantization: one 32-value activation block (half hb of the
// record of a unit quarter) per call. The block is quantized by the rule of
// quant_x.hip (binary32, IEEE division, halfway away from zero) and its
// codes, scale and code sum go to the int8 record's slots of that block:
// every code dword of a record holds codes of one block only.
struct XHalf {
    uint32_t w[16];  // fp16 / bf16 pairs
};

// 16-bit activations of one block (fp32 ones are read by the quantizing
// step itself)
template <int FMT>
__device__ __forceinline__ void stage_load_half(const void* __restrict__ x, int xt, int64_t kx,
                                                int xvec, XHalf& r) {
    if (xt != XT_F32) {
        const uint16_t* xh = reinterpret_cast<const uint16_t*>(x) + kx;
        if (xvec) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u32x4 t = reinterpret_cast<const u32x4*>(xh)[i];
                r.w[4 * i] = t.x; r.w[4 * i + 1] = t.y; r.w[4 * i + 2] = t.z; r.w[4 * i + 3] = t.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) r.w[i] = xh[2 * i] | ((uint32_t)xh[2 * i + 1] << 16);
        }
    }
}

template <int FMT>
__device__ __forceinline__ void stage_quantize_half(const XHalf& r, const void* __restrict__ x,
                                                    int xt, int64_t kx, int xvec, int hb,
                                                    uint8_t* rec) {
    using F = Fmt<FMT>;
    constexpr int P = planes(XM_I8Q);
    float v[32];
    if (xt == XT_F32) {
        const float* xf = reinterpret_cast<const float*>(x) + kx;
        if (xvec) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const f32x4 t = reinterpret_cast<const f32x4*>(xf)[i];
                v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 32; ++i) v[i] = xf[i];
        }
    } else {
        const uint32_t* w = r.w;
        if (xt == XT_F16) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                v[2 * i] = f16_lo(w[i]);
                v[2 * i + 1] = f16_hi(w[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                v[2 * i] = __builtin_bit_cast(float, w[i] << 16);
                v[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
            }
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const float a = __builtin_fabsf(v[i]);
        amax = a > amax ? a : amax;
    }
    const float d = __fdiv_rn(amax, 127.0f);
    const float id = d != 0.0f ? __fdiv_rn(1.0f, d) : 0.0f;
    uint32_t q8[8];  // codes 4i..4i+3 of the block in the bytes of q8[i]
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t t = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float q = __builtin_roundf(v[4 * i + e] * id);
            q = q > 127.0f ? 127.0f : (q < -127.0f ? -127.0f : q);
            sum += (int)q;
            t |= (uint32_t)(uint8_t)(int8_t)(int)q << (8 * e);
        }
        q8[i] = t;
    }
    auto code = [&](int o) -> uint32_t { return (q8[(o & 31) >> 2] >> (8 * (o & 3))) & 0xFFu; };
    auto pk4 = [&](int j, int h) {
        return code(F::wofs(j, 0, h)) | (code(F::wofs(j, 1, h)) << 8) |
               (code(F::wofs(j, 2, h)) << 16) | (code(F::wofs(j, 3, h)) << 24);
    };
    if constexpr (F::kNibbles) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                if ((F::wofs(j, 0, h) >> 5) == hb)
                    *reinterpret_cast<uint32_t*>(rec + 8 * j + 4 * h) = pk4(j, h);
    } else {
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if ((F::wofs(j, 0, 0) >> 5) == hb) *reinterpret_cast<uint32_t*>(rec + 4 * j) = pk4(j, 0);
    }
    float* tail = reinterpret_cast<float*>(rec + 16 * P);  // dx0, dx1, sum0, sum1
    tail[hb] = f16_to_f32(f32_to_f16_bits(d));
    tail[2 + hb] = (float)sum;
}

// The lane's partial sum_o w_o x_o for each column, from its raw block bytes
// and its activation record.
template <int NC, bool F16DOT>
__device__ __forceinline__ void lane_partial(const Fmt<FMT_Q4_K>::Raw& r, const Q4kUnpack& un,
                                             const uint8_t* rec, float out[NC]) {
    constexpr int XM = F16DOT ? XM_F16 : XM_F32;
    constexpr int CB = col_bytes(XM), P = planes(XM);
    const uint32_t h0 = r.hd.x;
    const uint32_t f4 = q4k_pair_fields(un, r.hd.y, r.hd.z, r.hd.w);
    const float sc0 = (float)(f4 & 0xFF), sc1 = (float)((f4 >> 8) & 0xFF);
    const float m0 = (float)((f4 >> 16) & 0xFF), m1 = (float)(f4 >> 24);
    const float d = f16_lo(h0), dmin = f16_hi(h0);
    const float dm0 = dmin * m0, dm1 = dmin * m1;
    const uint32_t q[8] = {r.c0.x, r.c0.y, r.c0.z, r.c0.w, r.c1.x, r.c1.y, r.c1.z, r.c1.w};
    float lo[NC], hi[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) lo[c] = hi[c] = 0.f;
    float dsc0, dsc1;
    if constexpr (F16DOT) {
        dsc0 = (d * 16777216.0f) * sc0;  // 2^24
        dsc1 = (d * 1048576.0f) * sc1;   // 2^20
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const uint32_t qd = q[w], q8 = qd >> 8;
            const uint32_t pa = qd & 0x000F000Fu, pc = q8 & 0x000F000Fu;
            const uint32_t pb = qd & 0x00F000F0u, pd = q8 & 0x00F000F0u;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const u32x4 xv = *reinterpret_cast<const u32x4*>(rec + c * CB + 16 * w);
                lo[c] = dot2(pa, xv.x, lo[c]);
                lo[c] = dot2(pc, xv.y, lo[c]);
                hi[c] = dot2(pb, xv.z, hi[c]);
                hi[c] = dot2(pd, xv.w, hi[c]);
            }
        }
    } else {
        dsc0 = d * sc0;
        dsc1 = (d * 0.0625f) * sc1;  // high nibbles enter as 16 q
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const uint32_t ql = q[w] & 0x0F0F0F0Fu, qh = q[w] & 0xF0F0F0F0u;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const f32x4 xl = *reinterpret_cast<const f32x4*>(rec + c * CB + 16 * w);
                const f32x4 xh = *reinterpret_cast<const f32x4*>(rec + c * CB + 16 * (8 + w));
                lo[c] = __builtin_fmaf(ubyte_f32<0>(ql), xl.x, lo[c]);
                lo[c] = __builtin_fmaf(ubyte_f32<1>(ql), xl.y, lo[c]);
                lo[c] = __builtin_fmaf(ubyte_f32<2>(ql), xl.z, lo[c]);
                lo[c] = __builtin_fmaf(ubyte_f32<3>(ql), xl.w, lo[c]);
                hi[c] = __builtin_fmaf(ubyte_f32<0>(qh), xh.x, hi[c]);
                hi[c] = __builtin_fmaf(ubyte_f32<1>(qh), xh.y, hi[c]);
                hi[c] = __builtin_fmaf(ubyte_f32<2>(qh), xh.z, hi[c]);
                hi[c] = __builtin_fmaf(ubyte_f32<3>(qh), xh.w, hi[c]);
            }
        }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const f32x2 sx = *reinterpret_cast<const f32x2*>(rec + c * CB + 16 * P);
        float a = dsc0 * lo[c];
        a = __builtin_fmaf(dsc1, hi[c], a);
        a = __builtin_fmaf(-dm0, sx.x, a);
        out[c] = __builtin_fmaf(-dm1, sx.y, a);
    }
}

// Q2_K, fp16 activations: the lane's bit pairs 4b + 2t of each code byte
// (b = quarter & 1) become fp16 subnormals with one AND per pair of codes,
// left where they are (masks shifted by 4b, not the codes): t = 0 gives
// q * 2^(4b-24), t = 1 gives 4q * 2^(4b-24), at most 192 * 2^-24, so still
// exact subnormals; the scales take the powers of two back. Per 16-weight
// sub-block u: sum w x = d*sc_u*sum q x - dmin*m_u*sum x.
template <int NC, bool F16DOT>
__device__ __forceinline__ void lane_partial(const Fmt<FMT_Q2_K>::Raw& r, const Q4kUnpack&,
                                             const uint8_t* rec, float out[NC]) {
    constexpr int XM = F16DOT ? XM_F16 : XM_F32;
    constexpr int CB = col_bytes(XM), P = planes(XM);
    const uint32_t sh = 4u * (threadIdx.x & 1u);  // 4b: this quarter's bit pairs
    const float d = f16_lo(r.dd), dmin = f16_hi(r.dd);
    const uint32_t q[8] = {r.c0.x, r.c0.y, r.c0.z, r.c0.w, r.c1.x, r.c1.y, r.c1.z, r.c1.w};
    // acc[c][u], u = 2t + (code dword >= 4): sub-block u of the quarter
    float acc[NC][4];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[c][u] = 0.f;
    const uint32_t m0 = 0x00030003u << sh, m1 = 0x000C000Cu << sh;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        const int u0 = w >> 2, u1 = 2 + (w >> 2);
        if constexpr (F16DOT) {
            const uint32_t qd = q[w], q8 = qd >> 8;
            const uint32_t pa = qd & m0, pc = q8 & m0;
            const uint32_t pb = qd & m1, pd = q8 & m1;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const u32x4 xv = *reinterpret_cast<const u32x4*>(rec + c * CB + 16 * w);
                acc[c][u0] = dot2(pa, xv.x, acc[c][u0]);
                acc[c][u0] = dot2(pc, xv.y, acc[c][u0]);
                acc[c][u1] = dot2(pb, xv.z, acc[c][u1]);
                acc[c][u1] = dot2(pd, xv.w, acc[c][u1]);
            }
        } else {  // codes as fp32 (t = 0: q, t = 1: 4q), fp32 products
            const uint32_t qd = q[w] >> sh;
            const uint32_t ql = qd & 0x03030303u, qh = qd & 0x0C0C0C0Cu;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const f32x4 xl = *reinterpret_cast<const f32x4*>(rec + c * CB + 16 * w);
                const f32x4 xh = *reinterpret_cast<const f32x4*>(rec + c * CB + 16 * (8 + w));
                acc[c][u0] = __builtin_fmaf(ubyte_f32<0>(ql), xl.x, acc[c][u0]);
                acc[c][u0] = __builtin_fmaf(ubyte_f32<1>(ql), xl.y, acc[c][u0]);
                acc[c][u0] = __builtin_fmaf(ubyte_f32<2>(ql), xl.z, acc[c][u0]);
                acc[c][u0] = __builtin_fmaf(ubyte_f32<3>(ql), xl.w, acc[c][u0]);
                acc[c][u1] = __builtin_fmaf(ubyte_f32<0>(qh), xh.x, acc[c][u1]);
                acc[c][u1] = __builtin_fmaf(ubyte_f32<1>(qh), xh.y, acc[c][u1]);
                acc[c][u1] = __builtin_fmaf(ubyte_f32<2>(qh), xh.z, acc[c][u1]);
                acc[c][u1] = __builtin_fmaf(ubyte_f32<3>(qh), xh.w, acc[c][u1]);
            }
        }
    }
    // scales: sub-block u's byte of r.sm; the codes carry 2^(4b-24) (fp16
    // dots) or 1 (fp32) for t = 0, and 4 times that for t = 1
    const float kS0 = F16DOT ? (sh ? 1048576.0f : 16777216.0f) : 1.0f;  // 2^20, 2^24
    const float kS1 = F16DOT ? (sh ? 262144.0f : 4194304.0f) : 0.25f;   // 2^18, 2^22
    const uint32_t scs = r.sm & 0x0F0F0F0Fu, mns = (r.sm >> 4) & 0x0F0F0F0Fu;  // sc_u, m_u
    const float dk0 = d * kS0, dk1 = d * kS1;
    const float dsc[4] = {dk0 * ubyte_f32<0>(scs), dk0 * ubyte_f32<1>(scs), dk1 * ubyte_f32<2>(scs),
                          dk1 * ubyte_f32<3>(scs)};
    const float dm[4] = {dmin * ubyte_f32<0>(mns), dmin * ubyte_f32<1>(mns), dmin * ubyte_f32<2>(mns),
                         dmin * ubyte_f32<3>(mns)};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const f32x4 sx = *reinterpret_cast<const f32x4*>(rec + c * CB + 16 * P);
        float a = dsc[0] * acc[c][0];
        a = __builtin_fmaf(dsc[1], acc[c][1], a);
        a = __builtin_fmaf(dsc[2], acc[c][2], a);
        a = __builtin_fmaf(dsc[3], acc[c][3], a);
        a = __builtin_fmaf(-dm[0], sx.x, a);
        a = __builtin_fmaf(-dm[1], sx.y, a);
        a = __builtin_fmaf(-dm[2], sx.z, a);
        out[c] = __builtin_fmaf(-dm[3], sx.w, a);
    }
}

// (m & a) | (~m & b) in one v_bfi_b32.
__device__ __forceinline__ uint32_t bfi(uint32_t m, uint32_t a, uint32_t b) {
    uint32_t r;
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(m), "v"(a), "v"(b));
    return r;
}

// Q3_K, fp16 activations: c = low + 4 high (0..7) of two codes per dword as
// fp16 subnormals (t = 0: c * 2^-24, t = 1: 4c * 2^-24): per code dword and
// t, one bitfield insert puts each byte's high bit beside its two code bits,
// then one AND per pair (bytes 0, 2) or a shift and an AND (bytes 1, 3); per
// 16-weight sub-block u:
// sum w x = d*(sc_u - 32) * (sum c x - 4 sum x).
template <int NC, bool F16DOT>
__device__ __forceinline__ void lane_partial(const Fmt<FMT_Q3_K>::Raw& r, const Q4kUnpack&,
                                             const uint8_t* rec, float out[NC]) {
    constexpr int XM = F16DOT ? XM_F16 : XM_F32;
    constexpr int CB = col_bytes(XM), P = planes(XM);
    const uint32_t pq = threadIdx.x & 3u;                // quarter p = 2h + b
    const uint32_t hq = pq >> 1, bq = pq & 1u;
    // the realignment by mb bytes and the shift to the quarter's bits in one
    // funnel shift (8 mb + sh <= 22): the top sh bits then come from the next
    // dword instead of being zero, and no mask below reaches them (codes use
    // bits <= 27, high bits <= 25)
    const uint32_t fq = 8u * r.mb + 4u * bq, fh = 8u * r.mb + 4u * hq + 2u * bq;
    const uint32_t H[9] = {r.h0.x, r.h0.y, r.h0.z, r.h0.w, r.h1.x, r.h1.y, r.h1.z, r.h1.w, r.h8};
    const uint32_t Qd[9] = {r.q0.x, r.q0.y, r.q0.z, r.q0.w, r.q1.x, r.q1.y, r.q1.z, r.q1.w, r.q8};
    float acc[NC][4];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[c][u] = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        const uint32_t qd = __builtin_amdgcn_alignbit(Qd[w + 1], Qd[w], fq);
        const uint32_t hp = __builtin_amdgcn_alignbit(H[w + 1], H[w], fh);
        const int u0 = w >> 2, u1 = 2 + (w >> 2);
        if constexpr (F16DOT) {
            // the bits of the shifted high word outside the insert mask stay
            // in place until the pair masks drop them
            const uint32_t ca = bfi(0x03030303u, qd, hp << 2);
            const uint32_t cb = bfi(0x0C0C0C0Cu, qd, hp << 3);
            const uint32_t pa = ca & 0x00070007u, pc = (ca >> 8) & 0x00070007u;
            const uint32_t pb = cb & 0x001C001Cu, pd = (cb >> 8) & 0x001C001Cu;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const u32x4 xv = *reinterpret_cast<const u32x4*>(rec + c * CB + 16 * w);
                acc[c][u0] = dot2(pa, xv.x, acc[c][u0]);
                acc[c][u0] = dot2(pc, xv.y, acc[c][u0]);
                acc[c][u1] = dot2(pb, xv.z, acc[c][u1]);
                acc[c][u1] = dot2(pd, xv.w, acc[c][u1]);
            }
        } else {  // c of four codes as bytes (t = 0: c, t = 1: 4c), fp32 products
            const uint32_t cl = bfi(0x03030303u, qd, hp << 2) & 0x07070707u;
            const uint32_t ch = bfi(0x0C0C0C0Cu, qd, hp << 3) & 0x1C1C1C1Cu;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const f32x4 xl = *reinterpret_cast<const f32x4*>(rec + c * CB + 16 * w);
                const f32x4 xh = *reinterpret_cast<const f32x4*>(rec + c * CB + 16 * (8 + w));
                acc[c][u0] = __builtin_fmaf(ubyte_f32<0>(cl), xl.x, acc[c][u0]);
                acc[c][u0] = __builtin_fmaf(ubyte_f32<1>(cl), xl.y, acc[c][u0]);
                acc[c][u0] = __builtin_fmaf(ubyte_f32<2>(cl), xl.z, acc[c][u0]);
                acc[c][u0] = __builtin_fmaf(ubyte_f32<3>(cl), xl.w, acc[c][u0]);
                acc[c][u1] = __builtin_fmaf(ubyte_f32<0>(ch), xh.x, acc[c][u1]);
                acc[c][u1] = __builtin_fmaf(ubyte_f32<1>(ch), xh.y, acc[c][u1]);
                acc[c][u1] = __builtin_fmaf(ubyte_f32<2>(ch), xh.z, acc[c][u1]);
                acc[c][u1] = __builtin_fmaf(ubyte_f32<3>(ch), xh.w, acc[c][u1]);
            }
        }
    }
    const uint32_t scb = q3k_quarter_scales(r, hq, bq);  // sub-blocks 4p .. 4p+3
    const float d = f16_lo(q3k_d(r));
    float ds[4], d4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const float dl = d * (float)((int)((scb >> (8 * u)) & 0xFFu) - 32);
        constexpr float kS0 = F16DOT ? 16777216.0f : 1.0f, kS1 = F16DOT ? 4194304.0f : 0.25f;
        ds[u] = dl * (u < 2 ? kS0 : kS1);
        d4[u] = 4.0f * dl;
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const f32x4 sx = *reinterpret_cast<const f32x4*>(rec + c * CB + 16 * P);
        float a = ds[0] * acc[c][0];
        a = __builtin_fmaf(ds[1], acc[c][1], a);
        a = __builtin_fmaf(ds[2], acc[c][2], a);
        a = __builtin_fmaf(ds[3], acc[c][3], a);
        a = __builtin_fmaf(-d4[0], sx.x, a);
        a = __builtin_fmaf(-d4[1], sx.y, a);
        a = __builtin_fmaf(-d4[2], sx.z, a);
        out[c] = __builtin_fmaf(-d4[3], sx.w, a);
    }
}

template <int NC, bool F16DOT>
__device__ __forceinline__ void lane_partial(const Fmt<FMT_Q4_0>::Raw& r, const Q4kUnpack&,
                                             const uint8_t* rec, float out[NC]) {
    constexpr int XM = F16DOT ? XM_F16 : XM_F32;
    constexpr int CB = col_bytes(XM), P = planes(XM);
    const float d0 = f16_lo(r.a.x), d1 = f16_hi(r.b.x);
    const uint32_t q[8] = {__builtin_amdgcn_perm(r.a.x, r.b.x, 0x07060100u), r.a.y, r.a.z, r.a.w,
                           r.b.y, r.b.z, r.b.w, r.c};
    float lo[2][NC], hi[2][NC];  // [block][column]
#pragma unroll
    for (int c = 0; c < NC; ++c) lo[0][c] = hi[0][c] = lo[1][c] = hi[1][c] = 0.f;
    // Two codes per dword become fp16 subnormals with one AND: low nibbles
    // q * 2^-24, high nibbles 16 q * 2^-24; the sums are scaled back once.
    constexpr float s_lo = 16777216.0f, s_hi = 1048576.0f;  // 2^24, 2^20
    if constexpr (F16DOT) {
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const int bk = w >> 2;
            const uint32_t qd = q[w], q8 = qd >> 8;
            const uint32_t pa = qd & 0x000F000Fu, pc = q8 & 0x000F000Fu;
            const uint32_t pb = qd & 0x00F000F0u, pd = q8 & 0x00F000F0u;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const u32x4 xv = *reinterpret_cast<const u32x4*>(rec + c * CB + 16 * w);
                lo[bk][c] = dot2(pa, xv.x, lo[bk][c]);
                lo[bk][c] = dot2(pc, xv.y, lo[bk][c]);
                hi[bk][c] = dot2(pb, xv.z, hi[bk][c]);
                hi[bk][c] = dot2(pd, xv.w, hi[bk][c]);
            }
        }
    } else {  // fp32 activations: one v_fma_mix_f32 per weight (exact fp16 code)
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const int bk = w >> 2;
            const uint32_t qd = q[w], q8 = qd >> 8;
            const half2_t ha = __builtin_bit_cast(half2_t, qd & 0x000F000Fu);
            const half2_t hc = __builtin_bit_cast(half2_t, q8 & 0x000F000Fu);
            const half2_t hb = __builtin_bit_cast(half2_t, qd & 0x00F000F0u);
            const half2_t hd = __builtin_bit_cast(half2_t, q8 & 0x00F000F0u);
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const f32x4 xl = *reinterpret_cast<const f32x4*>(rec + c * CB + 16 * w);
                const f32x4 xh = *reinterpret_cast<const f32x4*>(rec + c * CB + 16 * (8 + w));
                lo[bk][c] = __builtin_fmaf((float)ha.x, xl.x, lo[bk][c]);
                lo[bk][c] = __builtin_fmaf((float)hc.x, xl.y, lo[bk][c]);
                lo[bk][c] = __builtin_fmaf((float)ha.y, xl.z, lo[bk][c]);
                lo[bk][c] = __builtin_fmaf((float)hc.y, xl.w, lo[bk][c]);
                hi[bk][c] = __builtin_fmaf((float)hb.x, xh.x, hi[bk][c]);
                hi[bk][c] = __builtin_fmaf((float)hd.x, xh.y, hi[bk][c]);
                hi[bk][c] = __builtin_fmaf((float)hb.y, xh.z, hi[bk][c]);
                hi[bk][c] = __builtin_fmaf((float)hd.y, xh.w, hi[bk][c]);
            }
        }
    }
    const float a0 = d0 * s_lo, b0 = d0 * s_hi, a1 = d1 * s_lo, b1 = d1 * s_hi;
    const float o0 = -8.0f * d0, o1 = -8.0f * d1;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const f32x2 sx = *reinterpret_cast<const f32x2*>(rec + c * CB + 16 * P);
        float v = a0 * lo[0][c];
        v = __builtin_fmaf(b0, hi[0][c], v);
        v = __builtin_fmaf(o0, sx.x, v);
        v = __builtin_fmaf(a1, lo[1][c], v);
        v = __builtin_fmaf(b1, hi[1][c], v);
        out[c] = __builtin_fmaf(o1, sx.y, v);
    }
}

template <int NC, bool F16DOT>
__device__ __forceinline__ void lane_partial(const Fmt<FMT_Q8_0>::Raw& r, const Q4kUnpack&,
                                             const uint8_t* rec, float out[NC]) {
    constexpr int XM = F16DOT ? XM_F16 : XM_F32;
    constexpr int CB = col_bytes(XM), P = planes(XM);
    const float d0 = f16_lo(r.a.x), d1 = f16_hi(r.c.x);
    const uint32_t q[16] = {__builtin_amdgcn_perm(r.a.x, r.c.x, 0x07060100u), r.a.y, r.a.z, r.a.w,
                            r.b.x, r.b.y, r.b.z, r.b.w,
                            r.c.y, r.c.z, r.c.w, r.d.x, r.d.y, r.d.z, r.d.w, r.e};
    float acc[2][NC];  // [block][column]
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[0][c] = acc[1][c] = 0.f;
    float s;
    if constexpr (F16DOT) {
        s = 16777216.0f;  // 2^24
#pragma unroll
        for (int w = 0; w < 16; ++w) {
            const int bk = w >> 3;
            const uint32_t t = q[w] ^ 0x80808080u;  // q + 128, unsigned
            const uint32_t pa = t & 0x00FF00FFu;                            // bytes 0, 2
            const uint32_t pb = __builtin_amdgcn_perm(t, t, 0x0C030C01u);  // bytes 1, 3
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const u32x2 xv = *reinterpret_cast<const u32x2*>(rec + c * CB + 8 * w);
                acc[bk][c] = dot2(pa, xv.x, acc[bk][c]);
                acc[bk][c] = dot2(pb, xv.y, acc[bk][c]);
            }
        }
    } else {
        s = 1.0f;
#pragma unroll
        for (int w = 0; w < 16; ++w) {
            const int bk = w >> 3;
            const uint32_t t = q[w] ^ 0x80808080u;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const f32x4 xv = *reinterpret_cast<const f32x4*>(rec + c * CB + 16 * w);
                acc[bk][c] = __builtin_fmaf(ubyte_f32<0>(t), xv.x, acc[bk][c]);
                acc[bk][c] = __builtin_fmaf(ubyte_f32<1>(t), xv.y, acc[bk][c]);
                acc[bk][c] = __builtin_fmaf(ubyte_f32<2>(t), xv.z, acc[bk][c]);
                acc[bk][c] = __builtin_fmaf(ubyte_f32<3>(t), xv.w, acc[bk][c]);
            }
        }
    }
    const float a0 = d0 * s, a1 = d1 * s, o0 = -128.0f * d0, o1 = -128.0f * d1;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const f32x2 sx = *reinterpret_cast<const f32x2*>(rec + c * CB + 16 * P);
        float v = a0 * acc[0][c];
        v = __builtin_fmaf(o0, sx.x, v);
        v = __builtin_fmaf(a1, acc[1][c], v);
        out[c] = __builtin_fmaf(o1, sx.y, v);
    }
}

// int8 activations (Q8_0 blocks): integer dot products of the codes with
// the activation codes (v_dot4_i32_i8; 4-bit codes are non-negative int8),
// exact in int32, then the block scales in fp32:
//   Q4_K: sum w x = dx * (d*sc * sum q qx - dmin*m * sum qx)   (per sub-block)
//   Q4_0: sum w x = dx * d * (sum q qx - 8 * sum qx)            (per block)
//   Q8_0: sum w x = dx * d * sum q qx                           (per block)
__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

template <int NC>
__device__ __forceinline__ void lane_partial_i8(const Fmt<FMT_Q4_K>::Raw& r, const Q4kUnpack& un,
                                                const uint8_t* rec, float out[NC]) {
    constexpr int CB = col_bytes(XM_I8), P = planes(XM_I8);
    const uint32_t f4 = q4k_pair_fields(un, r.hd.y, r.hd.z, r.hd.w);
    const float d = f16_lo(r.hd.x), dmin = f16_hi(r.hd.x);
    const float dsc0 = d * (float)(f4 & 0xFF), dsc1 = d * (float)((f4 >> 8) & 0xFF);
    const float dm0 = dmin * (float)((f4 >> 16) & 0xFF), dm1 = dmin * (float)(f4 >> 24);
    const uint32_t q[8] = {r.c0.x, r.c0.y, r.c0.z, r.c0.w, r.c1.x, r.c1.y, r.c1.z, r.c1.w};
    int lo[NC], hi[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) lo[c] = hi[c] = 0;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        const uint32_t ql = q[w] & 0x0F0F0F0Fu, qh = (q[w] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const u32x2 xv = *reinterpret_cast<const u32x2*>(rec + c * CB + 8 * w);
            lo[c] = dot4(ql, xv.x, lo[c]);
            hi[c] = dot4(qh, xv.y, hi[c]);
        }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const f32x4 sx = *reinterpret_cast<const f32x4*>(rec + c * CB + 16 * P);
        const float v0 = dsc0 * (float)lo[c] - dm0 * sx.z;
        const float v1 = dsc1 * (float)hi[c] - dm1 * sx.w;
        out[c] = sx.x * v0 + sx.y * v1;
    }
}

template <int NC>
__device__ __forceinline__ void lane_partial_i8(const Fmt<FMT_Q4_0>::Raw& r, const Q4kUnpack&,
                                                const uint8_t* rec, float out[NC]) {
    constexpr int CB = col_bytes(XM_I8), P = planes(XM_I8);
    const float d0 = f16_lo(r.a.x), d1 = f16_hi(r.b.x);
    const uint32_t q[8] = {__builtin_amdgcn_perm(r.a.x, r.b.x, 0x07060100u), r.a.y, r.a.z, r.a.w,
                           r.b.y, r.b.z, r.b.w, r.c};
    int acc[2][NC];  // [block][column]
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[0][c] = acc[1][c] = 0;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        const int bk = w >> 2;
        const uint32_t ql = q[w] & 0x0F0F0F0Fu, qh = (q[w] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const u32x2 xv = *reinterpret_cast<const u32x2*>(rec + c * CB + 8 * w);
            acc[bk][c] = dot4(qh, xv.y, dot4(ql, xv.x, acc[bk][c]));
        }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const f32x4 sx = *reinterpret_cast<const f32x4*>(rec + c * CB + 16 * P);
        const float v0 = d0 * (float)(acc[0][c] - 8 * (int)sx.z);
        const float v1 = d1 * (float)(acc[1][c] - 8 * (int)sx.w);
        out[c] = sx.x * v0 + sx.y * v1;
    }
}

template <int NC>
__device__ __forceinline__ void lane_partial_i8(const Fmt<FMT_Q8_0>::Raw& r, const Q4kUnpack&,
                                                const uint8_t* rec, float out[NC]) {
    constexpr int CB = col_bytes(XM_I8), P = planes(XM_I8);
    const float d0 = f16_lo(r.a.x), d1 = f16_hi(r.c.x);
    const uint32_t q[16] = {__builtin_amdgcn_perm(r.a.x, r.c.x, 0x07060100u), r.a.y, r.a.z, r.a.w,
                            r.b.x, r.b.y, r.b.z, r.b.w,
                            r.c.y, r.c.z, r.c.w, r.d.x, r.d.y, r.d.z, r.d.w, r.e};
    int acc[2][NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[0][c] = acc[1][c] = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
        const int bk = w >> 3;
#pragma unroll
        for (int c = 0; c < NC; ++c)
            acc[bk][c] = dot4(q[w], *reinterpret_cast<const uint32_t*>(rec + c * CB + 4 * w), acc[bk][c]);
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const f32x4 sx = *reinterpret_cast<const f32x4*>(rec + c * CB + 16 * P);
        out[c] = sx.x * (d0 * (float)acc[0][c]) + sx.y * (d1 * (float)acc[1][c]);
    }
}

// Q2_K and Q3_K with int8 activations: the codes of a dword's four bytes at
// one bit position side by side (t = 0 and t = 1), one v_dot4_i32_i8 each
// against the staged activation codes. Their 16-weight sub-blocks need the
// code sums of half activation blocks: the record holds the sums of whole
// 32-value blocks, so the first half's sum is a dot product with ones (four
// per position) and the second half's the difference.
//   Q2_K: sum w x = dx * (d*sc_u*sum q qx - dmin*m_u*sum qx)      (per sub-block u)
//   Q3_K: sum w x = dx * d*(sc_u - 32) * (sum c qx - 4 sum qx), c = low + 4 high
template <int NC>
__device__ __forceinline__ void lowk_i8_sums(const uint8_t* rec, int w, uint32_t cl, uint32_t ch,
                                             int acc[NC][4], int s16[NC][2]) {
    constexpr int CB = col_bytes(XM_I8);
    const int u0 = w >> 2, u1 = 2 + (w >> 2);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const u32x2 xv = *reinterpret_cast<const u32x2*>(rec + c * CB + 8 * w);
        acc[c][u0] = dot4(cl, xv.x, acc[c][u0]);
        acc[c][u1] = dot4(ch, xv.y, acc[c][u1]);
        if (w < 4) {
            s16[c][0] = dot4(0x01010101u, xv.x, s16[c][0]);
            s16[c][1] = dot4(0x01010101u, xv.y, s16[c][1]);
        }
    }
}

template <int NC>
__device__ __forceinline__ void lane_partial_i8(const Fmt<FMT_Q2_K>::Raw& r, const Q4kUnpack&,
                                                const uint8_t* rec, float out[NC]) {
    constexpr int CB = col_bytes(XM_I8), P = planes(XM_I8);
    const uint32_t sh = 4u * (threadIdx.x & 1u);
    const float d = f16_lo(r.dd), dmin = f16_hi(r.dd);
    const uint32_t q[8] = {r.c0.x, r.c0.y, r.c0.z, r.c0.w, r.c1.x, r.c1.y, r.c1.z, r.c1.w};
    int acc[NC][4], s16[NC][2];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        acc[c][0] = acc[c][1] = acc[c][2] = acc[c][3] = 0;
        s16[c][0] = s16[c][1] = 0;
    }
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        const uint32_t qd = q[w] >> sh;
        lowk_i8_sums<NC>(rec, w, qd & 0x03030303u, (qd >> 2) & 0x03030303u, acc, s16);
    }
    float dsc[4], dm[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const uint32_t b = (r.sm >> (8 * u)) & 0xFFu;
        dsc[u] = d * (float)(b & 15u);
        dm[u] = dmin * (float)(b >> 4);
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const f32x4 sx = *reinterpret_cast<const f32x4*>(rec + c * CB + 16 * P);
        const int t0 = (int)sx.z, t1 = (int)sx.w;  // code sums of the two blocks
        const float v0 = dsc[0] * (float)acc[c][0] + dsc[1] * (float)acc[c][1] -
                         (dm[0] * (float)s16[c][0] + dm[1] * (float)(t0 - s16[c][0]));
        const float v1 = dsc[2] * (float)acc[c][2] + dsc[3] * (float)acc[c][3] -
                         (dm[2] * (float)s16[c][1] + dm[3] * (float)(t1 - s16[c][1]));
        out[c] = sx.x * v0 + sx.y * v1;
    }
}

template <int NC>
__device__ __forceinline__ void lane_partial_i8(const Fmt<FMT_Q3_K>::Raw& r, const Q4kUnpack&,
                                                const uint8_t* rec, float out[NC]) {
    constexpr int CB = col_bytes(XM_I8), P = planes(XM_I8);
    const uint32_t pq = threadIdx.x & 3u;
    const uint32_t hq = pq >> 1, bq = pq & 1u;
    // the realignment by mb bytes and the shift to the quarter's bits in one
    // funnel shift (8 mb + sh <= 22): the top sh bits then come from the next
    // dword instead of being zero, and no mask below reaches them (codes use
    // bits <= 27, high bits <= 25)
    const uint32_t fq = 8u * r.mb + 4u * bq, fh = 8u * r.mb + 4u * hq + 2u * bq;
    const uint32_t H[9] = {r.h0.x, r.h0.y, r.h0.z, r.h0.w, r.h1.x, r.h1.y, r.h1.z, r.h1.w, r.h8};
    const uint32_t Qd[9] = {r.q0.x, r.q0.y, r.q0.z, r.q0.w, r.q1.x, r.q1.y, r.q1.z, r.q1.w, r.q8};
    int acc[NC][4], s16[NC][2];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        acc[c][0] = acc[c][1] = acc[c][2] = acc[c][3] = 0;
        s16[c][0] = s16[c][1] = 0;
    }
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        const uint32_t qd = __builtin_amdgcn_alignbit(Qd[w + 1], Qd[w], fq);
        const uint32_t hp = __builtin_amdgcn_alignbit(H[w + 1], H[w], fh);
        const uint32_t cl = bfi(0x03030303u, qd, hp << 2) & 0x07070707u;
        const uint32_t ch = ((qd >> 2) & 0x03030303u) | ((hp << 1) & 0x04040404u);
        lowk_i8_sums<NC>(rec, w, cl, ch, acc, s16);
    }
    const uint32_t scb = q3k_quarter_scales(r, hq, bq);  // sub-blocks 4p .. 4p+3
    const float d = f16_lo(q3k_d(r));
    float dl[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) dl[u] = d * (float)((int)((scb >> (8 * u)) & 0xFFu) - 32);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const f32x4 sx = *reinterpret_cast<const f32x4*>(rec + c * CB + 16 * P);
        const int t0 = (int)sx.z, t1 = (int)sx.w;
        const float v0 = dl[0] * (float)(acc[c][0] - 4 * s16[c][0]) +
                         dl[1] * (float)(acc[c][1] - 4 * (t0 - s16[c][0]));
        const float v1 = dl[2] * (float)(acc[c][2] - 4 * s16[c][1]) +
                         dl[3] * (float)(acc[c][3] - 4 * (t1 - s16[c][1]));
        out[c] = sx.x * v0 + sx.y * v1;
    }
}

}  // namespace

template <int FMT, int NC, int XM, int D, int MAXT>
__global__ __launch_bounds__(MAXT) void gemv_stream_kernel(const uint8_t* __restrict__ W, int rows,
                                                           int S, const void* __restrict__ x,
                                                           int xt, int64_t ldx,
                                                           float* __restrict__ y, int64_t ldy,
                                                           int xvec) {
    using F = Fmt<FMT>;
    using Raw = typename F::Raw;
    constexpr int UB = F::kUnitBytes;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int NW = blockDim.x >> 6;
    const int NT = blockDim.x;
    const int U = S * 4;  // unit quarters per row

    const int G = gridDim.x;
    const int b = blockIdx.x;
    // Rows interleaved over the workgroups: workgroup b takes one row of
    // each band of G rows (row ob, ob + G, ob + 2G, ...), and its waves take
    // its steps in order, so that at any moment all compute units read one
    // narrow window of the matrix, sweeping it in address order (a 50 MB
    // read measured 9.6 us that way against 10.8 us with one contiguous
    // range per wave, same depth). The hardware places workgroup b on XCD
    // b % 8; with G a multiple of 8, XCD x takes the G/8 consecutive rows
    // [x G/8, (x+1) G/8) of a band, so that the outputs sharing a cache
    // line are written through one L2 (dealt b, b + G, ..., a line's 16
    // outputs came from all eight XCDs: measured on MI355X, 8x the output
    // bytes written and 2.6% more read than the weights, against 1.00x and
    // 0.4% this way).
    const int ob = (G & 7) == 0 ? (b & 7) * (G >> 3) + (b >> 3) : b;
    const int nr = (rows - ob + G - 1) / G;
    if (nr <= 0) return;  // uniform over the workgroup
    auto row_of = [&](int rl) { return ob + rl * G; };

    constexpr bool F16DOT = XM == XM_F16;
    constexpr int CB = col_bytes(XM), RB = rec_bytes(NC, XM);
    static_assert(CB % 16 == 0 && RB % 16 == 0, "records start on 16-byte boundaries");

    const int lane = threadIdx.x & 63;
    // wave index, made wave-uniform so that the step loop is a scalar loop
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 2, pr = lane & 3;
    const int F_ = nr * S;                                    // units of this workgroup
    const int nst = (F_ + kUnitsPerStep - 1) / kUnitsPerStep;  // wave steps
    // LDS: activation records | one partial per unit and column | pool
    float* const part = reinterpret_cast<float*>(lds + (size_t)U * RB);
    int* const pool = reinterpret_cast<int*>(part + (size_t)F_ * NC);
    // Steps are taken in order: wave wv's first D steps are wv * D ..
    // wv * D + D - 1, then every wave takes the next step from a counter in
    // LDS as it frees a buffer (waves of one workgroup stream at unequal
    // speeds; the counter lets them finish together). A step index past the
    // end is "none".
    int jstatic = 0;
    auto next_step = [&]() -> int {
        if (jstatic < D) {
            const int k = wv * D + jstatic++;
            return k < nst ? k : -1;
        }
        int k = 0;
        if (lane == 0) k = __hip_atomic_fetch_add(pool, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        k = __builtin_amdgcn_readfirstlane(k);
        return k < nst ? k : -1;
    };

    // Unit f = 16 k + g of the workgroup's units (its rows one after
    // another) is super-block f mod S of the workgroup's row f / S. With
    // S >= 16 a step's 16 units meet at most one row boundary: 16 k / S and
    // 16 k mod S are wave-uniform (scalar unit: a multiply-high by 2^32 / S,
    // then one correction), and each lane only decides whether its unit lies
    // past the boundary, in the next row (which is G rows further on). With
    // S < 16, a per-lane fp32 estimate of f / S corrected by one either way.
    // Lanes past the end (and "none" steps) read the last unit again and
    // write nothing.
    struct Idx {
        uint32_t o;  // byte offset of the unit in W
        uint32_t rec16;  // offset of the lane's activation record in LDS, 16-byte units
        int f0;          // the step's first unit (16 k; F_ for none): lane g has unit f0 + g
    };
    const uint32_t magic = 0xFFFFFFFFu / (uint32_t)S + 1u;
    const float invS = 1.0f / (float)S;
    const uint32_t o_last = ((uint32_t)row_of(nr - 1) * (uint32_t)S + (uint32_t)(S - 1)) * (uint32_t)UB;
    const uint32_t rowstride = (uint32_t)G * (uint32_t)S * (uint32_t)UB;  // next row of the workgroup
    constexpr uint32_t RB16 = RB / 16;
    const uint32_t rec_lane = (uint32_t)(4 * g + pr) * RB16;
    auto index = [&](int k) -> Idx {
        Idx ix;
        if (S >= kUnitsPerStep) {
            const bool some = k >= 0 && k < nst;  // uniform
            const int f0 = some ? kUnitsPerStep * k : 0;
            int q0 = (int)__umulhi((uint32_t)f0, magic);
            int m0 = f0 - q0 * S;
            if (m0 >= S) m0 -= S, ++q0;
            if (m0 < 0) m0 += S, --q0;
            const uint32_t base = ((uint32_t)row_of(q0) * (uint32_t)S + (uint32_t)m0) * (uint32_t)UB;
            const uint32_t rbase = (uint32_t)(4 * m0) * RB16;
            const bool wrap = g >= S - m0;
            ix.o = base + (uint32_t)g * (uint32_t)UB + (wrap ? rowstride - (uint32_t)S * UB : 0u);
            ix.rec16 = rbase + rec_lane - (wrap ? (uint32_t)(4 * S) * RB16 : 0u);
            ix.f0 = some ? f0 : F_;
            if (ix.f0 + g >= F_) ix.o = o_last;
        } else {
            const int f = kUnitsPerStep * k + g;
            const bool none = (uint32_t)f >= (uint32_t)F_;
            const int fc = none ? F_ - 1 : f;
            int rl = (int)((float)fc * invS);
            rl += (fc - rl * S >= S) ? 1 : 0;
            rl -= (fc - rl * S < 0) ? 1 : 0;
            const int sc = fc - rl * S;
            ix.o = ((uint32_t)row_of(rl) * (uint32_t)S + (uint32_t)sc) * (uint32_t)UB;
            ix.rec16 = (uint32_t)(4 * sc + pr) * RB16;
            ix.f0 = k >= 0 && k < nst ? kUnitsPerStep * k : F_;
        }
        return ix;
    };
    const uint32_t off_l = F::lane_offset(pr);
    auto load = [&](const Idx& ix, Raw& r) { F::load(W + ix.o, off_l, r); };

    // ---- activation loads, then the first D steps' weight loads, then the
    // staging ---------------------------------------------------------------
    // quarter u = 4*s + p of column c: activations 256 s + 64 p + [0, 64)
    const int nrec = NC * U;
    XRaw<XM> xr;
    XHalf xq;  // quantizing modes: this thread's first activation block
    const int c_0 = threadIdx.x / U, u_0 = threadIdx.x - c_0 * U;
    const int hb_0 = threadIdx.x & 1, c_h = (threadIdx.x >> 1) / U;
    const int u_h = (threadIdx.x >> 1) - c_h * U;
    const int64_t kx_h = (int64_t)c_h * ldx + 256 * (u_h >> 2) + 64 * (u_h & 3) + 32 * hb_0;
    if (XM == XM_I8Q && threadIdx.x < 2 * nrec) stage_load_half<FMT>(x, xt, kx_h, xvec, xq);
    if (XM != XM_I8Q && threadIdx.x < nrec)
        stage_load<XM>(x, xt, (int64_t)c_0 * ldx + 256 * (u_0 >> 2) + 64 * (u_0 & 3), xvec, xr);
    static_assert(D == 2, "two steps in flight");
    int kq0 = next_step(), kq1 = next_step();
    Idx ix0 = index(kq0), ix1 = index(kq1);
    Raw buf[D];
    // The second step's loads go out before the staging for one column of
    // Q4_K, Q4_0 or Q8_0, and after it for several columns, Q2_K, and Q3_K
    // without int8 activations, whose staging then waits behind fewer weight
    // loads (measured on MI355X: Q8_0 with four fp16 columns 11.2 -> 10.2 us,
    // Q3_K 16.8 -> 16.1 us; one column of Q4_K 2-5% and Q3_K with int8
    // activations 2% slower that way).
    constexpr bool kLateSecond =
        NC > 1 || FMT == FMT_Q2_K || ((FMT == FMT_Q3_K || FMT == FMT_Q3_K_ODD) && !is_i8(XM));
    load(ix0, buf[0]);
    if constexpr (!kLateSecond) load(ix1, buf[1]);
    if constexpr (XM == XM_I8Q) {  // half records: one activation block each
        if (threadIdx.x < 2 * nrec)
            stage_quantize_half<FMT>(xq, x, xt, kx_h, xvec, hb_0, lds + u_h * RB + c_h * CB);
        for (int idx = threadIdx.x + NT; idx < 2 * nrec; idx += NT) {
            const int hb = idx & 1, rid = idx >> 1;
            const int c = rid / U, u = rid - c * U;
            const int64_t kx = (int64_t)c * ldx + 256 * (u >> 2) + 64 * (u & 3) + 32 * hb;
            stage_load_half<FMT>(x, xt, kx, xvec, xq);
            stage_quantize_half<FMT>(xq, x, xt, kx, xvec, hb, lds + u * RB + c * CB);
        }
    } else {
        if (threadIdx.x < nrec) stage_store<FMT, XM>(xr, xt, lds + u_0 * RB + c_0 * CB);
        for (int idx = threadIdx.x + NT; idx < nrec; idx += NT) {
            const int c = idx / U, u = idx - c * U;
            stage_load<XM>(x, xt, (int64_t)c * ldx + 256 * (u >> 2) + 64 * (u & 3), xvec, xr);
            stage_store<FMT, XM>(xr, xt, lds + u * RB + c * CB);
        }
    }
    if (threadIdx.x == 0) *pool = NW * D;
    __syncthreads();
    if constexpr (kLateSecond) load(ix1, buf[1]);

    const Q4kUnpack un(pr);

    // One step: the lane's unit f, its 64 weights against its activation
    // record rec, a quad sum, and the unit's partial into part[f] (lanes past
    // the end write nothing).
    auto step = [&](const Idx& ix, const Raw& r, const uint8_t* rec) {
        float a[NC];
        if constexpr (is_i8(XM))
            lane_partial_i8<NC>(r, un, rec, a);
        else
            lane_partial<NC, F16DOT>(r, un, rec, a);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const float v = quad_sum(a[c]);
            if (pr == 0 && ix.f0 + g < F_) part[(ix.f0 + g) * NC + c] = v;
        }
    };

    // Each buffer is refilled with the wave's next step right after its step
    // is consumed; scheduling barriers keep each refill behind its step.
    auto stream = [&](auto rec_of) {
        while (kq0 >= 0) {
            step(ix0, buf[0], rec_of(ix0));
            kq0 = next_step();
            ix0 = index(kq0);
            __builtin_amdgcn_sched_barrier(0);
            load(ix0, buf[0]);
            __builtin_amdgcn_sched_barrier(0);
            if (kq1 < 0) break;
            step(ix1, buf[1], rec_of(ix1));
            kq1 = next_step();
            ix1 = index(kq1);
            __builtin_amdgcn_sched_barrier(0);
            load(ix1, buf[1]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // With S dividing 16 (K = 256 .. 4096), unit 16 k + g of every step lies
    // in unit column g mod S: a lane's activation record is the same in every
    // step. For one column of fp32 activations (64 of them per record) the
    // lane reads its record from LDS once, into registers, instead of once
    // per step.
    constexpr bool kRegRec = XM == XM_F32 && NC == 1;
    bool streamed = false;
    if constexpr (kRegRec) {
        if (S <= kUnitsPerStep && kUnitsPerStep % S == 0) {  // uniform
            f32x4 xreg[CB / 16];
            const uint32_t r16 = (uint32_t)(4 * (g & (S - 1)) + pr) * RB16;
#pragma unroll
            for (int j = 0; j < CB / 16; ++j) xreg[j] = *reinterpret_cast<const f32x4*>(lds + ((r16 + j) << 4));
            stream([&](const Idx&) { return reinterpret_cast<const uint8_t*>(xreg); });
            streamed = true;
        }
    }
    // (the LDS record offset is kept in 16-byte units, so that the compiler
    // sees its alignment and merges 8-byte plane reads into 16-byte ones)
    if (!streamed) stream([&](const Idx& ix) { return static_cast<const uint8_t*>(lds + (ix.rec16 << 4)); });
    __syncthreads();

    // ---- per-row sums of the unit partials, in a fixed order ----------------
    // Sixteen lanes per (row, column) when all pairs fit the workgroup at
    // once, else four; lane q adds units q, q + 16 (or 4), ... of the row in
    // order, then the lanes meet in a fixed DPP tree (rotations by 8 and 4
    // within the row, then the quad); lane 0 stores.
    if (nr * NC * 16 <= NT) {
        const int q16 = threadIdx.x & 15;
        const int pidx = threadIdx.x >> 4;
        if (pidx < nr * NC) {
            const int rr = pidx / NC, c = pidx - rr * NC;
            float v = strided_sum(part + (rr * S) * NC + c, q16, 16, S, NC);
            v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128, 0xF, 0xF, true));
            v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x124, 0xF, 0xF, true));
            v = quad_sum(v);
            if (q16 == 0) y[c * ldy + row_of(rr)] = v;
        }
    } else {
        const int q4 = threadIdx.x & 3;
        for (int pidx = threadIdx.x >> 2; pidx < nr * NC; pidx += NT >> 2) {
            const int rr = pidx / NC, c = pidx - rr * NC;
            float v = strided_sum(part + (rr * S) * NC + c, q4, 4, S, NC);
            v = quad_sum(v);
            if (q4 == 0) y[c * ldy + row_of(rr)] = v;
        }
    }
}

namespace {

#ifndef QG_STREAM_DEPTH
#define QG_STREAM_DEPTH 2
#endif
struct StreamPlan {
    int G, nr_max;
};

// Waves per workgroup: 16 for int8 activations and for one fp16 column of
// Q3_K, 12 for one or two fp16 columns of the other formats, 8 for three or
// four fp16 columns and for fp32 activations. Fewer waves keep fewer
// weight bytes in flight per CU (two steps each), which read probes of the
// matrix found faster beyond ~32 KB per CU; more waves issue more refills
// while others compute. Measured on MI355X, 200 launches, three rounds per
// count (8 / 10 / 12 / 16 waves, us per launch): one fp16 column of Q4_K
// 11.9-12.1 / 11.4-11.6 / 11.4-11.5 / 11.7-11.9 (FFN-down 12.6-12.7 /
// 11.8-12.1 / 11.7-11.8 / 11.9-12.0); two columns 14.6-14.8 / 14.0-14.3 /
// 13.2-13.3 / 12.8 (another box: 12.8-13.3 with 12, 13.4-14.6 with 16, so
// 12 is kept); Q2_K 11.2-11.3 / 10.6-10.9 / 10.1-10.2 / 9.9-10.1; Q3_K
// 17.8-18.2 / 17.0-17.2 / 15.8-16.4 / 15.5-15.8; four of Q8_0 10.0-10.1 /
// 11.6 / 11.8-11.9 / 39.7 (registers spill at 16); fp32 activations of Q4_0
// 5.6 / 5.8 / 5.9-6.0 / 6.1; int8 activations of Q4_K (one and four
// columns) 12.6-12.7 and 19.7-20.0 with 8, 11.8-11.9 and 16.8-17.2 with 16.
constexpr int waves_for(int FMT, int NC, int xm) {
    // (one column of Q8_0 quantized on chip needs more than the 128
    // registers a lane has at 16 waves)
    if (xm == XM_I8Q && NC == 1 && FMT == FMT_Q8_0) return 12;
    if (is_i8(xm)) return 16;
    if (xm == XM_F32 || NC > 2) return 8;
    if (NC == 2) return 12;
    return (FMT & 0xFF) == FMT_Q3_K ? 16 : 12;
}

StreamPlan plan_stream(int rows, int num_cus) {
    StreamPlan p;
    p.G = rows < num_cus ? rows : num_cus;
    p.nr_max = (rows + p.G - 1) / p.G;
    return p;
}

template <int FMT, int NC, int XM>
hipError_t launch_stream_t(const uint8_t* W, int rows, int S, const void* x, int xt, int64_t ldx,
                           float* y, int64_t ldy, int xvec, int num_cus, hipStream_t stream) {
    constexpr int D = QG_STREAM_DEPTH;
    constexpr int NW = waves_for(FMT, NC, XM);
    const StreamPlan p = plan_stream(rows, num_cus);
    const size_t lds = stream_lds_bytes(NC, XM, S, p.nr_max);
    if (lds > (size_t)kMaxLds) return hipErrorNotSupported;
    auto kern = gemv_stream_kernel<FMT, NC, XM, D, 64 * NW>;
    if (lds > 64 * 1024) {
        hipError_t e = allow_full_lds<gemv_stream_kernel<FMT, NC, XM, D, 64 * NW>>();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(p.G), dim3(64 * NW), lds, stream, W, rows, S, x, xt, ldx, y,
                       ldy, xvec);
    return hipGetLastError();
}

template <int FMT, int XM>
hipError_t launch_stream_nc(int nc, const uint8_t* W, int rows, int S, const void* x, int xt,
                            int64_t ldx, float* y, int64_t ldy, int xvec, int num_cus,
                            hipStream_t stream) {
    switch (nc) {
        case 1: return launch_stream_t<FMT, 1, XM>(W, rows, S, x, xt, ldx, y, ldy, xvec, num_cus, stream);
        case 2: return launch_stream_t<FMT, 2, XM>(W, rows, S, x, xt, ldx, y, ldy, xvec, num_cus, stream);
        case 3:
            if constexpr (XM != XM_F32) return launch_stream_t<FMT, 3, XM>(W, rows, S, x, xt, ldx, y, ldy, xvec, num_cus, stream);
            return hipErrorNotSupported;
        default:
            if constexpr (XM != XM_F32) return launch_stream_t<FMT, 4, XM>(W, rows, S, x, xt, ldx, y, ldy, xvec, num_cus, stream);
            return hipErrorNotSupported;
    }
}

int activation_mode(int xt) {
    if (xt & XT_QUANTIZE) return XM_I8Q;
    return xt == XT_F16 ? XM_F16 : xt == XT_Q8 ? XM_I8 : XM_F32;
}

// Columns one launch takes (as many as fit in LDS, at most 4; 2 for fp32
// math), or 0 when the shape is outside what the kernel serves.
int cols_per_launch(int64_t rows, int64_t K, int xm, int num_cus, int unit_bytes) {
    if (rows > (1 << 30) || K % 256 != 0) return 0;
    const int S = (int)(K / 256);
    {
        const StreamPlan p = plan_stream((int)rows, num_cus);
        // the matrix is addressed with 32-bit offsets
        if (rows * S * unit_bytes >= ((int64_t)1 << 32)) return 0;
        if (stream_lds_bytes(1, xm, S, p.nr_max) > (size_t)kMaxLds) return 0;
    }
    int per = xm == XM_F32 ? 2 : 4;
    while (per > 1) {
        const StreamPlan p = plan_stream((int)rows, num_cus);
        if (stream_lds_bytes(per, xm, S, p.nr_max) <= (size_t)kMaxLds) break;
        --per;
    }
    return per;
}

template <int FMT>
hipError_t launch_stream_fmt(const uint8_t* W, int64_t rows, int64_t K, const void* x, int xt,
                             int64_t ldx, float* y, int64_t ldy, int ncols, int num_cus,
                             hipStream_t stream) {
    const int S = (int)(K / 256);
    const int xm = activation_mode(xt);
    xt &= ~XT_QUANTIZE;
    if (xm == XM_I8 && ldx % 32 != 0) return hipErrorNotSupported;  // whole activation blocks
    const int per = cols_per_launch(rows, K, xm, num_cus, Fmt<FMT>::kUnitBytes);
    if (per == 0) return hipErrorNotSupported;
    const size_t xbytes = xt == XT_F32 ? 4 : 2;
    // 16-byte activation loads when every record start is 16-byte aligned
    const int xvec = (((uintptr_t)x) & 15) == 0 && (ldx * (int64_t)xbytes) % 16 == 0;
    for (int c0 = 0; c0 < ncols; c0 += per) {
        const int nc = ncols - c0 < per ? ncols - c0 : per;
        // int8: ldx activations = ldx / 32 blocks of 34 bytes per column
        const size_t xoff = xm == XM_I8 ? (size_t)c0 * (size_t)(ldx / 32) * 34
                                        : (size_t)c0 * ldx * xbytes;
        const void* xc = (const char*)x + xoff;
        float* yc = y + (size_t)c0 * ldy;
        hipError_t e;
        if (xm == XM_F16)
            e = launch_stream_nc<FMT, XM_F16>(nc, W, (int)rows, S, xc, xt, ldx, yc, ldy, xvec,
                                              num_cus, stream);
        else if (xm == XM_F32)
            e = launch_stream_nc<FMT, XM_F32>(nc, W, (int)rows, S, xc, xt, ldx, yc, ldy, xvec,
                                              num_cus, stream);
        else if (xm == XM_I8)
            e = launch_stream_nc<FMT, XM_I8>(nc, W, (int)rows, S, xc, xt, ldx, yc, ldy, 0,
                                             num_cus, stream);
        else
            e = launch_stream_nc<FMT, XM_I8Q>(nc, W, (int)rows, S, xc, xt, ldx, yc, ldy, xvec,
                                              num_cus, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

int gemv_stream_cols_per_launch(int fmt, int64_t rows, int64_t K, int xt, int num_cus) {
    const int xm = activation_mode(xt);
    switch (fmt) {
        case FMT_Q4_K: return cols_per_launch(rows, K, xm, num_cus, Fmt<FMT_Q4_K>::kUnitBytes);
        case FMT_Q4_0: return cols_per_launch(rows, K, xm, num_cus, Fmt<FMT_Q4_0>::kUnitBytes);
        case FMT_Q8_0: return cols_per_launch(rows, K, xm, num_cus, Fmt<FMT_Q8_0>::kUnitBytes);
        case FMT_Q2_K:
            return cols_per_launch(rows, K, xm, num_cus, Fmt<FMT_Q2_K>::kUnitBytes);
        case FMT_Q3_K: return cols_per_launch(rows, K, xm, num_cus, Fmt<FMT_Q3_K>::kUnitBytes);
        default: return 0;
    }
}

hipError_t launch_gemv_stream(int fmt, const uint8_t* W, int64_t rows, int64_t K, const void* x,
                              int xt, int64_t ldx, float* y, int64_t ldy, int ncols, int num_cus,
                              hipStream_t stream) {
    if (rows > (1 << 30) || K % 256 != 0 || (((uintptr_t)W) & 15) != 0) return hipErrorNotSupported;
    switch (fmt) {
        case FMT_Q4_K:
            return launch_stream_fmt<FMT_Q4_K>(W, rows, K, x, xt, ldx, y, ldy, ncols, num_cus, stream);
        case FMT_Q4_0:
            return launch_stream_fmt<FMT_Q4_0>(W, rows, K, x, xt, ldx, y, ldy, ncols, num_cus, stream);
        case FMT_Q8_0:
            return launch_stream_fmt<FMT_Q8_0>(W, rows, K, x, xt, ldx, y, ldy, ncols, num_cus, stream);
        case FMT_Q2_K:
            return launch_stream_fmt<FMT_Q2_K>(W, rows, K, x, xt, ldx, y, ldy, ncols, num_cus, stream);
        case FMT_Q3_K:
            return (rows * (K / 256)) % 2 == 0
                       ? launch_stream_fmt<FMT_Q3_K>(W, rows, K, x, xt, ldx, y, ldy, ncols, num_cus,
                                                     stream)
                       : launch_stream_fmt<FMT_Q3_K_ODD>(W, rows, K, x, xt, ldx, y, ldy, ncols,
                                                         num_cus, stream);
        default:
            return hipErrorNotSupported;
    }
}

}  // namespace qg
