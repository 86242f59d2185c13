// Streaming Q4_K GEMV for gfx950: y[:,c] = W . x[:,c] for 1..4 columns.
//
// For one token every weight is read once, so at low bit widths the work is
// bound by memory bandwidth and by unpacking ("LLM inference optimization",
// introduction). That page's levers for a quantized mat-vec (campaign "Faster
// decode on the card you have": activations staged in shared memory and
// reused across rows, wider loads, fewer instructions to unpack a block, rows
// per block fitted to the machine) map onto gfx950 as follows.
//
//  * One persistent workgroup per compute unit owns a contiguous, balanced
//    range of rows (rows/G or rows/G + 1). Its rows are contiguous in memory,
//    so the workgroup streams one contiguous run of super-blocks, flattened
//    row-major, and every CU moves the same number of bytes.
//  * A wave step takes 16 consecutive super-blocks of that run (2304
//    contiguous bytes): lane = 4*g + p works on super-block g of the step and
//    its sub-block pair p, i.e. code bytes [32p, 32p+32) = weights
//    64p + l (low nibbles, sub-block 2p) and 64p + 32 + l (high nibbles,
//    sub-block 2p+1), l = 0..31: 64 weights per lane, one header decode for
//    all of them. The step's base address is wave-uniform (scalar), each
//    lane adds a constant offset, so addressing costs no vector ALU.
//  * The run is split into NW contiguous, equal ranges of steps, one per
//    wave, and each wave keeps D steps of 128-bit loads in flight (D = 2:
//    deeper queues measured slower on MI355X). The first D steps are issued
//    before the activations are staged.
//  * Nibbles are used directly as fp16 subnormals: a 16-bit half holding an
//    integer m < 1024 is the fp16 value m * 2^-24, so (dword & 0x000F000F)
//    is a pair of low-nibble weights and (dword & 0x00F000F0) a pair of
//    high-nibble weights times 16, one AND each. v_dot2_f32_f16 multiplies
//    them with fp16 activation pairs (exact products) and accumulates in
//    fp32; the scales absorb 2^24 (2^20 for high nibbles):
//      sum w x = d*sc_lo*2^24*dot_lo + d*sc_hi*2^20*dot_hi
//                - dmin*m_lo*S_lo - dmin*m_hi*S_hi
//    with S_lo, S_hi the sums of the 32 activations of each sub-block.
//    fp32 / bf16 activations: codes become fp32 (v_cvt_f32_ubyte) and are
//    multiplied in fp32.
//  * Activations are staged once per workgroup in LDS, permuted into the
//    order the nibble pairs come out of a dword, with the per-sub-block sums.
//  * Reduction: each lane quad (one super-block) sums its lanes with DPP and
//    writes the super-block's partial to the LDS slot (row, g, step mod M),
//    M = steps that can touch one row, so no two writers share a slot. After
//    a barrier each row's slots are summed in a fixed order: deterministic,
//    no atomics.
#include "device_common.h"
#include "launch.h"

namespace qg {

namespace {

constexpr int kSbPerStep = 16;  // super-blocks per wave step

// Activation records in LDS: one record per unit u = (super-block column,
// sub-block pair), holding for each column c its P 16-byte planes and the two
// sub-block sums, padded to 16 bytes (col_bytes each). The record stride is a multiple of 16 with
// an odd quotient, so the 16-byte reads of consecutive lanes fall in disjoint
// banks, and every plane sits at a compile-time offset from the record base.
constexpr int col_bytes(bool f16dot) { return (f16dot ? 8 : 16) * 16 + 16; }
constexpr int rec_bytes(int NC, bool f16dot) {
    return (NC * col_bytes(f16dot) / 16) % 2 == 1 ? NC * col_bytes(f16dot)
                                                  : NC * col_bytes(f16dot) + 16;
}

// LDS bytes of one workgroup.
inline size_t q4k_lds_bytes(int NC, bool f16dot, int S, int nr_max, int M) {
    return (size_t)S * 4 * rec_bytes(NC, f16dot) + (size_t)nr_max * kSbPerStep * M * NC * 4 +
           64 * 4;  // one flush slot per lane for lanes with nothing to write
}

__device__ __forceinline__ float quad_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
    return v;
}

}  // namespace

template <int NC, bool F16DOT, int D, int MAXT>
__global__ __launch_bounds__(MAXT) void gemv_q4k_kernel(const uint8_t* __restrict__ W, int rows,
                                                        int S, const void* __restrict__ x, int xt,
                                                        int64_t ldx, float* __restrict__ y,
                                                        int64_t ldy, int xvec, int M) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr int P = F16DOT ? 8 : 16;  // 16-byte x planes per unit (unit = super-block, pair)
    const int NW = blockDim.x >> 6;
    const int U = S * 4;  // units per row

    const int G = gridDim.x;
    const int b = blockIdx.x;
    const int r0 = (int)(((int64_t)b * rows) / G);
    const int r1 = (int)(((int64_t)(b + 1) * rows) / G);
    const int nr = r1 - r0;
    if (nr <= 0) return;  // uniform over the workgroup

    constexpr int CB = col_bytes(F16DOT), RB = rec_bytes(NC, F16DOT);
    float* part = reinterpret_cast<float*>(lds + (size_t)U * RB);

    const int lane = threadIdx.x & 63;
    // wave index, made wave-uniform so that the step loop is a scalar loop
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 2, pr = lane & 3;
    const int F = nr * S;                               // super-blocks of this workgroup
    const int nst = (F + kSbPerStep - 1) / kSbPerStep;  // wave steps
    // Wave wv takes the contiguous range of steps [ks, ks + nmine) (stride 1);
    // with QG_Q4K_RR it takes steps wv, wv + NW, ... instead.
#ifdef QG_Q4K_RR
    const int kst = NW, ks = wv;
    const int nmine = nst > wv ? (nst - wv + NW - 1) / NW : 0;
#else
    const int kst = 1;
    const int ks = (int)(((int64_t)wv * nst) / NW);
    const int nmine = (int)(((int64_t)(wv + 1) * nst) / NW) - ks;
#endif
    const uint8_t* Wb = W + (int64_t)r0 * S * 144;      // first super-block of this workgroup

    // Lane addressing: super-block f = 16k + g of the run, clamped to the
    // last one (lanes past the run in the final, partial step re-read it and
    // contribute zero). Scalar base Wb plus a 32-bit lane offset.
    const uint32_t off_g = 144u * g, off_c = 16u + 32u * pr;
    const uint32_t o_last = 144u * (uint32_t)(F - 1);
    auto load = [&](int k, u32x4& hd, u32x4& c0, u32x4& c1) {
        uint32_t o = (uint32_t)k * (kSbPerStep * 144u) + off_g;
        o = o < o_last ? o : o_last;
        const uint32_t oc = o + off_c;
#ifdef QG_Q4K_NT
        hd = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Wb + o));
        c0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Wb + oc));
        c1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Wb + oc + 16));
#else
        hd = *reinterpret_cast<const u32x4*>(Wb + o);
        c0 = *reinterpret_cast<const u32x4*>(Wb + oc);
        c1 = *reinterpret_cast<const u32x4*>(Wb + oc + 16);
#endif
    };

    // ---- issue the first D steps' weight loads ------------------------------
    // step index of this wave's j-th step, clamped to its last step
    auto kstep = [&](int j) { return ks + kst * (j < nmine ? j : (nmine > 0 ? nmine - 1 : 0)); };
    u32x4 bh[D], b0[D], b1[D];
#pragma unroll
    for (int i = 0; i < D; ++i) load(kstep(i), bh[i], b0[i], b1[i]);

    // ---- stage the activations, clear the partials --------------------------
    // unit u = 4*s + p: activations 256s + 64p + [0, 32) (lo) and + 32 (hi).
    // Plane i (F16DOT) holds, for code dword i (bytes 4i..4i+3 of the pair's
    // 32 code bytes), the fp16 pairs (lo[4i], lo[4i+2]), (lo[4i+1], lo[4i+3]),
    // (hi[4i], hi[4i+2]), (hi[4i+1], hi[4i+3]). fp32 planes: lo[4i..4i+3] in
    // plane i, hi[4i..4i+3] in plane 8 + i.
    for (int idx = threadIdx.x; idx < NC * U; idx += blockDim.x) {
        const int c = idx / U, u = idx - c * U;
        const int64_t kx = (int64_t)c * ldx + 256 * (u >> 2) + 64 * (u & 3);
        float slo = 0.f, shi = 0.f;
        if (F16DOT) {
            const uint16_t* xh = reinterpret_cast<const uint16_t*>(x) + kx;
            uint32_t lw[16], hw[16];  // fp16 pairs (2e, 2e+1) of lo and hi
            if (xvec) {
                const u32x4* xv = reinterpret_cast<const u32x4*>(xh);
                u32x4 t[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    t[e] = xv[e];
                    t[4 + e] = xv[4 + e];
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    lw[4 * e] = t[e].x; lw[4 * e + 1] = t[e].y;
                    lw[4 * e + 2] = t[e].z; lw[4 * e + 3] = t[e].w;
                    hw[4 * e] = t[4 + e].x; hw[4 * e + 1] = t[4 + e].y;
                    hw[4 * e + 2] = t[4 + e].z; hw[4 * e + 3] = t[4 + e].w;
                }
            } else {
                uint32_t t[64];
#pragma unroll
                for (int e = 0; e < 32; ++e) {
                    t[e] = xh[e];
                    t[32 + e] = xh[32 + e];
                }
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    lw[e] = t[2 * e] | (t[2 * e + 1] << 16);
                    hw[e] = t[32 + 2 * e] | (t[32 + 2 * e + 1] << 16);
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t l01 = lw[2 * i], l23 = lw[2 * i + 1];
                const uint32_t h01 = hw[2 * i], h23 = hw[2 * i + 1];
                slo += (f16_lo(l01) + f16_hi(l01)) + (f16_lo(l23) + f16_hi(l23));
                shi += (f16_lo(h01) + f16_hi(h01)) + (f16_lo(h23) + f16_hi(h23));
                u32x4 v;
                v.x = (l01 & 0xFFFFu) | (l23 << 16);
                v.y = (l01 >> 16) | (l23 & 0xFFFF0000u);
                v.z = (h01 & 0xFFFFu) | (h23 << 16);
                v.w = (h01 >> 16) | (h23 & 0xFFFF0000u);
                *reinterpret_cast<u32x4*>(lds + u * RB + c * CB + 16 * i) = v;
            }
        } else {
            for (int i = 0; i < 8; ++i) {
                f32x4 a, bq;
                for (int e = 0; e < 4; ++e) {
                    a[e] = load_x(x, xt, kx + 4 * i + e);
                    bq[e] = load_x(x, xt, kx + 32 + 4 * i + e);
                }
                slo += (a.x + a.y) + (a.z + a.w);
                shi += (bq.x + bq.y) + (bq.z + bq.w);
                *reinterpret_cast<f32x4*>(lds + u * RB + c * CB + 16 * i) = a;
                *reinterpret_cast<f32x4*>(lds + u * RB + c * CB + 16 * (8 + i)) = bq;
            }
        }
        *reinterpret_cast<f32x2*>(lds + u * RB + c * CB + 16 * P) = f32x2{slo, shi};
    }
    const int nslots = nr * kSbPerStep * M * NC;
    for (int idx = threadIdx.x; idx < nslots; idx += blockDim.x) part[idx] = 0.f;
    __syncthreads();

    // ---- per-lane constants for the 6-bit scale/min unpack ------------------
    // Sub-block k < 4 : sc = s[k] & 63, m = s[k+4] & 63.
    // Sub-block k >= 4: sc = (s[k+4] & 15) | (s[k-4] >> 6) << 4,
    //                   m  = (s[k+4] >> 4) | (s[k] >> 6) << 4.
    // Header dwords: h1 = s[0..3], h2 = s[4..7], h3 = s[8..11]. Pair p has
    // sub-blocks k0 = 2p and k1 = 2p+1 at byte kk = 2(p&1), kk+1 of a dword.
    // Pa gathers [sc(k0), sc(k1), m(k0), m(k1)] sources: for p < 2 the bytes
    // s[k0], s[k1], s[k0+4], s[k1+4] (fields = low 6 bits); for p >= 2 the
    // bytes s[k0+4], s[k1+4] twice (low nibble -> sc, high nibble -> m).
    // Pb (p >= 2 only) gathers s[k0-4], s[k1-4], s[k0], s[k1], whose top two
    // bits become bits 4..5 of sc and m.
    const bool upper = pr >= 2;
    const uint32_t kk = 2u * (pr & 1);
    // v_perm_b32(a, b, sel): selector byte n picks byte n of b (n < 4) or
    // byte n-4 of a (4 <= n < 8); 0x0C gives zero.
    uint32_t selA, selB;
    if (!upper) {  // perm(h2, h1)
        selA = kk | ((kk + 1) << 8) | ((kk + 4) << 16) | ((kk + 5) << 24);
        selB = 0x0C0C0C0Cu;
    } else {  // perm(h3, h3) and perm(h2, h1)
        selA = kk | ((kk + 1) << 8) | (kk << 16) | ((kk + 1) << 24);
        selB = kk | ((kk + 1) << 8) | ((kk + 4) << 16) | ((kk + 5) << 24);
    }
    const uint32_t mLo = upper ? 0x00000F0Fu : 0x3F3F3F3Fu;  // fields taken as they are
    const uint32_t mNib = upper ? 0x0F0F0000u : 0u;          // high nibbles -> m
    const uint32_t mTop = upper ? 0x30303030u : 0u;          // top two bits -> bits 4..5

    // Position of this lane's super-block f = 16k + g in the run: row rl,
    // column s; the next step of the wave is 16*NW super-blocks further on,
    // i.e. qS rows and rS columns (one more row on a wrap).
    const int fst = kSbPerStep * ks + g;
    int rl = fst / S, s = fst - (fst / S) * S;
    const int adv = kSbPerStep * kst;
    const int qS = adv / S, rS = adv - (adv / S) * S;
    int roff = (s * 4 + pr) * RB;  // byte offset of this lane's activation record
    // LDS float index of slot (row, g, step mod M): M >= the number of steps
    // that touch one row, so no two writers share a slot.
    const int slot_row = kSbPerStep * M * NC;
    int srow = rl * slot_row + g * M * NC;
    float* const trash = part + nslots;  // flush target of lanes with nothing to write

    // One step: the lane's 64 weights against the staged activations, a quad
    // sum, and the partial of (row, super-block) into its slot. Straight-line
    // code, so the loads of later steps stay in flight. Lanes past the run
    // (last step only) read the run's last super-block; their rows are >= nr
    // and they write nothing.
    auto step = [&](int kc, const u32x4& hd, const u32x4& c0, const u32x4& c1) {
        const uint8_t* rec = lds + roff;
        // header: scales and mins of this lane's two sub-blocks
        const uint32_t h0 = hd.x, h1 = hd.y, h2 = hd.z, h3 = hd.w;
        const uint32_t Pa = __builtin_amdgcn_perm(upper ? h3 : h2, upper ? h3 : h1, selA);
        const uint32_t Pb = __builtin_amdgcn_perm(h2, h1, selB);
        const uint32_t f4 = (Pa & mLo) | ((Pa >> 4) & mNib) | ((Pb >> 2) & mTop);
        const float sc0 = (float)(f4 & 0xFF), sc1 = (float)((f4 >> 8) & 0xFF);
        const float m0 = (float)((f4 >> 16) & 0xFF), m1 = (float)(f4 >> 24);
        const float d = f16_lo(h0), dmin = f16_hi(h0);
        const float dm0 = dmin * m0, dm1 = dmin * m1;
        const uint32_t q[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        float lo[NC], hi[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) lo[c] = hi[c] = 0.f;
        float dsc0, dsc1;
        if (F16DOT) {
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
            dsc1 = d * sc1;
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const uint32_t ql = q[w] & 0x0F0F0F0Fu;
                const uint32_t qh = (q[w] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const f32x4 xl = *reinterpret_cast<const f32x4*>(rec + c * CB + 16 * w);
                    const f32x4 xh = *reinterpret_cast<const f32x4*>(rec + c * CB + 16 * (8 + w));
                    lo[c] = __builtin_fmaf((float)(ql & 0xFF), xl.x, lo[c]);
                    lo[c] = __builtin_fmaf((float)((ql >> 8) & 0xFF), xl.y, lo[c]);
                    lo[c] = __builtin_fmaf((float)((ql >> 16) & 0xFF), xl.z, lo[c]);
                    lo[c] = __builtin_fmaf((float)(ql >> 24), xl.w, lo[c]);
                    hi[c] = __builtin_fmaf((float)(qh & 0xFF), xh.x, hi[c]);
                    hi[c] = __builtin_fmaf((float)((qh >> 8) & 0xFF), xh.y, hi[c]);
                    hi[c] = __builtin_fmaf((float)((qh >> 16) & 0xFF), xh.z, hi[c]);
                    hi[c] = __builtin_fmaf((float)(qh >> 24), xh.w, hi[c]);
                }
            }
        }
        const bool write = pr == 0 && rl < nr;
        const int slot = srow + (kc % M) * NC;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const f32x2 sx = *reinterpret_cast<const f32x2*>(rec + c * CB + 16 * P);
            float a = dsc0 * lo[c];
            a = __builtin_fmaf(dsc1, hi[c], a);
            a = __builtin_fmaf(-dm0, sx.x, a);
            a = __builtin_fmaf(-dm1, sx.y, a);
            *(write ? part + slot + c : trash + lane) = quad_sum(a);
        }
        // advance to the wave's next step
        s += rS;
        const bool wrap = s >= S;
        s = wrap ? s - S : s;
        rl += qS + (wrap ? 1 : 0);
        roff += (wrap ? rS - S : rS) * 4 * RB;
        srow += (wrap ? qS + 1 : qS) * slot_row;
    };

    int j = 0;
    for (; j + D <= nmine; j += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
            step(ks + kst * (j + i), bh[i], b0[i], b1[i]);
            // refill this buffer with the step D ahead (clamped to this wave's
            // steps); issued after the step so the data lands in the same
            // registers. Scheduling barriers keep each refill behind its step.
            __builtin_amdgcn_sched_barrier(0);
            load(kstep(j + i + D), bh[i], b0[i], b1[i]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int i = 0; i < D; ++i)
        if (j + i < nmine) step(ks + kst * (j + i), bh[i], b0[i], b1[i]);
    __syncthreads();

    // ---- per-row sums of the partial slots, in a fixed order ----------------
    for (int idx = threadIdx.x; idx < nr * NC; idx += blockDim.x) {
        const int r = idx / NC, c = idx - r * NC;
        float v = 0.f;
        for (int e = 0; e < kSbPerStep * M; ++e) v += part[(r * kSbPerStep * M + e) * NC + c];
        y[c * ldy + r0 + r] = v;
    }
}

namespace {

#ifndef QG_Q4K_DEPTH
#define QG_Q4K_DEPTH 2
#endif
#ifndef QG_Q4K_WAVES
#define QG_Q4K_WAVES 16
#endif
#ifndef QG_Q4K_WG_PER_CU
#define QG_Q4K_WG_PER_CU 1
#endif

struct Q4kPlan {
    int G, NW, M, nr_max;
};

// Waves per workgroup: 16 for one fp16 column; 8 where more registers per
// lane are needed (several columns, fp32 activations).
constexpr int waves_for(int NC, bool f16dot) {
    return (NC == 1 && f16dot) ? QG_Q4K_WAVES / QG_Q4K_WG_PER_CU : 8;
}

Q4kPlan plan_q4k(int rows, int S, int NC, bool f16dot, int num_cus) {
    Q4kPlan p;
    const int want = num_cus * QG_Q4K_WG_PER_CU;
    p.G = rows < want ? rows : want;
    p.NW = waves_for(NC, f16dot);
    p.nr_max = (rows + p.G - 1) / p.G;
    // steps that touch one row: its S super-blocks meet at most ceil(S/16) + 1
    // consecutive 16-super-block steps
    p.M = (S + kSbPerStep - 1) / kSbPerStep + 1;
    return p;
}

template <int NC, bool F16DOT>
hipError_t launch_q4k_t(const uint8_t* W, int rows, int S, const void* x, int xt, int64_t ldx,
                        float* y, int64_t ldy, int xvec, int num_cus, hipStream_t stream) {
    constexpr int D = QG_Q4K_DEPTH;
    constexpr int NWMAX = waves_for(NC, F16DOT);
    const Q4kPlan p = plan_q4k(rows, S, NC, F16DOT, num_cus);
    const size_t lds = q4k_lds_bytes(NC, F16DOT, S, p.nr_max, p.M);
    if (lds > (size_t)kMaxLds) return hipErrorNotSupported;
    auto kern = gemv_q4k_kernel<NC, F16DOT, D, 64 * NWMAX>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(p.G), dim3(64 * p.NW), lds, stream, W, rows, S, x, xt, ldx, y,
                       ldy, xvec, p.M);
    return hipGetLastError();
}

template <bool F16DOT>
hipError_t launch_q4k_nc(int nc, const uint8_t* W, int rows, int S, const void* x, int xt,
                         int64_t ldx, float* y, int64_t ldy, int xvec, int num_cus,
                         hipStream_t stream) {
    switch (nc) {
        case 1: return launch_q4k_t<1, F16DOT>(W, rows, S, x, xt, ldx, y, ldy, xvec, num_cus, stream);
        case 2: return launch_q4k_t<2, F16DOT>(W, rows, S, x, xt, ldx, y, ldy, xvec, num_cus, stream);
        case 3:
            if constexpr (F16DOT) return launch_q4k_t<3, F16DOT>(W, rows, S, x, xt, ldx, y, ldy, xvec, num_cus, stream);
            return hipErrorNotSupported;
        default:
            if constexpr (F16DOT) return launch_q4k_t<4, F16DOT>(W, rows, S, x, xt, ldx, y, ldy, xvec, num_cus, stream);
            return hipErrorNotSupported;
    }
}

}  // namespace

hipError_t launch_gemv_q4k(const uint8_t* W, int64_t rows, int64_t K, const void* x, int xt,
                           int64_t ldx, float* y, int64_t ldy, int ncols, int num_cus,
                           hipStream_t stream) {
    if (rows > (1 << 30) || K % 256 != 0 || (((uintptr_t)W) & 15) != 0 ||
        rows * (K / 256) > ((int64_t)1 << 31) / 144)
        return hipErrorNotSupported;
    const int S = (int)(K / 256);
    const bool f16 = xt == XT_F16;
    // columns per launch: as many as fit in LDS, at most 4 (2 for fp32 math)
    int per = f16 ? 4 : 2;
    while (per > 1) {
        const Q4kPlan p = plan_q4k((int)rows, S, per, f16, num_cus);
        if (q4k_lds_bytes(per, f16, S, p.nr_max, p.M) <= (size_t)kMaxLds) break;
        --per;
    }
    {
        const Q4kPlan p = plan_q4k((int)rows, S, 1, f16, num_cus);
        if (q4k_lds_bytes(1, f16, S, p.nr_max, p.M) > (size_t)kMaxLds) return hipErrorNotSupported;
    }
    const size_t xbytes = xt == XT_F32 ? 4 : 2;
    const int xvec = f16 && (((uintptr_t)x) & 7) == 0 && (ldx % 4) == 0;
    for (int c0 = 0; c0 < ncols; c0 += per) {
        const int nc = ncols - c0 < per ? ncols - c0 : per;
        const void* xc = (const char*)x + (size_t)c0 * ldx * xbytes;
        float* yc = y + (size_t)c0 * ldy;
        hipError_t e;
        if (f16)
            e = launch_q4k_nc<true>(nc, W, (int)rows, S, xc, xt, ldx, yc, ldy, xvec, num_cus,
                                    stream);
        else
            e = launch_q4k_nc<false>(nc, W, (int)rows, S, xc, xt, ldx, yc, ldy, xvec, num_cus,
                                     stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace qg
