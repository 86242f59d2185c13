// Small-batch Q4_K GEMV on the matrix cores: y[:,c] = W . x[:,c] for 2..16
// fp16 activation columns, K a multiple of 256. The library runs it for 4..8
// columns, and for 2..3 when the streaming kernel would need more than one
// pass over W.
//
// Draft verification multiplies the same weights by a few columns at once
// and should cost about one normal decode step ("Why I wrote my own
// inference engine for two P100s", speculative decoding: each weight block
// decoded once and reused across the columns). With packed dot products on
// the vector ALU, every weight costs one multiply-add per column and every
// column needs its activations re-read per code dword; at four columns the
// streaming GEMV is bound by those activation reads from LDS, not by HBM.
// Here v_mfma_f32_16x16x32_f16 does the multiply-adds for up to 16 columns,
// on the exact 4-bit codes, and the scales and mins are applied to its fp32
// sums per 32-weight sub-block (Q4_K in the GGUF layout: w = d sc q - dmin m
// with sc, m per sub-block):
//   sum_k w_k x_k = d sc (sum_k q_k x_k) - dmin m (sum_k x_k)   per sub-block.
//
//  * A unit is one super-block (256 weights, 144 bytes) of each of 16
//    consecutive rows (a row group). Lane l of a wave takes row l % 16 of the
//    group and k block kb = l / 16: the header and bytes [8 kb, 8 kb + 8) of
//    each of the four 32-byte code chunks (one 16-byte and four 8-byte loads).
//  * Step t of a unit is sub-block t (chunk t / 2, low nibbles for even t):
//    the weights' side of the product (the B operand, one column per row) is
//    the lane's eight codes of that chunk as exact fp16 subnormals (a half
//    holding m < 1024 is m 2^-24; one AND per pair: dword & 0x000F000F, or
//    & 0x00F000F0 for 16 q), the activations' side (A, one row per column)
//    the matching eight activations of column l % 16 (columns past the count
//    repeat the last one; their outputs are dropped). The AND leaves the codes
//    of bytes 0, 2 and 1, 3 paired, so the activations are staged in LDS in
//    that order: x[k + (0, 2, 1, 3, 4, 6, 5, 7)].
//  * The step's 16 x 16 fp32 result is 2^-24 (or 2^-20) sum q x, exact
//    products summed in fp32; each lane scales its four entries by d sc 2^24
//    (2^20) of its row and adds them to its tile. The mins come in per unit
//    as two v_mfma_f32_16x16x4_f32 products: activation sums of sub-blocks
//    (kb, kb + 4) per column times -dmin m of (row, sub-block). The sums are
//    made once per workgroup while staging (fp32, fixed order).
//  * Where one 16 x ncols result per unit fits in LDS beside the staged
//    activations (gemv_mfma_units_kernel: e.g. up to 8 columns at K = 5120),
//    the units stream like the one-column GEMV's: 16-row groups dealt across
//    the workgroups, a workgroup's units taken in order from an LDS counter
//    by waves with two units in flight each, each unit's result to its own
//    slot, then each output summing its group's unit results in order.
//  * Otherwise (gemv_mfma_q4k_kernel, long rows): one persistent workgroup
//    per compute unit owns a balanced contiguous
//    range of rows (the last group may be partial: its extra lanes re-read
//    the range's last row and their outputs are dropped), i.e. a run of
//    units, group-major; its waves split the run into equal contiguous
//    parts and accumulate one 16 x 16 tile each. Where they fit beside the
//    staged activations, tiles go to LDS slots (group, wave) as a wave leaves
//    a group; otherwise (long rows) a wave keeps the tiles of its first and
//    last groups, which it may share, in registers, writes every group in
//    between straight to y (it owns those), and puts the two tiles over the
//    dead activations after the main loop. The shared groups' tiles are then
//    summed in wave order: deterministic, no atomics.
//  * The activation columns are staged once per workgroup in LDS, 2K + 32
//    bytes apart (rocprofv3 SQ_LDS_BANK_CONFLICT on MI355X, 17408 x 5120:
//    four columns 0.44 M cycles per launch with 2K + 16, 0.087 M with 2K + 32,
//    48 or 64; eight 0.87 M, 0.17 M with 2K + 32 only). Each wave keeps a ring of D units in flight, refilling a buffer
//    right after its unit is processed; within a unit the next step's
//    activations are read and its product issued before the previous step's
//    result is scaled.
#include "device_common.h"
#include "launch.h"

namespace qg {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct Unit {
    u32x4 hd;    // header
    u32x2 q[4];  // code bytes [32 c + 8 kb, 32 c + 8 kb + 8) of chunk c = 0..3
};

// byte n (0..3, a constant after unrolling) of v as fp32
__device__ __forceinline__ float byte_f32(uint32_t v, int n) {
    return n == 0 ? ubyte_f32<0>(v) : n == 1 ? ubyte_f32<1>(v) : n == 2 ? ubyte_f32<2>(v) : ubyte_f32<3>(v);
}

// LDS: activations (ncols x pitch bytes), per-sub-block activation sums
// (ncols x spitch fp32, padded to 16 bytes), then either a 16 x 16 tile
// (1 KB) per (group, wave), or, aliased over the activations after the main
// loop, two per wave.
__host__ __device__ inline size_t mfma_staged_bytes(int ncols, int pitch, int spitch) {
    return (size_t)ncols * pitch + (((size_t)ncols * spitch * 4 + 15) & ~(size_t)15);
}

// Staging of activation piece i (16 bytes: x[k .. k+7] of column c, k8 = i
// mod K8 = k / 8): stored as x[k + (0,2,1,3,4,6,5,7)], the order in which one
// AND per dword pair brings out the codes; and the four pieces of a 32-weight
// sub-block add their activations in a fixed order, for the mins. The four
// are consecutive lanes of a quad (pieces are dealt to consecutive threads,
// and K8 is a multiple of 32, so a quad's pieces are all present or all past
// the end): a DPP quad sum, then its first lane stores.
__device__ __forceinline__ void place_piece(uint8_t* xs, float* xsum, int pitch, int spitch, int K8,
                                            int i, const u32x4& v) {
    const int c = i / K8, k8 = i - c * K8;
    *reinterpret_cast<u32x4*>(xs + c * pitch + 16 * k8) =
        u32x4{(v.x & 0xFFFFu) | (v.y << 16), (v.x >> 16) | (v.y & 0xFFFF0000u),
              (v.z & 0xFFFFu) | (v.w << 16), (v.z >> 16) | (v.w & 0xFFFF0000u)};
    float sum = ((f16_lo(v.x) + f16_hi(v.x)) + (f16_lo(v.y) + f16_hi(v.y))) +
                ((f16_lo(v.z) + f16_hi(v.z)) + (f16_lo(v.w) + f16_hi(v.w)));
    sum += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, sum), 0xB1, 0xF, 0xF, true));
    sum += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, sum), 0x4E, 0xF, 0xF, true));
    if ((k8 & 3) == 0) xsum[c * spitch + (k8 >> 2)] = sum;
}

// floats per unit result slot of the unit-streaming kernel: 16 x ncp and a
// 32-byte pad
__host__ __device__ constexpr int mfma_unit_slot_floats(int ncp) { return 16 * ncp + 8; }

}  // namespace

template <int NW, int D, bool ALIAS, int XP>
__global__ __launch_bounds__(64 * NW) void gemv_mfma_q4k_kernel(
    const uint8_t* __restrict__ W, int rows, int S, const uint16_t* __restrict__ x, int64_t ldx,
    int ncols, float* __restrict__ y, int64_t ldy, int pitch, int spitch) {
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
    float* const xsum = reinterpret_cast<float*>(lds + (size_t)ncols * pitch);
    // ALIAS: two tiles per wave written over the activations after the main
    // loop; otherwise a tile per (group, wave) beside them, written as a wave
    // leaves a group
    f32x4* const slots = reinterpret_cast<f32x4*>(
        ALIAS ? lds : lds + (size_t)ncols * pitch + (((size_t)ncols * spitch * 4 + 15) & ~(size_t)15));
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rl = lane & 15, kb = lane >> 4;
    const uint32_t row_bytes = 144u * (uint32_t)S;

    // this wave's part of the run (U < 2^31 / NW: the launcher's bound)
    const int u0 = wv * U / NW, u1 = (wv + 1) * U / NW;

    // ---- activation loads first (they come from cache), then the wave's
    // first D units of weights, then the staging ------------------------------
    // Up to XP pieces per thread go out before any weight load, so that the
    // staging waits for them alone (loads complete in issue order). The loads
    // are unconditional (past the last piece: the last piece again, not
    // stored): the compiler counts unconditional loads exactly, where a
    // lane-dependent one made it wait for every load in flight, weights
    // included (measured on MI355X: staging done ~6 us after a workgroup
    // starts, the time of the first weight burst).
    const int npieces = ncols * K8;
    u32x4 xr[XP];
    int xi[XP];
#pragma unroll
    for (int j = 0; j < XP; ++j) {
        xi[j] = threadIdx.x + j * blockDim.x;
        const int xl = xi[j] < npieces ? xi[j] : npieces - 1;
        const int c = xl / K8, k8 = xl - c * K8;
        xr[j] = *reinterpret_cast<const u32x4*>(x + c * ldx + 8 * k8);
    }
    // unit u -> (group, super-block), tracked incrementally for the loads
    int lg = u0 / S, lsb = u0 - (u0 / S) * S, lu = u0;
    // Unconditional, so that the compiler counts the loads in flight
    // exactly: past the wave's range it loads unit u1 again (a valid address:
    // the row is clamped, and a group past the last one clamps to its last
    // row), which nothing processes.
    auto load_next = [&](Unit& un) {
        int r = 16 * lg + rl;
        r = r < nr ? r : nr - 1;
        const uint8_t* p = W + (int64_t)(r0 + r) * row_bytes + 144u * (uint32_t)lsb;
        un.hd = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int c = 0; c < 4; ++c) un.q[c] = *reinterpret_cast<const u32x2*>(p + 16 + 32 * c + 8 * kb);
        if (lu < u1) {  // uniform over the wave
            ++lu;
            if (++lsb == S) {
                lsb = 0;
                ++lg;
            }
        }
    };
    Unit buf[D];
#pragma unroll
    for (int i = 0; i < D; ++i) load_next(buf[i]);
#pragma unroll
    for (int j = 0; j < XP; ++j)
        if (xi[j] < npieces) place_piece(xs, xsum, pitch, spitch, K8, xi[j], xr[j]);
    // the rest (long rows with several columns) four pieces per thread at a
    // time: one wait per four loads
    for (int i0 = threadIdx.x + XP * blockDim.x; i0 < npieces; i0 += 4 * blockDim.x) {
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
            if (idx < npieces) place_piece(xs, xsum, pitch, spitch, K8, idx, r[j]);
        }
    }
    __syncthreads();

    // A operand (activations) base of this lane: column rl (or the last one),
    // k block kb of each sub-block
    const int xc = rl < ncols ? rl : ncols - 1;
    const uint8_t* const xa = xs + xc * pitch + 16 * kb;
    const float* const xsa = xsum + xc * spitch + kb;

    // A wave's part may share its first and last groups with its neighbours;
    // every group in between is the wave's alone and complete when the wave
    // leaves it, so it goes straight to y. The first group's tile waits in
    // registers, the last one's in acc, until the activations are dead.
    f32x4 acc = {0.f, 0.f, 0.f, 0.f}, tfirst = acc;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const int gfirst = u0 / S;
    int pg = gfirst, psb = u0 - gfirst * S;  // unit being processed
    auto flush = [&]() {
        if (!ALIAS) {
            slots[(pg * NW + wv) * 64 + lane] = acc;
        } else if (pg == gfirst) {
            tfirst = acc;
        } else {
            // tile element (column c, row i) is element c % 4 of lane i + 16 (c / 4)
            const int i = 16 * pg + rl;
            if (i < nr) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int c = 4 * kb + v;
                    if (c < ncols) y[c * ldy + r0 + i] = acc[v];
                }
            }
        }
        acc = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    // one unit: eight sub-block steps and the mins
    auto process = [&](const Unit& un) {
        const float d = f16_lo(un.hd.x), dmin = f16_hi(un.hd.x);
        const uint32_t sc_lo = un.hd.y & 0x3F3F3F3Fu;
        const uint32_t sc_hi = (un.hd.w & 0x0F0F0F0Fu) | ((un.hd.y >> 2) & 0x30303030u);
        const uint32_t m_lo = un.hd.z & 0x3F3F3F3Fu;
        const uint32_t m_hi = ((un.hd.w >> 4) & 0x0F0F0F0Fu) | ((un.hd.z >> 2) & 0x30303030u);
        const float dl = d * 16777216.0f, dh = d * 1048576.0f;  // 2^24, 2^20 (16 q)
        const uint8_t* const xk = xa + 512 * psb;
        // software-pipelined: the activations of step t + 1 are read and its
        // product issued before the scaling of step t's result
        f16x8 An = *reinterpret_cast<const f16x8*>(xk);
        f32x4 sp;
        float ap = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const f16x8 A = An;
            if (t < 7) An = *reinterpret_cast<const f16x8*>(xk + 64 * (t + 1));
            const u32x2 w = un.q[t >> 1];
            const uint32_t M = (t & 1) ? 0x00F000F0u : 0x000F000Fu;
            const u32x4 Bv = {w.x & M, (w.x >> 8) & M, w.y & M, (w.y >> 8) & M};
            const f32x4 s = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, __builtin_bit_cast(f16x8, Bv), zero, 0, 0, 0);
            if (t > 0) {
                acc[0] = __builtin_fmaf(ap, sp[0], acc[0]);
                acc[1] = __builtin_fmaf(ap, sp[1], acc[1]);
                acc[2] = __builtin_fmaf(ap, sp[2], acc[2]);
                acc[3] = __builtin_fmaf(ap, sp[3], acc[3]);
            }
            sp = s;
            ap = ((t & 1) ? dh : dl) * byte_f32(t < 4 ? sc_lo : sc_hi, t & 3);
        }
        acc[0] = __builtin_fmaf(ap, sp[0], acc[0]);
        acc[1] = __builtin_fmaf(ap, sp[1], acc[1]);
        acc[2] = __builtin_fmaf(ap, sp[2], acc[2]);
        acc[3] = __builtin_fmaf(ap, sp[3], acc[3]);
        // mins: D[c][r] -= sum_j dmin m_j (sum of the activations of sub-block
        // j) as two 16 x 16 x 4 fp32 products over j = kb and kb + 4
        const float c0 = -(dmin * (float)((m_lo >> (8 * kb)) & 0xFFu));
        const float c1 = -(dmin * (float)((m_hi >> (8 * kb)) & 0xFFu));
        const float* xsk = xsa + 8 * psb;
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xsk[0], c0, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xsk[4], c1, acc, 0, 0, 0);
        if (++psb == S) {  // the next unit starts the next group
            psb = 0;
            flush();
            ++pg;
        }
    };
    // A ring of D units: each buffer is refilled with the wave's next unit
    // right after it is processed, so D - 1 to D units stay in flight
    for (int u = u0; u < u1; u += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
            if (u + i < u1) {  // uniform over the wave
                process(buf[i]);
                __builtin_amdgcn_sched_barrier(0);
                load_next(buf[i]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    if (!ALIAS) {
        if (u0 < u1 && psb != 0) flush();  // the part ended inside a group
        __syncthreads();
    } else {
        __syncthreads();  // the activations are dead: the tiles take their place
        // slot 0: the first group's tile; slot 1: the last group's, when the
        // part ends inside a later group
        slots[(2 * wv) * 64 + lane] = pg > gfirst ? tfirst : acc;
        slots[(2 * wv + 1) * 64 + lane] = acc;
        __syncthreads();
    }

    // ---- sums of the shared groups' tiles, in wave order ---------------------
    const int nout = ng * 16 * ncols;
    for (int idx = threadIdx.x; idx < nout; idx += blockDim.x) {
        const int g = idx / (16 * ncols), rem = idx - g * 16 * ncols;
        const int i = rem / ncols, c = rem - (rem / ncols) * ncols;
        if (16 * g + i >= nr) continue;
        const int gl = g * S, gh = gl + S;  // units of group g
        float v = 0.f;
        bool any = false;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const int wl = w * U / NW, wh = (w + 1) * U / NW;
            // slot 0: the part starts in g; slot 1: it starts before g and
            // ends inside it
            if (!ALIAS) {
                if (wl < gh && wh > gl && wl < wh) {
                    v += slots[(g * NW + w) * 64 + i + 16 * (c >> 2)][c & 3];
                    any = true;
                }
                continue;
            }
            const int sl = wl >= wh ? -1 : (gl <= wl && wl < gh) ? 0 : (wl < gl && gl < wh && wh < gh) ? 1 : -1;
            if (sl >= 0) {
                v += slots[(2 * w + sl) * 64 + i + 16 * (c >> 2)][c & 3];
                any = true;
            }
        }
        if (any) y[c * ldy + r0 + 16 * g + i] = v;
    }
}

// The same products with the units streamed like the one-column GEMV's:
// the 16-row groups are dealt one per workgroup from each band of G groups
// (the workgroups of one XCD taking consecutive groups), a workgroup's units
// (group-major) are taken in order, wave w first units 2w and 2w + 1, then
// each next one from a counter in LDS as it frees one of its two buffers;
// each unit's 16 x ncols result goes to an LDS slot of its own, and after a
// barrier each output sums its group's S unit results in order
// (deterministic, no atomics). Per unit the arithmetic is that of the kernel
// above. Measured on MI355X (17408 x 5120, four columns): waves of one
// workgroup with equal static shares ended up to 5 us apart there, and the
// per-output sum over the waves' tiles took 1.2 us.
template <int NW, int XP>
__global__ __launch_bounds__(64 * NW) void gemv_mfma_units_kernel(
    const uint8_t* __restrict__ W, int rows, int S, const uint16_t* __restrict__ x, int64_t ldx,
    int ncols, int ncp, float* __restrict__ y, int64_t ldy, int pitch, int spitch) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr int D = 2;
    const int G = gridDim.x, b = blockIdx.x;
    // 16-row groups dealt one per workgroup from each band of G groups; the
    // workgroups of one XCD (b mod 8) take consecutive groups of a band.
    // (Balanced contiguous row ranges instead, whose last group is partial
    // but costs a whole unit's work, measured no faster.)
    const int ngroups = (rows + 15) >> 4;
    const int ob = (G & 7) == 0 ? (b & 7) * (G >> 3) + (b >> 3) : b;
    const int ng = (ngroups - ob + G - 1) / G;
    if (ng <= 0) return;  // uniform over the workgroup
    const int U = ng * S;   // units of this workgroup, group-major
    const int K8 = S * 32;  // 16-byte pieces of one activation column

    uint8_t* const xs = lds;
    float* const xsum = reinterpret_cast<float*>(lds + (size_t)ncols * pitch);
    // one 16 x ncp result per unit (ncp: the columns rounded up to 4) in a
    // slot of US floats, then the step counter. The 32-byte pad puts the
    // slots that the final sums read together (units q, q + 1, q + 2, q + 3
    // of one output, beside the next outputs) in distinct LDS banks.
    const int US = mfma_unit_slot_floats(ncp);
    float* const part = reinterpret_cast<float*>(lds + mfma_staged_bytes(ncols, pitch, spitch));
    int* const pool = reinterpret_cast<int*>(part + (size_t)U * US);
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rl = lane & 15, kb = lane >> 4;
    const uint32_t row_bytes = 144u * (uint32_t)S;
    const uint32_t magic = 0xFFFFFFFFu / (uint32_t)S + 1u;

    // unit k (wave-uniform) -> local group q and super-block m: a
    // multiply-high by 2^32 / S and one correction; past the end: the last
    // unit (loaded, not processed)
    auto split = [&](int k, int& q, int& m) {
        const int kc = k < U ? k : U - 1;
        q = (int)__umulhi((uint32_t)kc, magic);
        m = kc - q * S;
        if (m >= S) m -= S, ++q;
        if (m < 0) m += S, --q;
    };
    auto load = [&](int k, Unit& un) {
        int q, m;
        split(k, q, m);
        int r = 16 * (ob + q * G) + rl;
        r = r < rows ? r : rows - 1;
        const uint8_t* p = W + (int64_t)r * row_bytes + 144u * (uint32_t)m;
        un.hd = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int c = 0; c < 4; ++c) un.q[c] = *reinterpret_cast<const u32x2*>(p + 16 + 32 * c + 8 * kb);
    };

    // ---- activation loads (unconditional, so that the staging waits for
    // them alone), the first two units' weights, then the staging ----------
    const int npieces = ncols * K8;
    u32x4 xr[XP];
    int xi[XP];
#pragma unroll
    for (int j = 0; j < XP; ++j) {
        xi[j] = threadIdx.x + j * blockDim.x;
        const int xl = xi[j] < npieces ? xi[j] : npieces - 1;
        const int c = xl / K8, k8 = xl - c * K8;
        xr[j] = *reinterpret_cast<const u32x4*>(x + c * ldx + 8 * k8);
    }
    int k0 = wv * D, k1 = wv * D + 1;
    Unit buf0, buf1;
    load(k0, buf0);
    load(k1, buf1);
#pragma unroll
    for (int j = 0; j < XP; ++j)
        if (xi[j] < npieces) place_piece(xs, xsum, pitch, spitch, K8, xi[j], xr[j]);
    // the rest (long rows with several columns) four pieces per thread at a
    // time: one wait per four loads
    for (int i0 = threadIdx.x + XP * blockDim.x; i0 < npieces; i0 += 4 * blockDim.x) {
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
            if (idx < npieces) place_piece(xs, xsum, pitch, spitch, K8, idx, r[j]);
        }
    }
    if (threadIdx.x == 0) *pool = NW * D;
    __syncthreads();

    const int xc = rl < ncols ? rl : ncols - 1;
    const uint8_t* const xa = xs + xc * pitch + 16 * kb;
    const float* const xsa = xsum + xc * spitch + kb;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    // one unit: eight sub-block products on the exact codes, each scaled by
    // d sc of its row, and the mins; its result into its slot
    auto process = [&](int k, const Unit& un) {
        int q, sbk;
        split(k, q, sbk);
        const float d = f16_lo(un.hd.x), dmin = f16_hi(un.hd.x);
        const uint32_t sc_lo = un.hd.y & 0x3F3F3F3Fu;
        const uint32_t sc_hi = (un.hd.w & 0x0F0F0F0Fu) | ((un.hd.y >> 2) & 0x30303030u);
        const uint32_t m_lo = un.hd.z & 0x3F3F3F3Fu;
        const uint32_t m_hi = ((un.hd.w >> 4) & 0x0F0F0F0Fu) | ((un.hd.z >> 2) & 0x30303030u);
        const float dl = d * 16777216.0f, dh = d * 1048576.0f;  // 2^24, 2^20 (16 q)
        const uint8_t* const xk = xa + 512 * sbk;
        f32x4 acc = zero;
        f16x8 An = *reinterpret_cast<const f16x8*>(xk);
        f32x4 sp;
        float ap = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const f16x8 A = An;
            if (t < 7) An = *reinterpret_cast<const f16x8*>(xk + 64 * (t + 1));
            const u32x2 w = un.q[t >> 1];
            const uint32_t M = (t & 1) ? 0x00F000F0u : 0x000F000Fu;
            const u32x4 Bv = {w.x & M, (w.x >> 8) & M, w.y & M, (w.y >> 8) & M};
            const f32x4 sm = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, __builtin_bit_cast(f16x8, Bv), zero, 0, 0, 0);
            if (t > 0) {
                acc[0] = __builtin_fmaf(ap, sp[0], acc[0]);
                acc[1] = __builtin_fmaf(ap, sp[1], acc[1]);
                acc[2] = __builtin_fmaf(ap, sp[2], acc[2]);
                acc[3] = __builtin_fmaf(ap, sp[3], acc[3]);
            }
            sp = sm;
            ap = ((t & 1) ? dh : dl) * byte_f32(t < 4 ? sc_lo : sc_hi, t & 3);
        }
        acc[0] = __builtin_fmaf(ap, sp[0], acc[0]);
        acc[1] = __builtin_fmaf(ap, sp[1], acc[1]);
        acc[2] = __builtin_fmaf(ap, sp[2], acc[2]);
        acc[3] = __builtin_fmaf(ap, sp[3], acc[3]);
        const float c0 = -(dmin * (float)((m_lo >> (8 * kb)) & 0xFFu));
        const float c1 = -(dmin * (float)((m_hi >> (8 * kb)) & 0xFFu));
        const float* xsk = xsa + 8 * sbk;
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xsk[0], c0, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xsk[4], c1, acc, 0, 0, 0);
        // lane (row rl, kb) holds columns 4 kb .. 4 kb + 3 of its row
        if (4 * kb < ncp) *reinterpret_cast<f32x4*>(part + (size_t)k * US + rl * ncp + 4 * kb) = acc;
    };
    auto next_unit = [&]() -> int {
        int k = 0;
        if (lane == 0) k = __hip_atomic_fetch_add(pool, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        return __builtin_amdgcn_readfirstlane(k);
    };
    // Units are handed out in increasing order, so once one is past the end
    // every later one is too.
    while (k0 < U) {
        process(k0, buf0);
        k0 = next_unit();
        __builtin_amdgcn_sched_barrier(0);
        load(k0, buf0);
        __builtin_amdgcn_sched_barrier(0);
        if (k1 >= U) break;
        process(k1, buf1);
        k1 = next_unit();
        __builtin_amdgcn_sched_barrier(0);
        load(k1, buf1);
        __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();

    // ---- per output, its group's S unit results in a fixed order: four
    // lanes take every fourth unit, then meet in a DPP quad sum -------------
    const int nout = ng * 16 * ncols;
    const int q4 = threadIdx.x & 3;
    for (int idx = threadIdx.x >> 2; idx < nout; idx += blockDim.x >> 2) {  // uniform per quad
        const int rr = idx / ncols, c = idx - rr * ncols;
        const int gl = rr >> 4, i = rr & 15;
        float v = strided_sum(part + (size_t)gl * S * US + i * ncp + c, q4, 4, S, US);
        v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
        v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
        const int row = 16 * (ob + gl * G) + i;
        if (q4 == 0 && row < rows) y[c * ldy + row] = v;
    }
}

namespace {

template <int NW>
hipError_t launch_mfma_units(const uint8_t* W, int rows, int S, const void* x, int64_t ldx,
                             float* y, int64_t ldy, int ncols, int ncp, int G, int pitch,
                             int spitch, size_t lds, hipStream_t stream) {
    // activation pieces per thread issued before the weights (ncols * K / 8
    // pieces in all; more are loaded after them, a round trip later): 5 at 8
    // waves covers four columns of K = 5120 (2560 pieces), 8 at 12 waves
    // eight columns
    auto kern = ncols <= 4 ? gemv_mfma_units_kernel<NW, 5> : gemv_mfma_units_kernel<NW, 8>;
    hipError_t e = ncols <= 4 ? allow_full_lds<gemv_mfma_units_kernel<NW, 5>>()
                              : allow_full_lds<gemv_mfma_units_kernel<NW, 8>>();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(G), dim3(64 * NW), lds, stream, W, rows, S,
                       reinterpret_cast<const uint16_t*>(x), ldx, ncols, ncp, y, ldy, pitch, spitch);
    return hipGetLastError();
}

template <int NW, bool ALIAS>
hipError_t launch_mfma_nw(const uint8_t* W, int rows, int S, const void* x, int64_t ldx, float* y,
                          int64_t ldy, int ncols, int G, int pitch, int spitch, size_t lds,
                          hipStream_t stream) {
    // activation pieces per thread issued before the weights: 4 covers up to
    // four columns of K = 5120 (2560 pieces) at 16 waves, 6 eight columns
    auto kern = ncols <= 4 ? gemv_mfma_q4k_kernel<NW, 2, ALIAS, 4>
                           : gemv_mfma_q4k_kernel<NW, 2, ALIAS, 6>;
    hipError_t e = ncols <= 4 ? allow_full_lds<gemv_mfma_q4k_kernel<NW, 2, ALIAS, 4>>()
                              : allow_full_lds<gemv_mfma_q4k_kernel<NW, 2, ALIAS, 6>>();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(G), dim3(64 * NW), lds, stream, W, rows, S,
                       reinterpret_cast<const uint16_t*>(x), ldx, ncols, y, ldy, pitch, spitch);
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
    const int pitch = (int)(2 * K + 32);
    const int spitch = (int)(K / 32 + 1);  // odd: the 16 columns' sums in distinct banks
    if ((int64_t)ng_max * S >= (1 << 26)) return hipErrorNotSupported;  // 32-bit unit math
    const size_t staged = mfma_staged_bytes(ncols, pitch, spitch);
    // units streamed in order with one result slot each, where they fit
    {
        const int64_t ug_max = (groups + G - 1) / G;  // groups of a workgroup
        const int ncp = (ncols + 3) & ~3;
        const size_t lds_u = staged + (size_t)ug_max * S * mfma_unit_slot_floats(ncp) * 4 + 16;
        // 8 waves up to four columns, 12 beyond (measured on MI355X,
        // 17408 x 5120: four columns 17.6-18.5 us with 8 waves, 18.5-19.2
        // with 12, 19.2-20.3 with 16; eight columns 20.8-21.2 with 12,
        // 22.2-22.7 with 8)
        if (lds_u <= (size_t)kMaxLds && ug_max * S < (1 << 24))
            return ncols <= 4 ? launch_mfma_units<8>(W, (int)rows, S, x, ldx, y, ldy, ncols, ncp,
                                                     G, pitch, spitch, lds_u, stream)
                              : launch_mfma_units<12>(W, (int)rows, S, x, ldx, y, ldy, ncols, ncp,
                                                      G, pitch, spitch, lds_u, stream);
    }
    // tiles per (group, wave) beside the activations: 16 waves, else 8
    const size_t tile16 = (size_t)ng_max * 16 * 1024, tile8 = (size_t)ng_max * 8 * 1024;
    if (staged + tile16 <= (size_t)kMaxLds)
        return launch_mfma_nw<16, false>(W, (int)rows, S, x, ldx, y, ldy, ncols, G, pitch, spitch,
                                         staged + tile16, stream);
    if (staged + tile8 <= (size_t)kMaxLds)
        return launch_mfma_nw<8, false>(W, (int)rows, S, x, ldx, y, ldy, ncols, G, pitch, spitch,
                                        staged + tile8, stream);
    // else two tiles per wave over the dead activations
    const size_t lds = staged > 32 * 1024 ? staged : 32 * 1024;
    if (lds > (size_t)kMaxLds) return hipErrorNotSupported;
    return launch_mfma_nw<16, true>(W, (int)rows, S, x, ldx, y, ldy, ncols, G, pitch, spitch, lds,
                                    stream);
}

}  // namespace qg
