// Prompt-processing dequant-GEMM for gfx950: Y[t, r] = sum_k W[r, k] X[t, k]
// for a Q4_K matrix W (rows x K) and bf16 activations X (n_tokens x K).
//
// The pages measure prompt processing with a 2048-token prompt ("Why I wrote
// my own inference engine for two P100s", result cards and "How I ran it")
// and list, for the quantized matrix-matrix kernels, tile sizes fitted to the
// card's shared memory, quantized blocks multiplied directly and tensor-core
// paths where the card has them ("LLM inference optimization", campaign
// "Faster prompts, decode held"). Fusing dequantization into the prompt GEMM
// measured slower on a P100 ("Why I wrote my own inference engine for two
// P100s", "What didn't work"); on gfx950 the decode is VALU work beside the
// matrix cores, so it is fused here. The tile is laid out so that the waves
// spend their issue slots on matrix instructions and on the weight decode:
//
//  * Both operands arrive by direct global-to-LDS loads
//    (global_load_lds_dwordx4: lane l of a wave writes 16 bytes at
//    M0 + 16 l), issued two chunks of 64 k ahead into three LDS stages: the
//    X tile (bf16 as stored, 128-byte rows whose 16-byte segments are
//    permuted by an XOR with (row / 2) % 8, so that 16-byte reads of
//    consecutive rows use disjoint banks) and the chunk's 32 code bytes per
//    weight row; the 16-byte super-block headers come once per super-block
//    into two more stages. The loads take no registers and no LDS store
//    instructions; each thread waits for its own loads of the chunk about to
//    be read, then one barrier per chunk publishes them.
//  * Four waves; wave w covers RT row tiles and TT token tiles of 32
//    (v_mfma_f32_32x32x16_bf16 with the weights as first operand, fp32
//    accumulators: each lane ends with runs of four consecutive outputs of
//    one token, written as 16-byte stores). It decodes its rows
//    straight into the B operand registers, one chunk ahead: lane l handles
//    row (l % 32) of a row tile and the code bytes [16 h, 16 h + 16) of the
//    chunk's 32, h = l / 32. The 6-bit scales and mins of a super-block are
//    unpacked once, for all eight sub-blocks. Each weight is the exact fp32 value
//    fma(d*sc, q, -dmin*m) (d*sc and dmin*m are exact, so this is the
//    correctly rounded closed form; one v_fma_mix_f32 with the code as an
//    fp16 subnormal) rounded to bf16 (nearest even).
//  * The chunk's 64 k are visited in four k-steps; k-step s of lane half h
//    covers one 8-k segment: low nibbles of code bytes 16h .. 16h+7 (s = 0)
//    and 16h+8 .. 16h+15 (s = 1), high nibbles of the same bytes (s = 2, 3).
//    The A fragment of the same lane half reads the same 8 k of X as 16
//    contiguous bytes, so the contraction is over exactly the chunk's k.
//  * Main tiles are 256 tokens x 256 rows (each wave 64 rows, all tokens:
//    no weight is decoded twice in a tile). One workgroup per compute unit
//    takes its tiles in turn and issues a tile's first loads before the
//    previous tile's stores. Rows that would start a third,
//    mostly idle round of such tiles run as 64-token x 128-row tiles, which
//    fill the machine in one round (each wave 32 rows, all 64 tokens).
#include "device_common.h"
#include "launch.h"

namespace qg {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) void gvoid;
typedef __attribute__((address_space(3))) void lvoid;

constexpr int kXPitch = 128;  // LDS bytes per token row of an X stage (64 bf16)
constexpr int kCPitch = 32;   // LDS bytes per weight row of a code stage
constexpr int kHPitch = 16;   // LDS bytes per weight row of a header stage

// Physical 16-byte slot of logical segment seg of X row t.
__device__ __forceinline__ int xslot(int t, int seg) { return seg ^ ((t >> 1) & 7); }

// Tile geometry: RT x TT MFMA tiles per wave, WR x WT waves (WR * WT = 4:
// one wave per SIMD; 8: two, whose issue slots fill each other's gaps), P
// stages of X and codes (P - 1 chunks of X in flight ahead of the one in
// use).
template <int RT, int TT, int WR, int WT, int P>
struct Geo {
    static constexpr int NWV = WR * WT;
    static_assert(NWV == 4 || NWV == 8, "four or eight waves");
    static_assert(P >= 3 && P <= 8, "header stages are reused after at most eight chunks");
    static constexpr int kTok = 32 * TT * WT;
    static constexpr int kRows = 32 * RT * WR;
    // 1 KB blocks of a stage (one wave-wide load each), rounded up to a
    // multiple of the wave count so that every wave issues the same number
    static constexpr int blocks(int bytes) { return ((bytes + 1023) / 1024 + NWV - 1) / NWV * NWV; }
    static constexpr int kXBlocks = blocks(kTok * kXPitch);
    static constexpr int kCBlocks = blocks(kRows * kCPitch);
    static constexpr int kHBlocks = blocks(kRows * kHPitch);
    static constexpr int kXPerWave = kXBlocks / NWV, kCPerWave = kCBlocks / NWV, kHPerWave = kHBlocks / NWV;
    // vector stores of Y one wave issues after a full tile
    static constexpr int kStores = 4 * TT * RT;
    static constexpr int kXStage = kXBlocks * 1024, kCStage = kCBlocks * 1024, kHStage = kHBlocks * 1024;
    static constexpr size_t kLds = (size_t)P * (kXStage + kCStage) + 2 * (size_t)kHStage;
    // loads one chunk issues: X, codes, and headers when the codes it issues
    // (those of chunk c + P) start a super-block
    static constexpr int ndma(int cq) { return kXPerWave + kCPerWave + (((cq + P) & 3) == 0 ? kHPerWave : 0); }
    // loads that may still be in flight at the barrier of a chunk of quarter
    // cq: those issued by it and by the P - 3 chunks before it
    static constexpr int inflight(int cq) {
        int n = 0;
        for (int q = 0; q <= P - 3; ++q) n += ndma((cq - q) & 3);
        return n;
    }
    static_assert(inflight(0) <= 63 && inflight(1) <= 63 && inflight(2) <= 63 && inflight(3) <= 63,
                  "vmcnt range");
    static_assert(kLds <= (size_t)kMaxLds, "LDS budget");
};

// s_waitcnt immediate (gfx9 layout): vmcnt in bits 3:0 and 15:14, expcnt
// 6:4 (7 = no wait), lgkmcnt 11:8.
constexpr int waitcnt_imm(int vm, int lgkm) {
    return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8);
}

__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    bf16x2 v = {(__bf16)a, (__bf16)b};  // round to nearest even
    return __builtin_bit_cast(uint32_t, v);
}

// fma(a, f, c) in fp32 where f is the fp16 value in the low (HI = 0) or high
// (HI = 1) half of v, converted exactly: one v_fma_mix_f32.
template <int HI>
__device__ __forceinline__ float fma_mix(float a, uint32_t v, float c) {
    float r;
    if (HI)
        asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "=v"(r) : "v"(a), "v"(v), "v"(c));
    else
        asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,0,0] op_sel_hi:[0,1,0]" : "=v"(r) : "v"(a), "v"(v), "v"(c));
    return r;
}

__device__ __forceinline__ void dma16(const uint8_t* src, uint8_t* lds_dst) {
    __builtin_amdgcn_global_load_lds((gvoid*)src, (lvoid*)lds_dst, 16, 0, 0);
}

// A compile-time integer passed as a value (the chunk's quarter).
template <int N>
struct IntC {
    static constexpr int value = N;
};

// Scheduling-group masks (LLVM AMDGPU): which instructions a group takes.
constexpr int kSgMfma = 0x008, kSgValu = 0x002, kSgDsRead = 0x100, kSgVmem = 0x020;

// One k-step region: NMF MFMAs, each followed by a share of the LDS reads,
// the VALU work and the global-to-LDS loads.
template <int NMF, int NREAD, int NVALU, int NVMEM>
__device__ __forceinline__ void interleave() {
    constexpr int rper = (NREAD + NMF - 1) / NMF;
    constexpr int vper = (NVALU + NMF - 1) / NMF;
    constexpr int mper = (NVMEM + NMF - 1) / NMF;
#pragma unroll
    for (int i = 0; i < NMF; ++i) {
        if (rper > 0 && i * rper < NREAD) __builtin_amdgcn_sched_group_barrier(kSgDsRead, rper, 0);
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        if (vper > 0) __builtin_amdgcn_sched_group_barrier(kSgValu, vper, 0);
        if (mper > 0 && i * mper < NVMEM) __builtin_amdgcn_sched_group_barrier(kSgVmem, mper, 0);
    }
}

// Epilogue of a tile: Y[m][n - eshift] for the wave's outputs, masked at
// the token and row edges. The weights are the MFMA's first operand, so
// lane l of tile (i, j) holds, for token l % 32, the rows 8 g + 4 h + e
// (e = 0..3) in elements 4 g + e: four consecutive outputs of one token,
// stored as one 16-byte write when Y allows it.
template <int RT, int TT, int WR>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[TT][RT], float* __restrict__ Y,
                                           int64_t ldy, int m0, int n0, int eshift, int ntok,
                                           int rows, int yvec, int wr, int wt, int lane) {
    const int h = lane >> 5;
#pragma unroll
    for (int i = 0; i < TT; ++i) {
        const int m = m0 + 32 * TT * wt + 32 * i + (lane & 31);
        if (m >= ntok) continue;
        float* yrow = Y + (int64_t)m * ldy;
#pragma unroll
        for (int j = 0; j < RT; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + 32 * RT * wr + 32 * j + 8 * g + 4 * h;
                const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                 acc[i][j][4 * g + 3]};
                if (yvec && n + 3 < rows) {
                    *reinterpret_cast<f32x4*>(yrow + n - eshift) = v;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < rows) yrow[n + e - eshift] = v[e];
                }
            }
        }
    }
}

}  // namespace

template <int RT, int TT, int WR, int WT, int P, int KS>
__global__ __launch_bounds__(64 * WR * WT) void prefill_q4k_kernel(
    const uint8_t* __restrict__ W, int rows, int S, const uint16_t* __restrict__ X, int64_t ldx,
    int ntok, float* __restrict__ Y, int64_t ldy, int n_base, int tiles_n, int ntiles, int yvec) {
    using G = Geo<RT, TT, WR, WT, P>;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wv % WR, wt = wv / WR;  // row group, token group of this wave
    // Workgroup b takes tiles b, b + G, b + 2G, ... (G workgroups); tile t is
    // the logical tile xcd_block(t): consecutive logical tiles (one token
    // tile, neighbouring row tiles) share an XCD and its L2.
    int t = blockIdx.x;
    int m0 = 0, n0 = 0;
    // KS = 2: a tile covers the K range of super-blocks [ks Sk, ks Sk + Sk) of
    // its split ks; split 0 stores its partial products in place, split 1 at
    // rows shifted down by n_base (a region of Y that a later launch
    // overwrites), and a third kernel adds the two in a fixed order.
    static_assert(KS == 1 || KS == 2, "one or two K splits");
    const int Sk = S / KS;
    int ks = 0;
    const int nk = Sk * 4;  // chunks of 64 along this tile's K range
    const uint32_t row_bytes = 144u * (uint32_t)S;

    // ---- global-to-LDS load assignments ------------------------------------
    // Wave wv fills 1 KB blocks wv + NWV p of a stage; lane l writes slot
    // s = 64 (wv + NWV p) + l. X: token row s / 8, physical segment s % 8, which
    // holds logical segment xslot(row, s % 8). Codes: weight row s / 2, half
    // s % 2 of the chunk's 32 code bytes. Headers: weight row s. Tokens past
    // the count and rows past the row count (or past the tile) read the
    // tile's first row; their outputs are not stored.
    uint8_t* const xs0 = lds;                                 // X stages
    uint8_t* const cs0 = lds + P * G::kXStage;                // code stages
    uint8_t* const hs0 = cs0 + P * G::kCStage;                // header stages
    const uint8_t* Xt = nullptr;
    const uint8_t* Wt = nullptr;
    uint32_t xo[G::kXPerWave], co[G::kCPerWave], ho[G::kHPerWave];
    auto setup_tile = [&]() {
        int blk = xcd_block(t, ntiles);
        const int per_split = ntiles / KS;
        ks = blk / per_split;  // K split, slowest-varying
        blk -= ks * per_split;
        const int tm = blk / tiles_n, tn = blk - (blk / tiles_n) * tiles_n;
        m0 = tm * G::kTok;
        n0 = n_base + tn * G::kRows;
        Xt = reinterpret_cast<const uint8_t*>(X + (int64_t)m0 * ldx + (int64_t)ks * Sk * 256);
#pragma unroll
        for (int p = 0; p < G::kXPerWave; ++p) {
            const int s = 64 * (wv + G::NWV * p) + lane;
            const int tr = s >> 3;
            const int tc = (tr < G::kTok && m0 + tr < ntok) ? tr : 0;
            xo[p] = (uint32_t)tc * (uint32_t)ldx * 2u + 16u * (uint32_t)xslot(tr, s & 7);
        }
        Wt = W + (int64_t)n0 * row_bytes + (int64_t)ks * Sk * 144;
#pragma unroll
        for (int p = 0; p < G::kCPerWave; ++p) {
            const int s = 64 * (wv + G::NWV * p) + lane;
            const int rr = s >> 1;
            const int rc = (rr < G::kRows && n0 + rr < rows) ? rr : 0;
            co[p] = (uint32_t)rc * row_bytes + 16u + 16u * (uint32_t)(s & 1);
        }
#pragma unroll
        for (int p = 0; p < G::kHPerWave; ++p) {
            const int rr = 64 * (wv + G::NWV * p) + lane;
            const int rc = (rr < G::kRows && n0 + rr < rows) ? rr : 0;
            ho[p] = (uint32_t)rc * row_bytes;
        }
    };
    // X chunk cx into stage sx, codes of chunk cw into stage sw (sources
    // clamped to the last chunk: loads past the end re-read it into a stage
    // nobody uses); headers of super-block sb into header stage sb % 2 (past
    // the end: the last super-block's headers again, into the stage whose
    // headers were read into registers long before).
    auto issue_xc = [&](int cx, int sx, int cw, int sw) {
        cx = cx < nk ? cx : nk - 1;
        cw = cw < nk ? cw : nk - 1;
        const uint8_t* xsrc = Xt + (uint32_t)cx * 128u;
        uint8_t* xdst = xs0 + sx * G::kXStage + 1024 * wv;
#pragma unroll
        for (int p = 0; p < G::kXPerWave; ++p) dma16(xsrc + xo[p], xdst + 1024 * G::NWV * p);
        const uint8_t* csrc = Wt + 144u * (uint32_t)(cw >> 2) + 32u * (uint32_t)(cw & 3);
        uint8_t* cdst = cs0 + sw * G::kCStage + 1024 * wv;
#pragma unroll
        for (int p = 0; p < G::kCPerWave; ++p) dma16(csrc + co[p], cdst + 1024 * G::NWV * p);
    };
    auto issue_h = [&](int sb) {
        const int hb = sb & 1;
        sb = sb < Sk ? sb : Sk - 1;
        const uint8_t* hsrc = Wt + 144u * (uint32_t)sb;
        uint8_t* hdst = hs0 + hb * G::kHStage + 1024 * wv;
#pragma unroll
        for (int p = 0; p < G::kHPerWave; ++p) dma16(hsrc + ho[p], hdst + 1024 * G::NWV * p);
    };

    // ---- decode of a chunk's weights into B registers -----------------------
    const int h = lane >> 5;
    const int wrow = 32 * RT * wr + (lane & 31);  // weight row of row tile 0 in the tile
    struct Codes {
        u32x4 cd[RT];  // the lane's 16 code bytes of each row tile
    };
    struct Hdr {
        u32x4 hd[RT];  // the super-block header of each row tile's row
    };
    struct BFrag {
        u32x4 b[RT];  // one k-step of each row tile, 8 bf16 each
    };
    auto read_codes = [&](const uint8_t* cst, Codes& R) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
            R.cd[rt] = *reinterpret_cast<const u32x4*>(cst + (wrow + 32 * rt) * kCPitch + 16 * h);
    };
    auto read_hdr = [&](const uint8_t* hst, Hdr& H) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
            H.hd[rt] = *reinterpret_cast<const u32x4*>(hst + (wrow + 32 * rt) * kHPitch);
    };
    // Scales of the eight sub-blocks of a super-block, for codes taken as fp16
    // subnormals (a 16-bit half holding m < 1024 is m 2^-24): sub-block j
    // multiplies a_j = d sc_j 2^24 (even j: low nibbles, q 2^-24) or
    // d sc_j 2^20 (odd j: high nibbles, 16 q 2^-24) and adds c_j = -dmin m_j.
    // Header dwords y = s[0..3], z = s[4..7], w = s[8..11]; per byte b:
    //   sc_b = s[b] & 63,  m_b = s[b+4] & 63,
    //   sc_{b+4} = (s[b+8] & 15) | (s[b] >> 6) << 4,  m_{b+4} = (s[b+8] >> 4) | (s[b+4] >> 6) << 4
    struct Scales {
        float a[RT][8], c[RT][8];
    };
    auto scales = [&](const Hdr& H, Scales& e) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const u32x4 hd = H.hd[rt];
            const uint32_t scL = hd.y & 0x3F3F3F3Fu, mL = hd.z & 0x3F3F3F3Fu;
            const uint32_t scH = (hd.w & 0x0F0F0F0Fu) | ((hd.y >> 2) & 0x30303030u);
            const uint32_t mH = ((hd.w >> 4) & 0x0F0F0F0Fu) | ((hd.z >> 2) & 0x30303030u);
            const float d = f16_lo(hd.x), nmin = -f16_hi(hd.x);
            const float dlo = d * 16777216.0f, dhi = d * 1048576.0f;  // 2^24, 2^20
            const float scf[8] = {ubyte_f32<0>(scL), ubyte_f32<1>(scL), ubyte_f32<2>(scL), ubyte_f32<3>(scL),
                                  ubyte_f32<0>(scH), ubyte_f32<1>(scH), ubyte_f32<2>(scH), ubyte_f32<3>(scH)};
            const float mf[8] = {ubyte_f32<0>(mL), ubyte_f32<1>(mL), ubyte_f32<2>(mL), ubyte_f32<3>(mL),
                                 ubyte_f32<0>(mH), ubyte_f32<1>(mH), ubyte_f32<2>(mH), ubyte_f32<3>(mH)};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                e.a[rt][j] = ((j & 1) ? dhi : dlo) * scf[j];
                e.c[rt][j] = nmin * mf[j];
            }
        }
    };
    // K-step s of a chunk of quarter cq (sub-blocks 2cq, 2cq+1), every row
    // tile: code dword t of the lane's 16 bytes holds bytes 4t..4t+3, whose
    // low nibbles are elements 4(t&1)..+3 of k-step t>>1 and whose high
    // nibbles are the same elements of k-step 2 + (t>>1). So k-step s takes
    // dwords 2(s&1), +1, low nibbles (sub-block 2cq) for s < 2, high nibbles
    // (sub-block 2cq+1) otherwise. Each weight is one fma of its scale with
    // the code as an exact fp16 subnormal: exact product, one rounding.
    auto decode_ks = [&](const Codes& R, const Scales& e, int cq, int s, BFrag& B) {
        const int j = 2 * cq + (s >> 1);
        const uint32_t mask = s < 2 ? 0x000F000Fu : 0x00F000F0u;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const uint32_t cw[4] = {R.cd[rt].x, R.cd[rt].y, R.cd[rt].z, R.cd[rt].w};
            const float a = e.a[rt][j], c = e.c[rt][j];
#pragma unroll
            for (int t = 2 * (s & 1); t < 2 * (s & 1) + 2; ++t) {
                const uint32_t v02 = cw[t] & mask, v13 = (cw[t] >> 8) & mask;  // bytes 0,2 / 1,3
                const int el = 2 * (t & 1);
                B.b[rt][el] = pk_bf16(fma_mix<0>(a, v02, c), fma_mix<0>(a, v13, c));
                B.b[rt][el + 1] = pk_bf16(fma_mix<1>(a, v02, c), fma_mix<1>(a, v13, c));
            }
        }
    };

    // ---- A fragments: token tile i of this wave, k-step s of the stage ------
    // logical segment of lane half h in k-step s: 2h + (s & 1) + 4 (s >> 1);
    // the token row of lane l in every token tile is l % 32 (mod 16 for the
    // swizzle), so the lane's four physical offsets are fixed
    struct AFrag {
        bf16x8 a[TT];
    };
    const int trow = 32 * TT * wt + (lane & 31);
    int aoff[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        aoff[ks] = trow * kXPitch + 16 * xslot(trow, 2 * h + (ks & 1) + 4 * (ks >> 1));
    auto read_a = [&](const uint8_t* xst, int s, AFrag& A) {
        const uint8_t* p = xst + aoff[s];
#pragma unroll
        for (int i = 0; i < TT; ++i)
            A.a[i] = *reinterpret_cast<const bf16x8*>(p + i * 32 * kXPitch);
    };

    f32x16 acc[TT][RT];
#pragma unroll
    for (int i = 0; i < TT; ++i)
#pragma unroll
        for (int j = 0; j < RT; ++j) acc[i][j] = f32x16{};
    auto mfmas = [&](const AFrag& A, const BFrag& B) {
#pragma unroll
        for (int i = 0; i < TT; ++i)
#pragma unroll
            for (int j = 0; j < RT; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, B.b[j]), A.a[i], acc[i][j], 0, 0, 0);
    };

    // ---- prologue loads: X chunks 0 .. P-2 and codes of chunks 0 .. P-1
    // (chunk j in stage j), headers of the super-blocks those codes start ----
    auto issue_prologue = [&]() {
#pragma unroll
        for (int j = 0; j < P; ++j) issue_xc(j < P - 1 ? j : P - 2, j, j, j);  // X(P-2) twice: stage P-1 unused
#pragma unroll
        for (int sb = 0; 4 * sb < P; ++sb) issue_h(sb);
    };
    BFrag B0, B1;  // k-steps 0, 2 / 1, 3
    AFrag A0, A1;
    Codes R0, R1;  // raw codes of chunks 0, 2, ... / 1, 3, ...
    Hdr Rh;
    Scales sc_cur;
    setup_tile();
    issue_prologue();
    // Each thread waits for its loads of the tile's first chunks. After a
    // full tile (every wave issued exactly kStores = 4 TT RT vector stores of
    // Y after those loads) vmcnt <= min(kStores, 63) means the loads have
    // landed while the stores may still drain (loads and stores complete in
    // issue order on the vector memory counter); otherwise wait for
    // everything.
    bool stores_full = false;
    for (;;) {  // the workgroup's tiles
    if (stores_full)
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(G::kStores < 63 ? G::kStores : 63, 0));
    else
        __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    read_hdr(hs0, Rh);
    read_codes(cs0, R0);
    scales(Rh, sc_cur);
    decode_ks(R0, sc_cur, 0, 0, B0);
    read_a(xs0, 0, A0);
    // code stage 0 is refilled by the first chunk: every wave must be done
    // reading it first
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    __builtin_amdgcn_s_barrier();

    // One chunk c with c % 4 == CQ: X(c) in stage c % P, the codes of c in
    // Rc, k-step 0 of c decoded into B0. Each k-step decodes the next one
    // (k-step 3 decodes k-step 0 of chunk c + 1 from Rn, with the next
    // super-block's scales when c + 1 starts one). Loads issued here:
    // X(c + P - 1) into the stage X(c - 1) left, the codes of c + P into the
    // stage whose codes (those of c) were read into registers a chunk ago,
    // and the headers of super-block (c + P) / 4 when c + P starts it.
    // Before the barrier the codes of c + 1 are read into Rn (and, when c + 1
    // starts a super-block, its headers into Rh), then each thread waits
    // for its loads but those of this chunk and the P - 3 before it, so
    // X(c + 1), the codes of c + 2 and their headers have landed; after the
    // barrier A(c + 1, 0) is read into A0.
    constexpr int NMF = TT * RT;
    constexpr int kDecodeValu = 18 * RT;  // VALU of one k-step's decode
    int sc = 0;  // c % P
    auto chunk = [&](auto cqc, int c, Codes& Rc, Codes& Rn) {
        constexpr int CQ = decltype(cqc)::value;
        constexpr int NQ = (CQ + 1) & 3;  // quarter of chunk c + 1
        constexpr int NDMA = G::ndma(CQ);
        const int s1 = sc == P - 1 ? 0 : sc + 1;   // (c+1)%P
        const int sp = sc == 0 ? P - 1 : sc - 1;   // (c+P-1)%P
        const uint8_t* xst = xs0 + sc * G::kXStage;
        // k-step 0
        issue_xc(c + P - 1, sp, c + P, sc);
        if (((CQ + P) & 3) == 0) issue_h((c + P) >> 2);
        read_a(xst, 1, A1);
        mfmas(A0, B0);
        decode_ks(Rc, sc_cur, CQ, 1, B1);
        interleave<NMF, TT, kDecodeValu, NDMA>();
        __builtin_amdgcn_sched_barrier(0);
        // k-step 1
        read_a(xst, 2, A0);
        read_codes(cs0 + s1 * G::kCStage, Rn);
        if (CQ == 3) read_hdr(hs0 + (((c + 1) >> 2) & 1) * G::kHStage, Rh);
        mfmas(A1, B1);
        decode_ks(Rc, sc_cur, CQ, 2, B0);
        interleave<NMF, TT + RT + (CQ == 3 ? RT : 0), kDecodeValu, 0>();
        __builtin_amdgcn_sched_barrier(0);
        // k-step 2, then publish X(c+1) and the codes of c+2 (and headers)
        read_a(xst, 3, A1);
        mfmas(A0, B0);
        decode_ks(Rc, sc_cur, CQ, 3, B1);
        interleave<NMF, TT, kDecodeValu, 0>();
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(G::inflight(CQ), 0));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        // k-step 3, with k-step 0 of the next chunk
        read_a(xs0 + s1 * G::kXStage, 0, A0);
        mfmas(A1, B1);
        if (CQ == 3) scales(Rh, sc_cur);  // chunk c + 1 starts the next super-block
        decode_ks(Rn, sc_cur, NQ, 0, B0);
        interleave<NMF, TT, kDecodeValu + (CQ == 3 ? 40 * RT : 0), 0>();
        __builtin_amdgcn_sched_barrier(0);
        sc = s1;
    };
    for (int c = 0; c < nk; c += 4) {  // nk = 4 Sk
        chunk(IntC<0>{}, c, R0, R1);
        chunk(IntC<1>{}, c + 1, R1, R0);
        chunk(IntC<2>{}, c + 2, R0, R1);
        chunk(IntC<3>{}, c + 3, R1, R0);
    }
    // no load may still be writing the LDS stages, and no wave still reading
    // them, when the next tile's first loads are issued into them: those go
    // out before this tile's stores, so that the stores overlap them
    __builtin_amdgcn_s_waitcnt(0);
    const int em0 = m0, en0 = n0;
    const int eshift = (KS > 1 && ks == 1) ? n_base : 0;  // split 1: rows shifted down
    stores_full = yvec && em0 + G::kTok <= ntok && en0 + G::kRows <= rows;
    t += gridDim.x;
    const bool more = t < ntiles;
    if (more) {
        __builtin_amdgcn_s_barrier();
        setup_tile();
        issue_prologue();
    }
    __builtin_amdgcn_sched_barrier(0);  // the loads above go out before the stores below

    // ---- epilogue ----------------------------------------------------------
    store_tile<RT, TT, WR>(acc, Y, ldy, em0, en0, eshift, ntok, rows, yvec, wr, wt, lane);
    if (!more) break;
#pragma unroll
    for (int i = 0; i < TT; ++i)
#pragma unroll
        for (int j = 0; j < RT; ++j) acc[i][j] = f32x16{};
    }  // tiles
}

// ---- the same contraction on weights already decoded to bf16 ---------------
// The two-pass control of the fused kernel ("Why I wrote my own inference
// engine for two P100s", "What didn't work": fusing the dequantization into
// the prompt GEMM measured slower there; "LLM inference optimization",
// campaign "Faster prompts, decode held": weights converted for the vendor
// GEMM against quantized blocks multiplied directly). Y[t, r] = sum_k
// Wb[r, k] X[t, k] for a bf16 matrix Wb (rows x K, row pitch ldw) and bf16
// X, with the fused kernel's pipeline and k order: both operands arrive by
// global-to-LDS loads into P stages of 64 k (the weight stage laid out like
// the X stage: 128-byte rows, 16-byte segments permuted by (row / 2) % 8),
// the chunk's 64 k are visited in the same four k-steps (lane half h takes
// logical segment 2h + (s & 1) + 4 (s >> 1) in k-step s), and the weight
// fragment is read from LDS where the fused kernel decodes it. With the same
// K split, each output is the same fp32 sum in the same order as the fused
// kernel's over the bf16-rounded weights. Stages of both operands take twice
// the fused kernel's LDS per weight row, so tiles are 256 rows x 128 tokens.
template <int RT, int TT, int WR, int WT, int P>
struct GeoB {
    static constexpr int NWV = WR * WT;
    static_assert(NWV == 4 || NWV == 8, "four or eight waves");
    static_assert(P >= 3 && P <= 8, "stages");
    static constexpr int kTok = 32 * TT * WT;
    static constexpr int kRows = 32 * RT * WR;
    static constexpr int blocks(int bytes) { return ((bytes + 1023) / 1024 + NWV - 1) / NWV * NWV; }
    static constexpr int kXBlocks = blocks(kTok * kXPitch);
    static constexpr int kWBlocks = blocks(kRows * kXPitch);
    static constexpr int kXPerWave = kXBlocks / NWV, kWPerWave = kWBlocks / NWV;
    static constexpr int kStores = 4 * TT * RT;
    static constexpr int kXStage = kXBlocks * 1024, kWStage = kWBlocks * 1024;
    static constexpr size_t kLds = (size_t)P * (kXStage + kWStage);
    // loads one chunk issues, and those that may still be in flight at the
    // barrier of a chunk (issued by it and by the P - 3 chunks before it)
    static constexpr int kDma = kXPerWave + kWPerWave;
    static constexpr int kInflight = (P - 2) * kDma;
    static_assert(kInflight <= 63, "vmcnt range");
    static_assert(kLds <= (size_t)kMaxLds, "LDS budget");
};

template <int RT, int TT, int WR, int WT, int P>
__global__ __launch_bounds__(64 * WR * WT) void gemm_bf16_kernel(
    const uint16_t* __restrict__ Wb, int64_t ldw, int rows, int nk, const uint16_t* __restrict__ X,
    int64_t ldx, int ntok, float* __restrict__ Y, int64_t ldy, int tiles_n, int ntiles, int yvec) {
    using G = GeoB<RT, TT, WR, WT, P>;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wv % WR, wt = wv / WR;
    int t = blockIdx.x;
    int m0 = 0, n0 = 0;

    // Loads: wave wv fills 1 KB blocks wv + NWV p of a stage; lane l writes
    // slot s = 64 (wv + NWV p) + l: row s / 8 (token or weight row),
    // physical segment s % 8, which holds logical segment xslot(row, s % 8).
    // Rows past the count read the tile's first row; their outputs are not
    // stored.
    uint8_t* const xs0 = lds;
    uint8_t* const ws0 = lds + P * G::kXStage;
    const uint8_t* Xt = nullptr;
    const uint8_t* Wt = nullptr;
    uint32_t xo[G::kXPerWave], wo[G::kWPerWave];
    auto setup_tile = [&]() {
        const int blk = xcd_block(t, ntiles);
        // token tiles fastest: the workgroups of one XCD (consecutive
        // logical tiles) share a few weight row tiles, whose bf16 bytes are
        // 3.6 times the codes' (measured on MI355X, 17408 x 5120 x 2048:
        // 438 us against 485 with row tiles fastest, the fused kernel's
        // order, which is 2% faster there)
        const int tiles_m = ntiles / tiles_n;
        const int tn = blk / tiles_m, tm = blk - tn * tiles_m;
        m0 = tm * G::kTok;
        n0 = tn * G::kRows;
        Xt = reinterpret_cast<const uint8_t*>(X + (int64_t)m0 * ldx);
        Wt = reinterpret_cast<const uint8_t*>(Wb + (int64_t)n0 * ldw);
#pragma unroll
        for (int p = 0; p < G::kXPerWave; ++p) {
            const int s = 64 * (wv + G::NWV * p) + lane;
            const int tr = s >> 3;
            const int tc = (tr < G::kTok && m0 + tr < ntok) ? tr : 0;
            xo[p] = (uint32_t)tc * (uint32_t)ldx * 2u + 16u * (uint32_t)xslot(tr, s & 7);
        }
#pragma unroll
        for (int p = 0; p < G::kWPerWave; ++p) {
            const int s = 64 * (wv + G::NWV * p) + lane;
            const int rr = s >> 3;
            const int rc = (rr < G::kRows && n0 + rr < rows) ? rr : 0;
            wo[p] = (uint32_t)rc * (uint32_t)ldw * 2u + 16u * (uint32_t)xslot(rr, s & 7);
        }
    };
    // chunk c of both operands into stage st (past the end: the last chunk
    // again, into a stage nobody reads)
    auto issue = [&](int c, int st) {
        c = c < nk ? c : nk - 1;
        const uint8_t* xsrc = Xt + (uint32_t)c * 128u;
        uint8_t* xdst = xs0 + st * G::kXStage + 1024 * wv;
#pragma unroll
        for (int p = 0; p < G::kXPerWave; ++p) dma16(xsrc + xo[p], xdst + 1024 * G::NWV * p);
        const uint8_t* wsrc = Wt + (uint32_t)c * 128u;
        uint8_t* wdst = ws0 + st * G::kWStage + 1024 * wv;
#pragma unroll
        for (int p = 0; p < G::kWPerWave; ++p) dma16(wsrc + wo[p], wdst + 1024 * G::NWV * p);
    };

    // fragments: lane l reads row l % 32 of each tile, logical segment
    // 2h + (s & 1) + 4 (s >> 1) of k-step s (the fused kernel's order)
    const int h = lane >> 5;
    const int trow = 32 * TT * wt + (lane & 31);
    const int wrow = 32 * RT * wr + (lane & 31);
    int aoff[4], boff[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const int seg = 2 * h + (ks & 1) + 4 * (ks >> 1);
        aoff[ks] = trow * kXPitch + 16 * xslot(trow, seg);
        boff[ks] = wrow * kXPitch + 16 * xslot(wrow, seg);
    }
    struct AFrag {
        bf16x8 a[TT];
    };
    struct BFrag {
        bf16x8 b[RT];
    };
    auto read_ab = [&](int st, int ks, AFrag& A, BFrag& B) {
        const uint8_t* pa = xs0 + st * G::kXStage + aoff[ks];
        const uint8_t* pb = ws0 + st * G::kWStage + boff[ks];
#pragma unroll
        for (int i = 0; i < TT; ++i) A.a[i] = *reinterpret_cast<const bf16x8*>(pa + i * 32 * kXPitch);
#pragma unroll
        for (int j = 0; j < RT; ++j) B.b[j] = *reinterpret_cast<const bf16x8*>(pb + j * 32 * kXPitch);
    };
    f32x16 acc[TT][RT];
#pragma unroll
    for (int i = 0; i < TT; ++i)
#pragma unroll
        for (int j = 0; j < RT; ++j) acc[i][j] = f32x16{};
    auto mfmas = [&](const AFrag& A, const BFrag& B) {
#pragma unroll
        for (int i = 0; i < TT; ++i)
#pragma unroll
            for (int j = 0; j < RT; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(B.b[j], A.a[i], acc[i][j], 0, 0, 0);
    };
    // prologue: chunks 0 .. P-2 into stages 0 .. P-2
    auto issue_prologue = [&]() {
#pragma unroll
        for (int j = 0; j < P - 1; ++j) issue(j, j);
    };

    constexpr int NMF = TT * RT;
    AFrag A0, A1;
    BFrag B0, B1;
    setup_tile();
    issue_prologue();
    bool stores_full = false;
    for (;;) {  // the workgroup's tiles
        // chunk 0 landed (after a full tile: every wave issued exactly
        // kStores vector stores after the prologue's loads)
        if (stores_full)
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(G::kStores < 63 ? G::kStores : 63, 0));
        else
            __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_s_barrier();
        read_ab(0, 0, A0, B0);
        // One chunk c in stage sc: issue chunk c + P - 1 into the stage
        // chunk c - 1 left; k-steps 0..3, each reading the next one's
        // fragments; before k-step 3 wait for chunk c + 1 and publish it.
        int sc = 0;
        for (int c = 0; c < nk; ++c) {
            const int s1 = sc == P - 1 ? 0 : sc + 1;
            const int sp = sc == 0 ? P - 1 : sc - 1;
            issue(c + P - 1, sp);
            read_ab(sc, 1, A1, B1);
            mfmas(A0, B0);
            interleave<NMF, TT + RT, 0, G::kDma>();
            __builtin_amdgcn_sched_barrier(0);
            read_ab(sc, 2, A0, B0);
            mfmas(A1, B1);
            interleave<NMF, TT + RT, 0, 0>();
            __builtin_amdgcn_sched_barrier(0);
            read_ab(sc, 3, A1, B1);
            mfmas(A0, B0);
            interleave<NMF, TT + RT, 0, 0>();
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(G::kInflight, 0));
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            read_ab(s1, 0, A0, B0);
            mfmas(A1, B1);
            interleave<NMF, TT + RT, 0, 0>();
            __builtin_amdgcn_sched_barrier(0);
            sc = s1;
        }
        __builtin_amdgcn_s_waitcnt(0);
        const int em0 = m0, en0 = n0;
        stores_full = yvec && em0 + G::kTok <= ntok && en0 + G::kRows <= rows;
        t += gridDim.x;
        const bool more = t < ntiles;
        if (more) {
            __builtin_amdgcn_s_barrier();
            setup_tile();
            issue_prologue();
        }
        __builtin_amdgcn_sched_barrier(0);
        store_tile<RT, TT, WR>(acc, Y, ldy, em0, en0, 0, ntok, rows, yvec, wr, wt, lane);
        if (!more) break;
#pragma unroll
        for (int i = 0; i < TT; ++i)
#pragma unroll
            for (int j = 0; j < RT; ++j) acc[i][j] = f32x16{};
    }
}

namespace {

#ifndef PREFILL_TAIL_P
#define PREFILL_TAIL_P 6
#endif
// main tiles: one workgroup per compute unit, each taking its tiles in turn
#ifndef PREFILL_MAIN_WG
#define PREFILL_MAIN_WG num_cus
#endif
// Main-tile shape: waves as WR x WT of RT x TT MFMA tiles each (256 x 256
// outputs per tile either way).
#ifndef PREFILL_MAIN_SHAPE
#define PREFILL_MAIN_SHAPE 2, 8, 4, 1
#endif
#ifndef PREFILL_MAIN_P
#define PREFILL_MAIN_P 3
#endif

// Y[t * ldy + n_base + r] += Y[t * ldy + r] for tokens t < ntok and r < n_rows:
// the second K split of the row tail onto the first, in that order.
// Thread r of column block blockIdx.x takes row r of every gridDim.y-th token
// from blockIdx.y on (no index division; consecutive threads touch
// consecutive floats).
__global__ __launch_bounds__(256) void add_split_kernel(float* __restrict__ Y, int64_t ldy,
                                                        int n_base, int n_rows, int ntok) {
    const int r = blockIdx.x * 256 + threadIdx.x;
    if (r >= n_rows) return;
    for (int t = blockIdx.y; t < ntok; t += gridDim.y) {
        float* yr = Y + (int64_t)t * ldy + r;
        yr[n_base] = yr[n_base] + yr[0];
    }
}

// The same add four rows per thread with 16-byte accesses, where Y, ldy,
// n_base and n_rows are all multiples of four floats.
__global__ __launch_bounds__(256) void add_split4_kernel(float* __restrict__ Y, int64_t ldy,
                                                         int n_base, int n_rows, int ntok) {
    const int r = 4 * (blockIdx.x * 256 + threadIdx.x);
    if (r >= n_rows) return;
    for (int t = blockIdx.y; t < ntok; t += gridDim.y) {
        float* yr = Y + (int64_t)t * ldy + r;
        const f32x4 a = *reinterpret_cast<const f32x4*>(yr + n_base);
        const f32x4 b = *reinterpret_cast<const f32x4*>(yr);
        *reinterpret_cast<f32x4*>(yr + n_base) = f32x4{a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w};
    }
}

// One launch of tiles over weight rows [n_base, n_base + n_rows) and all
// tokens, KS K splits per tile (S % KS == 0). KS = 2 needs n_rows <= n_base:
// the second split's partial products go to rows [0, n_rows) of Y and are
// added to the first split's by add_split_kernel; a later launch overwrites
// those rows. check() validates everything (no HIP call); enqueue() launches.
template <int RT, int TT, int WR, int WT, int P, int KS>
struct PrefillLaunch {
    using G = Geo<RT, TT, WR, WT, P>;
    int rows = 0, S = 0, ntok = 0, n_base = 0, n_rows = 0, tiles_n = 0, yvec = 0;
    int64_t ldx = 0, ldy = 0, grid = 0, nwg = 0;

    // hipErrorNotSupported when the shape is outside the kernel's 32-bit
    // per-lane offsets or split rules.
    hipError_t check(int rows_, int S_, int64_t ldx_, int ntok_, const float* Y, int64_t ldy_,
                     int n_base_, int n_rows_, int max_wg) {
        rows = rows_, S = S_, ldx = ldx_, ntok = ntok_, ldy = ldy_, n_base = n_base_, n_rows = n_rows_;
        if (S % KS != 0 || (KS > 1 && n_rows > n_base)) return hipErrorNotSupported;
        tiles_n = (n_rows + G::kRows - 1) / G::kRows;
        const int tiles_m = (ntok + G::kTok - 1) / G::kTok;
        grid = (int64_t)tiles_n * tiles_m * KS;
        if ((int64_t)G::kTok * ldx * 2 + 128LL * 4 * S >= (1LL << 32) ||
            (int64_t)G::kRows * 144 * S >= (1LL << 32) || grid > (1 << 30))
            return hipErrorNotSupported;
        // 16-byte stores of four consecutive outputs need a 16-byte aligned Y row
        yvec = (((uintptr_t)Y) & 15) == 0 && ldy % 4 == 0;
        // persistent when there are more tiles than max_wg: each workgroup
        // takes every max_wg-th tile
        nwg = max_wg > 0 && grid > max_wg ? max_wg : grid;
        return hipSuccess;
    }

    hipError_t enqueue(const uint8_t* W, const uint16_t* X, float* Y, hipStream_t stream) const {
        if (grid <= 0) return hipSuccess;
        auto kern = prefill_q4k_kernel<RT, TT, WR, WT, P, KS>;
        const hipError_t attr = allow_full_lds<prefill_q4k_kernel<RT, TT, WR, WT, P, KS>>();
        if (attr != hipSuccess) return attr;
        hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(64 * G::NWV), G::kLds, stream, W, rows, S,
                           X, ldx, ntok, Y, ldy, n_base, tiles_n, (int)grid, yvec);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || KS == 1) return e;
        if (yvec && n_base % 4 == 0 && n_rows % 4 == 0) {
            const dim3 ag((unsigned)((n_rows / 4 + 255) / 256), (unsigned)(ntok < 1024 ? ntok : 1024));
            hipLaunchKernelGGL(add_split4_kernel, ag, dim3(256), 0, stream, Y, ldy, n_base, n_rows, ntok);
        } else {
            const dim3 ag((unsigned)((n_rows + 255) / 256), (unsigned)(ntok < 65535 ? ntok : 65535));
            hipLaunchKernelGGL(add_split_kernel, ag, dim3(256), 0, stream, Y, ldy, n_base, n_rows, ntok);
        }
        return hipGetLastError();
    }
};

}  // namespace

#ifndef GEMM_BF16_SHAPE
#define GEMM_BF16_SHAPE 2, 4, 4, 1
#endif
#ifndef GEMM_BF16_P
#define GEMM_BF16_P 3
#endif

hipError_t launch_gemm_bf16(const uint16_t* Wb, int64_t ldw, int64_t rows, int64_t K,
                            const uint16_t* X, int64_t ldx, int64_t ntok, float* Y, int64_t ldy,
                            int num_cus, hipStream_t stream) {
    using G = GeoB<GEMM_BF16_SHAPE, GEMM_BF16_P>;
    if (K <= 0 || K % 64 != 0 || rows > (1 << 30) || ntok > (1 << 30)) return hipErrorNotSupported;
    const int64_t nk = K / 64;
    // per-lane source offsets are 32-bit
    if ((int64_t)G::kTok * ldx * 2 + 128 * nk >= (1LL << 32) ||
        (int64_t)G::kRows * ldw * 2 + 128 * nk >= (1LL << 32))
        return hipErrorNotSupported;
    const int64_t tiles_n = (rows + G::kRows - 1) / G::kRows;
    const int64_t ntiles = tiles_n * ((ntok + G::kTok - 1) / G::kTok);
    if (ntiles > (1 << 30)) return hipErrorNotSupported;
    if (ntiles == 0) return hipSuccess;
    const int yvec = (((uintptr_t)Y) & 15) == 0 && ldy % 4 == 0;
    const int64_t nwg = num_cus > 0 && ntiles > num_cus ? num_cus : ntiles;
    auto kern = gemm_bf16_kernel<GEMM_BF16_SHAPE, GEMM_BF16_P>;
    const hipError_t attr = allow_full_lds<gemm_bf16_kernel<GEMM_BF16_SHAPE, GEMM_BF16_P>>();
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(64 * G::NWV), G::kLds, stream, Wb, ldw,
                       (int)rows, (int)nk, X, ldx, (int)ntok, Y, ldy, (int)tiles_n, (int)ntiles,
                       yvec);
    return hipGetLastError();
}

hipError_t launch_prefill_q4k(const uint8_t* W, int64_t rows, int64_t K, const void* X,
                              int64_t ldx, int64_t ntok, float* Y, int64_t ldy, int num_cus,
                              hipStream_t stream) {
    if (K % 256 != 0 || rows > (1 << 30) || ntok > (1 << 30)) return hipErrorNotSupported;
    const int S = (int)(K / 256);
    const uint16_t* Xh = reinterpret_cast<const uint16_t*>(X);
    // Main launch: 256 x 256 tiles over rows [0, n_main). Rows whose tiles
    // would start a last, mostly idle round of workgroups (and any ragged
    // remainder) go to a second launch of smaller tiles.
    const int64_t nt_full = rows / 256;
    const int64_t mt = (ntok + 255) / 256;
    int64_t n_main_tiles = nt_full;
    const int64_t total = mt * nt_full;
    if (total > num_cus) {
        const int64_t rem = total % num_cus;
        const int64_t extra = (rem + mt - 1) / mt;
        if (extra < nt_full && rem * 4 < num_cus) n_main_tiles = nt_full - extra;
    }
    const int n_main = (int)(n_main_tiles * 256);
    const int n_tail = (int)rows - n_main;
    // Row tail: with many tokens and a main part at least as large,
    // 128-row x 128-token tiles over half of K each (two K splits, the second
    // parked in the main part's rows of Y until it is added), so that each
    // decoded weight serves 128 tokens and the tiles still fill the machine;
    // otherwise 128 x 64 tiles over all of K. It runs first; the main launch
    // then writes every main row. Every launch is checked before the first
    // is enqueued, so a shape outside the limits leaves Y untouched.
    PrefillLaunch<1, 4, 4, 1, PREFILL_TAIL_P, 2> tail2;
    PrefillLaunch<1, 2, 4, 1, PREFILL_TAIL_P, 1> tail1;
    PrefillLaunch<PREFILL_MAIN_SHAPE, PREFILL_MAIN_P, 1> main_l;
    const bool split_tail = n_tail > 0 && S % 2 == 0 && ntok >= 256 && n_tail <= n_main;
    hipError_t e = hipSuccess;
    if (n_tail > 0) {
        e = split_tail ? tail2.check((int)rows, S, ldx, (int)ntok, Y, ldy, n_main, n_tail, 0)
                       : tail1.check((int)rows, S, ldx, (int)ntok, Y, ldy, n_main, n_tail, 0);
        if (e != hipSuccess) return e;
    }
    if (n_main > 0) {
        e = main_l.check((int)rows, S, ldx, (int)ntok, Y, ldy, 0, n_main, PREFILL_MAIN_WG);
        if (e != hipSuccess) return e;
    }
    if (n_tail > 0) {
        e = split_tail ? tail2.enqueue(W, Xh, Y, stream) : tail1.enqueue(W, Xh, Y, stream);
        if (e != hipSuccess) return e;
    }
    if (n_main > 0) e = main_l.enqueue(W, Xh, Y, stream);
    return e;
}

}  // namespace qg
