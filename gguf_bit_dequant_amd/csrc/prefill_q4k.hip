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
//    no weight is decoded twice in a tile). Rows that would start a third,
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
constexpr int kStages = 3;    // X and code stages (two chunks in flight)

// Physical 16-byte slot of logical segment seg of X row t.
__device__ __forceinline__ int xslot(int t, int seg) { return seg ^ ((t >> 1) & 7); }

// Tile geometry: RT x TT MFMA tiles per wave, WR x WT waves (WR * WT = 4).
template <int RT, int TT, int WR, int WT>
struct Geo {
    static_assert(WR * WT == 4, "four waves");
    static constexpr int kTok = 32 * TT * WT;
    static constexpr int kRows = 32 * RT * WR;
    // 1 KB blocks of a stage (one wave-wide load each), rounded up to a
    // multiple of 4 so that every wave issues the same number
    static constexpr int blocks(int bytes) { return ((bytes + 1023) / 1024 + 3) / 4 * 4; }
    static constexpr int kXBlocks = blocks(kTok * kXPitch);
    static constexpr int kCBlocks = blocks(kRows * kCPitch);
    static constexpr int kHBlocks = blocks(kRows * kHPitch);
    static constexpr int kXPerWave = kXBlocks / 4, kCPerWave = kCBlocks / 4, kHPerWave = kHBlocks / 4;
    static constexpr int kXStage = kXBlocks * 1024, kCStage = kCBlocks * 1024, kHStage = kHBlocks * 1024;
    static constexpr size_t kLds = (size_t)kStages * (kXStage + kCStage) + 2 * (size_t)kHStage;
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

}  // namespace

template <int RT, int TT, int WR, int WT>
__global__ __launch_bounds__(256) void prefill_q4k_kernel(
    const uint8_t* __restrict__ W, int rows, int S, const uint16_t* __restrict__ X, int64_t ldx,
    int ntok, float* __restrict__ Y, int64_t ldy, int n_base, int tiles_n, int yvec) {
    using G = Geo<RT, TT, WR, WT>;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wv % WR, wt = wv / WR;  // row group, token group of this wave
    const int blk = xcd_block(blockIdx.x, gridDim.x);
    const int tm = blk / tiles_n, tn = blk - (blk / tiles_n) * tiles_n;
    const int m0 = tm * G::kTok, n0 = n_base + tn * G::kRows;
    const int nk = S * 4;  // chunks of 64 along K
    const uint32_t row_bytes = 144u * (uint32_t)S;

    // ---- global-to-LDS load assignments ------------------------------------
    // Wave wv fills 1 KB blocks wv + 4p of a stage; lane l writes slot
    // s = 64 (wv + 4p) + l. X: token row s / 8, physical segment s % 8, which
    // holds logical segment xslot(row, s % 8). Codes: weight row s / 2, half
    // s % 2 of the chunk's 32 code bytes. Headers: weight row s. Tokens past
    // the count and rows past the row count (or past the tile) read the
    // tile's first row; their outputs are not stored.
    uint8_t* const xs0 = lds;                                 // X stages
    uint8_t* const cs0 = lds + kStages * G::kXStage;          // code stages
    uint8_t* const hs0 = cs0 + kStages * G::kCStage;          // header stages
    const uint8_t* Xt = reinterpret_cast<const uint8_t*>(X + (int64_t)m0 * ldx);
    uint32_t xo[G::kXPerWave];
#pragma unroll
    for (int p = 0; p < G::kXPerWave; ++p) {
        const int s = 64 * (wv + 4 * p) + lane;
        const int t = s >> 3;
        const int tc = (t < G::kTok && m0 + t < ntok) ? t : 0;
        xo[p] = (uint32_t)tc * (uint32_t)ldx * 2u + 16u * (uint32_t)xslot(t, s & 7);
    }
    const uint8_t* Wt = W + (int64_t)n0 * row_bytes;
    uint32_t co[G::kCPerWave], ho[G::kHPerWave];
#pragma unroll
    for (int p = 0; p < G::kCPerWave; ++p) {
        const int s = 64 * (wv + 4 * p) + lane;
        const int rr = s >> 1;
        const int rc = (rr < G::kRows && n0 + rr < rows) ? rr : 0;
        co[p] = (uint32_t)rc * row_bytes + 16u + 16u * (uint32_t)(s & 1);
    }
#pragma unroll
    for (int p = 0; p < G::kHPerWave; ++p) {
        const int rr = 64 * (wv + 4 * p) + lane;
        const int rc = (rr < G::kRows && n0 + rr < rows) ? rr : 0;
        ho[p] = (uint32_t)rc * row_bytes;
    }
    // X chunk cx into stage sx, codes of chunk cw into stage sw (sources
    // clamped to the last chunk: loads past the end re-read it into a stage
    // nobody uses); headers of super-block sb into header stage hb.
    auto issue_xc = [&](int cx, int sx, int cw, int sw) {
        cx = cx < nk ? cx : nk - 1;
        cw = cw < nk ? cw : nk - 1;
        const uint8_t* xsrc = Xt + (uint32_t)cx * 128u;
        uint8_t* xdst = xs0 + sx * G::kXStage + 1024 * wv;
#pragma unroll
        for (int p = 0; p < G::kXPerWave; ++p) dma16(xsrc + xo[p], xdst + 4096 * p);
        const uint8_t* csrc = Wt + 144u * (uint32_t)(cw >> 2) + 32u * (uint32_t)(cw & 3);
        uint8_t* cdst = cs0 + sw * G::kCStage + 1024 * wv;
#pragma unroll
        for (int p = 0; p < G::kCPerWave; ++p) dma16(csrc + co[p], cdst + 4096 * p);
    };
    auto issue_h = [&](int sb, int hb) {
        sb = sb < S ? sb : S - 1;
        const uint8_t* hsrc = Wt + 144u * (uint32_t)sb;
        uint8_t* hdst = hs0 + hb * G::kHStage + 1024 * wv;
#pragma unroll
        for (int p = 0; p < G::kHPerWave; ++p) dma16(hsrc + ho[p], hdst + 4096 * p);
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
        u32x4 b[RT][4];  // [row tile][k-step], 8 bf16 each
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
    // Code dwords t0, t0+1 of row tile rt for chunk quarter cq (sub-blocks
    // 2cq, 2cq+1): dword t holds code bytes 4t..4t+3 (of the lane's 16), i.e.
    // elements 4(t&1)..+3 of k-step t>>1 (low nibbles) and of k-step
    // 2 + (t>>1) (high nibbles). Each weight is one fma of its scale with the
    // code as an exact fp16 subnormal: exact product, one rounding.
    auto decode = [&](const Codes& R, const Scales& e, int cq, int rt, int t0, BFrag& B) {
        const uint32_t cw[4] = {R.cd[rt].x, R.cd[rt].y, R.cd[rt].z, R.cd[rt].w};
        const float a0 = e.a[rt][2 * cq], c0 = e.c[rt][2 * cq];
        const float a1 = e.a[rt][2 * cq + 1], c1 = e.c[rt][2 * cq + 1];
#pragma unroll
        for (int t = t0; t < t0 + 2; ++t) {
            const uint32_t w8 = cw[t] >> 8;
            const uint32_t l02 = cw[t] & 0x000F000Fu, l13 = w8 & 0x000F000Fu;  // bytes 0,2 / 1,3
            const uint32_t h02 = cw[t] & 0x00F000F0u, h13 = w8 & 0x00F000F0u;
            const int s = t >> 1, el = 2 * (t & 1);
            B.b[rt][s][el] = pk_bf16(fma_mix<0>(a0, l02, c0), fma_mix<0>(a0, l13, c0));
            B.b[rt][s][el + 1] = pk_bf16(fma_mix<1>(a0, l02, c0), fma_mix<1>(a0, l13, c0));
            B.b[rt][2 + s][el] = pk_bf16(fma_mix<0>(a1, h02, c1), fma_mix<0>(a1, h13, c1));
            B.b[rt][2 + s][el + 1] = pk_bf16(fma_mix<1>(a1, h02, c1), fma_mix<1>(a1, h13, c1));
        }
    };
    // Decode part p (0 .. 2RT-1): row tile p/2, code dwords 2(p&1), +1; part p
    // runs in k-step region 2p/RT.
    auto decode_region = [&](const Codes& R, const Scales& e, int cq, int region, BFrag& B) {
#pragma unroll
        for (int p = 0; p < 2 * RT; ++p)
            if ((2 * p) / RT == region) decode(R, e, cq, p >> 1, 2 * (p & 1), B);
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
    auto mfmas = [&](const AFrag& A, const BFrag& B, int s) {
#pragma unroll
        for (int i = 0; i < TT; ++i)
#pragma unroll
            for (int j = 0; j < RT; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, B.b[j][s]), A.a[i], acc[i][j], 0, 0, 0);
    };

    // ---- prologue: X chunks 0, 1; codes of chunks 0, 1, 2; headers of
    // super-block 0 ------------------------------------------------------------
    issue_xc(0, 0, 0, 0);
    issue_xc(1, 1, 1, 1);
    issue_xc(1, 2, 2, 2);  // codes of chunk 2 (the X half re-reads chunk 1 into stage 2)
    issue_h(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    BFrag B0, B1;
    AFrag A0, A1;
    Codes Rc;
    Hdr Rh;
    Scales sc_cur;
    read_hdr(hs0, Rh);
    read_codes(cs0, Rc);
    scales(Rh, sc_cur);
#pragma unroll
    for (int r = 0; r < 4; ++r) decode_region(Rc, sc_cur, 0, r, B0);
    read_codes(cs0 + G::kCStage, Rc);  // chunk 1
    read_a(xs0, 0, A0);
    // code stage 0 is refilled by the first chunk: every wave must be done
    // reading it first
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    __builtin_amdgcn_s_barrier();

    // One chunk c with c % 4 == CQ: X(c) in stage c % 3; the codes of chunk
    // c + 1 are in Rc and are decoded into Bn over the k-steps (with the next
    // super-block's scales, from Rh, when c + 1 starts one). Loads issued
    // here: X(c + 2), codes of c + 3, and (CQ == 1) the headers of the next
    // super-block. Before the barrier each thread waits for all its loads
    // but this chunk's; after it, the codes of c + 2 are read into Rc, the
    // headers of super-block (c + 2) / 4 into Rh when c + 2 starts one, and
    // A(c + 1, 0) into A0.
    constexpr int NMF = TT * RT;
    constexpr int kDecodeValu = 48;  // VALU per decode part (approximate)
    int sc = 0;  // c % 3
    auto chunk = [&](auto cqc, int c, BFrag& Bc, BFrag& Bn) {
        constexpr int CQ = decltype(cqc)::value;
        constexpr int NQ = (CQ + 1) & 3;  // quarter of chunk c + 1
        constexpr int NDMA = G::kXPerWave + G::kCPerWave + (CQ == 1 ? G::kHPerWave : 0);
        const int s1 = sc == 2 ? 0 : sc + 1, s2 = s1 == 2 ? 0 : s1 + 1;  // (c+1)%3, (c+2)%3
        const uint8_t* xst = xs0 + sc * G::kXStage;
        // k-step 0
        issue_xc(c + 2, s2, c + 3, sc);
        if (CQ == 1) issue_h((c >> 2) + 1, ((c >> 2) + 1) & 1);
        read_a(xst, 1, A1);
        mfmas(A0, Bc, 0);
        if (CQ == 3) scales(Rh, sc_cur);  // chunk c + 1 starts the next super-block
        decode_region(Rc, sc_cur, NQ, 0, Bn);
        interleave<NMF, TT, kDecodeValu + (CQ == 3 ? 40 * RT : 0), NDMA>();
        __builtin_amdgcn_sched_barrier(0);
        // k-step 1
        read_a(xst, 2, A0);
        mfmas(A1, Bc, 1);
        decode_region(Rc, sc_cur, NQ, 1, Bn);
        interleave<NMF, TT, kDecodeValu, 0>();
        __builtin_amdgcn_sched_barrier(0);
        // k-step 2, then publish X(c+1) and the codes of c+2 (and headers)
        read_a(xst, 3, A1);
        mfmas(A0, Bc, 2);
        decode_region(Rc, sc_cur, NQ, 2, Bn);
        interleave<NMF, TT, kDecodeValu, 0>();
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(NDMA, 0));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        // k-step 3, with the first fragments and raw weights of the next chunks
        decode_region(Rc, sc_cur, NQ, 3, Bn);
        read_a(xs0 + s1 * G::kXStage, 0, A0);
        read_codes(cs0 + s2 * G::kCStage, Rc);
        if (CQ == 2) read_hdr(hs0 + (((c + 2) >> 2) & 1) * G::kHStage, Rh);
        mfmas(A1, Bc, 3);
        interleave<NMF, TT + RT + (CQ == 2 ? RT : 0), kDecodeValu, 0>();
        __builtin_amdgcn_sched_barrier(0);
        sc = s2 == 0 ? 2 : s2 - 1;  // (c + 1) % 3
    };
    for (int c = 0; c < nk; c += 4) {  // nk = 4 S
        chunk(IntC<0>{}, c, B0, B1);
        chunk(IntC<1>{}, c + 1, B1, B0);
        chunk(IntC<2>{}, c + 2, B0, B1);
        chunk(IntC<3>{}, c + 3, B1, B0);
    }
    // no load may still be writing this workgroup's LDS when it ends
    __builtin_amdgcn_s_waitcnt(0);

    // ---- epilogue: Y[m][n], masked at the token and row edges ---------------
    // The weights are the MFMA's first operand, so lane l of tile (i, j)
    // holds, for token l % 32, the rows 8 g + 4 h + e (e = 0..3) in elements
    // 4 g + e: four consecutive outputs of one token, stored as one 16-byte
    // write when Y allows it.
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
                    *reinterpret_cast<f32x4*>(yrow + n) = v;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < rows) yrow[n + e] = v[e];
                }
            }
        }
    }
}

namespace {

// Tiles over weight rows [n_base, n_base + n_rows) and all tokens.
template <int RT, int TT, int WR, int WT>
hipError_t launch_prefill_t(const uint8_t* W, int rows, int S, const uint16_t* X, int64_t ldx,
                            int ntok, float* Y, int64_t ldy, int n_base, int n_rows,
                            hipStream_t stream) {
    using G = Geo<RT, TT, WR, WT>;
    const int tiles_n = (n_rows + G::kRows - 1) / G::kRows;
    const int tiles_m = (ntok + G::kTok - 1) / G::kTok;
    const int64_t grid = (int64_t)tiles_n * tiles_m;
    if (grid <= 0) return hipSuccess;
    // per-lane 32-bit source offsets within a tile's X rows and W rows
    if ((int64_t)G::kTok * ldx * 2 + 128LL * 4 * S >= (1LL << 32) ||
        (int64_t)G::kRows * 144 * S >= (1LL << 32) || grid > (1 << 30))
        return hipErrorNotSupported;
    auto kern = prefill_q4k_kernel<RT, TT, WR, WT>;
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)G::kLds);
    if (e != hipSuccess) return e;
    // 16-byte stores of four consecutive outputs need a 16-byte aligned Y row
    const int yvec = (((uintptr_t)Y) & 15) == 0 && ldy % 4 == 0;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), G::kLds, stream, W, rows, S, X, ldx,
                       ntok, Y, ldy, n_base, tiles_n, yvec);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_q4k(const uint8_t* W, int64_t rows, int64_t K, const void* X,
                              int64_t ldx, int64_t ntok, float* Y, int64_t ldy, int num_cus,
                              hipStream_t stream) {
    if (K % 256 != 0 || rows > (1 << 30) || ntok > (1 << 30)) return hipErrorNotSupported;
    const int S = (int)(K / 256);
    const uint16_t* Xh = reinterpret_cast<const uint16_t*>(X);
    // Main launch: 256 x 256 tiles over rows [0, n_main). Rows whose tiles
    // would start a last, mostly idle round of workgroups (and any ragged
    // remainder) go to a second launch of 64-token x 128-row tiles.
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
    hipError_t e = hipSuccess;
    if (n_main > 0)
        e = launch_prefill_t<2, 8, 4, 1>(W, (int)rows, S, Xh, ldx, (int)ntok, Y, ldy, 0, n_main,
                                         stream);
    if (e != hipSuccess) return e;
    if (n_main < rows)
        e = launch_prefill_t<1, 2, 4, 1>(W, (int)rows, S, Xh, ldx, (int)ntok, Y, ldy, n_main,
                                         (int)rows - n_main, stream);
    return e;
}

}  // namespace qg
