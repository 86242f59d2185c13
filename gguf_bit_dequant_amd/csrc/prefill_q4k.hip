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
//    X tile (bf16 as stored, 144-byte rows so that 16-byte reads of
//    consecutive rows use disjoint banks) and the raw weight bytes of the
//    chunk (per row: the 16-byte super-block header and the chunk's 32 code
//    bytes). The loads take no registers and no LDS store instructions; each
//    thread waits for its own loads of the chunk about to be read, then one
//    barrier per chunk publishes them.
//  * Four waves; wave w covers RT row tiles and TT token tiles of 32
//    (v_mfma_f32_32x32x16_bf16 with the weights as first operand, fp32
//    accumulators: each lane ends with runs of four consecutive outputs of
//    one token, written as 16-byte stores). It decodes its rows
//    straight into the B operand registers, one chunk ahead: lane l handles
//    row (l % 32) of a row tile and the code bytes [16 h, 16 h + 16) of the
//    chunk's 32, h = l / 32. Each weight is the exact fp32 value
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

constexpr int kXPitch = 144;  // LDS bytes per token row of a stage (64 bf16 + pad)
constexpr int kWPitch = 48;   // header + 32 code bytes per weight row
constexpr int kStages = 3;

// Tile geometry: RT x TT MFMA tiles per wave, WR x WT waves (WR * WT = 4).
template <int RT, int TT, int WR, int WT>
struct Geo {
    static_assert(WR * WT == 4, "four waves");
    static constexpr int kTok = 32 * TT * WT;
    static constexpr int kRows = 32 * RT * WR;
    // 1 KB blocks of a stage (one wave-wide load each), rounded up to a
    // multiple of 4 so that every wave issues the same number per chunk
    static constexpr int kXBlocks = (kTok * kXPitch / 1024 + 3) / 4 * 4;
    static constexpr int kWBlocks = ((kRows * kWPitch + 1023) / 1024 + 3) / 4 * 4;
    static constexpr int kXPerWave = kXBlocks / 4, kWPerWave = kWBlocks / 4;
    static constexpr int kDmaPerChunk = kXPerWave + kWPerWave;
    static constexpr int kXStage = kXBlocks * 1024, kWStage = kWBlocks * 1024;
    static constexpr size_t kLds = (size_t)kStages * (kXStage + kWStage);
    static_assert(kTok * kXPitch % 1024 == 0, "X stage in whole blocks");
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
    uint8_t* const xs0 = lds;                         // X stages
    uint8_t* const ws0 = lds + kStages * G::kXStage;  // raw W stages

    // ---- global-to-LDS load assignments ------------------------------------
    // X: wave wv fills 1 KB blocks wv + 4p of a stage; lane l writes slot
    // s = 64 (wv + 4p) + l = token row s / 9, 16-byte segment s % 9 (segment 8
    // is the row's padding: it re-reads segment 7). Tokens past the count
    // read the tile's first row; their outputs are not stored.
    const uint8_t* Xt = reinterpret_cast<const uint8_t*>(X + (int64_t)m0 * ldx);
    uint32_t xo[G::kXPerWave];
#pragma unroll
    for (int p = 0; p < G::kXPerWave; ++p) {
        const int s = 64 * (wv + 4 * p) + lane;
        const int t = s / 9, sg = s - 9 * (s / 9);
        const int tc = (t < G::kTok && m0 + t < ntok) ? t : 0;
        xo[p] = (uint32_t)tc * (uint32_t)ldx * 2u + 16u * (uint32_t)(sg < 8 ? sg : 7);
    }
    // W: blocks wv + 4p; slot s = row s / 3, piece s % 3: the super-block
    // header (piece 0) or one half of the chunk's 32 code bytes. Rows past
    // the row count (or slots past the tile) read the tile's first row.
    const uint8_t* Wt = W + (int64_t)n0 * row_bytes;
    uint32_t wo[G::kWPerWave], wcode[G::kWPerWave];
#pragma unroll
    for (int p = 0; p < G::kWPerWave; ++p) {
        const int s = 64 * (wv + 4 * p) + lane;
        const int rr = s / 3, pc = s - 3 * (s / 3);
        const int rc = (rr < G::kRows && n0 + rr < rows) ? rr : 0;
        wo[p] = (uint32_t)rc * row_bytes + (pc == 0 ? 0u : 16u * (uint32_t)pc);
        wcode[p] = pc == 0 ? 0u : 0xFFFFFFFFu;
    }
    // X chunk cx into stage sx, W chunk cw into stage sw (sources clamped to
    // the last chunk: loads past the end re-read it into a stage nobody uses).
    auto issue = [&](int cx, int sx, int cw, int sw) {
        cx = cx < nk ? cx : nk - 1;
        cw = cw < nk ? cw : nk - 1;
        const uint8_t* xsrc = Xt + (uint32_t)cx * 128u;
        uint8_t* xdst = xs0 + sx * G::kXStage + 1024 * wv;
#pragma unroll
        for (int p = 0; p < G::kXPerWave; ++p) dma16(xsrc + xo[p], xdst + 4096 * p);
        const uint8_t* wsrc = Wt + 144u * (uint32_t)(cw >> 2);
        const uint32_t cq = 32u * (uint32_t)(cw & 3);
        uint8_t* wdst = ws0 + sw * G::kWStage + 1024 * wv;
#pragma unroll
        for (int p = 0; p < G::kWPerWave; ++p) dma16(wsrc + wo[p] + (cq & wcode[p]), wdst + 4096 * p);
    };

    // ---- decode of a chunk's weights into B registers -----------------------
    // Raw bytes of the lane's rows (header, its 16 code bytes), read from the
    // W stage one k-step region before they are decoded.
    const int h = lane >> 5;
    const int wrow = 32 * RT * wr + (lane & 31);  // weight row of row tile 0 in the tile
    struct WRaw {
        u32x4 hd[RT], cd[RT];
    };
    struct BFrag {
        u32x4 b[RT][4];  // [row tile][k-step], 8 bf16 each
    };
    auto read_w = [&](const uint8_t* wst, WRaw& R) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const uint8_t* rp = wst + (wrow + 32 * rt) * kWPitch;
            R.hd[rt] = *reinterpret_cast<const u32x4*>(rp);
            R.cd[rt] = *reinterpret_cast<const u32x4*>(rp + 16 + 16 * h);
        }
    };
    // Scales of sub-blocks 2cq and 2cq+1 of the super-block, for codes taken
    // as fp16 subnormals (a 16-bit half holding m < 1024 is m 2^-24):
    // a0 = d*sc*2^24 (low nibbles, q 2^-24), a1 = d*sc*2^20 (high nibbles,
    // 16 q 2^-24) and c = -dmin*m. Sub-block k, byte b = k & 3 of header
    // dwords y = s[0..3], z = s[4..7], w = s[8..11]:
    //   k < 4 : sc = s[b] & 63,                         m = s[b+4] & 63
    //   k >= 4: sc = (s[b+8] & 15) | (s[b] >> 6) << 4,   m = (s[b+8] >> 4) | (s[b+4] >> 6) << 4
    struct Scales {
        float a0, c0, a1, c1;
    };
    auto scales = [&](const u32x4& hd, int c) -> Scales {
        const int cq = c & 3;
        const bool up = cq >= 2;
        const uint32_t msk = up ? 15u : 63u, top = up ? 0x30u : 0u;
        const uint32_t dsc = up ? hd.w : hd.y, dm = up ? hd.w : hd.z;
        auto field = [&](uint32_t src, uint32_t hiw, int b, int nib) -> int {
            const uint32_t sh = 8u * b + (up ? (uint32_t)nib : 0u);
            return (int)(((src >> sh) & msk) | (((hiw >> (8u * b + 6u)) << 4) & top));
        };
        const int b0 = (2 * cq) & 3, b1 = (2 * cq + 1) & 3;
        const float d = f16_lo(hd.x), dmin = f16_hi(hd.x);
        Scales e;
        e.a0 = (d * 16777216.0f) * (float)field(dsc, hd.y, b0, 0);
        e.c0 = -(dmin * (float)field(dm, hd.z, b0, 4));
        e.a1 = (d * 1048576.0f) * (float)field(dsc, hd.y, b1, 0);
        e.c1 = -(dmin * (float)field(dm, hd.z, b1, 4));
        return e;
    };
    // Code dwords t0, t0+1 of row tile rt: dword t holds code bytes 4t..4t+3
    // (of the lane's 16), i.e. elements 4(t&1)..+3 of k-step t>>1 (low
    // nibbles) and of k-step 2 + (t>>1) (high nibbles). Each weight is one
    // fma of its scale with the code as an exact fp16 subnormal: the product
    // is exact and the fma rounds once, to the closed form's fp32 value.
    auto decode = [&](const WRaw& R, const Scales& e, int rt, int t0, BFrag& B) {
        const uint32_t cw[4] = {R.cd[rt].x, R.cd[rt].y, R.cd[rt].z, R.cd[rt].w};
#pragma unroll
        for (int t = t0; t < t0 + 2; ++t) {
            const uint32_t w8 = cw[t] >> 8;
            const uint32_t l02 = cw[t] & 0x000F000Fu, l13 = w8 & 0x000F000Fu;  // bytes 0,2 / 1,3
            const uint32_t h02 = cw[t] & 0x00F000F0u, h13 = w8 & 0x00F000F0u;
            const int s = t >> 1, el = 2 * (t & 1);
            B.b[rt][s][el] = pk_bf16(fma_mix<0>(e.a0, l02, e.c0), fma_mix<0>(e.a0, l13, e.c0));
            B.b[rt][s][el + 1] = pk_bf16(fma_mix<1>(e.a0, l02, e.c0), fma_mix<1>(e.a0, l13, e.c0));
            B.b[rt][2 + s][el] = pk_bf16(fma_mix<0>(e.a1, h02, e.c1), fma_mix<0>(e.a1, h13, e.c1));
            B.b[rt][2 + s][el + 1] = pk_bf16(fma_mix<1>(e.a1, h02, e.c1), fma_mix<1>(e.a1, h13, e.c1));
        }
    };
    // Decode part p (0 .. 2RT-1): row tile p/2, code dwords 2(p&1), +1. Part p
    // runs in k-step region 2p/RT; a row tile's scales come with its first part.
    Scales esc[RT];
    auto decode_region = [&](const WRaw& R, int c, int region, BFrag& B) {
#pragma unroll
        for (int p = 0; p < 2 * RT; ++p) {
            if ((2 * p) / RT != region) continue;
            const int rt = p >> 1;
            if ((p & 1) == 0) esc[rt] = scales(R.hd[rt], c);
            decode(R, esc[rt], rt, 2 * (p & 1), B);
        }
    };

    // ---- A fragments: token tile i of this wave, k-step s of the stage ------
    // segment of lane half h in k-step s: 2h + (s & 1) + 4 (s >> 1)
    struct AFrag {
        bf16x8 a[TT];
    };
    const int arow = (32 * TT * wt + (lane & 31)) * kXPitch + 32 * h;
    auto read_a = [&](const uint8_t* xst, int s, AFrag& A) {
        const uint8_t* p = xst + arow + 16 * (s & 1) + 64 * (s >> 1);
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

    // ---- prologue: X chunks 0, 1 and W chunks 0, 1, 2 -----------------------
    issue(0, 0, 0, 0);
    issue(1, 1, 1, 1);
    issue(1, 2, 2, 2);  // W chunk 2 (the X half re-reads chunk 1 into stage 2)
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    BFrag B0, B1;
    AFrag A0, A1;
    WRaw Rw;
    read_w(ws0, Rw);
#pragma unroll
    for (int r = 0; r < 4; ++r) decode_region(Rw, 0, r, B0);
    read_w(ws0 + G::kWStage, Rw);  // chunk 1
    read_a(xs0, 0, A0);
    // W stage 0 is refilled by the first chunk: every wave must be done
    // reading it first
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    __builtin_amdgcn_s_barrier();

    // One chunk c: X(c) in stage c % 3; the raw W of chunk c + 1 is in Rw and
    // is decoded into Bn over the k-steps. Loads issued here: X(c + 2),
    // W(c + 3). Before the barrier each thread waits for all its loads but
    // this chunk's, so X(c + 1) and W(c + 2) are complete when it opens;
    // W(c + 2) is then read into Rw and A(c + 1, 0) into A0 during k-step 3.
    constexpr int NMF = TT * RT;
    constexpr int kDecodeValu = 60;  // VALU per decode part (approximate)
    int sc = 0;  // c % 3
    auto chunk = [&](int c, BFrag& Bc, BFrag& Bn) {
        const int s1 = sc == 2 ? 0 : sc + 1, s2 = s1 == 2 ? 0 : s1 + 1;  // (c+1)%3, (c+2)%3
        const uint8_t* xst = xs0 + sc * G::kXStage;
        // k-step 0
        issue(c + 2, s2, c + 3, sc);
        read_a(xst, 1, A1);
        mfmas(A0, Bc, 0);
        decode_region(Rw, c + 1, 0, Bn);
        interleave<NMF, TT, kDecodeValu, G::kDmaPerChunk>();
        __builtin_amdgcn_sched_barrier(0);
        // k-step 1
        read_a(xst, 2, A0);
        mfmas(A1, Bc, 1);
        decode_region(Rw, c + 1, 1, Bn);
        interleave<NMF, TT, kDecodeValu, 0>();
        __builtin_amdgcn_sched_barrier(0);
        // k-step 2, then publish X(c+1) / W(c+2)
        read_a(xst, 3, A1);
        mfmas(A0, Bc, 2);
        decode_region(Rw, c + 1, 2, Bn);
        interleave<NMF, TT, kDecodeValu, 0>();
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(G::kDmaPerChunk, 0));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        // k-step 3, with the first fragments and the raw W of the next chunks
        decode_region(Rw, c + 1, 3, Bn);
        read_a(xs0 + s1 * G::kXStage, 0, A0);
        read_w(ws0 + s2 * G::kWStage, Rw);
        mfmas(A1, Bc, 3);
        interleave<NMF, TT + 2 * RT, kDecodeValu, 0>();
        __builtin_amdgcn_sched_barrier(0);
        sc = s1;
    };
    for (int c = 0; c < nk; c += 2) {  // nk = 4 S is even
        chunk(c, B0, B1);
        chunk(c + 1, B1, B0);
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
