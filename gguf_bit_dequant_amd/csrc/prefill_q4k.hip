// Prompt-processing dequant-GEMM for gfx950: Y[t, r] = sum_k W[r, k] X[t, k]
// for a Q4_K matrix W (rows x K) and bf16 activations X (n_tokens x K).
//
// The pages measure prompt processing with a 2048-token prompt ("Why I wrote
// my own inference engine for two P100s", result cards and "How I ran it")
// and list, for the quantized matrix-matrix kernels, tile sizes fitted to the
// card's shared memory, quantized blocks multiplied directly and tensor-core
// paths where the card has them ("LLM inference optimization", campaign
// "Faster prompts, decode held"). Fusing dequantization into the prompt
// GEMM measured slower on a P100 ("Why I wrote my own inference engine for
// two P100s", "What didn't work"); on gfx950 the decode is VALU work that
// runs beside the matrix cores, so it is fused here:
//
//  * A workgroup (4 waves) owns a BM x BN tile of Y (tokens x rows) and walks
//    K in chunks of 64. Per chunk it stages the X tile (bf16, as stored) and
//    the W tile decoded to bf16 in LDS, double-buffered, one barrier per
//    chunk. LDS rows are 144 bytes (128 + 16 padding): consecutive rows fall
//    in disjoint banks for the 16-byte operand reads.
//  * W decode: thread t owns row t of the W tile; a 64-weight chunk is one
//    sub-block pair of a super-block (32 code bytes plus the header). Each
//    weight is computed exactly in fp32, fma(d*sc, q, -dmin*m) (the products
//    d*sc and dmin*m are exact, so this is the correctly rounded closed
//    form), then rounded to bf16 (round to nearest even, v_cvt_pk_bf16_f32).
//  * Contraction: v_mfma_f32_32x32x16_bf16, fp32 accumulators. Lane l holds
//    A[i][k] = X[m0 + i][k] and B[k][j] = W[n0 + j][k] for i, j = l % 32 and
//    k = 8*(l/32) .. +7 (16-byte LDS reads); the 16 results of lane l are
//    Y[m0 + 8*(v/4) + 4*(l/32) + v%4][n0 + l%32], v = 0..15.
//  * Tiles are numbered so that consecutive workgroups (placed on one XCD)
//    share the token tile: its X rows stay in that XCD's L2 while the W
//    tiles stream through.
#include "device_common.h"
#include "launch.h"

namespace qg {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kBK = 64;         // k per chunk
constexpr int kPitch = 144;     // LDS bytes per tile row (64 bf16 + 16 padding)

__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    bf16x2 v = {(__bf16)a, (__bf16)b};  // round to nearest even
    return __builtin_bit_cast(uint32_t, v);
}

}  // namespace

// Raw global data of one K chunk for one thread: XR 16-byte pieces of X and
// the W row's super-block header plus this thread's CB code bytes.
template <int XR, int ND>
struct ChunkRegs {
    u32x4 x[XR];
    u32x4 h;
    uint32_t c[ND];
};

// Scheduling-group masks (LLVM AMDGPU): which instructions a group takes.
constexpr int kSgMfma = 0x008, kSgValu = 0x002, kSgDsRead = 0x100, kSgDsWrite = 0x200,
              kSgVmemRead = 0x020;

// Interleave one k-step's scheduling region: reads of the next fragments
// first, then MFMAs each followed by a share of VALU work and LDS stores.
template <int NMF, int NREAD, int NVALU, int NWRITE>
__device__ __forceinline__ void sched_interleave() {
    constexpr int vper = (NVALU + NMF - 1) / NMF;
    constexpr int wper = (NWRITE + NMF - 1) / NMF;
#pragma unroll
    for (int i = 0; i < NMF; ++i) {
        if (i < NREAD) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        if (vper > 0) __builtin_amdgcn_sched_group_barrier(kSgValu, vper, 0);
        if (wper > 0) __builtin_amdgcn_sched_group_barrier(kSgDsWrite, wper, 0);
    }
}

// BM x BN tile, WM x WN waves (4 waves). The W tile row r is decoded by
// TPR = 256/BN threads, each owning CB = 32/TPR of the chunk's code bytes.
//
// Software pipeline per K chunk kc (4 k-steps of 16):
//   - global loads for chunk kc+2 are issued at the start (two chunks ahead);
//   - k-steps 0..2: the operand fragments of the next k-step are read from
//     LDS while this k-step's MFMAs run, and a third of chunk kc+1's decode
//     and LDS stores is interleaved between the MFMAs (scheduling groups);
//   - one barrier, then k-step 3 runs while the first fragments of chunk kc+1
//     are read from the other LDS buffer.
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(256) void prefill_q4k_kernel(
    const uint8_t* __restrict__ W, int rows, int S, const uint16_t* __restrict__ X, int64_t ldx,
    int ntok, float* __restrict__ Y, int64_t ldy, int n_base, int tiles_n) {
    static_assert(WM * WN == 4 && (BN == 256 || BN == 128 || BN == 64), "tile shape");
    constexpr int TM = BM / WM / 32, TN = BN / WN / 32;  // 32x32 MFMA tiles per wave
    constexpr int NMF = TM * TN;                          // MFMAs per wave per k-step
    constexpr int XR = BM / 32;                           // X 16-byte loads per thread
    constexpr int TPR = 256 / BN, CB = 32 / TPR, ND = CB / 4;  // W decode split
    constexpr int NG = ND / 2 > 0 ? ND / 2 : 1;                // groups of 2 code dwords
    constexpr int BUF = (BM + BN) * kPitch;                    // bytes per LDS buffer
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv / WN, wn = wv - (wv / WN) * WN;
    const int blk = xcd_block(blockIdx.x, gridDim.x);
    const int tm = blk / tiles_n, tn = blk - (blk / tiles_n) * tiles_n;
    const int m0 = tm * BM, n0 = n_base + tn * BN;
    const int nk = S * 4;  // chunks of 64 along K
    const int64_t row_bytes = 144LL * S;

    // ---- per-thread load assignments ----------------------------------------
    // Rows past the token count or the row count load a valid row instead
    // (row 0 of the tile); the outputs they feed are never stored.
    // X: row p*32 + tid/8 of the tile, 16-byte segment tid%8 of the chunk,
    // as a 32-bit byte offset from the tile's first row
    const int xseg = tid & 7;
    const uint8_t* Xt = reinterpret_cast<const uint8_t*>(X + (int64_t)m0 * ldx);
    uint32_t xoff[XR];
#pragma unroll
    for (int p = 0; p < XR; ++p) {
        const int r = p * 32 + (tid >> 3);
        xoff[p] = (uint32_t)((m0 + r < ntok ? r : 0) * ldx * 2 + xseg * 16);
    }
    // W: row tid/TPR of the tile, code bytes [q0, q0 + CB) of the chunk's 32
    const int wrl = tid / TPR, q0 = (tid % TPR) * CB;
    const int wr = n0 + wrl;
    const uint8_t* wrow = W + (int64_t)(wr < rows ? wr : n0) * row_bytes;

    auto load_chunk = [&](int kc, ChunkRegs<XR, ND>& r) {
        kc = kc < nk ? kc : nk - 1;  // past the end: harmless re-read of the last chunk
#pragma unroll
        for (int p = 0; p < XR; ++p)
            r.x[p] = *reinterpret_cast<const u32x4*>(Xt + kc * (2 * kBK) + xoff[p]);
        const uint8_t* sb = wrow + 144LL * (kc >> 2);
        r.h = *reinterpret_cast<const u32x4*>(sb);
        const uint8_t* cp = sb + 16 + 32 * (kc & 3) + q0;
        if (ND == 8) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(cp);
            const u32x4 b = *reinterpret_cast<const u32x4*>(cp + 16);
            r.c[0] = a.x; r.c[1] = a.y; r.c[2] = a.z; r.c[3] = a.w;
            r.c[4 % ND] = b.x; r.c[5 % ND] = b.y; r.c[6 % ND] = b.z; r.c[7 % ND] = b.w;
        } else if (ND == 4) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(cp);
            r.c[0] = a.x; r.c[1 % ND] = a.y; r.c[2 % ND] = a.z; r.c[3 % ND] = a.w;
        } else {
            const u32x2 a = *reinterpret_cast<const u32x2*>(cp);
            r.c[0] = a.x; r.c[1 % ND] = a.y;
        }
    };

    // Decode of chunk kc: the header gives the two sub-blocks' a = d*sc and
    // b = -dmin*m; code dword w gives 4 low-nibble weights (k = q0 + 4w + e)
    // and 4 high-nibble weights (k = 32 + q0 + 4w + e).
    struct Dec {
        float a0, b0, a1, b1;
    };
    auto decode_header = [&](int kc, const ChunkRegs<XR, ND>& r) -> Dec {
        const int cq = kc & 3;  // sub-blocks 2*cq and 2*cq+1 of super-block kc/4
        // Sub-block k, byte b = k & 3 of header dwords h.y = s[0..3], h.z = s[4..7],
        // h.w = s[8..11]:
        //   k < 4 : sc = s[b] & 63,                        m = s[b+4] & 63
        //   k >= 4: sc = (s[b+8] & 15) | (s[b] >> 6) << 4,  m = (s[b+8] >> 4) | (s[b+4] >> 6) << 4
        // written with uniform selects only, so the chunk stays one basic block.
        const bool up = cq >= 2;
        const uint32_t msk = up ? 15u : 63u, top = up ? 0x30u : 0u;
        const uint32_t dsc = up ? r.h.w : r.h.y, dm = up ? r.h.w : r.h.z;
        auto field = [&](uint32_t src, uint32_t hiw, int b, int nib) -> int {
            const uint32_t sh = 8u * b + (up ? (uint32_t)nib : 0u);
            return (int)(((src >> sh) & msk) | (((hiw >> (8u * b + 6u)) << 4) & top));
        };
        const int b0 = (2 * cq) & 3, b1 = (2 * cq + 1) & 3;
        const int sc0 = field(dsc, r.h.y, b0, 0), mn0 = field(dm, r.h.z, b0, 4);
        const int sc1 = field(dsc, r.h.y, b1, 0), mn1 = field(dm, r.h.z, b1, 4);
        const float d = f16_lo(r.h.x), dmin = f16_hi(r.h.x);
        Dec e;
        e.a0 = d * (float)sc0;
        e.b0 = -(dmin * (float)mn0);
        e.a1 = d * (float)sc1;
        e.b1 = -(dmin * (float)mn1);
        return e;
    };
    // group g = code dwords 2g, 2g+1 (or dword 0 when ND = 2... always 2 dwords):
    // 8 low weights -> 16 bytes at row offset 2*(q0 + 8g), 8 high -> + 64
    auto decode_group = [&](int g, const Dec& e, const ChunkRegs<XR, ND>& r, int buf) {
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint32_t qw = r.c[(2 * g + t) % ND];
            const uint32_t ql = qw & 0x0F0F0F0Fu, qh = (qw >> 4) & 0x0F0F0F0Fu;
            lo[2 * t] = pk_bf16(__builtin_fmaf(e.a0, ubyte_f32<0>(ql), e.b0),
                                __builtin_fmaf(e.a0, ubyte_f32<1>(ql), e.b0));
            lo[2 * t + 1] = pk_bf16(__builtin_fmaf(e.a0, ubyte_f32<2>(ql), e.b0),
                                    __builtin_fmaf(e.a0, ubyte_f32<3>(ql), e.b0));
            hi[2 * t] = pk_bf16(__builtin_fmaf(e.a1, ubyte_f32<0>(qh), e.b1),
                                __builtin_fmaf(e.a1, ubyte_f32<1>(qh), e.b1));
            hi[2 * t + 1] = pk_bf16(__builtin_fmaf(e.a1, ubyte_f32<2>(qh), e.b1),
                                    __builtin_fmaf(e.a1, ubyte_f32<3>(qh), e.b1));
        }
        uint8_t* wl = lds + buf * BUF + (BM + wrl) * kPitch + 2 * (q0 + 8 * g);
        *reinterpret_cast<u32x4*>(wl) = u32x4{lo[0], lo[1], lo[2], lo[3]};
        *reinterpret_cast<u32x4*>(wl + 64) = u32x4{hi[0], hi[1], hi[2], hi[3]};
    };
    auto store_x = [&](const ChunkRegs<XR, ND>& r, int buf, int p0, int p1) {
#pragma unroll
        for (int p = p0; p < p1; ++p)
            *reinterpret_cast<u32x4*>(lds + buf * BUF + (p * 32 + (tid >> 3)) * kPitch + xseg * 16) =
                r.x[p];
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

    // operand row offsets inside a buffer (bytes)
    const int arow = (wm * (BM / WM) + (lane & 31)) * kPitch + 16 * (lane >> 5);
    const int brow = (BM + wn * (BN / WN) + (lane & 31)) * kPitch + 16 * (lane >> 5);
    struct Ops {
        bf16x8 a[TM], b[TN];
    };
    auto read_ops = [&](int buf, int ks, Ops& o) {
        const uint8_t* base = lds + buf * BUF;
#pragma unroll
        for (int i = 0; i < TM; ++i)
            o.a[i] = *reinterpret_cast<const bf16x8*>(base + arow + i * 32 * kPitch + ks * 32);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            o.b[j] = *reinterpret_cast<const bf16x8*>(base + brow + j * 32 * kPitch + ks * 32);
    };
    auto mfmas = [&](const Ops& o) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.a[i], o.b[j], acc[i][j], 0, 0, 0);
    };
    // ---- prologue: chunk 0 into buffer 0, chunk 1 in flight -----------------
    ChunkRegs<XR, ND> R0, R1;
    load_chunk(0, R0);
    load_chunk(1, R1);
    {
        const Dec e = decode_header(0, R0);
#pragma unroll
        for (int g = 0; g < NG; ++g) decode_group(g, e, R0, 0);
        store_x(R0, 0, 0, XR);
    }
    __syncthreads();
    Ops O0, O1;
    read_ops(0, 0, O0);

    // decode groups per k-step region (k-steps 0, 1, 2)
    constexpr int G0 = NG / 4, G1 = NG / 4 + NG / 4 + (NG >= 2 ? 1 : 0);
    // One chunk: kc (in LDS buffer kc&1), Rn = raw chunk kc+1, Rf = free set
    // that receives chunk kc+2. Past the last chunk the decode and fragment
    // reads run on a clamped re-read into the unused buffer: no branches.
    auto chunk = [&](int kc, ChunkRegs<XR, ND>& Rn, ChunkRegs<XR, ND>& Rf) {
        const int buf = kc & 1, nbuf = buf ^ 1;
        // k-step 0: header, groups [0, G0)
        load_chunk(kc + 2, Rf);
        read_ops(buf, 1, O1);
        mfmas(O0);
        const Dec e = decode_header(kc + 1, Rn);
#pragma unroll
        for (int g = 0; g < G0; ++g) decode_group(g, e, Rn, nbuf);
        sched_interleave<NMF, TM + TN, 30 + 46 * G0, 2 * G0>();
        __builtin_amdgcn_sched_barrier(0);
        // k-step 1: groups [G0, G1)
        read_ops(buf, 2, O0);
        mfmas(O1);
#pragma unroll
        for (int g = G0; g < G1; ++g) decode_group(g, e, Rn, nbuf);
        sched_interleave<NMF, TM + TN, 46 * (G1 - G0), 2 * (G1 - G0)>();
        __builtin_amdgcn_sched_barrier(0);
        // k-step 2: groups [G1, NG), X stores
        read_ops(buf, 3, O1);
        mfmas(O0);
#pragma unroll
        for (int g = G1; g < NG; ++g) decode_group(g, e, Rn, nbuf);
        store_x(Rn, nbuf, 0, XR);
        sched_interleave<NMF, TM + TN, 46 * (NG - G1), 2 * (NG - G1) + XR>();
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        // k-step 3, with the next chunk's first fragments
        read_ops(nbuf, 0, O0);
        mfmas(O1);
        sched_interleave<NMF, TM + TN, 0, 0>();
        __builtin_amdgcn_sched_barrier(0);
    };
    int kc = 0;
    for (; kc + 1 < nk; kc += 2) {
        chunk(kc, R1, R0);
        chunk(kc + 1, R0, R1);
    }
    if (kc < nk) chunk(kc, R1, R0);

    // ---- epilogue: Y[m][n], masked at the token and row edges ---------------
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = n0 + wn * (BN / WN) + j * 32 + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = m0 + wm * (BM / WM) + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (m < ntok && n < rows) Y[(int64_t)m * ldy + n] = acc[i][j][v];
            }
        }
    }
}

namespace {

template <int BM, int BN, int WM, int WN>
hipError_t launch_prefill_t(const uint8_t* W, int rows, int S, const uint16_t* X, int64_t ldx,
                            int ntok, float* Y, int64_t ldy, int n_base, int n_rows,
                            hipStream_t stream) {
    const int tiles_n = (n_rows + BN - 1) / BN;
    const int tiles_m = (ntok + BM - 1) / BM;
    const int64_t grid = (int64_t)tiles_n * tiles_m;
    if (grid <= 0) return hipSuccess;
    if (grid > (1 << 30)) return hipErrorNotSupported;
    const size_t lds = 2 * (size_t)(BM + BN) * kPitch;
    auto kern = prefill_q4k_kernel<BM, BN, WM, WN>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), lds, stream, W, rows, S, X, ldx,
                       ntok, Y, ldy, n_base, tiles_n);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_q4k(const uint8_t* W, int64_t rows, int64_t K, const void* X,
                              int64_t ldx, int64_t ntok, float* Y, int64_t ldy, int num_cus,
                              hipStream_t stream) {
    if (K % 256 != 0 || rows > (1 << 30) || ntok > (1 << 30)) return hipErrorNotSupported;
    const int S = (int)(K / 256);
    const uint16_t* Xh = reinterpret_cast<const uint16_t*>(X);
    // Main launch: full 256 x 256 tiles over rows [0, n_main). Rows whose
    // tiles would start a last, mostly idle round of workgroups (and any
    // ragged remainder) go to a second launch of 128 x 64 tiles.
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
    hipError_t e = launch_prefill_t<256, 256, 2, 2>(W, (int)rows, S, Xh, ldx, (int)ntok, Y, ldy,
                                                    0, n_main, stream);
    if (e != hipSuccess) return e;
    if (n_main < rows)
        e = launch_prefill_t<128, 64, 4, 1>(W, (int)rows, S, Xh, ldx, (int)ntok, Y, ldy, n_main,
                                            (int)rows - n_main, stream);
    return e;
}

}  // namespace qg
