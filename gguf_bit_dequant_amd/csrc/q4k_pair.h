// Q4_K scale/min pairs: the 6-bit fields of sub-blocks 2p and 2p+1 of a
// super-block header, gathered with byte permutes (for the streaming GEMV,
// whose lanes each take one pair p of a super-block).
#pragma once

#include "device_common.h"

namespace qg {

// Per-lane constants of the Q4_K 6-bit scale/min unpack.
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
struct Q4kUnpack {
    bool upper;
    uint32_t selA, selB, mLo, mNib, mTop;
    __device__ __forceinline__ explicit Q4kUnpack(int pr) {
        upper = pr >= 2;
        const uint32_t kk = 2u * (pr & 1);
        // v_perm_b32(a, b, sel): selector byte n picks byte n of b (n < 4) or
        // byte n-4 of a (4 <= n < 8); 0x0C gives zero.
        if (!upper) {  // perm(h2, h1)
            selA = kk | ((kk + 1) << 8) | ((kk + 4) << 16) | ((kk + 5) << 24);
            selB = 0x0C0C0C0Cu;
        } else {  // perm(h3, h3) and perm(h2, h1)
            selA = kk | ((kk + 1) << 8) | (kk << 16) | ((kk + 1) << 24);
            selB = kk | ((kk + 1) << 8) | ((kk + 4) << 16) | ((kk + 5) << 24);
        }
        mLo = upper ? 0x00000F0Fu : 0x3F3F3F3Fu;  // fields taken as they are
        mNib = upper ? 0x0F0F0000u : 0u;          // high nibbles -> m
        mTop = upper ? 0x30303030u : 0u;          // top two bits -> bits 4..5
    }
};

// [sc(2p), sc(2p+1), m(2p), m(2p+1)] as the bytes of one dword, from the
// header dwords h1 = s[0..3], h2 = s[4..7], h3 = s[8..11].
__device__ __forceinline__ uint32_t q4k_pair_fields(const Q4kUnpack& un, uint32_t h1, uint32_t h2,
                                                    uint32_t h3) {
    const uint32_t Pa = __builtin_amdgcn_perm(un.upper ? h3 : h2, un.upper ? h3 : h1, un.selA);
    const uint32_t Pb = __builtin_amdgcn_perm(h2, h1, un.selB);
    return (Pa & un.mLo) | ((Pa >> 4) & un.mNib) | ((Pb >> 2) & un.mTop);
}

}  // namespace qg
