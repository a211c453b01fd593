// nf4_device.h -- device-side building blocks shared by the HIP kernels.
//
// gfx950 (CDNA4) only: wave64, v_mfma_f32_16x16x32_bf16, v_cvt_pk_bf16_f32,
// v_dot2c_f32_bf16.  Nothing here is shared with the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x2_t __attribute__((ext_vector_type(2)));

namespace nf4dev {

// The 16 NF4 levels as binary32 bit patterns, index = 4-bit code ("QLoRA
// explained", "Common misconceptions"; "From LoRA to QLoRA", "Pillar 1" table).
__host__ __device__ inline uint32_t level_bits(int i) {
    constexpr uint32_t t[16] = {
        0xbf800000u, 0xbf3239b1u, 0xbf066b30u, 0xbeca32a0u, 0xbe91a24du, 0xbe3d353fu,
        0xbdba7871u, 0x00000000u, 0x3da2faffu, 0x3e24cae3u, 0x3e7c04ddu, 0x3ead033au,
        0x3ee1a4b8u, 0x3f1007abu, 0x3f3913b3u, 0x3f800000u};
    return t[i & 15];
}

// Decision thresholds for the nearest-level search.  For k = 0..14 let m_k be
// the exact midpoint (T[k] + T[k+1]) / 2.  cut_bits(k) is the smallest binary32
// value strictly greater than m_k.  For a binary32 w', "m_k < w'" is then
// "w' >= cut_k", so code = #{k : w' >= cut_k} is the nearest level with an
// exact tie going to the lower index.  (Six midpoints are themselves binary32
// values -- between levels 2|3, 6|7, 7|8, 9|10, 11|12 and 13|14 -- and the cut
// is the next value above them.)  Only called with constant k.
__host__ __device__ constexpr uint32_t cut_bits(int k) {
    return k == 0 ? 0xbf591cd8u : k == 1 ? 0xbf1c5270u : k == 2 ? 0xbeeb847fu
         : k == 3 ? 0xbeadea76u : k == 4 ? 0xbe703cecu : k == 5 ? 0xbe0d38bbu
         : k == 6 ? 0xbd3a7870u : k == 7 ? 0x3d22fb00u : k == 8 ? 0x3df64863u
         : k == 9 ? 0x3e5067e1u : k == 10 ? 0x3e9582d5u : k == 11 ? 0x3ec753fau
         : k == 12 ? 0x3f006d04u : k == 13 ? 0x3f248db0u : 0x3f5c89dau;
}

__device__ __forceinline__ float bits_f(uint32_t b) { return __builtin_bit_cast(float, b); }
__device__ __forceinline__ uint32_t f_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

// Two fp32 -> packed bf16 (lo = a, hi = b), round to nearest even
// (v_cvt_pk_bf16_f32).  Inputs here are always finite.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2_t p;
    p[0] = (__bf16)a;
    p[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ uint16_t to_bf16(float a) {
    return __builtin_bit_cast(uint16_t, (__bf16)a);
}

__device__ __forceinline__ float bf16_lo(uint32_t p) { return bits_f(p << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t p) { return bits_f(p & 0xffff0000u); }
__device__ __forceinline__ float bf16_f(uint16_t p) { return bits_f(uint32_t(p) << 16); }

// acc + a.lo*b.lo + a.hi*b.hi in fp32 (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(s16x2_t, a),
                                           __builtin_bit_cast(s16x2_t, b), acc, false);
}

// D += A(16x32) * B(32x16), bf16 in, fp32 accumulate.  Lane l supplies A row
// (l % 16) and B column (l % 16), k elements [8*(l/16), 8*(l/16)+8); it holds
// D rows [4*(l/16), +4) of column (l % 16).
__device__ __forceinline__ f32x4_t mfma16(const u32x4_t& a, const u32x4_t& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                    __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// fl32(q / 127) for an int8 scale code, as one correctly rounded division.
__device__ __forceinline__ float q_over_127(int q) { return __fdiv_rn((float)q, 127.0f); }

// Split an fp32 value into bf16 hi + bf16 lo with hi + lo == v to within
// 2^-16 |v| (hi = RNE(v), lo = RNE(v - hi); v - hi is exact).
__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
    hi = to_bf16(v);
    lo = to_bf16(__fsub_rn(v, bf16_f(hi)));
}

// Philox-4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC 2011): the four output words for the
// counter (lo, hi of ctr, 0, 0) and the key (lo, hi of seed).  Each round
// forms the 64-bit products of words 0 and 2 with the two multipliers; the
// new words are (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1,
// lo(M0 c0)), and the key advances by the two increments between rounds.
__device__ __forceinline__ uint4 philox4(uint64_t ctr, uint64_t seed) {
    uint32_t c0 = uint32_t(ctr), c1 = uint32_t(ctr >> 32), c2 = 0u, c3 = 0u;
    uint32_t k0 = uint32_t(seed), k1 = uint32_t(seed >> 32);
#pragma unroll
    for (int rnd = 0; rnd < 10; ++rnd) {
        if (rnd) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint32_t lo0 = c0 * 0xD2511F53u, hi0 = __umulhi(c0, 0xD2511F53u);
        const uint32_t lo1 = c2 * 0xCD9E8D57u, hi1 = __umulhi(c2, 0xCD9E8D57u);
        c0 = hi1 ^ c1 ^ k0;
        c1 = lo1;
        c2 = hi0 ^ c3 ^ k1;
        c3 = lo0;
    }
    return make_uint4(c0, c1, c2, c3);
}

}  // namespace nf4dev
