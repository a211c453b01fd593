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

// FP4, the other quant type, read as the 4-bit float E2M1 (sign bit 3,
// exponent bits 2..1 with bias 1, mantissa bit 0; exponent 0 subnormal; no
// Inf/NaN -- the OCP Microscaling element type): level = fl32(value / 6), so
// the block's absmax maps to 1.  Index = the E2M1 bit pattern: magnitudes 0,
// 1/12, 1/6, 1/4, 1/3, 1/2, 2/3, 1 and their negatives (code 8 is -0).
__host__ __device__ inline uint32_t fp4_level_bits(int i) {
    constexpr uint32_t t[8] = {0x00000000u, 0x3daaaaabu, 0x3e2aaaabu, 0x3e800000u,
                               0x3eaaaaabu, 0x3f000000u, 0x3f2aaaabu, 0x3f800000u};
    return t[i & 7] | ((i & 8) ? 0x80000000u : 0u);
}

// Decision thresholds of the FP4 magnitude search, as cut_bits does for NF4:
// the smallest binary32 above the exact midpoint of magnitudes k and k+1, so
// mag = #{k : |w'| >= cut_k}.  Only the midpoint of 0 and fl32(1/12) is a
// binary32 value; a tie there goes to code 0, the even (and lower) code.
__host__ __device__ constexpr uint32_t fp4_cut_bits(int k) {
    return k == 0 ? 0x3d2aaaacu : k == 1 ? 0x3e000001u : k == 2 ? 0x3e555556u : k == 3 ? 0x3e955556u
         : k == 4 ? 0x3ed55556u : k == 5 ? 0x3f155556u : 0x3f555556u;
}

// Level bits of quant type qt (0 = NF4, 1 = FP4) for code i.
__host__ __device__ inline uint32_t qt_level_bits(int qt, int i) {
    return qt ? fp4_level_bits(i) : level_bits(i);
}

// The same for a wave-uniform qt and constant i, as a scalar register (the
// select would otherwise be made per lane and hold a vector register).
__device__ __forceinline__ float uniform_level(int qt, int i) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(qt_level_bits(qt, i)));
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

// The table slot {0, bf16(v)} (low half zero, the product in the high half,
// so the dword read back is the fp32 value of the bf16) in one conversion:
// v_cvt_pk_bf16_f32 with a constant 0 for the low half.
__device__ __forceinline__ uint32_t slot_bf16(float v) {
    uint32_t d;
    asm("v_cvt_pk_bf16_f32 %0, 0, %1" : "=v"(d) : "v"(v));
    return d;
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

// fp32 block scales of a double-quantized weight, fl32(fl32(q_b/127) * c_g)
// with g = b >> gshift (GSH) or b / group, for blocks [0, nbk), spread over
// the threads of `nwg` workgroups of which this one is number `wg`.  The
// workgroup first tabulates fl32(q/127) for the 256 int8 codes in `tab`
// (LDS, the same division), then a thread takes four consecutive blocks at
// a time (one 4-byte code load, one 16-byte store) when the arrays are
// aligned for it, and single blocks for the rest.  Every thread of the
// workgroup must call it (it synchronizes the workgroup once).
template <bool GSH>
__device__ __forceinline__ void block_scales_wg(const int8_t* __restrict__ qcodes, const float* __restrict__ gabs,
                                                int group, int gshift, int64_t nbk, float* __restrict__ sc,
                                                int64_t wg, int64_t nwg, float* tab) {
    const int nt = int(blockDim.x);
    for (int i = int(threadIdx.x); i < 256; i += nt) tab[i] = q_over_127(int8_t(i));
    __syncthreads();
    auto grp = [&](int64_t k) { return GSH ? (k >> gshift) : (k / group); };
    const int64_t t0 = wg * nt + threadIdx.x, stride = nwg * nt;
    const bool vec = (reinterpret_cast<uintptr_t>(qcodes) & 3) == 0 && (reinterpret_cast<uintptr_t>(sc) & 15) == 0;
    const int64_t nu = vec ? nbk / 4 : 0;
    for (int64_t u = t0; u < nu; u += stride) {
        const uint32_t c = reinterpret_cast<const uint32_t*>(qcodes)[u];
        const int64_t k = 4 * u;
        float4 o;
        o.x = __fmul_rn(tab[c & 255u], gabs[grp(k)]);
        o.y = __fmul_rn(tab[(c >> 8) & 255u], gabs[grp(k + 1)]);
        o.z = __fmul_rn(tab[(c >> 16) & 255u], gabs[grp(k + 2)]);
        o.w = __fmul_rn(tab[c >> 24], gabs[grp(k + 3)]);
        reinterpret_cast<float4*>(sc)[u] = o;
    }
    for (int64_t k = 4 * nu + t0; k < nbk; k += stride) sc[k] = __fmul_rn(tab[uint8_t(qcodes[k])], gabs[grp(k)]);
}

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

// ---------------------------------------------------------------------------
// Register lookup of NF4 weights: a block's 16 products bf16(s~ T[e]) held as
// eight byte planes, and eight code nibbles turned into four bf16 pairs with
// byte permutes (no memory access).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// Byte planes of a block's 16 bf16 products: pl[0..3] low bytes of entries
// 0-3, 4-7, 8-11, 12-15, pl[4..7] the high bytes.
struct Planes { uint32_t v[8]; };

// The planes from the block's 16 products packed in pairs: w[i] = bf16 pair
// (entry 2i, entry 2i+1).
__device__ __forceinline__ Planes planes_of_pairs(const uint32_t (&w)[8]) {
    Planes t;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        t.v[g] = perm(w[2 * g + 1], w[2 * g], 0x06040200u);      // low bytes of entries 4g..4g+3
        t.v[4 + g] = perm(w[2 * g + 1], w[2 * g], 0x07050301u);  // high bytes
    }
    return t;
}

// Levels of a quant type as floats, held in (wave-uniform) registers.
struct Levels {
    float v[16];
    __device__ __forceinline__ void init(int qt) {
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] = uniform_level(qt, e);
    }
};

__device__ __forceinline__ Planes make_planes(float s, const Levels& lv) {
    float p[16];
    // (level 0 too: s * 0 is -0 for a negative scale and NaN for a NaN one)
#pragma unroll
    for (int e = 0; e < 16; ++e) p[e] = __fmul_rn(s, lv.v[e]);
    uint32_t w[8];  // w[i] = bf16 pair (entry 2i, entry 2i+1)
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = pack_bf16x2(p[2 * i], p[2 * i + 1]);
    Planes t;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        t.v[g] = perm(w[2 * g + 1], w[2 * g], 0x06040200u);      // low bytes of entries 4g..4g+3
        t.v[4 + g] = perm(w[2 * g + 1], w[2 * g], 0x07050301u);  // high bytes
    }
    return t;
}

// Constants of the nibble decode, held in VGPRs so that the selector
// arithmetic fuses into single VOP3 operations.
struct DecK {
    uint32_t m7, m4, id, sa, sb;
    __device__ __forceinline__ void init() {
        m7 = 0x07070707u;
        m4 = 0x04040404u;
        id = 0x03020100u;
        sa = 0x05010400u;
        sb = 0x07030602u;
        asm volatile("" : "+v"(m7), "+v"(m4), "+v"(id), "+v"(sa), "+v"(sb));
    }
};

// Eight nibbles (one code dword: element 2i in the high nibble of byte i,
// element 2i+1 in the low nibble) -> four bf16 pairs in element order.
__device__ __forceinline__ void lookup8(const DecK& k, const Planes& t, uint32_t cd, u32x4_t& out) {
    const uint32_t c4 = cd >> 4;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        // bytes: element 4h, 4h+1, 4h+2, 4h+3 codes in the low nibbles
        const uint32_t raw = perm(cd, c4, half ? k.sb : k.sa);
        const uint32_t s3 = raw & k.m7;
        const uint32_t s2 = ((raw >> 1) & k.m4) | k.id;  // byte i, or 4+i if bit 3
        const uint32_t lo = perm(perm(t.v[3], t.v[2], s3), perm(t.v[1], t.v[0], s3), s2);
        const uint32_t hi = perm(perm(t.v[7], t.v[6], s3), perm(t.v[5], t.v[4], s3), s2);
        out[2 * half] = perm(hi, lo, k.sa);      // elements 4h, 4h+1
        out[2 * half + 1] = perm(hi, lo, k.sb);  // elements 4h+2, 4h+3
    }
}

}  // namespace nf4dev
