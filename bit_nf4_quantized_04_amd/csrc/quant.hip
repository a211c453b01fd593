// quant.hip -- NF4 (or FP4) blockwise quantizer, double quantization of the
// block scales, and dequantization to fp32 / bf16.
//
// Quantizer: "QLoRA Finetuner", section "2. Block-by-Block NormalFloat4 (NF4)
// Quantization" (absmax per 64-element block, division by it, nearest of the
// 16 levels) and "From LoRA to QLoRA", "Pillar 1" (two codes per byte, first
// element in the high nibble).  Double quantization: "QLoRA explained",
// "Double quantization" (scale / absmax * 127, rounded, int8) with the group
// size of "From LoRA to QLoRA", "Pillar 2" (256 blocks).
#include "nf4_device.h"
#include "nf4_internal.h"

using namespace nf4dev;

namespace {

// Nearest level for a normalized value: code = #{k : w >= cut_k}, found with
// a four-step binary search over the 15 sorted cuts (ties already resolved by
// the choice of cuts, see cut_bits).
__device__ __forceinline__ uint32_t nearest_code(float w) {
#define CUT(k) bits_f(cut_bits(k))
    uint32_t c = (w >= CUT(7)) ? 8u : 0u;
    float t = (c & 8u) ? CUT(11) : CUT(3);
    c |= (w >= t) ? 4u : 0u;
    t = (c & 8u) ? ((c & 4u) ? CUT(13) : CUT(9)) : ((c & 4u) ? CUT(5) : CUT(1));
    c |= (w >= t) ? 2u : 0u;
    float lo = (c & 8u) ? ((c & 4u) ? ((c & 2u) ? CUT(14) : CUT(12)) : ((c & 2u) ? CUT(10) : CUT(8)))
                        : ((c & 4u) ? ((c & 2u) ? CUT(6) : CUT(4)) : ((c & 2u) ? CUT(2) : CUT(0)));
    c |= (w >= lo) ? 1u : 0u;
#undef CUT
    return c;
}

// FP4 code of a normalized value: the sign bit of w and the nearest of the
// eight magnitudes, mag = #{k : |w| >= fp4_cut_k} by a three-step binary search.
__device__ __forceinline__ uint32_t nearest_code_fp4(float w) {
#define CUT(k) bits_f(fp4_cut_bits(k))
    const float a = fabsf(w);
    uint32_t c = (a >= CUT(3)) ? 4u : 0u;
    c |= (a >= ((c & 4u) ? CUT(5) : CUT(1))) ? 2u : 0u;
    const float lo = (c & 4u) ? ((c & 2u) ? CUT(6) : CUT(4)) : ((c & 2u) ? CUT(2) : CUT(0));
    c |= (a >= lo) ? 1u : 0u;
#undef CUT
    return c | ((f_bits(w) >> 28) & 8u);
}

template <bool FP4>
__device__ __forceinline__ uint32_t code_of(float w) {
    if constexpr (FP4) return nearest_code_fp4(w);
    else return nearest_code(w);
}

// Four consecutive input elements as fp32: an fp32 input, or bf16 bit
// patterns widened exactly.
__device__ __forceinline__ float4 load4(const float4* W, int64_t i) { return W[i]; }
__device__ __forceinline__ float4 load4(const uint2* W, int64_t i) {
    const uint2 p = W[i];
    return make_float4(bits_f(p.x << 16), bits_f(p.x & 0xffff0000u), bits_f(p.y << 16), bits_f(p.y & 0xffff0000u));
}

// One thread = 4 consecutive elements; L lanes = one block of 4L elements
// (16 lanes for 64, 32 for 128).  The absmax is an L-lane butterfly max of
// the magnitude bits (the integer order of |w| for finite w; Inf and NaN
// sort above every finite value); codes of 4 elements pack into 2 bytes.
template <int L, typename In, bool FP4>
__global__ __launch_bounds__(256) void k_quant_blocks(const In* __restrict__ W, int64_t n4,
                                                      uint16_t* __restrict__ codes,
                                                      float* __restrict__ absmax) {
    constexpr int LSH = L == 16 ? 4 : 5;
    const int64_t stride = int64_t(gridDim.x) * 256;
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n4; i += stride) {
        // n4 is a multiple of L and so is `stride`: the L lanes of a block
        // enter and leave the loop together.
        const float4 v = load4(W, i);
        constexpr uint32_t MAG = 0x7fffffffu;
        uint32_t mb = max(max(f_bits(v.x) & MAG, f_bits(v.y) & MAG), max(f_bits(v.z) & MAG, f_bits(v.w) & MAG));
#pragma unroll
        for (int off = L / 2; off >= 1; off >>= 1) mb = max(mb, uint32_t(__shfl_xor(int(mb), off, L)));
        float m = bits_f(mb);
        uint32_t packed;
        // the code of level 0: 7 for NF4, 0 (+0) for FP4
        constexpr uint32_t ZERO4 = FP4 ? 0x0000u : 0x7777u;
        if (mb >= 0x7f800000u) {
            // a block holding Inf or NaN: scale NaN, every code the level-0
            // code, so the whole block dequantizes to NaN
            packed = ZERO4;
            m = bits_f(0x7fc00000u);
        } else if (mb == 0u) {
            packed = ZERO4;  // an all-zero block: every element is level 0.0
        } else {
            const uint32_t c0 = code_of<FP4>(__fdiv_rn(v.x, m));
            const uint32_t c1 = code_of<FP4>(__fdiv_rn(v.y, m));
            const uint32_t c2 = code_of<FP4>(__fdiv_rn(v.z, m));
            const uint32_t c3 = code_of<FP4>(__fdiv_rn(v.w, m));
            packed = ((c0 << 4) | c1) | (((c2 << 4) | c3) << 8);
        }
        codes[i] = uint16_t(packed);
        if ((threadIdx.x & (L - 1)) == 0) absmax[i >> LSH] = m;
    }
}

// One wave per group of `G` consecutive block scales.
__global__ __launch_bounds__(256) void k_dq_scales(const float* __restrict__ absmax, int64_t nb,
                                                   int G, int8_t* __restrict__ q,
                                                   float* __restrict__ gabs) {
    const int lane = threadIdx.x & 63;
    const int64_t g = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const int64_t ng = (nb + G - 1) / G;
    if (g >= ng) return;  // whole wave
    const int64_t b0 = g * G;
    const int64_t len = (nb - b0 < G) ? (nb - b0) : G;
    float m = 0.0f;
    int bad = 0;  // a NaN scale (a block that held Inf or NaN) in the group
    for (int64_t j = lane; j < len; j += 64) {
        const float v = absmax[b0 + j];
        bad |= v != v;
        m = fmaxf(m, v);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    bad = __any(bad);
    // such a group gets constant NaN and codes 0: all its weights dequantize to NaN
    if (lane == 0) gabs[g] = bad ? bits_f(0x7fc00000u) : m;
    for (int64_t j = lane; j < len; j += 64) {
        int code = 0;
        if (!bad && m != 0.0f) code = (int)rintf(__fmul_rn(__fdiv_rn(absmax[b0 + j], m), 127.0f));
        q[b0 + j] = int8_t(code);
    }
}

// One thread = one dword of codes = 8 elements of one block (dword i is in
// block i >> dsh: 8 dwords per 64-element block, 16 per 128).
template <bool BF16>
__global__ __launch_bounds__(256) void k_dequant(const uint32_t* __restrict__ codes,
                                                 const float* __restrict__ absmax,
                                                 const int8_t* __restrict__ qcodes,
                                                 const float* __restrict__ gabs, int G, int dsh, int64_t n8,
                                                 int qt, void* __restrict__ out) {
    __shared__ float lv[16];
    if (threadIdx.x < 16) lv[threadIdx.x] = bits_f(qt_level_bits(qt, threadIdx.x));
    __syncthreads();
    const int64_t stride = int64_t(gridDim.x) * 256;
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n8; i += stride) {
        const int64_t b = i >> dsh;
        float s;
        if (qcodes) {
            s = __fmul_rn(q_over_127(qcodes[b]), gabs[b / G]);
        } else {
            s = absmax[b];
        }
        const uint32_t c = codes[i];
        float w[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            w[2 * j] = __fmul_rn(s, lv[(c >> (8 * j + 4)) & 15u]);
            w[2 * j + 1] = __fmul_rn(s, lv[(c >> (8 * j)) & 15u]);
        }
        if constexpr (BF16) {
            uint4 o;
            o.x = pack_bf16x2(w[0], w[1]);
            o.y = pack_bf16x2(w[2], w[3]);
            o.z = pack_bf16x2(w[4], w[5]);
            o.w = pack_bf16x2(w[6], w[7]);
            reinterpret_cast<uint4*>(out)[i] = o;
        } else {
            float4* o = reinterpret_cast<float4*>(out) + 2 * i;
            o[0] = make_float4(w[0], w[1], w[2], w[3]);
            o[1] = make_float4(w[4], w[5], w[6], w[7]);
        }
    }
}

// Half-block j of a 128-element-block weight takes the scale (or the int8
// scale code) of block j / 2.  A thread writes 16 bytes of dst (16 codes or
// 4 scales) from the 8 or 2 source entries they repeat; dst is 16-byte
// aligned, src is read entry by entry (it need not be).
template <typename T>
__global__ __launch_bounds__(256) void k_expand_scales(const T* __restrict__ src, int64_t n64,
                                                       T* __restrict__ dst) {
    constexpr int E = 16 / int(sizeof(T));  // entries of dst per thread
    const int64_t nv = n64 / E;
    const int64_t stride = int64_t(gridDim.x) * 256;
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < nv; i += stride) {
        T v[E];
#pragma unroll
        for (int k = 0; k < E / 2; ++k) v[2 * k] = v[2 * k + 1] = src[i * (E / 2) + k];
        *reinterpret_cast<uint4*>(dst + i * E) = __builtin_bit_cast(uint4, v);
    }
    // the last n64 % E entries
    const int64_t j = nv * E + int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (blockIdx.x == 0 && j < n64) dst[j] = src[j >> 1];
}

inline unsigned grid_for(int64_t items, int64_t per_block) {
    int64_t g = (items + per_block - 1) / per_block;
    const int64_t cap = 256 * 64;  // enough to fill the chip; the kernels grid-stride
    if (g > cap) g = cap;
    if (g < 1) g = 1;
    return unsigned(g);
}

}  // namespace

namespace nf4 {

int launch_quantize(const void* W, bool bf16, int64_t n, int block, int dq, int group, int qt, uint8_t* codes,
                    float* absmax, int8_t* qcodes, float* gabs, hipStream_t s) {
    const int64_t n4 = n / 4;
    uint16_t* c16 = reinterpret_cast<uint16_t*>(codes);
    const bool b128 = block == 128, fp4 = qt == 1;
    if (bf16) {
        auto kern = fp4 ? (b128 ? k_quant_blocks<32, uint2, true> : k_quant_blocks<16, uint2, true>)
                        : (b128 ? k_quant_blocks<32, uint2, false> : k_quant_blocks<16, uint2, false>);
        hipLaunchKernelGGL(kern, dim3(grid_for(n4, 256)), dim3(256), 0, s, static_cast<const uint2*>(W), n4, c16,
                           absmax);
    } else {
        auto kern = fp4 ? (b128 ? k_quant_blocks<32, float4, true> : k_quant_blocks<16, float4, true>)
                        : (b128 ? k_quant_blocks<32, float4, false> : k_quant_blocks<16, float4, false>);
        hipLaunchKernelGGL(kern, dim3(grid_for(n4, 256)), dim3(256), 0, s, static_cast<const float4*>(W), n4, c16,
                           absmax);
    }
    if (hipPeekAtLastError() != hipSuccess) return launch_status();
    if (dq) {
        const int64_t nb = n / block;
        const int64_t ng = (nb + group - 1) / group;
        hipLaunchKernelGGL(k_dq_scales, dim3(unsigned((ng + 3) / 4)), dim3(256), 0, s, absmax, nb,
                           group, qcodes, gabs);
        if (hipPeekAtLastError() != hipSuccess) return launch_status();
    }
    return NF4_OK;
}

int launch_dequant_f32(const QView& q, float* out, hipStream_t s) {
    const int64_t n8 = q.rows * q.cols / 8;
    hipLaunchKernelGGL(k_dequant<false>, dim3(grid_for(n8, 256)), dim3(256), 0, s, q.codes,
                       q.absmax, q.dq ? q.qcodes : nullptr, q.gabs, q.group, q.bshift - 3, n8, q.qt, (void*)out);
    return hipPeekAtLastError() == hipSuccess ? NF4_OK : launch_status();
}

int launch_dequant_bf16(const QView& q, uint16_t* out, hipStream_t s) {
    const int64_t n8 = q.rows * q.cols / 8;
    hipLaunchKernelGGL(k_dequant<true>, dim3(grid_for(n8, 256)), dim3(256), 0, s, q.codes,
                       q.absmax, q.dq ? q.qcodes : nullptr, q.gabs, q.group, q.bshift - 3, n8, q.qt, (void*)out);
    return hipPeekAtLastError() == hipSuccess ? NF4_OK : launch_status();
}

int expand_scales(const QView& q, void* s64, hipStream_t s) {
    const int64_t n64 = q.rows * q.cols / 64;
    if (q.dq)
        hipLaunchKernelGGL(k_expand_scales<int8_t>, dim3(grid_for(n64 / 16 + 1, 256)), dim3(256), 0, s, q.qcodes,
                           n64, static_cast<int8_t*>(s64));
    else
        hipLaunchKernelGGL(k_expand_scales<float>, dim3(grid_for(n64 / 4 + 1, 256)), dim3(256), 0, s, q.absmax,
                           n64, static_cast<float*>(s64));
    return hipPeekAtLastError() == hipSuccess ? NF4_OK : launch_status();
}

}  // namespace nf4
