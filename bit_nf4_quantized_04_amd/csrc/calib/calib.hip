// calib.hip -- the measurement kernels declared in include/nf4calib.h: a
// plain streaming read (the achievable HBM read rate for a given size), a
// loop of bf16 matrix-core instructions (the achievable MFMA rate under a
// sustained load), and the same loop fed the way the fused GEMM's inner
// loop feeds it (the ceiling of that structure).  Nothing here is used by
// the layer's kernels.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../nf4_device.h"
#include "nf4calib.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Each thread reads 16-byte pieces strided by the whole grid, four loads in
// flight per thread per iteration; the XOR of all words is reduced per
// workgroup and stored to sink[workgroup] (plain stores: atomics on one
// address would serialize thousands of waves at the end).
__global__ __launch_bounds__(256) void k_read(const uint4* __restrict__ p, int64_t n16, uint32_t* __restrict__ sink) {
    __shared__ uint32_t red[4];
    const int64_t stride = int64_t(gridDim.x) * 256;
    int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < n16; i += stride) {
        const uint4 a = p[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = (red[0] ^ red[1]) ^ (red[2] ^ red[3]);
}

// 8 independent accumulator sets per wave, so consecutive instructions do
// not wait on each other.  The operands are bf16 values with random mantissa
// bits (magnitudes in [0.5, 1)) whose mantissas change every iteration (an
// XOR with a per-iteration pattern), as in a real GEMM: a loop on constant or
// low-entropy operands draws less power and keeps a higher clock than a GEMM
// on random data can.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t mix32(uint32_t v) {
    v ^= v >> 16;
    v *= 0x7feb352dU;
    v ^= v >> 15;
    v *= 0x846ca68bU;
    v ^= v >> 16;
    return v;
}

__global__ __launch_bounds__(512) void k_mfma(int iters, float* __restrict__ sink) {
    const uint32_t seed = blockIdx.x * 512u + threadIdx.x;
    u32x4_t a, b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        a[e] = (mix32(seed * 8u + e) & 0x807F807Fu) | 0x3F003F00u;
        b[e] = (mix32(seed * 8u + 4u + e) & 0x807F807Fu) | 0x3F003F00u;
    }
    f32x16_t acc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[t][e] = 0.0f;
    uint32_t pat = mix32(seed ^ 0x9E3779B9u) & 0x007F007Fu;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
            acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, (t & 1) ? b : a),
                                                             __builtin_bit_cast(bf16x8_t, (t & 1) ? a : b), acc[t],
                                                             0, 0, 0);
        pat = (pat * 5u + 0x00130029u) & 0x007F007Fu;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a[e] ^= pat;
            b[e] ^= pat >> 1 & 0x007F007Fu;
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[t][e];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    if (threadIdx.x == 0) sink[blockIdx.x] = s;
}

// The inner loop of the fused forward GEMM without its memory traffic: one
// workgroup of eight waves per CU (the 96 KB of LDS keep a second one off),
// each wave a 256 x 32 slab of eight 32x32 accumulators.  Per iteration
// (one 16-k slice) the wave issues eight v_mfma_f32_32x32x16_bf16, each
// followed by the 16-byte LDS read of its A fragment for the next slice
// (eight waves read the same 8 KB, as they share the token tile); with
// `DEQ` it also turns one code dword into the next slice's B operand with
// the byte-plane lookup the layer's kernels use (four bf16 pairs from eight
// 4-bit codes).  The LDS holds bf16 values with random mantissas.
constexpr int TILE_LDS = 6144;  // uint4 entries: 96 KB

template <bool DEQ>
__global__ __launch_bounds__(512, 1) void k_mfma_tile(int iters, float* __restrict__ sink) {
    __shared__ uint4 buf[TILE_LDS];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    for (int i = tid; i < TILE_LDS; i += 512) {
        const uint32_t s = uint32_t(blockIdx.x) * TILE_LDS + uint32_t(i);
        buf[i] = make_uint4((mix32(4 * s) & 0x807F807Fu) | 0x3F003F00u, (mix32(4 * s + 1) & 0x807F807Fu) | 0x3F003F00u,
                            (mix32(4 * s + 2) & 0x807F807Fu) | 0x3F003F00u,
                            (mix32(4 * s + 3) & 0x807F807Fu) | 0x3F003F00u);
    }
    __syncthreads();
    const uint32_t seed = blockIdx.x * 512u + uint32_t(tid);
    nf4dev::DecK dk;
    dk.init();
    nf4dev::Levels lv;
    lv.init(0);
    const nf4dev::Planes pl = nf4dev::make_planes(0.01f + float(seed & 255u) * 1e-4f, lv);
    u32x4_t fr[8], b;
#pragma unroll
    for (int i = 0; i < 8; ++i) fr[i] = __builtin_bit_cast(u32x4_t, buf[(i * 64 + lane + w * 512) % TILE_LDS]);
#pragma unroll
    for (int e = 0; e < 4; ++e) b[e] = (mix32(seed * 8u + 4u + e) & 0x807F807Fu) | 0x3F003F00u;
    f32x16_t acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][e] = 0.0f;
    uint32_t cd = mix32(seed);
    const uint32_t base = uint32_t(w * 512 + lane) % 4096u;
    for (int it = 0; it < iters; ++it) {
        const uint32_t ib = (base + uint32_t(it & 7) * 512u) % 4096u;  // < 4096 + 7 * 64 < TILE_LDS
        u32x4_t bn;
        if constexpr (DEQ)
            nf4dev::lookup8(dk, pl, cd, bn);
        else
            bn = b ^ uint32_t(it & 0x007F007F);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fr[i]),
                                                             __builtin_bit_cast(bf16x8_t, b), acc[i], 0, 0, 0);
            fr[i] = __builtin_bit_cast(u32x4_t, buf[ib + uint32_t(i) * 64u]);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {  // the forward kernel's schedule: MFMA, LDS read, up to four VALU
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
        b = bn;
        cd = cd * 1664525u + 1013904223u;
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[i][e];
        s += float(fr[i][0] & 255u);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    if (lane == 0) sink[blockIdx.x * 8 + w] = s;
}

int resident(const void* kern, int threads) {
    int dev = 0, cus = 0, per = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kern, threads, 0) != hipSuccess || cus <= 0 ||
        per <= 0) {
        (void)hipGetLastError();
        return 0;
    }
    return cus * per;
}

int cus_of_device() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return cus;
}

}  // namespace

extern "C" {

int nf4calib_default_workgroups(int which) {
    if (which == 0) return resident(reinterpret_cast<const void*>(k_read), 256);
    return 4 * cus_of_device();
}

int nf4calib_read(const void* buf, size_t bytes, uint32_t* sink, int workgroups, void* stream) {
    if (!buf || !sink || (reinterpret_cast<uintptr_t>(buf) & 15) || bytes % 16 || workgroups < 0) return 1;
    if (workgroups == 0) workgroups = nf4calib_default_workgroups(0);
    if (workgroups <= 0) return 5;
    hipLaunchKernelGGL(k_read, dim3(unsigned(workgroups)), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint4*>(buf), int64_t(bytes / 16), sink);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

int nf4calib_mfma(int iters, int workgroups, int waves, float* sink, void* stream) {
    if (!sink || iters < 1 || workgroups < 0 || waves < 1 || waves > 8) return 1;
    if (workgroups == 0) workgroups = nf4calib_default_workgroups(1);
    if (workgroups <= 0) return 5;
    hipLaunchKernelGGL(k_mfma, dim3(unsigned(workgroups)), dim3(unsigned(64 * waves)), 0,
                       static_cast<hipStream_t>(stream), iters, sink);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

int nf4calib_mfma_tile(int iters, int workgroups, int dequant, float* sink, void* stream) {
    if (!sink || iters < 1 || workgroups < 0 || (dequant != 0 && dequant != 1)) return 1;
    if (workgroups == 0) workgroups = cus_of_device();
    if (workgroups <= 0) return 5;
    if (dequant)
        hipLaunchKernelGGL(k_mfma_tile<true>, dim3(unsigned(workgroups)), dim3(512), 0,
                           static_cast<hipStream_t>(stream), iters, sink);
    else
        hipLaunchKernelGGL(k_mfma_tile<false>, dim3(unsigned(workgroups)), dim3(512), 0,
                           static_cast<hipStream_t>(stream), iters, sink);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // extern "C"
