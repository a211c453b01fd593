// dropout.hip -- LoRA dropout on the adapter input ("QLoRA Finetuner",
// section "1. Low-Rank Adaptation (LoRA)" and its adapter-branch diagram:
// h = W0 x + (alpha/r) B(A(dropout(x))); "QLoRA explained", "Concrete
// example: Fine-tuning Llama-3-8B on a 24 GB GPU", uses a rate of 0.05).
// Inverted dropout: element e = m*K + k of x [M, K] is kept iff output word
// e mod 4 of Philox-4x32-10 at counter floor(e/4) under the seed is
// >= ceil(p 2^32), and the kept elements are scaled by 1/(1 - p).  The layer
// calls run the adapter branch on xd = keep * x (exact in bf16) with
// 1/(1 - p) folded into the scales.  The dX term keep * (dU A) / (1 - p)
// would need the mask per output element inside the dX product, so that
// product runs without the rank-r term into fp32 (split partials) and a pass
// of its own adds the partials and the masked term and rounds once, reading
// the keep bits that the backward's masking pass stored.
#include <algorithm>
#include <cmath>

#include "nf4_device.h"
#include "nf4_internal.h"

using namespace nf4dev;

namespace {

// xd = keep ? x : 0 over the flattened [M][K] input, 8 elements (two
// generator counters) per thread; with `bits`, byte i of it holds the keep
// decisions of elements 8i .. 8i + 7 (bit b for element 8i + b).
__global__ __launch_bounds__(256) void k_dropout_x(const uint4* __restrict__ x, int64_t n8, uint32_t thr,
                                                   uint64_t seed, uint4* __restrict__ xd, uint8_t* __restrict__ bits) {
    const int64_t stride = int64_t(gridDim.x) * 256;
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n8; i += stride) {
        const uint4 v = x[i];
        const uint4 g0 = philox4(uint64_t(2 * i), seed), g1 = philox4(uint64_t(2 * i + 1), seed);
        const uint32_t wd[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        uint32_t kb = 0;
#pragma unroll
        for (int b = 0; b < 8; ++b) kb |= uint32_t(wd[b] >= thr) << b;
        // dword e of the 16 bytes: element 2e in the low half, 2e + 1 in the high half
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
            w[e] &= (((kb >> (2 * e)) & 1u) ? 0x0000ffffu : 0u) | (((kb >> (2 * e + 1)) & 1u) ? 0xffff0000u : 0u);
        xd[i] = make_uint4(w[0], w[1], w[2], w[3]);
        if (bits) bits[i] = uint8_t(kb);
    }
}

__global__ __launch_bounds__(256) void k_scale_f32(float* __restrict__ v, int64_t n, float f) {
    const int64_t stride = int64_t(gridDim.x) * 256;
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride) v[i] *= f;
}

// dX[m][i] = bf16( P[m][i] + f * keep(m, i) * sum_j dU[m][j] A[j][i] ), P
// the fp32 dH Wb given as Z split partials [Z][M][K], added in split order
// (one rounding for the whole sum).  A workgroup takes DXD_ROWS rows x 512
// columns, each thread two adjacent columns of every row: each A pair is
// loaded once for all the rows, the dU values are workgroup-uniform (scalar
// loads).  K is even.
constexpr int DXD_ROWS = 32;

__global__ __launch_bounds__(256) void k_dx_dropout_add(uint16_t* __restrict__ dx, const float* __restrict__ part,
                                                        int Z, const float* __restrict__ du,
                                                        const uint16_t* __restrict__ A,
                                                        const uint8_t* __restrict__ bits, int64_t M, int64_t K,
                                                        int r, float f) {
    const int64_t ntc = (K + 511) / 512, ntr = (M + DXD_ROWS - 1) / DXD_ROWS, tiles = ntr * ntc;
    for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
        const int64_t m0 = (t / ntc) * DXD_ROWS, i = (t % ntc) * 512 + 2 * threadIdx.x;
        if (i >= K) continue;
        float acc[DXD_ROWS][2];
#pragma unroll
        for (int mm = 0; mm < DXD_ROWS; ++mm) acc[mm][0] = acc[mm][1] = 0.0f;
        // four adapter columns per step: the dU values of a row are then four
        // consecutive floats (one wide scalar load)
        int j = 0;
        for (; j + 4 <= r; j += 4) {
            float a0[4], a1[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                a0[jj] = bf16_f(A[int64_t(j + jj) * K + i]);
                a1[jj] = bf16_f(A[int64_t(j + jj) * K + i + 1]);
            }
#pragma unroll
            for (int mm = 0; mm < DXD_ROWS; ++mm) {
                const int64_t m = m0 + mm < M ? m0 + mm : M - 1;  // uniform
                const float* d = du + m * r + j;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    acc[mm][0] = __builtin_fmaf(d[jj], a0[jj], acc[mm][0]);
                    acc[mm][1] = __builtin_fmaf(d[jj], a1[jj], acc[mm][1]);
                }
            }
        }
        for (; j < r; ++j) {
            const float a0 = bf16_f(A[int64_t(j) * K + i]), a1 = bf16_f(A[int64_t(j) * K + i + 1]);
#pragma unroll
            for (int mm = 0; mm < DXD_ROWS; ++mm) {
                const int64_t m = m0 + mm < M ? m0 + mm : M - 1;  // uniform
                const float d = du[m * r + j];
                acc[mm][0] = __builtin_fmaf(d, a0, acc[mm][0]);
                acc[mm][1] = __builtin_fmaf(d, a1, acc[mm][1]);
            }
        }
#pragma unroll
        for (int mm = 0; mm < DXD_ROWS; ++mm) {
            const int64_t m = m0 + mm;
            if (m >= M) break;
            const int64_t e = m * K + i;
            const uint32_t kb = bits[e >> 3] >> (e & 7);
            float2 base = *reinterpret_cast<const float2*>(part + e);
            for (int z = 1; z < Z; ++z) {
                const float2 q = *reinterpret_cast<const float2*>(part + int64_t(z) * M * K + e);
                base.x += q.x;
                base.y += q.y;
            }
            const float v0 = base.x + ((kb & 1u) ? f * acc[mm][0] : 0.0f);
            const float v1 = base.y + ((kb & 2u) ? f * acc[mm][1] : 0.0f);
            *reinterpret_cast<uint32_t*>(dx + e) = pack_bf16x2(v0, v1);
        }
    }
}

inline unsigned grid_of(int64_t items) {
    return unsigned(std::max<int64_t>(1, std::min<int64_t>((items + 255) / 256, 8192)));
}

}  // namespace

namespace nf4 {

uint32_t dropout_threshold(float p) {
    const double t = std::ceil(double(p) * 4294967296.0);
    return t >= 4294967295.0 ? 0xffffffffu : uint32_t(t);
}

int dropout_x(const uint16_t* x, int64_t M, int64_t K, uint32_t thr, uint64_t seed, uint16_t* xd, uint8_t* bits,
              hipStream_t st) {
    const int64_t n8 = M * K / 8;  // K % 64 == 0
    hipLaunchKernelGGL(k_dropout_x, dim3(grid_of(n8)), dim3(256), 0, st, reinterpret_cast<const uint4*>(x), n8, thr,
                       seed, reinterpret_cast<uint4*>(xd), bits);
    return hipPeekAtLastError() == hipSuccess ? NF4_OK : launch_status();
}

int scale_f32(float* v, int64_t n, float f, hipStream_t st) {
    if (n <= 0) return NF4_OK;
    hipLaunchKernelGGL(k_scale_f32, dim3(grid_of(n)), dim3(256), 0, st, v, n, f);
    return hipPeekAtLastError() == hipSuccess ? NF4_OK : launch_status();
}

int dx_dropout_add(uint16_t* dx, const float* part, int Z, const float* du, const uint16_t* A, const uint8_t* bits,
                   int64_t M, int64_t K, int r, float f, hipStream_t st) {
    if (K % 2) return NF4_ESHAPE;
    const int64_t tiles = cdiv(M, DXD_ROWS) * cdiv(K, 512);
    hipLaunchKernelGGL(k_dx_dropout_add, dim3(unsigned(std::min<int64_t>(tiles, 65536))), dim3(256), 0, st, dx, part,
                       Z, du, A, bits, M, K, r, f);
    return hipPeekAtLastError() == hipSuccess ? NF4_OK : launch_status();
}

}  // namespace nf4
