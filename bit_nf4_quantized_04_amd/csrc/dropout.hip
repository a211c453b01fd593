// dropout.hip -- LoRA dropout on the adapter input ("QLoRA Finetuner",
// section "1. Low-Rank Adaptation (LoRA)" and its adapter-branch diagram:
// h = W0 x + (alpha/r) B(A(dropout(x))); "QLoRA explained", "Concrete
// example: Fine-tuning Llama-3-8B on a 24 GB GPU", uses a rate of 0.05).
// Inverted dropout: element (m, k) of x [M, K] is kept iff the first
// Philox-4x32-10 word of counter m*K + k under the seed is >= ceil(p 2^32),
// and the kept elements are scaled by 1/(1 - p).  The layer calls run the
// adapter branch on xd = keep * x (exact in bf16) with 1/(1 - p) folded into
// the scales.  The dX term keep * (dU A) / (1 - p) would need the mask per
// output element inside the dX product, so that product runs without the
// rank-r term into fp32 (split partials) and a pass of its own adds the
// partials and the masked term and rounds once.
#include <algorithm>
#include <cmath>

#include "nf4_device.h"
#include "nf4_internal.h"

using namespace nf4dev;

namespace {

// xd = keep ? x : 0 over the flattened [M][K] input, 8 elements per thread.
__global__ __launch_bounds__(256) void k_dropout_x(const uint4* __restrict__ x, int64_t n8, uint32_t thr,
                                                   uint64_t seed, uint4* __restrict__ xd) {
    const int64_t stride = int64_t(gridDim.x) * 256;
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n8; i += stride) {
        const uint4 v = x[i];
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint64_t idx = uint64_t(i) * 8 + 2 * e;
            const uint32_t lo = philox_w0(idx, seed) >= thr ? 0x0000ffffu : 0u;
            const uint32_t hi = philox_w0(idx + 1, seed) >= thr ? 0xffff0000u : 0u;
            w[e] &= lo | hi;
        }
        xd[i] = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

__global__ __launch_bounds__(256) void k_scale_f32(float* __restrict__ v, int64_t n, float f) {
    const int64_t stride = int64_t(gridDim.x) * 256;
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride) v[i] *= f;
}

// dX[m][i] = bf16( P[m][i] + f * keep(m, i) * sum_j dU[m][j] A[j][i] ), P
// the fp32 dH Wb given as Z split partials [Z][M][K], added in split order
// (one rounding for the whole sum): a workgroup takes 256 consecutive columns
// of one row (the dU row is the same for the whole workgroup).
__global__ __launch_bounds__(256) void k_dx_dropout_add(uint16_t* __restrict__ dx, const float* __restrict__ part,
                                                        int Z, const float* __restrict__ du,
                                                        const uint16_t* __restrict__ A, int64_t M, int64_t K, int r,
                                                        uint32_t thr, uint64_t seed, float f) {
    const int64_t ntk = (K + 255) / 256, tiles = M * ntk;
    for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
        const int64_t m = t / ntk, i = (t - m * ntk) * 256 + threadIdx.x;
        if (i >= K) continue;
        const float* dr = du + m * r;
        float acc = 0.0f;
        for (int j = 0; j < r; ++j) acc = __builtin_fmaf(dr[j], bf16_f(A[int64_t(j) * K + i]), acc);
        const int64_t e = m * K + i;
        const float add = philox_w0(uint64_t(e), seed) >= thr ? f * acc : 0.0f;
        float base = part[e];
        for (int z = 1; z < Z; ++z) base += part[int64_t(z) * M * K + e];
        dx[e] = to_bf16(base + add);
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

int dropout_x(const uint16_t* x, int64_t M, int64_t K, uint32_t thr, uint64_t seed, uint16_t* xd, hipStream_t st) {
    const int64_t n8 = M * K / 8;  // K % 64 == 0
    hipLaunchKernelGGL(k_dropout_x, dim3(grid_of(n8)), dim3(256), 0, st, reinterpret_cast<const uint4*>(x), n8, thr,
                       seed, reinterpret_cast<uint4*>(xd));
    return hipPeekAtLastError() == hipSuccess ? NF4_OK : launch_status();
}

int scale_f32(float* v, int64_t n, float f, hipStream_t st) {
    if (n <= 0) return NF4_OK;
    hipLaunchKernelGGL(k_scale_f32, dim3(grid_of(n)), dim3(256), 0, st, v, n, f);
    return hipPeekAtLastError() == hipSuccess ? NF4_OK : launch_status();
}

int dx_dropout_add(uint16_t* dx, const float* part, int Z, const float* du, const uint16_t* A, int64_t M, int64_t K,
                   int r, uint32_t thr, uint64_t seed, float f, hipStream_t st) {
    const int64_t tiles = M * cdiv(K, 256);
    hipLaunchKernelGGL(k_dx_dropout_add, dim3(unsigned(std::min<int64_t>(tiles, 65536))), dim3(256), 0, st, dx, part,
                       Z, du, A, M, K, r, thr, seed, f);
    return hipPeekAtLastError() == hipSuccess ? NF4_OK : launch_status();
}

}  // namespace nf4
