// adamw.hip -- one AdamW step on the adapter parameters.
//
// Only the adapters train; they and their optimizer state (the Adam moments)
// stay in full precision, the moments possibly paged to host memory ("QLoRA
// Specification for EMEP Fine-Tuning", "GPU Orchestration"; "QLoRA
// explained", "Paged optimizers").  The update is the published AdamW
// (decoupled weight decay, bias-corrected moments):
//
//   p <- p - lr*wd*p
//   m <- beta1*m + (1-beta1)*g,   v <- beta2*v + (1-beta2)*g^2
//   p <- p - lr * (m*c1) / (sqrt(v*c2) + eps),   c1 = 1/(1-beta1^t), c2 = 1/(1-beta2^t)
//
// in fp32, four parameters per thread step (16-byte accesses), and the bf16
// copy the layer calls read written in the same pass.  The moments may be
// device memory or pinned host memory (hipHostMalloc): the kernel reads and
// writes them in place either way, so a caller can keep the state of many
// adapters off the GPU.
#include <algorithm>
#include <cmath>

#include "nf4_device.h"
#include "nf4_internal.h"

using namespace nf4dev;

namespace {

struct AdamH {
    float lr, b1, b2, eps, decay, c1, c2;  // decay = 1 - lr*wd
};

__device__ __forceinline__ void adam1(const AdamH& h, float& p, float g, float& m, float& v) {
    p = p * h.decay;
    m = __builtin_fmaf(h.b1, m, (1.0f - h.b1) * g);
    v = __builtin_fmaf(h.b2, v, (1.0f - h.b2) * (g * g));
    p = p - h.lr * (m * h.c1) / (__builtin_sqrtf(v * h.c2) + h.eps);
}

__global__ __launch_bounds__(256) void k_adamw(float* __restrict__ p, const float* __restrict__ g, float* m,
                                               float* v, uint16_t* __restrict__ pb, int64_t n, AdamH h) {
    const int64_t n4 = n / 4;
    const int64_t stride = int64_t(gridDim.x) * 256;
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n4; i += stride) {
        float4 pp = reinterpret_cast<float4*>(p)[i];
        const float4 gg = reinterpret_cast<const float4*>(g)[i];
        float4 mm = reinterpret_cast<float4*>(m)[i];
        float4 vv = reinterpret_cast<float4*>(v)[i];
        adam1(h, pp.x, gg.x, mm.x, vv.x);
        adam1(h, pp.y, gg.y, mm.y, vv.y);
        adam1(h, pp.z, gg.z, mm.z, vv.z);
        adam1(h, pp.w, gg.w, mm.w, vv.w);
        reinterpret_cast<float4*>(p)[i] = pp;
        reinterpret_cast<float4*>(m)[i] = mm;
        reinterpret_cast<float4*>(v)[i] = vv;
        if (pb) reinterpret_cast<uint2*>(pb)[i] = make_uint2(pack_bf16x2(pp.x, pp.y), pack_bf16x2(pp.z, pp.w));
    }
    // the last n % 4 parameters
    const int64_t j = 4 * n4 + int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (j < n) {
        float pp = p[j], mm = m[j], vv = v[j];
        adam1(h, pp, g[j], mm, vv);
        p[j] = pp;
        m[j] = mm;
        v[j] = vv;
        if (pb) pb[j] = to_bf16(pp);
    }
}

}  // namespace

namespace nf4 {

int adamw_step(float* p, const float* g, float* m, float* v, uint16_t* pb, int64_t n, int step, float lr,
               float beta1, float beta2, float eps, float weight_decay, hipStream_t st) {
    if (n == 0) return NF4_OK;
    AdamH h;
    h.lr = lr;
    h.b1 = beta1;
    h.b2 = beta2;
    h.eps = eps;
    h.decay = float(1.0 - double(lr) * double(weight_decay));
    h.c1 = float(1.0 / (1.0 - std::pow(double(beta1), step)));
    h.c2 = float(1.0 / (1.0 - std::pow(double(beta2), step)));
    const int64_t blocks = std::min<int64_t>(std::max<int64_t>(cdiv(n / 4, 256), 1), 4096);
    hipLaunchKernelGGL(k_adamw, dim3(unsigned(blocks)), dim3(256), 0, st, p, g, m, v, pb, n, h);
    return hipPeekAtLastError() == hipSuccess ? NF4_OK : launch_status();
}

}  // namespace nf4
