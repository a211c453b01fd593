// api.hip -- the extern "C" entry points declared in include/nf4qlora.h:
// argument validation, then the launches.  No allocation, no synchronization.
#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "nf4_device.h"
#include "nf4_internal.h"

namespace {

thread_local int g_last_hip_error = 0;
hipEvent_t g_prof_start = nullptr, g_prof_stop = nullptr;
int g_prof_mode = 0;

inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Validates an nf4_tensor for a linear call (cols % 64 == 0, rows*cols a
// whole number of blocks) or for dequantization (a whole number of blocks).
int view_of(const nf4_tensor* t, bool linear, nf4::QView* v) {
    if (!t) return NF4_EINVAL;
    if (t->cfg.block_size != 64 && t->cfg.block_size != 128) return NF4_EUNSUPPORTED;
    if (t->rows < 0 || t->cols < 0) return NF4_EINVAL;
    if (t->cfg.double_quant != 0 && t->cfg.double_quant != 1) return NF4_EINVAL;
    if (t->cfg.double_quant && t->cfg.dq_group < 1) return NF4_EUNSUPPORTED;
    if (t->cfg.quant_type != NF4_QUANT_NF4 && t->cfg.quant_type != NF4_QUANT_FP4) return NF4_EUNSUPPORTED;
    const int64_t n = t->rows * t->cols;
    if ((linear && t->cols % 64 != 0) || n % t->cfg.block_size != 0) return NF4_ESHAPE;
    if (n / 64 >= (int64_t(1) << 31)) return NF4_EINVAL;  // block indices are 32-bit
    if (n > 0) {
        if (!t->codes || !al16(t->codes)) return NF4_EINVAL;
        if (t->cfg.double_quant) {
            if (!t->scale_codes || !t->group_absmax) return NF4_EINVAL;
        } else if (!t->absmax) {
            return NF4_EINVAL;
        }
    }
    v->codes = reinterpret_cast<const uint32_t*>(t->codes);
    v->absmax = t->absmax;
    v->qcodes = t->scale_codes;
    v->gabs = t->group_absmax;
    v->rows = t->rows;
    v->cols = t->cols;
    v->dq = t->cfg.double_quant;
    v->group = t->cfg.double_quant ? t->cfg.dq_group : 1;
    v->gshift = -1;
    for (int sh = 0; sh < 31; ++sh)
        if ((1 << sh) == v->group) v->gshift = sh;
    v->bshift = t->cfg.block_size == 128 ? 7 : 6;
    v->qt = t->cfg.quant_type;
    return NF4_OK;
}

// Bytes at the front of a layer call's workspace that hold the per-half-block
// scales of a 128-element-block weight.
inline size_t expand_bytes(int64_t rows, int64_t cols) {
    return (size_t(rows * cols / 64) * 4 + 255) / 256 * 256;
}

// A layer call on a 128-element-block weight runs the 64-block kernels on
// the expanded scales or scale codes (the same dequantized values); the
// expansion takes the front of the workspace, the call gets the rest.
int layer_view(nf4::QView* v, void** ws, size_t* ws_bytes, hipStream_t st) {
    if (v->bshift == 6) return NF4_OK;
    const size_t eb = expand_bytes(v->rows, v->cols);
    if (!*ws || *ws_bytes < eb || !al16(*ws)) return NF4_EWORKSPACE;
    const int rc = nf4::expand_scales(*v, *ws, st);
    if (rc) return rc;
    if (v->dq) {  // int8 codes per half-block; a group of G blocks is 2G halves
        v->qcodes = static_cast<const int8_t*>(*ws);
        // (G >= 2^30 blocks of 128 covers any accepted tensor, which has
        // fewer than 2^30 of them: one group, any size past the end will do)
        v->group = v->group >= (1 << 30) ? 0x7fffffff : 2 * v->group;
        v->gshift = -1;
        for (int sh = 0; sh < 31; ++sh)
            if ((1 << sh) == v->group) v->gshift = sh;
    } else {
        v->absmax = static_cast<const float*>(*ws);
    }
    v->bshift = 6;
    *ws = static_cast<char*>(*ws) + eb;
    *ws_bytes -= eb;
    return NF4_OK;
}

inline bool bad_ptr(const void* p) { return !p || !al16(p); }

// Scratch memory of qlora_linear_forward_noalloc: one array in every
// device's global memory (allocated with the code object, held until the
// process ends).  Host code never passes `scratch` itself to a kernel (in
// host code the name is a host-side stand-in): the device address comes
// from hipGetSymbolAddress, once per device, and only that pointer is used.
constexpr size_t kNoAllocScratch = size_t(QLORA_NOALLOC_SCRATCH_BYTES);
__device__ __align__(256) unsigned char scratch[kNoAllocScratch];
constexpr int kMaxDevices = 256;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The calling thread's current device's copy of `scratch`.
int scratch_ptr(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return NF4_EINVAL;
    }
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lk(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p) {
                g_last_hip_error = int(e != hipSuccess ? e : hipErrorInvalidSymbol);
                (void)hipGetLastError();
                return NF4_ELAUNCH;
            }
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return NF4_OK;
}

}  // namespace

namespace nf4 {
namespace {
thread_local bool g_prof_start_taken = false;
}
void prof_events(hipEvent_t* start, hipEvent_t* stop) {
    *start = g_prof_start;
    *stop = g_prof_stop;
}
bool prof_start_before() { return g_prof_mode == 1; }
bool& prof_start_taken() { return g_prof_start_taken; }
int launch_status() {
    const hipError_t e = hipGetLastError();
    g_last_hip_error = int(e);
    return e == hipSuccess ? NF4_OK : NF4_ELAUNCH;
}
}  // namespace nf4

extern "C" {

namespace {
struct LevelTable {
    float v[16];
    explicit LevelTable(int qt) {
        for (int i = 0; i < 16; ++i) {
            const uint32_t b = nf4dev::qt_level_bits(qt, i);
            memcpy(&v[i], &b, 4);
        }
    }
};
}  // namespace

const float* nf4_table(void) {
    static const LevelTable t(NF4_QUANT_NF4);  // initialised once, thread-safe (C++11 function-local static)
    return t.v;
}

const float* nf4_levels(int32_t quant_type) {
    static const LevelTable fp4(NF4_QUANT_FP4);
    if (quant_type == NF4_QUANT_NF4) return nf4_table();
    return quant_type == NF4_QUANT_FP4 ? fp4.v : nullptr;
}

const char* nf4_strerror(int code) {
    switch (code) {
        case NF4_OK: return "ok";
        case NF4_EINVAL: return "invalid argument (null or misaligned pointer, negative size, bad rank or scale)";
        case NF4_ESHAPE: return "shape not a multiple of the 64-element block (linear calls: cols % 64 != 0)";
        case NF4_EUNSUPPORTED:
            return "unsupported configuration (block_size must be 64 or 128, dq_group >= 1, quant_type NF4 or FP4)";
        case NF4_EWORKSPACE: return "workspace missing or smaller than qlora_workspace_bytes()";
        case NF4_ELAUNCH: return "HIP kernel launch failed (see nf4_last_hip_error)";
        case NF4_ETOOLARGE:
            return "the call needs more scratch than qlora_linear_forward_noalloc holds "
                   "(QLORA_NOALLOC_SCRATCH_BYTES); use qlora_linear_forward with a workspace";
        default: return "unknown error code";
    }
}

int nf4_version(void) { return NF4QLORA_VERSION; }

int nf4_last_hip_error(void) { return g_last_hip_error; }

int nf4_profile_events(void* start, void* stop, int mode) {
    if ((start == nullptr) != (stop == nullptr) || (mode != 0 && mode != 1)) return NF4_EINVAL;
    g_prof_start = static_cast<hipEvent_t>(start);
    g_prof_stop = static_cast<hipEvent_t>(stop);
    g_prof_mode = mode;
    nf4::prof_start_taken() = false;
    return NF4_OK;
}

int nf4_storage_sizes(int64_t rows, int64_t cols, const nf4_config* cfg, size_t* code_bytes,
                      size_t* scale_bytes, size_t* group_bytes) {
    if (!cfg || rows < 0 || cols < 0) return NF4_EINVAL;
    if (cfg->block_size < 1) return NF4_EINVAL;
    const int64_t n = rows * cols;
    if (n % 2 != 0 || n % cfg->block_size != 0) return NF4_ESHAPE;
    const int64_t nb = n / cfg->block_size;
    if (cfg->double_quant && cfg->dq_group < 1) return NF4_EUNSUPPORTED;
    if (code_bytes) *code_bytes = size_t(n / 2);
    if (scale_bytes) *scale_bytes = size_t(cfg->double_quant ? nb : nb * 4);
    if (group_bytes)
        *group_bytes = cfg->double_quant ? size_t((nb + cfg->dq_group - 1) / cfg->dq_group) * 4 : 0;
    return NF4_OK;
}

namespace {

int quantize_any(const void* W, bool bf16, int64_t rows, int64_t cols, const nf4_config* cfg, uint8_t* codes,
                 float* absmax, int8_t* scale_codes, float* group_absmax, void* stream) {
    if (!cfg) return NF4_EINVAL;
    if (cfg->block_size != 64 && cfg->block_size != 128) return NF4_EUNSUPPORTED;
    if (cfg->double_quant != 0 && cfg->double_quant != 1) return NF4_EINVAL;
    if (cfg->double_quant && cfg->dq_group < 1) return NF4_EUNSUPPORTED;
    if (cfg->quant_type != NF4_QUANT_NF4 && cfg->quant_type != NF4_QUANT_FP4) return NF4_EUNSUPPORTED;
    if (rows < 0 || cols < 0) return NF4_EINVAL;
    const int64_t n = rows * cols;
    if (n % cfg->block_size != 0) return NF4_ESHAPE;
    if (n == 0) return NF4_OK;
    if (bad_ptr(W) || bad_ptr(codes) || bad_ptr(absmax)) return NF4_EINVAL;
    if (cfg->double_quant && (bad_ptr(scale_codes) || bad_ptr(group_absmax))) return NF4_EINVAL;
    return nf4::launch_quantize(W, bf16, n, cfg->block_size, cfg->double_quant, cfg->dq_group, cfg->quant_type,
                                codes, absmax, scale_codes, group_absmax, static_cast<hipStream_t>(stream));
}

}  // namespace

int nf4_quantize(const float* W, int64_t rows, int64_t cols, const nf4_config* cfg, uint8_t* codes,
                 float* absmax, int8_t* scale_codes, float* group_absmax, void* stream) {
    return quantize_any(W, false, rows, cols, cfg, codes, absmax, scale_codes, group_absmax, stream);
}

int nf4_quantize_bf16(const uint16_t* W, int64_t rows, int64_t cols, const nf4_config* cfg, uint8_t* codes,
                      float* absmax, int8_t* scale_codes, float* group_absmax, void* stream) {
    return quantize_any(W, true, rows, cols, cfg, codes, absmax, scale_codes, group_absmax, stream);
}

int nf4_dequantize(const nf4_tensor* W, float* W_out, void* stream) {
    nf4::QView v;
    int rc = view_of(W, false, &v);
    if (rc) return rc;
    if (v.rows * v.cols == 0) return NF4_OK;
    if (bad_ptr(W_out)) return NF4_EINVAL;
    return nf4::launch_dequant_f32(v, W_out, static_cast<hipStream_t>(stream));
}

int nf4_dequantize_bf16(const nf4_tensor* W, uint16_t* W_out, void* stream) {
    nf4::QView v;
    int rc = view_of(W, false, &v);
    if (rc) return rc;
    if (v.rows * v.cols == 0) return NF4_OK;
    if (bad_ptr(W_out)) return NF4_EINVAL;
    return nf4::launch_dequant_bf16(v, W_out, static_cast<hipStream_t>(stream));
}

size_t qlora_workspace_bytes(int op, int64_t rows, int64_t cols, int64_t M, int32_t r,
                             int32_t n_adapters) {
    if (rows < 0 || cols < 0 || M < 0 || r < 0 || r > 256) return 0;
    const size_t base = nf4::workspace_bytes(op & ~(QLORA_OP_BLOCK128 | QLORA_OP_DROPOUT), rows, cols, M, r,
                                             n_adapters);
    // dropout: xd bf16 [M][in]; the backward also the fp32 dH Wb [M][in] and the keep bits
    const int base_op = op & ~(QLORA_OP_BLOCK128 | QLORA_OP_DROPOUT);
    const size_t mk = size_t(M) * size_t(cols);
    const size_t xd = (op & QLORA_OP_DROPOUT)
                          ? (mk * 2 + 255) / 256 * 256 +
                                (base_op == QLORA_OP_BACKWARD ? (mk * 4 + 255) / 256 * 256 + (mk / 8 + 255) / 256 * 256
                                                              : 0)
                          : 0;
    return ((op & QLORA_OP_BLOCK128) ? expand_bytes(rows, cols) : 0) + xd + base;
}

int qlora_linear_forward(const nf4_tensor* W, const uint16_t* x, int64_t M, const uint16_t* A,
                         const uint16_t* B, int32_t r, float scale, uint16_t* h, float* u_out,
                         void* ws, size_t ws_bytes, void* stream) {
    nf4::QView v;
    int rc = view_of(W, true, &v);
    if (rc) return rc;
    if (M < 0 || r < 0 || r > 256 || !isfinite(scale)) return NF4_EINVAL;
    if (!A || !B) r = 0;
    if (M == 0 || v.rows == 0) return NF4_OK;
    if (bad_ptr(x) || bad_ptr(h)) return NF4_EINVAL;
    if (r > 0 && (bad_ptr(A) || bad_ptr(B))) return NF4_EINVAL;
    if (u_out && !al16(u_out)) return NF4_EINVAL;
    if (v.cols == 0) return NF4_EINVAL;
    // (the single-token kernel reads the scales of 128-element blocks as they are)
    if (!nf4::gemv1_takes(v, M, r) && (rc = layer_view(&v, &ws, &ws_bytes, static_cast<hipStream_t>(stream))))
        return rc;
    return nf4::forward_impl(v, x, M, A, B, r, scale, h, r > 0 ? u_out : nullptr, ws, ws_bytes,
                             static_cast<hipStream_t>(stream));
}

int qlora_linear_forward_noalloc(const nf4_tensor* W, const uint16_t* x, int64_t M, const uint16_t* A,
                                 const uint16_t* B, int32_t r, float scale, uint16_t* h, float* u_out,
                                 void* stream) {
    nf4::QView v;
    int rc = view_of(W, true, &v);
    if (rc) return rc;
    if (M < 0 || r < 0 || r > 256 || !isfinite(scale)) return NF4_EINVAL;
    const int rr = (A && B) ? r : 0;
    const int op = QLORA_OP_FORWARD | (v.bshift == 7 ? QLORA_OP_BLOCK128 : 0);
    if (qlora_workspace_bytes(op, v.rows, v.cols, M, rr, 0) > kNoAllocScratch) return NF4_ETOOLARGE;
    if (M == 0 || v.rows == 0) return NF4_OK;
    void* ws = nullptr;
    if ((rc = scratch_ptr(&ws))) return rc;
    return qlora_linear_forward(W, x, M, A, B, r, scale, h, u_out, ws, kNoAllocScratch, stream);
}

int qlora_linear_forward_multi(const nf4_tensor* W, const uint16_t* x, int64_t M,
                               const uint16_t* A_bank, const uint16_t* B_bank, int32_t n_adapters,
                               int32_t r, const float* scales, const int32_t* ids, uint16_t* h,
                               void* ws, size_t ws_bytes, void* stream) {
    nf4::QView v;
    int rc = view_of(W, true, &v);
    if (rc) return rc;
    if (M < 0 || r < 1 || r > 256 || n_adapters < 1) return NF4_EINVAL;
    if (M == 0 || v.rows == 0) return NF4_OK;
    if (v.cols == 0) return NF4_EINVAL;
    if (bad_ptr(x) || bad_ptr(h) || bad_ptr(A_bank) || bad_ptr(B_bank) || bad_ptr(scales) ||
        bad_ptr(ids))
        return NF4_EINVAL;
    if ((rc = layer_view(&v, &ws, &ws_bytes, static_cast<hipStream_t>(stream)))) return rc;
    return nf4::forward_multi_impl(v, x, M, A_bank, B_bank, n_adapters, r, scales, ids, h, ws,
                                   ws_bytes, static_cast<hipStream_t>(stream));
}

int qlora_linear_backward(const nf4_tensor* W, const uint16_t* x, const uint16_t* dH, int64_t M,
                          const uint16_t* A, const uint16_t* B, int32_t r, float scale,
                          const float* u, uint16_t* dX, float* dA, float* dB, void* ws,
                          size_t ws_bytes, void* stream) {
    nf4::QView v;
    int rc = view_of(W, true, &v);
    if (rc) return rc;
    if (M < 0 || r < 1 || r > 256 || !isfinite(scale)) return NF4_EINVAL;
    if (bad_ptr(A) || bad_ptr(B) || bad_ptr(dA) || bad_ptr(dB)) return NF4_EINVAL;
    if (v.rows == 0 || v.cols == 0) return NF4_EINVAL;
    if (M > 0 && (bad_ptr(x) || bad_ptr(dH))) return NF4_EINVAL;
    if (u && !al16(u)) return NF4_EINVAL;
    if (dX && !al16(dX)) return NF4_EINVAL;
    if (M == 0) {
        // Empty batch: every gradient is an empty sum.
        hipStream_t st = static_cast<hipStream_t>(stream);
        rc = nf4::zero_f32(dA, int64_t(r) * v.cols, st);
        if (rc) return rc;
        return nf4::zero_f32(dB, v.rows * int64_t(r), st);
    }
    if ((rc = layer_view(&v, &ws, &ws_bytes, static_cast<hipStream_t>(stream)))) return rc;
    return nf4::backward_impl(v, x, dH, M, A, B, r, scale, u, dX, dA, dB, ws, ws_bytes,
                              static_cast<hipStream_t>(stream));
}

namespace {

// The dropout settings: the keep threshold and 1/(1 - p); p in [0, 1).
bool dropout_ok(const qlora_dropout* d) { return d && isfinite(d->p) && d->p >= 0.0f && d->p < 1.0f; }

// xd = keep * x at the front of the workspace (after a block-128 expansion);
// with `bits`, the keep bits (M*cols/8 bytes) right after it.
int dropout_input(const qlora_dropout* d, const uint16_t* x, int64_t M, int64_t cols, void** ws, size_t* ws_bytes,
                  hipStream_t st, uint16_t** xd, uint8_t** bits) {
    const size_t xb = (size_t(M) * size_t(cols) * 2 + 255) / 256 * 256;
    const size_t bb = bits ? (size_t(M) * size_t(cols) / 8 + 255) / 256 * 256 : 0;
    if (!*ws || *ws_bytes < xb + bb || !al16(*ws)) return NF4_EWORKSPACE;
    *xd = static_cast<uint16_t*>(*ws);
    if (bits) *bits = static_cast<uint8_t*>(*ws) + xb;
    const int rc = nf4::dropout_x(x, M, cols, nf4::dropout_threshold(d->p), d->seed, *xd, bits ? *bits : nullptr, st);
    if (rc) return rc;
    *ws = static_cast<char*>(*ws) + xb + bb;
    *ws_bytes -= xb + bb;
    return NF4_OK;
}

}  // namespace

int qlora_linear_forward_dropout(const nf4_tensor* W, const uint16_t* x, int64_t M, const uint16_t* A,
                                 const uint16_t* B, int32_t r, float scale, const qlora_dropout* drop,
                                 uint16_t* h, float* u_out, void* ws, size_t ws_bytes, void* stream) {
    if (!dropout_ok(drop)) return NF4_EINVAL;
    nf4::QView v;
    int rc = view_of(W, true, &v);
    if (rc) return rc;
    if (M < 0 || r < 0 || r > 256 || !isfinite(scale)) return NF4_EINVAL;
    if (!A || !B) r = 0;
    if (M == 0 || v.rows == 0) return NF4_OK;
    if (bad_ptr(x) || bad_ptr(h)) return NF4_EINVAL;
    if (r > 0 && (bad_ptr(A) || bad_ptr(B))) return NF4_EINVAL;
    if (u_out && !al16(u_out)) return NF4_EINVAL;
    if (v.cols == 0) return NF4_EINVAL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((rc = layer_view(&v, &ws, &ws_bytes, st))) return rc;
    if (r == 0) return nf4::forward_impl(v, x, M, A, B, 0, scale, h, nullptr, ws, ws_bytes, st);
    uint16_t* xd;
    if ((rc = dropout_input(drop, x, M, v.cols, &ws, &ws_bytes, st, &xd, nullptr))) return rc;
    const float ik = float(1.0 / (1.0 - double(drop->p)));
    if ((rc = nf4::forward_impl(v, x, M, A, B, r, scale * ik, h, u_out, ws, ws_bytes, st, xd))) return rc;
    return u_out ? nf4::scale_f32(u_out, M * r, ik, st) : NF4_OK;
}

int qlora_linear_backward_dropout(const nf4_tensor* W, const uint16_t* x, const uint16_t* dH, int64_t M,
                                  const uint16_t* A, const uint16_t* B, int32_t r, float scale,
                                  const qlora_dropout* drop, const float* u, uint16_t* dX, float* dA, float* dB,
                                  void* ws, size_t ws_bytes, void* stream) {
    if (!dropout_ok(drop)) return NF4_EINVAL;
    nf4::QView v;
    int rc = view_of(W, true, &v);
    if (rc) return rc;
    if (M < 0 || r < 1 || r > 256 || !isfinite(scale)) return NF4_EINVAL;
    if (bad_ptr(A) || bad_ptr(B) || bad_ptr(dA) || bad_ptr(dB)) return NF4_EINVAL;
    if (v.rows == 0 || v.cols == 0) return NF4_EINVAL;
    if (M > 0 && (bad_ptr(x) || bad_ptr(dH))) return NF4_EINVAL;
    if (u && !al16(u)) return NF4_EINVAL;
    if (dX && !al16(dX)) return NF4_EINVAL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (M == 0) {
        rc = nf4::zero_f32(dA, int64_t(r) * v.cols, st);
        if (rc) return rc;
        return nf4::zero_f32(dB, v.rows * int64_t(r), st);
    }
    if ((rc = layer_view(&v, &ws, &ws_bytes, st))) return rc;
    uint16_t* xd;
    uint8_t* bits;
    if ((rc = dropout_input(drop, x, M, v.cols, &ws, &ws_bytes, st, &xd, &bits))) return rc;
    const size_t fb = (size_t(M) * size_t(v.cols) * 4 + 255) / 256 * 256;  // fp32 dH Wb
    if (ws_bytes < fb) return NF4_EWORKSPACE;
    float* dxf = static_cast<float*>(ws);
    ws = static_cast<char*>(ws) + fb;
    ws_bytes -= fb;
    const nf4::BwdDropout bd{xd, dxf, bits, float(1.0 / (1.0 - double(drop->p)))};
    return nf4::backward_impl(v, x, dH, M, A, B, r, scale, u, dX, dA, dB, ws, ws_bytes, st, &bd);
}

int qlora_merge(const nf4_tensor* W, const uint16_t* A, const uint16_t* B, int32_t r, float scale,
                uint16_t* W_out, void* stream) {
    nf4::QView v;
    int rc = view_of(W, true, &v);
    if (rc) return rc;
    if (r < 1 || r > 256 || !isfinite(scale)) return NF4_EINVAL;
    if (v.rows == 0 || v.cols == 0) return NF4_EINVAL;
    if (bad_ptr(A) || bad_ptr(B) || bad_ptr(W_out)) return NF4_EINVAL;
    return nf4::merge_adapter(v, A, B, r, scale, W_out, static_cast<hipStream_t>(stream));
}

int qlora_adamw_step(float* p, const float* g, float* m, float* v, uint16_t* p_bf16, int64_t n,
                     int32_t step, float lr, float beta1, float beta2, float eps,
                     float weight_decay, void* stream) {
    if (n < 0 || step < 1) return NF4_EINVAL;
    if (!isfinite(lr) || !isfinite(beta1) || !isfinite(beta2) || !isfinite(eps) || !isfinite(weight_decay))
        return NF4_EINVAL;
    if (!(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f) || !(eps > 0.0f)) return NF4_EINVAL;
    if (n == 0) return NF4_OK;
    if (bad_ptr(p) || bad_ptr(g) || bad_ptr(m) || bad_ptr(v) || (p_bf16 && !al16(p_bf16))) return NF4_EINVAL;
    return nf4::adamw_step(p, g, m, v, p_bf16, n, step, lr, beta1, beta2, eps, weight_decay,
                           static_cast<hipStream_t>(stream));
}

}  // extern "C"
