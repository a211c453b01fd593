// nf4_internal.h -- host-side declarations shared by the library's .hip files.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "nf4qlora.h"  // from include/ (on the -I path)

namespace nf4 {

// Records a failed launch for nf4_last_hip_error() and returns NF4_ELAUNCH.
int launch_status();

struct QView {  // a validated nf4_tensor
    const uint32_t* codes;  // rows*cols/8 dwords
    const float* absmax;
    const int8_t* qcodes;
    const float* gabs;
    int64_t rows, cols;
    int dq;        // 0/1
    int group;     // dq_group
    int gshift;    // log2(group) when group is a power of two, else -1
    int bshift;    // log2(block size): 6 (64 elements) or 7 (128)
    int qt;        // quant type: 0 NF4, 1 FP4 (the level table of the codes)
};

// W: fp32, or bf16 bit patterns when `bf16`
int launch_quantize(const void* W, bool bf16, int64_t n, int block, int dq, int group, int qt, uint8_t* codes,
                    float* absmax, int8_t* qcodes, float* gabs, hipStream_t s);
// Every 64-element half of a 128-element block takes its block's fp32 scale,
// or with double quant its int8 scale code (the group of dq_group blocks is
// then 2 dq_group halves), into s64[rows*cols/64]: the layer kernels see a
// 64-block weight that dequantizes to the same values.
int expand_scales(const QView& q, void* s64, hipStream_t s);
int launch_dequant_f32(const QView& q, float* out, hipStream_t s);
int launch_dequant_bf16(const QView& q, uint16_t* out, hipStream_t s);

// Layer passes (defined in the GEMM / skinny / LoRA files).  `xl`, when
// not null, is the input of the adapter branch (x with dropout applied);
// the base product always reads x.
int forward_impl(const QView& q, const uint16_t* x, int64_t M, const uint16_t* A,
                 const uint16_t* B, int r, float scale, uint16_t* h, float* u_out, void* ws,
                 size_t ws_bytes, hipStream_t s, const uint16_t* xl = nullptr);
int forward_multi_impl(const QView& q, const uint16_t* x, int64_t M, const uint16_t* Ab,
                       const uint16_t* Bb, int n, int r, const float* scales, const int32_t* ids,
                       uint16_t* h, void* ws, size_t ws_bytes, hipStream_t s);
// Adapter-input dropout in the backward (dropout.hip): xd = keep * x, the
// rescale 1/(1 - p), and the mask of the dX term.
struct BwdDropout {
    const uint16_t* xd;
    float* dxf;  // [M][in] fp32: dH Wb, before the masked term and the one rounding
    const uint8_t* bits;  // keep bits of x, M*in/8 bytes
    float inv_keep;
};
int backward_impl(const QView& q, const uint16_t* x, const uint16_t* dH, int64_t M,
                  const uint16_t* A, const uint16_t* B, int r, float scale, const float* u,
                  uint16_t* dX, float* dA, float* dB, void* ws, size_t ws_bytes, hipStream_t s,
                  const BwdDropout* drop = nullptr);
// dropout.hip
uint32_t dropout_threshold(float p);  // ceil(p 2^32)
// bits: null, or M*K/8 bytes of keep bits (byte i: elements 8i .. 8i + 7, bit b for 8i + b)
int dropout_x(const uint16_t* x, int64_t M, int64_t K, uint32_t thr, uint64_t seed, uint16_t* xd, uint8_t* bits,
              hipStream_t st);
int scale_f32(float* v, int64_t n, float f, hipStream_t st);
int dx_dropout_add(uint16_t* dx, const float* part, int Z, const float* du, const uint16_t* A, const uint8_t* bits,
                   int64_t M, int64_t K, int r, float f, hipStream_t st);
// Profiling hook: the caller's events (or null) that bracket the dominant
// kernel of a call, attached to kernel dispatches (hipExtLaunchKernelGGL).
// Mode 0: both events attach to the dominant kernel's own dispatch.  Mode 1:
// the kernel launched just before the dominant one, when launched with
// launch_before_dominant, records the start event at its end (the pair then
// also spans the gap between the two kernels).
void prof_events(hipEvent_t* start, hipEvent_t* stop);
bool prof_start_before();  // mode 1
bool& prof_start_taken();  // per thread: the start event was attached to the previous kernel

template <typename Kernel, typename... Args>
void launch_before_dominant(Kernel kernel, dim3 grid, dim3 block, size_t shmem, hipStream_t st,
                            Args... args) {
    hipEvent_t a, b;
    prof_events(&a, &b);
    if (a && b && prof_start_before()) {
        hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, nullptr, a, 0, args...);
        prof_start_taken() = true;
    } else {
        hipLaunchKernelGGL(kernel, grid, block, shmem, st, args...);
    }
}

template <typename Kernel, typename... Args>
void launch_dominant(Kernel kernel, dim3 grid, dim3 block, size_t shmem, hipStream_t st,
                     Args... args) {
    hipEvent_t a, b;
    prof_events(&a, &b);
    if (a && b) {
        if (prof_start_taken())
            hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, nullptr, b, 0, args...);
        else
            hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, a, b, 0, args...);
        prof_start_taken() = false;
    } else {
        hipLaunchKernelGGL(kernel, grid, block, shmem, st, args...);
    }
}
// Decode path (M <= kSkinnyMaxM, r <= kSkinnyMaxR): partial down-projection
// kernel + fused dequant-GEMV kernel.
constexpr int64_t kSkinnyMaxM = 16;
constexpr int kSkinnyMaxR = 64;
size_t skinny_ws_bytes(int64_t M, int r);
bool gemv1_takes(const QView& q, int64_t M, int r);  // M = 1 kernel; it accepts bshift 6 or 7
int forward_skinny(const QView& q, const uint16_t* x, int64_t M, const uint16_t* A, const uint16_t* B,
                   int r, float scale, uint16_t* h, float* u_out, char* ws, hipStream_t st,
                   const uint16_t* xl = nullptr);
// Large-M fused dequant-GEMMs (256 x 256 tiles).
bool use_big_gemm(int64_t Mr, int64_t Nc);
int forward_big(const QView& q, const uint16_t* x, int64_t M, const uint16_t* ext, int KL,
                const uint16_t* B, int r, uint16_t* h, hipStream_t st);
// Forward with the weight dequantized into MFMA operand registers (256 x 256
// tiles); double quant needs rd_scales_bytes() of workspace for the fp32
// block scales.
size_t rd_scales_bytes(int64_t rows, int64_t cols);
bool use_rd(const QView& q, int64_t M, int r, int KL);
// When the tiles leave a partial last pass over the CUs, that pass's tiles
// split their reduction (fwd_tail_bytes() of workspace for the partials).
size_t fwd_tail_bytes(int64_t M, int64_t rows, int64_t cols);
int forward_rd(const QView& q, const uint16_t* x, int64_t M, const uint16_t* ext, int KL,
               const uint16_t* B, int r, uint16_t* h, float* scale_ws, float* tail_ws, hipStream_t st);
// One AdamW step on adapter parameters (adamw.hip).
int adamw_step(float* p, const float* g, float* m, float* v, uint16_t* pb, int64_t n, int step, float lr,
               float beta1, float beta2, float eps, float weight_decay, hipStream_t st);
// The adapter merged into the bf16 base weight (merge.hip).
int merge_adapter(const QView& q, const uint16_t* A, const uint16_t* B, int r, float scale, uint16_t* W_out,
                  hipStream_t st);
// The backward for a few tokens (M <= kBwdSmallMaxM, bwd_small.hip): fp32
// rank-r kernels and the transposed dequant-GEMV for dX, with
// bwd_small_ws_bytes() of workspace.
constexpr int64_t kBwdSmallMaxM = 16;
bool use_bwd_small(int64_t rows, int64_t cols, int64_t M);
size_t bwd_small_ws_bytes(int64_t rows, int64_t cols, int64_t M, int r);
int backward_small(const QView& q, const uint16_t* x, const uint16_t* dH, int64_t M, const uint16_t* A, int r,
                   const uint16_t* B, float scale, const float* u, uint16_t* dX, float* dA, float* dB, char* ws,
                   hipStream_t st);
// dX with the weight dequantized into a row-major LDS tile read transposed
// (256 x 256 tiles); double quant needs rd_scales_bytes() of workspace.
// (Both take grids from 16-32 tiles of 256 x 256 up; dX splits its
// reduction when the tiles are too few to fill the GPU, with
// dx_rd_part_bytes() of workspace for the fp32 partials.)
bool use_rd_grid(int64_t M, int64_t N);
// The multi-adapter forward on the same kernel: no rank-r K steps, the
// gathered term s_id u B_id added in the epilogue (su 16-byte aligned).
// On a small grid its reduction is split (fwd_multi_part_bytes() of
// workspace for the fp32 partials) and the gather moves to the partial sum.
size_t fwd_multi_part_bytes(int64_t M, int64_t rows, int64_t cols);
// scales_ready: scale_ws already holds the decoded block scales.
int forward_rd_multi(const QView& q, const uint16_t* x, int64_t M, const float* su, const int32_t* ids,
                     const uint16_t* Bb, int n_ad, int r, uint16_t* h, float* scale_ws, float* part_ws,
                     const struct MultiSort* ms, hipStream_t st, bool scales_ready = false);
// Multi-adapter tokens bucketed by adapter id (multi.hip): bucket order,
// bucket and segment offsets (segments of up to 16 tokens of one bucket).
constexpr int kMultiSortMaxAdapters = 4096;
struct MultiSort {
    int32_t* perm;  // [M] token indices in bucket order
    int32_t* off;   // [n_ad + 2] first position of each bucket (bucket n_ad: invalid ids)
    int32_t* seg;   // [n_ad + 2] first segment of each bucket
    int n_ad;
    int bound;      // an upper bound on the number of segments (the launch grid)
};
bool use_multi_sort(int64_t M, int n_ad, int r);
size_t multi_sort_bytes(int64_t M, int n_ad);
// With q (double-quantized) and sc_out, the same launch also decodes the
// weight's fp32 block scales into sc_out.
int multi_sort(const int32_t* ids, int64_t M, int n_ad, char* ws, MultiSort* ms, hipStream_t st,
               const QView* q = nullptr, float* sc_out = nullptr);
// su[t] = s_id x_t A_id^T for every token of a valid id (r <= 64, K % 32 == 0)
int multi_down_seg(const MultiSort& ms, const uint16_t* x, int64_t K, const uint16_t* Ab, int r,
                   const float* scales, float* su, hipStream_t st);
// h = bf16(the Z partials [Z][M][N] summed in order + the gathered term)
int multi_fin_seg(const MultiSort& ms, const float* part, int Z, int64_t M, int64_t N, const float* su, int r,
                  const uint16_t* Bb, uint16_t* h, hipStream_t st);
bool use_dx_rd(const QView& q, int64_t M, int r, int KL);
size_t dx_rd_part_bytes(int64_t M, int64_t rows, int64_t cols);
int dx_splits(int64_t M, int64_t rows, int64_t cols);
// f32: dX not written; the fp32 partials [dx_splits][M][in] go to part_ws
// (also for one split), for the caller to finish.
int dx_rd(const QView& q, const uint16_t* dH, int64_t M, const uint16_t* duext, int KL, const uint16_t* A,
          int r, uint16_t* dX, float* scale_ws, float* part_ws, hipStream_t st, bool f32 = false);
int dx_big(const QView& q, const uint16_t* dH, int64_t M, const uint16_t* duext, int KL,
           const uint16_t* A, int r, uint16_t* dX, hipStream_t st);
// Skinny rank-r products (lora_bwd.hip), r <= 64: fp32 partials over Z
// splits of the reduction.
int nt_splits(int64_t M, int64_t K);
int tn_splits(int64_t RR, int64_t M);
int nt_product(hipStream_t st, const uint16_t* P, int64_t M, int64_t K, const uint16_t* Q, int J, int Z,
               float* part);
int tn_product(hipStream_t st, const uint16_t* P, int64_t M, int64_t RR, const uint16_t* Q2, int J, int Z,
               float* part);
// The dU partials summed and scaled, written as the dX extension (hi | lo |
// pad, [M][KL]) and as hi/lo [M][128] for the dA product, with u's hi/lo too.
int fin_du(hipStream_t st, const float* part, int Z, int64_t M, int r, int KL, float scale, const float* u,
           uint16_t* duext, uint16_t* duq, uint16_t* uq, float* du = nullptr);
int transpose16(hipStream_t st, const uint16_t* b, int64_t n, int r, uint16_t* bt);
// transpose16 and the fp32 block scales of a double-quantized q into sc, one launch
int transpose_bs(hipStream_t st, const uint16_t* b, int64_t n, int r, uint16_t* bt, const QView& q, float* sc);
// dB = sb * sum of Zb partials [Zb][nb], and dA = the transposed reduce of
// Za partials [Za][na][r] scaled by sa, one launch
int reduce_pair(hipStream_t st, const float* pb, int Zb, int64_t nb, float sb, float* outb, const float* pa, int Za,
                int64_t na, int r, float sa, float* outa);
int reduce_t(hipStream_t st, const float* part, int Z, int64_t n, int r, float scale, float* out);
int zero_f32(float* p, int64_t n, hipStream_t s);  // fill kernel (graph-capture safe)
size_t workspace_bytes(int op, int64_t rows, int64_t cols, int64_t M, int r, int n_adapters);

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

}  // namespace nf4
