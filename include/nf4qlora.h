/*
 * nf4qlora.h -- C ABI of the MI355X (gfx950) NF4 QLoRA linear-layer library.
 *
 * The library computes the QLoRA linear layer
 *
 *     h = Wb x + (alpha/r) B (A x),        Wb = bf16( s~_b * NF4[code] )
 *
 * whose frozen base weight is stored as 4-bit NormalFloat codes (or FP4
 * codes, the other quant type) in blocks of 64 (or 128) elements, each block
 * with an absmax scale that may itself be quantized to int8 ("double
 * quantization").  Sources, by page title and
 * section:
 *
 *  [P1] "QLoRA Finetuner", sections "1. Low-Rank Adaptation (LoRA)" (forward
 *       h = W0 x + (alpha/r) B(A x)) and "2. Block-by-Block NormalFloat4 (NF4)
 *       Quantization" (64-element blocks, absmax scale, division by the scale,
 *       nearest of 16 levels, dequantization as scale times level).
 *  [P2] "QLoRA Specification for EMEP Fine-Tuning", "Hyperparameters"
 *       (quant type nf4, double quant on, compute dtype bfloat16), "GPU
 *       Orchestration" (adapters and optimizer state in full precision).
 *  [P3] "QLoRA explained: fine-tuning in 4-bit precision", "Double
 *       quantization" (scales divided by their absmax, times 127, rounded to
 *       int8), "The LoRA adapter path" (layout x W^T, (x A^T) B^T * scale; the
 *       dequantized weight is cast to bfloat16 and receives no gradient),
 *       "The quantization backbone" (blocks of 64 or 128 weights),
 *       "Common misconceptions" (the 16 NF4 levels), "Paged optimizers" (the
 *       Adam moments of the adapters paged to host memory), "Merging and deploying"
 *       (the adapter fused into a standalone 16-bit model).
 *  [P4] "How Fine-Tuning LLMs with LoRA and QLoRA Works", FAQ on merging
 *       adapters into the base weights (W_new = W + (alpha/r) B A).
 *  [P5] "Parameter-Efficient Fine-Tuning: From LoRA to QLoRA", "Pillar 1"
 *       (level table, worked example, two codes per byte, first element in
 *       the high nibble), "Block-Wise (Chunking) Quantization" (block size
 *       64 or 128), "Pillar 2" (8-bit scales in groups of 256), "The
 *       Real-World Bottleneck" (one resident base, adapter chosen per request).
 *
 * Conventions shared by every call:
 *  - Tensor pointers are DEVICE pointers to contiguous row-major memory owned
 *    by the caller, each aligned to 16 bytes (NF4_EINVAL otherwise).  The library never allocates, frees or synchronizes; it
 *    enqueues kernels on `stream` (a hipStream_t; NULL = the null stream) and
 *    returns.  Outputs must not alias inputs.
 *  - bf16 tensors are passed as uint16_t bit patterns.
 *  - Layouts follow nn.Linear [P3 "The LoRA adapter path"]: W is [out, in]
 *    (rows = out, cols = in), x is [M, in], A is [r, in], B is [out, r],
 *    h is [M, out].
 *  - Every call returns NF4_OK (0) or an error code; on error nothing has been
 *    enqueued (except NF4_ELAUNCH, after which the HIP error is available from
 *    nf4_last_hip_error(), per thread).  No exception crosses the ABI.
 *  - Weights should be finite.  The calls are asynchronous and never
 *    synchronize, so a status cannot depend on device data: instead a block
 *    that holds Inf or NaN is quantized to scale NaN with the level-0 code
 *    everywhere (7 for NF4, 0 for FP4)
 *    (with double quant its group gets constant NaN and scale codes 0), so
 *    every weight of that block (group) dequantizes to NaN and every output
 *    that reads it is NaN.  Activations and adapters are used as given.
 */
#ifndef NF4QLORA_H
#define NF4QLORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NF4QLORA_VERSION 2

enum {
    NF4_OK = 0,
    NF4_EINVAL = 1,        /* null pointer, negative size, r outside [0, 256], bad scale */
    NF4_ESHAPE = 2,        /* rows*cols not a multiple of the block; linear calls: cols % 64 != 0 */
    NF4_EUNSUPPORTED = 3,  /* block_size not 64 or 128, dq_group < 1, unknown quant_type */
    NF4_EWORKSPACE = 4,    /* workspace pointer NULL or smaller than qlora_workspace_bytes() */
    NF4_ELAUNCH = 5,       /* a HIP launch failed; see nf4_last_hip_error() */
    NF4_ETOOLARGE = 6      /* qlora_linear_forward_noalloc: more scratch needed than it holds */
};

/* Quant types [P2 "Hyperparameters": nf4 or fp4].  NF4: the 16 levels of
 * [P3 "Common misconceptions"], code = level index.  FP4: the pages call it
 * an IEEE-style exponent/mantissa format [P3 "Common misconceptions"]; this
 * library reads it as the 4-bit float E2M1 (1 sign, 2 exponent bits with
 * bias 1, 1 mantissa bit, subnormals, no Inf/NaN: the element type of the
 * OCP Microscaling Formats specification v1.0), the code being its bit
 * pattern and the level fl32(value / 6), so that +-absmax maps to +-1 as
 * with NF4.  FP4 quantization keeps the sign of w' and takes the nearest of
 * the eight magnitudes (an exact tie to the even code: on float32 inputs it
 * can only occur between 0 and 1/12, where that is code 0); the level-0 code
 * (all-zero and non-finite blocks) is 0 (+0). */
enum { NF4_QUANT_NF4 = 0, NF4_QUANT_FP4 = 1 };

/* Quantization settings [P2 "Hyperparameters"].  The compute dtype is bf16,
 * fixed. */
typedef struct nf4_config {
    int32_t block_size;    /* elements per block: 64 [P1 section 2] or 128 [P3 "The quantization
                              backbone"; P5 "Block-Wise (Chunking) Quantization"] */
    int32_t double_quant;  /* 0: fp32 block scales; 1: int8 scale codes + fp32 group constants */
    int32_t dq_group;      /* blocks per second-level group, >= 1 (256 [P5 Pillar 2]);
                              dq_group >= number of blocks gives one global constant [P3] */
    int32_t quant_type;    /* NF4_QUANT_NF4 (default) or NF4_QUANT_FP4; other values give
                              NF4_EUNSUPPORTED */
} nf4_config;

/* A quantized weight [rows, cols] in caller-owned device buffers.
 *  codes:        rows*cols/2 bytes; element e of the row-major flattening is
 *                the high nibble of byte e/2 when e is even, the low nibble
 *                when e is odd [P5 "Pillar 1", byte packing].
 *  absmax:       rows*cols/block_size fp32 block scales (read when double_quant == 0).
 *  scale_codes:  rows*cols/block_size int8 codes q_b (double_quant == 1); nf4_quantize
 *                writes codes in [0, 127].
 *  group_absmax: ceil(nblocks/dq_group) fp32 group constants c_g (double_quant == 1).
 * The scale used for block b is s_b, or fl32(fl32(q_b/127) * c_g) with
 * g = b / dq_group (the operation-by-operation inverse of the quantizer).
 * Every call decodes a scale code this way, a negative code from another
 * producer included (it gives a negative scale). */
typedef struct nf4_tensor {
    const uint8_t* codes;
    const float* absmax;
    const int8_t* scale_codes;
    const float* group_absmax;
    int64_t rows;
    int64_t cols;
    nf4_config cfg;
} nf4_tensor;

/* Host copy of the 16 NF4 levels (index = 4-bit code) [P3 "Common
 * misconceptions"; P5 "Pillar 1" table].  Never NULL. */
const float* nf4_table(void);
/* Host copy of the 16 levels of a quant type (index = 4-bit code): the NF4
 * table, or for NF4_QUANT_FP4 fl32(E2M1 value / 6).  NULL for an unknown
 * type. */
const float* nf4_levels(int32_t quant_type);
const char* nf4_strerror(int code);
int nf4_version(void);
/* The last hipError_t recorded by a failed launch on the calling thread. */
int nf4_last_hip_error(void);

/* Storage of a [rows, cols] weight in bytes (host-only arithmetic): codes,
 * first-level scale bytes stored (4 per block, or 1 per block with double
 * quant), second-level bytes (4 per group, double quant only).  Any output
 * pointer may be NULL.  [P5 worked example: 6 fp32 weights in one block take
 * 3 + 4 = 7 bytes; P5 "Pillar 2": 0.5 bits/param of fp32 scales fall to about
 * 0.127 with 8-bit scales in groups of 256.] */
int nf4_storage_sizes(int64_t rows, int64_t cols, const nf4_config* cfg,
                      size_t* code_bytes, size_t* scale_bytes, size_t* group_bytes);

/* Quantize W (fp32 [rows, cols], device) [P1 section 2; P5 "Pillar 1"]:
 * per contiguous block of block_size (64 or 128) elements of the row-major
 * flattening,
 *   s_b = max |w|, w' = fl32(w / s_b), code = nearest NF4 level to w'
 *   (an exact tie goes to the lower level; an all-zero block gets code 7),
 *   or with cfg->quant_type == NF4_QUANT_FP4 the FP4 code of w' (see the
 *   quant types above; an all-zero block gets code 0).
 * Writes `codes` and `absmax` (always).  With double quant [P3 "Double
 * quantization"; P5 "Pillar 2"] also writes, per group of dq_group blocks,
 *   c_g = max s_b,  q_b = round_half_even(fl32(fl32(s_b / c_g) * 127))
 * (q_b = 0 when c_g = 0) into scale_codes and group_absmax, which must then be
 * non-NULL.  Errors: NF4_EINVAL (NULL pointer, negative size), NF4_ESHAPE
 * (rows*cols % block_size != 0), NF4_EUNSUPPORTED (block_size not 64 or 128,
 * dq_group < 1). */
int nf4_quantize(const float* W, int64_t rows, int64_t cols, const nf4_config* cfg,
                 uint8_t* codes, float* absmax, int8_t* scale_codes, float* group_absmax,
                 void* stream);

/* Quantize a bf16 matrix (bit patterns [rows, cols], device, 16-byte
 * aligned): exactly nf4_quantize of its fp32 values (bf16 widens to fp32
 * without rounding), with the same outputs, contract and errors.  It takes a
 * merged 16-bit weight (qlora_merge) back to 4-bit storage [P3 "Merging and
 * deploying": the merged model may be re-quantized to 4 bits for deployment;
 * the pages name calibration-based GPTQ/AWQ there, this library's reading
 * uses its own calibration-free NF4 quantizer]. */
int nf4_quantize_bf16(const uint16_t* W, int64_t rows, int64_t cols, const nf4_config* cfg,
                      uint8_t* codes, float* absmax, int8_t* scale_codes, float* group_absmax,
                      void* stream);

/* Dequantize to fp32 [rows, cols]: w~ = fl32(scale_b * T[code]) with T the
 * levels of W->cfg.quant_type (NF4 or FP4) [P1
 * section 2, last item].  Bit-exact contract. */
int nf4_dequantize(const nf4_tensor* W, float* W_out, void* stream);
/* Dequantize to bf16 bits [rows, cols]: round-to-nearest-even of w~ [P3 "The
 * LoRA adapter path" casts the dequantized weight to bfloat16]. */
int nf4_dequantize_bf16(const nf4_tensor* W, uint16_t* W_out, void* stream);

/* Workspace sizes for the layer calls (bytes; 0 means none is needed).  For
 * a weight with 128-element blocks OR QLORA_OP_BLOCK128 into `op`: the call
 * then also keeps one fp32 scale per 64-element half-block (rows*cols/16
 * bytes, rounded up to 256) at the front of the workspace, and the kernels
 * of the 64-element layout run on it (every weight is dequantized to the
 * same value). */
enum {
    QLORA_OP_FORWARD = 1,
    QLORA_OP_BACKWARD = 2,
    QLORA_OP_FORWARD_MULTI = 3,
    QLORA_OP_BLOCK128 = 0x100,  /* OR'ed in: the weight has 128-element blocks */
    QLORA_OP_DROPOUT = 0x200    /* OR'ed in: the *_dropout calls (M*in*2 bytes more, the backward
                                   M*in*6 + M*in/8, each part rounded to 256) */
};
size_t qlora_workspace_bytes(int op, int64_t rows, int64_t cols, int64_t M, int32_t r,
                             int32_t n_adapters);

/* Forward of the QLoRA linear layer [P1 section 1; P3 "The LoRA adapter path"]:
 *   u = x A^T (fp32 [M, r]),   h = x Wb^T + scale * u B^T   (h as bf16)
 * W: rows = out, cols = in (cols % 64 == 0).  x bf16 [M, in]; A bf16 [r, in];
 * B bf16 [out, r]; h bf16 [M, out], overwritten.  u_out (fp32 [M, r]) may be
 * NULL; when given it receives u for the backward pass.  r == 0 or A/B NULL
 * gives the base product only.  No dropout on the adapter branch (p = 0; see
 * qlora_linear_forward_dropout).  M == 0 is a successful no-op.  ws must hold
 * qlora_workspace_bytes(QLORA_OP_FORWARD, ...).  Products use bf16 operands
 * with fp32 accumulation; u stays fp32 (hi+lo bf16 pair inside the MFMA). */
int qlora_linear_forward(const nf4_tensor* W, const uint16_t* x, int64_t M,
                         const uint16_t* A, const uint16_t* B, int32_t r, float scale,
                         uint16_t* h, float* u_out, void* ws, size_t ws_bytes, void* stream);

/* qlora_linear_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The same kernels, results, arguments
 * and errors as qlora_linear_forward; instead of a caller's workspace it uses
 * a scratch array that the library keeps in each device's global memory
 * (QLORA_NOALLOC_SCRATCH_BYTES = 64 MiB per device the library runs on, held
 * until the process ends).  A call whose workspace query,
 * qlora_workspace_bytes(QLORA_OP_FORWARD [| QLORA_OP_BLOCK128], ...),
 * exceeds that size returns NF4_ETOOLARGE before anything is enqueued
 * (every decode shape fits; for example 8192 -> 28672 at M = 4096 needs
 * 24 MiB, 4096 -> 11008 at M = 2048 about 52 MiB).  The scratch array is
 * shared by every call on a device and keeps the last call's contents; the
 * kernels read nothing from it that the same call did not write first.
 * Calls that overlap on one device (concurrent streams or threads) race on
 * it: serialize them. */
#define QLORA_NOALLOC_SCRATCH_BYTES (64u << 20)
int qlora_linear_forward_noalloc(const nf4_tensor* W, const uint16_t* x, int64_t M,
                                 const uint16_t* A, const uint16_t* B, int32_t r, float scale,
                                 uint16_t* h, float* u_out, void* stream);

/* Multi-adapter forward [P5 "The Real-World Bottleneck"]: token t uses
 * adapter ids[t] (device int32 [M]):
 *   h_t = x_t Wb^T + scales[id] * (x_t A_id^T) B_id^T
 * A_bank bf16 [n, r, in]; B_bank bf16 [n, out, r]; scales: device fp32 [n]
 * (alpha/r of each adapter).  A token whose id is outside [0, n) gets the base
 * output only (the pages do not say; this is the library's choice). */
int qlora_linear_forward_multi(const nf4_tensor* W, const uint16_t* x, int64_t M,
                               const uint16_t* A_bank, const uint16_t* B_bank,
                               int32_t n_adapters, int32_t r, const float* scales,
                               const int32_t* ids, uint16_t* h, void* ws, size_t ws_bytes,
                               void* stream);

/* Backward [P3 "The LoRA adapter path": gradients flow only into A and B; the
 * dequantized weight is a constant, so there is no dW].  With u = x A^T:
 *   dU = scale dH B,  dB = scale dH^T u,  dA = dU^T x,  dX = dH Wb + dU A.
 * dH bf16 [M, out]; u fp32 [M, r] saved by the forward, or NULL to recompute;
 * dX bf16 [M, in] (NULL: skipped); dA fp32 [r, in]; dB fp32 [out, r].  All
 * outputs are overwritten.  r must be >= 1. */
int qlora_linear_backward(const nf4_tensor* W, const uint16_t* x, const uint16_t* dH, int64_t M,
                          const uint16_t* A, const uint16_t* B, int32_t r, float scale,
                          const float* u, uint16_t* dX, float* dA, float* dB,
                          void* ws, size_t ws_bytes, void* stream);

/* The layer with dropout on the adapter input [P1 section 1 and its
 * adapter-branch diagram: h = W0 x + (alpha/r) B(A(dropout(x))); P3
 * "Concrete example: Fine-tuning Llama-3-8B on a 24 GB GPU": lora_dropout =
 * 0.05].  The pages give
 * the rate only; this library's reading: inverted dropout.  Element (m, k)
 * of x has flat index e = m*in + k.  One call of Philox-4x32-10 (Salmon,
 * Moraes, Dror, Shaw, SC 2011) serves four consecutive elements: with
 * counter (lo, hi of floor(e/4), 0, 0) and key (lo, hi of seed) it returns
 * four 32-bit words w0..w3, and element e is kept iff word w_(e mod 4) is
 * >= ceil(p * 2^32).  Kept elements are scaled by 1/(1 - p); the base
 * product always reads x.  Example: seed = 0, p = 0.5, elements 0..3 of x
 * are decided by the four words of the counter (0, 0, 0, 0), elements 4..7
 * by those of the counter (1, 0, 0, 0).  The same (p, seed) in the backward
 * regenerates the same mask.  p must be finite and in [0, 1) (NF4_EINVAL
 * otherwise). */
typedef struct qlora_dropout {
    float p;        /* dropout rate */
    uint32_t pad;   /* unused */
    uint64_t seed;  /* Philox key */
} qlora_dropout;

/* Forward with dropout: as qlora_linear_forward, with u_out = dropout(x) A^T
 * fp32.  Workspace: qlora_workspace_bytes(QLORA_OP_FORWARD |
 * QLORA_OP_DROPOUT [| QLORA_OP_BLOCK128], ...).  Arguments and errors as
 * qlora_linear_forward, plus NF4_EINVAL for a bad `drop`. */
int qlora_linear_forward_dropout(const nf4_tensor* W, const uint16_t* x, int64_t M, const uint16_t* A,
                                 const uint16_t* B, int32_t r, float scale, const qlora_dropout* drop,
                                 uint16_t* h, float* u_out, void* ws, size_t ws_bytes, void* stream);
/* Backward with dropout: dU = s dH B, dB = s dH^T u, dA = dU^T dropout(x),
 * dX = dH Wb + keep * (dU A) / (1 - p) (dH Wb in fp32, the masked term added
 * in fp32, one rounding to bf16).  u: dropout(x) A^T as the forward
 * returned it, or NULL to recompute it.  Workspace:
 * qlora_workspace_bytes(QLORA_OP_BACKWARD | QLORA_OP_DROPOUT [| ...], ...).
 * Arguments and errors as qlora_linear_backward, plus NF4_EINVAL for a bad
 * `drop`. */
int qlora_linear_backward_dropout(const nf4_tensor* W, const uint16_t* x, const uint16_t* dH, int64_t M,
                                  const uint16_t* A, const uint16_t* B, int32_t r, float scale,
                                  const qlora_dropout* drop, const float* u, uint16_t* dX, float* dA, float* dB,
                                  void* ws, size_t ws_bytes, void* stream);

/* Merge the adapter into the base weight for a standalone 16-bit model [P3
 * "Merging and deploying"; P4 FAQ on merging, W_new = W + (alpha/r) B A]:
 *   W_out[o][i] = bf16( Wb[o][i] + scale * sum_j B[o][j] A[j][i] )
 * Wb is the layer's dequantized bf16 weight.  W: rows = out, cols = in
 * (cols % 64 == 0); A bf16 [r, in]; B bf16 [out, r]; W_out bf16 [out, in],
 * overwritten, not aliasing the inputs.  1 <= r <= 256.  The rank-r product
 * uses bf16 operands with fp32 accumulation; Wb + scale * (B A) is formed in
 * fp32 and rounded to bf16 (nearest even).  Needs no workspace.  The merged
 * weight is not re-quantized. */
int qlora_merge(const nf4_tensor* W, const uint16_t* A, const uint16_t* B, int32_t r, float scale,
                uint16_t* W_out, void* stream);

/* One AdamW step on adapter parameters (only the adapters train; they and
 * their optimizer state stay in full precision, the state possibly paged to
 * host memory) [P2 "GPU Orchestration"; P3 "Paged optimizers"].  The rule is
 * the published AdamW, t = step >= 1:
 *   p <- p - lr*wd*p;  m <- b1*m + (1-b1)*g;  v <- b2*v + (1-b2)*g^2;
 *   p <- p - lr * (m / (1-b1^t)) / (sqrt(v / (1-b2^t)) + eps)
 * p, m, v fp32 [n], updated in place; g fp32 [n] (e.g. dA or dB of the
 * backward); p_bf16 [n] (may be NULL) receives bf16(p) for the next layer
 * call.  m and v may be device memory or pinned host memory from
 * hipHostMalloc (paged optimizer state): the kernel updates them in place.
 * fp32 arithmetic.  n == 0 is a no-op. */
int qlora_adamw_step(float* p, const float* g, float* m, float* v, uint16_t* p_bf16, int64_t n,
                     int32_t step, float lr, float beta1, float beta2, float eps,
                     float weight_decay, void* stream);

/* Profiling hook (for benchmarks; not thread-safe).  When both are non-NULL,
 * `start` and `stop` (hipEvent_t handles owned by the caller) are attached to
 * kernel dispatches on the call's stream around the dominant kernel of every
 * later qlora_linear_forward / _multi (the fused dequant product) and
 * qlora_linear_backward (the fused dequant dX product), so
 * hipEventElapsedTime gives that kernel's duration.  mode 0: both events on
 * the dominant kernel's own dispatch.  mode 1: on the few-token paths the
 * start event is recorded at the end of the kernel launched just before the
 * dominant one, so the pair also spans the gap between the two (an upper
 * bound on the kernel's time).  NULL, NULL disables.  NF4_EINVAL for one
 * NULL handle or another mode. */
int nf4_profile_events(void* start, void* stop, int mode);

#ifdef __cplusplus
}
#endif

#endif /* NF4QLORA_H */
