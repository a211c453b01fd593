// gemm.hip -- LDS-staged bf16 MFMA GEMM with on-the-fly NF4 dequantization,
// and the forward / backward / multi-adapter drivers built on it.
//
// The layer ("QLoRA Finetuner", "1. Low-Rank Adaptation"; "QLoRA explained",
// "The LoRA adapter path"):  h = x Wb^T + s (x A^T) B^T,  Wb = bf16(s~ T[code]).
// The rank-r branch is folded into the same K loop: after the base K range
// the loop continues over 2r extra columns whose A-operand is [su_hi | su_lo]
// (the fp32 s*u split into two bf16 halves) and whose B-operand is [B | B], so
// h is written exactly once and u keeps fp32 precision inside the MFMA.
//
// Backward (plain calculus of the forward; the dequantized weight is a
// constant, "QLoRA explained", "The LoRA adapter path"):
//   dU = s dH B,  dB = s dH^T u,  dA = dU^T x,  dX = dH Wb + dU A,
// with dX folded the same way ([dU_hi | dU_lo] x [A; A]).
#include "nf4_device.h"
#include "nf4_internal.h"

using namespace nf4dev;

namespace {

constexpr int BM = 128, BN = 128, BK = 32, BKP = BK + 8;
constexpr int NT = 256;

struct Smem {
    uint16_t As[BM][BKP];
    uint16_t Bs[BN][BKP];
    float lv[16];
    float q127[256];  // fl32(q/127) for the int8 code q, indexed by its byte
};

// ----------------------------------------------------------------- loaders
// Each loader fills a [128 rows][BK] bf16 tile (k contiguous) for tile rows
// starting at `row0` and K offset `k0` of its own phase.  Out-of-range
// elements are zero.

struct LdNone {
    __device__ void operator()(uint16_t (*)[BKP], int64_t, int64_t, const Smem&) const {}
};

// element (row, k) = p[row*ld + k]   (x, dH, SU, the A adapter as B-operand)
struct LdRowMajor {
    const uint16_t* p;
    int64_t rows, K, ld;
    bool vec;  // ld % 8 == 0 and p 16-byte aligned
    __device__ void operator()(uint16_t (*t)[BKP], int64_t row0, int64_t k0, const Smem&) const {
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int c = threadIdx.x + it * NT;  // 512 chunks of 8
            const int r = c >> 2, kc = (c & 3) * 8;
            const int64_t row = row0 + r, k = k0 + kc;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (row < rows) {
                const uint16_t* src = p + row * ld + k;
                if (vec && k + 8 <= K) {
                    v = *reinterpret_cast<const uint4*>(src);
                } else {
                    uint16_t e[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) e[j] = (k + j < K) ? src[j] : uint16_t(0);
                    v = make_uint4(e[0] | (uint32_t(e[1]) << 16), e[2] | (uint32_t(e[3]) << 16),
                                   e[4] | (uint32_t(e[5]) << 16), e[6] | (uint32_t(e[7]) << 16));
                }
            }
            *reinterpret_cast<uint4*>(&t[r][kc]) = v;
        }
    }
};

// element (row, k) = p[k*ld + row]   (dH^T for dB; x for dA; B adapter for dU;
// the split u / dU as [K=M][rows])
struct LdColMajor {
    const uint16_t* p;
    int64_t rows, K, ld;
    bool vec;
    __device__ void operator()(uint16_t (*t)[BKP], int64_t row0, int64_t k0, const Smem&) const {
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int c = threadIdx.x + it * NT;  // 32 k x 16 row-chunks of 8
            const int kk = c >> 4, rc = (c & 15) * 8;
            const int64_t k = k0 + kk, row = row0 + rc;
            uint16_t e[8];
            if (k < K) {
                const uint16_t* src = p + k * ld + row;
                if (vec && row + 8 <= rows) {
                    const uint4 v = *reinterpret_cast<const uint4*>(src);
                    e[0] = v.x; e[1] = v.x >> 16; e[2] = v.y; e[3] = v.y >> 16;
                    e[4] = v.z; e[5] = v.z >> 16; e[6] = v.w; e[7] = v.w >> 16;
                } else {
#pragma unroll
                    for (int j = 0; j < 8; ++j) e[j] = (row + j < rows) ? src[j] : uint16_t(0);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) e[j] = 0;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) t[rc + j][kk] = e[j];
        }
    }
};

__device__ __forceinline__ float block_scale(const nf4::QView& q, int64_t b, const Smem& sm) {
    if (q.dq) return __fmul_rn(sm.q127[uint8_t(q.qcodes[b])], q.gabs[b / q.group]);
    return q.absmax[b];
}

// NF4 weight rows as the tile rows (forward): element (n, k) = Wb[n][k].
struct LdNF4Rows {
    nf4::QView q;
    __device__ void operator()(uint16_t (*t)[BKP], int64_t row0, int64_t k0, const Smem& sm) const {
        const int r = threadIdx.x >> 1, half = threadIdx.x & 1;  // 16 weights per thread
        const int64_t row = row0 + r;
        uint4 o0 = make_uint4(0, 0, 0, 0), o1 = make_uint4(0, 0, 0, 0);
        if (row < q.rows) {
            const int64_t kw = k0 + half * 16;
            const int64_t e0 = row * q.cols + kw;
            const float s = block_scale(q, e0 >> 6, sm);
            const uint2 c = *reinterpret_cast<const uint2*>(q.codes + (e0 >> 3));
            uint32_t w[8];
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                const uint32_t cd = d ? c.y : c.x;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float a = __fmul_rn(s, sm.lv[(cd >> (8 * j + 4)) & 15u]);
                    const float b = __fmul_rn(s, sm.lv[(cd >> (8 * j)) & 15u]);
                    w[d * 4 + j] = pack_bf16x2(a, b);
                }
            }
            o0 = make_uint4(w[0], w[1], w[2], w[3]);
            o1 = make_uint4(w[4], w[5], w[6], w[7]);
        }
        *reinterpret_cast<uint4*>(&t[r][half * 16]) = o0;
        *reinterpret_cast<uint4*>(&t[r][half * 16 + 8]) = o1;
    }
};

// NF4 weight transposed (dX): tile row n = weight column, k = weight row:
// element (n, k) = Wb[k][n].  Each thread dequantizes rows k, k+1 of one
// 8-column chunk and writes (Wb[k][n], Wb[k+1][n]) pairs.
struct LdNF4Cols {
    nf4::QView q;
    __device__ void operator()(uint16_t (*t)[BKP], int64_t row0, int64_t k0, const Smem& sm) const {
        const int kp = threadIdx.x >> 4, dc = threadIdx.x & 15;
        const int64_t col = row0 + dc * 8;
        const int64_t k = k0 + 2 * kp;
        float w0[8], w1[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) { w0[e] = 0.0f; w1[e] = 0.0f; }
        if (col < q.cols) {
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                const int64_t wr = k + rr;
                if (wr < q.rows) {
                    const int64_t e0 = wr * q.cols + col;
                    const float s = block_scale(q, e0 >> 6, sm);
                    const uint32_t cd = q.codes[e0 >> 3];
                    float* w = rr ? w1 : w0;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        w[2 * j] = __fmul_rn(s, sm.lv[(cd >> (8 * j + 4)) & 15u]);
                        w[2 * j + 1] = __fmul_rn(s, sm.lv[(cd >> (8 * j)) & 15u]);
                    }
                }
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
            *reinterpret_cast<uint32_t*>(&t[dc * 8 + e][2 * kp]) = pack_bf16x2(w0[e], w1[e]);
    }
};

// LoRA extension, forward: element (n, c) = B[n][c mod r] for c < 2r, else 0.
struct LdDupRows {
    const uint16_t* B;
    int64_t rows;
    int r;
    __device__ void operator()(uint16_t (*t)[BKP], int64_t row0, int64_t k0, const Smem&) const {
        for (int i = threadIdx.x; i < BN * BK; i += NT) {
            const int rr = i / BK, kk = i % BK;
            const int64_t n = row0 + rr, c = k0 + kk;
            uint16_t v = 0;
            if (n < rows && c < 2 * r) v = B[n * r + (c % r)];
            t[rr][kk] = v;
        }
    }
};

// LoRA extension, dX: element (n, c) = A[c mod r][n] for c < 2r, else 0.
struct LdDupCols {
    const uint16_t* A;
    int64_t cols;
    int r;
    __device__ void operator()(uint16_t (*t)[BKP], int64_t row0, int64_t k0, const Smem&) const {
        for (int i = threadIdx.x; i < BN * BK; i += NT) {
            const int kk = i / BN, rr = i % BN;
            const int64_t n = row0 + rr, c = k0 + kk;
            uint16_t v = 0;
            if (n < cols && c < 2 * r) v = A[(c % r) * cols + n];
            t[rr][kk] = v;
        }
    }
};

// ----------------------------------------------------------------- outputs
struct OutBF16 {
    uint16_t* p;
    int64_t ld;
    __device__ void operator()(int, int64_t m, int64_t n, float v) const { p[m * ld + n] = to_bf16(v); }
};

struct OutPartial {  // split-K partial sums, [z][rows][cols] fp32
    float* p;
    int64_t rows, cols;
    __device__ void operator()(int z, int64_t m, int64_t n, float v) const {
        p[(int64_t(z) * rows + m) * cols + n] = v;
    }
};

// Multi-adapter: h[m][n] = base + sum_j su[m][j] * B_id[n][j] (su already
// scaled by the token's adapter scale; zero for an out-of-range id).
struct OutMulti {
    uint16_t* h;
    int64_t ld;
    const float* su;
    const int32_t* ids;
    const uint16_t* Bb;
    int n_ad, r;
    int64_t out;
    __device__ void operator()(int, int64_t m, int64_t n, float v) const {
        const int id = ids[m];
        if (id >= 0 && id < n_ad) {
            const uint16_t* b = Bb + (int64_t(id) * out + n) * r;
            const float* s = su + m * r;
            float l = 0.0f;
            for (int j = 0; j < r; ++j) l = fmaf(s[j], bf16_f(b[j]), l);
            v += l;
        }
        h[m * ld + n] = to_bf16(v);
    }
};

// Quant type of the NF4 operand among a product's loaders (NF4 when none).
template <class L>
__device__ __forceinline__ int loader_qt(const L&) { return 0; }
__device__ __forceinline__ int loader_qt(const LdNF4Rows& l) { return l.q.qt; }
__device__ __forceinline__ int loader_qt(const LdNF4Cols& l) { return l.q.qt; }

// ------------------------------------------------------------------ kernel
template <class LA1, class LB1, class LA2, class LB2, class OUT>
__global__ __launch_bounds__(NT) void k_gemm(LA1 la1, LB1 lb1, int64_t K1, LA2 la2, LB2 lb2,
                                             int64_t K2, OUT out, int64_t Mr, int64_t Nc,
                                             int splits) {
    __shared__ Smem sm;
    const int qt = loader_qt(la1) | loader_qt(lb1) | loader_qt(la2) | loader_qt(lb2);
    if (threadIdx.x < 16) sm.lv[threadIdx.x] = bits_f(qt_level_bits(qt, threadIdx.x));
    if (threadIdx.x < 256) sm.q127[threadIdx.x] = q_over_127(int8_t(threadIdx.x));
    const int64_t n0 = int64_t(blockIdx.x) * BN, m0 = int64_t(blockIdx.y) * BM;
    const int z = blockIdx.z;
    const int64_t S1 = (K1 + BK - 1) / BK, S2 = (K2 + BK - 1) / BK, S = S1 + S2;
    const int64_t sb = S * z / splits, se = S * (z + 1) / splits;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    __syncthreads();
    for (int64_t s = sb; s < se; ++s) {
        if (s < S1) {
            la1(sm.As, m0, s * BK, sm);
            lb1(sm.Bs, n0, s * BK, sm);
        } else {
            la2(sm.As, m0, (s - S1) * BK, sm);
            lb2(sm.Bs, n0, (s - S1) * BK, sm);
        }
        __syncthreads();
        u32x4_t a[4], b[4];
        const int kq = 8 * (lane >> 4), rl = lane & 15;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a[i] = *reinterpret_cast<const u32x4_t*>(&sm.As[wm * 64 + i * 16 + rl][kq]);
            b[i] = *reinterpret_cast<const u32x4_t*>(&sm.Bs[wn * 64 + i * 16 + rl][kq]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(a[i], b[j], acc[i][j]);
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t m = m0 + wm * 64 + i * 16 + 4 * (lane >> 4) + e;
                const int64_t n = n0 + wn * 64 + j * 16 + (lane & 15);
                if (m < Mr && n < Nc) out(z, m, n, acc[i][j][e]);
            }
}

template <class LA1, class LB1, class LA2, class LB2, class OUT>
int gemm(hipStream_t st, int64_t Mr, int64_t Nc, LA1 la1, LB1 lb1, int64_t K1, LA2 la2, LB2 lb2,
         int64_t K2, OUT out, int splits, bool dominant = false) {
    if (Mr <= 0 || Nc <= 0) return NF4_OK;
    dim3 grid(unsigned(nf4::cdiv(Nc, BN)), unsigned(nf4::cdiv(Mr, BM)), unsigned(splits));
    if (dominant)
        nf4::launch_dominant(k_gemm<LA1, LB1, LA2, LB2, OUT>, grid, dim3(NT), 0, st, la1, lb1, K1,
                             la2, lb2, K2, out, Mr, Nc, splits);
    else
        hipLaunchKernelGGL((k_gemm<LA1, LB1, LA2, LB2, OUT>), grid, dim3(NT), 0, st, la1, lb1, K1,
                           la2, lb2, K2, out, Mr, Nc, splits);
    return hipPeekAtLastError() == hipSuccess ? NF4_OK : nf4::launch_status();
}

// ------------------------------------------------------ small helper kernels
// out[i] = scale * sum_z part[z*n + i]
__global__ __launch_bounds__(256) void k_reduce(const float* __restrict__ part, int Z, int64_t n,
                                                float scale, float* __restrict__ out) {
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
        float a = 0.0f;
        for (int z = 0; z < Z; ++z) a += part[int64_t(z) * n + i];
        out[i] = a * scale;
    }
}

// u = the sum of the Z down-projection partials (in order), and ext [M][KL]
// = (bf16 hi of scale*u | bf16 lo | 0 pad), from one pass.
__global__ __launch_bounds__(256) void k_fin_u(const float* __restrict__ part, int Z, int64_t M, int r, int KL,
                                               float scale, float* __restrict__ u, uint16_t* __restrict__ ext) {
    const int64_t n = M * KL;
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
        const int64_t m = i / KL;
        const int c = int(i - m * KL);
        if (c < r) {
            float a = 0.0f;
            for (int z = 0; z < Z; ++z) a += part[(int64_t(z) * M + m) * r + c];
            u[m * r + c] = a;
            uint16_t h, l;
            split_bf16(__fmul_rn(scale, a), h, l);
            ext[i] = h;
            ext[i + r] = l;
        } else if (c >= 2 * r) {
            ext[i] = 0;
        }
    }
}

// k_fin_u (the first gu workgroups) and, in the same launch, the fp32 block
// scales fl32(fl32(q_b/127) * c_g) of a double-quantized weight for the
// register-dequant GEMM: two independent passes, one launch.
template <bool GSH>
__global__ __launch_bounds__(256) void k_fin_u_bs(const float* __restrict__ part, int Z, int64_t M, int r, int KL,
                                                  float scale, float* __restrict__ u, uint16_t* __restrict__ ext,
                                                  int gu, nf4::QView q, int64_t nbk, float* __restrict__ sc) {
    if (int(blockIdx.x) < gu) {
        const int64_t n = M * KL;
        for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gu) * 256) {
            const int64_t m = i / KL;
            const int c = int(i - m * KL);
            if (c < r) {
                float a = 0.0f;
                for (int z = 0; z < Z; ++z) a += part[(int64_t(z) * M + m) * r + c];
                u[m * r + c] = a;
                uint16_t h, l;
                split_bf16(__fmul_rn(scale, a), h, l);
                ext[i] = h;
                ext[i + r] = l;
            } else if (c >= 2 * r) {
                ext[i] = 0;
            }
        }
        return;
    }
    __shared__ float tab[256];
    block_scales_wg<GSH>(q.qcodes, q.gabs, q.group, q.gshift, nbk, sc, int64_t(blockIdx.x) - gu,
                         int64_t(gridDim.x) - gu, tab);
}

// From v [M][r] fp32: ext [M][KL] = (bf16 hi of scale*v | bf16 lo | 0 pad),
// and optionally hi/lo [M][r] of v itself.
__global__ __launch_bounds__(256) void k_splits(const float* __restrict__ v, int64_t M, int r, int KL,
                                                float scale, uint16_t* __restrict__ ext,
                                                uint16_t* __restrict__ hi, uint16_t* __restrict__ lo) {
    const int64_t n = M * KL;
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
        const int64_t m = i / KL;
        const int c = int(i % KL);
        if (ext) {
            uint16_t val = 0;
            if (c < 2 * r) {
                uint16_t h, l;
                split_bf16(__fmul_rn(scale, v[m * r + (c % r)]), h, l);
                val = c < r ? h : l;
            }
            ext[i] = val;
        }
        if (hi && c < r) {
            uint16_t h, l;
            split_bf16(v[m * r + c], h, l);
            hi[m * r + c] = h;
            lo[m * r + c] = l;
        }
    }
}

// Multi-adapter down-projection, one workgroup per token:
// su[t][j] = scales[id] * sum_k x[t][k] A_id[j][k]  (0 for an invalid id).
__global__ __launch_bounds__(256) void k_multi_down(const uint16_t* __restrict__ x, int64_t K,
                                                    const uint16_t* __restrict__ Ab, int n_ad, int r,
                                                    const float* __restrict__ scales,
                                                    const int32_t* __restrict__ ids,
                                                    float* __restrict__ su) {
    const int64_t t = blockIdx.x;
    const int id = ids[t];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int j = wave; j < r; j += 4) {
        float a = 0.0f;
        if (id >= 0 && id < n_ad) {
            const uint16_t* xa = x + t * K;
            const uint16_t* aa = Ab + (int64_t(id) * r + j) * K;
            for (int64_t k = lane * 8; k < K; k += 64 * 8) {
                const uint4 xv = *reinterpret_cast<const uint4*>(xa + k);
                const uint4 av = *reinterpret_cast<const uint4*>(aa + k);
                a = dot2_bf16(xv.x, av.x, a);
                a = dot2_bf16(xv.y, av.y, a);
                a = dot2_bf16(xv.z, av.z, a);
                a = dot2_bf16(xv.w, av.w, a);
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) a += __shfl_xor(a, off, 64);
        if (lane == 0) su[t * r + j] = (id >= 0 && id < n_ad) ? a * scales[id] : 0.0f;
    }
}

__global__ __launch_bounds__(256) void k_zero(float* __restrict__ p, int64_t n) {
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256)
        p[i] = 0.0f;
}

// --------------------------------------------------------------- planning
inline int choose_splits(int64_t tiles, int64_t ksteps) {
    if (tiles < 1) tiles = 1;  // (no tokens: a workspace query)
    int64_t z = (1024 + tiles - 1) / tiles;
    if (z > ksteps) z = ksteps;
    if (z > 64) z = 64;
    if (z < 1) z = 1;
    return int(z);
}

// Columns of the LoRA K-extension [hi | lo | 0 pad]: a multiple of 64 so both
// GEMM kernels step through it in whole K tiles.
inline int ext_cols(int r) { return int(nf4::cdiv(2 * r, 64) * 64); }

struct FwdPlan {
    int Zu;  // split-K of the down-projection
    size_t off_u, off_ext, off_part, off_sc, off_tail, total;
};

// Workspace of the GEMM-path down-projection: u, its bf16 hi/lo extension,
// split-K partials.
FwdPlan plan_down(int64_t rows, int64_t cols, int64_t M, int r) {
    FwdPlan p{};
    size_t o = 0;
    if (r > 0) {
        const int64_t tiles = nf4::cdiv(M, BM) * nf4::cdiv(r, BN);
        p.Zu = r <= 64 ? nf4::nt_splits(M, cols) : choose_splits(tiles, nf4::cdiv(cols, BK));
        p.off_u = o; o = nf4::align256(o + size_t(M) * r * 4);
        p.off_ext = o; o = nf4::align256(o + size_t(M) * ext_cols(r) * 2);
        p.off_part = o; o = nf4::align256(o + size_t(p.Zu) * M * r * 4);
    }
    (void)rows;
    p.total = o;
    return p;
}

FwdPlan plan_forward(int64_t rows, int64_t cols, int64_t M, int r) {
    if (M <= nf4::kSkinnyMaxM && r <= nf4::kSkinnyMaxR) {  // decode path: u partials
        FwdPlan p{};
        p.total = nf4::skinny_ws_bytes(M, r);
        return p;
    }
    FwdPlan p = plan_down(rows, cols, M, r);
    if (nf4::use_rd_grid(M, rows) || nf4::use_big_gemm(M, rows)) {  // register-dequant GEMM: fp32 block
        p.off_sc = p.total;                                           // scales, tail-split partials
        p.total = nf4::align256(p.total + nf4::rd_scales_bytes(rows, cols));
        p.off_tail = p.total;
        p.total += nf4::fwd_tail_bytes(M, rows, cols);
    }
    return p;
}

struct BwdPlan {
    FwdPlan f;       // recompute of u when it is not supplied
    int Zdu, Zdb, Zda;
    bool skinny;     // r <= 64: the lora_bwd.hip products
    size_t off_uh, off_ul, off_du, off_duext, off_duh, off_dul, off_bt, off_uq, off_duq, off_part, off_part_a,
        off_sc, off_dxv, off_dxp, total;
};

BwdPlan plan_backward(int64_t rows, int64_t cols, int64_t M, int r) {
    BwdPlan p{};
    p.f = plan_down(rows, cols, M, r);
    p.skinny = r <= 64 && rows % 16 == 0;  // dU streams dH rows 16 elements at a time
    size_t o = p.f.total;
    p.off_uh = o; o = nf4::align256(o + size_t(M) * r * 2);
    p.off_ul = o; o = nf4::align256(o + size_t(M) * r * 2);
    p.off_du = o; o = nf4::align256(o + size_t(M) * r * 4);
    p.off_duext = o; o = nf4::align256(o + size_t(M) * ext_cols(r) * 2);
    p.off_duh = o; o = nf4::align256(o + size_t(M) * r * 2);
    p.off_dul = o; o = nf4::align256(o + size_t(M) * r * 2);
    if (p.skinny) {
        p.off_bt = o; o = nf4::align256(o + size_t(rows) * r * 2);
        p.off_uq = o; o = nf4::align256(o + size_t(M) * 128 * 2);
        p.off_duq = o; o = nf4::align256(o + size_t(M) * 128 * 2);
        p.Zdu = nf4::nt_splits(M, rows);
        p.Zdb = nf4::tn_splits(rows, M);
        p.Zda = nf4::tn_splits(cols, M);
    } else {
        p.Zdu = choose_splits(nf4::cdiv(M, BM) * nf4::cdiv(r, BN), nf4::cdiv(rows, BK));
        p.Zdb = choose_splits(nf4::cdiv(rows, BM) * nf4::cdiv(r, BN), 2 * nf4::cdiv(M, BK));
        p.Zda = choose_splits(nf4::cdiv(r, BM) * nf4::cdiv(cols, BN), 2 * nf4::cdiv(M, BK));
    }
    size_t part = size_t(p.Zdu) * M * r;
    if (size_t(p.Zdb) * rows * r > part) part = size_t(p.Zdb) * rows * r;
    if (!p.skinny && size_t(p.Zda) * r * cols > part) part = size_t(p.Zda) * r * cols;
    p.off_part = o; o = nf4::align256(o + part * 4);
    if (p.skinny) {  // dA partials apart, so that one launch reduces dB and dA
        p.off_part_a = o;
        o = nf4::align256(o + size_t(p.Zda) * r * cols * 4);
    }
    if (!nf4::use_bwd_small(rows, cols, M) &&
        nf4::cdiv(M, 256) * nf4::cdiv(cols, 256) >= 16) {  // register-dequant dX: fp32 block scales,
        p.off_sc = o;                                       // split partials
        o = nf4::align256(o + nf4::rd_scales_bytes(rows, cols));
        p.off_dxp = o;
        o = nf4::align256(o + nf4::dx_rd_part_bytes(M, rows, cols));
    }
    if (nf4::use_bwd_small(rows, cols, M)) {  // the few-token backward
        p.off_dxv = o;
        o = nf4::align256(o + nf4::bwd_small_ws_bytes(rows, cols, M, r));
    }
    p.total = o;
    return p;
}

inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

unsigned ew_grid(int64_t n) {
    int64_t g = (n + 255) / 256;
    if (g > 8192) g = 8192;
    return unsigned(g < 1 ? 1 : g);
}

// u = x A^T (fp32 [M][r]) into u (split-K through `part`), then the bf16
// hi/lo extension of scale*u into ext.
// u = x A^T and its extension; with `bs` non-null also the fp32 block
// scales of the double-quantized q into bs, in the same launch as u's end.
int down_projection(hipStream_t st, const nf4::QView& q, const uint16_t* x, int64_t M,
                    const uint16_t* A, int r, float scale, const FwdPlan& fp, char* ws, float* u,
                    uint16_t* ext, float* bs = nullptr) {
    float* part = reinterpret_cast<float*>(ws + fp.off_part);
    int rc;
    if (r <= 64) {
        rc = nf4::nt_product(st, x, M, q.cols, A, r, fp.Zu, part);
    } else {
        LdRowMajor lx{x, M, q.cols, q.cols, al16(x)};
        LdRowMajor la{A, r, q.cols, q.cols, al16(A)};
        rc = gemm(st, M, r, lx, la, q.cols, LdNone{}, LdNone{}, 0, OutPartial{part, M, r}, fp.Zu);
    }
    if (rc) return rc;
    if (bs && q.dq) {
        const int gu = int(ew_grid(M * ext_cols(r)));
        const int64_t nbk = q.rows * q.cols / 64;
        const dim3 grid = dim3(unsigned(gu + std::min<int64_t>(nf4::cdiv(nbk, 1024), 4096)));
        if (q.gshift >= 0)
            hipLaunchKernelGGL(k_fin_u_bs<true>, grid, dim3(256), 0, st, part, fp.Zu, M, r, ext_cols(r), scale, u,
                               ext, gu, q, nbk, bs);
        else
            hipLaunchKernelGGL(k_fin_u_bs<false>, grid, dim3(256), 0, st, part, fp.Zu, M, r, ext_cols(r), scale, u,
                               ext, gu, q, nbk, bs);
    } else {
        hipLaunchKernelGGL(k_fin_u, dim3(ew_grid(M * ext_cols(r))), dim3(256), 0, st, part, fp.Zu, M, r,
                           ext_cols(r), scale, u, ext);
    }
    return hipPeekAtLastError() == hipSuccess ? NF4_OK : nf4::launch_status();
}

}  // namespace

namespace nf4 {

int zero_f32(float* p, int64_t n, hipStream_t st) {
    if (n <= 0) return NF4_OK;
    hipLaunchKernelGGL(k_zero, dim3(ew_grid(n)), dim3(256), 0, st, p, n);
    return hipPeekAtLastError() == hipSuccess ? NF4_OK : launch_status();
}

// Workspace of the multi-adapter forward: su [M][r] fp32, the token buckets
// (when used), then the fp32 block scales and split partials of the
// register-dequant kernel (when used).
struct MultiWs {
    size_t sort, sc, part, total;
};
MultiWs multi_ws_offsets(int64_t rows, int64_t cols, int64_t M, int r, int n) {
    MultiWs w{};
    size_t o = align256(size_t(M) * (r > 0 ? r : 0) * 4);
    w.sort = o;
    if (nf4::use_multi_sort(M, n, r)) o += nf4::multi_sort_bytes(M, n > 0 ? n : 0);
    w.sc = o;
    if (nf4::use_rd_grid(M, rows)) {
        o += align256(nf4::rd_scales_bytes(rows, cols));
        w.part = o;
        o += nf4::fwd_multi_part_bytes(M, rows, cols);
    }
    w.total = o;
    return w;
}

size_t workspace_bytes(int op, int64_t rows, int64_t cols, int64_t M, int r, int n_adapters) {
    if (op == QLORA_OP_FORWARD) return plan_forward(rows, cols, M, r).total;
    if (op == QLORA_OP_BACKWARD) return plan_backward(rows, cols, M, r).total;
    if (op == QLORA_OP_FORWARD_MULTI)  // su, the token buckets, the fp32 block scales and partials of the
        return multi_ws_offsets(rows, cols, M, r, n_adapters).total;  // register-dequant kernel
    return 0;
}

int forward_impl(const QView& q, const uint16_t* x, int64_t M, const uint16_t* A, const uint16_t* B,
                 int r, float scale, uint16_t* h, float* u_out, void* ws, size_t ws_bytes,
                 hipStream_t st, const uint16_t* xl) {
    const FwdPlan fp = plan_forward(q.rows, q.cols, M, r);
    if (ws_bytes < fp.total || (fp.total && !ws)) return NF4_EWORKSPACE;
    char* w = static_cast<char*>(ws);
    if (!xl) xl = x;
    if (M <= kSkinnyMaxM && r <= kSkinnyMaxR)
        return forward_skinny(q, x, M, A, B, r, scale, h, u_out, w, st, xl);
    LdRowMajor lx{x, M, q.cols, q.cols, al16(x)};
    LdNF4Rows lw{q};
    if (r == 0) {
        if (use_rd_grid(M, q.rows) && use_rd(q, M, 0, 0))
            return forward_rd(q, x, M, nullptr, 0, nullptr, 0, h, reinterpret_cast<float*>(w + fp.off_sc),
                              reinterpret_cast<float*>(w + fp.off_tail), st);
        if (use_big_gemm(M, q.rows)) return forward_big(q, x, M, nullptr, 0, nullptr, 0, h, st);
        return gemm(st, M, q.rows, lx, lw, q.cols, LdNone{}, LdNone{}, 0, OutBF16{h, q.rows}, 1, true);
    }
    float* u = u_out ? u_out : reinterpret_cast<float*>(w + fp.off_u);
    uint16_t* ext = reinterpret_cast<uint16_t*>(w + fp.off_ext);
    const bool rd = use_rd_grid(M, q.rows) && use_rd(q, M, r, ext_cols(r));
    float* scw = rd ? reinterpret_cast<float*>(w + fp.off_sc) : nullptr;
    int rc = down_projection(st, q, xl, M, A, r, scale, fp, w, u, ext, scw);
    if (rc) return rc;
    if (rd) {  // the block scales are decoded: the GEMM sees plain fp32 scales
        QView qv = q;
        if (q.dq) {
            qv.dq = 0;
            qv.absmax = scw;
        }
        return forward_rd(qv, x, M, ext, ext_cols(r), B, r, h, scw, reinterpret_cast<float*>(w + fp.off_tail), st);
    }
    if (use_big_gemm(M, q.rows)) return forward_big(q, x, M, ext, ext_cols(r), B, r, h, st);
    LdRowMajor le{ext, M, ext_cols(r), ext_cols(r), true};
    LdDupRows lb{B, q.rows, r};
    return gemm(st, M, q.rows, lx, lw, q.cols, le, lb, ext_cols(r), OutBF16{h, q.rows}, 1, true);
}

int backward_impl(const QView& q, const uint16_t* x, const uint16_t* dH, int64_t M, const uint16_t* A,
                  const uint16_t* B, int r, float scale, const float* u_in, uint16_t* dX, float* dA,
                  float* dB, void* ws, size_t ws_bytes, hipStream_t st, const BwdDropout* drop) {
    const BwdPlan bp = plan_backward(q.rows, q.cols, M, r);
    if (ws_bytes < bp.total || !ws) return NF4_EWORKSPACE;
    char* w = static_cast<char*>(ws);
    const int64_t out = q.rows, in = q.cols;
    const int KL = ext_cols(r);
    int rc;
    // u (recomputed when not supplied)
    const float* u = u_in;
    if (!u) {  // with dropout u = (xd A^T) / (1 - p)
        float* uu = reinterpret_cast<float*>(w + bp.f.off_u);
        rc = down_projection(st, q, drop ? drop->xd : x, M, A, r, scale, bp.f, w, uu,
                             reinterpret_cast<uint16_t*>(w + bp.f.off_ext));
        if (rc) return rc;
        if (drop && (rc = scale_f32(uu, M * r, drop->inv_keep, st))) return rc;
        u = uu;
    }
    const uint16_t* xa = drop ? drop->xd : x;             // the x of dA = dU^T x
    const float sa = drop ? drop->inv_keep : 1.0f;        // and its scale
    const bool small_plan = use_bwd_small(out, in, M);    // (no workspace for the large-tile dX then)
    uint16_t* uh = reinterpret_cast<uint16_t*>(w + bp.off_uh);
    uint16_t* ul = reinterpret_cast<uint16_t*>(w + bp.off_ul);
    float* du = reinterpret_cast<float*>(w + bp.off_du);
    uint16_t* duext = reinterpret_cast<uint16_t*>(w + bp.off_duext);
    uint16_t* duh = reinterpret_cast<uint16_t*>(w + bp.off_duh);
    uint16_t* dul = reinterpret_cast<uint16_t*>(w + bp.off_dul);
    float* part = reinterpret_cast<float*>(w + bp.off_part);
    if (small_plan && !drop)
        return backward_small(q, x, dH, M, A, r, B, scale, u, dX, dA, dB, w + bp.off_dxv, st);
    // with dropout the dX product runs without the rank-r term, into fp32
    // partials, and the masked term is added afterwards
    const int rdx = drop ? 0 : r, KLdx = drop ? 0 : KL;
    const bool dxrd = !small_plan && dX && use_dx_rd(q, M, rdx, KLdx);
    float* dx_rd_scales = (bp.skinny && dxrd && q.dq) ? reinterpret_cast<float*>(w + bp.off_sc) : nullptr;
    const bool dh_vec = al16(dH) && (out % 8 == 0);
    if (bp.skinny) {
        uint16_t* bt = reinterpret_cast<uint16_t*>(w + bp.off_bt);
        uint16_t* uq = reinterpret_cast<uint16_t*>(w + bp.off_uq);
        uint16_t* duq = reinterpret_cast<uint16_t*>(w + bp.off_duq);
        // dU = s dH B (B^T made contiguous along out first; the block scales of
        // the register-dequant dX product decoded in the same launch)
        if (dx_rd_scales) {
            if ((rc = transpose_bs(st, B, out, r, bt, q, dx_rd_scales))) return rc;
        } else if ((rc = transpose16(st, B, out, r, bt))) {
            return rc;
        }
        if ((rc = nt_product(st, dH, M, out, bt, r, bp.Zdu, part))) return rc;
        if ((rc = fin_du(st, part, bp.Zdu, M, r, KL, scale, u, duext, duq, uq, drop ? du : nullptr))) return rc;
        // dB = s dH^T u, dA = dU^T x: reductions over the tokens
        float* part_a = reinterpret_cast<float*>(w + bp.off_part_a);
        if ((rc = tn_product(st, dH, M, out, uq, r, bp.Zdb, part))) return rc;
        if ((rc = tn_product(st, xa, M, in, duq, r, bp.Zda, part_a))) return rc;
        if ((rc = reduce_pair(st, part, bp.Zdb, out * r, scale, dB, part_a, bp.Zda, in, r, sa, dA))) return rc;
    } else {
    hipLaunchKernelGGL(k_splits, dim3(ew_grid(M * r)), dim3(256), 0, st, u, M, r, r, 1.0f,
                       (uint16_t*)nullptr, uh, ul);
    if (hipPeekAtLastError() != hipSuccess) return launch_status();
    // dU = s dH B : [M][r], K = out.  B as [K=out][N=r].
    rc = gemm(st, M, r, LdRowMajor{dH, M, out, out, dh_vec}, LdColMajor{B, r, out, r, al16(B) && r % 8 == 0},
              out, LdNone{}, LdNone{}, 0, OutPartial{part, M, r}, bp.Zdu);
    if (rc) return rc;
    hipLaunchKernelGGL(k_reduce, dim3(ew_grid(M * r)), dim3(256), 0, st, part, bp.Zdu, M * r, scale, du);
    hipLaunchKernelGGL(k_splits, dim3(ew_grid(M * KL)), dim3(256), 0, st, du, M, r, KL, 1.0f, duext,
                       duh, dul);
    if (hipPeekAtLastError() != hipSuccess) return launch_status();
    // dB = s dH^T (u_hi + u_lo) : [out][r], K = M.
    rc = gemm(st, out, r, LdColMajor{dH, out, M, out, dh_vec}, LdColMajor{uh, r, M, r, r % 8 == 0}, M,
              LdColMajor{dH, out, M, out, dh_vec}, LdColMajor{ul, r, M, r, r % 8 == 0}, M,
              OutPartial{part, out, r}, bp.Zdb);
    if (rc) return rc;
    hipLaunchKernelGGL(k_reduce, dim3(ew_grid(out * r)), dim3(256), 0, st, part, bp.Zdb, out * r, scale, dB);
    if (hipPeekAtLastError() != hipSuccess) return launch_status();
    // dA = (dU_hi + dU_lo)^T x : [r][in], K = M.
    const bool x_vec = al16(xa);
    rc = gemm(st, r, in, LdColMajor{duh, r, M, r, r % 8 == 0}, LdColMajor{xa, in, M, in, x_vec}, M,
              LdColMajor{dul, r, M, r, r % 8 == 0}, LdColMajor{xa, in, M, in, x_vec}, M,
              OutPartial{part, r, in}, bp.Zda);
    if (rc) return rc;
    hipLaunchKernelGGL(k_reduce, dim3(ew_grid(r * in)), dim3(256), 0, st, part, bp.Zda, r * in, sa, dA);
    if (hipPeekAtLastError() != hipSuccess) return launch_status();
    }
    // dX = dH Wb + [dU_hi | dU_lo] [A; A] : [M][in], K = out (+ 2r).
    if (dX) {
        const uint16_t* ex = drop ? nullptr : duext;
        // with dropout: the fp32 dH Wb as Zdx split partials at dxp
        int Zdx = 1;
        float* dxp = drop ? drop->dxf : nullptr;
        if (dxrd) {
            QView qv = q;
            if (dx_rd_scales) {  // decoded already: plain fp32 scales
                qv.dq = 0;
                qv.absmax = dx_rd_scales;
            }
            float* part = reinterpret_cast<float*>(w + bp.off_dxp);
            if (drop && (Zdx = dx_splits(M, q.rows, q.cols)) == 1) part = dxp;
            if (drop) dxp = part;
            rc = dx_rd(qv, dH, M, ex, KLdx, A, rdx, dX, reinterpret_cast<float*>(w + bp.off_sc), part, st,
                       drop != nullptr);
        }
        else if (drop)
            rc = gemm(st, M, in, LdRowMajor{dH, M, out, out, dh_vec}, LdNF4Cols{q}, out, LdNone{}, LdNone{}, 0,
                      OutPartial{dxp, M, in}, 1, true);
        else if (use_big_gemm(M, in))
            rc = dx_big(q, dH, M, ex, KLdx, A, rdx, dX, st);
        else
            rc = gemm(st, M, in, LdRowMajor{dH, M, out, out, dh_vec}, LdNF4Cols{q}, out,
                      LdRowMajor{duext, M, KL, KL, true}, LdDupCols{A, in, r}, KL, OutBF16{dX, in}, 1,
                      true);
        if (rc) return rc;
        if (drop && (rc = dx_dropout_add(dX, dxp, Zdx, du, A, drop->bits, M, in, r, drop->inv_keep, st))) return rc;
    }
    return NF4_OK;
}

int forward_multi_impl(const QView& q, const uint16_t* x, int64_t M, const uint16_t* Ab,
                       const uint16_t* Bb, int n, int r, const float* scales, const int32_t* ids,
                       uint16_t* h, void* ws, size_t ws_bytes, hipStream_t st) {
    const MultiWs lay = multi_ws_offsets(q.rows, q.cols, M, r, n);
    if (ws_bytes < lay.total || !ws) return NF4_EWORKSPACE;
    char* w = static_cast<char*>(ws);
    float* su = reinterpret_cast<float*>(w);
    MultiSort ms{};
    const bool sorted = use_multi_sort(M, n, r) && al16(ws);
    const bool rd = use_rd_grid(M, q.rows) && use_rd(q, M, 0, 0) && al16(Bb) && al16(ws);
    float* sc_ws = reinterpret_cast<float*>(w + lay.sc);
    int rc;
    if (sorted) {  // tokens bucketed by adapter: each adapter's A read once per 16 tokens
        // (the sort's launch also decodes the base product's block scales)
        if ((rc = multi_sort(ids, M, n, w + lay.sort, &ms, st, rd ? &q : nullptr, rd ? sc_ws : nullptr)))
            return rc;
        if ((rc = multi_down_seg(ms, x, q.cols, Ab, r, scales, su, st))) return rc;
    } else {
        hipLaunchKernelGGL(k_multi_down, dim3(unsigned(M)), dim3(256), 0, st, x, q.cols, Ab, n, r,
                           scales, ids, su);
        if (hipPeekAtLastError() != hipSuccess) return launch_status();
    }
    if (rd)
        return forward_rd_multi(q, x, M, su, ids, Bb, n, r, h, sc_ws, reinterpret_cast<float*>(w + lay.part),
                                sorted ? &ms : nullptr, st, sorted);
    LdRowMajor lx{x, M, q.cols, q.cols, al16(x)};
    return gemm(st, M, q.rows, lx, LdNF4Rows{q}, q.cols, LdNone{}, LdNone{}, 0,
                OutMulti{h, q.rows, su, ids, Bb, n, r, q.rows}, 1, true);
}

}  // namespace nf4
