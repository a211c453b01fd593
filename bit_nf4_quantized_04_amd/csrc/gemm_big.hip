// gemm_big.hip -- the large-M fused dequant-GEMM (prefill / training):
// 256 x 256 output tiles, K in steps of 64 (one NF4 block per weight row),
// eight waves of 128 (M) x 64 (N), v_mfma_f32_32x32x16_bf16 with fp32
// accumulation; two waves per SIMD so one wave's loads, dequantization and
// LDS traffic overlap the other's MFMAs.
//
// Layer: h = x Wb^T + s (x A^T) B^T ("QLoRA Finetuner", "1. Low-Rank
// Adaptation"; "QLoRA explained", "The LoRA adapter path"), and the dX
// product dX = dH Wb + dU A of the backward pass (the dequantized weight is a
// constant there, same page).  Wb = bf16(s~ T[code]) is produced tile by tile
// in LDS and never stored to HBM.  The rank-r branch continues the same K loop
// as 2r extra columns ([hi | lo] bf16 split of the fp32 s*u or dU).
//
// Pipeline per K step: the global loads of step k+1 are issued into registers
// before the MFMAs of step k run out of LDS buffer k&1; then step k+1 is
// dequantized/stored into buffer (k+1)&1, and one barrier closes the step.
#include "nf4_device.h"
#include "nf4_internal.h"

using namespace nf4dev;

namespace {

constexpr int TM = 256, TN = 256, TK = 64, TKP = TK + 8;
constexpr int BT = 512;  // threads: 8 waves, 2 per SIMD

typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16_t mfma32(const u32x4_t& a, const u32x4_t& b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                    __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

struct BigSmem {
    uint16_t A[2][TM][TKP];
    uint16_t B[2][TN][TKP];
    // Per-lane 16-entry bf16 product tables of the B producers (waves 0-3):
    // [wave][entry][lane] dword slots, entry in the low half (16-bit typed).
    uint16_t tb[4][16][128];
};

typedef uint16_t (*Tile)[TKP];

// ------------------------------------------------------------------ loaders
// load(): global -> registers for the tile at (row0, k0).  store(): registers
// -> LDS tile [256][TK] (k contiguous), zero outside the operand.

struct NoLoad {
    struct R {};
    __device__ void load(R&, int64_t, int64_t) const {}
    __device__ void store(const R&, Tile, int64_t, int64_t, BigSmem&) const {}
};

// element (row, k) = p[row*ld + k].  Producer waves 4-7: thread 256 + t loads
// row t/8 + 32i (i = 0..7), 16-byte chunk t%8.
struct RowsBF16 {
    const uint16_t* p;
    int64_t rows, K, ld;
    bool vec;  // ld % 8 == 0 and p 16-byte aligned
    struct R { uint4 v[8]; };
    __device__ void load(R& r, int64_t row0, int64_t k0) const {
        if (threadIdx.x < 256) return;  // wave-uniform
        const int t = threadIdx.x - 256, ch = t & 7;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t row = row0 + (t >> 3) + 32 * i, k = k0 + ch * 8;
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
            r.v[i] = v;
        }
    }
    __device__ void store(const R& r, Tile t, int64_t, int64_t, BigSmem&) const {
        if (threadIdx.x < 256) return;
        const int tid = threadIdx.x - 256, ch = tid & 7;
#pragma unroll
        for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(&t[(tid >> 3) + 32 * i][ch * 8]) = r.v[i];
    }
};

// Scale of a block from its raw loads: fl32(fl32(q/127) * c_g) or the fp32 absmax.
__device__ __forceinline__ float blk_scale(const nf4::QView& q, uint32_t qb, float cg) {
    return q.dq ? __fmul_rn(q_over_127(int8_t(qb & 255u)), cg) : __builtin_bit_cast(float, qb);
}


// NF4 weight rows (forward): element (n, k) = Wb[n][k].  Producer waves 0-3:
// thread t < 256 owns the 64-element block of row row0 + t in this K step.
// It writes that block's 16 products bf16(s~ T[c]) to its own table column
// and looks every weight up there (two lookups = one packed bf16 pair), so
// each weight costs about two VALU operations instead of a multiply and a
// conversion.
struct NF4Rows {
    nf4::QView q;
    struct R { uint4 c0, c1; uint32_t qb; float cg; bool ok; };
    __device__ void load(R& r, int64_t row0, int64_t k0) const {
        if (threadIdx.x >= 256) return;  // wave-uniform
        const int64_t row = row0 + threadIdx.x;
        r.ok = row < q.rows;
        const int64_t crow = r.ok ? row : q.rows - 1;
        const int64_t e0 = crow * q.cols + k0;
        const uint4* cp = reinterpret_cast<const uint4*>(q.codes + (e0 >> 3));
        r.c0 = cp[0];
        r.c1 = cp[1];
        const int64_t b = e0 >> 6;
        if (q.dq) {
            r.qb = uint32_t(uint8_t(q.qcodes[b]));
            r.cg = q.gabs[q.gshift >= 0 ? (b >> q.gshift) : (b / q.group)];
        } else {
            r.qb = __builtin_bit_cast(uint32_t, q.absmax[b]);
            r.cg = 0.0f;
        }
    }
    __device__ void store(const R& r, Tile t, int64_t, int64_t, BigSmem& sm) const {
        if (threadIdx.x >= 256) return;  // wave-uniform
        const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
        const float s = r.ok ? blk_scale(q, r.qb, r.cg) : 0.0f;
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
            const uint32_t pk = pack_bf16x2(__fmul_rn(s, bits_f(qt_level_bits(q.qt, e))),
                                            __fmul_rn(s, bits_f(qt_level_bits(q.qt, e + 1))));
            sm.tb[w][e][2 * l] = uint16_t(pk);
            sm.tb[w][e + 1][2 * l] = uint16_t(pk >> 16);
        }
        // byte offset of tb[w][e][l] from tb[0]: e*256 + w*4096 + l*4
        const char* tbase = reinterpret_cast<const char*>(&sm.tb[0][0][0]);
        const uint32_t laneb = uint32_t(l) * 4u, P = uint32_t(w) * 0x10101010u;
        const uint32_t cw[8] = {r.c0.x, r.c0.y, r.c0.z, r.c0.w, r.c1.x, r.c1.y, r.c1.z, r.c1.w};
        uint16_t* dst = &t[threadIdx.x][0];
#pragma unroll
        for (int d = 0; d < 8; d += 2) {
            uint32_t w8[8];
#pragma unroll
            for (int dd = 0; dd < 2; ++dd) {
                const uint32_t cd = cw[d + dd];
                const uint32_t clo = (cd & 0x0F0F0F0Fu) | P;
                const uint32_t chi = ((cd >> 4) & 0x0F0F0F0Fu) | P;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t sel = 0x0C0C0000u | ((4u + j) << 8);
                    const uint32_t vh = *reinterpret_cast<const uint16_t*>(
                        tbase + __builtin_amdgcn_perm(chi, laneb, sel));
                    const uint32_t vl = *reinterpret_cast<const uint16_t*>(
                        tbase + __builtin_amdgcn_perm(clo, laneb, sel));
                    w8[dd * 4 + j] = vh | (vl << 16);
                }
            }
            *reinterpret_cast<uint4*>(dst + d * 8) = make_uint4(w8[0], w8[1], w8[2], w8[3]);
            *reinterpret_cast<uint4*>(dst + d * 8 + 8) = make_uint4(w8[4], w8[5], w8[6], w8[7]);
        }
    }
};

// NF4 weight transposed (dX): tile row n = weight column, k = weight row,
// element (n, k) = Wb[k][n].  Thread t: weight rows k0 + 2(t%32) and +1, and
// two 8-column chunks; it writes (Wb[k][n], Wb[k+1][n])
// pairs, consecutive lanes to consecutive LDS dwords.  (512 threads: chunks
// t/32 + 16i, i = 0..1.)
struct NF4Cols {
    nf4::QView q;
    struct R { uint32_t c[2][2]; uint32_t qb[2][2]; float cg[2][2]; bool ok[2][2]; };
    __device__ void load(R& r, int64_t row0, int64_t k0) const {
        const int kp = threadIdx.x & 31, dc = threadIdx.x >> 5;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int64_t col = row0 + (dc + 16 * i) * 8;
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                const int64_t wr = k0 + 2 * kp + rr;
                const bool ok = col < q.cols && wr < q.rows;
                r.ok[i][rr] = ok;
                const int64_t e0 = (ok ? wr : 0) * q.cols + (ok ? col : 0);
                r.c[i][rr] = q.codes[e0 >> 3];
                const int64_t b = e0 >> 6;
                if (q.dq) {
                    r.qb[i][rr] = uint32_t(uint8_t(q.qcodes[b]));
                    r.cg[i][rr] = q.gabs[q.gshift >= 0 ? (b >> q.gshift) : (b / q.group)];
                } else {
                    r.qb[i][rr] = __builtin_bit_cast(uint32_t, q.absmax[b]);
                    r.cg[i][rr] = 0.0f;
                }
            }
        }
    }
    __device__ void store(const R& r, Tile t, int64_t, int64_t, BigSmem&) const {
        const int kp = threadIdx.x & 31, dc = threadIdx.x >> 5;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            float w[2][8];
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                const float s = r.ok[i][rr] ? blk_scale(q, r.qb[i][rr], r.cg[i][rr]) : 0.0f;
                const uint32_t cd = r.c[i][rr];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    w[rr][2 * j] = __fmul_rn(s, bits_f(qt_level_bits(q.qt, (cd >> (8 * j + 4)) & 15u)));
                    w[rr][2 * j + 1] = __fmul_rn(s, bits_f(qt_level_bits(q.qt, (cd >> (8 * j)) & 15u)));
                }
            }
            const int n0 = (dc + 16 * i) * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                *reinterpret_cast<uint32_t*>(&t[n0 + e][2 * kp]) = pack_bf16x2(w[0][e], w[1][e]);
        }
    }
};

// LoRA extension, forward: element (n, c) = B[n][c mod r] for c < 2r, else 0.
struct DupRows {
    const uint16_t* B;
    int64_t rows;
    int r;
    struct R {};
    __device__ void load(R&, int64_t, int64_t) const {}
    __device__ void store(const R&, Tile t, int64_t row0, int64_t k0, BigSmem&) const {
        const int64_t n = row0 + (threadIdx.x >> 1);
        for (int kk = (threadIdx.x & 1) * 32; kk < (threadIdx.x & 1) * 32 + 32; ++kk) {
            const int64_t c = k0 + kk;
            t[threadIdx.x >> 1][kk] = (n < rows && c < 2 * r) ? B[n * r + (c % r)] : uint16_t(0);
        }
    }
};

// LoRA extension, dX: element (n, c) = A[c mod r][n] for c < 2r, else 0.
struct DupCols {
    const uint16_t* A;
    int64_t cols;
    int r;
    struct R {};
    __device__ void load(R&, int64_t, int64_t) const {}
    __device__ void store(const R&, Tile t, int64_t row0, int64_t k0, BigSmem&) const {
        const int64_t n = row0 + (threadIdx.x >> 1);
        for (int kk = (threadIdx.x & 1) * 32; kk < (threadIdx.x & 1) * 32 + 32; ++kk) {
            const int64_t c = k0 + kk;
            t[threadIdx.x >> 1][kk] = (n < cols && c < 2 * r) ? A[(c % r) * cols + n] : uint16_t(0);
        }
    }
};

// Register staging of the two K phases; one buffer when both phases use the
// same loader type (their live ranges never overlap).
template <class L1, class L2>
struct Staging {
    typename L1::R r1;
    typename L2::R r2;
    __device__ typename L1::R& first() { return r1; }
    __device__ typename L2::R& second() { return r2; }
};
template <class L>
struct Staging<L, L> {
    typename L::R r;
    __device__ typename L::R& first() { return r; }
    __device__ typename L::R& second() { return r; }
};

// ------------------------------------------------------------------ kernel
template <class LA1, class LB1, class LA2, class LB2>
__global__ __launch_bounds__(BT, 1) void k_gemm_big(LA1 la1, LB1 lb1, int64_t K1, LA2 la2, LB2 lb2,
                                                    int64_t K2, uint16_t* __restrict__ out,
                                                    int64_t ldo, int64_t Mr, int64_t Nc) {
    __shared__ __attribute__((aligned(16))) BigSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;  // 2 x 4 waves of 128 x 64

    // XCD-aware tile order: workgroups are dealt round-robin to the 8 XCDs;
    // give each XCD a contiguous run of tiles, walked in groups of 4 M-tiles
    // so neighbouring tiles on one XCD share x rows or W rows in its L2.
    const int64_t nMt = (Mr + TM - 1) / TM, nNt = (Nc + TN - 1) / TN, T = nMt * nNt;
    const int64_t b = blockIdx.x;
    const int64_t lin = (T % 8 == 0) ? (b % 8) * (T / 8) + b / 8 : b;
    const int64_t G = 4;
    const int64_t gsz = G * nNt;
    const int64_t grp = lin / gsz, first = grp * G;
    const int64_t gm = (nMt - first < G) ? (nMt - first) : G;
    const int64_t tm = first + (lin % gsz) % gm, tn = (lin % gsz) / gm;
    const int64_t m0 = tm * TM, n0 = tn * TN;

    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const int64_t S1 = (K1 + TK - 1) / TK, S2 = (K2 + TK - 1) / TK, S = S1 + S2;
    Staging<LA1, LA2> ra;
    Staging<LB1, LB2> rb;
    auto load = [&](int64_t s) {
        if (s < S1) {
            la1.load(ra.first(), m0, s * TK);
            lb1.load(rb.first(), n0, s * TK);
        } else {
            la2.load(ra.second(), m0, (s - S1) * TK);
            lb2.load(rb.second(), n0, (s - S1) * TK);
        }
    };
    auto store = [&](int64_t s, int buf) {
        if (s < S1) {
            la1.store(ra.first(), sm.A[buf], m0, s * TK, sm);
            lb1.store(rb.first(), sm.B[buf], n0, s * TK, sm);
        } else {
            la2.store(ra.second(), sm.A[buf], m0, (s - S1) * TK, sm);
            lb2.store(rb.second(), sm.B[buf], n0, (s - S1) * TK, sm);
        }
    };
    if (S > 0) {
        load(0);
        store(0, 0);
    }
    __syncthreads();
    const int rl = lane & 31, kh = 8 * (lane >> 5);
    auto mfma_k = [&](int buf, int kk) {
        u32x4_t a[4], bb[2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a[i] = *reinterpret_cast<const u32x4_t*>(&sm.A[buf][wm * 128 + i * 32 + rl][kk + kh]);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            bb[j] = *reinterpret_cast<const u32x4_t*>(&sm.B[buf][wn * 64 + j * 32 + rl][kk + kh]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(a[i], bb[j], acc[i][j]);
    };
    // The next step's dequantization and LDS stores are issued between this
    // step's MFMA k-slices so the matrix unit stays busy while they run.
    for (int64_t s = 0; s < S; ++s) {
        const int buf = int(s & 1);
        const bool more = s + 1 < S;
        if (more) load(s + 1);
        mfma_k(buf, 0);
        mfma_k(buf, 16);
        if (more) store(s + 1, buf ^ 1);
        mfma_k(buf, 32);
        mfma_k(buf, 48);
        __syncthreads();
    }
    // D layout of the 32x32 MFMA: lane holds column lane%32 and rows
    // 8*(v/4) + 4*(lane/32) + v%4, v = 0..15.
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t m = m0 + wm * 128 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                const int64_t n = n0 + wn * 64 + j * 32 + (lane & 31);
                if (m < Mr && n < Nc) out[m * ldo + n] = to_bf16(acc[i][j][v]);
            }
}

template <class LA1, class LB1, class LA2, class LB2>
int gemm_big(hipStream_t st, int64_t Mr, int64_t Nc, LA1 la1, LB1 lb1, int64_t K1, LA2 la2, LB2 lb2,
             int64_t K2, uint16_t* out, int64_t ldo) {
    const int64_t T = nf4::cdiv(Mr, TM) * nf4::cdiv(Nc, TN);
    nf4::launch_dominant(k_gemm_big<LA1, LB1, LA2, LB2>, dim3(unsigned(T)), dim3(BT), 0, st, la1, lb1,
                         K1, la2, lb2, K2, out, ldo, Mr, Nc);
    return hipPeekAtLastError() == hipSuccess ? NF4_OK : nf4::launch_status();
}

inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

namespace nf4 {

// The big-tile kernel pays off once the tile grid fills the chip a few times.
bool use_big_gemm(int64_t Mr, int64_t Nc) { return cdiv(Mr, TM) * cdiv(Nc, TN) >= 512; }

int forward_big(const QView& q, const uint16_t* x, int64_t M, const uint16_t* ext, int KL,
                const uint16_t* B, int r, uint16_t* h, hipStream_t st) {
    RowsBF16 lx{x, M, q.cols, q.cols, al16(x)};
    if (r == 0) return gemm_big(st, M, q.rows, lx, NF4Rows{q}, q.cols, NoLoad{}, NoLoad{}, 0, h, q.rows);
    return gemm_big(st, M, q.rows, lx, NF4Rows{q}, q.cols, RowsBF16{ext, M, KL, KL, true},
                    DupRows{B, q.rows, r}, KL, h, q.rows);
}

int dx_big(const QView& q, const uint16_t* dH, int64_t M, const uint16_t* duext, int KL,
           const uint16_t* A, int r, uint16_t* dX, hipStream_t st) {
    const int64_t out = q.rows, in = q.cols;
    RowsBF16 ld{dH, M, out, out, al16(dH) && out % 8 == 0};
    return gemm_big(st, M, in, ld, NF4Cols{q}, out, RowsBF16{duext, M, KL, KL, true},
                    DupCols{A, in, r}, KL, dX, in);
}

}  // namespace nf4
