// lora_bwd.hip -- the skinny products of the rank-r branch at large M:
//
//   u  = x A^T                (forward down-projection, [M][r], K = in)
//   dU = s dH B               ([M][r], K = out)
//   dB = s dH^T u             ([out][r], reduction over the M tokens)
//   dA = dU^T x               ([r][in], reduction over the M tokens)
//
// ("QLoRA Finetuner", "1. Low-Rank Adaptation": h = W0 x + (alpha/r) B(A x);
// the gradients are the plain derivative of that forward, and only A and B
// receive them: "QLoRA explained", "The LoRA adapter path".)
//
// All four stream one large bf16 operand (x or dH) against a small one
// (r <= 64 columns), so they are HBM-bound and split their reduction
// across the grid (fp32 partials, summed in a fixed order afterwards).
//
//  * k_nt: both operands contiguous along the reduction (u with A, dU with
//    B^T): MFMA operands are loaded straight from global memory.
//  * k_tn: both operands contiguous across it (dB: dH and u; dA: x and dU):
//    64-token tiles are staged row-major in LDS and read transposed with
//    ds_read_b64_tr_b16 (in each 16-lane group, lane 4e + g addresses row
//    k0 + e, column c0 + 4g; lane 4g + m then receives the four rows' values
//    of column c0 + 4g + m, i.e. four consecutive k of its own column).
//    The fp32 u / dU enter as a bf16 hi + lo pair ([M][128]: hi at column j,
//    lo at 64 + j), so they keep fp32 precision.
#include <algorithm>

#include "nf4_device.h"
#include "nf4_internal.h"

using namespace nf4dev;

namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

__device__ __forceinline__ f32x16_t mfma32(const u32x4_t& a, const u32x4_t& b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                    __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// ------------------------------------------------------------------ k_nt
// part[z][m][j] = sum over k in chunk z of P[m][k] * Q[j][k]; P [M][K],
// Q [J][K] bf16, J <= 16 * NJ, K % 16 == 0, chunks of whole 128-k pieces.
// A workgroup owns 128 rows (wave w: rows 32 w .. 32 w + 31) and one chunk,
// walked in pieces of 128 k that all four waves take together: each wave
// stages its 32 x 128 piece of P in its own LDS tile (four rows of 256
// contiguous bytes per load instruction), and the workgroup stages the
// J x 128 piece of Q once, in a tile all four waves read their MFMA B
// fragments from, so Q crosses the L2 once per 128 rows of P.  16-byte chunk
// c of tile row i is stored at chunk c ^ (i % 16): the stores and the
// fragment reads are free of bank conflicts.  The next piece's loads are
// issued before the current piece's MFMAs (two pieces in flight per lane).
// v_mfma_f32_16x16x32_bf16: lane (i, g) = (lane % 16, lane / 16) holds k
// 8g .. 8g + 7 of a 32-k slice of row (or Q row) i.  Each wave writes the
// fp32 partial of its own rows.  When the splits are a multiple of 8 the
// workgroups that share an XCD (consecutive ids go round the eight XCDs)
// share chunks, so each XCD's L2 holds an eighth of Q while P streams past.
constexpr int NT_ROWS = 128, NT_PIECE = 128;

template <int NJ>
__global__ __launch_bounds__(256) void k_nt(const uint16_t* __restrict__ P, int64_t M, int64_t K,
                                            const uint16_t* __restrict__ Q, int J, int64_t kchunk, int Z,
                                            float* __restrict__ part) {
    __shared__ __attribute__((aligned(16))) uint4 pt[4][32][16];   // per-wave P tiles
    __shared__ __attribute__((aligned(16))) uint4 qt[16 * NJ][16];  // the shared Q tile
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int li = lane & 15, g = lane >> 4;
    const int64_t lin = blockIdx.x;
    int64_t tile;
    int z;
    if ((Z & 7) == 0) {  // XCD lin % 8 takes splits lin % 8 + 8 i
        const int64_t rest = lin >> 3, q = Z >> 3;
        z = int(lin & 7) + 8 * int(rest % q);
        tile = rest / q;
    } else {
        z = int(lin % Z);
        tile = lin / Z;
    }
    const int64_t m0 = tile * NT_ROWS + 32 * w;  // the wave's first row
    const int64_t k0 = int64_t(z) * kchunk, k1 = std::min<int64_t>(K, k0 + kchunk);
    // P loads: instruction t, lane l -> row 4t + l/16 of the wave's 32,
    // 16-byte chunk l % 16 (rows past M read row M - 1; they are not stored)
    const uint16_t* pr = P + 8 * li;
    int64_t roff[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int64_t m = m0 + 4 * t + (lane >> 4);
        roff[t] = (m < M ? m : M - 1) * K;
    }
    // Q loads: instruction u, thread t -> Q row (t + 256 u) / 16, chunk t % 16
    // (rows past J repeat row J - 1; their columns are not stored)
    constexpr int QU = NJ;  // 16 NJ rows x 16 chunks / 256 threads
    const uint16_t* qsrc[QU];
#pragma unroll
    for (int u = 0; u < QU; ++u) {
        const int row = (tid + 256 * u) >> 4;
        qsrc[u] = Q + int64_t(row < J ? row : J - 1) * K + 8 * (tid & 15);
    }
    auto load = [&](int64_t kb, uint4 (&v)[8], uint4 (&qv)[QU]) {
        // zero past K: K % 16 == 0 keeps every 16-byte chunk either whole or
        // wholly past the end
        const bool full = kb + NT_PIECE <= k1;
        const bool pok = full || kb + 8 * li < k1;
#pragma unroll
        for (int t = 0; t < 8; ++t)
            v[t] = pok ? *reinterpret_cast<const uint4*>(pr + roff[t] + kb) : make_uint4(0u, 0u, 0u, 0u);
        const bool qok = full || kb + 8 * (tid & 15) < k1;
#pragma unroll
        for (int u = 0; u < QU; ++u)
            qv[u] = qok ? *reinterpret_cast<const uint4*>(qsrc[u] + kb) : make_uint4(0u, 0u, 0u, 0u);
    };
    f32x4_t acc[2][NJ];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int jb = 0; jb < NJ; ++jb) acc[rb][jb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    uint4 v[8], qv[QU];
    if (k0 < k1) load(k0, v, qv);
    for (int64_t kb = k0; kb < k1; kb += NT_PIECE) {
        __syncthreads();  // every wave is done reading the previous piece's tiles
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int row = 4 * t + (lane >> 4);
            pt[w][row][li ^ (row & 15)] = v[t];
        }
#pragma unroll
        for (int u = 0; u < QU; ++u) {
            const int row = (tid + 256 * u) >> 4, ch = tid & 15;
            qt[row][ch ^ (row & 15)] = qv[u];
        }
        __syncthreads();  // the piece's tiles are in
        if (kb + NT_PIECE < k1) load(kb + NT_PIECE, v, qv);  // the next piece in flight
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) {
            u32x4_t b[NJ];
#pragma unroll
            for (int jb = 0; jb < NJ; ++jb) {
                const int row = 16 * jb + li;
                b[jb] = __builtin_bit_cast(u32x4_t, qt[row][(4 * sl + g) ^ (row & 15)]);
            }
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const int row = 16 * rb + li;
                const u32x4_t a = __builtin_bit_cast(u32x4_t, pt[w][row][(4 * sl + g) ^ (row & 15)]);
#pragma unroll
                for (int jb = 0; jb < NJ; ++jb) acc[rb][jb] = mfma16(a, b[jb], acc[rb][jb]);
            }
        }
    }
    // D layout of the 16x16 MFMA: lane holds column li and rows 4g + e
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int jb = 0; jb < NJ; ++jb) {
            const int j = 16 * jb + li;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t m = m0 + 16 * rb + 4 * g + e;
                if (m < M && j < J) part[(int64_t(z) * M + m) * J + j] = acc[rb][jb][e];
            }
        }
}

// ------------------------------------------------------------------ k_tn
// part[z][R][j] = sum over tokens m in chunk z of P[m][R] * (Qh[m][j] + Ql[m][j])
// with Q2 = [M][128] (hi at j, lo at 64 + j), j < J <= 64.  Block bx owns
// columns R0 = 128 bx .. +127 of P; wave w the 32 of them at 32 w.  Narrow
// column stripes leave room for few token chunks, so the fp32 partials stay
// well below the streamed operand.
constexpr int TN_COLS = 128;
constexpr int TN_PS = TN_COLS + 32;  // LDS row stride of the P tile (elements): 320 bytes
constexpr int TN_QS = 128 + 32;  // of the Q tile: 320 bytes

// Four consecutive k (rows kb + 8(q>>1) + 4h .. +3) of column cb + (lane % 32),
// for h = 0 and 1: the eight k of an MFMA operand fragment.
__device__ __forceinline__ u32x4_t tr_frag(const uint16_t* tile, int stride, int kb, int cb, int lane) {
    const int q = lane >> 4, i = lane & 15;
    const int col = cb + 16 * (q & 1) + 4 * (i & 3);
    const int row = kb + 8 * (q >> 1) + (i >> 2);
    const uint16_t* p0 = tile + row * stride + col;
    const uint16_t* p1 = p0 + 4 * stride;
    const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p0));
    const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p1));
    const uint2 d0 = __builtin_bit_cast(uint2, v0), d1 = __builtin_bit_cast(uint2, v1);
    return u32x4_t{d0.x, d0.y, d1.x, d1.y};
}

__global__ __launch_bounds__(256) void k_tn(const uint16_t* __restrict__ P, int64_t M, int64_t RR,
                                            const uint16_t* __restrict__ Q2, int J, int64_t mchunk,
                                            float* __restrict__ part) {
    __shared__ __attribute__((aligned(16))) uint16_t pt[64 * TN_PS];
    __shared__ __attribute__((aligned(16))) uint16_t qt[64 * TN_QS];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t R0 = int64_t(blockIdx.x) * TN_COLS;
    const int z = blockIdx.y;
    const int64_t m0 = int64_t(z) * mchunk, m1 = std::min<int64_t>(M, m0 + mchunk);
    const bool pvec = RR % 8 == 0;

    // tile loads into registers: P chunk c = tid + 256 i (row c/16, 16-byte
    // chunk c%16), Q chunk c = tid + 256 i (row c/16, chunk c%16); rows past
    // the chunk are zero (they would otherwise count twice)
    uint4 pv[4], qv[4];
    auto load = [&](int64_t mb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i;
            const int64_t mm = mb + (c >> 4), rr = R0 + 8 * (c & 15);
            uint4 v = make_uint4(0, 0, 0, 0);
            if (mm < m1) {
                const uint16_t* src = P + mm * RR + rr;
                if (pvec && rr + 8 <= RR) {
                    v = *reinterpret_cast<const uint4*>(src);
                } else {
                    uint16_t e[8];
#pragma unroll
                    for (int t = 0; t < 8; ++t) e[t] = rr + t < RR ? src[t] : uint16_t(0);
                    v = make_uint4(e[0] | (uint32_t(e[1]) << 16), e[2] | (uint32_t(e[3]) << 16),
                                   e[4] | (uint32_t(e[5]) << 16), e[6] | (uint32_t(e[7]) << 16));
                }
            }
            pv[i] = v;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i;
            const int64_t mm = mb + (c >> 4);
            qv[i] = mm < m1 ? *reinterpret_cast<const uint4*>(Q2 + mm * 128 + 8 * (c & 15)) : make_uint4(0, 0, 0, 0);
        }
    };
    auto store = [&]() {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i;
            *reinterpret_cast<uint4*>(&pt[(c >> 4) * TN_PS + 8 * (c & 15)]) = pv[i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i;
            *reinterpret_cast<uint4*>(&qt[(c >> 4) * TN_QS + 8 * (c & 15)]) = qv[i];
        }
    };

    f32x16_t acc[4];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[f][v] = 0.0f;

    if (m0 < m1) load(m0);
    for (int64_t mb = m0; mb < m1; mb += 64) {
        __syncthreads();  // the previous step's reads are done
        store();
        __syncthreads();
        if (mb + 64 < m1) load(mb + 64);
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) {
            u32x4_t b[4];
            const u32x4_t a = tr_frag(pt, TN_PS, 16 * sl, 32 * w, lane);
#pragma unroll
            for (int f = 0; f < 4; ++f) b[f] = tr_frag(qt, TN_QS, 16 * sl, 32 * f, lane);
#pragma unroll
            for (int f = 0; f < 4; ++f) acc[f] = mfma32(a, b[f], acc[f]);
        }
    }
    // C[R][j] = hi part (frags 0, 1) + lo part (frags 2, 3)
    const int rl = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        const int j = 32 * f + rl;
        if (j >= J) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int64_t R = R0 + 32 * w + 8 * (v >> 2) + 4 * hh + (v & 3);
            if (R < RR) part[(int64_t(z) * RR + R) * J + j] = acc[f][v] + acc[f + 2][v];
        }
    }
}

// The end of dU: du = scale * (sum of the Z partials, in order), and the
// bf16 forms the later products read, all from one pass (r <= 64):
// duext [M][KL] = [hi | lo of du | 0 pad] for the dX rank-r steps, and
// duq / uq [M][128] = hi at column j, lo at 64 + j (zero past r) of du and u.
__global__ __launch_bounds__(256) void k_fin_du(const float* __restrict__ part, int Z, int64_t M, int r,
                                                int KL, float scale, const float* __restrict__ u,
                                                uint16_t* __restrict__ duext, uint16_t* __restrict__ duq,
                                                uint16_t* __restrict__ uq, float* __restrict__ du) {
    const int64_t n = M * 64;
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
        const int64_t m = i >> 6;
        const int j = int(i & 63);
        uint16_t dh = 0, dl = 0, uh = 0, ul = 0;
        if (j < r) {
            float a = 0.0f;
            for (int z = 0; z < Z; ++z) a += part[(int64_t(z) * M + m) * r + j];
            if (du) du[m * r + j] = a * scale;
            split_bf16(a * scale, dh, dl);
            split_bf16(u[m * r + j], uh, ul);
            duext[m * KL + j] = dh;
            duext[m * KL + r + j] = dl;
        }
        if (2 * r + j < KL) duext[m * KL + 2 * r + j] = 0;
        duq[m * 128 + j] = dh;
        duq[m * 128 + 64 + j] = dl;
        uq[m * 128 + j] = uh;
        uq[m * 128 + 64 + j] = ul;
    }
}

// A workgroup takes 64 rows of b (one contiguous slab of 64 r elements),
// transposes them through LDS and writes 64 consecutive elements of each of
// the r rows of bt.  r <= 64.
__device__ __forceinline__ void transpose_tile(const uint16_t* __restrict__ b, int64_t n, int r,
                                               uint16_t* __restrict__ bt, int64_t bx) {
    __shared__ uint16_t tile[64][66];
    const int tid = threadIdx.x;
    const int64_t o0 = bx * 64;
    const int rows = int(n - o0 < 64 ? n - o0 : 64);
    const uint16_t* src = b + o0 * r;
    for (int e = tid; e < rows * r; e += 256) {
        const int o = e / r;
        tile[o][e - o * r] = src[e];
    }
    __syncthreads();
    for (int e = tid; e < r * 64; e += 256) {
        const int j = e >> 6, o = e & 63;
        if (o < rows) bt[int64_t(j) * n + o0 + o] = tile[o][j];
    }
}

__global__ __launch_bounds__(256) void k_transpose16(const uint16_t* __restrict__ b, int64_t n, int r,
                                                     uint16_t* __restrict__ bt) {
    transpose_tile(b, n, r, bt, blockIdx.x);
}

// The transpose (the first gt workgroups) and, in the same launch, the fp32
// block scales fl32(fl32(q_b/127) * c_g) of a double-quantized weight for
// the register-dequant dX product: two independent passes, one launch.
template <bool GSH>
__global__ __launch_bounds__(256) void k_tr_bs(const uint16_t* __restrict__ b, int64_t n, int r,
                                               uint16_t* __restrict__ bt, int gt, nf4::QView q, int64_t nbk,
                                               float* __restrict__ sc) {
    if (int(blockIdx.x) < gt) {
        transpose_tile(b, n, r, bt, blockIdx.x);
        return;
    }
    __shared__ float tab[256];
    block_scales_wg<GSH>(q.qcodes, q.gabs, q.group, q.gshift, nbk, sc, int64_t(blockIdx.x) - gt,
                         int64_t(gridDim.x) - gt, tab);
}

// out[j][i] = scale * sum_z part[z][i][j]  (i < n, j < r): the transposed reduce of dA
__device__ __forceinline__ void reduce_t_tile(const float* __restrict__ part, int Z, int64_t n, int r,
                                              float scale, float* __restrict__ out, int64_t bx, int by) {
    // out[j][i] = scale * sum_z part[z][i][j]; a workgroup takes 16 i x 64 j:
    // partial rows are read along j (contiguous), summed in split order,
    // transposed through LDS and written along i
    __shared__ float tile[16][65];
    const int64_t i0 = bx * 16;
    const int j0 = by * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // 64 x 4
    const int j = j0 + tx;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int ii = ty + 4 * k;
        const int64_t i = i0 + ii;
        float a = 0.0f;
        if (i < n && j < r) {
            const float* p = part + i * r + j;
#pragma unroll 8
            for (int z = 0; z < Z; ++z) a += p[int64_t(z) * n * r];
        }
        tile[ii][tx] = a;
    }
    __syncthreads();
    // 64 j x 16 i outputs: thread (jj, iq) writes i0 + 4iq .. +3 of row j0 + jj
    const int jj = threadIdx.x >> 2, iq = threadIdx.x & 3;
    const int jo = j0 + jj;
    if (jo < r)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t i = i0 + 4 * iq + e;
            if (i < n) out[int64_t(jo) * n + i] = tile[4 * iq + e][jj] * scale;
        }
}

__global__ __launch_bounds__(256) void k_reduce_t(const float* __restrict__ part, int Z, int64_t n, int r,
                                                  float scale, float* __restrict__ out) {
    reduce_t_tile(part, Z, n, r, scale, out, blockIdx.x, int(blockIdx.y));
}

// dB = sb * (the Zb partials [Zb][nb] summed in split order), in the first
// gb workgroups, and the transposed reduce of dA in the rest: one launch.
__global__ __launch_bounds__(256) void k_reduce_pair(const float* __restrict__ pb, int Zb, int64_t nb, float sb,
                                                     float* __restrict__ outb, int gb,
                                                     const float* __restrict__ pa, int Za, int64_t na, int r,
                                                     float sa, float* __restrict__ outa) {
    if (int(blockIdx.x) < gb) {
        for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < nb; i += int64_t(gb) * 256) {
            float a = 0.0f;
            for (int z = 0; z < Zb; ++z) a += pb[int64_t(z) * nb + i];
            outb[i] = a * sb;
        }
        return;
    }
    const int64_t t = int64_t(blockIdx.x) - gb, ti = (na + 15) / 16;
    reduce_t_tile(pa, Za, na, r, sa, outa, t % ti, int(t / ti));
}

unsigned ew(int64_t n) { return unsigned(std::max<int64_t>(1, std::min<int64_t>(8192, (n + 255) / 256))); }

}  // namespace

namespace nf4 {

// Splits of the reduction so that the grid holds about 1024 workgroups.
// Splits of the reduction: one per slab when there are fewer than eight
// slabs, else a multiple of 8 (at least 512 workgroups when the rows allow);
// chunks are whole slabs, and a trailing chunk past K adds zero.
int64_t nt_chunk(int64_t K, int Z) { return cdiv(cdiv(K, Z), NT_PIECE) * NT_PIECE; }
int nt_splits(int64_t M, int64_t K) {
    const int64_t pieces = cdiv(K, NT_PIECE);
    if (pieces < 8) return int(std::max<int64_t>(1, pieces));
    // about one workgroup per CU: a workgroup keeps two pieces of 128 rows in flight
    const int64_t tiles = std::max<int64_t>(1, cdiv(M, NT_ROWS));  // (M = 0: a workspace query)
    const int64_t z = 8 * std::max<int64_t>(1, std::min<int64_t>(cdiv(256, 8 * tiles), pieces / 8));
    return int(cdiv(K, nt_chunk(K, int(z))));  // no empty chunk
}
// Token chunks of the column-stripe products: about 512 workgroups, chunks
// of whole 64-token steps, and no empty chunk.
int64_t tn_chunk(int64_t RR, int64_t M) {
    const int64_t tiles = cdiv(RR, TN_COLS);
    const int64_t z = std::max<int64_t>(1, std::min<int64_t>(cdiv(512, tiles), cdiv(M, 64)));
    return std::max<int64_t>(1, cdiv(cdiv(M, z), 64)) * 64;  // (at least one step: M = 0 in a query)
}
int tn_splits(int64_t RR, int64_t M) { return int(cdiv(M, tn_chunk(RR, M))); }

int nt_product(hipStream_t st, const uint16_t* P, int64_t M, int64_t K, const uint16_t* Q, int J, int Z,
               float* part) {
    if (Z != nt_splits(M, K)) return NF4_EINVAL;
    const int64_t kchunk = nt_chunk(K, Z);
    const int64_t nwg = cdiv(M, NT_ROWS) * Z;
    if (nwg >= (int64_t(1) << 31)) return NF4_ESHAPE;
    const dim3 grid = dim3(unsigned(nwg));
    if (J <= 16)
        hipLaunchKernelGGL(k_nt<1>, grid, dim3(256), 0, st, P, M, K, Q, J, kchunk, Z, part);
    else if (J <= 32)
        hipLaunchKernelGGL(k_nt<2>, grid, dim3(256), 0, st, P, M, K, Q, J, kchunk, Z, part);
    else
        hipLaunchKernelGGL(k_nt<4>, grid, dim3(256), 0, st, P, M, K, Q, J, kchunk, Z, part);
    return hipPeekAtLastError() == hipSuccess ? NF4_OK : launch_status();
}

int tn_product(hipStream_t st, const uint16_t* P, int64_t M, int64_t RR, const uint16_t* Q2, int J, int Z,
               float* part) {
    if (Z != tn_splits(RR, M)) return NF4_EINVAL;
    const int64_t mchunk = tn_chunk(RR, M);
    hipLaunchKernelGGL(k_tn, dim3(unsigned(cdiv(RR, TN_COLS)), unsigned(Z)), dim3(256), 0, st, P, M, RR, Q2, J,
                       mchunk, part);
    return hipPeekAtLastError() == hipSuccess ? NF4_OK : launch_status();
}

int fin_du(hipStream_t st, const float* part, int Z, int64_t M, int r, int KL, float scale, const float* u,
           uint16_t* duext, uint16_t* duq, uint16_t* uq, float* du) {
    hipLaunchKernelGGL(k_fin_du, dim3(ew(M * 64)), dim3(256), 0, st, part, Z, M, r, KL, scale, u, duext, duq, uq, du);
    return hipPeekAtLastError() == hipSuccess ? NF4_OK : launch_status();
}

int transpose16(hipStream_t st, const uint16_t* b, int64_t n, int r, uint16_t* bt) {
    if (r > 64) return NF4_EINVAL;
    hipLaunchKernelGGL(k_transpose16, dim3(unsigned(cdiv(n, 64))), dim3(256), 0, st, b, n, r, bt);
    return hipPeekAtLastError() == hipSuccess ? NF4_OK : launch_status();
}

int transpose_bs(hipStream_t st, const uint16_t* b, int64_t n, int r, uint16_t* bt, const QView& q, float* sc) {
    if (r > 64 || !q.dq) return NF4_EINVAL;
    const int gt = int(cdiv(n, 64));
    const int64_t nbk = q.rows * q.cols / 64;
    const int64_t gs = std::min<int64_t>(cdiv(nbk, 1024), 4096);
    const dim3 grid = dim3(unsigned(gt + gs));
    if (q.gshift >= 0)
        hipLaunchKernelGGL(k_tr_bs<true>, grid, dim3(256), 0, st, b, n, r, bt, gt, q, nbk, sc);
    else
        hipLaunchKernelGGL(k_tr_bs<false>, grid, dim3(256), 0, st, b, n, r, bt, gt, q, nbk, sc);
    return hipPeekAtLastError() == hipSuccess ? NF4_OK : launch_status();
}

int reduce_pair(hipStream_t st, const float* pb, int Zb, int64_t nb, float sb, float* outb, const float* pa, int Za,
                int64_t na, int r, float sa, float* outa) {
    const int gb = int(ew(nb));
    const int64_t ga = cdiv(na, 16) * cdiv(r, 64);
    hipLaunchKernelGGL(k_reduce_pair, dim3(unsigned(gb + ga)), dim3(256), 0, st, pb, Zb, nb, sb, outb, gb, pa, Za, na,
                       r, sa, outa);
    return hipPeekAtLastError() == hipSuccess ? NF4_OK : launch_status();
}

int reduce_t(hipStream_t st, const float* part, int Z, int64_t n, int r, float scale, float* out) {
    hipLaunchKernelGGL(k_reduce_t, dim3(unsigned(cdiv(n, 16)), unsigned(cdiv(r, 64))), dim3(256), 0, st, part, Z, n,
                       r, scale, out);
    return hipPeekAtLastError() == hipSuccess ? NF4_OK : launch_status();
}

}  // namespace nf4
