// bwd_small.hip -- the backward of the layer for a few tokens (M <= 16).
//
// dU = s dH B, dB = s dH^T u, dA = dU^T x, dX = dH Wb + dU A (the backward of
// the layer with the dequantized weight a constant, "QLoRA explained", "The
// LoRA adapter path"), for decode-sized M.  The time is in dX, the
// transposed dequant-GEMV over the whole weight; dU rides in the same pass
// over the weight rows (the rank-r slabs below), dB and dA are small fp32
// FMA kernels (a few MFLOP).
//
// dX: the reduction runs down the weight's rows, so the weight is streamed
// row by row exactly as in the forward GEMV, and each lane keeps one fp32
// accumulator per weight column it owns:
//
//   lane l of a wave owns 64-block j = l % 16 of a 16-block slab (1024
//   columns), row lane rs = l / 16.  A workgroup's four waves take rows
//   16i + 4w + rs of its row chunk, so every load instruction reads four
//   rows x 512 contiguous bytes of codes.  Per row, the lane builds the
//   block's 16 products bf16(s~*T[e]) as a table in its own LDS column
//   (slots hold the bf16 in the high half, so a 32-bit read is the value as
//   fp32), then looks up each of its 64 weights and accumulates
//   dH[row]*w with one FMA (the product of two bf16 values is exact in fp32).
//
// At the end of the chunk the four row lanes and the four waves are summed
// in a fixed order and the workgroup writes one fp32 partial of its 1024
// columns; k_dxv_fin adds the chunk partials in a fixed order, adds the
// rank-r term dU A, and rounds to bf16.  Tokens are the fastest-varying workgroup
// index, so the workgroups that read the same weight rows for different
// tokens run together and share the rows through the caches.
#include "nf4_device.h"
#include "nf4_internal.h"

using namespace nf4dev;

namespace {

constexpr int DV_SLAB = 16;  // 64-blocks per slab
constexpr int DV_ROWS = 16;  // rows per workgroup iteration (4 waves x 4 row lanes)

// The rank-r slabs of the same pass: dU partials sum_o dH[o] B[o][j] over
// the chunk's rows, four adapter columns per lane (64 per slab), written
// after the weight columns of the partial row.
__device__ __forceinline__ void bslab_partials(const uint16_t* __restrict__ dht, const uint16_t* __restrict__ B,
                                               int r, int bslab, int64_t row0, int64_t row_end, float* red,
                                               float* __restrict__ prow) {
    const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
    const int j = l & 15, rs = l >> 4;
    const int c0 = bslab * 64 + 4 * j;
    float a[4] = {0.f, 0.f, 0.f, 0.f};
    if ((r & 3) == 0 && (reinterpret_cast<uintptr_t>(B) & 7) == 0) {  // one 8-byte load per row
        const bool cok = c0 < r;
#pragma unroll 4
        for (int64_t o = row0 + 4 * w + rs; o < row_end; o += DV_ROWS) {
            const float d = bf16_f(dht[o]);
            const uint2 bv = cok ? *reinterpret_cast<const uint2*>(B + o * r + c0) : make_uint2(0u, 0u);
            a[0] = __builtin_fmaf(d, bf16_lo(bv.x), a[0]);
            a[1] = __builtin_fmaf(d, bf16_hi(bv.x), a[1]);
            a[2] = __builtin_fmaf(d, bf16_lo(bv.y), a[2]);
            a[3] = __builtin_fmaf(d, bf16_hi(bv.y), a[3]);
        }
    } else {
#pragma unroll 4
        for (int64_t o = row0 + 4 * w + rs; o < row_end; o += DV_ROWS) {
            const float d = bf16_f(dht[o]);
            const uint16_t* br = B + o * r;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (c0 + e < r) a[e] = __builtin_fmaf(d, bf16_f(br[c0 + e]), a[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        a[e] += __shfl_xor(a[e], 16);
        a[e] += __shfl_xor(a[e], 32);
    }
    if (rs == 0)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[w * 64 + 4 * j + e] = a[e];
    __syncthreads();
    if (tid < 64 && bslab * 64 + tid < r)
        prow[bslab * 64 + tid] = ((red[tid] + red[64 + tid]) + red[128 + tid]) + red[192 + tid];
}

template <bool DQ, bool GSH>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_dxv(
    nf4::QView q, const uint16_t* __restrict__ dh, int M, int nslab, int rows_chunk,
    const uint16_t* __restrict__ B, int r, int64_t pstride, float* __restrict__ part) {
    __shared__ __attribute__((aligned(16))) uint32_t tbl[4][16][64];  // [wave][entry][lane]
    __shared__ float q127[256];  // fl32(q/127) for the int8 code q, indexed by its byte
    __shared__ __attribute__((aligned(16))) float red[4][DV_SLAB * 64];  // per-wave column sums
    const int tid = threadIdx.x, l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t N = q.rows, K = q.cols;
    const int nkb = int(K / 64);
    const int nbs = (r + 63) / 64;  // rank-r slabs
    const int nchunk = int((N + rows_chunk - 1) / rows_chunk);
    // XCD-aware order (workgroups are dealt round-robin to the 8 XCDs): each
    // XCD walks a contiguous run of work items, so the slabs of one row
    // chunk share that XCD's L2 for the chunk's scale-code lines.  The grid
    // is padded to a multiple of 8; the padding exits at once.
    const int items = M * (nslab + nbs) * nchunk;
    const int per = int(gridDim.x) / 8;
    const int lin = int(blockIdx.x % 8u) * per + int(blockIdx.x / 8u);
    if (lin >= items) return;
    const int tok = lin % M;
    const int rest = lin / M;
    const int slab = rest % (nslab + nbs), chunk = rest / (nslab + nbs);
    const int64_t row0 = int64_t(chunk) * rows_chunk;
    const int64_t row_end = (row0 + rows_chunk < N) ? row0 + rows_chunk : N;
    float* prow = part + (int64_t(tok) * nchunk + chunk) * pstride;
    if (slab >= nslab) {  // workgroup-uniform
        bslab_partials(dh + int64_t(tok) * N, B, r, slab - nslab, row0, row_end, &red[0][0], prow + K);
        return;
    }
    const int j = l & 15, rs = l >> 4;
    const int blk = slab * DV_SLAB + j;
    const bool blk_ok = blk < nkb;
    const int cb = blk_ok ? blk : nkb - 1;
    const int n_it = int((row_end - row0 + DV_ROWS - 1) / DV_ROWS);

    if (DQ) q127[tid] = q_over_127(int8_t(tid));
    char* tb = reinterpret_cast<char*>(&tbl[0][0][0]);
    char* mine = tb + (w * 16 * 64 + l) * 4;  // slot (w, 0, l); entry stride 256 B
    const uint32_t laneb = uint32_t(l) * 4u;
    const uint32_t P = uint32_t(w) * 0x10101010u;
    uint32_t nmask = 0x0F0F0F0Fu;  // in a VGPR: (c & mask) | P is one v_and_or_b32
    asm volatile("" : "+v"(nmask));

    struct Fetch {  // raw loads only
        uint4 c0, c1;
        uint32_t qb;
        float cg;
        uint32_t dv;
        bool ok;
    };
    // 32-bit byte offsets from wave-uniform bases (the launcher keeps the code
    // array under 4 GB)
    const uint32_t row_bytes = uint32_t(K / 2);
    const uint32_t lane_bytes = uint32_t(cb) * 32u;
    const char* codes = reinterpret_cast<const char*>(q.codes);
    const uint16_t* dht = dh + int64_t(tok) * N;
    auto fetch = [&](int it, Fetch& f) {
        const int64_t row = row0 + DV_ROWS * it + 4 * w + rs;
        const bool rok = row < row_end;
        const uint32_t crow = uint32_t(rok ? row : row_end - 1);
        f.ok = rok && blk_ok;
        const uint32_t off = crow * row_bytes + lane_bytes;
        f.c0 = *reinterpret_cast<const uint4*>(codes + off);
        f.c1 = *reinterpret_cast<const uint4*>(codes + off + 16u);
        const uint32_t b = crow * uint32_t(nkb) + uint32_t(cb);
        if (DQ) {
            const uint32_t gi = GSH ? (b >> q.gshift) : (b / uint32_t(q.group));
            f.qb = uint32_t(uint8_t(q.qcodes[b]));
            f.cg = q.gabs[gi];
        } else {
            f.qb = __builtin_bit_cast(uint32_t, q.absmax[b]);
            f.cg = 0.0f;
        }
        f.dv = dht[crow];
    };

    float acc[64];
#pragma unroll
    for (int c = 0; c < 64; ++c) acc[c] = 0.0f;

    // the levels of the weight's quant type (wave-uniform)
    float lvf[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) lvf[e] = uniform_level(q.qt, e);
    auto process = [&](const Fetch& f) {
        const float sc = DQ ? __fmul_rn(q127[f.qb], f.cg) : bits_f(f.qb);
        const float s = f.ok ? sc : 0.0f;
        // every entry is the slot {0, bf16(s * T[e])}, level 0 included (NaN
        // for the NaN scale of a non-finite block); entries e and e+1 are
        // 256 B apart, so the compiler pairs the stores into ds_write2st64
#pragma unroll
        for (int e = 0; e < 16; ++e) *reinterpret_cast<uint32_t*>(mine + e * 256) = slot_bf16(__fmul_rn(s, lvf[e]));
        const float d = f.ok ? bf16_f(uint16_t(f.dv)) : 0.0f;
        const uint32_t cw[8] = {f.c0.x, f.c0.y, f.c0.z, f.c0.w, f.c1.x, f.c1.y, f.c1.z, f.c1.w};
        // the lookups of code dword st+1 are issued before the FMAs of dword
        // st (the scheduling barriers keep that order and bound the values
        // in flight to two dwords' worth)
        auto look = [&](uint32_t cd, float (&wv)[8]) {
            const uint32_t clo = (cd & nmask) | P;         // odd elements (low nibbles)
            const uint32_t chi = ((cd >> 4) & nmask) | P;  // even elements (high nibbles)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t sel = 0x0C0C0000u | ((4u + t) << 8);
                const uint32_t ah = __builtin_amdgcn_perm(chi, laneb, sel);
                const uint32_t al = __builtin_amdgcn_perm(clo, laneb, sel);
                wv[2 * t] = bits_f(*reinterpret_cast<const uint32_t*>(tb + ah));
                wv[2 * t + 1] = bits_f(*reinterpret_cast<const uint32_t*>(tb + al));
            }
        };
        float wv[2][8];
        look(cw[0], wv[0]);
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            if (st < 7) look(cw[st + 1], wv[(st + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[8 * st + e] = __builtin_fmaf(d, wv[st & 1][e], acc[8 * st + e]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    __syncthreads();  // q127 ready
    // one row in flight ahead of the one being processed (the scheduling
    // barriers keep each row's loads issued a whole row ahead of their use)
    Fetch fa, fb;
    fetch(0, fa);
    int it = 0;
    for (; it + 1 < n_it; it += 2) {
        fetch(it + 1, fb);
        __builtin_amdgcn_sched_barrier(0);
        process(fa);
        fetch(it + 2 < n_it ? it + 2 : it + 1, fa);
        __builtin_amdgcn_sched_barrier(0);
        process(fb);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (it < n_it) process(fa);

    // the four row lanes of each block, then the four waves, in a fixed order
#pragma unroll
    for (int c = 0; c < 64; ++c) {
        acc[c] += __shfl_xor(acc[c], 16);
        acc[c] += __shfl_xor(acc[c], 32);
    }
    if (rs == 0) {
        float4* dst = reinterpret_cast<float4*>(&red[w][64 * j]);
#pragma unroll
        for (int c = 0; c < 16; ++c) dst[c] = make_float4(acc[4 * c], acc[4 * c + 1], acc[4 * c + 2], acc[4 * c + 3]);
    }
    __syncthreads();
    const int cc = 4 * tid;  // four columns of the slab per thread
    const int64_t col = int64_t(slab) * DV_SLAB * 64 + cc;
    if (col < K) {
        const float4 a0 = *reinterpret_cast<const float4*>(&red[0][cc]);
        const float4 a1 = *reinterpret_cast<const float4*>(&red[1][cc]);
        const float4 a2 = *reinterpret_cast<const float4*>(&red[2][cc]);
        const float4 a3 = *reinterpret_cast<const float4*>(&red[3][cc]);
        float4 v;
        v.x = ((a0.x + a1.x) + a2.x) + a3.x;
        v.y = ((a0.y + a1.y) + a2.y) + a3.y;
        v.z = ((a0.z + a1.z) + a2.z) + a3.z;
        v.w = ((a0.w + a1.w) + a2.w) + a3.w;
        *reinterpret_cast<float4*>(prow + col) = v;
    }
}

// dU[m][j] = scale * sum over chunks of part[m][chunk][K + j]: 64 outputs per
// workgroup, sixteen strided chunk groups combined in a fixed order.
__global__ __launch_bounds__(1024) void k_du_fin(const float* __restrict__ part, int nchunk, int64_t K,
                                                 int64_t pstride, int M, int r, float scale,
                                                 float* __restrict__ du) {
    __shared__ float red[16][64];
    const int tid = threadIdx.x, c = tid & 63, g = tid >> 6;
    const int i = blockIdx.x * 64 + c;  // m * r + j
    float a = 0.0f;
    if (i < M * r) {
        const int m = i / r, jj = i % r;
        const float* p = part + int64_t(m) * nchunk * pstride + K + jj;
        for (int ch = g; ch < nchunk; ch += 16) a += p[int64_t(ch) * pstride];
    }
    red[g][c] = a;
    __syncthreads();
    if (tid < 64 && i < M * r) {
        float v = 0.0f;
#pragma unroll
        for (int gg = 0; gg < 16; ++gg) v += red[gg][c];
        du[i] = scale * v;
    }
}

// Per workgroup of 16 columns k: dX[m][k] = bf16( sum over chunks of
// part[m][chunk][k] + sum_j dU[m][j] A[j][k] ) for every token m, and
// dA[j][k] = sum_m dU[m][j] x[m][k].  Narrow column groups keep every
// thread's chain of dependent loads short: 64 chunk groups of 4 column
// quads, then 16 groups of adapter rows, each combined in LDS in a fixed
// order.
constexpr int FIN_COLS = 16;

__global__ __launch_bounds__(256) void k_dxv_fin(const float* __restrict__ part, int nchunk, int64_t K,
                                                 int64_t pstride, int M, const float* __restrict__ du,
                                                 const uint16_t* __restrict__ A, int r,
                                                 const uint16_t* __restrict__ x, uint16_t* __restrict__ dx,
                                                 float* __restrict__ da) {
    __shared__ float4 ps[64][4];
    __shared__ float rk[16][FIN_COLS];
    const int tid = threadIdx.x;
    const int64_t k0 = int64_t(blockIdx.x) * FIN_COLS;
    const int c = tid & 15, g16 = tid >> 4;
    for (int m = 0; m < (dx ? M : 0); ++m) {
        {
            const int cq = tid & 3, g = tid >> 2;
            const float* p = part + int64_t(m) * nchunk * pstride + k0 + 4 * cq;
            float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 2
            for (int ch = g; ch < nchunk; ch += 64) {
                const float4 v = *reinterpret_cast<const float4*>(p + int64_t(ch) * pstride);
                a.x += v.x;
                a.y += v.y;
                a.z += v.z;
                a.w += v.w;
            }
            ps[g][cq] = a;
        }
        {
            const float* dum = du + int64_t(m) * r;
            float a = 0.0f;
#pragma unroll 4
            for (int jj = g16; jj < r; jj += 16) a = __builtin_fmaf(dum[jj], bf16_f(A[int64_t(jj) * K + k0 + c]), a);
            rk[g16][c] = a;
        }
        __syncthreads();
        if (tid < FIN_COLS) {
            const float* pf = reinterpret_cast<const float*>(&ps[0][0]);
            float v = 0.0f;
            for (int g = 0; g < 64; ++g) v += pf[g * FIN_COLS + tid];
            float t = 0.0f;
#pragma unroll
            for (int g = 0; g < 16; ++g) t += rk[g][tid];
            dx[int64_t(m) * K + k0 + tid] = to_bf16(v + t);
        }
        __syncthreads();
    }
    // dA for these columns (x of every token held in registers)
    float xv[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) xv[m] = m < M ? bf16_f(x[int64_t(m) * K + k0 + c]) : 0.0f;
#pragma unroll 4
    for (int jj = g16; jj < r; jj += 16) {
        float a = 0.0f;
#pragma unroll
        for (int m = 0; m < 16; ++m)
            if (m < M) a = __builtin_fmaf(du[int64_t(m) * r + jj], xv[m], a);
        da[int64_t(jj) * K + k0 + c] = a;
    }
}

// dB[o][j] = scale * sum_m dH[m][o] u[m][j], four adapter columns per thread
// (one 16-byte store when r is a multiple of 4)
__global__ __launch_bounds__(256) void k_bs_db(const uint16_t* __restrict__ dh, int M, int64_t out,
                                               const float* __restrict__ u, int r, float scale,
                                               float* __restrict__ db) {
    const int rq = (r + 3) / 4;
    const int64_t n = out * rq;
    const bool vec = (r & 3) == 0 && ((reinterpret_cast<uintptr_t>(u) | reinterpret_cast<uintptr_t>(db)) & 15) == 0;
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
        const int64_t o = i / rq;
        const int j0 = int(i % rq) * 4;
        float a[4] = {0.f, 0.f, 0.f, 0.f};
        for (int m = 0; m < M; ++m) {
            const float d = bf16_f(dh[int64_t(m) * out + o]);
            const float* um = u + int64_t(m) * r + j0;
            if (vec) {
                const float4 uv = *reinterpret_cast<const float4*>(um);
                a[0] = __builtin_fmaf(d, uv.x, a[0]);
                a[1] = __builtin_fmaf(d, uv.y, a[1]);
                a[2] = __builtin_fmaf(d, uv.z, a[2]);
                a[3] = __builtin_fmaf(d, uv.w, a[3]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (j0 + e < r) a[e] = __builtin_fmaf(d, um[e], a[e]);
            }
        }
        float* dst = db + o * r + j0;
        if (vec) {
            *reinterpret_cast<float4*>(dst) = make_float4(scale * a[0], scale * a[1], scale * a[2], scale * a[3]);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (j0 + e < r) dst[e] = scale * a[e];
        }
    }
}

struct DxvPlan {
    int nslab, nchunk, rows_chunk;
};

DxvPlan dxv_plan(int64_t M, int64_t rows, int64_t cols, int r) {
    DxvPlan p{};
    const int64_t nkb = cols / 64;
    p.nslab = int(nf4::cdiv(nkb, DV_SLAB));
    // at most 768 workgroups in all, weight and rank-r slabs (three resident
    // per CU: one pass), whole 16-row steps
    const int64_t want = std::max<int64_t>(1, 768 / (M * (p.nslab + nf4::cdiv(r, 64))));
    const int64_t rc = nf4::cdiv(nf4::cdiv(rows, want), DV_ROWS) * DV_ROWS;
    p.rows_chunk = int(rc);
    p.nchunk = int(nf4::cdiv(rows, rc));
    return p;
}

}  // namespace

namespace nf4 {

bool use_bwd_small(int64_t rows, int64_t cols, int64_t M) {
    return M >= 1 && M <= kBwdSmallMaxM && cols % 64 == 0 && rows * cols / 2 < (int64_t(1) << 32) &&
           rows * (cols / 64) < (int64_t(1) << 32);
}

// partial rows: the weight's columns, then the rank-r slabs
static int64_t part_stride(int64_t cols, int r) { return cols + 64 * cdiv(r, 64); }

size_t bwd_small_ws_bytes(int64_t rows, int64_t cols, int64_t M, int r) {
    if (!use_bwd_small(rows, cols, M)) return 0;
    const DxvPlan p = dxv_plan(M, rows, cols, r);
    return align256(size_t(M) * size_t(p.nchunk) * size_t(part_stride(cols, r)) * 4) + align256(size_t(M) * r * 4);
}

int backward_small(const QView& q, const uint16_t* x, const uint16_t* dH, int64_t M, const uint16_t* A, int r,
                   const uint16_t* B, float scale, const float* u, uint16_t* dX, float* dA, float* dB, char* ws,
                   hipStream_t st) {
    const int64_t out = q.rows, in = q.cols;
    const DxvPlan p = dxv_plan(M, out, in, r);
    const int64_t ps = part_stride(in, r);
    float* part = reinterpret_cast<float*>(ws);
    float* du = reinterpret_cast<float*>(ws + align256(size_t(M) * size_t(p.nchunk) * size_t(ps) * 4));
    // dB = s dH^T u
    launch_before_dominant(k_bs_db, dim3(unsigned(std::min<int64_t>(cdiv(out * cdiv(r, 4), 256), 4096))), dim3(256),
                           0, st, dH, int(M), out, u, r, scale, dB);
    if (hipPeekAtLastError() != hipSuccess) return launch_status();
    // one pass over the weight rows: dX partials (dH Wb) and dU partials (dH
    // B); without dX only the rank-r slabs run
    const int nsl = dX ? p.nslab : 0;
    const dim3 grid(unsigned(cdiv(M * (nsl + cdiv(r, 64)) * p.nchunk, 8) * 8));
    if (q.dq) {
        if (q.gshift >= 0)
            launch_dominant(k_dxv<true, true>, grid, dim3(256), 0, st, q, dH, int(M), nsl, p.rows_chunk, B, r, ps,
                            part);
        else
            launch_dominant(k_dxv<true, false>, grid, dim3(256), 0, st, q, dH, int(M), nsl, p.rows_chunk, B, r, ps,
                            part);
    } else {
        launch_dominant(k_dxv<false, true>, grid, dim3(256), 0, st, q, dH, int(M), nsl, p.rows_chunk, B, r, ps, part);
    }
    if (hipPeekAtLastError() != hipSuccess) return launch_status();
    hipLaunchKernelGGL(k_du_fin, dim3(unsigned(cdiv(M * r, 64))), dim3(1024), 0, st, part, p.nchunk, in, ps, int(M),
                       r, scale, du);
    // dX = sum of the partials + dU A (when asked for), and dA = dU^T x
    hipLaunchKernelGGL(k_dxv_fin, dim3(unsigned(in / FIN_COLS)), dim3(256), 0, st, part, p.nchunk, in, ps, int(M), du,
                       A, r, x, dX, dA);
    return hipPeekAtLastError() == hipSuccess ? NF4_OK : launch_status();
}

}  // namespace nf4
