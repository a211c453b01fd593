// skinny.hip -- decode path (M <= 16 tokens): fused NF4 dequant-GEMV on MFMA.
//
// h = x Wb^T + s u B^T with u = x A^T ("QLoRA Finetuner", "1. Low-Rank
// Adaptation"; "QLoRA explained", "The LoRA adapter path"), Wb = bf16(s~ T[c])
// ("QLoRA Finetuner", section 2, last item; the bf16 cast of "The LoRA
// adapter path").
//
// Layout of the work: v_mfma_f32_16x16x32_bf16 with the tokens as the A rows
// (padded to 16) and 16 weight rows as the B columns.  Lane (j = l%16,
// g = l/16) owns one whole 64-element block of weight row j per block-step
// (4 blocks of a row per step, 256 k); its 8 code dwords feed 8 MFMAs, the
// k order inside the step being permuted identically for x and W.  Because a
// lane owns a block, it builds that block's 16 bf16 products s~*T[c] once and
// keeps them in LDS as a [entry][lane] table: every lookup of a wave hits 64
// distinct banks-by-lane, i.e. no bank conflicts.  Two lookups (high and low
// nibble of a code byte) give one packed bf16 pair, i.e. one MFMA B register.
// The block's weights are read from HBM exactly once, as 2 x 16 B per lane.
#include "nf4_device.h"
#include "nf4_internal.h"

using namespace nf4dev;

namespace {

constexpr int SKW = 4;  // waves per workgroup; they split the K range of 16 rows

// Partial down-projections for M <= 16 tokens: part[z][i][c] = sum over the
// z-th K chunk of x[i][k] A[c][k] (bf16 products, fp32 accumulation).  Grid:
// (r/16 adapter-row tiles, DOWN_SPLIT K chunks), 4 waves per workgroup that
// split the chunk further and reduce in LDS.
constexpr int DOWN_SPLIT = 16;

__global__ __launch_bounds__(256) void k_down_small(const uint16_t* __restrict__ x, int M,
                                                    int64_t K, const uint16_t* __restrict__ A,
                                                    int r, float* __restrict__ part) {
    __shared__ float red[4][16][17];
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int i = l & 15, g = l >> 4;
    const int c = blockIdx.x * 16 + i;  // adapter row of this lane's B column
    const int z = blockIdx.y;
    const int64_t steps = K / 32;
    const int64_t zb = steps * z / DOWN_SPLIT, ze = steps * (z + 1) / DOWN_SPLIT;
    const int64_t s0 = zb + (ze - zb) * w / 4, s1 = zb + (ze - zb) * (w + 1) / 4;
    const uint16_t* xr = x + int64_t(i < M ? i : 0) * K + g * 8;
    const uint16_t* ar = A + int64_t(c < r ? c : 0) * K + g * 8;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    int64_t s = s0;
    for (; s + 4 <= s1; s += 4) {  // four independent loads in flight per lane
        u32x4_t xa[4], ab[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            xa[t] = *reinterpret_cast<const u32x4_t*>(xr + (s + t) * 32);
            ab[t] = *reinterpret_cast<const u32x4_t*>(ar + (s + t) * 32);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) acc = mfma16(xa[t], ab[t], acc);
    }
    for (; s < s1; ++s)
        acc = mfma16(*reinterpret_cast<const u32x4_t*>(xr + s * 32),
                     *reinterpret_cast<const u32x4_t*>(ar + s * 32), acc);
    // rows i >= M and columns c >= r hold clamped-input garbage and are dropped
#pragma unroll
    for (int e = 0; e < 4; ++e) red[w][4 * g + e][i] = acc[e];
    __syncthreads();
    const int tok = threadIdx.x >> 4, col = threadIdx.x & 15;
    const int cc = blockIdx.x * 16 + col;
    if (tok < M && cc < r) {
        const float a = (red[0][tok][col] + red[1][tok][col]) + (red[2][tok][col] + red[3][tok][col]);
        part[(int64_t(z) * M + tok) * r + cc] = a;
    }
}

// Shared memory of the decode kernel.
template <int MT>
struct SkinnySmem {
    // [wave][entry][lane] dword slots; the bf16 entry sits in the low half.
    // Every C++ access is 16-bit typed.  After the main loop the storage
    // holds the cross-wave reduction.
    uint16_t tbl[SKW][16][128];
    uint16_t xs[SKW][MT][256];  // x slice of the current block-step, per wave
    float q127[128];
    float us[16 * 64];  // u for the epilogue (r <= 64 here)
};

// MT = token capacity (1, 4 or 16); the kernel handles any M <= MT.
template <bool DQ, int MT>
__global__ __launch_bounds__(256) void k_skinny(nf4::QView q, const uint16_t* __restrict__ x, int M,
                                                const float* __restrict__ upart, int r,
                                                const uint16_t* __restrict__ B, float scale,
                                                uint16_t* __restrict__ h, float* __restrict__ u_out) {
    __shared__ __attribute__((aligned(16))) SkinnySmem<MT> sm;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int j = l & 15, g = l >> 4;
    const int64_t N = q.rows, K = q.cols;
    const int nkb = int(K / 64);  // block indices fit in 32 bits (checked by the API)
    const int64_t o0 = int64_t(blockIdx.x) * 16;
    if (DQ && tid < 128) sm.q127[tid] = q_over_127(tid);
    // The lookup addresses assume the table starts at LDS offset 0.
    __syncthreads();

    const int S = (nkb + 3) / 4;
    const int sb = S * w / SKW, se = S * (w + 1) / SKW;
    // Branch-free streaming: a lane whose row or block lies outside W reads a
    // clamped, valid block and uses scale 0 (its products vanish).
    const int64_t row = o0 + j;
    const bool row_ok = row < N;
    const int64_t crow = row_ok ? row : N - 1;
    const uint4* cbase = reinterpret_cast<const uint4*>(q.codes) + crow * (K / 32);
    const uint32_t sbase = uint32_t(crow) * uint32_t(nkb);
    const int8_t* qrow = DQ ? q.qcodes + sbase : nullptr;
    const float* arow = DQ ? nullptr : q.absmax + sbase;
    // Byte offset of tbl[w][e][l] = e*256 + w*4096 + l*4: byte 0 is l*4,
    // byte 1 is (w << 4 | e).  P puts w<<4 into every byte of a nibble word.
    const uint32_t laneb = uint32_t(l) * 4u;
    const uint32_t P = uint32_t(w) * 0x10101010u;
    const char* tb = reinterpret_cast<const char*>(&sm.tbl[0][0][0]);

    // One block-step = 4 blocks of 16 rows (256 k).  Everything it needs from
    // memory -- codes, the block scale, the x slice (lane l holds k 4l..4l+3
    // of every token) -- is fetched one step ahead into a ping-pong buffer.
    struct Fetch {  // raw loads only: nothing here waits for memory
        uint4 c0, c1;
        uint32_t qb;  // int8 scale code (DQ) or the fp32 absmax bits
        float cg;     // group constant (DQ)
        bool ok;
        uint2 xv[MT];
    };
    auto fetch = [&](int kb, Fetch& f) {
        const int blk = kb * 4 + g;
        f.ok = row_ok && blk < nkb;
        const int cb = f.ok ? blk : nkb - 1;
        f.c0 = cbase[2 * cb];
        f.c1 = cbase[2 * cb + 1];
        if (DQ) {
            const uint32_t b = sbase + uint32_t(cb);
            const uint32_t gi = q.gshift >= 0 ? (b >> q.gshift) : (b / uint32_t(q.group));
            f.qb = uint32_t(uint8_t(qrow[cb]));
            f.cg = q.gabs[gi];
        } else {
            f.qb = __builtin_bit_cast(uint32_t, arow[cb]);
            f.cg = 0.0f;
        }
        int64_t kx = int64_t(kb) * 256 + 4 * l;
        if (kx + 4 > K) kx = K - 4;  // past the end only for zero-scale blocks
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            f.xv[m] = make_uint2(0, 0);
            if (m < M) f.xv[m] = *reinterpret_cast<const uint2*>(x + int64_t(m) * K + kx);
        }
    };

    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    auto process = [&](const Fetch& f) {
        // stage the x slice (this wave only: LDS operations of a wave are in order)
#pragma unroll
        for (int m = 0; m < MT; ++m)
            if (m < M) *reinterpret_cast<uint2*>(&sm.xs[w][m][4 * l]) = f.xv[m];
        const float sc = DQ ? __fmul_rn(sm.q127[f.qb & 127u], f.cg) : bits_f(f.qb);
        const float sblk = f.ok ? sc : 0.0f;
        // the block's 16 products, bf16, into this lane's table column
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
            const uint32_t pk = pack_bf16x2(__fmul_rn(sblk, bits_f(level_bits(e))),
                                            __fmul_rn(sblk, bits_f(level_bits(e + 1))));
            sm.tbl[w][e][2 * l] = uint16_t(pk);
            sm.tbl[w][e + 1][2 * l] = uint16_t(pk >> 16);
        }
        const uint32_t cw[8] = {f.c0.x, f.c0.y, f.c0.z, f.c0.w, f.c1.x, f.c1.y, f.c1.z, f.c1.w};
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            u32x4_t xa = {0u, 0u, 0u, 0u};  // MFMA rows >= M are never stored
            if (j < M)
                xa = *reinterpret_cast<const u32x4_t*>(&sm.xs[w][j < MT ? j : 0][g * 64 + st * 8]);
            const uint32_t cd = cw[st];
            const uint32_t clo = (cd & 0x0F0F0F0Fu) | P;         // low nibbles: odd elements
            const uint32_t chi = ((cd >> 4) & 0x0F0F0F0Fu) | P;  // high nibbles: even elements
            u32x4_t bw;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t sel = 0x0C0C0000u | ((4u + t) << 8);  // [laneb, byte t, 0, 0]
                const uint32_t ah = __builtin_amdgcn_perm(chi, laneb, sel);
                const uint32_t al = __builtin_amdgcn_perm(clo, laneb, sel);
                const uint32_t vh = *reinterpret_cast<const uint16_t*>(tb + ah);
                const uint32_t vl = *reinterpret_cast<const uint16_t*>(tb + al);
                bw[t] = vh | (vl << 16);
            }
            acc = mfma16(xa, bw, acc);
        }
    };

    Fetch fa, fb;
    if (sb < se) fetch(sb, fa);
    for (int kb = sb; kb < se; kb += 2) {
        if (kb + 1 < se) fetch(kb + 1, fb);
        process(fa);
        if (kb + 1 >= se) break;
        if (kb + 2 < se) fetch(kb + 2, fa);
        process(fb);
    }

    // lane holds D[token 4g+e][row j]; sum the 4 K quarters in LDS (reusing
    // the table storage once every wave is done with it)
    __syncthreads();
    float (*red)[16][17] = reinterpret_cast<float (*)[16][17]>(&sm.tbl[0][0][0]);
#pragma unroll
    for (int e = 0; e < 4; ++e) red[w][4 * g + e][j] = acc[e];
    __syncthreads();
    // u = sum of the down-projection partials, in a fixed order
    for (int idx = tid; idx < M * r; idx += 256) {
        float a = 0.0f;
#pragma unroll 4
        for (int zz = 0; zz < DOWN_SPLIT; ++zz) a += upart[int64_t(zz) * M * r + idx];
        sm.us[idx] = a;
        if (blockIdx.x == 0 && u_out) u_out[idx] = a;
    }
    __syncthreads();
    // epilogue: output (i, jj) of the tile is finished by 16 lanes that split
    // the rank-r dot product s * u[i] . B[o]
    for (int oi = tid >> 4; oi < M * 16; oi += 16) {
        const int i = oi >> 4, jj = oi & 15, sub = tid & 15;
        const int64_t o = o0 + jj;
        float ls = 0.0f;
        if (o < N) {
            const float* ui = &sm.us[i * r];
            const uint16_t* br = B + o * r;
            for (int c = sub; c < r; c += 16) ls = fmaf(ui[c], bf16_f(br[c]), ls);
        }
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) ls += __shfl_xor(ls, off, 16);
        if (sub == 0 && o < N) {
            float v = (red[0][i][jj] + red[1][i][jj]) + (red[2][i][jj] + red[3][i][jj]);
            if (r > 0) v += scale * ls;
            h[int64_t(i) * N + o] = to_bf16(v);
        }
    }
}

// ---------------------------------------------------------------------------
// M = 1: the "diagonal" dequant-GEMV.
//
// A region is 64 consecutive blocks (4096 weights, 2 KB of codes) of one row.
// Lane l owns block l of the region: its two 16-byte code loads make the
// wave read the region's 2 KB contiguously, and it builds the block's own
// 16-entry bf16 table ([entry][lane] in LDS, conflict-free).  In MFMA terms
// lane l is A-row (l%16) and B-column (l%16) with k-chunk l/16, and both the
// A fragment (x at block l) and the B fragment (W at block l) come from the
// same block, so D[i][i] = sum over the 4 lanes {i, i+16, i+32, i+48} of x.w
// over their blocks: the diagonal of D summed over i is the region's dot
// product.  The off-diagonal entries are discarded (M = 1 wastes 15/16 of the
// MFMA either way).  x at the lane's block is loaded once per wave and reused
// for every row the wave visits.
constexpr int G1_ITEMS = 8;  // rows per wave

template <bool DQ, bool GSH>
__global__ __launch_bounds__(256) void k_gemv1(nf4::QView q, const uint16_t* __restrict__ x,
                                               const float* __restrict__ upart, int r,
                                               const uint16_t* __restrict__ B, float scale,
                                               uint16_t* __restrict__ h, float* __restrict__ u_out,
                                               int R) {
    __shared__ __attribute__((aligned(16))) uint16_t tbl[4][16][128];  // [wave][entry][lane]
    __shared__ float q127[128];
    __shared__ float part[4][G1_ITEMS];  // per-wave row partials
    __shared__ float dlds[4][G1_ITEMS][16];  // diagonal D[i][i] per (wave, row, i)
    __shared__ float us[64];
    const int tid = threadIdx.x, l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int64_t N = q.rows, K = q.cols;
    const int nkb = int(K / 64);
    // workgroup: (4 / R) * G1_ITEMS rows; wave w -> region w % R, row subset w / R
    const int rows_wg = (4 / R) * G1_ITEMS;
    const int64_t o0 = int64_t(blockIdx.x) * rows_wg;
    const int rho = w % R, sub = w / R;
    if (DQ && tid < 128) q127[tid] = q_over_127(tid);

    const int blk = rho * 64 + l;  // this lane's block within a row
    const bool blk_ok = blk < nkb;
    const int cb = blk_ok ? blk : nkb - 1;
    // x at this lane's block: 8 fragments of 8 bf16, reused for every row
    u32x4_t xa[8];
    {
        const u32x4_t* xp = reinterpret_cast<const u32x4_t*>(x + int64_t(cb) * 64);
#pragma unroll
        for (int st = 0; st < 8; ++st) xa[st] = xp[st];
    }
    const uint32_t laneb = uint32_t(l) * 4u;
    const uint32_t P = uint32_t(w) * 0x10101010u;
    const char* tb = reinterpret_cast<const char*>(&tbl[0][0][0]);

    struct Fetch {  // raw loads only
        uint4 c0, c1;
        uint32_t qb;
        float cg;
        bool ok;
    };
    // rows of this wave: r0 + it, it < G1_ITEMS (wave-uniform); row pointers
    // advance by one row per item
    const int64_t r0 = o0 + int64_t(sub) * G1_ITEMS;
    const uint4* cp0 = reinterpret_cast<const uint4*>(q.codes) + 2 * int64_t(cb);
    const int64_t row_u4 = K / 32;
    auto fetch = [&](int it, Fetch& f) {
        const int64_t row = r0 + it;
        const bool rok = row < N;  // uniform
        const int64_t crow = rok ? row : N - 1;
        f.ok = blk_ok && rok;
        const uint4* cp = cp0 + crow * row_u4;
        f.c0 = cp[0];
        f.c1 = cp[1];
        const uint32_t b = uint32_t(crow) * uint32_t(nkb) + uint32_t(cb);
        if (DQ) {
            const uint32_t gi = GSH ? (b >> q.gshift) : (b / uint32_t(q.group));
            f.qb = uint32_t(uint8_t(q.qcodes[b]));
            f.cg = q.gabs[gi];
        } else {
            f.qb = __builtin_bit_cast(uint32_t, q.absmax[b]);
            f.cg = 0.0f;
        }
    };
    // the diagonal element held by this lane: D[4(l/16)+e][l%16] with e = l%16 - 4(l/16)
    const int de = (l & 15) - 4 * (l >> 4);
    __syncthreads();  // q127 ready

    auto process = [&](const Fetch& f, int it) {
        const float sc = DQ ? __fmul_rn(q127[f.qb & 127u], f.cg) : bits_f(f.qb);
        const float sblk = f.ok ? sc : 0.0f;
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
            const uint32_t pk = pack_bf16x2(__fmul_rn(sblk, bits_f(level_bits(e))),
                                            __fmul_rn(sblk, bits_f(level_bits(e + 1))));
            tbl[w][e][2 * l] = uint16_t(pk);
            tbl[w][e + 1][2 * l] = uint16_t(pk >> 16);
        }
        const uint32_t cw[8] = {f.c0.x, f.c0.y, f.c0.z, f.c0.w, f.c1.x, f.c1.y, f.c1.z, f.c1.w};
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            const uint32_t cd = cw[st];
            const uint32_t clo = (cd & 0x0F0F0F0Fu) | P;
            const uint32_t chi = ((cd >> 4) & 0x0F0F0F0Fu) | P;
            u32x4_t bw;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t sel = 0x0C0C0000u | ((4u + t) << 8);
                const uint32_t ah = __builtin_amdgcn_perm(chi, laneb, sel);
                const uint32_t al = __builtin_amdgcn_perm(clo, laneb, sel);
                const uint32_t vh = *reinterpret_cast<const uint16_t*>(tb + ah);
                const uint32_t vl = *reinterpret_cast<const uint16_t*>(tb + al);
                bw[t] = vh | (vl << 16);
            }
            acc = mfma16(xa[st], bw, acc);
        }
        float d = 0.0f;
        d = (de == 0) ? acc[0] : d;
        d = (de == 1) ? acc[1] : d;
        d = (de == 2) ? acc[2] : d;
        d = (de == 3) ? acc[3] : d;
        if (de >= 0 && de < 4) dlds[w][it][l & 15] = d;  // the 16 diagonal holders
    };

    // Ping-pong prefetch; the scheduling barriers keep each row's loads issued
    // a whole row ahead of their use (the scheduler would otherwise sink them).
    Fetch fa, fb;
    fetch(0, fa);
#pragma unroll
    for (int it = 0; it < G1_ITEMS; it += 2) {
        fetch(it + 1, fb);
        __builtin_amdgcn_sched_barrier(0);
        process(fa, it);
        if (it + 2 < G1_ITEMS) fetch(it + 2, fa);
        __builtin_amdgcn_sched_barrier(0);
        process(fb, it + 1);
    }
    // row sums of the diagonal values: lanes 0..G1_ITEMS-1 of each wave sum
    // one row's 64 entries in order
    if (l < G1_ITEMS) {
        float v = 0.0f;
        for (int k = 0; k < 16; ++k) v += dlds[w][l][k];
        part[w][l] = v;
    }
    // u = sum of the down-projection partials, in a fixed order
    for (int idx = tid; idx < r; idx += 256) {
        float a = 0.0f;
        for (int zz = 0; zz < DOWN_SPLIT; ++zz) a += upart[int64_t(zz) * r + idx];
        us[idx] = a;
        if (blockIdx.x == 0 && u_out) u_out[idx] = a;
    }
    __syncthreads();
    // epilogue: row (sub, it) = regions summed + s * u . B[o]; 16 lanes per row
    for (int ri = tid >> 4; ri < rows_wg; ri += 16) {
        const int sb2 = ri / G1_ITEMS, it = ri % G1_ITEMS, ln = tid & 15;
        const int64_t o = o0 + ri;
        float ls = 0.0f;
        if (o < N) {
            const uint16_t* br = B + o * r;
            for (int c = ln; c < r; c += 16) ls = fmaf(us[c], bf16_f(br[c]), ls);
        }
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) ls += __shfl_xor(ls, off, 16);
        if (ln == 0 && o < N) {
            float v = 0.0f;
            for (int rr = 0; rr < R; ++rr) v += part[sb2 * R + rr][it];
            if (r > 0) v += scale * ls;
            h[o] = to_bf16(v);
        }
    }
}

}  // namespace

namespace nf4 {

size_t skinny_ws_bytes(int64_t M, int r) {
    return align256(size_t(DOWN_SPLIT) * size_t(M) * (r > 0 ? r : 0) * 4);
}

int forward_skinny(const QView& q, const uint16_t* x, int64_t M, const uint16_t* A, const uint16_t* B,
                   int r, float scale, uint16_t* h, float* u_out, float* part, hipStream_t st) {
    if (r > 0) {
        hipLaunchKernelGGL(k_down_small, dim3(unsigned(cdiv(r, 16)), DOWN_SPLIT), dim3(256), 0, st, x,
                           int(M), q.cols, A, r, part);
        if (hipPeekAtLastError() != hipSuccess) return launch_status();
    }
    const int64_t nkb = q.cols / 64;
    const int R = nkb <= 64 ? 1 : nkb <= 128 ? 2 : nkb <= 256 ? 4 : 0;
    if (M == 1 && R > 0 && r <= 64) {
        const int rows_wg = (4 / R) * G1_ITEMS;
        const dim3 grid1(unsigned(cdiv(q.rows, rows_wg)));
        if (q.dq) {
            if (q.gshift >= 0)
                launch_dominant(k_gemv1<true, true>, grid1, dim3(256), 0, st, q, x, part, r, B, scale, h, u_out, R);
            else
                launch_dominant(k_gemv1<true, false>, grid1, dim3(256), 0, st, q, x, part, r, B, scale, h, u_out, R);
        } else {
            launch_dominant(k_gemv1<false, true>, grid1, dim3(256), 0, st, q, x, part, r, B, scale, h, u_out, R);
        }
        return hipPeekAtLastError() == hipSuccess ? NF4_OK : launch_status();
    }
    const dim3 grid(unsigned(cdiv(q.rows, 16)));
#define NF4_SKINNY(DQV, MTV)                                                                       \
    launch_dominant(k_skinny<DQV, MTV>, grid, dim3(256), 0, st, q, x, int(M), part, r, B, scale, h, \
                    u_out)
    if (q.dq) {
        if (M <= 1) NF4_SKINNY(true, 1);
        else if (M <= 4) NF4_SKINNY(true, 4);
        else NF4_SKINNY(true, 16);
    } else {
        if (M <= 1) NF4_SKINNY(false, 1);
        else if (M <= 4) NF4_SKINNY(false, 4);
        else NF4_SKINNY(false, 16);
    }
#undef NF4_SKINNY
    return hipPeekAtLastError() == hipSuccess ? NF4_OK : launch_status();
}

}  // namespace nf4
