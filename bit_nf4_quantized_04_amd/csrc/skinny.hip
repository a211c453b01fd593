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

// u = x A^T for M <= 16 tokens, exact fp32 accumulation of bf16 products.
// Workgroup (16 adapter rows) x 16 waves that split K; LDS reduction.
__global__ __launch_bounds__(1024) void k_down_small(const uint16_t* __restrict__ x, int M,
                                                     int64_t K, const uint16_t* __restrict__ A,
                                                     int r, float* __restrict__ u) {
    __shared__ float red[16][16][17];
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int i = l & 15, g = l >> 4;
    const int c = blockIdx.x * 16 + i;  // adapter row of this lane's B column
    const int64_t steps = K / 32;
    const int64_t s0 = steps * w / 16, s1 = steps * (w + 1) / 16;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int64_t s = s0; s < s1; ++s) {
        const int64_t k = s * 32 + g * 8;
        u32x4_t xa = {0u, 0u, 0u, 0u}, ab = {0u, 0u, 0u, 0u};
        if (i < M) xa = *reinterpret_cast<const u32x4_t*>(x + int64_t(i) * K + k);
        if (c < r) ab = *reinterpret_cast<const u32x4_t*>(A + int64_t(c) * K + k);
        acc = mfma16(xa, ab, acc);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) red[w][4 * g + e][i] = acc[e];
    __syncthreads();
    if (threadIdx.x < 256) {
        const int tok = threadIdx.x >> 4, col = threadIdx.x & 15;
        const int cc = blockIdx.x * 16 + col;
        if (tok < M && cc < r) {
            float a = 0.0f;
#pragma unroll
            for (int ww = 0; ww < 16; ++ww) a += red[ww][tok][col];
            u[tok * r + cc] = a;
        }
    }
}

template <bool DQ>
__global__ __launch_bounds__(256) void k_skinny(nf4::QView q, const uint16_t* __restrict__ x, int M,
                                                const float* __restrict__ u, int r,
                                                const uint16_t* __restrict__ B, float scale,
                                                uint16_t* __restrict__ h) {
    // [wave][entry][lane] dword slots; the bf16 entry sits in the low half.
    // Every access is 16-bit typed.
    __shared__ uint16_t tbl[SKW][16][128];
    __shared__ float q127[128];
    __shared__ float red[SKW][16][17];
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int j = l & 15, g = l >> 4;
    const int64_t N = q.rows, K = q.cols, nkb = K / 64;
    const int64_t o0 = int64_t(blockIdx.x) * 16;
    if (DQ && tid < 128) q127[tid] = q_over_127(tid);
    __syncthreads();

    const int64_t row = o0 + j;
    const bool row_ok = row < N;
    const int64_t S = (nkb + 3) / 4;
    const int64_t sb = S * w / SKW, se = S * (w + 1) / SKW;
    // LDS byte address of tbl[w][e][l] = e*256 + w*4096 + l*4: byte 0 is l*4,
    // byte 1 is (w << 4 | e).  P puts w<<4 into every byte of a nibble word.
    const uint32_t laneb = uint32_t(l) * 4u;
    const uint32_t P = uint32_t(w) * 0x10101010u;
    const char* tb = reinterpret_cast<const char*>(&tbl[0][0][0]);

    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int64_t kb = sb; kb < se; ++kb) {
        const int64_t blk = kb * 4 + g;
        const bool ok = row_ok && blk < nkb;
        uint4 c0 = make_uint4(0, 0, 0, 0), c1 = make_uint4(0, 0, 0, 0);
        float s = 0.0f;
        u32x4_t xa[8];
        if (ok) {
            const int64_t e0 = row * K + blk * 64;
            const uint4* cp = reinterpret_cast<const uint4*>(q.codes + (e0 >> 3));
            c0 = cp[0];
            c1 = cp[1];
            const int64_t b = e0 >> 6;
            if (DQ) s = __fmul_rn(q127[q.qcodes[b] & 127], q.gabs[b / q.group]);
            else s = q.absmax[b];
        }
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            xa[st] = u32x4_t{0u, 0u, 0u, 0u};
            if (j < M && blk < nkb)
                xa[st] = *reinterpret_cast<const u32x4_t*>(x + int64_t(j) * K + blk * 64 + st * 8);
        }
        // the block's 16 products, bf16, into this lane's table column
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
            const uint32_t pk = pack_bf16x2(__fmul_rn(s, bits_f(level_bits(e))),
                                            __fmul_rn(s, bits_f(level_bits(e + 1))));
            tbl[w][e][2 * l] = uint16_t(pk);
            tbl[w][e + 1][2 * l] = uint16_t(pk >> 16);
        }
        const uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
        for (int st = 0; st < 8; ++st) {
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
            acc = mfma16(xa[st], bw, acc);
        }
    }
    // lane holds D[token 4g+e][row j]; sum the 4 K quarters in LDS
#pragma unroll
    for (int e = 0; e < 4; ++e) red[w][4 * g + e][j] = acc[e];
    __syncthreads();
    const int i = tid >> 4, jj = tid & 15;
    const int64_t o = o0 + jj;
    if (i < M && o < N) {
        float v = (red[0][i][jj] + red[1][i][jj]) + (red[2][i][jj] + red[3][i][jj]);
        if (r > 0) {
            const float* ui = u + int64_t(i) * r;
            const uint16_t* br = B + o * r;
            float ls = 0.0f;
            if ((r & 7) == 0) {
                for (int c = 0; c < r; c += 8) {
                    const uint4 bv = *reinterpret_cast<const uint4*>(br + c);
                    ls = fmaf(ui[c + 0], bf16_lo(bv.x), ls);
                    ls = fmaf(ui[c + 1], bf16_hi(bv.x), ls);
                    ls = fmaf(ui[c + 2], bf16_lo(bv.y), ls);
                    ls = fmaf(ui[c + 3], bf16_hi(bv.y), ls);
                    ls = fmaf(ui[c + 4], bf16_lo(bv.z), ls);
                    ls = fmaf(ui[c + 5], bf16_hi(bv.z), ls);
                    ls = fmaf(ui[c + 6], bf16_lo(bv.w), ls);
                    ls = fmaf(ui[c + 7], bf16_hi(bv.w), ls);
                }
            } else {
                for (int c = 0; c < r; ++c) ls = fmaf(ui[c], bf16_f(br[c]), ls);
            }
            v += scale * ls;
        }
        h[int64_t(i) * N + o] = to_bf16(v);
    }
}

}  // namespace

namespace nf4 {

size_t skinny_ws_bytes(int64_t M, int r) { return align256(size_t(M) * (r > 0 ? r : 0) * 4); }

int forward_skinny(const QView& q, const uint16_t* x, int64_t M, const uint16_t* A, const uint16_t* B,
                   int r, float scale, uint16_t* h, float* u, hipStream_t st) {
    if (r > 0) {
        hipLaunchKernelGGL(k_down_small, dim3(unsigned(cdiv(r, 16))), dim3(1024), 0, st, x, int(M),
                           q.cols, A, r, u);
        if (hipPeekAtLastError() != hipSuccess) return launch_status();
    }
    const dim3 grid(unsigned(cdiv(q.rows, 16)));
    prof_begin(st);
    if (q.dq)
        hipLaunchKernelGGL(k_skinny<true>, grid, dim3(256), 0, st, q, x, int(M), u, r, B, scale, h);
    else
        hipLaunchKernelGGL(k_skinny<false>, grid, dim3(256), 0, st, q, x, int(M), u, r, B, scale, h);
    prof_end(st);
    return hipPeekAtLastError() == hipSuccess ? NF4_OK : launch_status();
}

}  // namespace nf4
