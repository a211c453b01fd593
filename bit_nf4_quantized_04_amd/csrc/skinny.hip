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
#include <algorithm>
#include <atomic>

#include "nf4_device.h"
#include "nf4_internal.h"

using namespace nf4dev;

namespace {

// k_skinny: waves per workgroup (they split the K range of 16 rows): 4, or 8
// when the weight has too few row tiles for two workgroups per CU
constexpr int SKW = 4;
constexpr int SKW_WIDE = 8;

// Partial down-projections for M <= 16 tokens: part[z][i][c] = sum over the
// z-th K chunk of x[i][k] A[c][k] (bf16 products, fp32 accumulation).  Grid:
// (r/16 adapter-row tiles, DOWN_SPLIT K chunks), 4 waves per workgroup that
// split the chunk further and reduce in LDS.
constexpr int DOWN_SPLIT = 16;

__global__ __launch_bounds__(256) void k_down_small(const uint16_t* __restrict__ x, int M,
                                                    int64_t K, const uint16_t* __restrict__ A,
                                                    int r, float* __restrict__ part) {
    __shared__ float red[4][16][17];
    if (r <= 0) return;
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

// Whether the decode kernel for MT tokens loads its MFMA A fragments (x)
// straight from memory (16 tokens: each lane's eight fragments of a
// block-step are eight 16-byte loads) rather than staging the step's x slice
// through LDS (fewer tokens: one 8-byte load per token per lane).
#ifndef NF4_SKINNY_XDIRECT
#define NF4_SKINNY_XDIRECT 16
#endif
template <int MT>
constexpr bool skinny_xdirect() { return MT >= NF4_SKINNY_XDIRECT; }

// Waves per SIMD the few-token kernel's registers must leave room for: five
// at 2 to 4 tokens (the compiler otherwise takes 100 registers, i.e. four
// waves: 8 % slower on the 70B weight at 4 tokens); no bound at 16 tokens,
// whose x fragments need 144 registers (held to four waves they spill).
template <int MT>
constexpr int skinny_min_waves() { return MT == 4 ? 5 : 1; }

// Shared memory of the decode kernel.
template <int MT, int NWV>
struct SkinnySmem {
    static constexpr bool XS = !skinny_xdirect<MT>();
    // [wave][entry][lane] dword slots; the bf16 entry sits in the low half.
    // Every C++ access is 16-bit typed.  After the main loop the storage
    // holds the cross-wave reduction.
    uint16_t tbl[NWV][16][128];
    uint16_t xs[XS ? NWV : 1][XS ? MT : 1][256];  // x slice of the current block-step, per wave
    float q127[256];  // fl32(q/127) for the int8 code q, indexed by its byte
    float us[16 * 64];  // u for the epilogue (r <= 64 here)
    uint16_t bs[16 * 64];  // the tile's 16 rows of B, for the epilogue
};

// MT = token capacity (1, 4 or 16); the kernel handles any M <= MT.  NWV:
// waves per workgroup.
template <bool DQ, int MT, int NWV>
__global__ __launch_bounds__(64 * NWV) __attribute__((amdgpu_waves_per_eu(skinny_min_waves<MT>()))) void k_skinny(nf4::QView q, const uint16_t* __restrict__ x, int M,
                                                const float* __restrict__ upart, int r,
                                                const uint16_t* __restrict__ B, float scale,
                                                uint16_t* __restrict__ h, float* __restrict__ u_out) {
    __shared__ __attribute__((aligned(16))) SkinnySmem<MT, NWV> sm;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int j = l & 15, g = l >> 4;
    const int64_t N = q.rows, K = q.cols;
    const int nkb = int(K / 64);  // block indices fit in 32 bits (checked by the API)
    const int64_t o0 = int64_t(blockIdx.x) * 16;
    if (DQ && tid < 256) sm.q127[tid] = q_over_127(int8_t(tid));
    // The lookup addresses assume the table starts at LDS offset 0.
    __syncthreads();

    const int S = (nkb + 3) / 4;
    const int sb = S * w / NWV, se = S * (w + 1) / NWV;
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
    // memory -- codes, the block scale, and x: either the step's slice (lane
    // l holds k 4l..4l+3 of every token, staged through LDS) or, direct, the
    // lane's own A fragments (token j, k 64g + 8st .. +7 of the step) -- is
    // fetched one step ahead into a ping-pong buffer.
    constexpr bool XD = skinny_xdirect<MT>();
    struct Fetch {  // raw loads only: nothing here waits for memory
        uint4 c0, c1;
        uint32_t qb;  // int8 scale code (DQ) or the fp32 absmax bits
        float cg;     // group constant (DQ)
        bool ok;
        uint2 xv[XD ? 1 : MT];
        u32x4_t xa[XD ? 8 : 1];
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
        if constexpr (XD) {
            // token j's k chunk g of the step (a block past the end of the row
            // has zero scales for every row: any finite x will do there)
            const int64_t kx = int64_t(blk < nkb ? blk : nkb - 1) * 64;
            const uint16_t* xp = x + int64_t(j < M ? j : 0) * K + kx;
#pragma unroll
            for (int st = 0; st < 8; ++st) {
                f.xa[st] = u32x4_t{0u, 0u, 0u, 0u};
                if (j < M) f.xa[st] = *reinterpret_cast<const u32x4_t*>(xp + st * 8);
            }
        } else {
            int64_t kx = int64_t(kb) * 256 + 4 * l;
            if (kx + 4 > K) kx = K - 4;  // past the end only for zero-scale blocks
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                f.xv[m] = make_uint2(0, 0);
                if (m < M) f.xv[m] = *reinterpret_cast<const uint2*>(x + int64_t(m) * K + kx);
            }
        }
    };

    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    auto process = [&](const Fetch& f) {
        // stage the x slice (this wave only: LDS operations of a wave are in order)
        if constexpr (!XD) {
#pragma unroll
            for (int m = 0; m < MT; ++m)
                if (m < M) *reinterpret_cast<uint2*>(&sm.xs[w][m][4 * l]) = f.xv[m];
        }
        const float sc = DQ ? __fmul_rn(sm.q127[f.qb], f.cg) : bits_f(f.qb);
        const float sblk = f.ok ? sc : 0.0f;
        // the block's 16 products, bf16, into this lane's table column
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
            const uint32_t pk = pack_bf16x2(__fmul_rn(sblk, bits_f(qt_level_bits(q.qt, e))),
                                            __fmul_rn(sblk, bits_f(qt_level_bits(q.qt, e + 1))));
            sm.tbl[w][e][2 * l] = uint16_t(pk);
            sm.tbl[w][e + 1][2 * l] = uint16_t(pk >> 16);
        }
        const uint32_t cw[8] = {f.c0.x, f.c0.y, f.c0.z, f.c0.w, f.c1.x, f.c1.y, f.c1.z, f.c1.w};
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            u32x4_t xa = {0u, 0u, 0u, 0u};  // MFMA rows >= M are never stored
            if constexpr (XD)
                xa = f.xa[st];
            else if (j < M)
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
    // u = sum of the down-projection partials, in a fixed order, and the
    // tile's rows of B, into LDS while the first block-step's loads are in
    // flight (the epilogue reads both after the barriers that follow the
    // main loop)
    for (int idx = tid; idx < 16 * r; idx += 64 * NWV) {
        const int64_t o = o0 + idx / r;
        sm.bs[idx] = o < N ? B[o * r + idx % r] : uint16_t(0);
    }
    for (int idx = tid; idx < M * r; idx += 64 * NWV) {
        float a = 0.0f;
#pragma unroll 4
        for (int zz = 0; zz < DOWN_SPLIT; ++zz) a += upart[int64_t(zz) * M * r + idx];
        sm.us[idx] = a;
        if (blockIdx.x == 0 && u_out) u_out[idx] = a;
    }
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
    // epilogue: output (i, jj) of the tile is finished by 16 lanes that split
    // the rank-r dot product s * u[i] . B[o]
    for (int oi = tid >> 4; oi < M * 16; oi += 4 * NWV) {
        const int i = oi >> 4, jj = oi & 15, sub = tid & 15;
        const int64_t o = o0 + jj;
        float ls = 0.0f;
        if (o < N) {
            const float* ui = &sm.us[i * r];
            const uint16_t* br = &sm.bs[jj * r];
            for (int c = sub; c < r; c += 16) ls = fmaf(ui[c], bf16_f(br[c]), ls);
        }
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) ls += __shfl_xor(ls, off, 16);
        if (sub == 0 && o < N) {
            float v = (red[0][i][jj] + red[1][i][jj]) + (red[2][i][jj] + red[3][i][jj]);
            if constexpr (NWV == 8)
                v += (red[4][i][jj] + red[5][i][jj]) + (red[6][i][jj] + red[7][i][jj]);
            if (r > 0) v += scale * ls;
            h[int64_t(i) * N + o] = to_bf16(v);
        }
    }
}

// v as held by another lane of the same quad (DPP quad_perm: 0x55 reads quad
// position 1, 0xAA position 2, 0xFF position 3), and one lane's v for the
// whole wave
template <int CTRL>
__device__ __forceinline__ float quad_from(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_val(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
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
//
// Table slots are 4 bytes: the low half is zero (written once), the high half
// holds the bf16 product s~*T[e].  A 16-bit read of the high half gives the
// pair {w, 0} and a 32-bit read of the slot gives {0, w}, so the even and the
// odd weights of a code byte form two B operands with no packing instruction;
// the two MFMAs against the same x fragment add both halves of the k range.
//
// The rank-r term s*u.B[o] rides on the same diagonal: lane l < r adds one
// MFMA step whose A fragment is {hi, lo} of s*u[l] (a bf16 pair, so u keeps
// fp32 precision) and whose B fragment is {B[o][l], B[o][l]}.
//
// Work is handed out in chunks of G1_NC rows per wave (a workgroup's four
// waves are R regions x 4/R row subsets of one chunk).  The grid is the number
// of resident workgroups (at most), and workgroup b takes chunks b, b + G,
// b + 2G, ... of the G-strided sequence: neighbouring workgroups stream
// neighbouring rows, and no counter or atomic is involved.
constexpr int G1_NC = 4;  // rows per wave per chunk (and fetch ring slots)
#ifndef NF4_GEMV_NV
#define NF4_GEMV_NV 0
#endif

// SH: log2(block size / 64), 0 or 1 (the scales of 128-element blocks are
// read as they are, one per two of the lanes' 64-element halves).  NV: code
// dwords of each lane's block (of 8) whose weights come from register byte
// planes instead of the LDS table, which moves that share of the lookups
// from the LDS pipe to the VALU.
template <bool DQ, bool GSH, int SH, int NV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_gemv1(
    nf4::QView q, const uint16_t* __restrict__ x, const float* __restrict__ upart, int r,
    const uint16_t* __restrict__ B, float scale, uint16_t* __restrict__ h,
    float* __restrict__ u_out, int R, int nchunks) {
    __shared__ __attribute__((aligned(16))) uint32_t tbl[4][16][64];  // [wave][entry][lane]
    __shared__ float q127[256];  // fl32(q/127) for the int8 code q, indexed by its byte
    __shared__ float dlds[2][4][G1_NC];  // the wave's region sum per (parity, wave, row)
    __shared__ float us[64];
    const int tid = threadIdx.x, l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int N = int(q.rows);  // rows < 2^31 (the launcher checks the code bytes)
    const int nkb = int(q.cols / 64);
    const int S = 4 / R, rows_chunk = S * G1_NC;
    const int rho = w % R, sub = w / R;
    if (DQ) q127[tid] = q_over_127(int8_t(tid));
    char* tb = reinterpret_cast<char*>(&tbl[0][0][0]);
    char* mine = tb + (w * 16 * 64 + l) * 4;  // slot (w, 0, l); entry stride 256 B
    // u = sum of the down-projection partials, in a fixed order
    for (int idx = tid; idx < r; idx += 256) {
        float a = 0.0f;
        for (int zz = 0; zz < DOWN_SPLIT; ++zz) a += upart[int64_t(zz) * r + idx];
        us[idx] = a;
        if (blockIdx.x == 0 && u_out) u_out[idx] = a;
    }

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
    // nibble mask kept in a VGPR so that (c & mask) | P is one v_and_or_b32
    uint32_t nmask = 0x0F0F0F0Fu;
    asm volatile("" : "+v"(nmask));
    DecK dk;
    if constexpr (NV > 0) dk.init();
    const bool lora = r > 0 && rho == 0;  // wave-uniform: region-0 waves add s*u.B
    const bool lane_r = l < r;
    const uint32_t lane_rc = uint32_t(lane_r ? l : 0);  // clamped B column

    struct Fetch {  // raw loads only
        uint4 c0, c1;
        uint32_t qb;
        float cg;
        uint32_t bv;
    };
    // every load is a uniform base plus a 32-bit per-lane byte offset (the
    // launcher keeps the code array under 4 GB)
    const uint32_t row_bytes = uint32_t(q.cols / 2);
    const uint32_t lane_bytes = uint32_t(cb) * 32u;
    const char* codes = reinterpret_cast<const char*>(q.codes);
    // the adapter's B row of the lane (without an adapter the load reads the
    // codes instead: the same load count on every path, the value unused)
    const char* bsrc = lora ? reinterpret_cast<const char*>(B) : codes;
    const uint32_t bstride = lora ? uint32_t(r) * 2u : 0u;
    const uint32_t boff = lora ? lane_rc * 2u : 0u;
    auto fetch = [&](int row, Fetch& f) {  // row: wave-uniform
        const uint32_t crow = uint32_t(row < N ? row : N - 1);
        const uint32_t off = crow * row_bytes + lane_bytes;
        f.c0 = *reinterpret_cast<const uint4*>(codes + off);
        f.c1 = *reinterpret_cast<const uint4*>(codes + off + 16u);
        // the lane's 64-element half-block, and the index of its scale: the
        // block itself, or with blocks of 128 the block holding the half
        const uint32_t b = (crow * uint32_t(nkb) + uint32_t(cb)) >> SH;
        if (DQ) {
            const uint32_t gi = GSH ? (b >> q.gshift) : (b / uint32_t(q.group));
            f.qb = uint32_t(*reinterpret_cast<const uint8_t*>(reinterpret_cast<const char*>(q.qcodes) + b));
            f.cg = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(q.gabs) + (gi << 2));
        } else {
            f.qb = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(q.absmax) + (b << 2));
            f.cg = 0.0f;
        }
        f.bv = *reinterpret_cast<const uint16_t*>(bsrc + (crow * bstride + boff));
    };
    __syncthreads();  // q127, us ready
    // A fragment of the rank-r step: {hi, lo} of s*u[l] in the first dword
    // (zeros after it, so the B fragment may repeat one dword)
    u32x4_t ua = {0u, 0u, 0u, 0u};
    if (lora && lane_r) {
        uint16_t hi, lo;
        split_bf16(__fmul_rn(scale, us[l]), hi, lo);
        ua[0] = uint32_t(hi) | (uint32_t(lo) << 16);
    }

    // the levels of the weight's quant type (wave-uniform)
    float lvf[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) lvf[e] = uniform_level(q.qt, e);
    auto process = [&](const Fetch& f, bool ok, int par, int i) {
        const float sc = DQ ? __fmul_rn(q127[f.qb], f.cg) : bits_f(f.qb);
        const float s = (ok && blk_ok) ? sc : 0.0f;
        // the block's 16 products; the LDS table holds them as {0, v} slots,
        // written two per instruction (entries e and e+1 are 256 B apart)
        // (level 0 included: s * 0 is NaN for the NaN scale of a non-finite block)
        float p[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) p[e] = __fmul_rn(s, lvf[e]);
        if constexpr (NV < 8) {
#pragma unroll
            for (int e = 0; e < 16; ++e) *reinterpret_cast<uint32_t*>(mine + e * 256) = slot_bf16(p[e]);
        }
        Planes pl;
        if constexpr (NV > 0) {
            uint32_t wp[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) wp[k] = pack_bf16x2(p[2 * k], p[2 * k + 1]);
            pl = planes_of_pairs(wp);
        }
        const uint32_t cw[8] = {f.c0.x, f.c0.y, f.c0.z, f.c0.w, f.c1.x, f.c1.y, f.c1.z, f.c1.w};
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        if (lora) {
            uint32_t bv = lane_r ? f.bv * 0x10001u : 0u;  // {B[o][l], B[o][l]}
            const u32x4_t bb = {bv, bv, bv, bv};
            acc = mfma16(ua, bb, acc);
        }
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            const uint32_t cd = cw[st];
            if (st >= 8 - NV) {  // register byte planes: four bf16 pairs, one MFMA
                u32x4_t wv;
                lookup8(dk, pl, cd, wv);
                acc = mfma16(xa[st], wv, acc);
                continue;
            }
            const uint32_t clo = (cd & nmask) | P;         // odd elements (low nibbles)
            const uint32_t chi = ((cd >> 4) & nmask) | P;  // even elements (high nibbles)
            u32x4_t we, wo;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t sel = 0x0C0C0000u | ((4u + t) << 8);
                const uint32_t ah = __builtin_amdgcn_perm(chi, laneb, sel);
                const uint32_t al = __builtin_amdgcn_perm(clo, laneb, sel);
                we[t] = *reinterpret_cast<const uint16_t*>(tb + ah + 2);
                wo[t] = *reinterpret_cast<const uint32_t*>(tb + al);
            }
            acc = mfma16(xa[st], we, acc);
            acc = mfma16(xa[st], wo, acc);
        }
        // the region sum is the trace of D: lane 20g + e holds D[4g+e][4g+e]
        // in acc[e], so the quad at lane 20g gathers its four diagonal
        // entries and the four quads (lanes 0, 20, 40, 60) add up
        const float qd = (acc[0] + quad_from<0x55>(acc[1])) + (quad_from<0xAA>(acc[2]) + quad_from<0xFF>(acc[3]));
        const float t = (lane_val(qd, 0) + lane_val(qd, 20)) + (lane_val(qd, 40) + lane_val(qd, 60));
        if (l == 0) dlds[par][w][i] = t;
    };

    // The wave's rows in order: chunk c contributes rows c*rows_chunk +
    // sub*G1_NC + {0 .. G1_NC-1}, and the chunks are blockIdx.x, +G, +2G, ...
    // A ring of G1_NC fetch slots keeps the next G1_NC - 1 rows in flight
    // while one row is processed (past the end the fetches read the clamped
    // last row, which keeps the load counts of every path equal).  The
    // scheduling barriers keep each row's loads issued that far ahead.
    const int G = int(gridDim.x);
    int c = blockIdx.x;
    auto seq_row = [&](int cc, int j) {  // row j of the ring, counted from chunk cc
        return (cc + (j / G1_NC) * G) * rows_chunk + sub * G1_NC + (j % G1_NC);
    };
    Fetch ring[G1_NC];
#pragma unroll
    for (int j = 0; j < G1_NC - 1; ++j) fetch(seq_row(c, j), ring[j]);
    for (int k = 0; c < nchunks; ++k, c += G) {
#pragma unroll
        for (int i = 0; i < G1_NC; ++i) {
            fetch(seq_row(c, i + G1_NC - 1), ring[(i + G1_NC - 1) % G1_NC]);
            __builtin_amdgcn_sched_barrier(0);
            process(ring[i], seq_row(c, i) < N, k & 1, i);
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
        // finish the chunk's rows: regions summed, in order
        if (tid < rows_chunk) {
            const int sb = tid / G1_NC, i = tid % G1_NC;
            const int o = c * rows_chunk + tid;
            float v = 0.0f;
            for (int rr = 0; rr < R; ++rr) v += dlds[k & 1][sb * R + rr][i];
            if (o < N) h[o] = to_bf16(v);
        }
    }
}

// Resident workgroups of a kernel on the current device (computed once).
template <typename Kern>
int resident_wgs(Kern kernel, int threads, int cache_slot) {
    static std::atomic<int> cache[8];
    int v = cache[cache_slot].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int dev = 0, cus = 0, per = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, threads, 0) != hipSuccess ||
        cus <= 0 || per <= 0) {
        (void)hipGetLastError();
        return 256 * 4;  // a safe guess: it only sizes the work per wave
    }
    v = cus * per;
    cache[cache_slot].store(v, std::memory_order_relaxed);
    return v;
}

}  // namespace

namespace nf4 {

size_t skinny_ws_bytes(int64_t M, int r) {
    // down-projection partials
    return align256(size_t(DOWN_SPLIT) * size_t(M) * (r > 0 ? r : 0) * 4);
}

// The single-token product runs in k_gemv1 (the one kernel here that also
// reads the scales of 128-element blocks directly).
bool gemv1_takes(const QView& q, int64_t M, int r) {
    const int64_t nkb = q.cols / 64;
    // (32-bit byte offsets inside the kernel: codes under 4 GB)
    return M == 1 && r <= kSkinnyMaxR && r <= 64 && nkb <= 256 && q.rows * q.cols / 2 < (int64_t(1) << 32) &&
           q.rows < (int64_t(1) << 31);
}

int forward_skinny(const QView& q, const uint16_t* x, int64_t M, const uint16_t* A, const uint16_t* B,
                   int r, float scale, uint16_t* h, float* u_out, char* ws, hipStream_t st, const uint16_t* xl) {
    float* part = reinterpret_cast<float*>(ws);
    const int64_t nkb = q.cols / 64;
    const int R = nkb <= 64 ? 1 : nkb <= 128 ? 2 : nkb <= 256 ? 4 : 0;
    const bool gemv1 = gemv1_takes(q, M, r);
    if (!gemv1 && q.bshift != 6) return NF4_EINVAL;  // the other kernels take 64-element scales only
    launch_before_dominant(k_down_small, dim3(unsigned(std::max<int64_t>(1, cdiv(r, 16))), DOWN_SPLIT),
                           dim3(256), 0, st, xl ? xl : x, int(M), q.cols, A, r, part);
    if (hipPeekAtLastError() != hipSuccess) return launch_status();
    if (gemv1) {
        const bool b128 = q.bshift == 7;
        constexpr int NV = NF4_GEMV_NV;
        auto kern = b128 ? (q.dq ? (q.gshift >= 0 ? k_gemv1<true, true, 1, NV> : k_gemv1<true, false, 1, NV>)
                                 : k_gemv1<false, true, 1, NV>)
                         : (q.dq ? (q.gshift >= 0 ? k_gemv1<true, true, 0, NV> : k_gemv1<true, false, 0, NV>)
                                 : k_gemv1<false, true, 0, NV>);
        const int slot = (q.dq ? (q.gshift >= 0 ? 0 : 1) : 2) + (b128 ? 3 : 0);
        const int64_t rows_chunk = (4 / R) * G1_NC;
        const int64_t nchunks = cdiv(q.rows, rows_chunk);
        const int64_t grid = std::min<int64_t>(nchunks, resident_wgs(kern, 256, slot));
        launch_dominant(kern, dim3(unsigned(grid)), dim3(256), 0, st, q, x, part, r, B, scale, h,
                        u_out, R, int(nchunks));
        return hipPeekAtLastError() == hipSuccess ? NF4_OK : launch_status();
    }
    const dim3 grid(unsigned(cdiv(q.rows, 16)));
    // fewer row tiles than two per CU: eight waves split each tile's K range
    const bool wide = cdiv(q.rows, 16) < 512;
#define NF4_SKINNY(DQV, MTV)                                                                              \
    (wide ? launch_dominant(k_skinny<DQV, MTV, SKW_WIDE>, grid, dim3(64 * SKW_WIDE), 0, st, q, x, int(M), \
                            part, r, B, scale, h, u_out)                                                  \
          : launch_dominant(k_skinny<DQV, MTV, SKW>, grid, dim3(64 * SKW), 0, st, q, x, int(M), part, r, B,  \
                            scale, h, u_out))
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
