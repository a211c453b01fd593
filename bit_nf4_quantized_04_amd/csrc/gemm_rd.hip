// gemm_rd.hip -- large-M forward fused dequant-GEMM with the NF4 weight
// dequantized straight into MFMA operand registers.
//
// Layer: h = x Wb^T + s (x A^T) B^T ("QLoRA Finetuner", "1. Low-Rank
// Adaptation"; "QLoRA explained", "The LoRA adapter path"), with
// Wb = bf16(s~ T[code]) ("QLoRA Finetuner", section 2, last item, and the
// bf16 cast of "The LoRA adapter path").
//
// Tiles of 256 tokens x 256 weight rows, K in steps of 64 (one NF4 block per
// weight row).  NW waves (eight, two per SIMD, for the single-adapter
// product; four for the gathered multi-adapter epilogue); wave w owns the
// 256 x (256/NW) slab of weight rows [w 256/NW, (w+1) 256/NW) and its fp32
// accumulator.  v_mfma_f32_32x32x16_bf16: the tokens are the A rows (x tile
// staged in LDS, shared by the waves) and the weight rows the B columns.
//
// The B operand never touches LDS.  In the 32x32x16 layout lane (n, hh)
// (n = lane % 32, hh = lane / 32) supplies 8 k values of column n; here the
// k order inside a 64-block is permuted so that lane hh of slice s holds
// elements 32hh + 8s .. 32hh + 8s + 7 of the block, i.e. one code dword of a
// 16-byte half block (the x tile is read with the same permutation).  The
// lane builds the block's 16 products bf16(fl32(s~ T[e])) once, as eight
// byte planes (low bytes and high bytes of entries 0-3, 4-7, 8-11, 12-15),
// and turns 8 nibbles into 8 bf16 values with byte permutes: two half-table
// selects and a merge on bit 3 per byte plane, then one interleave of low and
// high bytes per bf16 pair.  So each weight costs about three VALU operations
// and no LDS traffic, leaving the LDS to the shared x tile.
//
// The rank-r branch continues the K loop over the [hi | lo] bf16 split of
// s*u (2r columns, zero padded to a multiple of 64) against [B | B], so h is
// written once and u keeps fp32 precision.
//
// Every global read of the K loop is an LDS DMA (a buffer load with the LDS
// bit, on a raw buffer resource per operand), so that all outstanding loads
// are of one kind and a wait count can name exactly the ones a step needs
// (the MUBUF form, not the global one: while a global-segment LDS DMA is in
// flight the compiler treats the LDS wait counter as unordered and waits for
// every outstanding LDS read at each use, so a fragment read issued long
// before its MFMA would still wait for the reads issued after it): the x tile of step t+3 goes into a ring of four shared
// tiles, and each lane's own code half-blocks and fp32 block scales of step
// t+2 into a ring of two per-wave slots.  The block scales are made by a
// small pass before the GEMM (fl32(fl32(q/127) * c_g) per block, the same
// expression as every other dequantization here).
#include <algorithm>

#include "nf4_device.h"
#include "nf4_internal.h"

using namespace nf4dev;

namespace {

constexpr int RM = 256, RN = 256, RKS = 64;
constexpr int RT = 256;  // 4 waves

typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16_t mfma32(const u32x4_t& a, const u32x4_t& b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                    __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// x tile [256 rows][64 k] bf16 in LDS: row-major 128 B rows of eight 16-byte
// chunks, chunk c of row m stored at position c ^ ((m >> 1) & 7).  Sixteen
// consecutive rows then cover all 64 banks once for a given chunk, so both
// the fragment reads and the tile writes are conflict-free.
__device__ __forceinline__ int xpos(int m, int c) { return m * 8 + (c ^ ((m >> 1) & 7)); }

struct FwdArgs {
    const uint8_t* codes;  // [N][K/2]
    const float* scales;   // [N * K / 64] fp32 block scales
    const uint16_t* x;     // [M][K]
    const uint16_t* ext;   // [M][KL] (hi | lo of s*u, zero padded), or null
    const uint16_t* B;     // [N][r]
    uint16_t* h;           // [M][N]
    int64_t M, N, K;
    int KL, r;
    // multi-adapter epilogue (su null: none): h[m][n] += sum_j su[m][j] Bb[ids[m]][n][j]
    const float* su;       // [M][rm] s_id * x A_id^T
    const int32_t* ids;    // [M]; an id outside [0, n_ad) adds nothing
    const uint16_t* Bb;    // [n_ad][N][rm]
    int n_ad, rm;
    // split reduction (gridDim.y > 1): fp32 partials [nsplit][M][N], split z
    // taking weight steps [z*spl, z*spl + spl) (and the rank-r steps if last)
    float* part;
    int spl;
    // tail split (gridDim.y == 1, ztail > 1): the first tfull tiles take the
    // whole reduction; each later tile is split ztail ways (spl_tail steps
    // each) into tile-local fp32 partials [ztail][tile - tfull][RM][RN] at part
    int64_t tfull;
    int ztail, spl_tail;
    int qt;  // quant type of the codes: 0 NF4, 1 FP4
};

// The gathered rank-r term of one output of the multi-adapter forward, fp32
// (id: the token's adapter).
__device__ __forceinline__ float multi_term(const FwdArgs& a, int id, int64_t m, int64_t n) {
    if (id < 0 || id >= a.n_ad) return 0.0f;
    const int rm = a.rm;
    const float* s = a.su + m * rm;
    const uint16_t* b = a.Bb + (int64_t(id) * a.N + n) * rm;
    float l = 0.0f;
    if ((rm & 7) == 0) {  // 16-byte rows of B, 32-byte rows of su (the launcher checks alignment)
        for (int j = 0; j < rm; j += 8) {
            const uint4 bv = *reinterpret_cast<const uint4*>(b + j);
            const float4 s0 = *reinterpret_cast<const float4*>(s + j);
            const float4 s1 = *reinterpret_cast<const float4*>(s + j + 4);
            l = __builtin_fmaf(s0.x, bf16_lo(bv.x), l);
            l = __builtin_fmaf(s0.y, bf16_hi(bv.x), l);
            l = __builtin_fmaf(s0.z, bf16_lo(bv.y), l);
            l = __builtin_fmaf(s0.w, bf16_hi(bv.y), l);
            l = __builtin_fmaf(s1.x, bf16_lo(bv.z), l);
            l = __builtin_fmaf(s1.y, bf16_hi(bv.z), l);
            l = __builtin_fmaf(s1.z, bf16_lo(bv.w), l);
            l = __builtin_fmaf(s1.w, bf16_hi(bv.w), l);
        }
    } else {
        for (int j = 0; j < rm; ++j) l = __builtin_fmaf(s[j], bf16_f(b[j]), l);
    }
    return l;
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer resource over `bytes` bytes at `base` (the launchers keep every
// operand of these kernels under 4 GiB; word 3 selects 32-bit data).
__device__ __forceinline__ rsrc_t rsrc_of(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(uint32_t(bytes)), 0x00020000);
}
// LDS DMA of SZ bytes per lane from byte voff + soff of buffer r; lane l's
// bytes land at dst + SZ l
template <int SZ>
__device__ __forceinline__ void dma(rsrc_t r, uint32_t voff, uint32_t soff, void* dst) {
    static_assert(SZ == 16 || SZ == 4, "16- or 4-byte lanes");
    if constexpr (SZ == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)dst, 16, voff, soff, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)dst, 4, voff, soff, 0, 0);
}

constexpr int XBUF = RM * 8;  // one x tile: 256 rows x 8 chunks of 16 bytes

// The forward kernel's shape for NW waves: wave w owns the 256 x (256/NW)
// slab of weight rows [CPW w, CPW w + CPW), i.e. J = CPW/32 column groups of
// the 32x32 MFMA; each lane DMAs XD 16-byte chunks of every x tile.
template <int NW>
struct FwdShape {
    static constexpr int CPW = RN / NW;
    static constexpr int J = CPW / 32;
    static constexpr int XD = RM * 8 / (64 * NW);
    // per-wave weight slot: codes [j][64 lanes][16 B], then scales [j][64][4 B]
    static constexpr int WSLOT = J * 64 * 16 + J * 64 * 4;
    // DMA instructions per lane: XD per x tile, 2J per weight slot.  Issue
    // order: step t DMAs x tile t+3 in its first slice and weights t+3 in its
    // second.  At the wait in step t's second slice (x tile t+1 and weights
    // t+1 needed) x tile t+2, weights t+2 and x tile t+3 may be in flight.
    static constexpr int VM_XTILE = XD, VM_WSLOT = 2 * J;
    static constexpr int VM_STEP_WAIT = 2 * VM_XTILE + VM_WSLOT;
};

struct Frag { u32x4_t v[8]; };

template <int NW>
struct FwdCtx {
    using Sh = FwdShape<NW>;
    static constexpr int J = Sh::J, XD = Sh::XD, WSLOT = Sh::WSLOT;
    const FwdArgs& a;
    int S1, S;
    int nl, hh, w, lane;
    bool wok[J];
    uint32_t xoff[XD], eoff[XD];  // byte offsets of this lane's x / extension DMA sources
    uint32_t coff[J];             // byte offset of this lane's code half-block, step 0
    uint32_t soff[J];             // byte offset of row j's block scale, step 0
    DecK dk;
    Levels lv;                    // the levels of the codes' quant type
    rsrc_t rx, re, rc, rs;        // buffers: x, the extension, codes, block scales

    // x tile of step s into LDS tile `dst`: DMA instruction i of wave w fills
    // chunk positions 64(XD w + i) .. +63 (one 16-byte chunk per lane).
    __device__ __forceinline__ void xdma(int s, uint4* dst) const {
        const bool main = s < S1;
        const rsrc_t r = main ? rx : re;
        const uint32_t so = uint32_t(main ? s : s - S1) * (RKS * 2);
#pragma unroll
        for (int i = 0; i < XD; ++i) dma<16>(r, main ? xoff[i] : eoff[i], so, dst + 64 * (XD * w + i));
    }
    // this lane's codes and block scales of step s into its wave's slot
    __device__ __forceinline__ void wdma(int s, char* slot) const {
        char* mine = slot + w * WSLOT;
#pragma unroll
        for (int j = 0; j < J; ++j) dma<16>(rc, coff[j], uint32_t(s) * 32, mine + j * 1024);
#pragma unroll
        for (int j = 0; j < J; ++j) dma<4>(rs, soff[j], uint32_t(s) * 4, mine + J * 1024 + j * 256);
    }
    // (a lane whose weight row is past N holds row N-1's codes and scale: its
    // accumulator column is never stored)
    __device__ __forceinline__ void wread(const char* slot, uint4 (&cw)[J], float (&sc)[J]) const {
        const char* mine = slot + w * WSLOT;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            cw[j] = *reinterpret_cast<const uint4*>(mine + j * 1024 + lane * 16);
            const float v = *reinterpret_cast<const float*>(mine + J * 1024 + j * 256 + lane * 4);
            sc[j] = v;
        }
    }
    // A fragments of slice sl: rows 32i + nl, logical chunk 4hh + sl
    __device__ __forceinline__ void aread(const uint4* xb, int sl, Frag& f) const {
#pragma unroll
        for (int i = 0; i < 8; ++i) f.v[i] = __builtin_bit_cast(u32x4_t, xb[xpos(32 * i + nl, 4 * hh + sl)]);
    }
    // rank-r operand: element c of the extension (c < 2r) is B[n][c mod r]
    __device__ __forceinline__ void bload(int s, int64_t row, bool ok, int sl, u32x4_t& out) const {
        const int r = a.r;
        const int c0 = (s - S1) * RKS + 32 * hh + 8 * sl;
        uint16_t e[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int c = c0 + t;
            e[t] = (c < 2 * r && ok) ? a.B[row * r + (c % r)] : uint16_t(0);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) out[t] = uint32_t(e[2 * t]) | (uint32_t(e[2 * t + 1]) << 16);
    }
    __device__ __forceinline__ void lookups(const Planes (&p)[J], const uint4 (&cw)[J], int sl, u32x4_t (&bf)[J]) const {
#pragma unroll
        for (int j = 0; j < J; ++j)
            lookup8(dk, p[j], sl == 0 ? cw[j].x : sl == 1 ? cw[j].y : sl == 2 ? cw[j].z : cw[j].w, bf[j]);
    }
};

template <int J>
__device__ __forceinline__ void mma(f32x16_t (&acc)[8][J], const Frag& af, const u32x4_t (&bf)[J]) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < J; ++j) acc[i][j] = mfma32(af.v[i], bf[j], acc[i][j]);
}

// Interleave the N MFMAs of a slice with the slice's other work: after each
// MFMA one LDS read, up to four VALU operations and one DMA.
template <int N>
__device__ __forceinline__ void interleave() {
#pragma unroll
    for (int k = 0; k < N; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
    }
}

constexpr uint32_t vmcnt_imm(int n) {  // s_waitcnt vmcnt(n), other counters unconstrained
    return uint32_t((n & 15) | (((n >> 4) & 3) << 14) | (0x7 << 4) | (0xf << 8));
}

// One 16-k slice: acc[i][j] += f.v[i] * b[j] for the eight A fragments, each
// MFMA followed by the LDS read of fragment i of the next slice (x tile
// `nb`, slice `nsl`) into the register it frees, so a single set of A
// fragments is live; after each MFMA the schedule places that read, up to
// four VALU operations of the next slice's dequantization and one DMA.
template <int NW, int J>
__device__ __forceinline__ void slice_mma(const FwdCtx<NW>& c, f32x16_t (&acc)[8][J], Frag& f, const u32x4_t (&b)[J],
                                          const uint4* nb, int nsl) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int j = 0; j < J; ++j) acc[i][j] = mfma32(f.v[i], b[j], acc[i][j]);
        f.v[i] = __builtin_bit_cast(u32x4_t, nb[xpos(32 * i + c.nl, 4 * c.hh + nsl)]);
    }
#pragma unroll
    for (int k = 0; k < 8 * J; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        if (k % J == J - 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
    }
}

// One NF4 step t.  x tiles: `cur` = step t, `nxt` = step t+1, `xd` receives
// step t+3.  Weight slot `wn` holds step t+1: it is read in the second slice
// and then receives step t+3 (the other slot holds step t+2).  On entry f/ba
// are slice 0's operands and cw/pl the codes and planes of step t; the step
// builds cwn/pln for step t+1 and leaves f/ba as its slice 0 operands.
template <int NW, int J = FwdShape<NW>::J>
__device__ __forceinline__ void nf4_step(const FwdCtx<NW>& c, int t, const uint4* cur, const uint4* nxt,
                                         uint4* xd, char* wn, f32x16_t (&acc)[8][J], Frag& f,
                                         u32x4_t (&ba)[J], const uint4 (&cw)[J], const Planes (&pl)[J],
                                         uint4 (&cwn)[J], Planes (&pln)[J]) {
    constexpr int VM_STEP_WAIT = FwdShape<NW>::VM_STEP_WAIT;
    u32x4_t bb[J];
    float sc[J];
    // slice 0: slice 1's B operand; DMA the x tile of step t+3
    c.lookups(pl, cw, 1, bb);
    c.xdma(t + 3 < c.S ? t + 3 : c.S - 1, xd);
    slice_mma<NW, J>(c, acc, f, ba, cur, 1);
    // slice 1: this lane's weights of step t+1 (and x tile t+1) complete; they
    // go to registers, the slot receives step t+3's; slice 2's B operand
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(VM_STEP_WAIT));
    c.wread(wn, cwn, sc);
    c.wdma(t + 3 < c.S1 ? t + 3 : c.S1 - 1, wn);
    c.lookups(pl, cw, 2, ba);
    slice_mma<NW, J>(c, acc, f, bb, cur, 2);
    // slice 2: slice 3's B operand, the planes of step t+1 (their scales read
    // a slice earlier)
    c.lookups(pl, cw, 3, bb);
#pragma unroll
    for (int j = 0; j < J; ++j) pln[j] = make_planes(sc[j], c.lv);
    slice_mma<NW, J>(c, acc, f, ba, cur, 3);
    // slice 3: every wave's share of x tile t+1 is in (its fragments are read
    // during this slice); step t+1's first B operand
    __builtin_amdgcn_s_barrier();
    c.lookups(pln, cwn, 0, ba);
    slice_mma<NW, J>(c, acc, f, bb, nxt, 0);
}

// XCD-aware tile order (workgroups are dealt round-robin to the 8 XCDs): a
// run of consecutive `lin` goes to one XCD, and consecutive `lin` walk 4
// token tiles at a time across the output tiles, so neighbouring tiles on
// one XCD share x rows or weight rows in its L2.
__device__ __forceinline__ int64_t xcd_lin(int64_t bid, int64_t T) {
    return (T % 8 == 0) ? (bid % 8) * (T / 8) + bid / 8 : bid;
}
__device__ __forceinline__ void tile_of(int64_t lin, int64_t nMt, int64_t nNt, int64_t& tm, int64_t& tn) {
    const int64_t G = 4, gsz = G * nNt;
    const int64_t grp = lin / gsz, first = grp * G;
    const int64_t gm = (nMt - first < G) ? (nMt - first) : G;
    tm = first + (lin % gsz) % gm;
    tn = (lin % gsz) / gm;
}

template <bool MULTI, int NW>
__global__ __launch_bounds__(64 * NW, 1) void k_fwd_rd(FwdArgs a) {
    using Sh = FwdShape<NW>;
    constexpr int J = Sh::J, CPW = Sh::CPW;
    static_assert(!MULTI || NW == 4, "the gathered epilogue stages 64-column slabs");
    // the ring of x tiles and the two weight slots: separate arrays, so that
    // the compiler can see that a DMA into one never overlaps reads of another
    __shared__ __attribute__((aligned(16))) uint4 xs0[XBUF], xs1[XBUF], xs2[XBUF], xs3[XBUF];
    __shared__ __attribute__((aligned(16))) char wb0[NW * Sh::WSLOT], wb1[NW * Sh::WSLOT];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t N = a.N, K = a.K, M = a.M;

    // the workgroup's tile and its share of the reduction
    const int64_t nMt = (M + RM - 1) / RM, nNt = (N + RN - 1) / RN, T = nMt * nNt;
    const int64_t bid = blockIdx.x;
    int64_t lin, tt = 0;
    int z, nz, spl;
    if (gridDim.y > 1) {  // every tile split
        lin = xcd_lin(bid, T);
        z = int(blockIdx.y);
        nz = int(gridDim.y);
        spl = a.spl;
    } else if (a.ztail <= 1 || bid < a.tfull) {  // whole reduction
        lin = xcd_lin(bid, a.ztail <= 1 ? T : a.tfull);
        z = 0;
        nz = 1;
        spl = int(K / RKS);
    } else {  // a tail tile, split
        tt = (bid - a.tfull) / a.ztail;
        lin = a.tfull + tt;
        z = int((bid - a.tfull) % a.ztail);
        nz = a.ztail;
        spl = a.spl_tail;
    }
    int64_t tm, tn;
    tile_of(lin, nMt, nNt, tm, tn);
    const int64_t m0 = tm * RM, n0 = tn * RN;

    FwdCtx<NW> c{a};
    c.S1 = int(K / RKS);
    c.S = c.S1 + (a.ext ? a.KL / RKS : 0);
    c.nl = lane & 31;
    c.hh = lane >> 5;
    c.w = w;
    c.lane = lane;
    c.dk.init();
    c.lv.init(a.qt);
    c.rx = rsrc_of(a.x, M * K * 2);
    c.re = rsrc_of(a.ext, M * a.KL * 2);
    c.rc = rsrc_of(a.codes, N * K / 2);
    c.rs = rsrc_of(a.scales, N * (K / 64) * 4);
    int64_t wrow[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int64_t rr = n0 + CPW * w + 32 * j + c.nl;
        c.wok[j] = rr < N;
        wrow[j] = c.wok[j] ? rr : N - 1;
        c.coff[j] = uint32_t(wrow[j] * (K / 2) + 16 * c.hh);
        c.soff[j] = uint32_t(wrow[j] * (K / 64) * 4);
    }
#pragma unroll
    for (int i = 0; i < Sh::XD; ++i) {
        const int p = 64 * (Sh::XD * w + i) + lane;  // chunk position this lane's DMA writes
        const int m = p >> 3;
        const int ch = (p & 7) ^ ((m >> 1) & 7);  // logical chunk stored there
        int64_t row = m0 + m;
        row = row < M ? row : M - 1;  // rows past M are computed and dropped
        c.xoff[i] = uint32_t((row * K + 8 * ch) * 2);
        c.eoff[i] = uint32_t((row * a.KL + 8 * ch) * 2);
    }

    f32x16_t acc[8][J];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const int S1 = c.S1, S = c.S;
    const bool last = z == nz - 1;
    const int sb = z * spl;
    const int se = (sb + spl < S1) ? sb + spl : S1;
    // ---- prologue, in the issue order of the steady state: x tile s, then
    // weights s, for s = sb, sb+1, sb+2 (weights sb+2 go into slot 0 once
    // weights sb are in registers)
    c.xdma(sb, xs0);
    c.wdma(sb, wb0);
    c.xdma(sb + 1 < S ? sb + 1 : S - 1, xs1);
    c.wdma(sb + 1 < S1 ? sb + 1 : S1 - 1, wb1);
    c.xdma(sb + 2 < S ? sb + 2 : S - 1, xs2);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * Sh::VM_XTILE + Sh::VM_WSLOT));
    __syncthreads();  // x tile sb and the step-sb weights ready
    uint4 cw[J], cw2[J];
    Planes pl[J], pl2[J];
    {
        float sc[J];
        c.wread(wb0, cw, sc);
        c.wdma(sb + 2 < S1 ? sb + 2 : S1 - 1, wb0);
#pragma unroll
        for (int j = 0; j < J; ++j) pl[j] = make_planes(sc[j], c.lv);
    }
    Frag fa;
    u32x4_t ba[J];
    c.aread(xs0, 0, fa);
    c.lookups(pl, cw, 0, ba);

    // four steps per iteration so every ring index is static (the launcher
    // guarantees S1 % 4 == 0)
    for (int t = sb; t < se; t += 4) {
        nf4_step<NW>(c, t, xs0, xs1, xs3, wb1, acc, fa, ba, cw, pl, cw2, pl2);
        nf4_step<NW>(c, t + 1, xs1, xs2, xs0, wb0, acc, fa, ba, cw2, pl2, cw, pl);
        nf4_step<NW>(c, t + 2, xs2, xs3, xs1, wb1, acc, fa, ba, cw, pl, cw2, pl2);
        nf4_step<NW>(c, t + 3, xs3, xs0, xs2, wb0, acc, fa, ba, cw2, pl2, cw, pl);
    }

    // ---- rank-r steps (at most three, all already DMA'd): x tile from the
    // ring, the B operand gathered from global memory
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int s = S1; s < (last ? S : S1); ++s) {
        const int k = s & 3;
        const uint4* tl = k == 0 ? xs0 : k == 1 ? xs1 : k == 2 ? xs2 : xs3;
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) {
            Frag f;
            u32x4_t bf[J];
            c.aread(tl, sl, f);
#pragma unroll
            for (int j = 0; j < J; ++j) c.bload(s, wrow[j], c.wok[j], sl, bf[j]);
            mma<J>(acc, f, bf);
        }
    }

    // D layout of the 32x32 MFMA: lane holds column lane%32 and rows
    // 8*(v/4) + 4*(lane/32) + v%4, v = 0..15.
    if (nz > 1 && gridDim.y == 1) {  // a split tail tile: tile-local fp32 partials
        float* pz = a.part + (int64_t(z) * (T - a.tfull) + tt) * (RM * RN);
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int ln = CPW * w + 32 * j + c.nl;
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) pz[(32 * i + 8 * (v >> 2) + 4 * c.hh + (v & 3)) * RN + ln] = acc[i][j][v];
        }
    } else if (gridDim.y > 1) {  // one split of the reduction: fp32 partials
        float* pz = a.part + int64_t(z) * M * N;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int64_t n = n0 + CPW * w + 32 * j + c.nl;
            if (n >= N) continue;
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int64_t m = m0 + 32 * i + 8 * (v >> 2) + 4 * c.hh + (v & 3);
                    if (m < M) pz[m * N + n] = acc[i][j][v];
                }
        }
    } else if constexpr (!MULTI) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int64_t n = n0 + CPW * w + 32 * j + c.nl;
            if (n >= N) continue;
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int64_t m = m0 + 32 * i + 8 * (v >> 2) + 4 * c.hh + (v & 3);
                    if (m < M) a.h[m * N + n] = to_bf16(acc[i][j][v]);
                }
        }
    } else {
        // Gathered rank-r term: each 32-row slab of the wave's accumulators
        // goes through LDS (the x ring is free now), then lane l finishes
        // column 64w + l row by row, so the token's id and su row are
        // wave-uniform and the B_id rows are read contiguously.
        __syncthreads();  // every wave is past its last read of the x ring
        float* stg = reinterpret_cast<float*>(xs0) + w * (32 * 64);
        const int64_t n = n0 + 64 * w + lane;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
            for (int j = 0; j < J; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    stg[(8 * (v >> 2) + 4 * c.hh + (v & 3)) * 64 + 32 * j + c.nl] = acc[i][j][v];
            // the slab's 32 ids, one per lane, read back wave-uniform
            const int64_t mi = m0 + 32 * i + (lane & 31);
            const int idv = mi < M ? a.ids[mi] : -1;
#pragma unroll 8
            for (int rr = 0; rr < 32; ++rr) {
                const int64_t m = m0 + 32 * i + rr;
                const int id = __builtin_amdgcn_readlane(idv, rr);
                if (m < M && n < N) a.h[m * N + n] = to_bf16(stg[rr * 64 + lane] + multi_term(a, id, m, n));
            }
        }
    }
}

// ------------------------------------------------------------------ dX
// dX = dH Wb + [dU_hi | dU_lo] [A; A]  (the backward of the same layer; the
// dequantized weight is a constant there, "QLoRA explained", "The LoRA
// adapter path").  Tiles of 256 tokens x 256 input features, K = out in
// steps of 32 weight rows.  Eight waves, two per SIMD: waves w and w + 4 own
// the 128 x 64 slabs of columns [64w, 64w + 64), rows [0, 128) and
// [128, 256); waves 0-3 also issue the DMAs and dequantize (the same work
// per thread as with four waves), waves 4-7 only multiply, so that one
// wave's dequantization overlaps the other's MFMAs on the same SIMD.  (The
// four-wave form, one 256 x 64 slab per wave with its accumulator in AGPRs,
// remains as a build option.)
//
// Here the reduction runs across weight rows, so the weight is dequantized
// in its natural layout: thread t makes 32 consecutive columns (half an NF4
// block) of one weight row with the byte-plane lookup and writes them to a
// row-major LDS tile; the MFMA B operand is read from that tile transposed
// with ds_read_b64_tr_b16 (in each 16-lane group lane 4e + g addresses row
// k0 + e, column c0 + 4g, and lane 4g + m receives column c0 + 4g + m of
// those four rows: four consecutive k of one column).  The dH tile (A
// operand) and each thread's own codes and block scale come by DMA into a
// ring of four LDS buffers (one per step: the dH tile, then the staging), so
// the K loop issues no other global load and its wait counts name exactly
// the DMAs a step needs.
constexpr int DK = 32;                   // weight rows per K step
constexpr int DHBUF = RM * 4;            // dH tile: 256 rows x 4 chunks of 16 bytes
constexpr int WTS = 256 + 32;            // W tile row stride (elements), 576 bytes
constexpr int WTBUF = DK * WTS;          // W tile (elements)
constexpr int DSLOT = 64 * 16 + 64 * 4;  // staging per wave: codes, then the scale
constexpr int DXBUF = DHBUF + 4 * DSLOT / 16;  // one ring buffer (uint4): dH tile, staging
constexpr int DX_VM_STEP = 6;            // DMAs per thread per step: 4 dH, 2 staging

struct DxArgs {
    const uint8_t* codes;  // [out][in/2]
    const float* scales;   // [out * in / 64]
    const uint16_t* dh;    // [M][out]
    const uint16_t* ext;   // [M][KL] (dU hi | lo), or null
    const uint16_t* A;     // [r][in]
    uint16_t* dx;          // [M][in] (one split)
    float* part;           // [nsplit][M][in] fp32 partials (several splits)
    int64_t M, out, in;
    int KL, r;
    int spl;               // weight-row steps per split (a multiple of four)
    int f32;               // nonzero: fp32 partials even for one split
    int qt;                // quant type of the codes: 0 NF4, 1 FP4
};

// W tile layout: row-major with a 576-byte row stride, and the 16-byte chunk
// cc (8 weights) of row `row` stored at position cc ^ wt_swizzle(row, cc).
// The XOR touches the two low bits of cc only and depends on row mod 4 and
// bit 4 of cc, so moving 4 or 16 rows or 4 chunks (32 columns) moves the
// address by a constant (the transposed reads use immediate offsets), while
// the dequantizing threads' 16-byte stores (a 16-lane group: two rows, eight
// chunk positions) and the transposed 8-byte reads both hit 64 distinct
// banks.
__device__ __forceinline__ int wt_swizzle(int row, int cc) { return (row + 2 * ((cc >> 4) & 1)) & 3; }

// dH tile layout: row m of 4 chunks, chunk c stored at c ^ ((m >> 2) & 3)
// (sixteen consecutive rows then hit sixteen distinct bank groups)
__device__ __forceinline__ int dpos(int m, int c) { return m * 4 + (c ^ ((m >> 2) & 3)); }

struct DxCtx {
    const DxArgs& a;
    int S1, S;
    int w, lane, tid;
    uint32_t hoff[4], eoff[4];  // byte offsets of this lane's dH / extension DMA sources
    uint32_t coff;              // byte offset of this thread's code half-block, step 0
    uint32_t soff;              // byte offset of its block scale, step 0
    uint32_t tro;               // byte offset of this lane's first transposed read in a W tile
    int arow0;                  // first dH-tile row of this wave's accumulator slab
    DecK dk;
    Levels lv;                  // the levels of the codes' quant type
    rsrc_t rh, re, rc, rs;      // buffers: dH, the extension, codes, block scales

    __device__ __forceinline__ void hdma(int s, uint4* dst) const {
        const bool main = s < S1;
        const rsrc_t r = main ? rh : re;
        const uint32_t so = uint32_t(main ? s : s - S1) * (DK * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) dma<16>(r, main ? hoff[i] : eoff[i], so, dst + 64 * (4 * w + i));
    }
    __device__ __forceinline__ void sdma(int s, uint4* buf) const {
        char* mine = reinterpret_cast<char*>(buf + DHBUF) + w * DSLOT;
        dma<16>(rc, coff, uint32_t(s) * uint32_t(DK * (a.in / 2)), mine);
        dma<4>(rs, soff, uint32_t(s) * uint32_t(DK * (a.in / 64) * 4), mine + 1024);
    }
    // this thread's 32 weights (staged in `slot`) into W tile `wt`
    __device__ __forceinline__ void dequant(const uint4* buf, uint16_t* wt) const {
        const char* mine = reinterpret_cast<const char*>(buf + DHBUF) + w * DSLOT;
        const uint4 cw = *reinterpret_cast<const uint4*>(mine + lane * 16);
        const float sc = *reinterpret_cast<const float*>(mine + 1024 + lane * 4);
        const Planes p = make_planes(sc, lv);
        u32x4_t o[4];
        lookup8(dk, p, cw.x, o[0]);
        lookup8(dk, p, cw.y, o[1]);
        lookup8(dk, p, cw.z, o[2]);
        lookup8(dk, p, cw.w, o[3]);
        const int unit = tid >> 1, half = tid & 1;
        const int row = unit >> 2, q = unit & 3;
        uint16_t* dst = wt + row * WTS + 64 * q + 32 * half;
        const int f = wt_swizzle(row, 8 * q);  // the same for the thread's four chunks
#pragma unroll
        for (int d = 0; d < 4; ++d) *reinterpret_cast<u32x4_t*>(dst + 8 * (d ^ f)) = o[d];
    }
    // rank-r rows of the B operand: row c of the extension (c < 2r) is A[c mod r]
    __device__ __forceinline__ void afill(int s, int64_t i0, uint16_t* wt) const {
        const int r = a.r;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int e = tid + 256 * k;  // 1024 chunks: 32 rows x 32 chunks of 8
            const int row = e >> 5, ch = e & 31;
            const int c = (s - S1) * DK + row;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (c < 2 * r) v = *reinterpret_cast<const uint4*>(a.A + int64_t(c % r) * a.in + i0 + 8 * ch);
            *reinterpret_cast<uint4*>(wt + row * WTS + 8 * (ch ^ wt_swizzle(row, ch))) = v;
        }
    }
    // A fragment i of slice sl of dH tile `ht`
    __device__ __forceinline__ u32x4_t afrag(const uint4* ht, int i, int sl) const {
        return __builtin_bit_cast(u32x4_t, ht[dpos(arow0 + 32 * i + (lane & 31), 2 * sl + (lane >> 5))]);
    }
    // the step's B operand (2 slices x 2 column frags) from W tile `wt`: eight
    // transposed 8-byte reads off one address (the compiler places the waits)
    __device__ __forceinline__ void bread(const uint16_t* wt, u32x4_t (&b0)[2], u32x4_t (&b1)[2]) const {
        typedef short s16x4_t __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
        char* base = const_cast<char*>(reinterpret_cast<const char*>(wt)) + tro;
        auto rd = [&](int off) {
            return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(base + off)));
        };
        // offsets: +4 rows = 2304 B, +32 columns = 64 B, +16 rows (slice 1) = 9216 B
        const uint2 v0 = rd(0), v1 = rd(2304), v2 = rd(64), v3 = rd(2368);
        const uint2 v4 = rd(9216), v5 = rd(11520), v6 = rd(9280), v7 = rd(11584);
        b0[0] = u32x4_t{v0.x, v0.y, v1.x, v1.y};
        b0[1] = u32x4_t{v2.x, v2.y, v3.x, v3.y};
        b1[0] = u32x4_t{v4.x, v4.y, v5.x, v5.y};
        b1[1] = u32x4_t{v6.x, v6.y, v7.x, v7.y};
    }
};

// One K step t of a wave with FI 32-row blocks: MFMAs on ring buffer `bc`
// (dH tile of step t) and W tile `wc`.  A producing wave (PROD) also issues
// the DMAs of step t+3 into buffer `bd` and dequantizes step t+1 (staged in
// buffer `bn`) into W tile `wn`: it first waits for its own DMAs of step t+1
// (issued two steps earlier), so the dequantization can run between all of
// the step's MFMAs (64/FI VALU operations after each MFMA pair, the staged
// codes read first and the four W-tile stores in the second half).  One set
// of A fragments is live: during slice 0 each fragment, once its two MFMAs
// are issued, is reloaded with slice 1's.
template <int FI, bool PROD>
__device__ __forceinline__ void dx_step(const DxCtx& c, int t, const uint4* bc, const uint4* bn, uint4* bd,
                                        const uint16_t* wc, uint16_t* wn, f32x16_t (&acc)[FI][2], Frag& f) {
    u32x4_t ba[2], bb[2];
    c.bread(wc, ba, bb);
#pragma unroll
    for (int i = 0; i < FI; ++i) f.v[i] = c.afrag(bc, i, 0);
    if constexpr (PROD) {
        c.hdma(t + 3 < c.S ? t + 3 : c.S - 1, bd);
        c.sdma(t + 3 < c.S1 ? t + 3 : c.S1 - 1, bd);
        // step t+1's DMAs (dH tile and staging) are complete: issued two steps ago
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * DX_VM_STEP));
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (PROD) c.dequant(bn, wn);
#pragma unroll
    for (int i = 0; i < FI; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(f.v[i], ba[j], acc[i][j]);
        f.v[i] = c.afrag(bc, i, 1);
    }
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(f.v[i], bb[j], acc[i][j]);
    if constexpr (PROD) {
        constexpr int NV = 64 / FI;  // VALU operations after each MFMA pair
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read: the staged codes and scale
#pragma unroll
        for (int k = 0; k < FI; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
            __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);  // VALU
        }
#pragma unroll
        for (int k = 0; k < FI; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);  // VALU
            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // DS write
        }
        // W tile t+1 (LDS writes) complete before the barrier; no fence:
        // nothing else must be waited for
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * DX_VM_STEP) & ~0xf00u);
    } else {
#pragma unroll
        for (int k = 0; k < FI; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    }
    __builtin_amdgcn_s_barrier();
}

// The K loop over the ring of four buffers, four steps per iteration so the
// ring indices are static (the launcher guarantees a multiple of four
// steps).  The buffers are separate arrays so that the compiler can see that
// a DMA into one never overlaps reads of another.
template <int FI, bool PROD>
__device__ __forceinline__ void dx_loop(const DxCtx& c, int sb, int se, uint4* __restrict__ B0,
                                        uint4* __restrict__ B1, uint4* __restrict__ B2, uint4* __restrict__ B3,
                                        uint16_t* __restrict__ W0, uint16_t* __restrict__ W1,
                                        f32x16_t (&acc)[FI][2]) {
    Frag f;
    for (int t = sb; t < se; t += 4) {
        dx_step<FI, PROD>(c, t, B0, B1, B3, W0, W1, acc, f);
        dx_step<FI, PROD>(c, t + 1, B1, B2, B0, W1, W0, acc, f);
        dx_step<FI, PROD>(c, t + 2, B2, B3, B1, W0, W1, acc, f);
        dx_step<FI, PROD>(c, t + 3, B3, B0, B2, W1, W0, acc, f);
    }
}

template <int DW>
__global__ __launch_bounds__(64 * DW, 1) void k_dx_rd(DxArgs a) {
    static_assert(DW == 4 || DW == 8, "four or eight waves");
    constexpr int FI = DW == 8 ? 4 : 8;  // 32-row blocks of the wave's accumulator slab
    __shared__ __attribute__((aligned(16))) uint4 h0[DXBUF], h1[DXBUF], h2[DXBUF], h3[DXBUF];
    __shared__ __attribute__((aligned(16))) uint16_t wt0[WTBUF], wt1[WTBUF];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t M = a.M, N = a.in;

    // XCD-aware tile order, as in the forward
    const int64_t nMt = (M + RM - 1) / RM, nNt = (N + RN - 1) / RN, T = nMt * nNt;
    const int64_t bid = blockIdx.x;
    const int64_t lin = (T % 8 == 0) ? (bid % 8) * (T / 8) + bid / 8 : bid;
    const int64_t G = 4, gsz = G * nNt;
    const int64_t grp = lin / gsz, first = grp * G;
    const int64_t gm = (nMt - first < G) ? (nMt - first) : G;
    const int64_t tm = first + (lin % gsz) % gm, tn = (lin % gsz) / gm;
    const int64_t m0 = tm * RM, i0 = tn * RN;
    // split z of the reduction: weight-row steps [sb, se); the last split
    // also takes the rank-r steps
    const int z = int(blockIdx.y);
    const bool last = z == int(gridDim.y) - 1;

    DxCtx c{a};
    c.S1 = int(a.out / DK);
    c.S = c.S1 + (a.ext ? a.KL / DK : 0);
    const int sb = z * a.spl;
    const int se = (sb + a.spl < c.S1) ? sb + a.spl : c.S1;
    c.w = w;
    c.lane = lane;
    c.tid = tid;
    // slab of wave w: all 256 rows x 64 columns (four waves), or 128 rows x 64
    // columns (eight waves: waves w and w + 4 share the columns)
    const int cg = DW == 8 ? (w & 3) : w;
    c.arow0 = DW == 8 ? 128 * (w >> 2) : 0;
    const bool prod = w < 4;  // the waves that issue the DMAs and dequantize
    c.dk.init();
    c.lv.init(a.qt);
    c.rh = rsrc_of(a.dh, M * a.out * 2);
    c.re = rsrc_of(a.ext, M * a.KL * 2);
    c.rc = rsrc_of(a.codes, a.out * N / 2);
    c.rs = rsrc_of(a.scales, a.out * (N / 64) * 4);
    {
        const int unit = tid >> 1, half = tid & 1;
        const int64_t row = unit >> 2, q = unit & 3;
        c.coff = uint32_t(row * (N / 2) + (i0 + 64 * q) / 2 + 16 * half);
        c.soff = uint32_t((row * (N / 64) + i0 / 64 + q) * 4);
        const int qq = lane >> 4, i = lane & 15;
        const int col = 64 * cg + 16 * (qq & 1) + 4 * (i & 3);
        const int rw = 8 * (qq >> 1) + (i >> 2);
        const int cc = col >> 3;
        c.tro = uint32_t((rw * WTS + 8 * (cc ^ wt_swizzle(rw, cc)) + (col & 7)) * 2);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = 64 * (4 * w + i) + lane;  // chunk position this lane's DMA writes
        const int m = p >> 2;
        const int ch = (p & 3) ^ ((m >> 2) & 3);  // logical chunk stored there
        int64_t row = m0 + m;
        row = row < M ? row : M - 1;  // rows past M are computed and dropped
        c.hoff[i] = uint32_t((row * a.out + 8 * ch) * 2);
        c.eoff[i] = uint32_t((row * a.KL + 8 * ch) * 2);
    }

    f32x16_t acc[FI][2];
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const int S1 = c.S1, S = c.S;
    // ---- prologue: steps sb, sb+1, sb+2 (dH tile, then staging) in flight
    if (prod) {
        c.hdma(sb, h0);
        c.sdma(sb, h0);
        c.hdma(sb + 1 < S ? sb + 1 : S - 1, h1);
        c.sdma(sb + 1 < S1 ? sb + 1 : S1 - 1, h1);
        c.hdma(sb + 2 < S ? sb + 2 : S - 1, h2);
        c.sdma(sb + 2 < S1 ? sb + 2 : S1 - 1, h2);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * DX_VM_STEP));  // step sb
        c.dequant(h0, wt0);
    }
    __syncthreads();

    if (prod)
        dx_loop<FI, true>(c, sb, se, h0, h1, h2, h3, wt0, wt1, acc);
    else
        dx_loop<FI, false>(c, sb, se, h0, h1, h2, h3, wt0, wt1, acc);
    // the loop's last steps prefetched past the split: let those DMAs land
    // before the workgroup can end
    __builtin_amdgcn_s_waitcnt(0);

    // ---- rank-r steps (last split): dH-side tiles from the ring (the first
    // three were DMA'd by the loop), the B rows copied from A
    for (int s = S1; s < (last ? S : S1); ++s) {
        const int k = s & 3;
        uint4* ht = k == 0 ? h0 : k == 1 ? h1 : k == 2 ? h2 : h3;
        if (s + 3 < S && prod) c.hdma(s + 3, k == 0 ? h3 : k == 1 ? h0 : k == 2 ? h1 : h2);
        if (prod) c.afill(s, i0, wt0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        Frag f0, f1;
        u32x4_t b0[2], b1[2];
        c.bread(wt0, b0, b1);
#pragma unroll
        for (int i = 0; i < FI; ++i) {
            f0.v[i] = c.afrag(ht, i, 0);
            f1.v[i] = c.afrag(ht, i, 1);
        }
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                acc[i][j] = mfma32(f0.v[i], b0[j], acc[i][j]);
                acc[i][j] = mfma32(f1.v[i], b1[j], acc[i][j]);
            }
        __syncthreads();
    }

    // D layout: lane holds column lane%32 and rows 8(v/4) + 4(lane/32) + v%4
    float* pz = a.part + int64_t(z) * M * N;
    const bool split = gridDim.y > 1 || a.f32;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t n = i0 + 64 * cg + 32 * j + (lane & 31);
        if (n >= N) continue;
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t m = m0 + c.arow0 + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (m < M) {
                    if (split)
                        pz[m * N + n] = acc[i][j][v];
                    else
                        a.dx[m * N + n] = to_bf16(acc[i][j][v]);
                }
            }
    }
}

// dX = bf16 of the sum of the split partials, in split order
__global__ __launch_bounds__(256) void k_split_sum(const float* __restrict__ part, int Z, int64_t n,
                                                   uint16_t* __restrict__ out) {
    for (int64_t i = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4; i < n; i += int64_t(gridDim.x) * 1024) {
        float4 a = *reinterpret_cast<const float4*>(part + i);
        for (int zz = 1; zz < Z; ++zz) {
            const float4 b = *reinterpret_cast<const float4*>(part + int64_t(zz) * n + i);
            a.x += b.x;
            a.y += b.y;
            a.z += b.z;
            a.w += b.w;
        }
        *reinterpret_cast<uint2*>(out + i) = make_uint2(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w));
    }
}

// h of the split tail tiles: the tile-local partials summed in split order.
// One workgroup per 4 rows of a tail tile, four consecutive columns per
// thread (16-byte partial reads).
__global__ __launch_bounds__(256) void k_tail_sum(FwdArgs a) {
    const int64_t M = a.M, N = a.N;
    const int64_t nMt = (M + RM - 1) / RM, nNt = (N + RN - 1) / RN, T = nMt * nNt;
    const int64_t trem = T - a.tfull;
    const int64_t tt = blockIdx.x / (RM / 4);
    const int lr = int(blockIdx.x % (RM / 4)) * 4 + (threadIdx.x >> 6), lc = 4 * (threadIdx.x & 63);
    int64_t tm, tn;
    tile_of(a.tfull + tt, nMt, nNt, tm, tn);
    const int64_t m = tm * RM + lr, col = tn * RN + lc;
    if (m >= M || col >= N) return;
    const float* p = a.part + tt * (RM * RN) + lr * RN + lc;
    float4 v = *reinterpret_cast<const float4*>(p);
    for (int zz = 1; zz < a.ztail; ++zz) {
        const float4 b = *reinterpret_cast<const float4*>(p + int64_t(zz) * trem * (RM * RN));
        v.x += b.x;
        v.y += b.y;
        v.z += b.z;
        v.w += b.w;
    }
    const float vv[4] = {v.x, v.y, v.z, v.w};
    for (int e = 0; e < 4; ++e)
        if (col + e < N) a.h[m * N + col + e] = to_bf16(vv[e]);
}

// The multi-adapter forward after a split reduction: h[m][n] = bf16( the
// partials summed in split order + the gathered rank-r term ).  A wave takes
// 64 consecutive columns of one row, so the token's id and su row are
// wave-uniform and the B_id row segment is contiguous.
__global__ __launch_bounds__(256) void k_multi_fin(FwdArgs a, int Z) {
    const int64_t M = a.M, N = a.N, n = M * N;
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
        const int64_t m = i / N, col = i % N;
        float v = a.part[i];
        for (int zz = 1; zz < Z; ++zz) v += a.part[int64_t(zz) * n + i];
        a.h[i] = to_bf16(v + multi_term(a, a.ids[m], m, col));
    }
}

// fp32 block scales of a double-quantized weight: fl32(fl32(q_b/127) * c_g).
template <bool GSH>
__global__ __launch_bounds__(256) void k_block_scales(nf4::QView q, int64_t nb, float* __restrict__ out) {
    __shared__ float tab[256];
    block_scales_wg<GSH>(q.qcodes, q.gabs, q.group, q.gshift, nb, out, blockIdx.x, gridDim.x, tab);
}

}  // namespace

namespace nf4 {

size_t rd_scales_bytes(int64_t rows, int64_t cols) { return align256(size_t(rows * cols / 64) * 4); }

bool use_rd(const QView& q, int64_t M, int r, int KL) {
    // at most three rank-r steps, NF4 steps in fours, 32-bit offsets
    return !((r > 0 && KL > 3 * RKS) || q.cols % (4 * RKS) != 0 ||
             q.rows * q.cols / 2 >= (int64_t(1) << 32) || M * q.cols * 2 >= (int64_t(1) << 32) ||
             (r > 0 && M * KL * 2 >= (int64_t(1) << 32)));
}

// fp32 block scales: the absmax array, or the double-quant decode into scale_ws
int block_scales(const QView& q, float* scale_ws, const float** scales, hipStream_t st) {
    *scales = q.absmax;
    if (!q.dq) return NF4_OK;
    const int64_t nb = q.rows * q.cols / 64;
    const unsigned g = unsigned(std::min<int64_t>(cdiv(nb, 1024), 4096));
    if (q.gshift >= 0)
        hipLaunchKernelGGL(k_block_scales<true>, dim3(g), dim3(256), 0, st, q, nb, scale_ws);
    else
        hipLaunchKernelGGL(k_block_scales<false>, dim3(g), dim3(256), 0, st, q, nb, scale_ws);
    if (hipPeekAtLastError() != hipSuccess) return launch_status();
    *scales = scale_ws;
    return NF4_OK;
}

bool use_rd_grid(int64_t M, int64_t N) { return cdiv(M, RM) * cdiv(N, RN) >= 32; }

bool use_dx_rd(const QView& q, int64_t M, int r, int KL) {
    // whole steps of 32 weight rows in fours, whole 256-column tiles, 32-bit offsets
    return cdiv(M, RM) * cdiv(q.cols, RN) >= 16 && q.rows % (4 * DK) == 0 && q.cols % RN == 0 &&
           (r == 0 || KL % DK == 0) && q.rows * q.cols / 2 < (int64_t(1) << 32) &&
           M * q.rows * 2 < (int64_t(1) << 32) && (r == 0 || M * KL * 2 < (int64_t(1) << 32));
}

// Splits of the dX reduction: enough workgroups for the GPU when the output
// tiles alone are too few, each split a whole number of four-step groups.
int dx_splits(int64_t M, int64_t rows, int64_t cols) {
    const int64_t T = cdiv(M, RM) * cdiv(cols, RN);
    int64_t Z = T >= 192 ? 1 : std::min<int64_t>(8, std::max<int64_t>(1, 256 / T));
    const int64_t S1 = rows / DK;
    const int64_t spl = cdiv(cdiv(S1, Z), 4) * 4;
    return int(cdiv(S1, spl));
}

size_t dx_rd_part_bytes(int64_t M, int64_t rows, int64_t cols) {
    const int Z = dx_splits(M, rows, cols);
    return Z > 1 ? align256(size_t(Z) * size_t(M) * size_t(cols) * 4) : 0;
}

// Waves of the dX kernel: four (one per SIMD, each with a 256 x 64 slab,
// every wave dequantizing), or eight (two per SIMD: waves 0-3 issue the DMAs
// and dequantize, waves 4-7 only multiply; 128 x 64 slabs), so that one
// wave's dequantization overlaps the other's MFMAs.
#ifndef NF4_DX_WAVES
#define NF4_DX_WAVES 8
#endif
constexpr int kDxWaves = NF4_DX_WAVES;

int dx_rd(const QView& q, const uint16_t* dH, int64_t M, const uint16_t* duext, int KL, const uint16_t* A,
          int r, uint16_t* dX, float* scale_ws, float* part_ws, hipStream_t st, bool f32) {
    const float* scales;
    int rc = block_scales(q, scale_ws, &scales, st);
    if (rc) return rc;
    const int Z = dx_splits(M, q.rows, q.cols);
    const int S1 = int(q.rows / DK);
    const int spl = int(cdiv(cdiv(S1, Z), 4) * 4);
    DxArgs a{reinterpret_cast<const uint8_t*>(q.codes), scales, dH, r > 0 ? duext : nullptr, A, dX, part_ws,
             M, q.rows, q.cols, KL, r, spl, f32 ? 1 : 0, q.qt};
    const int64_t T = cdiv(M, RM) * cdiv(q.cols, RN);
    launch_dominant(k_dx_rd<kDxWaves>, dim3(unsigned(T), unsigned(Z)), dim3(64 * kDxWaves), 0, st, a);
    if (hipPeekAtLastError() != hipSuccess) return launch_status();
    if (Z > 1 && !f32) {
        const int64_t n = M * q.cols;  // a multiple of 256
        hipLaunchKernelGGL(k_split_sum, dim3(unsigned(std::min<int64_t>(cdiv(n, 1024), 8192))), dim3(256), 0, st,
                           part_ws, Z, n, dX);
        if (hipPeekAtLastError() != hipSuccess) return launch_status();
    }
    return NF4_OK;
}

// Waves of the single-adapter forward kernel: eight (two per SIMD, each
// with a 256 x 32 accumulator slab) so that one wave's dequantization and
// waits overlap the other's MFMAs.
#ifndef NF4_FWD_WAVES
#define NF4_FWD_WAVES 8
#endif
constexpr int kFwdWaves = NF4_FWD_WAVES;

struct TailPlan {
    int64_t T, tfull, grid;
    int z, spl;
};

static TailPlan tail_plan(int64_t M, int64_t rows, int64_t cols) {
    constexpr int64_t kCUs = 256;  // one workgroup per CU (the LDS of this kernel)
    TailPlan p{};
    p.T = cdiv(M, RM) * cdiv(rows, RN);
    p.tfull = p.T / kCUs * kCUs;
    const int64_t trem = p.T - p.tfull;
    const int64_t S1 = cols / RKS;
    p.z = 1;
    p.spl = int(S1);
    if (trem > 0) {
        const int64_t z = std::min<int64_t>(4, std::max<int64_t>(1, kCUs / trem));
        const int64_t spl = cdiv(cdiv(S1, z), 4) * 4;
        p.z = int(cdiv(S1, spl));
        p.spl = int(spl);
    }
    if (p.z <= 1) {
        p.z = 1;
        p.tfull = p.T;
    }
    p.grid = p.tfull + (p.T - p.tfull) * p.z;
    return p;
}

int forward_rd(const QView& q, const uint16_t* x, int64_t M, const uint16_t* ext, int KL,
               const uint16_t* B, int r, uint16_t* h, float* scale_ws, float* tail_ws, hipStream_t st) {
    const float* scales = q.absmax;
    const int64_t nb = q.rows * q.cols / 64;
    if (q.dq) {
        const unsigned g = unsigned(std::min<int64_t>(cdiv(nb, 1024), 4096));
        if (q.gshift >= 0)
            hipLaunchKernelGGL(k_block_scales<true>, dim3(g), dim3(256), 0, st, q, nb, scale_ws);
        else
            hipLaunchKernelGGL(k_block_scales<false>, dim3(g), dim3(256), 0, st, q, nb, scale_ws);
        if (hipPeekAtLastError() != hipSuccess) return launch_status();
        scales = scale_ws;
    }
    const TailPlan tp = tail_plan(M, q.rows, q.cols);
    FwdArgs a{reinterpret_cast<const uint8_t*>(q.codes), scales, x, r > 0 ? ext : nullptr, B, h,
              M, q.rows, q.cols, KL, r, nullptr, nullptr, nullptr, 0, 0, tail_ws, int(q.cols / RKS),
              tp.tfull, tp.z, tp.spl, q.qt};
    launch_dominant(k_fwd_rd<false, kFwdWaves>, dim3(unsigned(tp.grid)), dim3(64 * kFwdWaves), 0, st, a);
    if (hipPeekAtLastError() != hipSuccess) return launch_status();
    if (tp.z > 1) {
        hipLaunchKernelGGL(k_tail_sum, dim3(unsigned((tp.T - tp.tfull) * (RM / 4))), dim3(256), 0, st, a);
        if (hipPeekAtLastError() != hipSuccess) return launch_status();
    }
    return NF4_OK;
}

// One full pass of the GPU (kCUs workgroups) over the first tiles, then the
// remaining tiles split so that their pass is shorter.
size_t fwd_tail_bytes(int64_t M, int64_t rows, int64_t cols) {
    const TailPlan tp = tail_plan(M, rows, cols);
    return tp.z > 1 ? align256(size_t(tp.z) * size_t(tp.T - tp.tfull) * RM * RN * 4) : 0;
}

// Splits of the forward reduction for the multi-adapter pass: enough
// workgroups for the GPU when the output tiles alone are too few.
int fwd_multi_splits(int64_t M, int64_t rows, int64_t cols) {
    const int64_t T = cdiv(M, RM) * cdiv(rows, RN);
    const int64_t Z = T >= 192 ? 1 : std::min<int64_t>(4, std::max<int64_t>(1, 256 / T));
    const int64_t S1 = cols / RKS;
    const int64_t spl = cdiv(cdiv(S1, Z), 4) * 4;
    return int(cdiv(S1, spl));
}

size_t fwd_multi_part_bytes(int64_t M, int64_t rows, int64_t cols) {
    const int Z = fwd_multi_splits(M, rows, cols);
    return Z > 1 ? align256(size_t(Z) * size_t(M) * size_t(rows) * 4) : 0;
}

int forward_rd_multi(const QView& q, const uint16_t* x, int64_t M, const float* su, const int32_t* ids,
                     const uint16_t* Bb, int n_ad, int r, uint16_t* h, float* scale_ws, float* part_ws,
                     const MultiSort* ms, hipStream_t st, bool scales_ready) {
    const float* scales = scale_ws;
    if (!(scales_ready && q.dq)) {
        const int rc = block_scales(q, scale_ws, &scales, st);
        if (rc) return rc;
    }
    const int Z = fwd_multi_splits(M, q.rows, q.cols);
    const int S1 = int(q.cols / RKS);
    const int spl = int(cdiv(cdiv(S1, Z), 4) * 4);
    FwdArgs a{reinterpret_cast<const uint8_t*>(q.codes), scales, x, nullptr, nullptr, h,
              M, q.rows, q.cols, 0, 0, su, ids, Bb, n_ad, r, part_ws, spl, 0, 1, spl, q.qt};
    const int64_t T = cdiv(M, RM) * cdiv(q.rows, RN);
    // split: the plain forward kernel (eight waves) writes the fp32 partials
    // and the gather follows; one split: the gathered epilogue in the kernel
    if (Z > 1)
        launch_dominant(k_fwd_rd<false, kFwdWaves>, dim3(unsigned(T), unsigned(Z)), dim3(64 * kFwdWaves), 0, st, a);
    else
        launch_dominant(k_fwd_rd<true, 4>, dim3(unsigned(T), 1u), dim3(256), 0, st, a);
    if (hipPeekAtLastError() != hipSuccess) return launch_status();
    if (Z > 1) {
        if (ms) return multi_fin_seg(*ms, part_ws, Z, M, q.rows, su, r, Bb, h, st);
        hipLaunchKernelGGL(k_multi_fin, dim3(unsigned(std::min<int64_t>(cdiv(M * q.rows, 256), 8192))), dim3(256), 0,
                           st, a, Z);
        if (hipPeekAtLastError() != hipSuccess) return launch_status();
    }
    return NF4_OK;
}

}  // namespace nf4
