// merge.hip -- the adapter merged into the base weight (a 16-bit model).
//
//   W_out[o][i] = bf16( Wb[o][i] + scale * sum_j B[o][j] A[j][i] )
//
// ("How Fine-Tuning LLMs with LoRA and QLoRA Works", FAQ on merging adapters
// back into the base weights; "QLoRA explained", "Merging and deploying").
// Wb is the layer's dequantized bf16 weight, bf16(fl32(s~ * T[code])).
//
// One workgroup per 256 columns and four 64-row slabs, four waves, wave w
// owning columns [64w, 64w + 64).  The rank-r product runs on the 32x32x16
// bf16 MFMA in chunks of 64 adapter rows: the B rows of a slab (64 x 64) and
// the A rows (64 x 256, staged once for all four slabs when r <= 64) sit in
// LDS with zero padding past r; the A operand (rows of B) is read row-wise,
// the B operand (columns of A) transposed with ds_read_b64_tr_b16.  The
// epilogue goes through LDS one 32-row half at a time, so that each thread
// finishes eight consecutive columns of a row: one code dword, one block
// scale, a 16-byte store.  The time is in streaming the codes in and the bf16
// weight out, so the epilogue's code and scale loads of a slab are issued
// with its B staging (one memory round trip per slab), and the workgroup
// barriers wait for LDS only, leaving the stores and those loads in flight.
#include "nf4_device.h"
#include "nf4_internal.h"

using namespace nf4dev;

namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int MG_ROWS = 64, MG_COLS = 256, MG_KC = 64;
constexpr int MG_SLABS = 4;  // 64-row slabs per workgroup (the A chunk is reused across them)
constexpr int MG_AS = MG_COLS + 32;  // A chunk row stride (elements): conflict-free transposed reads
constexpr int MG_BS = MG_KC + 8;     // B chunk row stride (elements): conflict-free row reads
constexpr int MG_SS = MG_COLS + 4;   // output staging row stride (floats)

__device__ __forceinline__ f32x16_t mfma32(const u32x4_t& a, const u32x4_t& b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                    c, 0, 0, 0);
}

// Workgroup barrier for LDS hazards only: the wave's LDS operations are
// complete, global loads and stores may still be in flight (the compiler
// waits for a load where its value is used).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <bool DQ, bool GSH>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_merge(nf4::QView q, const uint16_t* __restrict__ A,
                                               const uint16_t* __restrict__ B, int r, float scale,
                                               uint16_t* __restrict__ W_out) {
    __shared__ __attribute__((aligned(16))) uint16_t at[MG_KC * MG_AS];   // A chunk
    __shared__ __attribute__((aligned(16))) float stg[32 * MG_SS];        // output staging, one 32-row half
    __shared__ __attribute__((aligned(16))) uint16_t bt[MG_ROWS * MG_BS];  // B chunk of the slab
    __shared__ float lv[16];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t N = q.rows, K = q.cols;
    const int64_t nct = (K + MG_COLS - 1) / MG_COLS;
    const int64_t r0 = int64_t(blockIdx.x / nct) * (MG_ROWS * MG_SLABS), i0 = int64_t(blockIdx.x % nct) * MG_COLS;
    if (tid < 16) lv[tid] = bits_f(qt_level_bits(q.qt, tid));

    // this lane's transposed-read position: in each 16-lane group lane 4e + g
    // addresses k row 8(qq/2) + e, column 16(qq%2) + 4g of the wave's slab
    const int qq = lane >> 4, li = lane & 15;
    const uint32_t tro = uint32_t(((8 * (qq >> 1) + (li >> 2)) * MG_AS + 64 * w + 16 * (qq & 1) + 4 * (li & 3)) * 2);
    const uint32_t atb = uint32_t(reinterpret_cast<uintptr_t>(at));
    const int rpad = (r + 15) / 16 * 16;
    const bool one_chunk = rpad <= MG_KC;  // the A chunk is staged once for all slabs
    const bool bvec = (r & 7) == 0;        // 16-byte rows of B
    const char* codes = reinterpret_cast<const char*>(q.codes);

    // Staging loops have fixed trip counts and load from clamped (valid)
    // addresses, the values past r or K replaced by zeros afterwards, so all
    // of a loop's loads are in flight together before its LDS writes.
    // (component-wise, so that the staged values stay in registers)
    auto keep4 = [](bool ok, const uint4& v) {
        return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
    };
    auto stage_a = [&](int kc) {  // A rows [kc, kc + 64) x the tile's 256 columns, in two passes
#pragma unroll
        for (int ps = 0; ps < 2; ++ps) {
            uint4 v[4];
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int e = tid + 256 * (4 * ps + it), kr = e >> 5, ch = e & 31;
                const int64_t col = i0 + 8 * ch;
                const int64_t rr = kc + kr < r ? kc + kr : r - 1, cc = col < K ? col : K - 8;
                v[it] = *reinterpret_cast<const uint4*>(A + rr * K + cc);
            }
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int e = tid + 256 * (4 * ps + it), kr = e >> 5, ch = e & 31;
                const bool ok = kc + kr < r && i0 + 8 * ch < K;
                *reinterpret_cast<uint4*>(at + kr * MG_AS + 8 * ch) = keep4(ok, v[it]);
            }
        }
    };

    for (int sb = 0; sb < MG_SLABS; ++sb) {
        const int64_t o0 = r0 + int64_t(sb) * MG_ROWS;
        if (o0 >= N) break;  // workgroup-uniform
        // the epilogue's loads: item tid + 256k of half hf is row (item >> 5)
        // of the half, columns 8 (item & 31) .. + 7
        uint32_t pcd[2][4];
        int pq[2][4];
        float pg[2][4];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int item = tid + 256 * k;
                // clamped to a valid element: the values of items past N or K are not used
                int64_t o = o0 + 32 * hf + (item >> 5), col = i0 + 8 * (item & 31);
                o = o < N ? o : N - 1;
                col = col < K ? col : K - 8;
                const int64_t el = o * K + col;
                pcd[hf][k] = *reinterpret_cast<const uint32_t*>(codes + el / 2);
                const int64_t b = el >> q.bshift;
                if (DQ) {
                    pq[hf][k] = q.qcodes[b];
                    pg[hf][k] = q.gabs[GSH ? (b >> q.gshift) : (b / q.group)];
                } else {
                    pq[hf][k] = 0;
                    pg[hf][k] = q.absmax[b];
                }
            }
        f32x16_t acc[2][2];
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

        for (int kc = 0; kc < rpad; kc += MG_KC) {
            lds_barrier();  // the previous chunk's (or slab's) reads are done
            if (!one_chunk || sb == 0) stage_a(kc);
            // B rows [o0, o0 + 64) x adapter columns [kc, kc + 64), zero past r
            if (bvec) {
                uint4 v[MG_ROWS * (MG_KC / 8) / 256];
#pragma unroll
                for (int it = 0; it < MG_ROWS * (MG_KC / 8) / 256; ++it) {
                    const int e = tid + 256 * it, ro = e >> 3, ch = e & 7;
                    const int64_t o = o0 + ro < N ? o0 + ro : N - 1;
                    const int kk = kc + 8 * ch < r ? kc + 8 * ch : r - 8;
                    v[it] = *reinterpret_cast<const uint4*>(B + o * r + kk);
                }
#pragma unroll
                for (int it = 0; it < MG_ROWS * (MG_KC / 8) / 256; ++it) {
                    const int e = tid + 256 * it, ro = e >> 3, ch = e & 7;
                    const bool ok = o0 + ro < N && kc + 8 * ch < r;
                    *reinterpret_cast<uint4*>(bt + ro * MG_BS + 8 * ch) = keep4(ok, v[it]);
                }
            } else {
                uint16_t v[MG_ROWS * MG_KC / 256];
#pragma unroll
                for (int it = 0; it < MG_ROWS * MG_KC / 256; ++it) {
                    const int e = tid + 256 * it, ro = e >> 6, kk = e & 63;
                    const int64_t o = o0 + ro < N ? o0 + ro : N - 1;
                    v[it] = B[o * r + (kc + kk < r ? kc + kk : r - 1)];
                }
#pragma unroll
                for (int it = 0; it < MG_ROWS * MG_KC / 256; ++it) {
                    const int e = tid + 256 * it, ro = e >> 6, kk = e & 63;
                    bt[ro * MG_BS + kk] = (o0 + ro < N && kc + kk < r) ? v[it] : uint16_t(0);
                }
            }
            lds_barrier();
            const int ksteps = (rpad - kc < MG_KC ? rpad - kc : MG_KC) / 16;
            for (int ks = 0; ks < ksteps; ++ks) {
                // B operand: columns of A, 8 consecutive k per lane from two transposed reads
                u32x4_t bo[2];
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) {
                    const uint32_t ad = atb + tro + uint32_t((16 * ks * MG_AS + 32 * cb) * 2);
                    uint2 v0, v1;
                    asm volatile(
                        "ds_read_b64_tr_b16 %0, %2\n\t"
                        "ds_read_b64_tr_b16 %1, %2 offset:2304\n\t"
                        "s_waitcnt lgkmcnt(0)"
                        : "=&v"(v0), "=&v"(v1)
                        : "v"(ad)
                        : "memory");
                    bo[cb] = u32x4_t{v0.x, v0.y, v1.x, v1.y};
                }
                // A operand: rows of B, 8 consecutive k per lane
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    const u32x4_t ao = *reinterpret_cast<const u32x4_t*>(
                        bt + (32 * rb + (lane & 31)) * MG_BS + 16 * ks + 8 * (lane >> 5));
#pragma unroll
                    for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = mfma32(ao, bo[cb], acc[rb][cb]);
                }
            }
        }

        // epilogue of the slab, one 32-row half at a time through LDS
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            if (hf) lds_barrier();  // the previous half is no longer read
            // D layout of the 32x32 MFMA: lane holds column lane%32, rows 8(v/4) + 4(lane/32) + v%4
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    stg[(8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)) * MG_SS + 64 * w + 32 * cb + (lane & 31)] =
                        acc[hf][cb][v];
            lds_barrier();
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int item = tid + 256 * k;  // 32 rows x 32 chunks of 8 columns
                const int row = item >> 5, ch = item & 31;
                const int64_t o = o0 + 32 * hf + row, col = i0 + 8 * ch;
                if (o >= N || col >= K) continue;
                const int64_t el = o * K + col;
                const uint32_t cd = pcd[hf][k];
                const float s = DQ ? __fmul_rn(q_over_127(pq[hf][k]), pg[hf][k]) : pg[hf][k];
                const float4 p0 = *reinterpret_cast<const float4*>(stg + row * MG_SS + 8 * ch);
                const float4 p1 = *reinterpret_cast<const float4*>(stg + row * MG_SS + 8 * ch + 4);
                const float pv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
                uint32_t outw[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    // byte t of the dword: element 2t in the high nibble, 2t+1 in the low
                    const uint32_t by = (cd >> (8 * t)) & 0xFFu;
                    const float w0 = bf16_f(to_bf16(__fmul_rn(s, lv[by >> 4])));
                    const float w1 = bf16_f(to_bf16(__fmul_rn(s, lv[by & 15u])));
                    outw[t] = pack_bf16x2(__builtin_fmaf(scale, pv[2 * t], w0),
                                          __builtin_fmaf(scale, pv[2 * t + 1], w1));
                }
                *reinterpret_cast<uint4*>(W_out + el) = make_uint4(outw[0], outw[1], outw[2], outw[3]);
            }
        }
    }
}

}  // namespace

namespace nf4 {

int merge_adapter(const QView& q, const uint16_t* A, const uint16_t* B, int r, float scale, uint16_t* W_out,
                  hipStream_t st) {
    const int64_t tiles = cdiv(q.rows, MG_ROWS * MG_SLABS) * cdiv(q.cols, MG_COLS);
    if (tiles >= (int64_t(1) << 31)) return NF4_ESHAPE;
    const dim3 grid = dim3(unsigned(tiles));
    auto kern = q.dq ? (q.gshift >= 0 ? k_merge<true, true> : k_merge<true, false>) : k_merge<false, true>;
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, q, A, B, r, scale, W_out);
    return hipPeekAtLastError() == hipSuccess ? NF4_OK : launch_status();
}

}  // namespace nf4
