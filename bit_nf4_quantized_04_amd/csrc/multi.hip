// multi.hip -- the adapter terms of the multi-adapter forward with the tokens
// bucketed by adapter id:
//
//   h_t = x_t Wb^T + s_id (x_t A_id^T) B_id^T,  id = ids[t]
//
// ("From LoRA to QLoRA", "The Real-World Bottleneck": one resident base and
// an adapter chosen per request; an id outside [0, n) adds nothing).
//
// Taken token by token, every token rereads its adapter's A (r x in) for the
// down-projection and every output element its adapter's B row; grouped by
// adapter, each A and B piece is read once per segment of up to 16 tokens.
//  * k_multi_sort: one workgroup counts the tokens per bucket (bucket n for
//    the invalid ids), prefix-sums the counts into bucket offsets and into
//    segment offsets (segments of SEG tokens never span two buckets), and
//    scatters the token indices into bucket order.  The order inside a
//    bucket is whatever the LDS atomics give; every output is computed from
//    its own token's data only, so it does not depend on that order.
//  * k_multi_down_seg: per segment of a valid bucket a, su[t][j] = s_a *
//    sum_k x[t][k] A_a[j][k] on the 16x16x32 MFMA (tokens as A rows, the r
//    adapter rows as B columns), the K range split over the four waves and
//    summed in LDS.
//  * k_multi_fin_seg: after a split base reduction, per segment and 256
//    columns, h[t][n] = bf16(sum of the partials in split order + sum_j
//    su[t][j] B_a[n][j]); each thread keeps its column's B row in registers
//    for the whole segment, and the su rows are workgroup-uniform.
#include "nf4_device.h"
#include "nf4_internal.h"

using namespace nf4dev;

namespace {

constexpr int SEG = 16;  // tokens per segment: one MFMA row block

// Buckets b = id (valid) or n_ad.  off[b]: first bucket-ordered position of
// bucket b, off[n_ad + 1] = M; seg[b]: first segment of bucket b,
// seg[n_ad + 1] = number of segments.
// Workgroups after the first, when the launch has them, decode the fp32
// block scales of a double-quantized weight for the base product
// (fl32(fl32(q_b/127) * c_g) into sc_out), which then needs no launch of
// its own.
__global__ __launch_bounds__(1024) void k_multi_sort(const int32_t* __restrict__ ids, int M, int n_ad,
                                                     int32_t* __restrict__ perm, int32_t* __restrict__ off,
                                                     int32_t* __restrict__ seg, nf4::QView q, int64_t nblk,
                                                     float* __restrict__ sc_out) {
    __shared__ int cnt[nf4::kMultiSortMaxAdapters + 1];
    __shared__ int cur[nf4::kMultiSortMaxAdapters + 1];
    if (blockIdx.x > 0) {  // workgroup-uniform
        __shared__ float tab[256];
        if (q.gshift >= 0)
            block_scales_wg<true>(q.qcodes, q.gabs, q.group, q.gshift, nblk, sc_out, blockIdx.x - 1,
                                  gridDim.x - 1, tab);
        else
            block_scales_wg<false>(q.qcodes, q.gabs, q.group, q.gshift, nblk, sc_out, blockIdx.x - 1,
                                   gridDim.x - 1, tab);
        return;
    }
    const int tid = threadIdx.x, nb = n_ad + 1;
    for (int b = tid; b < nb; b += 1024) cnt[b] = 0;
    __syncthreads();
    for (int t = tid; t < M; t += 1024) {
        const int id = ids[t];
        atomicAdd(&cnt[(id >= 0 && id < n_ad) ? id : n_ad], 1);
    }
    __syncthreads();
    if (tid < 64) {  // wave 0: lane l scans buckets [l*per, l*per + per), then the lanes' totals
        const int per = (nb + 63) / 64, b0 = tid * per, b1 = min(nb, b0 + per);
        int tc = 0, ts = 0;
        for (int b = b0; b < b1; ++b) {
            tc += cnt[b];
            ts += (cnt[b] + SEG - 1) / SEG;
        }
        int ic = tc, is = ts;  // inclusive scans across the lanes
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int c2 = __shfl_up(ic, d, 64), s2 = __shfl_up(is, d, 64);
            if (tid >= d) {
                ic += c2;
                is += s2;
            }
        }
        int oc = ic - tc, os = is - ts;
        for (int b = b0; b < b1; ++b) {
            off[b] = oc;
            seg[b] = os;
            cur[b] = oc;
            oc += cnt[b];
            os += (cnt[b] + SEG - 1) / SEG;
        }
        if (tid == 63) {
            off[nb] = ic;
            seg[nb] = is;
        }
    }
    __syncthreads();
    for (int t = tid; t < M; t += 1024) {
        const int id = ids[t];
        const int pos = atomicAdd(&cur[(id >= 0 && id < n_ad) ? id : n_ad], 1);
        perm[pos] = t;
    }
}

// The bucket of segment w: the largest b in [0, nb) with seg[b] <= w.
__device__ __forceinline__ int bucket_of(const int32_t* seg, int nb, int w) {
    int lo = 0, hi = nb - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (seg[mid] <= w) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// su[t][j] for the tokens of one segment of a valid bucket.  NJ blocks of 16
// adapter rows (r <= 16 NJ); NWD waves split the K range (32-k slices w,
// w + NWD, ...) and their sums are added in LDS in wave order.  K % 32 == 0.
template <int NJ, int NWD>
__global__ __launch_bounds__(64 * NWD) void k_multi_down_seg(const uint16_t* __restrict__ x, int64_t K,
                                                        const uint16_t* __restrict__ Ab, int n_ad, int r,
                                                        const float* __restrict__ scales,
                                                        const int32_t* __restrict__ perm,
                                                        const int32_t* __restrict__ off,
                                                        const int32_t* __restrict__ seg, float* __restrict__ su) {
    constexpr int RS = 16 * NJ + 4;  // the four row groups of a fragment 16 banks apart
    __shared__ float red[NWD][SEG][RS];
    const int w_idx = blockIdx.x;
    if (w_idx >= seg[n_ad]) return;  // past the segments of the valid buckets (workgroup-uniform)
    const int a = bucket_of(seg, n_ad, w_idx);
    const int p0 = off[a] + (w_idx - seg[a]) * SEG, p1 = min(off[a + 1], p0 + SEG);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int li = lane & 15, g = lane >> 4;
    const int tok = perm[p0 + li < p1 ? p0 + li : p0];  // rows past the segment repeat its first token
    const uint16_t* xr = x + int64_t(tok) * K + 8 * g;
    const uint16_t* ar[NJ];
#pragma unroll
    for (int jb = 0; jb < NJ; ++jb) {
        const int j = 16 * jb + li;
        ar[jb] = Ab + (int64_t(a) * r + (j < r ? j : r - 1)) * K + 8 * g;
    }
    f32x4_t acc[NJ];
#pragma unroll
    for (int jb = 0; jb < NJ; ++jb) acc[jb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // 32-k slices s = w, w + NWD, ...; four in flight
    constexpr int KS = 32 * NWD;
    int64_t k = 32 * w;
    for (; k + 3 * KS < K; k += 4 * KS) {
        u32x4_t xa[4], ab[4][NJ];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            xa[u] = *reinterpret_cast<const u32x4_t*>(xr + k + KS * u);
#pragma unroll
            for (int jb = 0; jb < NJ; ++jb) ab[u][jb] = *reinterpret_cast<const u32x4_t*>(ar[jb] + k + KS * u);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int jb = 0; jb < NJ; ++jb) acc[jb] = mfma16(xa[u], ab[u][jb], acc[jb]);
    }
    for (; k < K; k += KS) {
        const u32x4_t xa = *reinterpret_cast<const u32x4_t*>(xr + k);
#pragma unroll
        for (int jb = 0; jb < NJ; ++jb)
            acc[jb] = mfma16(xa, *reinterpret_cast<const u32x4_t*>(ar[jb] + k), acc[jb]);
    }
    // D: lane holds adapter row 16 jb + li of token rows 4g + e
#pragma unroll
    for (int jb = 0; jb < NJ; ++jb)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[w][4 * g + e][16 * jb + li] = acc[jb][e];
    __syncthreads();
    const float s = scales[a];
    const int n = p1 - p0;
    for (int idx = tid; idx < n * r; idx += 64 * NWD) {
        const int i = idx / r, j = idx - i * r;
        float v = red[0][i][j];
#pragma unroll
        for (int ww = 1; ww < NWD; ++ww) v += red[ww][i][j];
        su[int64_t(perm[p0 + i]) * r + j] = v * s;
    }
}

// h for the tokens of one segment (any bucket) and 256 columns after a split
// reduction of Z partials [Z][M][N].  r <= RR.  Token indices and su rows
// are the same for the whole workgroup (scalar loads); each thread holds its
// column's B row (16-byte loads when r % 8 == 0).
template <int RR>
__global__ __launch_bounds__(256) void k_multi_fin_seg(const float* __restrict__ part, int Z, int64_t M, int64_t N,
                                                       const float* __restrict__ su, int r,
                                                       const uint16_t* __restrict__ Bb, int n_ad,
                                                       const int32_t* __restrict__ perm,
                                                       const int32_t* __restrict__ off,
                                                       const int32_t* __restrict__ seg, uint16_t* __restrict__ h) {
    const int w_idx = blockIdx.x;
    if (w_idx >= seg[n_ad + 1]) return;  // workgroup-uniform
    const int a = bucket_of(seg, n_ad + 1, w_idx);
    const bool valid = a < n_ad;
    const int p0 = off[a] + (w_idx - seg[a]) * SEG, p1 = min(off[a + 1], p0 + SEG);
    const int64_t n = int64_t(blockIdx.y) * 256 + threadIdx.x;
    if (n >= N) return;
    float b[RR];
#pragma unroll
    for (int j = 0; j < RR; ++j) b[j] = 0.0f;
    if (valid) {
        const uint16_t* br = Bb + (int64_t(a) * N + n) * r;
        if ((r & 7) == 0) {
#pragma unroll
            for (int j8 = 0; j8 < RR / 8; ++j8)
                if (8 * j8 < r) {
                    const uint4 v = *reinterpret_cast<const uint4*>(br + 8 * j8);
                    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        b[8 * j8 + 2 * e] = bf16_lo(w4[e]);
                        b[8 * j8 + 2 * e + 1] = bf16_hi(w4[e]);
                    }
                }
        } else {
#pragma unroll
            for (int j = 0; j < RR; ++j)
                if (j < r) b[j] = bf16_f(br[j]);
        }
    }
    // every token's partials in flight at once (rows past the segment repeat
    // its first token and are not stored)
    const int cnt = p1 - p0;
    int64_t t[SEG];
    float v[SEG];
#pragma unroll
    for (int i = 0; i < SEG; ++i) {
        t[i] = perm[i < cnt ? p0 + i : p0];
        v[i] = part[t[i] * N + n];
    }
    for (int zz = 1; zz < Z; ++zz)
#pragma unroll
        for (int i = 0; i < SEG; ++i) v[i] += part[(int64_t(zz) * M + t[i]) * N + n];
#pragma unroll
    for (int i = 0; i < SEG; ++i) {
        float l = 0.0f;
        if (valid) {
            const float* srow = su + t[i] * r;
            if (r == RR) {  // whole rows: wide scalar loads
#pragma unroll
                for (int j = 0; j < RR; ++j) l = __builtin_fmaf(srow[j], b[j], l);
            } else {
#pragma unroll
                for (int j = 0; j < RR; ++j)
                    if (j < r) l = __builtin_fmaf(srow[j], b[j], l);
            }
        }
        if (i < cnt) h[t[i] * N + n] = to_bf16(v[i] + l);
    }
}

}  // namespace

namespace nf4 {

size_t multi_sort_bytes(int64_t M, int n_ad) {
    return align256(size_t(M) * 4) + 2 * align256(size_t(n_ad + 2) * 4);
}

bool use_multi_sort(int64_t M, int n_ad, int r) {
    return n_ad <= kMultiSortMaxAdapters && r <= 64 && M < (int64_t(1) << 30);
}

int multi_sort(const int32_t* ids, int64_t M, int n_ad, char* ws, MultiSort* ms, hipStream_t st, const QView* q,
               float* sc_out) {
    ms->perm = reinterpret_cast<int32_t*>(ws);
    ms->off = reinterpret_cast<int32_t*>(ws + align256(size_t(M) * 4));
    ms->seg = reinterpret_cast<int32_t*>(ws + align256(size_t(M) * 4) + align256(size_t(n_ad + 2) * 4));
    ms->n_ad = n_ad;
    ms->bound = int(cdiv(M, SEG)) + n_ad + 1;  // segments: at most one partial per bucket
    const bool scales = q && q->dq && sc_out;
    const int64_t nblk = scales ? q->rows * q->cols / 64 : 0;
    const unsigned extra = scales ? unsigned(std::min<int64_t>(cdiv(nblk, 4096), 1024)) : 0u;
    hipLaunchKernelGGL(k_multi_sort, dim3(1 + extra), dim3(1024), 0, st, ids, int(M), n_ad, ms->perm, ms->off,
                       ms->seg, scales ? *q : QView{}, nblk, sc_out);
    return hipPeekAtLastError() == hipSuccess ? NF4_OK : launch_status();
}

int multi_down_seg(const MultiSort& ms, const uint16_t* x, int64_t K, const uint16_t* Ab, int r,
                   const float* scales, float* su, hipStream_t st) {
    // sixteen waves per segment: the segments alone are fewer than the CUs
    const dim3 grid(unsigned(ms.bound));
    if (r <= 16)
        hipLaunchKernelGGL((k_multi_down_seg<1, 16>), grid, dim3(1024), 0, st, x, K, Ab, ms.n_ad, r, scales, ms.perm,
                           ms.off, ms.seg, su);
    else if (r <= 32)
        hipLaunchKernelGGL((k_multi_down_seg<2, 16>), grid, dim3(1024), 0, st, x, K, Ab, ms.n_ad, r, scales, ms.perm,
                           ms.off, ms.seg, su);
    else
        hipLaunchKernelGGL((k_multi_down_seg<4, 16>), grid, dim3(1024), 0, st, x, K, Ab, ms.n_ad, r, scales, ms.perm,
                           ms.off, ms.seg, su);
    return hipPeekAtLastError() == hipSuccess ? NF4_OK : launch_status();
}

int multi_fin_seg(const MultiSort& ms, const float* part, int Z, int64_t M, int64_t N, const float* su, int r,
                  const uint16_t* Bb, uint16_t* h, hipStream_t st) {
    const dim3 grid(unsigned(ms.bound), unsigned(cdiv(N, 256)));
    if (r <= 16)
        hipLaunchKernelGGL(k_multi_fin_seg<16>, grid, dim3(256), 0, st, part, Z, M, N, su, r, Bb, ms.n_ad, ms.perm,
                           ms.off, ms.seg, h);
    else if (r <= 32)
        hipLaunchKernelGGL(k_multi_fin_seg<32>, grid, dim3(256), 0, st, part, Z, M, N, su, r, Bb, ms.n_ad, ms.perm,
                           ms.off, ms.seg, h);
    else
        hipLaunchKernelGGL(k_multi_fin_seg<64>, grid, dim3(256), 0, st, part, Z, M, N, su, r, Bb, ms.n_ad, ms.perm,
                           ms.off, ms.seg, h);
    return hipPeekAtLastError() == hipSuccess ? NF4_OK : launch_status();
}

}  // namespace nf4
