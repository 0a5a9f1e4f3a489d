// Router top-k and the device route map.
//
// Follows the OLMo-core 3 tutorial's routing-tax section (paragraph on
// GPU-resident routing metadata): per-expert counts, per-expert row offsets
// and the per-expert permutation are produced on the GPU so the loop never
// waits for the host.  Three kernels, all deterministic (no atomics decide
// an order):
//   1. route_topk_kernel: one segment of LPT lanes per token selects the k
//      largest fp32 logits by k rounds of a segmented butterfly arg-max
//      (ties -> lower expert index), computes the softmax over the selected
//      logits, and for its block of 64 tokens the per-expert histogram and
//      each pair's rank among the block's earlier pairs of the same expert.
//   2. route_scan_kernel (one workgroup): column prefix sums of the block
//      histograms (-> each block's base rank per expert), counts, and the
//      exclusive scan of counts (-> offsets).
//   3. route_finalize_kernel: dst_row = offsets[e] + base + local rank (or
//      the padded row), src_slot as its inverse, padding rows -1.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int TB = kRouteTokensPerBlock;

struct Cand {
    float v;
    int i;
};

__device__ __forceinline__ bool better(float v1, int i1, float v2, int i2)
{
    return v1 > v2 || (v1 == v2 && i1 < i2);
}

// LPT lanes per token (power of two, <= 64); VPL logits per lane (E <= LPT*VPL)
template <int LPT, int VPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w,
                                                         int32_t* __restrict__ lrank,
                                                         int32_t* __restrict__ hist,
                                                         int32_t* __restrict__ dev_err)
{
    constexpr int TPI = 256 / LPT;  // tokens handled concurrently by the block
    __shared__ int s_exp[TB * kMaxTopK];
    __shared__ int s_hist[kMaxExperts];

    const int tid = threadIdx.x;
    const int lane = tid % LPT;
    const int seg = tid / LPT;
    const int t0 = blockIdx.x * TB;
    const int nt = min(TB, T - t0);

    for (int e = tid; e < E; e += 256) s_hist[e] = 0;

    bool bad = false;
    for (int tl = seg; tl < TB; tl += TPI) {
        const int t = t0 + tl;
        const bool active = tl < nt;
        float v[VPL];
#pragma unroll
        for (int s = 0; s < VPL; ++s) {
            const int e = lane + s * LPT;
            float x = -INFINITY;
            if (active && e < E) {
                x = logits[(int64_t)t * E + e];
                if (!__builtin_isfinite(x)) {
                    bad = true;
                    x = -INFINITY;
                }
            }
            v[s] = x;
        }
        uint32_t taken = 0;
        float sel_v[kMaxTopK];
        int sel_i[kMaxTopK];
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j) {
            if (j < k) {
                // lane-local best among not-taken valid entries
                float bv = -INFINITY;
                int bi = 0x7fffffff;
#pragma unroll
                for (int s = 0; s < VPL; ++s) {
                    const int e = lane + s * LPT;
                    if (e < E && !(taken & (1u << s)) && better(v[s], e, bv, bi)) {
                        bv = v[s];
                        bi = e;
                    }
                }
                // segmented butterfly arg-max
#pragma unroll
                for (int off = LPT / 2; off > 0; off >>= 1) {
                    const float ov = __shfl_xor(bv, off, 64);
                    const int oi = __shfl_xor(bi, off, 64);
                    if (better(ov, oi, bv, bi)) {
                        bv = ov;
                        bi = oi;
                    }
                }
                if (bi % LPT == lane) taken |= 1u << (bi / LPT);
                sel_v[j] = bv;
                sel_i[j] = bi;
            }
        }
        if (active && lane == 0) {
            // softmax over the selected logits, shifted by the largest
            float ex[kMaxTopK];
            float den = 0.0f;
#pragma unroll
            for (int j = 0; j < kMaxTopK; ++j) {
                ex[j] = 0.0f;
                if (j < k) {
                    const float z = sel_v[0] == -INFINITY ? 0.0f : sel_v[j] - sel_v[0];
                    ex[j] = expf(z);
                    den += ex[j];
                }
            }
#pragma unroll
            for (int j = 0; j < kMaxTopK; ++j) {
                if (j < k) {
                    topk_idx[(int64_t)t * k + j] = sel_i[j];
                    topk_w[(int64_t)t * k + j] = ex[j] / den;
                    s_exp[tl * k + j] = sel_i[j];
                }
            }
        }
    }
    if (bad && dev_err) atomicOr(dev_err, (int)MOE_ERR_NONFINITE_LOGIT);
    __syncthreads();

    // rank of each pair among the block's earlier pairs of the same expert
    const int P = nt * k;
    for (int p = tid; p < P; p += 256) {
        const int e = s_exp[p];
        int r = 0;
        for (int q = 0; q < p; ++q) r += (s_exp[q] == e);
        lrank[(int64_t)t0 * k + p] = r;
        atomicAdd(&s_hist[e], 1);  // integer count: order-independent
    }
    __syncthreads();
    for (int e = tid; e < E; e += 256) hist[(int64_t)blockIdx.x * E + e] = s_hist[e];
}

// One workgroup of 1024 threads.  hist [nblk, E] is replaced by its exclusive
// column prefix (the first rank of each block per expert).
__global__ __launch_bounds__(1024) void route_scan_kernel(int32_t* __restrict__ hist, int nblk,
                                                          int E, int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets)
{
    __shared__ int s_part[1024];
    __shared__ int s_cnt[kMaxExperts];
    __shared__ int s_wsum[16];
    const int tid = threadIdx.x;

    const int ech = E < 1024 ? E : 1024;          // experts per pass
    const int S = 1024 / ech;                     // row segments per expert
    for (int e0 = 0; e0 < E; e0 += ech) {
        const int el = tid % ech;
        const int s = tid / ech;
        const int e = e0 + el;
        const bool act = s < S && e < E;
        const int r0 = (int)((int64_t)nblk * s / S);
        const int r1 = (int)((int64_t)nblk * (s + 1) / S);
        int part = 0;
        if (act)
            for (int r = r0; r < r1; ++r) part += hist[(int64_t)r * E + e];
        s_part[tid] = part;
        __syncthreads();
        if (act) {
            int base = 0, total = 0;
            for (int q = 0; q < S; ++q) {
                const int pv = s_part[q * ech + el];
                if (q < s) base += pv;
                total += pv;
            }
            for (int r = r0; r < r1; ++r) {
                const int c = hist[(int64_t)r * E + e];
                hist[(int64_t)r * E + e] = base;
                base += c;
            }
            if (s == 0) {
                counts[e] = total;
                s_cnt[e] = total;
            }
        }
        __syncthreads();
    }
    // exclusive scan of counts -> offsets (E <= 1024, one value per thread)
    const int wave = tid / 64, lane = tid % 64;
    int v = tid < E ? s_cnt[tid] : 0;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    int wbase = 0;
    for (int w = 0; w < wave; ++w) wbase += s_wsum[w];
    if (tid < E) offsets[tid] = wbase + incl - v;
    if (tid == E - 1) offsets[E] = wbase + incl;
    if (E == 0 && tid == 0) offsets[0] = 0;
}

__global__ __launch_bounds__(256) void route_finalize_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ lrank,
    const int32_t* __restrict__ base, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ counts, int T, int E, int k, int C, int32_t* __restrict__ dst_row,
    int32_t* __restrict__ src_slot, int64_t total)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const int64_t P = (int64_t)T * k;
    if (i < P) {
        const int64_t t = i / k;
        const int e = topk_idx[i];
        const int rank = base[(t / TB) * E + e] + lrank[i];
        int64_t dst;
        if (C > 0) dst = rank < C ? (int64_t)e * C + rank : -1;
        else dst = (int64_t)offsets[e] + rank;
        dst_row[i] = (int32_t)dst;
        if (dst >= 0) src_slot[dst] = (int32_t)i;
    }
    if (C > 0 && i < (int64_t)E * C) {
        const int e = (int)(i / C);
        const int r = (int)(i % C);
        if (r >= counts[e]) src_slot[i] = -1;
    }
}

template <int LPT, int VPL>
void launch_topk(int nblk, hipStream_t s, const float* logits, int T, int E, int k,
                 int32_t* topk_idx, float* topk_w, int32_t* lrank, int32_t* hist,
                 int32_t* dev_err)
{
    hipLaunchKernelGGL((route_topk_kernel<LPT, VPL>), dim3(nblk), dim3(256), 0, s, logits, T, E,
                       k, topk_idx, topk_w, lrank, hist, dev_err);
}

}  // namespace

hipError_t launch_route(const float* logits, int T, int E, int k, int capacity, int32_t* topk_idx,
                        float* topk_w, int32_t* counts, int32_t* offsets, int32_t* dst_row,
                        int32_t* src_slot, int64_t n_rows, int32_t* lrank, int32_t* hist,
                        int32_t* dev_err, hipStream_t s)
{
    const int nblk = (T + TB - 1) / TB;
    if (nblk > 0) {
        if (E <= 8) launch_topk<8, 1>(nblk, s, logits, T, E, k, topk_idx, topk_w, lrank, hist, dev_err);
        else if (E <= 16) launch_topk<16, 1>(nblk, s, logits, T, E, k, topk_idx, topk_w, lrank, hist, dev_err);
        else if (E <= 32) launch_topk<32, 1>(nblk, s, logits, T, E, k, topk_idx, topk_w, lrank, hist, dev_err);
        else if (E <= 64) launch_topk<64, 1>(nblk, s, logits, T, E, k, topk_idx, topk_w, lrank, hist, dev_err);
        else if (E <= 128) launch_topk<64, 2>(nblk, s, logits, T, E, k, topk_idx, topk_w, lrank, hist, dev_err);
        else if (E <= 256) launch_topk<64, 4>(nblk, s, logits, T, E, k, topk_idx, topk_w, lrank, hist, dev_err);
        else if (E <= 512) launch_topk<64, 8>(nblk, s, logits, T, E, k, topk_idx, topk_w, lrank, hist, dev_err);
        else launch_topk<64, 16>(nblk, s, logits, T, E, k, topk_idx, topk_w, lrank, hist, dev_err);
    }
    hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, s, hist, nblk, E, counts, offsets);
    const int64_t P = (int64_t)T * k;
    const int64_t total = capacity > 0 ? (P > n_rows ? P : n_rows) : P;
    if (total > 0) {
        const int64_t grid = (total + 255) / 256;
        hipLaunchKernelGGL(route_finalize_kernel, dim3((unsigned)grid), dim3(256), 0, s, topk_idx,
                           lrank, hist, offsets, counts, T, E, k, capacity, dst_row, src_slot,
                           total);
    }
    return hipGetLastError();
}

}  // namespace moe
