// Router top-k and the device route map.
//
// Follows the OLMo-core 3 tutorial's routing-tax section (paragraph on
// GPU-resident routing metadata): per-expert counts, per-expert row offsets
// and the per-expert permutation are produced on the GPU so the loop never
// waits for the host.  Three kernels, all deterministic (no atomics decide
// an order):
//   1. route_topk_kernel: one segment of LPT lanes per token (16 logits per
//      lane) selects the k largest fp32 logits by k rounds of a lane-local
//      pass and a segmented butterfly arg-max (ties -> lower expert index),
//      computes the softmax over the selected logits, and for its block of
//      64 tokens the per-expert histogram (stored expert-major) and each
//      pair's rank among the block's earlier pairs of the same expert.
//   2. route_scan_kernel (one workgroup): prefix sums along each expert's
//      row of block histograms (-> each block's base rank per expert),
//      counts, and the exclusive scan of counts (-> offsets).
//   3. route_finalize_kernel: dst_row = offsets[e] + base + local rank (or
//      the padded row), src_slot as its inverse, padding rows -1.
#include <algorithm>

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

// LPT lanes per token (power of two, <= 64); lane l of a token's segment owns
// the VPL consecutive logits [l*VPL, l*VPL + VPL) (E <= LPT*VPL).  A block of
// NTHR = min(TB * LPT, 1024) threads handles TB tokens, NTHR/LPT at a time
// (all of them at once up to 16 lanes per token).
template <int LPT, int VPL, int NTHR = (TB * LPT < 1024 ? (TB * LPT < 64 ? 64 : TB * LPT) : 1024)>
__global__ __launch_bounds__(NTHR) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int nblk,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w,
                                                         int32_t* __restrict__ lrank,
                                                         int32_t* __restrict__ hist,
                                                         int32_t* __restrict__ dev_err)
{
    constexpr int TPI = NTHR / LPT;  // tokens handled concurrently by the block
    static_assert(VPL <= 32, "taken mask");
    __shared__ int s_exp[TB * kMaxTopK];
    __shared__ int s_hist[kMaxExperts];

    const int tid = threadIdx.x;
    const int lane = tid % LPT;
    const int seg = tid / LPT;
    const int t0 = blockIdx.x * TB;
    const int nt = min(TB, T - t0);
    // 16-byte loads of whole lane ranges when every row start is 16-byte aligned
    const bool vec = (E % 4) == 0 && (VPL % 4) == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0;

    for (int e = tid; e < E; e += NTHR) s_hist[e] = 0;

    bool bad = false;
    for (int tl = seg; tl < TB; tl += TPI) {
        const int t = t0 + tl;
        const bool active = tl < nt;
        const int e0 = lane * VPL;
        float v[VPL];
        if (vec && active && e0 + VPL <= E) {
            const float4* src = reinterpret_cast<const float4*>(logits + (int64_t)t * E + e0);
#pragma unroll
            for (int s = 0; s < VPL / 4; ++s) {
                const float4 q = src[s];
                v[4 * s] = q.x;
                v[4 * s + 1] = q.y;
                v[4 * s + 2] = q.z;
                v[4 * s + 3] = q.w;
            }
        } else {
#pragma unroll
            for (int s = 0; s < VPL; ++s)
                v[s] = active && e0 + s < E ? logits[(int64_t)t * E + e0 + s] : -INFINITY;
        }
#pragma unroll
        for (int s = 0; s < VPL; ++s) {
            if (active && e0 + s < E && !__builtin_isfinite(v[s])) bad = true;
            if (!__builtin_isfinite(v[s])) v[s] = -INFINITY;
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
                    const int e = e0 + s;
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
                if (bi / VPL == lane) taken |= 1u << (bi % VPL);
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
    for (int p = tid; p < P; p += NTHR) {
        const int e = s_exp[p];
        int r = 0;
        for (int q = 0; q < p; ++q) r += (s_exp[q] == e);
        lrank[(int64_t)t0 * k + p] = r;
        atomicAdd(&s_hist[e], 1);  // integer count: order-independent
    }
    __syncthreads();
    // expert-major: hist[e][block]
    for (int e = tid; e < E; e += NTHR) hist[(int64_t)e * nblk + blockIdx.x] = s_hist[e];
}

// One wave per expert: hist [E, nblk] (expert-major) is replaced by its
// exclusive prefix along each expert's row (the first rank of each block
// per expert) and counts[e] is the row total.  Each lane takes 8 consecutive
// blocks per chunk of 512, all loads of a chunk in flight together.
__global__ __launch_bounds__(256) void route_scan_kernel(int32_t* __restrict__ hist, int nblk,
                                                         int E, int32_t* __restrict__ counts)
{
    constexpr int CH = 8;
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (e >= E) return;
    int32_t* row = hist + (int64_t)e * nblk;
    int carry = 0;
    for (int c0 = 0; c0 < nblk; c0 += 64 * CH) {
        const int b0 = c0 + lane * CH;
        int v[CH];
#pragma unroll
        for (int q = 0; q < CH; ++q) v[q] = b0 + q < nblk ? row[b0 + q] : 0;
        int sum = 0;
#pragma unroll
        for (int q = 0; q < CH; ++q) sum += v[q];
        // wave inclusive scan of the lane sums
        int incl = sum;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int o = __shfl_up(incl, off, 64);
            if (lane >= off) incl += o;
        }
        int run = carry + incl - sum;
#pragma unroll
        for (int q = 0; q < CH; ++q) {
            if (b0 + q < nblk) row[b0 + q] = run;
            run += v[q];
        }
        carry += __shfl(incl, 63, 64);
    }
    if (lane == 0) counts[e] = carry;
}

// exclusive scan of counts[0..E) into s_off[0..E] by one block of 256 threads
__device__ __forceinline__ void block_offsets(const int32_t* __restrict__ counts, int E, int* s_off,
                                              int* s_wsum)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int PER = kMaxExperts / 256;   // 4 counts per thread
    int v[PER], sum = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int e = tid * PER + q;
        v[q] = e < E ? counts[e] : 0;
        sum += v[q];
    }
    int incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    int run = incl - sum;
    for (int w = 0; w < wave; ++w) run += s_wsum[w];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int e = tid * PER + q;
        if (e < E) s_off[e] = run;
        run += v[q];
    }
    if (tid == 255) s_off[E] = run;   // the last thread ends on the grand total
    __syncthreads();
}

// dst_row / src_slot of every pair; each block first forms the expert
// offsets (exclusive scan of counts) in LDS, block 0 also stores them
__global__ __launch_bounds__(256) void route_finalize_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ lrank,
    const int32_t* __restrict__ base, int32_t* __restrict__ offsets,
    const int32_t* __restrict__ counts, int T, int E, int k, int C, int nblk,
    int32_t* __restrict__ dst_row, int32_t* __restrict__ src_slot, int64_t total)
{
    __shared__ int s_off[kMaxExperts + 1];
    __shared__ int s_wsum[4];
    block_offsets(counts, E, s_off, s_wsum);
    if (blockIdx.x == 0)
        for (int e = threadIdx.x; e <= E; e += 256) offsets[e] = s_off[e];
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const int64_t P = (int64_t)T * k;
    if (i < P) {
        const int64_t t = i / k;
        const int e = topk_idx[i];
        const int rank = base[(int64_t)e * nblk + t / TB] + lrank[i];
        int64_t dst;
        if (C > 0) dst = rank < C ? (int64_t)e * C + rank : -1;
        else dst = (int64_t)s_off[e] + rank;
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
    constexpr int NTHR = TB * LPT < 1024 ? (TB * LPT < 64 ? 64 : TB * LPT) : 1024;
    hipLaunchKernelGGL((route_topk_kernel<LPT, VPL, NTHR>), dim3(nblk), dim3(NTHR), 0, s, logits, T, E,
                       k, nblk, topk_idx, topk_w, lrank, hist, dev_err);
}

// Shared experts as extra groups: every token also takes slots k .. k+S-1,
// expert E + s with weight 1, whose rows follow the routed rows expert by
// expert (row R + s*T + t).  Copies the routed slots into the wider [T, k+S]
// arrays, renumbers the routed rows' source slots (t*k + j -> t*(k+S) + j),
// and extends counts and offsets (offsets become the group starts also in
// the padded layout: e*C for the routed experts).
__global__ __launch_bounds__(256) void route_add_shared_kernel(
    const int32_t* __restrict__ idx_in, const float* __restrict__ w_in, const int32_t* __restrict__ dst_in,
    const int32_t* __restrict__ counts_in, const int32_t* __restrict__ offsets_in,
    const int32_t* __restrict__ src_in, int T, int E, int k, int S, int capacity, int64_t R,
    int32_t* __restrict__ idx_out, float* __restrict__ w_out, int32_t* __restrict__ counts_out,
    int32_t* __restrict__ offsets_out, int32_t* __restrict__ dst_out, int32_t* __restrict__ src_out)
{
    const int KS = k + S;
    const int64_t n_slots = (int64_t)T * KS;
    const int64_t n_rows = R + (int64_t)S * T;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_slots; i += stride) {
        const int64_t t = i / KS;
        const int j = (int)(i - t * KS);
        if (j < k) {
            idx_out[i] = idx_in[t * k + j];
            w_out[i] = w_in[t * k + j];
            dst_out[i] = dst_in[t * k + j];
        } else {
            idx_out[i] = E + (j - k);
            w_out[i] = 1.0f;
            dst_out[i] = (int32_t)(R + (int64_t)(j - k) * T + t);
        }
    }
    for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < n_rows; r += stride) {
        if (r < R) {
            const int32_t p = src_in[r];
            src_out[r] = p < 0 ? -1 : (int32_t)((p / k) * KS + p % k);
        } else {
            const int64_t q = r - R;
            const int64_t t = q % T;
            src_out[r] = (int32_t)(t * KS + k + q / T);
        }
    }
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e <= E + S; e += stride) {
        if (e < E + S) counts_out[e] = e < E ? counts_in[e] : T;
        offsets_out[e] = e <= E ? (capacity > 0 ? (int32_t)(e * capacity) : offsets_in[e])
                                : (int32_t)(R + (e - E) * (int64_t)T);
    }
}

}  // namespace

hipError_t launch_route_add_shared(const int32_t* idx_in, const float* w_in, const int32_t* dst_in,
                                   const int32_t* counts_in, const int32_t* offsets_in,
                                   const int32_t* src_in, int T, int E, int k, int S, int capacity,
                                   int64_t R, int32_t* idx_out, float* w_out, int32_t* counts_out,
                                   int32_t* offsets_out, int32_t* dst_out, int32_t* src_out, hipStream_t s)
{
    const int64_t n = std::max<int64_t>({(int64_t)T * (k + S), R + (int64_t)S * T, (int64_t)E + S + 1});
    const int64_t grid = std::min<int64_t>((n + 255) / 256, 65535);
    hipLaunchKernelGGL(route_add_shared_kernel, dim3((unsigned)grid), dim3(256), 0, s, idx_in, w_in, dst_in,
                       counts_in, offsets_in, src_in, T, E, k, S, capacity, R, idx_out, w_out, counts_out,
                       offsets_out, dst_out, src_out);
    return hipGetLastError();
}

hipError_t launch_route(const float* logits, int T, int E, int k, int capacity, int32_t* topk_idx,
                        float* topk_w, int32_t* counts, int32_t* offsets, int32_t* dst_row,
                        int32_t* src_slot, int64_t n_rows, int32_t* lrank, int32_t* hist,
                        int32_t* dev_err, hipStream_t s)
{
    const int nblk = (T + TB - 1) / TB;
    if (nblk > 0) {
        // 16 logits per lane (8 below 9 experts): a token's segment is E/16 lanes
        if (E <= 8) launch_topk<1, 8>(nblk, s, logits, T, E, k, topk_idx, topk_w, lrank, hist, dev_err);
        else if (E <= 16) launch_topk<1, 16>(nblk, s, logits, T, E, k, topk_idx, topk_w, lrank, hist, dev_err);
        else if (E <= 32) launch_topk<2, 16>(nblk, s, logits, T, E, k, topk_idx, topk_w, lrank, hist, dev_err);
        else if (E <= 64) launch_topk<4, 16>(nblk, s, logits, T, E, k, topk_idx, topk_w, lrank, hist, dev_err);
        else if (E <= 128) launch_topk<8, 16>(nblk, s, logits, T, E, k, topk_idx, topk_w, lrank, hist, dev_err);
        else if (E <= 256) launch_topk<16, 16>(nblk, s, logits, T, E, k, topk_idx, topk_w, lrank, hist, dev_err);
        else if (E <= 512) launch_topk<32, 16>(nblk, s, logits, T, E, k, topk_idx, topk_w, lrank, hist, dev_err);
        else launch_topk<64, 16>(nblk, s, logits, T, E, k, topk_idx, topk_w, lrank, hist, dev_err);
    }
    // also for T = 0: the scan then writes zero counts
    hipLaunchKernelGGL(route_scan_kernel, dim3((unsigned)((E + 3) / 4)), dim3(256), 0, s, hist, nblk, E,
                       counts);
    const int64_t P = (int64_t)T * k;
    const int64_t total = capacity > 0 ? (P > n_rows ? P : n_rows) : P;
    {   // at least one block: it stores the offsets
        const int64_t grid = total > 0 ? (total + 255) / 256 : 1;
        hipLaunchKernelGGL(route_finalize_kernel, dim3((unsigned)grid), dim3(256), 0, s, topk_idx,
                           lrank, hist, offsets, counts, T, E, k, capacity, nblk, dst_row, src_slot,
                           total);
    }
    return hipGetLastError();
}

}  // namespace moe
