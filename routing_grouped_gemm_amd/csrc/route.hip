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
//      computes the softmax over the selected logits, and counts its block's
//      64 tokens' pairs per expert (the block histogram, stored expert-major).
//   2. route_scan_kernel (one workgroup per expert): exclusive prefix sums
//      along each expert's row of block histograms (-> each block's first
//      rank per expert) and the expert's count.
//   3. route_finalize_kernel (one workgroup per block of 64 tokens): the
//      expert offsets (exclusive scan of counts), then each pair's rank among
//      its block's earlier pairs of the same expert -- found with a few wave
//      ballots, one per bit of the expert index, that give each lane the
//      mask of lanes holding its expert -- and dst_row = offsets[e] + block
//      base + rank (or the padded row), src_slot as its inverse, padding rows
//      -1.  The ranks are recomputed here rather than stored by kernel 1.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int TB = kRouteTokensPerBlock;

// maximum of a 64-bit value over aligned segments of L lanes (L a power of
// two <= 64), every lane of a segment ending with it.  Within 16 lanes the
// exchanges are DPP lane permutations (a maximum needs only some pairing per
// step, not xor: quad swaps, then mirrored half-rows and rows); wider
// segments exchange through ds_bpermute.
template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t x)
{
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)x, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(x >> 32), CTRL, 0xF, 0xF, false);
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

template <int L>
__device__ __forceinline__ uint64_t segment_max(uint64_t x)
{
    auto mx = [](uint64_t a, uint64_t b) __attribute__((always_inline)) { return a > b ? a : b; };
    if constexpr (L >= 2) x = mx(x, dpp64<0xB1>(x));     // quad_perm [1,0,3,2]
    if constexpr (L >= 4) x = mx(x, dpp64<0x4E>(x));     // quad_perm [2,3,0,1]
    if constexpr (L >= 8) x = mx(x, dpp64<0x141>(x));    // row_half_mirror
    if constexpr (L >= 16) x = mx(x, dpp64<0x140>(x));   // row_mirror
#pragma unroll
    for (int off = 16; off < L; off <<= 1) {
        const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)x, off, 64);
        const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(x >> 32), off, 64);
        x = mx(x, ((uint64_t)hi << 32) | lo);
    }
    return x;
}

// LPT lanes per token (power of two, <= 64); lane l of a token's segment owns
// the VPL consecutive logits [l*VPL, l*VPL + VPL) (E <= LPT*VPL).  A block of
// NTHR = min(TB * LPT, 1024) threads handles TB tokens, NTHR/LPT at a time
// (all of them at once up to 16 lanes per token).
// FULL: E == LPT * VPL, so every lane's logits lie inside the row (no
// per-logit range test).
template <int LPT, int VPL, int NTHR = (TB * LPT < 1024 ? (TB * LPT < 64 ? 64 : TB * LPT) : 1024), bool FULL = false>
__global__ __launch_bounds__(NTHR) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int nblk,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w,
                                                         int32_t* __restrict__ hist,
                                                         int32_t* __restrict__ dev_err)
{
    constexpr int TPI = NTHR / LPT;  // tokens handled concurrently by the block
    __shared__ int s_hist[kMaxExperts];

    const int tid = threadIdx.x;
    const int lane = tid % LPT;
    const int seg = tid / LPT;
    // 16-byte loads of whole lane ranges when every row start is 16-byte aligned
    const bool vec = (E % 4) == 0 && (VPL % 4) == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0;

    for (int e = tid; e < E; e += NTHR) s_hist[e] = 0;
    __syncthreads();

    bool bad = false;
    const int t0 = blockIdx.x * TB;
    const int nt = min(TB, T - t0);
    for (int tl = seg; tl < TB; tl += TPI) {
        const int t = t0 + tl;
        const bool active = tl < nt;
        const int e0 = lane * VPL;
        float v[VPL];
        if (vec && active && (FULL || e0 + VPL <= E)) {
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
                v[s] = active && (FULL || e0 + s < E) ? logits[(int64_t)t * E + e0 + s] : -INFINITY;
        }
        // one 64-bit key per logit: the high word orders the fp32 values as
        // unsigned integers (-0 taken as +0, non-finite as -inf), the low
        // word is ~e, so a larger key is a larger logit or, for equal
        // logits, a lower expert index.  Logits past E get key 0, below
        // every real one.
        uint64_t key[VPL];
#pragma unroll
        for (int s = 0; s < VPL; ++s) {
            const bool in = FULL || e0 + s < E;
            float x = v[s];
            if (active && in && !__builtin_isfinite(x)) bad = true;
            x = __builtin_isfinite(x) ? x : -INFINITY;
            uint32_t u = __float_as_uint(x);
            u = (u << 1) == 0 ? 0u : u;                       // -0 -> +0
            const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
            key[s] = in ? ((uint64_t)ord << 32) | (uint32_t)~(uint32_t)(e0 + s) : 0ull;
        }
        // k rounds: each lane's best key below the previous winner, then the
        // segment's maximum (keys are distinct, so nothing is taken twice)
        uint64_t thr = ~0ull;
        float sel_v[kMaxTopK];
        int sel_i[kMaxTopK];
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j) {
            if (j < k) {
                uint64_t best = 0;
#pragma unroll
                for (int s = 0; s < VPL; ++s) best = ((key[s] < thr) & (key[s] > best)) ? key[s] : best;
                best = segment_max<LPT>(best);
                thr = best;
                const uint32_t hi = (uint32_t)(best >> 32);
                sel_v[j] = __uint_as_float((hi & 0x80000000u) ? (hi & 0x7fffffffu) : ~hi);
                sel_i[j] = (int)~(uint32_t)best;
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
                    atomicAdd(&s_hist[sel_i[j]], 1);   // integer count: order-independent
                }
            }
        }
    }
    if (bad && dev_err) atomicOr(dev_err, (int)MOE_ERR_NONFINITE_LOGIT);
    __syncthreads();
    // expert-major: hist[e][block]
    for (int e = tid; e < E; e += NTHR) hist[(int64_t)e * nblk + blockIdx.x] = s_hist[e];
}

// One workgroup of SNT threads per expert: hist [E, nblk] (expert-major) is
// replaced by its exclusive prefix along each expert's row (the first rank
// of each block per expert) and counts[e] is the row total.  Per chunk of
// SNT * SCH blocks (all of a 2^20-token batch's 16384 in one pass) each
// thread sums SCH consecutive entries (all loads in flight together), the
// wave sums are scanned through LDS, and the chunk's total carries into the
// next.
constexpr int SCH = 16, SNT = 1024;
__global__ __launch_bounds__(SNT) void route_scan_kernel(int32_t* __restrict__ hist, int nblk,
                                                         int E, int32_t* __restrict__ counts)
{
    constexpr int NWS = SNT / 64;
    __shared__ int s_w[NWS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int e = blockIdx.x;
    int32_t* row = hist + (int64_t)e * nblk;
    const bool vec = (nblk & 3) == 0 && (reinterpret_cast<uintptr_t>(hist) & 15) == 0;
    int carry = 0;
    for (int c0 = 0; c0 < nblk; c0 += SNT * SCH) {
        const int b0 = c0 + tid * SCH;
        int v[SCH];
        if (vec && b0 + SCH <= nblk) {       // whole 16-byte vectors
#pragma unroll
            for (int q = 0; q < SCH / 4; ++q) {
                const int4 w = reinterpret_cast<const int4*>(row + b0)[q];
                v[4 * q] = w.x;
                v[4 * q + 1] = w.y;
                v[4 * q + 2] = w.z;
                v[4 * q + 3] = w.w;
            }
        } else {
#pragma unroll
            for (int q = 0; q < SCH; ++q) v[q] = b0 + q < nblk ? row[b0 + q] : 0;
        }
        int sum = 0;
#pragma unroll
        for (int q = 0; q < SCH; ++q) sum += v[q];
        int incl = sum;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int o = __shfl_up(incl, off, 64);
            if (lane >= off) incl += o;
        }
        if (lane == 63) s_w[wave] = incl;
        __syncthreads();
        int before = carry, chunk = 0;
#pragma unroll
        for (int w = 0; w < NWS; ++w) {
            if (w < wave) before += s_w[w];
            chunk += s_w[w];
        }
        int run = before + incl - sum;
        if (vec && b0 + SCH <= nblk) {
#pragma unroll
            for (int q = 0; q < SCH / 4; ++q) {
                int4 w;
                w.x = run;
                run += v[4 * q];
                w.y = run;
                run += v[4 * q + 1];
                w.z = run;
                run += v[4 * q + 2];
                w.w = run;
                run += v[4 * q + 3];
                reinterpret_cast<int4*>(row + b0)[q] = w;
            }
        } else {
#pragma unroll
            for (int q = 0; q < SCH; ++q) {
                if (b0 + q < nblk) row[b0 + q] = run;
                run += v[q];
            }
        }
        carry += chunk;
        __syncthreads();   // s_w is rewritten by the next chunk
    }
    if (tid == 0) counts[e] = carry;
}

// exclusive scan of counts[0..E) into s_off[0..E] by one block of NT threads
template <int NT>
__device__ __forceinline__ void block_offsets(const int32_t* __restrict__ counts, int E, int* s_off,
                                              int* s_wsum)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int PER = kMaxExperts / NT;    // counts per thread
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
    if (tid == NT - 1) s_off[E] = run;   // the last thread ends on the grand total
    __syncthreads();
}

// One workgroup per route block: S consecutive histogram blocks of TB tokens,
// whose pairs are a contiguous run of the pair index, taken as chunks of 64
// (FT threads; wave w takes chunks w, w + 8, ...).
//  - Every chunk's expert indices are loaded first (one memory round trip).
//  - A pair's rank among the route block's earlier pairs of the same expert:
//    per chunk, one wave ballot per bit of the expert index gives each lane
//    the mask of the chunk's lanes with its expert (its population below the
//    lane is the rank in the chunk, its first lane records the chunk's count
//    of that expert); one thread per expert then turns the per-chunk counts
//    into prefixes over the chunks, whose total is the block's count of the
//    expert, and X is the exclusive scan of those totals over the experts.
//  - dst_row = offsets[e] + base[e][block] + rank (or e * C + rank when below
//    the capacity C, else -1) goes out per pair (offsets = exclusive scan of
//    counts, block 0 stores them); the pair is also placed at X[e] + rank in
//    LDS, so that src_slot leaves as one run of consecutive rows per expert
//    instead of a scatter.
//  - With C > 0 every row of [e * C + counts[e], (e + 1) * C) gets src_slot
//    -1 (grid-stride).
constexpr int FT = TB * kMaxTopK;   // 512 threads
__global__ __launch_bounds__(FT) void route_finalize_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ base, int32_t* __restrict__ offsets,
    const int32_t* __restrict__ counts, int T, int E, int k, int C, int nsub, int S, int nbits,
    int32_t* __restrict__ dst_row, int32_t* __restrict__ src_slot)
{
    constexpr int NWF = FT / 64;
    constexpr int CPW = kRouteMaxPairsPerBlock / FT;     // chunks per wave, at most
    __shared__ int s_off[kMaxExperts + 1];
    __shared__ int s_x[kMaxExperts + 1];
    __shared__ int s_wsum[NWF];
    __shared__ int s_tot[kMaxExperts];
    __shared__ int s_cnt[kRouteMaxChunkCounts];          // [chunk][expert]
    __shared__ int s_pair[kRouteMaxPairsPerBlock];
    __shared__ uint16_t s_e[kRouteMaxPairsPerBlock];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.x;
    const int sb0 = b * S;                               // first histogram block
    const int64_t p0 = (int64_t)sb0 * TB * k;            // first pair
    const int64_t PB64 = sb0 < nsub ? min((int64_t)S * TB, (int64_t)T - (int64_t)sb0 * TB) * k : 0;
    const int PB = (int)(PB64 > 0 ? PB64 : 0);           // pairs of this route block
    const int nch = (PB + 63) / 64;
    int ev[CPW];
#pragma unroll
    for (int q = 0; q < CPW; ++q) {
        const int p = (wave + q * NWF) * 64 + lane;
        ev[q] = p < PB ? topk_idx[p0 + p] : 0;
    }
    for (int q = tid; q < nch * E; q += FT) s_cnt[q] = 0;
    block_offsets<FT>(counts, E, s_off, s_wsum);         // (its barriers also order the clearing above)
    if (b == 0)
        for (int e = tid; e <= E; e += FT) offsets[e] = s_off[e];
    // per chunk: rank in the chunk, chunk count per expert
    int rk[CPW];
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int q = 0; q < CPW; ++q) {
        const int c = wave + q * NWF;
        const bool valid = c * 64 + lane < PB;
        const int e = ev[q];
        uint64_t same = __ballot(valid);
        for (int bit = 0; bit < nbits; ++bit) {
            const uint64_t on = __ballot(valid && ((e >> bit) & 1));
            same &= ((e >> bit) & 1) ? on : ~on;
        }
        rk[q] = __popcll(same & below);
        if (valid && rk[q] == 0) s_cnt[c * E + e] = __popcll(same);
    }
    __syncthreads();
    // per expert: prefixes over the chunks and the block's total
    for (int e = tid; e < E; e += FT) {
        int run = 0;
        for (int c = 0; c < nch; ++c) {
            const int v = s_cnt[c * E + e];
            s_cnt[c * E + e] = run;
            run += v;
        }
        s_tot[e] = run;
    }
    __syncthreads();
    // one histogram block (small batches): runs of a pair or two per expert,
    // src_slot is written straight from each pair
    const bool staged = S > 1;
    if (staged) block_offsets<FT>(s_tot, E, s_x, s_wsum);   // LDS source; its barriers order the reads
#pragma unroll
    for (int q = 0; q < CPW; ++q) {
        const int c = wave + q * NWF;
        const int p = c * 64 + lane;
        if (p < PB) {
            const int e = ev[q];
            const int loc = s_cnt[c * E + e] + rk[q];
            const int rank = base[(int64_t)e * nsub + sb0] + loc;
            int64_t dst;
            if (C > 0) dst = rank < C ? (int64_t)e * C + rank : -1;
            else dst = (int64_t)s_off[e] + rank;
            dst_row[p0 + p] = (int32_t)dst;
            if (staged) {
                s_pair[s_x[e] + loc] = (int32_t)(p0 + p);
                s_e[s_x[e] + loc] = (uint16_t)e;
            } else if (dst >= 0) {
                src_slot[dst] = (int32_t)(p0 + p);
            }
        }
    }
    if (staged) __syncthreads();
    // src_slot, one run of consecutive rows per expert
    for (int q = tid; staged && q < PB; q += FT) {
        const int e = s_e[q];
        const int rank = base[(int64_t)e * nsub + sb0] + (q - s_x[e]);
        int64_t dst;
        if (C > 0) dst = rank < C ? (int64_t)e * C + rank : -1;
        else dst = (int64_t)s_off[e] + rank;
        if (dst >= 0) src_slot[dst] = s_pair[q];
    }
    if (C > 0) {
        const int64_t rows = (int64_t)E * C;
        for (int64_t r = (int64_t)b * FT + tid; r < rows; r += (int64_t)gridDim.x * FT) {
            const int ee = (int)(r / C), rr = (int)(r % C);
            if (rr >= counts[ee]) src_slot[r] = -1;
        }
    }
}

template <int LPT, int VPL>
void launch_topk(int nblk, hipStream_t s, const float* logits, int T, int E, int k,
                 int32_t* topk_idx, float* topk_w, int32_t* hist, int32_t* dev_err)
{
    constexpr int NTHR = TB * LPT < 1024 ? (TB * LPT < 64 ? 64 : TB * LPT) : 1024;
    if (E == LPT * VPL)
        hipLaunchKernelGGL((route_topk_kernel<LPT, VPL, NTHR, true>), dim3(nblk), dim3(NTHR), 0, s, logits, T, E,
                           k, nblk, topk_idx, topk_w, hist, dev_err);
    else
        hipLaunchKernelGGL((route_topk_kernel<LPT, VPL, NTHR>), dim3(nblk), dim3(NTHR), 0, s, logits, T, E,
                           k, nblk, topk_idx, topk_w, hist, dev_err);
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
                        int32_t* src_slot, int64_t n_rows, int32_t* hist, int32_t* dev_err, hipStream_t s)
{
    (void)n_rows;
    const int S = route_subblocks(T, E, k);    // histogram blocks per finalize workgroup
    const int nblk = (T + TB - 1) / TB;          // histogram blocks (top-k workgroups)
    if (nblk > 0) {
        // 16 logits per lane (8 below 9 experts): a token's segment is E/16 lanes
        if (E <= 8) launch_topk<1, 8>(nblk, s, logits, T, E, k, topk_idx, topk_w, hist, dev_err);
        else if (E <= 16) launch_topk<1, 16>(nblk, s, logits, T, E, k, topk_idx, topk_w, hist, dev_err);
        else if (E <= 32) launch_topk<2, 16>(nblk, s, logits, T, E, k, topk_idx, topk_w, hist, dev_err);
        else if (E <= 64) launch_topk<4, 16>(nblk, s, logits, T, E, k, topk_idx, topk_w, hist, dev_err);
        else if (E <= 128) launch_topk<8, 16>(nblk, s, logits, T, E, k, topk_idx, topk_w, hist, dev_err);
        else if (E <= 256) launch_topk<16, 16>(nblk, s, logits, T, E, k, topk_idx, topk_w, hist, dev_err);
        else if (E <= 512) launch_topk<32, 16>(nblk, s, logits, T, E, k, topk_idx, topk_w, hist, dev_err);
        else launch_topk<64, 16>(nblk, s, logits, T, E, k, topk_idx, topk_w, hist, dev_err);
    }
    // also for T = 0: the scan then writes zero counts
    hipLaunchKernelGGL(route_scan_kernel, dim3((unsigned)E), dim3(SNT), 0, s, hist, nblk, E, counts);
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    // at least one block: it stores the offsets; padded rows beyond the counts
    // are covered grid-stride by however many blocks there are
    const int nroute = (nblk + S - 1) / S;
    const int grid = nroute > 0 ? nroute : 1;
    hipLaunchKernelGGL(route_finalize_kernel, dim3((unsigned)grid), dim3(FT), 0, s, topk_idx, hist, offsets,
                       counts, T, E, k, capacity, nblk, S, nbits, dst_row, src_slot);
    return hipGetLastError();
}

}  // namespace moe
