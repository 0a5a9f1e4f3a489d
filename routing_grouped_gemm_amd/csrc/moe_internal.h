// Internal declarations shared by the HIP sources of libmoe (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// ---------------------------------------------------------------- bf16 helpers
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// fp32 -> bf16, round to nearest even, NaN kept quiet
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// ---------------------------------------------------------------- E4M3FN / E8M0
// fp32 -> E4M3FN, round to nearest even, saturating to +-448, NaN -> 0x7F.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v)
{
    uint32_t u = __float_as_uint(v);
    uint32_t sign = (u >> 24) & 0x80u;
    u &= 0x7fffffffu;
    if (u > 0x7f800000u) return 0x7fu;
    float a = __uint_as_float(u);
    if (a >= 448.0f) return sign | 0x7eu;
    if (a < 0.015625f) {                               // below 2^-6: subnormal grid 2^-9
        uint32_t q = (uint32_t)__builtin_rintf(a * 512.0f);   // 0..8, 8 = 2^-6
        return sign | q;
    }
    int ex = (int)(u >> 23) - 127;                     // -6 .. 8
    uint32_t mant = u & 0x7fffffu;
    uint32_t r = mant + 0x7ffffu + ((mant >> 20) & 1u);
    ex += (int)(r >> 23);
    uint32_t m3 = (r >> 20) & 7u;
    if (ex > 8 || (ex == 8 && m3 > 6)) return sign | 0x7eu;
    return sign | ((uint32_t)(ex + 7) << 3) | m3;
}

// smallest e in [-127, 127] with amax <= 448 * 2^e (amax >= 0); an infinite
// block maximum takes the largest exponent
__device__ __forceinline__ int mx_scale_exp(float amax)
{
    if (!(amax > 0.0f)) return -127;
    if (!(amax <= 3.402823466e38f)) return 127;
    // amax = m * 2^E, m in [1,2) (subnormal amax handled by frexp)
    int E;
    float m = __builtin_frexpf(amax, &E);              // amax = m * 2^E, m in [0.5, 1)
    // 448 * 2^e >= amax  <=>  e >= log2(amax / 448) = E - 1 + log2(2m) - log2(1.75) - 8
    int e = E - 9 + ((2.0f * m) > 1.75f ? 1 : 0);
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

// ---------------------------------------------------------------- device tile schedule
// Group g owns rows [goff(g), goff(g+1)): group_off[g], or g*capacity when
// capacity > 0.  Values are clamped to [0, n_rows] so that a corrupt offsets
// array can never move a tile outside the row buffer.
__device__ __forceinline__ int64_t group_begin(const int32_t* group_off, int capacity, int g,
                                               int64_t n_rows)
{
    const int64_t v = capacity > 0 ? (int64_t)g * capacity : (int64_t)group_off[g];
    return v < 0 ? 0 : (v > n_rows ? n_rows : v);
}

// rows of group g (never negative)
__device__ __forceinline__ int64_t group_rows(const int32_t* group_off, int capacity, int g,
                                              int64_t n_rows)
{
    const int64_t m = group_begin(group_off, capacity, g + 1, n_rows) -
                      group_begin(group_off, capacity, g, n_rows);
    return m > 0 ? m : 0;
}

// Block-wide exclusive prefix over groups of ceil(m_g / tile) * mult, written
// to s_pref[0..E] (s_pref[E] = total).  s_part needs NT ints.  All NT threads
// of the block must call it.  E <= 1024.
template <int NT>
__device__ int block_tile_prefix(const int32_t* group_off, int capacity, int E, int64_t n_rows,
                                 int tile, int mult, int* s_pref, int* s_part)
{
    const int tid = threadIdx.x;
    const int per = (E + NT - 1) / NT;
    const int g0 = tid * per;
    int local = 0;
    for (int g = g0; g < g0 + per && g < E; ++g)
        local += (int)((group_rows(group_off, capacity, g, n_rows) + tile - 1) / tile) * mult;
    s_part[tid] = local;
    __syncthreads();
    // Hillis-Steele inclusive scan over NT partial sums
    for (int off = 1; off < NT; off <<= 1) {
        const int v = tid >= off ? s_part[tid - off] : 0;
        __syncthreads();
        s_part[tid] += v;
        __syncthreads();
    }
    int run = s_part[tid] - local;
    for (int g = g0; g < g0 + per && g < E; ++g) {
        s_pref[g] = run;
        run += (int)((group_rows(group_off, capacity, g, n_rows) + tile - 1) / tile) * mult;
    }
    if (tid == NT - 1) s_pref[E] = s_part[NT - 1];
    __syncthreads();
    return s_pref[E];
}

// the group g with s_pref[g] <= L < s_pref[g+1] (0 <= L < s_pref[E]): the
// largest g with s_pref[g] <= L, which skips empty groups
__device__ __forceinline__ int find_group(const int* s_pref, int E, int L)
{
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_pref[mid] <= L) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// ---------------------------------------------------------------- launch helpers
constexpr int kRouteTokensPerBlock = 64;
// The route's finalize handles S histogram blocks of 64 tokens per
// workgroup: S = 1 below 65536 tokens, else as many as keep its pairs within
// kRouteMaxPairsPerBlock (at most 16), so that large batches write their
// source slots in fewer, longer per-expert runs of destination rows.
constexpr int kRouteMaxPairsPerBlock = 4096;
constexpr int kRouteMaxChunkCounts = 8192;   // (pairs / 64) x experts of one finalize workgroup
inline int route_subblocks(int64_t T, int E, int k)
{
    if (T < 65536) return 1;
    int s = kRouteMaxPairsPerBlock / (kRouteTokensPerBlock * k);
    const int s2 = kRouteMaxChunkCounts / (k * E);
    s = s < s2 ? s : s2;
    return s < 16 ? (s < 1 ? 1 : s) : 16;
}

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 8;
constexpr int kMxColPad = 128;   // column-wise MXFP8 groups are padded to this many rows
// Leading bytes of a grouped-GEMM workspace that hold the weight-gradient
// launch's control words (written by a small kernel ahead of the launch).
constexpr size_t kGemmCtlBytes = 256;

inline hipStream_t as_stream(moe_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

// route
hipError_t launch_route(const float* logits, int T, int E, int k, int capacity, int32_t* topk_idx,
                        float* topk_w, int32_t* counts, int32_t* offsets, int32_t* dst_row,
                        int32_t* src_slot, int64_t n_rows, int32_t* hist,
                        int32_t* dev_err, hipStream_t stream);
hipError_t launch_route_add_shared(const int32_t* idx_in, const float* w_in, const int32_t* dst_in,
                                   const int32_t* counts_in, const int32_t* offsets_in,
                                   const int32_t* src_in, int T, int E, int k, int S, int capacity,
                                   int64_t R, int32_t* idx_out, float* w_out, int32_t* counts_out,
                                   int32_t* offsets_out, int32_t* dst_out, int32_t* src_out, hipStream_t s);
// permute / combine / quantise
hipError_t launch_permute(int dtype, const void* x, int T, int d, int k, const int32_t* dst_row,
                          const int32_t* src_slot, const float* row_scale, int64_t n_rows,
                          void* x_perm, uint8_t* x_scales, int32_t* dev_err, hipStream_t stream);
hipError_t launch_combine(int dtype, const void* y_perm, const int32_t* dst_row, const float* w,
                          int T, int k, int d, int64_t n_rows, void* out, int32_t* dev_err,
                          hipStream_t stream);
hipError_t launch_quantize_rows(const uint16_t* src, int64_t rows, int K, uint8_t* codes,
                                uint8_t* scales, hipStream_t stream);
hipError_t launch_quantize_cols(const uint16_t* src, int64_t rows, int K, const int32_t* group_off,
                                int capacity, int n_groups, uint8_t* codes, uint8_t* scales,
                                hipStream_t stream);
hipError_t launch_dequant_requant_cols(const uint8_t* codes_row, const uint8_t* scales_row,
                                       int64_t rows, int K, const int32_t* group_off,
                                       int capacity, int n_groups, uint8_t* codes,
                                       uint8_t* scales, hipStream_t stream);

// router scores and the gradient through the gate weights
hipError_t launch_router_logits(const uint16_t* x, const uint16_t* w, int T, int E, int d, float* logits,
                                hipStream_t s);
hipError_t launch_gate_grad(const void* dout, const void* y_perm, const int32_t* topk_idx,
                            const float* topk_w, const int32_t* dst_row, int T, int E, int k, int d,
                            int64_t n_rows, float* dlogits, float* dw, void* dy_perm, int32_t* dev_err,
                            hipStream_t stream);

// grouped GEMMs (bf16 MFMA, fp32 SIMT, MXFP8 MFMA)
struct GroupSpec {
    const int32_t* group_off;  // [E+1] device, or nullptr with capacity > 0
    int capacity;
    int E;
    int64_t n_rows;
};
hipError_t gemm_op_bf16(int op, const moe_gemm_tensors& t, GroupSpec g, int d, int f,
                        hipStream_t s);
hipError_t gemm_op_f32(int op, const moe_gemm_tensors& t, GroupSpec g, int d, int f,
                       hipStream_t s);
size_t gemm_ws_mxfp8(int E, int64_t n_rows, int d, int f);
hipError_t gemm_op_mxfp8(int op, const moe_gemm_tensors& t, GroupSpec g, int d, int f, void* ws,
                         hipStream_t s);

}  // namespace moe
