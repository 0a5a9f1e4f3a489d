// Rowwise dispatch (permute), un-permute/combine, and the MXFP8 quantisers.
//
// Permute follows the OLMo-core 3 tutorial's "rowwise EP" paragraph: each
// token row is written straight into the row of its expert's input buffer
// given by the route map; there is no pack step.  The kernel reads each
// token row once (16-byte loads) and writes it to its k destinations
// (16-byte stores); the combine reads the k rows of a token and writes one.
// All HBM accesses are whole 16-byte vectors, consecutive lanes on
// consecutive vectors of the same row.
//
// MXFP8 (tutorial, MXFP8 section): one E8M0 scale per 32 elements, the
// smallest power of two that keeps the block maximum within 448, codes by
// round-to-nearest-even into E4M3FN.
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t vu4;   // 16 bytes, for non-temporal access

// 8 x bf16 or 4 x fp32 per 16-byte vector
template <bool BF16>
__device__ __forceinline__ uint4 scale_vec(uint4 v, float s)
{
    if constexpr (BF16) {
        uint4 o;
        o.x = pack_bf16x2(s * bf16_lo(v.x), s * bf16_hi(v.x));
        o.y = pack_bf16x2(s * bf16_lo(v.y), s * bf16_hi(v.y));
        o.z = pack_bf16x2(s * bf16_lo(v.z), s * bf16_hi(v.z));
        o.w = pack_bf16x2(s * bf16_lo(v.w), s * bf16_hi(v.w));
        return o;
    } else {
        uint4 o;
        o.x = __float_as_uint(s * __uint_as_float(v.x));
        o.y = __float_as_uint(s * __uint_as_float(v.y));
        o.z = __float_as_uint(s * __uint_as_float(v.z));
        o.w = __float_as_uint(s * __uint_as_float(v.w));
        return o;
    }
}

// thread i handles vector (i % nvec) of token row (i / nvec).  K (= top-k)
// is a template parameter: the token's K destinations and scales are read
// first, then its K stores go out back to back.  ROW (rows of at least 256
// vectors): one workgroup per token, each thread its vectors tid, tid + 256,
// ...; the destinations and scales are then workgroup-uniform (scalar loads,
// once per token instead of once per vector).
template <bool BF16, bool SCALE, int K, bool ROW = false>
__global__ __launch_bounds__(256) void permute_kernel(const uint4* __restrict__ x, int T, int nvec,
                                                      const int32_t* __restrict__ dst_row,
                                                      const float* __restrict__ row_scale,
                                                      int64_t n_rows, uint4* __restrict__ x_perm,
                                                      int32_t* __restrict__ dev_err)
{
    if constexpr (ROW) {
        const int64_t t = blockIdx.x;
        int32_t dst[K];
        float sc[K];
        bool bad = false;
#pragma unroll
        for (int j = 0; j < K; ++j) {
            dst[j] = dst_row[t * K + j];
            sc[j] = SCALE ? row_scale[t * K + j] : 1.0f;
            bad |= dst[j] >= n_rows;
        }
        for (int v = threadIdx.x; v < nvec; v += 256) {
            const uint4 val = x[t * nvec + v];
#pragma unroll
            for (int j = 0; j < K; ++j)
                if (dst[j] >= 0 && dst[j] < n_rows)
                    x_perm[(int64_t)dst[j] * nvec + v] = SCALE ? scale_vec<BF16>(val, sc[j]) : val;
        }
        if (bad && dev_err && threadIdx.x == 0) atomicOr(dev_err, (int)MOE_ERR_ROW_RANGE);
        return;
    }
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)T * nvec) return;
    const int64_t t = i / nvec;
    const int v = (int)(i - t * nvec);
    int32_t dst[K];
    float sc[K];
#pragma unroll
    for (int j = 0; j < K; ++j) dst[j] = dst_row[t * K + j];
    if constexpr (SCALE) {
#pragma unroll
        for (int j = 0; j < K; ++j) sc[j] = row_scale[t * K + j];
    }
    const uint4 val = x[i];
    bool bad = false;
#pragma unroll
    for (int j = 0; j < K; ++j) {
        bad |= dst[j] >= n_rows;
        if (dst[j] < 0 || dst[j] >= n_rows) continue;
        x_perm[(int64_t)dst[j] * nvec + v] = SCALE ? scale_vec<BF16>(val, sc[j]) : val;
    }
    if (bad && dev_err) atomicOr(dev_err, (int)MOE_ERR_ROW_RANGE);
}

// zero the rows nobody fills (padded layout); 16 rows per block
__global__ __launch_bounds__(256) void zero_rows_kernel(const int32_t* __restrict__ src_slot,
                                                        int64_t n_rows, int nvec,
                                                        uint4* __restrict__ buf,
                                                        uint8_t* __restrict__ scales, int nsc)
{
    const int64_t r0 = (int64_t)blockIdx.x * 16;
    for (int64_t r = r0; r < r0 + 16 && r < n_rows; ++r) {
        if (src_slot[r] >= 0) continue;
        for (int v = threadIdx.x; v < nvec; v += 256) buf[r * nvec + v] = make_uint4(0, 0, 0, 0);
        if (scales)
            for (int b = threadIdx.x; b < nsc; b += 256) scales[r * nsc + b] = 0;
    }
}

// One 32-element block: the scale exponent and the 32 E4M3FN codes (four per
// word, element 4*wi + b in byte b of w[wi]).  When every element is finite
// the scaled values lie within +-448 and the hardware packed conversion
// (round to nearest even) gives the codes; it was checked to agree with
// f32_to_e4m3 on every finite input of magnitude <= 448 tried: each E4M3
// value, each midpoint between neighbours and their fp32 neighbours, and
// four million random values over the range and over scales 2^-20 .. 2^9.
// Blocks with a NaN or an infinity take f32_to_e4m3 (saturation and NaN rules
// of the format).
__device__ __forceinline__ int quant_block32(const float (&vals)[32], uint32_t (&w)[8])
{
    float amax = 0.0f;
    bool finite = true;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const float a = fabsf(vals[i]);
        amax = fmaxf(amax, a);
        finite &= a <= 3.402823466e38f;   // false for NaN and infinities
    }
    const int e = mx_scale_exp(amax);
    if (finite) {
#pragma unroll
        for (int wi = 0; wi < 8; ++wi) {
            // ldexp keeps the exact product even when 2^-e overflows fp32 (e = -127)
            const float q0 = __builtin_ldexpf(vals[wi * 4 + 0], -e), q1 = __builtin_ldexpf(vals[wi * 4 + 1], -e);
            const float q2 = __builtin_ldexpf(vals[wi * 4 + 2], -e), q3 = __builtin_ldexpf(vals[wi * 4 + 3], -e);
            const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
            w[wi] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, lo, true);
        }
    } else {
#pragma unroll
        for (int wi = 0; wi < 8; ++wi) {
            uint32_t word = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) word |= f32_to_e4m3(__builtin_ldexpf(vals[wi * 4 + b], -e)) << (8 * b);
            w[wi] = word;
        }
    }
    return e;
}

// quantise 32 bf16 (four 16-byte vectors) into 32 E4M3FN codes + scale exponent
__device__ __forceinline__ int quant32(const uint4 (&in)[4], uint4 (&out)[2])
{
    float vals[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t w[4] = {in[q].x, in[q].y, in[q].z, in[q].w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            vals[q * 8 + 2 * p] = bf16_lo(w[p]);
            vals[q * 8 + 2 * p + 1] = bf16_hi(w[p]);
        }
    }
    uint32_t c[8];
    const int e = quant_block32(vals, c);
    out[0] = make_uint4(c[0], c[1], c[2], c[3]);
    out[1] = make_uint4(c[4], c[5], c[6], c[7]);
    return e;
}

// MXFP8 dispatch: thread i quantises 32-element block (i % nblk32) of token row
// (i / nblk32) and writes it to the k destinations
__global__ __launch_bounds__(256) void permute_mx_kernel(const uint4* __restrict__ x, int T,
                                                         int nb32, int k,
                                                         const int32_t* __restrict__ dst_row,
                                                         int64_t n_rows, uint4* __restrict__ codes,
                                                         uint8_t* __restrict__ scales,
                                                         int32_t* __restrict__ dev_err)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)T * nb32) return;
    const int64_t t = i / nb32;
    const int b = (int)(i - t * nb32);
    uint4 in[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) in[q] = x[i * 4 + q];
    uint4 out[2];
    const int e = quant32(in, out);
    bool bad = false;
    for (int j = 0; j < k; ++j) {
        const int64_t dst = dst_row[t * k + j];
        if (dst < 0) continue;
        if (dst >= n_rows) {
            bad = true;
            continue;
        }
        codes[(dst * nb32 + b) * 2] = out[0];
        codes[(dst * nb32 + b) * 2 + 1] = out[1];
        scales[dst * nb32 + b] = (uint8_t)(e + 127);
    }
    if (bad && dev_err) atomicOr(dev_err, (int)MOE_ERR_ROW_RANGE);
}

// row-wise quantiser: thread i handles block (i % nb32) of row (i / nb32)
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint4* __restrict__ src,
                                                         int64_t rows, int nb32,
                                                         uint4* __restrict__ codes,
                                                         uint8_t* __restrict__ scales)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= rows * nb32) return;
    uint4 in[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) in[q] = src[i * 4 + q];
    uint4 out[2];
    const int e = quant32(in, out);
    codes[i * 2] = out[0];
    codes[i * 2 + 1] = out[1];
    scales[i] = (uint8_t)(e + 127);
}

// Column-wise quantiser inside row groups.  Each group's rows are padded to a
// multiple of kMxColPad (zero codes) and stored transposed, so that a GEMM
// over the group reads whole 128-element K-steps and 4-byte scale words.
// Block (cb, L): columns [cb*128, cb*128+128) of the L-th 128-row tile in the
// concatenation of all groups' padded rows (device schedule from the group
// offsets).  The tile comes into LDS with coalesced row loads; each thread
// then quantises one column over two of the tile's four 32-row blocks, and
// the codes leave as whole 128-byte runs of the transposed layout (one
// column's 128 rows), eight lanes per run.
template <bool FROM_MX>
__global__ __launch_bounds__(256) void quant_cols_kernel(const uint16_t* __restrict__ src,
                                                         const uint8_t* __restrict__ src_codes,
                                                         const uint8_t* __restrict__ src_scales,
                                                         int64_t rows, int K,
                                                         const int32_t* __restrict__ group_off,
                                                         int capacity, int n_groups,
                                                         uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales)
{
    constexpr int TR = kMxColPad;   // 128 rows per tile
    constexpr int TC = 128;         // columns per tile
    constexpr int EB = FROM_MX ? 1 : 2;   // input bytes per element
    __shared__ int s_pref[kMaxExperts + 1];
    __shared__ int s_part[256];
    // the input tile (row-major); after the quantisation the codes reuse it
    // as [block b][column c][32 rows]
    static_assert(TR * TC * EB >= 4 * TC * 32, "codes fit the input tile");
    __shared__ __align__(16) uint8_t s_in[TR * TC * EB];
    __shared__ uint32_t s_rsc[FROM_MX ? TR : 1];            // FROM_MX: each row's 4 scale bytes
    __shared__ uint8_t s_osc[TC * 4];                       // scales as [column c][block b]
    uint8_t* s_out = s_in;
    int g = 0, rt = blockIdx.y;
    int64_t g0 = 0, g1 = rows, P = 0;
    if (group_off || capacity > 0) {
        const int total = block_tile_prefix<256>(group_off, capacity, n_groups, rows, TR, 1, s_pref, s_part);
        if ((int)blockIdx.y >= total) return;
        g = find_group(s_pref, n_groups, blockIdx.y);
        rt = blockIdx.y - s_pref[g];
        g0 = group_begin(group_off, capacity, g, rows);
        g1 = g0 + group_rows(group_off, capacity, g, rows);
        P = (int64_t)s_pref[g] * TR;              // padded rows of earlier groups
    } else if ((int64_t)rt * TR >= rows) {
        return;
    }
    const int64_t mpad = (g1 - g0 + TR - 1) / TR * TR;
    const int c0 = blockIdx.x * TC;
    const int64_t r0 = g0 + (int64_t)rt * TR;
    const int tid = threadIdx.x;

    // the input tile: TR rows x TC columns (rows past the group and columns
    // past K read as zero), 16 bytes per lane per load
    constexpr int CPR = TC * EB / 16;             // 16-byte chunks per tile row
    constexpr int NLD = TR * CPR / 256;           // loads per thread, all in flight together
    uint4 ld[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        const int q = tid + i * 256;
        const int r = q / CPR, cc = q % CPR;
        const int64_t row = r0 + r;
        const int col = c0 + cc * (16 / EB);
        ld[i] = make_uint4(0, 0, 0, 0);
        if (row < g1 && col < K) {
            if constexpr (FROM_MX)
                ld[i] = *reinterpret_cast<const uint4*>(src_codes + row * K + col);
            else
                ld[i] = *reinterpret_cast<const uint4*>(src + row * K + col);
        }
    }
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        const int q = tid + i * 256;
        *reinterpret_cast<uint4*>(s_in + (q / CPR) * (TC * EB) + (q % CPR) * 16) = ld[i];
    }
    if constexpr (FROM_MX) {
        if (tid < TR) {
            const int64_t row = r0 + tid;
            uint32_t w = 0;
            if (row < g1) {
#pragma unroll
                for (int b = 0; b < TC / 32; ++b) {
                    const int cb = c0 / 32 + b;
                    if (cb < K / 32) w |= (uint32_t)src_scales[row * (K / 32) + cb] << (8 * b);
                }
            }
            s_rsc[tid] = w;
        }
    }
    __syncthreads();

    // one column, 32-row blocks b and b + 2
    const int c = tid % TC;
    uint4 cw[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int b = tid / TC + 2 * h;
        float vals[32];
#pragma unroll
        for (int r = 0; r < 32; ++r) {
            const int rr = b * 32 + r;
            float v;
            if constexpr (FROM_MX) {
                // E4M3FN decode (exact; 0x7F / 0xFF are NaN) times the row's block scale
                const int code = s_in[rr * TC + c];
                const int se = (int)((s_rsc[rr] >> (8 * (c / 32))) & 0xffu) - 127;
                v = __builtin_ldexpf(__builtin_amdgcn_cvt_f32_fp8(code, 0), se);
            } else {
                v = bf16_to_f32(*reinterpret_cast<const uint16_t*>(s_in + rr * (TC * 2) + c * 2));
            }
            vals[r] = v;
        }
        uint32_t w[8];
        const int e = quant_block32(vals, w);
        cw[h][0] = make_uint4(w[0], w[1], w[2], w[3]);
        cw[h][1] = make_uint4(w[4], w[5], w[6], w[7]);
        s_osc[c * 4 + b] = (uint8_t)(e + 127);
    }
    __syncthreads();   // every thread has read its columns: the tile's LDS takes the codes
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        uint4* o = reinterpret_cast<uint4*>(s_out + ((tid / TC + 2 * h) * TC + c) * 32);
        o[0] = cw[h][0];
        o[1] = cw[h][1];
    }
    __syncthreads();

    // codes: column c's 128 rows are one 128-byte run of the group layout
    uint8_t* gcodes = codes + (int64_t)K * P + rt * TR;
#pragma unroll
    for (int q = tid; q < TC * 8; q += 256) {
        const int cc = q / 8, hh = q % 8;          // column, 16-byte piece of its run
        if (c0 + cc < K)
            *reinterpret_cast<uint4*>(gcodes + (int64_t)(c0 + cc) * mpad + hh * 16) =
                *reinterpret_cast<const uint4*>(s_out + ((hh / 2) * TC + cc) * 32 + (hh % 2) * 16);
    }
    if (tid < TC && c0 + tid < K)
        *reinterpret_cast<uint32_t*>(scales + (int64_t)K * P / 32 + (int64_t)(c0 + tid) * (mpad / 32) + rt * 4) =
            *reinterpret_cast<const uint32_t*>(s_osc + tid * 4);
}

// vector v of token t of the combine (flag: this thread reports a row out of range)
template <bool BF16, int K>
__device__ __forceinline__ void combine_vec(const uint4* __restrict__ y, const int32_t* __restrict__ dst_row,
                                            const float* __restrict__ w, int64_t t, int v, int nvec, int64_t n_rows,
                                            uint4* __restrict__ out, int32_t* __restrict__ dev_err, bool flag)
{
    const int64_t i = t * nvec + v;
    constexpr int NE = BF16 ? 8 : 4;
    int32_t dst[K];
    float wt[K];
#pragma unroll
    for (int j = 0; j < K; ++j) dst[j] = dst_row[t * K + j];
#pragma unroll
    for (int j = 0; j < K; ++j) wt[j] = w ? w[t * K + j] : 1.0f;
    // the expert rows are read once and the output written once: both
    // streams are non-temporal (they do not displace what the GEMMs reuse)
    vu4 val[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        val[j] = vu4{0, 0, 0, 0};
        if (dst[j] >= 0 && dst[j] < n_rows)
            val[j] = __builtin_nontemporal_load(reinterpret_cast<const vu4*>(y) + (int64_t)dst[j] * nvec + v);
    }
    float acc[NE];
#pragma unroll
    for (int q = 0; q < NE; ++q) acc[q] = 0.0f;
    bool bad = false;
#pragma unroll
    for (int j = 0; j < K; ++j) {
        bad |= dst[j] >= n_rows;
        if (dst[j] < 0 || dst[j] >= n_rows) continue;
        const uint32_t ww[4] = {val[j][0], val[j][1], val[j][2], val[j][3]};
        if constexpr (BF16) {
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                acc[2 * p] = fmaf(wt[j], bf16_lo(ww[p]), acc[2 * p]);
                acc[2 * p + 1] = fmaf(wt[j], bf16_hi(ww[p]), acc[2 * p + 1]);
            }
        } else {
#pragma unroll
            for (int p = 0; p < 4; ++p) acc[p] = fmaf(wt[j], __uint_as_float(ww[p]), acc[p]);
        }
    }
    vu4 o;
    if constexpr (BF16) {
        o = vu4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                pack_bf16x2(acc[6], acc[7])};
    } else {
        o = vu4{__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                __float_as_uint(acc[3])};
    }
    __builtin_nontemporal_store(o, reinterpret_cast<vu4*>(out) + i);
    if (bad && dev_err && flag) atomicOr(dev_err, (int)MOE_ERR_ROW_RANGE);
}

// thread i makes vector (i % nvec) of token (i / nvec): the K destination
// rows and weights are read first, then the K row loads are all in flight
// before the fp32 accumulation in slot order.  ROW (rows of at least 256
// vectors): one workgroup per token, each thread its vectors tid, tid + 256,
// ... (workgroup-uniform destinations and weights: scalar loads).
template <bool BF16, int K, bool ROW = false>
__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ y,
                                                      const int32_t* __restrict__ dst_row,
                                                      const float* __restrict__ w, int T, int nvec,
                                                      int64_t n_rows, uint4* __restrict__ out,
                                                      int32_t* __restrict__ dev_err)
{
    if constexpr (ROW) {
        for (int v = threadIdx.x; v < nvec; v += 256) combine_vec<BF16, K>(y, dst_row, w, blockIdx.x, v, nvec, n_rows, out,
                                                                          dev_err, threadIdx.x == 0 && v == (int)threadIdx.x);
        return;
    }
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)T * nvec) return;
    combine_vec<BF16, K>(y, dst_row, w, i / nvec, (int)(i - (i / nvec) * nvec), nvec, n_rows, out, dev_err, true);
}


// Gradient through the gate weights (the backward of the weighted combine
// with respect to the weights, then the softmax over the selected logits):
// one wave per token.  Lane i takes the 16-byte vectors i, i + 64, ... of
// the token's dout row and of its K expert rows y_perm[dst]; the K partial
// dot products are summed across the wave; then, with dw_j = <dout, y_j>
// (0 for a dropped slot), dlogits[t, topk_idx[t,j]] = w_j (dw_j - sum_m w_m
// dw_m) and every other entry of the token's row is 0.  FUSE also writes
// the combine backward, dy_perm[dst] = w_j * dout (as the row-scaled permute
// does), from the dout vectors already in registers.
template <int K, bool FUSE>
__global__ __launch_bounds__(256) void gate_grad_kernel(const uint4* __restrict__ dout,
                                                        const uint4* __restrict__ y, int T, int E,
                                                        int nvec, const int32_t* __restrict__ topk_idx,
                                                        const float* __restrict__ topk_w,
                                                        const int32_t* __restrict__ dst_row,
                                                        int64_t n_rows, float* __restrict__ dlogits,
                                                        float* __restrict__ dw_out,
                                                        uint4* __restrict__ dy_perm,
                                                        int32_t* __restrict__ dev_err)
{
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;   // wave-uniform
    const int lane = threadIdx.x & 63;
    int32_t dst[K];
    int idx[K];
    float w[K];
    bool bad = false;
#pragma unroll
    for (int j = 0; j < K; ++j) {
        dst[j] = dst_row[(int64_t)t * K + j];
        idx[j] = topk_idx[(int64_t)t * K + j];
        w[j] = topk_w[(int64_t)t * K + j];
        bad |= dst[j] >= n_rows;
        if (dst[j] >= n_rows) dst[j] = -1;
    }
    float acc[K];
#pragma unroll
    for (int j = 0; j < K; ++j) acc[j] = 0.0f;
    // the expert rows are read once here: non-temporal loads
#pragma unroll 2
    for (int v = lane; v < nvec; v += 64) {
        const uint4 g = dout[(int64_t)t * nvec + v];
        uint4 yv[K];
#pragma unroll
        for (int j = 0; j < K; ++j)
            if (dst[j] >= 0) {
                const vu4 q = __builtin_nontemporal_load(reinterpret_cast<const vu4*>(y) + (int64_t)dst[j] * nvec + v);
                yv[j] = make_uint4(q[0], q[1], q[2], q[3]);
            }
        const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
        for (int j = 0; j < K; ++j) {
            if (dst[j] < 0) continue;
            const uint32_t yw[4] = {yv[j].x, yv[j].y, yv[j].z, yv[j].w};
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                acc[j] = fmaf(bf16_lo(gw[p]), bf16_lo(yw[p]), acc[j]);
                acc[j] = fmaf(bf16_hi(gw[p]), bf16_hi(yw[p]), acc[j]);
            }
            if constexpr (FUSE) dy_perm[(int64_t)dst[j] * nvec + v] = scale_vec<true>(g, w[j]);
        }
    }
#pragma unroll
    for (int j = 0; j < K; ++j)
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) acc[j] += __shfl_xor(acc[j], off, 64);
    float wdw = 0.0f;
#pragma unroll
    for (int j = 0; j < K; ++j) wdw = fmaf(w[j], acc[j], wdw);
    for (int e = lane; e < E; e += 64) {
        float v = 0.0f;
#pragma unroll
        for (int j = 0; j < K; ++j)
            if (idx[j] == e) v = w[j] * (acc[j] - wdw);
        dlogits[(int64_t)t * E + e] = v;
    }
    if (dw_out) {
#pragma unroll
        for (int j = 0; j < K; ++j)
            if (lane == j) dw_out[(int64_t)t * K + j] = acc[j];
    }
    if (bad && lane == 0 && dev_err) atomicOr(dev_err, (int)MOE_ERR_ROW_RANGE);
}

// run f(integral_constant<int, k>) for k in 1..kMaxTopK
template <class F>
hipError_t with_k(int k, F&& f)
{
    switch (k) {
    case 1: f(std::integral_constant<int, 1>{}); break;
    case 2: f(std::integral_constant<int, 2>{}); break;
    case 3: f(std::integral_constant<int, 3>{}); break;
    case 4: f(std::integral_constant<int, 4>{}); break;
    case 5: f(std::integral_constant<int, 5>{}); break;
    case 6: f(std::integral_constant<int, 6>{}); break;
    case 7: f(std::integral_constant<int, 7>{}); break;
    case 8: f(std::integral_constant<int, 8>{}); break;
    default: return hipErrorInvalidValue;
    }
    return hipSuccess;
}

inline unsigned grid_for(int64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

hipError_t launch_permute(int dtype, const void* x, int T, int d, int k, const int32_t* dst_row,
                          const int32_t* src_slot, const float* row_scale, int64_t n_rows,
                          void* x_perm, uint8_t* x_scales, int32_t* dev_err, hipStream_t s)
{
    const bool padded = n_rows != (int64_t)T * k;
    if (dtype == MOE_MXFP8) {
        const int nb32 = d / 32;
        const int64_t n = (int64_t)T * nb32;
        if (n > 0)
            hipLaunchKernelGGL(permute_mx_kernel, dim3(grid_for(n)), dim3(256), 0, s,
                               (const uint4*)x, T, nb32, k, dst_row, n_rows, (uint4*)x_perm,
                               x_scales, dev_err);
        if (padded && n_rows > 0)
            hipLaunchKernelGGL(zero_rows_kernel, dim3((unsigned)((n_rows + 15) / 16)), dim3(256), 0,
                               s, src_slot, n_rows, d / 16, (uint4*)x_perm, x_scales, nb32);
        return hipGetLastError();
    }
    const bool bf = dtype == MOE_BF16;
    const int nvec = bf ? d / 8 : d / 4;
    const int64_t n = (int64_t)T * nvec;
    if (n > 0) {
        // rows of at least 256 vectors: one workgroup per token when a token
        // has at most 2 slots, or for the row-scaled form (measured: 7-19%
        // faster at k = 1 and 5% for the scaled copy at k = 4, 2% slower for
        // the plain copy at k = 4)
        const bool row = nvec >= 256 && (k <= 2 || row_scale);
        const dim3 grid(row ? (unsigned)T : grid_for(n)), blk(256);
        const hipError_t e = with_k(k, [&](auto kc) {
            constexpr int K = decltype(kc)::value;
            auto go = [&](auto BF_, auto SC_) {
                constexpr bool BF = decltype(BF_)::value, SC = decltype(SC_)::value;
                if (row)
                    hipLaunchKernelGGL((permute_kernel<BF, SC, K, true>), grid, blk, 0, s, (const uint4*)x, T, nvec,
                                       dst_row, row_scale, n_rows, (uint4*)x_perm, dev_err);
                else
                    hipLaunchKernelGGL((permute_kernel<BF, SC, K>), grid, blk, 0, s, (const uint4*)x, T, nvec,
                                       dst_row, row_scale, n_rows, (uint4*)x_perm, dev_err);
            };
            using T_ = std::true_type;
            using F_ = std::false_type;
            if (bf && row_scale) go(T_{}, T_{});
            else if (bf) go(T_{}, F_{});
            else if (row_scale) go(F_{}, T_{});
            else go(F_{}, F_{});
        });
        if (e != hipSuccess) return e;
    }
    if (padded && n_rows > 0)
        hipLaunchKernelGGL(zero_rows_kernel, dim3((unsigned)((n_rows + 15) / 16)), dim3(256), 0, s,
                           src_slot, n_rows, nvec, (uint4*)x_perm, (uint8_t*)nullptr, 0);
    return hipGetLastError();
}

hipError_t launch_combine(int dtype, const void* y_perm, const int32_t* dst_row, const float* w,
                          int T, int k, int d, int64_t n_rows, void* out, int32_t* dev_err,
                          hipStream_t s)
{
    const bool bf = dtype == MOE_BF16;
    const int nvec = bf ? d / 8 : d / 4;
    const int64_t n = (int64_t)T * nvec;
    if (n > 0) {
        // rows of at least 256 vectors and at most 2 slots per token: one
        // workgroup per token (11-19% faster at k = 1, 2-3.5% slower at k = 4)
        const bool row = nvec >= 256 && k <= 2;
        const dim3 grid(row ? (unsigned)T : grid_for(n));
        const hipError_t e = with_k(k, [&](auto kc) {
            constexpr int K = decltype(kc)::value;
            if (bf && row)
                hipLaunchKernelGGL((combine_kernel<true, K, true>), grid, dim3(256), 0, s,
                                   (const uint4*)y_perm, dst_row, w, T, nvec, n_rows, (uint4*)out, dev_err);
            else if (bf)
                hipLaunchKernelGGL((combine_kernel<true, K>), grid, dim3(256), 0, s,
                                   (const uint4*)y_perm, dst_row, w, T, nvec, n_rows, (uint4*)out, dev_err);
            else if (row)
                hipLaunchKernelGGL((combine_kernel<false, K, true>), grid, dim3(256), 0, s,
                                   (const uint4*)y_perm, dst_row, w, T, nvec, n_rows, (uint4*)out, dev_err);
            else
                hipLaunchKernelGGL((combine_kernel<false, K>), grid, dim3(256), 0, s,
                                   (const uint4*)y_perm, dst_row, w, T, nvec, n_rows, (uint4*)out, dev_err);
        });
        if (e != hipSuccess) return e;
    }
    return hipGetLastError();
}

hipError_t launch_gate_grad(const void* dout, const void* y_perm, const int32_t* topk_idx,
                            const float* topk_w, const int32_t* dst_row, int T, int E, int k, int d,
                            int64_t n_rows, float* dlogits, float* dw, void* dy_perm, int32_t* dev_err,
                            hipStream_t s)
{
    if (T == 0) return hipSuccess;
    const int nvec = d / 8;
    const unsigned grid = (unsigned)((T + 3) / 4);
    const hipError_t e = with_k(k, [&](auto kc) {
        constexpr int K = decltype(kc)::value;
        if (dy_perm)
            hipLaunchKernelGGL((gate_grad_kernel<K, true>), dim3(grid), dim3(256), 0, s, (const uint4*)dout,
                               (const uint4*)y_perm, T, E, nvec, topk_idx, topk_w, dst_row, n_rows, dlogits, dw,
                               (uint4*)dy_perm, dev_err);
        else
            hipLaunchKernelGGL((gate_grad_kernel<K, false>), dim3(grid), dim3(256), 0, s, (const uint4*)dout,
                               (const uint4*)y_perm, T, E, nvec, topk_idx, topk_w, dst_row, n_rows, dlogits, dw,
                               (uint4*)nullptr, dev_err);
    });
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

hipError_t launch_quantize_rows(const uint16_t* src, int64_t rows, int K, uint8_t* codes,
                                uint8_t* scales, hipStream_t s)
{
    const int nb32 = K / 32;
    const int64_t n = rows * nb32;
    if (n > 0)
        hipLaunchKernelGGL(quant_rows_kernel, dim3(grid_for(n)), dim3(256), 0, s,
                           (const uint4*)src, rows, nb32, (uint4*)codes, scales);
    return hipGetLastError();
}

static hipError_t launch_cols(bool from_mx, const uint16_t* src, const uint8_t* sc,
                              const uint8_t* ss, int64_t rows, int K, const int32_t* group_off,
                              int capacity, int n_groups, uint8_t* codes, uint8_t* scales,
                              hipStream_t s)
{
    // bound on the number of 128-row tiles over all padded groups
    const int64_t ngr = group_off || capacity > 0 ? n_groups : 1;
    const int64_t nrt = (rows + ngr * kMxColPad) / kMxColPad;
    if (nrt == 0 || K == 0) return hipGetLastError();
    const dim3 grid((unsigned)((K + 127) / 128), (unsigned)nrt);
    if (from_mx)
        hipLaunchKernelGGL((quant_cols_kernel<true>), grid, dim3(256), 0, s, src, sc, ss, rows, K,
                           group_off, capacity, n_groups, codes, scales);
    else
        hipLaunchKernelGGL((quant_cols_kernel<false>), grid, dim3(256), 0, s, src, sc, ss, rows, K,
                           group_off, capacity, n_groups, codes, scales);
    return hipGetLastError();
}

hipError_t launch_quantize_cols(const uint16_t* src, int64_t rows, int K, const int32_t* group_off,
                                int capacity, int n_groups, uint8_t* codes, uint8_t* scales,
                                hipStream_t s)
{
    return launch_cols(false, src, nullptr, nullptr, rows, K, group_off, capacity, n_groups, codes,
                       scales, s);
}

hipError_t launch_dequant_requant_cols(const uint8_t* codes_row, const uint8_t* scales_row,
                                       int64_t rows, int K, const int32_t* group_off,
                                       int capacity, int n_groups, uint8_t* codes,
                                       uint8_t* scales, hipStream_t s)
{
    return launch_cols(true, nullptr, codes_row, scales_row, rows, K, group_off, capacity,
                       n_groups, codes, scales, s);
}

}  // namespace moe
