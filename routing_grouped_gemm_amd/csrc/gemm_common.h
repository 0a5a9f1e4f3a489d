// Shared device code of the grouped GEMMs (bf16 and MXFP8): operand buffer
// descriptors, the device tile schedule, accumulator layout and epilogues.
// Included by gemm_bf16.hip and gemm_mxfp8.hip only.
#pragma once

#include "moe_internal.h"


namespace moe {
namespace gemm {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int BN = 256;
constexpr int NTH = 256;
constexpr uint32_t kOOB = 0x80000000u;  // a buffer offset past every range: loads return 0

enum { EPI_STORE = 0, EPI_SWIGLU_FWD = 1, EPI_SWIGLU_BWD = 2 };

// Raw buffer descriptor over [base, base + bytes) as four scalar words
// (base, base[47:32] with stride 0, num_records, flags).  Loads at or past
// `bytes` return zero, which masks tile rows / columns / k outside the
// operand.
typedef __attribute__((ext_vector_type(4))) uint32_t desc_t;

__device__ __forceinline__ desc_t make_desc(const void* base, int64_t bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t n = bytes > 0x7fffffff ? 0x7fffffffu : (uint32_t)(bytes < 0 ? 0 : bytes);
    return desc_t{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, n, 0x00020000u};
}

// a descriptor chosen per wave (the compiler cannot tell it is uniform)
__device__ __forceinline__ desc_t wave_uniform(desc_t d)
{
    return desc_t{(uint32_t)__builtin_amdgcn_readfirstlane(d[0]), (uint32_t)__builtin_amdgcn_readfirstlane(d[1]),
                  (uint32_t)__builtin_amdgcn_readfirstlane(d[2]), (uint32_t)__builtin_amdgcn_readfirstlane(d[3])};
}

// Global -> LDS without VGPRs: lane l's BYTES (4 or 16) bytes from
// desc + voff + soff land at LDS address lds + BYTES * l.  Issued from
// inline assembly on purpose: the compiler then keeps no record of an
// asynchronous LDS write and so adds no wait before the LDS reads of the
// other stage.  The caller owns the ordering: s_waitcnt vmcnt plus a
// barrier before any wave reads what these loads wrote.  M0 takes the LDS
// base (M0 is reserved: the compiler sets it wherever it needs it); one wait
// state separates an M0 write from an LDS DMA.  `desc` and `soff` must be
// wave-uniform.
template <int BYTES>
__device__ __forceinline__ void dma_to_lds(desc_t desc, const void* lds, uint32_t voff, uint32_t soff)
{
    const auto lp = (__attribute__((address_space(3))) const void*)lds;
    const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lp);
    if constexpr (BYTES == 16)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                     :: "s"(base), "v"(voff), "s"(desc), "s"(soff) : "memory");
    else
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                     :: "s"(base), "v"(voff), "s"(desc), "s"(soff) : "memory");
}

// LDS byte address of a pointer into shared memory, as a wave-uniform value
__device__ __forceinline__ uint32_t lds_addr(const void* p)
{
    const auto lp = (__attribute__((address_space(3))) const void*)p;
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lp);
}

// dma_to_lds<16> with the LDS destination given as a wave-uniform byte
// address (no pointer conversion at the issue point)
__device__ __forceinline__ void dma16_to_lds_at(desc_t desc, uint32_t lds, uint32_t voff, uint32_t soff)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds), "v"(voff), "s"(desc), "s"(soff) : "memory");
}

// A ROWS x BK tile source.  K-major: element (r, k) at p[r*ld + k], rows split
// into two halves with their own bases and valid counts.  MN-major: element
// (r, k) at p[k*ld + r] with rows0 valid rows.
struct TileSrc {
    const uint16_t* p0;
    const uint16_t* p1;
    int64_t ld;
    int rows0, rows1;
    int K;
};

// LDS tiles are unpadded and XOR-swizzled in 16-byte chunks (8 bf16):
//  K-major  [ROWS][BK]: row r at r*BK*2 B.  BK = 64: k-chunk c (of 8) stored at
//           chunk c ^ ((r >> 1) & 7); BK = 32: chunk c (of 4) at c ^ ((r >> 2) & 3).
//           The 16 lanes of a 16-byte read (16 consecutive rows, one k-chunk)
//           then hit 16 distinct bank groups.
//  MN-major [BK][ROWS]: k-row k at k*ROWS*2 B; row-chunk c stored at chunk
//           c ^ (4 * (k & 3)).  A transposed read (4 k-rows x 2 chunks per 16
//           lanes, 2 groups per 32 lanes) then hits 16 distinct bank groups.
// Both are filled by direct global->LDS loads: every wave instruction writes
// 1 KB of LDS lane-linearly (16 B per lane), each lane fetching the global
// element that belongs at its LDS position.
template <bool MN, int BK>
__device__ __forceinline__ uint32_t lds_chunk(int row_or_k, int c)
{
    if constexpr (MN) return (uint32_t)(c ^ (4 * (row_or_k & 3)));
    else if constexpr (BK == 64) return (uint32_t)(c ^ ((row_or_k >> 1) & 7));
    else return (uint32_t)(c ^ ((row_or_k >> 2) & 3));
}

template <int ROWS, int BK, bool MN, int NW = 4>
struct DirectLoader {
    static constexpr int TILE_BYTES = ROWS * BK * 2;
    static constexpr int PER_WAVE = TILE_BYTES / 1024 / NW;  // 1 KB instructions per wave per K-step
    static constexpr int HALF = ROWS / 2;
    static constexpr int CPR_K = BK / 8;                     // 16-byte chunks per K-major row
    static constexpr int RPC_K = 1024 / (BK * 2);            // K-major rows per 1 KB chunk
    desc_t r0, r1;
    uint32_t off[PER_WAVE];   // per-lane byte offset of its element at k = 0
    uint32_t kstep;           // bytes a K-step advances (scalar)
    uint32_t m0w;             // LDS byte address of this wave's first 1 KB chunk in the stage-0 tile
    int K;
    // whether instruction i of this wave loads rows of the second half (K-major):
    // a function of i alone when every chunk row-block of one i lies in one
    // half for all waves, else of i and the (wave-uniform) wave index
    __device__ __forceinline__ bool half_of(int i) const
    {
        if constexpr (MN) {
            return false;
        } else if constexpr (HALF % (NW * RPC_K) == 0) {
            return i * NW * RPC_K >= HALF;
        } else {
            const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
            return (i * NW + w) * RPC_K >= HALF;
        }
    }
    __device__ __forceinline__ void init(const TileSrc& s, uint32_t lds_tile = 0) { init_tid(s, lds_tile, threadIdx.x); }
    // init with the thread index passed in (a caller inside a loop can pass a
    // value the compiler cannot hoist, so the per-lane offsets are recomputed
    // where they are needed instead of being kept live across the loop)
    __device__ __forceinline__ void init_tid(const TileSrc& s, uint32_t lds_tile, int tid)
    {
        const int lane = tid & 63;
        const int w = tid >> 6;
        K = s.K;
        m0w = lds_tile + (uint32_t)__builtin_amdgcn_readfirstlane(w) * 1024u;
        if constexpr (!MN) {
            r0 = wave_uniform(make_desc(s.p0, (int64_t)s.rows0 * s.ld * 2));
            r1 = wave_uniform(make_desc(s.p1, (int64_t)s.rows1 * s.ld * 2));
            kstep = BK * 2;
#pragma unroll
            for (int i = 0; i < PER_WAVE; ++i) {
                const int q = i * NW + w;
                const int row = q * RPC_K + lane / CPR_K;
                const int c = (int)lds_chunk<false, BK>(row, lane % CPR_K);   // XOR is an involution
                const int rr = row >= HALF ? row - HALF : row;
                off[i] = (uint32_t)(rr * s.ld * 2 + c * 16);
            }
        } else {
            r0 = r1 = wave_uniform(make_desc(s.p0, (int64_t)s.K * s.ld * 2));
            kstep = (uint32_t)(BK * s.ld * 2);
            constexpr int KROWS = 1024 / (ROWS * 2);   // k-rows per 1 KB chunk
            constexpr int CPR = ROWS / 8;              // 16-byte chunks per k-row
#pragma unroll
            for (int i = 0; i < PER_WAVE; ++i) {
                const int q = i * NW + w;
                const int k = q * KROWS + lane / CPR;
                const int c = (int)lds_chunk<true, BK>(k, lane % CPR);
                off[i] = c * 8 < s.rows0 ? (uint32_t)(k * s.ld * 2 + c * 16) : kOOB;
            }
        }
    }
    // instruction i (of PER_WAVE) of this wave's share of K-step kt into `tile`
    __device__ __forceinline__ void issue_one(uint16_t* tile, int kt, int i)
    {
        const int w = threadIdx.x >> 6;
        const uint32_t so = (uint32_t)kt * kstep;
        const int q = i * NW + w;
        uint32_t o = off[i];
        if (!MN && (kt + 1) * BK > K) {  // k-chunks at or past K read zero
            const int lane = threadIdx.x & 63;
            const int row = q * RPC_K + lane / CPR_K;
            const int c = (int)lds_chunk<false, BK>(row, lane % CPR_K);
            if (kt * BK + c * 8 >= K) o = kOOB;
        }
        const bool hi = half_of(i);
        dma_to_lds<16>(hi ? r1 : r0, tile + q * 512, o, so);
    }
    // instruction i of K-step kt into the tile at LDS byte address
    // (stage-0 tile) + stage_off, without the K-tail test: K-step kt must lie
    // inside K when the rows are K-major (MN-major tiles are masked past K by
    // the descriptor)
    __device__ __forceinline__ void issue_fast(uint32_t stage_off, int kt, int i)
    {
        const bool hi = half_of(i);
        dma16_to_lds_at(hi ? r1 : r0, m0w + stage_off + (uint32_t)(i * NW * 1024), off[i],
                        (uint32_t)kt * kstep);
    }
    // issue_fast, or (inside false) the same instruction with the scalar
    // offset at the buffer's range, so that every lane's offset lies past it
    // (and below 2^32 for the masked lanes at kOOB): it writes zeros to its
    // LDS chunk without a memory access
    __device__ __forceinline__ void issue_ring(uint32_t stage_off, int kt, int i, bool inside)
    {
        const bool hi = half_of(i);
        const desc_t d = hi ? r1 : r0;
        dma16_to_lds_at(d, m0w + stage_off + (uint32_t)(i * NW * 1024), off[i], inside ? (uint32_t)kt * kstep : d[2]);
    }
    // global -> LDS for K-step kt into the tile at `tile` (TILE_BYTES bytes)
    __device__ __forceinline__ void issue(uint16_t* tile, int kt)
    {
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) issue_one(tile, kt, i);
    }
};

// logistic function with the hardware reciprocal (about 1 ulp; results are
// stored as bf16), and silu(g) = g * sigmoid(g)
__device__ __forceinline__ float sigmoid_f(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }
__device__ __forceinline__ float silu_f(float g) { return g * sigmoid_f(g); }

// Wave layout of a BM x 256 output tile.  NW = 4: 2 x 2 waves of (BM/2) x
// 128, sub-tiles j = 0..3 at columns (j>>1)*128 + wn*64 + (j&1)*32.  NW = 8
// (two waves per SIMD): 2 x 4 waves of (BM/2) x 64, sub-tiles j = 0..1 at
// columns j*128 + wn*32.  Either way sub-tiles j and j + NJ/2 of a wave are
// the same columns of the two 128-column halves of the tile (the gate and up
// columns of the SwiGLU forward).
template <int NW>
struct WL {
    static_assert(NW == 4 || NW == 8, "4 or 8 waves");
    static constexpr int NJ = NW == 4 ? 4 : 2;   // 32-column sub-tiles per wave
    static constexpr int NT = 64 * NW;           // threads
    __device__ static int wm(int wave) { return NW == 4 ? wave >> 1 : wave >> 2; }
    __device__ static int wn(int wave) { return NW == 4 ? wave & 1 : wave & 3; }
    __device__ static int sub_col(int wn, int j) { return NW == 4 ? (j >> 1) * 128 + wn * 64 + (j & 1) * 32 : j * 128 + wn * 32; }
};

// first column (0..255) of the 32-wide sub-tile j of wave column wn (4 waves)
__device__ __forceinline__ int sub_col(int wn, int j) { return WL<4>::sub_col(wn, j); }

// Accumulator layout.  The MFMA is issued with the B fragment as its first
// operand, so acc[i][j] holds the transpose of sub-tile (i, j): lane l owns
// tile row  wm*(BM/2) + 32*i + (l & 31)  and, for g = 0..3, the four
// consecutive columns  sub_col(wn, j) + 8*g + 4*(l >> 5) + {0,1,2,3}  in
// acc[i][j][4g .. 4g+3].
template <int NW = 4>
__device__ __forceinline__ int acc_col(int wn, int j, int g, int lane)
{
    return WL<NW>::sub_col(wn, j) + 8 * g + 4 * (lane >> 5);
}

__device__ __forceinline__ uint2 pack4_bf16(float a, float b, float c, float d)
{
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    const bf16x2 lo = {(__bf16)a, (__bf16)b};
    const bf16x2 hi = {(__bf16)c, (__bf16)d};
    return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

__device__ __forceinline__ void unpack4_bf16(uint2 v, float (&o)[4])
{
    o[0] = bf16_lo(v.x);
    o[1] = bf16_hi(v.x);
    o[2] = bf16_lo(v.y);
    o[3] = bf16_hi(v.y);
}

// vmcnt(n) with n known at compile time (expcnt / lgkmcnt left unconstrained)
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

struct MParams {
    const uint16_t* A;     // grouped rows, K-major [n_rows, K]
    int64_t lda;
    const uint16_t* B;     // per-expert weight: B + e * sB
    int64_t ldb, sB;
    int N;                 // output columns (f for the SwiGLU forward)
    int K;
    const int32_t* group_off;
    int capacity, E;
    int64_t n_rows;
    int ntn;               // N tiles
    uint16_t* C;           // STORE: out; SWIGLU_FWD: gu; SWIGLU_BWD: dgu
    int64_t ldc;
    uint16_t* H;           // SWIGLU_FWD: h
    int64_t ldh;
    const uint16_t* G;     // SWIGLU_BWD: saved gu
    int64_t ldg;
    int f;                 // SWIGLU: column offset of the u half in gu / dgu
    // optional (MXFP8 stages): the row-wise MXFP8 copy of h (SWIGLU_FWD) or
    // of dgu (SWIGLU_BWD), codes [rows, ldq] and E8M0 scales [rows, ldq / 32],
    // made from the bf16 values the epilogue stores
    uint8_t* Mq;
    uint8_t* Ms;
    int64_t ldq;
};

// Row-wise MXFP8 of 32 bf16 held as 8 by each of four consecutive lanes
// (lanes 4j .. 4j+3, in element order): the block maximum and finiteness are
// combined across the quad with DPP lane exchanges, then each lane encodes its
// 8 elements -- the same arithmetic as the standalone quantiser (scale rule,
// hardware round-to-nearest-even conversion for finite blocks, the software
// encoder for blocks with a NaN or an infinity).  All four lanes must execute
// it.  Returns the scale exponent; codes in element order, byte b of word w
// = element 4w + b.
__device__ __forceinline__ int mx_quant8_quad(uint4 v, uint2& codes)
{
    float x[8];
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        x[2 * p] = bf16_lo(wv[p]);
        x[2 * p + 1] = bf16_hi(wv[p]);
    }
    float amax = 0.0f;
    int finite = 1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float a = fabsf(x[i]);
        amax = fmaxf(amax, a);
        finite &= a <= 3.402823466e38f ? 1 : 0;
    }
    amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(amax), 0xB1, 0xF, 0xF, false)));
    amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(amax), 0x4E, 0xF, 0xF, false)));
    finite &= __builtin_amdgcn_update_dpp(0, finite, 0xB1, 0xF, 0xF, false);
    finite &= __builtin_amdgcn_update_dpp(0, finite, 0x4E, 0xF, 0xF, false);
    const int e = mx_scale_exp(amax);
    uint32_t w[2];
    if (finite) {
#pragma unroll
        for (int wi = 0; wi < 2; ++wi) {
            const float q0 = __builtin_ldexpf(x[wi * 4 + 0], -e), q1 = __builtin_ldexpf(x[wi * 4 + 1], -e);
            const float q2 = __builtin_ldexpf(x[wi * 4 + 2], -e), q3 = __builtin_ldexpf(x[wi * 4 + 3], -e);
            const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
            w[wi] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, lo, true);
        }
    } else {
#pragma unroll
        for (int wi = 0; wi < 2; ++wi) {
            uint32_t word = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) word |= f32_to_e4m3(__builtin_ldexpf(x[wi * 4 + b], -e)) << (8 * b);
            w[wi] = word;
        }
    }
    codes = make_uint2(w[0], w[1]);
    return e;
}

// Epilogues stage the bf16 result tile in LDS (free once the main loop has
// ended) and store it row by row: each lane writes 16 contiguous bytes and a
// wave two whole tile rows, instead of 32 rows x 16 bytes per instruction
// straight from the accumulator layout.  A staged tile is ROWS x (CH*8) bf16,
// row pitch CH*16 bytes, 16-byte chunk c of row r at chunk c ^ (r & (CH-1)):
// the 32 rows one accumulator write touches then fall on distinct chunks, and
// a row read back is one contiguous swizzled row.
template <int CH>
__device__ __forceinline__ uint32_t stage_off(int r, int col)   // element (r, col), col % 4 == 0
{
    return (uint32_t)(r * (CH * 16) + (((col >> 3) ^ (r & (CH - 1))) << 4) + ((col & 4) << 1));
}

// 16-byte non-temporal (streaming) store, for outputs that nothing reads
// back while they could still be in L2 (the weight gradients: measured 6%
// faster than plain stores there, no change for the forward / dgrad outputs)
__device__ __forceinline__ void store16(uint16_t* p, uint4 v)
{
    typedef __attribute__((ext_vector_type(4))) uint32_t vu4;
    __builtin_nontemporal_store(vu4{v.x, v.y, v.z, v.w}, reinterpret_cast<vu4*>(p));
}

__device__ __forceinline__ void stage_put(uint8_t* lds, uint32_t off, uint2 v)
{
    *reinterpret_cast<uint2*>(lds + off) = v;
}

// After a barrier: thread t hands out chunks t, t + NTH, ... as put(r, c, v),
// all of its LDS reads first (one wait instead of one per chunk); a
// trailing barrier frees the LDS again.
template <int ROWS, int CH, int NT = NTH, class F>
__device__ __forceinline__ void stage_flush(const uint8_t* lds, F&& put)
{
    constexpr int N = ROWS * CH / NT;   // chunks per thread
    static_assert(ROWS * CH % NT == 0, "whole chunks per thread");
    __syncthreads();
    uint4 v[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const int q = (int)threadIdx.x + i * NT;
        const int r = q / CH, c = q % CH;
        v[i] = *reinterpret_cast<const uint4*>(lds + r * (CH * 16) + ((c ^ (r & (CH - 1))) << 4));
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const int q = (int)threadIdx.x + i * NT;
        put(q / CH, q % CH, v[i]);
    }
    __syncthreads();
}

// the accumulator tile (BM x 256) as bf16 into the staging layout
template <int BM, int NW = 4>
__device__ __forceinline__ void stage_acc(const f32x16 (&acc)[BM / 64][WL<NW>::NJ], uint8_t* lds)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = WL<NW>::wm(wave), wn = WL<NW>::wn(wave);
#pragma unroll
    for (int i = 0; i < BM / 64; ++i)
#pragma unroll
        for (int j = 0; j < WL<NW>::NJ; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                stage_put(lds, stage_off<32>(wm * (BM / 2) + i * 32 + (lane & 31), acc_col<NW>(wn, j, g, lane)),
                          pack4_bf16(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                     acc[i][j][4 * g + 3]));
}

// MXQ: the SwiGLU epilogues also write the row-wise MXFP8 copy of their
// bf16 output (h or dgu) to p.Mq / p.Ms
template <int BM, int EPI, int NW = 4, bool MXQ = false>
__device__ __forceinline__ void epilogue_m(const f32x16 (&acc)[BM / 64][WL<NW>::NJ], const MParams& p,
                                           int64_t row0, int rows_valid, int nt, uint8_t* lds)
{
    constexpr int MI = BM / 64;
    constexpr int NJ = WL<NW>::NJ;
    constexpr int NT = WL<NW>::NT;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int lane = threadIdx.x & 63;
    const int wm = WL<NW>::wm(wave), wn = WL<NW>::wn(wave);
    if constexpr (EPI == EPI_STORE) {
        stage_acc<BM, NW>(acc, lds);
        stage_flush<BM, 32, NT>(lds, [&](int r, int c, uint4 v) {
            const int n = nt * BN + 8 * c;
            if (r < rows_valid && n < p.N) *reinterpret_cast<uint4*>(p.C + (row0 + r) * p.ldc + n) = v;
        });
    } else if constexpr (EPI == EPI_SWIGLU_FWD) {
        // tile columns 0..127 are gate columns n0.., 128..255 the up columns f + n0..
        const int n0 = nt * 128;
        stage_acc<BM, NW>(acc, lds);
        stage_flush<BM, 32, NT>(lds, [&](int r, int c, uint4 v) {
            const int n = n0 + 8 * (c & 15);
            if (r < rows_valid && n < p.f)
                *reinterpret_cast<uint4*>(p.C + (row0 + r) * p.ldc + (c < 16 ? n : p.f + n)) = v;
        });
        // h = silu(g) * u from the unrounded fp32 accumulators
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ / 2; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float hv[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) hv[q] = silu_f(acc[i][j][4 * g + q]) * acc[i][j + NJ / 2][4 * g + q];
                    stage_put(lds, stage_off<16>(wm * (BM / 2) + i * 32 + (lane & 31), acc_col<NW>(wn, j, g, lane)),
                              pack4_bf16(hv[0], hv[1], hv[2], hv[3]));
                }
        if constexpr (MXQ) {
            // h also leaves as row-wise MXFP8: the four lanes of each 32-column block encode it together
            stage_flush<BM, 16, NT>(lds, [&](int r, int c, uint4 v) {
                const int n = n0 + 8 * c;
                uint2 q;
                const int e = mx_quant8_quad(v, q);
                if (r < rows_valid && n < p.f) {
                    *reinterpret_cast<uint4*>(p.H + (row0 + r) * p.ldh + n) = v;
                    *reinterpret_cast<uint2*>(p.Mq + (row0 + r) * p.ldq + n) = q;
                    if ((c & 3) == 0) p.Ms[(row0 + r) * (p.ldq / 32) + n / 32] = (uint8_t)(e + 127);
                }
            });
        } else {
            stage_flush<BM, 16, NT>(lds, [&](int r, int c, uint4 v) {
                const int n = n0 + 8 * c;
                if (r < rows_valid && n < p.f) *reinterpret_cast<uint4*>(p.H + (row0 + r) * p.ldh + n) = v;
            });
        }
    } else {
        // SwiGLU backward, 128 tile columns at a time (accumulator sub-tiles
        // j = 2*ch, 2*ch+1 of every wave): the g and u tiles of those columns
        // come into LDS (direct loads, staging layout), every lane overwrites
        // its g, u pairs in place with dg, du, and both tiles leave as rows of dgu
        constexpr int QTILE = BM * 16 * 16;                 // bytes of one BM x 128 bf16 tile
        static_assert(2 * QTILE <= 2 * (BM + BN) * 64 * 2, "staging fits the stage buffers");
        const int n0 = nt * BN;
        uint8_t* lg = lds;
        uint8_t* lu = lds + QTILE;
        const desc_t g_desc = make_desc(p.G + row0 * p.ldg, (int64_t)rows_valid * p.ldg * 2);
        // the two 128-column halves, each with its half index known at compile time
        auto half = [&](auto CH_) __attribute__((always_inline)) {
            constexpr int ch = decltype(CH_)::value;
            const int nc = n0 + 128 * ch;                   // first column of this half
#pragma unroll
            for (int i = 0; i < QTILE / 1024 / NW; ++i) {
                const int q = i * NW + wave;                // 1 KB slice of the tile
                const int slot = q * 64 + lane;             // 16-byte staging slot
                const int r = slot >> 4, c = (slot & 15) ^ (r & 15);
                const uint32_t off = (uint32_t)((r * p.ldg + nc + 8 * c) * 2);
                dma_to_lds<16>(g_desc, lg + q * 1024, off, 0);
                dma_to_lds<16>(g_desc, lu + q * 1024, off, (uint32_t)(p.f * 2));
            }
            wait_vmcnt<0>();
            __syncthreads();
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int jj = 0; jj < NJ / 2; ++jj)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int j = (NJ / 2) * ch + jj;
                        const uint32_t off = stage_off<16>(wm * (BM / 2) + i * 32 + (lane & 31),
                                                           acc_col<NW>(wn, j, g, lane) - 128 * ch);
                        float gv[4], uv[4], dgv[4], duv[4];
                        unpack4_bf16(*reinterpret_cast<const uint2*>(lg + off), gv);
                        unpack4_bf16(*reinterpret_cast<const uint2*>(lu + off), uv);
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            const float dh = acc[i][j][4 * g + t];
                            const float sg = sigmoid_f(gv[t]);
                            duv[t] = dh * gv[t] * sg;
                            dgv[t] = dh * uv[t] * sg * (1.0f + gv[t] * (1.0f - sg));
                        }
                        stage_put(lg, off, pack4_bf16(dgv[0], dgv[1], dgv[2], dgv[3]));
                        stage_put(lu, off, pack4_bf16(duv[0], duv[1], duv[2], duv[3]));
                    }
            __syncthreads();
            // both tiles out as rows of dgu, all LDS reads of a thread first
            constexpr int NQ = BM * 16 * 2 / NT;
            static_assert(BM * 16 * 2 % NT == 0, "whole chunks per thread");
            uint4 v[NQ];
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const int q = (int)threadIdx.x + i * NT;
                const int which = q / (BM * 16), qq = q % (BM * 16);
                const int r = qq >> 4, c = qq & 15;
                v[i] = *reinterpret_cast<const uint4*>((which ? lu : lg) + r * 256 + ((c ^ (r & 15)) << 4));
            }
            if constexpr (MXQ) {
                // dgu also leaves as row-wise MXFP8 (32-column blocks never straddle dg | du)
#pragma unroll
                for (int i = 0; i < NQ; ++i) {
                    const int q = (int)threadIdx.x + i * NT;
                    const int which = q / (BM * 16), qq = q % (BM * 16);
                    const int r = qq >> 4, c = qq & 15;
                    const int n = nc + 8 * c;
                    uint2 cq;
                    const int e = mx_quant8_quad(v[i], cq);
                    if (r < rows_valid && n < p.N) {
                        const int col = which ? p.f + n : n;
                        *reinterpret_cast<uint4*>(p.C + (row0 + r) * p.ldc + col) = v[i];
                        *reinterpret_cast<uint2*>(p.Mq + (row0 + r) * p.ldq + col) = cq;
                        if ((c & 3) == 0) p.Ms[(row0 + r) * (p.ldq / 32) + col / 32] = (uint8_t)(e + 127);
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < NQ; ++i) {
                    const int q = (int)threadIdx.x + i * NT;
                    const int which = q / (BM * 16), qq = q % (BM * 16);
                    const int r = qq >> 4, c = qq & 15;
                    const int n = nc + 8 * c;
                    if (r < rows_valid && n < p.N)
                        *reinterpret_cast<uint4*>(p.C + (row0 + r) * p.ldc + (which ? p.f + n : n)) = v[i];
                }
            }
            __syncthreads();
        };
        half(std::integral_constant<int, 0>{});
        half(std::integral_constant<int, 1>{});
    }
}

// one 256-thread workgroup per CU: each SIMD runs one wave that may use the
// whole register file (accumulators in AGPRs)
#define MOE_GEMM_KERNEL_ATTRS \
    __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(1, 1), amdgpu_flat_work_group_size(NTH, NTH)))
// NW waves: NW / 4 per SIMD, each with the register file share that allows
#define MOE_GEMM_KERNEL_ATTRS_NW(NW) \
    __launch_bounds__(64 * (NW)) __attribute__((amdgpu_waves_per_eu((NW) / 4, (NW) / 4), \
                                               amdgpu_flat_work_group_size(64 * (NW), 64 * (NW))))


// Tile (mt, nt) of the local-th tile of an mtn x ntn grid, walked in groups
// of GM tile rows (nt fastest across a group's columns, mt fastest within):
// a run of consecutive tiles then shares GM row slices of A and a few column
// slices of B, which stay in L2 while those tiles run together.
__device__ __forceinline__ void grouped_tile(int local, int mtn, int ntn, int GM, int& mt, int& nt)
{
    const int per_group = GM * ntn;
    const int g = local / per_group;
    const int first = g * GM;
    const int gm = min(mtn - first, GM);
    const int r = local - g * per_group;
    mt = first + r % gm;
    nt = r / gm;
}

// Device tile schedule of a grouped-M launch: every wave of a workgroup
// sums, lane by lane, the ceil(m_e / BM) * ntn tiles of the experts (lane l
// takes experts l*per .. l*per+per-1, per = ceil(E / 64)) and scans the lane
// sums across the wave (no LDS, no barrier), remaps the workgroup id so
// that a contiguous range of tiles lands on one XCD, and finds its expert,
// N-tile and M-tile.  Returns false for surplus workgroups.
// An expert's tiles go in groups of kMTileGroup M-tiles (N-tiles across a
// group, M-tiles fastest within): the 32 tiles an XCD runs at once then read
// a few M-slices of A and N-slices of B (with all of a large expert's M-tiles
// per N-tile, 32 concurrent tiles would read 32 A slices and one B slice).
constexpr int kMTileGroup = 4;

struct MTile {
    int e, nt, mt, rows_valid;
    int64_t row0;
};

template <int BM>
__device__ __forceinline__ bool schedule_m(const int32_t* group_off, int capacity, int E, int64_t n_rows,
                                           int ntn, MTile& t)
{
    const int lane = threadIdx.x & 63;
    const int per = (E + 63) >> 6;   // experts per lane (at most 16)
    const int gb = lane * per;
    auto tiles = [&](int g) __attribute__((always_inline)) {
        return (int)((group_rows(group_off, capacity, g, n_rows) + BM - 1) / BM) * ntn;
    };
    int cnt = 0;
    for (int k = 0; k < per && gb + k < E; ++k) cnt += tiles(gb + k);
    int incl = cnt;   // inclusive scan of the lane sums
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
    }
    const int total = __builtin_amdgcn_readlane(incl, 63);   // wave-uniform
    const int per_xcd = (total + 7) / 8;
    const int xcd = blockIdx.x % 8;
    const int slot = blockIdx.x / 8;
    if (slot >= per_xcd) return false;
    const int L = xcd * per_xcd + slot;
    if (L >= total) return false;
    // the one lane whose experts hold tile L, then the expert within it
    const int excl = incl - cnt;
    const int src = __ffsll((unsigned long long)__ballot(excl <= L && L < incl)) - 1;
    int e = gb, first = excl;
    for (int k = 0, run = excl; k < per && gb + k < E; ++k) {
        const int c = tiles(gb + k);
        if (L >= run && L < run + c) {
            e = gb + k;
            first = run;
        }
        run += c;
    }
    t.e = __builtin_amdgcn_readlane(e, src);
    const int local = L - __builtin_amdgcn_readlane(first, src);
    const int64_t g0 = group_begin(group_off, capacity, t.e, n_rows);
    const int m_e = (int)group_rows(group_off, capacity, t.e, n_rows);
    const int mt_e = (m_e + BM - 1) / BM;
    grouped_tile(local, mt_e, ntn, kMTileGroup, t.mt, t.nt);
    t.row0 = g0 + (int64_t)t.mt * BM;
    t.rows_valid = min(BM, m_e - t.mt * BM);
    return true;
}

// add a BM x 256 accumulator tile into fp32 rows of C (rows [0, rows),
// columns col0 + [0, 256) below N; N % 4 == 0, C 16-byte aligned) straight
// from the accumulator layout: each lane reads, adds and writes back its
// four consecutive columns of one row, 32 rows at a time (all of a 32-row
// block's reads before its writes).  Staging the fp32 tile through the LDS
// for whole-row accesses measured no faster in the one-workgroup-per-tile
// kernel, where the tiles finish together and the read-modify-write is bound
// by their simultaneous HBM traffic (the persistent walk, whose tiles finish
// at different times, uses the staged form below).
template <int BM, int NW>
__device__ __forceinline__ void add_tile_f32(const f32x16 (&acc)[BM / 64][WL<NW>::NJ], float* C, int64_t ldc,
                                             int rows, int col0, int N)
{
    constexpr int NJ = WL<NW>::NJ;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = WL<NW>::wm(wave), wn = WL<NW>::wn(wave);
#pragma unroll
    for (int i = 0; i < BM / 64; ++i) {
        const int r = wm * (BM / 2) + i * 32 + (lane & 31);
        float4 v[NJ][4];
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c = col0 + acc_col<NW>(wn, j, g, lane);
                if (r < rows && c < N) v[j][g] = *reinterpret_cast<const float4*>(C + r * ldc + c);
            }
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c = col0 + acc_col<NW>(wn, j, g, lane);
                if (r < rows && c < N) {
                    float4 o = v[j][g];
                    o.x += acc[i][j][4 * g];
                    o.y += acc[i][j][4 * g + 1];
                    o.z += acc[i][j][4 * g + 2];
                    o.w += acc[i][j][4 * g + 3];
                    *reinterpret_cast<float4*>(C + r * ldc + c) = o;
                }
            }
    }
}

// store a BM x 256 accumulator tile as bf16 rows of C (rows [0, rows), columns
// col0 + [0, 256) below N), through the LDS staging above
template <int BM, int NW = 4>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[BM / 64][WL<NW>::NJ], uint16_t* C, int64_t ldc,
                                           int rows, int col0, int N, uint8_t* lds)
{
    stage_acc<BM, NW>(acc, lds);
    stage_flush<BM, 32, WL<NW>::NT>(lds, [&](int r, int c, uint4 v) {
        const int n = col0 + 8 * c;
        if (r < rows && n < N) store16(C + r * ldc + n, v);
    });
}

// Columns [128 PASS, 128 PASS + 128) of a 256 x 256 accumulator tile (sub-tile
// j = PASS of every wave) as bf16 rows of C: staged through the 64 KB at lds
// as 256 rows x 128 columns, then 8 non-temporal 16-byte buffer stores per
// thread, a wave instruction covering 4 rows x 256 contiguous bytes, always
// issued: an element outside rows x (N - col0) gets an offset past the
// buffer's range and the hardware drops it.  Ct is row 0, column 0 of the
// tile (wave-uniform) and every in-range byte offset (row * ldc + col) * 2 is
// below 2^31.  A barrier before the LDS reads and one after them.  Every wave
// converts and stages in both passes (splitting the rows instead left half of
// the waves idle while the other half staged: 1.3% slower weight gradient).
template <int NW, int PASS>
__device__ __forceinline__ void store_colhalf_nt(const f32x16 (&acc)[4][WL<NW>::NJ], uint16_t* Ct, int64_t ldc,
                                                 int rows, int col0, int N, uint8_t* lds)
{
    static_assert(NW == 8, "sub-tile j of every wave is one 128-column half");
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(Ct, (short)0, 0x7fffffff, 0x00020000);
    constexpr int NT = WL<NW>::NT;
    constexpr int PER = 256 * 16 / NT;            // 16-byte chunks per thread
    // the thread index through an empty asm: the offsets below are then
    // computed here rather than hoisted out of a caller's tile loop
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int wm = WL<NW>::wm(wave), wn = WL<NW>::wn(wave);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            stage_put(lds, stage_off<16>(wm * 128 + i * 32 + (lane & 31), wn * 32 + 8 * g + 4 * (lane >> 5)),
                      pack4_bf16(acc[i][PASS][4 * g], acc[i][PASS][4 * g + 1], acc[i][PASS][4 * g + 2],
                                 acc[i][PASS][4 * g + 3]));
    __syncthreads();
    uint4 v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int q = tid + i * NT;
        const int r = q >> 4, c = q & 15;
        v[i] = *reinterpret_cast<const uint4*>(lds + r * 256 + ((c ^ (r & 15)) << 4));
    }
    typedef __attribute__((ext_vector_type(4))) uint32_t vu4;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int q = tid + i * NT;
        const int r = q >> 4, n = col0 + PASS * 128 + 8 * (q & 15);
        const uint32_t off = r < rows && n < N ? (uint32_t)((r * ldc + n) * 2) : kOOB;
        __builtin_amdgcn_raw_buffer_store_b128(vu4{v[i].x, v[i].y, v[i].z, v[i].w}, rsrc, (int)off, 0,
                                               2 /* non-temporal */);
    }
    __syncthreads();
}

// A 256 x 256 accumulator tile added into fp32 rows of C, in four passes of
// 64 tile rows: pass i is accumulator sub-tile i of every wave (rows 32i ..
// 32i + 31 and 128 + 32i .. 128 + 32i + 31), staged through the 64 KB at lds
// as 64 rows x 256 fp32 (16-byte chunk c of staged row r at chunk c ^ (r & 63),
// so both the accumulator-layout writes and the row reads spread over the
// banks).  Every thread first loads its 8 chunks of C for the pass (a wave
// instruction covers one row's 1 KB), then the tile is staged, and after a
// barrier each thread adds its chunks and stores them back in place
// (non-temporal); a barrier frees the LDS for the next pass.  Every load and
// store is issued, 64 per thread, whatever the tile's extent: a chunk outside
// rows x (N - col0) gets an offset past the buffer's range (the load returns
// zeros, the store is dropped).  C is row 0, column 0 of the tile
// (wave-uniform), every in-range byte offset below 2^31, N % 4 == 0.
template <int NW>
__device__ __forceinline__ void add_tile_f32_rows(const f32x16 (&acc)[4][WL<NW>::NJ], float* C, int64_t ldc,
                                                  int rows, int col0, int N, uint8_t* lds)
{
    static_assert(NW == 8, "sub-tile i of every wave is one 64-row pass");
    constexpr int NT = WL<NW>::NT;
    constexpr int PER = 64 * 64 / NT;             // 16-byte chunks per thread and pass
    typedef __attribute__((ext_vector_type(4))) uint32_t vu4;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(C, (short)0, 0x7fffffff, 0x00020000);
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));                 // offsets computed here, not hoisted out of the tile loop
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int wm = WL<NW>::wm(wave), wn = WL<NW>::wn(wave);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // this thread's chunks: staged row (wave + 8n), chunk lane
        auto offset = [&](int pr) __attribute__((always_inline)) {
            const int tr = (pr < 32 ? 0 : 128 - 32) + i * 32 + pr, col = col0 + 4 * lane;
            return tr < rows && col < N ? (uint32_t)((tr * ldc + col) * 4) : kOOB;
        };
        vu4 cv[PER];
#pragma unroll
        for (int n = 0; n < PER; ++n) cv[n] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)offset(wave + 8 * n), 0, 0);
#pragma unroll
        for (int j = 0; j < WL<NW>::NJ; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int pr = wm * 32 + (lane & 31);
                const int c = (WL<NW>::sub_col(wn, j) + 8 * g + 4 * (lane >> 5)) >> 2;
                *reinterpret_cast<float4*>(lds + pr * 1024 + ((c ^ (pr & 63)) << 4)) =
                    make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
            }
        __syncthreads();
#pragma unroll
        for (int n = 0; n < PER; ++n) {
            const int pr = wave + 8 * n;
            const float4 a = *reinterpret_cast<const float4*>(lds + pr * 1024 + ((lane ^ (pr & 63)) << 4));
            const vu4 o = {__float_as_uint(__uint_as_float(cv[n].x) + a.x), __float_as_uint(__uint_as_float(cv[n].y) + a.y),
                           __float_as_uint(__uint_as_float(cv[n].z) + a.z), __float_as_uint(__uint_as_float(cv[n].w) + a.w)};
            __builtin_amdgcn_raw_buffer_store_b128(o, rsrc, (int)offset(pr), 0, 2 /* non-temporal */);
        }
        __syncthreads();
    }
}

}  // namespace gemm
}  // namespace moe
