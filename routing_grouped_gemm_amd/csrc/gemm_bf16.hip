// Grouped SwiGLU GEMMs on bf16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16).
//
// The OLMo-core 3 tutorial (routing-tax section, second tax) describes one
// device-scheduled grouped GEMM over the exact per-expert row counts, with
// no padding to a common capacity and no host launches per expert.  Here:
//   - every launch covers all experts; its grid is sized from host-known
//     bounds (n_rows / BM + E M-tiles) and each workgroup finds its
//     (expert, N-tile, M-tile) from the device-resident group offsets by a
//     block-wide prefix over ceil(m_e / BM) and a binary search;
//   - tile order is expert-major with the M-tiles of one (expert, N-tile)
//     adjacent, and workgroup ids are remapped so that a contiguous range of
//     tiles lands on one XCD (consecutive ids go round-robin over the 8 XCDs):
//     the M-tiles sharing a weight tile then share that XCD's L2;
//   - tiles are 256 x 256 x 64, eight waves (two per SIMD) in a 2 x 4 grid,
//     each wave owning 128 x 64 fp32 accumulators; operands go from HBM to
//     LDS with direct loads (no VGPR staging) into two XOR-swizzled stages;
//   - operands stored with M/N contiguous (the weight in dgrad, both operands
//     of wgrad) are read from LDS with the gfx950 transposing reads;
//   - two main loops: the default one (fragment reads one k-slice ahead, the
//     last slice's MFMAs after the next barrier, the next K-step's loads
//     spread over the first MFMAs) and a ping-pong one for K-major weights
//     (the two waves of a SIMD alternate between MFMA-only and memory ticks);
//   - epilogues, staged through LDS so that each lane stores 16 contiguous
//     bytes: plain bf16 store; the SwiGLU forward (each wave holds the gate
//     and up accumulators of the same columns, so h = silu(g) * u is formed
//     in registers and g, u, h are stored); the SwiGLU backward (reads the
//     saved g, u of its elements and stores dg, du).
// Accumulation is fp32; bf16 results are rounded to nearest even.
#include <type_traits>

#include "gemm_common.h"

namespace moe {
namespace {

using namespace gemm;

// Weight-gradient tiles are dealt to the XCDs in runs of this many tiles
// when contiguous ranges would load the XCDs unevenly.  A weight-gradient
// tile's cost is its group's row count, so with uneven groups (Zipf routing,
// shared experts) contiguous ranges leave one XCD with the big groups (e128
// under Zipf(1.2): 9.97 -> 2.97 ms, one shared expert 5.86 -> 3.70 ms).
// Dealt always, uniform e128 went 2.93 -> 2.97 ms with 2.9x the HBM reads
// (each XCD's L2 then sees every expert), hence the test ahead of each
// launch.  Runs of 16 measured the same, 32 slower.
constexpr int kKDealRun = 4;
// The direct loads of the next K-step go out spread evenly over the first
// kLoadSpan / 32 of a K-step's MFMAs (single-group loop, two LDS stages;
// best of 8 .. 28).  With a deeper ring the loads of K-step kt + NS - 1 go
// out over the first kLoadSpanRing / 32 of K-step kt's MFMAs.
constexpr int kLoadSpan = 12;
constexpr int kLoadSpanRing = 32;


// One MFMA operand fragment (8 consecutive k of one row) for lane `lane`:
// tile row row_base + (lane & 31), k = ks*16 + (lane >> 5)*8 + [0, 8).
template <int ROWS, int BK, bool MN>
__device__ __forceinline__ bf16x8 read_frag(const uint16_t* tile, int row_base, int ks, int lane)
{
    if constexpr (!MN) {
        const int row = row_base + (lane & 31);
        const int c = ks * 2 + (lane >> 5);
        return *reinterpret_cast<const bf16x8*>(tile + row * BK + lds_chunk<false, BK>(row, c) * 8);
    } else {
        // 16-lane group g reads rows row_base + (g & 1)*16 + [0,16) at k-chunk (g >> 1):
        // lanes 4r..4r+3 of the group supply k-row (kb + r), 4 rows each of 16 elements.
        typedef __attribute__((ext_vector_type(4))) short v4i16;
        typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
        const int g = lane >> 4;
        const int j = lane & 15;
        const int m = row_base + (g & 1) * 16 + 4 * (j & 3);   // first of 4 elements this lane supplies
        const int kb = ks * 16 + (g >> 1) * 8 + (j >> 2);
        v4i16 lo, hi;
        {
            const int k = kb;
            const uint16_t* p = tile + k * ROWS + lds_chunk<true, BK>(k, m >> 3) * 8 + (m & 7);
            lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(__attribute__((address_space(3))) const void*)p);
        }
        {
            const int k = kb + 4;
            const uint16_t* p = tile + k * ROWS + lds_chunk<true, BK>(k, m >> 3) * 8 + (m & 7);
            hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(__attribute__((address_space(3))) const void*)p);
        }
        typedef __attribute__((ext_vector_type(8))) short v8i16;
        const v8i16 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(bf16x8, v);
    }
}

// BM x 256 tile over s.K, accumulators acc[BM/64][NJ].  A ring of NS LDS
// stages of (BM + 256) x BK bf16: the direct loads of K-step kt + NS - 1 are
// in flight while the MFMAs of K-step kt run; one barrier per K-step.  With
// more than two stages (both operands MN-major, or K a multiple of BK) every
// K-step issues the loads NS - 1 steps ahead, past the end of K too, where
// they take an offset outside the buffer and write zeros to a stage nobody
// reads (a tail loop without loads made the accumulators spill).  The wait
// at a K-step counts the vector memory operations issued after its loads:
// they complete in issue order, those with every lane outside the buffer
// included (checked on the hardware for direct-to-LDS loads and for stores).
// Fragments of k-slice ks+1 are read while the MFMAs of slice ks run, and the
// MFMAs of each K-step's last slice are issued after the next barrier, so
// that they cover the latency of the first fragment reads of the new K-step.
// PRE: K-steps 0 .. PRE-1 were already issued into stages 0 .. PRE-1 by the
// caller (with loaders made from the same sources); stores16: the caller
// issued at least NDRAIN vector memory operations per wave after those loads
// (exactly 16 stores for the bf16 epilogue; 64 loads and stores, the last 8
// of them stores, for the fp32 one), so the last NDRAIN are waited for only
// from K-step PRE on and may drain during the first K-steps.
template <int BM, int BK, int NS, bool A_MN, bool B_MN, int NW, bool KAL, int PRE = 0, int NDRAIN = 16>
__device__ __forceinline__ void mainloop(const TileSrc& sa, const TileSrc& sb,
                                         f32x16 (&acc)[BM / 64][WL<NW>::NJ], uint16_t* smem,
                                         bool stores16 = false)
{
    constexpr int MI = BM / 64;
    constexpr int NJ = WL<NW>::NJ;
    constexpr int KS = BK / 16;             // k-slices per K-step
    constexpr int STAGE = (BM + BN) * BK;   // elements per stage
    using LA = DirectLoader<BM, BK, A_MN, NW>;
    using LB = DirectLoader<BN, BK, B_MN, NW>;
    constexpr int NA = LA::PER_WAVE;
    constexpr int NB = LB::PER_WAVE;
    constexpr int NQ = NA + NB;                    // load instructions per wave per K-step
    constexpr int SM = MI * NJ;                    // MFMAs per k-slice
    constexpr int SPN = (NS == 2 ? kLoadSpan : kLoadSpanRing) * KS * SM / 32;
    constexpr int SPAN = SPN < NQ ? NQ : SPN;
    static_assert(NS >= 2, "a ring of at least two LDS stages");
    static_assert(NS == 2 || KAL || (A_MN && B_MN), "deeper rings issue loads without the K-tail test");
    static_assert(PRE >= 0 && PRE < NS, "pre-issued K-steps fit the ring");
    static_assert(KS >= 2 && KS % 2 == 0, "an even number of k-slices per K-step");
    static_assert(SPAN <= KS * SM, "the loads fit the K-step's MFMAs");
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int wm = WL<NW>::wm(wave);
    const int wn = WL<NW>::wn(wave);

#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nk = (sa.K + BK - 1) / BK;
    if (nk == 0) return;
    LA la;
    LB lb;
    la.init(sa, lds_addr(smem));
    lb.init(sb, lds_addr(smem + BM * BK));
#pragma unroll
    for (int j = PRE; j <= NS - 2; ++j) {
        if constexpr (NS == 2) {
            la.issue(smem + j * STAGE, j);
            lb.issue(smem + j * STAGE + BM * BK, j);
        } else {
#pragma unroll
            for (int q = 0; q < NA; ++q) la.issue_ring((uint32_t)(j * STAGE * 2), j, q, j < nk);
#pragma unroll
            for (int q = 0; q < NB; ++q) lb.issue_ring((uint32_t)(j * STAGE * 2), j, q, j < nk);
        }
    }

    bf16x8 af[2][MI], bfr[2][NJ];
    auto read = [&](int buf, const uint16_t* a_s, const uint16_t* b_s, int ks) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < MI; ++i) af[buf][i] = read_frag<BM, BK, A_MN>(a_s, wm * (BM / 2) + i * 32, ks, lane);
#pragma unroll
        for (int j = 0; j < NJ; ++j) bfr[buf][j] = read_frag<BN, BK, B_MN>(b_s, WL<NW>::sub_col(wn, j), ks, lane);
    };
    // the MFMAs of one k-slice from fragment buffer buf; m0: index of its
    // first MFMA in the K-step's sequence (the previous K-step's last slice,
    // then slices 0 .. KS-2); load instruction q goes out after MFMA
    // (q + 1) * SPAN / NQ - 1
    auto slice = [&](int buf, int m0, auto&& load) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[buf][j], af[buf][i], acc[i][j], 0, 0, 0);
                const int m = m0 + i * NJ + j;
#pragma unroll
                for (int q = 0; q < NQ; ++q)
                    if ((q + 1) * SPAN / NQ - 1 == m) {
                        __builtin_amdgcn_sched_barrier(0);
                        load(q);
                        __builtin_amdgcn_sched_barrier(0);
                    }
            }
    };
    // RI: slice() with the fragments of k-slice ks of the stage at (a_s, b_s)
    // read into buffer rb between its MFMAs (fragment n after MFMA n), in
    // place of a burst of reads ahead of the slice
    auto slice_rd = [&](int buf, int m0, auto&& load, int rb, const uint16_t* a_s, const uint16_t* b_s,
                        int ks) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[buf][j], af[buf][i], acc[i][j], 0, 0, 0);
                const int n = i * NJ + j;
                if (n < MI) af[rb][n] = read_frag<BM, BK, A_MN>(a_s, wm * (BM / 2) + n * 32, ks, lane);
                else if (n < MI + NJ)
                    bfr[rb][n - MI] = read_frag<BN, BK, B_MN>(b_s, WL<NW>::sub_col(wn, n - MI), ks, lane);
                __builtin_amdgcn_sched_barrier(0);
                const int m = m0 + n;
#pragma unroll
                for (int q = 0; q < NQ; ++q)
                    if ((q + 1) * SPAN / NQ - 1 == m) {
                        load(q);
                        __builtin_amdgcn_sched_barrier(0);
                    }
            }
    };
    constexpr bool RI = A_MN && B_MN && MI * NJ >= MI + NJ;

    // one K-step.  MODE 1: the next K-step lies inside K (or is masked past K
    // by the descriptors), so its loads go out without the K-tail test;
    // 2: loads with the K-tail test, if there is a next K-step; 0: no loads
    auto kstep = [&](int kt, auto MODE) __attribute__((always_inline)) {
        constexpr int md = decltype(MODE)::value;
        // this wave's loads of K-step kt have landed (those of the NS - 2
        // K-steps after it, and stores the caller issued after them, may not)
        if (PRE > 0 && stores16 && kt < PRE) wait_vmcnt<NQ * (NS - 2) + NDRAIN>();
        else wait_vmcnt<NQ * (NS - 2)>();
        __syncthreads();     // everyone's have, and the stage loaded next is no longer read
        int so = (kt % NS) * STAGE;
        // one stage base in a scalar register, rather than per-stage copies
        // of every fragment address kept live across the loop
        if constexpr (NS > 2) asm volatile("" : "+s"(so));
        const uint16_t* a_s = smem + so;
        const uint16_t* b_s = a_s + BM * BK;
        const int kn = kt + NS - 1;                                      // the K-step loaded now
        const uint32_t nso = (uint32_t)((kn % NS) * STAGE * 2);          // its stage, bytes
        auto load = [&](int q) __attribute__((always_inline)) {
            if constexpr (md == 1 && NS > 2) {
                if (q < NA) la.issue_ring(nso, kn, q, kn < nk);
                else lb.issue_ring(nso, kn, q - NA, kn < nk);
            } else if constexpr (md == 1) {
                if (q < NA) la.issue_fast(nso, kn, q);
                else lb.issue_fast(nso, kn, q - NA);
            } else if (md == 2 && kt + 1 < nk) {
                uint16_t* nxt = smem + ((kt + 1) & 1) * STAGE;
                if (q < NA) la.issue_one(nxt, kt + 1, q);
                else lb.issue_one(nxt + BM * BK, kt + 1, q - NA);
            }
        };
        if (RI && kt > 0) {
            slice_rd(1, 0, load, 0, a_s, b_s, 0);   // the last k-slice of K-step kt-1
        } else {
            read(0, a_s, b_s, 0);
            __builtin_amdgcn_sched_barrier(0);
            if (kt > 0) {
                slice(1, 0, load);   // the last k-slice of K-step kt-1
            } else {
#pragma unroll
                for (int q = 0; q < NQ; ++q)
                    if ((q + 1) * SPAN / NQ - 1 < SM) load(q);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks + 1 < KS; ++ks) {
            if constexpr (RI) {
                slice_rd(ks & 1, (ks + 1) * SM, load, (ks + 1) & 1, a_s, b_s, ks + 1);
            } else {
                read((ks + 1) & 1, a_s, b_s, ks + 1);
                __builtin_amdgcn_sched_barrier(0);
                slice(ks & 1, (ks + 1) * SM, load);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // KAL: K is a multiple of BK (or both operands are MN-major), so every
    // K-step loaded lies inside K
    if constexpr (NS == 2 && (KAL || (A_MN && B_MN))) {
        for (int kt = 0; kt + 1 < nk; ++kt) kstep(kt, std::integral_constant<int, 1>{});
        kstep(nk - 1, std::integral_constant<int, 0>{});
    } else if constexpr (NS > 2) {
        for (int kt = 0; kt < nk; ++kt) kstep(kt, std::integral_constant<int, 1>{});
    } else {
        for (int kt = 0; kt < nk; ++kt) kstep(kt, std::integral_constant<int, 2>{});
    }
    slice(1, KS * SM, [](int) __attribute__((always_inline)) {});   // the last k-slice of the last K-step
    if constexpr (NS > 2) wait_vmcnt<0>();   // the zero loads past K have landed too
    __syncthreads();  // the LDS may be reused by the caller
}

// Direct loads of half of a K-major 256 x 64 tile (the layout DirectLoader
// writes): 1 KB chunks half*16 + 4i + w4, i = 0..3, of the 32 chunks of a
// K-step; half 0 is rows 0..127, half 1 rows 128..255.
template <int ROWS, int BK>
struct HalfLoader {
    static_assert(ROWS == 256 && BK == 64, "256 x 64 tiles");
    static constexpr int CPR_K = BK / 8;          // 16-byte chunks per row
    static constexpr int RPC_K = 1024 / (BK * 2); // rows per 1 KB chunk
    desc_t d;
    uint32_t off[4];
    uint32_t m0w;     // LDS byte address of chunk half*16 + w4 of the stage-0 tile
    __device__ __forceinline__ void init(const TileSrc& s, uint32_t lds_tile, int half, int w4)
    {
        const int lane = threadIdx.x & 63;
        m0w = lds_tile + (uint32_t)(half * 16 + w4) * 1024u;
        d = wave_uniform(half ? make_desc(s.p1, (int64_t)s.rows1 * s.ld * 2)
                              : make_desc(s.p0, (int64_t)s.rows0 * s.ld * 2));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = half * 16 + i * 4 + w4;
            const int row = q * RPC_K + lane / CPR_K;
            const int c = (int)lds_chunk<false, BK>(row, lane % CPR_K);
            off[i] = (uint32_t)((row - half * (ROWS / 2)) * s.ld * 2 + c * 16);
        }
    }
    // this wave's 4 chunks of K-step kt into the stage at byte offset stage_off
    __device__ __forceinline__ void issue(uint32_t stage_off, int kt)
    {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dma16_to_lds_at(d, m0w + stage_off + (uint32_t)i * 4096u, off[i], (uint32_t)(kt * BK * 2));
    }
};

// Direct loads of half of an MN-major 64 x 256 tile (k-rows of 256 elements,
// the layout DirectLoader<256, 64, true> writes): 1 KB chunks (2 k-rows)
// half*16 + 4i + w4, i = 0..3; half 0 is k-rows 0..31, half 1 k-rows 32..63.
template <int ROWS, int BK>
struct HalfLoaderMN {
    static_assert(ROWS == 256 && BK == 64, "64 x 256 tiles");
    static constexpr int KROWS = 1024 / (ROWS * 2);   // k-rows per 1 KB chunk
    static constexpr int CPR = ROWS / 8;              // 16-byte chunks per k-row
    desc_t d;
    uint32_t off[4];
    uint32_t m0w;
    uint32_t kstep;
    __device__ __forceinline__ void init(const TileSrc& s, uint32_t lds_tile, int half, int w4)
    {
        const int lane = threadIdx.x & 63;
        m0w = lds_tile + (uint32_t)(half * 16 + w4) * 1024u;
        d = wave_uniform(make_desc(s.p0, (int64_t)s.K * s.ld * 2));
        kstep = (uint32_t)(BK * s.ld * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = half * 16 + i * 4 + w4;
            const int k = q * KROWS + lane / CPR;
            const int c = (int)lds_chunk<true, BK>(k, lane % CPR);
            off[i] = c * 8 < s.rows0 ? (uint32_t)(k * s.ld * 2 + c * 16) : kOOB;
        }
    }
    __device__ __forceinline__ void issue(uint32_t stage_off, int kt)
    {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dma16_to_lds_at(d, m0w + stage_off + (uint32_t)i * 4096u, off[i], (uint32_t)kt * kstep);
    }
};

// Direct loads of a column half of an MN-major 64 x 256 tile kept as two
// 64 x 128 sub-tiles (k-rows of 128 elements, sub-tile h = columns
// 128h..128h+127 at byte 16384h): 1 KB chunks (4 k-rows) 4i + w4, i = 0..3,
// of sub-tile `half`.  Chunk placement within a k-row follows lds_chunk<true>.
template <int BK>
struct ColHalfLoaderMN {
    static_assert(BK == 64, "64-deep tiles");
    static constexpr int CPR = 128 / 8;   // 16-byte chunks per k-row
    desc_t d;
    uint32_t off[4];
    uint32_t m0w;
    uint32_t kstep;
    __device__ __forceinline__ void init(const TileSrc& s, uint32_t lds_tile, int half, int w4)
    {
        const int lane = threadIdx.x & 63;
        m0w = lds_tile + (uint32_t)half * 16384u + (uint32_t)w4 * 1024u;
        d = wave_uniform(make_desc(s.p0, (int64_t)s.K * s.ld * 2));
        kstep = (uint32_t)(BK * s.ld * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = i * 4 + w4;
            const int k = q * 4 + lane / CPR;
            const int col = half * 128 + (int)lds_chunk<true, BK>(k, lane % CPR) * 8;
            off[i] = col < s.rows0 ? (uint32_t)(k * s.ld * 2 + col * 2) : kOOB;
        }
    }
    __device__ __forceinline__ void issue(uint32_t stage_off, int kt)
    {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dma16_to_lds_at(d, m0w + stage_off + (uint32_t)i * 4096u, off[i], (uint32_t)kt * kstep);
    }
};

// Ping-pong main loop of a 256 x 256 tile, 8 waves, K-major A, K a multiple
// of 64; B K-major (rows of [N, K] weights) or MN-major ([K, N] weights).
// The two waves of a SIMD belong to different groups (waves 0..3: tile rows
// 0..127, waves 4..7: rows 128..255) that alternate, tick by tick, between
// a compute tick and a memory tick, with a barrier at the end of every tick;
// group 1 runs one tick behind group 0, so on every SIMD one wave keeps the
// MFMA pipe busy while the other issues loads.
//  - compute tick: the 16 MFMAs of one half K-step (32 k) from registers,
//    with the fragments of the group's next half K-step read from LDS in
//    their shadow (one fragment after each of 12 MFMAs); the first k-slice
//    of the next half K-step goes into the registers of the first k-slice of
//    this one once its 8 MFMAs have issued, so three k-slices of fragments
//    are live instead of four;
//  - memory tick: this wave's 4 direct loads (4 KB) of one quarter of a
//    K-step, 16 KB per CU; a direct load blocks the issuing wave for about
//    as long as the CU's load path takes to accept the CU's 16 of them, so
//    none go out in compute ticks.
// The quarters of K-step j (2 LDS stages) go out at ticks 4j-7 (A rows
// 0..127, group 0), 4j-6 (B half 0, group 1), 4j-5 (B half 1, group 0) and
// 4j-4 (A rows 128..255, group 1); group 0 reads K-step j at ticks 4j-2 and
// 4j, group 1 at 4j-1 and 4j+1.  Each quarter is waited for by its loading
// group at the end of the tick before its first read and is loaded only
// after the last read of the K-step two back, at an earlier tick.  B halves
// are rows 0..127 / 128..255 of a K-major tile and k-rows 0..31 / 32..63 of
// an MN-major one; both groups read all of B.
template <bool A_MN, bool B_MN>
__device__ __forceinline__ void mainloop_pp(const TileSrc& sa, const TileSrc& sb, f32x16 (&acc)[4][2],
                                            uint16_t* smem)
{
    constexpr int BM = 256, BK = 64, MI = 4, NJ = 2;
    constexpr int STAGE = (BM + BN) * BK;   // elements per stage
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = wave >> 2;    // group
    const int w4 = wave & 3;    // wave column (and SIMD)

#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // MN-major operands: the rows past K (K = the group's rows) read as zeros
    const int nk = A_MN ? (sa.K + BK - 1) / BK : sa.K / BK;
    if (nk == 0) return;
    const int H = 2 * nk;   // half K-steps
    // group 0 loads A half 0 and B half 1, group 1 B half 0 and A half 1,
    // K-steps 0 and 1 up front
    std::conditional_t<A_MN, ColHalfLoaderMN<BK>, HalfLoader<BM, BK>> ha;
    std::conditional_t<B_MN, HalfLoaderMN<BN, BK>, HalfLoader<BN, BK>> hb;
    ha.init(sa, lds_addr(smem), g, w4);
    hb.init(sb, lds_addr(smem + BM * BK), 1 - g, w4);
    ha.issue(0, 0);
    hb.issue(0, 0);
    if (nk > 1) {
        ha.issue(STAGE * 2, 1);
        hb.issue(STAGE * 2, 1);
    }
    if (nk > 1) wait_vmcnt<8>();
    else wait_vmcnt<0>();
    __syncthreads();

    // fragments of one 16-deep k-slice: 4 A sub-tiles, 2 B sub-tiles
    struct Slot {
        bf16x8 a[MI], b[NJ];
    };
    // fragment m (A 0..3, B 4..5) of k-slice s2 of half K-step hs
    auto read_one = [&](int hs, int s2, int m, Slot& dst) __attribute__((always_inline)) {
        const uint16_t* a_s = smem + ((hs >> 1) & 1) * STAGE;
        const uint16_t* b_s = a_s + BM * BK;
        const int ks = (hs & 1) * 2 + s2;
        if (m < MI) {
            if constexpr (A_MN) dst.a[m] = read_frag<128, BK, true>(a_s + g * 128 * BK, m * 32, ks, lane);
            else dst.a[m] = read_frag<BM, BK, false>(a_s, g * 128 + m * 32, ks, lane);
        }
        else dst.b[m - MI] = read_frag<BN, BK, B_MN>(b_s, WL<8>::sub_col(w4, m - MI), ks, lane);
    };
    // the 16 MFMAs of k-slices p (first) and c1 (second); with RD, the
    // fragments of half K-step hs: its second k-slice into n1 during the
    // first 8 MFMAs, its first k-slice into p (free by then) during the last 8
    auto compute = [&](auto RD, int hs, Slot& p, Slot& c1, Slot& n1) __attribute__((always_inline)) {
        __builtin_amdgcn_s_setprio(1);   // ahead of the memory-phase wave of this SIMD
#pragma unroll
        for (int n = 0; n < 16; ++n) {
            const int i = (n >> 1) & 3, j = n & 1;
            if (n < 8) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(p.b[j], p.a[i], acc[i][j], 0, 0, 0);
            else acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(c1.b[j], c1.a[i], acc[i][j], 0, 0, 0);
            if constexpr (decltype(RD)::value) {
                if (n < 6) read_one(hs, 1, n, n1);
                else if (n >= 8 && n < 14) read_one(hs, 0, n - 8, p);
            }
        }
        if constexpr (decltype(RD)::value) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                // LDS reads per fragment (a transposed, MN-major one takes two)
                constexpr int NRA = A_MN ? 2 : 1, NRB = B_MN ? 2 : 1;
#pragma unroll
                for (int n = 0; n < MI; ++n) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, NRA, 0);
                }
#pragma unroll
                for (int n = 0; n < NJ; ++n) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, NRB, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            }
        }
        __builtin_amdgcn_s_setprio(0);
    };
    // this wave's direct loads of memory tick t
    auto loads = [&](int t) __attribute__((always_inline)) {
        int j;
        if (g == 0) {
            if ((t & 3) == 1) {          // A half 0 of K-step j
                j = (t + 7) >> 2;
                if (j >= 2 && j < nk) ha.issue((uint32_t)(j & 1) * STAGE * 2, j);
            } else {                     // t % 4 == 3: B half 1
                j = (t + 5) >> 2;
                if (j >= 2 && j < nk) hb.issue((uint32_t)(j & 1) * STAGE * 2, j);
            }
        } else {
            if ((t & 3) == 2) {          // B half 0
                j = (t + 6) >> 2;
                if (j >= 2 && j < nk) hb.issue((uint32_t)(j & 1) * STAGE * 2, j);
            } else {                     // t % 4 == 0: A half 1
                j = (t + 4) >> 2;
                if (j >= 2 && j < nk) ha.issue((uint32_t)(j & 1) * STAGE * 2, j);
            }
        }
    };
    // end of tick t: what the next tick reads has landed, then the barrier
    auto end_tick = [&](int t) __attribute__((always_inline)) {
        if ((t & 3) == 1) {
            // K-step j = (t+3)/4 is read from the next tick on: group 0 needs
            // its A half 0 and B half 1 (A half 0 of K-step j+1, issued this
            // tick, may stay in flight), group 1 its B half 0 (A half 1 of
            // K-step j may stay in flight)
            const int j = (t + 3) >> 2;
            const int jn = g == 0 ? j + 1 : j;
            if (jn >= 2 && jn < nk) wait_vmcnt<4>();
            else wait_vmcnt<0>();
        } else if ((t & 3) == 2 && g == 1) {
            // group 1 reads K-step (t+2)/4 from the next tick on and needs its
            // A half 1 (B half 0 of the next K-step, issued this tick, may
            // stay in flight)
            const int jn = ((t + 2) >> 2) + 1;
            if (jn >= 2 && jn < nk) wait_vmcnt<4>();
            else wait_vmcnt<0>();
        }
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
    };
    const std::integral_constant<bool, true> rd;
    const std::integral_constant<bool, false> no_rd;
    Slot sp, sq, sr;   // first k-slice; second k-slice, alternating between sq and sr
    auto read_all = [&](int hs) __attribute__((always_inline)) {
#pragma unroll
        for (int m = 0; m < 6; ++m) read_one(hs, 0, m, sp);
#pragma unroll
        for (int m = 0; m < 6; ++m) read_one(hs, 1, m, sq);
    };

    if (g == 0) {
        read_all(0);
        int u = 0;
        for (; u + 2 < H; u += 2) {
            compute(rd, u + 1, sp, sq, sr);                  // tick 2u
            end_tick(2 * u);
            loads(2 * u + 1);                                // tick 2u+1
            end_tick(2 * u + 1);
            compute(rd, u + 2, sp, sr, sq);                  // tick 2u+2
            end_tick(2 * u + 2);
            loads(2 * u + 3);                                // tick 2u+3
            end_tick(2 * u + 3);
        }
        compute(rd, u + 1, sp, sq, sr);                      // tick 2H-4
        end_tick(2 * u);
        loads(2 * u + 1);
        end_tick(2 * u + 1);
        compute(no_rd, 0, sp, sr, sq);                       // tick 2H-2
        end_tick(2 * u + 2);
        loads(2 * u + 3);
        end_tick(2 * u + 3);
    } else {
        loads(0);                                            // tick 0
        read_all(0);
        end_tick(0);
        int u = 0;
        for (; u + 2 < H; u += 2) {
            compute(rd, u + 1, sp, sq, sr);                  // tick 2u+1
            end_tick(2 * u + 1);
            loads(2 * u + 2);                                // tick 2u+2
            end_tick(2 * u + 2);
            compute(rd, u + 2, sp, sr, sq);                  // tick 2u+3
            end_tick(2 * u + 3);
            loads(2 * u + 4);                                // tick 2u+4
            end_tick(2 * u + 4);
        }
        compute(rd, u + 1, sp, sq, sr);                      // tick 2H-3
        end_tick(2 * u + 1);
        loads(2 * u + 2);
        end_tick(2 * u + 2);
        compute(no_rd, 0, sp, sr, sq);                       // tick 2H-1
        end_tick(2 * u + 3);
    }
}

// Grouped-M GEMM: C[rows of group e] = A[rows of group e] x B_e^T (B_MN = false:
// B_e stored [N, K]) or A x B_e (B_MN = true: B_e stored [K, N]).
// LDS stages of the main loop of a BMS-row tail tile (K a multiple of 64):
// a 64-row K-step is 512 MFMA cycles per SIMD against 40 KB of loads, so two
// stages left it waiting on the load latency most of the time (a 64-row
// tail took 80% of a full tile's time); four stages of 40 KB fill the 160 KB
// of LDS and keep three K-steps of loads in flight, three of 48 KB two.
template <int BMS>
constexpr int tail_stages() { return BMS == 64 ? 4 : 3; }

template <int BM, int BK, int NS, bool B_MN, int EPI, int NW, bool KAL>
__global__ MOE_GEMM_KERNEL_ATTRS_NW(NW) void gemm_grouped_m_kernel(MParams p)
{
    constexpr int SMEM = KAL && BM == 256 && BK == 64 ? tail_stages<64>() * (64 + BN) * BK : NS * (BM + BN) * BK;
    static_assert(SMEM >= NS * (BM + BN) * BK, "LDS for the full-tile loop");
    static_assert(!(KAL && BM == 256 && BK == 64) || SMEM >= tail_stages<128>() * (128 + BN) * BK,
                  "LDS for the tail-tile rings");
    __shared__ __align__(16) uint16_t smem[SMEM];

    // device tile schedule: expert-major, then groups of M-tiles (N-tiles
    // across a group, M-tiles fastest within)
    MTile tile;
    if (!schedule_m<BM>(p.group_off, p.capacity, p.E, p.n_rows, p.ntn, tile)) return;
    const int e = tile.e, nt = tile.nt;
    const int64_t row0 = tile.row0;
    const int rows_valid = tile.rows_valid;

    TileSrc sa;
    sa.p0 = p.A + row0 * p.lda;
    sa.p1 = sa.p0 + (int64_t)(BM / 2) * p.lda;
    sa.ld = p.lda;
    sa.rows0 = min(rows_valid, BM / 2);
    sa.rows1 = max(rows_valid - BM / 2, 0);
    sa.K = p.K;

    TileSrc sb;
    const uint16_t* Be = p.B + (int64_t)e * p.sB;
    sb.ld = p.ldb;
    sb.K = p.K;
    if constexpr (EPI == EPI_SWIGLU_FWD) {
        const int n0 = nt * 128;
        sb.p0 = Be + (int64_t)n0 * p.ldb;
        sb.p1 = Be + (int64_t)(p.f + n0) * p.ldb;
        sb.rows0 = sb.rows1 = min(128, p.f - n0);
    } else if constexpr (B_MN) {
        const int n0 = nt * BN;
        sb.p0 = sb.p1 = Be + n0;
        sb.rows0 = min(BN, p.N - n0);
        sb.rows1 = 0;
    } else {
        const int n0 = nt * BN;
        sb.p0 = Be + (int64_t)n0 * p.ldb;
        sb.p1 = sb.p0 + (int64_t)128 * p.ldb;
        sb.rows0 = max(min(128, p.N - n0), 0);
        sb.rows1 = max(min(128, p.N - n0 - 128), 0);
    }

    if constexpr (BM == 256) {
        // the last M-tile of an expert with at most 64 (128) rows: a 64-row
        // (128-row) tile, with a quarter (half) of the MFMAs and of the A
        // loads of a full tile
        auto small = [&](auto BMS_) __attribute__((always_inline)) {
            constexpr int BMS = decltype(BMS_)::value;
            TileSrc st = sa;
            st.p1 = st.p0 + (int64_t)(BMS / 2) * p.lda;
            st.rows0 = min(rows_valid, BMS / 2);
            st.rows1 = max(rows_valid - BMS / 2, 0);
            f32x16 acc_s[BMS / 64][WL<NW>::NJ];
            mainloop<BMS, BK, KAL ? tail_stages<BMS>() : NS, false, B_MN, NW, KAL>(st, sb, acc_s, smem);
            epilogue_m<BMS, EPI, NW>(acc_s, p, row0, rows_valid, nt, reinterpret_cast<uint8_t*>(smem));
        };
        if (rows_valid <= 64) {
            small(std::integral_constant<int, 64>{});
            return;
        }
        if (rows_valid <= 128) {
            small(std::integral_constant<int, 128>{});
            return;
        }
    }
    f32x16 acc[BM / 64][WL<NW>::NJ];
    if constexpr (KAL && NW == 8 && BM == 256 && BK == 64)
        mainloop_pp<false, B_MN>(sa, sb, acc, smem);
    else
        mainloop<BM, BK, NS, false, B_MN, NW, KAL>(sa, sb, acc, smem);
    epilogue_m<BM, EPI, NW>(acc, p, row0, rows_valid, nt, reinterpret_cast<uint8_t*>(smem));
}



struct KProblem {
    const uint16_t* A;     // [n_rows, M] (M contiguous); group e's rows are its K
    int64_t lda;
    const uint16_t* B;     // [n_rows, N] (N contiguous)
    int64_t ldb;
    int M, N;
    int mtn, ntn;
    uint16_t* C;           // [E, M, N]
    int64_t ldc, sC;
    float* Cf;             // if set: [E, M, N] fp32, added into instead of writing C
};

struct KParams {
    KProblem pr[2];        // up to two weight gradients in one launch
    int nprob;
    const int32_t* group_off;
    int capacity, E;
    int64_t n_rows;
    int* ctl;              // caller workspace: ctl[0] = tile mapping flag (k_deal_flag_kernel)
};

// Whether contiguous tile ranges would load the XCDs unevenly: a weight-gradient
// tile costs about its group's row count (its K) plus a fixed overhead
// (setup, first loads, output store) worth some 256 rows; uneven means the
// busiest XCD's share exceeds the mean by more than 5%.  One wave computes it
// from the group offsets (k_deal_flag_kernel below).
__device__ __forceinline__ bool k_tiles_uneven(const KParams& p, int tiles_e, int per_xcd)
{
    constexpr float kTileCostRows = 256.f;
    const int lane = threadIdx.x & 63;
    float xc[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) xc[x] = 0.f;
    for (int e = lane; e < p.E; e += 64) {
        const float c = (float)group_rows(p.group_off, p.capacity, e, p.n_rows) + kTileCostRows;
        const int64_t a = (int64_t)e * tiles_e, b = a + tiles_e;
#pragma unroll
        for (int x = 0; x < 8; ++x) {
            const int64_t lo = max(a, (int64_t)x * per_xcd), hi = min(b, (int64_t)(x + 1) * per_xcd);
            if (hi > lo) xc[x] += (float)(hi - lo) * c;
        }
    }
    float mx = 0.f, sum = 0.f;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
        float v = xc[x];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
        mx = fmaxf(mx, v);
        sum += v;
    }
    // lanes may round the sums differently: lane 0 decides for the wave
    return __builtin_amdgcn_readfirstlane(mx > 1.05f * (sum * 0.125f) ? 1 : 0) != 0;
}

// Writes p.ctl[0]: 1 if the weight-gradient tiles are dealt to the XCDs in
// runs, 0 for contiguous ranges; and clears the per-XCD tile counters
// p.ctl[1 .. 8] of the persistent kernel.  It runs ahead of every
// weight-gradient launch on the same stream; both live in that call's
// workspace.
__global__ __launch_bounds__(64) void k_deal_flag_kernel(KParams p, int tiles_e, int per_xcd)
{
    const bool d = k_tiles_uneven(p, tiles_e, per_xcd);
    if (threadIdx.x == 0) p.ctl[0] = d ? 1 : 0;
    if (threadIdx.x >= 1 && threadIdx.x <= 8) p.ctl[threadIdx.x] = 0;
}

// Grouped-K GEMM (weight gradients): C_e = A_e^T B_e over the rows of group e,
// for one or two problems sharing the groups.  Tiles are expert-major so the
// tiles reading one expert's rows run together on one XCD.
template <int BM, int BK, int NS, int NW>
__global__ MOE_GEMM_KERNEL_ATTRS_NW(NW) void gemm_grouped_k_kernel(KParams p)
{
    __shared__ __align__(16) uint16_t smem[NS * (BM + BN) * BK];
    const int t0 = p.pr[0].mtn * p.pr[0].ntn;
    const int tiles_e = t0 + (p.nprob > 1 ? p.pr[1].mtn * p.pr[1].ntn : 0);
    const int total = p.E * tiles_e;
    const int xcd = blockIdx.x % 8;
    const int slot = blockIdx.x / 8;
    const int per_xcd = (total + 7) / 8;
    // a contiguous range per XCD: its L2 serves a few groups' operands
    const int Lc = slot < per_xcd ? xcd * per_xcd + slot : total;
    // or runs of kKDealRun tiles dealt round-robin to the XCDs, so that
    // every group's tiles, whatever its row count (the K of its tiles), spread
    // over all XCDs, as the flag kernel decided.  The group bounds of both
    // candidate tiles are read with the flag (selected, not branched on, so
    // the loads stay together): one memory round trip, as for a fixed mapping.
    constexpr int RUN = kKDealRun;
    const int Ld = ((slot / RUN) * 8 + xcd) * RUN + slot % RUN;
    const int ec = min(Lc, total - 1) / tiles_e, ed = min(Ld, total - 1) / tiles_e;
    const int64_t gc0 = group_begin(p.group_off, p.capacity, ec, p.n_rows);
    const int64_t gc1 = group_begin(p.group_off, p.capacity, ec + 1, p.n_rows);
    const int64_t gd0 = group_begin(p.group_off, p.capacity, ed, p.n_rows);
    const int64_t gd1 = group_begin(p.group_off, p.capacity, ed + 1, p.n_rows);
    const bool deal = p.ctl[0] != 0;
    const int L = deal ? Ld : Lc;
    if (L >= total) return;
    const int e = L / tiles_e;
    const int64_t g0 = deal ? gd0 : gc0;
    const int m_e = (int)max((int64_t)0, deal ? gd1 - gd0 : gc1 - gc0);
    int local = L - e * tiles_e;
    const int which = local < t0 ? 0 : 1;
    if (which) local -= t0;
    const KProblem& q = p.pr[which];
    int mt, nt;
    grouped_tile(local, q.mtn, q.ntn, 4, mt, nt);

    TileSrc sa;
    sa.p0 = sa.p1 = q.A + g0 * q.lda + (int64_t)mt * BM;
    sa.ld = q.lda;
    sa.rows0 = min(BM, q.M - mt * BM);
    sa.rows1 = 0;
    sa.K = m_e;
    TileSrc sb;
    sb.p0 = sb.p1 = q.B + g0 * q.ldb + (int64_t)nt * BN;
    sb.ld = q.ldb;
    sb.rows0 = min(BN, q.N - nt * BN);
    sb.rows1 = 0;
    sb.K = m_e;

    // (the ping-pong loop, with both operands transposed and 8 K-steps per
    // tile, measured 5% slower here than the single-group loop)
    f32x16 acc[BM / 64][WL<NW>::NJ];
    mainloop<BM, BK, NS, true, true, NW, true>(sa, sb, acc, smem);

    if (q.Cf)
        add_tile_f32<BM, NW>(acc, q.Cf + (int64_t)e * q.sC + (int64_t)mt * BM * q.ldc, q.ldc, q.M - mt * BM,
                             nt * BN, q.N);
    else
        store_tile<BM, NW>(acc, q.C + (int64_t)e * q.sC + (int64_t)mt * BM * q.ldc, q.ldc, q.M - mt * BM,
                           nt * BN, q.N, reinterpret_cast<uint8_t*>(smem));
}

// Persistent weight-gradient GEMM, bf16 outputs.  One workgroup per CU walks
// the tiles of its XCD's list (the contiguous range or the dealt runs the
// flag kernel chose), taking positions from that XCD's counter in the
// workspace, so tiles of very different K (their group's rows) still spread
// evenly over the CUs.  Per tile, the arithmetic of gemm_grouped_k_kernel
// (the same MFMAs in the same k order), with K-steps of 32 through a ring of
// four LDS stages, so that the loads of a K-step go out three K-steps ahead
// of its MFMAs (two stages of 64 left the loads of the next K-step too little
// time under load).  Between two tiles:
//   - the next position is fetched while the current tile computes, and the
//     group bounds come from a copy in LDS made at the start;
//   - the next tile's first two K-steps go out to stages 0 and 1 before the
//     current tile's epilogue, whose latency then hides under the epilogue;
//   - the epilogue stages the result in stages 2 and 3, 128 columns at a time,
//     and leaves through 16 buffer stores per wave that are always issued
//     (out of range elements are dropped by the buffer's range), so the next
//     tile waits for the stores only from its third K-step on and they drain
//     while its first K-steps compute, instead of every CU storing at once
//     while none computes.  (Storing from the accumulators without LDS, 32
//     bytes of each of 32 rows per instruction, measured 3.1 ms against
//     2.8 ms at e128 with plain stores and 6.6 ms non-temporal.)
template <int NW, bool F32 = false>
__global__ MOE_GEMM_KERNEL_ATTRS_NW(NW) void gemm_grouped_k_persistent(KParams p)
{
    constexpr int BM = 256, BK = 32, NS = 4, PRE = 2;
    constexpr int STAGE = (BM + BN) * BK;           // elements per stage
    static_assert(2 * STAGE * 2 == BM * 128 * 2, "stages 2 and 3 hold 128 staged output columns");
    __shared__ __align__(16) uint16_t smem[NS * STAGE];
    __shared__ int s_pos[2];
    __shared__ int64_t s_gb[kMaxExperts + 1];       // group bounds
    for (int g = threadIdx.x; g <= p.E; g += blockDim.x) s_gb[g] = group_begin(p.group_off, p.capacity, g, p.n_rows);
    const int t0 = p.pr[0].mtn * p.pr[0].ntn;
    const int tiles_e = t0 + (p.nprob > 1 ? p.pr[1].mtn * p.pr[1].ntn : 0);
    const int total = p.E * tiles_e;
    const int xcd = blockIdx.x % 8;
    const int per_xcd = (total + 7) / 8;
    const bool deal = p.ctl[0] != 0;
    int* counter = p.ctl + 1 + xcd;
    // global tile at position j of this XCD's list, total past its end
    auto tile_at = [&](int j) __attribute__((always_inline)) {
        int L;
        if (deal) L = ((j / kKDealRun) * 8 + xcd) * kKDealRun + j % kKDealRun;
        else L = j < per_xcd ? xcd * per_xcd + j : total;
        return __builtin_amdgcn_readfirstlane(L < total ? L : total);
    };
    // a tile, every field wave-uniform (kept in scalar registers)
    struct KT {
        int e, which, mt, nt, m_e;
        int64_t g0;
    };
    auto uni64 = [](int64_t v) __attribute__((always_inline)) {
        const uint64_t u = (uint64_t)v;
        return (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(u >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u));
    };
    auto describe = [&](int L, KT& t) __attribute__((always_inline)) {
        t.e = L / tiles_e;
        int local = L - t.e * tiles_e;
        t.which = local < t0 ? 0 : 1;
        if (t.which) local -= t0;
        grouped_tile(local, t.which ? p.pr[1].mtn : p.pr[0].mtn, t.which ? p.pr[1].ntn : p.pr[0].ntn, 4,
                     t.mt, t.nt);
        t.mt = __builtin_amdgcn_readfirstlane(t.mt);
        t.nt = __builtin_amdgcn_readfirstlane(t.nt);
        const int64_t g0 = s_gb[t.e];
        const int64_t g1 = s_gb[t.e + 1];
        t.g0 = uni64(g0);
        t.m_e = __builtin_amdgcn_readfirstlane((int)max((int64_t)0, g1 - g0));
    };
    auto sources = [&](const KT& t, TileSrc& sa, TileSrc& sb) __attribute__((always_inline)) {
        const KProblem& q = t.which ? p.pr[1] : p.pr[0];
        sa.p0 = sa.p1 = q.A + t.g0 * q.lda + (int64_t)t.mt * BM;
        sa.ld = q.lda;
        sa.rows0 = min(BM, q.M - t.mt * BM);
        sa.rows1 = 0;
        sa.K = t.m_e;
        sb.p0 = sb.p1 = q.B + t.g0 * q.ldb + (int64_t)t.nt * BN;
        sb.ld = q.ldb;
        sb.rows0 = min(BN, q.N - t.nt * BN);
        sb.rows1 = 0;
        sb.K = t.m_e;
    };
    // K-steps 0 .. PRE-1 of tile t into stages 0 .. PRE-1
    auto first_loads = [&](const KT& t) __attribute__((always_inline)) {
        if (t.m_e == 0) return;
        TileSrc sa, sb;
        sources(t, sa, sb);
        DirectLoader<BM, BK, true, NW> la;
        DirectLoader<BN, BK, true, NW> lb;
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));    // recomputed here, not kept live across the tile loop
        la.init_tid(sa, lds_addr(smem), tid);
        lb.init_tid(sb, lds_addr(smem + BM * BK), tid);
        // (LDS byte addresses through M0, no generic pointers kept live;
        // K-steps past the group's rows load zeros)
#pragma unroll
        for (int j = 0; j < PRE; ++j) {
#pragma unroll
            for (int i = 0; i < decltype(la)::PER_WAVE; ++i)
                la.issue_ring((uint32_t)(j * STAGE * 2), j, i, j * BK < t.m_e);
#pragma unroll
            for (int i = 0; i < decltype(lb)::PER_WAVE; ++i)
                lb.issue_ring((uint32_t)(j * STAGE * 2), j, i, j * BK < t.m_e);
        }
    };

    if (threadIdx.x == 0) s_pos[1] = atomicAdd(counter, 1);
    __syncthreads();
    int L = tile_at(s_pos[1]);
    if (L >= total) return;
    KT cur;
    describe(L, cur);
    first_loads(cur);
    bool stores16 = false;
    for (int it = 0;; ++it) {
        int pos = 0;
        if (threadIdx.x == 0) pos = atomicAdd(counter, 1);   // the next tile's position
        TileSrc sa, sb;
        sources(cur, sa, sb);
        f32x16 acc[BM / 64][WL<NW>::NJ];
        mainloop<BM, BK, NS, true, true, NW, true, PRE, F32 ? 8 : 16>(sa, sb, acc, smem, stores16);
        if (threadIdx.x == 0) s_pos[it & 1] = pos;
        __syncthreads();
        const int Ln = tile_at(s_pos[it & 1]);
        KT nxt = cur;
        if (Ln < total) {
            describe(Ln, nxt);
            first_loads(nxt);
        }
        const KProblem& q = cur.which ? p.pr[1] : p.pr[0];
        const int rows = q.M - cur.mt * BM;
        uint8_t* stage23 = reinterpret_cast<uint8_t*>(smem + 2 * STAGE);
        if constexpr (F32) {
            // added into fp32 accumulators: 64 loads and stores per thread,
            // always issued; the last pass's 8 stores drain under the next
            // tile's first K-steps
            add_tile_f32_rows<NW>(acc, q.Cf + (int64_t)cur.e * q.sC + (int64_t)cur.mt * BM * q.ldc, q.ldc, rows,
                                  cur.nt * BN, q.N, stage23);
        } else {
            uint16_t* Ct = q.C + (int64_t)cur.e * q.sC + (int64_t)cur.mt * BM * q.ldc;
            store_colhalf_nt<NW, 0>(acc, Ct, q.ldc, rows, cur.nt * BN, q.N, stage23);
            store_colhalf_nt<NW, 1>(acc, Ct, q.ldc, rows, cur.nt * BN, q.N, stage23);
        }
        if (Ln >= total) return;
        cur = nxt;
        stores16 = true;
    }
}

// Router scores: logits [T, E] fp32 = x [T, d] . W_r [E, d]^T, bf16 operands,
// fp32 accumulate (the gating stays in high precision: tutorial, MXFP8
// section).  A skinny product (E = 128 at most per tile, K = d): the T x d
// activations stream from HBM once and set the pace.  A workgroup of 8
// waves owns 64 rows x 128 experts (each wave 32 x 32; two waves per SIMD,
// so one computes while the other waits on its loads), with the x and W_r
// K-steps of 64 moving HBM/L2 -> LDS by direct loads through a 3-stage ring
// (two K-steps in flight while one is read; 4- and 6-stage rings, 4 waves
// of 32 x 64, and staggering the workgroups' K order all measured slower).
// The scores leave straight from the accumulators, four consecutive fp32
// columns per lane.
constexpr int kRM = 64, kRN = 128, kRK = 64, kRS = 3;
constexpr int kRW = 8;                  // waves: each 32 x 32 (two waves per SIMD)
constexpr int kRJ = 1;                  // 32-expert blocks per wave

__global__ __launch_bounds__(64 * kRW) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ w, int T, int E,
                                                            int d, float* __restrict__ logits)
{
    constexpr int STAGE = (kRM + kRN) * kRK;   // elements per stage
    __shared__ __align__(16) uint16_t smem[kRS * STAGE];
    const int row0 = blockIdx.x * kRM;
    const int n0 = blockIdx.y * kRN;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = wave / (kRW / 2), wn = wave % (kRW / 2);   // rows wm*32 .., experts wn*32*kRJ ..
    TileSrc sa;
    sa.p0 = x + (int64_t)row0 * d;
    sa.p1 = sa.p0 + (int64_t)(kRM / 2) * d;
    sa.ld = d;
    sa.rows0 = max(min(T - row0, kRM / 2), 0);
    sa.rows1 = max(min(T - row0 - kRM / 2, kRM / 2), 0);
    sa.K = d;
    TileSrc sb;
    sb.p0 = w + (int64_t)n0 * d;
    sb.p1 = sb.p0 + (int64_t)(kRN / 2) * d;
    sb.ld = d;
    sb.rows0 = max(min(E - n0, kRN / 2), 0);
    sb.rows1 = max(min(E - n0 - kRN / 2, kRN / 2), 0);
    sb.K = d;
    DirectLoader<kRM, kRK, false, kRW> la;
    DirectLoader<kRN, kRK, false, kRW> lb;
    la.init(sa);
    lb.init(sb);
    constexpr int NQ = DirectLoader<kRM, kRK, false, kRW>::PER_WAVE + DirectLoader<kRN, kRK, false, kRW>::PER_WAVE;
    const int nk = (d + kRK - 1) / kRK;
    auto issue = [&](int kt) __attribute__((always_inline)) {
        uint16_t* st = smem + (kt % kRS) * STAGE;
        la.issue(st, kt);
        lb.issue(st + kRM * kRK, kt);
    };
    static_assert(kRS >= 2 && kRS <= 6, "the waits below cover up to four later K-steps");
    f32x16 acc[kRJ];
#pragma unroll
    for (int j = 0; j < kRJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
    for (int kt = 0; kt < kRS - 1 && kt < nk; ++kt) issue(kt);
    for (int kt = 0; kt < nk; ++kt) {
        // K-step kt has landed once at most the loads of the K-steps issued
        // after it (up to kRS - 2 of them) are outstanding
        switch (min(nk - 1 - kt, kRS - 2)) {
        case 0: wait_vmcnt<0>(); break;
        case 1: wait_vmcnt<NQ>(); break;
        case 2: wait_vmcnt<2 * NQ>(); break;
        case 3: wait_vmcnt<3 * NQ>(); break;
        default: wait_vmcnt<4 * NQ>(); break;
        }
        __syncthreads();   // everyone's loads of kt landed; K-step kt-1's stage is free
        if (kt + kRS - 1 < nk) issue(kt + kRS - 1);
        const uint16_t* a_s = smem + (kt % kRS) * STAGE;
        const uint16_t* b_s = a_s + kRM * kRK;
#pragma unroll
        for (int ks = 0; ks < kRK / 16; ++ks) {
            const bf16x8 af = read_frag<kRM, kRK, false>(a_s, wm * 32, ks, lane);
#pragma unroll
            for (int j = 0; j < kRJ; ++j) {
                const bf16x8 bf = read_frag<kRN, kRK, false>(b_s, (wn * kRJ + j) * 32, ks, lane);
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf, af, acc[j], 0, 0, 0);
            }
        }
    }
    // acc[j] holds the transposed 32 x 32 block (rows wm*32.., experts
    // (wn*kRJ + j)*32 ..): lane l has row (l & 31) and, for g = 0..3, the
    // four experts 8g + 4(l >> 5) + {0..3}
    const int r = row0 + wm * 32 + (lane & 31);
    if (r >= T) return;
#pragma unroll
    for (int j = 0; j < kRJ; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int c = n0 + (wn * kRJ + j) * 32 + 8 * g + 4 * (lane >> 5);
            float* dst = logits + (int64_t)r * E + c;
            if ((E & 3) == 0 && c + 3 < E) {
                *reinterpret_cast<float4*>(dst) =
                    make_float4(acc[j][4 * g], acc[j][4 * g + 1], acc[j][4 * g + 2], acc[j][4 * g + 3]);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (c + q < E) dst[q] = acc[j][4 * g + q];
            }
        }
}

template <int BM, int BK, int NS, bool B_MN, int EPI, int NW>
hipError_t launch_m(const MParams& p, int64_t n_rows, hipStream_t s)
{
    // host-known bound on the M-tiles: sum ceil(m_e / BM) <= n_rows / BM + E
    const int64_t bound = (n_rows / BM + p.E) * (int64_t)p.ntn;
    const int64_t grid = (bound + 7) / 8 * 8;
    if (grid == 0) return hipSuccess;
    // K a multiple of BK: the main loop needs no K-tail tests
    if (p.K % BK == 0)
        hipLaunchKernelGGL((gemm_grouped_m_kernel<BM, BK, NS, B_MN, EPI, NW, true>), dim3((unsigned)grid),
                           dim3(64 * NW), 0, s, p);
    else
        hipLaunchKernelGGL((gemm_grouped_m_kernel<BM, BK, NS, B_MN, EPI, NW, false>), dim3((unsigned)grid),
                           dim3(64 * NW), 0, s, p);
    return hipGetLastError();
}

// workgroups of a persistent launch: one per CU of the current device
// (a multiple of 8, so that every XCD's tile list has workgroups)
int persistent_grid()
{
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu < 8)
        ncu = 256;
    return ncu / 8 * 8;
}

template <int BM, int BK, int NS, int NW>
hipError_t launch_k(const KParams& p, hipStream_t s)
{
    int64_t tiles_e = 0;
    for (int i = 0; i < p.nprob; ++i) tiles_e += (int64_t)p.pr[i].mtn * p.pr[i].ntn;
    const int64_t total = (int64_t)p.E * tiles_e;
    // whole runs on each of the 8 XCDs
    const int64_t grid = (total + 8 * kKDealRun - 1) / (8 * kKDealRun) * (8 * kKDealRun);
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(k_deal_flag_kernel, dim3(1), dim3(64), 0, s, p, (int)tiles_e, (int)((total + 7) / 8));
    // the persistent kernel: for bf16 outputs whose tile offsets fit its
    // 31-bit buffer range, or (its fp32 form) when every problem adds into
    // fp32 accumulators whose tile offsets fit it
    bool persistent = BM == 256 && BK == 64 && NS == 2 && NW == 8, all_f32 = true;
    for (int i = 0; i < p.nprob; ++i) {
        all_f32 = all_f32 && p.pr[i].Cf;
        persistent = persistent && !p.pr[i].Cf && (int64_t)256 * p.pr[i].ldc * 2 < ((int64_t)1 << 31);
        all_f32 = all_f32 && (int64_t)256 * p.pr[i].ldc * 4 < ((int64_t)1 << 31);
    }
    const int64_t pgrid = std::min<int64_t>(persistent_grid(), (total + 7) / 8 * 8);
    if (persistent) {
        hipLaunchKernelGGL((gemm_grouped_k_persistent<NW>), dim3((unsigned)pgrid), dim3(64 * NW), 0, s, p);
    } else if (all_f32 && BM == 256 && BK == 64 && NS == 2 && NW == 8) {
        hipLaunchKernelGGL((gemm_grouped_k_persistent<NW, true>), dim3((unsigned)pgrid), dim3(64 * NW), 0, s, p);
    } else {
        hipLaunchKernelGGL((gemm_grouped_k_kernel<BM, BK, NS, NW>), dim3((unsigned)grid), dim3(64 * NW), 0, s, p);
    }
    return hipGetLastError();
}

constexpr int kBM = 256;   // M tile of the grouped-M (forward / dgrad) GEMMs
constexpr int kBMK = 256;  // M tile of the grouped-K (weight gradient) GEMM
constexpr int kBK = 64;    // K step
constexpr int kNS = 2;     // LDS pipeline stages
constexpr int kNW = 8;     // waves per workgroup (two per SIMD)

}  // namespace

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* w, int T, int E, int d, float* logits,
                                hipStream_t s)
{
    if (T == 0) return hipSuccess;
    const dim3 grid((unsigned)((T + kRM - 1) / kRM), (unsigned)((E + kRN - 1) / kRN));
    hipLaunchKernelGGL(router_logits_kernel, grid, dim3(64 * kRW), 0, s, x, w, T, E, d, logits);
    return hipGetLastError();
}

hipError_t gemm_op_bf16(int op, const moe_gemm_tensors& t, GroupSpec g, int d, int f,
                        hipStream_t s)
{
    MParams p{};
    p.group_off = g.group_off;
    p.capacity = g.capacity;
    p.E = g.E;
    p.n_rows = g.n_rows;
    p.f = f;
    switch (op) {
    case MOE_GEMM_GATE_UP:  // gu = x [Wg|Wu]^T, h = silu(g) * u
        p.A = (const uint16_t*)t.x_perm;
        p.lda = d;
        p.B = (const uint16_t*)t.w13;
        p.ldb = d;
        p.sB = (int64_t)2 * f * d;
        p.N = f;
        p.K = d;
        p.ntn = (f + 127) / 128;
        p.C = (uint16_t*)t.gu;
        p.ldc = 2 * f;
        p.H = (uint16_t*)t.h;
        p.ldh = f;
        return launch_m<kBM, kBK, kNS, false, EPI_SWIGLU_FWD, kNW>(p, g.n_rows, s);
    case MOE_GEMM_DOWN:  // y = h Wd^T
        p.A = (const uint16_t*)t.h;
        p.lda = f;
        p.B = (const uint16_t*)t.w2;
        p.ldb = f;
        p.sB = (int64_t)d * f;
        p.N = d;
        p.K = f;
        p.ntn = (d + BN - 1) / BN;
        p.C = (uint16_t*)t.y_perm;
        p.ldc = d;
        return launch_m<kBM, kBK, kNS, false, EPI_STORE, kNW>(p, g.n_rows, s);
    case MOE_GEMM_DGRAD_DOWN:  // dh = dy Wd (Wd_e stored [d, f] = [K, N]), SwiGLU backward
        p.A = (const uint16_t*)t.dy_perm;
        p.lda = d;
        p.B = (const uint16_t*)t.w2;
        p.ldb = f;
        p.sB = (int64_t)d * f;
        p.N = f;
        p.K = d;
        p.ntn = (f + BN - 1) / BN;
        p.C = (uint16_t*)t.dgu;
        p.ldc = 2 * f;
        p.G = (const uint16_t*)t.gu;
        p.ldg = 2 * f;
        return launch_m<kBM, kBK, kNS, true, EPI_SWIGLU_BWD, kNW>(p, g.n_rows, s);
    case MOE_GEMM_DGRAD_GATE_UP:  // dx = [dg | du] [Wg ; Wu] (W13_e stored [2f, d] = [K, N])
        p.A = (const uint16_t*)t.dgu;
        p.lda = 2 * f;
        p.B = (const uint16_t*)t.w13;
        p.ldb = d;
        p.sB = (int64_t)2 * f * d;
        p.N = d;
        p.K = 2 * f;
        p.ntn = (d + BN - 1) / BN;
        p.C = (uint16_t*)t.dx_perm;
        p.ldc = d;
        return launch_m<kBM, kBK, kNS, true, EPI_STORE, kNW>(p, g.n_rows, s);
    case MOE_GEMM_WGRAD: {  // dWd_e [d, f] = dy_e^T h_e ; dW13_e [2f, d] = dgu_e^T x_e
        KParams k{};
        k.group_off = g.group_off;
        k.capacity = g.capacity;
        k.E = g.E;
        k.n_rows = g.n_rows;
        k.ctl = static_cast<int*>(t.ws);
        k.nprob = 2;
        KProblem& a = k.pr[0];
        a.A = (const uint16_t*)t.dy_perm;
        a.lda = d;
        a.B = (const uint16_t*)t.h;
        a.ldb = f;
        a.M = d;
        a.N = f;
        a.mtn = (d + kBMK - 1) / kBMK;
        a.ntn = (f + BN - 1) / BN;
        a.C = (uint16_t*)t.dw2;
        a.Cf = t.dw2_f32;
        a.ldc = f;
        a.sC = (int64_t)d * f;
        KProblem& b = k.pr[1];
        b.A = (const uint16_t*)t.dgu;
        b.lda = 2 * f;
        b.B = (const uint16_t*)t.x_perm;
        b.ldb = d;
        b.M = 2 * f;
        b.N = d;
        b.mtn = (2 * f + kBMK - 1) / kBMK;
        b.ntn = (d + BN - 1) / BN;
        b.C = (uint16_t*)t.dw13;
        b.Cf = t.dw13_f32;
        b.ldc = d;
        b.sC = (int64_t)2 * f * d;
        return launch_k<kBMK, kBK, kNS, kNW>(k, s);
    }
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace moe
