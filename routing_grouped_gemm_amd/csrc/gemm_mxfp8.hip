// MXFP8 grouped GEMMs on gfx950's block-scaled MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 operands, one E8M0 scale per 32 k).
//
// The OLMo-core 3 tutorial (MXFP8 section) runs all three GEMMs of each
// linear (forward, activation gradient, weight gradient) in MXFP8: E4M3
// elements with one power-of-two scale per 32 elements along the contraction
// dimension, with forward- and backward-direction weight caches.  Every GEMM
// here therefore reads both operands with K contiguous:
//   forward   gu = x Wg|Wu^T       x row-wise (dispatch payload), W13 forward cache
//             y  = h Wd^T          h row-wise (made by the gate/up epilogue), W2 forward cache
//   dgrad     dh = dy Wd           dy row-wise,  Wd^T  (backward cache [E, f, d])
//             dx = dgu [Wg;Wu]     dgu row-wise (made by the dgrad-down epilogue),
//                                  W13^T (backward cache [E, d, 2f])
//   wgrad     dWd = dy^T h, dW13 = dgu^T x   all four quantised column-wise
//             inside each expert's rows, stored group-transposed and padded
//             to 128 rows, so the tokens are the contiguous K.
// Tiles, LDS layout, schedule and epilogues are those of the bf16 kernels:
// a 128-byte K-step row of fp8 codes is the same LDS tile as 64 bf16.  Each
// K-step also brings a [rows][4] tile of scale bytes (four 32-k blocks per
// row); lane i passes its row's scale of the first 32-k block of an MFMA
// k-slice, lane i+32 that of the second.
#include "gemm_common.h"

namespace moe {

namespace {

using namespace gemm;

typedef __attribute__((ext_vector_type(8))) int i32x8;

constexpr int MBK = 128;   // K-step in fp8 elements (128 bytes per row)
constexpr int MNS = 2;     // LDS stages

// K-major MXFP8 operand tile source: codes [rows][K] bytes, scales [rows][K/32].
struct MxSrc {
    const uint8_t* c0;   // codes of rows [0, half)
    const uint8_t* c1;   // codes of rows [half, 2*half)
    const uint8_t* s0;   // scales of the same rows
    const uint8_t* s1;
    int64_t ldc;         // code row stride in bytes (>= K)
    int rows0, rows1;
    int K;               // multiple of 128
};

// scale bytes of a ROWS-row tile for one K-step: [ROWS][4] bytes in LDS, filled
// by 4-byte direct loads (64 rows per wave instruction, NW waves)
template <int ROWS, int NW = 4>
struct ScaleLoader {
    static constexpr int PER_WAVE = ROWS / 64 / NW > 0 ? ROWS / 64 / NW : 1;
    static constexpr int INSTR = ROWS / 64;   // instructions per tile
    static constexpr int HALF = ROWS / 2;
    desc_t r0, r1;
    uint32_t off[PER_WAVE];
    __device__ __forceinline__ void init(const MxSrc& s)
    {
        const int lane = threadIdx.x & 63;
        const int w = threadIdx.x >> 6;
        const int64_t lds_ = s.ldc / 32;   // scale row stride in bytes
        r0 = make_desc(s.s0, (int64_t)s.rows0 * lds_);
        r1 = make_desc(s.s1, (int64_t)s.rows1 * lds_);
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) {
            const int q = i * NW + w;
            const int row = q * 64 + lane;
            const int rr = row >= HALF ? row - HALF : row;
            off[i] = q < INSTR ? (uint32_t)(rr * lds_) : kOOB;
        }
    }
    __device__ __forceinline__ void issue(uint8_t* tile, int kt)
    {
        const int w = threadIdx.x >> 6;
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) {
            const int q = i * NW + w;
            if (q < INSTR) {
                const bool hi = q * 64 >= HALF;
                dma_to_lds<4>(wave_uniform(hi ? r1 : r0), tile + q * 256, off[i], (uint32_t)kt * 4);
            }
        }
    }
};

__device__ __forceinline__ TileSrc codes_as_tile(const MxSrc& s)
{
    // two fp8 codes per 16-bit "element": a 128-byte code row is a 64-element tile row
    TileSrc t;
    t.p0 = reinterpret_cast<const uint16_t*>(s.c0);
    t.p1 = reinterpret_cast<const uint16_t*>(s.c1);
    t.ld = s.ldc / 2;
    t.rows0 = s.rows0;
    t.rows1 = s.rows1;
    t.K = s.K / 2;
    return t;
}

// A-/B-operand of one block-scaled MFMA for k-slice ks (64 k = 32-k blocks
// 2ks and 2ks+1) of tile row row_base + (lane & 31).  The instruction takes
// block 0 from bytes 0..15 of lanes i and i+32 together (scale from lane i)
// and block 1 from bytes 16..31 of both (scale from lane i+32), so lane half
// h holds the h-th 16-code chunk of each block.
__device__ __forceinline__ i32x8 read_frag_mx(const uint16_t* tile, int row_base, int ks, int lane)
{
    const int row = row_base + (lane & 31);
    const int c = ks * 4 + (lane >> 5);   // chunk of block 2ks; block 2ks+1 is two chunks on
    const uint4 lo = *reinterpret_cast<const uint4*>(tile + row * 64 + lds_chunk<false, 64>(row, c) * 8);
    const uint4 hi = *reinterpret_cast<const uint4*>(tile + row * 64 + lds_chunk<false, 64>(row, c + 2) * 8);
    const i32x8 v = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    return v;
}

template <int BM, int NW>
__device__ __forceinline__ void mainloop_mx(const MxSrc& sa, const MxSrc& sb,
                                            f32x16 (&acc)[BM / 64][WL<NW>::NJ], uint8_t* smem)
{
    constexpr int MI = BM / 64;
    constexpr int NJ = WL<NW>::NJ;
    constexpr int CODE_BYTES = (BM + BN) * MBK;
    constexpr int STAGE = CODE_BYTES + (BM + BN) * 4;   // codes then scales
    using LA = DirectLoader<BM, 64, false, NW>;
    using LB = DirectLoader<BN, 64, false, NW>;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int wm = WL<NW>::wm(wave);
    const int wn = WL<NW>::wn(wave);
    const int half = lane >> 5;

#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nk = sa.K / MBK;
    if (nk == 0) return;
    LA la;
    LB lb;
    la.init(codes_as_tile(sa));
    lb.init(codes_as_tile(sb));
    ScaleLoader<BM, NW> ska;
    ScaleLoader<BN, NW> skb;
    ska.init(sa);
    skb.init(sb);
    auto issue = [&](int kt, int stage) {
        uint8_t* st = smem + stage * STAGE;
        la.issue(reinterpret_cast<uint16_t*>(st), kt);
        lb.issue(reinterpret_cast<uint16_t*>(st + BM * MBK), kt);
        ska.issue(st + CODE_BYTES, kt);
        skb.issue(st + CODE_BYTES + BM * 4, kt);
    };
    issue(0, 0);
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        wait_vmcnt<0>();
        __syncthreads();
        if (kt + 1 < nk) issue(kt + 1, cur ^ 1);
        const uint8_t* st = smem + cur * STAGE;
        const uint16_t* a_s = reinterpret_cast<const uint16_t*>(st);
        const uint16_t* b_s = reinterpret_cast<const uint16_t*>(st + BM * MBK);
        const uint32_t* sa_s = reinterpret_cast<const uint32_t*>(st + CODE_BYTES);
        const uint32_t* sb_s = reinterpret_cast<const uint32_t*>(st + CODE_BYTES + BM * 4);
        // scale words of this lane's rows: byte b = 32-k block b of the K-step
        uint32_t sca[MI], scb[NJ];
#pragma unroll
        for (int i = 0; i < MI; ++i) sca[i] = sa_s[wm * (BM / 2) + i * 32 + (lane & 31)];
#pragma unroll
        for (int j = 0; j < NJ; ++j) scb[j] = sb_s[WL<NW>::sub_col(wn, j) + (lane & 31)];
#pragma unroll
        for (int ks = 0; ks < MBK / 64; ++ks) {
            i32x8 af[MI], bfr[NJ];
#pragma unroll
            for (int i = 0; i < MI; ++i) af[i] = read_frag_mx(a_s, wm * (BM / 2) + i * 32, ks, lane);
#pragma unroll
            for (int j = 0; j < NJ; ++j) bfr[j] = read_frag_mx(b_s, WL<NW>::sub_col(wn, j), ks, lane);
            const int sh = 8 * (2 * ks + half);
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        bfr[j], af[i], acc[i][j], 0, 0, 0, (int)((scb[j] >> sh) & 0xffu), 0,
                        (int)((sca[i] >> sh) & 0xffu));
        }
    }
    __syncthreads();
}

struct MxMParams {
    MParams p;             // shapes, schedule and epilogue outputs (p.A / p.B unused)
    const uint8_t* Aq;     // [n_rows, K] codes
    const uint8_t* As;     // [n_rows, K/32] scales
    const uint8_t* Bq;     // per expert [N_total, K] codes at Bq + e * sBq
    const uint8_t* Bs;
    int64_t sBq;           // bytes between experts' codes (scales: sBq / 32)
};

template <int BM, int EPI, int NW>
__global__ MOE_GEMM_KERNEL_ATTRS_NW(NW) void mx_grouped_m_kernel(MxMParams mp)
{
    __shared__ __align__(16) uint8_t smem[MNS * ((BM + BN) * MBK + (BM + BN) * 4)];
    const MParams& p = mp.p;
    MTile tile;
    if (!schedule_m<BM>(p.group_off, p.capacity, p.E, p.n_rows, p.ntn, tile)) return;
    const int e = tile.e, nt = tile.nt;
    const int64_t K = p.K;

    MxSrc sa;
    sa.c0 = mp.Aq + tile.row0 * K;
    sa.c1 = sa.c0 + (int64_t)(BM / 2) * K;
    sa.s0 = mp.As + tile.row0 * (K / 32);
    sa.s1 = sa.s0 + (int64_t)(BM / 2) * (K / 32);
    sa.ldc = K;
    sa.rows0 = min(tile.rows_valid, BM / 2);
    sa.rows1 = max(tile.rows_valid - BM / 2, 0);
    sa.K = (int)K;

    MxSrc sb;
    const uint8_t* Bq = mp.Bq + (int64_t)e * mp.sBq;
    const uint8_t* Bs = mp.Bs + (int64_t)e * (mp.sBq / 32);
    sb.ldc = K;
    sb.K = (int)K;
    int r_lo, r_hi;
    if constexpr (EPI == EPI_SWIGLU_FWD) {
        const int n0 = nt * 128;
        r_lo = n0;
        r_hi = p.f + n0;
        sb.rows0 = sb.rows1 = min(128, p.f - n0);
    } else {
        const int n0 = nt * BN;
        r_lo = n0;
        r_hi = n0 + 128;
        sb.rows0 = max(min(128, p.N - n0), 0);
        sb.rows1 = max(min(128, p.N - n0 - 128), 0);
    }
    sb.c0 = Bq + (int64_t)r_lo * K;
    sb.c1 = Bq + (int64_t)r_hi * K;
    sb.s0 = Bs + (int64_t)r_lo * (K / 32);
    sb.s1 = Bs + (int64_t)r_hi * (K / 32);

    f32x16 acc[BM / 64][WL<NW>::NJ];
    mainloop_mx<BM, NW>(sa, sb, acc, smem);
    // the SwiGLU epilogues also write the row-wise MXFP8 h / dgu the next stage reads
    epilogue_m<BM, EPI, NW, EPI != EPI_STORE>(acc, p, tile.row0, tile.rows_valid, nt, smem);
}

// weight gradient over group-transposed operands: C_e = A_e B_e^T with
// A_e = [M][Kp_e], B_e = [N][Kp_e] at byte offset M * P_e (resp. N * P_e)
struct MxKProblem {
    const uint8_t* Aq;
    const uint8_t* As;
    const uint8_t* Bq;
    const uint8_t* Bs;
    int M, N, mtn, ntn;
    uint16_t* C;           // [E, M, N] bf16
    int64_t ldc, sC;
};

struct MxKParams {
    MxKProblem pr[2];
    const int32_t* group_off;
    int capacity, E;
    int64_t n_rows;
    int* ctl;              // caller workspace: ctl[0] = tile mapping flag (mx_k_deal_flag_kernel)
};

// Weight-gradient tiles go to the XCDs as contiguous ranges, or dealt in runs
// of kMxDealRun when contiguous ranges would load the XCDs unevenly: a tile
// costs about its group's padded row count (its K) plus a fixed overhead
// worth some 256 rows, and uneven means the busiest XCD's share exceeds the
// mean by more than 5%.  One wave decides ahead of each launch and leaves the
// answer in the call's workspace (p.ctl[0]).
constexpr int kMxDealRun = 4;

__global__ __launch_bounds__(64) void mx_k_deal_flag_kernel(MxKParams p, int tiles_e, int per_xcd)
{
    const int lane = threadIdx.x & 63;
    float xc[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) xc[x] = 0.f;
    for (int e = lane; e < p.E; e += 64) {
        const int64_t m = group_rows(p.group_off, p.capacity, e, p.n_rows);
        const float c = (float)((m + kMxColPad - 1) / kMxColPad * kMxColPad) + 256.f;
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
    // lanes may round the sums differently: lane 0 decides
    if (threadIdx.x == 0) p.ctl[0] = mx > 1.05f * (sum * 0.125f) ? 1 : 0;
}

template <int BM, int NW>
__global__ MOE_GEMM_KERNEL_ATTRS_NW(NW) void mx_grouped_k_kernel(MxKParams p)
{
    __shared__ __align__(16) uint8_t smem[MNS * ((BM + BN) * MBK + (BM + BN) * 4)];
    __shared__ int s_pref[kMaxExperts + 1];
    __shared__ int s_part[64 * NW];
    // padded row offsets of the groups: P_e = 128 * s_pref[e]
    block_tile_prefix<64 * NW>(p.group_off, p.capacity, p.E, p.n_rows, kMxColPad, 1, s_pref, s_part);
    const int t0 = p.pr[0].mtn * p.pr[0].ntn;
    const int tiles_e = t0 + p.pr[1].mtn * p.pr[1].ntn;
    const int total = p.E * tiles_e;
    const int per_xcd = (total + 7) / 8;
    const int xcd = blockIdx.x % 8;
    const int slot = blockIdx.x / 8;
    const int L = p.ctl[0] ? ((slot / kMxDealRun) * 8 + xcd) * kMxDealRun + slot % kMxDealRun
                              : (slot < per_xcd ? xcd * per_xcd + slot : total);
    if (L >= total) return;
    const int e = L / tiles_e;
    int local = L - e * tiles_e;
    const int which = local < t0 ? 0 : 1;
    if (which) local -= t0;
    const MxKProblem& q = p.pr[which];
    int mt, nt;
    grouped_tile(local, q.mtn, q.ntn, 4, mt, nt);
    const int64_t P = (int64_t)s_pref[e] * kMxColPad;
    const int64_t Kp = (int64_t)(s_pref[e + 1] - s_pref[e]) * kMxColPad;

    MxSrc sa;
    sa.ldc = Kp;
    sa.K = (int)Kp;
    const int64_t a_row0 = (int64_t)mt * BM;
    sa.c0 = q.Aq + (int64_t)q.M * P + a_row0 * Kp;
    sa.c1 = sa.c0 + (int64_t)(BM / 2) * Kp;
    sa.s0 = q.As + (int64_t)q.M * P / 32 + a_row0 * (Kp / 32);
    sa.s1 = sa.s0 + (int64_t)(BM / 2) * (Kp / 32);
    const int arows = min(BM, q.M - mt * BM);
    sa.rows0 = min(arows, BM / 2);
    sa.rows1 = max(arows - BM / 2, 0);
    MxSrc sb;
    sb.ldc = Kp;
    sb.K = (int)Kp;
    const int64_t b_row0 = (int64_t)nt * BN;
    sb.c0 = q.Bq + (int64_t)q.N * P + b_row0 * Kp;
    sb.c1 = sb.c0 + (int64_t)128 * Kp;
    sb.s0 = q.Bs + (int64_t)q.N * P / 32 + b_row0 * (Kp / 32);
    sb.s1 = sb.s0 + (int64_t)128 * (Kp / 32);
    const int brows = min(BN, q.N - nt * BN);
    sb.rows0 = min(brows, 128);
    sb.rows1 = max(brows - 128, 0);

    f32x16 acc[BM / 64][WL<NW>::NJ];
    mainloop_mx<BM, NW>(sa, sb, acc, smem);
    store_tile<BM, NW>(acc, q.C + (int64_t)e * q.sC + a_row0 * q.ldc, q.ldc, arows, nt * BN, q.N, smem);
}

constexpr int kMxBM = 256;
// waves per workgroup of the MXFP8 GEMMs: two per SIMD.  Eight waves of
// 128 x 64 measured 1-2% faster over the MXFP8 shard's step than four of
// 128 x 128 (down, both dgrads and the weight gradient 2-4% faster, gate/up
// 2% slower); spreading the next K-step's direct loads between the MFMAs, as
// the bf16 loop does, made it 10% slower here.
constexpr int kMxNW = 8;

template <int EPI>
hipError_t launch_mx_m(const MxMParams& mp, hipStream_t s)
{
    const int64_t bound = (mp.p.n_rows / kMxBM + mp.p.E) * (int64_t)mp.p.ntn;
    const int64_t grid = (bound + 7) / 8 * 8;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((mx_grouped_m_kernel<kMxBM, EPI, kMxNW>), dim3((unsigned)grid), dim3(64 * kMxNW), 0, s, mp);
    return hipGetLastError();
}

// workspace carve-up (all offsets 256-byte aligned)
struct MxWs {
    int* ctl;                                             // kGemmCtlBytes of control words
    uint8_t *hq, *hs, *dyq, *dys, *dguq, *dgus;           // row-wise
    uint8_t *dyT, *dyTs, *hT, *hTs, *dguT, *dguTs, *xT, *xTs;   // column-wise, group-transposed
};

inline size_t al(size_t v) { return (v + 255) / 256 * 256; }

size_t carve(void* ws, int E, int64_t R, int d, int f, MxWs* w)
{
    const size_t Rp = (size_t)R + (size_t)kMxColPad * E;
    const size_t sz[14] = {(size_t)R * f, (size_t)R * f / 32, (size_t)R * d, (size_t)R * d / 32,
                           (size_t)R * 2 * f, (size_t)R * 2 * f / 32, Rp * d, Rp * d / 32,
                           Rp * f, Rp * f / 32, Rp * 2 * f, Rp * 2 * f / 32, Rp * d, Rp * d / 32};
    uint8_t* base = reinterpret_cast<uint8_t*>(ws);
    if (w) w->ctl = reinterpret_cast<int*>(base);
    size_t off = kGemmCtlBytes;
    uint8_t** dst[14] = {w ? &w->hq : nullptr, w ? &w->hs : nullptr, w ? &w->dyq : nullptr,
                         w ? &w->dys : nullptr, w ? &w->dguq : nullptr, w ? &w->dgus : nullptr,
                         w ? &w->dyT : nullptr, w ? &w->dyTs : nullptr, w ? &w->hT : nullptr,
                         w ? &w->hTs : nullptr, w ? &w->dguT : nullptr, w ? &w->dguTs : nullptr,
                         w ? &w->xT : nullptr, w ? &w->xTs : nullptr};
    for (int i = 0; i < 14; ++i) {
        if (w) *dst[i] = base + off;
        off += al(sz[i]);
    }
    return off;
}

}  // namespace

size_t gemm_ws_mxfp8(int E, int64_t n_rows, int d, int f) { return carve(nullptr, E, n_rows, d, f, nullptr) + 256; }

// One stage of the MXFP8 grouped GEMM: the quantisation of the bf16
// operands it reads that no earlier stage left in the workspace, then one
// block-scaled GEMM.  GATE_UP and DGRAD_DOWN also write the row-wise MXFP8
// copy of their bf16 output (h, dgu) from their epilogues, which DOWN and
// DGRAD_GATE_UP read.  w13 / w2 are the forward caches for GATE_UP / DOWN and
// the backward (transposed, column-quantised) caches for the two DGRAD stages.
hipError_t gemm_op_mxfp8(int op, const moe_gemm_tensors& t, GroupSpec g, int d, int f, void* ws,
                         hipStream_t s)
{
    MxWs w;
    carve(ws, g.E, g.n_rows, d, f, &w);
    const int64_t R = g.n_rows;
    hipError_t err = hipSuccess;
    MxMParams a{};
    a.p.group_off = g.group_off;
    a.p.capacity = g.capacity;
    a.p.E = g.E;
    a.p.n_rows = R;
    a.p.f = f;
    a.Bq = static_cast<const uint8_t*>(op == MOE_GEMM_GATE_UP || op == MOE_GEMM_DGRAD_GATE_UP ? t.w13 : t.w2);
    a.Bs = op == MOE_GEMM_GATE_UP || op == MOE_GEMM_DGRAD_GATE_UP ? t.w13_scales : t.w2_scales;
    switch (op) {
    case MOE_GEMM_GATE_UP:   // gu = x [Wg | Wu]^T with the SwiGLU epilogue
        a.p.N = f;
        a.p.K = d;
        a.p.ntn = (f + 127) / 128;
        a.p.C = static_cast<uint16_t*>(t.gu);
        a.p.ldc = 2 * f;
        a.p.H = static_cast<uint16_t*>(t.h);
        a.p.ldh = f;
        a.p.Mq = w.hq;           // the row-wise MXFP8 h the down GEMM reads
        a.p.Ms = w.hs;
        a.p.ldq = f;
        a.Aq = static_cast<const uint8_t*>(t.x_perm);
        a.As = t.x_perm_scales;
        a.sBq = (int64_t)2 * f * d;
        return launch_mx_m<EPI_SWIGLU_FWD>(a, s);
    case MOE_GEMM_DOWN:      // y = h Wd^T, h quantised along f (by the GATE_UP epilogue)
        a.p.N = d;
        a.p.K = f;
        a.p.ntn = (d + BN - 1) / BN;
        a.p.C = static_cast<uint16_t*>(t.y_perm);
        a.p.ldc = d;
        a.Aq = w.hq;
        a.As = w.hs;
        a.sBq = (int64_t)d * f;
        return launch_mx_m<EPI_STORE>(a, s);
    case MOE_GEMM_DGRAD_DOWN:   // dh = dy Wd (cache Wd^T [E, f, d]) with the SwiGLU backward
        if ((err = launch_quantize_rows(static_cast<const uint16_t*>(t.dy_perm), R, d, w.dyq, w.dys, s)) !=
            hipSuccess)
            return err;
        a.p.N = f;
        a.p.K = d;
        a.p.ntn = (f + BN - 1) / BN;
        a.p.C = static_cast<uint16_t*>(t.dgu);
        a.p.ldc = 2 * f;
        a.p.G = static_cast<const uint16_t*>(t.gu);
        a.p.ldg = 2 * f;
        a.p.Mq = w.dguq;         // the row-wise MXFP8 dgu the gate/up dgrad GEMM reads
        a.p.Ms = w.dgus;
        a.p.ldq = 2 * f;
        a.Aq = w.dyq;
        a.As = w.dys;
        a.sBq = (int64_t)f * d;
        return launch_mx_m<EPI_SWIGLU_BWD>(a, s);
    case MOE_GEMM_DGRAD_GATE_UP:   // dx = [dg | du] [Wg ; Wu] (cache W13^T [E, d, 2f]), dgu quantised along
        a.p.N = d;                 // 2f by the DGRAD_DOWN epilogue
        a.p.K = 2 * f;
        a.p.ntn = (d + BN - 1) / BN;
        a.p.C = static_cast<uint16_t*>(t.dx_perm);
        a.p.ldc = d;
        a.Aq = w.dguq;
        a.As = w.dgus;
        a.sBq = (int64_t)d * 2 * f;
        return launch_mx_m<EPI_STORE>(a, s);
    case MOE_GEMM_WGRAD:
        break;
    default:
        return hipErrorInvalidValue;
    }
    // weight gradients: all four operands column-wise inside each expert's rows
    const uint16_t* dy = static_cast<const uint16_t*>(t.dy_perm);
    if ((err = launch_quantize_cols(dy, R, d, g.group_off, g.capacity, g.E, w.dyT, w.dyTs, s)) != hipSuccess)
        return err;
    if ((err = launch_quantize_cols(static_cast<const uint16_t*>(t.h), R, f, g.group_off, g.capacity, g.E, w.hT,
                                    w.hTs, s)) != hipSuccess)
        return err;
    if ((err = launch_quantize_cols(static_cast<const uint16_t*>(t.dgu), R, 2 * f, g.group_off, g.capacity, g.E,
                                    w.dguT, w.dguTs, s)) != hipSuccess)
        return err;
    if ((err = launch_dequant_requant_cols(static_cast<const uint8_t*>(t.x_perm), t.x_perm_scales, R, d,
                                           g.group_off, g.capacity, g.E, w.xT, w.xTs, s)) != hipSuccess)
        return err;
    MxKParams k{};
    k.group_off = g.group_off;
    k.capacity = g.capacity;
    k.E = g.E;
    k.n_rows = R;
    k.ctl = w.ctl;
    MxKProblem& p0 = k.pr[0];   // dWd [d, f] = dy^T h
    p0.Aq = w.dyT;
    p0.As = w.dyTs;
    p0.Bq = w.hT;
    p0.Bs = w.hTs;
    p0.M = d;
    p0.N = f;
    p0.mtn = (d + kMxBM - 1) / kMxBM;
    p0.ntn = (f + BN - 1) / BN;
    p0.C = static_cast<uint16_t*>(t.dw2);
    p0.ldc = f;
    p0.sC = (int64_t)d * f;
    MxKProblem& p1 = k.pr[1];   // dW13 [2f, d] = dgu^T x
    p1.Aq = w.dguT;
    p1.As = w.dguTs;
    p1.Bq = w.xT;
    p1.Bs = w.xTs;
    p1.M = 2 * f;
    p1.N = d;
    p1.mtn = (2 * f + kMxBM - 1) / kMxBM;
    p1.ntn = (d + BN - 1) / BN;
    p1.C = static_cast<uint16_t*>(t.dw13);
    p1.ldc = d;
    p1.sC = (int64_t)2 * f * d;
    const int64_t total = (int64_t)g.E * (p0.mtn * p0.ntn + p1.mtn * p1.ntn);
    // whole runs of dealt tiles on each of the 8 XCDs
    const int64_t grid = (total + 8 * kMxDealRun - 1) / (8 * kMxDealRun) * (8 * kMxDealRun);
    if (grid > 0) {
        hipLaunchKernelGGL(mx_k_deal_flag_kernel, dim3(1), dim3(64), 0, s, k,
                           p0.mtn * p0.ntn + p1.mtn * p1.ntn, (int)((total + 7) / 8));
        hipLaunchKernelGGL((mx_grouped_k_kernel<kMxBM, kMxNW>), dim3((unsigned)grid), dim3(64 * kMxNW), 0, s, k);
    }
    return hipGetLastError();
}

}  // namespace moe
