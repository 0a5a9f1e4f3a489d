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
//   - tiles are BM x 256 x 64, four waves in a 2 x 2 grid, each wave owning
//     (BM/2) x 128 of fp32 accumulators; operands are staged in LDS (row pitch
//     144 B: conflict-free 16-byte fragment reads), double-buffered so the
//     next K-step's global loads are in flight during the MFMAs;
//   - operands stored with K contiguous are copied to LDS as 16-byte
//     vectors; operands stored with M/N contiguous (the weight in dgrad, both
//     operands of wgrad) are read as 8 k-rows x 16 bytes per thread and
//     transposed in registers before the 16-byte LDS stores;
//   - epilogues: plain bf16 store; the SwiGLU forward (each wave holds the
//     gate and up accumulators of the same columns, so h = silu(g) * u is
//     formed in registers and g, u, h are stored); the SwiGLU backward (reads
//     the saved g, u of its elements and stores dg, du).
// Accumulation is fp32; bf16 results are rounded to nearest even.
#include "moe_internal.h"

namespace moe {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int BK = 64;
constexpr int BN = 256;
constexpr int NTH = 256;
constexpr int LDT = BK + 8;  // LDS row pitch, bf16 elements (144 bytes)

enum { EPI_STORE = 0, EPI_SWIGLU_FWD = 1, EPI_SWIGLU_BWD = 2 };

// A ROWS x BK tile source.  K-major: element (r, k) at p[r*ld + k] (rows split
// into two halves with their own bases and valid counts).  MN-major: element
// (r, k) at p[k*ld + r].
struct TileSrc {
    const uint16_t* p0;
    const uint16_t* p1;
    int64_t ld;
    int rows0, rows1;   // valid rows per half (K-major) / rows0 = valid rows (MN-major)
    int K;              // valid k
};

template <int ROWS>
struct KMajorLoader {
    static constexpr int NV = ROWS / 32;
    uint4 v[NV];
    __device__ __forceinline__ void load(const TileSrc& s, int k0)
    {
        const int kc = threadIdx.x & 7;
        const int rb = threadIdx.x >> 3;
        const int kk = k0 + kc * 8;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            constexpr int HALF = ROWS / 2;
            const bool hi = i * 32 >= HALF;
            const int r = i * 32 + rb - (hi ? HALF : 0);
            const uint16_t* p = hi ? s.p1 : s.p0;
            const int nrow = hi ? s.rows1 : s.rows0;
            uint4 val = make_uint4(0, 0, 0, 0);
            if (r < nrow && kk < s.K) val = *reinterpret_cast<const uint4*>(p + r * s.ld + kk);
            v[i] = val;
        }
    }
    __device__ __forceinline__ void store(uint16_t* lds) const
    {
        const int kc = threadIdx.x & 7;
        const int rb = threadIdx.x >> 3;
#pragma unroll
        for (int i = 0; i < NV; ++i)
            *reinterpret_cast<uint4*>(lds + (i * 32 + rb) * LDT + kc * 8) = v[i];
    }
};

// MN-major source: each thread owns KB k-rows x 8 rows (KB = 8 for 256 rows,
// 4 for 128), reads KB 16-byte vectors and transposes them in registers.
template <int ROWS>
struct MNMajorLoader {
    static constexpr int KB = ROWS == 256 ? 8 : 4;
    static constexpr int NKB = BK / KB;     // k-blocks per tile (8 or 16)
    uint4 v[KB];
    __device__ __forceinline__ void load(const TileSrc& s, int k0)
    {
        const int rblk = threadIdx.x / NKB;
        const int kblk = threadIdx.x % NKB;
        const bool rok = rblk * 8 < s.rows0;
#pragma unroll
        for (int q = 0; q < KB; ++q) {
            const int k = k0 + kblk * KB + q;
            uint4 val = make_uint4(0, 0, 0, 0);
            if (rok && k < s.K) val = *reinterpret_cast<const uint4*>(s.p0 + (int64_t)k * s.ld + rblk * 8);
            v[q] = val;
        }
    }
    __device__ __forceinline__ void store(uint16_t* lds) const
    {
        const int rblk = threadIdx.x / NKB;
        const int kblk = threadIdx.x % NKB;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            // k-values of row c: element c of each v[q]
            uint32_t e[KB];
#pragma unroll
            for (int q = 0; q < KB; ++q) {
                const uint32_t d = (c >> 1) == 0 ? v[q].x : (c >> 1) == 1 ? v[q].y : (c >> 1) == 2 ? v[q].z : v[q].w;
                e[q] = (c & 1) ? (d >> 16) : (d & 0xffffu);
            }
            uint16_t* dst = lds + (rblk * 8 + c) * LDT + kblk * KB;
            if constexpr (KB == 8) {
                *reinterpret_cast<uint4*>(dst) = make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16),
                                                            e[4] | (e[5] << 16), e[6] | (e[7] << 16));
            } else {
                *reinterpret_cast<uint2*>(dst) = make_uint2(e[0] | (e[1] << 16), e[2] | (e[3] << 16));
            }
        }
    }
};

template <int ROWS, bool MN>
using Loader = typename std::conditional<MN, MNMajorLoader<ROWS>, KMajorLoader<ROWS>>::type;

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

// column (0..255) of the tile that wave column wn, sub-tile j, lane covers
__device__ __forceinline__ int tile_col(int wn, int j, int lane)
{
    return (j >> 1) * 128 + wn * 64 + (j & 1) * 32 + (lane & 31);
}

// BM x 256 tile, K loop over s.K, accumulators acc[BM/64][4]
template <int BM, bool A_MN, bool B_MN>
__device__ __forceinline__ void mainloop(const TileSrc& sa, const TileSrc& sb, f32x16 (&acc)[BM / 64][4],
                                         uint16_t* smem)
{
    constexpr int MI = BM / 64;
    // stage s: A tile at smem + s * STAGE, B tile right after it.  Offsets (not
    // a table of pointers) keep every access in the LDS address space.
    constexpr int STAGE = (BM + BN) * LDT;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int wm = wave >> 1;
    const int wn = wave & 1;

#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nk = (sa.K + BK - 1) / BK;
    if (nk == 0) return;
    Loader<BM, A_MN> la;
    Loader<BN, B_MN> lb;
    la.load(sa, 0);
    lb.load(sb, 0);
    la.store(smem);
    lb.store(smem + BM * LDT);
    __syncthreads();

    const int arow = wm * (BM / 2) + (lane & 31);
    const int kofs = (lane >> 5) * 8;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
            la.load(sa, (kt + 1) * BK);
            lb.load(sb, (kt + 1) * BK);
        }
        const uint16_t* a_s = smem + cur * STAGE;
        const uint16_t* b_s = a_s + BM * LDT;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            bf16x8 af[MI], bfr[4];
#pragma unroll
            for (int i = 0; i < MI; ++i)
                af[i] = *reinterpret_cast<const bf16x8*>(a_s + (arow + i * 32) * LDT + ks * 16 + kofs);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int brow = (j >> 1) * 128 + wn * 64 + (j & 1) * 32 + (lane & 31);
                bfr[j] = *reinterpret_cast<const bf16x8*>(b_s + brow * LDT + ks * 16 + kofs);
            }
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (more) {
            uint16_t* nxt = smem + (cur ^ 1) * STAGE;
            la.store(nxt);
            lb.store(nxt + BM * LDT);
        }
        __syncthreads();
    }
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
};

template <int BM, int EPI>
__device__ __forceinline__ void epilogue_m(const f32x16 (&acc)[BM / 64][4], const MParams& p,
                                           int64_t row0, int rows_valid, int nt)
{
    constexpr int MI = BM / 64;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int wm = wave >> 1;
    const int wn = wave & 1;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = wm * (BM / 2) + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
            if (row >= rows_valid) continue;
            const int64_t grow = row0 + row;
            if constexpr (EPI == EPI_SWIGLU_FWD) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int n = nt * 128 + tile_col(wn, j, lane);
                    if (n >= p.f) continue;
                    const float g = acc[i][j][r];
                    const float u = acc[i][j + 2][r];
                    p.C[grow * p.ldc + n] = (uint16_t)f32_to_bf16_bits(g);
                    p.C[grow * p.ldc + p.f + n] = (uint16_t)f32_to_bf16_bits(u);
                    p.H[grow * p.ldh + n] = (uint16_t)f32_to_bf16_bits(silu_f(g) * u);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int n = nt * BN + tile_col(wn, j, lane);
                    if (n >= p.N) continue;
                    const float v = acc[i][j][r];
                    if constexpr (EPI == EPI_STORE) {
                        p.C[grow * p.ldc + n] = (uint16_t)f32_to_bf16_bits(v);
                    } else {
                        const float g = bf16_to_f32(p.G[grow * p.ldg + n]);
                        const float u = bf16_to_f32(p.G[grow * p.ldg + p.f + n]);
                        const float s = 1.0f / (1.0f + __expf(-g));
                        const float da = v * u;
                        const float du = v * g * s;
                        const float dg = da * s * (1.0f + g * (1.0f - s));
                        p.C[grow * p.ldc + n] = (uint16_t)f32_to_bf16_bits(dg);
                        p.C[grow * p.ldc + p.f + n] = (uint16_t)f32_to_bf16_bits(du);
                    }
                }
            }
        }
    }
}

// Grouped-M GEMM: C[rows of group e] = A[rows of group e] x B_e^T (B_MN = false:
// B_e stored [N, K]) or A x B_e (B_MN = true: B_e stored [K, N]).
template <int BM, bool B_MN, int EPI>
__global__ __launch_bounds__(NTH, 1) void gemm_grouped_m_kernel(MParams p)
{
    __shared__ __align__(16) uint16_t smem[2 * (BM + BN) * LDT];
    __shared__ int s_pref[kMaxExperts + 1];
    __shared__ int s_part[NTH];

    // device tile schedule: expert-major, N-tile, then M-tile
    const int total =
        block_tile_prefix<NTH>(p.group_off, p.capacity, p.E, p.n_rows, BM, p.ntn, s_pref, s_part);
    const int per_xcd = (total + 7) / 8;
    const int xcd = blockIdx.x % 8;
    const int slot = blockIdx.x / 8;
    if (slot >= per_xcd) return;
    const int L = xcd * per_xcd + slot;
    if (L >= total) return;
    const int e = find_group(s_pref, p.E, L);
    const int64_t g0 = group_begin(p.group_off, p.capacity, e, p.n_rows);
    const int m_e = (int)group_rows(p.group_off, p.capacity, e, p.n_rows);
    const int mt_e = (m_e + BM - 1) / BM;
    const int local = L - s_pref[e];
    const int nt = local / mt_e;
    const int mt = local - nt * mt_e;
    const int64_t row0 = g0 + (int64_t)mt * BM;
    const int rows_valid = min(BM, m_e - mt * BM);

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

    f32x16 acc[BM / 64][4];
    mainloop<BM, false, B_MN>(sa, sb, acc, smem);
    epilogue_m<BM, EPI>(acc, p, row0, rows_valid, nt);
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
};

struct KParams {
    KProblem pr[2];        // up to two weight gradients in one launch
    int nprob;
    const int32_t* group_off;
    int capacity, E;
    int64_t n_rows;
};

// Grouped-K GEMM (weight gradients): C_e = A_e^T B_e over the rows of group e,
// for one or two problems sharing the groups.  Tiles are expert-major so the
// tiles reading one expert's rows run together on one XCD.
template <int BM>
__global__ __launch_bounds__(NTH, 1) void gemm_grouped_k_kernel(KParams p)
{
    __shared__ __align__(16) uint16_t smem[2 * (BM + BN) * LDT];
    const int t0 = p.pr[0].mtn * p.pr[0].ntn;
    const int tiles_e = t0 + (p.nprob > 1 ? p.pr[1].mtn * p.pr[1].ntn : 0);
    const int total = p.E * tiles_e;
    const int per_xcd = (total + 7) / 8;
    const int xcd = blockIdx.x % 8;
    const int slot = blockIdx.x / 8;
    if (slot >= per_xcd) return;
    const int L = xcd * per_xcd + slot;
    if (L >= total) return;
    const int e = L / tiles_e;
    int local = L - e * tiles_e;
    const int which = local < t0 ? 0 : 1;
    if (which) local -= t0;
    const KProblem& q = p.pr[which];
    const int mt = local / q.ntn;
    const int nt = local - mt * q.ntn;
    const int64_t g0 = group_begin(p.group_off, p.capacity, e, p.n_rows);
    const int m_e = (int)group_rows(p.group_off, p.capacity, e, p.n_rows);

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

    f32x16 acc[BM / 64][4];
    mainloop<BM, true, true>(sa, sb, acc, smem);

    constexpr int MI = BM / 64;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int wm = wave >> 1;
    const int wn = wave & 1;
    uint16_t* Ce = q.C + (int64_t)e * q.sC;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = mt * BM + wm * (BM / 2) + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
            if (m >= q.M) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = nt * BN + tile_col(wn, j, lane);
                if (n < q.N) Ce[(int64_t)m * q.ldc + n] = (uint16_t)f32_to_bf16_bits(acc[i][j][r]);
            }
        }
}

template <int BM, bool B_MN, int EPI>
hipError_t launch_m(const MParams& p, int64_t n_rows, hipStream_t s)
{
    // host-known bound on the M-tiles: sum ceil(m_e / BM) <= n_rows / BM + E
    const int64_t bound = (n_rows / BM + p.E) * (int64_t)p.ntn;
    const int64_t grid = (bound + 7) / 8 * 8;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((gemm_grouped_m_kernel<BM, B_MN, EPI>), dim3((unsigned)grid), dim3(NTH), 0,
                       s, p);
    return hipGetLastError();
}

template <int BM>
hipError_t launch_k(const KParams& p, hipStream_t s)
{
    int64_t tiles_e = 0;
    for (int i = 0; i < p.nprob; ++i) tiles_e += (int64_t)p.pr[i].mtn * p.pr[i].ntn;
    const int64_t total = (int64_t)p.E * tiles_e;
    const int64_t grid = (total + 7) / 8 * 8;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((gemm_grouped_k_kernel<BM>), dim3((unsigned)grid), dim3(NTH), 0, s, p);
    return hipGetLastError();
}

constexpr int kBM = 128;

}  // namespace

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
        return launch_m<kBM, false, EPI_SWIGLU_FWD>(p, g.n_rows, s);
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
        return launch_m<kBM, false, EPI_STORE>(p, g.n_rows, s);
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
        return launch_m<kBM, true, EPI_SWIGLU_BWD>(p, g.n_rows, s);
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
        return launch_m<kBM, true, EPI_STORE>(p, g.n_rows, s);
    case MOE_GEMM_WGRAD: {  // dWd_e [d, f] = dy_e^T h_e ; dW13_e [2f, d] = dgu_e^T x_e
        KParams k{};
        k.group_off = g.group_off;
        k.capacity = g.capacity;
        k.E = g.E;
        k.n_rows = g.n_rows;
        k.nprob = 2;
        KProblem& a = k.pr[0];
        a.A = (const uint16_t*)t.dy_perm;
        a.lda = d;
        a.B = (const uint16_t*)t.h;
        a.ldb = f;
        a.M = d;
        a.N = f;
        a.mtn = (d + kBM - 1) / kBM;
        a.ntn = (f + BN - 1) / BN;
        a.C = (uint16_t*)t.dw2;
        a.ldc = f;
        a.sC = (int64_t)d * f;
        KProblem& b = k.pr[1];
        b.A = (const uint16_t*)t.dgu;
        b.lda = 2 * f;
        b.B = (const uint16_t*)t.x_perm;
        b.ldb = d;
        b.M = 2 * f;
        b.N = d;
        b.mtn = (2 * f + kBM - 1) / kBM;
        b.ntn = (d + BN - 1) / BN;
        b.C = (uint16_t*)t.dw13;
        b.ldc = d;
        b.sC = (int64_t)2 * f * d;
        return launch_k<kBM>(k, s);
    }
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace moe
