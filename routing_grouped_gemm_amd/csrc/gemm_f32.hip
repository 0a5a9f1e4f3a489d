// Grouped SwiGLU GEMMs in fp32 on the vector ALUs (the fp32 workload: fp32
// activations and weights, fp32 accumulate).  Same device tile schedule and
// epilogue semantics as the bf16 MFMA path; 64 x 64 tiles, 256 threads with a
// 4 x 4 register micro-tile each, operands staged in LDS as [k][row].
// For the SwiGLU forward a tile's 64 logical columns are 32 gate columns and
// the same 32 up columns, so the epilogue (through LDS) forms h = silu(g) * u.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int TM = 64, TN = 64, TK = 16;

enum { EPI_STORE = 0, EPI_SWIGLU_FWD = 1, EPI_SWIGLU_BWD = 2 };

struct F32M {
    const float* A;        // [n_rows, K] grouped rows
    int64_t lda;
    const float* B;        // per-expert weight, B + e * sB
    int64_t ldb, sB;
    bool b_mn;             // B_e stored [K, N] (else [N, K])
    int N, K;
    const int32_t* group_off;
    int capacity, E, ntn;
    int64_t n_rows;
    float* C;
    int64_t ldc;
    float* H;
    int64_t ldh;
    const float* G;
    int64_t ldg;
    int f;
};

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

template <int EPI>
__global__ __launch_bounds__(256) void f32_grouped_m_kernel(F32M p)
{
    __shared__ float sA[TK][TM + 4];
    __shared__ float sB[TK][TN + 4];
    __shared__ float sC[TM][TN + 1];
    __shared__ int s_pref[kMaxExperts + 1];
    __shared__ int s_part[256];

    const int total =
        block_tile_prefix<256>(p.group_off, p.capacity, p.E, p.n_rows, TM, p.ntn, s_pref, s_part);
    if ((int)blockIdx.x >= total) return;
    const int L = blockIdx.x;
    const int e = find_group(s_pref, p.E, L);
    const int64_t g0 = group_begin(p.group_off, p.capacity, e, p.n_rows);
    const int m_e = (int)group_rows(p.group_off, p.capacity, e, p.n_rows);
    const int mt_e = (m_e + TM - 1) / TM;
    const int local = L - s_pref[e];
    const int nt = local / mt_e;
    const int mt = local - nt * mt_e;
    const int64_t row0 = g0 + (int64_t)mt * TM;
    const int rows_valid = min(TM, m_e - mt * TM);
    const float* Be = p.B + (int64_t)e * p.sB;
    const int n0 = EPI == EPI_SWIGLU_FWD ? nt * (TN / 2) : nt * TN;

    const int tid = threadIdx.x;
    const int tx = tid % 16, ty = tid / 16;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < p.K; k0 += TK) {
        for (int idx = tid; idx < TM * TK; idx += 256) {
            const int r = idx / TK, kk = idx % TK;
            const int k = k0 + kk;
            sA[kk][r] = (r < rows_valid && k < p.K) ? p.A[(row0 + r) * p.lda + k] : 0.0f;
        }
        for (int idx = tid; idx < TN * TK; idx += 256) {
            const int c = idx / TK, kk = idx % TK;
            const int k = k0 + kk;
            int64_t brow;
            bool ok;
            if (EPI == EPI_SWIGLU_FWD) {
                const int n = n0 + (c % (TN / 2));
                ok = n < p.f;
                brow = c < TN / 2 ? n : p.f + n;
            } else {
                brow = n0 + c;
                ok = brow < p.N;
            }
            float v = 0.0f;
            if (ok && k < p.K) v = p.b_mn ? Be[(int64_t)k * p.ldb + brow] : Be[brow * p.ldb + k];
            sB[kk][c] = v;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < TK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = sB[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) sC[ty * 4 + i][tx * 4 + j] = acc[i][j];
    __syncthreads();
    if (EPI == EPI_SWIGLU_FWD) {
        for (int idx = tid; idx < TM * (TN / 2); idx += 256) {
            const int r = idx / (TN / 2), c = idx % (TN / 2);
            const int n = n0 + c;
            if (r >= rows_valid || n >= p.f) continue;
            const float g = sC[r][c], u = sC[r][c + TN / 2];
            const int64_t row = row0 + r;
            p.C[row * p.ldc + n] = g;
            p.C[row * p.ldc + p.f + n] = u;
            p.H[row * p.ldh + n] = silu(g) * u;
        }
    } else {
        for (int idx = tid; idx < TM * TN; idx += 256) {
            const int r = idx / TN, c = idx % TN;
            const int n = n0 + c;
            if (r >= rows_valid || n >= p.N) continue;
            const int64_t row = row0 + r;
            const float v = sC[r][c];
            if (EPI == EPI_STORE) {
                p.C[row * p.ldc + n] = v;
            } else {
                const float g = p.G[row * p.ldg + n], u = p.G[row * p.ldg + p.f + n];
                const float s = 1.0f / (1.0f + expf(-g));
                const float da = v * u;
                p.C[row * p.ldc + n] = da * s * (1.0f + g * (1.0f - s));
                p.C[row * p.ldc + p.f + n] = v * g * s;
            }
        }
    }
}

struct F32KProblem {
    const float* A;        // [n_rows, M]
    int64_t lda;
    const float* B;        // [n_rows, N]
    int64_t ldb;
    int M, N, mtn, ntn;
    float* C;              // [E, M, N]
    int64_t ldc, sC;
};

struct F32K {
    F32KProblem pr[2];
    int nprob;
    const int32_t* group_off;
    int capacity, E;
    int64_t n_rows;
};

__global__ __launch_bounds__(256) void f32_grouped_k_kernel(F32K p)
{
    __shared__ float sA[TK][TM + 4];
    __shared__ float sB[TK][TN + 4];
    const int t0 = p.pr[0].mtn * p.pr[0].ntn;
    const int tiles_e = t0 + (p.nprob > 1 ? p.pr[1].mtn * p.pr[1].ntn : 0);
    const int L = blockIdx.x;
    const int e = L / tiles_e;
    int local = L - e * tiles_e;
    const int which = local < t0 ? 0 : 1;
    if (which) local -= t0;
    const F32KProblem& q = p.pr[which];
    const int mt = local / q.ntn, nt = local - (local / q.ntn) * q.ntn;
    const int64_t g0 = group_begin(p.group_off, p.capacity, e, p.n_rows);
    const int m_e = (int)group_rows(p.group_off, p.capacity, e, p.n_rows);
    const int m0 = mt * TM, n0 = nt * TN;
    const int tid = threadIdx.x;
    const int tx = tid % 16, ty = tid / 16;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < m_e; k0 += TK) {
        for (int idx = tid; idx < TM * TK; idx += 256) {
            const int kk = idx / TM, c = idx % TM;
            const int k = k0 + kk;
            sA[kk][c] = (k < m_e && m0 + c < q.M) ? q.A[(g0 + k) * q.lda + m0 + c] : 0.0f;
            sB[kk][c] = (k < m_e && n0 + c < q.N) ? q.B[(g0 + k) * q.ldb + n0 + c] : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < TK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = sB[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
    float* Ce = q.C + (int64_t)e * q.sC;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
            if (m < q.M && n < q.N) Ce[(int64_t)m * q.ldc + n] = acc[i][j];
        }
}

template <int EPI>
hipError_t launch_m(const F32M& p, int64_t n_rows, hipStream_t s)
{
    const int64_t grid = (n_rows / TM + p.E) * (int64_t)p.ntn;
    if (grid > 0) hipLaunchKernelGGL((f32_grouped_m_kernel<EPI>), dim3((unsigned)grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_k(const F32K& p, hipStream_t s)
{
    int64_t tiles_e = 0;
    for (int i = 0; i < p.nprob; ++i) tiles_e += (int64_t)p.pr[i].mtn * p.pr[i].ntn;
    const int64_t grid = (int64_t)p.E * tiles_e;
    if (grid > 0) hipLaunchKernelGGL(f32_grouped_k_kernel, dim3((unsigned)grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t gemm_op_f32(int op, const moe_gemm_tensors& t, GroupSpec g, int d, int f,
                       hipStream_t s)
{
    F32M p{};
    p.group_off = g.group_off;
    p.capacity = g.capacity;
    p.E = g.E;
    p.n_rows = g.n_rows;
    p.f = f;
    switch (op) {
    case MOE_GEMM_GATE_UP:
        p.A = (const float*)t.x_perm;
        p.lda = d;
        p.B = (const float*)t.w13;
        p.ldb = d;
        p.sB = (int64_t)2 * f * d;
        p.b_mn = false;
        p.N = f;
        p.K = d;
        p.ntn = (f + TN / 2 - 1) / (TN / 2);
        p.C = (float*)t.gu;
        p.ldc = 2 * f;
        p.H = (float*)t.h;
        p.ldh = f;
        return launch_m<EPI_SWIGLU_FWD>(p, g.n_rows, s);
    case MOE_GEMM_DOWN:
        p.A = (const float*)t.h;
        p.lda = f;
        p.B = (const float*)t.w2;
        p.ldb = f;
        p.sB = (int64_t)d * f;
        p.b_mn = false;
        p.N = d;
        p.K = f;
        p.ntn = (d + TN - 1) / TN;
        p.C = (float*)t.y_perm;
        p.ldc = d;
        return launch_m<EPI_STORE>(p, g.n_rows, s);
    case MOE_GEMM_DGRAD_DOWN:
        p.A = (const float*)t.dy_perm;
        p.lda = d;
        p.B = (const float*)t.w2;
        p.ldb = f;
        p.sB = (int64_t)d * f;
        p.b_mn = true;
        p.N = f;
        p.K = d;
        p.ntn = (f + TN - 1) / TN;
        p.C = (float*)t.dgu;
        p.ldc = 2 * f;
        p.G = (const float*)t.gu;
        p.ldg = 2 * f;
        return launch_m<EPI_SWIGLU_BWD>(p, g.n_rows, s);
    case MOE_GEMM_DGRAD_GATE_UP:
        p.A = (const float*)t.dgu;
        p.lda = 2 * f;
        p.B = (const float*)t.w13;
        p.ldb = d;
        p.sB = (int64_t)2 * f * d;
        p.b_mn = true;
        p.N = d;
        p.K = 2 * f;
        p.ntn = (d + TN - 1) / TN;
        p.C = (float*)t.dx_perm;
        p.ldc = d;
        return launch_m<EPI_STORE>(p, g.n_rows, s);
    case MOE_GEMM_WGRAD: {
        F32K k{};
        k.group_off = g.group_off;
        k.capacity = g.capacity;
        k.E = g.E;
        k.n_rows = g.n_rows;
        k.nprob = 2;
        F32KProblem& a = k.pr[0];
        a.A = (const float*)t.dy_perm;
        a.lda = d;
        a.B = (const float*)t.h;
        a.ldb = f;
        a.M = d;
        a.N = f;
        a.mtn = (d + TM - 1) / TM;
        a.ntn = (f + TN - 1) / TN;
        a.C = (float*)t.dw2;
        a.ldc = f;
        a.sC = (int64_t)d * f;
        F32KProblem& b = k.pr[1];
        b.A = (const float*)t.dgu;
        b.lda = 2 * f;
        b.B = (const float*)t.x_perm;
        b.ldb = d;
        b.M = 2 * f;
        b.N = d;
        b.mtn = (2 * f + TM - 1) / TM;
        b.ntn = (d + TN - 1) / TN;
        b.C = (float*)t.dw13;
        b.ldc = d;
        b.sC = (int64_t)2 * f * d;
        return launch_k(k, s);
    }
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace moe
