/*
 * moe_oracle.c -- plain CPU oracle for one GPU's MoE feed-forward layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path
 * (the HIP library under routing_grouped_gemm_amd/) never calls it, shares
 * no code, header, table or helper with it, and must fail loudly when its
 * own extension is missing.
 *
 * Every floating-point value is held and accumulated in fp64.  Storage
 * rounding is modelled explicitly, only at the points where the layer
 * stores a tensor (round_mode: 0 = none, 1 = fp32, 2 = bf16, all
 * round-to-nearest-even).  Loops are written in the obvious order; no
 * blocking, fusion or reordering beyond what the definitions state.  Every
 * output element is produced by exactly one thread in a fixed summation
 * order, so results do not depend on the OpenMP thread count.
 *
 * Sources (the pages describing the OLMo-core 3 MoE training stack):
 *  - "OLMo-core 3: MoE 训练栈..." tutorial, section on the routing tax
 *    (paragraphs "rowwise EP" and "另外两处税: 主机同步与 padding"): the
 *    device-built route map (per-expert counts, row counts, per-expert
 *    permutation), rows written straight into their expert's input buffer,
 *    and one grouped GEMM over the exact per-expert row counts with no
 *    padding to a common capacity.
 *  - same tutorial, MXFP8 section: E4M3 elements with one power-of-two
 *    E8M0 scale per 32 elements, scale chosen from the block maximum and
 *    448 so that the block maximum does not overflow; three GEMMs per
 *    linear (forward, activation gradient, weight gradient).
 *  - "Ai2 Olmo-core 3: The Secret Behind 2.7x MoE Training Throughput",
 *    MoE explainer paragraph: each token activates only its top-k experts.
 * Where the pages are silent (router score function, gate normalisation,
 * tie-break, SwiGLU form, rounding points, capacity policy) the plainest
 * reading is taken; each such reading is named at the function below.
 *
 * Parity pins: every function here is checked in tests/ against something
 * other than itself (brute force, library routines, closed forms,
 * invariants), the MXFP8 composition of the FFN (mx_h, mx_dgu and the
 * substituted GEMM operands) against an independent torch chain and exact
 * operand probes, with planted mistakes that the checks must catch.  The
 * MXFP8 scale rounds the block maximum over 448 up to a power of two: of
 * the two power-of-two roundings it is the one that keeps the block maximum
 * from overflowing, the property the tutorial's MXFP8 paragraph states
 * (pinned); the pages do not print their own code, so agreement with it
 * cannot be checked beyond that property.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------ */
/* Storage rounding                                                    */
/* ------------------------------------------------------------------ */

/* Round a double to the nearest bfloat16 value (8 significant bits,
 * fp32 exponent range, subnormals kept), ties to even.  Done directly from
 * the double, a single rounding. */
static double round_bf16(double v)
{
    if (v == 0.0 || isnan(v) || isinf(v)) return v;
    double a = fabs(v);
    int ex;
    frexp(a, &ex);                 /* a = m * 2^ex, m in [0.5, 1) */
    /* bf16 quantum: 2^(ex-8) for normals (ex-1 >= -126), 2^-133 below */
    int qexp = ex - 8;
    if (ex - 1 < -126) qexp = -133;
    double q = ldexp(nearbyint(ldexp(a, -qexp)), qexp);
    const double bf16_max = ldexp(255.0, 120);   /* (2 - 2^-7) * 2^127 */
    if (q > bf16_max) q = INFINITY;
    return v < 0 ? -q : q;
}

static double round_store(double v, int round_mode)
{
    if (round_mode == 1) return (double)(float)v;
    if (round_mode == 2) return round_bf16(v);
    return v;
}

ORACLE_API double oracle_round(double v, int round_mode) { return round_store(v, round_mode); }

ORACLE_API void oracle_round_array(const double* in, double* out, long n, int round_mode)
{
    for (long i = 0; i < n; ++i) out[i] = round_store(in[i], round_mode);
}

/* ------------------------------------------------------------------ */
/* Route: top-k, gate weights, counts, offsets, per-expert permutation */
/* ------------------------------------------------------------------ */

/* Sparse top-k routing (each token activates its k best experts) and the
 * device route map (counts, per-expert offsets, per-expert permutation),
 * tutorial, routing-tax section.
 * Readings: selection compares the fp32 logits themselves; larger logit
 * first, equal logits ordered by lower expert index; gate weights are the
 * softmax over the k selected logits (they sum to one); rows inside an
 * expert group are ordered by token index then slot (a stable counting
 * sort of the (token, slot) pairs by expert).
 * Padded mode (capacity > 0): expert e owns rows [e*C, (e+1)*C); the pair
 * with within-expert rank r goes to e*C + r when r < C, otherwise it is
 * dropped (dst_row = -1).  Rows nobody fills have src_slot = -1.
 * Returns 0, or -1 on a non-finite logit or bad arguments. */
ORACLE_API int oracle_route(const float* logits, int T, int E, int k, int capacity,
                            int32_t* topk_idx, float* topk_w, int32_t* counts,
                            int32_t* offsets, int32_t* dst_row, int32_t* src_slot,
                            long n_rows)
{
    if (T < 0 || E < 1 || k < 1 || k > E) return -1;
    for (long i = 0; i < (long)T * E; ++i)
        if (!isfinite(logits[i])) return -1;

    /* selection: k rounds of "best among not yet chosen" */
    char* taken = (char*)calloc((size_t)E, 1);
    for (int t = 0; t < T; ++t) {
        const float* l = logits + (long)t * E;
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                /* strictly greater wins; equal keeps the lower index found first */
                if (best < 0 || l[e] > l[best]) best = e;
            }
            taken[best] = 1;
            topk_idx[(long)t * k + j] = best;
        }
        /* softmax over the selected logits, shifted by the largest one */
        double l0 = (double)l[topk_idx[(long)t * k]];
        double den = 0.0;
        for (int j = 0; j < k; ++j) den += exp((double)l[topk_idx[(long)t * k + j]] - l0);
        for (int j = 0; j < k; ++j)
            topk_w[(long)t * k + j] = (float)(exp((double)l[topk_idx[(long)t * k + j]] - l0) / den);
    }
    free(taken);

    /* counts and exclusive offsets */
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (long p = 0; p < (long)T * k; ++p) counts[topk_idx[p]] += 1;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];

    /* ranks in token order, destinations, inverse map */
    long rows = capacity > 0 ? (long)E * capacity : (long)T * k;
    if (n_rows != rows) return -1;
    for (long r = 0; r < rows; ++r) src_slot[r] = -1;
    int32_t* seen = (int32_t*)calloc((size_t)E, sizeof(int32_t));
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            long p = (long)t * k + j;
            int e = topk_idx[p];
            int rank = seen[e]++;
            long dst;
            if (capacity > 0) dst = rank < capacity ? (long)e * capacity + rank : -1;
            else dst = (long)offsets[e] + rank;
            dst_row[p] = (int32_t)dst;
            if (dst >= 0) src_slot[dst] = (int32_t)p;
        }
    }
    free(seen);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Permute (rowwise dispatch) and combine                              */
/* ------------------------------------------------------------------ */

/* Rowwise dispatch: token row t is written, unchanged, into the row of its
 * expert's input buffer chosen by the route map (tutorial, "rowwise EP").
 * With row_scale (the backward twin of the weighted combine) the written
 * row is row_scale[t*k+j] * x[t], rounded to storage.  Rows no pair writes
 * (padding) are zero. */
ORACLE_API void oracle_permute(const double* x, int T, int d, int k, const int32_t* dst_row,
                               const float* row_scale, long n_rows, int round_mode,
                               double* x_perm)
{
    memset(x_perm, 0, sizeof(double) * (size_t)n_rows * (size_t)d);
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            long p = (long)t * k + j;
            long dst = dst_row[p];
            if (dst < 0) continue;
            for (int i = 0; i < d; ++i) {
                double v = x[(long)t * d + i];
                if (row_scale) v = round_store((double)row_scale[p] * v, round_mode);
                x_perm[dst * d + i] = v;
            }
        }
}

/* Combine: the reverse transfer plus the weighted merge of each token's k
 * expert outputs (tutorial, "rowwise EP" dispatch/combine).  out[t] =
 * sum over non-dropped slots j, in slot order, of w[t,j] * y_perm[dst].
 * w == NULL gives the unweighted sum (the backward of the permute). */
ORACLE_API void oracle_combine(const double* y_perm, const int32_t* dst_row, const float* w,
                               int T, int k, int d, int round_mode, double* out)
{
    #pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t)
        for (int i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j) {
                long p = (long)t * k + j;
                long dst = dst_row[p];
                if (dst < 0) continue;
                double wt = w ? (double)w[p] : 1.0;
                acc += wt * y_perm[dst * d + i];
            }
            out[(long)t * d + i] = round_store(acc, round_mode);
        }
}

/* ------------------------------------------------------------------ */
/* Router scores and the gradient through the gate weights              */
/* ------------------------------------------------------------------ */

/* Router scores: logits[t,e] = sum_i x[t,i] * w_r[e,i], accumulated in
 * fp64 and stored with round_mode.  The layer stores them in fp32: the
 * tutorial's MXFP8 section (the DeepSeek-V3 paragraph) keeps the gating
 * in high precision.  Reading: a bias-free linear router over the token's
 * d features, weights [E, d] (the pages do not spell the router out). */
ORACLE_API void oracle_router_logits(const double* x, const double* w_r, int T, int E, int d,
                                     int round_mode, double* logits)
{
    #pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t)
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int i = 0; i < d; ++i) acc += x[(long)t * d + i] * w_r[(long)e * d + i];
            logits[(long)t * E + e] = round_store(acc, round_mode);
        }
}

/* Gradient of the layer output through the gate weights, back to the
 * router scores.  The combine gives out[t] = sum_j w[t,j] * y_perm[dst(t,j)]
 * over the non-dropped slots, so dw[t,j] = sum_i dout[t,i] *
 * y_perm[dst(t,j), i], and 0 for a dropped slot (it adds nothing to out).
 * The gate weights are the softmax over the k selected logits (the reading
 * the route takes), w_j = exp(l_j) / sum_m exp(l_m), whose Jacobian gives
 * dlogits[t, topk_idx[t,j]] = w[t,j] * (dw[t,j] - sum_m w[t,m] dw[t,m]);
 * the logits of the experts not selected get 0 (the selection is piecewise
 * constant in them).  fp64 throughout; dw kept in fp64, dlogits [T, E]
 * stored with round_mode. */
ORACLE_API void oracle_gate_grad(const double* dout, const double* y_perm, const int32_t* dst_row,
                                 const int32_t* topk_idx, const float* w, int T, int E, int k,
                                 int d, int round_mode, double* dw, double* dlogits)
{
    #pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            long p = (long)t * k + j;
            long dst = dst_row[p];
            double acc = 0.0;
            if (dst >= 0)
                for (int i = 0; i < d; ++i) acc += dout[(long)t * d + i] * y_perm[dst * d + i];
            dw[p] = acc;
        }
        double wdw = 0.0;
        for (int m = 0; m < k; ++m) wdw += (double)w[(long)t * k + m] * dw[(long)t * k + m];
        for (int e = 0; e < E; ++e) dlogits[(long)t * E + e] = 0.0;
        for (int j = 0; j < k; ++j) {
            long p = (long)t * k + j;
            dlogits[(long)t * E + topk_idx[p]] = round_store((double)w[p] * (dw[p] - wdw), round_mode);
        }
    }
}

/* ------------------------------------------------------------------ */
/* Expert SwiGLU FFN over contiguous groups of rows                     */
/* ------------------------------------------------------------------ */

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* One grouped pass of the expert FFN: expert e owns rows
 * [group_off[e], group_off[e+1]) of x_perm (tutorial: one grouped GEMM
 * over the exact per-expert row counts).  Reading (SwiGLU, pages silent on
 * its form): g = x Wg^T, u = x Wu^T, h = silu(g) * u, y = h Wd^T, no biases.
 * w13 is [E, 2f, d] with rows 0..f-1 = Wg, f..2f-1 = Wu; w2 is [E, d, f].
 * Stored: gu = [g | u] per row (rounded), h (rounded, computed from the
 * unrounded g, u), y (rounded, computed from the stored h).
 * mx_h != 0: the second GEMM reads h through the MXFP8 block quantiser
 * along f (its storage format for that GEMM); the stored h is unchanged. */
static void mx_qdq_vector(const double* v, long len, long stride, double* out, long ostride);

ORACLE_API void oracle_ffn_fwd(const double* x_perm, const double* w13, const double* w2,
                               const int32_t* group_off, int E, int d, int f, int round_mode,
                               int mx_h, double* gu, double* h, double* y)
{
    long n_rows = group_off[E];
    #pragma omp parallel for schedule(dynamic, 1)
    for (long r = 0; r < n_rows; ++r) {
        int e = 0;
        while (!(r >= group_off[e] && r < group_off[e + 1])) ++e;
        const double* xr = x_perm + r * d;
        const double* wg = w13 + (long)e * 2 * f * d;
        const double* wu = wg + (long)f * d;
        for (int n = 0; n < f; ++n) {
            double g = 0.0, u = 0.0;
            for (int i = 0; i < d; ++i) {
                g += xr[i] * wg[(long)n * d + i];
                u += xr[i] * wu[(long)n * d + i];
            }
            gu[r * 2 * f + n] = round_store(g, round_mode);
            gu[r * 2 * f + f + n] = round_store(u, round_mode);
            h[r * f + n] = round_store(g * sigmoid(g) * u, round_mode);
        }
    }
    /* the second GEMM reads h in its GEMM storage format */
    double* hq = NULL;
    const double* h_g = h;
    if (mx_h) {
        hq = (double*)malloc(sizeof(double) * (size_t)n_rows * f);
        for (long r = 0; r < n_rows; ++r) mx_qdq_vector(h + r * f, f, 1, hq + r * f, 1);
        h_g = hq;
    }
    #pragma omp parallel for schedule(dynamic, 1)
    for (long r = 0; r < n_rows; ++r) {
        int e = 0;
        while (!(r >= group_off[e] && r < group_off[e + 1])) ++e;
        const double* wd = w2 + (long)e * d * f;
        for (int i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int n = 0; n < f; ++n) acc += h_g[r * f + n] * wd[(long)i * f + n];
            y[r * d + i] = round_store(acc, round_mode);
        }
    }
    free(hq);
}

/* Backward of the expert FFN (the activation-gradient and weight-gradient
 * GEMMs of the three low-precision GEMMs per linear, tutorial MXFP8
 * section).  With dy = dL/dy for each row:
 *   dh = dy Wd ;  s = sigmoid(g) ; a = g s
 *   da = dh * u ; du = dh * a ; dg = da * s * (1 + g (1 - s))
 *   dx = dg Wg + du Wu
 *   dWd[e] = sum over rows of dy^T h ; dWg[e] = sum dg^T x ; dWu[e] = sum du^T x
 * g, u are read from the stored gu; dgu = [dg | du] is stored (rounded) and
 * the stored value feeds dx and dW13; dx, dW are rounded.  dh stays in the
 * accumulator (not stored).  Weight gradients overwrite (no accumulation
 * into an existing buffer).  Experts with no rows get zero gradients.
 * The optional *_q operands are the values the GEMMs read instead of the
 * stored tensor (MXFP8: each GEMM reads its own quantised copy); NULL
 * means "same as the stored tensor". */
ORACLE_API void oracle_ffn_bwd(const double* dy_perm, const double* x_perm, const double* gu,
                               const double* h, const double* w13, const double* w2,
                               const int32_t* group_off, int E, int d, int f, int round_mode,
                               const double* w2_dgrad, const double* w13_dgrad,
                               const double* dy_wgrad, const double* h_wgrad,
                               const double* x_wgrad, int mx_dgu,
                               double* dgu, double* dx_perm, double* dw13, double* dw2)
{
    long n_rows = group_off[E];
    if (!w2_dgrad) w2_dgrad = w2;
    if (!w13_dgrad) w13_dgrad = w13;
    if (!dy_wgrad) dy_wgrad = dy_perm;
    if (!h_wgrad) h_wgrad = h;
    if (!x_wgrad) x_wgrad = x_perm;

    /* dh, then the SwiGLU backward into dgu */
    #pragma omp parallel for schedule(dynamic, 1)
    for (long r = 0; r < n_rows; ++r) {
        int e = 0;
        while (!(r >= group_off[e] && r < group_off[e + 1])) ++e;
        const double* wd = w2_dgrad + (long)e * d * f;
        for (int n = 0; n < f; ++n) {
            double dh = 0.0;
            for (int i = 0; i < d; ++i) dh += dy_perm[r * d + i] * wd[(long)i * f + n];
            double g = gu[r * 2 * f + n], u = gu[r * 2 * f + f + n];
            double s = sigmoid(g);
            double a = g * s;
            double da = dh * u;
            double du = dh * a;
            double dg = da * s * (1.0 + g * (1.0 - s));
            dgu[r * 2 * f + n] = round_store(dg, round_mode);
            dgu[r * 2 * f + f + n] = round_store(du, round_mode);
        }
    }
    /* the GEMMs below read dgu in its GEMM storage format */
    double* dgu_q = NULL;
    const double* dgu_g = dgu;      /* dgrad operand (blocks along 2f) */
    if (mx_dgu) {
        dgu_q = (double*)malloc(sizeof(double) * (size_t)n_rows * 2 * f);
        for (long r = 0; r < n_rows; ++r)
            mx_qdq_vector(dgu + r * 2 * f, 2 * f, 1, dgu_q + r * 2 * f, 1);
        dgu_g = dgu_q;
    }
    /* dx = [dg | du] [Wg ; Wu] */
    #pragma omp parallel for schedule(dynamic, 1)
    for (long r = 0; r < n_rows; ++r) {
        int e = 0;
        while (!(r >= group_off[e] && r < group_off[e + 1])) ++e;
        const double* w = w13_dgrad + (long)e * 2 * f * d;
        for (int i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int n = 0; n < 2 * f; ++n) acc += dgu_g[r * 2 * f + n] * w[(long)n * d + i];
            dx_perm[r * d + i] = round_store(acc, round_mode);
        }
    }
    /* weight gradients: reduction over the rows of each group */
    double* dgu_w = NULL;
    const double* dgu_wg = dgu;     /* wgrad operand (blocks along rows in each group) */
    if (mx_dgu) {
        dgu_w = (double*)malloc(sizeof(double) * (size_t)n_rows * 2 * f);
        for (int e = 0; e < E; ++e) {
            long r0 = group_off[e], m = group_off[e + 1] - group_off[e];
            for (int n = 0; n < 2 * f; ++n)
                mx_qdq_vector(dgu + r0 * 2 * f + n, m, 2 * f, dgu_w + r0 * 2 * f + n, 2 * f);
        }
        dgu_wg = dgu_w;
    }
    for (int e = 0; e < E; ++e) {
        long r0 = group_off[e], r1 = group_off[e + 1];
        #pragma omp parallel for schedule(static)
        for (int i = 0; i < d; ++i)
            for (int n = 0; n < f; ++n) {
                double acc = 0.0;
                for (long r = r0; r < r1; ++r) acc += dy_wgrad[r * d + i] * h_wgrad[r * f + n];
                dw2[((long)e * d + i) * f + n] = round_store(acc, round_mode);
            }
        #pragma omp parallel for schedule(static)
        for (int n = 0; n < 2 * f; ++n)
            for (int i = 0; i < d; ++i) {
                double acc = 0.0;
                for (long r = r0; r < r1; ++r) acc += dgu_wg[r * 2 * f + n] * x_wgrad[r * d + i];
                dw13[((long)e * 2 * f + n) * d + i] = round_store(acc, round_mode);
            }
    }
    free(dgu_q);
    free(dgu_w);
}

/* ------------------------------------------------------------------ */
/* MXFP8: E4M3FN elements, one E8M0 scale per 32 elements              */
/* ------------------------------------------------------------------ */

/* E4M3FN (OCP, the "FN" variant: bias 7, no infinities, 0x7F/0xFF NaN,
 * largest finite 448 -- the tutorial's MXFP8 paragraph names 448 as the
 * E4M3 maximum). */
ORACLE_API double oracle_e4m3_decode(uint8_t code)
{
    int s = code >> 7, ex = (code >> 3) & 0xF, m = code & 7;
    double v;
    if (ex == 0xF && m == 7) return NAN;
    if (ex == 0) v = ldexp((double)m, -9);                 /* m/8 * 2^-6 */
    else v = ldexp(8.0 + m, ex - 7 - 3);                   /* (1 + m/8) * 2^(ex-7) */
    return s ? -v : v;
}

/* Round-to-nearest-even into E4M3FN, saturating to +-448 (never reached
 * by values already divided by the block scale chosen below). */
ORACLE_API uint8_t oracle_e4m3_encode(double v)
{
    if (isnan(v)) return 0x7F;
    uint8_t sign = (v < 0 || (v == 0 && signbit(v))) ? 0x80 : 0x00;
    double a = fabs(v);
    double q;
    if (a < ldexp(1.0, -6)) {
        q = nearbyint(ldexp(a, 9));            /* subnormal grid 2^-9; 8 -> 2^-6 */
        return (uint8_t)(sign | (uint8_t)q);   /* q in 0..8, code = q  */
    }
    int ex;
    frexp(a, &ex);                              /* a in [2^(ex-1), 2^ex) */
    q = ldexp(nearbyint(ldexp(a, -(ex - 1 - 3))), ex - 1 - 3);
    if (q > 448.0) q = 448.0;
    int eq;
    double mq = frexp(q, &eq);                  /* q = mq 2^eq, mq in [0.5,1) */
    int efield = (eq - 1) + 7;
    int mfield = (int)nearbyint((mq * 2.0 - 1.0) * 8.0);
    return (uint8_t)(sign | (efield << 3) | mfield);
}

ORACLE_API double oracle_e8m0_decode(uint8_t code)
{
    if (code == 0xFF) return NAN;
    return ldexp(1.0, (int)code - 127);
}

/* Block scale exponent for one 32-element block (tutorial MXFP8 paragraph:
 * divide the block maximum by 448, then take a power of two, so that the
 * block maximum does not overflow).  Reading of the garbled "three steps":
 * e = ceil(log2(amax / 448)), clamped to the E8M0 range [-127, 127];
 * amax == 0 gives e = -127. */
ORACLE_API int oracle_mx_scale_exp(double amax)
{
    if (!(amax > 0.0)) return -127;
    /* smallest e with amax <= 448 * 2^e; ldexp(448, e) is exact */
    int ex;
    frexp(amax / 448.0, &ex);
    int e = ex;
    while (e > -140 && ldexp(448.0, e - 1) >= amax) --e;
    while (ldexp(448.0, e) < amax) ++e;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* Quantise one vector of `len` elements (element i at v[i*stride]) in
 * consecutive 32-element blocks from its start; a short last block uses
 * only the elements present.  Writes codes (same indexing as v, ostride)
 * and one scale byte (E8M0, exponent + 127) per block. */
ORACLE_API void oracle_mx_quantize_vector(const double* v, long len, long stride,
                                          uint8_t* codes, long cstride, uint8_t* scales)
{
    for (long b0 = 0, blk = 0; b0 < len; b0 += 32, ++blk) {
        long b1 = b0 + 32 < len ? b0 + 32 : len;
        double amax = 0.0;
        for (long i = b0; i < b1; ++i) {
            double a = fabs(v[i * stride]);
            if (a > amax) amax = a;
        }
        int e = oracle_mx_scale_exp(amax);
        scales[blk] = (uint8_t)(e + 127);
        for (long i = b0; i < b1; ++i)
            codes[i * cstride] = oracle_e4m3_encode(ldexp(v[i * stride], -e));
    }
}

/* quantise-then-dequantise one vector (the value an MXFP8 GEMM operand
 * represents) */
static void mx_qdq_vector(const double* v, long len, long stride, double* out, long ostride)
{
    uint8_t c[32];
    for (long b0 = 0; b0 < len; b0 += 32) {
        long b1 = b0 + 32 < len ? b0 + 32 : len;
        double amax = 0.0;
        for (long i = b0; i < b1; ++i) {
            double a = fabs(v[i * stride]);
            if (a > amax) amax = a;
        }
        int e = oracle_mx_scale_exp(amax);
        for (long i = b0; i < b1; ++i) c[i - b0] = oracle_e4m3_encode(ldexp(v[i * stride], -e));
        for (long i = b0; i < b1; ++i) out[i * ostride] = ldexp(oracle_e4m3_decode(c[i - b0]), e);
    }
}

ORACLE_API void oracle_mx_qdq_vector(const double* v, long len, long stride, double* out,
                                     long ostride)
{
    mx_qdq_vector(v, len, stride, out, ostride);
}
