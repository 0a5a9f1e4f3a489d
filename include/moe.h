/*
 * moe.h -- C ABI of one GPU's MoE feed-forward layer on AMD Instinct MI355X
 * (gfx950): router top-k and route map, rowwise dispatch (permute), grouped
 * SwiGLU GEMM forward and backward, weighted un-permute/combine, and the
 * MXFP8 block quantiser.
 *
 * The operations follow the pages describing the OLMo-core 3 MoE training
 * stack ("OLMo-core 3: MoE 训练栈..." tutorial; "Ai2 Olmo-core 3: The Secret
 * Behind 2.7x MoE Training Throughput"):
 *   - route map kept on the device (tutorial, routing-tax section, paragraph
 *     on GPU-resident routing metadata): per-expert counts, row counts and a
 *     per-expert permutation are produced on the GPU, so nothing is copied
 *     back to the host;
 *   - rowwise dispatch (tutorial, "rowwise EP" paragraph): each token row is
 *     written straight into its expert's input buffer, no pack step;
 *   - device grouped GEMM (tutorial, same section, second tax): one launch
 *     over all experts using the exact per-expert row counts, no padding to a
 *     common capacity (a padded-to-capacity variant is provided for
 *     comparison);
 *   - MXFP8 (tutorial, MXFP8 section): E4M3 elements with one power-of-two
 *     E8M0 scale per 32 elements, used for the three GEMMs per linear.
 *
 * Conventions for every call:
 *   - Tensor arguments are device pointers owned by the caller.  The library
 *     never allocates, frees, copies to the host or synchronises: each call
 *     validates its arguments on the host, enqueues kernels on `stream` and
 *     returns.  Results are ready when the stream reaches them.
 *   - Tensors are dense row-major.  bf16 is stored as its 16-bit pattern.
 *   - Return value: MOE_OK, or a negative status found on the host from the
 *     arguments alone (nothing is enqueued then), or MOE_EHIP if a launch
 *     failed.  moe_status_string() names each status.
 *   - Data faults only visible on the device (a non-finite logit, a row
 *     index outside the destination) are OR-ed into *dev_err (a caller-owned
 *     device int32, may be NULL) with the MOE_ERR_* bits; the kernels then
 *     skip the offending element and finish normally.
 *   - Calls are re-entrant and keep no state between calls: everything a
 *     call's kernels write goes to the caller's tensors and workspace, so
 *     calls on different streams with different workspaces are independent.
 *     Results are bitwise reproducible for identical inputs (no
 *     floating-point atomics anywhere).
 *   - Limits: 1 <= E <= 1024, 1 <= k <= min(E, 8), row widths d and f
 *     multiples of 8 (MXFP8: 32 for the permute / quantiser, 128 for the
 *     grouped GEMMs), all pointers 16-byte aligned, n_rows < 2^31.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

/* A hipStream_t.  NULL selects the default (null) stream. */
typedef void* moe_stream_t;

enum moe_status {
    MOE_OK = 0,
    MOE_EINVAL = -1,        /* null pointer, negative or inconsistent size, k > E, ... */
    MOE_EALIGN = -2,        /* row width not a multiple of 8 (32 for MXFP8) or pointer not 16-B aligned */
    MOE_EUNSUPPORTED = -3,  /* dtype / option combination not provided */
    MOE_EWORKSPACE = -4,    /* workspace missing or smaller than the *_workspace_bytes() figure */
    MOE_EHIP = -5           /* a kernel launch failed (hipGetLastError) */
};

enum moe_dtype {
    MOE_F32 = 0,            /* fp32 activations and weights, fp32 accumulate */
    MOE_BF16 = 1,           /* bf16 storage, fp32 accumulate */
    MOE_MXFP8 = 2           /* E4M3FN codes + one E8M0 scale per 32 elements, fp32 accumulate */
};

enum moe_dev_err_bits {
    MOE_ERR_NONFINITE_LOGIT = 1,  /* a logit was NaN or +-Inf (selected as if -Inf) */
    MOE_ERR_ROW_RANGE = 2         /* a dst_row entry was >= n_rows (that row was skipped) */
};

/* Bytes of scratch moe_route_topk needs for T tokens, E experts, top-k. */
MOE_API size_t moe_route_workspace_bytes(int T, int E, int k);

/*
 * Router top-k and the device route map (tutorial, routing-tax section:
 * counts, per-expert row counts and the per-expert permutation, all made on
 * the device; each token activates only its top-k experts).
 *
 * in   logits     [T, E] fp32.
 * in   capacity   0 = unpadded (the method).  C > 0 = padded-to-capacity
 *                 variant: expert e owns rows [e*C, (e+1)*C); the first C
 *                 pairs routed to e in token order are kept, later ones are
 *                 dropped (dst_row = -1).
 * out  topk_idx   [T, k] int32: the k largest logits of each token, larger
 *                 first, equal logits ordered by lower expert index.
 * out  topk_w     [T, k] fp32: softmax over the k selected logits (sums to 1).
 * out  counts     [E] int32: pairs routed to each expert (before any drop).
 * out  offsets    [E+1] int32: exclusive prefix sum of counts; offsets[E] = T*k.
 * out  dst_row    [T*k] int32: destination row of pair (t, j) at t*k+j:
 *                 offsets[e] + (number of earlier tokens routed to e), or the
 *                 padded row / -1 as above.  Rows of one expert are in token order.
 * out  src_slot   [n_rows] int32: inverse map, row -> t*k+j, -1 for empty rows.
 * in   n_rows     T*k (unpadded) or E*C (padded).
 * in   ws         device scratch of at least moe_route_workspace_bytes(T,E,k).
 * out  dev_err    optional; MOE_ERR_NONFINITE_LOGIT.
 * T = 0 is allowed (counts and offsets become 0).  Three kernels; no host sync.
 */
MOE_API int moe_route_topk(const float* logits, int T, int E, int k, int capacity,
                   int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                   int32_t* dst_row, int32_t* src_slot, int64_t n_rows,
                   void* ws, size_t ws_bytes, int32_t* dev_err, moe_stream_t stream);

/*
 * moe_route_topk for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same call and results, with the scratch taken from a fixed array the
 * library holds on each GPU it runs on (MOE_ROUTE_NOALLOC_MAX_BYTES, 32 MiB,
 * kept until the process ends) instead of a caller workspace.  It calls no
 * allocator.  The current device must be the stream's device.  Returns
 * MOE_EWORKSPACE when moe_route_workspace_bytes(T, E, k) exceeds the array
 * (at E = 128: T up to 4 194 240 tokens), MOE_EHIP if the array's
 * device address cannot be looked up, otherwise as moe_route_topk.
 * Every call on one GPU uses that GPU's one array: calls that overlap on a
 * GPU (different streams or threads at once) race on it.  Nothing in the
 * array needs clearing between calls (the route writes all of it it reads).
 */
#define MOE_ROUTE_NOALLOC_MAX_BYTES ((size_t)32 << 20)
MOE_API int moe_route_topk_noalloc(const float* logits, int T, int E, int k, int capacity,
                                   int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                                   int32_t* dst_row, int32_t* src_slot, int64_t n_rows,
                                   int32_t* dev_err, moe_stream_t stream);

/*
 * Rowwise dispatch (tutorial, "rowwise EP" paragraph): token row t is written
 * into row dst_row[t*k+j] of x_perm for every slot j with dst_row >= 0.
 *
 * in   dtype      MOE_F32: x, x_perm fp32.  MOE_BF16: x, x_perm bf16 (an exact
 *                 copy).  MOE_MXFP8: x bf16; x_perm receives E4M3FN codes
 *                 [n_rows, d] and x_perm_scales E8M0 [n_rows, d/32] (dispatch
 *                 payload in MXFP8, tutorial MXFP8 section).
 * in   x          [T, d].
 * in   dst_row    [T*k] from moe_route_topk.
 * in   src_slot   [n_rows]; required when n_rows != T*k (padded): rows with
 *                 src_slot < 0 are zero-filled.  May be NULL otherwise.
 * in   row_scale  NULL, or [T*k] fp32: row (t, j) is written as
 *                 round(row_scale[t*k+j] * x[t]) (the backward of the weighted
 *                 combine).  Not combined with MOE_MXFP8.
 * out  x_perm     [n_rows, d].
 * out  dev_err    optional; MOE_ERR_ROW_RANGE.
 */
MOE_API int moe_permute(int dtype, const void* x, int T, int d, int k, const int32_t* dst_row,
                const int32_t* src_slot, const float* row_scale, int64_t n_rows,
                void* x_perm, uint8_t* x_perm_scales, int32_t* dev_err, moe_stream_t stream);

/* Bytes of scratch the grouped GEMM calls need: MOE_F32 none; MOE_BF16 the
 * weight-gradient stage's control words (256 bytes: a small kernel ahead of
 * that stage decides there how its tiles go to the XCDs); MOE_MXFP8 those
 * plus the quantised operands of every stage.  A workspace is 16-byte
 * aligned and used by one call at a time: calls that share one must run in
 * order on one stream. */
MOE_API size_t moe_gemm_workspace_bytes(int dtype, int E, int64_t n_rows, int d, int f);

/*
 * Grouped SwiGLU GEMM forward over uneven expert groups (tutorial: one device
 * grouped GEMM over the exact per-expert row counts).  For each expert e and
 * each row r of its group:  g = x Wg^T, u = x Wu^T (fp32 accumulate),
 * h = silu(g) * u, y = h Wd^T.  Two launches (gate/up with the SwiGLU
 * epilogue, then down); the tile schedule is built on the device from the
 * group offsets, the grid comes from host-known bounds.
 *
 * in   x_perm     [n_rows, d]   (MXFP8: codes, with x_perm_scales [n_rows, d/32])
 * in   w13        [E, 2f, d]: rows 0..f-1 = Wg, f..2f-1 = Wu of each expert
 *                 (MXFP8: codes with w13_scales [E, 2f, d/32]).
 * in   w2         [E, d, f] = Wd (MXFP8: codes with w2_scales [E, d, f/32]).
 * in   group_off  [E+1] device int32: expert e owns rows
 *                 [group_off[e], group_off[e+1]) (the route offsets).  Ignored
 *                 when capacity > 0: then expert e owns [e*C, (e+1)*C).
 * out  gu         [n_rows, 2f]: [g | u] per row (saved for the backward).
 * out  h          [n_rows, f]: silu(g) * u (saved for the backward).
 * out  y_perm     [n_rows, d].
 * gu, h, y_perm are fp32 for MOE_F32 and bf16 otherwise.  Rows outside every
 * group are not written.
 */
MOE_API int moe_grouped_gemm_fwd(int dtype, const void* x_perm, const uint8_t* x_perm_scales,
                         const void* w13, const uint8_t* w13_scales,
                         const void* w2, const uint8_t* w2_scales,
                         const int32_t* group_off, int capacity, int E, int64_t n_rows,
                         int d, int f, void* gu, void* h, void* y_perm,
                         void* ws, size_t ws_bytes, moe_stream_t stream);

/*
 * Grouped SwiGLU GEMM backward: the activation-gradient and weight-gradient
 * GEMMs (tutorial MXFP8 section: forward, dgrad and wgrad GEMMs per linear).
 *   dh = dy Wd ; s = sigmoid(g) ; dg = dh*u*s*(1 + g(1-s)) ; du = dh*g*s
 *   dx = dg Wg + du Wu
 *   dWd[e] = sum_r dy_r^T h_r ; dWg[e] = sum_r dg_r^T x_r ; dWu[e] = sum_r du_r^T x_r
 * Weight gradients overwrite dw13/dw2 (experts with no rows get zeros).
 *
 * in   dy_perm    [n_rows, d] (bf16 for MXFP8 too: quantised inside).
 * in   x_perm, gu, h  saved by the forward (x_perm as passed to it).
 * in   w13, w2    as in the forward for MOE_F32/MOE_BF16.  MOE_MXFP8 takes the
 *                 backward-direction caches: w13 codes [E, d, 2f] + scales
 *                 [E, d, 2f/32] (Wg|Wu transposed, blocks along 2f) and w2 codes
 *                 [E, f, d] + scales [E, f, d/32] (Wd transposed, blocks along d),
 *                 as made by moe_quantize_mxfp8(colwise=1) of the weights.
 * out  dgu        [n_rows, 2f]: [dg | du].
 * out  dx_perm    [n_rows, d].
 * out  dw13       [E, 2f, d], dw2 [E, d, f].
 * in   ws         workspace of moe_gemm_workspace_bytes() bytes (MOE_BF16 and
 *                 MOE_MXFP8; MOE_EWORKSPACE when missing or smaller).
 */
MOE_API int moe_grouped_gemm_bwd(int dtype, const void* dy_perm, const void* x_perm,
                         const uint8_t* x_perm_scales, const void* gu, const void* h,
                         const void* w13, const uint8_t* w13_scales,
                         const void* w2, const uint8_t* w2_scales,
                         const int32_t* group_off, int capacity, int E, int64_t n_rows,
                         int d, int f, void* dgu, void* dx_perm, void* dw13, void* dw2,
                         void* ws, size_t ws_bytes, moe_stream_t stream);

/* The grouped GEMM stages: one kernel launch each for MOE_F32 / MOE_BF16;
 * for MOE_MXFP8 the quantisation of the stage's bf16 operands into the
 * workspace, then one block-scaled GEMM launch. */
enum moe_gemm_op {
    MOE_GEMM_GATE_UP = 0,        /* gu = x [Wg | Wu]^T, h = silu(g) * u               */
    MOE_GEMM_DOWN = 1,           /* y = h Wd^T                                        */
    MOE_GEMM_DGRAD_DOWN = 2,     /* dh = dy Wd; dgu = [dg | du] from dh and saved gu  */
    MOE_GEMM_DGRAD_GATE_UP = 3,  /* dx = dg Wg + du Wu                                */
    MOE_GEMM_WGRAD = 4           /* dWd = sum dy^T h and dWg|dWu = sum dgu^T x        */
};

/* Operands of the grouped GEMM stages (device pointers; unused ones may be
 * NULL).  Shapes and layouts as in moe_grouped_gemm_fwd / _bwd.  MOE_MXFP8:
 * x_perm is codes + x_perm_scales (row-wise, as moe_permute writes them);
 * w13 / w2 (+ scales) hold the forward-direction caches for GATE_UP / DOWN
 * and the backward-direction caches for DGRAD_GATE_UP / DGRAD_DOWN; every
 * other activation is bf16; ws / ws_bytes is a workspace of at least
 * moe_gemm_workspace_bytes, needed by every MXFP8 stage and by the MOE_BF16
 * WGRAD stage.  MXFP8 stages hand operands on through it: GATE_UP leaves the
 * row-wise MXFP8 copy of h that DOWN reads, DGRAD_DOWN the copy of dgu that
 * DGRAD_GATE_UP reads, so those pairs run in order on one stream with one
 * workspace and the h / dgu they see are the ones those epilogues wrote. */
typedef struct moe_gemm_tensors {
    const void* x_perm;          /* [n_rows, d]                     */
    const uint8_t* x_perm_scales;
    const void* w13;             /* [E, 2f, d]                      */
    const uint8_t* w13_scales;
    const void* w2;              /* [E, d, f]                       */
    const uint8_t* w2_scales;
    void* gu;                    /* [n_rows, 2f]                    */
    void* h;                     /* [n_rows, f]                     */
    void* y_perm;                /* [n_rows, d]                     */
    const void* dy_perm;         /* [n_rows, d]                     */
    void* dgu;                   /* [n_rows, 2f]                    */
    void* dx_perm;               /* [n_rows, d]                     */
    void* dw13;                  /* [E, 2f, d]                      */
    void* dw2;                   /* [E, d, f]                       */
    void* ws;                    /* workspace (MXFP8 stages, bf16 WGRAD) */
    size_t ws_bytes;
    /* MOE_BF16 WGRAD only, optional (both or neither): fp32 weight-gradient
     * accumulators [E, 2f, d] and [E, d, f].  When set, WGRAD adds its sums
     * into them (dw13_f32 += dgu^T x, dw2_f32 += dy^T h, one fp32 addition per
     * element, no atomics) and does not write dw13 / dw2, which may be NULL. */
    float* dw13_f32;
    float* dw2_f32;
} moe_gemm_tensors;

/*
 * One stage of the grouped SwiGLU GEMM (the forward and backward calls above
 * are GATE_UP + DOWN and DGRAD_DOWN + DGRAD_GATE_UP + WGRAD, issued through
 * this same code).  Inputs a stage reads must have been produced by the
 * earlier stages on the same stream.  Errors as for the fwd / bwd calls;
 * MOE_EWORKSPACE when an MXFP8 stage that needs the workspace lacks it.
 */
MOE_API int moe_grouped_gemm_op(int op, int dtype, const moe_gemm_tensors* t,
                                const int32_t* group_off, int capacity, int E, int64_t n_rows,
                                int d, int f, moe_stream_t stream);

/*
 * Un-permute and combine (tutorial, "rowwise EP": the reverse transfer and
 * the merge of each token's k expert outputs):
 *   out[t] = sum over j with dst_row[t*k+j] >= 0, in slot order, of
 *            weights[t*k+j] * y_perm[dst_row[t*k+j]]
 * accumulated in fp32.  weights == NULL gives the unweighted sum (the
 * backward of moe_permute).
 * in   dtype      MOE_F32 (y_perm, out fp32) or MOE_BF16 (bf16).
 * out  out        [T, d].   out  dev_err  optional; MOE_ERR_ROW_RANGE.
 */
MOE_API int moe_unpermute_combine(int dtype, const void* y_perm, const int32_t* dst_row,
                          const float* weights, int T, int k, int d, int64_t n_rows,
                          void* out, int32_t* dev_err, moe_stream_t stream);

/*
 * MXFP8 block quantiser (tutorial MXFP8 section): E4M3FN codes with one E8M0
 * scale per 32 elements, scale = 2^e with e the smallest integer such that
 * block_max / 2^e <= 448 (clamped to [-127, 127]; an all-zero block gets
 * e = -127), codes = round-to-nearest-even(v / 2^e).
 *
 * in   src        [rows, K] bf16.
 * colwise = 0     blocks of 32 along K.  codes [rows, K], scales [rows, K/32].
 *                 K must be a multiple of 32.
 * colwise = 1     blocks of 32 along the rows inside each group
 *                 [group_off[g], group_off[g+1]) (device int32, n_groups+1
 *                 entries; NULL = one group of all rows).  Output is each
 *                 group transposed, its rows padded with zero codes to a
 *                 multiple of MOE_MX_COL_PAD (128): group g occupies
 *                 codes[K * P_g .. K * P_{g+1}) as [K][P_{g+1} - P_g] and
 *                 scales[K * P_g / 32 ..) as [K][(P_{g+1} - P_g) / 32], where
 *                 P_g = sum over earlier groups of their row count rounded up
 *                 to 128.  The buffers must hold K * (rows + 128 * n_groups)
 *                 codes and 1/32 of that in scales.  K must be a multiple
 *                 of 8 (16-byte source rows) and scales 4-byte aligned.
 * Errors: MOE_EINVAL (sizes, null pointers, n_groups outside 1..1024),
 * MOE_EALIGN (K, src / codes not 16-byte aligned, colwise scales not
 * 4-byte aligned).
 */
#define MOE_MX_COL_PAD 128
MOE_API int moe_quantize_mxfp8(const void* src, int64_t rows, int K, int colwise,
                       const int32_t* group_off, int n_groups, uint8_t* codes,
                       uint8_t* scales, moe_stream_t stream);

/*
 * Shared experts (the speed-read's training-recipe paragraph, the report's
 * section on the model recipe: ungated experts every token also uses, whose
 * merge with the routed output matters; several of them equal one wider
 * expert) as extra groups of the same grouped GEMM: from a
 * route of k slots, the route of k + n_shared slots in which slot k + s of
 * token t is expert E + s with weight 1 and row R + s*T + t, after the R
 * routed rows (R = T*k, or E*C padded).  Then permute, the grouped GEMM
 * (E + n_shared groups; weights of the shared experts after the routed
 * ones; group offsets = offsets_out, capacity 0) and combine run unchanged
 * on the wider route.
 * in   the route of moe_route_topk: topk_idx, topk_w, dst_row [T, k],
 *      counts [E], offsets [E+1], src_slot [n_rows]; capacity as given there.
 * out  topk_idx_out, topk_w_out, dst_row_out [T, k + n_shared];
 *      counts_out [E + n_shared]; offsets_out [E + n_shared + 1] (group
 *      starts: the routed offsets, or e*C when padded, then R + s*T);
 *      src_slot_out [n_rows + n_shared*T], routed rows renumbered to
 *      t*(k + n_shared) + j, padding rows -1.
 * Errors: MOE_EINVAL (sizes: n_shared >= 1, k + n_shared <= 8,
 * E + n_shared <= 1024, n_rows as the route; null pointers).
 */
MOE_API int moe_route_add_shared(int T, int E, int k, int n_shared, int capacity,
                                 const int32_t* topk_idx, const float* topk_w, const int32_t* dst_row,
                                 const int32_t* counts, const int32_t* offsets, const int32_t* src_slot,
                                 int64_t n_rows, int32_t* topk_idx_out, float* topk_w_out,
                                 int32_t* counts_out, int32_t* offsets_out, int32_t* dst_row_out,
                                 int32_t* src_slot_out, moe_stream_t stream);

/*
 * Router scores, the step before moe_route_topk:
 *   logits[t, e] = sum_i x[t, i] * w_router[e, i]
 * bf16 operands, fp32 accumulation and fp32 result (the tutorial's MXFP8
 * section keeps the gating in high precision; the pages do not spell the
 * router out, and this is the plainest reading: a bias-free linear map).
 * in   x          [T, d] bf16, 16-byte aligned, d % 8 == 0.
 * in   w_router   [E, d] bf16, 16-byte aligned; 1 <= E <= 1024.
 * out  logits     [T, E] fp32, 16-byte aligned.
 * Errors: MOE_EINVAL (sizes, null pointers), MOE_EALIGN (d % 8, alignment).
 */
MOE_API int moe_router_logits(const void* x, const void* w_router, int T, int E, int d,
                              float* logits, moe_stream_t stream);

/*
 * Gradient through the gate weights, back to the router scores (the
 * backward of the weighted combine with respect to its weights, then of the
 * softmax over the k selected logits that moe_route_topk forms):
 *   dw[t, j]                  = <dout[t], y_perm[dst_row[t*k+j]]>  (0 for a dropped slot)
 *   dlogits[t, topk_idx[t,j]] = topk_w[t,j] * (dw[t,j] - sum_m topk_w[t,m] * dw[t,m])
 *   dlogits[t, e]             = 0 for the experts not selected
 * with the dot products accumulated in fp32.
 * in   dout       [T, d] bf16 (upstream gradient of the layer output).
 * in   y_perm     [n_rows, d] bf16 (the expert outputs of the forward).
 * in   topk_idx, topk_w, dst_row  [T, k], as moe_route_topk wrote them.
 * out  dlogits    [T, E] fp32, every entry written.
 * out  dw         [T, k] fp32, optional (NULL: not written).
 * out  dy_perm    [n_rows, d] bf16, optional: also writes the combine
 *                 backward dy_perm[dst] = topk_w * dout[t] (what moe_permute
 *                 with row_scale = topk_w writes) from the same dout reads.
 *                 Unpadded layouts only (n_rows == T*k): MOE_EUNSUPPORTED
 *                 otherwise, as padding rows would stay unwritten.
 * out  dev_err    optional; MOE_ERR_ROW_RANGE for a destination >= n_rows
 *                 (that slot is then treated as dropped).
 * Errors: MOE_EINVAL (sizes: 1 <= k <= 8, k <= E <= 1024; null pointers),
 * MOE_EALIGN (d % 8, 16-byte alignment of dout, y_perm, dy_perm, dlogits),
 * MOE_EUNSUPPORTED (dy_perm with a padded layout).
 */
MOE_API int moe_gate_grad(const void* dout, const void* y_perm, const int32_t* topk_idx,
                          const float* topk_w, const int32_t* dst_row, int T, int E, int k, int d,
                          int64_t n_rows, float* dlogits, float* dw, void* dy_perm,
                          int32_t* dev_err, moe_stream_t stream);

/* Static text naming a status code. */
MOE_API const char* moe_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
MOE_API int moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
