// C ABI entry points of libmoe: host-side argument validation, workspace
// carving and kernel launches.  No entry point allocates, frees, copies to
// the host or synchronises; everything is enqueued on the caller's stream.
#include <mutex>

#include "moe_internal.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int status_of(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

constexpr int64_t kMaxRows = (int64_t)1 << 31;

// common validation of a grouped GEMM shape; returns MOE_OK or an error
int check_gemm_shape(int dtype, const int32_t* group_off, int capacity, int E, int64_t n_rows,
                     int d, int f)
{
    if (dtype != MOE_F32 && dtype != MOE_BF16 && dtype != MOE_MXFP8) return MOE_EUNSUPPORTED;
    if (E < 1 || E > kMaxExperts || n_rows < 0 || n_rows >= kMaxRows || d < 1 || f < 1 ||
        capacity < 0)
        return MOE_EINVAL;
    if (capacity > 0 && (int64_t)E * capacity != n_rows) return MOE_EINVAL;
    if (capacity == 0 && !group_off) return MOE_EINVAL;
    // MXFP8 GEMMs step K by 128 fp8 (whole 4-byte scale words per row)
    const int unit = dtype == MOE_MXFP8 ? 128 : (dtype == MOE_F32 ? 4 : 8);
    if (d % unit || f % unit) return MOE_EALIGN;
    if (n_rows * (int64_t)(d > 2 * f ? d : 2 * f) >= ((int64_t)1 << 40)) return MOE_EINVAL;
    return MOE_OK;
}

// one grouped GEMM stage in the given arithmetic
int run_gemm_op(int op, int dtype, const moe_gemm_tensors& t, const GroupSpec& g, int d, int f,
                hipStream_t s)
{
    hipError_t e;
    if (dtype == MOE_F32) e = gemm_op_f32(op, t, g, d, f, s);
    else if (dtype == MOE_BF16) e = gemm_op_bf16(op, t, g, d, f, s);
    else e = gemm_op_mxfp8(op, t, g, d, f, t.ws, s);
    return status_of(e);
}

// Scratch of moe_route_topk_noalloc: the route's per-pair ranks and per-block
// histograms, for callers that cannot allocate.  A __device__ array exists
// once per GPU, at that GPU's own address, from module load until the
// process ends.  Host code never uses the array's name as an address (on the
// host it is only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
constexpr size_t kNoAllocScratchBytes = MOE_ROUTE_NOALLOC_MAX_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// device address of the current device's scratch array
hipError_t scratch_of_current_device(void** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
    });
    if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
    *out = g_scratch_ptr[dev];
    return *out ? hipSuccess : hipErrorInvalidSymbol;
}

}  // namespace

extern "C" {

int moe_version(void) { return 100; }

const char* moe_status_string(int status)
{
    switch (status) {
    case MOE_OK: return "MOE_OK: success";
    case MOE_EINVAL: return "MOE_EINVAL: null pointer or invalid / inconsistent size";
    case MOE_EALIGN: return "MOE_EALIGN: row width or pointer alignment not supported";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED: dtype or option combination not provided";
    case MOE_EWORKSPACE: return "MOE_EWORKSPACE: workspace missing or too small";
    case MOE_EHIP: return "MOE_EHIP: kernel launch failed";
    default: return "unknown moe status";
    }
}

size_t moe_route_workspace_bytes(int T, int E, int k)
{
    if (T < 0 || E < 1 || k < 1) return 0;
    const size_t nblk = ((size_t)T + kRouteTokensPerBlock - 1) / kRouteTokensPerBlock;
    (void)k;
    return align_up(nblk * E * sizeof(int32_t)) + kAlign;
}

int moe_route_topk(const float* logits, int T, int E, int k, int capacity, int32_t* topk_idx,
                   float* topk_w, int32_t* counts, int32_t* offsets, int32_t* dst_row,
                   int32_t* src_slot, int64_t n_rows, void* ws, size_t ws_bytes,
                   int32_t* dev_err, moe_stream_t stream)
{
    if (T < 0 || E < 1 || E > kMaxExperts || k < 1 || k > kMaxTopK || k > E || capacity < 0)
        return MOE_EINVAL;
    if ((int64_t)T * k >= kMaxRows || (int64_t)E * capacity >= kMaxRows) return MOE_EINVAL;
    const int64_t want_rows = capacity > 0 ? (int64_t)E * capacity : (int64_t)T * k;
    if (n_rows != want_rows) return MOE_EINVAL;
    if (!counts || !offsets) return MOE_EINVAL;
    if (T > 0 && (!logits || !topk_idx || !topk_w || !dst_row)) return MOE_EINVAL;
    if (n_rows > 0 && !src_slot) return MOE_EINVAL;
    const size_t need = moe_route_workspace_bytes(T, E, k);
    if (!ws || ws_bytes < need) return MOE_EWORKSPACE;
    // the block histograms [E][nblk]
    int32_t* hist = reinterpret_cast<int32_t*>((reinterpret_cast<uintptr_t>(ws) + kAlign - 1) / kAlign * kAlign);
    return status_of(launch_route(logits, T, E, k, capacity, topk_idx, topk_w, counts, offsets,
                                  dst_row, src_slot, n_rows, hist, dev_err,
                                  as_stream(stream)));
}

int moe_route_topk_noalloc(const float* logits, int T, int E, int k, int capacity, int32_t* topk_idx,
                           float* topk_w, int32_t* counts, int32_t* offsets, int32_t* dst_row,
                           int32_t* src_slot, int64_t n_rows, int32_t* dev_err, moe_stream_t stream)
{
    // the route's scratch (the block histograms) is written in full before it
    // is read, so nothing is cleared
    void* ptr = nullptr;
    if (scratch_of_current_device(&ptr) != hipSuccess) return MOE_EHIP;
    return moe_route_topk(logits, T, E, k, capacity, topk_idx, topk_w, counts, offsets, dst_row, src_slot,
                          n_rows, ptr, kNoAllocScratchBytes, dev_err, stream);
}

int moe_route_add_shared(int T, int E, int k, int n_shared, int capacity, const int32_t* topk_idx,
                         const float* topk_w, const int32_t* dst_row, const int32_t* counts,
                         const int32_t* offsets, const int32_t* src_slot, int64_t n_rows,
                         int32_t* topk_idx_out, float* topk_w_out, int32_t* counts_out,
                         int32_t* offsets_out, int32_t* dst_row_out, int32_t* src_slot_out,
                         moe_stream_t stream)
{
    if (T < 0 || E < 1 || k < 1 || n_shared < 1 || k + n_shared > kMaxTopK || E + n_shared > kMaxExperts ||
        capacity < 0)
        return MOE_EINVAL;
    const int64_t want_rows = capacity > 0 ? (int64_t)E * capacity : (int64_t)T * k;
    if (n_rows != want_rows || n_rows + (int64_t)n_shared * T >= kMaxRows) return MOE_EINVAL;
    if (!counts || !offsets || !counts_out || !offsets_out) return MOE_EINVAL;
    if (T > 0 && (!topk_idx || !topk_w || !dst_row || !topk_idx_out || !topk_w_out || !dst_row_out ||
                  !src_slot_out))
        return MOE_EINVAL;
    if (n_rows > 0 && !src_slot) return MOE_EINVAL;
    return status_of(launch_route_add_shared(topk_idx, topk_w, dst_row, counts, offsets, src_slot, T, E, k,
                                             n_shared, capacity, n_rows, topk_idx_out, topk_w_out, counts_out,
                                             offsets_out, dst_row_out, src_slot_out, as_stream(stream)));
}

int moe_permute(int dtype, const void* x, int T, int d, int k, const int32_t* dst_row,
                const int32_t* src_slot, const float* row_scale, int64_t n_rows, void* x_perm,
                uint8_t* x_perm_scales, int32_t* dev_err, moe_stream_t stream)
{
    if (dtype != MOE_F32 && dtype != MOE_BF16 && dtype != MOE_MXFP8) return MOE_EUNSUPPORTED;
    if (T < 0 || d < 1 || k < 1 || k > kMaxTopK || n_rows < 0 || n_rows >= kMaxRows)
        return MOE_EINVAL;
    if ((int64_t)T * k >= kMaxRows) return MOE_EINVAL;
    const bool padded = n_rows != (int64_t)T * k;
    if (T > 0 && (!x || !dst_row)) return MOE_EINVAL;
    if (n_rows > 0 && !x_perm) return MOE_EINVAL;
    if (padded && n_rows > 0 && !src_slot) return MOE_EINVAL;
    const int unit = dtype == MOE_MXFP8 ? 32 : (dtype == MOE_F32 ? 4 : 8);
    if (d % unit) return MOE_EALIGN;
    if (!aligned16(x) || !aligned16(x_perm)) return MOE_EALIGN;
    if (dtype == MOE_MXFP8) {
        if (row_scale) return MOE_EUNSUPPORTED;
        if (n_rows > 0 && !x_perm_scales) return MOE_EINVAL;
    }
    return status_of(launch_permute(dtype, x, T, d, k, dst_row, src_slot, row_scale, n_rows,
                                    x_perm, x_perm_scales, dev_err, as_stream(stream)));
}

int moe_unpermute_combine(int dtype, const void* y_perm, const int32_t* dst_row,
                          const float* weights, int T, int k, int d, int64_t n_rows, void* out,
                          int32_t* dev_err, moe_stream_t stream)
{
    if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_EUNSUPPORTED;
    if (T < 0 || d < 1 || k < 1 || k > kMaxTopK || n_rows < 0 || n_rows >= kMaxRows)
        return MOE_EINVAL;
    if (T > 0 && (!dst_row || !out || (n_rows > 0 && !y_perm))) return MOE_EINVAL;
    const int unit = dtype == MOE_F32 ? 4 : 8;
    if (d % unit) return MOE_EALIGN;
    if (!aligned16(y_perm) || !aligned16(out)) return MOE_EALIGN;
    return status_of(launch_combine(dtype, y_perm, dst_row, weights, T, k, d, n_rows, out, dev_err,
                                    as_stream(stream)));
}

size_t moe_gemm_workspace_bytes(int dtype, int E, int64_t n_rows, int d, int f)
{
    if (E < 1 || n_rows < 0 || d < 1 || f < 1) return 0;
    if (dtype == MOE_BF16) return kGemmCtlBytes;
    if (dtype != MOE_MXFP8) return 0;
    return gemm_ws_mxfp8(E, n_rows, d, f);
}

int moe_grouped_gemm_fwd(int dtype, const void* x_perm, const uint8_t* x_perm_scales,
                         const void* w13, const uint8_t* w13_scales, const void* w2,
                         const uint8_t* w2_scales, const int32_t* group_off, int capacity, int E,
                         int64_t n_rows, int d, int f, void* gu, void* h, void* y_perm, void* ws,
                         size_t ws_bytes, moe_stream_t stream)
{
    int st = check_gemm_shape(dtype, group_off, capacity, E, n_rows, d, f);
    if (st != MOE_OK) return st;
    if (!w13 || !w2) return MOE_EINVAL;
    if (n_rows > 0 && (!x_perm || !gu || !h || !y_perm)) return MOE_EINVAL;
    for (const void* p : {x_perm, w13, w2, (const void*)gu, (const void*)h, (const void*)y_perm})
        if (!aligned16(p)) return MOE_EALIGN;
    if (dtype == MOE_MXFP8) {
        if (!x_perm_scales || !w13_scales || !w2_scales) return MOE_EINVAL;
        if (!ws || ws_bytes < moe_gemm_workspace_bytes(dtype, E, n_rows, d, f) || !aligned16(ws))
            return MOE_EWORKSPACE;
    }
    moe_gemm_tensors t{};
    t.x_perm = x_perm;
    t.x_perm_scales = x_perm_scales;
    t.w13 = w13;
    t.w13_scales = w13_scales;
    t.w2 = w2;
    t.w2_scales = w2_scales;
    t.gu = gu;
    t.h = h;
    t.y_perm = y_perm;
    t.ws = ws;
    t.ws_bytes = ws_bytes;
    const GroupSpec g{capacity > 0 ? nullptr : group_off, capacity, E, n_rows};
    for (int op : {MOE_GEMM_GATE_UP, MOE_GEMM_DOWN}) {
        const int st2 = run_gemm_op(op, dtype, t, g, d, f, as_stream(stream));
        if (st2 != MOE_OK) return st2;
    }
    return MOE_OK;
}

int moe_grouped_gemm_bwd(int dtype, const void* dy_perm, const void* x_perm,
                         const uint8_t* x_perm_scales, const void* gu, const void* h,
                         const void* w13, const uint8_t* w13_scales, const void* w2,
                         const uint8_t* w2_scales, const int32_t* group_off, int capacity, int E,
                         int64_t n_rows, int d, int f, void* dgu, void* dx_perm, void* dw13,
                         void* dw2, void* ws, size_t ws_bytes, moe_stream_t stream)
{
    int st = check_gemm_shape(dtype, group_off, capacity, E, n_rows, d, f);
    if (st != MOE_OK) return st;
    if (!w13 || !w2 || !dw13 || !dw2) return MOE_EINVAL;
    if (n_rows > 0 && (!dy_perm || !x_perm || !gu || !h || !dgu || !dx_perm)) return MOE_EINVAL;
    for (const void* p : {dy_perm, x_perm, gu, h, w13, w2, (const void*)dgu, (const void*)dx_perm,
                          (const void*)dw13, (const void*)dw2})
        if (!aligned16(p)) return MOE_EALIGN;
    if (dtype == MOE_MXFP8 && (!x_perm_scales || !w13_scales || !w2_scales)) return MOE_EINVAL;
    if (dtype != MOE_F32 &&
        (!ws || ws_bytes < moe_gemm_workspace_bytes(dtype, E, n_rows, d, f) || !aligned16(ws)))
        return MOE_EWORKSPACE;
    moe_gemm_tensors t{};
    t.x_perm = x_perm;
    t.x_perm_scales = x_perm_scales;
    t.w13 = w13;
    t.w13_scales = w13_scales;
    t.w2 = w2;
    t.w2_scales = w2_scales;
    t.gu = const_cast<void*>(gu);
    t.h = const_cast<void*>(h);
    t.dy_perm = dy_perm;
    t.dgu = dgu;
    t.dx_perm = dx_perm;
    t.dw13 = dw13;
    t.dw2 = dw2;
    t.ws = ws;
    t.ws_bytes = ws_bytes;
    const GroupSpec g{capacity > 0 ? nullptr : group_off, capacity, E, n_rows};
    for (int op : {MOE_GEMM_DGRAD_DOWN, MOE_GEMM_DGRAD_GATE_UP, MOE_GEMM_WGRAD}) {
        const int st2 = run_gemm_op(op, dtype, t, g, d, f, as_stream(stream));
        if (st2 != MOE_OK) return st2;
    }
    return MOE_OK;
}

int moe_grouped_gemm_op(int op, int dtype, const moe_gemm_tensors* t,
                        const int32_t* group_off, int capacity, int E, int64_t n_rows, int d,
                        int f, moe_stream_t stream)
{
    if (!t) return MOE_EINVAL;
    if (op < MOE_GEMM_GATE_UP || op > MOE_GEMM_WGRAD) return MOE_EINVAL;
    int st = check_gemm_shape(dtype, group_off, capacity, E, n_rows, d, f);
    if (st != MOE_OK) return st;
    if (dtype == MOE_MXFP8) {
        const bool w13_op = op == MOE_GEMM_GATE_UP || op == MOE_GEMM_DGRAD_GATE_UP;
        const bool w2_op = op == MOE_GEMM_DOWN || op == MOE_GEMM_DGRAD_DOWN;
        if ((w13_op && !t->w13_scales) || (w2_op && !t->w2_scales)) return MOE_EINVAL;
        if ((op == MOE_GEMM_GATE_UP || op == MOE_GEMM_WGRAD) && n_rows > 0 && !t->x_perm_scales)
            return MOE_EINVAL;
        if (!t->ws || t->ws_bytes < moe_gemm_workspace_bytes(dtype, E, n_rows, d, f) || !aligned16(t->ws))
            return MOE_EWORKSPACE;
    }
    // operands each stage reads (r) and writes (w)
    const void* need[4] = {nullptr, nullptr, nullptr, nullptr};
    int n = 0;
    switch (op) {
    case MOE_GEMM_GATE_UP: need[0] = t->x_perm; need[1] = t->w13; need[2] = t->gu; need[3] = t->h; n = 4; break;
    case MOE_GEMM_DOWN: need[0] = t->h; need[1] = t->w2; need[2] = t->y_perm; n = 3; break;
    case MOE_GEMM_DGRAD_DOWN: need[0] = t->dy_perm; need[1] = t->w2; need[2] = t->gu; need[3] = t->dgu; n = 4; break;
    case MOE_GEMM_DGRAD_GATE_UP: need[0] = t->dgu; need[1] = t->w13; need[2] = t->dx_perm; n = 3; break;
    default: break;
    }
    const bool acc_f32 = t->dw13_f32 || t->dw2_f32;
    if (acc_f32) {
        // fp32 accumulate-into weight gradients: bf16 WGRAD only, both targets
        if (op != MOE_GEMM_WGRAD || dtype != MOE_BF16) return MOE_EUNSUPPORTED;
        if (!t->dw13_f32 || !t->dw2_f32) return MOE_EINVAL;
        if (!aligned16(t->dw13_f32) || !aligned16(t->dw2_f32)) return MOE_EALIGN;
    }
    if (op == MOE_GEMM_WGRAD) {
        const void* wn[6] = {t->dy_perm, t->h, acc_f32 ? (const void*)t->dw2_f32 : t->dw2, t->dgu, t->x_perm,
                             acc_f32 ? (const void*)t->dw13_f32 : t->dw13};
        for (const void* p : wn) {
            if (!p) return MOE_EINVAL;
            if (!aligned16(p)) return MOE_EALIGN;
        }
    } else {
        for (int i = 0; i < n; ++i) {
            const bool weight = need[i] == t->w13 || need[i] == t->w2;
            if (!need[i] && (weight || n_rows > 0)) return MOE_EINVAL;
            if (!aligned16(need[i])) return MOE_EALIGN;
        }
    }
    // the bf16 weight gradient keeps its tile-mapping flag in the workspace
    if (dtype == MOE_BF16 && op == MOE_GEMM_WGRAD &&
        (!t->ws || t->ws_bytes < moe_gemm_workspace_bytes(dtype, E, n_rows, d, f) || !aligned16(t->ws)))
        return MOE_EWORKSPACE;
    const GroupSpec g{capacity > 0 ? nullptr : group_off, capacity, E, n_rows};
    return run_gemm_op(op, dtype, *t, g, d, f, as_stream(stream));
}

int moe_router_logits(const void* x, const void* w_router, int T, int E, int d, float* logits,
                      moe_stream_t stream)
{
    if (T < 0 || T >= kMaxRows || E < 1 || E > kMaxExperts || d < 1) return MOE_EINVAL;
    if (T > 0 && (!x || !w_router || !logits)) return MOE_EINVAL;
    if ((int64_t)T * d >= ((int64_t)1 << 40)) return MOE_EINVAL;
    if (d % 8) return MOE_EALIGN;
    if (!aligned16(x) || !aligned16(w_router) || !aligned16(logits)) return MOE_EALIGN;
    return status_of(launch_router_logits((const uint16_t*)x, (const uint16_t*)w_router, T, E, d, logits,
                                          as_stream(stream)));
}

int moe_gate_grad(const void* dout, const void* y_perm, const int32_t* topk_idx, const float* topk_w,
                  const int32_t* dst_row, int T, int E, int k, int d, int64_t n_rows, float* dlogits,
                  float* dw, void* dy_perm, int32_t* dev_err, moe_stream_t stream)
{
    if (T < 0 || k < 1 || k > kMaxTopK || E < k || E > kMaxExperts || d < 1 || n_rows < 0 ||
        n_rows >= kMaxRows || (int64_t)T * k >= kMaxRows)
        return MOE_EINVAL;
    if (T > 0 && (!dout || !topk_idx || !topk_w || !dst_row || !dlogits)) return MOE_EINVAL;
    if (T > 0 && n_rows > 0 && !y_perm) return MOE_EINVAL;
    if (d % 8) return MOE_EALIGN;
    if (!aligned16(dout) || !aligned16(y_perm) || !aligned16(dy_perm) || !aligned16(dlogits))
        return MOE_EALIGN;
    if (dy_perm && n_rows != (int64_t)T * k) return MOE_EUNSUPPORTED;
    return status_of(launch_gate_grad(dout, y_perm, topk_idx, topk_w, dst_row, T, E, k, d, n_rows, dlogits,
                                      dw, dy_perm, dev_err, as_stream(stream)));
}

int moe_quantize_mxfp8(const void* src, int64_t rows, int K, int colwise, const int32_t* group_off,
                       int n_groups, uint8_t* codes, uint8_t* scales, moe_stream_t stream)
{
    if (rows < 0 || rows >= kMaxRows || K < 1) return MOE_EINVAL;
    if (rows > 0 && (!src || !codes || !scales)) return MOE_EINVAL;
    if (!aligned16(src) || !aligned16(codes)) return MOE_EALIGN;
    hipStream_t s = as_stream(stream);
    if (!colwise) {
        if (K % 32) return MOE_EALIGN;
        return status_of(launch_quantize_rows((const uint16_t*)src, rows, K, codes, scales, s));
    }
    if (group_off && (n_groups < 1 || n_groups > kMaxExperts)) return MOE_EINVAL;
    // 16-byte loads along each source row; whole 32-bit scale words
    if (K % 8 || (reinterpret_cast<uintptr_t>(scales) & 3u)) return MOE_EALIGN;
    return status_of(launch_quantize_cols((const uint16_t*)src, rows, K, group_off, 0,
                                          group_off ? n_groups : 1, codes, scales, s));
}

}  // extern "C"
