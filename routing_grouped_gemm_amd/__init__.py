"""Python binding of libmoe: one GPU's MoE feed-forward layer on MI355X (gfx950).

Thin ctypes marshalling over the C ABI in ``include/moe.h``: every function
below has the name of the C entry point it calls, takes torch tensors that
already live on the GPU, passes their data pointers, sizes and the current
HIP stream, and raises ``MoeError`` on a non-OK status.  No computation
happens here and there is no CPU fallback: if ``libmoe.so`` has not been
built, importing the functions that need it raises ``ImportError``.

Build the library in-tree with ``python -m routing_grouped_gemm_amd.build``.
"""
import ctypes
import os

import torch

MOE_OK, MOE_EINVAL, MOE_EALIGN, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = 0, -1, -2, -3, -4, -5
MOE_F32, MOE_BF16, MOE_MXFP8 = 0, 1, 2
MOE_ERR_NONFINITE_LOGIT, MOE_ERR_ROW_RANGE = 1, 2

MOE_GEMM_GATE_UP, MOE_GEMM_DOWN, MOE_GEMM_DGRAD_DOWN, MOE_GEMM_DGRAD_GATE_UP, MOE_GEMM_WGRAD = \
    0, 1, 2, 3, 4

ABI_FUNCTIONS = ("moe_route_workspace_bytes", "moe_route_topk", "moe_route_topk_noalloc", "moe_permute",
                 "moe_gemm_workspace_bytes", "moe_grouped_gemm_fwd", "moe_grouped_gemm_bwd",
                 "moe_grouped_gemm_op", "moe_unpermute_combine", "moe_quantize_mxfp8",
                 "moe_route_add_shared", "moe_router_logits", "moe_gate_grad", "moe_status_string",
                 "moe_version")

GEMM_TENSOR_FIELDS = ("x_perm", "x_perm_scales", "w13", "w13_scales", "w2", "w2_scales", "gu",
                      "h", "y_perm", "dy_perm", "dgu", "dx_perm", "dw13", "dw2", "ws")
GEMM_TENSOR_FIELDS_F32 = ("dw13_f32", "dw2_f32")   # after ws_bytes: fp32 weight-gradient accumulators


class MoeGemmTensors(ctypes.Structure):
    """C struct moe_gemm_tensors (device pointers, NULL where unused)."""
    _fields_ = [(n, ctypes.c_void_p) for n in GEMM_TENSOR_FIELDS] + [("ws_bytes", ctypes.c_size_t)] + \
        [(n, ctypes.c_void_p) for n in GEMM_TENSOR_FIELDS_F32]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")
_lib = None


class MoeError(RuntimeError):
    def __init__(self, status, name):
        self.status = status
        msg = load().moe_status_string(status).decode()
        super().__init__(f"{name} returned {status}: {msg}")


def load():
    """Load libmoe.so (once).  Raises ImportError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m routing_grouped_gemm_amd.build` (there is no fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lib.moe_version.restype = I
    lib.moe_version.argtypes = []
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_status_string.argtypes = [I]
    lib.moe_route_workspace_bytes.restype = SZ
    lib.moe_route_workspace_bytes.argtypes = [I, I, I]
    lib.moe_route_topk.restype = I
    lib.moe_route_topk.argtypes = [P, I, I, I, I, P, P, P, P, P, P, I64, P, SZ, P, P]
    lib.moe_route_topk_noalloc.restype = I
    lib.moe_route_topk_noalloc.argtypes = [P, I, I, I, I, P, P, P, P, P, P, I64, P, P]
    lib.moe_permute.restype = I
    lib.moe_permute.argtypes = [I, P, I, I, I, P, P, P, I64, P, P, P, P]
    lib.moe_gemm_workspace_bytes.restype = SZ
    lib.moe_gemm_workspace_bytes.argtypes = [I, I, I64, I, I]
    lib.moe_grouped_gemm_fwd.restype = I
    lib.moe_grouped_gemm_fwd.argtypes = [I, P, P, P, P, P, P, P, I, I, I64, I, I, P, P, P, P, SZ, P]
    lib.moe_grouped_gemm_bwd.restype = I
    lib.moe_grouped_gemm_bwd.argtypes = [I, P, P, P, P, P, P, P, P, P, P, I, I, I64, I, I, P, P, P,
                                         P, P, SZ, P]
    lib.moe_grouped_gemm_op.restype = I
    lib.moe_grouped_gemm_op.argtypes = [I, I, ctypes.POINTER(MoeGemmTensors), P, I, I, I64, I, I,
                                        P]
    lib.moe_unpermute_combine.restype = I
    lib.moe_unpermute_combine.argtypes = [I, P, P, P, I, I, I, I64, P, P, P]
    lib.moe_quantize_mxfp8.restype = I
    lib.moe_quantize_mxfp8.argtypes = [P, I64, I, I, P, I, P, P, P]
    lib.moe_route_add_shared.restype = I
    lib.moe_route_add_shared.argtypes = [I, I, I, I, I, P, P, P, P, P, P, I64, P, P, P, P, P, P, P]
    lib.moe_router_logits.restype = I
    lib.moe_router_logits.argtypes = [P, P, I, I, I, P, P]
    lib.moe_gate_grad.restype = I
    lib.moe_gate_grad.argtypes = [P, P, P, P, P, I, I, I, I, I64, P, P, P, P, P]
    _lib = lib
    return lib


def lib_path():
    return LIB_PATH


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _s(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check(rc, name):
    if rc != MOE_OK:
        raise MoeError(rc, name)


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


# ------------------------------------------------------------------ ABI calls
def moe_version():
    return load().moe_version()


def moe_status_string(status):
    return load().moe_status_string(status).decode()


def moe_route_workspace_bytes(T, E, k):
    return int(load().moe_route_workspace_bytes(T, E, k))


def moe_route_topk(logits, k, capacity, topk_idx, topk_w, counts, offsets, dst_row, src_slot, ws,
                   dev_err=None, stream=None):
    """logits [T, E] fp32 -> topk_idx [T,k] i32, topk_w [T,k] f32, counts [E], offsets [E+1],
    dst_row [T*k], src_slot [n_rows] (n_rows = T*k, or E*capacity when padded)."""
    T, E = logits.shape
    n_rows = src_slot.numel()
    rc = load().moe_route_topk(_p(logits), T, E, k, capacity, _p(topk_idx), _p(topk_w),
                               _p(counts), _p(offsets), _p(dst_row), _p(src_slot), n_rows, _p(ws),
                               _nbytes(ws), _p(dev_err), _s(stream))
    _check(rc, "moe_route_topk")


ROUTE_NOALLOC_MAX_BYTES = 32 << 20    # MOE_ROUTE_NOALLOC_MAX_BYTES in moe.h


def moe_route_topk_noalloc(logits, k, capacity, topk_idx, topk_w, counts, offsets, dst_row, src_slot,
                           dev_err=None, stream=None):
    """moe_route_topk with the library's fixed per-GPU scratch instead of a workspace."""
    T, E = logits.shape
    n_rows = src_slot.numel()
    rc = load().moe_route_topk_noalloc(_p(logits), T, E, k, capacity, _p(topk_idx), _p(topk_w),
                                       _p(counts), _p(offsets), _p(dst_row), _p(src_slot), n_rows,
                                       _p(dev_err), _s(stream))
    _check(rc, "moe_route_topk_noalloc")


def moe_permute(dtype, x, k, dst_row, x_perm, src_slot=None, row_scale=None, x_perm_scales=None,
                dev_err=None, stream=None):
    """x [T, d] -> x_perm [n_rows, d] (MXFP8: codes + x_perm_scales [n_rows, d/32])."""
    T, d = x.shape
    n_rows = x_perm.shape[0]
    rc = load().moe_permute(dtype, _p(x), T, d, k, _p(dst_row), _p(src_slot), _p(row_scale),
                            n_rows, _p(x_perm), _p(x_perm_scales), _p(dev_err), _s(stream))
    _check(rc, "moe_permute")


def moe_gemm_workspace_bytes(dtype, E, n_rows, d, f):
    return int(load().moe_gemm_workspace_bytes(dtype, E, n_rows, d, f))


def moe_grouped_gemm_fwd(dtype, x_perm, w13, w2, group_off, capacity, gu, h, y_perm,
                         x_perm_scales=None, w13_scales=None, w2_scales=None, ws=None,
                         stream=None):
    """x_perm [n_rows, d], w13 [E, 2f, d], w2 [E, d, f] -> gu [n_rows, 2f], h [n_rows, f],
    y_perm [n_rows, d].  group_off [E+1] device int32 (ignored when capacity > 0, but its
    length still gives E)."""
    E = group_off.numel() - 1
    n_rows, d = x_perm.shape
    f = h.shape[1]
    rc = load().moe_grouped_gemm_fwd(dtype, _p(x_perm), _p(x_perm_scales), _p(w13),
                                     _p(w13_scales), _p(w2), _p(w2_scales), _p(group_off),
                                     capacity, E, n_rows, d, f, _p(gu), _p(h), _p(y_perm), _p(ws),
                                     _nbytes(ws), _s(stream))
    _check(rc, "moe_grouped_gemm_fwd")


def moe_grouped_gemm_bwd(dtype, dy_perm, x_perm, gu, h, w13, w2, group_off, capacity, dgu,
                         dx_perm, dw13, dw2, x_perm_scales=None, w13_scales=None, w2_scales=None,
                         ws=None, stream=None):
    """Activation and weight gradients of the grouped SwiGLU FFN (see include/moe.h)."""
    E = group_off.numel() - 1
    n_rows, d = dy_perm.shape
    f = h.shape[1]
    rc = load().moe_grouped_gemm_bwd(dtype, _p(dy_perm), _p(x_perm), _p(x_perm_scales), _p(gu),
                                     _p(h), _p(w13), _p(w13_scales), _p(w2), _p(w2_scales),
                                     _p(group_off), capacity, E, n_rows, d, f, _p(dgu),
                                     _p(dx_perm), _p(dw13), _p(dw2), _p(ws), _nbytes(ws),
                                     _s(stream))
    _check(rc, "moe_grouped_gemm_bwd")


def gemm_tensors(**tensors):
    """Build a MoeGemmTensors from keyword tensors (names as in GEMM_TENSOR_FIELDS;
    ws is a uint8 workspace tensor whose size becomes ws_bytes)."""
    bad = set(tensors) - set(GEMM_TENSOR_FIELDS) - set(GEMM_TENSOR_FIELDS_F32)
    if bad:
        raise TypeError(f"unknown operand(s) {sorted(bad)}")
    st = MoeGemmTensors(**{n: _p(t) for n, t in tensors.items()})
    if tensors.get("ws") is not None:
        st.ws_bytes = tensors["ws"].numel() * tensors["ws"].element_size()
    return st


def moe_grouped_gemm_op(op, dtype, tensors, group_off, capacity, E, n_rows, d, f, stream=None):
    """One grouped GEMM stage; tensors is a MoeGemmTensors (gemm_tensors())."""
    rc = load().moe_grouped_gemm_op(op, dtype, ctypes.byref(tensors), _p(group_off), capacity, E,
                                    n_rows, d, f, _s(stream))
    _check(rc, "moe_grouped_gemm_op")


def moe_unpermute_combine(dtype, y_perm, dst_row, weights, k, out, dev_err=None, stream=None):
    """out[t] = sum_j weights[t*k+j] * y_perm[dst_row[t*k+j]] (weights None: unweighted)."""
    T, d = out.shape
    n_rows = y_perm.shape[0]
    rc = load().moe_unpermute_combine(dtype, _p(y_perm), _p(dst_row), _p(weights), T, k, d,
                                      n_rows, _p(out), _p(dev_err), _s(stream))
    _check(rc, "moe_unpermute_combine")


def moe_route_add_shared(n_shared, capacity, topk_idx, topk_w, dst_row, counts, offsets, src_slot,
                         topk_idx_out, topk_w_out, counts_out, offsets_out, dst_row_out, src_slot_out,
                         stream=None):
    """The route of k slots -> the route of k + n_shared slots (shared experts E .. E+n_shared-1)."""
    T, k = topk_idx.shape
    E = counts.numel()
    rc = load().moe_route_add_shared(T, E, k, n_shared, capacity, _p(topk_idx), _p(topk_w), _p(dst_row),
                                     _p(counts), _p(offsets), _p(src_slot), src_slot.numel(), _p(topk_idx_out),
                                     _p(topk_w_out), _p(counts_out), _p(offsets_out), _p(dst_row_out),
                                     _p(src_slot_out), _s(stream))
    _check(rc, "moe_route_add_shared")


def moe_router_logits(x, w_router, logits, stream=None):
    """logits [T, E] fp32 = x [T, d] bf16 . w_router [E, d] bf16 ^T."""
    T, d = x.shape
    E = w_router.shape[0]
    rc = load().moe_router_logits(_p(x), _p(w_router), T, E, d, _p(logits), _s(stream))
    _check(rc, "moe_router_logits")


def moe_gate_grad(dout, y_perm, topk_idx, topk_w, dst_row, dlogits, dw=None, dy_perm=None,
                  dev_err=None, stream=None):
    """dlogits [T, E] (and optionally dw [T, k], and the combine backward into dy_perm)
    from dout [T, d] and the forward's expert outputs y_perm [n_rows, d]."""
    T, d = dout.shape
    k = topk_idx.shape[1]
    E = dlogits.shape[1]
    n_rows = y_perm.shape[0]
    rc = load().moe_gate_grad(_p(dout), _p(y_perm), _p(topk_idx), _p(topk_w), _p(dst_row), T, E, k, d,
                              n_rows, _p(dlogits), _p(dw), _p(dy_perm), _p(dev_err), _s(stream))
    _check(rc, "moe_gate_grad")


def moe_quantize_mxfp8(src, colwise, codes, scales, group_off=None, n_groups=0, stream=None):
    """bf16 src [rows, K] -> E4M3FN codes + E8M0 scales (row-wise or per-group column-wise)."""
    rows, K = src.shape
    rc = load().moe_quantize_mxfp8(_p(src), rows, K, int(colwise), _p(group_off), n_groups,
                                   _p(codes), _p(scales), _s(stream))
    _check(rc, "moe_quantize_mxfp8")
