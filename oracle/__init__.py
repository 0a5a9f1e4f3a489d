"""Plain CPU oracle for one GPU's MoE feed-forward layer -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``moe_oracle.c`` (plain C,
fp64 arithmetic, storage rounding modelled explicitly) through ctypes on
numpy arrays.  It shares no code with the HIP library and never imports it.

What each function computes, and the page passage it follows, is stated in
``moe_oracle.c``.  Rounding modes: ``NONE`` (keep fp64), ``FP32``, ``BF16``.

Parity status: every function is pinned in ``tests/test_oracle_*.py``
against brute force, library routines (torch / numpy), closed forms or
invariants; the MXFP8 composition of the FFN (``mx_h``, ``mx_dgu``, the
substituted operands and the ``mx_qdq_*`` wrappers) against an independent
torch float64 chain and exact operand probes, with planted mistakes in the
C source that the checks catch (``tests/test_oracle_mx_chain.py``).  The
MXFP8 scale-rounding direction (ceil of log2(amax/448)) is pinned against
the property the tutorial's MXFP8 paragraph states (the block maximum never
overflows 448, and the next smaller power of two would) and torch's
E4M3FN/E8M0 codecs; the pages print no implementation to compare beyond that.
"""
import ctypes
import os
import subprocess

import numpy as np

NONE, FP32, BF16 = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None


def build(force=True):
    """Compile moe_oracle.c with gcc (no fast-math: fp semantics preserved)."""
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-std=c11", "-Wall", "-shared", "-fPIC",
                           _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    _lib = open_library(_LIB_PATH)
    return _lib


def open_library(path):
    """Open a compiled oracle library at `path` with every entry point's
    argument types declared (the wrappers below call whichever library
    ``_load`` returns; the tests open deliberately broken builds this way to
    show their checks catch them)."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I, L, D = ctypes.c_int, ctypes.c_long, ctypes.c_double
    lib.oracle_round.argtypes = [D, I]
    lib.oracle_round.restype = D
    lib.oracle_round_array.argtypes = [P, P, L, I]
    lib.oracle_route.argtypes = [P, I, I, I, I, P, P, P, P, P, P, L]
    lib.oracle_route.restype = I
    lib.oracle_permute.argtypes = [P, I, I, I, P, P, L, I, P]
    lib.oracle_combine.argtypes = [P, P, P, I, I, I, I, P]
    lib.oracle_router_logits.argtypes = [P, P, I, I, I, I, P]
    lib.oracle_gate_grad.argtypes = [P, P, P, P, P, I, I, I, I, I, P, P]
    lib.oracle_ffn_fwd.argtypes = [P, P, P, P, I, I, I, I, I, P, P, P]
    lib.oracle_ffn_bwd.argtypes = [P, P, P, P, P, P, P, I, I, I, I, P, P, P, P, P, I,
                                   P, P, P, P]
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_decode.restype = D
    lib.oracle_e4m3_encode.argtypes = [D]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_e8m0_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e8m0_decode.restype = D
    lib.oracle_mx_scale_exp.argtypes = [D]
    lib.oracle_mx_scale_exp.restype = I
    lib.oracle_mx_quantize_vector.argtypes = [P, L, L, P, L, P]
    lib.oracle_mx_qdq_vector.argtypes = [P, L, L, P, L]
    return lib


def set_threads(n):
    """Set the OpenMP thread count the oracle uses (returns nothing)."""
    os.environ["OMP_NUM_THREADS"] = str(n)
    try:
        libgomp = ctypes.CDLL("libgomp.so.1")
        libgomp.omp_set_num_threads(ctypes.c_int(int(n)))
    except OSError:
        pass


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


# ---------------------------------------------------------------- rounding
def round_(v, mode):
    v = _f64(v)
    out = np.empty_like(v)
    _load().oracle_round_array(_p(v), _p(out), v.size, mode)
    return out


# ---------------------------------------------------------------- route
def route(logits, k, capacity=0):
    """Top-k selection, gate weights and the route map for fp32 logits [T, E].

    Returns a dict of numpy arrays: topk_idx [T,k] int32, topk_w [T,k] fp32,
    counts [E], offsets [E+1], dst_row [T*k] (-1 = dropped), src_slot
    [n_rows] (-1 = padding row) and n_rows (T*k, or E*capacity when padded).
    """
    lg = _f32(logits)
    T, E = lg.shape
    n_rows = E * capacity if capacity > 0 else T * k
    out = dict(topk_idx=np.empty((T, k), np.int32), topk_w=np.empty((T, k), np.float32),
               counts=np.empty(E, np.int32), offsets=np.empty(E + 1, np.int32),
               dst_row=np.empty(T * k, np.int32), src_slot=np.empty(n_rows, np.int32))
    rc = _load().oracle_route(_p(lg), T, E, k, capacity, _p(out["topk_idx"]), _p(out["topk_w"]),
                              _p(out["counts"]), _p(out["offsets"]), _p(out["dst_row"]),
                              _p(out["src_slot"]), n_rows)
    if rc != 0:
        raise ValueError("oracle_route rejected its input (non-finite logit or bad sizes)")
    out["n_rows"] = n_rows
    return out


def group_offsets(offsets, capacity=0):
    """Row ranges of the expert groups: the route offsets, or e*C when padded."""
    offsets = np.asarray(offsets)
    E = offsets.size - 1
    if capacity > 0:
        return (np.arange(E + 1) * capacity).astype(np.int32)
    return _i32(offsets)


# ---------------------------------------------------------------- permute / combine
def permute(x, dst_row, k, n_rows, row_scale=None, round_mode=NONE):
    x = _f64(x)
    T, d = x.shape
    out = np.empty((n_rows, d), np.float64)
    rs = None if row_scale is None else _f32(row_scale).reshape(-1)
    _load().oracle_permute(_p(x), T, d, k, _p(_i32(dst_row)), _p(rs), n_rows, round_mode,
                           _p(out))
    return out


def combine(y_perm, dst_row, w, T, k, round_mode=NONE):
    y = _f64(y_perm)
    d = y.shape[1]
    out = np.empty((T, d), np.float64)
    ww = None if w is None else _f32(w).reshape(-1)
    _load().oracle_combine(_p(y), _p(_i32(dst_row)), _p(ww), T, k, d, round_mode, _p(out))
    return out


# ---------------------------------------------------------------- router
def router_logits(x, w_r, round_mode=FP32):
    """Router scores [T, E] = x [T, d] . w_r [E, d]^T (fp64 sums, stored per round_mode)."""
    x = _f64(x)
    w = _f64(w_r)
    T, d = x.shape
    E = w.shape[0]
    assert w.shape == (E, d)
    out = np.empty((T, E))
    _load().oracle_router_logits(_p(x), _p(w), T, E, d, round_mode, _p(out))
    return out


def gate_grad(dout, y_perm, dst_row, topk_idx, topk_w, E, round_mode=FP32):
    """Gradient through the gate weights.  Returns (dw [T, k] fp64, dlogits [T, E])."""
    g = _f64(dout)
    y = _f64(y_perm)
    idx = _i32(topk_idx)
    T, k = idx.shape
    d = g.shape[1]
    assert y.shape[1] == d
    dw = np.empty((T, k))
    dl = np.empty((T, E))
    _load().oracle_gate_grad(_p(g), _p(y), _p(_i32(dst_row)), _p(idx), _p(_f32(topk_w)), T, E, k, d,
                             round_mode, _p(dw), _p(dl))
    return dw, dl


# ---------------------------------------------------------------- expert FFN
def ffn_fwd(x_perm, w13, w2, group_off, round_mode=NONE, mx_h=False):
    """Grouped SwiGLU FFN forward.  Returns (gu [R,2f], h [R,f], y [R,d])."""
    x = _f64(x_perm)
    w13 = _f64(w13)
    w2 = _f64(w2)
    go = _i32(group_off)
    E, two_f, d = w13.shape
    f = two_f // 2
    R = int(go[-1])
    assert x.shape[0] >= R and x.shape[1] == d and w2.shape == (E, d, f)
    gu = np.empty((R, 2 * f))
    h = np.empty((R, f))
    y = np.empty((R, d))
    _load().oracle_ffn_fwd(_p(x), _p(w13), _p(w2), _p(go), E, d, f, round_mode, int(mx_h),
                           _p(gu), _p(h), _p(y))
    return gu, h, y


def ffn_bwd(dy_perm, x_perm, gu, h, w13, w2, group_off, round_mode=NONE, w2_dgrad=None,
            w13_dgrad=None, dy_wgrad=None, h_wgrad=None, x_wgrad=None, mx_dgu=False):
    """Grouped SwiGLU FFN backward.  Returns (dgu [R,2f], dx_perm [R,d], dw13, dw2)."""
    dy = _f64(dy_perm)
    x = _f64(x_perm)
    gu = _f64(gu)
    h = _f64(h)
    w13 = _f64(w13)
    w2 = _f64(w2)
    go = _i32(group_off)
    E, two_f, d = w13.shape
    f = two_f // 2
    R = int(go[-1])
    opt = [None if a is None else _f64(a) for a in (w2_dgrad, w13_dgrad, dy_wgrad, h_wgrad,
                                                     x_wgrad)]
    dgu = np.empty((R, 2 * f))
    dx = np.empty((R, d))
    dw13 = np.empty((E, 2 * f, d))
    dw2 = np.empty((E, d, f))
    _load().oracle_ffn_bwd(_p(dy), _p(x), _p(gu), _p(h), _p(w13), _p(w2), _p(go), E, d, f,
                           round_mode, *[_p(a) for a in opt], int(mx_dgu), _p(dgu), _p(dx),
                           _p(dw13), _p(dw2))
    return dgu, dx, dw13, dw2


# ---------------------------------------------------------------- MXFP8
def e4m3_decode(code):
    return _load().oracle_e4m3_decode(int(code))


def e4m3_encode(v):
    return int(_load().oracle_e4m3_encode(float(v)))


def e8m0_decode(code):
    return _load().oracle_e8m0_decode(int(code))


def mx_scale_exp(amax):
    return int(_load().oracle_mx_scale_exp(float(amax)))


def mx_quantize_rows(v):
    """Row-wise MXFP8: 32-element blocks along the last axis of v [rows, K].

    Returns (codes uint8 [rows, K], scales uint8 [rows, ceil(K/32)])."""
    v = _f64(v)
    rows, K = v.shape
    nb = (K + 31) // 32
    codes = np.empty((rows, K), np.uint8)
    scales = np.empty((rows, nb), np.uint8)
    lib = _load()
    for r in range(rows):
        lib.oracle_mx_quantize_vector(_p(v[r]), K, 1, _p(codes[r]), 1, _p(scales[r]))
    return codes, scales


def mx_quantize_cols(v, group_off):
    """Column-wise MXFP8 inside row groups: for each group [g0, g1) of v [rows, K]
    and each column, 32-element blocks along the rows starting at g0.

    Returns (codes uint8 [rows, K] in v's layout, scales uint8 [K, nblk_total])
    where group e's blocks occupy scale columns [sb_e, sb_e + ceil(m_e/32))
    with sb_e the running sum of ceil(m/32) over earlier groups."""
    v = _f64(v)
    rows, K = v.shape
    go = np.asarray(group_off, np.int64)
    nblk = [(int(go[e + 1] - go[e]) + 31) // 32 for e in range(len(go) - 1)]
    codes = np.zeros((rows, K), np.uint8)
    scales = np.zeros((K, sum(nblk)), np.uint8)
    lib = _load()
    sb = 0
    for e in range(len(go) - 1):
        g0, g1 = int(go[e]), int(go[e + 1])
        if g1 > g0:
            for c in range(K):
                col_scales = np.empty(nblk[e], np.uint8)
                vc = np.ascontiguousarray(v[g0:g1, c])
                cc = np.empty(g1 - g0, np.uint8)
                lib.oracle_mx_quantize_vector(_p(vc), g1 - g0, 1, _p(cc), 1, _p(col_scales))
                codes[g0:g1, c] = cc
                scales[c, sb:sb + nblk[e]] = col_scales
        sb += nblk[e]
    return codes, scales


def mx_qdq_rows(v):
    """Value represented by row-wise MXFP8 of v (quantise then dequantise)."""
    v = _f64(v)
    out = np.empty_like(v)
    lib = _load()
    rows, K = v.shape
    for r in range(rows):
        lib.oracle_mx_qdq_vector(_p(v[r]), K, 1, _p(out[r]), 1)
    return out


def mx_qdq_cols(v, group_off):
    """Value represented by column-wise (per row group) MXFP8 of v."""
    v = _f64(v)
    out = np.zeros_like(v)
    go = np.asarray(group_off, np.int64)
    lib = _load()
    rows, K = v.shape
    vt = np.ascontiguousarray(v.T)
    ot = np.zeros_like(vt)
    for e in range(len(go) - 1):
        g0, g1 = int(go[e]), int(go[e + 1])
        if g1 > g0:
            for c in range(K):
                lib.oracle_mx_qdq_vector(_p(vt[c, g0:]), g1 - g0, 1, _p(ot[c, g0:]), 1)
    out[:] = ot.T
    return out


def mx_dequant_rows(codes, scales):
    """Decode row-wise MXFP8 (codes [rows, K], scales [rows, ceil(K/32)])."""
    codes = np.asarray(codes, np.uint8)
    scales = np.asarray(scales, np.uint8)
    table = np.array([e4m3_decode(c) for c in range(256)])
    rows, K = codes.shape
    s = np.array([e8m0_decode(c) for c in range(256)])[scales]
    return table[codes] * np.repeat(s, 32, axis=1)[:, :K]
