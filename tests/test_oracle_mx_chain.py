"""Pins for the oracle's MXFP8 composition of the grouped SwiGLU FFN.

The tutorial's MXFP8 section runs all three GEMMs of each linear (forward,
activation gradient, weight gradient) on E4M3 elements with one power-of-two
scale per 32 elements, kept in a forward and a backward cache.  The oracle
composes that from its codec: the down GEMM of the forward reads a row-wise
MX copy of h (``mx_h``), the activation-gradient GEMM of gate/up reads a
row-wise copy of dgu and the weight gradient a copy quantised along the
tokens of each expert group (``mx_dgu``), and every other GEMM operand is
substituted by the caller (``w2_dgrad``, ``w13_dgrad``, ``dy_wgrad``,
``h_wgrad``, ``x_wgrad``) with the wrappers ``mx_qdq_rows`` / ``mx_qdq_cols``.

The independent reference below is a torch float64 chain written from the
definitions alone: blocks of 32 along each GEMM's contraction axis (along
the tokens, restarting at each group's first row, for the weight gradient),
scale exponent read off the block maximum's binary exponent and mantissa
(2^e with e the least integer such that max / 2^e <= 448), elements cast
with torch's own float8_e4m3fn, bf16 storage rounding done by rounding to
odd into fp32 and then to nearest-even into bf16 (correct single rounding).
It shares nothing with the oracle's C code.

Both sides accumulate in fp64 and round at the same storage points, so they
agree to fp64 summation-order noise.  Each check is then repeated on
oracle builds with a planted mistake (wrong block axis, column blocks
shifted by one row, blocks not restarting at group starts, the stored dgu
fed where its quantised copy belongs, the row-wise copy fed to the weight
gradient) and must fail on every one of them.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

TOL = 1e-9          # relative to max|ref|: fp64 summation-order noise only
SRC = os.path.join(os.path.dirname(oracle.__file__), "moe_oracle.c")


# ------------------------------------------------------------ torch reference
def t_bf16(v):
    """float64 -> nearest bfloat16 (ties to even) as float64, by rounding to
    odd into float32 first (no double-rounding error)."""
    v = v.to(torch.float64)
    f = v.to(torch.float32)
    back = f.to(torch.float64)
    inexact = back != v
    over = inexact & (back.abs() > v.abs())
    bits = f.view(torch.int32)
    bits = torch.where(over, bits - 1, bits)          # one ulp toward zero (sign-magnitude)
    bits = torch.where(inexact, bits | 1, bits)       # sticky bit
    return bits.view(torch.float32).to(torch.bfloat16).to(torch.float64)


def t_mx_qdq_lastdim(v):
    """Value of MXFP8 with blocks of 32 along the last axis (from index 0;
    a short last block takes the elements present)."""
    n, L = v.shape
    pad = (-L) % 32
    b = F.pad(v, (0, pad)).reshape(n, -1, 32)
    amax = b.abs().amax(-1, keepdim=True)
    m, ex = torch.frexp(amax)                  # amax = m 2^ex, m in [0.5, 1)
    # least e with amax <= 1.75 * 2^(8+e): from amax's exponent and mantissa
    e = (ex - 9) + (2 * m > 1.75).to(ex.dtype)
    e = torch.where(amax > 0, e, torch.full_like(e, -127)).clamp(-127, 127)
    scale = torch.ldexp(torch.ones_like(amax), e)
    q = (b / scale).to(torch.float8_e4m3fn).to(torch.float64) * scale
    return q.reshape(n, -1)[:, :L]


def t_qrow(v):
    return t_mx_qdq_lastdim(v)


def t_qcol(v, go):
    """Blocks of 32 along the rows, restarting at each group's first row."""
    out = torch.zeros_like(v)
    for e in range(len(go) - 1):
        g0, g1 = int(go[e]), int(go[e + 1])
        if g1 > g0:
            out[g0:g1] = t_mx_qdq_lastdim(v[g0:g1].T.contiguous()).T
    return out


def t_chain(x, w13, w2, dy, go):
    """The MXFP8 expert FFN forward and backward, every GEMM operand
    quantised along that GEMM's contraction axis."""
    E, two_f, d = w13.shape
    f = two_f // 2
    R = x.shape[0]
    xq = t_qrow(x)                                                   # dispatch payload
    w13f = t_qrow(w13.reshape(-1, d)).reshape(E, 2 * f, d)           # fwd caches: along d / f
    w2f = t_qrow(w2.reshape(-1, f)).reshape(E, d, f)
    g13 = np.arange(E + 1) * 2 * f
    g2 = np.arange(E + 1) * d
    w13b = t_qcol(w13.reshape(-1, d), g13).reshape(E, 2 * f, d)      # bwd caches: along 2f / d
    w2b = t_qcol(w2.reshape(-1, f), g2).reshape(E, d, f)
    gu = torch.zeros(R, 2 * f, dtype=torch.float64)
    h = torch.zeros(R, f, dtype=torch.float64)
    for e in range(E):
        r0, r1 = int(go[e]), int(go[e + 1])
        g = xq[r0:r1] @ w13f[e, :f].T
        u = xq[r0:r1] @ w13f[e, f:].T
        gu[r0:r1, :f], gu[r0:r1, f:] = t_bf16(g), t_bf16(u)
        h[r0:r1] = t_bf16(F.silu(g) * u)
    hq = t_qrow(h)
    y = torch.zeros(R, d, dtype=torch.float64)
    for e in range(E):
        r0, r1 = int(go[e]), int(go[e + 1])
        y[r0:r1] = t_bf16(hq[r0:r1] @ w2f[e].T)
    # backward
    dyq = t_qrow(dy)
    dgu = torch.zeros(R, 2 * f, dtype=torch.float64)
    for e in range(E):
        r0, r1 = int(go[e]), int(go[e + 1])
        dh = dyq[r0:r1] @ w2b[e]                    # contraction over d
        g, u = gu[r0:r1, :f], gu[r0:r1, f:]
        s = torch.sigmoid(g)
        dgu[r0:r1, :f] = t_bf16(dh * u * s * (1 + g * (1 - s)))
        dgu[r0:r1, f:] = t_bf16(dh * g * s)
    dguq = t_qrow(dgu)
    dx = torch.zeros(R, d, dtype=torch.float64)
    for e in range(E):
        r0, r1 = int(go[e]), int(go[e + 1])
        dx[r0:r1] = t_bf16(dguq[r0:r1] @ w13b[e])    # contraction over 2f
    dyc, hc, dguc, xc = t_qcol(dy, go), t_qcol(h, go), t_qcol(dgu, go), t_qcol(xq, go)
    dw13 = torch.zeros(E, 2 * f, d, dtype=torch.float64)
    dw2 = torch.zeros(E, d, f, dtype=torch.float64)
    for e in range(E):
        r0, r1 = int(go[e]), int(go[e + 1])
        dw2[e] = t_bf16(dyc[r0:r1].T @ hc[r0:r1])
        dw13[e] = t_bf16(dguc[r0:r1].T @ xc[r0:r1])
    return dict(xq=xq, w13f=w13f, w2f=w2f, w13b=w13b, w2b=w2b, gu=gu, h=h, y=y, dgu=dgu, dx=dx,
                dw13=dw13, dw2=dw2, dyq=dyq, dyc=dyc, hc=hc, xc=xc)


# ------------------------------------------------------------ inputs
def _inputs(seed=7, d=64, f=64, rs=3, cs=3):
    """Four experts with 45 / 0 / 33 / 70 rows (ragged last blocks of 13, 1
    and 6 rows; one empty group), bf16-valued operands whose rows and
    columns carry spread-out magnitudes so that blocks along different axes
    get different scales."""
    g = torch.Generator().manual_seed(seed)
    E = 4
    counts = [45, 0, 33, 70]
    go = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(go[-1])

    def bf(*shape, rowspread=0, colspread=0, scale=1.0):
        v = torch.randn(*shape, generator=g, dtype=torch.float64) * scale
        if rowspread:
            v = v * torch.ldexp(torch.ones(shape[-2], 1, dtype=torch.float64),
                                torch.randint(-rowspread, rowspread + 1, (shape[-2], 1), generator=g))
        if colspread:
            v = v * torch.ldexp(torch.ones(shape[-1], dtype=torch.float64),
                                torch.randint(-colspread, colspread + 1, (shape[-1],), generator=g))
        return t_bf16(v)

    x = bf(R, d, rowspread=rs, colspread=cs)
    w13 = bf(E, 2 * f, d, rowspread=rs, colspread=cs, scale=0.1)
    w2 = bf(E, d, f, rowspread=rs, colspread=cs, scale=0.1)
    dy = bf(R, d, rowspread=rs, colspread=cs)
    return x, w13, w2, dy, go


def _oracle_chain(o, x, w13, w2, dy, go, ref):
    """The oracle's composition as the GPU parity tests drive it: the caches
    and the substituted operands come from the oracle's own wrappers."""
    E, two_f, d = w13.shape
    f = two_f // 2
    n = lambda t: t.numpy()
    g13 = np.arange(E + 1, dtype=np.int32) * 2 * f
    g2 = np.arange(E + 1, dtype=np.int32) * d
    w13f = o.mx_qdq_rows(n(w13).reshape(-1, d)).reshape(E, 2 * f, d)
    w2f = o.mx_qdq_rows(n(w2).reshape(-1, f)).reshape(E, d, f)
    w13b = o.mx_qdq_cols(n(w13).reshape(-1, d), g13).reshape(E, 2 * f, d)
    w2b = o.mx_qdq_cols(n(w2).reshape(-1, f), g2).reshape(E, d, f)
    xq = o.mx_qdq_rows(n(x))
    gu, h, y = o.ffn_fwd(xq, w13f, w2f, go, o.BF16, mx_h=True)
    dgu, dx, dw13, dw2 = o.ffn_bwd(o.mx_qdq_rows(n(dy)), xq, gu, h, w13f, w2f, go, o.BF16,
                                   w2_dgrad=w2b, w13_dgrad=w13b,
                                   dy_wgrad=o.mx_qdq_cols(n(dy), go),
                                   h_wgrad=o.mx_qdq_cols(h, go),
                                   x_wgrad=o.mx_qdq_cols(xq, go), mx_dgu=True)
    return dict(xq=xq, w13f=w13f, w2f=w2f, w13b=w13b, w2b=w2b, gu=gu, h=h, y=y, dgu=dgu, dx=dx,
                dw13=dw13, dw2=dw2)


def _errors(got, ref, names):
    out = {}
    for k in names:
        r = ref[k].numpy() if torch.is_tensor(ref[k]) else ref[k]
        out[k] = float(np.abs(np.asarray(got[k]) - r).max() / max(np.abs(r).max(), 1e-300))
    return out


ALL = ["gu", "h", "y", "dgu", "dx", "dw13", "dw2"]


@pytest.fixture(scope="module")
def case():
    x, w13, w2, dy, go = _inputs()
    return x, w13, w2, dy, go, t_chain(x, w13, w2, dy, go)


# ------------------------------------------------------------ the pins
def test_torch_reference_codec_facts():
    """The reference quantiser itself against what the definition fixes: a
    block whose maximum is exactly 448 * 2^e keeps scale 2^e (so an element
    1.125 * 2^(e-6), the smallest normal E4M3 exponent with one mantissa bit,
    stays exact); a maximum of 480 * 2^e (above 448 * 2^e) moves the scale to
    2^(e+1), where 480 is still exact (240) but that element becomes
    subnormal and rounds (4.5 -> 4 units of 2^-9, ties to even); an all-zero
    block stays zero; relative error at most 2^-4 for normal elements."""
    for e in (-20, 0, 7):
        v = torch.zeros(1, 32, dtype=torch.float64)
        v[0, 3] = 448.0 * 2.0 ** e
        v[0, 5] = 1.125 * 2.0 ** (e - 6)
        q = t_mx_qdq_lastdim(v)
        assert q[0, 3] == v[0, 3] and q[0, 5] == v[0, 5]
        v[0, 3] = 480.0 * 2.0 ** e
        q = t_mx_qdq_lastdim(v)
        assert q[0, 3] == v[0, 3]
        assert q[0, 5] == 2.0 ** (e - 6)
    assert torch.all(t_mx_qdq_lastdim(torch.zeros(2, 64, dtype=torch.float64)) == 0)
    x = _inputs()[0]
    q = t_mx_qdq_lastdim(x)
    rel = ((q - x).abs() / x.abs().clamp_min(1e-30))[x.abs() > x.abs().max() * 2 ** -6]
    assert float(rel.max()) <= 2.0 ** -4


def test_bf16_rounding_reference():
    """The reference's bf16 rounding against exact ties and near-ties built
    from bit patterns (fp32 -> bf16 in torch is correctly rounded; the fp64
    path must agree with it on fp32 inputs and resolve fp64-only ties)."""
    g = torch.Generator().manual_seed(3)
    f32 = torch.randn(100000, generator=g, dtype=torch.float32)
    assert torch.equal(t_bf16(f32.to(torch.float64)), f32.to(torch.bfloat16).to(torch.float64))
    one = torch.tensor([1.0], dtype=torch.float64)
    half_ulp = 2.0 ** -8
    # 1 + half ulp is a tie -> even (1.0); a hair above must round up
    assert float(t_bf16(one + half_ulp)) == 1.0
    assert float(t_bf16(one + half_ulp + 2.0 ** -40)) == 1.0 + 2.0 ** -7
    assert float(t_bf16(-(one + half_ulp + 2.0 ** -40))) == -(1.0 + 2.0 ** -7)


def test_qdq_wrappers_match_reference(case):
    """oracle.mx_qdq_rows / mx_qdq_cols (what the GPU parity tests use to
    build the substituted operands) equal the reference quantiser exactly,
    row-wise and per group along the tokens with a ragged and an empty group."""
    x, w13, w2, dy, go, ref = case
    assert np.array_equal(oracle.mx_qdq_rows(x.numpy()), t_qrow(x).numpy())
    assert np.array_equal(oracle.mx_qdq_cols(dy.numpy(), go), t_qcol(dy, go).numpy())
    assert np.array_equal(oracle.mx_qdq_cols(ref["xq"].numpy(), go), ref["xc"].numpy())
    E, two_f, d = w13.shape
    g13 = np.arange(E + 1, dtype=np.int32) * two_f
    assert np.array_equal(oracle.mx_qdq_cols(w13.numpy().reshape(-1, d), g13),
                          ref["w13b"].numpy().reshape(-1, d))


def test_mx_composition_matches_reference(case):
    x, w13, w2, dy, go, ref = case
    got = _oracle_chain(oracle, x, w13, w2, dy, go, ref)
    errs = _errors(got, ref, ALL)
    assert all(v <= TOL for v in errs.values()), errs
    # the composition is not the unquantised layer: MX changes every output
    E, two_f, d = w13.shape
    f = two_f // 2
    gu0, h0, y0 = oracle.ffn_fwd(x.numpy(), w13.numpy(), w2.numpy(), go, oracle.BF16)
    assert np.abs(y0 - ref["y"].numpy()).max() > 100 * TOL * np.abs(y0).max()


def test_mx_empty_group_gradients_zero(case):
    x, w13, w2, dy, go, ref = case
    got = _oracle_chain(oracle, x, w13, w2, dy, go, ref)
    assert np.all(got["dw13"][1] == 0) and np.all(got["dw2"][1] == 0)


# ------------------------------------------------------------ operand probes
# With an identity matrix in the other operand's place a GEMM returns its
# MX operand unchanged (one product per output, exact in bf16 since an MX
# value has 4 significant bits), so the quantised copies the oracle forms
# inside ffn_fwd / ffn_bwd can be compared element for element with the
# reference quantiser applied to the tensors the oracle itself stored.
PD, PF = 256, 128          # d >= 2f and f >= every group's row count


def _eye_groups(E, rows, cols):
    w = torch.zeros(E, rows, cols, dtype=torch.float64)
    for e in range(E):
        w[e].fill_diagonal_(1.0)
    return w


def _probe(o):
    """Returns {name: number of elements differing from the reference}."""
    x, w13, w2, dy, go = _inputs(seed=11, d=PD, f=PF, rs=10, cs=4)
    E = w13.shape[0]
    d, f = PD, PF
    R = int(go[-1])
    n = lambda t: t.numpy() if torch.is_tensor(t) else t
    xq = t_qrow(x)
    w13f = t_qrow(w13.reshape(-1, d)).reshape(E, 2 * f, d)
    out = {}
    # forward: y = Q_rows(h) I  ->  y == Q_rows(h_stored)
    w2_eye = _eye_groups(E, d, f)
    gu, h, y = o.ffn_fwd(n(xq), n(w13f), n(w2_eye), go, o.BF16, mx_h=True)
    out["fwd_h_rowwise"] = int((y[:, :f] != t_qrow(torch.from_numpy(h)).numpy()).sum())
    # backward: dx = Q_rows(dgu) I ; dw13[e] = Q_cols(dgu)^T I_rows ; dw2[e] = dy_wgrad^T I_rows
    w13_eye = _eye_groups(E, 2 * f, d)
    x_onehot = torch.zeros(R, d, dtype=torch.float64)
    h_onehot = torch.zeros(R, f, dtype=torch.float64)
    for e in range(E):
        r0, r1 = int(go[e]), int(go[e + 1])
        for r in range(r0, r1):
            x_onehot[r, r - r0] = 1.0
            h_onehot[r, r - r0] = 1.0
    dyc = t_qcol(dy, go)
    dyq = t_qrow(dy)
    w2f = t_qrow(w2.reshape(-1, f)).reshape(E, d, f)
    # the activation gradient reads w2_dgrad (identity here), not the forward cache w2f
    dgu, dx, dw13, dw2 = o.ffn_bwd(n(dyq), n(xq), gu, h, n(w13f), n(w2f), go, o.BF16,
                                   w2_dgrad=n(w2_eye), w13_dgrad=n(w13_eye), dy_wgrad=n(dyc),
                                   h_wgrad=n(h_onehot), x_wgrad=n(x_onehot), mx_dgu=True)
    dgu_t = torch.from_numpy(dgu)
    g, u = torch.from_numpy(gu[:, :f]), torch.from_numpy(gu[:, f:])
    dh = dyq[:, :f]
    sg = torch.sigmoid(g)
    want = torch.cat([t_bf16(dh * u * sg * (1 + g * (1 - sg))), t_bf16(dh * g * sg)], 1)
    out["dgrad_w2_operand"] = int(((dgu_t - want).abs() > 1e-6 * want.abs()).sum())
    out["dgrad_dgu_rowwise"] = int((dx[:, :2 * f] != t_qrow(dgu_t).numpy()).sum())
    dguc = t_qcol(dgu_t, go).numpy()
    bad13 = bad2 = 0
    for e in range(E):
        r0, r1 = int(go[e]), int(go[e + 1])
        m = r1 - r0
        bad13 += int((dw13[e][:, :m].T != dguc[r0:r1]).sum()) + int((dw13[e][:, m:] != 0).sum())
        bad2 += int((dw2[e][:, :m].T != dyc[r0:r1].numpy()).sum()) + int((dw2[e][:, m:] != 0).sum())
    out["wgrad_dgu_colwise"] = bad13
    out["wgrad_dy_operand"] = bad2
    return out


def test_mx_operand_copies_exact():
    """The quantised copies inside the oracle's MX composition equal the
    reference quantiser of the stored tensors, element for element: h along
    f for the down GEMM, dgu along 2f for the activation gradient, dgu along
    the tokens of each group (blocks restarting at the group's first row) for
    the weight gradient, and the caller's dy copy for dWd."""
    bad = _probe(oracle)
    assert all(v == 0 for v in bad.values()), bad


# ------------------------------------------------------------ planted mistakes
PLANTS = {
    # the down GEMM's h blocks along the rows (wrong axis) instead of along f
    "h_wrong_axis": (
        "for (long r = 0; r < n_rows; ++r) mx_qdq_vector(h + r * f, f, 1, hq + r * f, 1);",
        "for (long n = 0; n < f; ++n) mx_qdq_vector(h + n, n_rows, f, hq + n, f);"),
    # weight-gradient dgu blocks start one row after each group's first row
    "dgu_cols_shifted": (
        "mx_qdq_vector(dgu + r0 * 2 * f + n, m, 2 * f, dgu_w + r0 * 2 * f + n, 2 * f);",
        "if (m > 0) { mx_qdq_vector(dgu + r0 * 2 * f + n, 1, 2 * f, dgu_w + r0 * 2 * f + n, 2 * f);"
        " mx_qdq_vector(dgu + (r0 + 1) * 2 * f + n, m - 1, 2 * f, dgu_w + (r0 + 1) * 2 * f + n,"
        " 2 * f); }"),
    # weight-gradient dgu blocks run over all rows, ignoring group starts
    "dgu_cols_ungrouped": (
        "for (int e = 0; e < E; ++e) {\n            long r0 = group_off[e], m = group_off[e + 1] - group_off[e];",
        "for (int e = 0; e < 1; ++e) {\n            long r0 = 0, m = n_rows;"),
    # dx reads the stored dgu instead of its row-wise MX copy
    "dx_reads_stored_dgu": ("dgu_g = dgu_q;", "dgu_g = dgu;"),
    # the weight gradient reads the row-wise copy instead of the column-wise one
    "wgrad_reads_rowwise_dgu": ("dgu_wg = dgu_w;", "dgu_wg = dgu_q;"),
    # the activation gradient of the down GEMM reads the forward weight cache
    "dgrad_reads_forward_cache": ("const double* wd = w2_dgrad + (long)e * d * f;",
                                  "const double* wd = w2 + (long)e * d * f;"),
    # dW13 reads the row-wise dispatch payload instead of its column-wise copy
    "wgrad_reads_rowwise_x": ("acc += dgu_wg[r * 2 * f + n] * x_wgrad[r * d + i];",
                              "acc += dgu_wg[r * 2 * f + n] * x_perm[r * d + i];"),
    # dWd reads the stored dy instead of the caller's column-wise copy
    "wgrad_reads_stored_dy": ("acc += dy_wgrad[r * d + i] * h_wgrad[r * f + n];",
                              "acc += dy_perm[r * d + i] * h_wgrad[r * f + n];"),
}


@pytest.fixture(scope="module")
def planted_libs(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = open(SRC).read()
    out = {}
    d = tmp_path_factory.mktemp("planted")
    for name, (old, new) in PLANTS.items():
        assert src.count(old) == 1, f"plant {name}: anchor not found once in the oracle source"
        c = d / f"{name}.c"
        c.write_text(src.replace(old, new))
        so = d / f"{name}.so"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-std=c11", "-shared", "-fPIC", str(c),
                               "-o", str(so), "-lm"])
        out[name] = oracle.open_library(str(so))
    return out


@pytest.mark.parametrize("plant", sorted(PLANTS))
def test_planted_mistake_is_caught(case, planted_libs, plant, monkeypatch):
    """Every planted mistake fails the chain comparison (by far more than its
    tolerance) or the exact operand probes."""
    x, w13, w2, dy, go, ref = case
    monkeypatch.setattr(oracle, "_lib", planted_libs[plant])
    got = _oracle_chain(oracle, x, w13, w2, dy, go, ref)
    errs = _errors(got, ref, ALL)
    bad = _probe(oracle)
    assert max(errs.values()) > 1e3 * TOL or any(v > 0 for v in bad.values()), \
        f"planted mistake {plant} not caught: {errs} {bad}"
