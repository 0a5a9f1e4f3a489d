"""Pins for the oracle's router scores and its gradient through the gate weights.

The router scores are pinned by closed forms (one-hot tokens read out a weight
column), linearity, and the fp32 storage rounding; the gate gradient by central
finite differences of the layer output's inner product with dout (computed here
from a softmax written independently, in fp64), a hand-derived closed form for
k = 2, and the invariants of a softmax Jacobian (rows sum to zero, k = 1 gives
zero, experts not selected get zero, dropped slots contribute nothing).
"""
import numpy as np
import pytest


def test_router_logits_one_hot_tokens_read_weight_columns(oracle_lib):
    rng = np.random.default_rng(1)
    E, d = 6, 10
    w = rng.standard_normal((E, d))
    x = np.eye(d)                                   # token t = unit vector e_t
    lg = oracle_lib.router_logits(x, w, oracle_lib.NONE)
    np.testing.assert_array_equal(lg, w.T)


def test_router_logits_linear_and_fp32_rounded(oracle_lib):
    rng = np.random.default_rng(2)
    T, E, d = 9, 5, 33
    w = rng.standard_normal((E, d))
    x1, x2 = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    a, b = 0.75, -2.5
    l1 = oracle_lib.router_logits(x1, w, oracle_lib.NONE)
    l2 = oracle_lib.router_logits(x2, w, oracle_lib.NONE)
    l12 = oracle_lib.router_logits(a * x1 + b * x2, w, oracle_lib.NONE)
    np.testing.assert_allclose(l12, a * l1 + b * l2, rtol=1e-12, atol=1e-12)
    # stored scores are the fp64 sums rounded once to fp32
    f = oracle_lib.router_logits(x1, w, oracle_lib.FP32)
    np.testing.assert_array_equal(f, l1.astype(np.float32).astype(np.float64))


def _setup(T, E, k, d, seed, capacity=0):
    import oracle
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    r = oracle.route(logits, k, capacity=capacity)
    y = rng.standard_normal((r["n_rows"], d))
    dout = rng.standard_normal((T, d))
    return logits, r, y, dout


def _loss(logits_sel, r, y, dout, k):
    # sum_t <dout[t], out[t]>, out[t] = sum_j softmax(selected logits)_j * y[dst], fp64
    T = dout.shape[0]
    total = 0.0
    for t in range(T):
        l = logits_sel[t]
        e = np.exp(l - l.max())
        w = e / e.sum()
        for j in range(k):
            dst = r["dst_row"][t * k + j]
            if dst >= 0:
                total += w[j] * float(dout[t] @ y[dst])
    return total


@pytest.mark.parametrize("T,E,k,d,C", [(6, 5, 3, 7, 0), (8, 4, 2, 5, 0), (10, 3, 2, 4, 3)])
def test_gate_grad_matches_finite_differences(oracle_lib, T, E, k, d, C):
    logits, r, y, dout = _setup(T, E, k, d, seed=T + E + k, capacity=C)
    sel = np.take_along_axis(logits.astype(np.float64), r["topk_idx"].astype(np.int64), axis=1)
    # gate weights as the layer holds them (fp32), from the same selected logits
    dw, dl = oracle_lib.gate_grad(dout, y, r["dst_row"], r["topk_idx"], r["topk_w"], E,
                                  round_mode=oracle_lib.NONE)
    h = 1e-6
    for t in range(T):
        for j in range(k):
            lp, lm = sel.copy(), sel.copy()
            lp[t, j] += h
            lm[t, j] -= h
            fd = (_loss(lp, r, y, dout, k) - _loss(lm, r, y, dout, k)) / (2 * h)
            assert abs(dl[t, r["topk_idx"][t, j]] - fd) <= 1e-5 * (1 + abs(fd)), (t, j)
    # dw: the output is linear in each gate weight
    for t in range(T):
        for j in range(k):
            dst = r["dst_row"][t * k + j]
            expect = 0.0 if dst < 0 else float(np.dot(dout[t], y[dst]))
            assert abs(dw[t, j] - expect) <= 1e-12 * (1 + abs(expect))
    if C:
        assert (r["dst_row"] < 0).any(), "the padded case drops some pairs"


def test_gate_grad_k2_closed_form_and_invariants(oracle_lib):
    T, E, k, d = 12, 6, 2, 9
    logits, r, y, dout = _setup(T, E, k, d, seed=3)
    dw, dl = oracle_lib.gate_grad(dout, y, r["dst_row"], r["topk_idx"], r["topk_w"], E,
                                  round_mode=oracle_lib.NONE)
    w = r["topk_w"].astype(np.float64)
    # the fp32 gate weights sum to one only to within fp32 rounding, which
    # bounds how far the exact closed forms below can be off
    for t in range(T):
        e0, e1 = r["topk_idx"][t]
        # k = 2: dl_0 = w0 w1 (dw0 - dw1) = -dl_1
        c = w[t, 0] * w[t, 1] * (dw[t, 0] - dw[t, 1])
        scale = 1e-6 * (abs(dw[t, 0]) + abs(dw[t, 1]))
        assert abs(dl[t, e0] - c) <= scale
        assert abs(dl[t, e1] + c) <= scale
        others = [e for e in range(E) if e not in (e0, e1)]
        assert np.all(dl[t, others] == 0.0)
        assert abs(dl[t].sum()) <= scale


def test_gate_grad_top1_is_zero(oracle_lib):
    logits, r, y, dout = _setup(7, 4, 1, 5, seed=4)
    dw, dl = oracle_lib.gate_grad(dout, y, r["dst_row"], r["topk_idx"], r["topk_w"], 4)
    assert np.all(dl == 0.0)
    assert np.any(dw != 0.0)
