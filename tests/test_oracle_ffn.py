"""Pins for the oracle's permute, combine and grouped SwiGLU FFN (fwd + bwd).

Cross-checks: a dense SwiGLU FFN in torch float64 (E=1, k=1), brute-force
per-token evaluation of the routed layer in torch float64, torch.autograd
for the backward, central finite differences, and closed-form properties of
permute/combine.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import moe_synth


def _layer_inputs(T, d, E, f, k, seed):
    inp = moe_synth.make_inputs(T=T, d=d, E=E, f=f, k=k, seed=seed, act_dtype=torch.float64)
    # std 0.02 weights give tiny outputs; scale up so the checks are not trivially small
    inp["w13"] *= 10
    inp["w2"] *= 10
    inp["x"] *= 20
    return inp


def _oracle_layer(o, inp, k, capacity=0, mode=0):
    x = inp["x"].numpy()
    T = x.shape[0]
    r = o.route(inp["logits"].numpy(), k, capacity)
    go = o.group_offsets(r["offsets"], capacity)
    xp = o.permute(x, r["dst_row"], k, r["n_rows"], round_mode=mode)
    gu, h, y = o.ffn_fwd(xp, inp["w13"].numpy(), inp["w2"].numpy(), go, round_mode=mode)
    out = o.combine(y, r["dst_row"], r["topk_w"], T, k, round_mode=mode)
    return r, go, xp, gu, h, y, out


def _torch_expert(x, w13, w2, e, f):
    g = x @ w13[e, :f].T
    u = x @ w13[e, f:].T
    return (F.silu(g) * u) @ w2[e].T


def test_dense_reduction_e1_top1(oracle_lib):
    T, d, f = 37, 24, 40
    inp = _layer_inputs(T, d, 1, f, 1, seed=21)
    *_, out = _oracle_layer(oracle_lib, inp, 1)
    ref = _torch_expert(inp["x"], inp["w13"], inp["w2"], 0, f)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("T,d,E,f,k", [(29, 16, 4, 24, 2), (40, 8, 6, 16, 3)])
def test_brute_force_per_token(oracle_lib, T, d, E, f, k):
    inp = _layer_inputs(T, d, E, f, k, seed=T + E)
    r, *_, out = _oracle_layer(oracle_lib, inp, k)
    x, w13, w2 = inp["x"], inp["w13"], inp["w2"]
    for t in range(T):
        ref = torch.zeros(d, dtype=torch.float64)
        for j in range(k):
            e = int(r["topk_idx"][t, j])
            ref += float(r["topk_w"][t, j]) * _torch_expert(x[t:t + 1], w13, w2, e, f)[0]
        np.testing.assert_allclose(out[t], ref.numpy(), rtol=1e-11, atol=1e-13)


def test_saved_tensors_match_definition(oracle_lib):
    T, d, E, f, k = 20, 16, 3, 24, 2
    inp = _layer_inputs(T, d, E, f, k, seed=4)
    r, go, xp, gu, h, y, _ = _oracle_layer(oracle_lib, inp, k)
    w13 = inp["w13"].numpy()
    for e in range(E):
        rows = slice(go[e], go[e + 1])
        g = xp[rows] @ w13[e, :f].T
        u = xp[rows] @ w13[e, f:].T
        np.testing.assert_allclose(gu[rows, :f], g, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(gu[rows, f:], u, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(h[rows], g / (1 + np.exp(-g)) * u, rtol=1e-12, atol=1e-14)


def test_backward_matches_autograd(oracle_lib):
    T, d, E, f, k = 24, 16, 4, 20, 2
    inp = _layer_inputs(T, d, E, f, k, seed=9)
    o = oracle_lib
    r, go, xp, gu, h, y, out = _oracle_layer(o, inp, k)
    dout = inp["dout"].numpy()
    dy = o.permute(dout, r["dst_row"], k, r["n_rows"], row_scale=r["topk_w"])
    dgu, dxp, dw13, dw2 = o.ffn_bwd(dy, xp, gu, h, inp["w13"].numpy(), inp["w2"].numpy(), go)
    dx = o.combine(dxp, r["dst_row"], None, T, k)

    x = inp["x"].clone().requires_grad_(True)
    w13 = inp["w13"].clone().requires_grad_(True)
    w2 = inp["w2"].clone().requires_grad_(True)
    ref = torch.zeros(T, d, dtype=torch.float64)
    for t in range(T):
        for j in range(k):
            e = int(r["topk_idx"][t, j])
            ref[t] += float(r["topk_w"][t, j]) * _torch_expert(x[t:t + 1], w13, w2, e, f)[0]
    (ref * inp["dout"]).sum().backward()
    np.testing.assert_allclose(out, ref.detach().numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(dx, x.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dw13, w13.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dw2, w2.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_backward_central_finite_difference(oracle_lib):
    T, d, E, f, k = 12, 8, 3, 8, 2
    inp = _layer_inputs(T, d, E, f, k, seed=31)
    o = oracle_lib
    r, go, xp, gu, h, y, out = _oracle_layer(o, inp, k)
    dout = inp["dout"].numpy()
    dy = o.permute(dout, r["dst_row"], k, r["n_rows"], row_scale=r["topk_w"])
    _, dxp, dw13, dw2 = o.ffn_bwd(dy, xp, gu, h, inp["w13"].numpy(), inp["w2"].numpy(), go)
    dx = o.combine(dxp, r["dst_row"], None, T, k)

    def loss(x, w13, w2):
        xp2 = o.permute(x, r["dst_row"], k, r["n_rows"])
        _, _, y2 = o.ffn_fwd(xp2, w13, w2, go)
        return float((o.combine(y2, r["dst_row"], r["topk_w"], T, k) * dout).sum())

    base = [inp["x"].numpy().copy(), inp["w13"].numpy().copy(), inp["w2"].numpy().copy()]
    eps = 1e-6
    for which, grad, pos in [(0, dx, (3, 5)), (1, dw13, (1, 2, 4)), (1, dw13, (2, 11, 0)),
                             (2, dw2, (0, 7, 6)), (2, dw2, (2, 1, 3))]:
        plus = [a.copy() for a in base]
        minus = [a.copy() for a in base]
        plus[which][pos] += eps
        minus[which][pos] -= eps
        fd = (loss(*plus) - loss(*minus)) / (2 * eps)
        assert abs(fd - grad[pos]) <= 1e-6 * max(1.0, abs(fd)), (which, pos, fd, grad[pos])


def test_empty_expert_gets_zero_weight_gradient(oracle_lib):
    T, d, E, f, k = 16, 8, 5, 8, 2
    inp = _layer_inputs(T, d, E, f, k, seed=2)
    inp["logits"][:, 4] = -100.0                          # nobody picks expert 4
    o = oracle_lib
    r, go, xp, gu, h, y, out = _oracle_layer(o, inp, k)
    assert r["counts"][4] == 0
    dy = o.permute(inp["dout"].numpy(), r["dst_row"], k, r["n_rows"], row_scale=r["topk_w"])
    _, _, dw13, dw2 = o.ffn_bwd(dy, xp, gu, h, inp["w13"].numpy(), inp["w2"].numpy(), go)
    assert np.all(dw13[4] == 0) and np.all(dw2[4] == 0)


def test_padded_large_capacity_equals_unpadded(oracle_lib):
    T, d, E, f, k = 30, 16, 4, 16, 2
    inp = _layer_inputs(T, d, E, f, k, seed=8)
    r, *_, out = _oracle_layer(oracle_lib, inp, k)
    C = int(r["counts"].max()) + 2
    rp, gop, xpp, gup, hp, yp, outp = _oracle_layer(oracle_lib, inp, k, capacity=C)
    np.testing.assert_allclose(outp, out, rtol=1e-13, atol=1e-15)
    # padding rows are zero in and out
    pad = rp["src_slot"] < 0
    assert np.all(xpp[pad] == 0) and np.all(yp[pad] == 0)


def test_padded_drops_contribute_zero(oracle_lib):
    T, d, E, f, k = 40, 8, 4, 8, 2
    inp = _layer_inputs(T, d, E, f, k, seed=12)
    inp["logits"][:, 1] += 3.0
    C = 8
    rp, gop, xpp, gup, hp, yp, outp = _oracle_layer(oracle_lib, inp, k, capacity=C)
    x, w13, w2 = inp["x"], inp["w13"], inp["w2"]
    for t in range(T):
        ref = torch.zeros(d, dtype=torch.float64)
        for j in range(k):
            if rp["dst_row"][t * k + j] < 0:
                continue
            e = int(rp["topk_idx"][t, j])
            ref += float(rp["topk_w"][t, j]) * _torch_expert(x[t:t + 1], w13, w2, e, f)[0]
        np.testing.assert_allclose(outp[t], ref.numpy(), rtol=1e-11, atol=1e-13)


def test_permute_is_exact_copy_and_combine_identities(oracle_lib):
    T, d, E, k = 50, 12, 6, 3
    o = oracle_lib
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    x = rng.standard_normal((T, d))
    r = o.route(logits, k)
    xp = o.permute(x, r["dst_row"], k, r["n_rows"])
    np.testing.assert_array_equal(xp[r["dst_row"]], np.repeat(x, k, axis=0))
    # unweighted combine of the permuted rows is k * x; weighted (sum w = 1) is x
    np.testing.assert_allclose(o.combine(xp, r["dst_row"], None, T, k), k * x, rtol=1e-15)
    np.testing.assert_allclose(o.combine(xp, r["dst_row"], r["topk_w"], T, k), x, rtol=1e-6)
    # one-hot weights select one slot exactly
    oh = np.zeros((T, k), np.float32)
    oh[:, 1] = 1.0
    y = rng.standard_normal((T * k, d))
    np.testing.assert_array_equal(o.combine(y, r["dst_row"], oh, T, k),
                                  y[r["dst_row"].reshape(T, k)[:, 1]])
    # numpy fancy-index brute force of the weighted sum
    w = r["topk_w"].astype(np.float64)
    ref = (w[:, :, None] * y[r["dst_row"].reshape(T, k)]).sum(1)
    np.testing.assert_allclose(o.combine(y, r["dst_row"], r["topk_w"], T, k), ref, rtol=1e-14,
                               atol=1e-15)


def test_bf16_storage_rounding_points(oracle_lib):
    T, d, E, f, k = 32, 16, 4, 16, 2
    inp = _layer_inputs(T, d, E, f, k, seed=44)
    o = oracle_lib
    exact = _oracle_layer(o, inp, k, mode=o.NONE)
    rounded = _oracle_layer(o, inp, k, mode=o.BF16)
    for a, b in zip(exact[3:], rounded[3:]):          # gu, h, y, out
        np.testing.assert_array_equal(o.round_(b, o.BF16), b)   # representable in bf16
        scale = np.abs(a).max()
        assert np.abs(a - b).max() <= 2 ** -7 * scale * 4


@pytest.mark.parametrize("S,C", [(1, 0), (2, 0), (1, 40)])
def test_shared_experts_add_a_dense_ffn(oracle_lib, S, C):
    # a shared expert is an ungated expert every token uses: the layer with
    # shared experts equals the routed layer plus, per shared expert, the
    # dense SwiGLU FFN of x with that expert's weights (fp64, no rounding)
    import moe_synth
    from tests._chain import np64, oracle_layer, oracle_layer_shared
    T, d, E, f, k = 48, 16, 4, 24, 2
    inp = moe_synth.make_inputs(T=T, d=d, E=E + S, f=f, k=k, dtype="f32", seed=11 + S)
    inp["logits"] = inp["logits"][:, :E].contiguous()
    full = oracle_layer_shared(inp, k, S, capacity=C, round_mode=oracle_lib.NONE, bwd=False)
    routed_inp = dict(inp, w13=inp["w13"][:E], w2=inp["w2"][:E])
    routed = oracle_layer(routed_inp, k, capacity=C, round_mode=oracle_lib.NONE, bwd=False)
    x = np64(inp["x"])
    dense = np.zeros_like(x)
    for s_ in range(S):
        w13 = np64(inp["w13"][E + s_:E + s_ + 1])
        w2 = np64(inp["w2"][E + s_:E + s_ + 1])
        dense += oracle_lib.ffn_fwd(x, w13, w2, np.array([0, T], np.int32), oracle_lib.NONE)[2]
    np.testing.assert_allclose(full["out"], routed["out"] + dense, rtol=1e-12, atol=1e-14)


def test_shared_experts_equal_one_wider_expert(oracle_lib):
    # several ungated shared experts act as one expert of their summed width:
    # SwiGLU is elementwise over the hidden units and the down projection sums
    # over them, so S experts of width f equal one of width S*f whose gate
    # rows, up rows and down columns are the S experts' stacked (fp64, exact
    # up to summation order)
    import moe_synth
    from tests._chain import np64, oracle_layer_shared
    T, d, E, f, k, S = 40, 16, 4, 12, 2, 3
    inp = moe_synth.make_inputs(T=T, d=d, E=E + S, f=f, k=k, dtype="f32", seed=29)
    inp["logits"] = inp["logits"][:, :E].contiguous()
    full = oracle_layer_shared(inp, k, S, round_mode=oracle_lib.NONE, bwd=False)
    w13, w2 = np64(inp["w13"]), np64(inp["w2"])
    gate = np.concatenate([w13[E + s, :f] for s in range(S)])      # [S*f, d]
    up = np.concatenate([w13[E + s, f:] for s in range(S)])
    wide13 = np.concatenate([gate, up])[None]                      # [1, 2*S*f, d]
    wide2 = np.concatenate([w2[E + s] for s in range(S)], axis=1)[None]   # [1, d, S*f]
    x = np64(inp["x"])
    wide = oracle_lib.ffn_fwd(x, wide13, wide2, np.array([0, T], np.int32), oracle_lib.NONE)[2]
    # the routed part: the layer with the shared experts' outputs taken away
    y = full["y_perm"]
    R = full["route"]["n_rows"]
    routed_part = full["out"] - sum(y[R + s * T:R + (s + 1) * T] for s in range(S))
    scale = np.abs(wide).max()
    assert scale > 0, "the wide expert's output is not the trivial zero"
    np.testing.assert_allclose(routed_part + wide, full["out"], rtol=1e-12, atol=1e-12 * scale)
