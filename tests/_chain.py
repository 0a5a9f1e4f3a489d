"""Test helpers: the oracle's chain of the layer, and tensor comparison.

Only the oracle is called here (never the HIP library); inputs come from
moe_synth.  The oracle's outputs model the stored dtype of each tensor
(round_mode), so they are comparable element by element with the GPU's.
"""
import numpy as np
import torch

import oracle

BF16_TOL = 2e-2     # max|gpu - ref| <= BF16_TOL * max|ref|  (bf16 storage, fp32 accumulate)
F32_TOL = 1e-4      # fp32 storage and accumulate, K <= a few thousand


def np64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def oracle_layer(inp, k, capacity=0, round_mode=oracle.BF16, bwd=True, weights=None):
    """Route, permute, grouped SwiGLU FFN, combine (and the backward) on the CPU."""
    logits = inp["logits"].detach().cpu().numpy()
    T = logits.shape[0]
    r = oracle.route(logits, k, capacity)
    go = oracle.group_offsets(r["offsets"], capacity)
    w = r["topk_w"] if weights is None else np.asarray(weights, np.float32).reshape(T, k)
    x, w13, w2 = np64(inp["x"]), np64(inp["w13"]), np64(inp["w2"])
    xp = oracle.permute(x, r["dst_row"], k, r["n_rows"])
    gu, h, y = oracle.ffn_fwd(xp, w13, w2, go, round_mode)
    out = oracle.combine(y, r["dst_row"], w, T, k, round_mode)
    res = dict(route=r, go=go, x_perm=xp, gu=gu, h=h, y_perm=y, out=out, w=w)
    if bwd:
        dout = np64(inp["dout"])
        dy = oracle.permute(dout, r["dst_row"], k, r["n_rows"], row_scale=w, round_mode=round_mode)
        dgu, dxp, dw13, dw2 = oracle.ffn_bwd(dy, xp, gu, h, w13, w2, go, round_mode)
        dx = oracle.combine(dxp, r["dst_row"], None, T, k, round_mode)
        res.update(dy_perm=dy, dgu=dgu, dx_perm=dxp, dw13=dw13, dw2=dw2, dx=dx)
    return res


def widen_route(r, k, n_shared, capacity=0):
    """The oracle route r widened by n_shared shared experts: slot k+s of token
    t goes to row R + s*T + t with weight 1, the shared groups after the routed
    ones.  Returns dst [T*(k+S)], w [T, k+S], group offsets [E+S+1] and
    src [R+S*T] (the slot of each row, -1 for padding)."""
    S, K = n_shared, k + n_shared
    T = r["topk_idx"].shape[0]
    R = r["n_rows"]
    dst = np.empty((T, K), np.int32)
    dst[:, :k] = r["dst_row"].reshape(T, k)
    w = np.ones((T, K), np.float32)
    w[:, :k] = r["topk_w"]
    for s_ in range(S):
        dst[:, k + s_] = R + s_ * T + np.arange(T)
    dst = dst.reshape(-1)
    go = np.concatenate([oracle.group_offsets(r["offsets"], capacity),
                         R + T * np.arange(1, S + 1)]).astype(np.int32)
    src = -np.ones(R + S * T, np.int32)
    live = dst >= 0
    src[dst[live]] = np.nonzero(live)[0]
    return dst, w, go, src


def oracle_layer_shared(inp, k, n_shared, capacity=0, round_mode=oracle.BF16, bwd=True):
    """The layer with n_shared shared experts, read as ungated extra experts
    E .. E+n_shared-1 that every token uses with weight 1 (inp["w13"], inp["w2"]
    hold E + n_shared experts, the shared ones last): the oracle's own route,
    then its permute / FFN / combine over the k + n_shared slots of each token,
    the shared rows after the routed ones (row R + s*T + t)."""
    logits = inp["logits"].detach().cpu().numpy()
    T = logits.shape[0]
    S, K = n_shared, k + n_shared
    r = oracle.route(logits, k, capacity)
    dst, w, go, _ = widen_route(r, k, S, capacity)
    n = int(go[-1])
    x, w13, w2 = np64(inp["x"]), np64(inp["w13"]), np64(inp["w2"])
    xp = oracle.permute(x, dst, K, n)
    gu, h, y = oracle.ffn_fwd(xp, w13, w2, go, round_mode)
    out = oracle.combine(y, dst, w, T, K, round_mode)
    res = dict(route=r, dst=dst, w=w, go=go, x_perm=xp, gu=gu, h=h, y_perm=y, out=out)
    if bwd:
        dout = np64(inp["dout"])
        dy = oracle.permute(dout, dst, K, n, row_scale=w, round_mode=round_mode)
        dgu, dxp, dw13, dw2 = oracle.ffn_bwd(dy, xp, gu, h, w13, w2, go, round_mode)
        dx = oracle.combine(dxp, dst, None, T, K, round_mode)
        res.update(dy_perm=dy, dgu=dgu, dx_perm=dxp, dw13=dw13, dw2=dw2, dx=dx)
    return res


def rel_err(gpu, ref):
    """max|gpu - ref| / max|ref| (0 for empty tensors)."""
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    if r.size == 0:
        return 0.0
    scale = np.abs(r).max()
    err = np.abs(g - r).max()
    if scale == 0:
        return float(err)
    return float(err / scale)


def assert_close(gpu, ref, tol, name=""):
    g = np.asarray(gpu, np.float64)
    assert np.all(np.isfinite(g)), f"{name}: non-finite values"
    e = rel_err(g, ref)
    assert e <= tol, f"{name}: max|gpu-ref|/max|ref| = {e:.3e} > {tol:.1e}"
    return e
