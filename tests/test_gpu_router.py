"""GPU parity of the router scores and of the gradient through the gate weights.

Both accumulate bf16 products in fp32.  The products of two bf16 values are
exact in fp32, so in any summation order the error of a sum of n products is
at most n * 2^-24 * sum |products| (plus the final rounding); the tests check
every element against that bound computed from the inputs, with the oracle's
fp64 sums as the reference.  The zero pattern of dlogits (experts not
selected) and the fused combine backward (against moe_permute with the same
row scale) are checked bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

import moe_synth
import oracle
from tests._chain import np64

pytestmark = pytest.mark.gpu

DEV = "cuda"
U = 2.0 ** -24


def _say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def moe():
    import routing_grouped_gemm_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.load()
    return m


def _check_sum_bound(gpu, ref, abs_terms, n, name):
    # |gpu - ref| <= n * u * sum|terms| + u * |ref| (fp32 summation of exact products)
    bound = n * U * abs_terms + U * np.abs(ref) + 1e-30
    err = np.abs(gpu - ref)
    worst = np.max(err / bound)
    assert worst <= 1.0, f"{name}: error {err.max():.3e} exceeds the fp32 summation bound (x{worst:.2f})"


ROUTER_CASES = [
    # T, E, d
    (300, 128, 256),
    (200, 8, 200),      # d not a multiple of 64 (K tail)
    (130, 300, 128),    # two 256-expert tiles, the second ragged
    (97, 5, 64),        # E % 4 != 0 (scalar stores)
]


@pytest.mark.parametrize("T,E,d", ROUTER_CASES)
def test_router_logits_parity(moe, T, E, d):
    _say("router", T, E, d)
    inp = moe_synth.make_inputs(T=T, d=d, E=E, f=64, k=1, seed=T + E + d)
    x, w = inp["x"].to(DEV), inp["w_router"].to(DEV)
    lg = torch.empty(T, E, dtype=torch.float32, device=DEV)
    moe.moe_router_logits(x, w, lg)
    torch.cuda.synchronize()
    xr, wr = np64(inp["x"]), np64(inp["w_router"])
    ref = oracle.router_logits(xr, wr, oracle.NONE)
    _check_sum_bound(np64(lg), ref, np.abs(xr) @ np.abs(wr).T, d, "logits")


def test_router_logits_full_size_sampled_rows(moe):
    # e128: T = 16384 tokens, d = 4096, E = 128; rows checked: a sample spread over all tiles
    _say("router-e128")
    cfg = moe_synth.WORKLOADS["e128"]
    inp = moe_synth.make_inputs("e128", device=DEV)
    T, E, d = cfg["T"], cfg["E"], cfg["d"]
    lg = torch.empty(T, E, dtype=torch.float32, device=DEV)
    moe.moe_router_logits(inp["x"], inp["w_router"], lg)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, T, 257), [T - 1]]))
    xr = np64(inp["x"][rows])
    wr = np64(inp["w_router"])
    ref = oracle.router_logits(xr, wr, oracle.NONE)
    _check_sum_bound(np64(lg[rows]), ref, np.abs(xr) @ np.abs(wr).T, d, "logits")
    # the scores are about N(0, 1), as the routing workloads draw them
    assert 0.5 < float(lg.std()) < 2.0


def _gate_case(m, T, d, E, k, C, seed, fuse):
    inp = moe_synth.make_inputs(T=T, d=d, E=E, f=64, k=k, seed=seed)
    logits = inp["logits"].to(DEV)
    n_rows = E * C if C else T * k
    i32 = dict(dtype=torch.int32, device=DEV)
    r = dict(topk_idx=torch.empty(T, k, **i32), topk_w=torch.empty(T, k, dtype=torch.float32, device=DEV),
             counts=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
             dst_row=torch.empty(T * k, **i32), src_slot=torch.empty(n_rows, **i32))
    ws = torch.empty(m.moe_route_workspace_bytes(T, E, k), dtype=torch.uint8, device=DEV)
    m.moe_route_topk(logits, k, C, r["topk_idx"], r["topk_w"], r["counts"], r["offsets"], r["dst_row"],
                     r["src_slot"], ws)
    y = moe_synth.normal((n_rows, d), 0.05, seed + 11, DEV, torch.bfloat16)
    dout = inp["dout"].to(DEV)
    dl = torch.empty(T, E, dtype=torch.float32, device=DEV)
    dw = torch.empty(T, k, dtype=torch.float32, device=DEV)
    dyp = torch.empty(n_rows, d, dtype=torch.bfloat16, device=DEV) if fuse else None
    err = torch.zeros(1, **i32)
    m.moe_gate_grad(dout, y, r["topk_idx"], r["topk_w"], r["dst_row"], dl, dw=dw, dy_perm=dyp, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    return inp, r, y, dout, dl, dw, dyp


def _check_gate(r, y, dout, dl, dw, E, k, d, rows=None):
    idx = r["topk_idx"].cpu().numpy()
    w = r["topk_w"].cpu().numpy()
    dst = r["dst_row"].cpu().numpy().reshape(-1, k)
    T = idx.shape[0]
    toks = np.arange(T) if rows is None else rows
    # the rows of y the sampled tokens read, renumbered (keeps the oracle's input small)
    used = np.unique(dst[toks][dst[toks] >= 0])
    remap = -np.ones(max(int(y.shape[0]), 1), np.int64)
    remap[used] = np.arange(used.size)
    sub_dst = np.where(dst[toks] >= 0, remap[np.maximum(dst[toks], 0)], -1).astype(np.int32).reshape(-1)
    yr = np64(y[torch.as_tensor(used, device=y.device)]) if used.size else np.zeros((1, d))
    gr = np64(dout[torch.as_tensor(toks, device=dout.device)])
    ref_dw, ref_dl = oracle.gate_grad(gr, yr, sub_dst, idx[toks], w[toks], E, round_mode=oracle.NONE)
    # per-slot bound on dw from the products it sums
    e_dw = np.zeros((toks.size, k))
    for j in range(k):
        rr = sub_dst.reshape(-1, k)[:, j]
        ok = rr >= 0
        e_dw[ok, j] = d * U * np.sum(np.abs(gr[ok] * yr[rr[ok]]), axis=1)
    dwg = dw.cpu().numpy().astype(np.float64)[toks]
    assert np.all(np.abs(dwg - ref_dw) <= e_dw + U * np.abs(ref_dw) + 1e-30), "dw"
    dlg = dl.cpu().numpy().astype(np.float64)[toks]
    # dl_j = w_j (dw_j - sum_m w_m dw_m): each dw error enters at most twice (w <= 1)
    bound = 2 * e_dw.max(axis=1, keepdims=True) * k + 4 * U * np.abs(ref_dl) + 1e-30
    sel = np.zeros_like(dlg, dtype=bool)
    sel[np.arange(toks.size)[:, None], idx[toks]] = True
    assert np.all(np.abs(dlg - ref_dl)[sel] <= np.broadcast_to(bound, dlg.shape)[sel]), "dlogits"
    assert np.all(dlg[~sel] == 0.0), "experts not selected get exactly 0"


GATE_CASES = [
    # T, d, E, k, C, fused combine backward
    (300, 256, 8, 2, 0, True),
    (257, 128, 128, 4, 0, True),     # T % 4 != 0: a partly filled last workgroup
    (100, 64, 16, 8, 0, False),
    (64, 512, 4, 1, 0, True),        # k = 1: dlogits are exactly 0
    (400, 128, 8, 2, 70, False),     # padded: dropped slots
]


@pytest.mark.parametrize("T,d,E,k,C,fuse", GATE_CASES)
def test_gate_grad_parity(moe, T, d, E, k, C, fuse):
    _say("gate-grad", T, d, E, k, C, fuse)
    inp, r, y, dout, dl, dw, dyp = _gate_case(moe, T, d, E, k, C, seed=T + d + E, fuse=fuse)
    _check_gate(r, y, dout, dl, dw, E, k, d)
    if k == 1:
        assert torch.all(dl == 0)
    if C:
        assert bool((r["dst_row"] < 0).any()), "the padded case drops pairs"
    if fuse:
        ref = torch.empty_like(dyp)
        moe.moe_permute(moe.MOE_BF16, dout, k, r["dst_row"], ref, src_slot=r["src_slot"], row_scale=r["topk_w"])
        torch.cuda.synchronize()
        assert torch.equal(dyp, ref), "fused combine backward == moe_permute with the gate weights"


def test_gate_grad_full_size_sampled_tokens(moe):
    # e128 shapes: T = 16384, d = 4096, E = 128, k = 4; tokens checked: a sample
    _say("gate-grad-e128")
    cfg = moe_synth.WORKLOADS["e128"]
    T, d, E, k = cfg["T"], cfg["d"], cfg["E"], cfg["k"]
    inp, r, y, dout, dl, dw, dyp = _gate_case(moe, T, d, E, k, 0, seed=1002, fuse=True)
    toks = np.unique(np.concatenate([np.arange(0, T, 131), [T - 1]]))
    _check_gate(r, y, dout, dl, dw, E, k, d, rows=toks)
    ref = torch.empty_like(dyp)
    moe.moe_permute(moe.MOE_BF16, dout, k, r["dst_row"], ref, src_slot=r["src_slot"], row_scale=r["topk_w"])
    torch.cuda.synchronize()
    assert torch.equal(dyp, ref)


def test_router_and_gate_grad_empty(moe):
    # no tokens: both calls succeed and write nothing
    _say("router-empty")
    E, d, k = 8, 64, 2
    w = torch.randn(E, d, device=DEV).to(torch.bfloat16)
    x = torch.empty(0, d, dtype=torch.bfloat16, device=DEV)
    lg = torch.empty(0, E, dtype=torch.float32, device=DEV)
    moe.moe_router_logits(x, w, lg)
    i32 = dict(dtype=torch.int32, device=DEV)
    err = torch.zeros(1, **i32)
    moe.moe_gate_grad(torch.empty(0, d, dtype=torch.bfloat16, device=DEV),
                      torch.empty(0, d, dtype=torch.bfloat16, device=DEV), torch.empty(0, k, **i32),
                      torch.empty(0, k, dtype=torch.float32, device=DEV), torch.empty(0, **i32),
                      torch.empty(0, E, dtype=torch.float32, device=DEV), dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
