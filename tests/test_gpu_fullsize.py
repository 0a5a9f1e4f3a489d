"""GPU parity at the full workload sizes, in the launch configuration bench.py
times (MoELayer on one stream, the same kernels and tiles).

The oracle cannot run a whole E=128 layer in seconds, so the checks use
sub-problems that are exact by definition:
  * routing (top-k, counts, offsets, dst_row, src_slot) over all tokens,
    bit-exact;
  * the permute: every sampled row equals its source token row, bit-exact;
  * sampled rows (group edges, ragged tails, random rows): a one-row
    forward and backward with that row's expert weights gives the exact
    gu, h, y_perm, dy_perm, dgu, dx_perm rows; sampled tokens get out / dx
    from their k rows;
  * sampled experts and sampled columns n: the problem restricted to those
    columns (Wg[n], Wu[n] rows and Wd[:, n]) gives gu[:, n], h[:, n],
    dgu[:, n] for every row of the expert and dWd[:, n], dWg[n, :],
    dWu[n, :] exactly as the full problem defines them.
Tolerance: max|gpu - ref| <= 2e-2 * max|ref| per tensor (bf16 storage, fp32
accumulate); 6e-2 for the MXFP8 shard.
"""
import sys

import numpy as np
import pytest
import torch

import moe_synth
import oracle
from tests._chain import BF16_TOL, assert_close, np64, widen_route

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[gpu-fullsize]", *a, flush=True)
    sys.stdout.flush()


CASES = [("e8", False), ("e8_matched", False), ("e128", False), ("e128_zipf", False), ("e128_zipf", True),
         ("e128_shared", False)]


@pytest.fixture(scope="module")
def moe():
    import routing_grouped_gemm_amd as m
    assert torch.cuda.is_available()
    m.load()
    oracle.set_threads(16)
    return m


def _run(m, name, padded):
    from routing_grouped_gemm_amd.layer import MoELayer
    cfg = moe_synth.WORKLOADS[name]
    T, d, E, f, k = cfg["T"], cfg["d"], cfg["E"], cfg["f"], cfg["k"]
    cap = moe_synth.capacity_of(T, k, E, cfg.get("capacity_factor", 1.25)) if padded else 0
    inp = moe_synth.make_inputs(name, device="cuda")
    lay = MoELayer(T, d, E, f, k, m.MOE_BF16, capacity=cap, n_shared=cfg.get("n_shared", 0))
    lay.set_weights(inp["w13"], inp["w2"])
    # weight gradients start as NaN: a tile the weight-gradient GEMM never
    # writes stays NaN and is found below over the whole tensors
    lay._alloc_bwd()
    lay.dw13.fill_(float("nan"))
    lay.dw2.fill_(float("nan"))
    lay.forward(inp["logits"], inp["x"])
    lay.backward(inp["dout"])
    torch.cuda.synchronize()
    return cfg, cap, inp, lay


def _sample_rows(go, rng, per_group=2, extra=8):
    rows = []
    E = len(go) - 1
    big = np.argsort(np.diff(go))[::-1]
    for e in list(big[:3]) + list(big[-3:]) + list(rng.choice(E, size=min(E, 4), replace=False)):
        g0, g1 = int(go[e]), int(go[e + 1])
        if g1 > g0:
            rows += [g0, g1 - 1] + list(rng.integers(g0, g1, size=per_group))
    rows += list(rng.integers(0, int(go[-1]), size=extra))
    return sorted(set(int(r) for r in rows))


@pytest.mark.parametrize("name,padded", CASES)
def test_fullsize_layer(moe, name, padded):
    _say(name, "padded" if padded else "unpadded")
    cfg, cap, inp, lay = _run(moe, name, padded)
    T, d, E, f, k = cfg["T"], cfg["d"], cfg["E"], cfg["f"], cfg["k"]
    assert int(lay.dev_err.item()) == 0
    # every weight-gradient element written (the whole tensors, every expert)
    assert bool(torch.isfinite(lay.dw13).all()) and bool(torch.isfinite(lay.dw2).all())
    # fp32 accumulate-into from zero: the same tiles' sums added once, so
    # rounding them to bf16 gives the bf16 weight gradients bit for bit (a
    # tile skipped or added twice would not)
    if not padded:
        a13 = torch.zeros(lay.G, 2 * f, d, dtype=torch.float32, device="cuda")
        a2 = torch.zeros(lay.G, d, f, dtype=torch.float32, device="cuda")
        lay.wgrad_accumulate(a13, a2)
        torch.cuda.synchronize()
        assert torch.equal(a13.to(torch.bfloat16), lay.dw13), f"{name}: fp32-accumulated dW13"
        assert torch.equal(a2.to(torch.bfloat16), lay.dw2), f"{name}: fp32-accumulated dW2"
        del a13, a2
    # ---- routing, bit-exact over all tokens
    r = oracle.route(inp["logits"].cpu().numpy(), k, cap)
    np.testing.assert_array_equal(lay.topk_idx.cpu().numpy(), r["topk_idx"])
    np.testing.assert_array_equal(lay.counts.cpu().numpy(), r["counts"])
    np.testing.assert_array_equal(lay.offsets.cpu().numpy(), r["offsets"])
    np.testing.assert_array_equal(lay.dst_row.cpu().numpy(), r["dst_row"])
    np.testing.assert_array_equal(lay.src_slot.cpu().numpy(), r["src_slot"])
    np.testing.assert_allclose(lay.topk_w.cpu().numpy(), r["topk_w"], rtol=0, atol=1e-6)
    # shared experts: slots k .. k+S-1 of every token, groups E .. E+S-1
    S = cfg.get("n_shared", 0)
    dst_all, w_all, go, src = widen_route(r, k, S, cap)
    if not S:
        np.testing.assert_array_equal(src, r["src_slot"])
    else:
        np.testing.assert_array_equal(lay.s_dst.cpu().numpy(), dst_all)
        np.testing.assert_array_equal(lay.s_src.cpu().numpy(), src)
        np.testing.assert_array_equal(lay.s_off.cpu().numpy(), go)
        assert np.all(lay.s_w.cpu().numpy()[:, k:] == 1.0)
    k = k + S                                   # slots per token from here on
    w_pair = w_all.reshape(-1)
    rng = np.random.default_rng(sum(map(ord, name)) * 2 + int(padded))
    rows = [i for i in _sample_rows(go, rng) if src[i] >= 0]
    row_expert = np.searchsorted(go, rows, side="right") - 1

    # ---- permute: each sampled row is its token row, byte for byte
    x_cpu = inp["x"].cpu()
    xp = lay.x_perm[torch.tensor(rows, device="cuda")].cpu()
    toks = src[rows] // k
    assert torch.equal(xp, x_cpu[torch.from_numpy(toks).long()])

    # ---- one-row forward/backward problems for the sampled rows
    x64 = np64(x_cpu)
    dout64 = np64(inp["dout"].cpu())
    wcache = {}

    def wexp(e):
        if e not in wcache:
            wcache[e] = (np64(inp["w13"][e:e + 1].cpu()), np64(inp["w2"][e:e + 1].cpu()))
        return wcache[e]

    ref = {n: [] for n in ("gu", "h", "y", "dy", "dgu", "dx")}
    for r_i, e in zip(rows, row_expert):
        t = src[r_i] // k
        w13e, w2e = wexp(int(e))
        g1 = np.array([0, 1], np.int32)
        gu, h, y = oracle.ffn_fwd(x64[t:t + 1], w13e, w2e, g1, oracle.BF16)
        dy = oracle.permute(dout64[t:t + 1], np.array([0], np.int32), 1, 1,
                            row_scale=np.array([w_pair[src[r_i]]], np.float32),
                            round_mode=oracle.BF16)
        dgu, dxp, _, _ = oracle.ffn_bwd(dy, x64[t:t + 1], gu, h, w13e, w2e, g1, oracle.BF16)
        for n, v in (("gu", gu), ("h", h), ("y", y), ("dy", dy), ("dgu", dgu), ("dx", dxp)):
            ref[n].append(v[0])
    idx = torch.tensor(rows, device="cuda")
    for n, t in (("gu", lay.gu), ("h", lay.h), ("y", lay.y_perm), ("dy", lay.dy_perm),
                 ("dgu", lay.dgu), ("dx", lay.dx_perm)):
        assert_close(np64(t[idx]), np.stack(ref[n]), BF16_TOL, f"{name}:{n} rows")

    # ---- sampled experts, sampled columns: full-group exact sub-problems
    E_sel = [int(e) for e in np.argsort(np.diff(go))[::-1][[0, len(go) // 2]] if go[e + 1] > go[e]]
    n_sel = np.array(sorted(set([0, f - 1] + list(rng.integers(0, f, size=6)))))
    for e in E_sel:
        g0, g1 = int(go[e]), int(go[e + 1])
        valid = src[g0:g1] >= 0
        tok = np.where(valid, src[g0:g1] // k, 0)
        xe = np.where(valid[:, None], x64[tok], 0.0)
        dye = oracle.permute(dout64[tok], np.arange(g1 - g0, dtype=np.int32), 1, g1 - g0,
                             row_scale=np.where(valid, w_pair[src[g0:g1]], 0).astype(np.float32),
                             round_mode=oracle.BF16)
        w13 = np64(inp["w13"][e].cpu())
        w2 = np64(inp["w2"][e].cpu())
        w13s = np.concatenate([w13[n_sel], w13[f + n_sel]])[None]
        w2s = w2[:, n_sel][None]
        gs = np.array([0, g1 - g0], np.int32)
        gu_s, h_s, _ = oracle.ffn_fwd(xe, w13s, w2s, gs, oracle.BF16)
        dgu_s, _, dw13_s, dw2_s = oracle.ffn_bwd(dye, xe, gu_s, h_s, w13s, w2s, gs, oracle.BF16)
        ns = len(n_sel)
        cols = np.concatenate([n_sel, f + n_sel])
        assert_close(np64(lay.gu[g0:g1].cpu())[:, cols][valid], gu_s[valid], BF16_TOL,
                     f"{name}:gu expert {e}")
        assert_close(np64(lay.h[g0:g1].cpu())[:, n_sel][valid], h_s[valid], BF16_TOL,
                     f"{name}:h expert {e}")
        assert_close(np64(lay.dgu[g0:g1].cpu())[:, cols][valid], dgu_s[valid], BF16_TOL,
                     f"{name}:dgu expert {e}")
        assert_close(np64(lay.dw2[e].cpu())[:, n_sel], dw2_s[0], BF16_TOL, f"{name}:dw2 expert {e}")
        assert_close(np64(lay.dw13[e].cpu())[cols], dw13_s[0], BF16_TOL, f"{name}:dw13 expert {e}")
        assert ns > 0

    # ---- combine / permute-backward for sampled tokens
    t_sel = np.unique(np.concatenate([rng.choice(src[rows] // k, size=6), rng.integers(0, T, size=6)]))
    out_ref, dx_ref = [], []
    for t in t_sel:
        ys, dxs = np.zeros(d), np.zeros(d)
        for j in range(k):
            dst = dst_all[t * k + j]
            if dst < 0:
                continue
            e = int(np.searchsorted(go, dst, side="right") - 1)
            w13e, w2e = wexp(e)
            g1 = np.array([0, 1], np.int32)
            gu, h, y = oracle.ffn_fwd(x64[t:t + 1], w13e, w2e, g1, oracle.BF16)
            dy = oracle.permute(dout64[t:t + 1], np.array([0], np.int32), 1, 1,
                                row_scale=np.array([w_pair[t * k + j]], np.float32),
                                round_mode=oracle.BF16)
            _, dxp, _, _ = oracle.ffn_bwd(dy, x64[t:t + 1], gu, h, w13e, w2e, g1, oracle.BF16)
            ys += float(w_pair[t * k + j]) * y[0]
            dxs += dxp[0]
        out_ref.append(oracle.round_(ys, oracle.BF16))
        dx_ref.append(oracle.round_(dxs, oracle.BF16))
    tt = torch.from_numpy(t_sel).long().cuda()
    assert_close(np64(lay.out[tt]), np.stack(out_ref), BF16_TOL, f"{name}:out")
    assert_close(np64(lay.dx[tt]), np.stack(dx_ref), BF16_TOL, f"{name}:dx")


MX_TOL = 6e-2


def test_fullsize_mx_shard(moe):
    """The MXFP8 expert-parallel shard (32768 received rows, 16 local experts,
    k=1 with a per-row gate) at full size.  Every GEMM operand is taken
    through the MXFP8 quantiser in the direction its GEMM contracts over, so
    the sub-problems below are exact: row-wise quantisation only involves a
    row, column-wise only a column of one expert's rows."""
    from routing_grouped_gemm_amd.layer import MoELayer
    name = "mx_shard"
    _say(name)
    cfg = moe_synth.WORKLOADS[name]
    T, d, E, f, k = cfg["T"], cfg["d"], cfg["E"], cfg["f"], cfg["k"]
    inp = moe_synth.make_inputs(name, device="cuda")
    lay = MoELayer(T, d, E, f, k, moe.MOE_MXFP8)
    lay.set_weights(inp["w13"], inp["w2"])
    lay.forward(inp["logits"], inp["x"], weights=inp["gate"])
    lay.backward(inp["dout"], weights=inp["gate"])
    torch.cuda.synchronize()
    assert int(lay.dev_err.item()) == 0
    r = oracle.route(inp["logits"].cpu().numpy(), k)
    np.testing.assert_array_equal(lay.dst_row.cpu().numpy(), r["dst_row"])
    np.testing.assert_array_equal(lay.offsets.cpu().numpy(), r["offsets"])
    np.testing.assert_array_equal(lay.src_slot.cpu().numpy(), r["src_slot"])
    go = r["offsets"].astype(np.int32)
    src = r["src_slot"]
    gate = inp["gate"].cpu().numpy()
    rng = np.random.default_rng(4242)
    rows = _sample_rows(go, rng)
    row_expert = np.searchsorted(go, rows, side="right") - 1
    x64 = np64(inp["x"].cpu())
    dout64 = np64(inp["dout"].cpu())

    # ---- dispatch payload: codes and scales of sampled rows, bit-exact
    idx = torch.tensor(rows, device="cuda")
    rc, rs = oracle.mx_quantize_rows(x64[src[rows] // k])
    np.testing.assert_array_equal(lay.x_perm[idx].cpu().numpy(), rc)
    np.testing.assert_array_equal(lay.x_perm_scales[idx].cpu().numpy(), rs)

    caches = {}

    def cache(e):   # forward (blocks along the input dim) and backward (along the output dim)
        if e not in caches:
            w13 = np64(inp["w13"][e].cpu())
            w2 = np64(inp["w2"][e].cpu())
            caches[e] = (oracle.mx_qdq_rows(w13), oracle.mx_qdq_rows(w2),
                         oracle.mx_qdq_cols(w13, np.array([0, 2 * f], np.int32)),
                         oracle.mx_qdq_cols(w2, np.array([0, d], np.int32)))
        return caches[e]

    # ---- one-row problems for the sampled rows
    ref = {n: [] for n in ("gu", "h", "y", "dy", "dgu", "dx", "out")}
    g1 = np.array([0, 1], np.int32)
    for r_i, e in zip(rows, row_expert):
        t = src[r_i] // k
        w13f, w2f, w13b, w2b = cache(int(e))
        xq = oracle.mx_qdq_rows(x64[t:t + 1])
        gu, h, y = oracle.ffn_fwd(xq, w13f[None], w2f[None], g1, oracle.BF16, mx_h=True)
        dy = oracle.permute(dout64[t:t + 1], np.array([0], np.int32), 1, 1,
                            row_scale=gate[t:t + 1], round_mode=oracle.BF16)
        dgu, dxp, _, _ = oracle.ffn_bwd(oracle.mx_qdq_rows(dy), xq, gu, h, w13f[None], w2f[None], g1,
                                        oracle.BF16, w2_dgrad=w2b[None], w13_dgrad=w13b[None],
                                        mx_dgu=True)
        out = oracle.combine(y, np.array([0], np.int32), gate[t:t + 1], 1, 1, oracle.BF16)
        for n, v in (("gu", gu), ("h", h), ("y", y), ("dy", dy), ("dgu", dgu), ("dx", dxp),
                     ("out", out)):
            ref[n].append(v[0])
    toks = torch.from_numpy(src[rows] // k).long().cuda()
    for n, t in (("gu", lay.gu[idx]), ("h", lay.h[idx]), ("y", lay.y_perm[idx]),
                 ("dgu", lay.dgu[idx]), ("dx", lay.dx_perm[idx]), ("out", lay.out[toks])):
        assert_close(np64(t), np.stack(ref[n]), MX_TOL, f"{name}:{n} rows")
    assert_close(np64(lay.dy_perm[idx]), np.stack(ref["dy"]), BF16_TOL, f"{name}:dy rows")
    assert_close(np64(lay.dx[toks]), np.stack(ref["dx"]), MX_TOL, f"{name}:dx tokens")

    # ---- sampled experts and columns: weight gradients over whole groups
    counts = np.diff(go)
    n_sel = np.array(sorted(set([0, f - 1] + list(rng.integers(0, f, size=6)))))
    cols = np.concatenate([n_sel, f + n_sel])
    for e in (int(np.argmax(counts)), int(np.argmin(counts))):
        g0, g1e = int(go[e]), int(go[e + 1])
        m = g1e - g0
        tok = src[g0:g1e] // k
        w13f, w2f, w13b, w2b = cache(e)
        gs = np.array([0, m], np.int32)
        xq = oracle.mx_qdq_rows(x64[tok])
        dye = oracle.permute(dout64[tok], np.arange(m, dtype=np.int32), 1, m,
                             row_scale=gate[tok], round_mode=oracle.BF16)
        gu_s, h_s, _ = oracle.ffn_fwd(xq, w13f[cols][None], w2f[:, n_sel][None], gs, oracle.BF16)
        dgu_s, _, dw13_s, dw2_s = oracle.ffn_bwd(
            oracle.mx_qdq_rows(dye), xq, gu_s, h_s, w13f[cols][None], w2f[:, n_sel][None], gs,
            oracle.BF16, w2_dgrad=w2b[:, n_sel][None], w13_dgrad=w13b[cols][None],
            dy_wgrad=oracle.mx_qdq_cols(dye, gs), h_wgrad=oracle.mx_qdq_cols(h_s, gs),
            x_wgrad=oracle.mx_qdq_cols(xq, gs), mx_dgu=True)
        assert_close(np64(lay.gu[g0:g1e].cpu())[:, cols], gu_s, MX_TOL, f"{name}:gu expert {e}")
        assert_close(np64(lay.h[g0:g1e].cpu())[:, n_sel], h_s, MX_TOL, f"{name}:h expert {e}")
        assert_close(np64(lay.dgu[g0:g1e].cpu())[:, cols], dgu_s, MX_TOL, f"{name}:dgu expert {e}")
        assert_close(np64(lay.dw2[e].cpu())[:, n_sel], dw2_s[0], MX_TOL, f"{name}:dw2 expert {e}")
        assert_close(np64(lay.dw13[e].cpu())[cols], dw13_s[0], MX_TOL, f"{name}:dw13 expert {e}")
