"""GPU parity of the HIP path against the CPU oracle at sizes the oracle runs in
seconds (several tiles per dimension, ragged tails, empty experts, ties).

Integer outputs (top-k indices, counts, offsets, dst_row, src_slot, permuted
bytes) must match bit for bit; topk_w within 1e-6; bf16 tensors within
max|gpu - ref| <= 2e-2 * max|ref| (fp32 tensors 1e-4).
"""
import sys

import numpy as np
import pytest
import torch

import moe_synth
import oracle
from tests._chain import BF16_TOL, F32_TOL, assert_close, np64, oracle_layer, oracle_layer_shared

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def moe():
    import routing_grouped_gemm_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.load()
    return m


def _gpu_route(m, logits, k, capacity=0):
    from routing_grouped_gemm_amd.layer import MoELayer
    T, E = logits.shape
    lay = MoELayer(T, 8, E, 8, k, m.MOE_BF16, capacity=capacity)
    lay.route(logits.to(DEV))
    torch.cuda.synchronize()
    return lay


def _check_route(lay, ref):
    np.testing.assert_array_equal(lay.topk_idx.cpu().numpy(), ref["topk_idx"])
    np.testing.assert_array_equal(lay.counts.cpu().numpy(), ref["counts"])
    np.testing.assert_array_equal(lay.offsets.cpu().numpy(), ref["offsets"])
    np.testing.assert_array_equal(lay.dst_row.cpu().numpy(), ref["dst_row"])
    np.testing.assert_array_equal(lay.src_slot.cpu().numpy(), ref["src_slot"])
    np.testing.assert_allclose(lay.topk_w.cpu().numpy(), ref["topk_w"], rtol=0, atol=1e-6)


ROUTE_CASES = [(300, 6, 2), (1000, 128, 4), (513, 8, 8), (777, 1024, 3), (64, 16, 1),
               (4097, 64, 4), (129, 256, 5), (65, 600, 8), (16384, 128, 4)]


@pytest.mark.parametrize("T,E,k", ROUTE_CASES)
def test_route_bit_exact(moe, T, E, k):
    _say("route", T, E, k)
    logits = moe_synth.normal((T, E), 1.0, seed=T * 7 + E)
    lay = _gpu_route(moe, logits, k)
    _check_route(lay, oracle.route(logits.numpy(), k))
    assert int(lay.dev_err.item()) == 0


@pytest.mark.parametrize("T,E,k", [(500, 8, 2), (300, 128, 4), (200, 1000, 8)])
def test_route_ties_lowest_index(moe, T, E, k):
    _say("route-ties", T, E, k)
    g = torch.Generator().manual_seed(E)
    logits = torch.randint(-2, 3, (T, E), generator=g).float()
    logits[::7] = 0.0
    logits[1::7, :] = -0.0
    lay = _gpu_route(moe, logits, k)
    _check_route(lay, oracle.route(logits.numpy(), k))


@pytest.mark.parametrize("T,E,k,C", [(400, 8, 2, 90), (1000, 16, 4, 300), (256, 8, 2, 200)])
def test_route_padded(moe, T, E, k, C):
    _say("route-padded", T, E, k, C)
    logits = moe_synth.router_logits(T, E, seed=C, routing="zipf")
    lay = _gpu_route(moe, logits, k, capacity=C)
    _check_route(lay, oracle.route(logits.numpy(), k, capacity=C))


# Batches of 65536 tokens and more: the finalize takes up to 16 histogram
# blocks per workgroup and writes source slots as per-expert runs (a ragged
# last block, padded layouts with drops, k = 8, and ties)
@pytest.mark.parametrize("T,E,k,C,routing", [(262144, 128, 4, 0, "uniform"), (200003, 64, 2, 7000, "zipf"),
                                             (70001, 16, 8, 0, "uniform"), (65536, 1024, 3, 0, "ties")])
def test_route_large_batch_bit_exact(moe, T, E, k, C, routing):
    _say("route-large", T, E, k, C, routing)
    if routing == "ties":
        g = torch.Generator().manual_seed(T)
        logits = torch.randint(-3, 4, (T, E), generator=g).float()
    else:
        logits = moe_synth.router_logits(T, E, seed=T + E, routing=routing)
    lay = _gpu_route(moe, logits, k, capacity=C)
    _check_route(lay, oracle.route(logits.numpy(), k, capacity=C))
    assert int(lay.dev_err.item()) == 0


def test_route_empty_and_nonfinite(moe):
    _say("route-empty")
    lay = _gpu_route(moe, torch.zeros(0, 8), 2)
    assert lay.counts.cpu().sum() == 0 and np.all(lay.offsets.cpu().numpy() == 0)
    _say("route-nonfinite")
    logits = moe_synth.normal((100, 8), 1.0, seed=3)
    logits[5, 2] = float("nan")
    logits[9, 0] = float("inf")
    lay = _gpu_route(moe, logits, 2)
    assert int(lay.dev_err.item()) & moe.MOE_ERR_NONFINITE_LOGIT
    ok = np.ones(100, bool)
    ok[[5, 9]] = False
    ref = oracle.route(logits.nan_to_num(nan=-np.inf, posinf=-np.inf).numpy().clip(min=-3e38), 2)
    np.testing.assert_array_equal(lay.topk_idx.cpu().numpy()[ok], ref["topk_idx"][ok])


def test_route_deterministic(moe):
    _say("route-determinism")
    logits = moe_synth.normal((5000, 128), 1.0, seed=77)
    a = _gpu_route(moe, logits, 4)
    b = _gpu_route(moe, logits, 4)
    for name in ("topk_idx", "topk_w", "dst_row", "src_slot", "offsets"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name


# ------------------------------------------------------------------ layer
LAYER_CASES = [
    # T, d, E, f, k, dtype, capacity
    (384, 256, 5, 384, 2, "bf16", 0),
    (200, 200, 7, 136, 3, "bf16", 0),
    (512, 128, 8, 256, 2, "bf16", 0),
    (300, 64, 1, 64, 1, "bf16", 0),
    (256, 128, 16, 64, 8, "bf16", 0),
    (400, 128, 8, 128, 2, "bf16", 70),
    (256, 128, 8, 256, 2, "f32", 0),
    (130, 72, 3, 40, 2, "f32", 0),
    # last M-tiles of at most 64 / 128 rows (the 64- and 128-row tile paths):
    # about 275, 53 and 350 rows per expert
    (1100, 256, 4, 256, 1, "bf16", 0),
    (160, 128, 6, 128, 2, "bf16", 0),
    (1400, 256, 4, 256, 1, "bf16", 0),
    (600, 128, 1024, 64, 8, "bf16", 0),     # the most experts and slots: ~5 rows per expert
    # rows of at least 256 16-byte vectors: permute and combine run one workgroup per token
    (150, 2048, 8, 128, 2, "bf16", 0),
    (130, 2056, 5, 64, 3, "bf16", 60),      # 257 vectors per row, padded
    (96, 1024, 4, 64, 2, "f32", 0),
]


def _run_layer(m, inp, k, dtype, capacity, empty_expert=None):
    from routing_grouped_gemm_amd.layer import MoELayer
    T, d = inp["x"].shape
    E, two_f, _ = inp["w13"].shape
    dt = m.MOE_F32 if dtype == "f32" else m.MOE_BF16
    lay = MoELayer(T, d, E, two_f // 2, k, dt, capacity=capacity)
    g = {n: inp[n].to(DEV) for n in ("logits", "x", "w13", "w2", "dout")}
    lay.set_weights(g["w13"], g["w2"])
    lay.forward(g["logits"], g["x"])
    lay.backward(g["dout"])
    torch.cuda.synchronize()
    return lay


@pytest.mark.parametrize("T,d,E,f,k,dtype,C", LAYER_CASES)
def test_layer_fwd_bwd_parity(moe, T, d, E, f, k, dtype, C):
    _say("layer", T, d, E, f, k, dtype, C)
    inp = moe_synth.make_inputs(T=T, d=d, E=E, f=f, k=k, dtype=dtype, seed=T + d + E + f + k)
    if E > 2:
        inp["logits"][:, E - 2] -= 1e30            # one expert gets no rows
    lay = _run_layer(moe, inp, k, dtype, C)
    rm = oracle.FP32 if dtype == "f32" else oracle.BF16
    tol = F32_TOL if dtype == "f32" else BF16_TOL
    ref = oracle_layer(inp, k, capacity=C, round_mode=rm)
    _check_route(lay, ref["route"])
    assert int(lay.dev_err.item()) == 0
    # permute is a byte copy of the token rows (padding rows zero)
    np.testing.assert_array_equal(np64(lay.x_perm), ref["x_perm"])
    rows = ref["route"]["src_slot"] >= 0
    assert_close(np64(lay.gu)[rows], ref["gu"][rows], tol, "gu")
    assert_close(np64(lay.h)[rows], ref["h"][rows], tol, "h")
    assert_close(np64(lay.y_perm)[rows], ref["y_perm"][rows], tol, "y_perm")
    assert_close(np64(lay.out), ref["out"], tol, "out")
    assert_close(np64(lay.dy_perm)[rows], ref["dy_perm"][rows], tol, "dy_perm")
    assert_close(np64(lay.dgu)[rows], ref["dgu"][rows], tol, "dgu")
    assert_close(np64(lay.dx_perm)[rows], ref["dx_perm"][rows], tol, "dx_perm")
    assert_close(np64(lay.dx), ref["dx"], tol, "dx")
    assert_close(np64(lay.dw13), ref["dw13"], tol, "dw13")
    assert_close(np64(lay.dw2), ref["dw2"], tol, "dw2")
    if E > 2:
        assert torch.all(lay.dw13[E - 2] == 0) and torch.all(lay.dw2[E - 2] == 0)


def test_layer_group_sizes_at_kstep_boundaries(moe):
    # top-1 routing that gives the experts 31, 32, 33, 64, 65, 96, 97, 1 and 0
    # rows: groups ending just before, at and just after the 32- and 64-row
    # K-steps of the weight-gradient loops, a one-row group and an empty one
    sizes = [31, 32, 33, 64, 65, 96, 97, 1, 0]
    E, d, f, k = len(sizes), 256, 256, 1
    T = sum(sizes)
    _say("layer-kstep-boundaries", sizes)
    inp = moe_synth.make_inputs(T=T, d=d, E=E, f=f, k=k, seed=77)
    owner = np.repeat(np.arange(E), sizes)
    np.random.default_rng(5).shuffle(owner)
    logits = inp["logits"].clone()
    logits[torch.arange(T), torch.from_numpy(owner)] += 1e4   # each token's expert
    inp["logits"] = logits
    lay = _run_layer(moe, inp, k, "bf16", 0)
    ref = oracle_layer(inp, k, capacity=0, round_mode=oracle.BF16)
    _check_route(lay, ref["route"])
    np.testing.assert_array_equal(lay.counts.cpu().numpy(), np.array(sizes))
    assert_close(np64(lay.dx), ref["dx"], BF16_TOL, "dx")
    assert_close(np64(lay.dw13), ref["dw13"], BF16_TOL, "dw13")
    assert_close(np64(lay.dw2), ref["dw2"], BF16_TOL, "dw2")
    for e, n in enumerate(sizes):
        if n == 0:
            continue
        # every expert's gradient on its own scale, so a small group cannot hide
        assert_close(np64(lay.dw13[e]), ref["dw13"][e], BF16_TOL, f"dw13[{e}]")
        assert_close(np64(lay.dw2[e]), ref["dw2"][e], BF16_TOL, f"dw2[{e}]")
    assert torch.all(lay.dw13[E - 1] == 0) and torch.all(lay.dw2[E - 1] == 0)


def test_layer_large_groups_partial_mtile_groups(moe):
    # top-1 routing with experts of 1300, 0, 2050 and 700 rows: 6, 0, 9 and 3
    # M-tiles, so the grouped-M tile order (groups of four M-tiles, N-tiles
    # across a group) ends on partial groups of 2 and 1 M-tiles, with 3 N-tiles
    # at gate/up, 2 (one partial) at dgrad-down and 1 at down / dgrad-gate/up
    sizes = [1300, 0, 2050, 700]
    E, d, f, k = len(sizes), 256, 384, 1
    T = sum(sizes)
    _say("layer-partial-mtile-groups", sizes)
    inp = moe_synth.make_inputs(T=T, d=d, E=E, f=f, k=k, seed=91)
    owner = np.repeat(np.arange(E), sizes)
    np.random.default_rng(9).shuffle(owner)
    logits = inp["logits"].clone()
    logits[torch.arange(T), torch.from_numpy(owner)] += 1e4   # each token's expert
    inp["logits"] = logits
    lay = _run_layer(moe, inp, k, "bf16", 0)
    ref = oracle_layer(inp, k, capacity=0, round_mode=oracle.BF16)
    _check_route(lay, ref["route"])
    np.testing.assert_array_equal(lay.counts.cpu().numpy(), np.array(sizes))
    assert_close(np64(lay.h), ref["h"], BF16_TOL, "h")
    assert_close(np64(lay.out), ref["out"], BF16_TOL, "out")
    assert_close(np64(lay.dx), ref["dx"], BF16_TOL, "dx")
    for e, n in enumerate(sizes):
        if n == 0:
            assert torch.all(lay.dw13[e] == 0) and torch.all(lay.dw2[e] == 0)
            continue
        assert_close(np64(lay.dw13[e]), ref["dw13"][e], BF16_TOL, f"dw13[{e}]")
        assert_close(np64(lay.dw2[e]), ref["dw2"][e], BF16_TOL, f"dw2[{e}]")


@pytest.mark.parametrize("T,d,E,f,k,C", [(384, 256, 5, 384, 2, 0), (400, 128, 8, 128, 2, 70),
                                         (1100, 256, 4, 256, 1, 0)])
def test_wgrad_fp32_accumulate(moe, T, d, E, f, k, C):
    # the weight-gradient stage adding into fp32 accumulators: twice onto a
    # random start, each addition against the oracle's weight gradient
    _say("wgrad-f32-accumulate", T, d, E, f, k, C)
    inp = moe_synth.make_inputs(T=T, d=d, E=E, f=f, k=k, seed=T + 3 * d)
    if E > 2:
        inp["logits"][:, E - 2] -= 1e30            # one expert gets no rows
    lay = _run_layer(moe, inp, k, "bf16", C)
    ref = oracle_layer(inp, k, capacity=C, round_mode=oracle.BF16)
    a13 = moe_synth.normal((E, 2 * f, d), 1e-3, 5, DEV)
    a2 = moe_synth.normal((E, d, f), 1e-3, 6, DEV)
    s13, s2 = a13.clone(), a2.clone()
    lay.wgrad_accumulate(a13, a2)
    torch.cuda.synchronize()
    one13, one2 = a13.clone(), a2.clone()
    lay.wgrad_accumulate(a13, a2)
    torch.cuda.synchronize()
    assert_close(np64(one13 - s13), ref["dw13"], BF16_TOL, "dw13 += (first)")
    assert_close(np64(one2 - s2), ref["dw2"], BF16_TOL, "dw2 += (first)")
    assert_close(np64(a13 - one13), ref["dw13"], BF16_TOL, "dw13 += (second)")
    assert_close(np64(a2 - one2), ref["dw2"], BF16_TOL, "dw2 += (second)")
    if E > 2:   # an expert with no rows adds exactly nothing
        assert torch.equal(a13[E - 2], s13[E - 2]) and torch.equal(a2[E - 2], s2[E - 2])
    # the bf16 gradients of the same backward are untouched
    assert_close(np64(lay.dw13), ref["dw13"], BF16_TOL, "dw13")


SHARED_CASES = [
    # T, d, E, f, k, shared experts, capacity
    (384, 256, 5, 384, 2, 1, 0),
    (256, 128, 8, 128, 2, 2, 0),
    (400, 128, 8, 128, 2, 1, 70),
    (300, 64, 4, 64, 1, 1, 0),
    (300, 128, 1023, 64, 7, 1, 0),      # E + S = 1024 groups, k + S = 8 slots
]


@pytest.mark.parametrize("T,d,E,f,k,S,C", SHARED_CASES)
def test_layer_shared_experts_parity(moe, T, d, E, f, k, S, C):
    # shared experts as extra groups E .. E+S-1 of the same grouped GEMM
    from routing_grouped_gemm_amd.layer import MoELayer
    _say("shared", T, d, E, f, k, S, C)
    inp = moe_synth.make_inputs(T=T, d=d, E=E + S, f=f, k=k, seed=T + 5 * S + C)
    inp["logits"] = inp["logits"][:, :E].contiguous()
    lay = MoELayer(T, d, E, f, k, moe.MOE_BF16, capacity=C, n_shared=S)
    g = {n: inp[n].to(DEV) for n in ("logits", "x", "w13", "w2", "dout")}
    lay.set_weights(g["w13"], g["w2"])
    lay.forward(g["logits"], g["x"])
    lay.backward(g["dout"])
    torch.cuda.synchronize()
    assert int(lay.dev_err.item()) == 0
    ref = oracle_layer_shared(inp, k, S, capacity=C, round_mode=oracle.BF16)
    # the widened route is integer data: bit-exact
    np.testing.assert_array_equal(lay.s_dst.cpu().numpy(), ref["dst"])
    sw = lay.s_w.cpu().numpy()
    assert np.all(sw[:, k:] == 1.0)                        # shared slots: weight exactly 1
    np.testing.assert_allclose(sw[:, :k], ref["w"][:, :k], rtol=0, atol=1e-6)   # as the route tests
    np.testing.assert_array_equal(lay.s_off.cpu().numpy(), ref["go"])
    idx = lay.s_idx.cpu().numpy()
    np.testing.assert_array_equal(idx[:, :k], ref["route"]["topk_idx"])
    np.testing.assert_array_equal(idx[:, k:], np.broadcast_to(E + np.arange(S), (T, S)))
    cnt = lay.s_counts.cpu().numpy()
    np.testing.assert_array_equal(cnt[:E], ref["route"]["counts"])
    assert np.all(cnt[E:] == T)
    # src_slot is the inverse of dst_row over the widened slots; pad rows hold -1
    src = lay.s_src.cpu().numpy()
    expect = -np.ones(src.size, np.int64)
    live = ref["dst"] >= 0
    expect[ref["dst"][live]] = np.nonzero(live)[0]
    np.testing.assert_array_equal(src, expect)
    np.testing.assert_array_equal(np64(lay.x_perm), ref["x_perm"])
    assert_close(np64(lay.out), ref["out"], BF16_TOL, "out")
    assert_close(np64(lay.dx), ref["dx"], BF16_TOL, "dx")
    assert_close(np64(lay.dw13), ref["dw13"], BF16_TOL, "dw13")
    assert_close(np64(lay.dw2), ref["dw2"], BF16_TOL, "dw2")
    # the shared experts' own weight gradients, on their own scale
    assert_close(np64(lay.dw13[E:]), ref["dw13"][E:], BF16_TOL, "dw13 shared")
    assert_close(np64(lay.dw2[E:]), ref["dw2"][E:], BF16_TOL, "dw2 shared")


def test_layer_deterministic(moe):
    _say("layer-determinism")
    inp = moe_synth.make_inputs(T=384, d=256, E=5, f=384, k=2, seed=5)
    a = _run_layer(moe, inp, 2, "bf16", 0)
    b = _run_layer(moe, inp, 2, "bf16", 0)
    for name in ("gu", "h", "y_perm", "out", "dgu", "dx_perm", "dx", "dw13", "dw2"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name


def test_permute_row_range_error_is_flagged(moe):
    _say("permute-row-range")
    T, d, k = 16, 64, 2
    x = torch.randn(T, d, device=DEV).to(torch.bfloat16)
    dst = torch.arange(T * k, dtype=torch.int32, device=DEV)
    dst[5] = T * k + 3                                  # outside x_perm
    xp = torch.zeros(T * k, d, dtype=torch.bfloat16, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    moe.moe_permute(moe.MOE_BF16, x, k, dst, xp, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & moe.MOE_ERR_ROW_RANGE
    ok = torch.ones(T * k, dtype=torch.bool)
    ok[5] = False
    assert torch.equal(xp.cpu()[ok], x.cpu().repeat_interleave(k, 0)[ok])


@pytest.mark.parametrize("S", [0, 1])
def test_layer_empty_batch(moe, S):
    # no tokens: every group (shared ones included) is empty, the outputs are
    # empty and the weight gradients exactly zero
    from routing_grouped_gemm_amd.layer import MoELayer
    _say("layer-empty", S)
    T, d, E, f, k = 0, 128, 8, 128, 2
    inp = moe_synth.make_inputs(T=4, d=d, E=E + S, f=f, k=k, seed=21)
    lay = MoELayer(T, d, E, f, k, moe.MOE_BF16, n_shared=S)
    lay.set_weights(inp["w13"].to(DEV), inp["w2"].to(DEV))
    x = torch.empty(0, d, dtype=torch.bfloat16, device=DEV)
    out = lay.forward(torch.empty(0, E, device=DEV), x)
    dx, dw13, dw2 = lay.backward(torch.empty(0, d, dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()
    assert int(lay.dev_err.item()) == 0
    assert out.shape == (0, d) and dx.shape == (0, d)
    assert dw13.shape == (E + S, 2 * f, d) and dw2.shape == (E + S, d, f)
    assert torch.all(dw13 == 0) and torch.all(dw2 == 0)
    assert torch.all(lay.s_off == 0)
    assert torch.all(lay.s_counts == 0)
