"""GPU parity of the MXFP8 path against the CPU oracle.

Quantisers (row-wise, column-wise inside groups, decode-and-requantise, the
fused dispatch quantiser) must match the oracle's codes and scales bit for
bit on identical inputs.  The MXFP8 layer (block-scaled MFMA grouped GEMMs,
forward and backward) must be within max|gpu - ref| <= 6e-2 * max|ref| of
the oracle run on the same quantised operands (every GEMM operand passed
through the MXFP8 quantiser in the direction that GEMM contracts over).
"""
import sys

import numpy as np
import pytest
import torch

import moe_synth
import oracle
from tests._chain import BF16_TOL, assert_close, np64

pytestmark = pytest.mark.gpu
MX_TOL = 6e-2
PAD = 128


def _say(*a):
    print("[gpu-mx]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def moe():
    import routing_grouped_gemm_amd as m
    assert torch.cuda.is_available()
    m.load()
    return m


def _bf16(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    v = torch.randn(*shape, generator=g) * scale
    v[..., ::97] *= 64.0                      # spread the block maxima
    return v.to(torch.bfloat16)


def _unpack_cols(codes, scales, go, K):
    """Group-transposed padded layout -> (codes [rows, K], scales per group list)."""
    rows = int(go[-1])
    out = np.zeros((rows, K), np.uint8)
    sc = []
    P = 0
    for e in range(len(go) - 1):
        m = int(go[e + 1] - go[e])
        mp = (m + PAD - 1) // PAD * PAD
        blk = codes[K * P:K * (P + mp)].reshape(K, mp)
        out[go[e]:go[e + 1]] = blk[:, :m].T
        assert np.all(blk[:, m:] == 0), "padding rows must hold zero codes"
        sc.append(scales[K * P // 32:K * (P + mp) // 32].reshape(K, mp // 32))
        P += mp
    return out, sc


@pytest.mark.parametrize("rows,K", [(1, 32), (77, 256), (1000, 4096)])
def test_quantize_rows_bit_exact(moe, rows, K):
    _say("quant-rows", rows, K)
    x = _bf16((rows, K), rows + K, 0.02)
    codes = torch.empty(rows, K, dtype=torch.uint8, device="cuda")
    scales = torch.empty(rows, K // 32, dtype=torch.uint8, device="cuda")
    moe.moe_quantize_mxfp8(x.cuda(), 0, codes, scales)
    torch.cuda.synchronize()
    rc, rs = oracle.mx_quantize_rows(np64(x))
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)


def _check_cols(moe, x, go, K):
    rows, E = int(go[-1]), len(go) - 1
    n = K * (rows + PAD * E)
    codes = torch.full((n,), 0xAA, dtype=torch.uint8, device="cuda")
    scales = torch.full((n // 32,), 0xAA, dtype=torch.uint8, device="cuda")
    moe.moe_quantize_mxfp8(x.cuda(), 1, codes, scales, torch.from_numpy(go).cuda(), E)
    torch.cuda.synchronize()
    got, gs = _unpack_cols(codes.cpu().numpy(), scales.cpu().numpy(), go, K)
    rc, rs = oracle.mx_quantize_cols(np64(x), go)
    np.testing.assert_array_equal(got, rc)
    sb = 0
    for e, m in enumerate(np.diff(go)):
        nb = (m + 31) // 32
        np.testing.assert_array_equal(gs[e][:, :nb], rs[:, sb:sb + nb])
        assert np.all(gs[e][:, nb:] == 0)         # all-zero blocks: scale 2^-127
        sb += nb


@pytest.mark.parametrize("sizes,K", [([33, 0, 130, 257], 64), ([512, 511, 1], 256), ([200] * 5, 96)])
def test_quantize_cols_bit_exact(moe, sizes, K):
    _say("quant-cols", sizes, K)
    go = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    _check_cols(moe, _bf16((int(go[-1]), K), int(go[-1]) * 3 + K, 0.5), go, K)


def _special_bf16(rows, K, seed):
    """Blocks with NaN, infinities, the largest and smallest bf16 magnitudes,
    signed zeros and all-zero blocks, among ordinary values."""
    g = torch.Generator().manual_seed(seed)
    v = torch.randn(rows, K, generator=g)
    v[0, 3] = float("nan")
    v[1, 40] = float("inf")
    v[2, 70] = float("-inf")
    v[3, :32] = 0.0
    v[4, 33:64] = -0.0
    v[5, 5] = 3.3895e38                       # near the bf16 maximum
    v[6, 96:128] *= 1e-37                     # tiny block: scale near 2^-127
    v[7, 0:32] = 2.0 ** -133                  # bf16 subnormals
    v[8, 64:96] = torch.tensor([448.0 * 2.0 ** -3, 416.0 * 2.0 ** -3, 432.0 * 2.0 ** -3] * 10 + [1.0, -1.0])
    v[9:11, 10] = float("nan")
    v[12, :] = float("inf")
    return v.to(torch.bfloat16)


def test_quantize_special_values_bit_exact(moe):
    _say("quant-special")
    rows, K = 64, 128
    x = _special_bf16(rows, K, 5)
    codes = torch.empty(rows, K, dtype=torch.uint8, device="cuda")
    scales = torch.empty(rows, K // 32, dtype=torch.uint8, device="cuda")
    moe.moe_quantize_mxfp8(x.cuda(), 0, codes, scales)
    torch.cuda.synchronize()
    rc, rs = oracle.mx_quantize_rows(np64(x))
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)
    # column-wise over the same values (two groups, the first one ragged)
    go = np.array([0, 37, rows], np.int32)
    _check_cols(moe, x, go, K)


def test_permute_mx_and_requantise_cols_bit_exact(moe):
    _say("permute-mx")
    T, d, E, k = 700, 256, 6, 2
    inp = moe_synth.make_inputs(T=T, d=d, E=E, f=128, k=k, seed=77)
    from routing_grouped_gemm_amd.layer import MoELayer
    lay = MoELayer(T, d, E, 128, k, moe.MOE_MXFP8)
    lay.route(inp["logits"].cuda())
    lay.permute(inp["x"].cuda())
    torch.cuda.synchronize()
    r = oracle.route(inp["logits"].numpy(), k)
    xp = oracle.permute(np64(inp["x"]), r["dst_row"], k, r["n_rows"])
    rc, rs = oracle.mx_quantize_rows(xp)
    np.testing.assert_array_equal(lay.x_perm.cpu().numpy(), rc)
    np.testing.assert_array_equal(lay.x_perm_scales.cpu().numpy(), rs)
    # column-wise quantisation of the decoded dispatch payload (the operand
    # the gate/up weight gradient reads), per expert group
    go = r["offsets"].astype(np.int32)
    dq = oracle.mx_dequant_rows(rc, rs)
    _check_cols(moe, torch.from_numpy(dq).to(torch.bfloat16), go, d)   # decoded values are bf16-exact


def _mx_oracle(inp, k, gate=None):
    """The oracle on the operands each MXFP8 GEMM reads."""
    x = np64(inp["x"])
    T = x.shape[0]
    E, two_f, d = inp["w13"].shape
    f = two_f // 2
    r = oracle.route(inp["logits"].numpy(), k)
    go = r["offsets"].astype(np.int32)
    w = r["topk_w"] if gate is None else np.asarray(gate, np.float32).reshape(T, k)
    w13 = np64(inp["w13"]).reshape(E * 2 * f, d)
    w2 = np64(inp["w2"]).reshape(E * d, f)
    w13f = oracle.mx_qdq_rows(w13).reshape(E, 2 * f, d)          # forward caches
    w2f = oracle.mx_qdq_rows(w2).reshape(E, d, f)
    g13 = np.arange(E + 1, dtype=np.int32) * 2 * f
    g2 = np.arange(E + 1, dtype=np.int32) * d
    w13b = oracle.mx_qdq_cols(w13, g13).reshape(E, 2 * f, d)     # backward caches
    w2b = oracle.mx_qdq_cols(w2, g2).reshape(E, d, f)
    xp = oracle.permute(x, r["dst_row"], k, r["n_rows"])
    xq = oracle.mx_qdq_rows(xp)
    gu, h, y = oracle.ffn_fwd(xq, w13f, w2f, go, oracle.BF16, mx_h=True)
    out = oracle.combine(y, r["dst_row"], w, T, k, oracle.BF16)
    dy = oracle.permute(np64(inp["dout"]), r["dst_row"], k, r["n_rows"], row_scale=w,
                        round_mode=oracle.BF16)
    dgu, dxp, dw13, dw2 = oracle.ffn_bwd(
        oracle.mx_qdq_rows(dy), xq, gu, h, w13f, w2f, go, oracle.BF16, w2_dgrad=w2b,
        w13_dgrad=w13b, dy_wgrad=oracle.mx_qdq_cols(dy, go), h_wgrad=oracle.mx_qdq_cols(h, go),
        x_wgrad=oracle.mx_qdq_cols(xq, go), mx_dgu=True)
    dx = oracle.combine(dxp, r["dst_row"], None, T, k, oracle.BF16)
    return dict(route=r, gu=gu, h=h, y=y, out=out, dy=dy, dgu=dgu, dxp=dxp, dw13=dw13, dw2=dw2,
                dx=dx)


@pytest.mark.parametrize("T,d,E,f,k,empty", [(600, 256, 5, 128, 1, None), (512, 384, 4, 256, 2, None),
                                              (300, 128, 16, 128, 1, None), (700, 256, 6, 384, 2, 3),
                                              (400, 128, 4, 128, 1, None), (1500, 256, 4, 256, 1, None)])
def test_mx_layer_fwd_bwd(moe, T, d, E, f, k, empty):
    _say("mx-layer", T, d, E, f, k, "empty expert", empty)
    _mx_layer_case(moe, T, d, E, f, k, empty)


def test_mx_layer_skewed_groups(moe):
    # Zipf(1.2) rows over 16 experts: contiguous weight-gradient tile ranges
    # would load the XCDs unevenly, so the kernel deals its tiles (checked
    # here on the CPU with the same cost model)
    T, d, E, f, k = 1500, 256, 16, 128, 1
    _say("mx-layer-skewed", T, d, E, f, k)
    logits = moe_synth.router_logits(T, E, seed=41, routing="zipf")
    counts = np.bincount(oracle.route(logits.numpy(), k)["topk_idx"].reshape(-1), minlength=E)
    tiles_e = 2 * ((d + 255) // 256) * ((f + 255) // 256)
    per = (E * tiles_e + 7) // 8
    xc = np.zeros(8)
    for e in range(E):
        c = -(-counts[e] // 128) * 128 + 256.0
        for x in range(8):
            xc[x] += max(0, min((e + 1) * tiles_e, (x + 1) * per) - max(e * tiles_e, x * per)) * c
    assert xc.max() > 1.05 * xc.mean(), "the case exercises the dealt tile mapping"
    _mx_layer_case(moe, T, d, E, f, k, None, logits=logits)


def _mx_layer_case(moe, T, d, E, f, k, empty, logits=None):
    from routing_grouped_gemm_amd.layer import MoELayer
    inp = moe_synth.make_inputs(T=T, d=d, E=E, f=f, k=k, seed=T + E)
    if logits is not None:
        inp["logits"] = logits
    if empty is not None:   # an expert no token picks: a zero-row group in every GEMM
        inp["logits"][:, empty] = -1e4
    inp["w13"] = (inp["w13"].float() * 3).to(torch.bfloat16)
    inp["x"] = (inp["x"].float() * 5).to(torch.bfloat16)
    gate = moe_synth.uniform01((T * k,), seed=T) if k == 1 else None
    lay = MoELayer(T, d, E, f, k, moe.MOE_MXFP8)
    g = {n: inp[n].cuda() for n in ("logits", "x", "w13", "w2", "dout")}
    lay.set_weights(g["w13"], g["w2"])
    w = gate.cuda() if gate is not None else None
    lay.forward(g["logits"], g["x"], weights=w)
    lay.backward(g["dout"], weights=w)
    torch.cuda.synchronize()
    ref = _mx_oracle(inp, k, gate.numpy() if gate is not None else None)
    if empty is not None:
        assert ref["route"]["counts"][empty] == 0
        assert float(lay.dw13[empty].abs().max()) == 0.0 and float(lay.dw2[empty].abs().max()) == 0.0
    np.testing.assert_array_equal(lay.dst_row.cpu().numpy(), ref["route"]["dst_row"])
    for name, t, rv in (("gu", lay.gu, ref["gu"]), ("h", lay.h, ref["h"]), ("y", lay.y_perm, ref["y"]),
                        ("out", lay.out, ref["out"]), ("dgu", lay.dgu, ref["dgu"]),
                        ("dx_perm", lay.dx_perm, ref["dxp"]), ("dx", lay.dx, ref["dx"]),
                        ("dw13", lay.dw13, ref["dw13"]), ("dw2", lay.dw2, ref["dw2"])):
        assert_close(np64(t), rv, MX_TOL, name)
    assert_close(np64(lay.dy_perm), ref["dy"], BF16_TOL, "dy_perm")
