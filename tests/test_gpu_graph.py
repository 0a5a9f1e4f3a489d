"""The layer's forward + backward step captured in a HIP graph and replayed.

Every call of the library enqueues kernels on the current stream and nothing
else (no allocation, host copy, synchronisation or memset), so a whole step
can be captured once and replayed.  The kernels are deterministic, so each
replay must reproduce the eager step bit for bit: replays run with new inputs
copied into the captured input buffers, with the outputs overwritten and
eager steps run in between, and each is compared with an eager step on the
same inputs.
"""
import sys

import pytest
import torch

import moe_synth

pytestmark = pytest.mark.gpu

DEV = "cuda"
OUTS = ("x_perm", "gu", "h", "y_perm", "out", "dy_perm", "dgu", "dx_perm", "dx", "dw13", "dw2")


def _say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def moe():
    import routing_grouped_gemm_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.load()
    return m


CASES = [
    # T, d, E, f, k, dtype, shared experts, capacity
    (384, 256, 8, 256, 2, "bf16", 0, 0),
    (300, 256, 6, 256, 2, "bf16", 1, 0),
    (400, 128, 8, 128, 2, "bf16", 0, 70),
    (256, 256, 4, 256, 1, "mxfp8", 0, 0),
]


@pytest.mark.parametrize("T,d,E,f,k,dt,S,C", CASES)
def test_layer_step_graph_replay(moe, T, d, E, f, k, dt, S, C):
    from routing_grouped_gemm_amd.layer import MoELayer
    _say("graph", T, d, E, f, k, dt, S, C)
    dtype = {"bf16": moe.MOE_BF16, "mxfp8": moe.MOE_MXFP8}[dt]
    sets = []
    for seed in (3, 4, 5):
        inp = moe_synth.make_inputs(T=T, d=d, E=E + S, f=f, k=k, seed=seed + T)
        inp["logits"] = inp["logits"][:, :E].contiguous()
        sets.append({n: inp[n].to(DEV) for n in ("logits", "x", "dout")})
    w = moe_synth.make_inputs(T=T, d=d, E=E + S, f=f, k=k, seed=99)
    lay = MoELayer(T, d, E, f, k, dtype, capacity=C, n_shared=S)
    lay.set_weights(w["w13"].to(DEV), w["w2"].to(DEV))
    static = {n: v.clone() for n, v in sets[0].items()}

    def step(src):
        lay.forward(src["logits"], src["x"])
        lay.backward(src["dout"])

    def eager(src):
        step(src)
        torch.cuda.synchronize()
        assert int(lay.dev_err.item()) == 0
        return {n: getattr(lay, n).clone() for n in OUTS}

    eager(static)                      # binds the stage tensors, allocates the backward buffers
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(static)                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(static)
    torch.cuda.synchronize()

    for rep, src in enumerate(sets + sets[:1]):
        ref = eager(src)
        for n in OUTS:
            getattr(lay, n).fill_(0)
        for n, v in src.items():
            static[n].copy_(v)
        g.replay()
        torch.cuda.synchronize()
        assert int(lay.dev_err.item()) == 0
        for n in OUTS:
            assert torch.equal(getattr(lay, n), ref[n]), f"replay {rep}: {n} differs from the eager step"
