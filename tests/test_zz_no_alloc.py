"""moe_route_topk_noalloc (the route with the library's fixed per-GPU scratch
instead of a caller workspace) against moe_route_topk, through the C ABI.

Two calls in a row on the same GPU, the second with a smaller input (fewer
tokens, fewer experts, padded), each compared bit for bit with the
workspace entry point on the same logits; then a size beyond the fixed
array is refused on the host.
"""
import ctypes
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[no-alloc]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def m():
    import routing_grouped_gemm_amd as m
    assert torch.cuda.is_available()
    m.load()
    return m


def _route_outputs(T, E, k, capacity):
    i32 = dict(dtype=torch.int32, device="cuda")
    n_rows = E * capacity if capacity else T * k
    return dict(idx=torch.full((T, k), -7, **i32),
                w=torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda"),
                counts=torch.full((E,), -7, **i32), offsets=torch.full((E + 1,), -7, **i32),
                dst=torch.full((T * k,), -7, **i32), src=torch.full((n_rows,), -7, **i32),
                err=torch.zeros(1, **i32)), n_rows


def _call(m, noalloc, logits, k, capacity):
    lib = m.load()
    T, E = logits.shape
    o, n_rows = _route_outputs(T, E, k, capacity)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = [p(logits), T, E, k, capacity, p(o["idx"]), p(o["w"]), p(o["counts"]), p(o["offsets"]),
            p(o["dst"]), p(o["src"]), n_rows]
    if noalloc:
        rc = lib.moe_route_topk_noalloc(*args, p(o["err"]), stream)
    else:
        ws = torch.empty(lib.moe_route_workspace_bytes(T, E, k), dtype=torch.uint8, device="cuda")
        rc = lib.moe_route_topk(*args, p(ws), ws.numel(), p(o["err"]), stream)
    assert rc == m.MOE_OK, m.moe_status_string(rc)
    torch.cuda.synchronize()
    return o


def test_noalloc_route_matches_workspace_route(m):
    g = torch.Generator(device="cuda").manual_seed(2024)
    cases = [(16384, 128, 4, 0), (1000, 64, 2, 40)]    # the second smaller, padded
    for T, E, k, cap in cases:
        _say(f"T={T} E={E} k={k} capacity={cap}")
        logits = torch.randn(T, E, generator=g, device="cuda", dtype=torch.float32)
        want = _call(m, False, logits, k, cap)
        got = _call(m, True, logits, k, cap)
        for name in ("idx", "counts", "offsets", "dst", "src", "err"):
            assert torch.equal(got[name], want[name]), f"{name} differs (T={T} E={E} k={k} C={cap})"
        assert torch.equal(got["w"].view(torch.int32), want["w"].view(torch.int32)), "topk_w bits differ"
        assert int(got["err"].item()) == 0
        assert int(got["offsets"][-1].item()) == T * k


def test_noalloc_route_size_limit(m):
    """A route whose scratch exceeds the fixed array is refused on the host
    (nothing is launched); the largest one that fits is accepted."""
    lib = m.load()
    E, k = 128, 4
    cap_bytes = m.ROUTE_NOALLOC_MAX_BYTES
    T_max = 4194240                                       # moe.h: largest T at E = 128
    assert lib.moe_route_workspace_bytes(T_max, E, k) <= cap_bytes
    assert lib.moe_route_workspace_bytes(T_max + 1, E, k) > cap_bytes
    fake = ctypes.c_void_p(0x10000)                        # never dereferenced: refused first
    T = T_max + 1
    rc = lib.moe_route_topk_noalloc(fake, T, E, k, 0, fake, fake, fake, fake, fake, fake, T * k, None, None)
    assert rc == m.MOE_EWORKSPACE
