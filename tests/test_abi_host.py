"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/moe.h declares, and rejects bad arguments on the
host before anything is enqueued.  Every call below fails validation, so no
kernel is ever launched from these tests.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def m():
    import routing_grouped_gemm_amd as m
    if not os.path.exists(m.LIB_PATH):
        pytest.skip("libmoe.so not built")
    return m


def _declared():
    text = open(HEADER).read()
    return set(re.findall(r"MOE_API\s+[\w\s\*]*?\b(moe_\w+)\s*\(", text))


def test_header_declares_the_abi(m):
    assert _declared() == set(m.ABI_FUNCTIONS)


def test_library_exports_every_declared_symbol(m):
    out = subprocess.run(["nm", "-D", "--defined-only", m.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert _declared() <= exported
    lib = m.load()
    for name in _declared():
        assert hasattr(lib, name)


def test_header_compiles_as_c():
    src = '#include "moe.h"\nint main(void){return moe_version() > 0 ? 0 : 1;}\n'
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only",
                        "-I" + os.path.dirname(HEADER), "-x", "c", "-"], input=src,
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_version_and_status_strings(m):
    assert m.moe_version() >= 100
    for st in (m.MOE_OK, m.MOE_EINVAL, m.MOE_EALIGN, m.MOE_EUNSUPPORTED, m.MOE_EWORKSPACE,
               m.MOE_EHIP):
        assert m.moe_status_string(st).startswith("MOE_")
    assert "unknown" in m.moe_status_string(12345)


def test_route_workspace_formula(m):
    assert m.moe_route_workspace_bytes(-1, 8, 2) == 0
    a = m.moe_route_workspace_bytes(16384, 128, 4)
    # one histogram row of E int32 per 64 tokens, plus alignment slack
    assert a >= 256 * 128 * 4
    assert a < 256 * 128 * 4 + 1024
    # bf16: only the weight gradient's control words; fp32: none
    assert m.moe_gemm_workspace_bytes(m.MOE_BF16, 8, 1000, 128, 128) == 256
    assert m.moe_gemm_workspace_bytes(m.MOE_F32, 8, 1000, 128, 128) == 0


FAKE = 0x10000          # 16-byte aligned, never dereferenced (validation fails first)


def test_route_argument_validation(m):
    lib = m.load()
    P = FAKE
    ws = m.moe_route_workspace_bytes(100, 8, 2)

    def call(T=100, E=8, k=2, C=0, n_rows=200, wsb=ws, logits=P, counts=P, src=P):
        return lib.moe_route_topk(logits, T, E, k, C, P, P, counts, P, P, src, n_rows, P, wsb,
                                  None, None)
    assert call(k=9) == m.MOE_EINVAL                # k > 8
    assert call(E=4, k=5) == m.MOE_EINVAL           # k > E
    assert call(E=1025) == m.MOE_EINVAL             # too many experts
    assert call(T=-1) == m.MOE_EINVAL
    assert call(n_rows=199) == m.MOE_EINVAL         # n_rows != T*k
    assert call(C=30, n_rows=200) == m.MOE_EINVAL   # padded: n_rows must be E*C
    assert call(logits=None) == m.MOE_EINVAL
    assert call(counts=None) == m.MOE_EINVAL
    assert call(src=None) == m.MOE_EINVAL
    assert call(wsb=ws - 1) == m.MOE_EWORKSPACE
    assert call(C=-1) == m.MOE_EINVAL


def test_permute_and_combine_validation(m):
    lib = m.load()
    P = FAKE
    assert lib.moe_permute(9, P, 10, 64, 2, P, None, None, 20, P, None, None, None) == \
        m.MOE_EUNSUPPORTED
    assert lib.moe_permute(m.MOE_BF16, P, 10, 60, 2, P, None, None, 20, P, None, None, None) == \
        m.MOE_EALIGN                                # d % 8
    assert lib.moe_permute(m.MOE_BF16, P + 8, 10, 64, 2, P, None, None, 20, P, None, None,
                           None) == m.MOE_EALIGN     # pointer alignment
    assert lib.moe_permute(m.MOE_BF16, P, 10, 64, 2, P, None, None, 24, P, None, None, None) == \
        m.MOE_EINVAL                                # padded layout needs src_slot
    assert lib.moe_permute(m.MOE_MXFP8, P, 10, 64, 2, P, None, P, 20, P, P, None, None) == \
        m.MOE_EUNSUPPORTED                          # no row scale with MXFP8
    assert lib.moe_permute(m.MOE_MXFP8, P, 10, 48, 2, P, None, None, 20, P, P, None, None) == \
        m.MOE_EALIGN                                # d % 32 for MXFP8
    assert lib.moe_permute(m.MOE_BF16, P, 10, 64, 9, P, None, None, 90, P, None, None, None) == \
        m.MOE_EINVAL                                # k > 8
    assert lib.moe_unpermute_combine(m.MOE_MXFP8, P, P, None, 10, 2, 64, 20, P, None, None) == \
        m.MOE_EUNSUPPORTED
    assert lib.moe_unpermute_combine(m.MOE_BF16, P, None, None, 10, 2, 64, 20, P, None, None) == \
        m.MOE_EINVAL
    assert lib.moe_unpermute_combine(m.MOE_F32, P, P, None, 10, 2, 66, 20, P, None, None) == \
        m.MOE_EALIGN


def test_gemm_validation(m):
    lib = m.load()
    P = FAKE

    def fwd(dtype=m.MOE_BF16, goff=P, C=0, E=8, n_rows=100, d=128, f=128, w13=P, ws=None,
            wsb=0, xs=None):
        return lib.moe_grouped_gemm_fwd(dtype, P, xs, w13, xs, P, xs, goff, C, E, n_rows, d, f,
                                        P, P, P, ws, wsb, None)
    assert fwd(dtype=5) == m.MOE_EUNSUPPORTED
    assert fwd(goff=None) == m.MOE_EINVAL           # unpadded needs group offsets
    assert fwd(C=10, n_rows=100, goff=None) == m.MOE_EINVAL   # E*C != n_rows
    assert fwd(E=0) == m.MOE_EINVAL
    assert fwd(E=2000) == m.MOE_EINVAL
    assert fwd(d=100) == m.MOE_EALIGN
    assert fwd(f=12) == m.MOE_EALIGN
    assert fwd(w13=None) == m.MOE_EINVAL
    assert fwd(w13=P + 2) == m.MOE_EALIGN
    assert fwd(dtype=m.MOE_MXFP8, d=128, f=80) == m.MOE_EALIGN
    assert fwd(dtype=m.MOE_MXFP8, xs=None) == m.MOE_EINVAL    # scales required
    assert fwd(dtype=m.MOE_MXFP8, xs=P, ws=None) == m.MOE_EWORKSPACE
    assert lib.moe_grouped_gemm_bwd(m.MOE_BF16, P, P, None, P, P, P, None, P, None, P, 0, 8, 100,
                                    128, 128, P, P, None, P, None, 0, None) == m.MOE_EINVAL
    # the bf16 backward needs the (small) workspace of its weight-gradient stage
    wsb16 = lib.moe_gemm_workspace_bytes(m.MOE_BF16, 8, 100, 128, 128)
    assert wsb16 > 0 and lib.moe_gemm_workspace_bytes(m.MOE_F32, 8, 100, 128, 128) == 0
    for ws, wsb in ((None, wsb16), (P, wsb16 - 1), (P + 4, wsb16)):
        assert lib.moe_grouped_gemm_bwd(m.MOE_BF16, P, P, None, P, P, P, None, P, None, P, 0, 8, 100,
                                        128, 128, P, P, P, P, ws, wsb, None) == m.MOE_EWORKSPACE
    # one MXFP8 stage: scales of the operands it reads, and the workspace for
    # every stage (GATE_UP leaves the MXFP8 copy of h there for DOWN)
    t = m.MoeGemmTensors(**{n: P for n in m.GEMM_TENSOR_FIELDS})
    t.ws = None

    def op(o, t=t):
        return lib.moe_grouped_gemm_op(o, m.MOE_MXFP8, ctypes.byref(t), P, 0, 8, 100, 128, 128, None)
    for o in (m.MOE_GEMM_GATE_UP, m.MOE_GEMM_DOWN, m.MOE_GEMM_DGRAD_DOWN, m.MOE_GEMM_DGRAD_GATE_UP,
              m.MOE_GEMM_WGRAD):
        assert op(o) == m.MOE_EWORKSPACE
    t.ws, t.ws_bytes = P, lib.moe_gemm_workspace_bytes(m.MOE_MXFP8, 8, 100, 128, 128) - 1
    assert op(m.MOE_GEMM_DOWN) == m.MOE_EWORKSPACE
    t.w13_scales = None
    assert op(m.MOE_GEMM_GATE_UP) == m.MOE_EINVAL
    assert op(m.MOE_GEMM_DGRAD_GATE_UP) == m.MOE_EINVAL
    assert op(7) == m.MOE_EINVAL
    assert lib.moe_quantize_mxfp8(P, 10, 48, 0, None, 0, P, P, None) == m.MOE_EALIGN
    assert lib.moe_quantize_mxfp8(P, -1, 64, 0, None, 0, P, P, None) == m.MOE_EINVAL
    assert lib.moe_quantize_mxfp8(P, 10, 64, 1, P, 0, P, P, None) == m.MOE_EINVAL
    # column-wise: 16-byte source rows and whole scale words
    assert lib.moe_quantize_mxfp8(P, 10, 60, 1, None, 0, P, P, None) == m.MOE_EALIGN
    assert lib.moe_quantize_mxfp8(P, 10, 64, 1, None, 0, P, P + 2, None) == m.MOE_EALIGN


def test_router_and_gate_grad_validation(m):
    lib = m.load()
    P = FAKE

    def rl(x=P, w=P, T=100, E=8, d=64, lg=P):
        return lib.moe_router_logits(x, w, T, E, d, lg, None)
    assert rl(E=0) == m.MOE_EINVAL
    assert rl(E=1025) == m.MOE_EINVAL
    assert rl(T=-1) == m.MOE_EINVAL
    assert rl(x=None) == m.MOE_EINVAL
    assert rl(d=12) == m.MOE_EALIGN
    assert rl(x=P + 8) == m.MOE_EALIGN
    assert rl(T=0, x=None, w=None, lg=None) == m.MOE_OK     # nothing to do, nothing launched

    def gg(T=100, E=8, k=2, d=64, n_rows=200, dout=P, y=P, dl=P, dyp=None):
        return lib.moe_gate_grad(dout, y, P, P, P, T, E, k, d, n_rows, dl, None, dyp, None, None)
    assert gg(k=0) == m.MOE_EINVAL
    assert gg(k=9) == m.MOE_EINVAL
    assert gg(E=1, k=2) == m.MOE_EINVAL              # k > E
    assert gg(dout=None) == m.MOE_EINVAL
    assert gg(dl=None) == m.MOE_EINVAL
    assert gg(d=20) == m.MOE_EALIGN
    assert gg(y=P + 4) == m.MOE_EALIGN
    assert gg(n_rows=240, dyp=P) == m.MOE_EUNSUPPORTED      # padded layout + fused combine backward
    assert gg(T=0, n_rows=0, dout=None, y=None, dl=None) == m.MOE_OK


def test_route_add_shared_validation(m):
    lib = m.load()
    P = FAKE

    def call(T=100, E=8, k=2, S=1, C=0, n_rows=200, counts=P, src=P):
        return lib.moe_route_add_shared(T, E, k, S, C, P, P, P, counts, P, src, n_rows, P, P, P, P, P, P, None)
    assert call(S=0) == m.MOE_EINVAL
    assert call(k=7, S=2) == m.MOE_EINVAL          # k + n_shared > 8
    assert call(E=1024, S=1) == m.MOE_EINVAL       # E + n_shared > 1024
    assert call(n_rows=199) == m.MOE_EINVAL        # not the route's row count
    assert call(C=30, n_rows=200) == m.MOE_EINVAL  # padded: n_rows = E*C
    assert call(counts=None) == m.MOE_EINVAL
    assert call(src=None) == m.MOE_EINVAL


def test_wgrad_fp32_accumulate_validation(m):
    lib = m.load()
    P = FAKE
    t = m.MoeGemmTensors(**{n: P for n in m.GEMM_TENSOR_FIELDS})

    def op(o, dtype=m.MOE_BF16, t=t):
        return lib.moe_grouped_gemm_op(o, dtype, ctypes.byref(t), P, 0, 8, 0, 128, 128, None)
    t.dw13_f32, t.dw2_f32 = P, None
    assert op(m.MOE_GEMM_WGRAD) == m.MOE_EINVAL               # both accumulators or neither
    t.dw2_f32 = P + 8
    assert op(m.MOE_GEMM_WGRAD) == m.MOE_EALIGN
    t.dw2_f32 = P
    assert op(m.MOE_GEMM_DGRAD_GATE_UP) == m.MOE_EUNSUPPORTED  # accumulate-into is a WGRAD option
    assert op(m.MOE_GEMM_WGRAD, dtype=m.MOE_F32) == m.MOE_EUNSUPPORTED
    t.dw13_f32, t.dw2_f32, t.dy_perm = P, P, None
    assert op(m.MOE_GEMM_WGRAD) == m.MOE_EINVAL               # operands still required
    t.dy_perm, t.ws, t.ws_bytes = P, None, 0
    assert op(m.MOE_GEMM_WGRAD) == m.MOE_EWORKSPACE           # the stage's control words


def test_gemm_tensors_struct_matches_header(m, tmp_path):
    """The ctypes mirror of moe_gemm_tensors has the C struct's size and offsets."""
    fields = list(m.GEMM_TENSOR_FIELDS) + ["ws_bytes"] + list(m.GEMM_TENSOR_FIELDS_F32)
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "moe.h"\nint main(void){\n'
                   '  printf("%zu\\n", sizeof(moe_gemm_tensors));\n'
                   + "".join(f'  printf("%zu\\n", offsetof(moe_gemm_tensors, {f}));\n' for f in fields)
                   + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    assert got[0] == ctypes.sizeof(m.MoeGemmTensors)
    assert got[1:] == [getattr(m.MoeGemmTensors, f).offset for f in fields]
