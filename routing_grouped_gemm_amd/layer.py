"""One MoE feed-forward layer on one GPU, sequenced over the C ABI.

``MoELayer`` owns the device buffers of one layer shape and issues the ABI
calls in the order of the method (route -> permute -> grouped GEMM forward ->
combine, then the backward twins), all on one stream with no host
synchronisation.  It does no arithmetic of its own: every step runs in the
HIP library.  Buffers come from torch's caching allocator.

The backward of the layer with the routing held fixed:
    dy_perm = permute(dout, row_scale = topk_w)     (combine backward)
    dgu, dx_perm, dw13, dw2 = grouped_gemm_bwd(...)
    dx = unpermute_combine(dx_perm, weights = None) (permute backward)
"""
import torch

from . import (MOE_BF16, MOE_F32, MOE_GEMM_DGRAD_DOWN, MOE_GEMM_DGRAD_GATE_UP, MOE_GEMM_WGRAD,
               MOE_MXFP8,
               gemm_tensors, moe_gemm_workspace_bytes, moe_grouped_gemm_bwd, moe_grouped_gemm_fwd,
               moe_gate_grad, moe_grouped_gemm_op, moe_permute, moe_quantize_mxfp8,
               moe_route_add_shared, moe_route_topk, moe_route_workspace_bytes, moe_router_logits,
               moe_unpermute_combine)

_ACT = {MOE_F32: torch.float32, MOE_BF16: torch.bfloat16, MOE_MXFP8: torch.bfloat16}


class MoELayer:
    """n_shared > 0 adds that many shared experts (ungated, every token, weight
    1) as extra groups E .. E+n_shared-1 of the same grouped GEMM: weights are
    then [E + n_shared, ...] with the shared experts last, and the buffers hold
    the routed rows followed by n_shared * T shared rows."""

    def __init__(self, T, d, E, f, k, dtype=MOE_BF16, capacity=0, device="cuda", n_shared=0):
        self.T, self.d, self.E, self.f, self.k = T, d, E, f, k
        self.dtype, self.capacity, self.device = dtype, capacity, device
        self.S = n_shared
        self.K = k + n_shared                  # slots per token (routed, then shared)
        self.G = E + n_shared                  # GEMM groups
        self.R = E * capacity if capacity > 0 else T * k   # routed rows
        self.n_rows = self.R + n_shared * T
        R = self.n_rows
        act = _ACT[dtype]
        i32 = dict(dtype=torch.int32, device=device)
        self.topk_idx = torch.empty(T, k, **i32)
        self.topk_w = torch.empty(T, k, dtype=torch.float32, device=device)
        self.counts = torch.empty(E, **i32)
        self.offsets = torch.empty(E + 1, **i32)
        self.dst_row = torch.empty(T * k, **i32)
        self.src_slot = torch.empty(self.R, **i32)
        if n_shared:
            K, G = self.K, self.G
            self.s_idx = torch.empty(T, K, **i32)
            self.s_w = torch.empty(T, K, dtype=torch.float32, device=device)
            self.s_counts = torch.empty(G, **i32)
            self.s_off = torch.empty(G + 1, **i32)
            self.s_dst = torch.empty(T * K, **i32)
            self.s_src = torch.empty(R, **i32)
        else:
            self.s_idx, self.s_w, self.s_dst, self.s_src = self.topk_idx, self.topk_w, self.dst_row, self.src_slot
            self.s_counts, self.s_off = self.counts, self.offsets
        # group offsets and capacity the grouped GEMM takes (shared groups: explicit offsets)
        self.g_cap = 0 if n_shared else capacity
        self.dev_err = torch.zeros(1, **i32)
        self.route_ws = torch.empty(moe_route_workspace_bytes(T, E, k), dtype=torch.uint8,
                                    device=device)
        if dtype == MOE_MXFP8:
            self.x_perm = torch.empty(R, d, dtype=torch.uint8, device=device)
            self.x_perm_scales = torch.empty(R, d // 32, dtype=torch.uint8, device=device)
        else:
            self.x_perm = torch.empty(R, d, dtype=act, device=device)
            self.x_perm_scales = None
        self.gu = torch.empty(R, 2 * f, dtype=act, device=device)
        self.h = torch.empty(R, f, dtype=act, device=device)
        self.y_perm = torch.empty(R, d, dtype=act, device=device)
        self.out = torch.empty(T, d, dtype=act, device=device)
        self.gemm_ws = None
        wsb = moe_gemm_workspace_bytes(dtype, self.G, R, d, f)
        if wsb:
            self.gemm_ws = torch.empty(wsb, dtype=torch.uint8, device=device)
        self._bwd_alloc = False

    def _alloc_bwd(self):
        if self._bwd_alloc:
            return
        R, d, f, E = self.n_rows, self.d, self.f, self.G
        act = _ACT[self.dtype]
        dev = self.device
        self.dy_perm = torch.empty(R, d, dtype=act, device=dev)
        self.dgu = torch.empty(R, 2 * f, dtype=act, device=dev)
        self.dx_perm = torch.empty(R, d, dtype=act, device=dev)
        self.dx = torch.empty(self.T, d, dtype=act, device=dev)
        self.dw13 = torch.empty(E, 2 * f, d, dtype=act, device=dev)
        self.dw2 = torch.empty(E, d, f, dtype=act, device=dev)
        self._bwd_alloc = True

    # -------------------------------------------------------------- weights
    def set_weights(self, w13, w2):
        """Weights [E, 2f, d] and [E, d, f] (fp32 or bf16).  For MXFP8 the forward
        and backward MXFP8 caches are made here (once per optimizer step)."""
        self.w13, self.w2 = w13, w2
        self._stages = None
        if self.dtype != MOE_MXFP8:
            return
        E, f, d = self.G, self.f, self.d
        dev = self.device
        u8 = dict(dtype=torch.uint8, device=dev)
        # forward direction: blocks along the contraction dim of each GEMM
        self.w13_q = torch.empty(E * 2 * f, d, **u8)
        self.w13_s = torch.empty(E * 2 * f, d // 32, **u8)
        self.w2_q = torch.empty(E * d, f, **u8)
        self.w2_s = torch.empty(E * d, f // 32, **u8)
        # backward direction: each expert's matrix transposed, blocks along 2f / d
        # (column-wise quantiser layout: K * (rows + 128 * groups) codes)
        self._g13 = torch.arange(0, E + 1, dtype=torch.int32, device=dev) * (2 * f)
        self._g2 = torch.arange(0, E + 1, dtype=torch.int32, device=dev) * d
        n13 = d * (E * 2 * f + 128 * E)
        n2 = f * (E * d + 128 * E)
        self.w13t_q = torch.empty(n13, **u8)
        self.w13t_s = torch.empty(n13 // 32, **u8)
        self.w2t_q = torch.empty(n2, **u8)
        self.w2t_s = torch.empty(n2 // 32, **u8)
        self.requantize_weights()

    def requantize_weights(self):
        """MXFP8: rebuild the four weight caches (forward and backward direction
        of w13 and w2) from the bf16 weights in place, as an optimizer step does."""
        E, f, d = self.G, self.f, self.d
        moe_quantize_mxfp8(self.w13.reshape(E * 2 * f, d), 0, self.w13_q, self.w13_s)
        moe_quantize_mxfp8(self.w2.reshape(E * d, f), 0, self.w2_q, self.w2_s)
        moe_quantize_mxfp8(self.w13.reshape(E * 2 * f, d), 1, self.w13t_q, self.w13t_s, self._g13, E)
        moe_quantize_mxfp8(self.w2.reshape(E * d, f), 1, self.w2t_q, self.w2t_s, self._g2, E)

    # -------------------------------------------------------------- stages
    def _stage_tensors(self):
        """Operands of the five grouped GEMM stages: (forward-direction set,
        backward-direction set); they differ only in the MXFP8 weight caches."""
        self._alloc_bwd()
        common = dict(x_perm=self.x_perm, x_perm_scales=self.x_perm_scales, gu=self.gu, h=self.h,
                      y_perm=self.y_perm, dy_perm=self.dy_perm, dgu=self.dgu, dx_perm=self.dx_perm,
                      dw13=self.dw13, dw2=self.dw2, ws=self.gemm_ws)
        if self.dtype != MOE_MXFP8:
            t = gemm_tensors(w13=self.w13, w2=self.w2, **common)
            return t, t
        fwd = gemm_tensors(w13=self.w13_q, w13_scales=self.w13_s, w2=self.w2_q,
                           w2_scales=self.w2_s, **common)
        bwd = gemm_tensors(w13=self.w13t_q, w13_scales=self.w13t_s, w2=self.w2t_q,
                           w2_scales=self.w2t_s, **common)
        return fwd, bwd

    def gemm_stage(self, op):
        """Issue one grouped GEMM stage (MOE_GEMM_*) on the layer's buffers (the
        forward and backward calls are these stages in order).  Call
        set_weights first; the tensors are bound on first use."""
        if getattr(self, "_stages", None) is None:
            self._stages = self._stage_tensors()
        bwd = op in (MOE_GEMM_DGRAD_DOWN, MOE_GEMM_DGRAD_GATE_UP)
        moe_grouped_gemm_op(op, self.dtype, self._stages[1 if bwd else 0], self.s_off,
                            self.g_cap, self.G, self.n_rows, self.d, self.f)

    def wgrad_accumulate(self, dw13_f32, dw2_f32):
        """bf16: the weight-gradient stage adding into fp32 accumulators
        (dw13_f32 += dgu^T x_perm, dw2_f32 += dy_perm^T h, per expert) instead
        of writing the bf16 dw13 / dw2.  Call after backward (it reads dgu)."""
        self._alloc_bwd()
        t = gemm_tensors(x_perm=self.x_perm, h=self.h, dy_perm=self.dy_perm, dgu=self.dgu,
                         dw13_f32=dw13_f32, dw2_f32=dw2_f32, ws=self.gemm_ws)
        moe_grouped_gemm_op(MOE_GEMM_WGRAD, self.dtype, t, self.s_off, self.g_cap, self.G,
                            self.n_rows, self.d, self.f)

    # -------------------------------------------------------------- steps
    def route(self, logits):
        moe_route_topk(logits, self.k, self.capacity, self.topk_idx, self.topk_w, self.counts,
                       self.offsets, self.dst_row, self.src_slot, self.route_ws, self.dev_err)
        if self.S:
            moe_route_add_shared(self.S, self.capacity, self.topk_idx, self.topk_w, self.dst_row,
                                 self.counts, self.offsets, self.src_slot, self.s_idx, self.s_w,
                                 self.s_counts, self.s_off, self.s_dst, self.s_src)

    def permute(self, x):
        moe_permute(self.dtype, x, self.K, self.s_dst, self.x_perm, src_slot=self.s_src,
                    x_perm_scales=self.x_perm_scales, dev_err=self.dev_err)

    def gemm_fwd(self):
        if self.dtype == MOE_MXFP8:
            moe_grouped_gemm_fwd(self.dtype, self.x_perm, self.w13_q, self.w2_q, self.s_off,
                                 self.g_cap, self.gu, self.h, self.y_perm,
                                 x_perm_scales=self.x_perm_scales, w13_scales=self.w13_s,
                                 w2_scales=self.w2_s, ws=self.gemm_ws)
        else:
            moe_grouped_gemm_fwd(self.dtype, self.x_perm, self.w13, self.w2, self.s_off,
                                 self.g_cap, self.gu, self.h, self.y_perm)

    def _slot_weights(self, weights):
        if weights is None or weights is self.s_w:
            return self.s_w
        assert not self.S, "per-row weights are not combined with shared experts"
        return weights

    def combine(self, weights=None):
        moe_unpermute_combine(MOE_F32 if self.dtype == MOE_F32 else MOE_BF16, self.y_perm,
                              self.s_dst, self._slot_weights(weights), self.K, self.out,
                              dev_err=self.dev_err)

    def router_scores(self, x, w_router):
        """Router scores [T, E] fp32 = x . w_router^T (bf16 x and w_router [E, d])."""
        if getattr(self, "logits", None) is None:
            self.logits = torch.empty(self.T, self.E, dtype=torch.float32, device=x.device)
        moe_router_logits(x, w_router, self.logits)
        return self.logits

    def gate_grad(self, dout):
        """dlogits [T, E] fp32: the gradient of <dout, out> through the gate
        weights of the last forward (bf16 activations; call after forward)."""
        if getattr(self, "dlogits", None) is None:
            self.dlogits = torch.empty(self.T, self.E, dtype=torch.float32, device=dout.device)
        moe_gate_grad(dout, self.y_perm, self.topk_idx, self.topk_w, self.dst_row, self.dlogits,
                      dev_err=self.dev_err)
        return self.dlogits

    def forward(self, logits, x, weights=None):
        self.route(logits)
        self.permute(x)
        self.gemm_fwd()
        self.combine(weights)
        return self.out

    def backward(self, dout, weights=None):
        self._alloc_bwd()
        act_dt = MOE_F32 if self.dtype == MOE_F32 else MOE_BF16
        moe_permute(act_dt, dout, self.K, self.s_dst, self.dy_perm, src_slot=self.s_src,
                    row_scale=self._slot_weights(weights), dev_err=self.dev_err)
        if self.dtype == MOE_MXFP8:
            moe_grouped_gemm_bwd(self.dtype, self.dy_perm, self.x_perm, self.gu, self.h,
                                 self.w13t_q, self.w2t_q, self.s_off, self.g_cap, self.dgu,
                                 self.dx_perm, self.dw13, self.dw2,
                                 x_perm_scales=self.x_perm_scales, w13_scales=self.w13t_s,
                                 w2_scales=self.w2t_s, ws=self.gemm_ws)
        else:
            moe_grouped_gemm_bwd(self.dtype, self.dy_perm, self.x_perm, self.gu, self.h,
                                 self.w13, self.w2, self.s_off, self.g_cap, self.dgu,
                                 self.dx_perm, self.dw13, self.dw2, ws=self.gemm_ws)
        moe_unpermute_combine(act_dt, self.dx_perm, self.s_dst, None, self.K, self.dx,
                              dev_err=self.dev_err)
        return self.dx, self.dw13, self.dw2
