"""Benchmark of one GPU's MoE feed-forward layer (fwd + bwd) on MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload e128]

A step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM: route (top-k + route map) -> permute -> grouped
GEMM gate/up (+SwiGLU) -> grouped GEMM down -> combine, then the backward:
combine-backward (permute with row scale) -> grouped GEMM dgrad of the down
projection (+SwiGLU backward) -> grouped GEMM dgrad of gate/up -> grouped
GEMM weight gradients -> permute-backward (unweighted combine).  Every stage
is one C-ABI call on one stream; each is bracketed by HIP events in every
timed step.  Rank 0 prints one JSON line.

The default workload is the one the metric names (E=128 experts, top-4,
bf16): T=16384 tokens, d_model=4096, d_ff=1536, uniform-random routing.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + grouped-GEMM TFLOP/s (% MFMA peak), E=128 top-4 bf16"
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0        # MI355X dense fp8 (and MX-scaled fp8) MFMA
PEAK_F32_TFLOPS = 157.3         # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E

STAGES = ["route", "permute", "gemm_gate_up", "gemm_down", "combine", "combine_bwd",
          "gemm_dgrad_down", "gemm_dgrad_gate_up", "gemm_wgrad", "permute_bwd"]
KERNEL_NAMES = {
    "gemm_gate_up": "gemm_grouped_m_kernel<256, 64, 2, false, 1, 8, true> (gate/up + SwiGLU)",
    "gemm_down": "gemm_grouped_m_kernel<256, 64, 2, false, 0, 8, true> (down)",
    "gemm_dgrad_down": "gemm_grouped_m_kernel<256, 64, 2, true, 2, 8, true> (dgrad down + SwiGLU bwd)",
    "gemm_dgrad_gate_up": "gemm_grouped_m_kernel<256, 64, 2, true, 0, 8, true> (dgrad gate/up)",
    "gemm_wgrad": "k_deal_flag_kernel + gemm_grouped_k_persistent<8> (wgrad, dWd and dW13 in one launch)",
    "permute": "permute_kernel<true, false, {k}>",
    "combine": "combine_kernel<true, {k}>",
    "combine_bwd": "permute_kernel<true, true, {k}>",
    "permute_bwd": "combine_kernel<true, {k}>",
    "route": "route_topk_kernel + route_scan_kernel + route_finalize_kernel",
}
KERNEL_NAMES_MX = {
    "gemm_gate_up": "mx_grouped_m_kernel<256, 1, 8> (gate/up + SwiGLU)",
    "gemm_down": "mx_grouped_m_kernel<256, 0, 8> (down; h quantised by the gate/up epilogue)",
    "gemm_dgrad_down": "quant_rows_kernel (dy) + mx_grouped_m_kernel<256, 2, 8> (dgrad down + SwiGLU bwd)",
    "gemm_dgrad_gate_up": "mx_grouped_m_kernel<256, 0, 8> (dgrad gate/up; dgu quantised by the dgrad-down epilogue)",
    "gemm_wgrad": "4 x quant_cols_kernel + mx_k_deal_flag_kernel + mx_grouped_k_kernel<256, 8> (wgrad, dWd and dW13)",
    "permute": "permute_mx_kernel",
    "combine": "combine_kernel<true, {k}>",
    "combine_bwd": "permute_kernel<true, true, {k}>",
    "permute_bwd": "combine_kernel<true, {k}>",
    "route": "route_topk_kernel + route_scan_kernel + route_finalize_kernel",
}


def kernel_name(stage, k, mx=False):
    """The kernel(s) a stage launches (templates as the profiler names them)."""
    return (KERNEL_NAMES_MX if mx else KERNEL_NAMES).get(stage, stage).format(k=k)


PROFILES = os.path.join(ROOT, "profiles")
_CSRC = "routing_grouped_gemm_amd/csrc/"
# the sources each stage's kernels are compiled from (a traffic record is
# only valid for the exact sources it was measured on)
KERNEL_SOURCES = {"gemm": ["gemm_bf16.hip", "gemm_common.h", "moe_internal.h"],
                  "gemm_mx": ["gemm_mxfp8.hip", "gemm_common.h", "moe_internal.h", "permute.hip"],
                  "route": ["route.hip", "moe_internal.h"],
                  "permute": ["permute.hip", "moe_internal.h"],
                  "combine": ["permute.hip", "moe_internal.h"]}


def source_hash(stage, mx=False):
    import hashlib
    key = stage.split("_")[0]
    if key == "gemm" and mx:
        key = "gemm_mx"
    h = hashlib.sha256()
    for name in KERNEL_SOURCES.get(key, KERNEL_SOURCES["permute"]):
        h.update(open(os.path.join(ROOT, _CSRC, name), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(stage, workload, mx=False):
    """HBM bytes per launch of `stage` from the committed counter record
    (profiles/traffic_<stage>_<workload>.json), or None when there is none or
    the kernel source changed since the counters were taken."""
    path = os.path.join(PROFILES, f"traffic_{stage}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256_16") != source_hash(stage, mx):
        return None
    return rec.get("hbm_bytes_per_launch")


def copy_calibration(nbytes=1 << 31, iters=5):
    """A plain device copy of known size (for scaling FETCH_SIZE / WRITE_SIZE)."""
    import torch
    a = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").normal_()
    b = torch.empty_like(a)
    for _ in range(iters):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": nbytes, "bytes_written": nbytes,
                      "iters": iters}), flush=True)


def roofline(attainable_peak, bandwidth, intensity):
    """Attainable throughput = min(peak compute, peak bandwidth x intensity)."""
    return min(attainable_peak, bandwidth * intensity)


MX_ELEM = 1 + 1 / 32             # bytes per MXFP8 element: E4M3 code + its share of the E8M0 scale


def stage_work(name, T, d, E, f, k, R, elem=2, mx=False):
    """Algorithmic (FLOPs, HBM bytes) of one stage: useful work only, padding
    rows never counted; bytes = each operand read once and each result
    written once.  MXFP8 (mx=True): the dispatch payload and the weights are
    read as codes + scales, every other activation is bf16 (a stage's own
    quantisation of a bf16 operand is internal to the stage)."""
    if mx:
        return _stage_work_mx(name, T, d, E, f, k, R)
    a = elem
    if name == "route":
        return 0, T * E * 4 + T * k * (4 + 4 + 4) + R * 4 + E * 8
    if name in ("permute", "combine_bwd"):
        return 0, T * d * a + R * d * a + T * k * 4 + (T * k * 4 if name == "combine_bwd" else 0)
    if name in ("combine", "permute_bwd"):
        return 0, R * d * a + T * d * a + T * k * 4 + (T * k * 4 if name == "combine" else 0)
    W13, W2 = E * 2 * f * d * a, E * d * f * a
    if name == "gemm_gate_up":
        return 4 * R * d * f, R * d * a + W13 + R * 3 * f * a
    if name == "gemm_down":
        return 2 * R * d * f, R * f * a + W2 + R * d * a
    if name == "gemm_dgrad_down":
        return 2 * R * d * f, R * d * a + W2 + R * 2 * f * a * 2
    if name == "gemm_dgrad_gate_up":
        return 4 * R * d * f, R * 2 * f * a + W13 + R * d * a
    if name == "gemm_wgrad":
        return 6 * R * d * f, R * d * a + R * f * a + R * 2 * f * a + R * d * a + W13 + W2
    raise KeyError(name)


def _stage_work_mx(name, T, d, E, f, k, R):
    q, a = MX_ELEM, 2
    W13, W2 = E * 2 * f * d * q, E * d * f * q
    if name == "permute":
        return 0, T * d * a + R * d * q + T * k * 4
    if name == "gemm_gate_up":
        return 4 * R * d * f, R * d * q + W13 + R * 3 * f * a
    if name == "gemm_wgrad":
        return 6 * R * d * f, R * d * a + R * f * a + R * 2 * f * a + R * d * q + 2 * (W13 + W2) / q
    if name.startswith("gemm"):
        fl, by = stage_work(name, T, d, E, f, k, R, 2)
        return fl, by - (E * 2 * f * d * a if "gate_up" in name else E * d * f * a) + \
            (W13 if "gate_up" in name else W2)
    return stage_work(name, T, d, E, f, k, R, 2)


def run_gpu(args, cfg):
    import torch

    import moe_synth
    import routing_grouped_gemm_amd as m
    from routing_grouped_gemm_amd.layer import MoELayer

    T, d, E, f, k = cfg["T"], cfg["d"], cfg["E"], cfg["f"], cfg["k"]
    dt = {"bf16": m.MOE_BF16, "f32": m.MOE_F32, "mxfp8": m.MOE_MXFP8}[cfg["dtype"]]
    cap = 0
    if args.padded:
        cap = moe_synth.capacity_of(T, k, E, cfg.get("capacity_factor", 1.25))
    inp = moe_synth.make_inputs(args.workload, device="cuda")
    S = cfg.get("n_shared", 0)
    lay = MoELayer(T, d, E, f, k, dt, capacity=cap, n_shared=S)
    lay.set_weights(inp["w13"], inp["w2"])
    lay._alloc_bwd()
    R = lay.n_rows
    act_dt = m.MOE_F32 if dt == m.MOE_F32 else m.MOE_BF16
    # combine weights: the router's softmax weights, or the per-row gate a
    # received expert-parallel shard comes with
    wts = inp["gate"] if "gate" in inp else lay.s_w

    def step(ev):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        lay.route(inp["logits"])
        mark(1)
        lay.permute(inp["x"])
        mark(2)
        lay.gemm_stage(m.MOE_GEMM_GATE_UP)
        mark(3)
        lay.gemm_stage(m.MOE_GEMM_DOWN)
        mark(4)
        lay.combine(wts)
        mark(5)
        m.moe_permute(act_dt, inp["dout"], lay.K, lay.s_dst, lay.dy_perm, src_slot=lay.s_src,
                      row_scale=wts, dev_err=lay.dev_err)
        mark(6)
        lay.gemm_stage(m.MOE_GEMM_DGRAD_DOWN)
        mark(7)
        lay.gemm_stage(m.MOE_GEMM_DGRAD_GATE_UP)
        mark(8)
        lay.gemm_stage(m.MOE_GEMM_WGRAD)
        mark(9)
        m.moe_unpermute_combine(act_dt, lay.dx_perm, lay.s_dst, None, lay.K, lay.dx,
                                dev_err=lay.dev_err)
        mark(10)

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)]
           for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert int(lay.dev_err.item()) == 0, "device reported a data fault"
    stage_ms = {}
    for j, s in enumerate(STAGES):
        stage_ms[s] = sum(evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(K)) / K
    gpu_ms = sum(evs[i][0].elapsed_time(evs[i][len(STAGES)]) for i in range(K)) / K
    ms_per_step = wall * 1e3 / K
    counts = lay.counts.cpu()
    cold = cold_cache(lay, inp, wts, act_dt, T, d, k, max(5, min(K, 10))) if dt != m.MOE_F32 and not S else None
    f1 = router_steps(lay, inp, K) if dt == m.MOE_BF16 and not cap else None
    f4 = wgrad_f32_accumulate(lay, K) if dt == m.MOE_BF16 and not cap else None
    wq = weight_requant(lay, K) if dt == m.MOE_MXFP8 else None
    return dict(stage_ms=stage_ms, gpu_ms=gpu_ms, ms_per_step=ms_per_step, R=R, cap=cap, f1=f1, wq=wq, f4=f4,
                cold=cold,
                counts=counts, inp=inp, lay=lay)


def cold_cache(lay, inp, wts, act_dt, T, d, k, reps):
    """The HBM-bound stages timed one launch at a time with the caches cold:
    before each repetition a 1 GiB buffer is written (more than the 256 MB
    last-level cache and every L2 hold), so the stage's operands come from
    HBM.  Median over `reps` launches of permute, combine, combine-backward
    and permute-backward; bytes as in stage_work (each operand once)."""
    import torch
    import routing_grouped_gemm_amd as m
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    calls = {
        "permute": lambda: lay.permute(inp["x"]),
        "combine": lambda: lay.combine(wts),
        "combine_bwd": lambda: m.moe_permute(act_dt, inp["dout"], lay.K, lay.s_dst, lay.dy_perm,
                                             src_slot=lay.s_src, row_scale=wts, dev_err=lay.dev_err),
        "permute_bwd": lambda: m.moe_unpermute_combine(act_dt, lay.dx_perm, lay.s_dst, None, lay.K, lay.dx,
                                                       dev_err=lay.dev_err),
    }
    mx = lay.dtype == m.MOE_MXFP8
    out = {}
    for name, fn in calls.items():
        ms = []
        for _ in range(reps):
            flush.fill_(1)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        ms.sort()
        med = ms[len(ms) // 2]
        _, by = stage_work(name, T, d, lay.E, lay.f, k, lay.n_rows if not lay.capacity else
                           int((lay.dst_row >= 0).sum().item()), 2, mx and name == "permute")
        out[name] = {"ms": round(med, 4), "gbs": round(by / med / 1e6, 1),
                     "frac_hbm": round(by / med / 1e6 / PEAK_HBM_GBS, 4), "bytes": by}
    del flush
    return out


def route_stress(reps, T=1 << 20, E=128, k=4):
    """The route (top-k, histogram, scan, destination rows) alone at a large
    token count, where its HBM traffic is big enough to measure: T = 2^20
    tokens x E = 128 fp32 logits (537 MB), iid N(0, 1), top-4, each launch
    bracketed by events; bytes as in stage_work('route')."""
    import torch
    import moe_synth
    import routing_grouped_gemm_amd as m
    logits = moe_synth.normal((T, E), 1.0, 4242, "cuda")
    i32 = dict(dtype=torch.int32, device="cuda")
    idx = torch.empty(T, k, **i32)
    w = torch.empty(T, k, dtype=torch.float32, device="cuda")
    counts = torch.empty(E, **i32)
    offsets = torch.empty(E + 1, **i32)
    dst = torch.empty(T * k, **i32)
    src = torch.empty(T * k, **i32)
    ws = torch.empty(m.moe_route_workspace_bytes(T, E, k), dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, **i32)

    def run():
        m.moe_route_topk(logits, k, 0, idx, w, counts, offsets, dst, src, ws, dev_err=err)
    run()
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        run()
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    ms.sort()
    med = ms[len(ms) // 2]
    assert int(offsets[-1].item()) == T * k and int(err.item()) == 0
    _, by = stage_work("route", T, 0, E, 0, k, T * k)
    del logits, ws
    return {"tokens": T, "experts": E, "top_k": k, "ms": round(med, 4), "gbs": round(by / med / 1e6, 1),
            "frac_hbm": round(by / med / 1e6 / PEAK_HBM_GBS, 4), "bytes": by}


def router_steps(lay, inp, reps):
    """The steps either side of the layer (not part of the timed step): router
    scores x . W_r^T and the gradient through the gate weights (dlogits), each
    timed alone over `reps` launches after the layer's own step, on the same
    synthetic inputs (the gate gradient reads the last forward's expert
    outputs).  Returns {name: {"ms", "gbs", "frac_hbm", "bytes"}}."""
    import torch
    T, d, E, k, R = lay.T, lay.d, lay.E, lay.k, lay.n_rows
    work = {
        "router_logits": (lambda: lay.router_scores(inp["x"], inp["w_router"]),
                          T * d * 2 + E * d * 2 + T * E * 4),
        "gate_grad": (lambda: lay.gate_grad(inp["dout"]), T * d * 2 + R * d * 2 + T * E * 4 + T * k * 12),
    }
    out = {}
    for name, (fn, by) in work.items():
        fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        out[name] = {"ms": round(ms, 4), "gbs": round(by / ms / 1e6, 1),
                     "frac_hbm": round(by / ms / 1e6 / PEAK_HBM_GBS, 4), "bytes": by}
    return out


def wgrad_f32_accumulate(lay, reps):
    """The weight-gradient stage adding into fp32 accumulators (the training
    loop's accumulate-into variant of the bf16 overwrite the step runs),
    timed alone over `reps` launches after the layer's step.  Bytes: the four
    activation operands read once and the fp32 accumulators read and written."""
    import torch
    E, d, f, R = lay.E, lay.d, lay.f, lay.n_rows
    a13 = torch.zeros(lay.G, 2 * f, d, dtype=torch.float32, device="cuda")
    a2 = torch.zeros(lay.G, d, f, dtype=torch.float32, device="cuda")
    fl = 6 * R * d * f
    by = R * (2 * d + 3 * f) * 2 + 2 * (a13.numel() + a2.numel()) * 4
    lay.wgrad_accumulate(a13, a2)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        lay.wgrad_accumulate(a13, a2)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del a13, a2
    return {"ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 1), "gbs": round(by / ms / 1e6, 1),
            "frac_hbm": round(by / ms / 1e6 / PEAK_HBM_GBS, 4), "bytes": by, "flops": fl}


def weight_requant(lay, reps):
    """MXFP8: the per-optimizer-step rebuild of the four weight caches (both
    directions of w13 and w2), timed alone over `reps` rebuilds (not part of
    the layer step).  Bytes: the bf16 weights read once per direction, codes
    and scales written."""
    import torch
    E, d, f = lay.E, lay.d, lay.f
    n = E * 3 * f * d                        # weight elements (w13 and w2)
    by = 2 * n * 2 + int(2 * n * MX_ELEM)    # bf16 read per direction; codes + scales written
    lay.requantize_weights()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        lay.requantize_weights()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    return {"ms": round(ms, 4), "gbs": round(by / ms / 1e6, 1), "frac_hbm": round(by / ms / 1e6 / PEAK_HBM_GBS, 4),
            "bytes": by}


def cpu_baseline(args, cfg, inp):
    """The oracle, untuned, on a bounded sample: route over all T tokens, then
    the expert FFN forward + backward for the first cpu_rows rows of the
    first n_exp experts (gathered like the permute does), time scaled to all
    R routed rows."""
    import numpy as np
    import torch

    import oracle
    oracle.build(force=False)
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    oracle.set_threads(threads)
    T, d, E, f, k = cfg["T"], cfg["d"], cfg["E"], cfg["f"], cfg["k"]
    logits = inp["logits"].cpu().numpy()
    t0 = time.perf_counter()
    r = oracle.route(logits, k)
    t_route = time.perf_counter() - t0
    n_exp = max(1, min(E, args.cpu_experts))
    rows_total = int(r["offsets"][-1])
    lo = int(r["offsets"][0])
    hi = min(int(r["offsets"][n_exp]), lo + args.cpu_rows)
    toks = r["src_slot"][lo:hi] // k
    to64 = lambda t: t.detach().cpu().to(torch.float64).numpy()
    x = to64(inp["x"][torch.from_numpy(toks).long().to(inp["x"].device)])
    dout_rows = to64(inp["dout"][torch.from_numpy(toks).long().to(inp["x"].device)])
    if "gate" in inp:
        w = inp["gate"].cpu().numpy()[toks].astype(np.float64)
    else:
        w = r["topk_w"].reshape(-1)[r["src_slot"][lo:hi]].astype(np.float64)
    w13 = to64(inp["w13"][:n_exp])
    w2 = to64(inp["w2"][:n_exp])
    go = np.minimum(r["offsets"][:n_exp + 1], hi).astype(np.int32)
    rows = hi - lo
    ident = np.arange(rows, dtype=np.int32)
    mx = cfg["dtype"] == "mxfp8"
    if mx:   # weight caches are made once per optimizer step, outside the step
        g13 = np.arange(n_exp + 1, dtype=np.int32) * 2 * f
        g2 = np.arange(n_exp + 1, dtype=np.int32) * d
        w13f = oracle.mx_qdq_rows(w13.reshape(-1, d)).reshape(w13.shape)
        w2f = oracle.mx_qdq_rows(w2.reshape(-1, f)).reshape(w2.shape)
        w13b = oracle.mx_qdq_cols(w13.reshape(-1, d), g13).reshape(w13.shape)
        w2b = oracle.mx_qdq_cols(w2.reshape(-1, f), g2).reshape(w2.shape)
    t1 = time.perf_counter()
    if mx:
        xq = oracle.mx_qdq_rows(x)
        gu, h, y = oracle.ffn_fwd(xq, w13f, w2f, go, oracle.BF16, mx_h=True)
        dy = oracle.permute(dout_rows, ident, 1, rows, row_scale=w.astype(np.float32),
                            round_mode=oracle.BF16)
        oracle.ffn_bwd(oracle.mx_qdq_rows(dy), xq, gu, h, w13f, w2f, go, oracle.BF16,
                       w2_dgrad=w2b, w13_dgrad=w13b, dy_wgrad=oracle.mx_qdq_cols(dy, go),
                       h_wgrad=oracle.mx_qdq_cols(h, go), x_wgrad=oracle.mx_qdq_cols(xq, go),
                       mx_dgu=True)
    else:
        gu, h, y = oracle.ffn_fwd(x, w13, w2, go, oracle.BF16)
        dy = oracle.permute(dout_rows, ident, 1, rows, row_scale=w.astype(np.float32),
                            round_mode=oracle.BF16)
        oracle.ffn_bwd(dy, x, gu, h, w13, w2, go, oracle.BF16)
    t_ffn = time.perf_counter() - t1
    # shared experts run the same per-row FFN over T more rows each
    rows_total += cfg.get("n_shared", 0) * T
    t_full = t_route + t_ffn * rows_total / max(rows, 1)
    return {"value": T / t_full, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"oracle route over all {T} tokens ({t_route:.2f} s) + expert FFN fwd+bwd "
                       f"for the first {rows} rows of experts 0..{n_exp - 1} ({t_ffn:.2f} s), "
                       f"scaled to all {rows_total} expert rows"),
            "sample_seconds": round(t_route + t_ffn, 2)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="e128")
    ap.add_argument("--padded", action="store_true", help="padded-to-capacity variant")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-experts", type=int, default=1,
                    help="experts whose rows the CPU-oracle sample covers")
    ap.add_argument("--cpu-rows", type=int, default=512,
                    help="at most this many of those rows")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 2 GiB device copy (counter calibration) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py measures one GPU's share of the layer; --gpus {args.gpus} is not "
              "supported (the path and its measurement run on exactly one GPU).", file=sys.stderr)
        sys.exit(2)

    import moe_synth
    cfg = moe_synth.WORKLOADS[args.workload]
    T, d, E, f, k = cfg["T"], cfg["d"], cfg["E"], cfg["f"], cfg["k"]
    res = run_gpu(args, cfg)
    R = res["R"]
    mx = cfg["dtype"] == "mxfp8"
    elem = 4 if cfg["dtype"] == "f32" else 2
    # shared experts: extra groups of T rows each, extra slots per token
    S = cfg.get("n_shared", 0)
    routed = T * k - (0 if not args.padded else int((res["lay"].dst_row < 0).sum().item())) + S * T
    Eg, kg = E + S, k + S   # GEMM groups and slots per token
    stages = {}
    for s in STAGES:
        fl, by = stage_work(s, T, d, Eg, f, kg, routed, elem, mx)
        ms = res["stage_ms"][s]
        ent = {"ms": round(ms, 4)}
        if fl:
            ent["tflops"] = round(fl / ms / 1e9, 1)
        ent["gbs"] = round(by / ms / 1e6, 1)
        stages[s] = ent
    gemm = [s for s in STAGES if s.startswith("gemm")]
    gemm_ms = sum(res["stage_ms"][s] for s in gemm)
    gemm_flops = 18 * routed * d * f
    peak = PEAK_FP8_TFLOPS if mx else (PEAK_BF16_TFLOPS if elem == 2 else PEAK_F32_TFLOPS)
    dom = max(STAGES, key=lambda s: res["stage_ms"][s])
    fl, by = stage_work(dom, T, d, Eg, f, kg, routed, elem, mx)
    dom_ms = res["stage_ms"][dom]
    if fl:
        rl = {"bound": "alu" if elem == 4 else "mfma", "achieved": round(fl / dom_ms / 1e9, 1),
              "peak": peak, "unit": "TFLOP/s", "frac": round(fl / dom_ms / 1e9 / peak, 4)}
    else:
        rl = {"bound": "hbm", "achieved": round(by / dom_ms / 1e6, 1), "peak": PEAK_HBM_GBS,
              "unit": "GB/s", "frac": round(by / dom_ms / 1e6 / PEAK_HBM_GBS, 4)}
    rl["attainable"] = round(roofline(peak, PEAK_HBM_GBS / 1e3, fl / by), 1) if fl else None
    rl.update({"traffic": measured_traffic(dom, args.workload + ("_padded" if args.padded else ""), mx),
               "kernel": kernel_name(dom, k, mx), "stage": dom,
               "launch_ms": round(dom_ms, 4), "algorithmic_flops": fl, "algorithmic_bytes": by})
    value = T / (res["ms_per_step"] / 1e3)
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(res["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg["dtype"], "data": "synthetic",
        "config": {"workload": (f"{args.workload}: T={T} d_model={d} E={E} d_ff={f} top-{k} "
                                f"{cfg['dtype']} SwiGLU, {cfg['routing']} routing, fwd+bwd"
                                + (" padded C=%d" % res["cap"] if args.padded else "")
                                + (f", {S} shared expert(s)" if S else "")),
                   "tokens": T, "experts": E, "top_k": k, "d_model": d, "d_ff": f,
                   "routed_rows": routed, "executed_rows": R, "shared_experts": S,
                   "seed": moe_synth.seed_of(args.workload)},
        "gemm": {"ms": round(gemm_ms, 4), "tflops": round(gemm_flops / gemm_ms / 1e9, 1),
                 "frac_peak": round(gemm_flops / gemm_ms / 1e9 / peak, 4)},
        "stages": stages, "gpu_event_ms_per_step": round(res["gpu_ms"], 4),
        "roofline": rl,
        "expert_rows": {"min": int(res["counts"].min()), "max": int(res["counts"].max())},
    }
    if res["f1"]:
        out["router_and_gate_grad"] = res["f1"]
    if res["wq"]:
        out["mx_weight_requant"] = res["wq"]
    if res["f4"]:
        out["wgrad_fp32_accumulate"] = res["f4"]
    if res["cold"]:
        out["hbm_stages_cold_cache"] = res["cold"]
    if args.workload == "e128" and not args.padded:
        out["route_stress"] = route_stress(max(5, min(args.steps, 10)))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args, cfg, res["inp"])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
