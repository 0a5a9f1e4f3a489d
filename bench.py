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
PEAK_F32_TFLOPS = 157.3         # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E

STAGES = ["route", "permute", "gemm_gate_up", "gemm_down", "combine", "combine_bwd",
          "gemm_dgrad_down", "gemm_dgrad_gate_up", "gemm_wgrad", "permute_bwd"]
KERNEL_NAMES = {
    "gemm_gate_up": "gemm_grouped_m_kernel<256, 64, 2, false, 1> (gate/up + SwiGLU)",
    "gemm_down": "gemm_grouped_m_kernel<256, 64, 2, false, 0> (down)",
    "gemm_dgrad_down": "gemm_grouped_m_kernel<256, 64, 2, true, 2> (dgrad down + SwiGLU bwd)",
    "gemm_dgrad_gate_up": "gemm_grouped_m_kernel<256, 64, 2, true, 0> (dgrad gate/up)",
    "gemm_wgrad": "gemm_grouped_k_kernel<256, 64, 2> (wgrad, dWd and dW13 in one launch)",
    "permute": "permute_kernel<true, false>",
    "combine": "combine_kernel<true>",
}


PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {"gemm": "routing_grouped_gemm_amd/csrc/gemm_bf16.hip",
                  "route": "routing_grouped_gemm_amd/csrc/route.hip",
                  "permute": "routing_grouped_gemm_amd/csrc/permute.hip",
                  "combine": "routing_grouped_gemm_amd/csrc/permute.hip"}


def source_hash(stage):
    import hashlib
    key = "gemm" if stage.startswith("gemm") else stage.split("_")[0]
    path = os.path.join(ROOT, KERNEL_SOURCES.get(key, KERNEL_SOURCES["gemm"]))
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def measured_traffic(stage, workload):
    """HBM bytes per launch of `stage` from the committed counter record
    (profiles/traffic_<stage>_<workload>.json), or None when there is none or
    the kernel source changed since the counters were taken."""
    path = os.path.join(PROFILES, f"traffic_{stage}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256_16") != source_hash(stage):
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


def stage_work(name, T, d, E, f, k, R, elem=2):
    """Algorithmic (FLOPs, HBM bytes) of one stage: useful work only, padding
    rows never counted; bytes = each operand read once and each result
    written once."""
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


def run_gpu(args, cfg):
    import torch

    import moe_synth
    import routing_grouped_gemm_amd as m
    from routing_grouped_gemm_amd.layer import MoELayer

    T, d, E, f, k = cfg["T"], cfg["d"], cfg["E"], cfg["f"], cfg["k"]
    dt = {"bf16": m.MOE_BF16, "f32": m.MOE_F32}[cfg["dtype"]]
    cap = 0
    if args.padded:
        cap = moe_synth.capacity_of(T, k, E, cfg.get("capacity_factor", 1.25))
    inp = moe_synth.make_inputs(args.workload, device="cuda")
    lay = MoELayer(T, d, E, f, k, dt, capacity=cap)
    lay.set_weights(inp["w13"], inp["w2"])
    lay._alloc_bwd()
    R = lay.n_rows
    act_dt = dt
    ten = m.gemm_tensors(x_perm=lay.x_perm, w13=lay.w13, w2=lay.w2, gu=lay.gu, h=lay.h,
                         y_perm=lay.y_perm, dy_perm=lay.dy_perm, dgu=lay.dgu,
                         dx_perm=lay.dx_perm, dw13=lay.dw13, dw2=lay.dw2)
    goff = lay.offsets

    def step(ev):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        lay.route(inp["logits"])
        mark(1)
        lay.permute(inp["x"])
        mark(2)
        m.moe_grouped_gemm_op(m.MOE_GEMM_GATE_UP, dt, ten, goff, cap, E, R, d, f)
        mark(3)
        m.moe_grouped_gemm_op(m.MOE_GEMM_DOWN, dt, ten, goff, cap, E, R, d, f)
        mark(4)
        lay.combine()
        mark(5)
        m.moe_permute(act_dt, inp["dout"], k, lay.dst_row, lay.dy_perm, src_slot=lay.src_slot,
                      row_scale=lay.topk_w, dev_err=lay.dev_err)
        mark(6)
        m.moe_grouped_gemm_op(m.MOE_GEMM_DGRAD_DOWN, dt, ten, goff, cap, E, R, d, f)
        mark(7)
        m.moe_grouped_gemm_op(m.MOE_GEMM_DGRAD_GATE_UP, dt, ten, goff, cap, E, R, d, f)
        mark(8)
        m.moe_grouped_gemm_op(m.MOE_GEMM_WGRAD, dt, ten, goff, cap, E, R, d, f)
        mark(9)
        m.moe_unpermute_combine(act_dt, lay.dx_perm, lay.dst_row, None, k, lay.dx,
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
    return dict(stage_ms=stage_ms, gpu_ms=gpu_ms, ms_per_step=ms_per_step, R=R, cap=cap,
                counts=counts, inp=inp, lay=lay)


def cpu_baseline(args, cfg, inp):
    """The oracle, untuned, on a bounded sample: route over all T tokens, then
    the expert FFN forward + backward for the rows of the first n_exp experts
    (their rows are gathered like the permute does), time scaled to all R
    routed rows."""
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
    lo, hi = int(r["offsets"][0]), int(r["offsets"][n_exp])
    toks = r["src_slot"][lo:hi] // k
    to64 = lambda t: t.detach().cpu().to(torch.float64).numpy()
    x = to64(inp["x"][torch.from_numpy(toks).long().to(inp["x"].device)])
    dout_rows = to64(inp["dout"][torch.from_numpy(toks).long().to(inp["x"].device)])
    w = r["topk_w"].reshape(-1)[r["src_slot"][lo:hi]].astype(np.float64)
    w13 = to64(inp["w13"][:n_exp])
    w2 = to64(inp["w2"][:n_exp])
    go = r["offsets"][:n_exp + 1].astype(np.int32)
    rows = hi - lo
    t1 = time.perf_counter()
    gu, h, y = oracle.ffn_fwd(x, w13, w2, go, oracle.BF16)
    ident = np.arange(rows, dtype=np.int32)
    dy = oracle.permute(dout_rows, ident, 1, rows, row_scale=w.astype(np.float32),
                        round_mode=oracle.BF16)
    oracle.ffn_bwd(dy, x, gu, h, w13, w2, go, oracle.BF16)
    t_ffn = time.perf_counter() - t1
    t_full = t_route + t_ffn * rows_total / max(rows, 1)
    return {"value": T / t_full, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"oracle route over all {T} tokens ({t_route:.2f} s) + expert FFN fwd+bwd "
                       f"for the {rows} rows of experts 0..{n_exp - 1} ({t_ffn:.2f} s), "
                       f"scaled to all {rows_total} routed rows"),
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
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 2 GiB device copy (counter calibration) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py measures one GPU's share of the layer; --gpus {args.gpus} is not "
              "supported (this build runs on exactly one GPU).", file=sys.stderr)
        sys.exit(2)

    import moe_synth
    cfg = moe_synth.WORKLOADS[args.workload]
    if cfg["dtype"] not in ("bf16", "f32"):
        print(f"workload {args.workload} ({cfg['dtype']}) is not benchmarked here", file=sys.stderr)
        sys.exit(2)
    T, d, E, f, k = cfg["T"], cfg["d"], cfg["E"], cfg["f"], cfg["k"]
    res = run_gpu(args, cfg)
    R = res["R"]
    elem = 2 if cfg["dtype"] == "bf16" else 4
    routed = T * k - (0 if not args.padded else int((res["lay"].dst_row < 0).sum().item()))
    stages = {}
    for s in STAGES:
        fl, by = stage_work(s, T, d, E, f, k, routed, elem)
        ms = res["stage_ms"][s]
        ent = {"ms": round(ms, 4)}
        if fl:
            ent["tflops"] = round(fl / ms / 1e9, 1)
        ent["gbs"] = round(by / ms / 1e6, 1)
        stages[s] = ent
    gemm = [s for s in STAGES if s.startswith("gemm")]
    gemm_ms = sum(res["stage_ms"][s] for s in gemm)
    gemm_flops = 18 * routed * d * f
    peak = PEAK_BF16_TFLOPS if elem == 2 else PEAK_F32_TFLOPS
    dom = max(STAGES, key=lambda s: res["stage_ms"][s])
    fl, by = stage_work(dom, T, d, E, f, k, routed, elem)
    dom_ms = res["stage_ms"][dom]
    if fl:
        rl = {"bound": "mfma" if elem == 2 else "alu", "achieved": round(fl / dom_ms / 1e9, 1),
              "peak": peak, "unit": "TFLOP/s", "frac": round(fl / dom_ms / 1e9 / peak, 4)}
    else:
        rl = {"bound": "hbm", "achieved": round(by / dom_ms / 1e6, 1), "peak": PEAK_HBM_GBS,
              "unit": "GB/s", "frac": round(by / dom_ms / 1e6 / PEAK_HBM_GBS, 4)}
    rl["attainable"] = round(roofline(peak, PEAK_HBM_GBS / 1e3, fl / by), 1) if fl else None
    rl.update({"traffic": measured_traffic(dom, args.workload + ("_padded" if args.padded else "")),
               "kernel": KERNEL_NAMES.get(dom, dom), "stage": dom,
               "launch_ms": round(dom_ms, 4), "algorithmic_flops": fl, "algorithmic_bytes": by})
    value = T / (res["ms_per_step"] / 1e3)
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(res["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg["dtype"], "data": "synthetic",
        "config": {"workload": (f"{args.workload}: T={T} d_model={d} E={E} d_ff={f} top-{k} "
                                f"{cfg['dtype']} SwiGLU, {cfg['routing']} routing, fwd+bwd"
                                + (" padded C=%d" % res["cap"] if args.padded else "")),
                   "tokens": T, "experts": E, "top_k": k, "d_model": d, "d_ff": f,
                   "routed_rows": routed, "executed_rows": R, "seed": moe_synth.seed_of(args.workload)},
        "gemm": {"ms": round(gemm_ms, 4), "tflops": round(gemm_flops / gemm_ms / 1e9, 1),
                 "frac_peak": round(gemm_flops / gemm_ms / 1e9 / peak, 4)},
        "stages": stages, "gpu_event_ms_per_step": round(res["gpu_ms"], 4),
        "roofline": rl,
        "expert_rows": {"min": int(res["counts"].min()), "max": int(res["counts"].max())},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args, cfg, res["inp"])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
