"""Seeded synthetic inputs for the MoE feed-forward layer.

This module only draws random numbers; it holds none of the layer's
arithmetic.  Both the HIP path and the CPU oracle take their inputs from
here (the oracle never sees anything the HIP path produced).

Workloads (the pages measure their systems under random routing with
uniform expert load; no dataset is involved):
  tiny    T=256   d=128  E=8   f=256  k=2  fp32, fwd only
  e8      T=8192  d=2048 E=8   f=1024 k=4  bf16, fwd+bwd
  e128    T=16384 d=4096 E=128 f=1536 k=4  bf16, fwd+bwd      (the metric's workload)
  e8_matched       T=16384 d=4096 E=8 f=1536 k=4 (same active FLOPs as e128)
  e128_zipf        e128 shapes, expert choice ~ Zipf(1.2) (Gumbel top-k)
  mx_shard         32768 received rows, 16 local experts, d=4096 f=1536, MXFP8
Values: activations and weights ~ N(0, 0.02), router logits ~ N(0, 1),
upstream gradient ~ N(0, 1); bf16 tensors are the RNE rounding of the drawn
fp32 values (torch's conversion).  Seeds are 1000 + workload index.
"""
import math

import torch

WORKLOADS = {
    "tiny": dict(idx=0, T=256, d=128, E=8, f=256, k=2, dtype="f32", routing="uniform",
                 bwd=False),
    "e8": dict(idx=1, T=8192, d=2048, E=8, f=1024, k=4, dtype="bf16", routing="uniform",
               bwd=True),
    "e128": dict(idx=2, T=16384, d=4096, E=128, f=1536, k=4, dtype="bf16", routing="uniform",
                 bwd=True),
    "e128_zipf": dict(idx=3, T=16384, d=4096, E=128, f=1536, k=4, dtype="bf16", routing="zipf",
                      bwd=True, capacity_factor=1.25),
    "mx_shard": dict(idx=4, T=32768, d=4096, E=16, f=1536, k=1, dtype="mxfp8",
                     routing="uniform", bwd=True, gate="uniform01"),
    "e8_matched": dict(idx=5, T=16384, d=4096, E=8, f=1536, k=4, dtype="bf16",
                       routing="uniform", bwd=True),
    # e128 plus one shared expert (ungated, every token) of the same width
    "e128_shared": dict(idx=6, T=16384, d=4096, E=128, f=1536, k=4, n_shared=1, dtype="bf16",
                        routing="uniform", bwd=True),
    # the MXFP8 shard with Zipf(1.2)-skewed rows over its 16 experts
    "mx_shard_zipf": dict(idx=7, T=32768, d=4096, E=16, f=1536, k=1, dtype="mxfp8",
                          routing="zipf", bwd=True, gate="uniform01"),
}

ZIPF_S = 1.2


def seed_of(name):
    return 1000 + WORKLOADS[name]["idx"]


def capacity_of(T, k, E, factor):
    """Expert capacity C = ceil(factor * T * k / E)."""
    return int(math.ceil(factor * T * k / E))


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, std, seed, device="cpu", dtype=torch.float32):
    g = _gen(seed, device)
    v = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        v.mul_(std)
    return v.to(dtype)


def uniform01(shape, seed, device="cpu"):
    g = _gen(seed, device)
    return torch.rand(*shape, generator=g, device=device, dtype=torch.float32)


def router_logits(T, E, seed, routing="uniform", device="cpu"):
    """fp32 router logits.  uniform: iid N(0,1).  zipf: ln p_e + Gumbel(0,1)
    with p_e proportional to (e+1)^-1.2, so the top-k of a row is a draw of k
    distinct experts without replacement with probabilities p."""
    if routing == "uniform":
        return normal((T, E), 1.0, seed, device)
    if routing == "zipf":
        u = uniform01((T, E), seed, device).clamp_(min=1e-12, max=1.0 - 1e-7)
        gumbel = -torch.log(-torch.log(u))
        p = torch.arange(1, E + 1, device=device, dtype=torch.float64).pow(-ZIPF_S)
        logp = torch.log(p / p.sum()).to(torch.float32)
        return (gumbel + logp[None, :]).contiguous()
    raise ValueError(routing)


def make_inputs(name=None, device="cpu", seed=None, act_dtype=None, **over):
    """Inputs of a named workload, or of explicit sizes passed as keywords
    (T, d, E, f, k, dtype, routing).  Returns a dict of torch tensors:
    logits [T,E] fp32, x [T,d], w13 [E,2f,d], w2 [E,d,f], dout [T,d],
    and gate [T] fp32 for the MXFP8 shard (per-row combine weight)."""
    cfg = dict(WORKLOADS[name]) if name else dict(T=64, d=64, E=4, f=64, k=2, dtype="bf16",
                                                  routing="uniform", bwd=True, idx=99)
    cfg.update(over)
    if seed is None:
        seed = 1000 + cfg["idx"]
    T, d, E, f = cfg["T"], cfg["d"], cfg["E"], cfg["f"]
    if act_dtype is None:
        act_dtype = torch.float32 if cfg["dtype"] == "f32" else torch.bfloat16
    s = seed * 16
    out = dict(cfg=cfg, seed=seed)
    out["logits"] = router_logits(T, E, s + 1, cfg["routing"], device)
    out["x"] = normal((T, d), 0.02, s + 2, device, act_dtype)
    Ew = E + cfg.get("n_shared", 0)   # expert weights: the routed ones, then the shared ones
    out["w13"] = normal((Ew, 2 * f, d), 0.02, s + 3, device, act_dtype)
    out["w2"] = normal((Ew, d, f), 0.02, s + 4, device, act_dtype)
    out["dout"] = normal((T, d), 1.0, s + 5, device, act_dtype)
    # router weights [E, d]: std 1 / (0.02 sqrt(d)), so that with x ~ N(0, 0.02)
    # the router scores x . W_r^T are about N(0, 1) like the logits above
    out["w_router"] = normal((E, d), 1.0 / (0.02 * math.sqrt(d)), s + 7, device, act_dtype)
    if cfg.get("gate") == "uniform01":
        out["gate"] = uniform01((T,), s + 6, device)
    return out
