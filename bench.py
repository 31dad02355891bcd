#!/usr/bin/env python3
"""Benchmark of the MoE layer forward on one MI355X.

One step = one moe_forward call (gate + histogram/offsets, permute, grouped
SwiGLU FFN, combine) over the Mixtral-shaped layer (T=8192, d=4096, E=8, K=2,
n=14336, bf16, fp32 accumulation), inputs resident in HBM.  Prints ONE JSON line:
  value       = active layer TFLOPS = 6*T*K*d*n / time per step
  gate        = fused gate Gtokens/s on [T=262144, E=128, K=8] (cold MALL)
  steps_us    = per-entry-point times of the layer (HIP events, median)
  roofline    = the grouped FFN (moe_grouped_ffn: the SwiGLU GEMM then the
                down-projection GEMM), MFMA-bound, against 2.5 PFLOP/s dense bf16
  cpu_baseline= the CPU oracle (per-token loop, fp64 accumulation) on a bounded
                sample of the same layer, on this host's cores
Inputs are seeded synthetic tensors (see synth/); nothing is read from disk
except the optional HBM-traffic table under profiles/.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
TRAFFIC_TABLE = os.path.join(ROOT, "profiles", "traffic.json")
FFN_SOURCE = os.path.join(ROOT, "mixture_experts_routing_gate_amd", "csrc", "ffn.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def event_time_ms(torch, fn, iters, flush=None):
    """Median per-call time from HIP events recorded on torch's current stream
    (the stream every library call is enqueued on)."""
    times = []
    for _ in range(iters):
        if flush is not None:
            flush()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        e.synchronize()
        times.append(s.elapsed_time(e))
    return statistics.median(times), times


def ffn_traffic(cfg_name):
    """HBM bytes per grouped-FFN call from the committed rocprofv3 counter table,
    or None when absent or taken from a different ffn.hip."""
    try:
        tab = json.load(open(TRAFFIC_TABLE))
        src = hashlib.sha256(open(FFN_SOURCE, "rb").read()).hexdigest()
        ent = tab.get(cfg_name, {})
        if ent.get("ffn_source_sha256") != src:
            return None
        return ent.get("ffn_hbm_bytes")
    except (OSError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1 (multi-GPU sharding is "
                                   "described in DESIGN.md but not built)", "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import mixture_experts_routing_gate_amd as moe
    import synth

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    moe.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    cfg = synth.CONFIGS["mixtral"]
    T, d, E, K, n = cfg.T, cfg.d, cfg.E, cfg.K, cfg.n
    A = T * K
    flops = 6.0 * A * d * n
    g = synth.make_inputs(cfg, dev, seed=0)
    plan = moe.ForwardPlan(T, d, E, K, n, cfg.torch_dtype, dev)

    def step():
        plan(g["X"], g["logits"], g["W1"], g["W3"], g["W2"])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    tflops = flops / (ms_per_step * 1e-3) / 1e12

    # Per-entry-point times of the same layer (events around each ABI call).
    idx, w, counts, offsets = moe.moe_route(g["logits"], K)
    sp, inv, Xp = moe.moe_permute(g["X"], idx, E)
    Act, Y = moe.moe_grouped_ffn(Xp, g["W1"], g["W3"], g["W2"], counts, offsets, K)
    torch.cuda.synchronize()
    r_ms, _ = event_time_ms(torch, lambda: moe.moe_route(g["logits"], K), 20)
    p_ms, _ = event_time_ms(torch, lambda: moe.moe_permute(g["X"], idx, E), 20)
    f_ms, f_all = event_time_ms(torch, lambda: moe.moe_grouped_ffn(Xp, g["W1"], g["W3"], g["W2"], counts, offsets, K),
                                max(5, args.steps // 2))
    c_ms, _ = event_time_ms(torch, lambda: moe.moe_combine(Y, w, inv), 20)
    s = 2  # bf16 bytes
    perm_bytes = T * (s * d * (1 + K) + 12 * K)
    comb_bytes = T * (s * d * (K + 1) + 8 * K)
    route_bytes = T * (4 * E + 8 * K)
    ffn_tflops = flops / (f_ms * 1e-3) / 1e12
    counts_h = counts.cpu().numpy()

    # Gate on the large gate-only workload, MALL flushed before every call.
    gcfg = synth.CONFIGS["gate_l"]
    glg = synth.make_inputs(gcfg, dev, seed=0)["logits"]
    flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    moe.moe_route(glg, gcfg.K)
    torch.cuda.synchronize()
    g_ms, _ = event_time_ms(torch, lambda: moe.moe_route(glg, gcfg.K), 20, flush=lambda: flush_buf.fill_(1))
    gate_bytes = gcfg.T * (4 * gcfg.E + 8 * gcfg.K)
    gate = {"workload": "gate-only fp32 logits [T=262144, E=128], K=8 (N(0,1))",
            "value": gcfg.T / (g_ms * 1e-3) / 1e9, "unit": "Gtokens/s", "us_per_call": g_ms * 1e3,
            "roofline": {"bound": "hbm", "achieved": gate_bytes / (g_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": gate_bytes / (g_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         "traffic": None}}
    del flush_buf

    out = {
        "metric": "MoE layer fwd active TFLOPS + gate Gtokens/s on 1 MI355X (vs roofline)",
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; X~N(0,1), logits=X@Wr, Wr~N(0,1/d), W1,W3~N(0,1/d), W2~N(0,1/n))",
        "config": {"workload": "mixtral-shaped MoE layer forward", "T": T, "d": d, "E": E, "K": K, "n": n,
                   "active_flops_per_step": flops, "expert_counts": counts_h.tolist()},
        "gate": gate,
        "steps_us": {
            "route": {"us": r_ms * 1e3, "GB/s": route_bytes / (r_ms * 1e-3) / 1e9},
            "permute": {"us": p_ms * 1e3, "GB/s": perm_bytes / (p_ms * 1e-3) / 1e9,
                        "frac_hbm": perm_bytes / (p_ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
            "grouped_ffn": {"us": f_ms * 1e3, "TFLOPS": ffn_tflops},
            "combine": {"us": c_ms * 1e3, "GB/s": comb_bytes / (c_ms * 1e-3) / 1e9,
                        "frac_hbm": comb_bytes / (c_ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
        },
        "roofline": {"kernel": "moe_grouped_ffn (ffn_wide_kernel: SwiGLU GEMM launch + down-projection launch)",
                     "bound": "mfma", "achieved": round(ffn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(ffn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": ffn_traffic("mixtral"),
                     "algorithmic_flops_per_call": flops},
    }

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, g, args.cpu_seconds, np, torch, synth)
    print(json.dumps(out), flush=True)


def cpu_baseline(cfg, g, budget_s, np, torch, synth):
    """The oracle's per-token layer loop, as it stands, on a bounded token sample."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    X = synth.to_numpy(g["X"])
    lg = synth.to_numpy(g["logits"])
    W1, W3, W2 = (synth.to_numpy(g[k]) for k in ("W1", "W3", "W2"))
    rng = np.random.default_rng(0)
    per_tok = 6.0 * cfg.K * cfg.d * cfg.n
    ntok = max(cores, 4)
    t0 = time.perf_counter()
    oracle.layer(X, lg, W1, W3, W2, cfg.K, tokens=rng.choice(cfg.T, ntok, replace=False).astype(np.int32))
    dt = time.perf_counter() - t0
    ntok2 = int(min(cfg.T, max(ntok, ntok * (budget_s - dt) / max(dt, 1e-3))))
    toks = rng.choice(cfg.T, ntok2, replace=False).astype(np.int32)
    t0 = time.perf_counter()
    oracle.layer(X, lg, W1, W3, W2, cfg.K, tokens=toks)
    dt2 = time.perf_counter() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    return {"value": per_tok * ntok2 / dt2 / 1e12, "unit": "TFLOPS", "cores": min(threads, cores),
            "kind": "oracle",
            "sample": f"{ntok2} of {cfg.T} tokens of the mixtral-shaped layer through the oracle's per-token "
                      f"loop (route + {cfg.K} expert SwiGLU MLPs + combine, fp64 accumulation), "
                      f"{dt2:.1f} s wall; scaled to active TFLOPS of those tokens"}


if __name__ == "__main__":
    main()
