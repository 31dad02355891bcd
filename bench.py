#!/usr/bin/env python3
"""Benchmark of the MoE layer forward on one MI355X.

One step = one moe_forward call (gate + histogram/offsets, permute, grouped
SwiGLU FFN, combine) over the Mixtral-shaped layer (T=8192, d=4096, E=8, K=2,
n=14336, bf16, fp32 accumulation), inputs resident in HBM.  Prints ONE JSON line:
  value       = active layer TFLOPS = 6*T*K*d*n / time per step
  gate        = fused gate Gtokens/s on [T=262144, E=128, K=8] (cold caches: read flush)
  steps_us    = per-entry-point times of the layer (HIP events, median)
  roofline    = the dominant kernel, the SwiGLU GEMM (moe_ffn_up: one launch
                of the pipelined MFMA kernel), MFMA-bound, against 2.5 PFLOP/s
                dense bf16; its HBM traffic comes from the committed rocprofv3
                counter table (profiles/traffic.json) when it matches ffn.hip
  token_rounding = the layer with Token Rounding at tile height 256 beside
                plain top-K on the same inputs (mixtral here; the other shapes
                under other_workloads), with its plan and combine back to back
  backward_data = moe_backward_data (dX and the router-logit gradient) on the
                same layer, per call, with the rate of its grouped GEMMs, and
                moe_backward (the expert-weight gradients too)
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
CSRC = os.path.join(ROOT, "mixture_experts_routing_gate_amd", "csrc")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the DeepSeek-V3-shaped and fine-grained layer timings")
    ap.add_argument("--backward-probe", action="store_true",
                    help="run moe_backward_data on the mixtral-shaped layer once, then 3 times back to back, "
                         "for a kernel trace, and print its time")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run a plain copy of known size and each step once (for rocprofv3 --pmc) and exit")
    ap.add_argument("--probe", choices=["mixtral", "dsv3", "fine", "gate_l"],
                    help="run the steps of one workload a few times (the router, moe_route, moe_permute, "
                         "moe_ffn_up, moe_ffn_down, moe_combine, then moe_forward), each call after a 512 MiB "
                         "read flush with --cold, for a rocprofv3 kernel trace or counter pass, and exit")
    ap.add_argument("--cold", action="store_true", help="with --probe: a read flush before every call")
    ap.add_argument("--copy-probe", action="store_true",
                    help="a plain 512 MiB device copy, for calibrating FETCH_SIZE / WRITE_SIZE, and exit")
    ap.add_argument("--blas-ref", action="store_true",
                    help="time the mixtral-shaped grouped GEMMs against hipBLASLt (torch.matmul per expert) on the "
                         "same rows and weights, each at steady state, and exit")
    ap.add_argument("--ref-seconds", type=float, default=1.0,
                    help="with --blas-ref: back-to-back run before each timing")
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


def make_flush(torch, dev):
    """A 512 MiB read (a sum into one float): evicts earlier data from L2 and the
    256 MB Infinity Cache without leaving dirty lines for the timed call to write
    back (a write flush would)."""
    buf = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    res = torch.empty(1, dtype=torch.float32, device=dev)
    return lambda: torch.sum(buf, 0, keepdim=True, out=res)


def b2b_time_ms(torch, fn, n=20, reps=3):
    """Per-call time of n calls issued back to back (best of `reps`), from HIP
    events on the current stream: the steady-state rate without the launch
    latency that a single timed call includes."""
    fn()
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(reps):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(n):
            fn()
        e.record()
        e.synchronize()
        best = min(best, s.elapsed_time(e) / n)
    return best


def kernel_traffic(workload, kernel):
    """Calibrated bytes per launch of `kernel` from the committed rocprofv3
    counter table (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy), or None when
    absent or when the kernel's source file changed since the counters were taken."""
    try:
        tab = json.load(open(TRAFFIC_TABLE))
        ent = tab["workloads"][workload][kernel]
        src = ent["source"]
        now = hashlib.sha256(open(os.path.join(CSRC, src), "rb").read()).hexdigest()
        if tab["sources"].get(src) != now:
            return None
        return ent["hbm_bytes"]
    except (OSError, ValueError, KeyError):
        return None


def traffic_probe(moe, synth, torch, dev):
    """A plain copy of known size, then the router projection and each step of
    the layer once on the mixtral-shaped workload and the gate on the large gate
    workload (each after one warm-up call), for FETCH_SIZE / WRITE_SIZE counter
    runs."""
    n = 256 << 20  # 512 MiB of bf16
    src = torch.ones(n, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    cfg = synth.CONFIGS["mixtral"]
    g = synth.make_inputs(cfg, dev, seed=0)
    Wr, rb = synth.make_router(cfg, dev, seed=0)
    for _ in range(2):
        moe.moe_router(g["X"], Wr, rb)
        idx, w, counts, offsets = moe.moe_route(g["logits"], cfg.K)
        sp, inv, Xp = moe.moe_permute(g["X"], idx, cfg.E)
        Act = moe.moe_ffn_up(Xp, g["W1"], g["W3"], counts, offsets, cfg.K)
        Y = moe.moe_ffn_down(Act, g["W2"], counts, offsets, cfg.K)
        moe.moe_combine(Y, w, inv)
    torch.cuda.synchronize()
    del g, Xp, Act, Y
    gcfg = synth.CONFIGS["gate_l"]
    glg = synth.make_inputs(gcfg, dev, seed=0)["logits"]
    for _ in range(2):
        moe.moe_route(glg, gcfg.K)
    torch.cuda.synchronize()
    print(json.dumps({"traffic_probe": "done", "copy_bytes_each_way": 2 * n}), flush=True)


def workload_probe(name, cold, moe, synth, torch, dev, reps=3):
    """Each step of one workload `reps` times (after one warm-up round), for a
    rocprofv3 kernel trace or counter pass; with `cold`, a 512 MiB read before
    every call.  Prints one line per round (progress for long profiled runs)."""
    cfg = synth.CONFIGS[name]
    g = synth.make_inputs(cfg, dev, seed=0)
    flush = make_flush(torch, dev) if cold else (lambda: None)
    if cfg.gate_only:
        out = moe.moe_route(g["logits"], cfg.K)
        for r in range(reps + 1):
            flush()
            moe.moe_route(g["logits"], cfg.K, out=out)
            torch.cuda.synchronize()
            print(json.dumps({"probe": name, "pass": r}), flush=True)
        return
    Wr, rb = synth.make_router(cfg, dev, seed=0)
    plan = moe.ForwardPlan(cfg.T, cfg.d, cfg.E, cfg.K, cfg.n, cfg.torch_dtype, dev)
    for r in range(reps + 1):
        flush()
        moe.moe_router(g["X"], Wr, rb)
        flush()
        idx, w, counts, offsets = moe.moe_route(g["logits"], cfg.K)
        flush()
        sp, inv, Xp = moe.moe_permute(g["X"], idx, cfg.E)
        flush()
        Act = moe.moe_ffn_up(Xp, g["W1"], g["W3"], counts, offsets, cfg.K)
        flush()
        Y = moe.moe_ffn_down(Act, g["W2"], counts, offsets, cfg.K)
        flush()
        moe.moe_combine(Y, w, inv)
        flush()
        plan(g["X"], g["logits"], g["W1"], g["W3"], g["W2"])
        torch.cuda.synchronize()
        del Xp, Act, Y
        print(json.dumps({"probe": name, "pass": r}), flush=True)


def blas_reference(moe, synth, torch, dev, seconds, iters=10):
    """The mixtral-shaped grouped GEMMs next to hipBLASLt, reached through
    torch.matmul with one GEMM per expert, on the same expert-sorted rows and
    weights.  The weights are given as stored (n-contiguous) and, for
    hipBLASLt only, also as k-contiguous copies made beforehand.  The card's
    clock settles under its power cap within about a second of sustained
    work, so each candidate first runs back to back for `seconds`, and then
    the median of `iters` event-timed calls is taken.  The rounds alternate
    the candidates twice."""
    cfg = synth.CONFIGS["mixtral"]
    T, d, E, K, n = cfg.T, cfg.d, cfg.E, cfg.K, cfg.n
    A = T * K
    g = synth.make_inputs(cfg, dev, seed=0)
    idx, w, counts, offsets = moe.moe_route(g["logits"], K)
    sp, inv, Xp = moe.moe_permute(g["X"], idx, E)
    W1, W3, W2 = g["W1"], g["W3"], g["W2"]
    W1t, W3t, W2t = (W.transpose(1, 2).contiguous() for W in (W1, W3, W2))
    off = offsets.cpu().tolist()
    segs = [(e, off[e], off[e + 1]) for e in range(E) if off[e + 1] > off[e]]
    ws = moe.load_library().moe_ffn_workspace_bytes(d, n, moe.dtype_code(Xp.dtype))
    ws = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
    Act = moe.moe_ffn_up(Xp, W1, W3, counts, offsets, K, ws=ws)
    Y = moe.moe_ffn_down(Act, W2, counts, offsets, K, ws=ws)
    H1 = torch.empty(A, n, dtype=Xp.dtype, device=dev)
    H3 = torch.empty_like(H1)
    Yb = torch.empty(A, d, dtype=Xp.dtype, device=dev)

    def blas_up(kc):
        for e, a, b in segs:
            torch.matmul(Xp[a:b], W1t[e].T if kc else W1[e], out=H1[a:b])
            torch.matmul(Xp[a:b], W3t[e].T if kc else W3[e], out=H3[a:b])

    def blas_down(kc):
        for e, a, b in segs:
            torch.matmul(Act[a:b], W2t[e].T if kc else W2[e], out=Yb[a:b])

    cands = {
        "up": (4.0 * A * d * n, {
            "ours": lambda: moe.moe_ffn_up(Xp, W1, W3, counts, offsets, K, ws=ws, out=Act),
            "hipblaslt_n": lambda: blas_up(False),
            "hipblaslt_k": lambda: blas_up(True)}),
        "down": (2.0 * A * d * n, {
            "ours": lambda: moe.moe_ffn_down(Act, W2, counts, offsets, K, ws=ws, out=Y),
            "hipblaslt_n": lambda: blas_down(False),
            "hipblaslt_k": lambda: blas_down(True)}),
    }
    res = {}
    for rnd in range(2):
        for gemm, (flops, fns) in cands.items():
            for name, fn in fns.items():
                t_end = time.perf_counter() + seconds
                while time.perf_counter() < t_end:
                    for _ in range(5):
                        fn()
                    torch.cuda.synchronize()
                ms, _ = event_time_ms(torch, fn, iters)
                r = res.setdefault(gemm, {}).setdefault(name, {"ms": []})
                r["ms"].append(round(ms, 4))
                print(json.dumps({"blas_ref_round": rnd, "gemm": gemm, "candidate": name, "ms": round(ms, 4)}),
                      flush=True)
    for gemm, (flops, _) in cands.items():
        for name, r in res[gemm].items():
            r["tflops"] = [round(flops / (m * 1e-3) / 1e12, 1) for m in r["ms"]]
            r["frac_of_bf16_peak"] = [round(t / 2500.0, 4) for t in r["tflops"]]
    return {"workload": "mixtral T=8192 d=4096 E=8 K=2 n=14336 bf16", "steady_state_seconds": seconds,
            "iters": iters, "gemms": res}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "one GPU only: --gpus must be 1 (the expert-parallel sharding across GPUs "
                                   "is not built)", "n_gpus": args.gpus}))
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
    if args.traffic_probe:
        traffic_probe(moe, synth, torch, dev)
        return
    if args.copy_probe:
        n = 256 << 20  # 512 MiB of bf16
        src = torch.ones(n, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe": "done", "bytes_each_way": 2 * n}), flush=True)
        return
    if args.probe:
        workload_probe(args.probe, args.cold, moe, synth, torch, dev)
        return
    if args.blas_ref:
        print(json.dumps({"blas_ref": blas_reference(moe, synth, torch, dev, args.ref_seconds)}), flush=True)
        return
    if args.backward_probe:
        c = synth.CONFIGS["mixtral"]
        print(json.dumps({"backward_probe": backward_data(c, synth.make_inputs(c, dev, seed=0), moe, torch, dev)}),
              flush=True)
        return

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
    f_ms, _ = event_time_ms(torch, lambda: moe.moe_grouped_ffn(Xp, g["W1"], g["W3"], g["W2"], counts, offsets, K),
                            max(5, args.steps // 2))
    # The dominant kernel alone: the SwiGLU GEMM (one launch), then the down GEMM.
    up_ms, up_times = event_time_ms(torch, lambda: moe.moe_ffn_up(Xp, g["W1"], g["W3"], counts, offsets, K),
                                    max(5, args.steps // 2))
    up_mean_ms = statistics.mean(up_times)
    dn_ms, _ = event_time_ms(torch, lambda: moe.moe_ffn_down(Act, g["W2"], counts, offsets, K),
                             max(5, args.steps // 2))
    up_flops = 4.0 * A * d * n
    up_tflops = up_flops / (up_ms * 1e-3) / 1e12
    up_tflops_mean = up_flops / (up_mean_ms * 1e-3) / 1e12
    c_ms, _ = event_time_ms(torch, lambda: moe.moe_combine(Y, w, inv), 20)
    # Router projection upstream of the gate (logits = X Wr for this workload).
    Wr, rb = synth.make_router(cfg, dev, seed=0)
    rws = torch.empty(max(moe.load_library().moe_router_workspace_bytes(d, E, 1), 1), dtype=torch.uint8, device=dev)
    rt_ms, _ = event_time_ms(torch, lambda: moe.moe_router(g["X"], Wr, rb, ws=rws), 20)
    rt_b2b = b2b_time_ms(torch, lambda: moe.moe_router(g["X"], Wr, rb, ws=rws))
    router_bytes = T * d * 2 + d * E * 4 + T * E * 4
    layer_x = layer_from_x(cfg, g, Wr, rb, moe, torch, dev, args, r_ms, rt_ms)
    p_b2b = b2b_time_ms(torch, lambda: moe.moe_permute(g["X"], idx, E))
    c_b2b = b2b_time_ms(torch, lambda: moe.moe_combine(Y, w, inv))
    # Cold: the same 512 MiB read before every call as for the gate, so that the
    # steps' working sets (about 200 MB here) are not served from the 256 MB
    # Infinity Cache; outputs and workspace preallocated.
    flush = make_flush(torch, dev)
    p_out = (torch.empty_like(sp), torch.empty_like(inv), torch.empty_like(Xp))
    p_ws = torch.empty(moe.load_library().moe_permute_workspace_bytes(T, E, K), dtype=torch.uint8, device=dev)
    c_out = torch.empty((T, d), dtype=cfg.torch_dtype, device=dev)
    p_cold, _ = event_time_ms(torch, lambda: moe.moe_permute(g["X"], idx, E, out=p_out, ws=p_ws), 20, flush=flush)
    c_cold, _ = event_time_ms(torch, lambda: moe.moe_combine(Y, w, inv, out=c_out), 20, flush=flush)
    del p_out, p_ws, c_out
    s = 2  # bf16 bytes
    perm_bytes = T * (s * d * (1 + K) + 12 * K)
    comb_bytes = T * (s * d * (K + 1) + 8 * K)
    route_bytes = T * (4 * E + 8 * K)
    ffn_tflops = flops / (f_ms * 1e-3) / 1e12
    counts_h = counts.cpu().numpy()

    # Gate on the large gate-only workload with cold caches: before every call
    # a 512 MiB buffer is read (not written, so that the call does not pay for
    # writing back someone else's dirty lines), which evicts the 134 MB of
    # logits from L2 and the 256 MB Infinity Cache.
    gcfg = synth.CONFIGS["gate_l"]
    glg = synth.make_inputs(gcfg, dev, seed=0)["logits"]
    g_out = moe.moe_route(glg, gcfg.K)  # outputs and workspace reused: no allocation between the events
    g_ws = torch.empty(max(moe.load_library().moe_route_workspace_bytes(gcfg.T, gcfg.E, gcfg.K), 1),
                       dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    g_ms, _ = event_time_ms(torch, lambda: moe.moe_route(glg, gcfg.K, out=g_out, ws=g_ws), 20, flush=flush)
    # warm: 20 calls back to back on the same logits (steady state, no launch gaps)
    gs, ge = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gs.record()
    for _ in range(20):
        moe.moe_route(glg, gcfg.K, out=g_out, ws=g_ws)
    ge.record()
    ge.synchronize()
    g_warm_ms = gs.elapsed_time(ge) / 20
    gate_bytes = gcfg.T * (4 * gcfg.E + 8 * gcfg.K)
    # the small gate workload: launch-bound, reported for context (warm, back to back)
    scfg = synth.CONFIGS["gate_s"]
    slg = synth.make_inputs(scfg, dev, seed=0)["logits"]
    s_out = moe.moe_route(slg, scfg.K)  # preallocated outputs and workspace: no allocation inside the timed calls
    s_ws = torch.empty(max(moe.load_library().moe_route_workspace_bytes(scfg.T, scfg.E, scfg.K), 1),
                       dtype=torch.uint8, device=dev)
    s_ms = b2b_time_ms(torch, lambda: moe.moe_route(slg, scfg.K, out=s_out, ws=s_ws))
    gate_small = {"workload": f"gate-only fp32 logits [T={scfg.T}, E={scfg.E}], K={scfg.K} (N(0,1))",
                  "value": scfg.T / (s_ms * 1e-3) / 1e9, "unit": "Gtokens/s", "us_per_call_back_to_back": s_ms * 1e3,
                  "note": "two launches of a few us each; back to back, the host's launch time per call bounds it"}
    gate = {"workload": "gate-only fp32 logits [T=262144, E=128], K=8 (N(0,1))",
            "value": gcfg.T / (g_ms * 1e-3) / 1e9, "unit": "Gtokens/s", "us_per_call": g_ms * 1e3,
            "us_per_call_warm": g_warm_ms * 1e3,
            "roofline": {"bound": "hbm", "achieved": gate_bytes / (g_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": gate_bytes / (g_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         "traffic": kernel_traffic("gate_l", "gate_kernel")}}
    del flush

    # Practical HBM ceiling: a plain 1 GiB device-to-device copy (torch copy_),
    # 20 copies back to back, best of 3; bytes = read + write.
    cp_src = torch.ones(256 << 20, dtype=torch.float32, device=dev)
    cp_dst = torch.empty_like(cp_src)
    cp_ms = b2b_time_ms(torch, lambda: cp_dst.copy_(cp_src))
    hbm_copy = {"what": "torch copy_ of 1 GiB, device to device, 20 back to back, best of 3; read + write bytes",
                "GB/s": 2 * cp_src.numel() * 4 / (cp_ms * 1e-3) / 1e9}
    hbm_copy["frac_of_8TBs"] = hbm_copy["GB/s"] / PEAK_HBM_GBS
    del cp_src, cp_dst

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
                   "active_flops_per_step": flops, "expert_counts": counts_h.tolist(),
                   "load": load_stats(counts_h, A, E)},
        "gate": gate,
        "gate_small": gate_small,
        "layer_from_x": layer_x,
        "hbm_copy": hbm_copy,
        "steps_us": {
            "router": {"us": rt_ms * 1e3, "us_back_to_back": rt_b2b * 1e3,
                       "frac_hbm_back_to_back": router_bytes / (rt_b2b * 1e-3) / 1e9 / PEAK_HBM_GBS},
            "route_x": layer_x.pop("route_x"),
            "route": {"us": r_ms * 1e3, "GB/s": route_bytes / (r_ms * 1e-3) / 1e9},
            "permute": {"us": p_ms * 1e3, "us_cold": p_cold * 1e3, "GB/s_cold": perm_bytes / (p_cold * 1e-3) / 1e9,
                        "frac_hbm": perm_bytes / (p_cold * 1e-3) / 1e9 / PEAK_HBM_GBS,
                        "us_back_to_back": p_b2b * 1e3,
                        "frac_hbm_back_to_back": perm_bytes / (p_b2b * 1e-3) / 1e9 / PEAK_HBM_GBS,
                        "note": "frac_hbm: one call (three launches) after a 512 MiB read flush; back to back "
                                "the working set partly stays in the Infinity Cache (context only)"},
            "grouped_ffn": {"us": f_ms * 1e3, "TFLOPS": ffn_tflops},
            "ffn_up": {"us": up_ms * 1e3, "TFLOPS": up_tflops},
            "ffn_down": {"us": dn_ms * 1e3, "TFLOPS": 2.0 * A * d * n / (dn_ms * 1e-3) / 1e12},
            "combine": {"us": c_ms * 1e3, "us_cold": c_cold * 1e3, "GB/s_cold": comb_bytes / (c_cold * 1e-3) / 1e9,
                        "frac_hbm": comb_bytes / (c_cold * 1e-3) / 1e9 / PEAK_HBM_GBS,
                        "us_back_to_back": c_b2b * 1e3,
                        "frac_hbm_back_to_back": comb_bytes / (c_b2b * 1e-3) / 1e9 / PEAK_HBM_GBS,
                        "note": "frac_hbm: one call after a 512 MiB read flush; back to back: context only"},
        },
        "roofline": {"kernel": "ffn_p4_kernel<true, false> (moe_ffn_up: Act = SiLU(Xp W1) * (Xp W3), one launch)",
                     "bound": "mfma", "achieved": round(up_tflops_mean, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(up_tflops_mean / PEAK_BF16_TFLOPS, 4),
                     "traffic": kernel_traffic("mixtral", "ffn_up"),
                     "algorithmic_flops_per_launch": up_flops, "us_per_launch_mean": up_mean_ms * 1e3,
                     "us_per_launch_median": up_ms * 1e3, "launches_timed": len(up_times),
                     "note": "achieved = 4*T*K*d*n FLOPs / the mean of single moe_ffn_up calls, each between "
                             "two HIP events on the library's stream (the GEMM launch and its split-tail fixup)"},
    }

    if not args.no_other_workloads:
        out["token_rounding"] = {"mixtral": token_rounding(cfg, g, plan, moe, torch, np, dev)}
        out["backward_data"] = backward_data(cfg, g, moe, torch, dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, g, args.cpu_seconds, np, torch, synth)
    if not args.no_other_workloads:
        del g, plan, Xp, Act, Y
        torch.cuda.empty_cache()
        out["other_workloads"] = {name: other_workload(name, moe, synth, torch, np, dev)
                                  for name in ("dsv3", "fine")}
    print(json.dumps(out), flush=True)


def layer_from_x(cfg, g, Wr, rb, moe, torch, dev, args, route_ms, router_ms):
    """The layer from the tokens and the router weights (moe_forward_x: the router
    projection fused with the gate, no logits round trip), per step as the headline
    is timed, and moe_route_x alone beside moe_router + moe_route."""
    T, d, E, K, n = cfg.T, cfg.d, cfg.E, cfg.K, cfg.n
    xplan = moe.ForwardXPlan(T, d, E, K, n, cfg.torch_dtype, dev)

    def step_x():
        xplan(g["X"], Wr, rb, g["W1"], g["W3"], g["W2"])

    for _ in range(args.warmup):
        step_x()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step_x()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    lib = moe.load_library()
    ws = torch.empty(lib.moe_route_x_workspace_bytes(T, d, E, K, 1), dtype=torch.uint8, device=dev)
    out = moe.moe_route_x(g["X"], Wr, rb, K, want_logits=False, ws=ws)
    rx_ms, _ = event_time_ms(torch, lambda: moe.moe_route_x(g["X"], Wr, rb, K, ws=ws, out=out), 20)
    rx_b2b = b2b_time_ms(torch, lambda: moe.moe_route_x(g["X"], Wr, rb, K, ws=ws, out=out))
    fused = bool(E <= 64 and d % 256 == 0)
    res = {"what": "moe_forward_x: the layer from X, Wr (and the bias) -- the router projection "
                   + ("fused with the gate (no logits round trip)" if fused else "then the gate"),
           "ms_per_step": round(ms, 4), "TFLOPS": 6.0 * T * K * d * n / (ms * 1e-3) / 1e12,
           "route_x": {"us": rx_ms * 1e3, "us_back_to_back": rx_b2b * 1e3, "fused": fused,
                       "router_plus_route_us": (router_ms + route_ms) * 1e3,
                       "note": "moe_route_x (split of Wr + the fused router-gate kernel + the scan) against "
                               "moe_router then moe_route, single calls"}}
    del xplan, ws, out
    torch.cuda.empty_cache()
    return res


def other_workload(name, moe, synth, torch, np, dev, steps=5):
    """Whole-layer time of another workload shape (context, not the headline):
    active TFLOP/s and the fraction of a per-step roofline that sums, over the
    kernels, max(FLOPs / bf16 peak, algorithmic bytes / HBM peak), with the
    weights of non-empty experts read once."""
    c = synth.CONFIGS[name]
    g = synth.make_inputs(c, dev, seed=0)
    plan = moe.ForwardPlan(c.T, c.d, c.E, c.K, c.n, c.torch_dtype, dev)

    def run():
        plan(g["X"], g["logits"], g["W1"], g["W3"], g["W2"])

    for _ in range(2):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    counts = plan.counts.cpu().numpy().astype(np.int64)
    A, d, n, E, K, T, s = c.T * c.K, c.d, c.n, c.E, c.K, c.T, 2
    # the router projection and the memory-bound steps on their own, back to back
    Wr, rb = synth.make_router(c, dev, seed=0)
    rws = torch.empty(max(moe.load_library().moe_router_workspace_bytes(d, E, 1), 1), dtype=torch.uint8, device=dev)
    rt = b2b_time_ms(torch, lambda: moe.moe_router(g["X"], Wr, rb, ws=rws))
    pt = b2b_time_ms(torch, lambda: moe.moe_permute(g["X"], plan.topk_idx, E))
    Yc = torch.zeros((A, d), dtype=c.torch_dtype, device=dev)
    ct = b2b_time_ms(torch, lambda: moe.moe_combine(Yc, plan.topk_w, plan.inv))
    BW = PEAK_HBM_GBS * 1e9
    steps = {"router_us": round(rt * 1e3, 1),
             "router_frac_of_roof": (max(2.0 * T * d * E / (PEAK_BF16_TFLOPS * 1e12),
                                         (T * d * s + d * E * 4 + T * E * 4) / BW) * 1e3) / rt,
             "permute_us": round(pt * 1e3, 1), "permute_frac_hbm": T * (s * d * (1 + K) + 12 * K) / BW * 1e3 / pt,
             "combine_us": round(ct * 1e3, 1), "combine_frac_hbm": T * (s * d * (K + 1) + 8 * K) / BW * 1e3 / ct}
    e_act = int((counts > 0).sum())
    P, BW = PEAK_BF16_TFLOPS * 1e12, PEAK_HBM_GBS * 1e9
    roof_s = (T * (4 * E + 8 * K)) / BW                                                        # gate
    roof_s += 2 * T * (s * d * (K + 1)) / BW                                                   # permute + combine
    roof_s += max(4.0 * A * d * n / P, (2 * e_act * d * n * s + A * (d + n) * s) / BW)        # SwiGLU GEMM
    roof_s += max(2.0 * A * d * n / P, (e_act * n * d * s + A * (n + d) * s) / BW)            # down GEMM
    # rows the MFMA tiles compute: whole 256-row tiles, and the last tile of an
    # expert at 32, 64 or 128 rows when its remainder fits
    def rows_computed(c):
        full, rem = divmod(int(c), 256)
        return full * 256 + (0 if rem == 0 else next(h for h in (32, 64, 128, 256) if rem <= h))
    padded = sum(rows_computed(x) for x in counts)
    res = {"workload": f"{name}: T={T}, d={d}, E={E}, K={K}, n={n}, {c.dtype}, logits {c.logits}"
                       + (f" (per-expert bias variance {c.bias_var})" if c.bias_var else ""),
           "ms_per_step": round(ms, 4), "TFLOPS": 6.0 * A * d * n / (ms * 1e-3) / 1e12,
           "roofline_ms": round(roof_s * 1e3, 4), "frac_of_roofline": roof_s * 1e3 / ms,
           "experts_nonempty": e_act, "max_count": int(counts.max()), "load": load_stats(counts, A, E),
           "steps_back_to_back": steps,
           "tile_padding": padded / A - 1.0,
           "token_rounding": token_rounding(c, g, plan, moe, torch, np, dev)}
    del g, plan, Yc, Wr, rb, rws
    torch.cuda.empty_cache()
    return res


def backward_data(c, g, moe, torch, dev, calls=3):
    """moe_backward_data on the same layer (dX and the router-logit gradient for a
    seeded dout): time per call, 3 calls back to back after one warm-up, and the
    rate of its grouped GEMMs, 10*d*n FLOPs per assignment (H1 and H3 recomputed,
    dA = dY W2^T, dXp = [dh1 | dh3] [W1^T ; W3^T])."""
    lib = moe.load_library()
    ws = torch.empty(lib.moe_backward_data_workspace_bytes(c.T, c.d, c.E, c.K, c.n, 1), dtype=torch.uint8,
                     device=dev)
    gen = torch.Generator(device="cpu").manual_seed(12)
    dout = torch.randn((c.T, c.d), generator=gen).to(c.torch_dtype).to(dev)

    def run():
        moe.moe_backward_data(g["X"], g["logits"], g["W1"], g["W3"], g["W2"], c.K, dout, ws=ws)

    ms = b2b_time_ms(torch, run, n=calls, reps=1)
    flops = 10.0 * c.T * c.K * c.d * c.n
    res = {"what": "dX, dlogits and dw (no weight gradients)", "ms_per_call": round(ms, 4),
           "TFLOPS": flops / (ms * 1e-3) / 1e12, "flops_per_call": flops}
    res["frac_of_bf16_peak"] = res["TFLOPS"] / PEAK_BF16_TFLOPS
    del ws
    # with the expert-weight gradients: 6*d*n more FLOPs per assignment
    wsw = torch.empty(lib.moe_backward_workspace_bytes(c.T, c.d, c.E, c.K, c.n, 1), dtype=torch.uint8, device=dev)

    def run_w():
        moe.moe_backward(g["X"], g["logits"], g["W1"], g["W3"], g["W2"], c.K, dout, ws=wsw)

    ms_w = b2b_time_ms(torch, run_w, n=calls, reps=1)
    flops_w = 16.0 * c.T * c.K * c.d * c.n
    res["with_weight_gradients"] = {"ms_per_call": round(ms_w, 4), "TFLOPS": flops_w / (ms_w * 1e-3) / 1e12,
                                    "flops_per_call": flops_w}
    res["with_weight_gradients"]["frac_of_bf16_peak"] = res["with_weight_gradients"]["TFLOPS"] / PEAK_BF16_TFLOPS
    del wsw, dout
    torch.cuda.empty_cache()
    return res


def load_stats(counts, A, E):
    """Expert load of the routing: smallest and largest count, empty experts,
    and the variance of the load fractions f_e = count_e / (T*K) around 1/E."""
    f = [int(x) / A for x in counts]
    return {"min": int(min(counts)), "max": int(max(counts)), "empty": int(sum(1 for x in counts if int(x) == 0)),
            "var_f": sum((x - 1.0 / E) ** 2 for x in f) / E}


def token_rounding(c, g, plan_topk, moe, torch, np, dev, steps=5, M=256):
    """The layer with Token Rounding (page "MoE architecture optimisation and
    SonicMoE practice", section 3) at tile height M, timed beside plain top-K
    routing on the same inputs in the same run: time per step, rows the grouped
    GEMMs compute, and the plan and its combine on their own, back to back,
    against their algorithmic bytes."""
    T, d, E, K, n, s = c.T, c.d, c.E, c.K, c.n, 2
    trp = moe.ForwardTRPlan(T, d, E, K, n, M, c.torch_dtype, dev)

    def run_tr():
        trp(g["X"], g["logits"], g["W1"], g["W3"], g["W2"])

    def run_topk():
        plan_topk(g["X"], g["logits"], g["W1"], g["W3"], g["W2"])

    def per_step(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    ms_tr = per_step(run_tr)
    ms_topk = per_step(run_topk)
    R = int(trp.offsets_r[-1].item())
    counts_r = trp.counts_r.cpu().numpy().astype(np.int64)
    counts = plan_topk.counts.cpu().numpy().astype(np.int64)
    kept_routed = int(np.minimum(counts, counts_r).sum())  # routed pairs an expert keeps
    idx, _, cnt, _ = moe.moe_route(g["logits"], K)
    plan_ms = b2b_time_ms(torch, lambda: moe.moe_token_round(g["logits"], idx, cnt, M))
    Yr = torch.zeros((max(R, 1), d), dtype=c.torch_dtype, device=dev)
    comb_ms = b2b_time_ms(torch, lambda: moe.moe_tr_combine(Yr, trp.slot_row, trp.slot_w))
    BW = PEAK_HBM_GBS * 1e9
    plan_bytes = 12 * T * E + 4 * T * K + 4 * R
    comb_bytes = 8 * T * E + (R + T) * d * s
    res = {"M": M, "ms_per_step": round(ms_tr, 4), "ms_per_step_topk_same_run": round(ms_topk, 4),
           "rows": R, "rows_topk": T * K, "routed_pairs_dropped": T * K - kept_routed,
           "pairs_added": R - kept_routed, "tile_padding": 0.0 if R == 0 else float(
               sum(-(-int(x) // 256) * 256 for x in counts_r) / R - 1.0),
           "TFLOPS_of_rows": 6.0 * R * d * n / (ms_tr * 1e-3) / 1e12,
           "plan_us_back_to_back": round(plan_ms * 1e3, 2), "plan_frac_hbm": plan_bytes / BW * 1e3 / plan_ms,
           "combine_us_back_to_back": round(comb_ms * 1e3, 2), "combine_frac_hbm": comb_bytes / BW * 1e3 / comb_ms}
    del trp, Yr
    torch.cuda.empty_cache()
    return res


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, g, budget_s, np, torch, synth):
    """The oracle, as it stands: its route (softmax, top-K, histogram, offsets)
    and permutation over all T, timed alone, and its per-token layer loop on a
    bounded token sample."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    X = synth.to_numpy(g["X"])
    lg = synth.to_numpy(g["logits"])
    route_s = []
    for _ in range(3):
        t0 = time.perf_counter()
        idx, _, _, _ = oracle.route(lg, cfg.K)
        oracle.permute(idx, cfg.E)
        route_s.append(time.perf_counter() - t0)
    route_s = statistics.median(route_s)
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
            "cpu_model": cpu_model(), "kind": "oracle",
            "route_s_all_tokens": route_s, "route_Gtokens_per_s": cfg.T / route_s / 1e9,
            "layer_s_per_token": dt2 / ntok2, "layer_s_all_tokens_estimate": dt2 / ntok2 * cfg.T,
            "sample": f"route + permutation: all {cfg.T} tokens (median of 3); layer: {ntok2} of {cfg.T} tokens "
                      f"of the mixtral-shaped layer through the oracle's per-token loop (route + {cfg.K} expert "
                      f"SwiGLU MLPs + combine, fp64 accumulation), {dt2:.1f} s wall; value = active TFLOPS of "
                      f"those tokens"}


if __name__ == "__main__":
    main()
