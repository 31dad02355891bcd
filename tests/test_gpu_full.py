"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: routing and permutation compared in full (the oracle does
those for every token in seconds); the layer output, Act and Y compared on
sampled tokens/rows that the oracle computes one by one.  Inputs are drawn on
the GPU (weights are gigabytes) and copied to the host for the oracle."""
import numpy as np
import pytest
import torch

import mixture_experts_routing_gate_amd as moe
import oracle
import synth
from parity_util import check_close, check_equal, check_weights, to_np

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def sample_tokens(T, idx, counts, n_rand=12, seed=0):
    rng = np.random.default_rng(seed)
    toks = set(rng.choice(T, size=min(n_rand, T), replace=False).tolist()) | {0, T - 1}
    # tokens routed to the smallest non-empty expert (ragged tails)
    nz = np.nonzero(counts)[0]
    small = nz[np.argmin(counts[nz])]
    toks |= set(np.nonzero((idx == small).any(1))[0][:2].tolist())
    return np.array(sorted(toks), np.int32)


@pytest.mark.parametrize("name", ["gate_s", "gate_l"])
def test_full_gate(name):
    cfg = synth.CONFIGS[name]
    lg = synth.make_inputs(cfg, "cuda", 0)["logits"]
    idx, w, counts, offsets = moe.moe_route(lg, cfg.K)
    torch.cuda.synchronize()
    ridx, rw, rc, ro = oracle.route(to_np(lg), cfg.K)
    check_equal(idx, ridx, "topk_idx")
    check_equal(counts, rc, "counts")
    check_equal(offsets, ro, "offsets")
    check_weights(w.cpu().numpy(), rw)


@pytest.mark.parametrize("name", ["mixtral", "fine", "dsv3"])
def test_full_layer(name):
    cfg = synth.CONFIGS[name]
    print(f"[full] {name}: generating inputs", flush=True)
    g = synth.make_inputs(cfg, "cuda", 0)
    plan = moe.ForwardPlan(cfg.T, cfg.d, cfg.E, cfg.K, cfg.n, cfg.torch_dtype, "cuda")
    print(f"[full] {name}: moe_forward", flush=True)
    out = plan(g["X"], g["logits"], g["W1"], g["W3"], g["W2"])
    torch.cuda.synchronize()

    lg = to_np(g["logits"])
    ridx, rw, rc, ro = oracle.route(lg, cfg.K)
    check_equal(plan.topk_idx, ridx, "topk_idx")
    check_equal(plan.counts, rc, "counts")
    check_equal(plan.offsets, ro, "offsets")
    check_weights(plan.topk_w.cpu().numpy(), rw)
    rsp, rinv = oracle.permute(ridx, cfg.E)
    check_equal(plan.sorted_pair, rsp, "sorted_pair")
    check_equal(plan.inv, rinv, "inv")

    # the steps one by one on the same inputs, to expose Xp, Act and Y
    print(f"[full] {name}: step-by-step entry points", flush=True)
    sp, inv, Xp = moe.moe_permute(g["X"], plan.topk_idx, cfg.E)
    Act, Y = moe.moe_grouped_ffn(Xp, g["W1"], g["W3"], g["W2"], plan.counts, plan.offsets, cfg.K)
    out2 = moe.moe_combine(Y, plan.topk_w, inv)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16)), "forward != step-by-step"

    print(f"[full] {name}: host copies + oracle on sampled tokens", flush=True)
    X_h = to_np(g["X"])
    W_h = {k: to_np(g[k]) for k in ("W1", "W3", "W2")}
    toks = sample_tokens(cfg.T, ridx, rc)
    ref = oracle.layer(X_h, lg, W_h["W1"], W_h["W3"], W_h["W2"], cfg.K, tokens=toks)
    check_close(out[torch.from_numpy(toks).long().cuda()], ref, cfg.dtype, "out (sampled tokens)")

    rows = np.unique(np.concatenate([rinv[(toks[:, None] * cfg.K + np.arange(cfg.K)).ravel()],
                                     ro[:-1][rc > 0], (ro[1:] - 1)[rc > 0]]))[:96].astype(np.int32)
    check_equal(Xp[torch.from_numpy(rows).long().cuda()], X_h[rsp[rows] // cfg.K], "Xp (sampled rows)")
    row_expert = ridx.ravel()[rsp[rows]].astype(np.int32)
    ract, ry = oracle.expert_ffn(X_h[rsp[rows] // cfg.K], row_expert, W_h["W1"], W_h["W3"], W_h["W2"])
    sel = torch.from_numpy(rows).long().cuda()
    check_close(Act[sel], ract, cfg.dtype, "Act (sampled rows)")
    check_close(Y[sel], ry, cfg.dtype, "Y (sampled rows)")
