"""GPU parity of moe_forward (the whole layer) against the oracle's per-token
layer loop, on small configs where the oracle covers every token, plus the
degenerate cases of the method."""
import numpy as np
import pytest
import torch

import mixture_experts_routing_gate_amd as moe
import oracle
import synth
from parity_util import check_close, check_equal, check_weights, cuda, to_np

pytestmark = pytest.mark.gpu

CASES = [
    synth.CONFIGS["tiny"],
    synth.MoEConfig("small_bf16", T=512, d=256, E=8, K=2, n=384),
    synth.MoEConfig("ragged_bias", T=1000, d=256, E=64, K=4, n=128, logits="bias", bias_var=2.0),
    synth.MoEConfig("dense_e1", T=130, d=128, E=1, K=1, n=256),
    synth.MoEConfig("k_equals_e", T=100, d=128, E=8, K=8, n=128),
    synth.MoEConfig("t1", T=1, d=128, E=16, K=4, n=128),
    synth.MoEConfig("min_dims", T=257, d=128, E=4, K=2, n=128),
    synth.MoEConfig("fine_small", T=2048, d=256, E=128, K=4, n=128, logits="bias", bias_var=2.0),
    synth.MoEConfig("f32_e256", T=300, d=64, E=256, K=8, n=64, dtype="f32"),
    # every expert short (a few rows each): short tiles, tile claiming, gathered loads
    synth.MoEConfig("bf16_e256_k8", T=600, d=256, E=256, K=8, n=128, logits="bias", bias_var=1.5),
]


def run_forward(cfg, inp, logits=None):
    lg = inp["logits"] if logits is None else logits
    out, plan = moe.moe_forward(cuda(inp["X"]), cuda(lg), cuda(inp["W1"]), cuda(inp["W3"]), cuda(inp["W2"]), cfg.K)
    torch.cuda.synchronize()
    return out, plan


def check_layer(cfg, inp, out, plan, lg_np):
    ridx, rw, rc, ro = oracle.route(lg_np, cfg.K)
    check_equal(plan.topk_idx, ridx, "topk_idx")
    check_equal(plan.counts, rc, "counts")
    check_equal(plan.offsets, ro, "offsets")
    check_weights(plan.topk_w.cpu().numpy(), rw)
    rsp, rinv = oracle.permute(ridx, cfg.E)
    check_equal(plan.sorted_pair, rsp, "sorted_pair")
    check_equal(plan.inv, rinv, "inv")
    ref = oracle.layer(to_np(inp["X"]), lg_np, to_np(inp["W1"]), to_np(inp["W3"]), to_np(inp["W2"]), cfg.K)
    return check_close(out, ref, cfg.dtype, "out")


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_forward_matches_oracle(cfg):
    inp = synth.make_inputs(cfg, "cpu", 0)
    out, plan = run_forward(cfg, inp)
    check_layer(cfg, inp, out, plan, to_np(inp["logits"]))


def test_forward_one_expert_takes_all():
    cfg = synth.MoEConfig("dominant", T=600, d=128, E=16, K=2, n=128)
    inp = synth.make_inputs(cfg, "cpu", 4)
    lg = inp["logits"].clone()
    lg[:, 5] += 30.0
    out, plan = run_forward(cfg, inp, lg)
    assert int(plan.counts[5]) == cfg.T
    check_layer(cfg, inp, out, plan, lg.numpy())


def test_forward_all_equal_logits_tie_break():
    cfg = synth.MoEConfig("ties", T=300, d=128, E=8, K=3, n=128)
    inp = synth.make_inputs(cfg, "cpu", 5)
    lg = torch.zeros(cfg.T, cfg.E)
    out, plan = run_forward(cfg, inp, lg)
    assert (plan.topk_idx.cpu() == torch.tensor([0, 1, 2], dtype=torch.int32)).all()
    check_layer(cfg, inp, out, plan, lg.numpy())


def test_forward_identical_experts_equal_dense_mlp():
    """All experts equal: the layer is the dense SwiGLU MLP whatever the routing."""
    cfg = synth.MoEConfig("ident", T=256, d=128, E=16, K=4, n=256)
    inp = synth.make_inputs(cfg, "cpu", 6)
    for k in ("W1", "W3", "W2"):
        inp[k] = inp[k][:1].repeat(cfg.E, 1, 1).contiguous()
    out, plan = run_forward(cfg, inp)
    dense = oracle.layer(to_np(inp["X"]), np.zeros((cfg.T, 1), np.float32), to_np(inp["W1"][:1]),
                         to_np(inp["W3"][:1]), to_np(inp["W2"][:1]), 1)
    check_close(out, dense, "bf16", "out vs dense MLP")


def test_forward_is_bitwise_deterministic():
    cfg = synth.MoEConfig("det", T=2048, d=256, E=32, K=4, n=256, logits="bias", bias_var=2.0)
    inp = synth.make_inputs(cfg, "cpu", 7)
    g = {k: cuda(v) for k, v in inp.items()}
    plan = moe.ForwardPlan(cfg.T, cfg.d, cfg.E, cfg.K, cfg.n, cfg.torch_dtype, "cuda")
    plan(g["X"], g["logits"], g["W1"], g["W3"], g["W2"])
    first = plan.out.clone()
    for _ in range(2):
        plan(g["X"], g["logits"], g["W1"], g["W3"], g["W2"])
        assert torch.equal(plan.out.view(torch.int16), first.view(torch.int16))
