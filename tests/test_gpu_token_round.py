"""GPU parity of Token Rounding (page "MoE architecture optimisation and
SonicMoE practice", section 3) against the oracle: the plan (row counts,
offsets, row tokens, slot rows) bit for bit and the renormalised weights to
1e-5 relative; the combine over a plan; the whole layer with Token Rounding
on small configs in full, and at the Mixtral and DeepSeek-V3 sizes on sampled
tokens."""
import numpy as np
import pytest
import torch

import mixture_experts_routing_gate_amd as moe
import oracle
import synth
from parity_util import check_close, check_equal, check_weights, cuda, to_np

pytestmark = pytest.mark.gpu


def _logits(T, E, seed, levels=0, bias_var=0.0):
    rng = np.random.default_rng(seed)
    if levels:
        lg = rng.integers(0, levels, size=(T, E)).astype(np.float32) * np.float32(0.25)
    else:
        lg = rng.standard_normal((T, E)).astype(np.float32)
    if bias_var:
        lg = (lg + np.sqrt(bias_var) * rng.standard_normal(E)).astype(np.float32)
    return lg


def _check_plan(plan, ref):
    check_equal(plan["counts_r"], ref["counts_r"], "counts_r")
    check_equal(plan["offsets_r"], ref["offsets_r"], "offsets_r")
    rows = int(ref["offsets_r"][-1])
    check_equal(plan["row_tok"][:rows], ref["row_tok"], "row_tok")
    check_equal(plan["slot_row"], ref["slot_row"], "slot_row")
    check_weights(plan["slot_w"].cpu().numpy(), ref["slot_w"])


PLAN_CASES = [
    # (name, T, E, K, M, cap_tiles, levels, bias_var)
    ("small", 256, 8, 2, 16, 0, 0, 0.0),
    ("ties", 1000, 16, 4, 32, 0, 6, 0.0),          # coarse logits: ties inside experts
    ("cap2", 3000, 8, 2, 64, 2, 0, 0.0),           # the page's limit of 2M rows
    ("m1", 777, 8, 2, 1, 0, 0, 0.0),               # M = 1: plain top-K
    ("k_eq_e", 300, 4, 4, 64, 0, 0, 0.0),          # every token routed to every expert
    ("t_below_m", 5, 4, 2, 8, 0, 0, 0.0),          # rounding up past T rounds down
    ("skewed_e64", 70001, 64, 4, 128, 0, 0, 2.0),  # many select blocks, ragged last block
    ("t_16384", 16384, 16, 2, 256, 0, 5, 1.0),     # largest T whose tokens the select stages in LDS
    ("t_16385", 16385, 16, 2, 256, 0, 5, 1.0),     # one past it: 17 tokens a thread, read from global memory
    ("mixtral_routing", 8192, 8, 2, 256, 0, 0, 0.0),
    ("dsv3_routing", 8192, 256, 8, 256, 0, 0, 1.5),
]


@pytest.mark.parametrize("case", PLAN_CASES, ids=lambda c: c[0])
def test_plan_matches_oracle(case):
    name, T, E, K, M, cap, levels, bias_var = case
    print(f"[tr] plan {name}: T={T} E={E} K={K} M={M} cap={cap}", flush=True)
    lg = _logits(T, E, 7, levels, bias_var)
    lg_d = cuda(torch.from_numpy(lg))
    idx, _, counts, _ = moe.moe_route(lg_d, K)
    plan = moe.moe_token_round(lg_d, idx, counts, M, cap)
    torch.cuda.synchronize()
    _check_plan(plan, oracle.token_round(lg, K, M, cap))


def test_plan_repeats_bit_for_bit():
    lg = _logits(5000, 32, 9, 4)
    lg_d = cuda(torch.from_numpy(lg))
    idx, _, counts, _ = moe.moe_route(lg_d, 4)
    a = moe.moe_token_round(lg_d, idx, counts, 64)
    b = moe.moe_token_round(lg_d, idx, counts, 64)
    torch.cuda.synchronize()
    rows = int(a["offsets_r"][-1])
    assert rows == int(b["offsets_r"][-1])
    a["row_tok"], b["row_tok"] = a["row_tok"][:rows], b["row_tok"][:rows]  # entries past rows are not written
    for k in a:
        assert torch.equal(a[k].view(torch.int32), b[k].view(torch.int32)), k


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_tr_combine_matches_oracle(dtype):
    T, E, K, M, d = 1500, 16, 4, 32, 384 if dtype == "bf16" else 96
    lg = _logits(T, E, 3)
    ref = oracle.token_round(lg, K, M)
    rows = int(ref["offsets_r"][-1])
    rng = np.random.default_rng(5)
    Yf = rng.standard_normal((rows, d)).astype(np.float32)
    Yt = torch.from_numpy(Yf).to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    out = moe.moe_tr_combine(cuda(Yt), cuda(torch.from_numpy(ref["slot_row"])),
                             cuda(torch.from_numpy(ref["slot_w"])))
    torch.cuda.synchronize()
    want = oracle.tr_combine(Yt.float().numpy(), ref["slot_row"], ref["slot_w"])
    check_close(out, want, dtype, "tr_combine out")
    # tokens that kept no expert get zero rows
    none = ~(ref["slot_row"] >= 0).any(axis=1)
    assert torch.all(out.float().cpu()[torch.from_numpy(none)] == 0)


LAYER_CASES = [
    synth.MoEConfig("tiny", T=256, d=128, E=8, K=2, n=256, dtype="f32"),
    synth.MoEConfig("small_bf16", T=512, d=256, E=8, K=2, n=384),
    synth.MoEConfig("ragged_bias", T=1000, d=256, E=64, K=4, n=128, logits="bias", bias_var=2.0),
    synth.MoEConfig("fine_small", T=2048, d=256, E=128, K=4, n=128, logits="bias", bias_var=2.0),
]


@pytest.mark.parametrize("cfg", LAYER_CASES, ids=lambda c: c.name)
@pytest.mark.parametrize("M,cap", [(256, 0), (64, 0), (32, 2)])
def test_forward_tr_matches_oracle(cfg, M, cap):
    print(f"[tr] forward {cfg.name} M={M} cap={cap}", flush=True)
    inp = synth.make_inputs(cfg, "cpu", 0)
    lg = to_np(inp["logits"])
    out, plan = moe.moe_forward_tr(cuda(inp["X"]), cuda(inp["logits"]), cuda(inp["W1"]), cuda(inp["W3"]),
                                   cuda(inp["W2"]), cfg.K, M, cap)
    torch.cuda.synchronize()
    ref = oracle.token_round(lg, cfg.K, M, cap)
    _check_plan({"counts_r": plan.counts_r, "offsets_r": plan.offsets_r, "row_tok": plan.row_tok,
                 "slot_row": plan.slot_row, "slot_w": plan.slot_w}, ref)
    want = oracle.tr_layer(to_np(inp["X"]), ref["slot_row"], ref["slot_w"], to_np(inp["W1"]), to_np(inp["W3"]),
                           to_np(inp["W2"]))
    check_close(out, want, cfg.dtype, "out")


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["mixtral", "dsv3", "fine"])
def test_forward_tr_full_size(name):
    cfg = synth.CONFIGS[name]
    print(f"[tr] full {name}: generating inputs", flush=True)
    g = synth.make_inputs(cfg, "cuda", 0)
    plan = moe.ForwardTRPlan(cfg.T, cfg.d, cfg.E, cfg.K, cfg.n, 256, cfg.torch_dtype, "cuda")
    print(f"[tr] full {name}: moe_forward_tr", flush=True)
    out = plan(g["X"], g["logits"], g["W1"], g["W3"], g["W2"])
    torch.cuda.synchronize()
    lg = to_np(g["logits"])
    ref = oracle.token_round(lg, cfg.K, 256)
    _check_plan({"counts_r": plan.counts_r, "offsets_r": plan.offsets_r, "row_tok": plan.row_tok,
                 "slot_row": plan.slot_row, "slot_w": plan.slot_w}, ref)
    assert np.all(ref["counts_r"] % 256 == 0)
    print(f"[tr] full {name}: oracle on all {cfg.T} tokens", flush=True)
    X_h = to_np(g["X"])
    want = oracle.tr_layer(X_h, ref["slot_row"], ref["slot_w"], to_np(g["W1"]), to_np(g["W3"]), to_np(g["W2"]))
    check_close(out, want, cfg.dtype, "out (every token)")
    # the tokens whose expert set changed (a kept expert outside the top-K, or a
    # dropped one) and those that kept none, on their own
    kept = ref["slot_row"] >= 0
    idx, _, _, _ = oracle.route(lg, cfg.K)
    routed = np.zeros_like(kept)
    routed[np.repeat(np.arange(cfg.T), cfg.K), idx.reshape(-1)] = True
    changed = np.nonzero((kept != routed).any(axis=1))[0]
    if changed.size:
        sel = torch.from_numpy(changed).long().cuda()
        check_close(out[sel], want[changed], cfg.dtype, f"out ({changed.size} tokens with a changed expert set)")
    none = np.nonzero(~kept.any(axis=1))[0]
    if none.size:
        assert not out[torch.from_numpy(none).long().cuda()].float().abs().max().item(), "token with no row"
