"""GPU parity of the calls that start from the tokens: moe_route_x (the router
projection fused with the gate for bf16, d % 256 == 0, E <= 64; the router
then the gate elsewhere) and moe_forward_x (the whole layer from X and Wr).

The fused kernel computes the logits exactly as moe_router does, so:
  * the logits it can return equal moe_router's bit for bit, and stay within
    the router's error bound of the oracle's fp64 sums;
  * the routing equals the oracle's gate on those GPU logits: indices, counts
    and offsets bit for bit, weights within 1e-5 relative;
  * moe_forward_x has moe_forward's routing on those logits (indices and the
    permutation bit for bit; the weights of the two gates may differ in the
    last bits, since they sum the K exponentials in different orders), and its
    output equals moe_forward's bit for bit on every token whose weights are
    identical (the same kernels after the routing); the other tokens, and the
    whole output on small shapes, are checked against the oracle's layer."""
import numpy as np
import pytest
import torch

import mixture_experts_routing_gate_amd as moe
import oracle
import synth
from parity_util import check_close, check_equal, check_weights, cuda, to_np
from test_gpu_router import _check_logits

pytestmark = pytest.mark.gpu


def _router_inputs(T, d, E, dt, bv, seed=5):
    cfg = synth.MoEConfig("rx", T=T, d=d, E=E, K=1, n=128, dtype=dt, logits="proj_bias" if bv else "proj",
                          bias_var=bv)
    X = synth._normal((T, d), 1.0, cfg.torch_dtype, torch.device("cpu"), synth._gen("cpu", seed, "X"))
    Wr, b = synth.make_router(cfg, "cpu", seed)
    return X, Wr, b


def _check_route(lg, idx, w, counts, offsets, K):
    ridx, rw, rc, ro = oracle.route(lg.cpu().numpy(), K)
    check_equal(idx, ridx, "topk_idx")
    check_equal(counts, rc, "counts")
    check_equal(offsets, ro, "offsets")
    check_weights(w.cpu().numpy(), rw)


# (T, d, E, K, dtype, bias variance).  Fused: E <= 64 with bf16 and d % 256 == 0
# (E padded to 32 or 64, 4 or 8 gate lanes per token, ragged last tiles, one
# token, K up to 8).  Not fused: E > 64, d % 256 != 0, fp32.
CASES = [
    (300, 512, 8, 2, "bf16", 0.0),
    (1000, 256, 16, 4, "bf16", 1.0),
    (33, 1024, 32, 8, "bf16", 0.5),
    (1, 256, 8, 1, "bf16", 0.0),
    (513, 768, 40, 3, "bf16", 2.0),
    (257, 256, 64, 8, "bf16", 1.5),
    (70001, 256, 8, 2, "bf16", 0.0),
    (257, 768, 256, 8, "bf16", 1.5),
    (100, 1536, 128, 4, "bf16", 2.0),
    (33, 384, 8, 2, "bf16", 0.0),
    (256, 128, 8, 2, "f32", 0.0),
    # staged E <= 32 with E not a multiple of 8
    (130, 512, 12, 3, "bf16", 0.5),
    (500, 768, 27, 5, "bf16", 1.0),
]


@pytest.mark.parametrize("T,d,E,K,dt,bv", CASES, ids=lambda v: str(v))
def test_route_x_matches_router_and_oracle(T, d, E, K, dt, bv):
    print(f"[route_x] T={T} d={d} E={E} K={K} {dt}", flush=True)
    X, Wr, b = _router_inputs(T, d, E, dt, bv)
    Xg, Wg, bg = cuda(X), cuda(Wr), None if b is None else cuda(b)
    idx, w, counts, offsets, lg = moe.moe_route_x(Xg, Wg, bg, K)
    lg_r = moe.moe_router(Xg, Wg, bg)
    idx2, w2, counts2, offsets2, none = moe.moe_route_x(Xg, Wg, bg, K, want_logits=False)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(lg.view(torch.int32), lg_r.view(torch.int32)), "logits differ from moe_router's"
    rows = None if T <= 2000 else np.unique(np.r_[np.random.default_rng(2).choice(T, 64, replace=False), 0, T - 1])
    _check_logits(lg, to_np(X), Wr.numpy(), None if b is None else b.numpy(), rows=rows)
    _check_route(lg, idx, w, counts, offsets, K)
    # without the logits output the routing is the same, bit for bit
    for a, c in ((idx, idx2), (w, w2), (counts, counts2), (offsets, offsets2)):
        assert torch.equal(a.view(torch.int32), c.view(torch.int32))


def test_route_x_ties():
    """Zero token rows make the logits equal the bias exactly: a bias with
    repeated values and +-0.0 gives exact ties, which go to the lower expert;
    two equal columns of Wr tie on every row."""
    T, d, E, K = 200, 256, 32, 8
    X, Wr, _ = _router_inputs(T, d, E, "bf16", 0.0, seed=9)
    X[::3] = 0
    Wr[:, 7] = Wr[:, 3]
    Wr[:, 30] = Wr[:, 12]
    b = torch.tensor([0.5, -0.0, 0.5, 0.0, 1.25, 1.25, 0.0, -0.0] * 4, dtype=torch.float32)
    idx, w, counts, offsets, lg = moe.moe_route_x(cuda(X), cuda(Wr), cuda(b), K)
    torch.cuda.synchronize()
    _check_route(lg, idx, w, counts, offsets, K)
    zr = idx[::3].cpu().numpy()
    # the bias ranks 1.25 (4,5,12,13,...), then 0.5 (0,2,8,10,...): lower index first among equals
    assert zr[0, :4].tolist() == [4, 5, 12, 13], zr[0]


FWD_CASES = [
    synth.MoEConfig("fx_small", T=512, d=256, E=8, K=2, n=384, logits="proj"),
    synth.MoEConfig("fx_e64", T=700, d=512, E=64, K=4, n=128, logits="proj_bias", bias_var=2.0),
    synth.MoEConfig("fx_e128", T=300, d=256, E=128, K=4, n=128, logits="proj_bias", bias_var=2.0),
    synth.MoEConfig("fx_tile128", T=300, d=384, E=16, K=2, n=128, logits="proj"),
    synth.MoEConfig("fx_f32", T=256, d=128, E=8, K=2, n=256, dtype="f32", logits="proj"),
]


@pytest.mark.parametrize("cfg", FWD_CASES, ids=lambda c: c.name)
def test_forward_x_matches_forward_and_oracle(cfg):
    inp = synth.make_inputs(cfg, "cpu", 0)
    Wr, b = synth.make_router(cfg, "cpu", 0)
    g = {k: cuda(v) for k, v in inp.items()}
    Wg, bg = cuda(Wr), None if b is None else cuda(b)
    out_x, plan_x = moe.moe_forward_x(g["X"], Wg, bg, g["W1"], g["W3"], g["W2"], cfg.K)
    lg = moe.moe_router(g["X"], Wg, bg)
    out, plan = moe.moe_forward(g["X"], lg, g["W1"], g["W3"], g["W2"], cfg.K)
    torch.cuda.synchronize()
    assert torch.equal(plan_x.logits.view(torch.int32), lg.view(torch.int32))
    for k in ("topk_idx", "counts", "offsets", "sorted_pair", "inv"):
        assert torch.equal(getattr(plan_x, k), getattr(plan, k)), k
    _check_route(lg, plan_x.topk_idx, plan_x.topk_w, plan_x.counts, plan_x.offsets, cfg.K)
    _same_where_weights_equal(out_x, out, plan_x.topk_w, plan.topk_w, cfg)
    ref = oracle.layer(to_np(inp["X"]), lg.cpu().numpy(), to_np(inp["W1"]), to_np(inp["W3"]), to_np(inp["W2"]), cfg.K)
    check_close(out_x, ref, cfg.dtype, "out")


def _same_where_weights_equal(out_x, out, w_x, w, cfg):
    """Tokens whose weights are bit-identical get bit-identical outputs; returns the others."""
    same = (w_x.view(torch.int32) == w.view(torch.int32)).all(dim=1)
    bits = torch.int16 if cfg.dtype == "bf16" else torch.int32
    assert torch.equal(out_x[same].view(bits), out[same].view(bits)), "outputs differ where the routing is identical"
    return np.nonzero(~same.cpu().numpy())[0].astype(np.int32)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["mixtral", "dsv3"])
def test_forward_x_full_size(name):
    """The layer from X at full size (fused router-gate on the mixtral shape, router
    then gate on the DeepSeek-V3 one): routing bit-exact against the oracle's gate on
    the GPU's logits, the logits within the router bound on sampled rows, and the
    output equal to moe_forward's on those logits bit for bit."""
    cfg = synth.CONFIGS[name]
    print(f"[forward_x] {name}", flush=True)
    g = synth.make_inputs(cfg, "cuda", 0)
    Wr, b = synth.make_router(cfg, "cuda", 0)
    plan_x = moe.ForwardXPlan(cfg.T, cfg.d, cfg.E, cfg.K, cfg.n, cfg.torch_dtype, "cuda", want_logits=True)
    out_x = plan_x(g["X"], Wr, b, g["W1"], g["W3"], g["W2"])
    lg = plan_x.logits
    plan = moe.ForwardPlan(cfg.T, cfg.d, cfg.E, cfg.K, cfg.n, cfg.torch_dtype, "cuda")
    out = plan(g["X"], lg, g["W1"], g["W3"], g["W2"])
    torch.cuda.synchronize()
    _check_route(lg, plan_x.topk_idx, plan_x.topk_w, plan_x.counts, plan_x.offsets, cfg.K)
    rsp, rinv = oracle.permute(plan_x.topk_idx.cpu().numpy(), cfg.E)
    check_equal(plan_x.sorted_pair, rsp, "sorted_pair")
    check_equal(plan_x.inv, rinv, "inv")
    rows = np.unique(np.r_[np.random.default_rng(3).choice(cfg.T, 48, replace=False), 0, cfg.T - 1])
    X_h = to_np(g["X"])
    _check_logits(lg, X_h, Wr.cpu().numpy(), None if b is None else b.cpu().numpy(), rows=rows)
    for k in ("topk_idx", "counts", "offsets", "sorted_pair", "inv"):
        assert torch.equal(getattr(plan_x, k), getattr(plan, k)), k
    other = _same_where_weights_equal(out_x, out, plan_x.topk_w, plan.topk_w, cfg)
    print(f"[forward_x] {name}: {other.size} tokens with weights unlike moe_forward's", flush=True)
    if other.size:
        toks = other[:64]
        ref = oracle.layer(X_h, lg.cpu().numpy(), to_np(g["W1"]), to_np(g["W3"]), to_np(g["W2"]), cfg.K, tokens=toks)
        check_close(out_x[torch.from_numpy(toks).long().cuda()], ref, cfg.dtype, "out (tokens with other weights)")
