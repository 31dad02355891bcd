"""GPU parity of moe_permute, moe_grouped_ffn and moe_combine, each fed the
oracle's exact upstream outputs so that every step is tested on its own."""
import numpy as np
import pytest
import torch

import mixture_experts_routing_gate_amd as moe
import oracle
import synth
from parity_util import as_f64, check_close, check_equal, cuda, from_np, to_np

pytestmark = pytest.mark.gpu


def routed(cfg: synth.MoEConfig, seed=0):
    """Host inputs of a small config plus the oracle's routing of them."""
    inp = synth.make_inputs(cfg, "cpu", seed)
    lg = to_np(inp["logits"])
    idx, w, counts, offsets = oracle.route(lg, cfg.K)
    sp, inv = oracle.permute(idx, cfg.E)
    return inp, lg, idx, w, counts, offsets, sp, inv


def forced_counts_idx(counts, K=1):
    """topk_idx [T,1] whose histogram is exactly `counts` (tokens dealt round-robin)."""
    E = len(counts)
    rem = list(counts)
    out = []
    e = 0
    while sum(rem):
        if rem[e]:
            out.append(e)
            rem[e] -= 1
        e = (e + 1) % E
    return np.array(out, np.int32).reshape(-1, K)


PERMUTE_CASES = [
    synth.MoEConfig("p1", T=1, d=128, E=4, K=1, n=128),
    synth.MoEConfig("p2", T=300, d=256, E=8, K=2, n=128),
    synth.MoEConfig("p3", T=1000, d=384, E=64, K=4, n=128, logits="bias", bias_var=2.0),
    synth.MoEConfig("p4", T=513, d=128, E=256, K=8, n=128, dtype="f32"),
    synth.MoEConfig("p5", T=70001, d=128, E=16, K=2, n=128),
    # many chunks times many experts: the scan runs as its own launch
    synth.MoEConfig("p6", T=70001, d=128, E=256, K=2, n=128),
]


@pytest.mark.parametrize("cfg", PERMUTE_CASES, ids=lambda c: c.name)
def test_permute_matches_oracle(cfg):
    rng = np.random.default_rng(cfg.T)
    lg = (rng.normal(size=(cfg.T, cfg.E)) + rng.normal(0, 2, cfg.E)).astype(np.float32)
    idx, _, _, _ = oracle.route(lg, cfg.K)
    X = synth._normal((cfg.T, cfg.d), 1.0, cfg.torch_dtype, torch.device("cpu"), synth._gen("cpu", 1, "X"))
    sp, inv, Xp = moe.moe_permute(cuda(X), cuda(torch.from_numpy(idx)), cfg.E)
    torch.cuda.synchronize()
    rsp, rinv = oracle.permute(idx, cfg.E)
    check_equal(sp, rsp, "sorted_pair")
    check_equal(inv, rinv, "inv")
    check_equal(Xp, oracle.gather_rows(to_np(X), rsp, cfg.K), "Xp")


FFN_CASES = [
    synth.CONFIGS["tiny"],
    synth.MoEConfig("ffn_bf16", T=512, d=256, E=8, K=2, n=384),
    synth.MoEConfig("ffn_ragged", T=300, d=128, E=16, K=4, n=256, logits="bias", bias_var=2.0),
    synth.MoEConfig("ffn_sparse", T=1000, d=256, E=64, K=4, n=128, logits="bias", bias_var=4.0),
    synth.MoEConfig("ffn_t1", T=1, d=128, E=4, K=1, n=128),
    synth.MoEConfig("ffn_dense", T=200, d=256, E=1, K=1, n=256),
    synth.MoEConfig("ffn_f32_ragged", T=333, d=192, E=8, K=3, n=128, dtype="f32", logits="bias", bias_var=2.0),
]


def _ffn_check(cfg, Xp_np, row_expert, counts, offsets, W):
    Act, Y = moe.moe_grouped_ffn(cuda(from_np(Xp_np)), cuda(W["W1"]), cuda(W["W3"]), cuda(W["W2"]),
                                 cuda(torch.from_numpy(counts)), cuda(torch.from_numpy(offsets)), cfg.K)
    torch.cuda.synchronize()
    ract, ry = oracle.expert_ffn(Xp_np, row_expert, to_np(W["W1"]), to_np(W["W3"]), to_np(W["W2"]))
    check_close(Act, ract, cfg.dtype, "Act")
    check_close(Y, ry, cfg.dtype, "Y")


@pytest.mark.parametrize("cfg", FFN_CASES, ids=lambda c: c.name)
def test_grouped_ffn_matches_oracle(cfg):
    inp, lg, idx, w, counts, offsets, sp, inv = routed(cfg)
    Xp = oracle.gather_rows(to_np(inp["X"]), sp, cfg.K)
    _ffn_check(cfg, Xp, idx.ravel()[sp], counts, offsets, inp)


@pytest.mark.parametrize("counts", [[1, 127, 128, 129], [0, 0, 255, 1], [128, 0, 0, 0], [0, 0, 0, 300]])
def test_grouped_ffn_ragged_tails(counts):
    cfg = synth.MoEConfig("tails", T=sum(counts), d=128, E=4, K=1, n=256)
    idx = forced_counts_idx(counts)
    c = np.bincount(idx.ravel(), minlength=4).astype(np.int32)
    assert list(c) == counts
    off = np.concatenate([[0], np.cumsum(c)]).astype(np.int32)
    sp, inv = oracle.permute(idx, 4)
    inp = synth.make_inputs(cfg, "cpu", 2)
    Xp = oracle.gather_rows(to_np(inp["X"]), sp, 1)
    _ffn_check(cfg, Xp, idx.ravel()[sp], c, off, inp)


COMBINE_CASES = [
    synth.CONFIGS["tiny"],
    synth.MoEConfig("cmb_bf16", T=700, d=384, E=16, K=4, n=128, logits="bias", bias_var=2.0),
    synth.MoEConfig("cmb_k8", T=129, d=7168 // 4, E=32, K=8, n=128),
    synth.MoEConfig("cmb_k1", T=50, d=128, E=4, K=1, n=128),
]


@pytest.mark.parametrize("cfg", COMBINE_CASES, ids=lambda c: c.name)
def test_combine_matches_oracle(cfg):
    rng = np.random.default_rng(cfg.T)
    lg = (rng.normal(size=(cfg.T, cfg.E)) + rng.normal(0, 2, cfg.E)).astype(np.float32)
    idx, w, counts, offsets = oracle.route(lg, cfg.K)
    sp, inv = oracle.permute(idx, cfg.E)
    Y = torch.from_numpy(rng.normal(size=(cfg.T * cfg.K, cfg.d)).astype(np.float32)).to(cfg.torch_dtype)
    out = moe.moe_combine(cuda(Y), cuda(torch.from_numpy(w)), cuda(torch.from_numpy(inv)))
    torch.cuda.synchronize()
    ref = oracle.combine(Y.float().numpy(), w, inv)
    check_close(out, ref, cfg.dtype, "out")


UPDOWN_CASES = [
    synth.CONFIGS["tiny"],
    synth.MoEConfig("ud_bf16", T=512, d=256, E=8, K=2, n=384),
    synth.MoEConfig("ud_sparse", T=1000, d=512, E=64, K=4, n=256, logits="bias", bias_var=4.0),
    synth.MoEConfig("ud_narrow", T=300, d=128, E=16, K=4, n=256, logits="bias", bias_var=2.0),
]


@pytest.mark.parametrize("cfg", UPDOWN_CASES, ids=lambda c: c.name)
def test_ffn_up_and_down_separately(cfg):
    """Step 4a and 4b through their own entry points, each against the oracle."""
    inp, lg, idx, w, counts, offsets, sp, inv = routed(cfg)
    Xp = oracle.gather_rows(to_np(inp["X"]), sp, cfg.K)
    re = idx.ravel()[sp]
    c_d, o_d = cuda(torch.from_numpy(counts)), cuda(torch.from_numpy(offsets))
    Act = moe.moe_ffn_up(cuda(from_np(Xp)), cuda(inp["W1"]), cuda(inp["W3"]), c_d, o_d, cfg.K)
    torch.cuda.synchronize()
    ract, _ = oracle.expert_ffn(Xp, re, to_np(inp["W1"]), to_np(inp["W3"]), to_np(inp["W2"]))
    check_close(Act, ract, cfg.dtype, "Act")
    # down-projection fed the oracle's activation in the storage dtype
    act_in = torch.from_numpy(ract).to(cfg.torch_dtype)
    Y = moe.moe_ffn_down(cuda(act_in), cuda(inp["W2"]), c_d, o_d, cfg.K)
    torch.cuda.synchronize()
    ry = oracle.expert_down(to_np(act_in), re, to_np(inp["W2"]))
    check_close(Y, ry, cfg.dtype, "Y")


SPLIT_CASES = [
    # few tiles: the whole grid is one partial round, split along K into several parts
    synth.MoEConfig("split_small", T=512, d=512, E=4, K=2, n=1024),
    # ragged experts, some empty, rows not multiples of the tile height
    synth.MoEConfig("split_ragged", T=900, d=256, E=32, K=4, n=512, logits="bias", bias_var=4.0),
]


@pytest.mark.parametrize("cfg", SPLIT_CASES, ids=lambda c: c.name)
def test_ffn_split_tail_matches_unsplit_and_oracle(cfg):
    """The K-split of the last partial round (with the workspace) and the plain
    schedule (without) both match the oracle, and agree with each other to
    fp32 rounding; the split result is the same on a second call."""
    inp, lg, idx, w, counts, offsets, sp, inv = routed(cfg)
    Xp = oracle.gather_rows(to_np(inp["X"]), sp, cfg.K)
    re = idx.ravel()[sp]
    c_d, o_d = cuda(torch.from_numpy(counts)), cuda(torch.from_numpy(offsets))
    xp_d = cuda(from_np(Xp))
    w1, w3, w2 = cuda(inp["W1"]), cuda(inp["W3"]), cuda(inp["W2"])
    act_s, y_s = moe.moe_grouped_ffn(xp_d, w1, w3, w2, c_d, o_d, cfg.K, split=True)
    act_s2, y_s2 = moe.moe_grouped_ffn(xp_d, w1, w3, w2, c_d, o_d, cfg.K, split=True)
    act_u, y_u = moe.moe_grouped_ffn(xp_d, w1, w3, w2, c_d, o_d, cfg.K, split=False)
    torch.cuda.synchronize()
    ract, ry = oracle.expert_ffn(Xp, re, to_np(inp["W1"]), to_np(inp["W3"]), to_np(inp["W2"]))
    check_close(act_s, ract, cfg.dtype, "Act (split)")
    check_close(act_u, ract, cfg.dtype, "Act (unsplit)")
    check_close(y_u, ry, cfg.dtype, "Y (unsplit)")
    # Y of the split run is computed from its own Act
    ry_s = oracle.expert_down(to_np(act_s), re, to_np(inp["W2"]))
    check_close(y_s, ry_s, cfg.dtype, "Y (split)")
    assert torch.equal(act_s.view(torch.int16), act_s2.view(torch.int16)), "split Act not deterministic"
    assert torch.equal(y_s.view(torch.int16), y_s2.view(torch.int16)), "split Y not deterministic"
    # split and unsplit differ only by fp32 summation order before one bf16 rounding
    da = (act_s.float() - act_u.float()).abs().max().item()
    assert da <= 2e-2 * act_u.float().abs().max().item(), da


# Expert row counts that give every tile height of the pipelined bf16 kernel
# (d % 256 == 0, n % 128 == 0): remainder tiles of 1..32, 33..64 and 65..128
# rows, full-height tiles, several tiles per expert, and an empty expert.
SHORT_TILE_COUNTS = [1, 31, 32, 33, 64, 65, 100, 128, 129, 200, 256, 257, 300, 0, 520]


@pytest.mark.parametrize("split", [False, True], ids=["whole", "split"])
def test_grouped_ffn_short_tiles(split):
    counts = SHORT_TILE_COUNTS
    E = len(counts)
    cfg = synth.MoEConfig("short_tiles", T=sum(counts), d=256, E=E, K=1, n=256)
    idx = forced_counts_idx(counts)
    c = np.bincount(idx.ravel(), minlength=E).astype(np.int32)
    assert list(c) == counts
    off = np.concatenate([[0], np.cumsum(c)]).astype(np.int32)
    sp, inv = oracle.permute(idx, E)
    inp = synth.make_inputs(cfg, "cpu", 3)
    Xp = oracle.gather_rows(to_np(inp["X"]), sp, 1)
    re = idx.ravel()[sp]
    Act, Y = moe.moe_grouped_ffn(cuda(from_np(Xp)), cuda(inp["W1"]), cuda(inp["W3"]), cuda(inp["W2"]),
                                 cuda(torch.from_numpy(c)), cuda(torch.from_numpy(off)), 1, split=split)
    torch.cuda.synchronize()
    ract, ry = oracle.expert_ffn(Xp, re, to_np(inp["W1"]), to_np(inp["W3"]), to_np(inp["W2"]))
    check_close(Act, ract, cfg.dtype, "Act")
    check_close(Y, ry, cfg.dtype, "Y")
    # row by row (relative L2 of each row), so that a wrong row or column slice
    # of a short tile cannot hide in the whole-tensor norms
    for name, o, r in (("Act", as_f64(Act), as_f64(ract)), ("Y", as_f64(Y), as_f64(ry))):
        rel = np.linalg.norm(o - r, axis=1) / np.linalg.norm(r, axis=1)
        bad = np.flatnonzero(rel > 1e-2)
        assert bad.size == 0, (name, [(int(np.searchsorted(off, b, "right") - 1), int(b)) for b in bad[:8]],
                               rel[bad[:8]])
