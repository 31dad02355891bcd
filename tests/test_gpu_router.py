"""GPU parity of moe_router (the router projection upstream of the gate)
against the oracle, and of the routing that follows it."""
import numpy as np
import pytest
import torch

import mixture_experts_routing_gate_amd as moe
import oracle
import synth
from parity_util import check_equal, cuda, to_np

pytestmark = pytest.mark.gpu


def _check_logits(lg_gpu, X_h, Wr_h, b_h, rows=None):
    """|logit - oracle| <= 2^-16 * sum_i |X[t,i] Wr[i,e]| (+ a tiny floor), element by element."""
    Xf = oracle.bf16_to_f32(X_h) if X_h.dtype == np.uint16 else X_h
    if rows is not None:
        X_h, Xf = X_h[rows], Xf[rows]
    ref = oracle.router(X_h, Wr_h, b_h).astype(np.float64)
    S = np.abs(Xf.astype(np.float64)) @ np.abs(Wr_h.astype(np.float64))
    got = lg_gpu.cpu().numpy().astype(np.float64)
    if rows is not None:
        got = got[rows]
    err = np.abs(got - ref)
    bound = 2.0 ** -16 * S + 2.0 ** -40
    bad = np.argwhere(err > bound)
    assert bad.size == 0, (f"{len(bad)} logits out of bound, first {bad[:3].tolist()}: "
                           f"err {err[tuple(bad[0])]:.3e} bound {bound[tuple(bad[0])]:.3e}")
    return float((err / np.maximum(S, 1e-30)).max())


CASES = [
    # (T, d, E, dtype, bias variance): E padded to 32 or 64, ragged token tiles,
    # d not a multiple of 256 (the FMA path), fp32 X, a single token
    (300, 512, 8, "bf16", 0.0),
    (257, 768, 256, "bf16", 1.5),
    (100, 1536, 128, "bf16", 2.0),
    (65, 256, 40, "bf16", 1.0),
    (33, 384, 8, "bf16", 0.0),
    (256, 128, 8, "f32", 0.0),
    (1, 1024, 64, "bf16", 0.5),
    # E a multiple of 128 and d >= 4096: the grouped GEMM's kernel with every
    # tile split along K (4 parts; 3 parts of uneven length), ragged tokens
    (8000, 4096, 256, "bf16", 1.5),
    (16385, 4096, 128, "bf16", 0.0),
    # two token tiles, one short (so tiles are claimed), each split in 32 parts
    (300, 4096, 128, "bf16", 0.5),
    # the same E with a shorter d, and too many token tiles for that path: the
    # LDS-staged tile kernel
    (16385, 256, 128, "bf16", 0.0),
    (33000, 256, 128, "bf16", 1.0),
    # tile kernel: a second expert group half made of zero rows; E not a
    # multiple of 4 (element stores) with a ragged last token tile; one token
    (1000, 512, 96, "bf16", 1.0),
    (130, 1024, 65, "bf16", 0.5),
    (1, 256, 200, "bf16", 0.0),
    # E <= 32, staged through LDS in pieces of 8 weight rows: E not a multiple
    # of 8 (rows past E read as zeros), each piece count, ragged token tiles
    (77, 512, 12, "bf16", 0.5),
    (300, 1024, 20, "bf16", 1.0),
    (1025, 256, 27, "bf16", 0.0),
    (64, 4096, 32, "bf16", 0.0),
    (33, 768, 5, "bf16", 2.0),
]


@pytest.mark.parametrize("T,d,E,dt,bv", CASES, ids=lambda v: str(v))
def test_router_matches_oracle(T, d, E, dt, bv):
    cfg = synth.MoEConfig("r", T=T, d=d, E=E, K=1, n=128, dtype=dt, logits="proj_bias" if bv else "proj",
                          bias_var=bv)
    X = synth._normal((T, d), 1.0, cfg.torch_dtype, torch.device("cpu"), synth._gen("cpu", 3, "X"))
    Wr, b = synth.make_router(cfg, "cpu", 3)
    lg = moe.moe_router(cuda(X), cuda(Wr), None if b is None else cuda(b))
    torch.cuda.synchronize()
    _check_logits(lg, to_np(X), Wr.numpy(), None if b is None else b.numpy())
    # the same call twice gives the same bits
    lg2 = moe.moe_router(cuda(X), cuda(Wr), None if b is None else cuda(b))
    torch.cuda.synchronize()
    assert torch.equal(lg, lg2)


@pytest.mark.parametrize("name", ["mixtral", "dsv3", "fine"])
def test_router_full_size_then_route(name):
    """Full-size router (every row on the fine-grained shape, sampled rows on the
    other two), then the gate on the GPU logits matches the oracle's gate on
    those same logits bit for bit."""
    cfg = synth.CONFIGS[name]
    X = synth._normal((cfg.T, cfg.d), 1.0, cfg.torch_dtype, torch.device("cuda"), synth._gen("cuda", 0, "X"))
    Wr, b = synth.make_router(cfg, "cuda", 0)
    lg = moe.moe_router(X, Wr, b)
    torch.cuda.synchronize()
    rows = (None if name == "fine" else
            np.unique(np.r_[np.random.default_rng(1).choice(cfg.T, 48, replace=False), 0, cfg.T - 1]))
    _check_logits(lg, to_np(X), Wr.cpu().numpy(), None if b is None else b.cpu().numpy(), rows=rows)
    idx, w, counts, offsets = moe.moe_route(lg, cfg.K)
    torch.cuda.synchronize()
    ridx, rw, rc, ro = oracle.route(lg.cpu().numpy(), cfg.K)
    check_equal(idx, ridx, "topk_idx")
    check_equal(counts, rc, "counts")
