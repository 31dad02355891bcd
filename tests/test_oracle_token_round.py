"""Pins for the oracle's Token Rounding (the routing variant of page "MoE
architecture optimisation and SonicMoE practice", sections 3.1 and 3.2):
hand-worked examples, the rounding rule's defining properties, a brute-force
check that every expert keeps the best-ranked candidates, the reduction to
plain top-K at M = 1, and closed forms for the combine and the layer.  CPU only."""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "token_round_worked_examples.json")


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _kept_sets(slot_row):
    return [sorted(np.nonzero(r >= 0)[0].tolist()) for r in slot_row]


def _check_layout(plan, T, E, M, cap_tiles):
    """Rows expert by expert, tokens ascending inside an expert, slot_row the inverse of row_tok."""
    cr, off, rt, sr = plan["counts_r"], plan["offsets_r"], plan["row_tok"], plan["slot_row"]
    assert off[0] == 0 and np.array_equal(np.diff(off), cr) and rt.size == off[E]
    for e in range(E):
        assert cr[e] % M == 0 and cr[e] <= T
        if cap_tiles:
            assert cr[e] <= cap_tiles * M
        seg = rt[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.array_equal(sr[seg, e], np.arange(off[e], off[e + 1]))
    assert int((sr >= 0).sum()) == rt.size


def test_worked_examples():
    g = json.load(open(GOLDEN))
    for ex in g["examples"]:
        lg = np.array(ex["logits"], np.float32)
        T, E = lg.shape
        plan = oracle.token_round(lg, ex["K"], ex["M"], ex["cap_tiles"])
        assert plan["counts_r"].tolist() == ex["counts_r"], ex["name"]
        assert plan["offsets_r"].tolist() == ex["offsets_r"], ex["name"]
        assert plan["row_tok"].tolist() == ex["row_tok"], ex["name"]
        assert _kept_sets(plan["slot_row"]) == ex["kept"], ex["name"]
        _check_layout(plan, T, E, ex["M"], ex["cap_tiles"])
        for t in range(T):
            kept = ex["kept"][t]
            w = plan["slot_w"][t]
            if str(t) in ex["weights_closed_form"]:
                want = [eval(f, {"exp": math.exp}) for f in ex["weights_closed_form"][str(t)]]
                np.testing.assert_allclose(w[kept], want, rtol=1e-6)
            elif len(kept) == 1:
                assert w[kept[0]] == 1.0
            assert np.all(w[[e for e in range(E) if e not in kept]] == 0.0)


def test_target_rule_cases_and_properties():
    g = json.load(open(GOLDEN))
    for f, M, T, cap, want in g["targets"]["cases"]:
        assert oracle.tr_target(f, M, T, cap) == want, (f, M, T, cap)
    rng = np.random.default_rng(3)
    for _ in range(2000):
        M = int(rng.integers(1, 300))
        T = int(rng.integers(1, 5000))
        f = int(rng.integers(0, T + 1))
        r = oracle.tr_target(f, M, T, 0)
        assert r % M == 0 and 0 <= r <= T
        # no multiple of M within [0, T] is nearer to f; a half goes up
        for q in (r - M, r + M):
            if 0 <= q <= T:
                assert abs(q - f) > abs(r - f) or (abs(q - f) == abs(r - f) and q < r)
        cap = int(rng.integers(1, 4))
        assert oracle.tr_target(f, M, T, cap) == min(r, cap * M)


@pytest.mark.parametrize("T,E,K,M,cap,levels,seed", [
    (40, 4, 1, 8, 0, 5, 1),       # coarse logits: many ties
    (97, 6, 2, 16, 0, 0, 2),
    (128, 8, 2, 32, 0, 7, 3),
    (200, 16, 4, 8, 0, 0, 4),
    (64, 8, 3, 8, 1, 4, 5),       # limit of one tile
    (33, 5, 5, 4, 0, 3, 6),       # K = E: every token picks every expert
])
def test_every_expert_keeps_its_best_candidates(T, E, K, M, cap, levels, seed):
    """Brute force: for each expert, every kept candidate ranks ahead of every
    candidate it did not keep, by (logit descending, token ascending)."""
    rng = np.random.default_rng(seed)
    if levels:
        lg = rng.integers(0, levels, size=(T, E)).astype(np.float32) * np.float32(0.5)
    else:
        lg = rng.standard_normal((T, E)).astype(np.float32)
    idx, _, counts, _ = oracle.route(lg, K)
    plan = oracle.token_round(lg, K, M, cap)
    _check_layout(plan, T, E, M, cap)
    routed = np.zeros((T, E), bool)
    routed[np.repeat(np.arange(T), K), idx.reshape(-1)] = True
    kept = plan["slot_row"] >= 0
    for e in range(E):
        f = int(routed[:, e].sum())
        assert f == counts[e]
        r = oracle.tr_target(f, M, T, cap)
        assert kept[:, e].sum() == r
        if r <= f:
            assert not np.any(kept[:, e] & ~routed[:, e])
            cand = np.nonzero(routed[:, e])[0]
        else:
            assert np.all(kept[routed[:, e], e])
            cand = np.nonzero(~routed[:, e])[0]
        rank = lambda t: (-float(lg[t, e]), int(t))
        ins = [rank(t) for t in cand if kept[t, e]]
        outs = [rank(t) for t in cand if not kept[t, e]]
        if ins and outs:
            assert max(ins) < min(outs)


def test_weights_are_softmax_over_kept():
    rng = np.random.default_rng(11)
    T, E, K, M = 150, 8, 2, 16
    lg = (3.0 * rng.standard_normal((T, E))).astype(np.float32)
    plan = oracle.token_round(lg, K, M)
    kept = plan["slot_row"] >= 0
    w = plan["slot_w"].astype(np.float64)
    for t in range(T):
        ks = np.nonzero(kept[t])[0]
        if ks.size == 0:
            assert np.all(w[t] == 0)
            continue
        np.testing.assert_allclose(w[t].sum(), 1.0, rtol=1e-6)
        # ratios follow the logit differences: w_a / w_b = exp(l_a - l_b)
        a, b = ks[0], ks[-1]
        np.testing.assert_allclose(w[t, a] / w[t, b], math.exp(float(lg[t, a]) - float(lg[t, b])), rtol=1e-5)


def test_m1_is_plain_top_k():
    rng = np.random.default_rng(12)
    T, E, K = 120, 8, 2
    lg = rng.standard_normal((T, E)).astype(np.float32)
    idx, w, counts, _ = oracle.route(lg, K)
    plan = oracle.token_round(lg, K, 1)
    assert np.array_equal(plan["counts_r"], counts)
    for t in range(T):
        assert _kept_sets(plan["slot_row"][t:t + 1])[0] == sorted(idx[t].tolist())
        np.testing.assert_allclose(plan["slot_w"][t, idx[t]], w[t], rtol=1e-6)
    # the combine then equals the plain combine, up to the summation order
    sp, inv = oracle.permute(idx, E)
    d = 16
    Y = rng.standard_normal((T * K, d)).astype(np.float32)
    # rows of the two layouts hold the same (token, expert) pairs in the same order
    assert np.array_equal(plan["row_tok"], sp // K)
    np.testing.assert_allclose(oracle.tr_combine(Y, plan["slot_row"], plan["slot_w"]),
                               oracle.combine(Y, w, inv), rtol=1e-6, atol=1e-6)


def test_combine_special_cases():
    rng = np.random.default_rng(13)
    T, E, K, M = 90, 6, 2, 8
    lg = rng.standard_normal((T, E)).astype(np.float32)
    plan = oracle.token_round(lg, K, M)
    rows = plan["row_tok"].size
    # rows holding one-hot of their expert: the output is the weight row itself
    row_e = np.repeat(np.arange(E), plan["counts_r"])
    Y = np.zeros((rows, E), np.float32)
    Y[np.arange(rows), row_e] = 1.0
    np.testing.assert_array_equal(oracle.tr_combine(Y, plan["slot_row"], plan["slot_w"]), plan["slot_w"])
    # rows holding their token index: out[t] = t * (sum of weights) = t, or 0 for a token with nothing
    Y = np.repeat(plan["row_tok"].astype(np.float32)[:, None], 3, axis=1)
    out = oracle.tr_combine(Y, plan["slot_row"], plan["slot_w"])
    has = (plan["slot_row"] >= 0).any(axis=1)
    np.testing.assert_allclose(out[has], np.repeat(np.arange(T)[has, None], 3, 1).astype(np.float64), rtol=1e-6)
    assert np.all(out[~has] == 0)


def test_layer_with_identical_experts_is_the_dense_mlp():
    """Every expert the same MLP and weights summing to 1: each token's output is
    that MLP on its row (library matmuls), or zero for a token that kept nothing."""
    rng = np.random.default_rng(14)
    T, d, E, K, n, M = 48, 16, 4, 1, 24, 8
    X = rng.standard_normal((T, d)).astype(np.float32)
    w1 = (rng.standard_normal((d, n)) / 4).astype(np.float32)
    w3 = (rng.standard_normal((d, n)) / 4).astype(np.float32)
    w2 = (rng.standard_normal((n, d)) / 5).astype(np.float32)
    W1, W3, W2 = (np.repeat(a[None], E, 0) for a in (w1, w3, w2))
    lg = rng.standard_normal((T, E)).astype(np.float32)
    plan = oracle.token_round(lg, K, M, cap_tiles=1)
    out = oracle.tr_layer(X, plan["slot_row"], plan["slot_w"], W1, W3, W2)
    Xd = X.astype(np.float64)
    h1 = Xd @ w1.astype(np.float64)
    act = (_silu(h1) * (Xd @ w3.astype(np.float64))).astype(np.float32).astype(np.float64)
    dense = act @ w2.astype(np.float64)
    has = (plan["slot_row"] >= 0).any(axis=1)
    assert has.any() and (~has).any()
    np.testing.assert_allclose(out[has], dense[has], rtol=2e-5, atol=2e-6)
    assert np.all(out[~has] == 0)
