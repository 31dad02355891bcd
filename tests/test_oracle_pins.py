"""Pins for the CPU oracle: each check compares the oracle with something other
than itself -- a hand-derived worked example, closed forms, invariants, an
independent brute force, or a library routine -- so that a plausible mistake
in the oracle (a dropped term, a wrong sign or index, a transposed operand)
fails at least one of them.  CPU only."""
import collections
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _dense_swiglu(X, W1, W3, W2):
    """Dense SwiGLU MLP from library matmuls in fp64: (SiLU(X W1) * (X W3)) W2."""
    X = X.astype(np.float64)
    return (_silu(X @ W1.astype(np.float64)) * (X @ W3.astype(np.float64))) @ W2.astype(np.float64)


def _rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# ----------------------------------------------------------------- worked example

def test_worked_example_route_and_permute(oracle_lib):
    g = json.load(open(os.path.join(GOLDEN, "route_worked_example.json")))
    lg = np.array(g["logits"], np.float32)
    assert math.copysign(1.0, float(lg[3, 0])) < 0  # the -0.0 survived the fixture
    idx, w, counts, offsets = oracle.route(lg, g["K"])
    np.testing.assert_array_equal(idx, np.array(g["topk_idx"], np.int32))
    np.testing.assert_allclose(w, np.array(g["topk_w"]), rtol=0, atol=g["weight_tolerance"])
    np.testing.assert_array_equal(counts, g["counts"])
    np.testing.assert_array_equal(offsets, g["offsets"])
    sp, inv = oracle.permute(idx, g["E"])
    np.testing.assert_array_equal(sp, g["sorted_pair"])
    np.testing.assert_array_equal(inv, g["inv"])


# ------------------------------------------------------------------------ softmax

@pytest.mark.parametrize("E", [1, 2, 7, 8, 128, 256])
def test_softmax_rows_sum_to_one(oracle_lib, E):
    lg = _rng(E).normal(0, 3, size=(64, E)).astype(np.float32)
    p = oracle.softmax(lg)
    assert np.all(p > 0)
    assert np.max(np.abs(p.sum(1) - 1.0)) <= E * 2.0 ** -52 * 4


def test_softmax_two_experts_is_logistic(oracle_lib):
    lg = _rng(1).normal(0, 4, size=(200, 2)).astype(np.float32)
    p = oracle.softmax(lg)
    l0 = lg[:, 0].astype(np.float64)
    l1 = lg[:, 1].astype(np.float64)
    logistic = np.array([1.0 / (1.0 + math.exp(b - a)) for a, b in zip(l0, l1)])
    np.testing.assert_allclose(p[:, 0], logistic, rtol=1e-14, atol=0)


def test_softmax_equal_row_and_shift_invariance(oracle_lib):
    for E in (1, 3, 8, 100):
        p = oracle.softmax(np.full((3, E), 0.75, np.float32))
        np.testing.assert_allclose(p, 1.0 / E, rtol=1e-15)
    lg = _rng(2).normal(size=(32, 16)).astype(np.float32)
    p0 = oracle.softmax(lg)
    p1 = oracle.softmax(lg + np.float32(64.0))   # exact shift: small ints added to values in [-5, 5]
    np.testing.assert_allclose(p0, p1, rtol=1e-5)  # inputs change by fp32 rounding of the shift only
    # monotone: probabilities order exactly as logits do
    for r in range(lg.shape[0]):
        order_l = np.argsort(-lg[r].astype(np.float64), kind="stable")
        order_p = np.argsort(-p0[r], kind="stable")
        np.testing.assert_array_equal(order_l, order_p)


def test_softmax_rejects_non_finite(oracle_lib):
    lg = np.zeros((2, 4), np.float32)
    lg[1, 2] = np.inf
    with pytest.raises(ValueError):
        oracle.softmax(lg)


# ------------------------------------------------------------------------- top-K

def _brute_topk(row, K):
    # independent full sort: key (-logit, expert); Python compares -0.0 == 0.0
    return sorted(range(len(row)), key=lambda e: (-float(row[e]), e))[:K]


@pytest.mark.parametrize("E", [1, 2, 3, 5, 8, 16])
def test_topk_matches_full_sort_with_ties(oracle_lib, E):
    rng = _rng(10 + E)
    T = 64
    # small integer-valued logits make ties common; sprinkle signed zeros
    lg = rng.integers(-3, 4, size=(T, E)).astype(np.float32)
    zeros = rng.random((T, E)) < 0.2
    lg[zeros] = np.where(rng.random(zeros.sum()) < 0.5, -0.0, 0.0)
    for K in range(1, E + 1):
        idx, _, _, _ = oracle.route(lg, K)
        for t in range(T):
            assert list(idx[t]) == _brute_topk(lg[t], K), (t, K, lg[t])


def test_topk_k_equals_e_is_full_order(oracle_lib):
    lg = _rng(3).normal(size=(40, 8)).astype(np.float32)
    idx, w, counts, _ = oracle.route(lg, 8)
    for t in range(40):
        assert list(idx[t]) == list(np.argsort(-lg[t].astype(np.float64), kind="stable"))
    np.testing.assert_array_equal(counts, np.full(8, 40))
    # with every expert selected the weights are the plain softmax
    np.testing.assert_allclose(w, np.take_along_axis(oracle.softmax(lg), idx.astype(np.int64), 1), rtol=1e-6)


# ----------------------------------------------------------------------- weights

def test_weights_sum_to_one_and_ratio(oracle_lib):
    lg = _rng(4).normal(0, 2, size=(300, 32)).astype(np.float32)
    idx, w, _, _ = oracle.route(lg, 6)
    assert np.max(np.abs(w.astype(np.float64).sum(1) - 1.0)) <= 1e-6
    # w_a / w_b = exp(l_a - l_b): the softmax denominator and the renormaliser cancel
    la = np.take_along_axis(lg, idx.astype(np.int64), 1).astype(np.float64)
    ratio = w[:, 1:].astype(np.float64) / w[:, :1]
    np.testing.assert_allclose(ratio, np.exp(la[:, 1:] - la[:, :1]), rtol=1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)  # slots are in descending weight


def test_weights_k1_is_one_and_two_expert_closed_form(oracle_lib):
    lg = _rng(5).normal(size=(100, 8)).astype(np.float32)
    _, w, _, _ = oracle.route(lg, 1)
    assert np.all(w == 1.0)
    lg2 = _rng(6).normal(0, 3, size=(100, 2)).astype(np.float32)
    idx, w, _, _ = oracle.route(lg2, 2)
    hi = np.maximum(lg2[:, 0], lg2[:, 1]).astype(np.float64)
    lo = np.minimum(lg2[:, 0], lg2[:, 1]).astype(np.float64)
    np.testing.assert_allclose(w[:, 0], 1.0 / (1.0 + np.exp(lo - hi)), rtol=2e-7)
    np.testing.assert_allclose(w[:, 1], 1.0 / (1.0 + np.exp(hi - lo)), rtol=2e-7)


# ---------------------------------------------------------------- counts/offsets

@pytest.mark.parametrize("T,E,K", [(1, 1, 1), (257, 8, 2), (500, 128, 8), (64, 256, 8), (33, 5, 5)])
def test_counts_offsets_brute(oracle_lib, T, E, K):
    lg = (_rng(T + E).normal(size=(T, E)) + _rng(7).normal(0, 2, size=E)).astype(np.float32)
    idx, _, counts, offsets = oracle.route(lg, K)
    c = collections.Counter(idx.ravel().tolist())
    np.testing.assert_array_equal(counts, [c.get(e, 0) for e in range(E)])
    assert counts.sum() == T * K
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    # every token's K experts are distinct
    assert all(len(set(r)) == K for r in idx.tolist())


# ------------------------------------------------------------------- permutation

@pytest.mark.parametrize("T,E,K", [(1, 1, 1), (300, 8, 2), (257, 64, 4), (128, 256, 8)])
def test_permutation_properties(oracle_lib, T, E, K):
    lg = (_rng(11).normal(size=(T, E)) + _rng(12).normal(0, 1.5, size=E)).astype(np.float32)
    idx, _, counts, offsets = oracle.route(lg, K)
    sp, inv = oracle.permute(idx, E)
    A = T * K
    np.testing.assert_array_equal(inv[sp], np.arange(A))        # round trip both ways
    np.testing.assert_array_equal(sp[inv], np.arange(A))
    flat = idx.ravel()
    for e in range(E):
        seg = sp[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e)                            # segment purity
        assert np.all(np.diff(seg // K) > 0)                     # strictly ascending tokens
    # a library stable sort of the row-major (token, slot) list by expert is the same order
    np.testing.assert_array_equal(sp, np.argsort(flat, kind="stable"))


def test_gather_rows_matches_fancy_indexing(oracle_lib):
    T, E, K, d = 50, 6, 3, 24
    idx, _, _, _ = oracle.route(_rng(13).normal(size=(T, E)).astype(np.float32), K)
    sp, _ = oracle.permute(idx, E)
    X = _rng(14).normal(size=(T, d)).astype(np.float32)
    np.testing.assert_array_equal(oracle.gather_rows(X, sp, K), X[sp // K])
    Xb = _rng(15).integers(0, 65535, size=(T, d)).astype(np.uint16)
    np.testing.assert_array_equal(oracle.gather_rows(Xb, sp, K), Xb[sp // K])


# ----------------------------------------------------------------- FFN + combine

def _weights(E, d, n, seed, dtype=np.float32):
    r = _rng(seed)
    W1 = (r.normal(size=(E, d, n)) / math.sqrt(d)).astype(dtype)
    W3 = (r.normal(size=(E, d, n)) / math.sqrt(d)).astype(dtype)
    W2 = (r.normal(size=(E, n, d)) / math.sqrt(n)).astype(dtype)
    return W1, W3, W2


def test_single_expert_layer_is_dense_swiglu(oracle_lib):
    T, d, n = 40, 32, 48
    X = _rng(20).normal(size=(T, d)).astype(np.float32)
    W1, W3, W2 = _weights(1, d, n, 21)
    lg = _rng(22).normal(size=(T, 1)).astype(np.float32)
    out = oracle.layer(X, lg, W1, W3, W2, K=1)
    ref = _dense_swiglu(X, W1[0], W3[0], W2[0])
    assert _rel_l2(out, ref) < 1e-6
    # a transposed-W1 or SiLU-on-the-wrong-branch oracle would fail this:
    wrong = _dense_swiglu(X, W3[0], W1[0], W2[0])
    assert _rel_l2(wrong, ref) > 1e-2


def test_identical_experts_reduce_to_dense_mlp(oracle_lib):
    """With every expert equal, sum_k w_k = 1 makes the layer the dense MLP for any routing."""
    T, d, n, E, K = 64, 16, 32, 8, 3
    X = _rng(30).normal(size=(T, d)).astype(np.float32)
    W1, W3, W2 = _weights(1, d, n, 31)
    W1, W3, W2 = (np.repeat(W, E, 0) for W in (W1, W3, W2))
    lg = _rng(32).normal(0, 2, size=(T, E)).astype(np.float32)
    out = oracle.layer(X, lg, W1, W3, W2, K=K)
    assert _rel_l2(out, _dense_swiglu(X, W1[0], W3[0], W2[0])) < 2e-6
    # and via the permuted step-by-step route
    idx, w, counts, offsets = oracle.route(lg, K)
    sp, inv = oracle.permute(idx, E)
    Xp = oracle.gather_rows(X, sp, K)
    act, Y = oracle.expert_ffn(Xp, idx.ravel()[sp], W1, W3, W2)
    assert _rel_l2(oracle.combine(Y, w, inv), _dense_swiglu(X, W1[0], W3[0], W2[0])) < 2e-6


def test_expert_ffn_rows_against_library_matmuls(oracle_lib):
    rows, d, n, E = 30, 24, 40, 5
    Xp = _rng(40).normal(size=(rows, d)).astype(np.float32)
    re = _rng(41).integers(0, E, size=rows).astype(np.int32)
    W1, W3, W2 = _weights(E, d, n, 42)
    act, y = oracle.expert_ffn(Xp, re, W1, W3, W2)
    for r in range(rows):
        e = re[r]
        x = Xp[r:r + 1].astype(np.float64)
        a_ref = _silu(x @ W1[e].astype(np.float64)) * (x @ W3[e].astype(np.float64))
        np.testing.assert_allclose(act[r], a_ref[0], rtol=1e-6, atol=1e-7)
        np.testing.assert_allclose(y[r], (act[r:r + 1].astype(np.float64) @ W2[e].astype(np.float64))[0],
                                   rtol=1e-6, atol=1e-7)
    # selecting rows returns the same values in the requested order
    sel = np.array([7, 0, 29, 7], np.int32)
    a2, y2 = oracle.expert_ffn(Xp, re, W1, W3, W2, rows=sel)
    np.testing.assert_array_equal(a2, act[sel])
    np.testing.assert_array_equal(y2, y[sel])


def test_zero_row_and_exact_scaling(oracle_lib):
    T, d, n, E, K = 20, 16, 16, 4, 2
    X = _rng(50).normal(size=(T, d)).astype(np.float32)
    X[5] = 0.0
    W1, W3, W2 = _weights(E, d, n, 51)
    lg = _rng(52).normal(size=(T, E)).astype(np.float32)
    out = oracle.layer(X, lg, W1, W3, W2, K)
    assert np.all(out[5] == 0.0)
    out2 = oracle.layer(X, lg, W1, W3, (W2 * np.float32(2)).astype(np.float32), K)
    np.testing.assert_array_equal(out2, 2 * out)


def test_combine_properties(oracle_lib):
    T, K, d = 30, 3, 12
    A = T * K
    Y = _rng(60).normal(size=(A, d)).astype(np.float32)
    inv = _rng(61).permutation(A).astype(np.int32)
    one = np.zeros((T, K), np.float32)
    one[:, 0] = 1.0
    np.testing.assert_array_equal(oracle.combine(Y, one, inv), Y[inv.reshape(T, K)[:, 0]])
    # equal rows under one token with weights summing to 1 give that row back
    Yt = np.repeat(_rng(62).normal(size=(T, d)).astype(np.float32), K, 0)
    inv_id = np.arange(A, dtype=np.int32)
    w = _rng(63).random((T, K)).astype(np.float64)
    w = (w / w.sum(1, keepdims=True)).astype(np.float32)
    np.testing.assert_allclose(oracle.combine(Yt, w, inv_id), Yt[::K], rtol=1e-6, atol=1e-7)


def test_layer_matches_permuted_steps(oracle_lib):
    """The per-token layer and the gather -> expert MLP -> combine chain agree."""
    T, d, n, E, K = 90, 16, 24, 12, 4
    X = _rng(70).normal(size=(T, d)).astype(np.float32)
    W1, W3, W2 = _weights(E, d, n, 71)
    lg = (_rng(72).normal(size=(T, E)) + _rng(73).normal(0, 2, E)).astype(np.float32)
    out = oracle.layer(X, lg, W1, W3, W2, K)
    idx, w, counts, offsets = oracle.route(lg, K)
    sp, inv = oracle.permute(idx, E)
    _, Y = oracle.expert_ffn(oracle.gather_rows(X, sp, K), idx.ravel()[sp], W1, W3, W2)
    np.testing.assert_allclose(oracle.combine(Y, w, inv), out, rtol=1e-6, atol=1e-7)
    sub = np.array([89, 3, 3, 0], np.int32)
    np.testing.assert_array_equal(oracle.layer(X, lg, W1, W3, W2, K, tokens=sub), out[sub])


def test_bf16_storage_widens_exactly(oracle_lib):
    """bf16 inputs give the same result as their exact fp32 widening (widened here by torch)."""
    cfg = synth.MoEConfig("t", T=24, d=16, E=4, K=2, n=32, dtype="bf16")
    inp = synth.make_inputs(cfg, "cpu", seed=3)
    Xb, W1b, W3b, W2b = (synth.to_numpy(inp[k]) for k in ("X", "W1", "W3", "W2"))
    Xf, W1f, W3f, W2f = (inp[k].float().numpy() for k in ("X", "W1", "W3", "W2"))
    lg = synth.to_numpy(inp["logits"])
    ob = oracle.layer(Xb, lg, W1b, W3b, W2b, cfg.K)
    of = oracle.layer(Xf, lg, W1f, W3f, W2f, cfg.K)
    np.testing.assert_array_equal(ob, of)
    np.testing.assert_array_equal(oracle.bf16_to_f32(Xb), Xf)


def test_synth_is_deterministic_and_shaped():
    cfg = synth.CONFIGS["tiny"]
    a = synth.make_inputs(cfg, "cpu", 0)
    b = synth.make_inputs(cfg, "cpu", 0)
    for k in a:
        assert torch.equal(a[k], b[k])
    assert a["X"].shape == (256, 128) and a["W1"].shape == (8, 128, 256) and a["W2"].shape == (8, 256, 128)
    assert abs(float(a["W1"].std()) - 1 / math.sqrt(128)) < 0.01
    assert abs(float(a["W2"].std()) - 1 / math.sqrt(256)) < 0.01
    c = synth.make_inputs(cfg, "cpu", 1)
    assert not torch.equal(a["X"], c["X"])


def test_expert_down_matches_expert_ffn_and_matmul(oracle_lib):
    """The down-projection alone reproduces expert_ffn's y from its act, and a library matmul."""
    rows, d, n, E = 25, 16, 40, 3
    Xp = _rng(80).normal(size=(rows, d)).astype(np.float32)
    re = _rng(81).integers(0, E, size=rows).astype(np.int32)
    W1, W3, W2 = _weights(E, d, n, 82)
    act, y = oracle.expert_ffn(Xp, re, W1, W3, W2)
    np.testing.assert_array_equal(oracle.expert_down(act, re, W2), y)
    for r in range(rows):
        np.testing.assert_allclose(oracle.expert_down(act[r:r + 1], re[r:r + 1], W2)[0],
                                   act[r].astype(np.float64) @ W2[re[r]].astype(np.float64), rtol=1e-6, atol=1e-7)
    # bf16 storage widens exactly
    ab = _rng(83).integers(0x3000, 0x4000, size=(rows, n)).astype(np.uint16)
    W2b = _rng(84).integers(0x3000, 0x3c00, size=(E, n, d)).astype(np.uint16)
    np.testing.assert_array_equal(oracle.expert_down(ab, re, W2b),
                                  oracle.expert_down(oracle.bf16_to_f32(ab), re, oracle.bf16_to_f32(W2b)))


# ---- router projection (logits = X @ Wr + bias) ----

def test_router_matches_library_matmul(oracle_lib):
    """fp64 library matmul (a different summation order) agrees to fp32 rounding."""
    rng = np.random.default_rng(7)
    X = rng.normal(size=(37, 96)).astype(np.float32)
    W = (rng.normal(size=(96, 12)) / np.sqrt(96)).astype(np.float32)
    b = rng.normal(size=12).astype(np.float32)
    got = oracle.router(X, W, b).astype(np.float64)
    ref = X.astype(np.float64) @ W.astype(np.float64) + b.astype(np.float64)
    assert np.all(np.abs(got - ref) <= 2.0 ** -23 * np.abs(ref) + 1e-30)
    got0 = oracle.router(X, W).astype(np.float64)
    ref0 = X.astype(np.float64) @ W.astype(np.float64)
    assert np.all(np.abs(got0 - ref0) <= 2.0 ** -23 * np.abs(ref0) + 1e-30)


def test_router_one_hot_rows_and_columns(oracle_lib):
    """A unit row of X picks a row of Wr exactly (plus the bias); a unit column of
    Wr copies a column of X exactly.  A transposed Wr index or a dropped bias fails."""
    rng = np.random.default_rng(8)
    d, E = 24, 5
    W = rng.normal(size=(d, E)).astype(np.float32)
    b = np.array([0.5, -1.0, 2.0, 0.0, 3.25], np.float32)
    X = np.zeros((d, d), np.float32)
    X[np.arange(d), np.arange(d)] = 1.0
    lg = oracle.router(X, W, b)
    assert np.array_equal(lg, (W.astype(np.float64) + b).astype(np.float32))
    Xr = rng.normal(size=(9, d)).astype(np.float32)
    Wc = np.zeros((d, E), np.float32)
    for e in range(E):
        Wc[(3 * e + 1) % d, e] = 1.0
    lg2 = oracle.router(Xr, Wc)
    for e in range(E):
        assert np.array_equal(lg2[:, e], Xr[:, (3 * e + 1) % d])


def test_router_bf16_input_widens_exactly(oracle_lib):
    rng = np.random.default_rng(9)
    Xf = rng.normal(size=(11, 64)).astype(np.float32)
    Xb = synth.to_numpy(torch.from_numpy(Xf).to(torch.bfloat16))
    W = rng.normal(size=(64, 8)).astype(np.float32)
    assert np.array_equal(oracle.router(Xb, W), oracle.router(oracle.bf16_to_f32(Xb), W))
