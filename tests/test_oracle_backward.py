"""Pins for the oracle's layer backward (the gradient of oracle.layer: page
"MoE architecture optimisation and SonicMoE practice", section 2.2 names the
dH and dS products of the backward, section 5 measures it).  CPU only.

- Central finite differences of the oracle's own forward layer, for every
  element of X, the router logits and the three expert weight tensors.
- The section 2.2 identity dS = <dA, A>: the routing-weight gradient equals
  <dout W2^T, act> built from the forward oracle's act and a library matmul.
- Softmax shift invariance (each token's logit gradient sums to zero), zeros
  for experts a token did not choose, K = 1 (weights fixed at 1), identical
  experts (routing cannot matter), exact linearity in dout, and exact bf16
  widening.
- The variants for large layers (some tokens; slices of the weight gradients)
  equal the full backward exactly on small inputs."""
import numpy as np
import pytest

import oracle


def _case(seed, T=5, d=8, E=4, K=2, n=16, identical=False):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, d)).astype(np.float32)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    W1 = (rng.standard_normal((E, d, n)) / np.sqrt(d)).astype(np.float32)
    W3 = (rng.standard_normal((E, d, n)) / np.sqrt(d)).astype(np.float32)
    W2 = (rng.standard_normal((E, n, d)) / np.sqrt(n)).astype(np.float32)
    if identical:
        W1[:], W3[:], W2[:] = W1[0], W3[0], W2[0]
    G = rng.standard_normal((T, d)).astype(np.float32)
    return X, lg, W1, W3, W2, G


def _loss(args, K, G):
    X, lg, W1, W3, W2 = args
    return float(np.sum(oracle.layer(X, lg, W1, W3, W2, K).astype(np.float64) * G.astype(np.float64)))


def _safe_logit(lg, t, e, K, h):
    """True when moving logit [t, e] by +-h cannot change the set of chosen experts."""
    row = np.sort(lg[t].astype(np.float64))[::-1]
    if K == lg.shape[1]:
        return True
    le = float(lg[t, e])
    if le >= row[K - 1]:          # chosen: must stay above the best unchosen logit
        return le - 2 * h > row[K]
    return le + 2 * h < row[K - 1]  # not chosen: must stay below the worst chosen one


@pytest.mark.parametrize("seed,K", [(0, 2), (1, 1), (2, 3)])
def test_gradients_match_central_differences(seed, K):
    X, lg, W1, W3, W2, G = _case(seed, K=K)
    got = oracle.layer_backward(X, lg, W1, W3, W2, K, G)
    names = ["X", "logits", "W1", "W3", "W2"]
    grads = [got["dX"], got["dlogits"], got["dW1"], got["dW3"], got["dW2"]]
    base = [X, lg, W1, W3, W2]
    for which, (name, an) in enumerate(zip(names, grads)):
        h = 1e-3 if name == "logits" else 1e-2
        fd = np.zeros(an.shape, np.float64)
        checked = np.zeros(an.shape, bool)
        for ix in np.ndindex(an.shape):
            if name == "logits" and not _safe_logit(lg, ix[0], ix[1], K, h):
                continue
            args_p = [a.copy() for a in base]
            args_m = [a.copy() for a in base]
            args_p[which][ix] = np.float32(base[which][ix] + h)
            args_m[which][ix] = np.float32(base[which][ix] - h)
            step = float(args_p[which][ix]) - float(args_m[which][ix])
            fd[ix] = (_loss(args_p, K, G) - _loss(args_m, K, G)) / step
            checked[ix] = True
        assert checked.sum() > 0.5 * checked.size, name
        scale = max(float(np.max(np.abs(an))), 1e-3)
        err = np.max(np.abs(fd[checked] - an.astype(np.float64)[checked]))
        assert err <= 2e-3 * scale, f"{name}: max |fd - analytic| = {err:.3e}, scale {scale:.3e}"


def test_routing_weight_gradient_is_the_dS_identity():
    """dw[t,k] = <dout[t], y_k> = <dout[t] W2[e]^T, act_k> (page section 2.2)."""
    X, lg, W1, W3, W2, G = _case(3, T=7, K=2)
    K = 2
    got = oracle.layer_backward(X, lg, W1, W3, W2, K, G)
    idx, _, _, _ = oracle.route(lg, K)
    rows = np.repeat(np.arange(X.shape[0]), K)
    act, y = oracle.expert_ffn(X[rows], idx.reshape(-1).astype(np.int32), W1, W3, W2)
    e = idx.reshape(-1)
    g = G[rows].astype(np.float64)
    via_y = np.sum(g * y.astype(np.float64), axis=1)
    gA = np.einsum("rc,rjc->rj", g, W2[e].astype(np.float64))
    via_act = np.sum(gA * act.astype(np.float64), axis=1)
    dw = got["dw"].reshape(-1).astype(np.float64)
    tol = 1e-5 * max(1.0, float(np.max(np.abs(dw))))
    assert np.max(np.abs(dw - via_y)) <= tol
    assert np.max(np.abs(dw - via_act)) <= tol


def test_logit_gradient_structure():
    X, lg, W1, W3, W2, G = _case(4, T=9, E=6, K=3)
    K = 3
    got = oracle.layer_backward(X, lg, W1, W3, W2, K, G)
    dl = got["dlogits"].astype(np.float64)
    idx, w, _, _ = oracle.route(lg, K)
    chosen = np.zeros(dl.shape, bool)
    chosen[np.repeat(np.arange(lg.shape[0]), K), idx.reshape(-1)] = True
    assert np.all(dl[~chosen] == 0.0)
    # softmax over the chosen logits is shift invariant: each row sums to zero
    assert np.max(np.abs(dl.sum(axis=1))) <= 1e-6 * max(1.0, float(np.max(np.abs(dl))))
    # closed form from the routing-weight gradient
    dw = got["dw"].astype(np.float64)
    wd = w.astype(np.float64)
    want = wd * (dw - np.sum(wd * dw, axis=1, keepdims=True))
    np.testing.assert_allclose(dl[np.repeat(np.arange(lg.shape[0]), K), idx.reshape(-1)], want.reshape(-1),
                               rtol=1e-5, atol=1e-7)


def test_k1_and_identical_experts_give_zero_logit_gradient():
    X, lg, W1, W3, W2, G = _case(5, K=1)
    assert np.all(oracle.layer_backward(X, lg, W1, W3, W2, 1, G)["dlogits"] == 0.0)
    X, lg, W1, W3, W2, G = _case(6, E=5, identical=True)
    got = oracle.layer_backward(X, lg, W1, W3, W2, 3, G)
    # every slot has the same dS; the fp32 weights sum to 1 only up to rounding
    assert np.max(np.abs(got["dlogits"])) <= 1e-6 * float(np.max(np.abs(got["dw"])))
    # every token sees the same dense MLP, so dX does not depend on the routing
    other = oracle.layer_backward(X, -lg, W1, W3, W2, 3, G)
    np.testing.assert_allclose(other["dX"], got["dX"], rtol=1e-6, atol=1e-7)


def test_linear_in_dout_and_exact_bf16_widening():
    X, lg, W1, W3, W2, G = _case(7, K=2)
    a = oracle.layer_backward(X, lg, W1, W3, W2, 2, G)
    b = oracle.layer_backward(X, lg, W1, W3, W2, 2, 2 * G)
    for k in a:
        assert np.array_equal(2 * a[k], b[k]), k
    # bf16 storage: the bit patterns widen exactly to the float32 values they hold
    def bf(x):
        return (np.ascontiguousarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    Xb, W1b, W3b, W2b = bf(X), bf(W1), bf(W3), bf(W2)
    wide = [oracle.bf16_to_f32(v) for v in (Xb, W1b, W3b, W2b)]
    c = oracle.layer_backward(Xb, lg, W1b, W3b, W2b, 2, G)
    d = oracle.layer_backward(wide[0], lg, wide[1], wide[2], wide[3], 2, G)
    for k in c:
        assert np.array_equal(c[k], d[k]), k


def test_rows_variant_equals_the_full_backward():
    X, lg, W1, W3, W2, G = _case(8, T=9, K=2)
    full = oracle.layer_backward(X, lg, W1, W3, W2, 2, G)
    toks = np.array([8, 0, 3, 3], np.int32)
    part = oracle.layer_backward_rows(X, lg, W1, W3, W2, 2, G, toks)
    for k in ("dX", "dlogits", "dw"):
        assert np.array_equal(part[k], full[k][toks]), k


@pytest.mark.parametrize("seed,K,E,bf16", [(9, 2, 4, False), (10, 3, 5, True), (11, 1, 6, False)])
def test_weight_grad_slices_equal_the_full_backward(seed, K, E, bf16):
    """Every (expert, column) slice: column j of dW1[e] and dW3[e], row j of
    dW2[e], bit for bit (same fp64 sums in the same order), experts without
    tokens included (T = 7 with 6 experts and K = 1 leaves some empty)."""
    X, lg, W1, W3, W2, G = _case(seed, T=7, E=E, K=K)
    if bf16:
        import torch
        X, W1, W3, W2 = (torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
                         for a in (X, W1, W3, W2))
    full = oracle.layer_backward(X, lg, W1, W3, W2, K, G)
    n = full["dW1"].shape[2]
    ex = np.repeat(np.arange(E, dtype=np.int32), n)
    cl = np.tile(np.arange(n, dtype=np.int32), E)
    sl = oracle.weight_grad_slices(X, lg, W1, W3, W2, K, G, ex, cl)
    assert np.array_equal(sl["dW1c"], full["dW1"][ex, :, cl])
    assert np.array_equal(sl["dW3c"], full["dW3"][ex, :, cl])
    assert np.array_equal(sl["dW2r"], full["dW2"][ex, cl, :])
    idx, _, counts, _ = oracle.route(lg, K)
    if (counts == 0).any():
        e0 = int(np.nonzero(counts == 0)[0][0])
        assert not sl["dW1c"][ex == e0].any() and not sl["dW2r"][ex == e0].any()

