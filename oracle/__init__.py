"""CPU oracle for the MoE layer forward pass and its backward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports it, and this package imports nothing from
the product: the two share no code.

The arithmetic lives in ``moe_oracle.c`` (plain C, fp64 accumulation); this
module only builds/loads it and marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")

F32 = 0
BF16 = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (IEEE arithmetic: no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.oracle_softmax.argtypes = [P, I, I, P]
        lib.oracle_route.argtypes = [P, I, I, I, P, P, P, P]
        lib.oracle_permute.argtypes = [P, I, I, I, P, P]
        lib.oracle_gather_rows.argtypes = [P, I, I, I, I, P, P]
        lib.oracle_expert_ffn.argtypes = [P, I, I, P, P, I, P, P, P, I, I, I, P, P]
        lib.oracle_combine.argtypes = [P, P, P, I, I, I, P]
        lib.oracle_expert_down.argtypes = [P, I, I, P, P, I, I, I, P]
        lib.oracle_layer.argtypes = [P, I, P, P, P, P, I, I, I, I, I, P, I, P]
        lib.oracle_router.argtypes = [P, I, P, P, I, I, I, P]
        L = ctypes.c_int64
        lib.oracle_tr_target.argtypes = [ctypes.c_int32, I, I, I]
        lib.oracle_tr_target.restype = ctypes.c_int32
        lib.oracle_token_round.argtypes = [P, I, I, I, I, I, P, P, P, L, P, P]
        lib.oracle_tr_combine.argtypes = [P, P, P, I, I, I, L, P]
        lib.oracle_tr_layer.argtypes = [P, I, P, P, P, P, P, I, I, I, I, P, I, P]
        lib.oracle_layer_backward.argtypes = [P, I, P, P, P, P, I, I, I, I, I, P, P, P, P, P, P, P]
        lib.oracle_layer_backward_rows.argtypes = [P, I, P, P, P, P, I, I, I, I, I, P, P, I, P, P, P]
        lib.oracle_weight_grad_slices.argtypes = [P, I, P, P, P, P, I, I, I, I, I, P, P, P, I, P, P, P]
        for f in (lib.oracle_softmax, lib.oracle_route, lib.oracle_permute, lib.oracle_gather_rows,
                  lib.oracle_expert_ffn, lib.oracle_combine, lib.oracle_layer, lib.oracle_expert_down,
                  lib.oracle_router, lib.oracle_token_round, lib.oracle_tr_combine, lib.oracle_tr_layer,
                  lib.oracle_layer_backward, lib.oracle_layer_backward_rows, lib.oracle_weight_grad_slices):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc: int, name: str):
    if rc != 0:
        raise ValueError(f"{name} rejected its arguments (rc={rc})")


def _storage(x: np.ndarray):
    """Return (contiguous array, dtype code).  bf16 tensors arrive as uint16 bit patterns."""
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x), BF16
    return np.ascontiguousarray(x, dtype=np.float32), F32


def router(X, Wr, bias=None) -> np.ndarray:
    """Router logits X @ Wr (+ bias), fp64 sums rounded to fp32.  -> float32 [T, E]."""
    Xs, dt = _storage(X)
    W = _c(Wr, np.float32)
    T, d = Xs.shape
    d_, E = W.shape
    assert d_ == d
    b = None if bias is None else _c(bias, np.float32)
    assert b is None or b.shape == (E,)
    out = np.empty((T, E), np.float32)
    _check(_load().oracle_router(_ptr(Xs), dt, _ptr(W), None if b is None else _ptr(b), T, d, E, _ptr(out)),
           "oracle_router")
    return out


def softmax(logits: np.ndarray) -> np.ndarray:
    lg = _c(logits, np.float32)
    T, E = lg.shape
    p = np.empty((T, E), np.float64)
    _check(_load().oracle_softmax(_ptr(lg), T, E, _ptr(p)), "oracle_softmax")
    return p


def route(logits: np.ndarray, K: int):
    """-> (idx int32 [T,K], w float32 [T,K], counts int32 [E], offsets int32 [E+1])."""
    lg = _c(logits, np.float32)
    T, E = lg.shape
    idx = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float32)
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    _check(_load().oracle_route(_ptr(lg), T, E, K, _ptr(idx), _ptr(w), _ptr(counts), _ptr(offsets)),
           "oracle_route")
    return idx, w, counts, offsets


def permute(idx: np.ndarray, E: int):
    """-> (sorted_pair int32 [T*K], inv int32 [T*K])."""
    ix = _c(idx, np.int32)
    T, K = ix.shape
    sp = np.empty(T * K, np.int32)
    inv = np.empty(T * K, np.int32)
    _check(_load().oracle_permute(_ptr(ix), T, E, K, _ptr(sp), _ptr(inv)), "oracle_permute")
    return sp, inv


def gather_rows(X: np.ndarray, sorted_pair: np.ndarray, K: int) -> np.ndarray:
    Xc = np.ascontiguousarray(X)
    T, d = Xc.shape
    sp = _c(sorted_pair, np.int32)
    Xp = np.empty((sp.size, d), Xc.dtype)
    _check(_load().oracle_gather_rows(_ptr(Xc), Xc.itemsize, T, d, K, _ptr(sp), _ptr(Xp)),
           "oracle_gather_rows")
    return Xp


def expert_ffn(Xp: np.ndarray, row_expert: np.ndarray, W1, W3, W2, rows=None):
    """Expert MLP on expert-ordered rows.  -> (act float32 [nsel,n], y float32 [nsel,d])."""
    Xs, dt = _storage(Xp)
    W1s, d1 = _storage(W1)
    W3s, d3 = _storage(W3)
    W2s, d2 = _storage(W2)
    if not (dt == d1 == d3 == d2):
        raise ValueError("Xp and the expert weights must share one storage dtype")
    nrows, d = Xs.shape
    E, d_, n = W1s.shape
    assert d_ == d and W3s.shape == (E, d, n) and W2s.shape == (E, n, d)
    re = _c(row_expert, np.int32)
    if rows is None:
        nsel, rp = nrows, None
    else:
        rr = _c(rows, np.int32)
        nsel, rp = rr.size, _ptr(rr)
    act = np.empty((nsel, n), np.float32)
    y = np.empty((nsel, d), np.float32)
    _check(_load().oracle_expert_ffn(_ptr(Xs), dt, nrows, _ptr(re), rp, nsel, _ptr(W1s), _ptr(W3s),
                                     _ptr(W2s), E, d, n, _ptr(act), _ptr(y)), "oracle_expert_ffn")
    return act, y


def expert_down(act: np.ndarray, row_expert: np.ndarray, W2) -> np.ndarray:
    """Second expert GEMM alone on expert-ordered rows.  -> y float32 [nrows, d]."""
    As, dt = _storage(act)
    W2s, d2 = _storage(W2)
    if dt != d2:
        raise ValueError("act and W2 must share one storage dtype")
    nrows, n = As.shape
    E, n_, d = W2s.shape
    assert n_ == n
    re = _c(row_expert, np.int32)
    y = np.empty((nrows, d), np.float32)
    _check(_load().oracle_expert_down(_ptr(As), dt, nrows, _ptr(re), _ptr(W2s), E, d, n, _ptr(y)),
           "oracle_expert_down")
    return y


def combine(Y: np.ndarray, w: np.ndarray, inv: np.ndarray) -> np.ndarray:
    Yc = _c(Y, np.float32)
    wc = _c(w, np.float32)
    T, K = wc.shape
    d = Yc.shape[1]
    invc = _c(inv, np.int32)
    out = np.empty((T, d), np.float32)
    _check(_load().oracle_combine(_ptr(Yc), _ptr(wc), _ptr(invc), T, d, K, _ptr(out)), "oracle_combine")
    return out


def layer(X, logits, W1, W3, W2, K: int, tokens=None) -> np.ndarray:
    """Whole layer, per-token loop over the selected experts.  -> float32 [ntok, d]."""
    Xs, dt = _storage(X)
    W1s, d1 = _storage(W1)
    W3s, d3 = _storage(W3)
    W2s, d2 = _storage(W2)
    if not (dt == d1 == d3 == d2):
        raise ValueError("X and the expert weights must share one storage dtype")
    lg = _c(logits, np.float32)
    T, d = Xs.shape
    E, _, n = W1s.shape
    if tokens is None:
        ntok, tp = T, None
    else:
        tk = _c(tokens, np.int32)
        ntok, tp = tk.size, _ptr(tk)
    out = np.empty((ntok, d), np.float32)
    _check(_load().oracle_layer(_ptr(Xs), dt, _ptr(lg), _ptr(W1s), _ptr(W3s), _ptr(W2s), T, d, E, K, n,
                                tp, ntok, _ptr(out)), "oracle_layer")
    return out


def layer_backward(X, logits, W1, W3, W2, K: int, dout):
    """Gradient of layer() given dout [T, d]: a dict of float32 arrays dX [T, d],
    dlogits [T, E], dW1, dW3 [E, d, n], dW2 [E, n, d] and dw [T, K] (the
    gradient of the renormalised routing weights)."""
    Xs, dt = _storage(X)
    W1s, d1 = _storage(W1)
    W3s, d3 = _storage(W3)
    W2s, d2 = _storage(W2)
    if not (dt == d1 == d3 == d2):
        raise ValueError("X and the expert weights must share one storage dtype")
    lg = _c(logits, np.float32)
    g = _c(dout, np.float32)
    T, d = Xs.shape
    E, _, n = W1s.shape
    assert g.shape == (T, d) and lg.shape == (T, E)
    r = {"dX": np.empty((T, d), np.float32), "dlogits": np.empty((T, E), np.float32),
         "dW1": np.empty((E, d, n), np.float32), "dW3": np.empty((E, d, n), np.float32),
         "dW2": np.empty((E, n, d), np.float32), "dw": np.empty((T, K), np.float32)}
    _check(_load().oracle_layer_backward(_ptr(Xs), dt, _ptr(lg), _ptr(W1s), _ptr(W3s), _ptr(W2s), T, d, E, K, n,
                                         _ptr(g), _ptr(r["dX"]), _ptr(r["dlogits"]), _ptr(r["dW1"]), _ptr(r["dW3"]),
                                         _ptr(r["dW2"]), _ptr(r["dw"])), "oracle_layer_backward")
    return r


def layer_backward_rows(X, logits, W1, W3, W2, K: int, dout, tokens):
    """layer_backward() for the listed tokens only, without weight gradients:
    a dict of dX [ntok, d], dlogits [ntok, E] and dw [ntok, K] (float32)."""
    Xs, dt = _storage(X)
    W1s, d1 = _storage(W1)
    W3s, d3 = _storage(W3)
    W2s, d2 = _storage(W2)
    if not (dt == d1 == d3 == d2):
        raise ValueError("X and the expert weights must share one storage dtype")
    lg = _c(logits, np.float32)
    g = _c(dout, np.float32)
    tk = _c(tokens, np.int32)
    T, d = Xs.shape
    E, _, n = W1s.shape
    m = tk.size
    r = {"dX": np.empty((m, d), np.float32), "dlogits": np.empty((m, E), np.float32),
         "dw": np.empty((m, K), np.float32)}
    _check(_load().oracle_layer_backward_rows(_ptr(Xs), dt, _ptr(lg), _ptr(W1s), _ptr(W3s), _ptr(W2s), T, d, E, K,
                                              n, _ptr(g), _ptr(tk), m, _ptr(r["dX"]), _ptr(r["dlogits"]),
                                              _ptr(r["dw"])), "oracle_layer_backward_rows")
    return r


def weight_grad_slices(X, logits, W1, W3, W2, K: int, dout, experts, cols):
    """Slices of layer_backward()'s weight gradients for pairs (experts[p], cols[p]):
    a dict of float32 arrays dW1c, dW3c [npair, d] (column cols[p] of dW1 and dW3
    of expert experts[p]) and dW2r [npair, d] (row cols[p] of its dW2)."""
    Xs, dt = _storage(X)
    W1s, d1 = _storage(W1)
    W3s, d3 = _storage(W3)
    W2s, d2 = _storage(W2)
    if not (dt == d1 == d3 == d2):
        raise ValueError("X and the expert weights must share one storage dtype")
    lg = _c(logits, np.float32)
    g = _c(dout, np.float32)
    ex = _c(experts, np.int32)
    cl = _c(cols, np.int32)
    T, d = Xs.shape
    E, _, n = W1s.shape
    m = ex.size
    assert cl.size == m and g.shape == (T, d) and lg.shape == (T, E)
    r = {"dW1c": np.empty((m, d), np.float32), "dW3c": np.empty((m, d), np.float32),
         "dW2r": np.empty((m, d), np.float32)}
    _check(_load().oracle_weight_grad_slices(_ptr(Xs), dt, _ptr(lg), _ptr(W1s), _ptr(W3s), _ptr(W2s), T, d, E, K,
                                             n, _ptr(g), _ptr(ex), _ptr(cl), m, _ptr(r["dW1c"]), _ptr(r["dW3c"]),
                                             _ptr(r["dW2r"])), "oracle_weight_grad_slices")
    return r


def tr_target(f: int, M: int, T: int, cap_tiles: int = 0) -> int:
    """Rows an expert with f routed tokens keeps under Token Rounding."""
    return int(_load().oracle_tr_target(int(f), int(M), int(T), int(cap_tiles)))


def token_round(logits: np.ndarray, K: int, M: int, cap_tiles: int = 0):
    """Token Rounding plan.  -> dict with counts_r int32 [E], offsets_r int32 [E+1],
    row_tok int32 [rows], slot_row int32 [T,E] (-1 where not kept), slot_w float32 [T,E]."""
    lg = _c(logits, np.float32)
    T, E = lg.shape
    cap = T * E
    counts_r = np.empty(E, np.int32)
    offsets_r = np.empty(E + 1, np.int32)
    row_tok = np.empty(max(cap, 1), np.int32)
    slot_row = np.empty((T, E), np.int32)
    slot_w = np.empty((T, E), np.float32)
    _check(_load().oracle_token_round(_ptr(lg), T, E, K, M, cap_tiles, _ptr(counts_r), _ptr(offsets_r),
                                      _ptr(row_tok), cap, _ptr(slot_row), _ptr(slot_w)), "oracle_token_round")
    return {"counts_r": counts_r, "offsets_r": offsets_r, "row_tok": row_tok[: int(offsets_r[E])].copy(),
            "slot_row": slot_row, "slot_w": slot_w}


def tr_combine(Y: np.ndarray, slot_row: np.ndarray, slot_w: np.ndarray) -> np.ndarray:
    """out[t] = sum over kept experts e (ascending) of slot_w[t,e] * Y[slot_row[t,e]] (fp64)."""
    Yc = _c(Y, np.float32)
    sr = _c(slot_row, np.int32)
    sw = _c(slot_w, np.float32)
    T, E = sr.shape
    nrows, d = Yc.shape
    out = np.empty((T, d), np.float32)
    _check(_load().oracle_tr_combine(_ptr(Yc), _ptr(sr), _ptr(sw), T, E, d, nrows, _ptr(out)),
           "oracle_tr_combine")
    return out


def tr_layer(X, slot_row, slot_w, W1, W3, W2, tokens=None) -> np.ndarray:
    """Layer after Token Rounding, per-token loop over the kept experts.  -> float32 [ntok, d]."""
    Xs, dt = _storage(X)
    W1s, d1 = _storage(W1)
    W3s, d3 = _storage(W3)
    W2s, d2 = _storage(W2)
    if not (dt == d1 == d3 == d2):
        raise ValueError("X and the expert weights must share one storage dtype")
    sr = _c(slot_row, np.int32)
    sw = _c(slot_w, np.float32)
    T, d = Xs.shape
    E, _, n = W1s.shape
    assert sr.shape == (T, E) and sw.shape == (T, E)
    if tokens is None:
        ntok, tp = T, None
    else:
        tk = _c(tokens, np.int32)
        ntok, tp = tk.size, _ptr(tk)
    out = np.empty((ntok, d), np.float32)
    _check(_load().oracle_tr_layer(_ptr(Xs), dt, _ptr(sr), _ptr(sw), _ptr(W1s), _ptr(W3s), _ptr(W2s), T, d, E,
                                   n, tp, ntok, _ptr(out)), "oracle_tr_layer")
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)
