"""Python binding of libmoe, the gfx950 MoE layer forward library.

Argument marshalling only: every step of the layer runs in the HIP kernels of
``libmoe.so`` (built in-tree by ``_build.build()``).  PyTorch provides device
memory and the current stream.  There is no CPU fallback: if the library is
missing, or a tensor is not on the GPU, the call raises.

The functions carry the names of the C entry points declared in
``include/moe.h``; each allocates its outputs and workspace with torch and
enqueues the library call on torch's current stream.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "moe.h")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16 = 0, 1

_lib = None


class MoEError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        super().__init__(f"{func}: status {status}: {detail}")
        self.status = status


def load_library() -> ctypes.CDLL:
    """Load libmoe.so and declare its C signatures (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, Z, L = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_longlong
    sig = {
        "moe_status_string": ([I], ctypes.c_char_p),
        "moe_last_error": ([], ctypes.c_char_p),
        "moe_workspace_bytes": ([I, I, I, I, I, I], Z),
        "moe_route_workspace_bytes": ([I, I, I], Z),
        "moe_permute_workspace_bytes": ([I, I, I], Z),
        "moe_forward_workspace_bytes": ([I, I, I, I, I, I], Z),
        "moe_ffn_workspace_bytes": ([I, I, I], Z),
        "moe_router_workspace_bytes": ([I, I, I], Z),
        "moe_router": ([P, I, I, I, I, P, P, P, P, Z, P], I),
        "moe_route": ([P, I, I, I, P, P, P, P, P, Z, P], I),
        "moe_route_noalloc": ([P, I, I, I, P, P, P, P, P], I),
        "moe_permute": ([P, I, I, I, I, I, P, P, P, P, P, Z, P], I),
        "moe_grouped_ffn": ([P, P, P, P, I, I, I, I, I, I, P, P, P, P, P, Z, P], I),
        "moe_ffn_up": ([P, P, P, I, I, I, I, I, I, P, P, P, P, Z, P], I),
        "moe_ffn_down": ([P, P, I, I, I, I, I, I, P, P, P, P, Z, P], I),
        "moe_combine": ([P, P, P, I, I, I, I, P, P], I),
        "moe_forward": ([P, P, P, P, P, I, I, I, I, I, I, P, P, P, P, P, P, P, P, Z, P], I),
        "moe_route_x_workspace_bytes": ([I, I, I, I, I], Z),
        "moe_route_x": ([P, I, I, I, I, I, P, P, P, P, P, P, P, P, Z, P], I),
        "moe_forward_x_workspace_bytes": ([I, I, I, I, I, I], Z),
        "moe_forward_x": ([P, P, P, P, P, P, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, Z, P], I),
        "moe_token_round_max_rows": ([I, I, I, I], L),
        "moe_token_round_workspace_bytes": ([I, I, I, I], Z),
        "moe_token_round": ([P, P, P, I, I, I, I, I, P, P, P, L, P, P, P, Z, P], I),
        "moe_tr_combine": ([P, P, P, I, I, I, I, L, P, P], I),
        "moe_forward_tr_workspace_bytes": ([I, I, I, I, I, I, I], Z),
        "moe_forward_tr": ([P, P, P, P, P, I, I, I, I, I, I, I, I, P, P, P, P, P, P, P, Z, P], I),
        "moe_backward_data_workspace_bytes": ([I, I, I, I, I, I], Z),
        "moe_backward_data": ([P, P, P, P, P, I, I, I, I, I, I, P, P, P, P, P, Z, P], I),
        "moe_backward_workspace_bytes": ([I, I, I, I, I, I], Z),
        "moe_backward": ([P, P, P, P, P, I, I, I, I, I, I, P, P, P, P, P, P, P, P, Z, P], I),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def header_functions() -> list[str]:
    """Names of the functions include/moe.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def _check(status: int, func: str):
    if status != MOE_OK:
        lib = load_library()
        raise MoEError(status, func, lib.moe_last_error().decode())


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return MOE_F32
    if dt == torch.bfloat16:
        return MOE_BF16
    raise ValueError(f"unsupported dtype {dt}")


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def moe_router(X: torch.Tensor, Wr: torch.Tensor, bias: torch.Tensor | None = None, ws: torch.Tensor | None = None):
    """Router projection.  X [T,d] (f32/bf16), Wr [d,E] f32, bias [E] f32 or None -> logits [T,E] f32."""
    lib = load_library()
    T, d = X.shape
    E = Wr.shape[1]
    dev = X.device
    dt = dtype_code(X.dtype)
    wsb = lib.moe_router_workspace_bytes(d, E, dt)
    if wsb and ws is None:
        ws = _workspace(wsb, dev)
    logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    _check(lib.moe_router(_dev(X, "X"), dt, T, d, E, _dev(Wr, "Wr", torch.float32),
                          0 if bias is None else _dev(bias, "bias", torch.float32), logits.data_ptr(),
                          0 if not wsb else ws.data_ptr(), wsb, _stream(dev)), "moe_router")
    return logits


def moe_route(logits: torch.Tensor, K: int, out=None, ws: torch.Tensor | None = None):
    """Steps 1-2.  logits [T,E] fp32 -> (topk_idx [T,K] i32, topk_w [T,K] f32, counts [E] i32, offsets [E+1] i32).
    `out` (optional) is such a tuple to write into and `ws` a workspace of moe_route_workspace_bytes bytes,
    so that repeated calls allocate nothing."""
    lib = load_library()
    T, E = logits.shape
    dev = logits.device
    if out is None:
        out = (torch.empty((T, K), dtype=torch.int32, device=dev), torch.empty((T, K), dtype=torch.float32, device=dev),
               torch.empty(E, dtype=torch.int32, device=dev), torch.empty(E + 1, dtype=torch.int32, device=dev))
    idx, w, counts, offsets = out
    for t, shape, dt, name in ((idx, (T, K), torch.int32, "topk_idx"), (w, (T, K), torch.float32, "topk_w"),
                               (counts, (E,), torch.int32, "counts"), (offsets, (E + 1,), torch.int32, "offsets")):
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must have shape {shape}, got {tuple(t.shape)}")
        _dev(t, name, dt)
    nws = lib.moe_route_workspace_bytes(T, E, K)
    if ws is None:
        ws = _workspace(nws, dev)
    elif ws.numel() < nws:
        raise ValueError(f"ws must hold {nws} bytes")
    _check(lib.moe_route(_dev(logits, "logits", torch.float32), T, E, K, idx.data_ptr(), w.data_ptr(),
                         counts.data_ptr(), offsets.data_ptr(), ws.data_ptr(), nws, _stream(dev)), "moe_route")
    return idx, w, counts, offsets


def moe_route_noalloc(logits: torch.Tensor, K: int, out):
    """Steps 1-2 with the library's static scratch instead of a workspace.  `out` is the
    (topk_idx [T,K] i32, topk_w [T,K] f32, counts [E] i32, offsets [E+1] i32) tuple written into."""
    lib = load_library()
    T, E = logits.shape
    idx, w, counts, offsets = out
    for t, shape, dt, name in ((idx, (T, K), torch.int32, "topk_idx"), (w, (T, K), torch.float32, "topk_w"),
                               (counts, (E,), torch.int32, "counts"), (offsets, (E + 1,), torch.int32, "offsets")):
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must have shape {shape}, got {tuple(t.shape)}")
        _dev(t, name, dt)
    _check(lib.moe_route_noalloc(_dev(logits, "logits", torch.float32), T, E, K, idx.data_ptr(), w.data_ptr(),
                                 counts.data_ptr(), offsets.data_ptr(), _stream(logits.device)), "moe_route_noalloc")
    return out


def moe_permute(X: torch.Tensor, topk_idx: torch.Tensor, E: int, out=None, ws: torch.Tensor | None = None):
    """Step 3.  X [T,d], topk_idx [T,K] -> (sorted_pair [T*K] i32, inv [T*K] i32, Xp [T*K,d]).
    `out` (optional) is such a tuple to write into and `ws` a workspace of moe_permute_workspace_bytes
    bytes, so that repeated calls allocate nothing."""
    lib = load_library()
    T, d = X.shape
    K = topk_idx.shape[1]
    dev = X.device
    if out is None:
        out = (torch.empty(T * K, dtype=torch.int32, device=dev), torch.empty(T * K, dtype=torch.int32, device=dev),
               torch.empty((T * K, d), dtype=X.dtype, device=dev))
    sp, inv, Xp = out
    for t, shape, tdt, name in ((sp, (T * K,), torch.int32, "sorted_pair"), (inv, (T * K,), torch.int32, "inv"),
                                (Xp, (T * K, d), X.dtype, "Xp")):
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must have shape {shape}, got {tuple(t.shape)}")
        _dev(t, name, tdt)
    nws = lib.moe_permute_workspace_bytes(T, E, K)
    if ws is None:
        ws = _workspace(nws, dev)
    elif ws.numel() < nws:
        raise ValueError(f"ws must hold {nws} bytes")
    _check(lib.moe_permute(_dev(X, "X"), dtype_code(X.dtype), T, d, E, K, _dev(topk_idx, "topk_idx", torch.int32),
                           sp.data_ptr(), inv.data_ptr(), Xp.data_ptr(), ws.data_ptr(), nws, _stream(dev)),
           "moe_permute")
    return sp, inv, Xp


def ffn_workspace(d: int, n: int, dtype, device, split: bool = True, ws: torch.Tensor | None = None):
    """(pointer, bytes) of the optional grouped-GEMM workspace: none when split
    is off or the sizes take no split; `ws` (uint8 tensor) is used when given."""
    if not split:
        return None, 0
    nbytes = load_library().moe_ffn_workspace_bytes(d, n, dtype_code(dtype))
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = _workspace(nbytes, device)
    if ws.numel() < nbytes:
        raise MoEError(MOE_ERR_WORKSPACE, "ffn workspace", f"needs {nbytes} bytes, got {ws.numel()}")
    return ws.data_ptr(), nbytes


def moe_grouped_ffn(Xp: torch.Tensor, W1: torch.Tensor, W3: torch.Tensor, W2: torch.Tensor,
                    counts: torch.Tensor, offsets: torch.Tensor, K: int, split: bool = True,
                    ws: torch.Tensor | None = None):
    """Step 4.  Xp [T*K,d], W1/W3 [E,d,n], W2 [E,n,d] -> (Act [T*K,n], Y [T*K,d]).
    split: let the last partial round of tiles be split along K (workspace `ws`
    or one allocated here)."""
    lib = load_library()
    A, d = Xp.shape
    E, _, n = W1.shape
    T = A // K
    dev = Xp.device
    Act = torch.empty((A, n), dtype=Xp.dtype, device=dev)
    Y = torch.empty((A, d), dtype=Xp.dtype, device=dev)
    wp, wn = ffn_workspace(d, n, Xp.dtype, dev, split, ws)
    _check(lib.moe_grouped_ffn(_dev(Xp, "Xp"), _dev(W1, "W1", Xp.dtype), _dev(W3, "W3", Xp.dtype),
                               _dev(W2, "W2", Xp.dtype), dtype_code(Xp.dtype), T, d, E, K, n,
                               _dev(counts, "counts", torch.int32), _dev(offsets, "offsets", torch.int32),
                               Act.data_ptr(), Y.data_ptr(), wp, wn, _stream(dev)), "moe_grouped_ffn")
    return Act, Y


def _out(out, shape, dtype, device, name):
    if out is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if tuple(out.shape) != tuple(shape) or out.dtype != dtype or not out.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}")
    return out


def moe_ffn_up(Xp: torch.Tensor, W1: torch.Tensor, W3: torch.Tensor, counts: torch.Tensor,
               offsets: torch.Tensor, K: int, split: bool = True, ws: torch.Tensor | None = None,
               out: torch.Tensor | None = None):
    """Step 4a.  Xp [T*K,d], W1/W3 [E,d,n] -> Act [T*K,n] = SiLU(Xp W1) * (Xp W3)
    (written into `out` when given)."""
    lib = load_library()
    A, d = Xp.shape
    E, _, n = W1.shape
    dev = Xp.device
    Act = _out(out, (A, n), Xp.dtype, dev, "out")
    wp, wn = ffn_workspace(d, n, Xp.dtype, dev, split, ws)
    _check(lib.moe_ffn_up(_dev(Xp, "Xp"), _dev(W1, "W1", Xp.dtype), _dev(W3, "W3", Xp.dtype), dtype_code(Xp.dtype),
                          A // K, d, E, K, n, _dev(counts, "counts", torch.int32),
                          _dev(offsets, "offsets", torch.int32), Act.data_ptr(), wp, wn, _stream(dev)),
           "moe_ffn_up")
    return Act


def moe_ffn_down(Act: torch.Tensor, W2: torch.Tensor, counts: torch.Tensor, offsets: torch.Tensor, K: int,
                 split: bool = True, ws: torch.Tensor | None = None, out: torch.Tensor | None = None):
    """Step 4b.  Act [T*K,n], W2 [E,n,d] -> Y [T*K,d] = Act W2 (written into `out` when given)."""
    lib = load_library()
    A, n = Act.shape
    E, _, d = W2.shape
    dev = Act.device
    Y = _out(out, (A, d), Act.dtype, dev, "out")
    wp, wn = ffn_workspace(d, n, Act.dtype, dev, split, ws)
    _check(lib.moe_ffn_down(_dev(Act, "Act"), _dev(W2, "W2", Act.dtype), dtype_code(Act.dtype), A // K, d, E, K, n,
                            _dev(counts, "counts", torch.int32), _dev(offsets, "offsets", torch.int32),
                            Y.data_ptr(), wp, wn, _stream(dev)), "moe_ffn_down")
    return Y


def moe_combine(Y: torch.Tensor, topk_w: torch.Tensor, inv: torch.Tensor, out: torch.Tensor | None = None):
    """Step 5.  Y [T*K,d], topk_w [T,K] f32, inv [T*K] i32 -> out [T,d] (written into `out` when given)."""
    lib = load_library()
    T, K = topk_w.shape
    d = Y.shape[1]
    dev = Y.device
    if out is None:
        out = torch.empty((T, d), dtype=Y.dtype, device=dev)
    elif tuple(out.shape) != (T, d) or out.dtype != Y.dtype:
        raise ValueError(f"out must be [{T}, {d}] of {Y.dtype}")
    _dev(out, "out")
    _check(lib.moe_combine(_dev(Y, "Y"), _dev(topk_w, "topk_w", torch.float32), _dev(inv, "inv", torch.int32),
                           dtype_code(Y.dtype), T, d, K, out.data_ptr(), _stream(dev)), "moe_combine")
    return out


class ForwardPlan:
    """Preallocated outputs and workspace for repeated moe_forward calls on one shape."""

    def __init__(self, T: int, d: int, E: int, K: int, n: int, dtype: torch.dtype, device):
        lib = load_library()
        self.T, self.d, self.E, self.K, self.n, self.dtype = T, d, E, K, n, dtype
        self.device = torch.device(device)
        self.ws_bytes = lib.moe_forward_workspace_bytes(T, d, E, K, n, dtype_code(dtype))
        if self.ws_bytes == 0:
            raise MoEError(MOE_ERR_UNSUPPORTED, "moe_forward_workspace_bytes", lib.moe_last_error().decode())
        dev = self.device
        self.ws = _workspace(self.ws_bytes, dev)
        self.out = torch.empty((T, d), dtype=dtype, device=dev)
        self.topk_idx = torch.empty((T, K), dtype=torch.int32, device=dev)
        self.topk_w = torch.empty((T, K), dtype=torch.float32, device=dev)
        self.counts = torch.empty(E, dtype=torch.int32, device=dev)
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        self.sorted_pair = torch.empty(T * K, dtype=torch.int32, device=dev)
        self.inv = torch.empty(T * K, dtype=torch.int32, device=dev)

    def __call__(self, X, logits, W1, W3, W2):
        lib = load_library()
        dt = self.dtype
        _check(lib.moe_forward(_dev(X, "X", dt), _dev(logits, "logits", torch.float32), _dev(W1, "W1", dt),
                               _dev(W3, "W3", dt), _dev(W2, "W2", dt), dtype_code(dt), self.T, self.d, self.E,
                               self.K, self.n, self.out.data_ptr(), self.topk_idx.data_ptr(),
                               self.topk_w.data_ptr(), self.counts.data_ptr(), self.offsets.data_ptr(),
                               self.sorted_pair.data_ptr(), self.inv.data_ptr(), self.ws.data_ptr(),
                               self.ws_bytes, _stream(self.device)), "moe_forward")
        return self.out


def moe_forward(X: torch.Tensor, logits: torch.Tensor, W1: torch.Tensor, W3: torch.Tensor, W2: torch.Tensor,
                K: int):
    """Whole layer.  Returns (out [T,d], plan) -- the plan also holds the routing outputs."""
    T, d = X.shape
    E, _, n = W1.shape
    plan = ForwardPlan(T, d, E, K, n, X.dtype, X.device)
    plan(X, logits, W1, W3, W2)
    return plan.out, plan


def moe_route_x(X: torch.Tensor, Wr: torch.Tensor, bias: torch.Tensor | None, K: int, want_logits: bool = True,
                ws: torch.Tensor | None = None, out=None):
    """Router projection and steps 1-2 from the tokens.  X [T,d], Wr [d,E] f32, bias [E] f32 or None ->
    (topk_idx [T,K] i32, topk_w [T,K] f32, counts [E] i32, offsets [E+1] i32, logits [T,E] f32 or None).
    `out` (optional) is such a tuple to write into and `ws` a workspace of moe_route_x_workspace_bytes bytes,
    so that repeated calls allocate nothing."""
    lib = load_library()
    T, d = X.shape
    E = Wr.shape[1]
    dev = X.device
    dt = dtype_code(X.dtype)
    nws = lib.moe_route_x_workspace_bytes(T, d, E, K, dt)
    if nws == 0:
        raise MoEError(MOE_ERR_UNSUPPORTED, "moe_route_x_workspace_bytes", lib.moe_last_error().decode())
    if ws is None:
        ws = _workspace(nws, dev)
    elif ws.numel() < nws:
        raise ValueError(f"ws must hold {nws} bytes")
    if out is None:
        out = (torch.empty((T, K), dtype=torch.int32, device=dev), torch.empty((T, K), dtype=torch.float32, device=dev),
               torch.empty(E, dtype=torch.int32, device=dev), torch.empty(E + 1, dtype=torch.int32, device=dev),
               torch.empty((T, E), dtype=torch.float32, device=dev) if want_logits else None)
    idx, w, counts, offsets, logits = out
    for t, shape, tdt, name in ((idx, (T, K), torch.int32, "topk_idx"), (w, (T, K), torch.float32, "topk_w"),
                                (counts, (E,), torch.int32, "counts"), (offsets, (E + 1,), torch.int32, "offsets")):
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must have shape {shape}, got {tuple(t.shape)}")
        _dev(t, name, tdt)
    if logits is not None and tuple(logits.shape) != (T, E):
        raise ValueError(f"logits must have shape {(T, E)}")
    _check(lib.moe_route_x(_dev(X, "X"), dt, T, d, E, K, _dev(Wr, "Wr", torch.float32),
                           0 if bias is None else _dev(bias, "bias", torch.float32),
                           0 if logits is None else logits.data_ptr(), idx.data_ptr(), w.data_ptr(),
                           counts.data_ptr(), offsets.data_ptr(), _dev(ws, "ws"), nws, _stream(dev)), "moe_route_x")
    return idx, w, counts, offsets, logits


class ForwardXPlan(ForwardPlan):
    """Preallocated outputs and workspace for repeated moe_forward_x calls (the layer from X and the router
    weights); `logits` is filled only when want_logits is set."""

    def __init__(self, T: int, d: int, E: int, K: int, n: int, dtype: torch.dtype, device, want_logits: bool = False):
        super().__init__(T, d, E, K, n, dtype, device)
        lib = load_library()
        self.ws_bytes = lib.moe_forward_x_workspace_bytes(T, d, E, K, n, dtype_code(dtype))
        if self.ws_bytes == 0:
            raise MoEError(MOE_ERR_UNSUPPORTED, "moe_forward_x_workspace_bytes", lib.moe_last_error().decode())
        self.ws = _workspace(self.ws_bytes, self.device)
        self.logits = torch.empty((T, E), dtype=torch.float32, device=self.device) if want_logits else None

    def __call__(self, X, Wr, bias, W1, W3, W2):
        lib = load_library()
        dt = self.dtype
        _check(lib.moe_forward_x(_dev(X, "X", dt), _dev(Wr, "Wr", torch.float32),
                                 0 if bias is None else _dev(bias, "bias", torch.float32), _dev(W1, "W1", dt),
                                 _dev(W3, "W3", dt), _dev(W2, "W2", dt), dtype_code(dt), self.T, self.d, self.E,
                                 self.K, self.n, self.out.data_ptr(),
                                 0 if self.logits is None else self.logits.data_ptr(), self.topk_idx.data_ptr(),
                                 self.topk_w.data_ptr(), self.counts.data_ptr(), self.offsets.data_ptr(),
                                 self.sorted_pair.data_ptr(), self.inv.data_ptr(), self.ws.data_ptr(),
                                 self.ws_bytes, _stream(self.device)), "moe_forward_x")
        return self.out


def moe_forward_x(X: torch.Tensor, Wr: torch.Tensor, bias: torch.Tensor | None, W1: torch.Tensor, W3: torch.Tensor,
                  W2: torch.Tensor, K: int, want_logits: bool = True):
    """Whole layer from X and the router weights.  Returns (out [T,d], plan) -- the plan holds the routing
    outputs and, with want_logits, the logits."""
    T, d = X.shape
    E, _, n = W1.shape
    plan = ForwardXPlan(T, d, E, K, n, X.dtype, X.device, want_logits)
    plan(X, Wr, bias, W1, W3, W2)
    return plan.out, plan


def moe_token_round(logits: torch.Tensor, topk_idx: torch.Tensor, counts: torch.Tensor, M: int,
                    cap_tiles: int = 0):
    """Token Rounding plan from logits [T,E] f32 and moe_route's topk_idx [T,K] / counts [E].
    Returns a dict: counts_r [E], offsets_r [E+1], row_tok [max rows] (the first offsets_r[E]
    entries are the plan's), slot_row [T,E] i32, slot_w [T,E] f32."""
    lib = load_library()
    T, E = logits.shape
    K = topk_idx.shape[1]
    dev = logits.device
    R = lib.moe_token_round_max_rows(T, E, K, M)
    nws = lib.moe_token_round_workspace_bytes(T, E, K, M)
    if R <= 0 or nws == 0:
        raise MoEError(MOE_ERR_UNSUPPORTED, "moe_token_round_max_rows", lib.moe_last_error().decode())
    ws = _workspace(nws, dev)
    plan = {
        "counts_r": torch.empty(E, dtype=torch.int32, device=dev),
        "offsets_r": torch.empty(E + 1, dtype=torch.int32, device=dev),
        "row_tok": torch.empty(R, dtype=torch.int32, device=dev),
        "slot_row": torch.empty((T, E), dtype=torch.int32, device=dev),
        "slot_w": torch.empty((T, E), dtype=torch.float32, device=dev),
    }
    _check(lib.moe_token_round(_dev(logits, "logits", torch.float32), _dev(topk_idx, "topk_idx", torch.int32),
                               _dev(counts, "counts", torch.int32), T, E, K, M, cap_tiles,
                               plan["counts_r"].data_ptr(), plan["offsets_r"].data_ptr(), plan["row_tok"].data_ptr(),
                               R, plan["slot_row"].data_ptr(), plan["slot_w"].data_ptr(), ws.data_ptr(), nws,
                               _stream(dev)), "moe_token_round")
    return plan


def moe_tr_combine(Y: torch.Tensor, slot_row: torch.Tensor, slot_w: torch.Tensor):
    """Combine after Token Rounding.  Y [rows,d], slot_row [T,E] i32, slot_w [T,E] f32 -> out [T,d]."""
    lib = load_library()
    T, E = slot_row.shape
    rows, d = Y.shape
    dev = Y.device
    out = torch.empty((T, d), dtype=Y.dtype, device=dev)
    _check(lib.moe_tr_combine(_dev(Y, "Y"), _dev(slot_row, "slot_row", torch.int32),
                              _dev(slot_w, "slot_w", torch.float32), dtype_code(Y.dtype), T, E, d, rows,
                              out.data_ptr(), _stream(dev)), "moe_tr_combine")
    return out


class ForwardTRPlan:
    """Preallocated outputs and workspace for repeated moe_forward_tr calls on one shape."""

    def __init__(self, T: int, d: int, E: int, K: int, n: int, M: int, dtype: torch.dtype, device,
                 cap_tiles: int = 0):
        lib = load_library()
        self.T, self.d, self.E, self.K, self.n, self.M, self.cap_tiles = T, d, E, K, n, M, cap_tiles
        self.dtype = dtype
        self.device = torch.device(device)
        self.ws_bytes = lib.moe_forward_tr_workspace_bytes(T, d, E, K, n, M, dtype_code(dtype))
        self.max_rows = lib.moe_token_round_max_rows(T, E, K, M)
        if self.ws_bytes == 0 or self.max_rows <= 0:
            raise MoEError(MOE_ERR_UNSUPPORTED, "moe_forward_tr_workspace_bytes", lib.moe_last_error().decode())
        dev = self.device
        self.ws = _workspace(self.ws_bytes, dev)
        self.out = torch.empty((T, d), dtype=dtype, device=dev)
        self.counts_r = torch.empty(E, dtype=torch.int32, device=dev)
        self.offsets_r = torch.empty(E + 1, dtype=torch.int32, device=dev)
        self.row_tok = torch.empty(self.max_rows, dtype=torch.int32, device=dev)
        self.slot_row = torch.empty((T, E), dtype=torch.int32, device=dev)
        self.slot_w = torch.empty((T, E), dtype=torch.float32, device=dev)

    def __call__(self, X, logits, W1, W3, W2):
        lib = load_library()
        dt = self.dtype
        _check(lib.moe_forward_tr(_dev(X, "X", dt), _dev(logits, "logits", torch.float32), _dev(W1, "W1", dt),
                                  _dev(W3, "W3", dt), _dev(W2, "W2", dt), dtype_code(dt), self.T, self.d, self.E,
                                  self.K, self.n, self.M, self.cap_tiles, self.out.data_ptr(),
                                  self.counts_r.data_ptr(), self.offsets_r.data_ptr(), self.row_tok.data_ptr(),
                                  self.slot_row.data_ptr(), self.slot_w.data_ptr(), self.ws.data_ptr(),
                                  self.ws_bytes, _stream(self.device)), "moe_forward_tr")
        return self.out


def moe_forward_tr(X: torch.Tensor, logits: torch.Tensor, W1: torch.Tensor, W3: torch.Tensor, W2: torch.Tensor,
                   K: int, M: int = 256, cap_tiles: int = 0):
    """Whole layer with Token Rounding.  Returns (out [T,d], plan)."""
    T, d = X.shape
    E, _, n = W1.shape
    plan = ForwardTRPlan(T, d, E, K, n, M, X.dtype, X.device, cap_tiles)
    plan(X, logits, W1, W3, W2)
    return plan.out, plan


def moe_backward_data(X: torch.Tensor, logits: torch.Tensor, W1: torch.Tensor, W3: torch.Tensor, W2: torch.Tensor,
                      K: int, dout: torch.Tensor, ws: torch.Tensor | None = None):
    """Data gradients of the layer: dX [T,d] (dtype of X) and dlogits [T,E] f32 given dout [T,d];
    also dw [T,K] f32, the gradient of the renormalised routing weights.  Returns a dict."""
    lib = load_library()
    T, d = X.shape
    E, _, n = W1.shape
    dt = X.dtype
    dev = X.device
    nws = lib.moe_backward_data_workspace_bytes(T, d, E, K, n, dtype_code(dt))
    if nws == 0:
        raise MoEError(MOE_ERR_UNSUPPORTED, "moe_backward_data_workspace_bytes", lib.moe_last_error().decode())
    if ws is None:
        ws = _workspace(nws, dev)
    r = {"dX": torch.empty((T, d), dtype=dt, device=dev),
         "dlogits": torch.empty((T, E), dtype=torch.float32, device=dev),
         "dw": torch.empty((T, K), dtype=torch.float32, device=dev)}
    _check(lib.moe_backward_data(_dev(X, "X", dt), _dev(logits, "logits", torch.float32), _dev(W1, "W1", dt),
                                 _dev(W3, "W3", dt), _dev(W2, "W2", dt), dtype_code(dt), T, d, E, K, n,
                                 _dev(dout, "dout", dt), r["dX"].data_ptr(), r["dlogits"].data_ptr(),
                                 r["dw"].data_ptr(), _dev(ws, "ws"), ws.numel(), _stream(dev)), "moe_backward_data")
    return r


def moe_backward(X: torch.Tensor, logits: torch.Tensor, W1: torch.Tensor, W3: torch.Tensor, W2: torch.Tensor,
                 K: int, dout: torch.Tensor, ws: torch.Tensor | None = None):
    """moe_backward_data plus the expert-weight gradients dW1, dW3 [E,d,n] and dW2 [E,n,d] (f32).
    Returns a dict with dX, dlogits, dw, dW1, dW3, dW2."""
    lib = load_library()
    T, d = X.shape
    E, _, n = W1.shape
    dt = X.dtype
    dev = X.device
    nws = lib.moe_backward_workspace_bytes(T, d, E, K, n, dtype_code(dt))
    if nws == 0:
        raise MoEError(MOE_ERR_UNSUPPORTED, "moe_backward_workspace_bytes", lib.moe_last_error().decode())
    if ws is None:
        ws = _workspace(nws, dev)
    f32 = torch.float32
    r = {"dX": torch.empty((T, d), dtype=dt, device=dev), "dlogits": torch.empty((T, E), dtype=f32, device=dev),
         "dw": torch.empty((T, K), dtype=f32, device=dev), "dW1": torch.empty((E, d, n), dtype=f32, device=dev),
         "dW3": torch.empty((E, d, n), dtype=f32, device=dev), "dW2": torch.empty((E, n, d), dtype=f32, device=dev)}
    _check(lib.moe_backward(_dev(X, "X", dt), _dev(logits, "logits", f32), _dev(W1, "W1", dt), _dev(W3, "W3", dt),
                            _dev(W2, "W2", dt), dtype_code(dt), T, d, E, K, n, _dev(dout, "dout", dt),
                            r["dX"].data_ptr(), r["dlogits"].data_ptr(), r["dw"].data_ptr(), r["dW1"].data_ptr(),
                            r["dW3"].data_ptr(), r["dW2"].data_ptr(), _dev(ws, "ws"), ws.numel(), _stream(dev)),
           "moe_backward")
    return r
