"""Guard canaries around every output and workspace of the layer's entry points.

Each output and workspace buffer is carved from the middle of a larger device
buffer whose margins (1 MiB on each side) hold seeded random bytes; the
interior starts filled with the same kind of bytes.  After the call the margins
must be unchanged, the inputs must equal their copies, and every output must
equal, bit for bit, what the same entry point writes into plain buffers (the
kernels are deterministic), so a stray store past an output, a store into an
input, and an element left unwritten all fail.  The configs take the kernels'
edge paths: short last tiles (at most 32, 64 or 128 rows), ragged tails,
empty experts, the split tail and per-XCD tile claiming (with the optional
grouped-GEMM workspace), the gathered X rows of moe_forward and moe_forward_tr,
the 128 x 128 kernel (d % 256 != 0) and the fp32 kernels, and both router
projection paths (the register-tiled kernel and the grouped GEMM's kernel with
every tile split along K).  These are ordinary runs of the kernels on valid
inputs; nothing is made to fault."""
import ctypes

import numpy as np
import pytest
import torch

import mixture_experts_routing_gate_amd as moe
import synth

pytestmark = pytest.mark.gpu

MARGIN = 1 << 20
_gen = torch.Generator(device="cpu").manual_seed(1234)


class Guarded:
    """`nbytes` of device memory at a 256-byte aligned offset inside a buffer
    with MARGIN bytes of seeded random guard bytes on each side."""

    def __init__(self, nbytes: int, dev):
        self.nbytes = max(int(nbytes), 16)
        self.size = (self.nbytes + 255) // 256 * 256
        total = 2 * MARGIN + self.size
        host = torch.randint(0, 256, (total,), dtype=torch.uint8, generator=_gen)
        self.buf = host.to(dev)
        self.lo = host[:MARGIN].clone()
        self.hi = host[MARGIN + self.size:].clone()

    @property
    def ptr(self) -> int:
        return self.buf.data_ptr() + MARGIN

    def view(self, dtype, shape):
        n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        return self.buf[MARGIN:MARGIN + n].view(dtype).view(*shape)

    def check(self, what: str):
        h = self.buf.cpu()
        lo_bad = int((h[:MARGIN] != self.lo).sum())
        hi_bad = int((h[MARGIN + self.size:] != self.hi).sum())
        assert lo_bad == 0 and hi_bad == 0, f"{what}: {lo_bad} bytes changed before it, {hi_bad} after it"


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ok(status, lib, name):
    assert status == 0, f"{name}: status {status}: {lib.moe_last_error().decode()}"


def _inputs(cfg):
    inp = synth.make_inputs(cfg, "cpu", 0)
    return {k: v.to("cuda").contiguous() for k, v in inp.items()}


def _inputs_unchanged(g, copies):
    for k, v in g.items():
        assert torch.equal(v.view(torch.uint8) if v.dtype != torch.uint8 else v,
                           copies[k].view(torch.uint8) if copies[k].dtype != torch.uint8 else copies[k]), \
            f"input {k} was written"


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _same(a, b, what):
    assert torch.equal(_bits(a.contiguous()), _bits(b.contiguous())), f"{what} differs from the unguarded call"


CASES = [
    # E=64, about 60 rows per expert: short tiles of 32 and 64 rows, claiming on, some empty experts
    synth.MoEConfig("short_ragged", T=1000, d=256, E=64, K=4, n=128, logits="bias", bias_var=2.0),
    # about 512 rows per expert: whole 256-row tiles, ragged tails and a split tail round
    synth.MoEConfig("whole_tiles", T=2048, d=512, E=8, K=2, n=384),
    # skewed E=128 (empty experts, 128-row short tiles)
    synth.MoEConfig("fine_small", T=2048, d=256, E=128, K=4, n=128, logits="bias", bias_var=2.0),
    # d % 256 != 0: the 128 x 128 kernel and the explicit Xp copy
    synth.MoEConfig("tile128", T=700, d=384, E=16, K=2, n=128, logits="bias", bias_var=1.0),
    synth.MoEConfig("f32", T=333, d=192, E=8, K=3, n=128, dtype="f32", logits="bias", bias_var=2.0),
]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_forward_canaries(cfg):
    lib = moe.load_library()
    dev = torch.device("cuda")
    g = _inputs(cfg)
    copies = {k: v.clone() for k, v in g.items()}
    T, d, E, K, n = cfg.T, cfg.d, cfg.E, cfg.K, cfg.n
    A, s, dt = T * K, (4 if cfg.dtype == "f32" else 2), (0 if cfg.dtype == "f32" else 1)
    wsb = lib.moe_forward_workspace_bytes(T, d, E, K, n, dt)
    bufs = {"out": Guarded(T * d * s, dev), "topk_idx": Guarded(A * 4, dev), "topk_w": Guarded(A * 4, dev),
            "counts": Guarded(E * 4, dev), "offsets": Guarded((E + 1) * 4, dev), "sorted_pair": Guarded(A * 4, dev),
            "inv": Guarded(A * 4, dev), "ws": Guarded(wsb, dev)}
    b = {k: v.ptr for k, v in bufs.items()}
    _ok(lib.moe_forward(g["X"].data_ptr(), g["logits"].data_ptr(), g["W1"].data_ptr(), g["W3"].data_ptr(),
                        g["W2"].data_ptr(), dt, T, d, E, K, n, b["out"], b["topk_idx"], b["topk_w"], b["counts"],
                        b["offsets"], b["sorted_pair"], b["inv"], b["ws"], wsb, _stream()), lib, "moe_forward")
    torch.cuda.synchronize()
    for k, v in bufs.items():
        v.check(f"moe_forward {k}")
    _inputs_unchanged(g, copies)
    out, plan = moe.moe_forward(g["X"], g["logits"], g["W1"], g["W3"], g["W2"], K)
    torch.cuda.synchronize()
    _same(bufs["out"].view(cfg.torch_dtype, (T, d)), out, "out")
    for k, shape, tdt in (("topk_idx", (T, K), torch.int32), ("topk_w", (T, K), torch.float32),
                          ("counts", (E,), torch.int32), ("offsets", (E + 1,), torch.int32),
                          ("sorted_pair", (A,), torch.int32), ("inv", (A,), torch.int32)):
        _same(bufs[k].view(tdt, shape), getattr(plan, k), k)


@pytest.mark.parametrize("with_ws", [False, True], ids=["plain", "split_ws"])
@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_step_by_step_canaries(cfg, with_ws):
    """moe_route, moe_permute, moe_grouped_ffn (with and without its optional
    workspace) and moe_combine, each output and workspace guarded."""
    lib = moe.load_library()
    dev = torch.device("cuda")
    g = _inputs(cfg)
    copies = {k: v.clone() for k, v in g.items()}
    T, d, E, K, n = cfg.T, cfg.d, cfg.E, cfg.K, cfg.n
    A, s, dt = T * K, (4 if cfg.dtype == "f32" else 2), (0 if cfg.dtype == "f32" else 1)
    st = _stream()
    rws = lib.moe_route_workspace_bytes(T, E, K)
    pws = lib.moe_permute_workspace_bytes(T, E, K)
    fws = lib.moe_ffn_workspace_bytes(d, n, dt) if with_ws else 0
    bufs = {"idx": Guarded(A * 4, dev), "w": Guarded(A * 4, dev), "counts": Guarded(E * 4, dev),
            "offsets": Guarded((E + 1) * 4, dev), "route_ws": Guarded(rws, dev), "sp": Guarded(A * 4, dev),
            "inv": Guarded(A * 4, dev), "Xp": Guarded(A * d * s, dev), "perm_ws": Guarded(pws, dev),
            "Act": Guarded(A * n * s, dev), "Y": Guarded(A * d * s, dev), "out": Guarded(T * d * s, dev)}
    if fws:
        bufs["ffn_ws"] = Guarded(fws, dev)
    b = {k: v.ptr for k, v in bufs.items()}
    _ok(lib.moe_route(g["logits"].data_ptr(), T, E, K, b["idx"], b["w"], b["counts"], b["offsets"], b["route_ws"],
                      rws, st), lib, "moe_route")
    _ok(lib.moe_permute(g["X"].data_ptr(), dt, T, d, E, K, b["idx"], b["sp"], b["inv"], b["Xp"], b["perm_ws"], pws,
                        st), lib, "moe_permute")
    _ok(lib.moe_grouped_ffn(b["Xp"], g["W1"].data_ptr(), g["W3"].data_ptr(), g["W2"].data_ptr(), dt, T, d, E, K, n,
                            b["counts"], b["offsets"], b["Act"], b["Y"], b.get("ffn_ws"), fws, st),
        lib, "moe_grouped_ffn")
    _ok(lib.moe_combine(b["Y"], b["w"], b["inv"], dt, T, d, K, b["out"], st), lib, "moe_combine")
    torch.cuda.synchronize()
    for k, v in bufs.items():
        v.check(k)
    _inputs_unchanged(g, copies)
    # the same calls into plain buffers (the grouped GEMMs with the same split setting)
    idx, w, counts, offsets = moe.moe_route(g["logits"], K)
    sp, inv, Xp = moe.moe_permute(g["X"], idx, E)
    Act, Y = moe.moe_grouped_ffn(Xp, g["W1"], g["W3"], g["W2"], counts, offsets, K, split=with_ws)
    out = moe.moe_combine(Y, w, inv)
    torch.cuda.synchronize()
    for k, want, shape, tdt in (("idx", idx, (T, K), torch.int32), ("w", w, (T, K), torch.float32),
                                ("counts", counts, (E,), torch.int32), ("offsets", offsets, (E + 1,), torch.int32),
                                ("sp", sp, (A,), torch.int32), ("inv", inv, (A,), torch.int32),
                                ("Xp", Xp, (A, d), cfg.torch_dtype), ("Act", Act, (A, n), cfg.torch_dtype),
                                ("Y", Y, (A, d), cfg.torch_dtype), ("out", out, (T, d), cfg.torch_dtype)):
        _same(bufs[k].view(tdt, shape), want, k)


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_forward_tr_canaries(cfg):
    lib = moe.load_library()
    dev = torch.device("cuda")
    g = _inputs(cfg)
    copies = {k: v.clone() for k, v in g.items()}
    T, d, E, K, n, M = cfg.T, cfg.d, cfg.E, cfg.K, cfg.n, 64
    s, dt = (4 if cfg.dtype == "f32" else 2), (0 if cfg.dtype == "f32" else 1)
    R = lib.moe_token_round_max_rows(T, E, K, M)
    wsb = lib.moe_forward_tr_workspace_bytes(T, d, E, K, n, M, dt)
    bufs = {"out": Guarded(T * d * s, dev), "counts_r": Guarded(E * 4, dev), "offsets_r": Guarded((E + 1) * 4, dev),
            "row_tok": Guarded(R * 4, dev), "slot_row": Guarded(T * E * 4, dev), "slot_w": Guarded(T * E * 4, dev),
            "ws": Guarded(wsb, dev)}
    b = {k: v.ptr for k, v in bufs.items()}
    _ok(lib.moe_forward_tr(g["X"].data_ptr(), g["logits"].data_ptr(), g["W1"].data_ptr(), g["W3"].data_ptr(),
                           g["W2"].data_ptr(), dt, T, d, E, K, n, M, 0, b["out"], b["counts_r"], b["offsets_r"],
                           b["row_tok"], b["slot_row"], b["slot_w"], b["ws"], wsb, _stream()), lib, "moe_forward_tr")
    torch.cuda.synchronize()
    for k, v in bufs.items():
        v.check(f"moe_forward_tr {k}")
    _inputs_unchanged(g, copies)
    out, plan = moe.moe_forward_tr(g["X"], g["logits"], g["W1"], g["W3"], g["W2"], K, M, 0)
    torch.cuda.synchronize()
    _same(bufs["out"].view(cfg.torch_dtype, (T, d)), out, "out")
    _same(bufs["slot_row"].view(torch.int32, (T, E)), plan.slot_row, "slot_row")
    rows = int(plan.offsets_r[-1].item())
    _same(bufs["row_tok"].view(torch.int32, (R,))[:rows], plan.row_tok[:rows], "row_tok")


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_backward_canaries(cfg):
    lib = moe.load_library()
    dev = torch.device("cuda")
    g = _inputs(cfg)
    T, d, E, K, n = cfg.T, cfg.d, cfg.E, cfg.K, cfg.n
    s, dt = (4 if cfg.dtype == "f32" else 2), (0 if cfg.dtype == "f32" else 1)
    gen = torch.Generator(device="cpu").manual_seed(5)
    g["dout"] = torch.randn((T, d), generator=gen).to(cfg.torch_dtype).to(dev)
    copies = {k: v.clone() for k, v in g.items()}
    wsb = lib.moe_backward_workspace_bytes(T, d, E, K, n, dt)
    bufs = {"dX": Guarded(T * d * s, dev), "dlogits": Guarded(T * E * 4, dev), "dw": Guarded(T * K * 4, dev),
            "dW1": Guarded(E * d * n * 4, dev), "dW3": Guarded(E * d * n * 4, dev), "dW2": Guarded(E * n * d * 4, dev),
            "ws": Guarded(wsb, dev)}
    b = {k: v.ptr for k, v in bufs.items()}
    _ok(lib.moe_backward(g["X"].data_ptr(), g["logits"].data_ptr(), g["W1"].data_ptr(), g["W3"].data_ptr(),
                         g["W2"].data_ptr(), dt, T, d, E, K, n, g["dout"].data_ptr(), b["dX"], b["dlogits"], b["dw"],
                         b["dW1"], b["dW3"], b["dW2"], b["ws"], wsb, _stream()), lib, "moe_backward")
    torch.cuda.synchronize()
    for k, v in bufs.items():
        v.check(f"moe_backward {k}")
    _inputs_unchanged(g, copies)
    r = moe.moe_backward(g["X"], g["logits"], g["W1"], g["W3"], g["W2"], K, g["dout"])
    torch.cuda.synchronize()
    for k, shape, tdt in (("dX", (T, d), cfg.torch_dtype), ("dlogits", (T, E), torch.float32),
                          ("dw", (T, K), torch.float32), ("dW1", (E, d, n), torch.float32),
                          ("dW3", (E, d, n), torch.float32), ("dW2", (E, n, d), torch.float32)):
        _same(bufs[k].view(tdt, shape), r[k], k)


ROUTER_CASES = [
    # (T, d, E, bias variance): the grouped GEMM's kernel (E % 128 == 0, d >= 4096),
    # with two token tiles (one short, claimed, 32 parts each) and with 16 tiles
    (300, 4096, 128, 0.5),
    (2000, 4096, 256, 1.5),
    # the LDS-staged tile kernel (E > 64 with a short d; a half-empty expert
    # group), the register-tiled kernel (E padded to 64), and the staged E <= 32
    # kernel (a ragged last token tile)
    (1000, 1536, 128, 2.0),
    (130, 512, 96, 0.5),
    (700, 512, 40, 1.0),
    (77, 768, 20, 0.0),
]


@pytest.mark.parametrize("T,d,E,bv", ROUTER_CASES, ids=lambda v: str(v))
def test_router_canaries(T, d, E, bv):
    """moe_router: the logits and the workspace guarded, X, Wr and the bias
    unchanged, the logits equal to an unguarded call's bit for bit."""
    lib = moe.load_library()
    dev = torch.device("cuda")
    cfg = synth.MoEConfig("r", T=T, d=d, E=E, K=1, n=128, logits="proj_bias" if bv else "proj", bias_var=bv)
    X = synth._normal((T, d), 1.0, torch.bfloat16, torch.device("cpu"), synth._gen("cpu", 3, "X")).to(dev)
    Wr, b = synth.make_router(cfg, "cpu", 3)
    g = {"X": X, "Wr": Wr.to(dev)}
    if b is not None:
        g["bias"] = b.to(dev)
    copies = {k: v.clone() for k, v in g.items()}
    wsb = lib.moe_router_workspace_bytes(d, E, 1)
    bufs = {"logits": Guarded(T * E * 4, dev), "ws": Guarded(wsb, dev)}
    _ok(lib.moe_router(g["X"].data_ptr(), 1, T, d, E, g["Wr"].data_ptr(),
                       g["bias"].data_ptr() if "bias" in g else None, bufs["logits"].ptr, bufs["ws"].ptr, wsb,
                       _stream()), lib, "moe_router")
    torch.cuda.synchronize()
    for k, v in bufs.items():
        v.check(f"moe_router {k}")
    _inputs_unchanged(g, copies)
    ref = moe.moe_router(g["X"], g["Wr"], g.get("bias"))
    torch.cuda.synchronize()
    _same(bufs["logits"].view(torch.float32, (T, E)), ref, "logits")


@pytest.mark.parametrize("T,d,E,K,bv", [(1000, 512, 40, 4, 1.0), (333, 1024, 8, 2, 0.0), (600, 4096, 256, 8, 1.5),
                                          (77, 768, 20, 3, 0.5)],
                         ids=lambda v: str(v))
def test_route_x_canaries(T, d, E, K, bv):
    """moe_route_x (fused router-gate for E <= 64, router then gate above):
    logits, routing outputs and workspace guarded, equal to an unguarded call."""
    lib = moe.load_library()
    dev = torch.device("cuda")
    cfg = synth.MoEConfig("rx", T=T, d=d, E=E, K=K, n=128, logits="proj_bias" if bv else "proj", bias_var=bv)
    X = synth._normal((T, d), 1.0, torch.bfloat16, torch.device("cpu"), synth._gen("cpu", 5, "X")).to(dev)
    Wr, b = synth.make_router(cfg, "cpu", 5)
    g = {"X": X, "Wr": Wr.to(dev)}
    if b is not None:
        g["bias"] = b.to(dev)
    copies = {k: v.clone() for k, v in g.items()}
    wsb = lib.moe_route_x_workspace_bytes(T, d, E, K, 1)
    A = T * K
    bufs = {"logits": Guarded(T * E * 4, dev), "idx": Guarded(A * 4, dev), "w": Guarded(A * 4, dev),
            "counts": Guarded(E * 4, dev), "offsets": Guarded((E + 1) * 4, dev), "ws": Guarded(wsb, dev)}
    bb = {k: v.ptr for k, v in bufs.items()}
    _ok(lib.moe_route_x(g["X"].data_ptr(), 1, T, d, E, K, g["Wr"].data_ptr(),
                        g["bias"].data_ptr() if "bias" in g else None, bb["logits"], bb["idx"], bb["w"],
                        bb["counts"], bb["offsets"], bb["ws"], wsb, _stream()), lib, "moe_route_x")
    torch.cuda.synchronize()
    for k, v in bufs.items():
        v.check(f"moe_route_x {k}")
    _inputs_unchanged(g, copies)
    idx, w, counts, offsets, lg = moe.moe_route_x(g["X"], g["Wr"], g.get("bias"), K)
    torch.cuda.synchronize()
    for k, want, shape, tdt in (("logits", lg, (T, E), torch.float32), ("idx", idx, (T, K), torch.int32),
                                ("w", w, (T, K), torch.float32), ("counts", counts, (E,), torch.int32),
                                ("offsets", offsets, (E + 1,), torch.int32)):
        _same(bufs[k].view(tdt, shape), want, k)

