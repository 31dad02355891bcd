"""C-ABI checks that need no GPU: the library loads, exports every function
include/moe.h declares, and rejects bad arguments before launching anything.
Every call here carries at least one invalid argument, so no kernel is ever
launched (the fake pointers are never dereferenced)."""
import ctypes

import pytest

import mixture_experts_routing_gate_amd as moe

OK, INVALID, UNSUPPORTED, WORKSPACE, HIP = range(5)
P = 4096  # an aligned, never-dereferenced stand-in pointer


@pytest.fixture(scope="module")
def lib():
    return moe.load_library()


def test_exports_every_declared_function(lib):
    names = moe.header_functions()
    assert {"moe_route", "moe_permute", "moe_grouped_ffn", "moe_combine", "moe_forward"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings(lib):
    assert lib.moe_status_string(OK) == b"ok"
    for s in (INVALID, UNSUPPORTED, WORKSPACE, HIP):
        assert lib.moe_status_string(s) not in (b"ok", b"unknown status")
    assert lib.moe_status_string(99) == b"unknown status"


def test_workspace_sizes(lib):
    assert lib.moe_route_workspace_bytes(262144, 128, 8) == 256 * 128 * 4  # 256 chunks of 1024 tokens
    assert lib.moe_route_workspace_bytes(2048, 8, 2) == 256                 # 8 chunks, 256-byte aligned
    assert lib.moe_route_workspace_bytes(0, 8, 2) == 0
    assert lib.moe_route_workspace_bytes(16, 8, 9) == 0
    assert lib.moe_permute_workspace_bytes(8192, 8, 2) >= 2 * 32 * 8 * 4
    # forward holds Y and Act at least; Xp only where the SwiGLU GEMM cannot gather X rows
    # (bf16 with d % 256 == 0 gathers; d % 256 == 128 and fp32 take the permuted copy)
    T, d, E, K, n = 8192, 4096, 8, 2, 14336
    A = T * K
    gathered = lib.moe_forward_workspace_bytes(T, d, E, K, n, moe.MOE_BF16)
    assert A * (d + n) * 2 <= gathered < A * (2 * d + n) * 2
    copied = lib.moe_forward_workspace_bytes(T, d + 128, E, K, n, moe.MOE_BF16)
    assert copied >= A * (2 * (d + 128) + n) * 2
    assert lib.moe_forward_workspace_bytes(256, 128, 8, 2, 256, moe.MOE_F32) >= 512 * (2 * 128 + 256) * 4
    # one workspace for every forward-path call
    for args in ((T, d, E, K, n, moe.MOE_BF16), (256, 128, 8, 2, 256, moe.MOE_F32), (70001, 256, 256, 2, 128, 1)):
        Tt, dd, Ee, Kk, nn, dt = args
        allw = lib.moe_workspace_bytes(*args)
        assert allw >= lib.moe_forward_workspace_bytes(*args) > 0
        assert allw >= lib.moe_route_workspace_bytes(Tt, Ee, Kk)
        assert allw >= lib.moe_permute_workspace_bytes(Tt, Ee, Kk)
        assert allw >= lib.moe_ffn_workspace_bytes(dd, nn, dt)
    assert lib.moe_workspace_bytes(T, 100, E, K, n, moe.MOE_BF16) == 0
    assert lib.moe_forward_workspace_bytes(T, 100, E, K, n, moe.MOE_BF16) == 0  # d not a multiple of 128
    assert lib.moe_forward_workspace_bytes(T, d, E, K, n, 7) == 0               # unknown dtype


@pytest.mark.parametrize("T,E,K,code", [
    (0, 8, 2, INVALID), (16, 0, 1, INVALID), (16, 8, 0, INVALID), (16, 8, 9, INVALID),
    (16, 300, 2, UNSUPPORTED), (16, 16, 9, UNSUPPORTED), (2 ** 29, 8, 8, UNSUPPORTED)])
def test_route_rejects_sizes(lib, T, E, K, code):
    assert lib.moe_route(P, T, E, K, P, P, P, P, P, 1 << 30, None) == code
    assert lib.moe_last_error()


def test_route_rejects_pointers_and_workspace(lib):
    assert lib.moe_route(None, 16, 8, 2, P, P, P, P, P, 1 << 20, None) == INVALID
    assert lib.moe_route(P + 4, 16, 8, 2, P, P, P, P, P, 1 << 20, None) == INVALID  # misaligned
    assert lib.moe_route(P, 16, 8, 2, P, None, P, P, P, 1 << 20, None) == INVALID
    assert lib.moe_route(P, 16, 8, 2, P, P, P, P, None, 0, None) == WORKSPACE
    assert lib.moe_route(P, 16, 8, 2, P, P, P, P, P, 4, None) == WORKSPACE
    assert b"workspace" in lib.moe_last_error()


def test_permute_rejects(lib):
    ws = lib.moe_permute_workspace_bytes(16, 8, 2)
    assert lib.moe_permute(P, 1, 16, 128, 8, 2, P, P, P, None, P, ws, None) == INVALID
    assert lib.moe_permute(P, 5, 16, 128, 8, 2, P, P, P, P, P, ws, None) == UNSUPPORTED
    assert lib.moe_permute(P, 1, 16, 12, 8, 2, P, P, P, P, P, ws, None) == UNSUPPORTED  # 24-byte rows
    assert lib.moe_permute(P, 1, 16, 128, 8, 2, P, P, P, P, P, ws - 1, None) == WORKSPACE


def test_grouped_ffn_rejects(lib):
    args = dict(Xp=P, W1=P, W3=P, W2=P, dt=1, T=16, d=128, E=8, K=2, n=128, c=P, o=P, act=P, y=P)

    def call(**kw):
        a = dict(args, **kw)
        return lib.moe_grouped_ffn(a["Xp"], a["W1"], a["W3"], a["W2"], a["dt"], a["T"], a["d"], a["E"],
                                   a["K"], a["n"], a["c"], a["o"], a["act"], a["y"], a.get("ws"),
                                   a.get("wsb", 0), None)
    assert call(W3=None) == INVALID
    assert call(d=192) == UNSUPPORTED          # bf16 needs multiples of 128
    assert call(n=0) == INVALID
    assert call(dt=0, d=192, n=64, c=None) == INVALID
    assert call(K=3, E=2) == INVALID
    # the optional split workspace: NULL is fine, a too small one is rejected
    assert lib.moe_ffn_workspace_bytes(256, 128, 1) > 0
    assert lib.moe_ffn_workspace_bytes(64, 64, 0) == 0
    assert call(d=256, ws=P, wsb=4) == WORKSPACE


def test_combine_and_forward_reject(lib):
    assert lib.moe_combine(P, P, None, 1, 16, 128, 2, P, None) == INVALID
    assert lib.moe_combine(P, P, P, 1, 16, 128, 9, P, None) == UNSUPPORTED
    assert lib.moe_combine(P, P, P, 1, 0, 128, 2, P, None) == INVALID
    ws = lib.moe_forward_workspace_bytes(16, 128, 8, 2, 128, 1)
    base = [P, P, P, P, P, 1, 16, 128, 8, 2, 128, P, None, None, None, None, None, None]
    assert lib.moe_forward(*base, P, ws - 256, None) == WORKSPACE
    bad = list(base)
    bad[13] = P + 8  # misaligned optional output
    assert lib.moe_forward(*bad, P, ws, None) == INVALID
    bad = list(base)
    bad[1] = None
    assert lib.moe_forward(*bad, P, ws, None) == INVALID


def test_router_workspace_and_rejections(lib):
    assert lib.moe_router_workspace_bytes(4096, 8, 1) == 2 * 32 * 4096 * 2     # E padded to 32
    # E a multiple of 128: hi and lo [d, E], 256 bytes of schedule, and the split
    # slots of the grouped GEMM's kernel that then runs the projection
    assert lib.moe_router_workspace_bytes(7168, 256, 1) == \
        2 * 256 * 7168 * 2 + 256 + lib.moe_ffn_workspace_bytes(7168, 256, 1)
    assert lib.moe_router_workspace_bytes(4096, 128, 1) == \
        2 * 128 * 4096 * 2 + 256 + lib.moe_ffn_workspace_bytes(4096, 128, 1)
    assert lib.moe_router_workspace_bytes(1536, 128, 1) == 2 * 128 * 1536 * 2   # d < 4096: transposed only
    assert lib.moe_router_workspace_bytes(4096, 192, 1) == 2 * 192 * 4096 * 2   # E % 128 != 0
    assert lib.moe_router_workspace_bytes(1536, 40, 1) == 2 * 64 * 1536 * 2    # E padded to 64
    assert lib.moe_router_workspace_bytes(128, 8, 0) == 0                      # fp32: no split
    assert lib.moe_router_workspace_bytes(384, 8, 1) == 0                      # d % 256 != 0: no split
    assert lib.moe_router_workspace_bytes(4096, 257, 1) == 0
    wsb = lib.moe_router_workspace_bytes(4096, 8, 1)
    assert lib.moe_router(P, 1, 0, 4096, 8, P, None, P, P, wsb, None) == INVALID      # T = 0
    assert lib.moe_router(P, 1, 16, 4096, 0, P, None, P, P, wsb, None) == INVALID     # E = 0
    assert lib.moe_router(P, 1, 16, 4096, 300, P, None, P, P, wsb, None) == UNSUPPORTED
    assert lib.moe_router(None, 1, 16, 4096, 8, P, None, P, P, wsb, None) == INVALID  # X NULL
    assert lib.moe_router(P, 1, 16, 4096, 8, None, None, P, P, wsb, None) == INVALID  # Wr NULL
    assert lib.moe_router(P, 1, 16, 4096, 8, P, None, None, P, wsb, None) == INVALID  # logits NULL
    assert lib.moe_router(P, 1, 16, 4096, 8, P, None, P, None, 0, None) == WORKSPACE
    assert lib.moe_router(P, 1, 16, 4096, 8, P, None, P, P, wsb - 1, None) == WORKSPACE
    assert lib.moe_router(P + 8, 1, 16, 4096, 8, P, None, P, P, wsb, None) == INVALID  # X misaligned
    assert lib.moe_router(P, 7, 16, 4096, 8, P, None, P, P, wsb, None) == UNSUPPORTED  # dtype


def test_token_round_sizes_and_rejections(lib):
    # an expert rounds up by at most floor(M/2) rows and holds a token at most once
    assert lib.moe_token_round_max_rows(8192, 8, 2, 256) == 8192 * 2 + 8 * 128
    assert lib.moe_token_round_max_rows(100, 4, 2, 256) == 100 * 4
    assert lib.moe_token_round_max_rows(16, 8, 2, 0) == 0
    assert lib.moe_token_round_workspace_bytes(8192, 8, 2, 256) >= 8192 * 8 * 9
    assert lib.moe_token_round_workspace_bytes(16, 8, 9, 4) == 0
    R = lib.moe_token_round_max_rows(16, 8, 2, 4)
    good = [P, P, P, 16, 8, 2, 4, 0, P, P, P, R, P, P, P, 1 << 20, None]

    def call(**kw):
        a = list(good)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return lib.moe_token_round(*a)

    assert call(a6=0) == INVALID            # M
    assert call(a6=70000) == UNSUPPORTED
    assert call(a7=-1) == INVALID           # cap_tiles
    assert call(a11=R - 1) == INVALID       # row_tok too small
    assert call(a0=None) == INVALID
    assert call(a2=None) == INVALID         # counts
    assert call(a13=P + 4) == INVALID       # misaligned slot_row
    assert call(a15=0) == WORKSPACE
    assert call(a4=300) == UNSUPPORTED      # E
    assert lib.moe_last_error()


def test_tr_combine_and_forward_tr_reject(lib):
    assert lib.moe_tr_combine(P, P, P, moe.MOE_BF16, 0, 8, 128, 10, P, None) == INVALID
    assert lib.moe_tr_combine(P, P, P, moe.MOE_BF16, 16, 300, 128, 10, P, None) == UNSUPPORTED
    assert lib.moe_tr_combine(P, P, P, moe.MOE_BF16, 16, 8, 100, 10, P, None) == UNSUPPORTED  # row of 200 bytes
    assert lib.moe_tr_combine(P, P, P, moe.MOE_BF16, 16, 8, 128, -1, P, None) == INVALID
    assert lib.moe_tr_combine(P, None, P, moe.MOE_BF16, 16, 8, 128, 10, P, None) == INVALID
    T, d, E, K, n, M = 8192, 4096, 8, 2, 14336, 256
    R = lib.moe_token_round_max_rows(T, E, K, M)
    assert lib.moe_forward_tr_workspace_bytes(T, d, E, K, n, M, moe.MOE_BF16) >= R * (d + n) * 2
    assert lib.moe_forward_tr_workspace_bytes(T, d, E, K, n, 0, moe.MOE_BF16) == 0
    args = [P, P, P, P, P, moe.MOE_BF16, T, d, E, K, n, M, 0, P, None, None, None, None, None, P, 0, None]
    assert lib.moe_forward_tr(*args) == WORKSPACE
    args[11] = 0
    assert lib.moe_forward_tr(*args) == INVALID
