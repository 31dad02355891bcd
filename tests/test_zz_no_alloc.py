"""moe_route_noalloc (the route entry point on the library's static device
scratch) against moe_route (the same kernels on a caller workspace), through
the C ABI: two calls in a row, the second on a smaller input, so that the
second runs over scratch the first left dirty.  Indices, counts and offsets
bit-exact; gate weights within 1e-5 relative (they come from the same
kernels, so they are expected to be identical)."""
import ctypes

import numpy as np
import pytest
import torch

import mixture_experts_routing_gate_amd as moe
import synth

pytestmark = pytest.mark.gpu

MOE_OK, MOE_ERR_UNSUPPORTED = 0, 2


def _outputs(T, E, K, dev):
    return (torch.full((T, K), -7, dtype=torch.int32, device=dev), torch.full((T, K), -7.0, device=dev),
            torch.full((E,), -7, dtype=torch.int32, device=dev), torch.full((E + 1,), -7, dtype=torch.int32, device=dev))


def _call_noalloc(lib, lg, K, out, stream):
    T, E = lg.shape
    idx, w, counts, offsets = out
    return lib.moe_route_noalloc(lg.data_ptr(), T, E, K, idx.data_ptr(), w.data_ptr(), counts.data_ptr(),
                                 offsets.data_ptr(), ctypes.c_void_p(stream))


def _call_route(lib, lg, K, out, stream):
    T, E = lg.shape
    idx, w, counts, offsets = out
    nws = lib.moe_route_workspace_bytes(T, E, K)
    ws = torch.empty(nws, dtype=torch.uint8, device=lg.device)
    st = lib.moe_route(lg.data_ptr(), T, E, K, idx.data_ptr(), w.data_ptr(), counts.data_ptr(), offsets.data_ptr(),
                       ws.data_ptr(), nws, ctypes.c_void_p(stream))
    return st, ws


def _compare(a, b, what):
    for name, x, y in zip(("topk_idx", "topk_w", "counts", "offsets"), a, b):
        xh, yh = x.cpu().numpy(), y.cpu().numpy()
        if name == "topk_w":
            assert np.all(np.abs(xh.astype(np.float64) - yh) <= 1e-5 * np.abs(yh.astype(np.float64))), (what, name)
        else:
            assert np.array_equal(xh, yh), (what, name, np.argwhere(xh != yh)[:4])


def test_noalloc_matches_route_two_calls():
    lib = moe.load_library()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev).cuda_stream
    # first the large gate workload (256 chunks of 1024 tokens x 128 experts in the
    # scratch), then a smaller one with a different chunk size and expert count
    cases = [synth.CONFIGS["gate_l"], synth.MoEConfig("small", T=3000, d=0, E=16, K=4, n=0, dtype="f32", gate_only=True)]
    for cfg in cases:
        print(f"[noalloc] T={cfg.T} E={cfg.E} K={cfg.K}", flush=True)
        lg = synth.make_inputs(cfg, dev, 0)["logits"]
        got = _outputs(cfg.T, cfg.E, cfg.K, dev)
        ref = _outputs(cfg.T, cfg.E, cfg.K, dev)
        assert _call_noalloc(lib, lg, cfg.K, got, stream) == MOE_OK, lib.moe_last_error()
        st, ws = _call_route(lib, lg, cfg.K, ref, stream)
        assert st == MOE_OK, lib.moe_last_error()
        torch.cuda.synchronize()
        _compare(got, ref, f"T={cfg.T} E={cfg.E} K={cfg.K}")
        assert int(got[3][-1].item()) == cfg.T * cfg.K
        del ws


def test_noalloc_rejects_sizes_beyond_the_scratch():
    lib = moe.load_library()
    # 2048 chunks of 1024 tokens x 256 experts = 2 MiB of counts, above the 1 MiB scratch;
    # rejected before any launch (the pointers are never dereferenced)
    P = 4096
    assert lib.moe_route_noalloc(P, 1 << 21, 256, 8, P, P, P, P, None) == MOE_ERR_UNSUPPORTED
    assert b"scratch" in lib.moe_last_error()
