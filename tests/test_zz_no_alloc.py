"""The allocation-free layer entry point (moe_prefill_run_layer_noalloc) against
the handle-based moe_prefill_run_layer it varies: same kernels, with the
library's static per-device scratch array as the workspace.  Two calls in a row
(the second with fewer tokens, other inputs and other dimensions follow), each
compared with the handle-based call on the same inputs -- every exported
intermediate and y bit for bit, y also against the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import moe_prefill_ffn_amd as mp
import oracle
import workload as wl

SCRATCH_BYTES = 128 << 20
EXPORTS = ("eidx", "counts", "bounds", "rows", "pos", "xq", "dx", "hq", "dh", "dm")


def _raw_noalloc(d, f, E, k, T, workspace=0, ptr=0x100000):
    """Direct C call with placeholder device pointers: only for requests the host
    checks refuse before anything touches the device."""
    p = mp.moe_prefill_params_t()
    p.struct_size = ctypes.sizeof(p)
    p.d_model, p.d_ff, p.n_experts, p.top_k, p.max_tokens = d, f, E, k, T
    p.workspace = workspace
    io = mp.moe_layer_io_t()
    io.struct_size = ctypes.sizeof(io)
    io.layer = -1
    io.n_tokens = T
    io.weights_dev = io.x = io.logits = io.y = ptr
    rc = mp.lib().moe_prefill_run_layer_noalloc(ctypes.byref(p), ctypes.byref(io), None)
    return rc, mp.moe_prefill_last_error(None)


def test_noalloc_refuses_a_layer_above_the_scratch_on_the_host():
    # T=8192, d=4096, f=1536, E=256, top-8 needs about 1.2 GiB of workspace
    need = mp.moe_prefill_workspace_size(4096, 1536, 256, 8, 8192)
    assert need > SCRATCH_BYTES
    rc, msg = _raw_noalloc(4096, 1536, 256, 8, 8192)
    assert rc == mp.MOE_EINVAL and "static scratch" in msg
    rc, msg = _raw_noalloc(2048, 768, 128, 8, 1024, workspace=0x200000)
    assert rc == mp.MOE_EINVAL and "workspace must be NULL" in msg
    rc, _ = _raw_noalloc(2048, 768, 128, 8, 0)        # no tokens: nothing to do
    assert rc == mp.MOE_OK


def _inputs(w, layer, T):
    x = np.ascontiguousarray(wl.layer_activations(w, layer)[:T])
    lg = np.ascontiguousarray(wl.layer_logits(w, layer)[:T])
    return x, lg


def _exports(w, T):
    ex = {}
    for name in EXPORTS:
        from gpu_helpers import EXPORT_SHAPES
        shp, dt = EXPORT_SHAPES[name](w, T)
        ex[name] = torch.full(shp, -7, dtype=dt, device="cuda") if not dt.is_floating_point else \
            torch.full(shp, float("nan"), dtype=dt, device="cuda")
    return ex


@pytest.mark.gpu
def test_noalloc_equals_run_layer_on_consecutive_calls():
    from gpu_helpers import ExpertCache, assert_close, assert_equal, host_blob, say

    big = wl.WORKLOADS["resident"]          # T=1024, d=2048, f=768, E=128, top-8
    tiny = wl.WORKLOADS["tiny"]
    blob_big = host_blob(big, ExpertCache(big, 0, keep=False)).cuda()
    ex_tiny = ExpertCache(tiny, 0)
    blob_tiny = host_blob(tiny, ex_tiny).cuda()
    h_big = mp.moe_prefill_create(big.d, big.f, big.E, big.k, big.T)
    h_tiny = mp.moe_prefill_create(tiny.d, tiny.f, tiny.E, tiny.k, tiny.T)
    # the first call at the full size, the second with fewer tokens and other inputs, then
    # other dimensions (another scratch layout), then the full size again
    calls = [(big, h_big, blob_big, 0, big.T), (big, h_big, blob_big, 1, 300),
             (tiny, h_tiny, blob_tiny, 0, tiny.T), (big, h_big, blob_big, 2, 777)]
    for w, h, blob, layer, T in calls:
        say(f"[case] noalloc {w.name} inputs of layer {layer}, T={T}")
        assert mp.moe_prefill_workspace_size(w.d, w.f, w.E, w.k, T) <= SCRATCH_BYTES
        x, lg = _inputs(w, layer, T)
        xt, lt = torch.from_numpy(x).cuda(), torch.from_numpy(lg).cuda()
        y_ref = torch.full((T, w.d), float("nan"), device="cuda")
        ex_ref = _exports(w, T)
        mp.moe_prefill_run_layer(h, xt, lt, y_ref, weights=blob, exports=ex_ref)
        y = torch.full((T, w.d), float("nan"), device="cuda")
        ex = _exports(w, T)
        mp.moe_prefill_run_layer_noalloc(w.d, w.f, w.E, w.k, xt, lt, y, blob, exports=ex)
        torch.cuda.synchronize()
        for name in EXPORTS:
            assert_equal(f"{name} (T={T})", ex[name].cpu().numpy(), ex_ref[name].cpu().numpy())
        assert_equal(f"y (T={T})", y.cpu().numpy(), y_ref.cpu().numpy())
        if w is tiny:
            assert_close("y vs oracle", y.cpu().numpy(), oracle.layer(x, lg, w.k, ex_tiny, w.f)["y"])
    h_big.close()
    h_tiny.close()


@pytest.mark.gpu
def test_noalloc_layer_captured_in_a_hip_graph_replays_exactly():
    """The callers this entry point is for include code under HIP graph capture: one
    resident layer captured once, replayed with new inputs copied into the captured
    buffers and eager work (the handle-based entry point) between the replays; every
    replay equals the eager run bit for bit."""
    from gpu_helpers import ExpertCache, host_blob, say

    w = wl.WORKLOADS["resident"]
    say("[case] noalloc layer under graph capture")
    T = 512
    blob = host_blob(w, ExpertCache(w, 0, keep=False)).cuda()
    xs = [torch.from_numpy(np.ascontiguousarray(wl.layer_activations(w, l)[:T])).cuda() for l in (0, 1, 2)]
    lgs = [torch.from_numpy(np.ascontiguousarray(wl.layer_logits(w, l)[:T])).cuda() for l in (0, 1, 2)]
    h = mp.moe_prefill_create(w.d, w.f, w.E, w.k, T)
    ref = []
    for x, lg in zip(xs, lgs):
        y = torch.empty(T, w.d, device="cuda")
        mp.moe_prefill_run_layer(h, x, lg, y, weights=blob)
        torch.cuda.synchronize()
        ref.append(y.cpu())
    x_s, lg_s = xs[0].clone(), lgs[0].clone()
    y_s = torch.empty(T, w.d, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mp.moe_prefill_run_layer_noalloc(w.d, w.f, w.E, w.k, x_s, lg_s, y_s, blob, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="thread_local"):
        mp.moe_prefill_run_layer_noalloc(w.d, w.f, w.E, w.k, x_s, lg_s, y_s, blob)
    for rep in range(3):
        for i in (1, 0, 2):
            x_s.copy_(xs[i])
            lg_s.copy_(lgs[i])
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y_s.cpu(), ref[i]), (rep, i)
            y_e = torch.empty_like(y_s)
            mp.moe_prefill_run_layer(h, xs[i], lgs[i], y_e, weights=blob)
            torch.cuda.synchronize()
            assert torch.equal(y_e.cpu(), ref[i]), (rep, i, "eager")
    del g
    h.close()
