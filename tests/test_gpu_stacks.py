"""The two whole streamed stacks exactly as their workloads configure them,
through the slot pool:

  - 48 layers at T=3072, d_model=2048, d_ff=768, E=128, top-8 with an N(0, 0.5)
    expert bias; prefetch depth 2 and a VRAM budget of 7 layer slots, which the
    planner turns into 4 resident leading layers + the streaming slots;
  - 8 layers at T=8192, d_model=4096, d_ff=1536, E=256, top-8 with Zipf(1.1)
    expert skew; 3 slots, prefetch depth 2.

The pages' acceptance criterion for streaming is output identity with the
non-streamed run (stable-diffusion.cpp #1905 "Verification": every output hash
matches its reference run; #1906 "Verification": 0 differing channels), so every
layer of two passes (the first one cold) must equal that layer run resident bit
for bit.  Sampled tokens of a resident layer and of streamed layers at both ends
of each stack are checked against the CPU oracle (all routing, grouping and Xq
stages in full, y on the sampled tokens), so the pool path at these shapes is
tied to the oracle and not only to the HIP path itself."""
import os

import numpy as np
import pytest
import torch

import moe_prefill_ffn_amd as mp
import oracle
import workload as wl
from gpu_helpers import ExpertCache, assert_close, assert_equal, make_handle, say

pytestmark = pytest.mark.gpu


def _pack(w):
    lb = mp.moe_prefill_layer_bytes(w.d, w.f, w.E)
    threads = max(1, min(16, os.cpu_count() or 1))
    blobs = []
    for l in range(w.n_layers):
        b = torch.empty(lb, dtype=torch.uint8, pin_memory=True)
        mp.pack_layer(w.d, w.f, w.E, lambda e, l=l: wl.expert_weights(w, l, e), b, threads=threads)
        blobs.append(b)
    return blobs, lb


def _sample_tokens(w, lg, n, seed):
    """n random tokens plus tokens routed to the busiest expert and the first/last token."""
    rng = np.random.default_rng(seed)
    eidx, _ = oracle.route(lg, w.k)
    counts = np.bincount(eidx.reshape(-1), minlength=w.E)
    heavy = np.nonzero((eidx == int(np.argmax(counts))).any(1))[0]
    toks = set(rng.choice(w.T, n, replace=False).tolist()) | set(heavy[:4].tolist()) | {0, w.T - 1}
    return sorted(toks)


def _stack_case(key, oracle_layers, passes=2):
    w = wl.WORKLOADS[key]
    st = w.stream
    say(f"[case] {w.name}: packing {w.n_layers} pinned layer blobs")
    blobs, lb = _pack(w)
    xs = [torch.from_numpy(wl.layer_activations(w, l)).cuda() for l in range(w.n_layers)]
    lgs = [torch.from_numpy(wl.layer_logits(w, l)).cuda() for l in range(w.n_layers)]
    h = make_handle(w)

    say(f"[case] {w.name}: resident reference runs")
    ref = []
    for l in range(w.n_layers):
        dev = blobs[l].cuda()
        y = torch.empty(w.T, w.d, device="cuda")
        mp.moe_prefill_run_layer(h, xs[l], lgs[l], y, layer=-1, weights=dev)
        torch.cuda.synchronize()
        ref.append(y.cpu().numpy())
        del dev, y
    torch.cuda.empty_cache()

    say(f"[case] {w.name}: {passes} passes through the pool as configured")
    budget = st.budget_slots * lb if st.budget_slots else 0
    plan = mp.stream_pool_configure(h, blobs, prefetch_depth=st.depth, resident_layers=st.residents,
                                    max_vram_bytes=budget, requested_slots=st.slots)
    ys = [[torch.full((w.T, w.d), float("nan"), device="cuda") for _ in range(w.n_layers)]
          for _ in range(passes)]
    for p in range(passes):
        for l in range(w.n_layers):
            mp.moe_prefill_run_layer(h, xs[l], lgs[l], ys[p][l], layer=l)
        torch.cuda.synchronize()
        for l in range(w.n_layers):
            assert_equal(f"pass {p} layer {l}", ys[p][l].cpu().numpy(), ref[l])
    stats = mp.moe_prefill_get_stats(h)
    h.close()
    del ys, xs, lgs
    torch.cuda.empty_cache()

    for l in oracle_layers:
        say(f"[case] {w.name}: layer {l} against the oracle (sampled tokens)")
        x = wl.layer_activations(w, l)
        lg = wl.layer_logits(w, l)
        toks = _sample_tokens(w, lg, 16, seed=100 + l)
        r = oracle.layer(x, lg, w.k, ExpertCache(w, l, keep=False), w.f, tokens=toks)
        assert_close(f"layer {l} y[tokens]", ref[l][toks], r["y"])
    del blobs
    return w, plan, stats


def test_streamed_48_layer_stack_as_configured():
    w, plan, stats = _stack_case("stream48", oracle_layers=(0, 4, 47))
    assert (plan["slots"], plan["depth"], plan["residents"]) == (7, 2, 4)
    streamed = w.n_layers - plan["residents"]
    # every streamed layer of both passes found its prefetch except possibly the first one
    assert stats["sync_loads"] <= 1
    assert stats["prefetch_activated"] + stats["sync_loads"] == 2 * streamed
    assert stats["layers_run"] == w.n_layers * 3               # references + 2 passes


def test_skewed_8_layer_stack_as_configured():
    w, plan, stats = _stack_case("skew", oracle_layers=(0, 3, 7))
    assert (plan["slots"], plan["depth"], plan["residents"]) == (3, 2, 0)
    assert stats["sync_loads"] <= 1
    assert stats["prefetch_activated"] + stats["sync_loads"] == 2 * w.n_layers
