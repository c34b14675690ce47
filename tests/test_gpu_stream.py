"""Streamed stacks through the fixed-slot pool: every streamed configuration
must give outputs identical bit for bit to running the same layers resident
(the layer-streaming pages' acceptance criterion: matching output hashes with
and without streaming / pooling), and the prefetch counters must follow the
rolling-window policy.  Fault hooks force the synchronous fallback and pool
degradation from the host side; every kernel still runs normally."""
import os

import numpy as np
import pytest
import torch

import moe_prefill_ffn_amd as mp
import oracle
import workload as wl
from gpu_helpers import ExpertCache, assert_close, assert_equal, host_blob, make_handle, say

pytestmark = pytest.mark.gpu


class Stack:
    def __init__(self, w: wl.Workload, n_layers: int):
        self.w = w
        self.n = n_layers
        self.blobs = [host_blob(w, ExpertCache(w, l, keep=False), pinned=True) for l in range(n_layers)]
        self.x = [torch.from_numpy(wl.layer_activations(w, l)).cuda() for l in range(n_layers)]
        self.lg = [torch.from_numpy(wl.layer_logits(w, l)).cuda() for l in range(n_layers)]
        h = make_handle(w)
        self.ref = []
        for l in range(n_layers):
            dev = self.blobs[l].cuda()
            y = torch.empty(w.T, w.d, device="cuda")
            mp.moe_prefill_run_layer(h, self.x[l], self.lg[l], y, layer=-1, weights=dev)
            torch.cuda.synchronize()
            self.ref.append(y.cpu().numpy())
        h.close()

    def run_passes(self, h, passes: int, order=None):
        order = order or list(range(self.n))
        outs = []
        for _ in range(passes):
            for l in order:
                y = torch.full((self.w.T, self.w.d), float("nan"), device="cuda")
                mp.moe_prefill_run_layer(h, self.x[l], self.lg[l], y, layer=l)
                outs.append((l, y))
        torch.cuda.synchronize()
        return [(l, y.cpu().numpy()) for l, y in outs]

    def check(self, outs):
        for l, y in outs:
            assert_equal(f"layer {l}", y, self.ref[l])


@pytest.fixture(scope="module")
def tiny5():
    say("[case] 5-layer tiny stack")
    return Stack(wl.Workload("stack5_T64_d256_f512_E8_top2", 64, 256, 512, 8, 2, 5, 600), 5)


def _configure(h, st, **kw):
    return mp.stream_pool_configure(h, st.blobs, **kw)


def test_rolling_window_depth1_two_slots(tiny5):
    h = make_handle(tiny5.w)
    plan = _configure(h, tiny5, prefetch_depth=1, resident_layers=0, requested_slots=2)
    assert (plan["slots"], plan["depth"], plan["residents"]) == (2, 1, 0)
    tiny5.check(tiny5.run_passes(h, 2))
    s = mp.moe_prefill_get_stats(h)
    # pass 1: layer 0 loads synchronously; every later layer finds its prefetch
    assert s["sync_loads"] == 1
    assert s["prefetch_queued"] == 2 * 5
    assert s["prefetch_activated"] == 2 * 5 - 1
    assert s["prefetch_failed"] == 0
    h.close()


def test_streamed_atomic_combine_matches_resident_within_rounding(tiny5):
    """The atomic combine on pool slots (prefetched and loaded): the same y as the
    resident gather to within the rounding of a different order of the k adds."""
    h = make_handle(tiny5.w)
    _configure(h, tiny5, prefetch_depth=1, resident_layers=1, requested_slots=3)
    outs = []
    for l in range(tiny5.n):
        y = torch.full((tiny5.w.T, tiny5.w.d), float("nan"), device="cuda")
        mp.moe_prefill_run_layer(h, tiny5.x[l], tiny5.lg[l], y, layer=l, combine="atomic")
        outs.append((l, y))
    torch.cuda.synchronize()
    for l, y in outs:
        ref = tiny5.ref[l].astype(np.float64)
        assert np.abs(y.cpu().numpy() - ref).max() <= 1e-5 * np.abs(ref).max(), l
    h.close()


def test_depth0_is_load_then_compute(tiny5):
    h = make_handle(tiny5.w)
    plan = _configure(h, tiny5, prefetch_depth=0, resident_layers=0)
    assert (plan["slots"], plan["depth"]) == (1, 0)
    tiny5.check(tiny5.run_passes(h, 2))
    s = mp.moe_prefill_get_stats(h)
    assert s["sync_loads"] == 10 and s["prefetch_queued"] == 0
    h.close()


def test_depth2_three_slots_and_residents(tiny5):
    h = make_handle(tiny5.w)
    lb = tiny5.blobs[0].numel()
    slot = (lb + 65535) // 65536 * 65536
    plan = _configure(h, tiny5, prefetch_depth=2, resident_layers=-1, max_vram_bytes=5 * slot)
    assert (plan["slots"], plan["depth"], plan["residents"]) == (5, 2, 2)
    tiny5.check(tiny5.run_passes(h, 3))
    s = mp.moe_prefill_get_stats(h)
    assert s["eff_residents"] == 2 and s["prefetch_failed"] == 0
    # residents never stream: 3 streamed layers per pass after the first
    assert s["sync_loads"] == 0 or s["sync_loads"] == 1
    h.close()


def test_out_of_order_layers_still_match(tiny5):
    h = make_handle(tiny5.w)
    _configure(h, tiny5, prefetch_depth=1, resident_layers=0, requested_slots=2)
    tiny5.check(tiny5.run_passes(h, 2, order=[3, 1, 4, 4, 0, 2]))
    h.close()


def test_forced_prefetch_failure_falls_back(tiny5):
    os.environ["MOE_TEST_PREFETCH_FAIL"] = "2"
    try:
        h = make_handle(tiny5.w)
        _configure(h, tiny5, prefetch_depth=1, resident_layers=0, requested_slots=2)
    finally:
        del os.environ["MOE_TEST_PREFETCH_FAIL"]
    tiny5.check(tiny5.run_passes(h, 2))
    s = mp.moe_prefill_get_stats(h)
    assert s["prefetch_failed"] == 1
    assert s["sync_loads"] == 2
    h.close()


def test_pool_degrades_to_one_slot(tiny5):
    os.environ["MOE_TEST_POOL_MAX_SLOTS"] = "1"
    try:
        h = make_handle(tiny5.w)
        plan = _configure(h, tiny5, prefetch_depth=1, resident_layers=0, requested_slots=2)
    finally:
        del os.environ["MOE_TEST_POOL_MAX_SLOTS"]
    assert (plan["slots"], plan["depth"]) == (1, 0)
    assert plan["warnings"] & mp.MOE_WARN_POOL_DEGRADED
    tiny5.check(tiny5.run_passes(h, 2))
    h.close()


def test_one_slot_failure_is_an_error_and_reconfigure_works(tiny5):
    h = make_handle(tiny5.w)
    os.environ["MOE_TEST_POOL_FAIL_ALL"] = "1"
    try:
        with pytest.raises(mp.MoePrefillError) as ei:
            _configure(h, tiny5, prefetch_depth=1, resident_layers=0, requested_slots=2)
    finally:
        del os.environ["MOE_TEST_POOL_FAIL_ALL"]
    assert ei.value.code == mp.MOE_ENOMEM
    with pytest.raises(mp.MoePrefillError) as ei:
        tiny5.run_passes(h, 1)
    assert ei.value.code == mp.MOE_ESTATE
    _configure(h, tiny5, prefetch_depth=1, resident_layers=0, requested_slots=2)
    tiny5.check(tiny5.run_passes(h, 1))
    # a new plan releases the old pool first; tearing down works too
    _configure(h, tiny5, prefetch_depth=2, resident_layers=1, requested_slots=4)
    tiny5.check(tiny5.run_passes(h, 1))
    mp.stream_pool_configure(h, [], prefetch_depth=0)
    h.close()


def test_streamed_real_shape_stack_matches_resident_and_oracle():
    w = wl.WORKLOADS["stream4"]
    say(f"[case] {w.name}")
    st = Stack(w, w.n_layers)
    h = make_handle(w)
    plan = _configure(h, st, prefetch_depth=w.stream.depth, resident_layers=w.stream.residents,
                      requested_slots=w.stream.slots)
    assert (plan["slots"], plan["depth"], plan["residents"]) == (2, 1, 0)
    outs = st.run_passes(h, 2)
    st.check(outs)
    s = mp.moe_prefill_get_stats(h)
    assert s["bytes_h2d"] == (1 + s["prefetch_queued"]) * st.blobs[0].numel()
    h.close()
    # one streamed layer against the oracle too (sampled tokens)
    toks = [0, 1, 500, 1023]
    ref = oracle.layer(wl.layer_activations(w, 2), wl.layer_logits(w, 2), w.k, ExpertCache(w, 2, keep=False),
                       w.f, tokens=toks)
    assert_close("streamed layer 2 y", outs[2][1][toks], ref["y"])


# ------------------------------------------------------ active-expert loads ---

@pytest.fixture(scope="module")
def skew4():
    say("[case] 4-layer skewed stack (many empty experts)")
    w = wl.Workload("stack4_T96_d256_f320_E48_top2_zipf", 96, 256, 320, 48, 2, 4, 700, bias=("zipf", 1.1))
    return Stack(w, 4)


def _active_experts(st, layer):
    lg = wl.layer_logits(st.w, layer)
    top = np.argsort(-lg, axis=1, kind="stable")[:, :st.w.k]
    return np.unique(top).size


def test_stack_references_match_the_oracle(tiny5, skew4):
    """The resident runs every streamed stack here is compared with, against the
    oracle in full (every token of every layer): the pool tests then tie the
    streamed outputs to the oracle, not only to the HIP path itself."""
    for st in (tiny5, skew4):
        for l in range(st.n):
            say(f"[case] {st.w.name} layer {l} against the oracle")
            ref = oracle.layer(wl.layer_activations(st.w, l), wl.layer_logits(st.w, l), st.w.k,
                               ExpertCache(st.w, l), st.w.f)
            assert_close(f"{st.w.name} layer {l} y", st.ref[l], ref["y"])


def test_active_only_loads_only_routed_experts(skew4):
    h = make_handle(skew4.w)
    plan = _configure(h, skew4, prefetch_depth=2, resident_layers=0, requested_slots=2, active_only=True)
    assert plan["depth"] == 0 and plan["residents"] == 0      # routing decides the copy: no lookahead
    outs = skew4.run_passes(h, 2)
    skew4.check(outs)                                         # identical to the resident run
    s = mp.moe_prefill_get_stats(h)
    active = sum(_active_experts(skew4, l) for l in range(4))
    assert active < 4 * skew4.w.E                             # the case has idle experts
    eb = mp.moe_prefill_expert_bytes(skew4.w.d, skew4.w.f)
    assert s["sparse_loads"] == 8 and s["sync_loads"] == 0 and s["prefetch_queued"] == 0
    assert s["experts_loaded"] == 2 * active
    assert s["bytes_sparse"] == 2 * active * eb
    assert s["bytes_h2d"] == 0
    h.close()


def test_active_only_one_slot_reuse_and_residents(skew4):
    """One streaming slot rewritten by every layer (experts a layer does not use
    keep the previous layer's bytes and are never read), plus a resident layer
    that is uploaded whole and never reloaded."""
    h = make_handle(skew4.w)
    lb = skew4.blobs[0].numel()
    slot = (lb + 65535) // 65536 * 65536
    plan = _configure(h, skew4, prefetch_depth=1, resident_layers=1, max_vram_bytes=2 * slot,
                      active_only=True)
    assert (plan["slots"], plan["depth"], plan["residents"]) == (2, 0, 1)
    skew4.check(skew4.run_passes(h, 2, order=[0, 2, 1, 3, 2]))
    s = mp.moe_prefill_get_stats(h)
    assert s["sparse_loads"] == 2 * 4                         # every non-resident run loads again
    h.close()


def test_active_only_rejects_pageable_blobs(skew4):
    h = make_handle(skew4.w)
    pageable = [b.clone() for b in skew4.blobs]               # ordinary host memory
    assert not pageable[0].is_pinned()
    with pytest.raises(mp.MoePrefillError) as ei:
        _raw_configure(h, pageable)                           # rejected before any kernel runs
    assert ei.value.code == mp.MOE_EINVAL
    h.close()


def _raw_configure(h, blobs):
    """Calls the C entry point directly (the binding itself refuses unpinned tensors)."""
    import ctypes
    p = mp.stream_pool_params_t()
    p.struct_size = ctypes.sizeof(p)
    arr = (ctypes.c_void_p * len(blobs))(*[b.data_ptr() for b in blobs])
    p.n_layers = len(blobs)
    p.host_blobs = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    p.layer_bytes = blobs[0].numel()
    p.active_only = 1
    mp._check(mp.lib().stream_pool_configure(h.ptr, ctypes.byref(p)), h.ptr)


# ---------------------------------------------------------- memory pressure ---

def _slot_bytes(st):
    lb = st.blobs[0].numel()
    return (lb + 65535) // 65536 * 65536


def _passes_preallocated(st, h, passes, outs):
    for p in range(passes):
        for l in range(st.n):
            mp.moe_prefill_run_layer(h, st.x[l], st.lg[l], outs[p][l], layer=l)
    torch.cuda.synchronize()
    for p in range(passes):
        for l in range(st.n):
            assert_equal(f"pass {p} layer {l}", outs[p][l].cpu().numpy(), st.ref[l])


def test_budget_evicts_residents_from_the_end_and_returns_memory(tiny5):
    h = make_handle(tiny5.w)
    slot = _slot_bytes(tiny5)
    plan = _configure(h, tiny5, prefetch_depth=1, resident_layers=-1, max_vram_bytes=5 * slot)
    assert (plan["slots"], plan["depth"], plan["residents"]) == (5, 1, 3)
    tiny5.check(tiny5.run_passes(h, 1))
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    b = mp.stream_pool_set_budget(h, 3 * slot)
    free1 = torch.cuda.mem_get_info()[0]
    assert (b["slots"], b["depth"], b["residents"], b["released_bytes"]) == (3, 1, 1, 2 * slot)
    assert free1 - free0 >= 2 * slot - (1 << 20), (free0, free1)
    tiny5.check(tiny5.run_passes(h, 2))
    s = mp.moe_prefill_get_stats(h)
    assert (s["eff_residents"], s["eff_slots"], s["evicted_residents"], s["released_bytes"]) == (1, 3, 2, 2 * slot)
    assert s["prefetch_failed"] == 0
    # the budget only shrinks: a larger one changes nothing
    b = mp.stream_pool_set_budget(h, 10 * slot)
    assert (b["slots"], b["residents"], b["released_bytes"]) == (3, 1, 0)
    tiny5.check(tiny5.run_passes(h, 1))
    h.close()


def test_budget_on_an_all_resident_pool_keeps_a_streaming_slot(tiny5):
    h = make_handle(tiny5.w)
    slot = _slot_bytes(tiny5)
    plan = _configure(h, tiny5, prefetch_depth=1, resident_layers=-1)
    assert (plan["slots"], plan["depth"], plan["residents"]) == (5, 0, 5)
    tiny5.check(tiny5.run_passes(h, 1))
    b = mp.stream_pool_set_budget(h, 2 * slot)
    assert (b["slots"], b["depth"], b["residents"], b["released_bytes"]) == (2, 0, 1, 3 * slot)
    tiny5.check(tiny5.run_passes(h, 2))
    s = mp.moe_prefill_get_stats(h)
    assert s["evicted_residents"] == 4 and s["sync_loads"] > 0
    h.close()


def test_budget_below_one_slot_keeps_the_execution_slot(tiny5):
    h = make_handle(tiny5.w)
    slot = _slot_bytes(tiny5)
    _configure(h, tiny5, prefetch_depth=2, resident_layers=0, requested_slots=3)
    tiny5.check(tiny5.run_passes(h, 1))
    b = mp.stream_pool_set_budget(h, 1)
    assert (b["slots"], b["depth"], b["residents"], b["released_bytes"]) == (1, 0, 0, 2 * slot)
    assert b["warnings"] & mp.MOE_WARN_SLOT_OVER_BUDGET and b["warnings"] & mp.MOE_WARN_DEPTH_REDUCED
    tiny5.check(tiny5.run_passes(h, 2))
    assert mp.moe_prefill_get_stats(h)["sync_loads"] >= 10
    h.close()


def test_budget_needs_a_pool_and_a_positive_budget(tiny5):
    h = make_handle(tiny5.w)
    with pytest.raises(mp.MoePrefillError) as e:
        mp.stream_pool_set_budget(h, 1 << 30)
    assert e.value.code == mp.MOE_ESTATE
    _configure(h, tiny5, prefetch_depth=1, resident_layers=0, requested_slots=2)
    with pytest.raises(mp.MoePrefillError) as e:
        mp.stream_pool_set_budget(h, 0)
    assert e.value.code == mp.MOE_EINVAL
    h.close()


def test_reserve_shrinks_the_pool_when_a_pass_starts(tiny5):
    """Memory pressure from the host side: the reserve asks for more free device memory
    than there is, so the next pass start gives residents back (from the end of the
    prefix) until the shortfall is covered; later passes find the reserve met."""
    w = tiny5.w
    slot = _slot_bytes(tiny5)
    outs = [[torch.empty(w.T, w.d, device="cuda") for _ in range(tiny5.n)] for _ in range(3)]
    h = make_handle(w)
    _configure(h, tiny5, prefetch_depth=1, resident_layers=-1, max_vram_bytes=5 * slot)
    torch.cuda.synchronize()
    free_now = torch.cuda.mem_get_info()[0]
    plan = _configure(h, tiny5, prefetch_depth=1, resident_layers=-1, max_vram_bytes=5 * slot,
                      reserve_bytes=free_now + slot + slot // 2)
    assert plan["residents"] == 3
    _passes_preallocated(tiny5, h, 3, outs)
    s = mp.moe_prefill_get_stats(h)
    assert s["pressure_trims"] == 1, s
    assert (s["eff_residents"], s["evicted_residents"], s["released_bytes"]) == (1, 2, 2 * slot)
    h.close()


# ------------------------------------------------------ logging and debug ---

def test_log_sink_reports_degradations_and_pool_decisions(tiny5):
    msgs = []
    h = make_handle(tiny5.w)
    mp.moe_prefill_set_log(h, lambda lv, m: msgs.append((lv, m)), mp.MOE_LOG_INFO)
    slot = _slot_bytes(tiny5)
    os.environ["MOE_TEST_PREFETCH_FAIL"] = "2"
    try:
        _configure(h, tiny5, prefetch_depth=4, resident_layers=0, max_vram_bytes=3 * slot)
    finally:
        del os.environ["MOE_TEST_PREFETCH_FAIL"]
    tiny5.check(tiny5.run_passes(h, 1))
    mp.stream_pool_set_budget(h, 2 * slot)
    text = "\n".join(m for _, m in msgs)
    assert any(lv == mp.MOE_LOG_WARN and "prefetch depth reduced" in m for lv, m in msgs), text
    assert any(lv == mp.MOE_LOG_WARN and "failed (test hook)" in m for lv, m in msgs), text
    assert any(lv == mp.MOE_LOG_INFO and m.startswith("pool: 3 slots") for lv, m in msgs), text
    assert any(lv == mp.MOE_LOG_INFO and "released" in m for lv, m in msgs), text
    # WARN level drops the INFO messages; errors always come through
    msgs.clear()
    mp.moe_prefill_set_log(h, lambda lv, m: msgs.append((lv, m)), mp.MOE_LOG_WARN)
    tiny5.check(tiny5.run_passes(h, 1))
    assert all(lv <= mp.MOE_LOG_WARN for lv, _ in msgs)
    with pytest.raises(mp.MoePrefillError):
        mp.stream_pool_set_budget(h, 0)
    assert msgs and msgs[-1][0] == mp.MOE_LOG_ERROR
    mp.moe_prefill_set_log(h, None)
    h.close()


def _poisoned(st, **kw):
    os.environ["MOE_DEBUG_POISON"] = "1"
    try:
        h = make_handle(st.w)
        _configure(h, st, **kw)
    finally:
        del os.environ["MOE_DEBUG_POISON"]
    return h


def test_poisoned_slots_change_nothing(tiny5):
    """Debug mode: a slot is filled with NaN bytes right before every refill, so a
    read between a slot's free fence and its refill would turn outputs into NaN."""
    h = _poisoned(tiny5, prefetch_depth=2, resident_layers=0, requested_slots=3)
    tiny5.check(tiny5.run_passes(h, 2, order=[0, 1, 2, 3, 4, 2, 0]))
    h.close()


def test_poisoned_active_only_slots_never_read_unrouted_experts(skew4):
    """Active-expert loads into a NaN-filled slot: the experts a layer routes no
    rows to keep NaN bytes and must never be read."""
    assert sum(_active_experts(skew4, l) for l in range(4)) < 4 * skew4.w.E
    h = _poisoned(skew4, prefetch_depth=1, resident_layers=0, requested_slots=2, active_only=True)
    skew4.check(skew4.run_passes(h, 2))
    h.close()


def test_serialized_launches_give_the_same_outputs(tiny5, tmp_path):
    """Race check: the streamed stack in a child process with every kernel and copy
    serialised by the runtime (AMD_SERIALIZE_KERNEL=3, AMD_SERIALIZE_COPY=3) equals the
    reference bit for bit, as the normal overlapped run does."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = tmp_path / "y.npy"
    code = f"""
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {os.path.join(root, "tests")!r})
import numpy as np, torch
import moe_prefill_ffn_amd as mp, workload as wl
from gpu_helpers import ExpertCache, host_blob, make_handle
w = wl.Workload("stack5_T64_d256_f512_E8_top2", 64, 256, 512, 8, 2, 5, 600)
blobs = [host_blob(w, ExpertCache(w, l, keep=False), pinned=True) for l in range(5)]
h = make_handle(w)
mp.stream_pool_configure(h, blobs, prefetch_depth=2, resident_layers=0, requested_slots=3)
ys = []
for p in range(2):
    for l in range(5):
        y = torch.empty(w.T, w.d, device="cuda")
        x = torch.from_numpy(wl.layer_activations(w, l)).cuda()
        lg = torch.from_numpy(wl.layer_logits(w, l)).cuda()
        mp.moe_prefill_run_layer(h, x, lg, y, layer=l)
        ys.append(y)
torch.cuda.synchronize()
np.save({str(out)!r}, np.stack([y.cpu().numpy() for y in ys]))
h.close()
"""
    env = dict(os.environ, AMD_SERIALIZE_KERNEL="3", AMD_SERIALIZE_COPY="3")
    say("[case] serialized child process")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stderr[-2000:]
    ys = np.load(out)
    for i, y in enumerate(ys):
        assert_equal(f"serialized layer {i % 5}", y, tiny5.ref[i % 5])
