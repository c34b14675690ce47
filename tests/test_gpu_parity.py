"""GPU parity: the HIP path through the C ABI against the CPU oracle, stage by
stage, on seeded synthetic layers -- the tiny and real-shape resident layers in
full, edge cases (ragged T, single token, one expert, E not a multiple of 64,
partial K stages, empty experts, ties, zero input), and the large skewed /
biased shapes on sampled rows and tokens in the bench's launch configuration.
"""
import ctypes

import numpy as np
import pytest
import torch

import moe_prefill_ffn_amd as mp
import oracle
import workload as wl
from gpu_helpers import (EXPORT_SHAPES, ExpertCache, assert_close, assert_equal, check_full_parity,
                         check_sampled_parity, host_blob, make_handle, run_layer_gpu, say)

pytestmark = pytest.mark.gpu


def _full_case(w, layer=0, x=None, lg=None, override=None, max_tokens=None):
    say(f"[case] {w.name} layer {layer}")
    x = wl.layer_activations(w, layer) if x is None else x
    lg = wl.layer_logits(w, layer) if lg is None else lg
    ex = ExpertCache(w, layer, override=override)
    blob = host_blob(w, ex).cuda()
    h = make_handle(w, max_tokens)
    g = run_layer_gpu(h, w, x, lg, blob)
    ref = oracle.layer(x, lg, w.k, ex, w.f)
    h.close()
    return g, ref


def test_tiny_layer_all_stages():
    w = wl.WORKLOADS["tiny"]
    g, ref = _full_case(w)
    check_full_parity(w, g, ref)


def test_resident_real_shape_all_stages():
    w = wl.WORKLOADS["resident"]
    g, ref = _full_case(w)
    check_full_parity(w, g, ref)


@pytest.mark.parametrize("T,d,f,E,k,bias", [
    (1, 256, 512, 8, 2, None),          # a single token
    (97, 128, 192, 16, 3, None),        # ragged T, f/64 = 3 (partial K stage), odd k
    (200, 64, 64, 130, 7, None),        # E not a multiple of 64, minimal d and f
    (65, 128, 128, 1, 1, None),         # one expert: 65 rows = a full tile + 1 row
    (64, 128, 128, 1, 1, None),         # exactly one full 64-row tile
    (300, 256, 256, 64, 4, ("zipf", 1.1)),   # many empty experts
    (129, 192, 320, 5, 5, None),        # k = E: every expert gets every token
    (70, 64, 64, 257, 8, None),         # E > 256: 16 routing keys per lane
    (40, 64, 64, 1024, 12, None),       # the largest E
    (50, 224, 96, 6, 3, None),          # d and f odd multiples of 32: one-block K tail, one f-block group
    (33, 32, 32, 4, 2, None),           # the smallest d and f: a single K block
    (24, 64, 64, 100, 80, None),        # top_k above 64, rank-count routing (E <= 128)
    (40, 96, 160, 300, 100, None),      # top_k above 64, wave-maximum routing (E > 128)
    (8, 32, 64, 1024, 1024, None),      # k = E = 1024: every token goes to every expert
    (24, 16384, 16384, 2, 1, None),     # the largest d and f: 256 K pairs, 1,024 gate/up n-tiles
    (17, 16352, 16352, 3, 2, None),     # the largest odd multiples of 32: one-block K tails at K = 16352
    (65536, 32, 32, 64, 32, None),      # T * top_k = 2^21, the largest routed-row count
])
def test_edge_shapes(T, d, f, E, k, bias):
    w = wl.small_workload(T, d, f, E, k, seed_base=77 + T + E, bias=bias)
    g, ref = _full_case(w)
    check_full_parity(w, g, ref)
    if bias:
        assert (ref["counts"] == 0).sum() > 0     # the case really has empty experts


def test_tile_row_counts_at_every_group_boundary():
    """Experts with row counts on both sides of every 8-row register group of a
    GEMM row tile (128 rows = two 64-row halves, each one or two 32-row register
    halves): 1 .. 300 rows, i.e. partly filled groups in either half, an empty or
    partly filled second half, full tiles plus a tail of every kind; k = 1 and each
    token's logit for its assigned expert raised by 12, so the counts are exact."""
    counts = [1, 7, 8, 9, 16, 17, 24, 25, 31, 32, 33, 40, 41, 48, 49, 56, 57, 63, 64, 65, 72, 97,
              104, 120, 127, 128, 129, 160, 192, 193, 255, 256, 257, 300]
    E, k, d, f = len(counts) + 2, 1, 128, 192         # two experts get no rows
    T = sum(counts)
    w = wl.small_workload(T, d, f, E, k, seed_base=4242)
    owner = np.repeat(np.arange(len(counts)), counts)
    rng = np.random.default_rng(5)
    owner = owner[rng.permutation(T)]
    lg = wl.layer_logits(w, 0).copy()
    lg[np.arange(T), owner] += 12.0
    g, ref = _full_case(w, lg=lg)
    assert list(ref["counts"][:len(counts)]) == counts and ref["counts"][-2:].sum() == 0
    check_full_parity(w, g, ref)


def test_gemm_block_combination_worked_example():
    """The hand-derived case of tests/golden/gemm_block_order_worked_example.json run
    through the kernels: x is chosen so that its Q8 codes and scales are the example's
    (block 0: code -1 at k = 0, scale 1; block 1: code 3 at k = 32, scale 0x3EAAAAAB),
    and gate row 0 of the single expert holds weight 1 at k = 0 and k = 32 with fp16
    scales 1.0.  GU[0, 0] must be 2^-25 (one fma per block, ascending), the value
    neither a separate multiply nor the other block order gives."""
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "gemm_block_order_worked_example.json")))
    T, d, f, E, k = 1, 64, 32, 1, 1
    w = wl.small_workload(T, d, f, E, k, seed_base=9)
    x = np.zeros((T, d), np.float32)
    x[0, 0], x[0, 1] = -1.0, 127.0               # block 0: amax 127 -> scale 1, codes -1, 127
    x[0, 32], x[0, 33] = 1.0, 42.333336          # block 1: scale 0x3EAAAAAB, code 3 at k = 32
    lg = np.zeros((T, E), np.float32)
    base = wl.expert_weights(w, 0, 0)
    wgu_q = base.wgu_q.copy()
    wgu_s = base.wgu_s.copy()
    wgu_q[0, :] = 0
    wgu_q[0, 0] = wgu_q[0, 32] = 1
    wgu_s[0, :] = 0x3C00
    ex = wl.ExpertWeights(wgu_q, wgu_s, base.wd_q, base.wd_s)
    g_, ref = _full_case(w, x=x, lg=lg, override=lambda e: ex)
    assert ref["xq"][0, 0] == -1 and ref["xq"][0, 32] == 3
    assert ref["dx"].view(np.uint32)[0, 1] == int(g["a_scales_bits"][1], 16)
    assert ref["gu"].view(np.uint32)[0, 0] == int(g["expected_bits"], 16)
    assert g_["gu"].view(np.uint32)[0, 0] == int(g["expected_bits"], 16)
    check_full_parity(w, g_, ref)


@pytest.mark.parametrize("name", ["tiny", "resident"])
def test_hot_path_without_intermediate_exports(name):
    """The bench configuration: GU and H are not exported, so the gate/up GEMM
    writes only Hq and its scales from the fused epilogue."""
    w = wl.WORKLOADS[name]
    say(f"[case] {name} exporting hq, dh only")
    x, lg = wl.layer_activations(w, 0), wl.layer_logits(w, 0)
    ex = ExpertCache(w, 0)
    blob = host_blob(w, ex).cuda()
    h = make_handle(w)
    g = run_layer_gpu(h, w, x, lg, blob, exports=("hq", "dh", "rows"))
    ref = oracle.layer(x, lg, w.k, ex, w.f)
    h.close()
    assert_equal("rows", g["rows"], ref["rows"])
    assert_equal("hq", g["hq"], ref["hq"])
    assert_equal("dh", g["dh"], ref["dh"])
    assert_close("y", g["y"], ref["y"])


def test_kernel_timing_reports_every_launch():
    w = wl.WORKLOADS["tiny"]
    say("[case] kernel timing")
    x, lg = wl.layer_activations(w, 0), wl.layer_logits(w, 0)
    blob = host_blob(w, ExpertCache(w, 0)).cuda()
    h = make_handle(w)
    mp.moe_prefill_set_timing(h, True)
    for _ in range(3):
        run_layer_gpu(h, w, x, lg, blob, exports=())
    kt = mp.moe_prefill_kernel_times(h, reset=True)
    mp.moe_prefill_set_timing(h, False)
    h.close()
    assert list(kt) == ["route_quant", "group", "expert_load", "row_scatter", "gemm_gate_up", "gemm_down", "combine"]
    for name, (count, ms) in kt.items():
        if name == "expert_load":                 # only active-expert loads of streamed layers
            assert count == 0 and ms == 0.0, (name, count, ms)
        else:
            assert count == 3 and ms > 0.0, (name, count, ms)


def test_tied_logits_pick_lowest_experts():
    w = wl.small_workload(40, 128, 128, 12, 4, seed_base=5)
    lg = np.zeros((w.T, w.E), np.float32)
    lg[::2, 7] = 1.0                       # even tokens: expert 7 first, then 0, 1, 2
    lg[1::3, 3] = -0.0                     # -0 ties with +0
    g, ref = _full_case(w, lg=lg)
    check_full_parity(w, g, ref)
    assert np.array_equal(g["eidx"][1], [0, 1, 2, 3])
    assert np.array_equal(g["eidx"][0], [7, 0, 1, 2])


@pytest.mark.parametrize("E", [100, 200])
def test_tied_logits_both_routing_methods(E):
    """Ties (equal logits, -0 against +0) resolve to the lower expert index both
    where ranks are counted (E <= 128) and where slots are taken by repeated
    wave maxima (E > 128)."""
    w = wl.small_workload(36, 64, 64, E, 6, seed_base=11 + E)
    lg = np.zeros((w.T, w.E), np.float32)
    lg[::2, E - 1] = 1.0                   # even tokens: the last expert first, then 0, 1, ...
    lg[1::3, 5] = -0.0
    lg[2::5, [E // 2, E // 3]] = 0.5       # two equal logits above the zeros
    g, ref = _full_case(w, lg=lg)
    check_full_parity(w, g, ref)
    assert np.array_equal(g["eidx"][1], [0, 1, 2, 3, 4, 5])
    assert np.array_equal(g["eidx"][0], [E - 1, 0, 1, 2, 3, 4])
    assert np.array_equal(g["eidx"][7], [E // 3, E // 2, 0, 1, 2, 3])


def test_zero_activations_give_zero_output():
    w = wl.small_workload(50, 128, 192, 8, 2, seed_base=9)
    x = np.zeros((w.T, w.d), np.float32)
    g, ref = _full_case(w, x=x)
    check_full_parity(w, g, ref)
    assert np.all(g["y"] == 0) and np.all(g["xq"] == 0)


def test_tiny_and_huge_magnitudes():
    w = wl.small_workload(64, 128, 128, 8, 2, seed_base=11)
    x = wl.layer_activations(w, 0) * np.float32(1e-30)
    x[3] *= np.float32(1e-8)                # denormal scales
    x[5] = wl.layer_activations(w, 0)[5] * np.float32(1e10)
    g, ref = _full_case(w, x=x)
    check_full_parity(w, g, ref)


def test_out_of_range_block_scales_take_the_exact_gemm_path_layer_by_layer():
    """The GEMMs' 16x weight codes are exact only while every nonzero A block scale
    lies in [2^-98, 2^107]; the quantizers flag any other scale and the GEMM of that
    layer takes the plain codes.  Layers with X scales, or only H scales, outside the
    range alternate with ordinary ones on one handle: every layer bit-exact, so each
    flag is raised when needed and cleared for the next layer."""
    w = wl.small_workload(64, 128, 128, 8, 2, seed_base=11)
    ex = ExpertCache(w, 0)
    blob = host_blob(w, ex).cuda()
    lg = wl.layer_logits(w, 0)
    x0 = wl.layer_activations(w, 0)
    x_tiny = x0 * np.float32(1e-30)
    x_tiny[3] *= np.float32(1e-8)
    cases = [("ordinary", x0, None), ("tiny H scales", x0 * np.float32(1e-20), "h_low"),
             ("ordinary", x0, None), ("huge H scales", x0 * np.float32(1e17), "h_high"),
             ("tiny X scales", x_tiny, "x_low"), ("ordinary", x0, None)]
    h = make_handle(w)
    for name, x, want in cases:
        say(f"[case] {name}")
        ref = oracle.layer(x, lg, w.k, ex, w.f)
        dx, dh = np.abs(ref["dx"]), np.abs(ref["dh"])
        lo, hi = np.float32(2.0 ** -98), np.float32(2.0 ** 107)
        x_out = ((dx > 0) & ((dx < lo) | (dx > hi))).any()
        h_low, h_high = ((dh > 0) & (dh < lo)).any(), (dh > hi).any()
        # the case holds what its name says (checked on the oracle's scales)
        assert x_out == (want == "x_low")
        if want in ("h_low", "h_high"):
            assert {"h_low": h_low, "h_high": h_high}[want] and not x_out
        if want is None:
            assert not (x_out or h_low or h_high)
        g = run_layer_gpu(h, w, x, lg, blob)
        check_full_parity(w, g, ref)
    h.close()


def test_fewer_tokens_than_max_and_repeat_runs_are_identical():
    w = wl.WORKLOADS["tiny"]
    x = wl.layer_activations(w, 0)
    lg = wl.layer_logits(w, 0)
    ex = ExpertCache(w, 0)
    blob = host_blob(w, ex).cuda()
    h = make_handle(w, max_tokens=4 * w.T)
    g1 = run_layer_gpu(h, w, x, lg, blob)
    g2 = run_layer_gpu(h, w, x[:17], lg[:17], blob)
    g3 = run_layer_gpu(h, w, x, lg, blob)
    ref = oracle.layer(x, lg, w.k, ex, w.f)
    ref17 = oracle.layer(x[:17], lg[:17], w.k, ex, w.f)
    check_full_parity(w, g1, ref)
    check_full_parity(w, g2, ref17)
    for k in g1:
        assert_equal(k, g3[k], g1[k])
    # T = 0 is a no-op
    y0 = torch.zeros(0, w.d, device="cuda")
    mp.moe_prefill_run_layer(h, torch.zeros(0, w.d, device="cuda"), torch.zeros(0, w.E, device="cuda"),
                             y0, weights=blob)
    h.close()


def test_bad_arguments_fail_clearly():
    w = wl.WORKLOADS["tiny"]
    h = make_handle(w)
    x = torch.zeros(w.T + 1, w.d, device="cuda")
    lg = torch.zeros(w.T + 1, w.E, device="cuda")
    y = torch.zeros(w.T + 1, w.d, device="cuda")
    blob = torch.zeros(mp.moe_prefill_layer_bytes(w.d, w.f, w.E), dtype=torch.uint8, device="cuda")
    with pytest.raises(mp.MoePrefillError) as ei:
        mp.moe_prefill_run_layer(h, x, lg, y, weights=blob)          # T > max_tokens
    assert ei.value.code == mp.MOE_EINVAL
    with pytest.raises(mp.MoePrefillError) as ei:
        mp.moe_prefill_run_layer(h, x[:4], lg[:4], y[:4], layer=0)   # no pool configured
    assert ei.value.code == mp.MOE_ESTATE
    h.close()


def test_lent_workspace():
    w = wl.WORKLOADS["tiny"]
    nbytes = mp.moe_prefill_workspace_size(w.d, w.f, w.E, w.k, w.T)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    x = wl.layer_activations(w, 0)
    lg = wl.layer_logits(w, 0)
    ex = ExpertCache(w, 0)
    blob = host_blob(w, ex).cuda()
    h = mp.moe_prefill_create(w.d, w.f, w.E, w.k, w.T, workspace=ws)
    g = run_layer_gpu(h, w, x, lg, blob)
    check_full_parity(w, g, oracle.layer(x, lg, w.k, ex, w.f))
    h.close()
    with pytest.raises(mp.MoePrefillError) as ei:
        mp.moe_prefill_create(w.d, w.f, w.E, w.k, w.T, workspace=ws[: nbytes // 2])
    assert ei.value.code == mp.MOE_EINVAL


def _sampled_case(name, n_tok=24, seed=0, combine="gather"):
    w = wl.WORKLOADS[name]
    say(f"[case] {w.name} layer 0 (sampled, {combine} combine)")
    x = wl.layer_activations(w, 0)
    lg = wl.layer_logits(w, 0)
    blob_ex = ExpertCache(w, 0, keep=False)
    blob = host_blob(w, blob_ex).cuda()
    h = make_handle(w)
    ex = ("eidx", "weights", "counts", "bounds", "rows", "pos", "xq", "dx", "hq", "dh")
    g = run_layer_gpu(h, w, x, lg, blob, exports=ex + (("dm",) if combine == "gather" else ()), combine=combine)
    h.close()
    del blob
    torch.cuda.empty_cache()
    rng = np.random.default_rng(seed)
    eidx, _ = oracle.route(lg, w.k)
    counts = np.bincount(eidx.reshape(-1), minlength=w.E)
    big = int(np.argmax(counts))
    heavy = np.nonzero((eidx == big).any(1))[0]
    toks = set(rng.choice(w.T, n_tok, replace=False).tolist())
    toks |= set(heavy[:4].tolist()) | {0, w.T - 1}
    ref = oracle.layer(x, lg, w.k, ExpertCache(w, 0, keep=False), w.f, tokens=sorted(toks))
    return w, g, ref


def test_biased_48_layer_shape_sampled():
    w, g, ref = _sampled_case("stream48")
    check_sampled_parity(w, g, ref)


def test_skewed_large_shape_sampled():
    w, g, ref = _sampled_case("skew", n_tok=16)
    check_sampled_parity(w, g, ref)
    assert ref["counts"].max() > 1000 and (ref["counts"] == 0).sum() > 10


def test_skewed_large_shape_sampled_atomic_combine():
    w, g, ref = _sampled_case("skew", n_tok=16, seed=1, combine="atomic")
    check_sampled_parity(w, g, ref)


@pytest.mark.parametrize("name", ["tiny", "resident"])
def test_atomic_combine_matches_the_oracle(name):
    """MOE_COMBINE_ATOMIC: every stage up to Dm is the gather mode's (bit-exact against
    the oracle), y is within the combine's tolerance of the oracle, and repeated runs
    agree with each other and with the gather mode to within rounding (the order of
    the atomic adds varies)."""
    w = wl.WORKLOADS[name]
    say(f"[case] atomic combine {name}")
    x = wl.layer_activations(w, 0)
    lg = wl.layer_logits(w, 0)
    ex = ExpertCache(w, 0)
    blob = host_blob(w, ex).cuda()
    h = make_handle(w)
    names = tuple(n for n in EXPORT_SHAPES if n != "dm")
    g = run_layer_gpu(h, w, x, lg, blob, exports=names, combine="atomic")
    ref = oracle.layer(x, lg, w.k, ex, w.f)
    check_full_parity(w, g, ref)
    g2 = run_layer_gpu(h, w, x, lg, blob, exports=(), combine="atomic")
    y_gather = run_layer_gpu(h, w, x, lg, blob, exports=())["y"]
    h.close()
    # Both modes sum the same fp32 products w * Dm of each token's k rows; the gather
    # as an fma chain in slot order, the atomic mode as rounded products added in any
    # order.  Each result is within (k + 1) roundings of sum |w * Dm| of the exact sum,
    # so two results differ by at most 2 (k + 1) 2^-24 sum |w * Dm| per element.
    pos = ref["pos"].reshape(w.T, w.k)
    mag = np.einsum("tj,tjc->tc", np.abs(ref["w"]), np.abs(ref["dm"][pos]))
    bound = 2 * (w.k + 1) * 2.0 ** -24 * mag * 1.001
    for name, other in (("repeat", g2["y"]), ("gather", y_gather)):
        diff = np.abs(other.astype(np.float64) - g["y"])
        assert (diff <= bound).all(), (name, diff.max(), bound[np.unravel_index(diff.argmax(), diff.shape)])


def test_atomic_combine_captured_in_a_hip_graph():
    """The atomic combine's extra launches (zeroing y, clearing the mask) are fill
    kernels, so a layer in that mode captures and replays like the default one: every
    replay, with new inputs copied in and eager work between, agrees with the gather's
    y to within the rounding bound of the atomic test above."""
    w = wl.WORKLOADS["tiny"]
    say("[case] graph capture, atomic combine")
    ex = ExpertCache(w, 0)
    blob = host_blob(w, ex).cuda()
    h = make_handle(w)
    xs = [torch.from_numpy(wl.layer_activations(w, l)).cuda() for l in (0, 1)]
    lgs = [torch.from_numpy(wl.layer_logits(w, l)).cuda() for l in (0, 1)]
    ref = []
    for x, lg in zip(xs, lgs):
        y = torch.empty(w.T, w.d, device="cuda")
        mp.moe_prefill_run_layer(h, x, lg, y, weights=blob)
        torch.cuda.synchronize()
        ref.append(y.cpu().double())
    x_s, lg_s = xs[0].clone(), lgs[0].clone()
    y_s = torch.empty(w.T, w.d, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mp.moe_prefill_run_layer(h, x_s, lg_s, y_s, weights=blob, combine="atomic")
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="thread_local"):
        mp.moe_prefill_run_layer(h, x_s, lg_s, y_s, weights=blob, combine="atomic")
    for rep in range(2):
        for i in (1, 0):
            x_s.copy_(xs[i])
            lg_s.copy_(lgs[i])
            g.replay()
            torch.cuda.synchronize()
            diff = (y_s.cpu().double() - ref[i]).abs().max().item()
            assert diff <= 1e-5 * ref[i].abs().max().item(), (rep, i, diff)
            y_e = torch.empty_like(y_s)
            mp.moe_prefill_run_layer(h, xs[i], lgs[i], y_e, weights=blob)
            torch.cuda.synchronize()
            assert torch.equal(y_e.cpu().double(), ref[i]), (rep, i, "eager")
    del g
    h.close()


def test_noalloc_entry_point_with_the_atomic_combine():
    """The allocation-free entry point takes the combine mode too: its y agrees with the
    handle-based gather to within the rounding of a different add order."""
    w = wl.WORKLOADS["tiny"]
    say("[case] noalloc + atomic combine")
    blob = host_blob(w, ExpertCache(w, 0)).cuda()
    x = torch.from_numpy(wl.layer_activations(w, 0)).cuda()
    lg = torch.from_numpy(wl.layer_logits(w, 0)).cuda()
    h = make_handle(w)
    y_ref = torch.empty(w.T, w.d, device="cuda")
    mp.moe_prefill_run_layer(h, x, lg, y_ref, weights=blob)
    y = torch.full((w.T, w.d), float("nan"), device="cuda")
    mp.moe_prefill_run_layer_noalloc(w.d, w.f, w.E, w.k, x, lg, y, blob, combine="atomic")
    torch.cuda.synchronize()
    diff = (y.double() - y_ref.double()).abs().max().item()
    assert diff <= 1e-5 * y_ref.abs().max().item(), diff
    h.close()


def test_atomic_combine_refuses_a_dm_export_and_unknown_modes():
    w = wl.WORKLOADS["tiny"]
    x = torch.from_numpy(wl.layer_activations(w, 0)).cuda()
    lg = torch.from_numpy(wl.layer_logits(w, 0)).cuda()
    blob = host_blob(w, ExpertCache(w, 0)).cuda()
    h = make_handle(w)
    y = torch.empty(w.T, w.d, device="cuda")
    dm = torch.empty(w.T * w.k, w.d, device="cuda")
    with pytest.raises(mp.MoePrefillError) as ei:
        mp.moe_prefill_run_layer(h, x, lg, y, weights=blob, exports={"dm": dm}, combine="atomic")
    assert ei.value.code == mp.MOE_EINVAL and "dm" in str(ei.value)
    io = mp._layer_io(h.params, x, lg, y, -1, blob, None)
    io.combine = 7
    rc = mp.lib().moe_prefill_run_layer(h.ptr, ctypes.byref(io), None)   # rejected before any launch
    assert rc == mp.MOE_EINVAL and b"combine" in mp.lib().moe_prefill_last_error(h.ptr)
    h.close()


@pytest.mark.parametrize("name", ["tiny", "resident"])
def test_layer_captured_in_a_hip_graph_replays_exactly(name):
    """A resident layer is a fixed sequence of stream-ordered kernels (no host
    waits, no memsets), so it can be captured once and replayed: every replay,
    with new inputs copied into the captured buffers and eager work between the
    replays, must equal the eager run bit for bit."""
    w = wl.WORKLOADS[name]
    say(f"[case] graph capture {name}")
    layers = [0, 1, 2]
    blob = host_blob(w, ExpertCache(w, 0)).cuda()
    xs = [torch.from_numpy(wl.layer_activations(w, l)).cuda() for l in layers]
    lgs = [torch.from_numpy(wl.layer_logits(w, l)).cuda() for l in layers]
    h = make_handle(w)
    ref = []
    for x, lg in zip(xs, lgs):
        y = torch.empty(w.T, w.d, device="cuda")
        mp.moe_prefill_run_layer(h, x, lg, y, weights=blob)
        torch.cuda.synchronize()
        ref.append(y.cpu())
    x_s, lg_s = xs[0].clone(), lgs[0].clone()
    y_s = torch.empty(w.T, w.d, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up on the capture stream's side, as torch advises
        mp.moe_prefill_run_layer(h, x_s, lg_s, y_s, weights=blob)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="thread_local"):
        mp.moe_prefill_run_layer(h, x_s, lg_s, y_s, weights=blob)
    for rep in range(3):
        for i in (1, 0, 2):
            x_s.copy_(xs[i])
            lg_s.copy_(lgs[i])
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y_s.cpu(), ref[i]), (rep, i)
            # eager work between the replays
            y_e = torch.empty_like(y_s)
            mp.moe_prefill_run_layer(h, xs[i], lgs[i], y_e, weights=blob)
            torch.cuda.synchronize()
            assert torch.equal(y_e.cpu(), ref[i]), (rep, i, "eager")
    del g
    h.close()
