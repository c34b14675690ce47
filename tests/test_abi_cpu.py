"""Host-side checks of the C ABI that need no GPU: the library loads and exports
every entry point the header declares, the pool planner follows the
layer-streaming pages' policy tables, versioned structs behave, and the weight
packer writes the documented tile layout."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest
import torch

import moe_prefill_ffn_amd as mp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_prefill.h")
MiB = 1 << 20


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"^typedef[^;]*;", "", src, flags=re.M | re.S)     # function-pointer types declare nothing
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


def test_library_exports_every_declared_symbol():
    declared = _declared_functions()
    assert "moe_prefill_create" in declared and "stream_pool_configure" in declared
    assert "moe_prefill_run_layer" in declared
    L = mp.lib()
    for name in declared:
        assert hasattr(L, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", mp.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(line.split()[-1] for line in nm.splitlines() if " T " in line)
    for name in declared:
        assert name in exported, name
    assert sorted(mp.EXPORTED_SYMBOLS) == declared


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device error path")
def test_kernel_ids_and_names():
    names = [mp.lib().moe_prefill_kernel_name(i).decode() for i in range(mp.MOE_N_KERNELS)]
    assert names == ["route_quant", "group", "expert_load", "row_scatter", "gemm_gate_up", "gemm_down", "combine"]
    assert mp.lib().moe_prefill_kernel_name(mp.MOE_N_KERNELS) == b""
    assert mp.lib().moe_prefill_kernel_name(-1) == b""
    hdr = open(os.path.join(ROOT, "include", "moe_prefill.h")).read()
    assert f"#define MOE_N_KERNELS {mp.MOE_N_KERNELS}" in hdr


def test_create_without_gpu_fails_clearly():
    with pytest.raises(mp.MoePrefillError) as ei:
        mp.moe_prefill_create(256, 512, 8, 2, 64)
    assert ei.value.code in (mp.MOE_EUNSUPPORTED, mp.MOE_EHIP)
    assert mp.moe_prefill_last_error()


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device error path")
def test_errors_reach_stderr_when_MOE_LOG_LEVEL_is_set(capfd, monkeypatch):
    monkeypatch.setenv("MOE_LOG_LEVEL", "0")
    with pytest.raises(mp.MoePrefillError):
        mp.moe_prefill_create(256, 512, 8, 2, 64)
    err = capfd.readouterr().err
    assert "moe_prefill error:" in err and mp.moe_prefill_last_error() in err
    monkeypatch.setenv("MOE_LOG_LEVEL", "-1")
    with pytest.raises(mp.MoePrefillError):
        mp.moe_prefill_create(256, 512, 8, 2, 64)
    assert "moe_prefill" not in capfd.readouterr().err


def test_dimension_checks():
    for bad in [(100, 512, 8, 2, 64), (256, 500, 8, 2, 64), (256, 512, 0, 1, 64), (256, 512, 8, 9, 64),
                (256, 512, 8, 2, 0), (256, 512, 2000, 2, 64), (256, 512, 128, 129, 64), (16, 512, 8, 2, 64),
                (256, 16400, 8, 2, 64), (256, 512, 1024, 1024, 4096)]:
        with pytest.raises(mp.MoePrefillError) as ei:
            mp.moe_prefill_workspace_size(*bad)
        assert ei.value.code == mp.MOE_EINVAL
    # multiples of 32 (one Q8/Q4 block) and any top_k up to n_experts are accepted
    for ok in [(224, 96, 8, 2, 64), (32, 32, 1, 1, 1), (256, 512, 128, 65, 64), (64, 64, 1024, 1024, 2048)]:
        assert mp.moe_prefill_workspace_size(*ok) > 0
    a = mp.moe_prefill_workspace_size(2048, 768, 128, 8, 1024)
    b = mp.moe_prefill_workspace_size(2048, 768, 128, 8, 2048)
    assert 0 < a < b


def test_blob_sizes():
    # resident-layer shape: E=128, d=2048, f=768 -> 2 x 1.5 MiB-ish experts
    eb = mp.moe_prefill_expert_bytes(2048, 768)
    assert eb == 2 * 768 * 2048 // 2 + 2 * 768 * 64 * 2 + 2048 * 768 // 2 + 2048 * 24 * 2
    assert mp.moe_prefill_layer_bytes(2048, 768, 128) == 128 * eb
    assert mp.moe_prefill_layer_bytes(2048, 768, 128) == 324 * MiB
    assert mp.moe_prefill_expert_bytes(100, 768) == 0
    # K % 64 == 32: the last K pair of every n-tile is stored whole (one block of zero codes)
    pad = lambda x: (x + 255) // 256 * 256
    assert mp.moe_prefill_expert_bytes(224, 96) == (pad(2 * 96 * 4 * 32) + pad(2 * 96 * 8 * 2) +
                                                    pad(224 * 2 * 32) + pad(224 * 8 * 2))


# ------------------------------------------------------------- planner ---

S = 324 * MiB


def plan(L, depth, res, budget_slots=0, requested=0, max_alloc=0, slot=S):
    return mp.moe_prefill_plan_pool(L, slot, depth, res, budget_slots * slot, requested, max_alloc)


def test_plan_depth0_is_load_then_compute():
    p = plan(4, 0, 0)
    assert (p["rc"], p["slots"], p["depth"], p["residents"]) == (0, 1, 0, 0)


def test_plan_minimal_rolling_window():
    # no optional residents, depth 1: one active + one prefetched slot
    p = plan(4, 1, 0, budget_slots=2)
    assert (p["slots"], p["depth"], p["residents"], p["warnings"]) == (2, 1, 0, 0)
    p = plan(4, 1, 0, requested=2)
    assert (p["slots"], p["depth"], p["residents"]) == (2, 1, 0)


def test_plan_depth_reduced_to_fit_budget():
    p = plan(8, 10, 0, budget_slots=3)
    assert (p["slots"], p["depth"], p["residents"]) == (3, 2, 0)
    assert p["warnings"] & mp.MOE_WARN_DEPTH_REDUCED


def test_plan_auto_residents_use_the_leftover_budget():
    # 48-layer stack, depth 2, budget of 7 slots -> 4 resident leading layers
    p = plan(48, 2, -1, budget_slots=7)
    assert (p["slots"], p["depth"], p["residents"]) == (7, 2, 4)


def test_plan_resident_count_is_a_maximum_and_only_peak_slots_allocated():
    p = plan(48, 2, 2, budget_slots=7)
    assert (p["slots"], p["depth"], p["residents"]) == (5, 2, 2)
    p = plan(48, 2, 50, budget_slots=7)
    assert (p["slots"], p["depth"], p["residents"]) == (7, 2, 4)


def test_plan_prefetch_window_before_residents():
    p = plan(10, 3, -1, budget_slots=4)
    assert (p["slots"], p["depth"], p["residents"]) == (4, 3, 0)


def test_plan_budget_below_one_slot_keeps_the_mandatory_slot():
    p = mp.moe_prefill_plan_pool(4, S, 1, -1, S // 2, 0, 0)
    assert (p["rc"], p["slots"], p["depth"], p["residents"]) == (0, 1, 0, 0)
    assert p["warnings"] & mp.MOE_WARN_SLOT_OVER_BUDGET


def test_plan_allocation_failure_degrades_residents_first():
    p = plan(48, 2, -1, budget_slots=7, max_alloc=5)
    assert (p["rc"], p["slots"], p["depth"], p["residents"]) == (0, 5, 2, 2)
    assert p["warnings"] & mp.MOE_WARN_POOL_DEGRADED
    p = plan(48, 2, -1, budget_slots=7, max_alloc=2)
    assert (p["slots"], p["depth"], p["residents"]) == (2, 1, 0)
    p = plan(48, 2, -1, budget_slots=7, max_alloc=1)
    assert (p["slots"], p["depth"], p["residents"]) == (1, 0, 0)


def test_plan_one_slot_failure_is_an_error():
    p = plan(4, 1, 0, budget_slots=2, max_alloc=-1)
    assert p["rc"] == mp.MOE_ENOMEM


def test_plan_no_cap_means_everything_resident():
    p = plan(4, 1, -1)
    assert (p["slots"], p["depth"], p["residents"]) == (4, 0, 4)


def test_plan_depth_clipped_to_streamed_layers():
    p = plan(3, 5, 0)
    assert (p["slots"], p["depth"], p["residents"]) == (3, 2, 0)
    p = plan(1, 2, 0)
    assert (p["slots"], p["depth"], p["residents"]) == (1, 0, 0)


def test_plan_skewed_stack_three_slots():
    p = plan(8, 2, 0, requested=3)
    assert (p["slots"], p["depth"], p["residents"]) == (3, 2, 0)


# ---------------------------------------------------- versioned structs ---

def trim(L, residents, streaming, budget_slots):
    return mp.moe_prefill_plan_trim(L, residents, streaming, budget_slots)


def test_trim_evicts_from_the_end_of_the_resident_prefix_before_prefetch_slots():
    # 48 layers, 4 residents + 3 streaming (depth 2): a 5-slot budget costs two residents
    t = trim(48, 4, 3, 5)
    assert (t["rc"], t["residents"], t["streaming"], t["evicted"], t["released"]) == (0, 2, 3, 2, 2)
    assert t["converted"] == 0 and t["warnings"] == 0
    # 3 slots: every resident goes, the prefetch window stays
    t = trim(48, 4, 3, 3)
    assert (t["residents"], t["streaming"], t["evicted"], t["released"]) == (0, 3, 4, 4)


def test_trim_then_shrinks_the_prefetch_window():
    t = trim(48, 4, 3, 2)
    assert (t["residents"], t["streaming"], t["evicted"], t["released"]) == (0, 2, 4, 5)
    assert t["warnings"] & mp.MOE_WARN_DEPTH_REDUCED


def test_trim_keeps_one_slot_even_below_the_budget():
    t = trim(8, 0, 3, 0)
    assert (t["residents"], t["streaming"], t["released"]) == (0, 1, 2)
    assert t["warnings"] & mp.MOE_WARN_SLOT_OVER_BUDGET


def test_trim_of_an_all_resident_pool_keeps_a_streaming_slot():
    # every layer resident (no streaming slot): the first evicted layer's slot becomes it
    t = trim(4, 4, 0, 2)
    assert (t["residents"], t["streaming"], t["evicted"], t["converted"], t["released"]) == (1, 1, 3, 1, 2)


def test_trim_within_budget_changes_nothing():
    t = trim(48, 4, 3, 7)
    assert (t["residents"], t["streaming"], t["evicted"], t["released"], t["warnings"]) == (4, 3, 0, 0, 0)
    t = trim(48, 4, 3, 100)
    assert (t["residents"], t["streaming"], t["released"]) == (4, 3, 0)


def test_trim_rejects_pools_the_planner_never_makes():
    assert trim(4, 5, 1, 2)["rc"] == mp.MOE_EINVAL        # more residents than layers
    assert trim(4, 2, 0, 2)["rc"] == mp.MOE_EINVAL        # streamed layers but no streaming slot
    assert trim(4, 0, 0, 2)["rc"] == mp.MOE_EINVAL        # no slot at all


def test_undersized_struct_takes_defaults():
    p = mp.moe_pool_plan_t()
    p.n_layers, p.slot_bytes, p.prefetch_depth, p.resident_layers = 4, S, 1, 0
    p.max_vram_bytes = 2 * S
    p.requested_slots = 0
    p.max_alloc_slots = 1           # beyond the truncated size: must be ignored (default 0)
    p.struct_size = mp.moe_pool_plan_t.max_alloc_slots.offset
    assert mp.lib().moe_prefill_plan_pool(ctypes.byref(p)) == 0
    # outputs are not written past the caller's struct_size
    assert p.slots == 0


def test_oversized_struct_with_nonzero_tail_is_rejected():
    class Big(ctypes.Structure):
        _fields_ = [("base", mp.moe_pool_plan_t), ("extra", ctypes.c_int64)]
    b = Big()
    b.base.struct_size = ctypes.sizeof(Big)
    b.base.n_layers, b.base.slot_bytes, b.base.prefetch_depth = 4, S, 1
    b.extra = 0
    ptr = ctypes.cast(ctypes.byref(b), ctypes.POINTER(mp.moe_pool_plan_t))
    assert mp.lib().moe_prefill_plan_pool(ptr) == 0
    assert b.base.slots == 2
    b.extra = 7
    assert mp.lib().moe_prefill_plan_pool(ptr) == mp.MOE_EINVAL
    assert "struct_size" in mp.moe_prefill_last_error()


# -------------------------------------------------------------- packer ---

def _unpack_blob_matrix(buf: np.ndarray, N: int, K: int, interleave_f: int):
    """Read the tiled Q4 layout back, following the header's documented format (with
    K % 64 == 32 the padded second block of the last pair must hold code 8, weight 0)."""
    sx4 = lambda v: v - 8                        # offset-binary nibble
    npairs, nbk = -(-K // 64), K // 32
    qs = buf[: N * npairs * 32].reshape(N // 32, npairs, 64, 16)
    W = np.zeros((N, K), np.int8)
    for nt in range(N // 32):
        for lane in range(64):
            j, h = lane % 32, lane // 32
            n = ((interleave_f if nt % 2 else 0) + (nt // 2) * 32 + j) if interleave_f else nt * 32 + j
            for pr in range(npairs):
                by = [int(v) for v in qs[nt, pr, lane]]
                for q in range(2):
                    k0 = 32 * (2 * pr + q) + 16 * h
                    if k0 >= K:
                        assert by[8 * q: 8 * q + 8] == [0x88] * 8
                        continue
                    for i in range(4):
                        W[n, k0 + i] = sx4(by[8 * q + i] & 15)
                        W[n, k0 + 4 + i] = sx4(by[8 * q + i] >> 4)
                        W[n, k0 + 8 + i] = sx4(by[8 * q + 4 + i] & 15)
                        W[n, k0 + 12 + i] = sx4(by[8 * q + 4 + i] >> 4)
    return W


@pytest.mark.parametrize("d,f", [(128, 64), (320, 192), (224, 96), (32, 32)])
def test_pack_expert_layout_round_trip(d, f):
    r = np.random.default_rng(0)
    wgu_q = r.integers(-8, 8, (2 * f, d)).astype(np.int8)
    wgu_s = r.integers(0, 65535, (2 * f, d // 32)).astype(np.uint16)
    wd_q = r.integers(-8, 8, (d, f)).astype(np.int8)
    wd_s = r.integers(0, 65535, (d, f // 32)).astype(np.uint16)
    eb = mp.moe_prefill_expert_bytes(d, f)
    out = np.zeros(eb, np.uint8)
    mp.moe_prefill_pack_expert(d, f, wgu_q, wgu_s, wd_q, wd_s, out.ctypes.data)
    ngd, ngf = -(-(d // 32) // 8), -(-(f // 32) // 8)     # 8-block scale groups
    pairs = lambda K: -(-K // 64)
    gu_q_bytes = 2 * f * pairs(d) * 32
    gu_s_off = (gu_q_bytes + 255) // 256 * 256
    d_q_off = gu_s_off + ((2 * f * ngd * 8 * 2 + 255) // 256) * 256
    d_s_off = d_q_off + ((d * pairs(f) * 32 + 255) // 256) * 256
    assert eb == d_s_off + ((d * ngf * 8 * 2 + 255) // 256) * 256
    assert np.array_equal(_unpack_blob_matrix(out, 2 * f, d, f), wgu_q)
    assert np.array_equal(_unpack_blob_matrix(out[d_q_off:], d, f, 0), wd_q)

    def scales(sec, N, nbk, ng, row_of):
        # (nt, group, j) -> 8 fp16 scales of blocks 8g .. 8g+7 (zero past the last block)
        sc = sec.view(np.uint16).reshape(N // 32, ng, 32, 8)
        for nt in range(N // 32):
            rows = row_of(nt)
            got = sc[nt].transpose(1, 0, 2).reshape(32, ng * 8)
            assert np.array_equal(got[:, :nbk], rows)
            assert not got[:, nbk:].any()

    scales(out[gu_s_off:gu_s_off + 2 * f * ngd * 16], 2 * f, d // 32, ngd,
           lambda nt: wgu_s[(f if nt % 2 else 0) + (nt // 2) * 32 + np.arange(32)])
    scales(out[d_s_off:d_s_off + d * ngf * 16], d, f // 32, ngf,
           lambda nt: wd_s[nt * 32:(nt + 1) * 32])


def test_pack_rejects_out_of_range_weights():
    d, f = 64, 64
    wgu_q = np.zeros((2 * f, d), np.int8)
    wgu_q[3, 5] = 8
    z = lambda *s: np.zeros(s, np.uint16)
    out = np.zeros(mp.moe_prefill_expert_bytes(d, f), np.uint8)
    with pytest.raises(mp.MoePrefillError) as ei:
        mp.moe_prefill_pack_expert(d, f, wgu_q, z(2 * f, 2), np.zeros((d, f), np.int8), z(d, 2), out.ctypes.data)
    assert ei.value.code == mp.MOE_EINVAL
