#!/usr/bin/env python3
"""Benchmark of the MoE prompt (prefill) FFN layer on one MI355X.

One step = one whole layer through the C ABI (route + Xq, group, row table,
GU grouped GEMM with SwiGLU+requant, down grouped GEMM, combine).  The headline
is the largest configuration that fits one GPU: one resident layer of the
skewed stack's shape, T=8192 tokens, d_model=4096, d_ff=1536, E=256 experts,
top-8, Zipf(1.1) expert skew, Q4 weights resident in HBM, synthetic seeded
inputs.  value = tokens/s per layer.

Also reported on the same line:
  roofline      the gate/up grouped GEMM (the dominant kernel) of the headline
                layer: algorithmic int8 ops per launch / its mean device time,
                from HIP events on the launch stream over exactly the K timed
                layers, against the int8 MFMA dense peak (5.0 POPS), and against
                the measured MFMA-only peak and per-32-block epilogue ceiling
  denominators  microbenchmarks (libmoe_micro.so): int8 MFMA peak, the block
                epilogue ceiling in each arithmetic form, VALU instruction
                costs, a device copy, fp32 atomic adds
  resident_c1   the real-shape resident layer (T=1024, d_model=2048, d_ff=768,
                E=128, top-8), whose GEMMs are HBM-bound: its roofline against
                8 TB/s with the MFMA fraction beside it, per-kernel times, and
                the same layer captured in a HIP graph and replayed
  streamed      the 4-layer streamed stack (T=1024 shape, 2-slot pool, depth-1
                prefetch): tokens/s per pass, achieved H2D GB/s, measured PCIe
                GB/s, fraction of copy time hidden and overlap efficiency
  streamed_active_experts
                the first three layers of the skewed stack through a 2-slot pool:
                whole-layer streaming with depth-1 prefetch against active_only
                loads (only the routed experts, copied by a kernel after the
                routing): ms and GB per pass
  stacks        the two whole streamed stacks: 48 layers at T=3072 (4 resident
                leading layers, depth-2 prefetch, 7-slot budget) and the skewed 8-layer
                stack (3 slots, depth 2): tokens/s per pass, H2D GB/s achieved against
                the measured PCIe rate, copy-hidden fraction, overlap efficiency, and
                the resident per-layer kernel times and GEMM rates at those shapes
  cpu_baseline  the CPU oracle timed on this host's cores on a bounded token
                sample of the headline layer

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA, published
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
VALU_PEAK_TOPS = 78.6        # fp32 VALU lane-ops/s: 256 CU x 4 SIMD x 32 lanes x 2.4 GHz (fma = 1 op)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# how the streamed legs' overlap figures relate (hidden = copy + compute - wall time)
OVERLAP_NOTE = ("copy_hidden_frac = hidden / copy can be at most compute / copy "
                "(copy_hidden_frac_max) when the copies take longer than the compute; "
                "overlap_efficiency = hidden / min(copy, compute) is the share of the "
                "possible overlap achieved")


def kernel_source_hash() -> str:
    """Hash of the kernel sources with comments and blank space taken out, so that
    an edit of the comments alone keeps the recorded counter runs valid."""
    h = hashlib.sha256()
    for f in ("moe_kernels.hip", "moe_kernels.h", "moe_layout.h"):
        text = open(os.path.join(ROOT, "moe_prefill_ffn_amd", "csrc", f)).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source (else None)."""
    p = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(p):
        return None
    try:
        d = json.loads(open(p).read().split("JSON:", 1)[1])
    except Exception:
        return None
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def pack_blobs(mp, wl, torch, w, pinned: bool = True):
    """Pinned host blobs of every layer of workload w (generated and packed on the host cores)."""
    lb = mp.moe_prefill_layer_bytes(w.d, w.f, w.E)
    threads = max(1, min(16, os.cpu_count() or 1))
    blobs = []
    for l in range(w.n_layers):
        b = torch.empty(lb, dtype=torch.uint8, pin_memory=pinned)
        mp.pack_layer(w.d, w.f, w.E, lambda e, l=l: wl.expert_weights(w, l, e), b, threads=threads)
        blobs.append(b)
    return blobs, lb


def stack_leg(mp, wl, torch, dev, key: str, passes: int) -> dict:
    """One whole streamed stack: pass time through the slot pool with the workload's depth,
    slot count and VRAM budget, against the copy-only time (every streamed layer's blob over
    PCIe) and the compute-only time (every layer resident in HBM)."""
    w = wl.WORKLOADS[key]
    st = w.stream
    log(f"[bench] {w.name}: packing {w.n_layers} pinned layer blobs")
    t0 = time.perf_counter()
    blobs, lb = pack_blobs(mp, wl, torch, w)
    log(f"[bench] packed {w.n_layers} x {lb / 2**20:.0f} MiB in {time.perf_counter() - t0:.1f} s")
    xs = [torch.from_numpy(wl.layer_activations(w, l)).to(dev) for l in range(w.n_layers)]
    lgs = [torch.from_numpy(wl.layer_logits(w, l)).to(dev) for l in range(w.n_layers)]
    y = torch.empty(w.T, w.d, device=dev)
    h = mp.moe_prefill_create(w.d, w.f, w.E, w.k, w.T, device=0)
    R = w.T * w.k
    # compute only: all layers resident, per-kernel device times
    devb = [b.to(dev) for b in blobs]
    for l in range(w.n_layers):
        mp.moe_prefill_run_layer(h, xs[l], lgs[l], y, layer=-1, weights=devb[l])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(passes):
        for l in range(w.n_layers):
            mp.moe_prefill_run_layer(h, xs[l], lgs[l], y, layer=-1, weights=devb[l])
    torch.cuda.synchronize()
    t_comp_all = (time.perf_counter() - t0) / passes
    mp.moe_prefill_set_timing(h, True)
    for l in range(w.n_layers):
        mp.moe_prefill_run_layer(h, xs[l], lgs[l], y, layer=-1, weights=devb[l])
    torch.cuda.synchronize()
    kt = mp.moe_prefill_kernel_times(h, reset=True)
    mp.moe_prefill_set_timing(h, False)
    kern_us = {n: (ms / c * 1e3 if c else None) for n, (c, ms) in kt.items()}
    gu_tops = 2.0 * R * (2 * w.f) * w.d / (kern_us["gemm_gate_up"] * 1e-6) / 1e12
    dn_tops = 2.0 * R * w.d * w.f / (kern_us["gemm_down"] * 1e-6) / 1e12
    del devb
    torch.cuda.empty_cache()
    budget = st.budget_slots * lb if st.budget_slots else 0
    plan = mp.stream_pool_configure(h, blobs, prefetch_depth=st.depth, resident_layers=st.residents,
                                    max_vram_bytes=budget, requested_slots=st.slots)
    streamed = w.n_layers - plan["residents"]
    # copy only: the streamed layers' blobs, back to back on one stream (best of 2)
    dst = torch.empty(lb, dtype=torch.uint8, device=dev)
    t_copy = 1e9
    for _ in range(2):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for b in blobs[plan["residents"]:]:
            dst.copy_(b, non_blocking=True)
        torch.cuda.synchronize()
        t_copy = min(t_copy, time.perf_counter() - t0)
    del dst
    torch.cuda.empty_cache()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for l in range(w.n_layers):            # first (cold) pass: nothing prefetched yet
        mp.moe_prefill_run_layer(h, xs[l], lgs[l], y, layer=l)
    torch.cuda.synchronize()
    t_cold = time.perf_counter() - t0
    s0 = mp.moe_prefill_get_stats(h)
    t_pass = []
    for _ in range(passes):
        t0 = time.perf_counter()
        for l in range(w.n_layers):
            mp.moe_prefill_run_layer(h, xs[l], lgs[l], y, layer=l)
        torch.cuda.synchronize()
        t_pass.append(time.perf_counter() - t0)
    # the median pass: the host's PCIe share varies from pass to pass on a shared node
    t_wall = sorted(t_pass)[len(t_pass) // 2]
    s1 = mp.moe_prefill_get_stats(h)
    moved = (s1["bytes_h2d"] - s0["bytes_h2d"]) / passes
    pcie = streamed * lb / t_copy
    hidden = max(0.0, t_copy + t_comp_all - t_wall)
    out = {
        "workload": w.name, "layers": w.n_layers, "slots": plan["slots"], "depth": plan["depth"],
        "residents": plan["residents"], "streamed_layers": streamed,
        "tokens_per_s_per_pass": round(w.T / t_wall, 1), "ms_per_pass": round(t_wall * 1e3, 3),
        "ms_per_pass_all": [round(t * 1e3, 3) for t in t_pass],
        "cold_pass": {"ms": round(t_cold * 1e3, 3), "tokens_per_s": round(w.T / t_cold, 1)},
        "h2d_GB_per_pass": round(moved / 1e9, 3), "h2d_GBs_achieved": round(moved / t_wall / 1e9, 2),
        "pcie_h2d_GBs_measured": round(pcie / 1e9, 2),
        "pcie_roofline_frac": round((moved / pcie) / t_wall, 4) if pcie > 0 else None,
        "copy_ms_per_pass": round(t_copy * 1e3, 3), "compute_ms_per_pass": round(t_comp_all * 1e3, 3),
        "copy_hidden_frac": round(hidden / t_copy, 4) if t_copy > 0 else None,
        "copy_hidden_frac_max": round(min(1.0, t_comp_all / t_copy), 4) if t_copy > 0 else None,
        "overlap_efficiency": round(hidden / min(t_copy, t_comp_all), 4) if t_copy > 0 else None,
        "overlap_note": OVERLAP_NOTE,
        "prefetch_activated": (s1["prefetch_activated"] - s0["prefetch_activated"]) / passes,
        "sync_loads": (s1["sync_loads"] - s0["sync_loads"]) / passes,
        "resident_layer": {
            "us_per_layer": round(t_comp_all * 1e6 / w.n_layers, 1),
            "tokens_per_s_per_layer": round(w.T * w.n_layers / t_comp_all, 1),
            "kernels_us": {n: (round(v, 2) if v is not None else None) for n, v in kern_us.items()},
            "gemm_gate_up_TOPS": round(gu_tops, 2), "gemm_gate_up_frac": round(gu_tops / INT8_PEAK_TOPS, 4),
            "gemm_down_TOPS": round(dn_tops, 2), "gemm_down_frac": round(dn_tops / INT8_PEAK_TOPS, 4),
        },
    }
    h.close()
    del blobs, xs, lgs, y
    torch.cuda.empty_cache()
    return out


STACK_KEYS = ("stream48", "skew")


def trace_windows(wl, passes: int):
    """Per stack of the --stacks-only run: the half-open range of layer ordinals (counted
    over the whole run, in launch order) that are the timed streamed passes.  Each layer
    is one k_route_quant ... k_combine sequence; per stack the run does 1 + passes + 1
    compute-only passes, one cold streamed pass, then the timed streamed passes."""
    out, base = {}, 0
    for key in STACK_KEYS:
        n = wl.WORKLOADS[key].n_layers
        first = base + n * (passes + 2) + n
        out[key] = (first, first + n * passes)
        base = first + n * passes
    return out


def _intervals_union(iv):
    iv = sorted(iv)
    out = []
    for a, b in iv:
        if out and a <= out[-1][1]:
            out[-1][1] = max(out[-1][1], b)
        else:
            out.append([a, b])
    return out


def _overlap(u1, u2):
    i = j = 0
    tot = 0
    while i < len(u1) and j < len(u2):
        a = max(u1[i][0], u2[j][0])
        b = min(u1[i][1], u2[j][1])
        if b > a:
            tot += b - a
        if u1[i][1] < u2[j][1]:
            i += 1
        else:
            j += 1
    return tot


def summarize_trace(trace_dir: str, passes: int) -> dict:
    """Copy/compute overlap of the timed streamed passes, from rocprofv3's kernel and
    memory-copy traces of a `bench.py --stacks-only` run."""
    import csv
    import glob

    import workload as wl

    def one(pattern):
        f = sorted(glob.glob(os.path.join(trace_dir, "**", pattern), recursive=True))
        if not f:
            raise FileNotFoundError(f"no {pattern} under {trace_dir}")
        return list(csv.DictReader(open(f[0])))

    kern = one("*kernel_trace.csv")
    copies = one("*memory_copy_trace.csv")
    kiv = [(int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]) for r in kern]
    kiv.sort()
    rq = [iv for iv in kiv if iv[2].startswith("k_route_quant") or "k_route_quant" in iv[2]]
    cb = [iv for iv in kiv if "k_combine" in iv[2]]
    h2d = []
    for r in copies:
        dirn = r.get("Direction", "") + r.get("Operation", "") + r.get("Kind", "")
        if "HOST_TO_DEVICE" in dirn.upper() or "H2D" in dirn.upper():
            nbytes = None
            for key in ("Bytes", "Size", "Copy_Bytes"):
                if key in r and r[key] not in ("", None):
                    nbytes = int(r[key])
            h2d.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), nbytes))
    res = {}
    for key, (lo, hi) in trace_windows(wl, passes).items():
        if hi > len(rq) or hi > len(cb):
            res[key] = {"error": f"trace has {len(rq)} layers, window needs {hi}"}
            continue
        w0, w1 = rq[lo][0], cb[hi - 1][1]
        ku = _intervals_union([(a, b) for a, b, _ in kiv if b > w0 and a < w1])
        cin = [(max(a, w0), min(b, w1), n) for a, b, n in h2d if b > w0 and a < w1]
        cu = _intervals_union([(a, b) for a, b, _ in cin])
        copy_ns = sum(b - a for a, b in cu)
        kern_ns = sum(b - a for a, b in ku)
        hid = _overlap(cu, ku)
        nb = [n for _, _, n in cin]
        bytes_ = sum(nb) if nb and all(n is not None for n in nb) else None
        wall = (w1 - w0) / passes
        gaps = [cu[i + 1][0] - cu[i][1] for i in range(len(cu) - 1)]
        res[key] = {
            "window_ms_per_pass": round(wall / 1e6, 3),
            "h2d_copies": len(cin) / passes,
            "copy_busy_ms_per_pass": round(copy_ns / passes / 1e6, 3),
            "kernel_busy_ms_per_pass": round(kern_ns / passes / 1e6, 3),
            "copy_hidden_frac": round(hid / copy_ns, 4) if copy_ns else None,
            "kernel_time_under_copies_frac": round(hid / kern_ns, 4) if kern_ns else None,
            "h2d_GB_per_pass": round(bytes_ / passes / 1e9, 3) if bytes_ is not None else None,
            "h2d_GBs_over_window": round(bytes_ / (w1 - w0), 2) if bytes_ is not None else None,
            "h2d_GBs_while_copying": round(bytes_ / copy_ns, 2) if bytes_ and copy_ns else None,
            "copy_gap_ms": {"mean": round(sum(gaps) / len(gaps) / 1e6, 4) if gaps else None,
                            "max": round(max(gaps) / 1e6, 4) if gaps else None,
                            "total_per_pass": round(sum(gaps) / passes / 1e6, 3)},
        }
    return res


def gate_up_bytes(w, active: int) -> int:
    """Algorithmic HBM bytes of one gate/up launch: the active experts' Q4 gate/up weights
    (codes + fp16 scales), Xq + its scales read, Hq + its scales and the row table written."""
    R = w.T * w.k
    wgu = active * (2 * w.f * w.d // 2 + 2 * w.f * (w.d // 32) * 2)
    return wgu + w.T * w.d + w.T * (w.d // 32) * 4 + R * w.f + R * (w.f // 32) * 4 + R * 4


def down_bytes(w, active: int) -> int:
    """Algorithmic HBM bytes of one down launch: the active experts' Q4 down weights, Hq and
    its scales read, Dm written."""
    R = w.T * w.k
    wd = active * (w.d * w.f // 2 + w.d * (w.f // 32) * 2)
    return wd + R * w.f + R * (w.f // 32) * 4 + R * w.d * 4


def resident_leg(mp, wl, torch, dev, key: str, steps: int, warmup: int, micro, graph: bool = False,
                 events_in_timed: bool = True, atomic: bool = False) -> dict:
    """One resident layer of workload `key`, layer 0: W untimed layers, then K timed layers
    with HIP events between the kernels on the launch stream (the per-kernel device times of
    exactly the timed region), the gate/up GEMM's roofline and the memory-bound kernels' GB/s.
    events_in_timed=False: the K timed layers run without events and K more give the kernel
    times (a short layer's time is then free of the events' own cost)."""
    w = wl.WORKLOADS[key]
    T, d, f, E, k = w.T, w.d, w.f, w.E, w.k
    R = T * k
    log(f"[bench] {w.name}: generating inputs")
    x = torch.from_numpy(wl.layer_activations(w, 0)).to(dev)
    lg = torch.from_numpy(wl.layer_logits(w, 0)).to(dev)
    blob_h = torch.empty(mp.moe_prefill_layer_bytes(d, f, E), dtype=torch.uint8)
    mp.pack_layer(d, f, E, lambda e: wl.expert_weights(w, 0, e), blob_h, threads=max(1, min(16, os.cpu_count() or 1)))
    blob = blob_h.to(dev)
    del blob_h
    y = torch.empty(T, d, device=dev)
    h = mp.moe_prefill_create(d, f, E, k, T, device=0)
    stream = torch.cuda.current_stream(dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    mp.moe_prefill_run_layer(h, x, lg, y, layer=-1, weights=blob, stream=stream, exports={"counts": counts})
    active = int((counts.cpu() > 0).sum())

    def step():
        mp.moe_prefill_run_layer(h, x, lg, y, layer=-1, weights=blob, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    us_plain = None
    if not events_in_timed:       # the layer time without events, then the kernel times with them
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        us_plain = (time.perf_counter() - t0) * 1e6 / steps
    mp.moe_prefill_set_timing(h, True)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kt = mp.moe_prefill_kernel_times(h, reset=True)
    mp.moe_prefill_set_timing(h, False)
    us = (t1 - t0) * 1e6 / steps if us_plain is None else us_plain
    kern_us = {n: (ms / c * 1e3 if c else None) for n, (c, ms) in kt.items()}
    gu_us, dn_us = kern_us["gemm_gate_up"], kern_us["gemm_down"]
    ops_gu = 2.0 * R * (2 * f) * d           # int8 multiply-adds x 2, routed rows only
    ops_dn = 2.0 * R * d * f
    gu_tops = ops_gu / (gu_us * 1e-6) / 1e12
    dn_tops = ops_dn / (dn_us * 1e-6) / 1e12
    b_gu, b_dn = gate_up_bytes(w, active), down_bytes(w, active)
    gu_gbs = b_gu / (gu_us * 1e-6) / 1e9
    dn_gbs = b_dn / (dn_us * 1e-6) / 1e9
    ridge = INT8_PEAK_TOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    mfma = {"achieved": round(gu_tops, 2), "peak": INT8_PEAK_TOPS, "unit": "TOPS",
            "frac": round(gu_tops / INT8_PEAK_TOPS, 4)}
    hbm_roof = {"achieved": round(gu_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gu_gbs / HBM_PEAK_GBS, 4)}
    if micro:
        mfma["frac_of_measured_mfma_peak"] = round(gu_tops / micro["int8_mfma_peak_TOPS_measured"], 4)
        mfma["frac_of_epilogue_ceiling"] = round(gu_tops / micro["epilogue_ceiling_TOPS"], 4)
        hbm_roof["frac_of_measured_copy"] = round(gu_gbs / micro["copy_GBs"], 4)
    bound = "mfma" if ops_gu / b_gu > ridge else "hbm"
    roofline = dict(mfma if bound == "mfma" else hbm_roof)
    roofline.update({
        "bound": bound, "traffic": load_traffic("gemm_gate_up", key), "kernel": "gemm_gate_up",
        "workload": w.name, "ops_per_launch": ops_gu, "algorithmic_bytes_per_launch": b_gu,
        "arithmetic_intensity_ops_per_byte": round(ops_gu / b_gu, 1), "ridge_ops_per_byte": round(ridge, 1),
        "active_experts": active, "mean_us": round(gu_us, 2),
        "dtype": "int8 x int4 -> int32 blocks, fp32 epilogue",
        "note": "gate/up GEMM with the fused SwiGLU + Q8 epilogue (writes Hq, not GU); mean device time "
                "from HIP events on the launch stream over the timed layers",
    })
    roofline["mfma" if bound == "hbm" else "hbm"] = hbm_roof if bound == "mfma" else mfma
    q_bytes = T * E * 4 + R * 8 + T * d * 4 + T * d + T * (d // 32) * 4   # logits, eidx+w, X, Xq, dx
    c_bytes = R * d * 4 + R * 8 + T * d * 4
    out = {
        "workload": w.name, "us_per_layer": round(us, 2), "tokens_per_s_per_layer": round(T / (us * 1e-6), 1),
        "steps": steps, "warmup": warmup, "active_experts": active,
        "kernels_us": {n: (round(v, 2) if v is not None else None) for n, v in kern_us.items()},
        "roofline": roofline,
        "gemm_down": {"TOPS": round(dn_tops, 2), "frac_of_int8_peak": round(dn_tops / INT8_PEAK_TOPS, 4),
                      "GBs": round(dn_gbs, 1), "frac_of_hbm": round(dn_gbs / HBM_PEAK_GBS, 4),
                      "algorithmic_bytes_per_launch": b_dn, "mean_us": round(dn_us, 2)},
        "hbm": {"route_quant_GBs": round(q_bytes / (kern_us["route_quant"] * 1e-6) / 1e9, 1),
                "combine_GBs": round(c_bytes / (kern_us["combine"] * 1e-6) / 1e9, 1),
                "route_quant_bytes": q_bytes, "combine_bytes": c_bytes, "peak_GBs": HBM_PEAK_GBS},
    }
    # the whole layer against its floor: its int8 ops at the spec peak (and at the measured
    # per-block epilogue ceiling), or its unavoidable HBM bytes (the active experts' weights,
    # x, logits, y) at 8 TB/s, whichever is longer
    ops_layer = ops_gu + ops_dn
    min_bytes = active * mp.moe_prefill_expert_bytes(d, f) + T * d * 4 * 2 + T * E * 4
    floor_ops_us = ops_layer / (INT8_PEAK_TOPS * 1e12) * 1e6
    floor_hbm_us = min_bytes / (HBM_PEAK_GBS * 1e9) * 1e6
    floor_us = max(floor_ops_us, floor_hbm_us)
    out["layer_roofline"] = {
        "bound": "mfma" if floor_ops_us >= floor_hbm_us else "hbm", "floor_us": round(floor_us, 2),
        "frac": round(floor_us / us, 4), "int8_ops_per_layer": ops_layer, "min_hbm_bytes_per_layer": min_bytes,
        "floor_us_at_int8_peak": round(floor_ops_us, 2), "floor_us_at_hbm_peak": round(floor_hbm_us, 2),
    }
    if micro:
        ceil_us = ops_layer / (micro["epilogue_ceiling_TOPS"] * 1e12) * 1e6
        out["layer_roofline"]["floor_us_at_epilogue_ceiling"] = round(ceil_us, 2)
        out["layer_roofline"]["frac_of_epilogue_ceiling_floor"] = round(max(ceil_us, floor_hbm_us) / us, 4)
    if graph:
        out["graph_replay"] = graph_leg(mp, torch, h, x, lg, y, blob, stream, steps, warmup, T)
    if atomic:
        out["combine_atomic"] = atomic_leg(mp, torch, h, x, lg, y, blob, stream, steps, warmup, T, us,
                                           events_in_timed)
    h.close()
    del blob, x, lg, y
    torch.cuda.empty_cache()
    return out


def atomic_leg(mp, torch, h, x, lg, y, blob, stream, steps, warmup, T, us_gather,
               events_in_timed: bool = True) -> dict:
    """The same layer with the opt-in atomic combine (the down GEMM adds w * Dm into y,
    no Dm round trip, no gather kernel): its time and kernel times, timed the way the
    gather's layer time was, and its largest difference from the gather's y (the order
    of the fp32 adds varies)."""
    y_ref = y.clone()
    y_at = torch.empty_like(y)

    def step():
        mp.moe_prefill_run_layer(h, x, lg, y_at, layer=-1, weights=blob, stream=stream, combine="atomic")

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    us_plain = None
    if not events_in_timed:
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        us_plain = (time.perf_counter() - t0) * 1e6 / steps
    mp.moe_prefill_set_timing(h, True)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    us_at = (time.perf_counter() - t0) * 1e6 / steps if us_plain is None else us_plain
    kt = mp.moe_prefill_kernel_times(h, reset=True)
    mp.moe_prefill_set_timing(h, False)
    diff = (y_at - y_ref).abs().max().item()
    scale = y_ref.abs().max().item()
    return {"us_per_layer": round(us_at, 2), "tokens_per_s_per_layer": round(T / (us_at * 1e-6), 1),
            "saving_us_vs_gather": round(us_gather - us_at, 2),
            "kernels_us": {n: (round(ms / c * 1e3, 2) if c else None) for n, (c, ms) in kt.items()},
            "max_abs_diff_vs_gather": diff, "max_abs_y": scale,
            "note": "gemm_down includes zeroing y and the atomic adds; combine is only the mask clear"}


def graph_leg(mp, torch, h, x, lg, y, blob, stream, steps, warmup, T) -> dict:
    """The same resident layer captured once in a HIP graph and replayed (inputs in place)."""
    try:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            mp.moe_prefill_run_layer(h, x, lg, y, layer=-1, weights=blob, stream=side)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, capture_error_mode="thread_local"):
            mp.moe_prefill_run_layer(h, x, lg, y, layer=-1, weights=blob)
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        us_graph = (time.perf_counter() - t0) * 1e6 / steps
        del g
        return {"us_per_layer": round(us_graph, 2), "tokens_per_s_per_layer": round(T / (us_graph * 1e-6), 1)}
    except Exception as ex:          # reported, never fatal: the direct path is the measurement
        log(f"[bench] graph capture failed: {ex}")
        return {"error": str(ex)[:200]}


def cpu_leg(wl, w, seconds: float) -> dict:
    """The CPU oracle as it stands, on the host's cores, on a bounded sample of the layer:
    routing, grouping and Q8 of all T tokens plus every stage of the sampled tokens' rows.
    Two probes (64 and 256 tokens) size the sample to about `seconds` of oracle time."""
    import numpy as np

    import oracle

    x = wl.layer_activations(w, 0)
    lg = wl.layer_logits(w, 0)
    perm = np.random.default_rng(1234).permutation(w.T)
    eidx, _ = oracle.route(lg, w.k)
    cache = {}

    def pregen(toks):               # inputs of the timed call, generated before it
        for e in np.unique(eidx[toks]):
            if int(e) not in cache:
                cache[int(e)] = wl.expert_weights(w, 0, int(e))

    def timed(toks):
        pregen(toks)
        t0 = time.perf_counter()
        oracle.layer(x, lg, w.k, cache.__getitem__, w.f, tokens=toks)
        return time.perf_counter() - t0

    t64 = timed(perm[:64])                  # two probes: fixed cost (all tokens' routing, grouping,
    t256 = timed(perm[:256])                # Q8) + a cost per sampled token
    per_tok = max((t256 - t64) / 192, 1e-6)
    fixed = max(t64 - 64 * per_tok, 0.0)
    n = int(min(w.T, max(256, round((seconds - fixed) / per_tok))))
    toks = perm[:n]
    t = timed(toks)
    return {"value": round(n / t, 1), "unit": "tokens/s per layer", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{n} of the {w.T} tokens of {w.name} layer 0 (seeded random sample): routing, "
                      f"grouping and Q8 of all tokens plus every stage of the sampled tokens' {n * w.k} rows, "
                      f"{t:.1f} s (expert weights generated before the timed call)"}


def micro_leg(torch, dev) -> dict:
    """Measured denominators (libmoe_micro.so): the int8 MFMA peak, the per-32-block
    epilogue ceiling of the grouped GEMMs in each arithmetic form (register-only loops:
    MFMAs + the block epilogue, no memory), single-instruction VALU rates, a device copy
    and fp32 atomic adds into scattered rows."""
    from moe_prefill_ffn_amd import micro

    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    spec_mac_clk = INT8_PEAK_TOPS * 1e12 / 2 / (n_cu * 4 * 2.4e9)   # MACs per clock per SIMD at the spec
    out = {"n_cu": n_cu, "spec_int8_mac_per_clk_per_simd": round(spec_mac_clk, 1)}
    micro.block("mfma_i8", 2000, n_cu)                                # warm the clocks

    def simd_cycles(r, iters):
        """SIMD cycles per loop iteration: the launch's event time at the shader clock the
        waves read over their loops.  Every SIMD holds the same waves for the whole launch
        (n_cu x wps workgroups of four waves), so this is each SIMD's time; a wave's own
        cycle count is not, since the SIMD issues oldest-first and the waves that start
        first finish first."""
        return r["ms"] * 1e-3 * r["clock_ghz"] * 1e9 / iters

    forms = {}
    for name, iters in (("mfma_i8", 40000), ("cvt_fma_mscale", 20000), ("cvt_fma_vscale", 20000),
                        ("sub_fma_vscale", 20000), ("sub_fma_mscale", 20000), ("pipe_cvt_fma", 20000),
                        ("overlap_indep", 20000), ("f8split_fma_mscale", 20000), ("f6split_fma_mscale", 20000)):
        for wps in (4, 2):
            r = micro.block(name, iters, n_cu, wps)
            macs_iter = (4 if name == "mfma_i8" else 2) * 32768
            mac_clk = wps * macs_iter / simd_cycles(r, iters)
            forms[f"{name}@{wps}w"] = {
                "TOPS": round(r["work"] / (r["ms"] * 1e-3) / 1e12, 1),
                "frac_of_spec_peak": round(r["work"] / (r["ms"] * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
                "mac_per_clk_per_simd": round(mac_clk, 1),
                "frac_of_spec_per_clock": round(mac_clk / spec_mac_clk, 4),
                "clock_ghz": round(r["clock_ghz"], 3),
            }
    out["block_forms"] = forms
    out["int8_mfma_peak_TOPS_measured"] = forms["mfma_i8@4w"]["TOPS"]
    # the ceiling of the arithmetic the GEMMs run (int8 MFMA block sums); the fp8 x fp6 and
    # fp6 x fp6 split forms are alternative designs, reported beside it
    best = max((v["TOPS"], k) for k, v in forms.items()
               if not k.startswith(("mfma_i8", "overlap_indep", "f8split", "f6split")))
    out["epilogue_ceiling_TOPS"] = best[0]
    out["epilogue_ceiling_form"] = best[1]
    valu = {}
    for name in ("valu_fma", "valu_cvt", "valu_sub"):
        iters = 20000
        r = micro.block(name, iters, n_cu, 4)
        valu[name] = round(simd_cycles(r, iters) / (4 * 64), 3)   # SIMD cycles per wave64 instruction
    out["valu_cycles_per_wave_instr"] = valu
    # co-execution: SIMD cycles per loop iteration of the single-kind loops (per wave and
    # iteration: 64 fmas, 64 converts, four int8 MFMAs, two scale-product MFMAs taken at once
    # or chained through C) beside the loops that issue both kinds (two int8 MFMAs + 64 fmas
    # or converts; one scale-product MFMA + 64 fmas with its result taken at once, or
    # chained through C beside 64 fmas or converts), the VALU work independent of the MFMAs
    coexec = {}
    for wps in (1, 4):
        row = {}
        for name in ("valu_fma", "valu_cvt", "mfma_i8", "mfma_f32_scale", "mfma_f32_chain", "overlap_indep",
                     "overlap_cvt", "overlap_scale_fma", "overlap_scale_chain", "overlap_scale_cvt"):
            r = micro.block(name, 20000, n_cu, wps)
            row[name] = round(simd_cycles(r, 20000), 1)
        coexec[f"{wps}w"] = row
    out["coexec_simd_cycles_per_iter"] = coexec
    # matrix-core cycles per instruction with four waves per SIMD (four per wave and iteration):
    # int8 32x32x32 against fp6 x fp6 32x32x64
    rates = {}
    for name, key in (("mfma_i8", "i8_32x32x32"), ("mfma_f6", "f6_32x32x64")):
        iters = 20000
        r = micro.block(name, iters, n_cu, 4)
        rates[key] = round(simd_cycles(r, iters) / (4 * 4), 2)
    out["mfma_cycles_per_instr"] = rates
    iters = 20000
    r = micro.block("mfma_f32_scale", iters, n_cu, 4)
    # SIMD cycles per scale-product MFMA (4 waves per SIMD, 2 per iteration) and products/s
    out["mfma_f32_scale"] = {"cycles_per_instr": round(simd_cycles(r, iters) / (4 * 2), 2),
                             "G_products_per_s": round(r["work"] / 2 / (r["ms"] * 1e-3) / 1e9, 1)}
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    r = micro.copy(dst, src, n_cu * 16, 10)
    out["copy_GBs"] = round(r["work"] / (r["ms"] * 1e-3) / 1e9, 1)
    del src, dst
    rows, d, k = 8192, 2048, 8
    g = torch.Generator().manual_seed(5)
    perm = torch.randperm(rows, generator=g).to(torch.int32)
    dst_row = (perm // k).to(dev)
    srcm = torch.ones(rows, d, dtype=torch.float32, device=dev)
    y = torch.zeros(rows // k, d, dtype=torch.float32, device=dev)
    r = micro.atomic(srcm, dst_row, y, 10)
    out["atomic_add_f32"] = {"rows": rows, "d": d, "dest_rows": rows // k, "ms": round(r["ms"], 4),
                             "G_atomics_per_s": round(rows * d / (r["ms"] * 1e-3) / 1e9, 1),
                             "GBs": round(r["work"] / (r["ms"] * 1e-3) / 1e9, 1)}
    torch.cuda.synchronize()
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=300,
                    help="untimed layers first: the MI355X needs ~40 ms of sustained work to reach "
                         "its steady clocks (a cold layer takes ~290 us, a warm one ~195 us)")
    ap.add_argument("--stream-passes", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="target CPU time of the oracle baseline's token sample")
    ap.add_argument("--no-micro", action="store_true", help="skip the microbenchmark denominators")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the headline layer (no denominators, no T=1024 layer, no streaming, no CPU "
                         "baseline): the command the kernel-trace and counter profiles run")
    ap.add_argument("--workload", default="skew", choices=("skew", "resident", "stream48"),
                    help="with --headline-only: the layer to run (the T=1024 layer, or a resident layer of "
                         "the 48-layer stack's shape, for their own profiles)")
    ap.add_argument("--no-stream", action="store_true")
    ap.add_argument("--no-active", action="store_true", help="skip the active-expert streaming comparison")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-stacks", action="store_true", help="skip the 48-layer and skewed 8-layer stacks")
    ap.add_argument("--stack-passes", type=int, default=3)
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="summarise rocprofv3 kernel + memory-copy traces of a --stacks-only run")
    ap.add_argument("--stacks-only", action="store_true",
                    help="only the two whole streamed stacks (for traces of the streaming)")
    ap.add_argument("--micro", action="store_true",
                    help="only the microbenchmarks that set the roofline denominators")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain 256 MiB device-to-device copies (counter scale reference)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the MoE prefill FFN path here runs on a single "
              "MI355X (no layer split, no collectives); run it with --gpus 1", file=sys.stderr)
        return 2

    if args.summarize_trace:
        print(json.dumps(summarize_trace(args.summarize_trace, args.stack_passes), indent=1))
        return 0

    import numpy as np
    import torch

    import moe_prefill_ffn_amd as mp
    import workload as wl

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        # a plain copy of known size: reads and writes exactly 256 MiB per launch
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_launch": src.numel() * 4, "launches": 5}))
        return 0
    if args.micro:
        print(json.dumps({"micro": micro_leg(torch, dev)}), flush=True)
        return 0
    if args.stacks_only:
        out = {key: stack_leg(mp, wl, torch, dev, key, args.stack_passes) for key in STACK_KEYS}
        print(json.dumps({"stacks": out}), flush=True)
        return 0
    # ---- measured denominators first (this also brings the clocks to their loaded state)
    if args.workload != "skew" and not args.headline_only:
        print("--workload applies to --headline-only runs", file=sys.stderr)
        return 2
    if args.headline_only:
        args.no_micro = args.no_stream = args.no_cpu = True
    micro = None
    if not args.no_micro:
        micro = micro_leg(torch, dev)
        log(f"[bench] micro: int8 MFMA {micro['int8_mfma_peak_TOPS_measured']} TOPS, epilogue ceiling "
            f"{micro['epilogue_ceiling_TOPS']} TOPS ({micro['epilogue_ceiling_form']}), copy {micro['copy_GBs']} GB/s")

    # ---- headline: the largest single-GPU configuration, one resident layer of the skewed
    # 8-layer stack's shape (T=8192, d_model=4096, d_ff=1536, E=256, top-8, Zipf routing)
    # (the opt-in atomic combine is timed as an extra key, outside --headline-only, whose
    # kernel traces must hold the default path's launches only)
    head = resident_leg(mp, wl, torch, dev, args.workload, args.steps, args.warmup, micro,
                        atomic=not args.headline_only)
    w = wl.WORKLOADS[args.workload]
    log(f"[bench] headline {w.name}: {head['us_per_layer']:.1f} us/layer -> "
        f"{head['tokens_per_s_per_layer']:,.0f} tokens/s per layer; gate/up GEMM "
        f"{head['roofline']['achieved']} TOPS = {100 * head['roofline']['frac']:.2f}% of int8 peak")

    # ---- the real-shape resident layer (T=1024, d_model=2048, d_ff=768, E=128, top-8): HBM-bound GEMMs
    c1 = None
    if not args.headline_only:
        # a short layer: its own warm-up to steady clocks and a longer timed run (extra key)
        c1 = resident_leg(mp, wl, torch, dev, "resident", max(args.steps, 200), max(args.warmup, 300), micro,
                          graph=True, events_in_timed=False, atomic=True)
        log(f"[bench] {c1['workload']}: {c1['us_per_layer']:.1f} us/layer; gate/up GEMM "
            f"{c1['roofline']['achieved']} GB/s = {100 * c1['roofline']['frac']:.1f}% of HBM")

    line = {
        "metric": "MoE prefill tokens/s per layer (1 GPU); int8 MFMA %peak; H2D GB/s hidden %",
        "value": head["tokens_per_s_per_layer"], "unit": "tokens/s per layer", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(head["us_per_layer"] / 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic (seeded N(0,1) activations, N(0,1) logits + Zipf(1.1) expert bias, "
                "Q4 uniform int4 weights)",
        "config": {"workload": w.name, "T": w.T, "d_model": w.d, "d_ff": w.f, "n_experts": w.E, "top_k": w.k,
                   "weights": "resident in HBM", "global_batch": w.T, "seq_len": w.T, "parallelism": "none"},
        "roofline": head["roofline"], "layer_roofline": head["layer_roofline"],
        "kernels_us": head["kernels_us"], "hbm": head["hbm"],
        "gemm_down": head["gemm_down"], "combine_atomic": head.get("combine_atomic"), "denominators": micro,
        "resident_c1": c1,
    }
    # ---- streamed stack: 4 layers through a 2-slot pool with depth-1 prefetch
    if not args.no_stream:
        ws = wl.WORKLOADS["stream4"]
        log(f"[bench] {ws.name}: packing {ws.n_layers} pinned layer blobs")
        lb = mp.moe_prefill_layer_bytes(ws.d, ws.f, ws.E)
        blobs = []
        for l in range(ws.n_layers):
            b = torch.empty(lb, dtype=torch.uint8, pin_memory=True)
            mp.pack_layer(ws.d, ws.f, ws.E, lambda e, l=l: wl.expert_weights(ws, l, e), b)
            blobs.append(b)
        xs = [torch.from_numpy(wl.layer_activations(ws, l)).to(dev) for l in range(ws.n_layers)]
        lgs = [torch.from_numpy(wl.layer_logits(ws, l)).to(dev) for l in range(ws.n_layers)]
        ys = torch.empty(ws.T, ws.d, device=dev)
        hs = mp.moe_prefill_create(ws.d, ws.f, ws.E, ws.k, ws.T, device=0)
        # raw pinned H2D bandwidth (best of 3 over the whole stack)
        dst = torch.empty(lb, dtype=torch.uint8, device=dev)
        t_copy = 1e9
        for _ in range(3):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for b in blobs:
                dst.copy_(b, non_blocking=True)
            torch.cuda.synchronize()
            t_copy = min(t_copy, time.perf_counter() - t0)
        # compute only: the same layers resident
        devb = [b.to(dev) for b in blobs]
        for _ in range(2):
            for l in range(ws.n_layers):
                mp.moe_prefill_run_layer(hs, xs[l], lgs[l], ys, layer=-1, weights=devb[l])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.stream_passes):
            for l in range(ws.n_layers):
                mp.moe_prefill_run_layer(hs, xs[l], lgs[l], ys, layer=-1, weights=devb[l])
        torch.cuda.synchronize()
        t_comp = (time.perf_counter() - t0) / args.stream_passes
        del devb, dst
        torch.cuda.empty_cache()
        plan = mp.stream_pool_configure(hs, blobs, prefetch_depth=ws.stream.depth,
                                        resident_layers=ws.stream.residents,
                                        requested_slots=ws.stream.slots)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for l in range(ws.n_layers):       # first (cold) pass: nothing prefetched yet
            mp.moe_prefill_run_layer(hs, xs[l], lgs[l], ys, layer=l)
        torch.cuda.synchronize()
        t_cold = time.perf_counter() - t0
        s0 = mp.moe_prefill_get_stats(hs)
        t0 = time.perf_counter()
        for _ in range(args.stream_passes):
            for l in range(ws.n_layers):
                mp.moe_prefill_run_layer(hs, xs[l], lgs[l], ys, layer=l)
        torch.cuda.synchronize()
        t_wall = (time.perf_counter() - t0) / args.stream_passes
        s1 = mp.moe_prefill_get_stats(hs)
        moved = (s1["bytes_h2d"] - s0["bytes_h2d"]) / args.stream_passes
        hidden = max(0.0, t_copy + t_comp - t_wall)
        line["streamed"] = {
            "workload": ws.name, "layers": ws.n_layers, "slots": plan["slots"], "depth": plan["depth"],
            "tokens_per_s_per_pass": round(ws.T / t_wall, 1),
            "ms_per_pass": round(t_wall * 1e3, 3), "ms_per_layer": round(t_wall * 1e3 / ws.n_layers, 3),
            "cold_pass": {"ms": round(t_cold * 1e3, 3), "tokens_per_s": round(ws.T / t_cold, 1)},
            "h2d_GBs_achieved": round(moved / t_wall / 1e9, 2),
            "pcie_h2d_GBs_measured": round(ws.n_layers * lb / t_copy / 1e9, 2),
            "copy_ms_per_pass": round(t_copy * 1e3, 3), "compute_ms_per_pass": round(t_comp * 1e3, 3),
            "copy_hidden_frac": round(hidden / t_copy, 4),
            "copy_hidden_frac_max": round(min(1.0, t_comp / t_copy), 4),
            "overlap_efficiency": round(hidden / min(t_copy, t_comp), 4),
            "overlap_note": OVERLAP_NOTE,
            "prefetch_activated": s1["prefetch_activated"] - s0["prefetch_activated"],
            "sync_loads": s1["sync_loads"] - s0["sync_loads"],
        }
        log(f"[bench] streamed: {line['streamed']}")
        hs.close()
        del blobs
        torch.cuda.empty_cache()

    # ---- active-expert streaming: the first three layers of the skewed stack through a
    # 2-slot pool, whole-layer streaming (depth-1 prefetch) against loading only the routed
    # experts after routing
    if not args.no_stream and not args.no_active:
        wk = wl.WORKLOADS["skew"]
        nl = 3
        log(f"[bench] {wk.name}: packing {nl} pinned layer blobs")
        lbk = mp.moe_prefill_layer_bytes(wk.d, wk.f, wk.E)
        kblobs = []
        for l in range(nl):
            b = torch.empty(lbk, dtype=torch.uint8, pin_memory=True)
            mp.pack_layer(wk.d, wk.f, wk.E, lambda e, l=l: wl.expert_weights(wk, l, e), b)
            kblobs.append(b)
        kx = [torch.from_numpy(wl.layer_activations(wk, l)).to(dev) for l in range(nl)]
        klg = [torch.from_numpy(wl.layer_logits(wk, l)).to(dev) for l in range(nl)]
        ky = torch.empty(wk.T, wk.d, device=dev)
        hk = mp.moe_prefill_create(wk.d, wk.f, wk.E, wk.k, wk.T, device=0)

        def passes(active: bool):
            plan = mp.stream_pool_configure(hk, kblobs, prefetch_depth=1, resident_layers=0,
                                            requested_slots=2, active_only=active)
            for l in range(nl):            # first (cold) pass
                mp.moe_prefill_run_layer(hk, kx[l], klg[l], ky, layer=l)
            torch.cuda.synchronize()
            s0 = mp.moe_prefill_get_stats(hk)
            t0 = time.perf_counter()
            for _ in range(args.stream_passes):
                for l in range(nl):
                    mp.moe_prefill_run_layer(hk, kx[l], klg[l], ky, layer=l)
            torch.cuda.synchronize()
            t = (time.perf_counter() - t0) / args.stream_passes
            s1 = mp.moe_prefill_get_stats(hk)
            moved = (s1["bytes_h2d"] - s0["bytes_h2d"] + s1["bytes_sparse"] - s0["bytes_sparse"]) / args.stream_passes
            return plan, t, moved, (s1["experts_loaded"] - s0["experts_loaded"]) / args.stream_passes

        plan_f, t_full, moved_f, _ = passes(False)
        plan_a, t_act, moved_a, experts = passes(True)
        line["streamed_active_experts"] = {
            "workload": wk.name + f" (layers 0-{nl - 1})", "layers": nl,
            "whole_layer": {"slots": plan_f["slots"], "depth": plan_f["depth"],
                            "ms_per_pass": round(t_full * 1e3, 3), "GB_per_pass": round(moved_f / 1e9, 3),
                            "h2d_GBs_achieved": round(moved_f / t_full / 1e9, 2),
                            "tokens_per_s_per_pass": round(wk.T / t_full, 1)},
            "active_only": {"slots": plan_a["slots"], "depth": plan_a["depth"],
                            "ms_per_pass": round(t_act * 1e3, 3), "GB_per_pass": round(moved_a / 1e9, 3),
                            "h2d_GBs_achieved": round(moved_a / t_act / 1e9, 2),
                            "experts_per_pass": experts, "experts_total": nl * wk.E,
                            "tokens_per_s_per_pass": round(wk.T / t_act, 1)},
            "speedup": round(t_full / t_act, 3),
        }
        log(f"[bench] active-expert streaming: {line['streamed_active_experts']}")
        hk.close()
        del kblobs, kx, klg, ky
        torch.cuda.empty_cache()

    # ---- whole streamed stacks: the 48-layer prompt stack (T=3072, 4 resident leading layers,
    # depth 2) and the skewed 8-layer stack (T=8192, d_model=4096, d_ff=1536, E=256, 3 slots,
    # depth 2), each with its compute-only (all layers resident) and copy-only times
    if not args.no_stream and not args.no_stacks:
        line["stacks"] = {}
        for key in STACK_KEYS:
            line["stacks"][key] = stack_leg(mp, wl, torch, dev, key, args.stack_passes)
            log(f"[bench] stack {key}: {line['stacks'][key]}")

    # ---- CPU oracle on the host's cores, the headline layer on a bounded token sample
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_leg(wl, w, args.cpu_seconds)
        log(f"[bench] cpu oracle: {line['cpu_baseline']}")

    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
