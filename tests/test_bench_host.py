"""Host-side parts of bench.py, on the CPU: the interval arithmetic behind the
copy/compute overlap figures, the trace summary on a synthetic rocprofv3 trace,
the kernel-source hash that gates the recorded HBM-traffic figures, and the
refusal of more than one GPU."""
import json
import os
import random
import shutil
import subprocess
import sys

import bench
import workload as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _covered(ivs):
    """Brute force: the set of unit cells [x, x+1) that the intervals cover."""
    cells = set()
    for a, b in ivs:
        cells.update(range(a, b))
    return cells


def test_interval_union_and_overlap_match_brute_force():
    rng = random.Random(5)
    for _ in range(300):
        iv1 = [(a, a + rng.randint(0, 12)) for a in (rng.randint(0, 80) for _ in range(rng.randint(0, 9)))]
        iv2 = [(a, a + rng.randint(0, 12)) for a in (rng.randint(0, 80) for _ in range(rng.randint(0, 9)))]
        u1, u2 = bench._intervals_union(iv1), bench._intervals_union(iv2)
        # the union is sorted, disjoint and covers exactly the same cells
        assert all(u1[i][1] < u1[i + 1][0] for i in range(len(u1) - 1))
        assert _covered(u1) == _covered(iv1)
        assert bench._overlap(u1, u2) == len(_covered(iv1) & _covered(iv2))


def _fake_trace(tmp_path, passes):
    """A kernel trace with one k_route_quant .. k_combine sequence per layer (100 ns
    each, back to back) and, during the timed passes of each stack, one 150 ns H2D
    copy per layer that starts halfway through the layer."""
    wins = bench.trace_windows(wl, passes)
    n_layers = max(hi for _, hi in wins.values())
    kern, copies = [], []
    t = 1000
    for layer in range(n_layers):
        kern.append(("k_route_quant(args)", t, t + 40))
        kern.append(("k_combine(args)", t + 40, t + 100))
        if any(lo <= layer < hi for lo, hi in wins.values()):
            copies.append(("MEMORY_COPY_HOST_TO_DEVICE", t + 50, t + 200, 4096))
        t += 300                                   # 200 ns idle after each layer's kernels
    d = tmp_path / "trace"
    d.mkdir()
    with open(d / "s_kernel_trace.csv", "w") as f:
        f.write("Kernel_Name,Start_Timestamp,End_Timestamp\n")
        for name, a, b in kern:
            f.write(f'"{name}",{a},{b}\n')
    with open(d / "s_memory_copy_trace.csv", "w") as f:
        f.write("Direction,Start_Timestamp,End_Timestamp,Bytes\n")
        for dirn, a, b, n in copies:
            f.write(f"{dirn},{a},{b},{n}\n")
    return str(d), wins


def test_trace_summary_on_a_synthetic_trace(tmp_path):
    passes = 2
    trace_dir, wins = _fake_trace(tmp_path, passes)
    out = bench.summarize_trace(trace_dir, passes)
    for key, (lo, hi) in wins.items():
        r = out[key]
        n = (hi - lo) // passes                    # layers per pass
        N = hi - lo                                # copies in the window
        # each copy (150 ns) overlaps 50 ns of its layer's kernels and nothing else; the
        # window ends with the last k_combine, which cuts the last copy to 50 ns
        copy_ns = 150 * N - 100
        assert r["h2d_copies"] == n
        assert r["copy_busy_ms_per_pass"] == round(copy_ns / passes / 1e6, 3)
        assert r["kernel_busy_ms_per_pass"] == round(100 * n / 1e6, 3)
        assert r["copy_hidden_frac"] == round(50 * N / copy_ns, 4)
        assert r["kernel_time_under_copies_frac"] == round(50 / 100, 4)
        assert r["h2d_GB_per_pass"] == round(4096 * n / 1e9, 3)
        # copies start every 300 ns and last 150 ns: 150 ns gaps between them
        assert r["copy_gap_ms"]["mean"] == round(150 / 1e6, 4)


def _hash_tree(tmp_path):
    d = tmp_path / "tree"
    csrc = d / "moe_prefill_ffn_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in ("moe_kernels.hip", "moe_kernels.h", "moe_layout.h"):
        shutil.copy(os.path.join(ROOT, "moe_prefill_ffn_amd", "csrc", f), csrc / f)
    return d, csrc


def test_source_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    d, csrc = _hash_tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(d))
    h0 = bench.kernel_source_hash()
    assert h0 == bench.kernel_source_hash()
    src = (csrc / "moe_kernels.hip").read_text()
    (csrc / "moe_kernels.hip").write_text("// a new comment line\n" + src.replace("\n\n", "\n\n/* block */\n", 1) + "\n\n")
    assert bench.kernel_source_hash() == h0
    assert "kRing = 4" in src
    (csrc / "moe_kernels.hip").write_text(src.replace("kRing = 4", "kRing = 3", 1))
    assert bench.kernel_source_hash() != h0


def test_traffic_figure_is_used_only_for_the_same_kernel_source(tmp_path, monkeypatch):
    d, _ = _hash_tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(d))
    prof = d / "profiles"
    prof.mkdir()
    assert bench.load_traffic("gemm_gate_up", "resident") is None          # no file
    rec = {"kernel_source_hash": bench.kernel_source_hash(), "hbm_bytes_per_launch": 123456}
    (prof / "traffic_gemm_gate_up_resident.txt").write_text("header\n\nJSON: " + json.dumps(rec))
    assert bench.load_traffic("gemm_gate_up", "resident") == 123456
    rec["kernel_source_hash"] = "0" * 16
    (prof / "traffic_gemm_gate_up_resident.txt").write_text("JSON: " + json.dumps(rec))
    assert bench.load_traffic("gemm_gate_up", "resident") is None          # other source


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single" in r.stderr
    assert r.stdout == ""
