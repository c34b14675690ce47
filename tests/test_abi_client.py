"""A C99 program built with gcc against include/moe_prefill.h and linked to
libmoe_prefill.so (tests/abi_client.c): the struct layouts a C compiler gives the
public header must equal the ctypes layouts of the Python binding field by
field, and the library must accept the structs of a client compiled against
an older header (undersized), a current one, and a newer one (oversized with a
zero tail; a nonzero unknown tail is refused) -- the checks the layer-streaming
page lists under "Verification" (stable-diffusion.cpp #1905: current and
undersized versioned C API structures, an executable built against the
previous public API).  The GPU test runs a resident layer and a two-layer
pool from C through the first published struct layouts."""
import ctypes
import json
import os
import subprocess

import numpy as np
import pytest

import moe_prefill_ffn_amd as mp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "moe_prefill_ffn_amd")
SRC = os.path.join(ROOT, "tests", "abi_client.c")


def _build(out_dir, gpu=False):
    exe = os.path.join(str(out_dir), "abi_client_gpu" if gpu else "abi_client")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include")]
    if gpu:
        cmd += ["-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__", "-DABI_CLIENT_GPU"]
    cmd += [SRC, "-L", LIBDIR, "-l:libmoe_prefill.so"]
    rpath = LIBDIR
    if gpu:
        cmd += ["-L/opt/rocm/lib", "-lamdhip64"]
        rpath += ":/opt/rocm/lib"
    cmd += [f"-Wl,-rpath,{rpath}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.fixture(scope="module")
def client(tmp_path_factory):
    mp.lib()                                   # the library must be built
    return _build(tmp_path_factory.mktemp("abi"))


def _run(exe, *args, timeout=60):
    r = subprocess.run([exe, *map(str, args)], capture_output=True, text=True, timeout=timeout)
    assert r.returncode == 0, r.stdout + r.stderr
    return json.loads(r.stdout.strip().splitlines()[-1])


STRUCTS = ["moe_prefill_params_t", "moe_layer_io_t", "stream_pool_params_t", "stream_pool_budget_t",
           "moe_pool_plan_t", "moe_pool_trim_t", "moe_stats_t", "moe_kernel_times_t"]


def test_c_layouts_equal_the_binding_layouts(client):
    lay = _run(client, "layout")
    assert lay["abi_version"] == 1
    for name in STRUCTS:
        cls = getattr(mp, name)
        c = lay[name]
        assert c["size"] == ctypes.sizeof(cls), name
        assert list(c["fields"]) == [f for f, _ in cls._fields_], name
        for f, off in c["fields"].items():
            assert getattr(cls, f).offset == off, (name, f)


def test_first_published_layouts_are_prefixes_of_the_current_ones(client):
    lay = _run(client, "layout")
    v1 = lay["v1_sizes"]
    assert v1["stream_pool_params_v1"] == lay["stream_pool_params_t"]["fields"]["active_only"]
    assert v1["moe_stats_v1"] == lay["moe_stats_t"]["fields"]["sparse_loads"]
    assert v1["moe_layer_io_v1"] == lay["moe_layer_io_t"]["fields"]["combine"]


def test_current_undersized_and_oversized_structs(client):
    r = _run(client, "host")
    assert r["rc_ws_current"] == 0 and r["rc_ws_undersized"] == 0
    assert r["ws_current"] == r["ws_undersized"] > 0
    assert r["rc_oversized_zero_tail"] == 0
    assert (r["plan_slots"], r["plan_residents"], r["plan_depth"]) == (7, 4, 2)
    assert r["struct_size_kept"] == r["expected_oversized_size"]     # the caller's size stays
    assert r["rc_oversized_nonzero_tail"] == mp.MOE_EINVAL
    assert "nonzero" in r["err_oversized"]
    assert r["rc_trim"] == 0 and r["trim_new_residents"] == 2 and r["trim_released"] == 2
    assert r["rc_exp"] == 0 and abs(r["exp1"] - np.e) < 1e-6


def test_create_without_a_gpu_fails_clearly(client):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    r = _run(client, "host")
    assert r["rc_create"] == mp.MOE_EUNSUPPORTED and r["create_out_null"] == 1


@pytest.mark.gpu
def test_c_client_runs_a_layer_and_a_pool_through_old_struct_layouts(tmp_path):
    import oracle
    import workload as wl
    from gpu_helpers import ExpertCache, assert_close, assert_equal, host_blob, say

    say("[case] C client: resident layer + 2-layer pool through v1 structs")
    exe = _build(tmp_path, gpu=True)
    w = wl.WORKLOADS["tiny"]
    x = wl.layer_activations(w, 0)
    lg = wl.layer_logits(w, 0)
    ex = ExpertCache(w, 0)
    blob = host_blob(w, ex).numpy()
    x.tofile(tmp_path / "x.bin")
    lg.tofile(tmp_path / "logits.bin")
    blob.tofile(tmp_path / "blob.bin")
    r = _run(exe, "gpu", tmp_path, w.T, w.d, w.f, w.E, w.k, timeout=110)
    assert r["rc_create"] == 0 and r["rc_resident"] == 0 and r["rc_atomic"] == 0
    assert r["rc_pool"] == 0 and (r["eff_slots"], r["eff_depth"], r["eff_residents"]) == (2, 1, 0)
    assert r["rc_layer0"] == 0 and r["rc_layer1"] == 0 and r["rc_stats"] == 0
    assert r["pool_struct_size_kept"] == 64 and r["stats_struct_size_kept"] == 72
    assert r["layers_run"] == 4 and r["sync_loads"] == 1 and r["prefetch_activated"] == 1
    y_res = np.fromfile(tmp_path / "y_res.bin", dtype=np.float32).reshape(w.T, w.d)
    ref = oracle.layer(x, lg, w.k, ex, w.f)
    assert_close("C client y", y_res, ref["y"])
    for name in ("y_pool0.bin", "y_pool1.bin"):
        assert_equal(name, np.fromfile(tmp_path / name, dtype=np.float32).reshape(w.T, w.d), y_res)
    assert_close("C client y, atomic combine",
                 np.fromfile(tmp_path / "y_atomic.bin", dtype=np.float32).reshape(w.T, w.d), ref["y"])
