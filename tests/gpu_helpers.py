"""Shared helpers for the GPU tests: seeded inputs, packed blobs, running one
layer through the C ABI with every intermediate exported, and the parity
checks against the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import moe_prefill_ffn_amd as mp
import oracle
import workload as wl


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class ExpertCache:
    """expert e -> canonical weights, generated on demand (optionally kept)."""

    def __init__(self, w: wl.Workload, layer: int, keep: bool = True, override=None):
        self.w, self.layer, self.keep, self.override = w, layer, keep, override
        self.cache = {}

    def __call__(self, e):
        if e in self.cache:
            return self.cache[e]
        W = self.override(e) if self.override else wl.expert_weights(self.w, self.layer, e)
        if self.keep:
            self.cache[e] = W
        return W


def host_blob(w: wl.Workload, experts, pinned: bool = False) -> torch.Tensor:
    nbytes = mp.moe_prefill_layer_bytes(w.d, w.f, w.E)
    out = torch.empty(nbytes, dtype=torch.uint8, pin_memory=pinned)
    return mp.pack_layer(w.d, w.f, w.E, experts, out)


def make_handle(w: wl.Workload, max_tokens=None):
    return mp.moe_prefill_create(w.d, w.f, w.E, w.k, max_tokens or w.T, device=0)


EXPORT_SHAPES = {
    "eidx": lambda w, T: ((T, w.k), torch.int32),
    "weights": lambda w, T: ((T, w.k), torch.float32),
    "counts": lambda w, T: ((w.E,), torch.int32),
    "bounds": lambda w, T: ((w.E + 1,), torch.int32),
    "rows": lambda w, T: ((T * w.k,), torch.int32),
    "pos": lambda w, T: ((T * w.k,), torch.int32),
    "xq": lambda w, T: ((T, w.d), torch.int8),
    "dx": lambda w, T: ((T, w.d // 32), torch.float32),
    "gu": lambda w, T: ((T * w.k, 2 * w.f), torch.float32),
    "h": lambda w, T: ((T * w.k, w.f), torch.float32),
    "hq": lambda w, T: ((T * w.k, w.f), torch.int8),
    "dh": lambda w, T: ((T * w.k, w.f // 32), torch.float32),
    "dm": lambda w, T: ((T * w.k, w.d), torch.float32),
}


def run_layer_gpu(h, w: wl.Workload, x: np.ndarray, lg: np.ndarray, blob_dev: torch.Tensor,
                  exports=tuple(EXPORT_SHAPES), layer: int = -1, combine: str = "gather"):
    T = x.shape[0]
    dev = torch.device("cuda:0")
    xt = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    lt = torch.from_numpy(np.ascontiguousarray(lg)).to(dev)
    y = torch.full((T, w.d), float("nan"), dtype=torch.float32, device=dev)
    ex = {}
    for name in exports:
        shp, dt = EXPORT_SHAPES[name](w, T)
        ex[name] = torch.empty(shp, dtype=dt, device=dev)
        if dt.is_floating_point:
            ex[name].fill_(float("nan"))
        else:
            ex[name].fill_(-99)
    mp.moe_prefill_run_layer(h, xt, lt, y, layer=layer, weights=blob_dev, exports=ex, combine=combine)
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in ex.items()}
    out["y"] = y.cpu().numpy()
    return out


def close_mask(a: np.ndarray, ref: np.ndarray, rtol=1e-3, atol=1e-4):
    a = a.astype(np.float64)
    return np.abs(a - ref) <= atol + rtol * np.abs(ref)


def assert_close(name, a, ref, rtol=1e-3, atol=1e-4):
    ok = close_mask(a, ref, rtol, atol)
    if not ok.all():
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError(f"{name}: {(~ok).sum()} of {ok.size} outside |d| <= {atol} + {rtol}|ref|; "
                             f"first at {i}: got {a[i]!r} ref {ref[i]!r}")


def assert_equal(name, a, ref):
    a = np.asarray(a)
    ref = np.asarray(ref)
    assert a.shape == ref.shape, (name, a.shape, ref.shape)
    if a.dtype.kind == "f":
        eq = (a.view(np.uint32 if a.dtype == np.float32 else np.uint64) ==
              ref.astype(a.dtype).view(np.uint32 if a.dtype == np.float32 else np.uint64))
    else:
        eq = a == ref
    if not eq.all():
        bad = np.argwhere(~eq)
        i = tuple(bad[0])
        raise AssertionError(f"{name}: {(~eq).sum()} of {eq.size} differ; first at {i}: "
                             f"got {a[i]!r} ref {ref[i]!r}")


def weights_rtol(k: int) -> float:
    """Router weights: fp32 (exp, an ascending sum of k terms, one division) against the
    fp64 oracle.  2e-6 up to k = 8; beyond, the sum's rounding bound (k - 1) * 2^-24 of
    the total grows with k, so the bound grows by 2^-23 per slot."""
    return 2e-6 + max(0, k - 8) * 2.0 ** -23


def check_full_parity(w: wl.Workload, g: dict, ref: dict):
    """Every stage of one layer: integers bit-exact, GU/H (which decide Hq) bit-exact,
    fp outputs within 1e-3 relative + 1e-4 absolute of the fp64 oracle."""
    T = ref["eidx"].shape[0]
    assert_equal("eidx", g["eidx"], ref["eidx"])
    assert_close("weights", g["weights"], ref["w"], rtol=weights_rtol(w.k), atol=1e-7)
    assert_equal("counts", g["counts"], ref["counts"])
    assert_equal("bounds", g["bounds"], ref["bounds"])
    assert_equal("rows", g["rows"], ref["rows"])
    assert_equal("pos", g["pos"], ref["pos"].reshape(-1))
    assert_equal("xq", g["xq"], ref["xq"])
    assert_equal("dx", g["dx"], ref["dx"])
    assert_equal("gu", g["gu"], ref["gu"])
    assert_equal("h", g["h"], ref["h"])
    assert_equal("hq", g["hq"], ref["hq"])
    assert_equal("dh", g["dh"], ref["dh"])
    if "dm" in g:                     # not stored with the atomic combine
        assert_close("dm", g["dm"], ref["dm"])
    assert_close("y", g["y"], ref["y"])
    assert g["y"].shape == (T, w.d)


def check_sampled_parity(w: wl.Workload, g: dict, ref: dict):
    """Large layers: routing/grouping/Xq complete; GU/H/Hq/Dm on the sampled rows;
    y on the sampled tokens."""
    assert_equal("eidx", g["eidx"], ref["eidx"])
    assert_close("weights", g["weights"], ref["w"], rtol=2e-6, atol=1e-7)
    assert_equal("counts", g["counts"], ref["counts"])
    assert_equal("bounds", g["bounds"], ref["bounds"])
    assert_equal("rows", g["rows"], ref["rows"])
    assert_equal("pos", g["pos"], ref["pos"].reshape(-1))
    assert_equal("xq", g["xq"], ref["xq"])
    assert_equal("dx", g["dx"], ref["dx"])
    r = ref["sel_rows"]
    if "gu" in g:
        assert_equal("gu[rows]", g["gu"][r], ref["gu"])
    if "h" in g:
        assert_equal("h[rows]", g["h"][r], ref["h"])
    assert_equal("hq[rows]", g["hq"][r], ref["hq"])
    assert_equal("dh[rows]", g["dh"][r], ref["dh"])
    if "dm" in g:
        assert_close("dm[rows]", g["dm"][r], ref["dm"])
    assert_close("y[tokens]", g["y"][ref["tokens"]], ref["y"])
