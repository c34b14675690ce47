"""MI355X-native MoE prompt (prefill) FFN layer -- Python binding.

A thin ctypes binding of ``libmoe_prefill.so`` (C ABI in
``include/moe_prefill.h``).  It only marshals arguments: routing, grouping,
quantisation, both grouped GEMMs, SwiGLU, requantisation, the combine and the
slot pool's copies all run in the library (HIP kernels for gfx950 and its C++
host runtime).  PyTorch supplies device memory, pinned host memory and
streams; there is no CPU fallback -- if the library is missing, importing the
binding's entry points raises.

The function names are the C entry points' names.
"""
from __future__ import annotations

import ctypes
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Callable, Dict, Optional, Sequence

import numpy as np
import torch  # loaded first so the library binds to the same HIP runtime as torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_prefill.so")

MOE_OK, MOE_EINVAL, MOE_ENOMEM, MOE_EHIP, MOE_EUNSUPPORTED, MOE_ESTATE, MOE_ETIMEOUT = 0, -1, -2, -3, -4, -5, -6
MOE_WARN_SLOT_OVER_BUDGET, MOE_WARN_POOL_DEGRADED, MOE_WARN_DEPTH_REDUCED = 1, 2, 4
_NAMES = {0: "MOE_OK", -1: "MOE_EINVAL", -2: "MOE_ENOMEM", -3: "MOE_EHIP", -4: "MOE_EUNSUPPORTED",
          -5: "MOE_ESTATE", -6: "MOE_ETIMEOUT"}


class MoePrefillError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_NAMES.get(code, code)}: {msg}")
        self.code = code


_u32, _i32, _i64, _u64, _vp = ctypes.c_uint32, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p


class moe_prefill_params_t(ctypes.Structure):
    _fields_ = [("struct_size", _u32), ("d_model", _i32), ("d_ff", _i32), ("n_experts", _i32),
                ("top_k", _i32), ("max_tokens", _i32), ("device", _i32), ("reserved0", _i32),
                ("workspace", _vp), ("workspace_bytes", _u64)]


class moe_layer_io_t(ctypes.Structure):
    _fields_ = [("struct_size", _u32), ("layer", _i32), ("weights_dev", _vp), ("n_tokens", _i32),
                ("reserved0", _i32), ("x", _vp), ("logits", _vp), ("y", _vp),
                ("eidx", _vp), ("weights", _vp), ("counts", _vp), ("bounds", _vp), ("rows", _vp),
                ("pos", _vp), ("xq", _vp), ("dx", _vp), ("gu", _vp), ("h", _vp), ("hq", _vp),
                ("dh", _vp), ("dm", _vp), ("combine", _i32), ("reserved1", _i32)]


COMBINE_MODES = {"gather": 0, "atomic": 1}   # MOE_COMBINE_GATHER, MOE_COMBINE_ATOMIC


class stream_pool_params_t(ctypes.Structure):
    _fields_ = [("struct_size", _u32), ("n_layers", _i32), ("host_blobs", ctypes.POINTER(_vp)),
                ("layer_bytes", _u64), ("prefetch_depth", _i32), ("resident_layers", _i32),
                ("max_vram_bytes", _i64), ("requested_slots", _i32), ("eff_slots", _i32),
                ("eff_depth", _i32), ("eff_residents", _i32), ("warnings", _i32), ("reserved0", _i32),
                ("active_only", _i32), ("reserved1", _i32), ("reserve_bytes", _i64)]


class stream_pool_budget_t(ctypes.Structure):
    _fields_ = [("struct_size", _u32), ("reserved0", _i32), ("max_vram_bytes", _i64),
                ("eff_slots", _i32), ("eff_depth", _i32), ("eff_residents", _i32), ("warnings", _i32),
                ("released_bytes", _u64)]


class moe_pool_trim_t(ctypes.Structure):
    _fields_ = [("struct_size", _u32), ("n_layers", _i32), ("residents", _i32), ("streaming", _i32),
                ("budget_slots", _i64), ("new_residents", _i32), ("new_streaming", _i32),
                ("evicted", _i32), ("converted", _i32), ("released", _i32), ("warnings", _i32)]


class moe_pool_plan_t(ctypes.Structure):
    _fields_ = [("struct_size", _u32), ("n_layers", _i32), ("slot_bytes", _u64),
                ("prefetch_depth", _i32), ("resident_layers", _i32), ("max_vram_bytes", _i64),
                ("requested_slots", _i32), ("max_alloc_slots", _i32), ("slots", _i32),
                ("depth", _i32), ("residents", _i32), ("warnings", _i32)]


class moe_stats_t(ctypes.Structure):
    _fields_ = [("struct_size", _u32), ("reserved0", _i32), ("layers_run", _u64),
                ("prefetch_queued", _u64), ("prefetch_activated", _u64), ("sync_loads", _u64),
                ("prefetch_failed", _u64), ("bytes_h2d", _u64), ("eff_slots", _i32),
                ("eff_depth", _i32), ("eff_residents", _i32), ("warnings", _i32),
                ("sparse_loads", _u64), ("experts_loaded", _u64), ("bytes_sparse", _u64),
                ("evicted_residents", _u64), ("released_bytes", _u64), ("pressure_trims", _u64)]


MOE_N_KERNELS = 7
MOE_LOG_ERROR, MOE_LOG_WARN, MOE_LOG_INFO = 0, 1, 2
_LOG_FN = ctypes.CFUNCTYPE(None, _i32, ctypes.c_char_p, _vp)


class moe_kernel_times_t(ctypes.Structure):
    _fields_ = [("struct_size", _u32), ("n_kernels", _i32), ("launches", _u64 * MOE_N_KERNELS),
                ("total_ms", ctypes.c_double * MOE_N_KERNELS)]


EXPORTED_SYMBOLS = [
    "moe_prefill_workspace_size", "moe_prefill_create", "moe_prefill_destroy",
    "moe_prefill_last_error", "moe_prefill_expert_bytes", "moe_prefill_layer_bytes",
    "moe_prefill_pack_expert", "moe_prefill_run_layer", "stream_pool_configure",
    "moe_prefill_plan_pool", "moe_prefill_plan_trim", "stream_pool_set_budget",
    "moe_prefill_get_stats", "moe_prefill_set_log", "moe_prefill_set_timing",
    "moe_prefill_kernel_times", "moe_prefill_kernel_name",
    "moe_prefill_exp_host", "moe_prefill_exp_device", "moe_prefill_run_layer_noalloc",
]

_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python moe_prefill_ffn_amd/build.py` "
                          "(or __graft_entry__.build()); there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    L.moe_prefill_workspace_size.argtypes = [ctypes.POINTER(moe_prefill_params_t), ctypes.POINTER(_u64)]
    L.moe_prefill_create.argtypes = [ctypes.POINTER(moe_prefill_params_t), ctypes.POINTER(_vp)]
    L.moe_prefill_destroy.argtypes = [_vp]
    L.moe_prefill_destroy.restype = None
    L.moe_prefill_last_error.argtypes = [_vp]
    L.moe_prefill_last_error.restype = ctypes.c_char_p
    L.moe_prefill_expert_bytes.argtypes = [_i32, _i32]
    L.moe_prefill_expert_bytes.restype = _u64
    L.moe_prefill_layer_bytes.argtypes = [_i32, _i32, _i32]
    L.moe_prefill_layer_bytes.restype = _u64
    L.moe_prefill_pack_expert.argtypes = [_i32, _i32, _vp, _vp, _vp, _vp, _vp]
    L.moe_prefill_run_layer.argtypes = [_vp, ctypes.POINTER(moe_layer_io_t), _vp]
    L.stream_pool_configure.argtypes = [_vp, ctypes.POINTER(stream_pool_params_t)]
    L.moe_prefill_plan_pool.argtypes = [ctypes.POINTER(moe_pool_plan_t)]
    L.moe_prefill_plan_trim.argtypes = [ctypes.POINTER(moe_pool_trim_t)]
    L.stream_pool_set_budget.argtypes = [_vp, ctypes.POINTER(stream_pool_budget_t)]
    L.moe_prefill_get_stats.argtypes = [_vp, ctypes.POINTER(moe_stats_t)]
    L.moe_prefill_set_log.argtypes = [_vp, _LOG_FN, _vp, _i32]
    L.moe_prefill_set_timing.argtypes = [_vp, _i32]
    L.moe_prefill_kernel_times.argtypes = [_vp, ctypes.POINTER(moe_kernel_times_t), _i32]
    L.moe_prefill_kernel_name.argtypes = [_i32]
    L.moe_prefill_kernel_name.restype = ctypes.c_char_p
    L.moe_prefill_run_layer_noalloc.argtypes = [ctypes.POINTER(moe_prefill_params_t),
                                                ctypes.POINTER(moe_layer_io_t), _vp]
    L.moe_prefill_exp_host.argtypes = [_u32, _u64, _vp]
    L.moe_prefill_exp_device.argtypes = [_u32, _u64, _vp, _vp]
    _lib = L
    return L


def _check(rc: int, handle=None):
    if rc != MOE_OK:
        msg = lib().moe_prefill_last_error(handle).decode(errors="replace")
        raise MoePrefillError(rc, msg)


def moe_prefill_last_error(handle=None) -> str:
    return lib().moe_prefill_last_error(handle.ptr if handle else None).decode(errors="replace")


# ---------------------------------------------------------------- handle ---

class Handle:
    """Owner of a ``moe_prefill_t*`` plus references that must outlive it."""

    def __init__(self, ptr: int, params: dict, keep=()):
        self.ptr = ptr
        self.params = params
        self._keep = list(keep)
        self._pool_keep = []
        self._log_cb = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def close(self):
        if self.ptr:
            lib().moe_prefill_destroy(self.ptr)
            self.ptr = None
        self._pool_keep = []

    def __enter__(self):
        return self

    def __exit__(self, *a):
        self.close()


def _params(d_model, d_ff, n_experts, top_k, max_tokens, device=0, workspace=None):
    p = moe_prefill_params_t()
    p.struct_size = ctypes.sizeof(p)
    p.d_model, p.d_ff, p.n_experts, p.top_k, p.max_tokens, p.device = (
        d_model, d_ff, n_experts, top_k, max_tokens, device)
    if workspace is not None:
        p.workspace = workspace.data_ptr()
        p.workspace_bytes = workspace.numel() * workspace.element_size()
    return p


def moe_prefill_workspace_size(d_model: int, d_ff: int, n_experts: int, top_k: int, max_tokens: int) -> int:
    p = _params(d_model, d_ff, n_experts, top_k, max_tokens)
    out = _u64()
    _check(lib().moe_prefill_workspace_size(ctypes.byref(p), ctypes.byref(out)))
    return int(out.value)


def moe_prefill_create(d_model: int, d_ff: int, n_experts: int, top_k: int, max_tokens: int,
                       device: int = 0, workspace: Optional[torch.Tensor] = None) -> Handle:
    """Create a handle.  ``workspace``: optional lent device uint8 tensor."""
    p = _params(d_model, d_ff, n_experts, top_k, max_tokens, device, workspace)
    out = _vp()
    _check(lib().moe_prefill_create(ctypes.byref(p), ctypes.byref(out)))
    return Handle(out.value, dict(d_model=d_model, d_ff=d_ff, n_experts=n_experts, top_k=top_k,
                                  max_tokens=max_tokens, device=device),
                  keep=[workspace] if workspace is not None else [])


def moe_prefill_destroy(handle: Handle):
    handle.close()


# ----------------------------------------------------------------- blobs ---

def moe_prefill_expert_bytes(d_model: int, d_ff: int) -> int:
    return int(lib().moe_prefill_expert_bytes(d_model, d_ff))


def moe_prefill_layer_bytes(d_model: int, d_ff: int, n_experts: int) -> int:
    return int(lib().moe_prefill_layer_bytes(d_model, d_ff, n_experts))


def _np_ptr(a: np.ndarray, dtype) -> int:
    if a.dtype != dtype or not a.flags["C_CONTIGUOUS"]:
        raise TypeError(f"expected a C-contiguous {np.dtype(dtype)} array")
    return a.ctypes.data


def moe_prefill_pack_expert(d_model: int, d_ff: int, wgu_q: np.ndarray, wgu_s: np.ndarray,
                            wd_q: np.ndarray, wd_s: np.ndarray, dst_ptr: int) -> None:
    """Pack one expert's canonical weights into host memory at ``dst_ptr``."""
    for a, shp in ((wgu_q, (2 * d_ff, d_model)), (wgu_s, (2 * d_ff, d_model // 32)),
                   (wd_q, (d_model, d_ff)), (wd_s, (d_model, d_ff // 32))):
        if tuple(a.shape) != shp:
            raise ValueError(f"shape {a.shape} != {shp}")
    rc = lib().moe_prefill_pack_expert(
        d_model, d_ff, _np_ptr(wgu_q, np.int8), _np_ptr(wgu_s, np.uint16), _np_ptr(wd_q, np.int8),
        _np_ptr(wd_s, np.uint16), dst_ptr)
    _check(rc)


def pack_layer(d_model: int, d_ff: int, n_experts: int, expert_fn: Callable, out: torch.Tensor,
               threads: int = 8) -> torch.Tensor:
    """Pack a whole layer blob into ``out`` (a host uint8 tensor, e.g. pinned).

    ``expert_fn(e)`` returns an object with ``wgu_q, wgu_s, wd_q, wd_s``.
    """
    eb = moe_prefill_expert_bytes(d_model, d_ff)
    if out.device.type != "cpu" or out.dtype != torch.uint8 or out.numel() < eb * n_experts:
        raise ValueError("out must be a host uint8 tensor of at least layer_bytes")
    base = out.data_ptr()

    def one(e):
        w = expert_fn(e)
        moe_prefill_pack_expert(d_model, d_ff, w.wgu_q, w.wgu_s, w.wd_q, w.wd_s, base + e * eb)

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(one, range(n_experts)))
    return out


# ------------------------------------------------------------- one layer ---

_EXPORTS = ("eidx", "weights", "counts", "bounds", "rows", "pos", "xq", "dx", "gu", "h", "hq", "dh", "dm")


def _dev_ptr(t: Optional[torch.Tensor], dtype, name: str, numel: Optional[int] = None) -> int:
    if t is None:
        return 0
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise TypeError(f"{name}: expected a contiguous {dtype} device tensor")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name}: needs at least {numel} elements")
    return t.data_ptr()


def _layer_io(P: dict, x: torch.Tensor, logits: torch.Tensor, y: torch.Tensor, layer: int,
              weights: Optional[torch.Tensor], exports: Optional[Dict[str, torch.Tensor]],
              combine: str = "gather") -> moe_layer_io_t:
    T = x.shape[0]
    io = moe_layer_io_t()
    io.struct_size = ctypes.sizeof(io)
    io.layer = layer
    io.n_tokens = T
    if combine not in COMBINE_MODES:
        raise ValueError(f"combine must be one of {sorted(COMBINE_MODES)}")
    io.combine = COMBINE_MODES[combine]
    io.x = _dev_ptr(x, torch.float32, "x", T * P["d_model"])
    io.logits = _dev_ptr(logits, torch.float32, "logits", T * P["n_experts"])
    io.y = _dev_ptr(y, torch.float32, "y", T * P["d_model"])
    if layer < 0:
        if weights is None:
            raise ValueError("layer=-1 needs a resident weight blob")
        io.weights_dev = _dev_ptr(weights, torch.uint8, "weights",
                                  moe_prefill_layer_bytes(P["d_model"], P["d_ff"], P["n_experts"]))
    dt = dict(eidx=torch.int32, weights=torch.float32, counts=torch.int32, bounds=torch.int32,
              rows=torch.int32, pos=torch.int32, xq=torch.int8, dx=torch.float32, gu=torch.float32,
              h=torch.float32, hq=torch.int8, dh=torch.float32, dm=torch.float32)
    R, d, f, E = T * P["top_k"], P["d_model"], P["d_ff"], P["n_experts"]
    need = dict(eidx=R, weights=R, counts=E, bounds=E + 1, rows=R, pos=R, xq=T * d, dx=T * d // 32,
                gu=R * 2 * f, h=R * f, hq=R * f, dh=R * f // 32, dm=R * d)
    for name, t in (exports or {}).items():
        if name not in _EXPORTS:
            raise KeyError(name)
        setattr(io, name, _dev_ptr(t, dt[name], name, need[name]))
    return io


def moe_prefill_run_layer(handle: Handle, x: torch.Tensor, logits: torch.Tensor, y: torch.Tensor,
                          layer: int = -1, weights: Optional[torch.Tensor] = None,
                          stream: Optional[torch.cuda.Stream] = None,
                          exports: Optional[Dict[str, torch.Tensor]] = None,
                          combine: str = "gather") -> None:
    """Enqueue one MoE prefill FFN layer on ``stream`` (default: torch's current stream).
    combine: "gather" (deterministic, default) or "atomic" (the down GEMM adds into y)."""
    io = _layer_io(handle.params, x, logits, y, layer, weights, exports, combine)
    s = stream if stream is not None else torch.cuda.current_stream(x.device)
    _check(lib().moe_prefill_run_layer(handle.ptr, ctypes.byref(io), _vp(s.cuda_stream)), handle.ptr)


def moe_prefill_run_layer_noalloc(d_model: int, d_ff: int, n_experts: int, top_k: int, x: torch.Tensor,
                                  logits: torch.Tensor, y: torch.Tensor, weights: torch.Tensor,
                                  device: int = 0, stream: Optional[torch.cuda.Stream] = None,
                                  exports: Optional[Dict[str, torch.Tensor]] = None,
                                  combine: str = "gather") -> None:
    """One resident layer with no handle and no device allocation: the library's static
    per-device scratch array is the workspace (calls on one device must not overlap)."""
    T = x.shape[0]
    P = dict(d_model=d_model, d_ff=d_ff, n_experts=n_experts, top_k=top_k, max_tokens=max(T, 1))
    io = _layer_io(P, x, logits, y, -1, weights, exports, combine)
    p = _params(d_model, d_ff, n_experts, top_k, max(T, 1), device)
    s = stream if stream is not None else torch.cuda.current_stream(x.device)
    _check(lib().moe_prefill_run_layer_noalloc(ctypes.byref(p), ctypes.byref(io), _vp(s.cuda_stream)))


# ----------------------------------------------------------- stream pool ---

def stream_pool_configure(handle: Handle, host_blobs: Sequence[torch.Tensor], prefetch_depth: int = 1,
                          resident_layers: int = 0, max_vram_bytes: int = 0,
                          requested_slots: int = 0, active_only: bool = False,
                          reserve_bytes: int = 0) -> dict:
    """Plan + allocate the slot pool over pinned host blobs (one per layer).
    active_only: streamed layers are loaded after their routing, only the experts with rows.
    reserve_bytes: device memory to keep free; checked when a pass starts (layer 0)."""
    p = stream_pool_params_t()
    p.struct_size = ctypes.sizeof(p)
    n = len(host_blobs)
    arr = (_vp * max(n, 1))()
    for i, b in enumerate(host_blobs):
        if b.device.type != "cpu" or b.dtype != torch.uint8 or not b.is_contiguous():
            raise TypeError("host blobs must be contiguous host uint8 tensors")
        if not b.is_pinned():
            raise TypeError("host blobs must be pinned (torch.empty(..., pin_memory=True))")
        arr[i] = b.data_ptr()
    p.n_layers = n
    p.host_blobs = ctypes.cast(arr, ctypes.POINTER(_vp))
    p.layer_bytes = host_blobs[0].numel() if n else 0
    p.prefetch_depth = prefetch_depth
    p.resident_layers = resident_layers
    p.max_vram_bytes = max_vram_bytes
    p.requested_slots = requested_slots
    p.active_only = 1 if active_only else 0
    p.reserve_bytes = reserve_bytes
    _check(lib().stream_pool_configure(handle.ptr, ctypes.byref(p)), handle.ptr)
    handle._pool_keep = list(host_blobs)
    return dict(slots=p.eff_slots, depth=p.eff_depth, residents=p.eff_residents, warnings=p.warnings)


def stream_pool_set_budget(handle: Handle, max_vram_bytes: int) -> dict:
    """Shrink the live pool to max_vram_bytes (memory pressure); returns the effective shape
    and the device bytes released."""
    p = stream_pool_budget_t()
    p.struct_size = ctypes.sizeof(p)
    p.max_vram_bytes = max_vram_bytes
    _check(lib().stream_pool_set_budget(handle.ptr, ctypes.byref(p)), handle.ptr)
    return dict(slots=p.eff_slots, depth=p.eff_depth, residents=p.eff_residents, warnings=p.warnings,
                released_bytes=p.released_bytes)


def moe_prefill_plan_trim(n_layers: int, residents: int, streaming: int, budget_slots: int) -> dict:
    p = moe_pool_trim_t()
    p.struct_size = ctypes.sizeof(p)
    p.n_layers, p.residents, p.streaming, p.budget_slots = n_layers, residents, streaming, budget_slots
    rc = lib().moe_prefill_plan_trim(ctypes.byref(p))
    return dict(rc=rc, residents=p.new_residents, streaming=p.new_streaming, evicted=p.evicted,
                converted=p.converted, released=p.released, warnings=p.warnings)


def moe_prefill_plan_pool(n_layers: int, slot_bytes: int, prefetch_depth: int, resident_layers: int,
                          max_vram_bytes: int = 0, requested_slots: int = 0,
                          max_alloc_slots: int = 0) -> dict:
    p = moe_pool_plan_t()
    p.struct_size = ctypes.sizeof(p)
    p.n_layers, p.slot_bytes, p.prefetch_depth, p.resident_layers = n_layers, slot_bytes, prefetch_depth, resident_layers
    p.max_vram_bytes, p.requested_slots, p.max_alloc_slots = max_vram_bytes, requested_slots, max_alloc_slots
    rc = lib().moe_prefill_plan_pool(ctypes.byref(p))
    out = dict(rc=rc, slots=p.slots, depth=p.depth, residents=p.residents, warnings=p.warnings)
    return out


def moe_prefill_get_stats(handle: Handle) -> dict:
    s = moe_stats_t()
    s.struct_size = ctypes.sizeof(s)
    _check(lib().moe_prefill_get_stats(handle.ptr, ctypes.byref(s)), handle.ptr)
    return {name: getattr(s, name) for name, _ in moe_stats_t._fields_ if name not in ("struct_size", "reserved0")}


# --------------------------------------------------------------- logging ---

def moe_prefill_set_log(handle: Handle, fn: Optional[Callable[[int, str], None]], level: int = MOE_LOG_WARN) -> None:
    """Route the handle's messages of level <= `level` to fn(level, text); fn=None removes the sink."""
    if fn is None:
        cb = ctypes.cast(None, _LOG_FN)
    else:
        cb = _LOG_FN(lambda lv, msg, user: fn(int(lv), msg.decode(errors="replace")))
    handle._log_cb = cb                    # the library keeps the pointer: keep the callback alive
    _check(lib().moe_prefill_set_log(handle.ptr, cb, None, level), handle.ptr)


# --------------------------------------------------------------- tracing ---

def moe_prefill_kernel_name(kernel_id: int) -> str:
    return lib().moe_prefill_kernel_name(kernel_id).decode()


def moe_prefill_set_timing(handle: Handle, enable: bool = True) -> None:
    _check(lib().moe_prefill_set_timing(handle.ptr, 1 if enable else 0), handle.ptr)


def moe_prefill_kernel_times(handle: Handle, reset: bool = True) -> dict:
    """{kernel name: (launches, total device ms)} of the timed launches so far."""
    t = moe_kernel_times_t()
    t.struct_size = ctypes.sizeof(t)
    _check(lib().moe_prefill_kernel_times(handle.ptr, ctypes.byref(t), 1 if reset else 0), handle.ptr)
    return {moe_prefill_kernel_name(i): (int(t.launches[i]), float(t.total_ms[i])) for i in range(t.n_kernels)}


def moe_prefill_exp_host(first_bits: int, out: np.ndarray) -> np.ndarray:
    """The library's fp32 exponential (host build) of the inputs with bit patterns
    first_bits .. first_bits + out.size - 1, written into out (float32, contiguous)."""
    assert out.dtype == np.float32 and out.flags["C_CONTIGUOUS"]
    _check(lib().moe_prefill_exp_host(first_bits, out.size, out.ctypes.data))
    return out


def moe_prefill_exp_device(first_bits: int, out: torch.Tensor, stream=None) -> torch.Tensor:
    """The kernels' fp32 exponential of the inputs with bit patterns first_bits ..
    first_bits + out.numel() - 1, enqueued on `stream` into the device tensor out."""
    assert out.dtype == torch.float32 and out.is_cuda and out.is_contiguous()
    st = stream if stream is not None else torch.cuda.current_stream(out.device)
    _check(lib().moe_prefill_exp_device(first_bits, out.numel(), out.data_ptr(), st.cuda_stream))
    return out
