"""CPU oracle for the MoE prompt (prefill) FFN layer -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package.  The product path (``moe_prefill_ffn_amd``) never
imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain loops, one function per step of the
prompt path named on the page "prefill: a layer split's idle card streams a
share of a one-chunk prompt's experts", Strata #663, section "What").  This
module only marshals numpy arrays and strings the steps together in the
page's order: route -> group -> Xq -> GU -> H -> Hq -> Dm -> combine.

Parity status of each function is pinned by ``tests/test_oracle_*.py``; see the
oracle header in ``oracle.c`` for the readings taken where the page is silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Callable, Iterable, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build() -> str:
    """Compile oracle.c (gcc; no contraction, no fast-math, OpenMP over rows)."""
    src = os.path.join(_HERE, "oracle.c")
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O3", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fno-unsafe-math-optimizations", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.oracle_f16_to_f64.restype = ctypes.c_double
    lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f64_array.argtypes = [i64, vp, vp]
    lib.oracle_exp_ref.restype = ctypes.c_float
    lib.oracle_exp_ref.argtypes = [ctypes.c_float]
    lib.oracle_exp_ref_array.argtypes = [i64, vp, vp]
    lib.oracle_route.argtypes = [i32, i32, i32, vp, vp, vp]
    lib.oracle_group.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp]
    lib.oracle_quant_q8.argtypes = [i64, i32, vp, vp, vp]
    lib.oracle_block_dots.argtypes = [i32, i32, i32, vp, vp, vp]
    lib.oracle_gemm_f32.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp]
    lib.oracle_gemm_f64.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp]
    lib.oracle_swiglu_f32.argtypes = [i64, i32, vp, vp]
    lib.oracle_combine_f64.argtypes = [i32, i32, i32, vp, vp, vp, vp]
    lib.oracle_num_threads.restype = i32
    _lib = lib
    return lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


# ----------------------------------------------------------------- steps ---

def f16_to_f64(h: np.ndarray) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, dtype=np.float64)
    _load().oracle_f16_to_f64_array(h.size, _p(h), _p(out))
    return out


def exp_ref(x: np.ndarray) -> np.ndarray:
    x = _c(x, np.float32)
    y = np.empty_like(x)
    _load().oracle_exp_ref_array(x.size, _p(x), _p(y))
    return y


def route(logits: np.ndarray, k: int):
    """Top-k experts per token (ties -> lower index) and fp64 softmax weights."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    if not (1 <= k <= E <= 4096):
        raise ValueError("need 1 <= k <= E <= 4096")
    eidx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    _load().oracle_route(T, E, k, _p(logits), _p(eidx), _p(w))
    return eidx, w


def group(eidx: np.ndarray, E: int):
    """counts [E], bounds [E+1], rows [T*k] (stable in p = t*k + j), pos [T*k]."""
    eidx = _c(eidx, np.int32)
    T, k = eidx.shape
    counts = np.empty(E, dtype=np.int32)
    bounds = np.empty(E + 1, dtype=np.int32)
    rows = np.empty(T * k, dtype=np.int32)
    pos = np.empty(T * k, dtype=np.int32)
    _load().oracle_group(T, k, E, _p(eidx), _p(counts), _p(bounds), _p(rows), _p(pos))
    return counts, bounds, rows, pos


def quant_q8(x: np.ndarray):
    """Q8 blocks of 32 along the last axis: int8 codes and fp32 scales."""
    x = _c(x, np.float32)
    n, K = x.shape
    if K % 32:
        raise ValueError("row length must be a multiple of 32")
    q = np.empty((n, K), dtype=np.int8)
    s = np.empty((n, K // 32), dtype=np.float32)
    _load().oracle_quant_q8(n, K, _p(x), _p(q), _p(s))
    return q, s


def block_dots(A: np.ndarray, W: np.ndarray) -> np.ndarray:
    A, W = _c(A, np.int8), _c(W, np.int8)
    M, K = A.shape
    N = W.shape[0]
    out = np.empty((M, N, K // 32), dtype=np.int32)
    _load().oracle_block_dots(M, N, K, _p(A), _p(W), _p(out))
    return out


def gemm_f32(A, a_scale, W, w_scale) -> np.ndarray:
    A, W = _c(A, np.int8), _c(W, np.int8)
    a_scale, w_scale = _c(a_scale, np.float32), _c(w_scale, np.uint16)
    M, K = A.shape
    N = W.shape[0]
    out = np.empty((M, N), dtype=np.float32)
    if M:
        _load().oracle_gemm_f32(M, N, K, _p(A), _p(a_scale), _p(W), _p(w_scale), _p(out))
    return out


def gemm_f64(A, a_scale, W, w_scale) -> np.ndarray:
    A, W = _c(A, np.int8), _c(W, np.int8)
    a_scale, w_scale = _c(a_scale, np.float32), _c(w_scale, np.uint16)
    M, K = A.shape
    N = W.shape[0]
    out = np.empty((M, N), dtype=np.float64)
    if M:
        _load().oracle_gemm_f64(M, N, K, _p(A), _p(a_scale), _p(W), _p(w_scale), _p(out))
    return out


def swiglu_f32(gu: np.ndarray) -> np.ndarray:
    gu = _c(gu, np.float32)
    M, two_f = gu.shape
    out = np.empty((M, two_f // 2), dtype=np.float32)
    _load().oracle_swiglu_f32(M, two_f // 2, _p(gu), _p(out))
    return out


def combine_f64(w: np.ndarray, pos: np.ndarray, dm: np.ndarray) -> np.ndarray:
    w, pos, dm = _c(w, np.float64), _c(pos, np.int32), _c(dm, np.float64)
    T, k = w.shape
    d = dm.shape[1]
    y = np.empty((T, d), dtype=np.float64)
    _load().oracle_combine_f64(T, k, d, _p(w), _p(pos), _p(dm), _p(y))
    return y


# ------------------------------------------------------------ the layer ---

def layer(x: np.ndarray, logits: np.ndarray, k: int, experts: Callable, f: int,
          tokens: Optional[Iterable[int]] = None) -> dict:
    """The whole prompt-path FFN layer.

    ``experts(e)`` returns that expert's canonical weights (an object with
    ``wgu_q [2f,d] int8, wgu_s [2f,d/32] fp16 bits, wd_q [d,f] int8,
    wd_s [d,f/32] fp16 bits``).  With ``tokens`` set, only those tokens' output
    rows are produced (GU/H/Hq/Dm for their rows only); routing, grouping and
    Xq are always complete.
    """
    T, d = x.shape
    E = logits.shape[1]
    eidx, w = route(logits, k)
    counts, bounds, rows, pos = group(eidx, E)
    xq, dx = quant_q8(x)
    out = dict(eidx=eidx, w=w, counts=counts, bounds=bounds, rows=rows, pos=pos, xq=xq, dx=dx)
    R = T * k
    if tokens is None:
        need = np.arange(R, dtype=np.int64)                       # every row
    else:
        tok = np.asarray(sorted(set(int(t) for t in tokens)), dtype=np.int64)
        need = np.sort(pos.reshape(T, k)[tok].reshape(-1).astype(np.int64))
    need_set = need
    res_rows, res_gu, res_h, res_hq, res_dh, res_dm = [], [], [], [], [], []
    for e in range(E):
        r0, r1 = int(bounds[e]), int(bounds[e + 1])
        if r1 == r0:
            continue
        sel = need_set[(need_set >= r0) & (need_set < r1)]
        if sel.size == 0:
            continue
        W = experts(e)
        tk = rows[sel] // k
        g = gemm_f32(xq[tk], dx[tk], W.wgu_q, W.wgu_s)
        h = swiglu_f32(g)
        hq, dh = quant_q8(h)
        dm = gemm_f64(hq, dh, W.wd_q, W.wd_s)
        res_rows.append(sel)
        res_gu.append(g)
        res_h.append(h)
        res_hq.append(hq)
        res_dh.append(dh)
        res_dm.append(dm)
    if res_rows:
        order_rows = np.concatenate(res_rows)
        perm = np.argsort(order_rows, kind="stable")
        sel_rows = order_rows[perm]
        cat = lambda L: np.concatenate(L)[perm]
        gu_s, h_s, hq_s, dh_s, dm_s = cat(res_gu), cat(res_h), cat(res_hq), cat(res_dh), cat(res_dm)
    else:
        sel_rows = np.zeros(0, dtype=np.int64)
        gu_s = np.zeros((0, 2 * f), np.float32)
        h_s = np.zeros((0, f), np.float32)
        hq_s = np.zeros((0, f), np.int8)
        dh_s = np.zeros((0, f // 32), np.float32)
        dm_s = np.zeros((0, d), np.float64)
    out.update(sel_rows=sel_rows, gu=gu_s, h=h_s, hq=hq_s, dh=dh_s, dm=dm_s)
    if tokens is None:
        out["y"] = combine_f64(w, pos, dm_s)
    else:
        tok = np.asarray(sorted(set(int(t) for t in tokens)), dtype=np.int64)
        # positions of the sampled tokens' rows inside the computed subset
        sub_pos = np.searchsorted(sel_rows, pos.reshape(T, k)[tok]).astype(np.int32)
        out["tokens"] = tok
        out["y"] = combine_f64(w[tok], sub_pos, dm_s)
    return out
