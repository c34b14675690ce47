"""Seeded synthetic workloads for the MoE prompt (prefill) FFN layer.

Holds only input generation: shapes, seeds and random draws (``gen.c``).  Both
the GPU path and the CPU oracle consume these arrays as inputs; nothing here
routes, quantises, multiplies or combines.

Workload shapes follow the prompt-path page (Strata #663, "What": a one-chunk
prompt streamed through an MoE layer's experts) and the layer-streaming pages
(stable-diffusion.cpp #1905/#1906: a stack of layers streamed through a fixed
slot pool with lookahead prefetch).  Distributions: activations and router
logits N(0,1) fp32; expert weights Q4 in blocks of 32 (int4 uniform in [-8, 7],
one fp16 scale per block, U(0.5, 1.5)/sqrt(d_in)).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmoegen.so")
_lib = None

# Stream ids (one independent counter-based stream per tensor kind).
T_X, T_LOGITS, T_BIAS, T_WGU_Q, T_WGU_S, T_WD_Q, T_WD_S = range(7)


def build() -> str:
    """Compile gen.c into libmoegen.so (gcc, OpenMP)."""
    src = os.path.join(_HERE, "gen.c")
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", src, "-o", tmp, "-lm"]
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
    u64, i64, i32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.gen_stream_key.restype = u64
    lib.gen_stream_key.argtypes = [u64, u64, u64]
    lib.gen_u64.argtypes = [u64, u64, i64, vp]
    lib.gen_normal_f32.argtypes = [u64, i64, ctypes.c_float, ctypes.c_float, vp]
    lib.gen_int4.argtypes = [u64, i64, vp]
    lib.gen_scale_f16.argtypes = [u64, i64, i32, vp]
    lib.gen_rank_perm.argtypes = [u64, i32, vp]
    lib.gen_add_bias.argtypes = [i64, i32, vp, vp]
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def stream_key(seed: int, tensor: int, expert: int = 0) -> int:
    return int(_load().gen_stream_key(seed, tensor, expert))


def u64(seed: int, tensor: int, expert: int, first: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    _load().gen_u64(stream_key(seed, tensor, expert), first, n, _ptr(out))
    return out


def normal(seed: int, tensor: int, n: int, mean: float = 0.0, std: float = 1.0,
           expert: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    _load().gen_normal_f32(stream_key(seed, tensor, expert), n, mean, std, _ptr(out))
    return out


def int4(seed: int, tensor: int, expert: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int8)
    _load().gen_int4(stream_key(seed, tensor, expert), n, _ptr(out))
    return out


def scale_f16(seed: int, tensor: int, expert: int, n: int, d_in: int) -> np.ndarray:
    """fp16 block scales, returned as raw binary16 bits (uint16)."""
    out = np.empty(n, dtype=np.uint16)
    _load().gen_scale_f16(stream_key(seed, tensor, expert), n, d_in, _ptr(out))
    return out


@dataclass(frozen=True)
class Stream:
    """How a stack is streamed through the slot pool."""
    depth: int
    residents: int           # max resident leading layers, -1 = as many as the budget allows
    slots: int = 0           # requested slot count (0 = derive from the budget)
    budget_slots: int = 0    # VRAM budget in units of one slot (0 = no cap)


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    f: int
    E: int
    k: int
    n_layers: int
    seed_base: int
    bias: Optional[tuple] = None        # ("normal", std) or ("zipf", s)
    stream: Optional[Stream] = None

    def seed(self, layer: int) -> int:
        return self.seed_base + layer

    @property
    def R(self) -> int:
        return self.T * self.k


# The five layer workloads (shapes, stack depth, pool and skew).
WORKLOADS = {
    "tiny": Workload("tiny_T64_d256_f512_E8_top2", 64, 256, 512, 8, 2, 1, 0),
    "resident": Workload("resident_T1024_d2048_f768_E128_top8", 1024, 2048, 768, 128, 8, 1, 1000),
    "stream4": Workload("streamed4_T1024_d2048_f768_E128_top8", 1024, 2048, 768, 128, 8, 4, 2000,
                        stream=Stream(depth=1, residents=0, slots=2)),
    "stream48": Workload("streamed48_T3072_d2048_f768_E128_top8_bias", 3072, 2048, 768, 128, 8, 48,
                         3000, bias=("normal", 0.5),
                         stream=Stream(depth=2, residents=-1, budget_slots=7)),
    "skew": Workload("skewed8_T8192_d4096_f1536_E256_top8_zipf", 8192, 4096, 1536, 256, 8, 8, 4000,
                     bias=("zipf", 1.1), stream=Stream(depth=2, residents=0, slots=3)),
}


def expert_bias(w: Workload, layer: int) -> Optional[np.ndarray]:
    """Per-expert router bias [E] fp32, or None.

    normal: N(0, std) with std = the stated 0.5.  zipf: -s * ln(rank_e) with rank a
    seeded permutation of 1..E, i.e. the log of a Zipf(s) popularity.
    """
    if w.bias is None:
        return None
    kind, par = w.bias
    seed = w.seed(layer)
    if kind == "normal":
        return normal(seed, T_BIAS, w.E, 0.0, float(par))
    if kind == "zipf":
        rank = np.empty(w.E, dtype=np.int32)
        _load().gen_rank_perm(stream_key(seed, T_BIAS, 0), w.E, _ptr(rank))
        return (-float(par) * np.log(rank.astype(np.float64))).astype(np.float32)
    raise ValueError(kind)


def layer_activations(w: Workload, layer: int) -> np.ndarray:
    """X [T, d] fp32."""
    return normal(w.seed(layer), T_X, w.T * w.d).reshape(w.T, w.d)


def layer_logits(w: Workload, layer: int) -> np.ndarray:
    """Router logits [T, E] fp32 (N(0,1) plus the workload's per-expert bias)."""
    lg = normal(w.seed(layer), T_LOGITS, w.T * w.E).reshape(w.T, w.E)
    b = expert_bias(w, layer)
    if b is not None:
        _load().gen_add_bias(w.T, w.E, _ptr(b), _ptr(lg))
    return lg


@dataclass
class ExpertWeights:
    """Canonical (unpacked) Q4 weights of one expert.

    wgu_q [2f, d] int8 in [-8, 7]: rows [0, f) are the gate projection, rows
    [f, 2f) the up projection.  wgu_s [2f, d/32] fp16 bits.  wd_q [d, f] int8,
    wd_s [d, f/32] fp16 bits.
    """
    wgu_q: np.ndarray
    wgu_s: np.ndarray
    wd_q: np.ndarray
    wd_s: np.ndarray


def expert_weights(w: Workload, layer: int, e: int) -> ExpertWeights:
    s = w.seed(layer)
    d, f = w.d, w.f
    return ExpertWeights(
        wgu_q=int4(s, T_WGU_Q, e, 2 * f * d).reshape(2 * f, d),
        wgu_s=scale_f16(s, T_WGU_S, e, 2 * f * (d // 32), d).reshape(2 * f, d // 32),
        wd_q=int4(s, T_WD_Q, e, d * f).reshape(d, f),
        wd_s=scale_f16(s, T_WD_S, e, d * (f // 32), f).reshape(d, f // 32),
    )


def small_workload(T: int, d: int, f: int, E: int, k: int, seed_base: int,
                   bias=None, name: Optional[str] = None) -> Workload:
    """An ad-hoc single-layer workload (edge cases and ragged sizes in tests)."""
    return Workload(name or f"adhoc_T{T}_d{d}_f{f}_E{E}_top{k}", T, d, f, E, k, 1, seed_base,
                    bias=bias)
