"""Binding of libmoe_micro.so: the microbenchmarks that set the roofline
denominators (int8 MFMA peak, the per-32-block epilogue ceiling of the grouped
GEMMs in each arithmetic form, a device copy, fp32 atomic adds).  Measurement
only; the layer path never loads this library."""
from __future__ import annotations

import ctypes
import os

import torch  # loaded first so the library binds to the same HIP runtime as torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_micro.so")

BLOCK_TESTS = {
    "mfma_i8": 0,          # int8 MFMAs alone (four chains)
    "cvt_fma_mscale": 1,   # scale products on the fp32 matrix cores, convert + fma on the VALU
    "cvt_fma_vscale": 2,   # scale products, convert and fma all on the VALU
    "sub_fma_vscale": 3,   # MFMA C seeded with 1.5*2^23: subtract instead of convert
    "sub_fma_mscale": 4,
    "valu_fma": 5,         # one VALU instruction kind alone
    "valu_cvt": 6,
    "valu_sub": 7,
    "overlap_indep": 8,    # two int8 MFMAs beside 64 fmas that do not depend on them
    "pipe_cvt_fma": 9,     # cvt_fma_mscale with the epilogue one block behind the MFMAs
    "mfma_f32_scale": 10,  # the fp32 scale-product MFMA (v_mfma_f32_32x32x1_2b_f32) alone
    "overlap_cvt": 11,     # two int8 MFMAs beside 64 independent converts
    "overlap_fma16": 12,   # two int8 MFMAs beside 16 independent fmas
    "overlap_mul": 13,     # two int8 MFMAs beside 64 independent multiplies
    "overlap_scale_fma": 14,  # one scale-product MFMA beside 64 independent fmas (result taken at once)
    "overlap_scale_chain": 15,  # one scale-product MFMA chained through C beside 64 fmas
    "overlap_scale_cvt": 16,    # one scale-product MFMA chained through C beside 64 converts
    "mfma_f32_chain": 17,       # two scale-product MFMAs chained through C, nothing else
    "f8split_fma_mscale": 18,   # alternative block form: fp8 x fp6 MFMAs give fp32 block sums, no convert
    "mfma_f6": 19,              # fp6 x fp6 MFMAs alone (four chains, K 64 each)
    "f6split_fma_mscale": 20,   # alternative block form: fp6 x fp6 MFMAs give fp32 block sums, no convert
}


class moe_micro_result_t(ctypes.Structure):
    _fields_ = [("ms", ctypes.c_double), ("cycles_per_wave", ctypes.c_double),
                ("clock_ghz", ctypes.c_double), ("work", ctypes.c_double)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python moe_prefill_ffn_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        R = ctypes.POINTER(moe_micro_result_t)
        i32, u64, vp = ctypes.c_int32, ctypes.c_uint64, ctypes.c_void_p
        L.moe_micro_block.argtypes = [i32, i32, i32, i32, R]
        L.moe_micro_copy.argtypes = [vp, vp, u64, i32, i32, R]
        L.moe_micro_atomic.argtypes = [vp, vp, vp, i32, i32, i32, R]
        _lib = L
    return _lib


def _res(rc: int, r: moe_micro_result_t, what: str) -> dict:
    if rc != 0:
        raise RuntimeError(f"{what} failed ({rc})")
    return {"ms": r.ms, "cycles_per_wave": r.cycles_per_wave, "clock_ghz": r.clock_ghz, "work": r.work}


def block(test: str, iters: int, n_cu: int, blocks_per_cu: int = 4) -> dict:
    r = moe_micro_result_t()
    return _res(lib().moe_micro_block(BLOCK_TESTS[test], iters, n_cu, blocks_per_cu, ctypes.byref(r)), r, test)


def copy(dst: torch.Tensor, src: torch.Tensor, grid: int, reps: int) -> dict:
    r = moe_micro_result_t()
    n = min(dst.numel() * dst.element_size(), src.numel() * src.element_size())
    return _res(lib().moe_micro_copy(dst.data_ptr(), src.data_ptr(), n, grid, reps, ctypes.byref(r)), r, "copy")


def atomic(src: torch.Tensor, dst_row: torch.Tensor, y: torch.Tensor, reps: int) -> dict:
    r = moe_micro_result_t()
    rows, d = src.shape
    return _res(lib().moe_micro_atomic(src.data_ptr(), dst_row.data_ptr(), y.data_ptr(), rows, d, reps,
                                       ctypes.byref(r)), r, "atomic")
