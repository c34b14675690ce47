"""The kernels' fp32 exponential against the oracle's, on every fp32 input in
[-104, 89] (about 2.24e9 values; the negative and the positive bit-pattern
ranges, the subnormal-result tail included).

H = silu(G) * U and therefore every Hq code rests on the two sides' exp giving
the same bits, so the comparison is exact.  The CPU test runs the host build of
the library's exp source; the GPU test runs the kernel build of the same source
through moe_prefill_exp_device.  Both compare against oracle.exp_ref, which is
pinned to fp64 exp separately (test_oracle_pins.py)."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import moe_prefill_ffn_amd as mp
import oracle

# fp32 bit patterns of the inputs in [-104, 89]: +0 .. 89.0 and -0 .. -104.0
POS = (0x00000000, 0x42B20000)        # 0x42B20000 = 89.0
NEG = (0x80000000, 0xC2D00000)        # 0xC2D00000 = -104.0
CHUNK = 1 << 24


def _chunks():
    for lo, hi in (POS, NEG):
        for a in range(lo, hi + 1, CHUNK):
            yield a, min(CHUNK, hi + 1 - a)


def _inputs(first: int, n: int) -> np.ndarray:
    return (np.arange(n, dtype=np.uint64) + first).astype(np.uint32).view(np.float32)


def _mismatch(first: int, got: np.ndarray, ref: np.ndarray):
    bad = np.nonzero(got.view(np.uint32) != ref.view(np.uint32))[0]
    if bad.size == 0:
        return None
    i = int(bad[0])
    x = _inputs(first + i, 1)[0]
    return f"{bad.size} differ from bits {first:#010x}; first x = {x!r}: got {got[i]!r} ref {ref[i]!r}"


def test_bounds_of_the_range():
    assert _inputs(POS[1], 1)[0] == np.float32(89.0)
    assert _inputs(NEG[1], 1)[0] == np.float32(-104.0)
    assert sum(n for _, n in _chunks()) == (POS[1] - POS[0] + 1) + (NEG[1] - NEG[0] + 1)


def test_host_build_exp_equals_oracle_on_every_input():
    def one(c):
        first, n = c
        got = mp.moe_prefill_exp_host(first, np.empty(n, np.float32))
        return _mismatch(first, got, oracle.exp_ref(_inputs(first, n)))

    with ThreadPoolExecutor(8) as ex:          # ctypes releases the GIL during the calls
        errs = [e for e in ex.map(one, list(_chunks())) if e]
    assert not errs, errs[:3]


@pytest.mark.gpu
def test_kernel_exp_equals_oracle_on_every_input():
    import torch

    print("[case] exhaustive exp on the device", flush=True)
    big = 1 << 27
    out = torch.empty(big, dtype=torch.float32, device="cuda")
    host = torch.empty(big, dtype=torch.float32, pin_memory=True)
    errs = []
    for lo, hi in (POS, NEG):
        for first in range(lo, hi + 1, big):
            n = min(big, hi + 1 - first)
            mp.moe_prefill_exp_device(first, out[:n])
            host[:n].copy_(out[:n])
            torch.cuda.synchronize()
            got = host[:n].numpy()
            e = _mismatch(first, got, oracle.exp_ref(_inputs(first, n)))
            if e:
                errs.append(e)
    assert not errs, errs[:3]
