"""Pins for the CPU oracle: each check ties an oracle step to something other
than the oracle itself -- brute force on tiny inputs, closed forms, library
routines (numpy float16, fp64 matmul, math.exp), invariants, exact special
cases and a hand-derived worked example.  A dropped term, a wrong sign or
index, or a transposed operand in ``oracle.c`` fails at least one of these.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(12345)


# ------------------------------------------------------------------ fp16 ---

def test_f16_to_f64_matches_numpy_exhaustively(oracle_lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.f16_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # sign of zero
    assert math.copysign(1.0, got[0x8000]) == -1.0


# ------------------------------------------------------------------- exp ---

def _ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    ia = a.view(np.int32).astype(np.int64)
    ib = b.view(np.int32).astype(np.int64)
    return np.abs(ia - ib)


def test_exp_ref_accuracy_within_2ulp(oracle_lib):
    lo = np.float32(-103.9).view(np.int32)
    # every 97th fp32 in [-103.9, 0] and [0, 88.7] plus random points
    neg = np.arange(np.float32(-0.0).view(np.int32), lo, 97, dtype=np.int64).astype(np.uint32)
    neg = neg.view(np.float32)
    hi = np.float32(88.7).view(np.int32)
    pos = np.arange(0, hi, 97, dtype=np.int32).view(np.float32)
    x = np.concatenate([neg, pos, rng.uniform(-103, 88, 200000).astype(np.float32)])
    y = oracle.exp_ref(x)
    ref = np.exp(x.astype(np.float64)).astype(np.float32)   # fp64 exp, rounded once
    normal = ref >= np.float32(1.17549435e-38)
    d = _ulp_diff(y[normal], ref[normal])
    assert d.max() <= 2, (d.max(), x[normal][d.argmax()])
    # subnormal results: absolute error within 2 ulp of the smallest normal
    sub = ~normal
    assert np.all(np.abs(y[sub].astype(np.float64) - np.exp(x[sub].astype(np.float64))) < 2 * 2.0 ** -149 * 4)


def test_exp_ref_special_values(oracle_lib):
    e = oracle_lib._load().oracle_exp_ref
    assert e(0.0) == 1.0
    assert e(-0.0) == 1.0
    assert abs(e(1.0) - math.e) <= 2 * np.spacing(np.float32(math.e))
    assert e(89.5) == math.inf
    assert e(1e30) == math.inf
    assert e(-104.5) == 0.0
    assert e(-1e30) == 0.0
    assert math.isnan(e(float("nan")))
    # monotone on a dense sorted sample (catches a sign slip in the reduction)
    x = np.sort(rng.uniform(-20, 20, 100000).astype(np.float32))
    y = oracle.exp_ref(x)
    assert np.all(np.diff(y) >= 0)
    # exp(a) * exp(-a) == 1 within a few ulp
    a = rng.uniform(-40, 40, 10000).astype(np.float32)
    prod = oracle.exp_ref(a).astype(np.float64) * oracle.exp_ref(-a).astype(np.float64)
    assert np.max(np.abs(prod - 1.0)) < 4 * 2.0 ** -23


# ----------------------------------------------------------------- route ---

def _brute_topk(l: np.ndarray, k: int):
    order = sorted(range(l.size), key=lambda e: (-float(l[e]), e))
    return order[:k]


@pytest.mark.parametrize("E,k", [(8, 1), (8, 2), (8, 8), (16, 5), (64, 8), (130, 7)])
def test_route_topk_brute_force(oracle_lib, E, k):
    T = 40
    lg = rng.standard_normal((T, E)).astype(np.float32)
    eidx, w = oracle.route(lg, k)
    for t in range(T):
        assert list(eidx[t]) == _brute_topk(lg[t], k)


def test_route_ties_go_to_lower_index(oracle_lib):
    T, E, k = 200, 12, 4
    vals = np.array([-1.0, 0.0, -0.0, 0.5, 1.0, 1.0], dtype=np.float32)
    lg = vals[rng.integers(0, vals.size, (T, E))]
    eidx, w = oracle.route(lg, k)
    for t in range(T):
        assert list(eidx[t]) == _brute_topk(lg[t], k)
        # equal chosen logits -> equal weights
        for a in range(k):
            for b in range(k):
                if lg[t, eidx[t, a]] == lg[t, eidx[t, b]]:
                    assert w[t, a] == w[t, b]


def test_route_weights_closed_forms(oracle_lib):
    # k = 1 -> weight exactly 1
    lg = rng.standard_normal((30, 9)).astype(np.float32)
    _, w = oracle.route(lg, 1)
    assert np.all(w == 1.0)
    # all-equal logits -> lowest k indices, weights 1/k
    lg = np.full((5, 10), 0.3, dtype=np.float32)
    eidx, w = oracle.route(lg, 4)
    assert np.all(eidx == np.arange(4))
    assert np.allclose(w, 0.25, rtol=0, atol=1e-15)
    # two selected logits a and a - ln 3 -> weights 3/4 and 1/4
    a = np.float32(0.7)
    b = np.float32(np.float64(a) - math.log(3.0))
    lg = np.array([[b, -5.0, a, -6.0]], dtype=np.float32)
    eidx, w = oracle.route(lg, 2)
    assert list(eidx[0]) == [2, 0]
    exact = 1.0 / (1.0 + math.exp(float(b) - float(a)))
    assert abs(w[0, 0] - exact) < 1e-15 and abs(w[0, 0] - 0.75) < 1e-7
    # sum to one; non-increasing along the slots
    lg = rng.standard_normal((500, 128)).astype(np.float32)
    eidx, w = oracle.route(lg, 8)
    assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-14)
    assert np.all(np.diff(w, axis=1) <= 0)


# ----------------------------------------------------------------- group ---

@pytest.mark.parametrize("T,E,k", [(64, 8, 2), (33, 5, 5), (100, 128, 8), (7, 3, 1)])
def test_group_brute_force_and_invariants(oracle_lib, T, E, k):
    lg = rng.standard_normal((T, E)).astype(np.float32)
    eidx, _ = oracle.route(lg, k)
    counts, bounds, rows, pos = oracle.group(eidx, E)
    R = T * k
    flat = eidx.reshape(-1)
    brute = [p for e in range(E) for p in range(R) if flat[p] == e]
    assert list(rows) == brute
    assert bounds[0] == 0 and bounds[E] == R
    assert np.all(np.diff(bounds) >= 0)
    assert np.array_equal(np.diff(bounds), counts)
    assert np.array_equal(np.sort(rows), np.arange(R))
    assert np.array_equal(pos[rows], np.arange(R))
    for e in range(E):
        g = rows[bounds[e]:bounds[e + 1]]
        assert np.all(np.diff(g) > 0)
        assert np.all(flat[g] == e)


def test_group_k_equals_E(oracle_lib):
    T, E = 17, 6
    lg = rng.standard_normal((T, E)).astype(np.float32)
    eidx, _ = oracle.route(lg, E)
    counts, bounds, rows, pos = oracle.group(eidx, E)
    assert np.all(counts == T)
    for e in range(E):
        toks = rows[bounds[e]:bounds[e + 1]] // E
        assert np.array_equal(toks, np.arange(T))


# -------------------------------------------------------------- quantise ---

def test_q8_worked_example(oracle_lib):
    fx = json.load(open(os.path.join(GOLDEN, "q8_worked_example.json")))
    x = np.array([b["x"] for b in fx["blocks"]], dtype=np.float32).reshape(1, -1)
    q, s = oracle.quant_q8(x)
    assert list(s[0]) == [b["scale"] for b in fx["blocks"]]
    assert list(q[0]) == [v for b in fx["blocks"] for v in b["q"]]


def test_q8_invariants(oracle_lib):
    x = (rng.standard_normal((300, 256)) * rng.uniform(1e-3, 1e3, (300, 1))).astype(np.float32)
    x[5, 32:64] = 0.0
    q, s = oracle.quant_q8(x)
    xb = x.reshape(300, 8, 32).astype(np.float64)
    qb = q.reshape(300, 8, 32).astype(np.float64)
    amax = np.abs(xb).max(-1)
    assert np.array_equal(s, (amax.astype(np.float32) / np.float32(127.0)))
    assert s[5, 1] == 0 and np.all(qb[5, 1] == 0)
    nz = s > 0
    # the amax element maps to +-127
    arg = np.abs(xb).argmax(-1)
    top = np.take_along_axis(qb, arg[..., None], -1)[..., 0]
    assert np.all(np.abs(top[nz]) == 127)
    # reconstruction error at most half a step (plus fp32 rounding of the quotient)
    err = np.abs(xb - qb * s[..., None].astype(np.float64))
    assert np.all(err <= s[..., None] * 0.5 * (1 + 2.0 ** -20) + 1e-45)
    assert np.all(np.abs(qb) <= 127)


# ------------------------------------------------------------------ GEMM ---

def _rand_case(M, N, K, seed):
    r = np.random.default_rng(seed)
    A = r.integers(-127, 128, (M, K)).astype(np.int8)
    W = r.integers(-8, 8, (N, K)).astype(np.int8)
    sa = r.uniform(0.01, 0.1, (M, K // 32)).astype(np.float32)
    sw = r.uniform(0.01, 0.05, (N, K // 32)).astype(np.float16).view(np.uint16)
    return A, W, sa, sw


def test_block_dots_match_int64_reference(oracle_lib):
    A, W, _, _ = _rand_case(19, 23, 128, 1)
    got = oracle.block_dots(A, W)
    ref = np.einsum("mbi,nbi->mnb", A.reshape(19, 4, 32).astype(np.int64),
                    W.reshape(23, 4, 32).astype(np.int64))
    assert np.array_equal(got, ref)


def test_gemm_unit_scales_is_integer_matmul(oracle_lib):
    M, N, K = 37, 53, 4096
    A, W, _, _ = _rand_case(M, N, K, 2)
    sa = np.ones((M, K // 32), np.float32)
    sw = np.full((N, K // 32), 0x3C00, np.uint16)    # fp16 1.0
    ref = A.astype(np.int64) @ W.astype(np.int64).T
    assert np.array_equal(oracle.gemm_f32(A, sa, W, sw).astype(np.int64), ref)
    assert np.array_equal(oracle.gemm_f64(A, sa, W, sw).astype(np.int64), ref)


def test_gemm_equals_dequantised_fp64_matmul(oracle_lib):
    M, N, K = 29, 61, 512
    A, W, sa, sw = _rand_case(M, N, K, 3)
    deq_a = A.astype(np.float64) * np.repeat(sa.astype(np.float64), 32, axis=1)
    deq_w = W.astype(np.float64) * np.repeat(sw.view(np.float16).astype(np.float64), 32, axis=1)
    ref = deq_a @ deq_w.T
    g64 = oracle.gemm_f64(A, sa, W, sw)
    g32 = oracle.gemm_f32(A, sa, W, sw).astype(np.float64)
    # absolute-value mass of the block terms bounds the rounding error
    dots = oracle.block_dots(A, W).astype(np.float64)
    mass = np.abs(dots * sa[:, None, :] * sw.view(np.float16).astype(np.float64)[None]).sum(-1)
    assert np.all(np.abs(g64 - ref) <= 1e-13 * mass + 1e-300)
    nb = K // 32
    assert np.all(np.abs(g32 - ref) <= (nb + 2) * 2.0 ** -24 * mass)
    # the fp32 result is not identically the fp64 one (it does round)
    assert np.any(g32 != g64)


def test_gemm_power_of_two_weight_scale(oracle_lib):
    M, N, K = 11, 17, 256
    A, W, sa, sw = _rand_case(M, N, K, 4)
    sw2 = (sw.view(np.float16) * np.float16(2)).view(np.uint16)
    assert np.array_equal(oracle.gemm_f32(A, sa, W, sw2), 2 * oracle.gemm_f32(A, sa, W, sw))


# ---------------------------------------------------------------- SwiGLU ---

def test_swiglu_against_fp64_formula(oracle_lib):
    M, f = 64, 96
    gu = (rng.standard_normal((M, 2 * f)) * 8).astype(np.float32)
    gu[0, 0] = 0.0
    gu[0, 1] = -200.0
    gu[0, 2] = 200.0
    h = oracle.swiglu_f32(gu)
    g = gu[:, :f].astype(np.float64)
    u = gu[:, f:].astype(np.float64)
    with np.errstate(over="ignore"):
        ref = g / (1.0 + np.exp(-g)) * u
    rel = np.abs(h - ref) / np.maximum(np.abs(ref), 1e-30)
    ok = np.abs(ref) > 1e-30
    assert np.max(rel[ok]) < 8 * 2.0 ** -24
    assert h[0, 0] == 0.0
    assert h[0, 1] == 0.0
    assert h[0, 2] == np.float32(200.0) * gu[0, f + 2]


# --------------------------------------------------------------- combine ---

def test_combine_matches_einsum(oracle_lib):
    T, k, d, R = 20, 3, 40, 60
    w = rng.uniform(0, 1, (T, k))
    pos = rng.permutation(R).astype(np.int32).reshape(T, k)
    dm = rng.standard_normal((R, d))
    y = oracle.combine_f64(w, pos, dm)
    ref = np.einsum("tj,tjn->tn", w, dm[pos])
    assert np.allclose(y, ref, rtol=1e-14, atol=1e-14)
    onehot = np.zeros((T, k))
    onehot[:, 1] = 1.0
    assert np.array_equal(oracle.combine_f64(onehot, pos, dm), dm[pos[:, 1]])


def test_gemm_block_combination_worked_example():
    """R9 pinned by a hand-derived case (tests/golden/gemm_block_order_worked_example.json):
    one fused multiply-add per block in ascending block order gives 2^-25; a separate
    multiply and add, or the reverse block order, gives 0.0."""
    g = json.load(open(os.path.join(GOLDEN, "gemm_block_order_worked_example.json")))
    K = g["K"]
    A = np.zeros((1, K), np.int8)
    W = np.zeros((1, K), np.int8)
    for k, v in g["a_codes"].items():
        A[0, int(k)] = v
    for k, v in g["w_codes"].items():
        W[0, int(k)] = v
    a_scale = np.array([[int(b, 16) for b in g["a_scales_bits"]]], np.uint32).view(np.float32)
    w_scale = np.array([[int(b, 16) for b in g["w_scales_fp16_bits"]]], np.uint16)
    out = oracle.gemm_f32(A, a_scale, W, w_scale)
    assert out.view(np.uint32)[0, 0] == int(g["expected_bits"], 16)
    assert out[0, 0] == np.float32(2.0 ** -25)
    assert int(g["mul_then_add_bits"], 16) != int(g["expected_bits"], 16)
