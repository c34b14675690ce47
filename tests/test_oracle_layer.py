"""Layer-level pins for the oracle: metamorphic relations that hold exactly for
the prompt-path FFN layer (token permutation, zero input, exact power-of-two
scalings, identical experts reducing to a dense FFN) plus the workload
generator's own determinism and distributions."""
import dataclasses

import numpy as np
import pytest

import oracle
import workload as wl


def _experts_fn(w, layer=0):
    cache = {}

    def get(e):
        if e not in cache:
            cache[e] = wl.expert_weights(w, layer, e)
        return cache[e]
    return get


@pytest.fixture(scope="module")
def tiny():
    w = wl.WORKLOADS["tiny"]
    x = wl.layer_activations(w, 0)
    lg = wl.layer_logits(w, 0)
    ex = _experts_fn(w)
    out = oracle.layer(x, lg, w.k, ex, w.f)
    return w, x, lg, ex, out


def test_tiny_layer_shapes_and_group_invariants(tiny):
    w, x, lg, ex, out = tiny
    R = w.T * w.k
    assert out["y"].shape == (w.T, w.d)
    assert np.array_equal(np.sort(out["rows"]), np.arange(R))
    assert out["bounds"][-1] == R
    assert np.allclose(out["w"].sum(1), 1.0, atol=1e-14)
    assert np.all(np.isfinite(out["y"]))


def test_token_permutation_permutes_output(tiny):
    w, x, lg, ex, out = tiny
    perm = np.random.default_rng(7).permutation(w.T)
    out2 = oracle.layer(x[perm], lg[perm], w.k, ex, w.f)
    assert np.array_equal(out2["y"], out["y"][perm])


def test_zero_input_gives_zero_output(tiny):
    w, x, lg, ex, out = tiny
    out2 = oracle.layer(np.zeros_like(x), lg, w.k, ex, w.f)
    assert np.all(out2["xq"] == 0) and np.all(out2["dx"] == 0)
    assert np.all(out2["y"] == 0)


def _scaled(ex, which):
    def get(e):
        W = ex(e)
        W = dataclasses.replace(W)
        if which == "down":
            W.wd_s = (W.wd_s.view(np.float16) * np.float16(2)).view(np.uint16)
        else:                                 # the up half of the gate/up matrix
            s = W.wgu_s.copy()
            f = s.shape[0] // 2
            s[f:] = (s[f:].view(np.float16) * np.float16(2)).view(np.uint16)
            W.wgu_s = s
        return W
    return get


@pytest.mark.parametrize("which", ["down", "up"])
def test_power_of_two_scale_doubles_output_exactly(tiny, which):
    w, x, lg, ex, out = tiny
    out2 = oracle.layer(x, lg, w.k, _scaled(ex, which), w.f)
    assert np.array_equal(out2["y"], 2 * out["y"])
    assert np.array_equal(out2["hq"], out["hq"])


def test_identical_experts_reduce_to_dense_ffn(tiny):
    w, x, lg, ex, out = tiny
    same = lambda e: ex(3)
    out_k = oracle.layer(x, lg, w.k, same, w.f)
    out_1 = oracle.layer(x, lg, 1, same, w.f)          # one expert, weight 1: a dense FFN
    assert np.allclose(out_k["y"], out_1["y"], rtol=1e-13, atol=1e-12)


def test_sampled_tokens_match_full_layer(tiny):
    w, x, lg, ex, out = tiny
    toks = [0, 5, 17, 63, 40]
    part = oracle.layer(x, lg, w.k, ex, w.f, tokens=toks)
    assert np.array_equal(part["y"], out["y"][sorted(toks)])


# -------------------------------------------------------------- generator ---

def test_generator_is_deterministic_and_counter_based():
    a = wl.u64(5, 1, 2, 0, 1000)
    b = wl.u64(5, 1, 2, 0, 1000)
    assert np.array_equal(a, b)
    # element i can be drawn on its own
    c = wl.u64(5, 1, 2, 600, 10)
    assert np.array_equal(c, a[600:610])
    assert not np.array_equal(wl.u64(5, 1, 3, 0, 10), a[:10])


def test_generator_distributions():
    z = wl.normal(11, wl.T_X, 400000)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01
    q = wl.int4(11, wl.T_WGU_Q, 0, 160000)
    assert q.min() == -8 and q.max() == 7
    cnt = np.bincount(q.astype(np.int64) + 8, minlength=16)
    assert np.all(np.abs(cnt / q.size - 1 / 16) < 0.005)
    s = wl.scale_f16(11, wl.T_WGU_S, 0, 50000, 2048).view(np.float16).astype(np.float64)
    assert s.min() >= 0.5 / np.sqrt(2048) * (1 - 1e-3) and s.max() <= 1.5 / np.sqrt(2048) * (1 + 1e-3)


def test_zipf_bias_and_skew():
    w = wl.WORKLOADS["skew"]
    b = wl.expert_bias(w, 0)
    ranks = np.rint(np.exp(-b.astype(np.float64) / 1.1)).astype(int)
    assert sorted(ranks) == list(range(1, w.E + 1))
