"""Property tests of the pool planner and the memory-pressure trim (host code, no
GPU), over random stacks, budgets and requests.  They state the layer-streaming
pages' policy as invariants rather than single cases: the execution slot is
mandatory and the budget otherwise caps the pool (page #1906, pool-behaviour
table); the prefetch window is filled before any layer is made resident and
residents are the leading layers (page #1905, "Summary"); under memory pressure
residents are evicted from the end of the resident prefix before the prefetch
window shrinks, and the active slot is never given up (page #1905, "Summary")."""
from hypothesis import given, settings, strategies as st

import moe_prefill_ffn_amd as mp

SLOT = 7 * (1 << 20)


def _plan(L, depth, res, budget_slots, requested, max_alloc, slack=0):
    budget = budget_slots * SLOT + slack if budget_slots > 0 else 0
    return mp.moe_prefill_plan_pool(L, SLOT, depth, res, budget, requested, max_alloc)


plans = st.tuples(st.integers(1, 64),              # layers
                  st.integers(0, 12),              # requested prefetch depth
                  st.integers(-1, 70),             # requested residents (-1: as many as fit)
                  st.integers(0, 80),              # budget in slots (0: none)
                  st.integers(0, 80),              # requested slots (0: none)
                  st.integers(0, 80),              # slots that can be allocated (0: any)
                  st.integers(0, SLOT - 1))        # budget bytes beyond whole slots


@settings(max_examples=400, deadline=None)
@given(plans)
def test_plan_shape_invariants(args):
    L, depth, res, budget, requested, max_alloc, slack = args
    p = _plan(L, depth, res, budget, requested, max_alloc, slack)
    assert p["rc"] == 0
    s, d, r = p["slots"], p["depth"], p["residents"]
    assert s >= 1 and d >= 0 and 0 <= r <= L
    if r == L:                                     # everything resident: no streaming slot
        assert (s, d) == (L, 0)
    else:
        assert s == r + 1 + d                      # residents + the active slot + the window
        assert d <= L - r - 1                      # never prefetch beyond the streamed layers
    assert d <= depth
    if res >= 0:
        assert r <= res
    # caps: the budget, the requested slots and what can be allocated, but never below one slot
    for cap in (budget if budget > 0 else 0, requested, max_alloc):
        if cap > 0:
            assert s <= max(cap, 1)
    # the prefetch window comes before residents
    if 0 < r < L:
        assert d == min(depth, L - r - 1)


@settings(max_examples=300, deadline=None)
@given(plans)
def test_plan_budget_is_monotone(args):
    L, depth, res, budget, requested, max_alloc, slack = args
    if budget == 0:
        return
    a = _plan(L, depth, res, budget, requested, max_alloc, slack)
    b = _plan(L, depth, res, budget + 1, requested, max_alloc, slack)
    assert b["slots"] >= a["slots"]
    assert b["residents"] >= a["residents"] or b["depth"] > a["depth"]


@settings(max_examples=300, deadline=None)
@given(st.integers(1, 64), st.integers(0, 12), st.integers(-1, 70))
def test_plan_one_slot_allocation_failure_is_an_error(L, depth, res):
    assert _plan(L, depth, res, 0, 0, -1)["rc"] == mp.MOE_ENOMEM


def _valid_pool(L, residents, streaming):
    """The pools the planner makes: residents <= L; a streaming slot whenever a layer
    streams; at least one slot."""
    return residents <= L and residents + streaming >= 1 and (residents == L or streaming >= 1)


@settings(max_examples=600, deadline=None)
@given(st.integers(1, 64), st.integers(0, 64), st.integers(0, 14), st.integers(-2, 90))
def test_trim_invariants(L, residents, streaming, budget):
    t = mp.moe_prefill_plan_trim(L, residents, streaming, budget)
    if not _valid_pool(L, residents, streaming):
        assert t["rc"] == mp.MOE_EINVAL
        return
    assert t["rc"] == 0
    r, s = t["residents"], t["streaming"]
    alive_before, alive = residents + streaming, r + s
    assert 0 <= r <= residents and 0 <= s
    assert t["evicted"] == residents - r                   # evicted layers are residents
    assert t["released"] == alive_before - alive           # released slots go back
    assert alive >= 1 and (r == L or s >= 1)               # the active slot stays
    target = max(budget, 1)
    if alive_before <= target:                             # within budget: nothing changes
        assert (r, s, t["evicted"], t["released"], t["converted"]) == (residents, streaming, 0, 0, 0)
    else:
        assert alive <= target or (r == 0 and s == 1)      # fits, unless only the active slot is left
    if s < streaming:                                      # the window shrinks only after every
        assert r == 0                                      # resident is gone
    # an all-resident pool turns its first evicted layer's slot into the streaming slot
    assert t["converted"] == (1 if streaming == 0 and t["evicted"] > 0 else 0)
    if streaming == 0 and t["evicted"] > 0:
        assert s == 1


@settings(max_examples=300, deadline=None)
@given(st.integers(1, 64), st.integers(0, 64), st.integers(1, 14), st.integers(1, 90), st.integers(1, 90))
def test_trim_is_monotone_in_the_budget(L, residents, streaming, b1, b2):
    if not _valid_pool(L, residents, streaming):
        return
    lo, hi = sorted((b1, b2))
    a = mp.moe_prefill_plan_trim(L, residents, streaming, lo)
    b = mp.moe_prefill_plan_trim(L, residents, streaming, hi)
    assert b["residents"] >= a["residents"] and b["streaming"] >= a["streaming"]
