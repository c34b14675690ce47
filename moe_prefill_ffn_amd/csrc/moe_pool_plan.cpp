// Slot-pool planning: a pure function of the request, the slot size and the
// allocator's (simulated) limit.  Policy from the layer-streaming pages:
//  - "feat: prefetch streamed layers during compute" (stable-diffusion.cpp
//    #1905), "Summary" and "Effective behavior": the effective prefetch depth
//    shrinks to fit the budget, the budget is never exceeded by optional
//    slots, the active segment is never evicted, residency is a maximum
//    (-1 = whatever the budget leaves), and the prefetch window is served
//    before optional residents;
//  - "feat: pool VRAM for streamed layer" (#1906), "Summary" and the
//    pool-behaviour table: only the peak slot count is allocated; the one
//    mandatory slot is execution memory and is tried even above the budget
//    (with a warning); on allocation failure progressively smaller pools of
//    the same slot size are tried; if one slot fails, creation fails clearly;
//  - #1905 "Summary": under runtime memory pressure residents are evicted from
//    the end of the resident prefix (plan_trim), the active segment never.
#include "moe_pool_plan.h"

#include <stdint.h>

namespace moe {

// Fit a request into n slots: window first, then residents.
static PoolShape refit(int64_t n, int L, int depth_req, int residents_req)
{
    PoolShape s;
    int64_t depth = depth_req < n - 1 ? depth_req : n - 1;
    if (depth < 0) depth = 0;
    int64_t avail = n - 1 - depth;
    int64_t res = residents_req < 0 ? avail : (residents_req < avail ? residents_req : avail);
    if (res > L) res = L;
    if (res < 0) res = 0;
    if (res == L) {
        s.residents = L;
        s.depth = 0;
        s.slots = L;
    } else {
        const int64_t streamed = L - res;
        if (depth > streamed - 1) depth = streamed - 1;
        s.residents = (int)res;
        s.depth = (int)depth;
        s.slots = (int)(res + 1 + depth);
    }
    return s;
}

PoolShape plan_initial(int L, uint64_t slot_bytes, int depth_req, int residents_req,
                       int64_t budget, int requested_slots, int* warnings)
{
    int64_t cap = INT64_MAX / 4;
    if (budget > 0) cap = budget / (int64_t)slot_bytes;
    if (requested_slots > 0 && requested_slots < cap) cap = requested_slots;
    if (cap < 1) {
        cap = 1;
        if (budget > 0 && (int64_t)slot_bytes > budget) *warnings |= kWarnSlotOverBudget;
    }
    PoolShape s = refit(cap, L, depth_req, residents_req);
    if (s.depth < depth_req && s.residents < L) *warnings |= kWarnDepthReduced;
    return s;
}

PoolShape plan_degrade(const PoolShape& cur, int L, int depth_req, int residents_req, int* warnings)
{
    PoolShape s = refit((int64_t)cur.slots - 1, L, depth_req, residents_req);
    *warnings |= kWarnPoolDegraded;
    if (s.depth < depth_req && s.residents < L) *warnings |= kWarnDepthReduced;
    return s;
}

PoolTrim plan_trim(int L, int residents, int streaming, int64_t budget_slots, int* warnings)
{
    PoolTrim t;
    t.residents = residents;
    t.streaming = streaming;
    int64_t alive = (int64_t)residents + streaming;
    int64_t target = budget_slots;
    if (target < 1) {
        target = 1;
        *warnings |= kWarnSlotOverBudget;
    }
    while (alive > target && t.residents > 0) {
        --t.residents;
        ++t.evicted;
        if (t.streaming == 0) {
            t.streaming = 1;       // the evicted layer's slot keeps it, now as a streaming slot
            t.converted = 1;
        } else {
            ++t.released;
            --alive;
        }
    }
    const int depth_before = streaming > 0 ? streaming - 1 : 0;
    while (alive > target && t.streaming > 1) {
        --t.streaming;
        ++t.released;
        --alive;
    }
    if (t.residents < L && t.streaming - 1 < depth_before) *warnings |= kWarnDepthReduced;
    return t;
}

}  // namespace moe
