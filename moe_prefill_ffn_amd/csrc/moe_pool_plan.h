// Slot-pool planner (pure; no device calls).
#pragma once

#include <stdint.h>

namespace moe {

constexpr int kWarnSlotOverBudget = 1;
constexpr int kWarnPoolDegraded = 2;
constexpr int kWarnDepthReduced = 4;

struct PoolShape {
    int slots = 0;       // total slots = residents + (residents < L ? 1 + depth : 0)
    int depth = 0;       // prefetch lookahead
    int residents = 0;   // resident leading layers
};

// First plan for L layers (L >= 1).
PoolShape plan_initial(int L, uint64_t slot_bytes, int depth_req, int residents_req,
                       int64_t budget, int requested_slots, int* warnings);

// The next smaller pool after an allocation of cur.slots slots failed
// (cur.slots >= 2): one slot fewer, prefetch window kept before residents.
PoolShape plan_degrade(const PoolShape& cur, int L, int depth_req, int residents_req, int* warnings);

// Shrinking a live pool to a budget of budget_slots slots (memory pressure).
struct PoolTrim {
    int residents = 0;      // resident leading layers left
    int streaming = 0;      // streaming slots left
    int evicted = 0;        // residents evicted (from the end of the resident prefix)
    int converted = 0;      // 1: the first evicted resident's slot became the streaming slot
    int released = 0;       // slots whose memory is returned
};

// residents + streaming alive slots of an L-layer stack.  Residents leave
// from the end of the prefix before any prefetch slot; the last slot is
// never released (execution memory, kept even above the budget: warning).  A
// pool without a streaming slot turns its first evicted resident into one.
PoolTrim plan_trim(int L, int residents, int streaming, int64_t budget_slots, int* warnings);

}  // namespace moe
