// Host runtime behind the C ABI (include/moe_prefill.h): handle + workspace,
// layer launch, fixed-slot pool with a lookahead prefetch queue on its own
// HIP stream, event fencing, stats and errors.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <array>
#include <chrono>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "../../include/moe_prefill.h"
#include "moe_kernels.h"
#include "moe_layout.h"
#include "moe_pool_plan.h"

namespace moe {
bool pack_expert(int d, int f, const int8_t* wgu_q, const uint16_t* wgu_s, const int8_t* wd_q,
                 const uint16_t* wd_s, uint8_t* dst);
}

using namespace moe;

struct moe_prefill {
    int dev = 0;
    int d = 0, f = 0, E = 0, k = 0, Tmax = 0;
    WsLayout L{};
    BlobLayout B{};
    uint8_t* ws = nullptr;
    bool ws_owned = false;
    hipStream_t copy = nullptr;
    std::string err;
    bool mask_dirty = false;

    // stream pool
    bool pool_on = false;
    int nl = 0;
    std::vector<const void*> blobs;
    bool active_only = false;
    std::vector<const uint8_t*> blobs_dev;   // device addresses of the pinned host blobs (active_only)
    uint64_t layer_bytes = 0, slot_bytes = 0;
    PoolShape shape;                 // the plan at configure time (shape.slots = address-range slots)
    int warnings = 0;
    uint8_t* pool = nullptr;
    // pool memory: one reserved device address range.  With virtual memory management
    // every slot has its own physical allocation, so a released slot returns its
    // memory; otherwise the range is one hipMalloc and nothing is released early.
    bool vmm = false;
    uint64_t va_bytes = 0;
    std::vector<hipMemGenericAllocationHandle_t> phys;
    std::vector<char> slot_kind;     // kSlotStreaming / kSlotResident / kSlotReleased
    int res_live = 0;                // resident leading layers now (layer i lives in slot i)
    int depth_live = 0;              // effective prefetch depth now
    int64_t reserve_bytes = 0;       // free device memory to keep (0: off)
    std::vector<int> slot_layer, layer_slot;
    std::vector<hipEvent_t> ev_ready, ev_free;
    std::vector<char> ready_set, free_set, from_prefetch;
    int active = -1;
    uint64_t prefetch_counter = 0;
    uint64_t fail_at = 0;   // test hook: this prefetch enqueue (1-based) is treated as failed

    moe_stats_t stats{};

    // logging
    moe_log_fn log_fn = nullptr;
    void* log_user = nullptr;
    int log_level = -1;               // sink threshold; -1: MOE_LOG_LEVEL decides (stderr)
    bool poison = false;              // MOE_DEBUG_POISON: fill a slot with NaN bytes before each refill

    // kernel timing
    bool timing = false;
    struct TimedLayer {
        std::array<hipEvent_t, kNumKernels + 1> ev{};
        uint32_t launched = 0;          // bit i: kernel i ran in this layer
    };
    std::vector<TimedLayer> t_pending;
    std::vector<std::array<hipEvent_t, kNumKernels + 1>> t_free;
    uint64_t t_launches[kNumKernels] = {};
    double t_ms[kNumKernels] = {};
};

static thread_local std::string g_err;

static int env_log_level()
{
    const char* e = getenv("MOE_LOG_LEVEL");
    return e ? atoi(e) : -1;
}

static void log_msg(const moe_prefill_t* h, int level, const std::string& msg)
{
    if (h && h->log_fn) {
        if (level <= h->log_level) h->log_fn(level, msg.c_str(), h->log_user);
        return;
    }
    if (level <= env_log_level()) {
        static const char* tag[3] = {"error", "warning", "info"};
        fprintf(stderr, "moe_prefill %s: %s\n", tag[level < 0 ? 0 : (level > 2 ? 2 : level)], msg.c_str());
    }
}

static int fail(moe_prefill_t* h, int code, const std::string& msg)
{
    if (h)
        h->err = msg;
    else
        g_err = msg;
    log_msg(h, MOE_LOG_ERROR, msg);
    return code;
}

// the MOE_WARN_* bits as one message (nothing if none is set)
static void log_warnings(const moe_prefill_t* h, int warn, const std::string& where)
{
    if (warn & kWarnSlotOverBudget) log_msg(h, MOE_LOG_WARN, where + ": the one mandatory slot exceeds the budget");
    if (warn & kWarnPoolDegraded) log_msg(h, MOE_LOG_WARN, where + ": allocation failed, a smaller pool is used");
    if (warn & kWarnDepthReduced) log_msg(h, MOE_LOG_WARN, where + ": prefetch depth reduced to fit");
}

static int hip_fail(moe_prefill_t* h, hipError_t e, const char* what)
{
    return fail(h, MOE_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

namespace {

struct DevGuard {
    int prev = -1;
    explicit DevGuard(int d)
    {
        if (hipGetDevice(&prev) != hipSuccess) prev = -1;
        (void)hipSetDevice(d);
    }
    ~DevGuard()
    {
        if (prev >= 0) (void)hipSetDevice(prev);
    }
};

// Versioned struct in: a smaller struct_size leaves trailing fields at 0; a
// larger one is accepted only if every unknown byte is zero.
template <class S>
bool read_struct(const void* src, S* dst, std::string* why)
{
    memset(dst, 0, sizeof(S));
    if (!src) {
        *why = "null struct pointer";
        return false;
    }
    uint32_t sz;
    memcpy(&sz, src, 4);
    if (sz < 8) {
        *why = "struct_size too small";
        return false;
    }
    if (sz <= sizeof(S)) {
        memcpy(dst, src, sz);
    } else {
        memcpy(dst, src, sizeof(S));
        const uint8_t* b = static_cast<const uint8_t*>(src);
        for (uint32_t i = sizeof(S); i < sz; ++i)
            if (b[i]) {
                *why = "struct_size larger than this library knows, with nonzero unknown fields";
                return false;
            }
    }
    dst->struct_size = sizeof(S);
    return true;
}

template <class S>
void write_struct(void* dst, const S& src)
{
    uint32_t sz;
    memcpy(&sz, dst, 4);
    S tmp = src;
    const uint32_t n = sz < sizeof(S) ? sz : (uint32_t)sizeof(S);
    memcpy(dst, &tmp, n);
    memcpy(dst, &sz, 4);   // keep the caller's struct_size
}

int64_t wait_budget_ms()
{
    const char* s = getenv("MOE_WAIT_MS");
    return s ? atoll(s) : 120000;
}

// Bounded host waits (a wait that expires returns MOE_ETIMEOUT).
int wait_stream(moe_prefill_t* h, hipStream_t st)
{
    const auto t0 = std::chrono::steady_clock::now();
    const int64_t lim = wait_budget_ms();
    for (;;) {
        const hipError_t e = hipStreamQuery(st);
        if (e == hipSuccess) return MOE_OK;
        if (e != hipErrorNotReady) return hip_fail(h, e, "hipStreamQuery");
        const auto ms = std::chrono::duration_cast<std::chrono::milliseconds>(
                            std::chrono::steady_clock::now() - t0).count();
        if (lim > 0 && ms > lim) return fail(h, MOE_ETIMEOUT, "copy stream wait timed out");
        std::this_thread::sleep_for(std::chrono::microseconds(50));
    }
}

int wait_event(moe_prefill_t* h, hipEvent_t ev)
{
    const auto t0 = std::chrono::steady_clock::now();
    const int64_t lim = wait_budget_ms();
    for (;;) {
        const hipError_t e = hipEventQuery(ev);
        if (e == hipSuccess) return MOE_OK;
        if (e != hipErrorNotReady) return hip_fail(h, e, "hipEventQuery");
        const auto ms = std::chrono::duration_cast<std::chrono::milliseconds>(
                            std::chrono::steady_clock::now() - t0).count();
        if (lim > 0 && ms > lim) return fail(h, MOE_ETIMEOUT, "event wait timed out");
        std::this_thread::sleep_for(std::chrono::microseconds(50));
    }
}

bool dims_ok(const moe_prefill_params_t& p, std::string* why)
{
    auto bad = [&](const char* m) {
        *why = m;
        return false;
    };
    if (p.d_model < 32 || p.d_model > 16384 || p.d_model % 32) return bad("d_model must be a multiple of 32 in [32, 16384]");
    if (p.d_ff < 32 || p.d_ff > 16384 || p.d_ff % 32) return bad("d_ff must be a multiple of 32 in [32, 16384]");
    if (p.n_experts < 1 || p.n_experts > 1024) return bad("n_experts must be in [1, 1024]");
    if (p.top_k < 1 || p.top_k > p.n_experts) return bad("top_k must be in [1, n_experts]");
    if (p.max_tokens < 1 || (int64_t)p.max_tokens * p.top_k > (1 << 21)) return bad("max_tokens must be >= 1 and max_tokens*top_k <= 2^21");
    return true;
}

// Workspace pointers of one layer launch (ws: the workspace base, L its layout).
void bind_layer(LayerLaunch& LL, uint8_t* w, const WsLayout& L, const BlobLayout& B)
{
    LL.W = L.W;
    LL.load_stats = reinterpret_cast<unsigned long long*>(w + L.load_stats);
    LL.expert_stride = B.expert_bytes;
    LL.gu_q_off = B.gu_q;
    LL.gu_s_off = B.gu_s;
    LL.d_q_off = B.d_q;
    LL.d_s_off = B.d_s;
    LL.eidx = reinterpret_cast<int32_t*>(w + L.eidx);
    LL.wts = reinterpret_cast<float*>(w + L.wts);
    LL.mask = reinterpret_cast<uint32_t*>(w + L.mask);
    LL.wprefix = reinterpret_cast<int32_t*>(w + L.wprefix);
    LL.counts = reinterpret_cast<int32_t*>(w + L.counts);
    LL.bounds = reinterpret_cast<int32_t*>(w + L.bounds);
    LL.tiles = reinterpret_cast<int32_t*>(w + L.tiles);
    LL.ntiles = reinterpret_cast<int32_t*>(w + L.ntiles);
    LL.rows = reinterpret_cast<int32_t*>(w + L.rows);
    LL.pos = reinterpret_cast<int32_t*>(w + L.pos);
    LL.rtok = reinterpret_cast<int32_t*>(w + L.rtok);
    LL.xq = reinterpret_cast<int8_t*>(w + L.xq);
    LL.dx = reinterpret_cast<float*>(w + L.dx);
    LL.hq = reinterpret_cast<int8_t*>(w + L.hq);
    LL.dh = reinterpret_cast<float*>(w + L.dh);
    LL.dm = reinterpret_cast<float*>(w + L.dm);
}

// Stream-ordered copies of the requested intermediate buffers out of the workspace.
// (rows x row_bytes, read with a source row stride of src_pitch bytes: the block-scale
// arrays are kept with a padded row stride in the workspace.)  GU is not here: the
// gate/up GEMM writes it straight into the caller's buffer.
hipError_t export_copies(const moe_layer_io_t& io, const uint8_t* ws, const WsLayout& L, int T, int d, int f,
                         int E, int k, hipStream_t st)
{
    const uint64_t R = (uint64_t)T * k;
    struct Ex {
        void* dst;
        uint64_t off, rows, row_bytes, src_pitch;
    } ex[] = {
        {io.eidx, L.eidx, 1, R * 4, R * 4},
        {io.weights, L.wts, 1, R * 4, R * 4},
        {io.counts, L.counts, 1, (uint64_t)E * 4, (uint64_t)E * 4},
        {io.bounds, L.bounds, 1, (uint64_t)(E + 1) * 4, (uint64_t)(E + 1) * 4},
        {io.rows, L.rows, 1, R * 4, R * 4},
        {io.pos, L.pos, 1, R * 4, R * 4},
        {io.xq, L.xq, 1, (uint64_t)T * d, (uint64_t)T * d},
        {io.dx, L.dx, (uint64_t)T, (uint64_t)(d / 32) * 4, (uint64_t)scale_stride(d) * 4},
        {io.hq, L.hq, 1, R * f, R * f},
        {io.dh, L.dh, R, (uint64_t)(f / 32) * 4, (uint64_t)scale_stride(f) * 4},
        {io.dm, L.dm, 1, R * d * 4, R * d * 4},
    };
    for (const Ex& x : ex) {
        if (!x.dst || x.rows == 0) continue;
        hipError_t e;
        if (x.rows == 1 || x.row_bytes == x.src_pitch)
            e = hipMemcpyAsync(x.dst, ws + x.off, x.rows * x.row_bytes, hipMemcpyDeviceToDevice, st);
        else
            e = hipMemcpy2DAsync(x.dst, x.row_bytes, ws + x.off, x.src_pitch, x.row_bytes, x.rows,
                                 hipMemcpyDeviceToDevice, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// The allocation-free entry point's device check (gfx950), once per device.
int noalloc_device_ok(int dev)
{
    static std::mutex mu;
    static std::vector<signed char> ok;                  // -1 unknown, 0 refused, 1 accepted
    std::lock_guard<std::mutex> lock(mu);
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) return fail(nullptr, MOE_EUNSUPPORTED, "no HIP device");
    if (dev < 0 || dev >= ndev) return fail(nullptr, MOE_EINVAL, "device ordinal out of range");
    if ((int)ok.size() < ndev) ok.resize(ndev, -1);
    if (ok[dev] < 0) {
        hipDeviceProp_t prop;
        const hipError_t e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return hip_fail(nullptr, e, "hipGetDeviceProperties");
        ok[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
    }
    if (!ok[dev]) return fail(nullptr, MOE_EUNSUPPORTED, "device is not gfx950");
    return MOE_OK;
}

// --------------------------------------------------------------- pool ops ---

// Layers of the prefetch window after `cur`: the next `depth` streamed layers
// in pass order (wrapping to the next pass), never `cur` itself.
enum : char { kSlotStreaming = 0, kSlotResident = 1, kSlotReleased = 2 };

std::vector<int> window_after(const moe_prefill_t* h, int cur)
{
    std::vector<int> w;
    const int res = h->res_live;
    if (res >= h->nl) return w;
    for (int i = 1; i < h->nl && (int)w.size() < h->depth_live; ++i) {
        const int y = (cur + i) % h->nl;
        if (y >= res && y != cur) w.push_back(y);
    }
    return w;
}

// Streaming slot to (re)fill: not `exclude`, not holding `cur` or a layer of
// cur's window; an empty slot first, else the one whose layer comes last.
int pick_victim(const moe_prefill_t* h, int cur, int exclude)
{
    const std::vector<int> win = window_after(h, cur);
    int best = -1;
    long best_score = -1;
    for (int s = 0; s < h->shape.slots; ++s) {
        if (s == exclude || h->slot_kind[s] != kSlotStreaming) continue;
        const int lay = h->slot_layer[s];
        bool keep = lay >= 0 && lay == cur;
        for (int y : win) keep = keep || lay == y;
        if (keep) continue;
        const long score = lay < 0 ? (1L << 40) : (long)((lay - cur + h->nl) % h->nl);
        if (score > best_score) {
            best_score = score;
            best = s;
        }
    }
    return best;
}

hipError_t enqueue_copy(moe_prefill_t* h, int s, int layer)
{
    const int old = h->slot_layer[s];
    if (old >= 0) h->layer_slot[old] = -1;
    h->slot_layer[s] = -1;
    h->from_prefetch[s] = 0;
    hipError_t e = hipSuccess;
    if (h->free_set[s]) e = hipStreamWaitEvent(h->copy, h->ev_free[s], 0);
    if (e == hipSuccess && h->poison)   // debug: a read of the slot between free and refill sees NaN
        e = launch_fill_u32(reinterpret_cast<uint32_t*>(h->pool + (uint64_t)s * h->slot_bytes),
                            (int64_t)(h->slot_bytes / 4), 0xFFFFFFFFu, h->copy);
    if (e == hipSuccess)
        e = hipMemcpyAsync(h->pool + (uint64_t)s * h->slot_bytes, h->blobs[layer], h->layer_bytes,
                           hipMemcpyHostToDevice, h->copy);
    if (e == hipSuccess) e = hipEventRecord(h->ev_ready[s], h->copy);
    if (e != hipSuccess) return e;
    h->ready_set[s] = 1;
    h->slot_layer[s] = layer;
    h->layer_slot[layer] = s;
    h->stats.bytes_h2d += h->layer_bytes;
    return hipSuccess;
}

// Pool memory for n slots of slot_bytes: a reserved address range with one physical
// allocation mapped per slot (vmm), else one hipMalloc.  On failure nothing is left allocated.
hipError_t pool_alloc(moe_prefill_t* h, int n, uint64_t slot_bytes)
{
    const uint64_t bytes = (uint64_t)n * slot_bytes;
    h->phys.assign(n, 0);
    if (!h->vmm) {
        h->va_bytes = bytes;
        return hipMalloc(reinterpret_cast<void**>(&h->pool), bytes);
    }
    void* va = nullptr;
    hipError_t e = hipMemAddressReserve(&va, bytes, 0, nullptr, 0);
    if (e != hipSuccess) return e;
    hipMemAllocationProp prop = {};
    prop.type = hipMemAllocationTypePinned;
    prop.location.type = hipMemLocationTypeDevice;
    prop.location.id = h->dev;
    hipMemAccessDesc acc = {};
    acc.location = prop.location;
    acc.flags = hipMemAccessFlagsProtReadWrite;
    int mapped = 0;
    for (; mapped < n && e == hipSuccess; ++mapped) {
        char* at = static_cast<char*>(va) + (uint64_t)mapped * slot_bytes;
        e = hipMemCreate(&h->phys[mapped], slot_bytes, &prop, 0);
        if (e != hipSuccess) break;
        e = hipMemMap(at, slot_bytes, 0, h->phys[mapped], 0);
        if (e != hipSuccess) {
            (void)hipMemRelease(h->phys[mapped]);
            break;
        }
        e = hipMemSetAccess(at, slot_bytes, &acc, 1);
        if (e != hipSuccess) {
            (void)hipMemUnmap(at, slot_bytes);
            (void)hipMemRelease(h->phys[mapped]);
            break;
        }
    }
    if (e != hipSuccess) {
        for (int i = 0; i < mapped; ++i) {
            (void)hipMemUnmap(static_cast<char*>(va) + (uint64_t)i * slot_bytes, slot_bytes);
            (void)hipMemRelease(h->phys[i]);
        }
        (void)hipMemAddressFree(va, bytes);
        h->phys.clear();
        return e;
    }
    h->pool = static_cast<uint8_t*>(va);
    h->va_bytes = bytes;
    return hipSuccess;
}

// Return slot s's memory (vmm only); its queued work must have finished.
hipError_t slot_unmap(moe_prefill_t* h, int s)
{
    hipError_t e = hipMemUnmap(h->pool + (uint64_t)s * h->slot_bytes, h->slot_bytes);
    if (e == hipSuccess) e = hipMemRelease(h->phys[s]);
    h->phys[s] = 0;
    h->slot_kind[s] = kSlotReleased;
    return e;
}

void pool_free_memory(moe_prefill_t* h)
{
    if (!h->pool) return;
    if (h->vmm) {
        for (size_t s = 0; s < h->phys.size(); ++s) {
            if (!h->phys[s]) continue;
            (void)hipMemUnmap(h->pool + (uint64_t)s * h->slot_bytes, h->slot_bytes);
            (void)hipMemRelease(h->phys[s]);
        }
        (void)hipMemAddressFree(h->pool, h->va_bytes);
    } else {
        (void)hipFree(h->pool);
    }
    h->phys.clear();
    h->pool = nullptr;
    h->va_bytes = 0;
}

// Wait (bounded) for the work queued on slot s: its last layer's kernels and any copy into it.
int slot_quiesce(moe_prefill_t* h, int s)
{
    if (h->free_set[s]) {
        const int rc = wait_event(h, h->ev_free[s]);
        if (rc != MOE_OK) return rc;
    }
    if (h->ready_set[s]) {
        const int rc = wait_event(h, h->ev_ready[s]);
        if (rc != MOE_OK) return rc;
    }
    return MOE_OK;
}

int count_slots(const moe_prefill_t* h, char kind)
{
    int n = 0;
    for (char k : h->slot_kind) n += k == kind;
    return n;
}

// Shrink the live pool to budget_bytes (memory pressure): residents leave from the end of
// the resident prefix, then prefetch slots, never the last slot (plan_trim).
int pool_trim(moe_prefill_t* h, int64_t budget_bytes, uint64_t* released, int* warn)
{
    const int n_stream = count_slots(h, kSlotStreaming);
    const int64_t budget_slots = budget_bytes > 0 ? budget_bytes / (int64_t)h->slot_bytes : 0;
    const PoolTrim t = plan_trim(h->nl, h->res_live, n_stream, budget_slots, warn);
    for (int i = 0; i < t.evicted; ++i) {
        const int r = h->res_live - 1;                    // layer r lives in slot r
        int rc = slot_quiesce(h, r);
        if (rc != MOE_OK) return rc;
        if (t.converted && i == 0) {
            h->slot_kind[r] = kSlotStreaming;             // keeps layer r, now as a streamed copy
            h->from_prefetch[r] = 0;
        } else {
            h->layer_slot[r] = -1;
            h->slot_layer[r] = -1;
            const hipError_t e = slot_unmap(h, r);
            if (e != hipSuccess) return hip_fail(h, e, "pool trim: release a resident slot");
            *released += h->slot_bytes;
        }
        --h->res_live;
        h->stats.evicted_residents++;
    }
    // prefetch slots: never the active one; empty slots first, then the layer needed last
    for (int n = count_slots(h, kSlotStreaming); n > t.streaming; --n) {
        int best = -1;
        long best_score = -1;
        for (int s = 0; s < h->shape.slots; ++s) {
            if (h->slot_kind[s] != kSlotStreaming || s == h->active) continue;
            const int lay = h->slot_layer[s];
            const int cur = h->active >= 0 && h->slot_layer[h->active] >= 0 ? h->slot_layer[h->active] : 0;
            const long score = lay < 0 ? (1L << 40) : (long)((lay - cur + h->nl) % h->nl);
            if (score > best_score) {
                best_score = score;
                best = s;
            }
        }
        if (best < 0) break;
        int rc = slot_quiesce(h, best);
        if (rc != MOE_OK) return rc;
        if (h->slot_layer[best] >= 0) h->layer_slot[h->slot_layer[best]] = -1;
        h->slot_layer[best] = -1;
        const hipError_t e = slot_unmap(h, best);
        if (e != hipSuccess) return hip_fail(h, e, "pool trim: release a prefetch slot");
        *released += h->slot_bytes;
    }
    const int streaming = count_slots(h, kSlotStreaming);
    h->depth_live = h->res_live < h->nl ? std::min(h->depth_live, streaming - 1) : 0;
    if (h->depth_live < 0) h->depth_live = 0;
    h->stats.released_bytes += *released;
    h->stats.eff_slots = h->res_live + streaming;
    h->stats.eff_depth = h->depth_live;
    h->stats.eff_residents = h->res_live;
    h->stats.warnings |= *warn;
    return MOE_OK;
}

void pool_release(moe_prefill_t* h)
{
    if (!h->pool_on && !h->pool) return;
    (void)wait_stream(h, h->copy);
    for (size_t s = 0; s < h->ev_free.size(); ++s)
        if (h->free_set[s]) (void)wait_event(h, h->ev_free[s]);
    for (hipEvent_t e : h->ev_ready) (void)hipEventDestroy(e);
    for (hipEvent_t e : h->ev_free) (void)hipEventDestroy(e);
    pool_free_memory(h);
    h->pool_on = false;
    h->nl = 0;
    h->blobs.clear();
    h->blobs_dev.clear();
    h->active_only = false;
    h->slot_layer.clear();
    h->layer_slot.clear();
    h->ev_ready.clear();
    h->ev_free.clear();
    h->ready_set.clear();
    h->free_set.clear();
    h->from_prefetch.clear();
    h->slot_kind.clear();
    h->res_live = h->depth_live = 0;
    h->reserve_bytes = 0;
    h->active = -1;
    h->shape = PoolShape();
    h->warnings = 0;
}

}  // namespace

// ======================================================================= ABI

extern "C" {

const char* moe_prefill_last_error(const moe_prefill_t* h)
{
    return h ? h->err.c_str() : g_err.c_str();
}

uint64_t moe_prefill_expert_bytes(int32_t d_model, int32_t d_ff)
{
    if (d_model < 32 || d_model % 32 || d_ff < 32 || d_ff % 32 || d_model > 16384 || d_ff > 16384) return 0;
    return blob_layout(d_model, d_ff).expert_bytes;
}

uint64_t moe_prefill_layer_bytes(int32_t d_model, int32_t d_ff, int32_t n_experts)
{
    if (n_experts < 1) return 0;
    return moe_prefill_expert_bytes(d_model, d_ff) * (uint64_t)n_experts;
}

int moe_prefill_pack_expert(int32_t d_model, int32_t d_ff, const int8_t* wgu_q, const uint16_t* wgu_s,
                            const int8_t* wd_q, const uint16_t* wd_s, void* dst)
{
    if (d_model < 32 || d_model % 32 || d_ff < 32 || d_ff % 32 || d_model > 16384 || d_ff > 16384)
        return fail(nullptr, MOE_EINVAL, "pack: d_model and d_ff must be multiples of 32 in [32, 16384]");
    if (!wgu_q || !wgu_s || !wd_q || !wd_s || !dst) return fail(nullptr, MOE_EINVAL, "pack: null pointer");
    if (!pack_expert(d_model, d_ff, wgu_q, wgu_s, wd_q, wd_s, static_cast<uint8_t*>(dst)))
        return fail(nullptr, MOE_EINVAL, "pack: weight outside [-8, 7]");
    return MOE_OK;
}

int moe_prefill_workspace_size(const moe_prefill_params_t* pin, uint64_t* bytes)
{
    moe_prefill_params_t p;
    std::string why;
    if (!bytes) return fail(nullptr, MOE_EINVAL, "null bytes pointer");
    if (!read_struct(pin, &p, &why)) return fail(nullptr, MOE_EINVAL, why);
    if (!dims_ok(p, &why)) return fail(nullptr, MOE_EINVAL, why);
    *bytes = ws_layout(p.d_model, p.d_ff, p.n_experts, p.top_k, p.max_tokens).total;
    return MOE_OK;
}

int moe_prefill_create(const moe_prefill_params_t* pin, moe_prefill_t** out)
{
    if (!out) return fail(nullptr, MOE_EINVAL, "null out pointer");
    *out = nullptr;
    moe_prefill_params_t p;
    std::string why;
    if (!read_struct(pin, &p, &why)) return fail(nullptr, MOE_EINVAL, why);
    if (!dims_ok(p, &why)) return fail(nullptr, MOE_EINVAL, why);

    int ndev = 0;
    hipError_t e = hipGetDeviceCount(&ndev);
    if (e != hipSuccess || ndev < 1) return fail(nullptr, MOE_EUNSUPPORTED, "no HIP device");
    if (p.device < 0 || p.device >= ndev) return fail(nullptr, MOE_EINVAL, "device ordinal out of range");
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, p.device);
    if (e != hipSuccess) return hip_fail(nullptr, e, "hipGetDeviceProperties");
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(nullptr, MOE_EUNSUPPORTED, std::string("device is ") + prop.gcnArchName + ", not gfx950");

    DevGuard guard(p.device);
    moe_prefill_t* h = new moe_prefill_t();
    h->dev = p.device;
    h->d = p.d_model;
    h->f = p.d_ff;
    h->E = p.n_experts;
    h->k = p.top_k;
    h->Tmax = p.max_tokens;
    h->L = ws_layout(h->d, h->f, h->E, h->k, h->Tmax);
    h->B = blob_layout(h->d, h->f);
    h->stats.struct_size = sizeof(moe_stats_t);

    if (p.workspace) {
        if (p.workspace_bytes < h->L.total) {
            delete h;
            return fail(nullptr, MOE_EINVAL, "lent workspace smaller than moe_prefill_workspace_size()");
        }
        if (reinterpret_cast<uintptr_t>(p.workspace) % 256) {
            delete h;
            return fail(nullptr, MOE_EINVAL, "lent workspace must be 256-byte aligned");
        }
        h->ws = static_cast<uint8_t*>(p.workspace);
    } else {
        e = hipMalloc(reinterpret_cast<void**>(&h->ws), h->L.total);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            delete h;
            return fail(nullptr, MOE_ENOMEM, "workspace allocation failed");
        }
        h->ws_owned = true;
    }
    e = hipStreamCreateWithFlags(&h->copy, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipMemset(h->ws + h->L.mask, 0, (size_t)mask_words(h->E, h->L.W) * 4);
    if (e == hipSuccess) e = hipMemset(h->ws + h->L.load_stats, 0, 16);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        const int rc = hip_fail(nullptr, e, "create");
        if (h->copy) (void)hipStreamDestroy(h->copy);
        if (h->ws_owned) (void)hipFree(h->ws);
        delete h;
        return rc;
    }
    *out = h;
    g_err.clear();
    return MOE_OK;
}

void moe_prefill_destroy(moe_prefill_t* h)
{
    if (!h) return;
    {
        DevGuard guard(h->dev);
        pool_release(h);
        for (auto& set : h->t_pending)
            for (hipEvent_t e : set.ev) (void)hipEventDestroy(e);
        for (auto& set : h->t_free)
            for (hipEvent_t e : set) (void)hipEventDestroy(e);
        if (h->copy) (void)hipStreamDestroy(h->copy);
        if (h->ws_owned && h->ws) (void)hipFree(h->ws);
    }
    delete h;
}

// Whether the combine mode of a layer call is valid (else why not).
static bool combine_ok(const moe_layer_io_t& io, std::string* why)
{
    if (io.combine != MOE_COMBINE_GATHER && io.combine != MOE_COMBINE_ATOMIC) {
        *why = "combine must be MOE_COMBINE_GATHER (0) or MOE_COMBINE_ATOMIC (1)";
        return false;
    }
    if (io.combine == MOE_COMBINE_ATOMIC && io.dm) {
        *why = "dm cannot be exported with MOE_COMBINE_ATOMIC (the down GEMM adds into y, Dm is not stored)";
        return false;
    }
    return true;
}

int moe_prefill_run_layer(moe_prefill_t* h, const moe_layer_io_t* io_in, void* stream)
{
    if (!h) return fail(nullptr, MOE_EINVAL, "null handle");
    moe_layer_io_t io;
    std::string why;
    if (!read_struct(io_in, &io, &why)) return fail(h, MOE_EINVAL, why);
    if (!combine_ok(io, &why)) return fail(h, MOE_EINVAL, why);
    const int T = io.n_tokens;
    if (T < 0 || T > h->Tmax) return fail(h, MOE_EINVAL, "n_tokens out of [0, max_tokens]");
    if (T == 0) return MOE_OK;
    if (!io.x || !io.logits || !io.y) return fail(h, MOE_EINVAL, "x, logits and y are required");
    if ((reinterpret_cast<uintptr_t>(io.x) | reinterpret_cast<uintptr_t>(io.y) |
         reinterpret_cast<uintptr_t>(io.h)) % 16)
        return fail(h, MOE_EINVAL, "x, y and h must be 16-byte aligned");
    hipStream_t st = static_cast<hipStream_t>(stream);
    DevGuard guard(h->dev);

    const uint8_t* blob = nullptr;
    int slot = -1, sparse_slot = -1;
    hipError_t e = hipSuccess;
    if (io.layer < 0) {
        if (!io.weights_dev) return fail(h, MOE_EINVAL, "layer == -1 needs weights_dev");
        blob = static_cast<const uint8_t*>(io.weights_dev);
    } else {
        if (!h->pool_on) return fail(h, MOE_ESTATE, "layer >= 0 but no stream pool is configured");
        if (io.layer >= h->nl) return fail(h, MOE_ESTATE, "layer index beyond the configured stack");
        if (io.layer == 0 && h->reserve_bytes > 0 && h->vmm) {
            // a pass starts: give memory back if the device runs short of the reserve
            size_t fr = 0, tot = 0;
            if (hipMemGetInfo(&fr, &tot) == hipSuccess && (int64_t)fr < h->reserve_bytes) {
                const int64_t live = (int64_t)(h->res_live + count_slots(h, kSlotStreaming)) * (int64_t)h->slot_bytes;
                uint64_t rel = 0;
                int w = 0;
                const int rc = pool_trim(h, live - (h->reserve_bytes - (int64_t)fr), &rel, &w);
                if (rc != MOE_OK) return rc;
                h->stats.pressure_trims++;
                h->warnings |= w;
                log_msg(h, MOE_LOG_WARN, "device memory below the reserve: the pool released " +
                        std::to_string(rel) + " bytes, " + std::to_string(h->res_live) + " residents left");
                log_warnings(h, w, "memory pressure");
            }
            (void)hipGetLastError();
        }
        slot = h->layer_slot[io.layer];
        if (slot >= 0) {
            if (h->slot_kind[slot] == kSlotStreaming && h->ready_set[slot])
                e = hipStreamWaitEvent(st, h->ev_ready[slot], 0);
            if (h->from_prefetch[slot]) {
                h->stats.prefetch_activated++;
                h->from_prefetch[slot] = 0;
            }
        } else if (h->active_only) {
            // active-expert load: the kernels of this layer fill the slot after routing
            slot = pick_victim(h, io.layer, -1);
            if (slot < 0) return fail(h, MOE_ESTATE, "no pool slot available");
            const int old = h->slot_layer[slot];
            if (old >= 0) h->layer_slot[old] = -1;
            h->slot_layer[slot] = -1;                     // a partial layer: never reused as whole
            if (h->free_set[slot]) e = hipStreamWaitEvent(st, h->ev_free[slot], 0);
            if (e == hipSuccess && h->poison)   // debug: the experts that are not loaded hold NaN bytes
                e = launch_fill_u32(reinterpret_cast<uint32_t*>(h->pool + (uint64_t)slot * h->slot_bytes),
                                    (int64_t)(h->slot_bytes / 4), 0xFFFFFFFFu, st);
            sparse_slot = slot;
            h->stats.sparse_loads++;
        } else {
            // load-then-compute: a stream-ordered copy into a free slot first
            slot = pick_victim(h, io.layer, -1);
            if (slot < 0) return fail(h, MOE_ESTATE, "no pool slot available");
            e = enqueue_copy(h, slot, io.layer);
            if (e == hipSuccess) e = hipStreamWaitEvent(st, h->ev_ready[slot], 0);
            h->stats.sync_loads++;
            log_msg(h, MOE_LOG_INFO, "layer " + std::to_string(io.layer) + ": not prefetched, loaded before compute");
        }
        if (e != hipSuccess) return hip_fail(h, e, "pool acquire");
        blob = h->pool + (uint64_t)slot * h->slot_bytes;
    }

    if (h->mask_dirty) {   // a launch failed part-way: restore the grouping state first
        e = launch_fill_u32(reinterpret_cast<uint32_t*>(h->ws + h->L.mask), (int64_t)mask_words(h->E, h->L.W), 0u, st);
        if (e != hipSuccess) return hip_fail(h, e, "grouping state reset");
        h->mask_dirty = false;
    }

    LayerLaunch LL;
    LL.T = T;
    LL.d = h->d;
    LL.f = h->f;
    LL.E = h->E;
    LL.k = h->k;
    LL.x = io.x;
    LL.logits = io.logits;
    LL.y = io.y;
    LL.blob = blob;
    LL.load_src = sparse_slot >= 0 ? h->blobs_dev[io.layer] : nullptr;
    LL.load_dst = sparse_slot >= 0 ? h->pool + (uint64_t)sparse_slot * h->slot_bytes : nullptr;
    bind_layer(LL, h->ws, h->L, h->B);
    LL.h_out = io.h;
    LL.gu = io.gu;
    LL.combine_atomic = io.combine == MOE_COMBINE_ATOMIC;
    LL.marks = nullptr;
    std::array<hipEvent_t, kNumKernels + 1> tset{};
    if (h->timing) {
        if (!h->t_free.empty()) {
            tset = h->t_free.back();
            h->t_free.pop_back();
        } else {
            for (auto& ev : tset) {
                e = hipEventCreate(&ev);
                if (e != hipSuccess) return hip_fail(h, e, "timing events");
            }
        }
        LL.marks = tset.data();
    }

    e = launch_layer(LL, st);
    if (e != hipSuccess) {
        h->mask_dirty = true;
        return hip_fail(h, e, "layer launch");
    }
    if (slot >= 0) {
        e = hipEventRecord(h->ev_free[slot], st);   // the down GEMM was the last reader
        if (e != hipSuccess) {
            h->mask_dirty = true;
            return hip_fail(h, e, "hipEventRecord");
        }
        h->free_set[slot] = 1;
        h->active = slot;
    }
    e = launch_combine(LL, st);
    if (e != hipSuccess) {
        h->mask_dirty = true;
        return hip_fail(h, e, "combine launch");
    }
    if (h->timing) {
        moe_prefill::TimedLayer tl;
        tl.ev = tset;
        tl.launched = ((1u << kNumKernels) - 1) & ~(sparse_slot >= 0 ? 0u : 1u << kExpertLoad);
        h->t_pending.push_back(tl);
    }

    e = export_copies(io, h->ws, h->L, T, h->d, h->f, h->E, h->k, st);
    if (e != hipSuccess) return hip_fail(h, e, "export copy");
    h->stats.layers_run++;

    // lookahead: queue the next streamed layers behind this one
    if (io.layer >= 0) {
        for (int y : window_after(h, io.layer)) {
            if (h->layer_slot[y] >= 0) continue;
            const int v = pick_victim(h, io.layer, h->active);
            if (v < 0) break;
            h->prefetch_counter++;
            if (h->fail_at && h->prefetch_counter == h->fail_at) {
                h->stats.prefetch_failed++;   // forced failure: this layer will load synchronously
                log_msg(h, MOE_LOG_WARN, "prefetch of layer " + std::to_string(y) + " failed (test hook): it will load synchronously");
                continue;
            }
            e = enqueue_copy(h, v, y);
            if (e != hipSuccess) {
                (void)hipGetLastError();
                h->stats.prefetch_failed++;
                log_msg(h, MOE_LOG_WARN, "prefetch of layer " + std::to_string(y) + " failed: it will load synchronously");
                continue;
            }
            h->from_prefetch[v] = 1;
            h->stats.prefetch_queued++;
        }
    }
    h->err.clear();
    return MOE_OK;
}

int moe_prefill_run_layer_noalloc(const moe_prefill_params_t* pin, const moe_layer_io_t* io_in, void* stream)
{
    moe_prefill_params_t p;
    moe_layer_io_t io;
    std::string why;
    if (!read_struct(pin, &p, &why)) return fail(nullptr, MOE_EINVAL, why);
    if (!read_struct(io_in, &io, &why)) return fail(nullptr, MOE_EINVAL, why);
    if (!combine_ok(io, &why)) return fail(nullptr, MOE_EINVAL, why);
    const int T = io.n_tokens;
    if (T < 0) return fail(nullptr, MOE_EINVAL, "noalloc: n_tokens < 0");
    p.max_tokens = T > 0 ? T : 1;                     // the workspace is laid out for this T
    if (!dims_ok(p, &why)) return fail(nullptr, MOE_EINVAL, why);
    if (p.workspace) return fail(nullptr, MOE_EINVAL, "noalloc: workspace must be NULL (the static scratch is the workspace)");
    if (T == 0) return MOE_OK;
    if (io.layer != -1 || !io.weights_dev)
        return fail(nullptr, MOE_EINVAL, "noalloc: resident weights only (layer = -1 and weights_dev)");
    if (!io.x || !io.logits || !io.y) return fail(nullptr, MOE_EINVAL, "x, logits and y are required");
    if ((reinterpret_cast<uintptr_t>(io.x) | reinterpret_cast<uintptr_t>(io.y) |
         reinterpret_cast<uintptr_t>(io.h)) % 16)
        return fail(nullptr, MOE_EINVAL, "x, y and h must be 16-byte aligned");
    const WsLayout L = ws_layout(p.d_model, p.d_ff, p.n_experts, p.top_k, T);
    if (L.total > kScratchBytes)
        return fail(nullptr, MOE_EINVAL, "noalloc: this layer needs " + std::to_string(L.total) +
                    " bytes of workspace, more than the static scratch of " + std::to_string(kScratchBytes) +
                    " bytes; use moe_prefill_run_layer");
    const int rc = noalloc_device_ok(p.device);
    if (rc != MOE_OK) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    DevGuard guard(p.device);
    uint8_t* ws = nullptr;
    hipError_t e = scratch_device_ptr(p.device, &ws);
    if (e != hipSuccess) return hip_fail(nullptr, e, "noalloc: static scratch address");
    // The membership mask and the scale flags must start at zero.  Their place in the
    // scratch depends on the dimensions and an earlier call may have left other data
    // there, so every call clears them (a kernel, not a memset: safe to capture).
    e = launch_fill_u32(reinterpret_cast<uint32_t*>(ws + L.mask), (int64_t)mask_words(p.n_experts, L.W), 0u, st);
    if (e != hipSuccess) return hip_fail(nullptr, e, "noalloc: grouping state reset");
    const BlobLayout B = blob_layout(p.d_model, p.d_ff);
    LayerLaunch LL;
    LL.T = T;
    LL.d = p.d_model;
    LL.f = p.d_ff;
    LL.E = p.n_experts;
    LL.k = p.top_k;
    LL.x = io.x;
    LL.logits = io.logits;
    LL.y = io.y;
    LL.blob = static_cast<const uint8_t*>(io.weights_dev);
    LL.load_src = nullptr;
    LL.load_dst = nullptr;
    bind_layer(LL, ws, L, B);
    LL.h_out = io.h;
    LL.gu = io.gu;
    LL.combine_atomic = io.combine == MOE_COMBINE_ATOMIC;
    LL.marks = nullptr;
    e = launch_layer(LL, st);
    if (e == hipSuccess) e = launch_combine(LL, st);
    if (e != hipSuccess) return hip_fail(nullptr, e, "noalloc: layer launch");
    e = export_copies(io, ws, L, T, p.d_model, p.d_ff, p.n_experts, p.top_k, st);
    if (e != hipSuccess) return hip_fail(nullptr, e, "noalloc: export copy");
    g_err.clear();
    return MOE_OK;
}

int moe_prefill_plan_pool(moe_pool_plan_t* inout)
{
    moe_pool_plan_t p;
    std::string why;
    if (!read_struct(inout, &p, &why)) return fail(nullptr, MOE_EINVAL, why);
    if (p.n_layers < 0 || p.prefetch_depth < 0 || p.resident_layers < -1)
        return fail(nullptr, MOE_EINVAL, "plan: bad request");
    p.slots = p.depth = p.residents = p.warnings = 0;
    if (p.n_layers == 0) {
        write_struct(inout, p);
        return MOE_OK;
    }
    if (p.slot_bytes == 0) return fail(nullptr, MOE_EINVAL, "plan: slot_bytes == 0");
    int warn = 0;
    PoolShape s = plan_initial(p.n_layers, p.slot_bytes, p.prefetch_depth, p.resident_layers,
                               p.max_vram_bytes, p.requested_slots, &warn);
    for (;;) {
        const bool fits = p.max_alloc_slots == 0 || (p.max_alloc_slots > 0 && s.slots <= p.max_alloc_slots);
        if (fits) break;
        if (s.slots <= 1) {
            p.warnings = warn;
            write_struct(inout, p);
            return fail(nullptr, MOE_ENOMEM, "plan: one slot does not fit");
        }
        s = plan_degrade(s, p.n_layers, p.prefetch_depth, p.resident_layers, &warn);
    }
    p.slots = s.slots;
    p.depth = s.depth;
    p.residents = s.residents;
    p.warnings = warn;
    write_struct(inout, p);
    return MOE_OK;
}

int moe_prefill_plan_trim(moe_pool_trim_t* inout)
{
    moe_pool_trim_t p;
    std::string why;
    if (!read_struct(inout, &p, &why)) return fail(nullptr, MOE_EINVAL, why);
    if (p.n_layers < 1 || p.residents < 0 || p.streaming < 0 || p.residents > p.n_layers ||
        p.residents + p.streaming < 1 || (p.residents < p.n_layers && p.streaming < 1))
        return fail(nullptr, MOE_EINVAL, "plan trim: not a pool the planner makes");
    int warn = 0;
    const PoolTrim t = plan_trim(p.n_layers, p.residents, p.streaming, p.budget_slots, &warn);
    p.new_residents = t.residents;
    p.new_streaming = t.streaming;
    p.evicted = t.evicted;
    p.converted = t.converted;
    p.released = t.released;
    p.warnings = warn;
    write_struct(inout, p);
    return MOE_OK;
}

int stream_pool_configure(moe_prefill_t* h, stream_pool_params_t* inout)
{
    if (!h) return fail(nullptr, MOE_EINVAL, "null handle");
    stream_pool_params_t p;
    std::string why;
    if (!read_struct(inout, &p, &why)) return fail(h, MOE_EINVAL, why);
    DevGuard guard(h->dev);

    // a new plan first releases stale prefetches and residents
    int rc = wait_stream(h, h->copy);
    if (rc != MOE_OK) return rc;
    pool_release(h);
    p.eff_slots = p.eff_depth = p.eff_residents = p.warnings = 0;
    h->stats.eff_slots = h->stats.eff_depth = h->stats.eff_residents = h->stats.warnings = 0;
    if (p.n_layers == 0) {
        write_struct(inout, p);
        return MOE_OK;
    }
    if (p.n_layers < 0 || !p.host_blobs) return fail(h, MOE_EINVAL, "pool: need n_layers > 0 and host_blobs");
    if (p.prefetch_depth < 0 || p.resident_layers < -1) return fail(h, MOE_EINVAL, "pool: bad depth or resident count");
    const uint64_t want = blob_layout(h->d, h->f).expert_bytes * (uint64_t)h->E;
    if (p.layer_bytes != want) return fail(h, MOE_EINVAL, "pool: layer_bytes != moe_prefill_layer_bytes()");
    for (int i = 0; i < p.n_layers; ++i)
        if (!p.host_blobs[i]) return fail(h, MOE_EINVAL, "pool: null host blob");

    // active_only: the kernel reads the host blobs itself, so they must be page-locked host memory
    // mapped for the device; its device address is taken from the runtime
    std::vector<const uint8_t*> blobs_dev;
    if (p.active_only) {
        for (int i = 0; i < p.n_layers; ++i) {
            hipPointerAttribute_t at{};
            const hipError_t e = hipPointerGetAttributes(&at, p.host_blobs[i]);
            if (e != hipSuccess || at.type != hipMemoryTypeHost || !at.devicePointer) {
                (void)hipGetLastError();
                return fail(h, MOE_EINVAL, "pool: active_only needs pinned host blobs mapped for the device");
            }
            const uint8_t* dp = static_cast<const uint8_t*>(at.devicePointer);
            if (reinterpret_cast<uintptr_t>(dp) % 16)
                return fail(h, MOE_EINVAL, "pool: active_only needs 16-byte aligned host blobs");
            blobs_dev.push_back(dp);
        }
    }
    int vmm = 0;
    if (hipDeviceGetAttribute(&vmm, hipDeviceAttributeVirtualMemoryManagementSupported, h->dev) != hipSuccess) {
        (void)hipGetLastError();
        vmm = 0;
    }
    h->vmm = vmm != 0;
    uint64_t align = 1 << 16;
    if (h->vmm) {
        hipMemAllocationProp prop = {};
        prop.type = hipMemAllocationTypePinned;
        prop.location.type = hipMemLocationTypeDevice;
        prop.location.id = h->dev;
        size_t gran = 0;
        if (hipMemGetAllocationGranularity(&gran, &prop, hipMemAllocationGranularityRecommended) == hipSuccess &&
            gran > align)
            align = gran;
        (void)hipGetLastError();
    }
    const uint64_t slot_bytes = align_up(p.layer_bytes, align);
    int warn = 0;
    const int want_depth = p.active_only ? 0 : p.prefetch_depth;   // routing decides the copy: no lookahead
    PoolShape s = plan_initial(p.n_layers, slot_bytes, want_depth, p.resident_layers,
                               p.max_vram_bytes, p.requested_slots, &warn);
    const char* cap_env = getenv("MOE_TEST_POOL_MAX_SLOTS");
    const int cap = cap_env ? atoi(cap_env) : 0;
    const bool fail_all = getenv("MOE_TEST_POOL_FAIL_ALL") && atoi(getenv("MOE_TEST_POOL_FAIL_ALL"));
    for (;;) {
        bool ok = !fail_all && !(cap > 0 && s.slots > cap);
        if (ok) {
            const hipError_t e = pool_alloc(h, s.slots, slot_bytes);
            if (e != hipSuccess) {
                (void)hipGetLastError();
                h->pool = nullptr;
                ok = false;
            }
        }
        if (ok) break;
        if (s.slots <= 1) {
            p.warnings = warn;
            write_struct(inout, p);
            return fail(h, MOE_ENOMEM, "pool: the mandatory one-slot pool could not be allocated");
        }
        s = plan_degrade(s, p.n_layers, want_depth, p.resident_layers, &warn);
    }

    h->pool_on = true;
    h->nl = p.n_layers;
    h->blobs.assign(p.host_blobs, p.host_blobs + p.n_layers);
    h->active_only = p.active_only != 0;
    h->blobs_dev = blobs_dev;
    h->layer_bytes = p.layer_bytes;
    h->slot_bytes = slot_bytes;
    h->shape = s;
    h->warnings = warn;
    h->slot_layer.assign(s.slots, -1);
    h->layer_slot.assign(p.n_layers, -1);
    h->ev_ready.assign(s.slots, nullptr);
    h->ev_free.assign(s.slots, nullptr);
    h->ready_set.assign(s.slots, 0);
    h->free_set.assign(s.slots, 0);
    h->from_prefetch.assign(s.slots, 0);
    h->slot_kind.assign(s.slots, kSlotStreaming);
    for (int i = 0; i < s.residents; ++i) h->slot_kind[i] = kSlotResident;
    h->res_live = s.residents;
    h->depth_live = s.depth;
    h->reserve_bytes = p.reserve_bytes > 0 ? p.reserve_bytes : 0;
    h->poison = getenv("MOE_DEBUG_POISON") && atoi(getenv("MOE_DEBUG_POISON"));
    h->active = -1;
    h->prefetch_counter = 0;
    const char* fa = getenv("MOE_TEST_PREFETCH_FAIL");
    h->fail_at = fa ? (uint64_t)atoll(fa) : 0;
    for (int i = 0; i < s.slots; ++i) {
        hipError_t e = hipEventCreateWithFlags(&h->ev_ready[i], hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&h->ev_free[i], hipEventDisableTiming);
        if (e != hipSuccess) {
            const int r = hip_fail(h, e, "pool events");
            pool_release(h);
            return r;
        }
    }
    // resident leading layers are uploaded now
    for (int i = 0; i < s.residents; ++i) {
        const hipError_t e = hipMemcpyAsync(h->pool + (uint64_t)i * slot_bytes, h->blobs[i], h->layer_bytes,
                                            hipMemcpyHostToDevice, h->copy);
        if (e != hipSuccess) {
            const int r = hip_fail(h, e, "resident upload");
            pool_release(h);
            return r;
        }
        h->slot_layer[i] = i;
        h->layer_slot[i] = i;
        h->stats.bytes_h2d += h->layer_bytes;
    }
    rc = wait_stream(h, h->copy);
    if (rc != MOE_OK) {
        pool_release(h);
        return rc;
    }
    p.eff_slots = s.slots;
    p.eff_depth = s.depth;
    p.eff_residents = s.residents;
    p.warnings = warn;
    h->stats.eff_slots = s.slots;
    h->stats.eff_depth = s.depth;
    h->stats.eff_residents = s.residents;
    h->stats.warnings = warn;
    write_struct(inout, p);
    log_warnings(h, warn, "pool");
    log_msg(h, MOE_LOG_INFO, "pool: " + std::to_string(s.slots) + " slots of " + std::to_string(slot_bytes) +
            " bytes, depth " + std::to_string(s.depth) + ", " + std::to_string(s.residents) + " residents" +
            (h->vmm ? " (one physical allocation per slot)" : " (one allocation)"));
    h->err.clear();
    return MOE_OK;
}

int stream_pool_set_budget(moe_prefill_t* h, stream_pool_budget_t* inout)
{
    if (!h) return fail(nullptr, MOE_EINVAL, "null handle");
    stream_pool_budget_t p;
    std::string why;
    if (!read_struct(inout, &p, &why)) return fail(h, MOE_EINVAL, why);
    if (!h->pool_on) return fail(h, MOE_ESTATE, "pool budget: no stream pool is configured");
    if (p.max_vram_bytes <= 0) return fail(h, MOE_EINVAL, "pool budget: max_vram_bytes must be > 0");
    if (!h->vmm)
        return fail(h, MOE_EUNSUPPORTED, "pool budget: the device has no virtual memory management, "
                                         "so the pool is one allocation; reconfigure it instead");
    DevGuard guard(h->dev);
    uint64_t rel = 0;
    int w = 0;
    const int rc = pool_trim(h, p.max_vram_bytes, &rel, &w);
    h->warnings |= w;
    log_warnings(h, w, "pool budget");
    if (rel) log_msg(h, MOE_LOG_INFO, "pool budget: released " + std::to_string(rel) + " bytes, " +
                     std::to_string(h->res_live) + " residents left");
    p.eff_slots = h->res_live + count_slots(h, kSlotStreaming);
    p.eff_depth = h->depth_live;
    p.eff_residents = h->res_live;
    p.warnings = w;
    p.released_bytes = rel;
    write_struct(inout, p);
    if (rc != MOE_OK) return rc;
    h->err.clear();
    return MOE_OK;
}

int moe_prefill_set_log(moe_prefill_t* h, moe_log_fn fn, void* user, int32_t level)
{
    if (!h) return fail(nullptr, MOE_EINVAL, "null handle");
    h->log_fn = fn;
    h->log_user = user;
    h->log_level = level;
    return MOE_OK;
}

int moe_prefill_set_timing(moe_prefill_t* h, int32_t enable)
{
    if (!h) return fail(nullptr, MOE_EINVAL, "null handle");
    h->timing = enable != 0;
    return MOE_OK;
}

const char* moe_prefill_kernel_name(int32_t id)
{
    static_assert(kNumKernels == MOE_N_KERNELS, "kernel ids of the header and the launcher agree");
    static const char* names[kNumKernels] = {"route_quant", "group", "expert_load", "row_scatter",
                                             "gemm_gate_up", "gemm_down", "combine"};
    return (id >= 0 && id < kNumKernels) ? names[id] : "";
}

int moe_prefill_kernel_times(moe_prefill_t* h, moe_kernel_times_t* inout, int32_t reset)
{
    if (!h) return fail(nullptr, MOE_EINVAL, "null handle");
    moe_kernel_times_t out;
    std::string why;
    if (!read_struct(inout, &out, &why)) return fail(h, MOE_EINVAL, why);
    DevGuard guard(h->dev);
    for (auto& set : h->t_pending) {
        const int rc = wait_event(h, set.ev[kNumKernels]);
        if (rc != MOE_OK) return rc;
        for (int i = 0; i < kNumKernels; ++i) {
            if (!(set.launched >> i & 1u)) continue;      // not launched in that layer
            float ms = 0.0f;
            if (hipEventElapsedTime(&ms, set.ev[i], set.ev[i + 1]) == hipSuccess) {
                h->t_ms[i] += ms;
                h->t_launches[i]++;
            }
        }
        h->t_free.push_back(set.ev);
    }
    h->t_pending.clear();
    out.n_kernels = kNumKernels;
    for (int i = 0; i < kNumKernels; ++i) {
        out.launches[i] = h->t_launches[i];
        out.total_ms[i] = h->t_ms[i];
        if (reset) {
            h->t_launches[i] = 0;
            h->t_ms[i] = 0.0;
        }
    }
    write_struct(inout, out);
    return MOE_OK;
}

int moe_prefill_exp_host(uint32_t first_bits, uint64_t n, float* out)
{
    if (n > 0 && !out) return fail(nullptr, MOE_EINVAL, "exp_host: null output");
    if ((uint64_t)first_bits + n > (1ull << 32)) return fail(nullptr, MOE_EINVAL, "exp_host: range beyond 2^32 patterns");
    exp_range_host(first_bits, n, out);
    return MOE_OK;
}

int moe_prefill_exp_device(uint32_t first_bits, uint64_t n, float* out, void* stream)
{
    if (n > 0 && !out) return fail(nullptr, MOE_EINVAL, "exp_device: null output");
    if ((uint64_t)first_bits + n > (1ull << 32)) return fail(nullptr, MOE_EINVAL, "exp_device: range beyond 2^32 patterns");
    const hipError_t e = launch_exp_range(first_bits, n, out, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(nullptr, e, "exp_device launch");
    return MOE_OK;
}

int moe_prefill_get_stats(const moe_prefill_t* h, moe_stats_t* inout)
{
    if (!h) return fail(nullptr, MOE_EINVAL, "null handle");
    moe_stats_t tmp;
    std::string why;
    if (!read_struct(inout, &tmp, &why)) return fail(nullptr, MOE_EINVAL, why);
    moe_stats_t out = h->stats;
    if (out.sparse_loads) {   // the device-side counters of the active-expert loads
        unsigned long long c[2] = {0, 0};
        DevGuard guard(h->dev);
        hipError_t e = hipDeviceSynchronize();
        if (e == hipSuccess) e = hipMemcpy(c, h->ws + h->L.load_stats, sizeof(c), hipMemcpyDeviceToHost);
        if (e != hipSuccess) return hip_fail(const_cast<moe_prefill_t*>(h), e, "stats read");
        out.experts_loaded = c[0];
        out.bytes_sparse = c[1];
    }
    write_struct(inout, out);
    return MOE_OK;
}

}  // extern "C"
