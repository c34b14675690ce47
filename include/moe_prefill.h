/*
 * moe_prefill.h -- C ABI of the MI355X (gfx950) MoE prompt (prefill) FFN layer.
 *
 * One call runs one mixture-of-experts FFN layer over a one-chunk prompt, the
 * prompt path described on the page "prefill: a layer split's idle card streams
 * a share of a one-chunk prompt's experts" (Strata #663, section "What"):
 * activations are quantised (Xq), tokens are routed top-k and grouped into a
 * row table with per-expert group bounds, a grouped Q4 x Q8 GEMM produces the
 * gate/up projection (GU), SwiGLU gives H, H is requantised (Hq), a second
 * grouped GEMM gives the down projection (Dm), and the expert rows are
 * combined back into token rows with the router weights.  Expert weights can
 * be streamed from pinned host memory into a fixed-slot device pool with
 * lookahead prefetch, as on the pages "feat: prefetch streamed layers during
 * compute" (stable-diffusion.cpp #1905, "Summary" and "Effective behavior")
 * and "feat: pool VRAM for streamed layer" (stable-diffusion.cpp #1906,
 * "Summary" and the pool-behaviour table).
 *
 * Conventions (all entry points):
 *  - Return 0 (MOE_OK) on success, a negative MOE_E* code otherwise; the
 *    message of the last failure on a handle is moe_prefill_last_error(h)
 *    (moe_prefill_last_error(NULL) for failures before a handle exists).
 *  - Versioned structs (pages #1905/#1906: controls exposed through a versioned
 *    params struct and additive constructors, existing layouts preserved).
 *    Every struct starts with uint32_t struct_size = sizeof() as the caller
 *    compiled it.  A smaller size is accepted: missing trailing fields take
 *    their defaults (0).  A larger size is accepted only if every byte past
 *    the fields this library knows is zero; otherwise MOE_EINVAL.
 *  - Pointers called "device" are HIP device memory on the handle's device
 *    (e.g. from torch.empty(..., device="cuda")); "host" pointers are ordinary
 *    CPU memory, "pinned" ones page-locked host memory (hipHostMalloc, or
 *    torch.empty(..., pin_memory=True)).  The caller owns every buffer it
 *    passes; the library never frees caller memory.
 *  - `stream` arguments are a hipStream_t passed as void* (NULL = the null
 *    stream).  Work is enqueued on it and the call returns before completion;
 *    moe_prefill_run_layer and the pool calls never call hipDeviceSynchronize
 *    (create does, once; moe_prefill_get_stats does when it reads device-side
 *    counters).
 *  - A handle is not thread-safe; separate handles are independent.
 *  - Degradations (smaller pool, shallower prefetch, one slot above the
 *    budget, synchronous fallback) are warnings: the call succeeds and the
 *    effective values are reported back.  A mandatory resource that cannot be
 *    had (workspace, the one pool slot) fails clearly with MOE_ENOMEM; there
 *    is no hidden fallback (page #1906, pool-behaviour table).
 */
#ifndef MOE_PREFILL_H
#define MOE_PREFILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_PREFILL_ABI_VERSION 1

enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,        /* bad argument, dimension or struct */
    MOE_ENOMEM = -2,        /* workspace or the mandatory pool slot not allocatable */
    MOE_EHIP = -3,          /* a HIP runtime call failed */
    MOE_EUNSUPPORTED = -4,  /* device is not gfx950, or lacks a feature the call needs */
    MOE_ESTATE = -5,        /* call not valid in the handle's state (e.g. layer >= 0 before a pool) */
    MOE_ETIMEOUT = -6       /* a bounded host wait expired */
};

typedef struct moe_prefill moe_prefill_t;

/* ------------------------------------------------------------- creation --- */

typedef struct moe_prefill_params {
    uint32_t struct_size;
    int32_t d_model;          /* d: multiple of 32 (one Q8/Q4 block), 32..16384 */
    int32_t d_ff;             /* f, per expert: multiple of 32, 32..16384 */
    int32_t n_experts;        /* E: 1..1024 */
    int32_t top_k;            /* k: 1..E */
    int32_t max_tokens;       /* largest T any run will use: >= 1, max_tokens*top_k <= 2^21 */
    int32_t device;           /* HIP device ordinal */
    int32_t reserved0;
    void* workspace;          /* NULL: the library allocates; else a caller-lent
                                 device buffer of >= moe_prefill_workspace_size()
                                 bytes, 256-byte aligned, owned by the caller and
                                 valid until moe_prefill_destroy (the page #663
                                 "What" lends every stage's prompt buffers the
                                 same way) */
    uint64_t workspace_bytes; /* size of `workspace` when lent */
} moe_prefill_params_t;

/* Device bytes of the per-handle workspace (routing tables, Xq, GU, Hq, Dm,
 * ...) for these dimensions.  Host only.  MOE_EINVAL on bad dimensions. */
int moe_prefill_workspace_size(const moe_prefill_params_t* p, uint64_t* bytes);

/* Checks the dimensions and the device (gfx950, else MOE_EUNSUPPORTED),
 * allocates or adopts the workspace, creates the copy stream and events.
 * The handle holds every buffer one layer of the prompt path needs (page #663,
 * "What": the stages' prompt buffers, the row table and the group bounds); the
 * workspace is the one mandatory resource, so a failed allocation is MOE_ENOMEM
 * with no fallback (page #1906, pool-behaviour table: mandatory execution
 * memory fails clearly).  On failure *out is NULL. */
int moe_prefill_create(const moe_prefill_params_t* p, moe_prefill_t** out);

/* Waits for the handle's copy stream, then releases the pool, events, streams
 * and a library-owned workspace, so no queued copy writes into freed memory
 * (page #1906, "Verification": lifecycle cleanup of the pool is among the
 * validated behaviours).  NULL is a no-op. */
void moe_prefill_destroy(moe_prefill_t* h);

/* Message of the last failure on h (h may be NULL: the last failure of a call
 * that had no handle, per thread).  Never NULL; "" after success.  Failures are
 * reported clearly rather than hidden behind a fallback (page #1906,
 * pool-behaviour table). */
const char* moe_prefill_last_error(const moe_prefill_t* h);

/* ---------------------------------------------------------- weight blob --- */
/*
 * A layer's weights are one blob: E experts back to back, each
 * moe_prefill_expert_bytes() long.  Inside an expert: the gate/up matrix
 * W_gu [2f, d] and the down matrix W_d [d, f], each as Q4 blocks of 32 along
 * its input dimension (4-bit integers in [-8, 7], one fp16 scale per block),
 * in a tiled order matched to the GEMM kernel (see moe_prefill_pack_expert).
 * Host and device layouts are the same, so filling a pool slot is one copy.
 */
uint64_t moe_prefill_expert_bytes(int32_t d_model, int32_t d_ff);
uint64_t moe_prefill_layer_bytes(int32_t d_model, int32_t d_ff, int32_t n_experts);

/* Packs one expert from its canonical arrays into `dst` (host memory,
 * moe_prefill_expert_bytes() bytes):
 *   wgu_q [2f][d]    int8 in [-8, 7]; rows [0, f) gate, rows [f, 2f) up
 *   wgu_s [2f][d/32] fp16 bits, scale of each block of 32 along d
 *   wd_q  [d][f]     int8 in [-8, 7]
 *   wd_s  [d][f/32]  fp16 bits
 * MOE_EINVAL on a bad dimension or a weight outside [-8, 7]. */
int moe_prefill_pack_expert(int32_t d_model, int32_t d_ff, const int8_t* wgu_q,
                            const uint16_t* wgu_s, const int8_t* wd_q, const uint16_t* wd_s,
                            void* dst);

/* ------------------------------------------------------------ one layer --- */

typedef struct moe_layer_io {
    uint32_t struct_size;
    int32_t layer;             /* >= 0: weights come from the stream pool (layer
                                  index of stream_pool_configure); -1: from
                                  weights_dev */
    const void* weights_dev;   /* device: a resident layer blob of
                                  moe_prefill_layer_bytes() bytes (layer == -1) */
    int32_t n_tokens;          /* T: 0..max_tokens (0 is a no-op) */
    int32_t reserved0;
    const float* x;            /* device [T, d] fp32 activations, 16-byte aligned */
    const float* logits;       /* device [T, E] fp32 router logits, finite */
    float* y;                  /* device [T, d] fp32 output, overwritten, 16-byte aligned */
    /* Optional device exports of the intermediate buffers (NULL = skip).
       Row index r is the position in the row table, grouped by expert. */
    int32_t* eidx;             /* [T, k]  expert of slot j of token t */
    float* weights;            /* [T, k]  router weight of that slot */
    int32_t* counts;           /* [E]     rows routed to each expert */
    int32_t* bounds;           /* [E+1]   group bounds, bounds[E] = T*k */
    int32_t* rows;             /* [T*k]   row table: row r holds pair p = t*k + j */
    int32_t* pos;              /* [T*k]   inverse: pos[p] = r */
    int8_t* xq;                /* [T, d]  Q8 codes of x */
    float* dx;                 /* [T, d/32] Q8 scales of x */
    float* gu;                 /* [T*k, 2f] gate | up */
    float* h;                  /* [T*k, f]  SwiGLU output (16-byte aligned) */
    int8_t* hq;                /* [T*k, f]  Q8 codes of h */
    float* dh;                 /* [T*k, f/32] Q8 scales of h */
    float* dm;                 /* [T*k, d]  down projection per row */
    /* Fields added after the first layout (a caller built against that layout
       passes its smaller struct_size and gets the defaults): */
    int32_t combine;           /* how the expert rows become token rows (the
                                  combine step, page #663 "What"):
                                  MOE_COMBINE_GATHER (0, default): the down GEMM
                                  writes Dm and a gather kernel sums each token's
                                  k rows in slot order -- deterministic, the
                                  same bits on every run;
                                  MOE_COMBINE_ATOMIC (1): the down GEMM's epilogue
                                  adds w * Dm straight into y with fp32 atomic
                                  adds (y is zeroed first), so Dm never goes
                                  through device memory.  The order of the adds
                                  changes from run to run, so y agrees with the
                                  gather only to rounding (page #663 "Output":
                                  another grouping rounds differently; such a
                                  variant is opt-in).  dm cannot be exported in
                                  this mode (MOE_EINVAL). */
    int32_t reserved1;         /* 0 */
} moe_layer_io_t;

enum { MOE_COMBINE_GATHER = 0, MOE_COMBINE_ATOMIC = 1 };

/*
 * Runs one MoE prefill FFN layer on `stream` (see the file comment for the
 * steps).  For layer >= 0 the weights are taken from the pool: a resident
 * slot, a prefetched slot (the stream waits for its copy), or -- when the
 * layer is not in the pool -- a stream-ordered load into a free slot first
 * (load-then-compute, page #1905 "Summary").  After enqueueing the layer it
 * queues prefetches of the next prefetch-depth streamed layers on the copy
 * stream; a prefetch never overwrites the active slot.
 * Errors: MOE_EINVAL (bad T or pointers, an unknown combine mode, dm with
 * MOE_COMBINE_ATOMIC), MOE_ESTATE (layer >= 0 with no pool, or layer out of
 * range), MOE_EHIP.
 */
int moe_prefill_run_layer(moe_prefill_t* h, const moe_layer_io_t* io, void* stream);

/*
 * Allocation-free variant of moe_prefill_run_layer, for callers that cannot
 * allocate device memory: code running under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It needs no handle and calls no
 * hipMalloc, hipFree or allocating library routine.
 *
 *  - p: the dimensions (d_model, d_ff, n_experts, top_k, device) with the same
 *    limits as moe_prefill_create; max_tokens is ignored (the workspace is laid
 *    out for io->n_tokens) and workspace must be NULL.
 *  - io: as for moe_prefill_run_layer, resident weights only (layer == -1,
 *    weights_dev set); the optional exports and the combine modes work as
 *    there.
 *  - The workspace is a static device array of 128 MiB (134217728 bytes) per
 *    device, 256-byte aligned, that the library holds until the process ends.
 *    A layer whose workspace (moe_prefill_workspace_size with max_tokens =
 *    n_tokens) is larger is refused with MOE_EINVAL before anything is enqueued
 *    (e.g. d_model=2048, d_ff=768, 128 experts, top-8 fits up to ~1700 tokens).
 *  - Every call on a device shares that device's array, which keeps the last
 *    call's contents; each call first clears, with a kernel on `stream`, the
 *    parts that must start at zero.  Calls that overlap on one device (other
 *    streams, other threads) race on the array: the caller serialises them.
 *  - Work is enqueued on `stream` and the call returns before completion.
 * Errors: MOE_EINVAL (bad dimensions, pointers, too large a layer),
 * MOE_EUNSUPPORTED (not gfx950), MOE_EHIP.
 */
int moe_prefill_run_layer_noalloc(const moe_prefill_params_t* p, const moe_layer_io_t* io, void* stream);

/* ---------------------------------------------------------- stream pool --- */

typedef struct stream_pool_params {
    uint32_t struct_size;
    int32_t n_layers;                /* L; 0 tears the pool down */
    const void* const* host_blobs;   /* [L] pinned host blobs of layer_bytes each,
                                        caller-owned, valid until reconfigure/destroy */
    uint64_t layer_bytes;            /* must equal moe_prefill_layer_bytes() */
    int32_t prefetch_depth;          /* requested lookahead N >= 0 (0 = load-then-compute) */
    int32_t resident_layers;         /* max resident leading layers; -1 = as many as the budget leaves */
    int64_t max_vram_bytes;          /* > 0: budget for the pool; 0: no cap */
    int32_t requested_slots;         /* > 0: cap on the slot count; 0: derive */
    /* outputs */
    int32_t eff_slots;               /* slots allocated (one device address range) */
    int32_t eff_depth;               /* effective prefetch depth */
    int32_t eff_residents;           /* resident leading layers */
    int32_t warnings;                /* MOE_WARN_* bits */
    int32_t reserved0;
    /* appended fields (a smaller struct_size leaves them 0) */
    int32_t active_only;             /* != 0: a streamed layer that is not in the pool is
                                        loaded after its routing, only the experts that
                                        received rows; no lookahead prefetch (eff_depth 0) */
    int32_t reserved1;
    int64_t reserve_bytes;           /* > 0: device memory to keep free.  When a pass starts
                                        (moe_prefill_run_layer with layer 0) and the device
                                        has less free memory than this, the pool shrinks by
                                        the difference as stream_pool_set_budget does: that
                                        layer-0 call then waits on the host (bounded) for the
                                        released slots' queued work, so it must not be
                                        captured in a HIP graph; callers that capture passes
                                        leave this 0 and call stream_pool_set_budget between
                                        passes.  0: off */
} stream_pool_params_t;

#define MOE_WARN_SLOT_OVER_BUDGET 1  /* the one mandatory slot exceeds max_vram_bytes */
#define MOE_WARN_POOL_DEGRADED    2  /* allocation failed; fewer slots than planned */
#define MOE_WARN_DEPTH_REDUCED    4  /* prefetch depth reduced to fit */

/*
 * Plans and allocates the slot pool (pages #1905 "Summary"/"Effective
 * behavior" and #1906 "Summary"/pool-behaviour table):
 *  - one slot is mandatory execution memory, tried even above the budget
 *    (warning); the prefetch window is served before optional residents;
 *    only residents + 1 + depth slots are allocated, never the whole budget;
 *  - the pool is one contiguous device address range of fixed-size slots
 *    (each slot its own physical allocation where the device has virtual
 *    memory management, else one allocation); on allocation failure fewer
 *    slots of the same size are tried (residents first, then depth) down to
 *    one; if one slot fails: MOE_ENOMEM;
 *  - resident layers are uploaded before returning;
 *  - active_only (copy only the experts that receive rows): the layer's
 *    routing decides its copy.  After the grouping step of moe_prefill_run_layer
 *    a kernel reads the experts with rows > 0 straight from the pinned host blob
 *    (PCIe reads by the GPU, no host round trip) into the slot; experts without
 *    rows are not copied and never read.  host_blobs must then be page-locked
 *    host memory mapped for the device (hipHostMalloc, torch pin_memory);
 *    anything else is MOE_EINVAL.  The slot then holds a partial layer, so a
 *    later run of the same layer loads again;
 *  - calling again first drains the copy stream and releases the previous
 *    pool, prefetches and residents.
 * Effective values are written back into *inout.
 */
int stream_pool_configure(moe_prefill_t* h, stream_pool_params_t* inout);

/* Memory pressure (page #1905 "Summary": residents are evicted from the end of
 * the resident prefix when memory runs short, and the active segment never).
 * Shrinks the configured pool to at most max_vram_bytes (> 0) of slots and
 * returns the freed device memory at once:
 *  - resident layers leave from the end of the resident prefix first and are
 *    streamed from then on; a pool without a streaming slot keeps the first
 *    evicted layer's slot (and its data) as its streaming slot;
 *  - then prefetch slots (the effective depth drops), never below one slot:
 *    that slot is execution memory and stays even above the budget
 *    (MOE_WARN_SLOT_OVER_BUDGET);
 *  - a slot is released only after the work queued on it (its last layer's
 *    kernels, a copy into it) has finished: a bounded host wait
 *    (MOE_ETIMEOUT when it expires);
 *  - the pool is one reserved device address range whose slots each have
 *    their own physical allocation (HIP virtual memory), so released slots
 *    return their memory without moving the others.  A device without
 *    virtual memory management gets a single allocation at configure time and
 *    MOE_EUNSUPPORTED here.
 * Later passes produce the same outputs, with more layers streamed.  The
 * budget only shrinks the pool; stream_pool_configure builds a larger one. */
typedef struct stream_pool_budget {
    uint32_t struct_size;
    int32_t reserved0;
    int64_t max_vram_bytes;          /* in: the new pool budget, > 0 */
    /* outputs */
    int32_t eff_slots;               /* slots still holding memory */
    int32_t eff_depth;               /* effective prefetch depth */
    int32_t eff_residents;           /* resident leading layers */
    int32_t warnings;                /* MOE_WARN_* bits */
    uint64_t released_bytes;         /* device memory returned by this call */
} stream_pool_budget_t;

int stream_pool_set_budget(moe_prefill_t* h, stream_pool_budget_t* inout);

/* Pure planning step of stream_pool_configure (no device, no allocation), for
 * callers that want to see the plan first.  max_alloc_slots simulates the
 * allocator: > 0 means a pool of more slots than this fails to allocate, -1
 * means every allocation fails, 0 means none fail. */
typedef struct moe_pool_plan {
    uint32_t struct_size;
    int32_t n_layers;
    uint64_t slot_bytes;
    int32_t prefetch_depth;
    int32_t resident_layers;
    int64_t max_vram_bytes;
    int32_t requested_slots;
    int32_t max_alloc_slots;
    /* outputs */
    int32_t slots, depth, residents, warnings;
} moe_pool_plan_t;

int moe_prefill_plan_pool(moe_pool_plan_t* inout);

/* Pure planning step of stream_pool_set_budget: which slots a live pool of
 * `residents` resident and `streaming` streaming slots (an n_layers stack)
 * gives up to fit budget_slots slots.  No device, no allocation. */
typedef struct moe_pool_trim {
    uint32_t struct_size;
    int32_t n_layers;
    int32_t residents;               /* in: resident slots now */
    int32_t streaming;               /* in: streaming slots now */
    int64_t budget_slots;            /* in: slots the budget holds (may be 0) */
    /* outputs */
    int32_t new_residents, new_streaming;
    int32_t evicted;                 /* residents evicted, from the end of the prefix */
    int32_t converted;               /* 1: the first evicted resident's slot became the streaming slot */
    int32_t released;                /* slots whose memory is returned */
    int32_t warnings;                /* MOE_WARN_* bits */
} moe_pool_trim_t;

int moe_prefill_plan_trim(moe_pool_trim_t* inout);

/* ---------------------------------------------------------------- stats --- */

typedef struct moe_stats {
    uint32_t struct_size;
    int32_t reserved0;
    uint64_t layers_run;
    uint64_t prefetch_queued;        /* prefetch copies enqueued */
    uint64_t prefetch_activated;     /* layers that found their prefetched slot */
    uint64_t sync_loads;             /* load-then-compute copies */
    uint64_t prefetch_failed;        /* prefetch enqueues that failed (fell back) */
    uint64_t bytes_h2d;              /* bytes copied into the pool by whole-layer copies */
    int32_t eff_slots, eff_depth, eff_residents, warnings;
    /* appended fields */
    uint64_t sparse_loads;           /* active-expert loads launched */
    uint64_t experts_loaded;         /* experts those loads copied (device-counted) */
    uint64_t bytes_sparse;           /* bytes they copied (device-counted) */
    uint64_t evicted_residents;      /* resident layers given up under memory pressure */
    uint64_t released_bytes;         /* device memory the pool returned under pressure */
    uint64_t pressure_trims;         /* shrinks started by reserve_bytes at a pass start */
} moe_stats_t;

/* Counters of the handle: layers run, prefetches queued against prefetches that
 * a layer found ready (page #1905, "Verification": prefetches activated out of
 * those queued), synchronous loads, bytes copied, and the pool's evictions.
 * experts_loaded and bytes_sparse are kept on the
 * device; reading them waits for the device to finish its queued work. */
int moe_prefill_get_stats(const moe_prefill_t* h, moe_stats_t* inout);

/* ------------------------------------------------------------- logging --- */

#define MOE_LOG_ERROR 0
#define MOE_LOG_WARN 1
#define MOE_LOG_INFO 2

/* One message: its level (MOE_LOG_*), text (valid during the call) and the
 * user pointer given to moe_prefill_set_log. */
typedef void (*moe_log_fn)(int32_t level, const char* message, void* user);

/* Log sink of the handle: failed calls (level ERROR), degradations (WARN: a
 * smaller pool, a reduced prefetch depth, a slot above the budget, a prefetch
 * that fell back to a synchronous load, memory-pressure evictions) and pool
 * decisions (INFO) with level <= `level` go to fn.  fn == NULL removes the
 * sink.  Without a sink, MOE_LOG_LEVEL=<n> in the environment prints messages
 * of level <= n to stderr.  Host only; the callback runs on the calling
 * thread inside the library call. */
int moe_prefill_set_log(moe_prefill_t* h, moe_log_fn fn, void* user, int32_t level);

/* ------------------------------------------------------------- tracing --- */

#define MOE_N_KERNELS 7
/* Kernel ids, in launch order inside moe_prefill_run_layer. */
enum {
    MOE_K_ROUTE_QUANT = 0,    /* top-k routing, router weights, membership mask; Xq = Q8(x) */
    MOE_K_GROUP = 1,          /* per-expert row counts and membership-word prefixes */
    MOE_K_EXPERT_LOAD = 2,    /* active-expert load of a streamed layer (active_only pools) */
    MOE_K_SCATTER = 3,        /* group bounds, GEMM row tiles and their order, row table */
    MOE_K_GEMM_GATE_UP = 4,   /* GU grouped GEMM with the SwiGLU + Q8 epilogue: Hq, its scales */
    MOE_K_GEMM_DOWN = 5,      /* Dm grouped GEMM */
    MOE_K_COMBINE = 6         /* y = weighted combine */
};

typedef struct moe_kernel_times {
    uint32_t struct_size;
    int32_t n_kernels;                  /* out: MOE_N_KERNELS */
    uint64_t launches[MOE_N_KERNELS];   /* out: timed launches per kernel */
    double total_ms[MOE_N_KERNELS];     /* out: summed device time per kernel */
} moe_kernel_times_t;

/* enable != 0: every kernel of the following moe_prefill_run_layer calls is
 * bracketed by HIP events recorded on the launch stream (one event record
 * between consecutive kernels); 0 stops it.  Host only.  A kernel that a
 * layer does not launch (the expert load outside active_only loads) is not
 * counted for that layer. */
int moe_prefill_set_timing(moe_prefill_t* h, int32_t enable);

/* Waits (bounded; MOE_ETIMEOUT) for the timed launches so far, adds their
 * per-kernel device durations to the handle's totals, writes the totals to
 * *inout and, if reset != 0, zeroes them. */
int moe_prefill_kernel_times(moe_prefill_t* h, moe_kernel_times_t* inout, int32_t reset);

/* Name of kernel id (MOE_K_*), or "" for an unknown id. */
const char* moe_prefill_kernel_name(int32_t id);

/* --------------------------------------------------- exponential check --- */
/*
 * The kernels' own fp32 exponential, the one inside H = SwiGLU(GU) (the page
 * #663 "What" names the H stage; silu(g) = g / (1 + exp(-g))) and the router
 * weights (softmax over the k selected logits).  Hq codes are decided by H, so
 * this function must give the same bits as any other implementation of the same
 * Cody-Waite + Taylor steps; these two calls let a test compare it input by
 * input, over any range of fp32 bit patterns.
 *
 * out[i] = exp(x) where x is the fp32 number whose bit pattern is first_bits + i,
 * for i < n; first_bits + n <= 2^32.
 *  - moe_prefill_exp_host: computed on the calling thread by the host build of
 *    the same source; out is host memory.
 *  - moe_prefill_exp_device: one kernel enqueued on `stream` (returns before
 *    completion); out is device memory of n floats, owned by the caller.
 * MOE_EINVAL for a null out with n > 0 or a range beyond 2^32 patterns;
 * MOE_EHIP if the launch fails.
 */
int moe_prefill_exp_host(uint32_t first_bits, uint64_t n, float* out);
int moe_prefill_exp_device(uint32_t first_bits, uint64_t n, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PREFILL_H */
