/*
 * A plain C99 client of include/moe_prefill.h, built by the tests with gcc and
 * linked against libmoe_prefill.so -- what an application built against the
 * public header does.  The layer-streaming pages verify "current and undersized
 * versioned C API structures" and "compatibility of an executable built against
 * the previous public API" (stable-diffusion.cpp #1905, "Verification"); this
 * client carries the first published layouts of the structs that have grown
 * since (stream_pool_params_v1, moe_stats_v1, moe_layer_io_v1) and calls the
 * library with them.
 *
 *   abi_client layout         sizeof / offsetof of every public struct (JSON)
 *   abi_client host           host-only calls with current, undersized and
 *                             oversized structs (JSON); needs no GPU
 *   abi_client gpu DIR T d f E k
 *                             one resident layer and a 2-layer pool through
 *                             the old struct layouts, and one resident layer
 *                             with the atomic combine through the current one;
 *                             inputs x.bin, logits.bin, blob.bin from DIR,
 *                             outputs y_res.bin, y_pool0.bin, y_pool1.bin,
 *                             y_atomic.bin into DIR (JSON of return codes and
 *                             counters on stdout)
 */
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_prefill.h"

/* First published layouts of the two structs that gained trailing fields. */
typedef struct stream_pool_params_v1 {
    uint32_t struct_size;
    int32_t n_layers;
    const void* const* host_blobs;
    uint64_t layer_bytes;
    int32_t prefetch_depth;
    int32_t resident_layers;
    int64_t max_vram_bytes;
    int32_t requested_slots;
    int32_t eff_slots, eff_depth, eff_residents, warnings;
    int32_t reserved0;
} stream_pool_params_v1;

typedef struct moe_layer_io_v1 {
    uint32_t struct_size;
    int32_t layer;
    const void* weights_dev;
    int32_t n_tokens;
    int32_t reserved0;
    const float* x;
    const float* logits;
    float* y;
    int32_t* eidx;
    float* weights;
    int32_t* counts;
    int32_t* bounds;
    int32_t* rows;
    int32_t* pos;
    int8_t* xq;
    float* dx;
    float* gu;
    float* h;
    int8_t* hq;
    float* dh;
    float* dm;
} moe_layer_io_v1;

typedef struct moe_stats_v1 {
    uint32_t struct_size;
    int32_t reserved0;
    uint64_t layers_run, prefetch_queued, prefetch_activated, sync_loads, prefetch_failed, bytes_h2d;
    int32_t eff_slots, eff_depth, eff_residents, warnings;
} moe_stats_v1;

#define FIELD(S, f) printf("%s\"%s\": %zu", first ? "" : ", ", #f, offsetof(S, f)), first = 0
#define BEGIN(S) printf("%s\"%s\": {\"size\": %zu, \"fields\": {", nstruct++ ? ", " : "", #S, sizeof(S)), first = 1
#define END() printf("}}")

static int layout(void)
{
    int first = 1, nstruct = 0;
    printf("{");
    BEGIN(moe_prefill_params_t);
    FIELD(moe_prefill_params_t, struct_size); FIELD(moe_prefill_params_t, d_model);
    FIELD(moe_prefill_params_t, d_ff); FIELD(moe_prefill_params_t, n_experts);
    FIELD(moe_prefill_params_t, top_k); FIELD(moe_prefill_params_t, max_tokens);
    FIELD(moe_prefill_params_t, device); FIELD(moe_prefill_params_t, reserved0);
    FIELD(moe_prefill_params_t, workspace); FIELD(moe_prefill_params_t, workspace_bytes);
    END();
    BEGIN(moe_layer_io_t);
    FIELD(moe_layer_io_t, struct_size); FIELD(moe_layer_io_t, layer); FIELD(moe_layer_io_t, weights_dev);
    FIELD(moe_layer_io_t, n_tokens); FIELD(moe_layer_io_t, reserved0); FIELD(moe_layer_io_t, x);
    FIELD(moe_layer_io_t, logits); FIELD(moe_layer_io_t, y); FIELD(moe_layer_io_t, eidx);
    FIELD(moe_layer_io_t, weights); FIELD(moe_layer_io_t, counts); FIELD(moe_layer_io_t, bounds);
    FIELD(moe_layer_io_t, rows); FIELD(moe_layer_io_t, pos); FIELD(moe_layer_io_t, xq);
    FIELD(moe_layer_io_t, dx); FIELD(moe_layer_io_t, gu); FIELD(moe_layer_io_t, h);
    FIELD(moe_layer_io_t, hq); FIELD(moe_layer_io_t, dh); FIELD(moe_layer_io_t, dm);
    FIELD(moe_layer_io_t, combine); FIELD(moe_layer_io_t, reserved1);
    END();
    BEGIN(stream_pool_params_t);
    FIELD(stream_pool_params_t, struct_size); FIELD(stream_pool_params_t, n_layers);
    FIELD(stream_pool_params_t, host_blobs); FIELD(stream_pool_params_t, layer_bytes);
    FIELD(stream_pool_params_t, prefetch_depth); FIELD(stream_pool_params_t, resident_layers);
    FIELD(stream_pool_params_t, max_vram_bytes); FIELD(stream_pool_params_t, requested_slots);
    FIELD(stream_pool_params_t, eff_slots); FIELD(stream_pool_params_t, eff_depth);
    FIELD(stream_pool_params_t, eff_residents); FIELD(stream_pool_params_t, warnings);
    FIELD(stream_pool_params_t, reserved0); FIELD(stream_pool_params_t, active_only);
    FIELD(stream_pool_params_t, reserved1); FIELD(stream_pool_params_t, reserve_bytes);
    END();
    BEGIN(stream_pool_budget_t);
    FIELD(stream_pool_budget_t, struct_size); FIELD(stream_pool_budget_t, reserved0);
    FIELD(stream_pool_budget_t, max_vram_bytes); FIELD(stream_pool_budget_t, eff_slots);
    FIELD(stream_pool_budget_t, eff_depth); FIELD(stream_pool_budget_t, eff_residents);
    FIELD(stream_pool_budget_t, warnings); FIELD(stream_pool_budget_t, released_bytes);
    END();
    BEGIN(moe_pool_plan_t);
    FIELD(moe_pool_plan_t, struct_size); FIELD(moe_pool_plan_t, n_layers); FIELD(moe_pool_plan_t, slot_bytes);
    FIELD(moe_pool_plan_t, prefetch_depth); FIELD(moe_pool_plan_t, resident_layers);
    FIELD(moe_pool_plan_t, max_vram_bytes); FIELD(moe_pool_plan_t, requested_slots);
    FIELD(moe_pool_plan_t, max_alloc_slots); FIELD(moe_pool_plan_t, slots); FIELD(moe_pool_plan_t, depth);
    FIELD(moe_pool_plan_t, residents); FIELD(moe_pool_plan_t, warnings);
    END();
    BEGIN(moe_pool_trim_t);
    FIELD(moe_pool_trim_t, struct_size); FIELD(moe_pool_trim_t, n_layers); FIELD(moe_pool_trim_t, residents);
    FIELD(moe_pool_trim_t, streaming); FIELD(moe_pool_trim_t, budget_slots);
    FIELD(moe_pool_trim_t, new_residents); FIELD(moe_pool_trim_t, new_streaming);
    FIELD(moe_pool_trim_t, evicted); FIELD(moe_pool_trim_t, converted); FIELD(moe_pool_trim_t, released);
    FIELD(moe_pool_trim_t, warnings);
    END();
    BEGIN(moe_stats_t);
    FIELD(moe_stats_t, struct_size); FIELD(moe_stats_t, reserved0); FIELD(moe_stats_t, layers_run);
    FIELD(moe_stats_t, prefetch_queued); FIELD(moe_stats_t, prefetch_activated);
    FIELD(moe_stats_t, sync_loads); FIELD(moe_stats_t, prefetch_failed); FIELD(moe_stats_t, bytes_h2d);
    FIELD(moe_stats_t, eff_slots); FIELD(moe_stats_t, eff_depth); FIELD(moe_stats_t, eff_residents);
    FIELD(moe_stats_t, warnings); FIELD(moe_stats_t, sparse_loads); FIELD(moe_stats_t, experts_loaded);
    FIELD(moe_stats_t, bytes_sparse); FIELD(moe_stats_t, evicted_residents);
    FIELD(moe_stats_t, released_bytes); FIELD(moe_stats_t, pressure_trims);
    END();
    BEGIN(moe_kernel_times_t);
    FIELD(moe_kernel_times_t, struct_size); FIELD(moe_kernel_times_t, n_kernels);
    FIELD(moe_kernel_times_t, launches); FIELD(moe_kernel_times_t, total_ms);
    END();
    printf(", \"v1_sizes\": {\"stream_pool_params_v1\": %zu, \"moe_stats_v1\": %zu, \"moe_layer_io_v1\": %zu}",
           sizeof(stream_pool_params_v1), sizeof(moe_stats_v1), sizeof(moe_layer_io_v1));
    printf(", \"abi_version\": %d}\n", MOE_PREFILL_ABI_VERSION);
    return 0;
}

static int host(void)
{
    moe_prefill_params_t p;
    memset(&p, 0, sizeof p);
    p.struct_size = sizeof p;
    p.d_model = 256;
    p.d_ff = 512;
    p.n_experts = 8;
    p.top_k = 2;
    p.max_tokens = 64;
    uint64_t ws_cur = 0, ws_old = 0;
    const int rc_cur = moe_prefill_workspace_size(&p, &ws_cur);
    /* undersized: a caller compiled before the workspace fields existed */
    p.struct_size = (uint32_t)offsetof(moe_prefill_params_t, workspace);
    const int rc_old = moe_prefill_workspace_size(&p, &ws_old);

    /* oversized: a caller compiled against a newer header; a zero tail is accepted,
       a nonzero one refused */
    struct {
        moe_pool_plan_t plan;
        int64_t future[2];
    } big;
    memset(&big, 0, sizeof big);
    big.plan.struct_size = sizeof big;
    big.plan.n_layers = 48;
    big.plan.slot_bytes = 339738624ull;
    big.plan.prefetch_depth = 2;
    big.plan.resident_layers = -1;
    big.plan.max_vram_bytes = 7 * 339738624ll;
    const int rc_big_zero = moe_prefill_plan_pool(&big.plan);
    const int plan_slots = big.plan.slots, plan_res = big.plan.residents, plan_depth = big.plan.depth;
    const uint32_t size_kept = big.plan.struct_size;
    big.future[1] = 7;
    const int rc_big_nonzero = moe_prefill_plan_pool(&big.plan);
    const char* err_big = moe_prefill_last_error(NULL);
    char err_copy[256];
    snprintf(err_copy, sizeof err_copy, "%s", err_big);
    for (char* c = err_copy; *c; ++c)
        if (*c == '"' || *c == '\\') *c = '\'';

    moe_pool_trim_t t;
    memset(&t, 0, sizeof t);
    t.struct_size = sizeof t;
    t.n_layers = 48;
    t.residents = 4;
    t.streaming = 3;
    t.budget_slots = 5;
    const int rc_trim = moe_prefill_plan_trim(&t);

    moe_prefill_t* h = (moe_prefill_t*)0x1;
    p.struct_size = sizeof p;
    const int rc_create = moe_prefill_create(&p, &h);   /* no GPU here: MOE_EUNSUPPORTED */
    const int h_null = h == NULL;

    float e[3];
    const int rc_exp = moe_prefill_exp_host(0x3f800000u, 3, e);   /* exp(1), exp(1+ulp), ... */

    printf("{\"rc_ws_current\": %d, \"ws_current\": %llu, \"rc_ws_undersized\": %d, \"ws_undersized\": %llu, "
           "\"rc_oversized_zero_tail\": %d, \"plan_slots\": %d, \"plan_residents\": %d, \"plan_depth\": %d, "
           "\"struct_size_kept\": %u, \"rc_oversized_nonzero_tail\": %d, \"err_oversized\": \"%s\", "
           "\"rc_trim\": %d, \"trim_new_residents\": %d, \"trim_released\": %d, "
           "\"rc_create\": %d, \"create_out_null\": %d, \"rc_exp\": %d, \"exp1\": %.9g, "
           "\"expected_oversized_size\": %zu}\n",
           rc_cur, (unsigned long long)ws_cur, rc_old, (unsigned long long)ws_old, rc_big_zero, plan_slots,
           plan_res, plan_depth, size_kept, rc_big_nonzero, err_copy, rc_trim, t.new_residents, t.released,
           rc_create, h_null, rc_exp, (double)e[0], sizeof big);
    return 0;
}

#ifdef ABI_CLIENT_GPU
#include <hip/hip_runtime_api.h>

static void* read_file(const char* dir, const char* name, size_t* n)
{
    char path[1024];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "rb");
    if (!f) return NULL;
    fseek(f, 0, SEEK_END);
    *n = (size_t)ftell(f);
    fseek(f, 0, SEEK_SET);
    void* p = malloc(*n);
    if (p && fread(p, 1, *n, f) != *n) {
        free(p);
        p = NULL;
    }
    fclose(f);
    return p;
}

static int write_dev(const char* dir, const char* name, const void* dev, size_t n)
{
    char path[1024];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    void* h = malloc(n);
    if (!h || hipMemcpy(h, dev, n, hipMemcpyDeviceToHost) != hipSuccess) return -1;
    FILE* f = fopen(path, "wb");
    const int ok = f && fwrite(h, 1, n, f) == n;
    if (f) fclose(f);
    free(h);
    return ok ? 0 : -1;
}

#define CK(x)                                                                      \
    do {                                                                           \
        if ((x) != hipSuccess) {                                                   \
            fprintf(stderr, "HIP call failed: %s\n", #x);                          \
            return 2;                                                              \
        }                                                                          \
    } while (0)

static int gpu(const char* dir, int T, int d, int f, int E, int k)
{
    size_t nx, nl, nb;
    float* x = (float*)read_file(dir, "x.bin", &nx);
    float* lg = (float*)read_file(dir, "logits.bin", &nl);
    void* blob = read_file(dir, "blob.bin", &nb);
    if (!x || !lg || !blob || nx != (size_t)T * d * 4 || nl != (size_t)T * E * 4 ||
        nb != moe_prefill_layer_bytes(d, f, E)) {
        fprintf(stderr, "bad inputs\n");
        return 2;
    }
    /* a caller compiled before the workspace fields existed: the library allocates */
    moe_prefill_params_t p;
    memset(&p, 0x5a, sizeof p);                 /* bytes past struct_size must not be read */
    p.struct_size = (uint32_t)offsetof(moe_prefill_params_t, workspace);
    p.d_model = d;
    p.d_ff = f;
    p.n_experts = E;
    p.top_k = k;
    p.max_tokens = T;
    p.device = 0;
    p.reserved0 = 0;
    moe_prefill_t* h = NULL;
    const int rc_create = moe_prefill_create(&p, &h);
    if (rc_create != MOE_OK) {
        printf("{\"rc_create\": %d}\n", rc_create);
        return 1;
    }
    float *dx, *dl, *y;
    void* dblob;
    CK(hipMalloc((void**)&dx, nx));
    CK(hipMalloc((void**)&dl, nl));
    CK(hipMalloc((void**)&y, nx));
    CK(hipMalloc(&dblob, nb));
    CK(hipMemcpy(dx, x, nx, hipMemcpyHostToDevice));
    CK(hipMemcpy(dl, lg, nl, hipMemcpyHostToDevice));
    CK(hipMemcpy(dblob, blob, nb, hipMemcpyHostToDevice));

    /* the first published layer layout: no combine field, so the default gather */
    moe_layer_io_v1 io;
    memset(&io, 0, sizeof io);
    io.struct_size = sizeof io;
    io.layer = -1;
    io.weights_dev = dblob;
    io.n_tokens = T;
    io.x = dx;
    io.logits = dl;
    io.y = y;
    const int rc_res = moe_prefill_run_layer(h, (const moe_layer_io_t*)&io, NULL);
    CK(hipDeviceSynchronize());
    if (write_dev(dir, "y_res.bin", y, nx)) return 2;

    /* the current layout with the atomic combine */
    moe_layer_io_t ioa;
    memset(&ioa, 0, sizeof ioa);
    ioa.struct_size = sizeof ioa;
    ioa.layer = -1;
    ioa.weights_dev = dblob;
    ioa.n_tokens = T;
    ioa.x = dx;
    ioa.logits = dl;
    ioa.y = y;
    ioa.combine = MOE_COMBINE_ATOMIC;
    const int rc_atomic = moe_prefill_run_layer(h, &ioa, NULL);
    CK(hipDeviceSynchronize());
    if (write_dev(dir, "y_atomic.bin", y, nx)) return 2;

    /* a two-layer pool configured through the first published stream-pool layout */
    void* pinned[2];
    CK(hipHostMalloc(&pinned[0], nb, 0));
    CK(hipHostMalloc(&pinned[1], nb, 0));
    memcpy(pinned[0], blob, nb);
    memcpy(pinned[1], blob, nb);
    stream_pool_params_v1 sp;
    memset(&sp, 0, sizeof sp);
    sp.struct_size = sizeof sp;
    sp.n_layers = 2;
    sp.host_blobs = (const void* const*)pinned;
    sp.layer_bytes = nb;
    sp.prefetch_depth = 1;
    sp.resident_layers = 0;
    const int rc_pool = stream_pool_configure(h, (stream_pool_params_t*)&sp);
    int rc_l0 = -100, rc_l1 = -100;
    io.weights_dev = NULL;
    io.layer = 0;
    rc_l0 = moe_prefill_run_layer(h, (const moe_layer_io_t*)&io, NULL);
    CK(hipDeviceSynchronize());
    if (write_dev(dir, "y_pool0.bin", y, nx)) return 2;
    io.layer = 1;
    rc_l1 = moe_prefill_run_layer(h, (const moe_layer_io_t*)&io, NULL);
    CK(hipDeviceSynchronize());
    if (write_dev(dir, "y_pool1.bin", y, nx)) return 2;

    moe_stats_v1 st;
    memset(&st, 0xff, sizeof st);
    st.struct_size = sizeof st;
    const int rc_stats = moe_prefill_get_stats(h, (moe_stats_t*)&st);
    printf("{\"rc_create\": %d, \"rc_resident\": %d, \"rc_atomic\": %d, \"rc_pool\": %d, \"eff_slots\": %d, \"eff_depth\": %d, "
           "\"eff_residents\": %d, \"pool_struct_size_kept\": %u, \"rc_layer0\": %d, \"rc_layer1\": %d, "
           "\"rc_stats\": %d, \"stats_struct_size_kept\": %u, \"layers_run\": %llu, \"prefetch_queued\": %llu, "
           "\"prefetch_activated\": %llu, \"sync_loads\": %llu, \"bytes_h2d\": %llu}\n",
           rc_create, rc_res, rc_atomic, rc_pool, sp.eff_slots, sp.eff_depth, sp.eff_residents, sp.struct_size, rc_l0, rc_l1,
           rc_stats, st.struct_size, (unsigned long long)st.layers_run, (unsigned long long)st.prefetch_queued,
           (unsigned long long)st.prefetch_activated, (unsigned long long)st.sync_loads,
           (unsigned long long)st.bytes_h2d);
    moe_prefill_destroy(h);
    (void)hipHostFree(pinned[0]);
    (void)hipHostFree(pinned[1]);
    (void)hipFree(dx);
    (void)hipFree(dl);
    (void)hipFree(y);
    (void)hipFree(dblob);
    free(x);
    free(lg);
    free(blob);
    return 0;
}
#endif

int main(int argc, char** argv)
{
    if (argc >= 2 && !strcmp(argv[1], "layout")) return layout();
    if (argc >= 2 && !strcmp(argv[1], "host")) return host();
#ifdef ABI_CLIENT_GPU
    if (argc >= 8 && !strcmp(argv[1], "gpu"))
        return gpu(argv[2], atoi(argv[3]), atoi(argv[4]), atoi(argv[5]), atoi(argv[6]), atoi(argv[7]));
#endif
    fprintf(stderr, "usage: abi_client layout | host | gpu DIR T d f E k\n");
    return 2;
}
