// Launch interface of the MoE prefill kernels (host side of moe_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct GemmArgs {
    const int8_t* A;          // activation codes [rows, K]
    const float* A_scale;     // their block scales [rows][a_scale_stride], blocks 0 .. K/32-1 used
    const int32_t* row_src;   // grouped row -> A row (gate/up launch; the down launch reads row r)
    const uint8_t* blob;      // layer weight blob
    uint64_t expert_stride;   // bytes per expert
    uint64_t q_off, s_off;    // matrix quant / scale section offsets in an expert
    const int32_t* tiles;     // [max_tiles][3]: expert, first row, end row
    const int32_t* ntiles;    // number of valid tiles (device)
    float* out;               // [R, N]; gate/up launch: GU, written only if not null
    int8_t* hq;               // gate/up launch: Hq [R, f] = Q8(SwiGLU(GU)) (else unused)
    float* dh;                // gate/up launch: its block scales [R][dh_stride]
    float* h_out;             // gate/up launch: optional H [R, f] (null: not written)
    int dh_stride;
    int N, K;
    int E;                    // experts in the blob (tile expert indices are clamped to it)
    int gu_f;                 // f of the interleaved gate/up matrix (gate/up launch only)
    int a_scale_stride;       // floats per A_scale row (a multiple of the 8-block scale group)
    const uint32_t* fold_flag;  // nonzero: some A scale is outside the range the 16x codes allow
    uint32_t* h_flag;         // gate/up launch: set when an H block scale is outside that range
    // down launch, atomic combine: y [T, N] += wts[rows[r]] * (row r of the product) for row r
    // of token rtok[r], fp32 atomic adds (out is then null); null: the product goes to out
    float* y_add;
    const int32_t* rows;      // row -> pair t*k + j
    const int32_t* rtok;      // row -> token
    const float* wts;         // pair -> router weight
};

struct LayerLaunch {
    int T, d, f, E, k, W;
    const float* x;
    const float* logits;
    float* y;
    const uint8_t* blob;
    uint64_t expert_stride, gu_q_off, gu_s_off, d_q_off, d_s_off;
    int32_t* eidx;
    float* wts;
    uint32_t* mask;
    int32_t* wprefix;
    int32_t* counts;
    int32_t* bounds;
    int32_t* tiles;
    int32_t* ntiles;
    int32_t* rows;
    int32_t* pos;
    int32_t* rtok;
    int8_t* xq;
    float* dx;
    float* gu;                // optional export of GU [R, 2f] (caller memory; nullptr: not written)
    int8_t* hq;
    float* dh;
    float* dm;
    const uint8_t* load_src;  // active-expert load: device-accessible pinned host blob of the
    uint8_t* load_dst;        // layer and its pool slot (load_src null: the blob is in place)
    unsigned long long* load_stats;   // [2] experts and bytes loaded (device counters)
    float* h_out;             // optional export of H (nullptr: not written)
    int combine_atomic = 0;   // 1: the down GEMM adds w * Dm into y with atomics (y zeroed first,
                              // Dm not stored); the combine launch then only clears the mask
    hipEvent_t* marks;        // optional: kNumKernels + 1 timing events (nullptr: none);
                              // marks[i] before kernel i, marks[kNumKernels] after the last
};

// kernel ids in launch order (timing)
enum KernelId { kRouteQuant, kGroup, kExpertLoad, kScatter, kGemmGateUp, kGemmDown, kCombine,
                kNumKernels };

// route + quantise X, group (bounds, tiles), the active-expert load (if load_src), the row table,
// GU GEMM with SwiGLU+Q8, down GEMM (last reader of the weights) -- everything up to the combine.
// The kExpertLoad mark is recorded whether or not that kernel runs.
hipError_t launch_layer(const LayerLaunch& L, hipStream_t st);
// combine (and clear the membership mask for the next layer)
hipError_t launch_combine(const LayerLaunch& L, hipStream_t st);
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t st);
// Device address of the static scratch array of device `dev` (which must be current);
// looked up once per device.  kScratchBytes bytes, 256-byte aligned.
constexpr uint64_t kScratchBytes = 128ull << 20;
hipError_t scratch_device_ptr(int dev, uint8_t** out);
// the kernels' fp32 exponential over the inputs with bit patterns first .. first + n - 1
hipError_t launch_exp_range(uint32_t first, uint64_t n, float* out, hipStream_t st);
void exp_range_host(uint32_t first, uint64_t n, float* out);

}  // namespace moe
