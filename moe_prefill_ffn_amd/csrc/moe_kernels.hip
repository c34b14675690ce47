// HIP kernels (CDNA4 / gfx950) of the MoE prompt (prefill) FFN layer.
//
// The steps follow the prompt path of the page "prefill: a layer split's idle
// card streams a share of a one-chunk prompt's experts" (Strata #663, section
// "What"): mixed activations -> Xq, router -> row table + group bounds,
// GU = grouped GEMM, H = SwiGLU, Hq, Dm = grouped GEMM, combine.  The page
// names these buffers only; the arithmetic read here is:
//   route     top-k of the E logits (ties to the lower expert index), weights =
//             softmax over the k selected logits (fp32)
//   group     stable counting sort of the pairs p = t*k + j on their expert
//   Q8        blocks of 32: scale = amax/127 (fp32), code = rint(x/scale) clamped
//   GEMM      Q4 weights (int4, fp16 scale per 32 along K) x Q8 activations,
//             exact int32 dot per 32-block on the int8 MFMA, blocks combined in
//             fp32 in ascending order: acc = fma((float)isum, a_scale*w_scale, acc)
//   SwiGLU    h = g / (1 + exp(-g)) * u
//   combine   y[t] = sum_j w[t,j] * Dm[pos(t,j)], j ascending, fma chain
//
// Build flags (see build.py): -ffp-contract=off, no fast-math, correctly
// rounded fp32 division, fp32 denormals kept, packed-fp32 instructions off.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "moe_kernels.h"
#include "moe_layout.h"
#include "moe_math.h"

namespace moe {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// exp_cw (moe_math.h): the fp32 exponential of the SwiGLU and the router weights.

// Q8 code of v given the block scale d (d > 0): rint(v / d) clamped to +-127.
__device__ __forceinline__ int q8_code(float v, float d)
{
    float q = __builtin_rintf(v / d);
    q = q > 127.0f ? 127.0f : q;
    q = q < -127.0f ? -127.0f : q;
    return (int)q;
}

__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d)
{
    return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
           ((uint32_t)(d & 0xff) << 24);
}

// Quantise the 4 values this lane holds of a 32-block spread over 8 lanes
// (lanes 8g .. 8g+7 of the wave hold one block).  Returns the packed codes;
// *scale gets the block scale.
__device__ __forceinline__ uint32_t q8_block_of8(float4 v, float* scale)
{
    float m = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    m = fmaxf(m, __shfl_xor(m, 4));
    const float d = m / 127.0f;
    *scale = d;
    if (d == 0.0f) return 0u;
    return pack4(q8_code(v.x, d), q8_code(v.y, d), q8_code(v.z, d), q8_code(v.w, d));
}

// ------------------------------------------------------- route + quantise ---
// One launch, two kinds of workgroup.  Workgroups [0, n_route) route tokens (up
// to 128 experts one token per workgroup, above that 4 per workgroup, one per
// wave); the rest quantise X to Q8 and flag block scales outside the range the
// GEMMs' 16x weight codes allow.
//
// Routing: with key(e) = (order-preserving bits of the logit, with -0 read as
// +0) << 32 | (2^32 - 1 - e), the order (larger logit first, ties to the lower
// expert index) is the unsigned order of the 64-bit keys, and all keys differ.
// Slot j of a token is the expert whose key has rank j.  Up to 128 experts the
// ranks are counted directly (a workgroup per token, every key compared with all
// E keys broadcast from LDS); above that, each lane keeps the keys of experts lane,
// lane + 64, ... in registers and slot j is the wave-wide maximum key after
// slots 0 .. j-1 were taken out (k rounds of a lane-local maximum and a 6-step
// butterfly): O(E k) instead of O(E^2) compares.  Both give the same slots.
// Router weights: softmax over the k selected logits, summed in ascending slot
// order.  Each selected (token, expert) also sets the token's bit in the expert
// membership mask read by the grouping step.
constexpr int kRouteMaxE = 1024;
constexpr int kRouteKeys = kRouteMaxE / 64;     // keys per lane
constexpr int kRankMaxE = 128;                  // rank counting up to this many experts

__device__ __forceinline__ uint64_t route_key(float v, int e)
{
    uint32_t u = v == 0.0f ? 0u : __float_as_uint(v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m)
{
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m);
    return ((uint64_t)hi << 32) | lo;
}

// router weights of the token's k slots, whose logits are in zsel[0 .. k) (k <= 1024):
// z_j = exp(l_j - l_0) (lane j % 64 computes slot j), S = z_0 + ... + z_{k-1} summed in
// ascending slot order, w_j = z_j / S
__device__ __forceinline__ void route_weights(int t, int k, float* __restrict__ wts, float* zsel)
{
    const int lane = threadIdx.x & 63;
    __builtin_amdgcn_wave_barrier();
    const float top = zsel[0];
    __builtin_amdgcn_wave_barrier();
    for (int j = lane; j < k; j += 64) zsel[j] = exp_cw(zsel[j] - top);
    __builtin_amdgcn_wave_barrier();
    float sum = 0.0f;
    for (int j = 0; j < k; ++j) sum += zsel[j];
    for (int j = lane; j < k; j += 64) wts[(int64_t)t * k + j] = zsel[j] / sum;
}

// E <= kRankMaxE: one token per workgroup.  Thread (e = tid % 128, part = tid / 128)
// counts the keys of part `part` of the experts (the first or second half of
// 0 .. E-1) that beat key e; the two partial ranks add up in LDS.  Splitting the
// E^2 compares over four waves per token keeps every SIMD busy with several
// routing waves instead of one long serial one.
__device__ __forceinline__ void route_token_rank(const float* __restrict__ logits, int t, int E,
                                                 int k, int32_t* __restrict__ eidx,
                                                 float* __restrict__ wts,
                                                 uint32_t* __restrict__ mask, int W,
                                                 uint64_t* keys, int* prank, float* zsel)
{
    const int tid = threadIdx.x;
    const float* lt = logits + (int64_t)t * E;
    if (tid < E) keys[tid] = route_key(lt[tid], tid);
    __syncthreads();
    const int e = tid & (kRankMaxE - 1), part = tid >> 7;   // part: uniform per wave
    const int hE = (E + 1) >> 1;
    const int c0 = part ? hE : 0, c1 = part ? E : hE;
    int rank = 0;
    if (e < E) {
        const uint64_t me = keys[e];
        for (int c = c0; c < c1; ++c) rank += keys[c] > me ? 1 : 0;
        if (part) prank[e] = rank;
    }
    __syncthreads();
    if (!part && e < E) {
        rank += prank[e];
        if (rank < k) {
            eidx[(int64_t)t * k + rank] = e;
            zsel[rank] = lt[e];
            atomicOr(&mask[(int64_t)e * W + (t >> 5)], 1u << (t & 31));
        }
    }
    __syncthreads();
    if (tid < 64) route_weights(t, k, wts, zsel);
}

template <int NK>   // keys per lane: E <= 64 * NK
__device__ __forceinline__ void route_token(const float* __restrict__ logits, int t, int E, int k,
                                            int32_t* __restrict__ eidx, float* __restrict__ wts,
                                            uint32_t* __restrict__ mask, int W, float* zsel)
{
    const int lane = threadIdx.x & 63;
    const float* lt = logits + (int64_t)t * E;
    uint64_t key[NK];
#pragma unroll
    for (int i = 0; i < NK; ++i) {
        const int e = lane + 64 * i;
        key[i] = e < E ? route_key(lt[e], e) : 0ull;   // 0: below every real key
    }
    for (int j = 0; j < k; ++j) {
        uint64_t m = key[0];
#pragma unroll
        for (int i = 1; i < NK; ++i) m = max_u64(m, key[i]);
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) m = max_u64(m, shfl_xor_u64(m, o));
        const int e = (int)(0xFFFFFFFFu - (uint32_t)m);  // the same on every lane
#pragma unroll
        for (int i = 0; i < NK; ++i) key[i] = key[i] == m ? 0ull : key[i];
        if (lane == 0) {
            eidx[(int64_t)t * k + j] = e;
            zsel[j] = lt[e];
            atomicOr(&mask[(int64_t)e * W + (t >> 5)], 1u << (t & 31));
        }
    }
    route_weights(t, k, wts, zsel);
}

// True when a nonzero block scale d lies outside [2^-98, 2^107] (NaN included).
// Inside that range every product d * w_scale with a nonzero fp16 weight scale
// (|w_scale| in [2^-24, 65504]) stays a normal fp32 number after a division by 16,
// which the grouped GEMM's 16x codes rely on.
__device__ __forceinline__ bool scale_outside_fold_range(float d)
{
    const float a = fabsf(d);
    return d != 0.0f && !(a >= 0x1p-98f && a <= 0x1p107f);
}

// x is a flat array of n_blocks 32-float blocks (a row-major [rows, K] matrix
// with K % 32 == 0); 8 lanes per block, 4 values per lane.  A wave takes
// kQuantBlocksPerWave consecutive blocks: its 8-lane group g the blocks b0 + g,
// + 8, + 16, + 24, so each of the four loads reads 1 KiB of contiguous X and all
// four are in flight together.  Block blk = row * nbk + b; its scale goes to
// scale[row * stride + b].  n_blocks < 2^31 (T * d / 32 <= 2^21 * 512).
constexpr int kQuantBlocksPerWave = 32;

__device__ __forceinline__ void quant_blocks_of_wave(const float* __restrict__ x, int64_t b0,
                                                     int64_t n_blocks, int nbk, int stride,
                                                     int8_t* __restrict__ q, float* __restrict__ scale,
                                                     uint32_t* __restrict__ flag)
{
    const int sub = threadIdx.x & 7;
    constexpr int kN = kQuantBlocksPerWave / 8;
    float4 v[kN];
#pragma unroll
    for (int j = 0; j < kN; ++j) {                // clamped: a block past the end is loaded, not used
        const int64_t blk = b0 + 8 * j < n_blocks ? b0 + 8 * j : n_blocks - 1;
        v[j] = *reinterpret_cast<const float4*>(x + blk * 32 + sub * 4);
    }
#pragma unroll
    for (int j = 0; j < kN; ++j) {
        const int64_t blk = b0 + 8 * j;
        if (blk >= n_blocks) break;               // uniform over the 8-lane group
        float d;
        const uint32_t packed = q8_block_of8(v[j], &d);
        *reinterpret_cast<uint32_t*>(q + blk * 32 + sub * 4) = packed;
        if (sub == 0) {
            const uint32_t row = (uint32_t)blk / (uint32_t)nbk;
            scale[(int64_t)row * stride + ((uint32_t)blk - row * (uint32_t)nbk)] = d;
            if (scale_outside_fold_range(d)) atomicOr(flag, 1u);
        }
    }
}

__global__ __launch_bounds__(256) void k_route_quant(const float* __restrict__ logits, int T, int E,
                                                     int k, int32_t* __restrict__ eidx,
                                                     float* __restrict__ wts,
                                                     uint32_t* __restrict__ mask, int W,
                                                     int n_route, const float* __restrict__ x,
                                                     int64_t n_blocks, int nbk, int dx_stride,
                                                     int8_t* __restrict__ xq, float* __restrict__ dx,
                                                     uint32_t* __restrict__ x_flag)
{
    __shared__ uint64_t keys[kRankMaxE];
    __shared__ int prank[kRankMaxE];
    __shared__ float zsel[4][kRouteMaxE];                 // selected logits, then their exps
    if ((int)blockIdx.x < n_route) {
        if (E <= kRankMaxE) {                             // one token per workgroup
            const int t = blockIdx.x;
            if (t < T) route_token_rank(logits, t, E, k, eidx, wts, mask, W, keys, prank, zsel[0]);
            return;
        }
        const int wave = threadIdx.x >> 6;                // one token per wave
        const int t = blockIdx.x * 4 + wave;
        if (t >= T) return;
        if (E <= 256)
            route_token<4>(logits, t, E, k, eidx, wts, mask, W, zsel[wave]);
        else
            route_token<kRouteKeys>(logits, t, E, k, eidx, wts, mask, W, zsel[wave]);
        return;
    }
    const int64_t wave = ((int64_t)(blockIdx.x - n_route) * 256 + threadIdx.x) >> 6;
    const int64_t b0 = wave * kQuantBlocksPerWave + ((threadIdx.x & 63) >> 3);
    if (b0 < n_blocks) quant_blocks_of_wave(x, b0, n_blocks, nbk, dx_stride, xq, dx, x_flag);
}

// ---------------------------------------------------------------- group ---
// The row table is a stable counting sort of the pairs p = t*k + j on their
// expert.  Word w of expert e in the membership mask holds tokens 32w..32w+31
// routed to e.
//
// k_group: one workgroup per expert writes the exclusive prefix of the word
// popcounts and the expert's row count.  No workgroup waits for another: the
// bounds are derived from the counts by every workgroup of the next kernel.
constexpr int kGroupThreads = 256;

__global__ __launch_bounds__(kGroupThreads) void k_group(const uint32_t* __restrict__ mask, int W,
                                                         int32_t* __restrict__ wprefix,
                                                         int32_t* __restrict__ counts)
{
    __shared__ int s_tot[4];
    const int e = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int running = 0;
    for (int base = 0; base < W; base += kGroupThreads) {
        const int w = base + tid;
        const int c = w < W ? __popc(mask[(int64_t)e * W + w]) : 0;
        int incl = c;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o);
            if (lane >= o) incl += y;
        }
        if (lane == 63) s_tot[wave] = incl;
        __syncthreads();
        int before = 0, total = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            before += i < wave ? s_tot[i] : 0;
            total += s_tot[i];
        }
        if (w < W) wprefix[(int64_t)e * W + w] = running + before + incl - c;
        running += total;
        __syncthreads();
    }
    if (tid == 0) counts[e] = running;
}

// -------------------------------------------------------- expert load ---
// Active-expert load of a streamed layer: once the grouping has counted the
// rows of every expert, copy only the experts that received rows from the
// pinned host blob (read over PCIe by the kernel itself, so the choice needs no
// host round trip) into the pool slot.  Every workgroup takes a grid-stride
// share of each active expert's 16-byte words, expert after expert.
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_expert_load(const uint8_t* __restrict__ src,
                                                     uint8_t* __restrict__ dst,
                                                     const int32_t* __restrict__ counts, int E,
                                                     uint64_t expert_bytes,
                                                     unsigned long long* __restrict__ stats)
{
    const uint64_t n16 = expert_bytes / 16;
    const uint64_t stride = (uint64_t)gridDim.x * 256;
    for (int e = 0; e < E; ++e) {
        if (counts[e] == 0) continue;                     // uniform
        const v4u* s = reinterpret_cast<const v4u*>(src + (uint64_t)e * expert_bytes);
        v4u* d = reinterpret_cast<v4u*>(dst + (uint64_t)e * expert_bytes);
        for (uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride)
            d[i] = __builtin_nontemporal_load(s + i);
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            atomicAdd(&stats[0], 1ull);
            atomicAdd(&stats[1], (unsigned long long)expert_bytes);
        }
    }
}

// ------------------------------------------------------------ row table ---
// Row table: pair p = t*k + j goes to row bounds[e] + prefix[e][t/32] + (tokens
// of word t/32 before t routed to e) -- stable in p.  Every workgroup first
// scans the E counts (E <= 1024: four per thread) into the group bounds in LDS;
// workgroup 0 also writes the bounds and the GEMM row-tile list (expert, first
// row, end row; kBM rows per tile; expert order) for the kernels that follow, a
// run of consecutive tiles per thread (the run's expert found by binary search
// over the experts' first tiles: empty experts own no tiles).
__global__ __launch_bounds__(256) void k_scatter(const int32_t* __restrict__ eidx, int64_t R, int k,
                                                 const uint32_t* __restrict__ mask,
                                                 const int32_t* __restrict__ wprefix,
                                                 const int32_t* __restrict__ counts, int E, int W,
                                                 int32_t* __restrict__ bounds,
                                                 int32_t* __restrict__ tiles,
                                                 int32_t* __restrict__ ntiles,
                                                 int32_t* __restrict__ rows, int32_t* __restrict__ pos,
                                                 int32_t* __restrict__ rtok)
{
    __shared__ int s_bounds[kRouteMaxE];
    __shared__ int s_tfirst[kRouteMaxE + 1];              // first tile of each expert (writer)
    __shared__ int s_wc[4], s_wt[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool writer = blockIdx.x == 0;
    int c4[4], t4[4], sc = 0, st = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ee = tid * 4 + i;
        c4[i] = ee < E ? counts[ee] : 0;
        t4[i] = (c4[i] + kBM - 1) / kBM;
        sc += c4[i];
        st += t4[i];
    }
    int ic = sc, it = st;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int yc = __shfl_up(ic, o);
        const int yt = __shfl_up(it, o);
        if (lane >= o) {
            ic += yc;
            it += yt;
        }
    }
    if (lane == 63) {
        s_wc[wave] = ic;
        s_wt[wave] = it;
    }
    __syncthreads();
    int bc = 0, bt = 0, all_c = 0, all_t = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        bc += i < wave ? s_wc[i] : 0;
        bt += i < wave ? s_wt[i] : 0;
        all_c += s_wc[i];
        all_t += s_wt[i];
    }
    int start = bc + ic - sc, tstart = bt + it - st;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ee = tid * 4 + i;
        if (ee < E) {
            s_bounds[ee] = start;
            s_tfirst[ee] = tstart;
            if (writer) bounds[ee] = start;
        }
        start += c4[i];
        tstart += t4[i];
    }
    if (tid == 0) s_tfirst[E] = all_t;
    if (writer && tid == 0) {
        bounds[E] = all_c;
        *ntiles = all_t;
    }
    __syncthreads();
    // tile tau belongs to the expert e with s_tfirst[e] <= tau < s_tfirst[e + 1]; each
    // thread takes a run of consecutive tiles (a binary search for the run's first
    // tile, then a walk).
    const int run = (all_t + 255) >> 8;
    const int t0 = tid * run, t1 = t0 + run < all_t ? t0 + run : all_t;
    int lo0 = 0;
    if (t0 < t1) {
        int hi = E - 1;
        while (lo0 < hi) {
            const int mid = (lo0 + hi + 1) >> 1;
            if (s_tfirst[mid] <= t0)
                lo0 = mid;
            else
                hi = mid - 1;
        }
    }
    auto tile_rows = [&](int tau, int& lo, int& r0, int& r1) {
        while (lo + 1 < E && s_tfirst[lo + 1] <= tau) ++lo;
        r0 = s_bounds[lo] + (tau - s_tfirst[lo]) * kBM;
        const int rend = lo + 1 < E ? s_bounds[lo + 1] : all_c;
        r1 = r0 + kBM < rend ? r0 + kBM : rend;
    };
    if (writer) {
        int lo = lo0, r0, r1;
        for (int tau = t0; tau < t1; ++tau) {
            tile_rows(tau, lo, r0, r1);
            tiles[3 * tau + 0] = lo;
            tiles[3 * tau + 1] = r0;
            tiles[3 * tau + 2] = r1;
        }
    }
    const int64_t p = (int64_t)blockIdx.x * 256 + tid;
    if (p >= R) return;
    const int t = (int)(p / k);
    int e = eidx[p];
    e = e < 0 ? 0 : (e >= E ? E - 1 : e);
    const int64_t wi = (int64_t)e * W + (t >> 5);
    const uint32_t below = mask[wi] & ((1u << (t & 31)) - 1u);
    int row = s_bounds[e] + wprefix[wi] + __popc(below);
    // a consistent table always gives row in [0, R); the clamp only keeps an
    // inconsistent one from writing outside the buffers
    row = row < 0 ? 0 : (row >= (int)R ? (int)R - 1 : row);
    rows[row] = (int32_t)p;
    pos[p] = row;
    rtok[row] = t;
}

// ---------------------------------------------------------- grouped GEMM ---
// out[r, n] = sum_b isum(r, n, b) * a_scale[src(r), b] * w_scale[e, n, b]
// for the rows r of each row tile (all of one expert e).
//
// Workgroup = 4 waves = one row tile (64 rows) x 4 weight n-tiles (128 output
// columns); wave w owns n-tile 4*ng + w for all 64 rows: two 32x32 tiles
// stacked along M that share the unpacked B operand.
//
// K advances one packed pair (2 blocks, 64 K) per stage through a 4-deep LDS
// ring filled by direct global->LDS loads (no register staging), issued three
// stages ahead: per stage and wave 1 KiB of gathered A rows and the wave's
// 1 KiB of packed Q4 weights.  A's 16-byte chunks are XOR-swizzled within each
// 64-byte row, which makes the MFMA operand reads bank-conflict free.  The block scales
// come in groups of 8 blocks (4 stages) into a double-buffered LDS area, one
// 16-byte load per lane: lanes 0-31 the fp16 scales of the wave's 32 weight
// columns, lanes 32-63 the fp32 A scales of 16 rows (two lanes per row).
//
// Per 32-block the matrix cores do all products: one v_mfma_f32_32x32x1_2b_f32
// gives the scale products a_scale[row] * w_scale[col] of both row halves (one
// rounding each, as a plain fp32 multiply), and per row half one
// v_mfma_i32_32x32x32_i8 gives the exact int32 block sums.  The VALU is left
// with unpacking the nibbles and the convert + fma per element.  The unpack
// places each 4-bit code in the high half of a byte (16x the weight), and the
// fp16 weight scale is divided by 16 in fp32 to match: 16 isum * (a_scale *
// w_scale / 16) is the same real product as isum * a_scale * w_scale, and with
// every nonzero A scale in [2^-98, 2^107] the scale product stays a normal
// number, so its rounding is that of the unscaled one.  The producers of the A
// scales flag any scale outside that range; a launch that sees the flag takes
// the plain unpack (kFold = false) and the exact unscaled arithmetic.  Both row
// halves' integer MFMAs are issued before the first half's convert + fma, so the
// second one runs under that VALU work; a wave stays within 124 VGPRs (four waves
// per SIMD).  A partly filled half converts only the 8-row register groups that
// hold rows of the tile.
//
// Workgroups are numbered so that each XCD (dispatch is round-robin over the
// 8 XCDs) receives a contiguous run of row tiles with all their n-groups: the
// n-groups of a row tile and the row tiles of an expert share that XCD's L2.
// Inside an XCD's run the tiles go in tile order, so an expert's tiles (a full
// one and its partial last one) run together and read its weights once.
constexpr int kGemmThreads = 256;         // 4 waves
constexpr int kRing = 4;                  // LDS stages = stages per scale group
constexpr int kA_OFF = 0;                 // [64 rows][4 chunks of 16 B], chunks swizzled per row
constexpr int kB_OFF = 4096;              // [4 waves][64 lanes][16 B]
constexpr int kStageBytes = 8192;
constexpr int kScaleBytes = 4096;         // [4 waves][ {32 cols x 8 fp16} | {16 rows x 8 fp32} ]
static_assert(kBM == 64, "a tile is one 64-row block of one expert");
static_assert(kRing * 2 == kScaleGroup, "one scale group per pass over the ring");

typedef float v32f __attribute__((ext_vector_type(32)));

__device__ __forceinline__ uint32_t nib_to_i8(uint32_t v)   // 4 offset-binary nibbles -> 4 int8
{
    return (v + 0x78787878u) ^ 0x80808080u;
}
// 8 offset-binary nibbles (code = q + 8) -> two words of 4 int8 each holding 16 * q:
// the code with its top bit flipped is q in 4-bit two's complement, and in the high
// half of a byte it reads as 16 * q.  Three instructions per 8 codes instead of seven.
__device__ __forceinline__ uint32_t nib_hi_i8x16(uint32_t w) { return (w & 0xF0F0F0F0u) ^ 0x80808080u; }
__device__ __forceinline__ uint32_t nib_lo_i8x16(uint32_t w) { return ((w << 4) & 0xF0F0F0F0u) ^ 0x80808080u; }

// B operand of one 32-block: codes of k 0-3 | 4-7 in w0 and 8-11 | 12-15 in w1
// (low | high nibbles).  kFold: the 16x form.
template <bool kFold>
__device__ __forceinline__ v4i unpack_b(uint32_t w0, uint32_t w1)
{
    v4i b;
    if (kFold) {
        b.x = (int)nib_lo_i8x16(w0);
        b.y = (int)nib_hi_i8x16(w0);
        b.z = (int)nib_lo_i8x16(w1);
        b.w = (int)nib_hi_i8x16(w1);
    } else {
        b.x = (int)nib_to_i8(w0 & 0x0F0F0F0Fu);
        b.y = (int)nib_to_i8((w0 >> 4) & 0x0F0F0F0Fu);
        b.z = (int)nib_to_i8(w1 & 0x0F0F0F0Fu);
        b.w = (int)nib_to_i8((w1 >> 4) & 0x0F0F0F0Fu);
    }
    return b;
}

// Direct global->LDS loads: lane i's 16 bytes from g land at LDS wave_base + 16 i.
// Issued as inline asm so the compiler's wait-count bookkeeping does not track
// them: the ring below waits for them explicitly (vmcnt) and never lets the
// compiler drain loads still meant to be in flight.
__device__ __forceinline__ uint32_t lds_addr(const void* p)
{
    return __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p);
}
// lds: wave-uniform LDS byte address of lane 0's destination
__device__ __forceinline__ void g2lds16(const void* g, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(g), "s"(lds) : "memory", "m0");
}

// A tile of a stage: 64 rows x 64 bytes, row-major; 16-byte chunk c of row r
// sits in slot c ^ a_swz(r).  Any 16 consecutive rows (one pass of a 128-bit
// LDS read) then touch 16 distinct 16-byte bank groups, and any 8 consecutive
// rows 8 distinct ones modulo 128 bytes.
__device__ __forceinline__ int a_swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }
__device__ __forceinline__ int a_lds_off(int r, int c) { return r * 64 + ((c ^ a_swz(r)) << 4); }

// Gate/up epilogue: SwiGLU + Q8 of the tile, fused.  Waves 2i and 2i+1 of the
// workgroup hold the gate and up columns of f-block 2*ng + i (n-tiles interleave
// gate and up).  The tile goes through LDS as fp32 [64 rows][kXsStride] (padded
// so the MFMA-layout writes are bank-conflict free); then each 8-lane group
// takes one (row, f-block): h = silu(gate) * up and its Q8 block, the same
// arithmetic as the standalone SwiGLU + Q8 step.  GU and H are written out only
// when asked for (g.out, g.h_out).
constexpr int kXsStride = 136;            // floats per staged row (128 + 8 pad)
constexpr int kXsBytes = kBM * kXsStride * 4;

__device__ __forceinline__ void swiglu_q8_epilogue(const GemmArgs& g, uint8_t* lds,
                                                   const float (&acc0)[16], const float (&acc1)[16],
                                                   int r0, int nrows, int ng, int nt, bool wave_on)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, j32 = lane & 31;
    if (g.out && wave_on) {
        const int col = gu_logical_row(nt, j32, g.gu_f);
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 8 * gq + 4 * h + i;
                if (row < nrows) g.out[(int64_t)(r0 + row) * g.N + col] = acc0[4 * gq + i];
                if (row + 32 < nrows) g.out[(int64_t)(r0 + row + 32) * g.N + col] = acc1[4 * gq + i];
            }
        }
    }
    float* xs = reinterpret_cast<float*>(lds);
    __syncthreads();                                      // every wave is done with the ring
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int row = 8 * (i >> 2) + 4 * h + (i & 3);
        xs[row * kXsStride + wave * 32 + j32] = acc0[i];
        xs[(row + 32) * kXsStride + wave * 32 + j32] = acc1[i];
    }
    __syncthreads();
    const int f = g.gu_f;
#pragma unroll
    for (int it = 0; it < kBM * 16 / kGemmThreads; ++it) {
        const int t = it * kGemmThreads + tid;            // (row, f-block of the pair, 4-column slice)
        const int row = t >> 4, fb = (t >> 3) & 1, sub = t & 7;
        if (row >= nrows) continue;                       // uniform over the 8-lane group
        if ((2 * ng + fb) * 32 >= f) continue;            // f % 64 == 32: the last group holds one f-block
        const float* xr = xs + row * kXsStride + fb * 64 + sub * 4;
        const float4 gv = *reinterpret_cast<const float4*>(xr);
        const float4 uv = *reinterpret_cast<const float4*>(xr + 32);
        float4 hv;
        hv.x = gv.x / (1.0f + exp_cw(-gv.x)) * uv.x;
        hv.y = gv.y / (1.0f + exp_cw(-gv.y)) * uv.y;
        hv.z = gv.z / (1.0f + exp_cw(-gv.z)) * uv.z;
        hv.w = gv.w / (1.0f + exp_cw(-gv.w)) * uv.w;
        const int64_t r = r0 + row;
        const int fblk = 2 * ng + fb;
        if (g.h_out) *reinterpret_cast<float4*>(g.h_out + r * f + fblk * 32 + sub * 4) = hv;
        float d;
        const uint32_t packed = q8_block_of8(hv, &d);
        *reinterpret_cast<uint32_t*>(g.hq + r * f + fblk * 32 + sub * 4) = packed;
        if (sub == 0) {
            g.dh[r * g.dh_stride + fblk] = d;
            if (scale_outside_fold_range(d)) atomicOr(g.h_flag, 1u);
        }
    }
}

// The work item of a workgroup: row tile (expert, first row, rows) and n-group.
struct GemmItem {
    int ng, e, r0, nrows;
};

// XCD x (dispatch is round-robin over the 8 XCDs) takes a contiguous range of row
// tiles with all their n-groups, in tile order.  Inside the range
// the workgroups go by super-groups of kSuperNG n-groups: all the range's tiles of
// n-groups 0-7, then of 8-15, ...  The workgroups an XCD runs at once then share
// each weight slice among many tiles and each tile's activation rows among 8
// n-groups, which keeps more of both in that XCD's L2 than taking each tile's n-groups
// together (tile-major) or each n-group's tiles together (n-group-major).
// False: this workgroup has no item.  Runs before the kernel picks its arithmetic
// path, so the tile-list reads stay scalar loads.
constexpr int kSuperNG = 8;

__device__ __forceinline__ bool gemm_item(const GemmArgs& g, GemmItem& it)
{
    const int NG = ((g.N >> 5) + 3) >> 2;                 // n-groups of 4 n-tiles
    int tile, ng;
    {
        const int nt_all = *g.ntiles;
        const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
        const int tq = nt_all >> 3, tr = nt_all & 7;
        const int ta = xcd * tq + (xcd < tr ? xcd : tr);
        const int tn = tq + (xcd < tr ? 1 : 0);
        if (slot >= tn * NG) return false;                // uniform across the workgroup
        const int full = NG / kSuperNG, per = tn * kSuperNG, sg = slot / per;
        int k;
        if (sg < full) {                                  // a whole super-group
            const int rem = slot - sg * per;
            k = rem / kSuperNG;
            ng = sg * kSuperNG + rem % kSuperNG;
        } else {                                          // the last, partial one
            const int rem = slot - full * per, part = NG - full * kSuperNG;
            k = rem / part;
            ng = full * kSuperNG + rem % part;
        }
        tile = ta + k;                                    // the range's tiles in tile order
    }
    const int te = g.tiles[3 * tile + 0];
    it.ng = ng;
    it.e = te < 0 ? 0 : (te >= g.E ? g.E - 1 : te);      // always valid; a no-op for a sound list
    it.r0 = g.tiles[3 * tile + 1];
    it.nrows = g.tiles[3 * tile + 2] - it.r0;            // 1 .. kBM
    return true;
}

template <bool kGateUp, bool kFold>
__device__ __forceinline__ void grouped_gemm_body(const GemmArgs& g, const GemmItem& it, uint8_t* lds)
{
    const int ng = it.ng, e = it.e, r0 = it.r0, nrows = it.nrows;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int K = g.K, N = g.N;
    const int npairs = k_pairs(K), ngroups = scale_groups(K);
    const bool half_tail = (K & 63) != 0;                 // K % 64 == 32: the last pair holds one block
    const int nt_real = ng * 4 + wave;
    const bool wave_on = nt_real < (N >> 5);
    const int nt = wave_on ? nt_real : (N >> 5) - 1;      // idle waves load valid memory

    uint8_t* const ring = lds;
    uint8_t* const sbuf = lds + kRing * kStageBytes;

    // ---- load sources (all addresses clamped in bounds)
    // A: this wave fills rows 16w..16w+15, lane -> row 16w + lane/4, slot lane%4
    const int8_t* a_src;
    int a_col;
    {
        const int row = 16 * wave + (lane >> 2);
        const int rr = r0 + (row < nrows ? row : nrows - 1);
        const int src = kGateUp ? g.row_src[rr] : rr;
        a_src = g.A + (int64_t)src * K;
        a_col = ((lane & 3) ^ a_swz(row)) * 16;
    }
    const uint8_t* ex = g.blob + (uint64_t)e * g.expert_stride;
    const uint8_t* wq = ex + g.q_off + (uint64_t)nt * npairs * 1024 + lane * 16;
    // scale groups: lanes 0-31 -> fp16 scales of weight column lane (16 B per group),
    // lanes 32-63 -> A scales of row 16w + (lane-32)/2, blocks 4*((lane-32)&1) .. +3
    const uint8_t* sc_src;
    int sc_step;
    if (lane < 32) {
        sc_src = ex + g.s_off + ((uint64_t)nt * ngroups * 32 + lane) * 16;
        sc_step = 32 * 16;
    } else {
        const int row = 16 * wave + ((lane - 32) >> 1);
        const int rr = r0 + (row < nrows ? row : nrows - 1);
        const int src = kGateUp ? g.row_src[rr] : rr;
        sc_src = reinterpret_cast<const uint8_t*>(g.A_scale + (int64_t)src * g.a_scale_stride +
                                                  ((lane - 32) & 1) * 4);
        sc_step = kScaleGroup * 4;
    }

    // stage = packed pair pr, scale group grp (clamped: tail loads repeat the
    // last one, never read)
    const uint32_t lds_wave = lds_addr(lds) + wave * 1024;   // this wave's 1 KiB in each area
    auto issue_stage = [&](int pr, int slot) {
        const int p = pr < npairs ? pr : npairs - 1;
        g2lds16(a_src + p * 64 + a_col, lds_wave + slot * kStageBytes + kA_OFF);
        g2lds16(wq + (uint64_t)p * 1024, lds_wave + slot * kStageBytes + kB_OFF);
    };
    auto issue_scales = [&](int grp, int buf) {
        const int gg = grp < ngroups ? grp : ngroups - 1;
        g2lds16(sc_src + (int64_t)gg * sc_step, lds_wave + kRing * kStageBytes + buf * kScaleBytes);
    };

    float acc0[16], acc1[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        acc0[i] = 0.0f;
        acc1[i] = 0.0f;
    }
    const int h = lane >> 5, j32 = lane & 31;
    const v16i zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    v32f fzero;
#pragma unroll
    for (int i = 0; i < 32; ++i) fzero[i] = 0.0f;
    // A-operand offsets (chunk index depends on the block of the pair: 2*q + h)
    const int a_off0[2] = {a_lds_off(j32, h), a_lds_off(j32, 2 + h)};
    const int a_off1[2] = {a_lds_off(32 + j32, h), a_lds_off(32 + j32, 2 + h)};
    // scale-area offsets: this lane's column scales, and the A scales of row = lane
    const int ws_off = wave * 1024 + j32 * 16;
    const int xs_off = (lane >> 4) * 1024 + 512 + (lane & 15) * 32;
    const int xs_off1h = (j32 >> 4) * 1024 + 512 + (j32 & 15) * 32;   // row j32, for one row half

    // acc[i] += (float)is[i] * t[off + i] for the register groups that hold tile rows: element
    // i of a lane is row 8*(i/4) + 4*h + i%4 of its half, so group g = i/4 covers rows
    // 8g .. 8g+7 (the first kG groups; kG = 0: the first G, known only at run time)
    auto fma_groups = [&](auto full_c, float(&acc)[16], const v16i& is, const v32f& t, int off, int G) {
        constexpr int kG = decltype(full_c)::value;     // groups fixed at compile time (0: G)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            if (kG ? g < kG : g < G) {
#pragma unroll
                for (int i = 4 * g; i < 4 * g + 4; ++i) acc[i] = __builtin_fmaf((float)is[i], t[off + i], acc[i]);
            }
        }
    };
    // one stage (U = position in the scale group): wait for its loads, sync,
    // queue the stage three ahead into the slot freed by the previous stage
    // (and, at a group start, the next group's scales), then two blocks of
    // MFMA + epilogue
    auto stage = [&](auto two_c, auto full_c, auto u_c, int s, int G) {
        constexpr bool kTwo = decltype(two_c)::value;
        constexpr int U = decltype(u_c)::value;
        // loads issued after this stage's: two per later stage in flight, plus the
        // scale load issued at the start of a group if that came after them
        constexpr int kLater = 2 * (kRing - 2) + ((U == 1 || U == 2) ? 1 : 0);
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" :: "n"(kLater) : "memory");
        const int grp = s >> 2;
        if (U == 0) issue_scales(grp + 1, (grp + 1) & 1);
        issue_stage(s + kRing - 1, (U + kRing - 1) % kRing);
        if (!wave_on) return;
        const bool one_block = half_tail && s == npairs - 1;   // skip the padded second block
        const uint8_t* sb = ring + U * kStageBytes;
        const uint8_t* sc = sbuf + (grp & 1) * kScaleBytes;
        const uint4 bq = *reinterpret_cast<const uint4*>(sb + kB_OFF + wave * 1024 + lane * 16);
        if (!kTwo) {
            // one row half: a single scale MFMA serves both blocks of the stage (lanes
            // 0-31 carry block 0's scales, lanes 32-63 block 1's, rows 0-31 either way):
            // t[i] = block 0 products, t[16 + i] = block 1 products
            const uint16_t hb = *reinterpret_cast<const uint16_t*>(sc + ws_off + U * 4 + h * 2);
            const float dw = (float)__builtin_bit_cast(_Float16, hb) * (kFold ? 0.0625f : 1.0f);
            const float dxv = *reinterpret_cast<const float*>(sc + xs_off1h + U * 8 + h * 4);
            const v32f t = __builtin_amdgcn_mfma_f32_32x32x1f32(dxv, dw, fzero, 0, 0, 0);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                if (q == 1 && one_block) break;
                const uint32_t w0 = q ? bq.z : bq.x;
                const uint32_t w1 = q ? bq.w : bq.y;
                const v4i bop = unpack_b<kFold>(w0, w1);
                const v4i a0 = *reinterpret_cast<const v4i*>(sb + kA_OFF + a_off0[q]);
                const v16i is0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, bop, zero, 0, 0, 0);
                fma_groups(std::integral_constant<int, 0>{}, acc0, is0, t, 16 * q, G);
                __builtin_amdgcn_sched_barrier(0);
            }
            return;
        }
        const uint32_t bs = *reinterpret_cast<const uint32_t*>(sc + ws_off + U * 4);
        const float2 dx = *reinterpret_cast<const float2*>(sc + xs_off + (U >> 1) * 16 + (U & 1) * 8);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            if (q == 1 && one_block) break;
            const uint32_t w0 = q ? bq.z : bq.x;
            const uint32_t w1 = q ? bq.w : bq.y;
            const v4i bop = unpack_b<kFold>(w0, w1);
            const uint16_t hb = (uint16_t)(q ? (bs >> 16) : (bs & 0xffffu));
            const float dw = (float)__builtin_bit_cast(_Float16, hb) * (kFold ? 0.0625f : 1.0f);
            // t[16*half + i] = a_scale(row of D element i in that half) * w_scale(col)
            const v32f t = __builtin_amdgcn_mfma_f32_32x32x1f32(q ? dx.y : dx.x, dw, fzero, 0, 0, 0);
            const v4i a0 = *reinterpret_cast<const v4i*>(sb + kA_OFF + a_off0[q]);
            v16i is0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, bop, zero, 0, 0, 0);
            if (kTwo) {
                const v4i a1 = *reinterpret_cast<const v4i*>(sb + kA_OFF + a_off1[q]);
                const v16i is1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, bop, zero, 0, 0, 0);
                // empty: orders the second MFMA before the first half's VALU work
                asm volatile("" : "+v"(is0) : "v"(is1));
                fma_groups(std::integral_constant<int, 4>{}, acc0, is0, t, 0, G);
                fma_groups(full_c, acc1, is1, t, 16, G);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // the partly filled row half (the second of two, or the only one) runs only the 8-row
    // register groups that hold rows of the tile
    auto run = [&](auto two_c, auto full_c) {
        constexpr bool kTwo = decltype(two_c)::value;
        const int G = ((kTwo ? nrows - 32 : nrows) + 7) >> 3;
        issue_scales(0, 0);
#pragma unroll
        for (int u = 0; u < kRing - 1; ++u) issue_stage(u, u);
        for (int s0 = 0; s0 < npairs; s0 += kRing) {
            stage(two_c, full_c, std::integral_constant<int, 0>{}, s0, G);
            if (s0 + 1 < npairs) stage(two_c, full_c, std::integral_constant<int, 1>{}, s0 + 1, G);
            if (s0 + 2 < npairs) stage(two_c, full_c, std::integral_constant<int, 2>{}, s0 + 2, G);
            if (s0 + 3 < npairs) stage(two_c, full_c, std::integral_constant<int, 3>{}, s0 + 3, G);
        }
    };
    if (!kFold) {                     // the rare exact path: two variants keep the code small
        if (nrows > 32)
            run(std::true_type{}, std::integral_constant<int, 4>{});
        else
            run(std::false_type{}, std::integral_constant<int, 0>{});
    } else if (nrows > 56)
        run(std::true_type{}, std::integral_constant<int, 4>{});
    else if (nrows > 48)
        run(std::true_type{}, std::integral_constant<int, 3>{});
    else if (nrows > 40)
        run(std::true_type{}, std::integral_constant<int, 2>{});
    else if (nrows > 32)
        run(std::true_type{}, std::integral_constant<int, 1>{});
    else
        run(std::false_type{}, std::integral_constant<int, 0>{});
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // drain the clamped tail loads before exit

    if (kGateUp) {
        swiglu_q8_epilogue(g, lds, acc0, acc1, r0, nrows, ng, nt, wave_on);
        return;
    }
    if (!wave_on) return;
    const int col = nt * 32 + j32;
    if (g.y_add) {                        // atomic combine: y[token] += w * row, no Dm
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 8 * gq + 4 * h + i;
                if (row < nrows) {
                    const int r = r0 + row;
                    atomicAdd(g.y_add + (int64_t)g.rtok[r] * N + col, g.wts[g.rows[r]] * acc0[4 * gq + i]);
                }
                if (row + 32 < nrows) {
                    const int r = r0 + row + 32;
                    atomicAdd(g.y_add + (int64_t)g.rtok[r] * N + col, g.wts[g.rows[r]] * acc1[4 * gq + i]);
                }
            }
        }
        return;
    }
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 8 * gq + 4 * h + i;
            if (row < nrows) g.out[(int64_t)(r0 + row) * N + col] = acc0[4 * gq + i];
            if (row + 32 < nrows) g.out[(int64_t)(r0 + row + 32) * N + col] = acc1[4 * gq + i];
        }
    }
}

// gate/up projection: A rows gathered from Xq through the row table, output
// columns in logical gate | up order.
constexpr int kGemmLdsRing = kRing * kStageBytes + 2 * kScaleBytes;
constexpr int kGemmLds = kGemmLdsRing > kXsBytes ? kGemmLdsRing : kXsBytes;   // 40 KiB: four workgroups per CU

// The launch reads the scale flag once and runs one of the two instantiations; the
// LDS is declared here, once, so both share it (a __shared__ array inside the
// template would be allocated per instantiation).
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_gemm_gate_up(GemmArgs g)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[kGemmLds];
    GemmItem it;
    if (!gemm_item(g, it)) return;
    if (*g.fold_flag == 0)
        grouped_gemm_body<true, true>(g, it, lds);
    else
        grouped_gemm_body<true, false>(g, it, lds);
}
// down projection: A = Hq in row-table order.
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_gemm_down(GemmArgs g)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[kGemmLds];
    GemmItem it;
    if (!gemm_item(g, it)) return;
    if (*g.fold_flag == 0)
        grouped_gemm_body<false, true>(g, it, lds);
    else
        grouped_gemm_body<false, false>(g, it, lds);
}

// -------------------------------------------------------------- combine ---
// y[t, :] = sum_j w[t, j] * dm[pos[t*k + j], :], j ascending, fma chain from 0.
// Also clears the membership mask and the scale flags for the next layer (dead here).
// Dm is read once and y written once: both go past the caches (non-temporal), which
// keeps the stream from evicting lines other work still uses (about 10% faster at
// 1.2 GB per launch).
typedef float v4f __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ dm,
                                                 const float* __restrict__ wts,
                                                 const int32_t* __restrict__ pos, int T, int k, int d,
                                                 float* __restrict__ y, uint32_t* __restrict__ mask,
                                                 int64_t mask_words)
{
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t nthreads = (int64_t)gridDim.x * 256;
    for (int64_t i = gid; i < mask_words; i += nthreads) mask[i] = 0u;
    const int d4 = d >> 2;
    if (gid >= (int64_t)T * d4) return;
    const int t = (int)(gid / d4);
    const int c = (int)(gid - (int64_t)t * d4) * 4;
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int j = 0; j < k; ++j) {
        const int r = pos[(int64_t)t * k + j];
        const float wt = wts[(int64_t)t * k + j];
        const v4f v = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(dm + (int64_t)r * d + c));
        acc.x = __builtin_fmaf(wt, v.x, acc.x);
        acc.y = __builtin_fmaf(wt, v.y, acc.y);
        acc.z = __builtin_fmaf(wt, v.z, acc.z);
        acc.w = __builtin_fmaf(wt, v.w, acc.w);
    }
    __builtin_nontemporal_store(acc, reinterpret_cast<v4f*>(y + (int64_t)t * d + c));
}

__global__ __launch_bounds__(256) void k_fill_u32(uint32_t* __restrict__ p, int64_t n, uint32_t v)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = v;
}

// ---------------------------------------------------------- exp check ---
// out[i] = exp_cw(the fp32 number with bit pattern first + i): lets a caller
// compare the kernels' exponential with an independent one input by input.
__global__ __launch_bounds__(256) void k_exp_range(uint32_t first, uint64_t n, float* __restrict__ out)
{
    const uint64_t stride = (uint64_t)gridDim.x * 256;
    for (uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride)
        out[i] = exp_cw(__builtin_bit_cast(float, (uint32_t)(first + i)));
}

hipError_t launch_exp_range(uint32_t first, uint64_t n, float* out, hipStream_t st)
{
    if (n == 0) return hipSuccess;
    const uint64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(k_exp_range, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, st, first, n,
                       out);
    return hipGetLastError();
}

void exp_range_host(uint32_t first, uint64_t n, float* out)
{
    for (uint64_t i = 0; i < n; ++i) out[i] = exp_cw(__builtin_bit_cast(float, (uint32_t)(first + i)));
}

// ------------------------------------------------------- static scratch ---
// Workspace of the allocation-free layer entry point: one array per device, held
// until the process ends.  In host code `scratch` names a host-side stand-in, not
// device memory: its device address comes from hipGetSymbolAddress, once per device
// with that device current, and only that address is ever handed to a kernel or a
// copy.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kScratchMaxDevices = 64;
static std::mutex g_scratch_mu;
static uint8_t* g_scratch_ptr[kScratchMaxDevices] = {};

hipError_t scratch_device_ptr(int dev, uint8_t** out)
{
    *out = nullptr;
    if (dev < 0 || dev >= kScratchMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;                                   // the caller made `dev` current
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = static_cast<uint8_t*>(p);
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

// ------------------------------------------------------------- launches ---
static inline unsigned nblk(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

static inline void mark(const LayerLaunch& L, int i, hipStream_t st)
{
    if (L.marks) (void)hipEventRecord(L.marks[i], st);
}

hipError_t launch_layer(const LayerLaunch& L, hipStream_t st)
{
    const int64_t R = (int64_t)L.T * L.k;
    const int n_route = L.E <= kRankMaxE ? L.T : (int)nblk(L.T, 4);   // routing workgroups
    const int64_t xblocks = (int64_t)L.T * (L.d / 32);
    mark(L, kRouteQuant, st);
    hipLaunchKernelGGL(k_route_quant, dim3(n_route + nblk(xblocks, 4 * kQuantBlocksPerWave)), dim3(256), 0, st,
                       L.logits, L.T, L.E, L.k, L.eidx, L.wts, L.mask, L.W, n_route, L.x, xblocks,
                       L.d / 32, scale_stride(L.d), L.xq, L.dx, L.mask + (int64_t)L.E * L.W);
    mark(L, kGroup, st);
    hipLaunchKernelGGL(k_group, dim3(L.E), dim3(kGroupThreads), 0, st, L.mask, L.W, L.wprefix,
                       L.counts);
    mark(L, kExpertLoad, st);
    if (L.load_src)
        hipLaunchKernelGGL(k_expert_load, dim3(512), dim3(256), 0, st, L.load_src, L.load_dst, L.counts,
                           L.E, L.expert_stride, L.load_stats);
    mark(L, kScatter, st);
    hipLaunchKernelGGL(k_scatter, dim3(nblk(R, 256)), dim3(256), 0, st, L.eidx, R, L.k, L.mask,
                       L.wprefix, L.counts, L.E, L.W, L.bounds, L.tiles, L.ntiles, L.rows, L.pos,
                       L.rtok);
    const int max_tiles_now = (int)((R + kBM - 1) / kBM) + (L.E < R ? L.E : (int)R);

    GemmArgs gu = {};
    gu.A = L.xq;
    gu.A_scale = L.dx;
    gu.a_scale_stride = scale_stride(L.d);
    gu.row_src = L.rtok;
    gu.blob = L.blob;
    gu.expert_stride = L.expert_stride;
    gu.q_off = L.gu_q_off;
    gu.s_off = L.gu_s_off;
    gu.tiles = L.tiles;
    gu.ntiles = L.ntiles;
    gu.out = L.gu;
    gu.hq = L.hq;
    gu.dh = L.dh;
    gu.dh_stride = scale_stride(L.f);
    gu.h_out = L.h_out;
    gu.N = 2 * L.f;
    gu.K = L.d;
    gu.E = L.E;
    gu.gu_f = L.f;
    gu.fold_flag = L.mask + (int64_t)L.E * L.W;           // X scales (set by k_route_quant)
    gu.h_flag = L.mask + (int64_t)L.E * L.W + 1;           // H scales (set by this launch)
    mark(L, kGemmGateUp, st);
    const unsigned tiles8 = 8 * nblk(max_tiles_now, 8);   // every XCD's tile range, rounded up
    hipLaunchKernelGGL(k_gemm_gate_up, dim3(nblk(gu.N / 32, 4) * tiles8), dim3(kGemmThreads), 0, st, gu);

    GemmArgs dn = gu;
    dn.A = L.hq;
    dn.A_scale = L.dh;
    dn.a_scale_stride = scale_stride(L.f);
    dn.row_src = nullptr;
    dn.q_off = L.d_q_off;
    dn.s_off = L.d_s_off;
    dn.out = L.combine_atomic ? nullptr : L.dm;
    dn.y_add = L.combine_atomic ? L.y : nullptr;
    dn.rows = L.rows;
    dn.rtok = L.rtok;
    dn.wts = L.wts;
    dn.hq = nullptr;
    dn.dh = nullptr;
    dn.h_out = nullptr;
    dn.N = L.d;
    dn.K = L.f;
    dn.gu_f = 0;
    dn.fold_flag = gu.h_flag;
    dn.h_flag = nullptr;
    mark(L, kGemmDown, st);
    if (L.combine_atomic) {               // the atomic combine adds into a zeroed y
        const hipError_t e = launch_fill_u32(reinterpret_cast<uint32_t*>(L.y), (int64_t)L.T * L.d, 0u, st);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_gemm_down, dim3(nblk(dn.N / 32, 4) * tiles8), dim3(kGemmThreads), 0, st, dn);
    mark(L, kCombine, st);
    return hipGetLastError();
}

hipError_t launch_combine(const LayerLaunch& L, hipStream_t st)
{
    const int64_t work = (int64_t)L.T * (L.d / 4);
    const int64_t mw = (int64_t)mask_words(L.E, L.W);    // the mask and the scale flags
    if (L.combine_atomic) {               // y is complete: only clear the grouping state
        const hipError_t e = launch_fill_u32(L.mask, mw, 0u, st);
        mark(L, kNumKernels, st);
        return e;
    }
    hipLaunchKernelGGL(k_combine, dim3(nblk(work > mw ? work : mw, 256)), dim3(256), 0, st, L.dm,
                       L.wts, L.pos, L.T, L.k, L.d, L.y, L.mask, mw);
    mark(L, kNumKernels, st);
    return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t st)
{
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_u32, dim3(nblk(n, 256)), dim3(256), 0, st, p, n, v);
    return hipGetLastError();
}

}  // namespace moe
