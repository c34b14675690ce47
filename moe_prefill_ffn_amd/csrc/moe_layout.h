// Internal layouts of the MoE prefill library: the packed expert blob and the
// per-handle workspace.  Host and device code both include this file.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define MOE_HD __host__ __device__
#else
#define MOE_HD
#endif

namespace moe {

constexpr int kBM = 64;          // rows (routed token slots) per GEMM tile
constexpr int kQBlock = 32;      // Q4 / Q8 block length along K

MOE_HD static inline uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

// ------------------------------------------------------------ expert blob ---
//
// One expert = [ W_gu quants | W_gu scales | W_d quants | W_d scales ], each
// section 256-byte aligned.  A matrix W [N, K] (N output rows, K input) is
// stored in tiles of 32 output rows ("n-tiles") by pairs of K-blocks (64 K):
//
//   quants: for nt < N/32, pr < ceil(K/64), lane < 64: 16 bytes at
//           ((nt * ceil(K/64) + pr) * 64 + lane) * 16 (K % 64 == 32: the second
//           block of the last pair holds code 8, i.e. weight 0)
//     lane = h * 32 + j  (j: row inside the n-tile, h: which 16-K half of a block)
//     bytes 8q .. 8q+7 hold block b = 2 pr + q, K range [32 b + 16 h, +16):
//       byte i   (i < 4): low nibble K+i,    high nibble K+4+i
//       byte 4+i (i < 4): low nibble K+8+i,  high nibble K+12+i
//     nibble = w + 8  (w in [-8, 7] stored offset-binary)
//   scales: in groups of kScaleGroup = 8 K-blocks (the last group zero-padded):
//           for nt < N/32, g < ceil(K/256), j < 32: 16 bytes at
//           ((nt * ceil(K/256) + g) * 32 + j) * 16 = fp16 scales of blocks
//           8g .. 8g+7 of row nt*32 + j.
//
// One wave-wide 16-byte load per (n-tile, K pair) therefore hands every lane
// exactly its B-operand bytes for two 32x32x32 int8 MFMAs, and one 512-byte load
// (lanes 0-31) the n-tile's scales for eight blocks.
//
// W_gu's n-tiles interleave gate and up: n-tile 2i holds gate rows
// [32 i, 32 i + 32), n-tile 2i+1 holds up rows [f + 32 i, f + 32 i + 32).
struct BlobLayout {
    uint64_t gu_q, gu_s, d_q, d_s;   // section offsets inside one expert
    uint64_t expert_bytes;
};

constexpr int kScaleGroup = 8;   // K-blocks per scale group

// K pairs (64 K each) of a K extent; with K % 64 == 32 the last pair holds one block
MOE_HD static inline int k_pairs(int K) { return (K + 63) / 64; }

// scale groups of a K extent, and the padded per-row stride (in blocks) of the
// activation block-scale arrays the GEMMs read a whole group at a time from
MOE_HD static inline int scale_groups(int K) { return (K / 32 + kScaleGroup - 1) / kScaleGroup; }
MOE_HD static inline int scale_stride(int K) { return scale_groups(K) * kScaleGroup; }

static inline BlobLayout blob_layout(int d, int f)
{
    BlobLayout L;
    uint64_t n_gu_q = (uint64_t)2 * f * k_pairs(d) * 32;
    uint64_t n_gu_s = (uint64_t)2 * f * scale_stride(d) * 2;
    uint64_t n_d_q = (uint64_t)d * k_pairs(f) * 32;
    uint64_t n_d_s = (uint64_t)d * scale_stride(f) * 2;
    L.gu_q = 0;
    L.gu_s = L.gu_q + align_up(n_gu_q, 256);
    L.d_q = L.gu_s + align_up(n_gu_s, 256);
    L.d_s = L.d_q + align_up(n_d_q, 256);
    L.expert_bytes = L.d_s + align_up(n_d_s, 256);
    return L;
}

// Logical output column of row j (< 32) of blob n-tile nt for W_gu (interleaved).
MOE_HD static inline int gu_logical_row(int nt, int j, int f)
{
    return ((nt & 1) ? f : 0) + (nt >> 1) * 32 + j;
}

// -------------------------------------------------------------- workspace ---
// The membership mask [E][W] is followed by kScaleFlagWords words: flag 0 is set
// when an X block scale, flag 1 when an H block scale, is zero-free and outside
// [2^-98, 2^107] (see the grouped GEMM).  Both are cleared with the mask.
constexpr int kScaleFlagWords = 2;
MOE_HD static inline uint64_t mask_words(int E, int W) { return (uint64_t)E * W + kScaleFlagWords; }

struct WsLayout {
    uint64_t eidx, wts, mask, wprefix, counts, bounds, tiles, ntiles, load_stats;
    uint64_t rows, pos, rtok, xq, dx, hq, dh, dm;
    uint64_t total;
    int W;            // 32-token words per expert in the membership mask
    int max_tiles;    // upper bound on GEMM row tiles
};

static inline WsLayout ws_layout(int d, int f, int E, int k, int Tmax)
{
    WsLayout L;
    const uint64_t R = (uint64_t)Tmax * k;
    L.W = (Tmax + 31) / 32;
    L.max_tiles = (int)((R + kBM - 1) / kBM) + (E < (int)R ? E : (int)R);
    uint64_t o = 0;
    auto take = [&](uint64_t bytes) { uint64_t at = o; o = align_up(o + bytes, 256); return at; };
    L.eidx = take(R * 4);
    L.wts = take(R * 4);
    L.mask = take(mask_words(E, L.W) * 4);
    L.wprefix = take((uint64_t)E * L.W * 4);
    L.counts = take((uint64_t)E * 4);
    L.bounds = take((uint64_t)(E + 1) * 4);
    L.tiles = take((uint64_t)L.max_tiles * 3 * 4);
    L.ntiles = take(4);
    L.load_stats = take(16);                              // experts, bytes of active-expert loads
    L.rows = take(R * 4);
    L.pos = take(R * 4);
    L.rtok = take(R * 4);
    L.xq = take((uint64_t)Tmax * d + 64);                // + 64: a half last K pair reads past a row
    L.dx = take((uint64_t)Tmax * scale_stride(d) * 4);   // [Tmax][scale_stride(d)]
    L.hq = take(R * f + 64);
    L.dh = take(R * scale_stride(f) * 4);                 // [R][scale_stride(f)]
    L.dm = take(R * d * 4);
    L.total = o;
    return L;
}

}  // namespace moe
