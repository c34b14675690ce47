// Host-side packing of one expert's canonical Q4 weights into the tiled blob
// layout read by the grouped GEMM (layout described in moe_layout.h).
#include <string.h>

#include "moe_layout.h"

namespace moe {

// W [N, K] int8 in [-8, 7], S [N, K/32] fp16 bits -> quant and scale sections
// (K a multiple of 32; with K % 64 == 32 the last K pair holds one block and zero codes).
// interleave_f > 0: W is the gate/up matrix with f = interleave_f (blob n-tile
// 2i = gate rows 32i.., 2i+1 = up rows f + 32i..).
static bool pack_matrix(int N, int K, const int8_t* W, const uint16_t* S, int interleave_f,
                        uint8_t* q_dst, uint8_t* s_dst)
{
    const int npairs = k_pairs(K), nbk = K / 32, ngroups = scale_groups(K);
    for (int64_t i = 0; i < (int64_t)N * K; ++i)
        if (W[i] < -8 || W[i] > 7) return false;
    for (int nt = 0; nt < N / 32; ++nt) {
        for (int pr = 0; pr < npairs; ++pr) {
            uint8_t* qt = q_dst + ((int64_t)nt * npairs + pr) * 64 * 16;
            for (int lane = 0; lane < 64; ++lane) {
                const int j = lane & 31, h = lane >> 5;
                const int n = interleave_f ? gu_logical_row(nt, j, interleave_f) : nt * 32 + j;
                const int8_t* wr = W + (int64_t)n * K;
                uint8_t* out = qt + lane * 16;
                for (int q = 0; q < 2; ++q) {
                    const int k0 = 32 * (2 * pr + q) + 16 * h;
                    if (k0 >= K) {                    // the second block of a half pair: weight 0
                        memset(out + 8 * q, 0x88, 8);
                        continue;
                    }
                    for (int i = 0; i < 4; ++i) {
                        out[8 * q + i] = (uint8_t)((wr[k0 + i] + 8) | ((wr[k0 + 4 + i] + 8) << 4));
                        out[8 * q + 4 + i] = (uint8_t)((wr[k0 + 8 + i] + 8) | ((wr[k0 + 12 + i] + 8) << 4));
                    }
                }
            }
        }
        for (int g = 0; g < ngroups; ++g) {
            uint16_t* st = reinterpret_cast<uint16_t*>(s_dst) + ((int64_t)nt * ngroups + g) * 32 * kScaleGroup;
            for (int j = 0; j < 32; ++j) {
                const int n = interleave_f ? gu_logical_row(nt, j, interleave_f) : nt * 32 + j;
                for (int b = 0; b < kScaleGroup; ++b) {
                    const int blk = g * kScaleGroup + b;
                    st[j * kScaleGroup + b] = blk < nbk ? S[(int64_t)n * nbk + blk] : (uint16_t)0;
                }
            }
        }
    }
    return true;
}

bool pack_expert(int d, int f, const int8_t* wgu_q, const uint16_t* wgu_s, const int8_t* wd_q,
                 const uint16_t* wd_s, uint8_t* dst)
{
    const BlobLayout L = blob_layout(d, f);
    memset(dst, 0, L.expert_bytes);
    if (!pack_matrix(2 * f, d, wgu_q, wgu_s, f, dst + L.gu_q, dst + L.gu_s)) return false;
    if (!pack_matrix(d, f, wd_q, wd_s, 0, dst + L.d_q, dst + L.d_s)) return false;
    return true;
}

}  // namespace moe
