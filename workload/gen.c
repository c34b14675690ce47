/*
 * Seeded synthetic inputs for the MoE prompt (prefill) FFN layer.
 *
 * This module only draws numbers.  It holds none of the layer's arithmetic
 * (no routing, quantisation, GEMM or combine): both the GPU path and the CPU
 * oracle take what it writes as *input*.
 *
 * Generator: SplitMix64 used as a counter-based generator (G. Steele, D. Lea,
 * C. Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014):
 * element i of a stream with key K is mix64(K + (i + 1) * GAMMA), so any element
 * can be produced on its own and in parallel.  A stream key is derived from
 * (seed, tensor id, expert) by chained mix64 calls.
 *
 * Normals: Box-Muller (G. E. P. Box, M. E. Muller, 1958), cosine branch only,
 * evaluated in double and rounded once to fp32.
 *
 * Workload shapes and distributions follow the prompt-path pages' layer:
 * activations and router logits N(0,1) fp32; expert weights as 4-bit integers
 * uniform in [-8, 7] with one fp16 scale per 32 weights along the input
 * dimension, scale ~ U(0.5, 1.5) / sqrt(d_in).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t gen_stream_key(uint64_t seed, uint64_t tensor, uint64_t expert)
{
    uint64_t k = mix64(seed + GAMMA);
    k = mix64(k ^ ((tensor + 1) * GAMMA));
    k = mix64(k ^ ((expert + 1) * GAMMA));
    return k;
}

static inline uint64_t draw(uint64_t key, uint64_t i)
{
    return mix64(key + (i + 1) * GAMMA);
}

/* Raw 64-bit draws (exposed so tests can pin the stream). */
void gen_u64(uint64_t key, uint64_t first, int64_t n, uint64_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = draw(key, first + (uint64_t)i);
}

/* N(0,1) fp32: element i uses draws 2i and 2i+1. */
void gen_normal_f32(uint64_t key, int64_t n, float mean, float std, float* out)
{
    const double two_pi = 6.283185307179586476925286766559;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        double u1 = ((double)(draw(key, 2 * (uint64_t)i) >> 11) + 1.0) * 0x1.0p-53; /* (0,1] */
        double u2 = (double)(draw(key, 2 * (uint64_t)i + 1) >> 11) * 0x1.0p-53;     /* [0,1) */
        double z = sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
        out[i] = (float)((double)mean + (double)std * z);
    }
}

/* 4-bit integers uniform in [-8, 7]: element i is nibble (i % 16) of draw i / 16. */
void gen_int4(uint64_t key, int64_t n, int8_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < (n + 15) / 16; ++c) {
        uint64_t u = draw(key, (uint64_t)c);
        int64_t base = c * 16;
        for (int j = 0; j < 16 && base + j < n; ++j)
            out[base + j] = (int8_t)((int)((u >> (4 * j)) & 15u) - 8);
    }
}

/* fp32 -> IEEE binary16 bits, round to nearest even (inputs here are normal
 * positive values well inside the half range, but the conversion is general). */
static uint16_t f32_to_f16_bits(float f)
{
    uint32_t x;
    memcpy(&x, &f, 4);
    uint32_t sign = (x >> 16) & 0x8000u;
    uint32_t ex = (x >> 23) & 0xFFu;
    uint32_t man = x & 0x7FFFFFu;
    if (ex == 0xFFu) return (uint16_t)(sign | 0x7C00u | (man ? 0x200u : 0u));
    int e = (int)ex - 127 + 15;
    if (e >= 31) return (uint16_t)(sign | 0x7C00u);
    if (e <= 0) {
        if (e < -10) return (uint16_t)sign;
        man |= 0x800000u;
        int shift = 14 - e;
        uint32_t h = man >> shift;
        uint32_t rem = man & ((1u << shift) - 1u);
        uint32_t half = 1u << (shift - 1);
        if (rem > half || (rem == half && (h & 1u))) h++;
        return (uint16_t)(sign | h);
    }
    uint32_t h = ((uint32_t)e << 10) | (man >> 13);
    uint32_t rem = man & 0x1FFFu;
    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h++;
    return (uint16_t)(sign | h);
}

/* Block scales: fp16(RNE) of fp32((0.5 + U) / sqrt(d_in)), U = top 24 bits of draw i. */
void gen_scale_f16(uint64_t key, int64_t n, int d_in, uint16_t* out)
{
    const double inv = 1.0 / sqrt((double)d_in);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        double u = (double)(draw(key, (uint64_t)i) >> 40) * 0x1.0p-24;
        out[i] = f32_to_f16_bits((float)((0.5 + u) * inv));
    }
}

/* A seeded permutation of 1..n (Fisher-Yates driven by the stream). */
void gen_rank_perm(uint64_t key, int n, int32_t* rank)
{
    for (int i = 0; i < n; ++i) rank[i] = i + 1;
    for (int i = n - 1; i > 0; --i) {
        uint64_t j = draw(key, (uint64_t)i) % (uint64_t)(i + 1);
        int32_t t = rank[i];
        rank[i] = rank[j];
        rank[j] = t;
    }
}

/* logits[t][e] += bias[e], in fp32, one rounding per element. */
void gen_add_bias(int64_t T, int E, const float* bias, float* logits)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int e = 0; e < E; ++e) logits[t * E + e] = logits[t * E + e] + bias[e];
}
