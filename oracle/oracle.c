/*
 * CPU ORACLE for the MoE prompt (prefill) FFN layer -- TEST INFRASTRUCTURE.
 *
 * Only the tests, the package's smoke check and the benchmark's CPU-baseline
 * leg may load or call this file.  The product path never does; it shares no
 * code, header, table or constant with it.
 *
 * What is computed (page "prefill: a layer split's idle card streams a share of
 * a one-chunk prompt's experts", Strata #663, section "What"): the prompt path
 * turns the mixed activations into Xq, runs the gate/up expert GEMM into GU,
 * SwiGLU into H, requantises H into Hq, runs the down GEMM into Dm, and combines
 * the expert rows back into token rows; tokens reach experts through a row
 * table with per-expert group bounds.  The page names these buffers but never
 * writes the arithmetic out; the readings taken here are:
 *
 *   route    top-k over the E router logits, ties to the lower expert index;
 *            weights = softmax over the k selected logits (fp64 here).
 *   group    counts, exclusive-scan bounds, row table stable in p = t*k + j.
 *   Q8       blocks of 32: scale = amax / 127 in fp32, q = round-half-even
 *            (x / scale) in fp32, clamped to [-127, 127]; scale 0 -> q 0.
 *   GEMM     Q4 weights (int4 in [-8,7], fp16 scale per 32 along K); per block
 *            an exact int32 dot; GU combines the blocks in fp32 in ascending
 *            block order with one fused multiply-add per block,
 *            acc = fma((float)isum, a_scale * w_scale, acc), because GU decides
 *            the integer codes of Hq and both sides must take that decision in
 *            the same precision.  Dm is evaluated in fp64 (plain definition).
 *   SwiGLU   H = silu(gate) * up with silu(g) = g / (1 + exp(-g)), in fp32,
 *            exp from oracle_exp_ref (Cody-Waite reduction + Taylor, below).
 *   combine  Y[t] = sum_j w[t,j] * Dm[pos(t,j)], fp64.
 *
 * Every loop is plain; OpenMP only splits independent rows across threads.
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp (no FTZ, no
 * contraction, correctly rounded fp32 division).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ---------------------------------------------------------------- fp16 --- */

/* IEEE binary16 bits -> value, written out from the format definition. */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1F;
    int man = h & 0x3FF;
    double v;
    if (ex == 0)
        v = ldexp((double)man, -24);                 /* subnormal: man * 2^-24 */
    else if (ex == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + man), ex - 25);    /* (1 + man/1024) * 2^(ex-15) */
    return sign ? -v : v;
}

void oracle_f16_to_f64_array(int64_t n, const uint16_t* h, double* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_to_f64(h[i]);
}

/* ---------------------------------------------------------------- exp ---- */

/*
 * exp_ref: fp32 exponential by Cody-Waite argument reduction (W. J. Cody,
 * W. Waite, "Software Manual for the Elementary Functions", 1980) and a
 * degree-7 Taylor polynomial in Horner form.  Every step is one IEEE fp32
 * operation, so any IEEE implementation of the same steps gives the same bits:
 *
 *   NaN -> NaN;  x > 89 -> +inf;  x < -104 -> +0
 *   n  = rint(x * LOG2E)                       (fp32 multiply, ties to even)
 *   r  = fma(-n, LN2_HI, x);  r = fma(-n, LN2_LO, r)
 *   p  = c7; p = fma(p, r, c_j) for j = 6..0   (c_j = 1/j! rounded to fp32)
 *   n1 = trunc(n / 2), n2 = n - n1;  result = (p * 2^n1) * 2^n2
 *
 * LOG2E = fp32(log2 e), LN2_HI = fp32(ln 2), LN2_LO = fp32(ln 2 - LN2_HI).
 */
static float pow2i(int n) /* 2^n for n in [-126, 127] */
{
    uint32_t b = (uint32_t)(n + 127) << 23;
    float f;
    memcpy(&f, &b, 4);
    return f;
}

float oracle_exp_ref(float x)
{
    const float LOG2E = 0x1.715476p+0f;
    const float LN2_HI = 0x1.62e430p-1f;
    const float LN2_LO = -0x1.05c610p-29f;
    const float c0 = 1.0f, c1 = 1.0f, c2 = 0.5f;
    const float c3 = 0x1.555556p-3f;   /* 1/6    */
    const float c4 = 0x1.555556p-5f;   /* 1/24   */
    const float c5 = 0x1.111112p-7f;   /* 1/120  */
    const float c6 = 0x1.6c16c2p-10f;  /* 1/720  */
    const float c7 = 0x1.a01a02p-13f;  /* 1/5040 */
    if (x != x) return x;
    if (x > 89.0f) return INFINITY;
    if (x < -104.0f) return 0.0f;
    float n = rintf(x * LOG2E);
    float r = fmaf(-n, LN2_HI, x);
    r = fmaf(-n, LN2_LO, r);
    float p = c7;
    p = fmaf(p, r, c6);
    p = fmaf(p, r, c5);
    p = fmaf(p, r, c4);
    p = fmaf(p, r, c3);
    p = fmaf(p, r, c2);
    p = fmaf(p, r, c1);
    p = fmaf(p, r, c0);
    int ni = (int)n;
    int n1 = ni / 2;
    int n2 = ni - n1;
    return (p * pow2i(n1)) * pow2i(n2);
}

void oracle_exp_ref_array(int64_t n, const float* x, float* y)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) y[i] = oracle_exp_ref(x[i]);
}

/* -------------------------------------------------------------- route ---- */

/* Top-k per token over E logits: k passes, each taking the largest logit not yet
 * taken; a strict '>' keeps the lower index on ties (and -0 == +0).  Weights are
 * the softmax over the k taken logits, in fp64. */
void oracle_route(int T, int E, int k, const float* logits, int32_t* eidx, double* w)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const float* l = logits + (int64_t)t * E;
        unsigned char taken[4096];
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;
            taken[best] = 1;
            eidx[(int64_t)t * k + j] = best;
        }
        double m = (double)l[eidx[(int64_t)t * k]];
        double z[4096];
        double s = 0.0;
        for (int j = 0; j < k; ++j) {
            z[j] = exp((double)l[eidx[(int64_t)t * k + j]] - m);
            s += z[j];
        }
        for (int j = 0; j < k; ++j) w[(int64_t)t * k + j] = z[j] / s;
    }
}

/* -------------------------------------------------------------- group ---- */

/* Row table by a stable counting sort of the pairs p = t*k + j on their expert. */
void oracle_group(int T, int k, int E, const int32_t* eidx, int32_t* counts, int32_t* bounds,
                  int32_t* rows, int32_t* pos)
{
    int64_t R = (int64_t)T * k;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t p = 0; p < R; ++p) counts[eidx[p]]++;
    bounds[0] = 0;
    for (int e = 0; e < E; ++e) bounds[e + 1] = bounds[e] + counts[e];
    int32_t fill[4096];
    for (int e = 0; e < E; ++e) fill[e] = bounds[e];
    for (int64_t p = 0; p < R; ++p) {
        int e = eidx[p];
        rows[fill[e]] = (int32_t)p;
        pos[p] = fill[e];
        fill[e]++;
    }
}

/* ------------------------------------------------------------ quantise --- */

/* Q8 blocks of 32 along each row of x [n_rows, K]. */
void oracle_quant_q8(int64_t n_rows, int K, const float* x, int8_t* q, float* scale)
{
    int nb = K / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n_rows; ++r) {
        for (int b = 0; b < nb; ++b) {
            const float* xb = x + r * K + 32 * b;
            int8_t* qb = q + r * K + 32 * b;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                float a = fabsf(xb[i]);
                if (a > amax) amax = a;
            }
            float d = amax / 127.0f;
            scale[r * nb + b] = d;
            for (int i = 0; i < 32; ++i) {
                if (d == 0.0f) {
                    qb[i] = 0;
                    continue;
                }
                float v = rintf(xb[i] / d);
                if (v > 127.0f) v = 127.0f;
                if (v < -127.0f) v = -127.0f;
                qb[i] = (int8_t)v;
            }
        }
    }
}

/* ---------------------------------------------------------------- GEMM --- */

/* Exact per-block int32 dot products: isum[m][n][b] = sum_{i<32} A[m][32b+i]*W[n][32b+i].
 * A [M, K] int8 (activation codes), W [N, K] int8 (weight integers). */
void oracle_block_dots(int M, int N, int K, const int8_t* A, const int8_t* W, int32_t* isum)
{
    int nb = K / 32;
#pragma omp parallel for schedule(static)
    for (int m = 0; m < M; ++m)
        for (int n = 0; n < N; ++n)
            for (int b = 0; b < nb; ++b) {
                int32_t s = 0;
                for (int i = 0; i < 32; ++i)
                    s += (int32_t)A[(int64_t)m * K + 32 * b + i] * (int32_t)W[(int64_t)n * K + 32 * b + i];
                isum[((int64_t)m * N + n) * nb + b] = s;
            }
}

/* out[m][n] = sum_b isum * a_scale[m][b] * w_scale[n][b], combined in fp32:
 * acc = 0; for b ascending: acc = fma((float)isum_b, a_scale * w_scale, acc). */
void oracle_gemm_f32(int M, int N, int K, const int8_t* A, const float* a_scale, const int8_t* W,
                     const uint16_t* w_scale, float* out)
{
    int nb = K / 32;
#pragma omp parallel for schedule(dynamic, 4)
    for (int m = 0; m < M; ++m) {
        for (int n = 0; n < N; ++n) {
            float acc = 0.0f;
            for (int b = 0; b < nb; ++b) {
                int32_t s = 0;
                for (int i = 0; i < 32; ++i)
                    s += (int32_t)A[(int64_t)m * K + 32 * b + i] * (int32_t)W[(int64_t)n * K + 32 * b + i];
                float ws = (float)oracle_f16_to_f64(w_scale[(int64_t)n * nb + b]);
                float sc = a_scale[(int64_t)m * nb + b] * ws;
                acc = fmaf((float)s, sc, acc);
            }
            out[(int64_t)m * N + n] = acc;
        }
    }
}

/* The same sum in fp64 (each term isum * a_scale * w_scale is exact in fp64). */
void oracle_gemm_f64(int M, int N, int K, const int8_t* A, const float* a_scale, const int8_t* W,
                     const uint16_t* w_scale, double* out)
{
    int nb = K / 32;
#pragma omp parallel for schedule(dynamic, 4)
    for (int m = 0; m < M; ++m) {
        for (int n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int b = 0; b < nb; ++b) {
                int32_t s = 0;
                for (int i = 0; i < 32; ++i)
                    s += (int32_t)A[(int64_t)m * K + 32 * b + i] * (int32_t)W[(int64_t)n * K + 32 * b + i];
                acc += (double)s * (double)a_scale[(int64_t)m * nb + b] *
                       oracle_f16_to_f64(w_scale[(int64_t)n * nb + b]);
            }
            out[(int64_t)m * N + n] = acc;
        }
    }
}

/* -------------------------------------------------------------- SwiGLU --- */

/* gu [M, 2f]: columns [0, f) gate, [f, 2f) up.  h[m][i] = silu(g) * u in fp32. */
void oracle_swiglu_f32(int64_t M, int f, const float* gu, float* h)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int i = 0; i < f; ++i) {
            float g = gu[m * 2 * f + i];
            float u = gu[m * 2 * f + f + i];
            float e = oracle_exp_ref(-g);
            float sg = g / (1.0f + e);
            h[m * f + i] = sg * u;
        }
}

/* ------------------------------------------------------------- combine --- */

/* y[t][n] = sum_{j<k} w[t][j] * dm[pos[t*k+j]][n], fp64, j ascending. */
void oracle_combine_f64(int T, int k, int d, const double* w, const int32_t* pos, const double* dm,
                        double* y)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t)
        for (int n = 0; n < d; ++n) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j)
                acc += w[(int64_t)t * k + j] * dm[(int64_t)pos[(int64_t)t * k + j] * d + n];
            y[(int64_t)t * d + n] = acc;
        }
}

int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
