/*
 * moe_oracle.c -- CPU oracle for the routed FP8 block-scaled MoE expert FFN.
 *
 * TEST INFRASTRUCTURE ONLY (see moe_oracle.h for the contract, the pages it
 * follows and every rounding point).  Plain loops in the order the method is
 * written; OpenMP only splits independent rows, so each element is computed
 * by exactly the same sequence of operations whatever the thread count.
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* O0: formats                                                          */
/* ------------------------------------------------------------------ */

#define E4M3_NAN NAN

/* OCP E4M3 ("FN"): code = s eeee mmm.  e == 0: (-1)^s * m * 2^-9;
 * e >= 1: (-1)^s * (8 + m) * 2^(e - 10); 0x7F and 0xFF are NaN.
 * Written out in full so it can be read against that closed form. */
static const float E4M3[256] = {
    /* 0x00 */ 0.0f, 0.001953125f, 0.00390625f, 0.005859375f, 0.0078125f, 0.009765625f, 0.01171875f, 0.013671875f,
    /* 0x08 */ 0.015625f, 0.017578125f, 0.01953125f, 0.021484375f, 0.0234375f, 0.025390625f, 0.02734375f, 0.029296875f,
    /* 0x10 */ 0.03125f, 0.03515625f, 0.0390625f, 0.04296875f, 0.046875f, 0.05078125f, 0.0546875f, 0.05859375f,
    /* 0x18 */ 0.0625f, 0.0703125f, 0.078125f, 0.0859375f, 0.09375f, 0.1015625f, 0.109375f, 0.1171875f,
    /* 0x20 */ 0.125f, 0.140625f, 0.15625f, 0.171875f, 0.1875f, 0.203125f, 0.21875f, 0.234375f,
    /* 0x28 */ 0.25f, 0.28125f, 0.3125f, 0.34375f, 0.375f, 0.40625f, 0.4375f, 0.46875f,
    /* 0x30 */ 0.5f, 0.5625f, 0.625f, 0.6875f, 0.75f, 0.8125f, 0.875f, 0.9375f,
    /* 0x38 */ 1.0f, 1.125f, 1.25f, 1.375f, 1.5f, 1.625f, 1.75f, 1.875f,
    /* 0x40 */ 2.0f, 2.25f, 2.5f, 2.75f, 3.0f, 3.25f, 3.5f, 3.75f,
    /* 0x48 */ 4.0f, 4.5f, 5.0f, 5.5f, 6.0f, 6.5f, 7.0f, 7.5f,
    /* 0x50 */ 8.0f, 9.0f, 10.0f, 11.0f, 12.0f, 13.0f, 14.0f, 15.0f,
    /* 0x58 */ 16.0f, 18.0f, 20.0f, 22.0f, 24.0f, 26.0f, 28.0f, 30.0f,
    /* 0x60 */ 32.0f, 36.0f, 40.0f, 44.0f, 48.0f, 52.0f, 56.0f, 60.0f,
    /* 0x68 */ 64.0f, 72.0f, 80.0f, 88.0f, 96.0f, 104.0f, 112.0f, 120.0f,
    /* 0x70 */ 128.0f, 144.0f, 160.0f, 176.0f, 192.0f, 208.0f, 224.0f, 240.0f,
    /* 0x78 */ 256.0f, 288.0f, 320.0f, 352.0f, 384.0f, 416.0f, 448.0f, E4M3_NAN,
    /* 0x80 */ -0.0f, -0.001953125f, -0.00390625f, -0.005859375f, -0.0078125f, -0.009765625f, -0.01171875f, -0.013671875f,
    /* 0x88 */ -0.015625f, -0.017578125f, -0.01953125f, -0.021484375f, -0.0234375f, -0.025390625f, -0.02734375f, -0.029296875f,
    /* 0x90 */ -0.03125f, -0.03515625f, -0.0390625f, -0.04296875f, -0.046875f, -0.05078125f, -0.0546875f, -0.05859375f,
    /* 0x98 */ -0.0625f, -0.0703125f, -0.078125f, -0.0859375f, -0.09375f, -0.1015625f, -0.109375f, -0.1171875f,
    /* 0xA0 */ -0.125f, -0.140625f, -0.15625f, -0.171875f, -0.1875f, -0.203125f, -0.21875f, -0.234375f,
    /* 0xA8 */ -0.25f, -0.28125f, -0.3125f, -0.34375f, -0.375f, -0.40625f, -0.4375f, -0.46875f,
    /* 0xB0 */ -0.5f, -0.5625f, -0.625f, -0.6875f, -0.75f, -0.8125f, -0.875f, -0.9375f,
    /* 0xB8 */ -1.0f, -1.125f, -1.25f, -1.375f, -1.5f, -1.625f, -1.75f, -1.875f,
    /* 0xC0 */ -2.0f, -2.25f, -2.5f, -2.75f, -3.0f, -3.25f, -3.5f, -3.75f,
    /* 0xC8 */ -4.0f, -4.5f, -5.0f, -5.5f, -6.0f, -6.5f, -7.0f, -7.5f,
    /* 0xD0 */ -8.0f, -9.0f, -10.0f, -11.0f, -12.0f, -13.0f, -14.0f, -15.0f,
    /* 0xD8 */ -16.0f, -18.0f, -20.0f, -22.0f, -24.0f, -26.0f, -28.0f, -30.0f,
    /* 0xE0 */ -32.0f, -36.0f, -40.0f, -44.0f, -48.0f, -52.0f, -56.0f, -60.0f,
    /* 0xE8 */ -64.0f, -72.0f, -80.0f, -88.0f, -96.0f, -104.0f, -112.0f, -120.0f,
    /* 0xF0 */ -128.0f, -144.0f, -160.0f, -176.0f, -192.0f, -208.0f, -224.0f, -240.0f,
    /* 0xF8 */ -256.0f, -288.0f, -320.0f, -352.0f, -384.0f, -416.0f, -448.0f, E4M3_NAN,
};

const float* oracle_e4m3_table(void) { return E4M3; }

float oracle_e4m3_decode(uint8_t code) { return E4M3[code]; }

/* Nearest finite E4M3 value to v; ties go to the code whose last mantissa
 * bit is 0; magnitudes above 448 give +-448; the sign of zero is kept. */
uint8_t oracle_e4m3_encode(float v)
{
    if (isnan(v)) return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    float a = fabsf(v);
    if (a >= 448.0f) return (uint8_t)(sign | 0x7E);
    /* Positive codes 0x00..0x7E increase strictly in value.  Bisect for
     * lo, hi = lo + 1 with E4M3[lo] <= a < E4M3[hi]. */
    int lo = 0x00, hi = 0x7E;
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (E4M3[mid] <= a) lo = mid; else hi = mid;
    }
    /* distances in double are exact for these fp32 operands */
    double dlo = (double)a - (double)E4M3[lo];
    double dhi = (double)E4M3[hi] - (double)a;
    int c;
    if (dlo < dhi) c = lo;
    else if (dhi < dlo) c = hi;
    else c = (lo & 1) ? hi : lo;
    return (uint8_t)(sign | c);
}

/* Same contract by exhaustive search over every finite code that carries
 * the sign of v.  Used only to check oracle_e4m3_encode. */
uint8_t oracle_e4m3_encode_linear(float v)
{
    if (isnan(v)) return 0x7F;
    int sgn = signbit(v) ? 1 : 0;
    int best = -1;
    double bestd = 0.0;
    for (int c = 0; c < 256; ++c) {
        if ((c & 0x7F) == 0x7F) continue;        /* NaN codes */
        if (((c >> 7) & 1) != sgn) continue;      /* sign must match v */
        double d = fabs((double)E4M3[c] - (double)v);
        if (best < 0 || d < bestd || (d == bestd && (c & 1) == 0)) {
            best = c;
            bestd = d;
        }
    }
    return (uint8_t)best;
}

void oracle_e4m3_encode_array(const float* v, int64_t n, uint8_t* out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) out[j] = oracle_e4m3_encode(v[j]);
}

static uint32_t f32_bits(float v) { uint32_t u; memcpy(&u, &v, 4); return u; }
static float bits_f32(uint32_t u) { float v; memcpy(&v, &u, 4); return v; }

float oracle_bf16_decode(uint16_t b) { return bits_f32((uint32_t)b << 16); }

/* Round an fp32 to the nearest bf16 (8-bit exponent, 7-bit fraction), ties
 * to the even bf16.  The two candidates are the truncation of v and the next
 * bf16 away from zero; both distances are exact in double. */
uint16_t oracle_bf16_encode(float v)
{
    if (isnan(v)) return 0x7FC0;
    uint32_t u = f32_bits(v);
    uint16_t lo = (uint16_t)(u >> 16);          /* truncation, same sign */
    if ((u & 0xFFFFu) == 0) return lo;           /* exactly representable */
    uint16_t hi = (uint16_t)(lo + 1);            /* next magnitude up */
    /* Past the largest finite bf16 the next candidate is infinity; IEEE
     * rounding compares against 2^128, the value an unbounded exponent
     * would give there. */
    double vhi = ((hi & 0x7FFFu) == 0x7F80u) ? copysign(0x1.0p128, (double)v)
                                            : (double)oracle_bf16_decode(hi);
    double dlo = fabs((double)v - (double)oracle_bf16_decode(lo));
    double dhi = fabs(vhi - (double)v);
    if (dlo < dhi) return lo;
    if (dhi < dlo) return hi;
    return (lo & 1) ? hi : lo;
}

/* ------------------------------------------------------------------ */
/* threads                                                              */
/* ------------------------------------------------------------------ */

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_get_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* 1x128 / 128x128 block quantisation                                   */
/* ------------------------------------------------------------------ */

/* Quantise n (<= 128) values that share one scale. */
static float quant_group(const float* v, int n, int stride, uint8_t* q, int qstride)
{
    float amax = 0.0f;
    for (int j = 0; j < n; ++j) {
        float a = fabsf(v[(int64_t)j * stride]);
        if (a > amax) amax = a;
    }
    float s = amax / 448.0f;
    for (int j = 0; j < n; ++j) {
        uint8_t c = 0x00;
        if (s != 0.0f) c = oracle_e4m3_encode(v[(int64_t)j * stride] / s);
        q[(int64_t)j * qstride] = c;
    }
    return s;
}

void oracle_quant_weight_block128(const float* w, int64_t batch, int N, int K,
                                  uint8_t* q, float* s)
{
    const int NB = N / 128, KB = K / 128;
    #pragma omp parallel for schedule(static)
    for (int64_t blk = 0; blk < batch * NB * KB; ++blk) {
        int64_t b = blk / (NB * KB);
        int nb = (int)((blk / KB) % NB);
        int kb = (int)(blk % KB);
        const float* base = w + (b * N + (int64_t)nb * 128) * K + (int64_t)kb * 128;
        uint8_t* qbase = q + (b * N + (int64_t)nb * 128) * K + (int64_t)kb * 128;
        float amax = 0.0f;
        for (int r = 0; r < 128; ++r)
            for (int c = 0; c < 128; ++c) {
                float a = fabsf(base[(int64_t)r * K + c]);
                if (a > amax) amax = a;
            }
        float sc = amax / 448.0f;
        for (int r = 0; r < 128; ++r)
            for (int c = 0; c < 128; ++c) {
                uint8_t code = 0x00;
                if (sc != 0.0f) code = oracle_e4m3_encode(base[(int64_t)r * K + c] / sc);
                qbase[(int64_t)r * K + c] = code;
            }
        s[blk] = sc;
    }
}

void oracle_act_quant(const uint16_t* x, int M, int K, uint8_t* q, float* s)
{
    const int KB = K / 128;
    #pragma omp parallel for schedule(static)
    for (int t = 0; t < M; ++t) {
        float row[128];
        for (int g = 0; g < KB; ++g) {
            for (int j = 0; j < 128; ++j)
                row[j] = oracle_bf16_decode(x[(int64_t)t * K + g * 128 + j]);
            s[(int64_t)t * KB + g] = quant_group(row, 128, 1, q + (int64_t)t * K + g * 128, 1);
        }
    }
}

/* ------------------------------------------------------------------ */
/* BF16 routing logits                                                  */
/* ------------------------------------------------------------------ */

void oracle_router_logits(const uint16_t* x, const uint16_t* wr, int M, int K, int E, float* logits)
{
    #pragma omp parallel for schedule(static)
    for (int t = 0; t < M; ++t) {
        const uint16_t* xr = x + (int64_t)t * K;
        for (int e = 0; e < E; ++e) {
            const uint16_t* w = wr + (int64_t)e * K;
            double acc = 0.0;
            for (int j = 0; j < K; ++j)
                acc += (double)oracle_bf16_decode(xr[j]) * (double)oracle_bf16_decode(w[j]);
            logits[(int64_t)t * E + e] = (float)acc;
        }
    }
}

/* ------------------------------------------------------------------ */
/* Front end: RMSNorm to bf16, then the 1x128 quantisation above        */
/* ------------------------------------------------------------------ */

void oracle_rmsnorm_act_quant(const uint16_t* x, const float* gamma, float eps, int M, int K,
                              uint16_t* y, uint8_t* q, float* s)
{
    const int KB = K / 128;
    #pragma omp parallel for schedule(static)
    for (int t = 0; t < M; ++t) {
        const uint16_t* xr = x + (int64_t)t * K;
        uint16_t* yr = y + (int64_t)t * K;
        /* mean of squares and its inverse square root, in float64 */
        double ss = 0.0;
        for (int c = 0; c < K; ++c) {
            const double v = (double)oracle_bf16_decode(xr[c]);
            ss += v * v;
        }
        const double ms = ss / (double)K;
        const float r = (float)(1.0 / sqrt(ms + (double)eps));
        /* normalised, weighted, rounded to bf16 */
        for (int c = 0; c < K; ++c) {
            const float n = oracle_bf16_decode(xr[c]) * r;
            const float wv = n * gamma[c];
            yr[c] = oracle_bf16_encode(wv);
        }
        /* the layer's activation quantisation of the bf16 row */
        float row[128];
        for (int g = 0; g < KB; ++g) {
            for (int j = 0; j < 128; ++j) row[j] = oracle_bf16_decode(yr[g * 128 + j]);
            s[(int64_t)t * KB + g] = quant_group(row, 128, 1, q + (int64_t)t * K + g * 128, 1);
        }
    }
}

/* ------------------------------------------------------------------ */
/* O2: router -- softmax, top-k on logits (ties to lower index), renorm */
/* ------------------------------------------------------------------ */

void oracle_router(const float* logits, int M, int E, int k, int32_t* ids, float* w)
{
    #pragma omp parallel for schedule(static)
    for (int t = 0; t < M; ++t) {
        const float* l = logits + (int64_t)t * E;
        float* p = (float*)malloc(sizeof(float) * (size_t)E);
        unsigned char* taken = (unsigned char*)calloc((size_t)E, 1);
        /* softmax */
        float mx = l[0];
        for (int e = 1; e < E; ++e) if (l[e] > mx) mx = l[e];
        float S = 0.0f;
        for (int e = 0; e < E; ++e) { p[e] = expf(l[e] - mx); S += p[e]; }
        for (int e = 0; e < E; ++e) p[e] = p[e] / S;
        /* top-k: k passes, each takes the largest remaining logit; a strict
         * '>' keeps the lower index among equal logits */
        for (int r = 0; r < k; ++r) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e;
            }
            taken[best] = 1;
            ids[(int64_t)t * k + r] = best;
        }
        /* renormalise over the picks */
        float ssel = 0.0f;
        for (int r = 0; r < k; ++r) ssel += p[ids[(int64_t)t * k + r]];
        for (int r = 0; r < k; ++r)
            w[(int64_t)t * k + r] = p[ids[(int64_t)t * k + r]] / ssel;
        free(p);
        free(taken);
    }
}

/* ------------------------------------------------------------------ */
/* O4: grouping by expert (stable counting sort)                        */
/* ------------------------------------------------------------------ */

void oracle_group(const int32_t* ids, int R, int E,
                  int32_t* counts, int32_t* offsets, int32_t* sorted)
{
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int p = 0; p < R; ++p) counts[ids[p]] += 1;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t* fill = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    for (int e = 0; e < E; ++e) fill[e] = offsets[e];
    for (int p = 0; p < R; ++p) sorted[fill[ids[p]]++] = p;
    free(fill);
}

/* ------------------------------------------------------------------ */
/* O5 / O7: block-scaled FP8 GEMM                                       */
/* ------------------------------------------------------------------ */

void oracle_block_gemm(const uint8_t* A, const float* As, const int32_t* arow,
                       const uint8_t* W, const float* Ws, const int32_t* wsel,
                       int R, int N, int K, float* out)
{
    const int KB = K / 128, NB = N / 128;
    #pragma omp parallel for schedule(static)
    for (int64_t rn = 0; rn < (int64_t)R * N; ++rn) {
        int r = (int)(rn / N), n = (int)(rn % N);
        const uint8_t* a = A + (int64_t)arow[r] * K;
        const float* as = As + (int64_t)arow[r] * KB;
        const uint8_t* wr = W + ((int64_t)wsel[r] * N + n) * K;
        const float* ws = Ws + ((int64_t)wsel[r] * NB + n / 128) * KB;
        float acc = 0.0f;
        for (int kb = 0; kb < KB; ++kb) {
            float blk = 0.0f;
            for (int kk = 0; kk < 128; ++kk)
                blk += E4M3[a[kb * 128 + kk]] * E4M3[wr[kb * 128 + kk]];
            acc += blk * (as[kb] * ws[kb]);
        }
        out[rn] = acc;
    }
}

/* ------------------------------------------------------------------ */
/* O6: SiLU(gate) * up, then 1x128 FP8 requantisation                   */
/* ------------------------------------------------------------------ */

void oracle_silu_mul_quant(const float* g, int R, int I, uint8_t* a2, float* a2s)
{
    const int IB = I / 128;
    #pragma omp parallel for schedule(static)
    for (int p = 0; p < R; ++p) {
        const float* gate = g + (int64_t)p * 2 * I;
        const float* up = gate + I;
        float v[128];
        for (int b = 0; b < IB; ++b) {
            for (int j = 0; j < 128; ++j) {
                float a = gate[b * 128 + j];
                float u = up[b * 128 + j];
                v[j] = (a / (1.0f + expf(-a))) * u;
            }
            a2s[(int64_t)p * IB + b] = quant_group(v, 128, 1, a2 + (int64_t)p * I + b * 128, 1);
        }
    }
}

/* ------------------------------------------------------------------ */
/* O8: fixed-order combine over the k routes of each token              */
/* ------------------------------------------------------------------ */

void oracle_combine(const float* y, const float* w, int M, int k, int H, uint16_t* out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t tn = 0; tn < (int64_t)M * H; ++tn) {
        int t = (int)(tn / H), n = (int)(tn % H);
        float acc = 0.0f;
        for (int r = 0; r < k; ++r)
            acc += w[(int64_t)t * k + r] * y[((int64_t)t * k + r) * H + n];
        out[tn] = oracle_bf16_encode(acc);
    }
}

/* ------------------------------------------------------------------ */
/* whole layer                                                          */
/* ------------------------------------------------------------------ */

int oracle_moe_forward(const uint16_t* x, const float* logits,
                       const uint8_t* w13, const float* s13,
                       const uint8_t* w2, const float* s2,
                       uint16_t* out, int M, int h, int i, int E, int k,
                       oracle_intermediates* dbg)
{
    if (M < 0 || h <= 0 || i <= 0 || E <= 0 || k < 1 || k > E) return -1;
    if (h % 128 != 0 || i % 128 != 0) return -1;
    if (M == 0) return 0;
    const int R = M * k;
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)R);
    float* tw = (float*)malloc(sizeof(float) * (size_t)R);
    uint8_t* xq = (uint8_t*)malloc((size_t)M * h);
    float* xs = (float*)malloc(sizeof(float) * (size_t)M * (h / 128));
    int32_t* counts = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    int32_t* offsets = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t* sorted = (int32_t*)malloc(sizeof(int32_t) * (size_t)R);
    int32_t* arow = (int32_t*)malloc(sizeof(int32_t) * (size_t)R);
    int32_t* wsel = (int32_t*)malloc(sizeof(int32_t) * (size_t)R);
    int32_t* prow = (int32_t*)malloc(sizeof(int32_t) * (size_t)R);
    float* g = (float*)malloc(sizeof(float) * (size_t)R * 2 * i);
    uint8_t* a2 = (uint8_t*)malloc((size_t)R * i);
    float* a2s = (float*)malloc(sizeof(float) * (size_t)R * (i / 128));
    float* y = (float*)malloc(sizeof(float) * (size_t)R * h);
    float* gs = (float*)malloc(sizeof(float) * (size_t)R * 2 * i);
    float* ys = (float*)malloc(sizeof(float) * (size_t)R * h);

    /* 1. routing */
    oracle_router(logits, M, E, k, ids, tw);
    /* 2. per-token 1x128 activation quantisation */
    oracle_act_quant(x, M, h, xq, xs);
    /* 3. group routes by expert */
    oracle_group(ids, R, E, counts, offsets, sorted);
    /* 4. gate/up GEMM over routes in grouped order: route p = sorted[j]
     *    reads token p / k with expert ids[p] */
    for (int j = 0; j < R; ++j) {
        arow[j] = sorted[j] / k;
        wsel[j] = ids[sorted[j]];
    }
    oracle_block_gemm(xq, xs, arow, w13, s13, wsel, R, 2 * i, h, gs);
    /* scatter back to route order */
    for (int j = 0; j < R; ++j)
        memcpy(g + (int64_t)sorted[j] * 2 * i, gs + (int64_t)j * 2 * i, sizeof(float) * 2 * (size_t)i);
    /* 5. SiLU(gate) * up with FP8 requantisation, per route */
    oracle_silu_mul_quant(g, R, i, a2, a2s);
    /* 6. down GEMM, grouped order, activation row = route */
    for (int j = 0; j < R; ++j) prow[j] = sorted[j];
    oracle_block_gemm(a2, a2s, prow, w2, s2, wsel, R, h, i, ys);
    for (int j = 0; j < R; ++j)
        memcpy(y + (int64_t)sorted[j] * h, ys + (int64_t)j * h, sizeof(float) * (size_t)h);
    /* 7. fixed-order combine */
    oracle_combine(y, tw, M, k, h, out);

    if (dbg) {
        if (dbg->ids) memcpy(dbg->ids, ids, sizeof(int32_t) * (size_t)R);
        if (dbg->topk_w) memcpy(dbg->topk_w, tw, sizeof(float) * (size_t)R);
        if (dbg->xq) memcpy(dbg->xq, xq, (size_t)M * h);
        if (dbg->xs) memcpy(dbg->xs, xs, sizeof(float) * (size_t)M * (h / 128));
        if (dbg->counts) memcpy(dbg->counts, counts, sizeof(int32_t) * (size_t)E);
        if (dbg->offsets) memcpy(dbg->offsets, offsets, sizeof(int32_t) * (size_t)(E + 1));
        if (dbg->sorted) memcpy(dbg->sorted, sorted, sizeof(int32_t) * (size_t)R);
        if (dbg->g) memcpy(dbg->g, g, sizeof(float) * (size_t)R * 2 * i);
        if (dbg->a2) memcpy(dbg->a2, a2, (size_t)R * i);
        if (dbg->a2s) memcpy(dbg->a2s, a2s, sizeof(float) * (size_t)R * (i / 128));
        if (dbg->y) memcpy(dbg->y, y, sizeof(float) * (size_t)R * h);
    }
    free(ids); free(tw); free(xq); free(xs); free(counts); free(offsets);
    free(sorted); free(arow); free(wsel); free(prow); free(g); free(a2);
    free(a2s); free(y); free(gs); free(ys);
    return 0;
}

/* ------------------------------------------------------------------ */
/* MXFP4 weight variant                                                 */
/* ------------------------------------------------------------------ */

/* E2M1 (OCP MX FP4): bit 3 sign, bits 2..1 exponent (bias 1), bit 0
 * mantissa.  Exponent 0 is subnormal (m * 0.5); otherwise (1 + m/2) *
 * 2^(e - 1).  No infinities or NaN; the largest magnitude is 6. */
static const float E2M1[16] = {
    0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f,
    -0.0f, -0.5f, -1.0f, -1.5f, -2.0f, -3.0f, -4.0f, -6.0f,
};

float oracle_e2m1_decode(uint8_t code) { return E2M1[code & 15]; }

/* Nearest E2M1 value; a tie goes to the code whose mantissa bit is 0
 * (round to nearest even); |v| above 6 gives +-6; the sign of zero is kept.
 * Found by comparing |v| with each non-negative value in ascending order. */
uint8_t oracle_e2m1_encode(float v)
{
    const uint8_t sign = signbit(v) ? 8 : 0;
    const double a = fabs((double)v);
    if (isnan(v)) return 7;
    if (a >= 6.0) return (uint8_t)(sign | 7);   /* saturation (also keeps huge |v| exact) */
    int best = 0;
    for (int c = 1; c < 8; ++c) {
        const double dc = fabs(a - (double)E2M1[c]), db = fabs(a - (double)E2M1[best]);
        if (dc < db || (dc == db && (c & 1) == 0)) best = c;
    }
    return (uint8_t)(sign | best);
}

/* E8M0 block scale: 2^(code - 127); code 255 is NaN (never produced here). */
double oracle_e8m0_decode(uint8_t code) { return code == 255 ? NAN : ldexp(1.0, (int)code - 127); }

/* OCP MX quantisation of fp32 rows [rows][K] in blocks of 32 along K:
 * shared exponent e = floor(log2(amax)) - 2 (2 = the largest E2M1 exponent),
 * clamped to [-127, 127], scale code e + 127; element code = E2M1(w * 2^-e)
 * (exact scaling by a power of two).  amax == 0 gives scale code 0 and zero
 * codes.  codes [rows][K/2]: element 2j in the low nibble of byte j, 2j + 1
 * in the high nibble; scales [rows][K/32]. */
void oracle_mxfp4_quantize(const float* w, int64_t rows, int K, uint8_t* codes, uint8_t* scales)
{
    const int nb = K / 32;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int b = 0; b < nb; ++b) {
            const float* v = w + r * K + (int64_t)b * 32;
            double amax = 0.0;
            for (int j = 0; j < 32; ++j) amax = fmax(amax, fabs((double)v[j]));
            int e = -127;
            if (amax > 0.0) {
                int ex;
                frexp(amax, &ex);          /* amax = f * 2^ex, f in [0.5, 1) */
                e = (ex - 1) - 2;          /* floor(log2(amax)) - 2 */
                if (e < -127) e = -127;
                if (e > 127) e = 127;
            }
            scales[r * nb + b] = (uint8_t)(amax > 0.0 ? e + 127 : 0);
            for (int j = 0; j < 32; j += 2) {
                uint8_t c0 = 0, c1 = 0;
                if (amax > 0.0) {
                    c0 = oracle_e2m1_encode((float)ldexp((double)v[j], -e));
                    c1 = oracle_e2m1_encode((float)ldexp((double)v[j + 1], -e));
                }
                codes[r * (K / 2) + (int64_t)b * 16 + j / 2] = (uint8_t)(c0 | (c1 << 4));
            }
        }
    }
}

/* One GEMM row of the MXFP4 variant: out[n] = fp32( sum over k of
 * E2M1(W[n][k]) * 2^(S[n][k/32] - 127) * E4M3(a[k]) * as[k/128] ), every
 * term exact in float64, summed in float64 in ascending k, rounded once. */
static void mx_gemm_row(const uint8_t* a, const float* as, const uint8_t* W, const uint8_t* S,
                        int N, int K, float* out)
{
    for (int n = 0; n < N; ++n) {
        const uint8_t* wr = W + (int64_t)n * (K / 2);
        const uint8_t* sr = S + (int64_t)n * (K / 32);
        double acc = 0.0;
        for (int kk = 0; kk < K; ++kk) {
            const uint8_t c = (uint8_t)((wr[kk / 2] >> ((kk & 1) * 4)) & 15);
            const double wv = (double)E2M1[c] * oracle_e8m0_decode(sr[kk / 32]);
            acc += wv * (double)E4M3[a[kk]] * (double)as[kk / 128];
        }
        out[n] = (float)acc;
    }
}

int oracle_moe_forward_mxfp4(const uint16_t* x, const float* logits,
                             const uint8_t* w13, const uint8_t* e13,
                             const uint8_t* w2, const uint8_t* e2,
                             uint16_t* out, int M, int h, int i, int E, int k,
                             oracle_intermediates* dbg)
{
    if (M < 0 || h <= 0 || i <= 0 || E <= 0 || k < 1 || k > E) return -1;
    if (h % 128 != 0 || i % 128 != 0) return -1;
    if (M == 0) return 0;
    const int R = M * k;
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)R);
    float* tw = (float*)malloc(sizeof(float) * (size_t)R);
    uint8_t* xq = (uint8_t*)malloc((size_t)M * h);
    float* xs = (float*)malloc(sizeof(float) * (size_t)M * (h / 128));
    float* g = (float*)malloc(sizeof(float) * (size_t)R * 2 * i);
    uint8_t* a2 = (uint8_t*)malloc((size_t)R * i);
    float* a2s = (float*)malloc(sizeof(float) * (size_t)R * (i / 128));
    float* y = (float*)malloc(sizeof(float) * (size_t)R * h);

    /* routing and the 1x128 activation quantisation as in the FP8 layer */
    oracle_router(logits, M, E, k, ids, tw);
    oracle_act_quant(x, M, h, xq, xs);
    /* gate/up per route (route p = t * k + r reads token t, expert ids[p]) */
    #pragma omp parallel for schedule(dynamic)
    for (int p = 0; p < R; ++p) {
        const int t = p / k, e = ids[p];
        mx_gemm_row(xq + (int64_t)t * h, xs + (int64_t)t * (h / 128),
                    w13 + (int64_t)e * 2 * i * (h / 2), e13 + (int64_t)e * 2 * i * (h / 32),
                    2 * i, h, g + (int64_t)p * 2 * i);
    }
    oracle_silu_mul_quant(g, R, i, a2, a2s);
    #pragma omp parallel for schedule(dynamic)
    for (int p = 0; p < R; ++p) {
        const int e = ids[p];
        mx_gemm_row(a2 + (int64_t)p * i, a2s + (int64_t)p * (i / 128),
                    w2 + (int64_t)e * h * (i / 2), e2 + (int64_t)e * h * (i / 32),
                    h, i, y + (int64_t)p * h);
    }
    oracle_combine(y, tw, M, k, h, out);

    if (dbg) {
        if (dbg->ids) memcpy(dbg->ids, ids, sizeof(int32_t) * (size_t)R);
        if (dbg->topk_w) memcpy(dbg->topk_w, tw, sizeof(float) * (size_t)R);
        if (dbg->xq) memcpy(dbg->xq, xq, (size_t)M * h);
        if (dbg->xs) memcpy(dbg->xs, xs, sizeof(float) * (size_t)M * (h / 128));
        if (dbg->g) memcpy(dbg->g, g, sizeof(float) * (size_t)R * 2 * i);
        if (dbg->a2) memcpy(dbg->a2, a2, (size_t)R * i);
        if (dbg->a2s) memcpy(dbg->a2s, a2s, sizeof(float) * (size_t)R * (i / 128));
        if (dbg->y) memcpy(dbg->y, y, sizeof(float) * (size_t)R * h);
    }
    free(ids); free(tw); free(xq); free(xs); free(g); free(a2); free(a2s); free(y);
    return 0;
}
