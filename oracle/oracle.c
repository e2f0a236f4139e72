/*
 * oracle.c -- plain, slow CPU oracle for the per-layer cached denoising step of a
 * diffusion LLM (refresh-row projection, rotary embedding, cache write, bidirectional
 * attention, attention mass, top-k tracking and the cosine drift test).
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load this library.  It shares no source, header, table or helper with
 * the HIP library, and it never calls it.
 *
 * Arithmetic: IEEE double throughout.  Every sum runs over its index in ascending order,
 * one output element per loop, and the file is built with -ffp-contract=off, so each output
 * depends only on its own inputs (never on which other rows are computed, nor on the
 * number of threads).  OpenMP only splits independent outputs across threads.
 *
 * Sources, by function:
 *   orc_linear          QKV projection of the refreshed rows (Flash-dLLM summary, paragraph
 *                       on the memory problem: projection -> RoPE -> cache write -> attention;
 *                       LaCache Technical Summary, Methodology 1: RoPECache holds hidden states
 *                       after the QKV projection and RoPE).
 *   orc_rope_rows       rotary embedding, rotate-half pairing (i, i + D/2), theta_i =
 *                       base^(-2i/D).  The pages give no formula; the dLLM-Cache record names
 *                       rotate_half / apply_rotary_pos_emb only.  Reading stated in the
 *                       design notes.
 *   orc_round_*         storage precision of the cache (bf16 / fp32), round to nearest even.
 *   orc_e4m3_*          OCP 8-bit floating point, E4M3 ("fn") variant: bias 7, max 448,
 *                       S.1111.111 = NaN, no infinities.  Written from that specification.
 *   orc_fp8_quantize_rows  per-group FP8 with one scale per 1 x 128 group (LaCache Technical
 *                       Summary, Methodology 2, granularity), applied to cache rows.
 *   orc_attention       softmax(Q K^T / sqrt(d)) V without a mask (Flash-Cache article,
 *                       section 3.1 pseudocode; LaCache Problem Statement: bidirectional
 *                       attention over the full context), plus log-sum-exp and the column
 *                       attention mass used to rank the most-attended tokens (Flash-dLLM
 *                       summary, paragraph on selective cache tracking).
 *   orc_attention_state the online-softmax state (running maximum m, normaliser l,
 *                       unnormalised output O~) of attention over a subset of the keys, the
 *                       quantities FACache keeps for query rows outside the current block
 *                       over the keys of the invariant region (LaCache Technical Summary,
 *                       Methodology 1, FACache).
 *   orc_topk            the k most-attended tokens per head (tracking budget 32).
 *   orc_drift           Elastic-Cache core idea: cosine similarity of the previous step's
 *                       most-attended tokens; refresh when it drops below gamma.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------ */
/* Storage rounding                                                                      */
/* ------------------------------------------------------------------------------------ */

/* Round a double to the nearest fp32 value (C conversion rounds to nearest even). */
double orc_round_f32(double x) { return (double)(float)x; }

/* Round a double to the nearest bf16 value, ties to even: 8 significant bits, the exponent
 * range of fp32 (smallest subnormal 2^-133), overflow to infinity. */
double orc_round_bf16(double x)
{
    if (isnan(x) || isinf(x) || x == 0.0) return x;
    int e;
    frexp(fabs(x), &e);              /* |x| in [2^(e-1), 2^e) */
    int ulp_exp = e - 8;             /* spacing of 8-bit significands in that binade */
    if (ulp_exp < -133) ulp_exp = -133;
    double r = nearbyint(ldexp(fabs(x), -ulp_exp)); /* default mode: nearest, ties even */
    double y = ldexp(r, ulp_exp);
    if (y >= ldexp(1.0, 128)) y = INFINITY;
    return copysign(y, x);
}

/* mode 0: keep double, 1: fp32, 2: bf16 (in place) */
void orc_round(double *x, int64_t n, int mode)
{
    if (mode == 0) return;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        x[i] = (mode == 1) ? orc_round_f32(x[i]) : orc_round_bf16(x[i]);
}

/* ------------------------------------------------------------------------------------ */
/* OCP FP8 E4M3 (fn) codec                                                               */
/* ------------------------------------------------------------------------------------ */

double orc_e4m3_decode(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);                /* subnormal: m/8 * 2^-6 */
    else v = ldexp((double)(8 + m), e - 10);             /* (1 + m/8) * 2^(e-7)  */
    return s ? -v : v;
}

/* Round to the nearest representable E4M3 value, ties to even, saturating to +-448;
 * NaN maps to the NaN code with its sign. */
uint8_t orc_e4m3_encode(double x)
{
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    if (isnan(x)) return sign | 0x7F;
    double a = fabs(x);
    if (a >= 448.0) return sign | 0x7E;
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                    /* a in [2^(e-1), 2^e) */
    int E = e - 1;                   /* unbiased exponent of a */
    if (E < -6) E = -6;              /* subnormals share the spacing of the smallest binade */
    int ulp_exp = E - 3;             /* 3 mantissa bits */
    double r = nearbyint(ldexp(a, -ulp_exp));
    double v = ldexp(r, ulp_exp);    /* the rounded magnitude, exact */
    if (v > 448.0) v = 448.0;
    if (v == 0.0) return sign;
    if (v < ldexp(1.0, -6)) return sign | (uint8_t)(int)ldexp(v, 9);   /* 1..7 */
    frexp(v, &e);
    E = e - 1;
    int mant = (int)ldexp(v, 3 - E) - 8;                                 /* 0..7 */
    return sign | (uint8_t)(((E + 7) << 3) | mant);
}

void orc_e4m3_encode_array(const double *x, int64_t n, uint8_t *codes)
{
    for (int64_t i = 0; i < n; i++) codes[i] = orc_e4m3_encode(x[i]);
}

void orc_e4m3_decode_array(const uint8_t *codes, int64_t n, double *x)
{
    for (int64_t i = 0; i < n; i++) x[i] = orc_e4m3_decode(codes[i]);
}

/* Per-group FP8 of cache rows: one group = one row of `group` values.
 *   amax  = max |x_t|
 *   scale = fp32(amax) / 448 computed in fp32; a zero row gets scale 1
 *   code  = e4m3(x_t / scale), the quotient formed in double
 *   deq_t = decode(code_t) * scale                                                        */
void orc_fp8_quantize_rows(const double *x, int64_t rows, int group, uint8_t *codes,
                           float *scales, double *deq)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        const double *row = x + r * group;
        double amax = 0.0;
        for (int t = 0; t < group; t++)
            if (fabs(row[t]) > amax) amax = fabs(row[t]);
        float s = (float)amax / 448.0f;
        if (amax == 0.0) s = 1.0f;
        scales[r] = s;
        for (int t = 0; t < group; t++) {
            uint8_t c = orc_e4m3_encode(row[t] / (double)s);
            codes[r * group + t] = c;
            if (deq) deq[r * group + t] = orc_e4m3_decode(c) * (double)s;
        }
    }
}

/* ------------------------------------------------------------------------------------ */
/* Projection and rotary embedding                                                       */
/* ------------------------------------------------------------------------------------ */

/* y[r][j] = sum_{k=0}^{H-1} x[r][k] * w[wrow[j]][k], summed in ascending k.
 *   x: [R, H] fp32, w: [Nw, H] fp32, wrow: [J] rows of w to use, y: [R, J] double. */
void orc_linear(const float *x, int64_t R, int64_t H, const float *w, const int32_t *wrow,
                int64_t J, double *y)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t r = 0; r < R; r++)
        for (int64_t j = 0; j < J; j++) {
            const float *xr = x + r * H;
            const float *wj = w + (int64_t)wrow[j] * H;
            double acc = 0.0;
            for (int64_t k = 0; k < H; k++) acc += (double)xr[k] * (double)wj[k];
            y[r * J + j] = acc;
        }
}

/* Rotary embedding, in place, on x: [R, nh, D] (nh heads per row) at absolute position
 * pos[r].  For i < D/2, theta_i = base^(-2i/D), phi = pos * theta_i:
 *   x'_i       = x_i cos(phi) - x_{i+D/2} sin(phi)
 *   x'_{i+D/2} = x_{i+D/2} cos(phi) + x_i sin(phi)                                        */
void orc_rope_rows(double *x, int64_t R, int nh, int D, const int32_t *pos, double base)
{
    int half = D / 2;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; r++)
        for (int h = 0; h < nh; h++) {
            double *v = x + (r * nh + h) * D;
            for (int i = 0; i < half; i++) {
                double theta = pow(base, -2.0 * (double)i / (double)D);
                double phi = (double)pos[r] * theta;
                double c = cos(phi), s = sin(phi);
                double a = v[i], b = v[i + half];
                v[i] = a * c - b * s;
                v[i + half] = b * c + a * s;
            }
        }
}

/* ------------------------------------------------------------------------------------ */
/* Bidirectional attention, log-sum-exp and column attention mass                        */
/* ------------------------------------------------------------------------------------ */

/* q: [B, n, Hq, D]; k, v: [B, Hkv, S, D]; query head h reads KV head h / (Hq/Hkv).
 * For every (b, h, i):  z_j = <q, k_j> * scale for all j < S (no mask),
 *   m = max_j z_j, l = sum_j exp(z_j - m), p_j = exp(z_j - m) / l,
 *   out = sum_j p_j v_j, lse = m + log(l).
 * mass (nullable): [B, Hq, S], mass[b,h,j] = sum_i p_ij, summed in ascending i.
 * out: [B, n, Hq, D], lse (nullable): [B, Hq, n]. */
void orc_attention(const double *q, const double *k, const double *v, int B, int n, int Hq,
                   int Hkv, int S, int D, double scale, double *out, double *lse, double *mass)
{
    int G = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; b++)
        for (int h = 0; h < Hq; h++) {
            int g = h / G;
            const double *K = k + ((int64_t)(b * Hkv + g) * S) * D;
            const double *V = v + ((int64_t)(b * Hkv + g) * S) * D;
            double *p = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
            double *a = mass ? mass + ((int64_t)(b * Hq + h)) * S : NULL;
            if (a)
                for (int j = 0; j < S; j++) a[j] = 0.0;
            for (int i = 0; i < n; i++) {
                const double *qi = q + (((int64_t)b * n + i) * Hq + h) * D;
                double *oi = out + (((int64_t)b * n + i) * Hq + h) * D;
                double m = -INFINITY;
                for (int j = 0; j < S; j++) {
                    double dot = 0.0;
                    for (int d = 0; d < D; d++) dot += qi[d] * K[(int64_t)j * D + d];
                    p[j] = dot * scale;
                    if (p[j] > m) m = p[j];
                }
                double l = 0.0;
                for (int j = 0; j < S; j++) {
                    p[j] = exp(p[j] - m);
                    l += p[j];
                }
                for (int j = 0; j < S; j++) p[j] = p[j] / l;
                for (int d = 0; d < D; d++) {
                    double o = 0.0;
                    for (int j = 0; j < S; j++) o += p[j] * V[(int64_t)j * D + d];
                    oi[d] = o;
                }
                if (lse) lse[((int64_t)(b * Hq + h)) * n + i] = m + log(l);
                if (a)
                    for (int j = 0; j < S; j++) a[j] += p[j];
            }
            free(p);
        }
}

/* Online-softmax state over the keys j with keep[b * S + j] != 0, for every (b, i, h):
 *   z_j = <q_i, K_j> * scale,  m = max z_j,  l = sum exp(z_j - m),  O~ = sum exp(z_j - m) V_j
 * (the running maximum, normaliser and unnormalised output accumulator that FACache stores;
 * O = O~ / l and m + log l are then the attention output and log-sum-exp over those keys).
 * No key kept: m = -inf, l = 0, O~ = 0.  m, l: [B, Hq, n]; o: [B, n, Hq, D]. */
void orc_attention_state(const double *q, const double *k, const double *v, const uint8_t *keep,
                         int B, int n, int Hq, int Hkv, int S, int D, double scale,
                         double *m_out, double *l_out, double *o_out)
{
    int G = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; b++)
        for (int h = 0; h < Hq; h++) {
            int g = h / G;
            const double *K = k + ((int64_t)(b * Hkv + g) * S) * D;
            const double *V = v + ((int64_t)(b * Hkv + g) * S) * D;
            const uint8_t *kp = keep + (int64_t)b * S;
            double *z = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
            for (int i = 0; i < n; i++) {
                const double *qi = q + (((int64_t)b * n + i) * Hq + h) * D;
                double *oi = o_out + (((int64_t)b * n + i) * Hq + h) * D;
                double m = -INFINITY;
                for (int j = 0; j < S; j++) {
                    if (!kp[j]) continue;
                    double dot = 0.0;
                    for (int d = 0; d < D; d++) dot += qi[d] * K[(int64_t)j * D + d];
                    z[j] = dot * scale;
                    if (z[j] > m) m = z[j];
                }
                double l = 0.0;
                for (int d = 0; d < D; d++) oi[d] = 0.0;
                for (int j = 0; j < S; j++) {
                    if (!kp[j]) continue;
                    double p = exp(z[j] - m);
                    l += p;
                    for (int d = 0; d < D; d++) oi[d] += p * V[(int64_t)j * D + d];
                }
                m_out[((int64_t)(b * Hq + h)) * n + i] = m;
                l_out[((int64_t)(b * Hq + h)) * n + i] = l;
            }
            free(z);
        }
}

/* ------------------------------------------------------------------------------------ */
/* Tracking set and drift test                                                           */
/* ------------------------------------------------------------------------------------ */

typedef struct { double a; int32_t j; } orc_rank;

static int orc_rank_cmp(const void *x, const void *y)
{
    const orc_rank *p = (const orc_rank *)x, *r = (const orc_rank *)y;
    if (p->a > r->a) return -1;          /* larger mass first */
    if (p->a < r->a) return 1;
    return (p->j < r->j) ? -1 : (p->j > r->j); /* then lower index first */
}

static int orc_int_cmp(const void *x, const void *y)
{
    int32_t p = *(const int32_t *)x, r = *(const int32_t *)y;
    return (p > r) - (p < r);
}

/* For each of P rows of a: [P, S], the k positions ranked first by (mass desc, index asc),
 * written in ascending index order to T: [P, k]; slots beyond S are -1. */
void orc_topk(const double *a, int64_t P, int S, int k, int32_t *T)
{
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < P; p++) {
        orc_rank *r = (orc_rank *)malloc(sizeof(orc_rank) * (size_t)(S > 0 ? S : 1));
        for (int j = 0; j < S; j++) { r[j].a = a[p * S + j]; r[j].j = j; }
        qsort(r, (size_t)S, sizeof(orc_rank), orc_rank_cmp);
        int take = S < k ? S : k;
        int32_t *t = T + p * k;
        for (int i = 0; i < take; i++) t[i] = r[i].j;
        qsort(t, (size_t)take, sizeof(int32_t), orc_int_cmp);
        for (int i = take; i < k; i++) t[i] = -1;
        free(r);
    }
}

/* Cosine drift of the tracked tokens.
 *   buf: [B, Hq, k, 2, D] the K and V rows saved when T was chosen (previous step)
 *   T:   [B, Hq, k] tracked positions, -1 = empty slot
 *   kc, vc: [B, Hkv, S, D] the cache after this step's refresh
 * For each (b, h): u = concat over valid slots t (in slot order) of buf K_t || V_t, and
 * w the same rows read from the cache now; sigma = <u, w> / (|u| |w|).  No valid slot:
 * sigma = 1.  |u| |w| = 0: sigma = 1 if u == w else 0.
 * refresh[b] = 1 iff min_h sigma[b, h] < gamma.                                           */
void orc_drift(const double *buf, const int32_t *T, const double *kc, const double *vc, int B,
               int Hq, int Hkv, int S, int D, int k, double gamma, double *sigma,
               uint8_t *refresh)
{
    int G = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; b++)
        for (int h = 0; h < Hq; h++) {
            int g = h / G;
            double uw = 0.0, uu = 0.0, ww = 0.0;
            int valid = 0, equal = 1;
            for (int t = 0; t < k; t++) {
                int32_t j = T[((int64_t)(b * Hq + h)) * k + t];
                if (j < 0 || j >= S) continue;
                valid++;
                const double *u = buf + (((int64_t)(b * Hq + h)) * k + t) * 2 * D;
                const double *kr = kc + (((int64_t)(b * Hkv + g)) * S + j) * D;
                const double *vr = vc + (((int64_t)(b * Hkv + g)) * S + j) * D;
                for (int part = 0; part < 2; part++) {
                    const double *w = part ? vr : kr;
                    const double *uu_ = u + part * D;
                    for (int d = 0; d < D; d++) {
                        uw += uu_[d] * w[d];
                        uu += uu_[d] * uu_[d];
                        ww += w[d] * w[d];
                        if (uu_[d] != w[d]) equal = 0;
                    }
                }
            }
            double s;
            if (!valid) s = 1.0;
            else {
                double denom = sqrt(uu) * sqrt(ww);
                s = (denom == 0.0) ? (equal ? 1.0 : 0.0) : uw / denom;
            }
            sigma[b * Hq + h] = s;
        }
    for (int b = 0; b < B; b++) {
        double mn = INFINITY;
        for (int h = 0; h < Hq; h++)
            if (sigma[b * Hq + h] < mn) mn = sigma[b * Hq + h];
        refresh[b] = (uint8_t)(mn < gamma);
    }
}
