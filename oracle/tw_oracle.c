/*
 * tw_oracle.c -- plain, slow CPU oracle for the decode-time ternary MoE FFN.
 *
 * TEST INFRASTRUCTURE ONLY (see tw_oracle.h for the pages cited, the readings taken and who may
 * load this library).  Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC.  The flag
 * -ffp-contract=off matters for the int8 spec mode: every fp32 step there is one rounding.
 *
 * Everything is written as the plain definition: loops over rows and columns, no blocking,
 * no reordering.  Threads (OpenMP) only split independent tokens.
 */
#include "tw_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static int64_t g_bad_codes = 0;

int64_t or_bad_codes(void) { return g_bad_codes; }
void or_reset_bad_codes(void) { g_bad_codes = 0; }

/* ---- packing: two bits per weight, four weights per byte -------------------------------------
 * [MacMini] "What Ternary Actually Means": four ternary weights share a single byte.
 * Reading: 00 -> 0, 01 -> +1, 10 -> -1, weight 4b+j in bits 2j..2j+1 of byte b. */

static int code_of_value(int8_t w, int64_t *bad)
{
    if (w == 0) return 0;
    if (w == 1) return 1;
    if (w == -1) return 2;
    (*bad)++;
    return 0;
}

int64_t or_pack(const int8_t *w, int64_t rows, int64_t cols, uint8_t *packed)
{
    int64_t stride = (cols + 3) / 4, bad = 0;
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t b = 0; b < stride; b++) {
            unsigned byte = 0;
            for (int j = 0; j < 4; j++) {
                int64_t i = 4 * b + j;
                if (i < cols) byte |= (unsigned)code_of_value(w[r * cols + i], &bad) << (2 * j);
            }
            packed[r * stride + b] = (uint8_t)byte;
        }
    }
    return bad;
}

/* The value of weight i of a packed row.  Code 11 is never written by or_pack; meeting it is
 * counted as an error and it contributes nothing. */
static int trit_at(const uint8_t *row, int64_t i)
{
    int c = (row[i / 4] >> (2 * (i % 4))) & 3;
    if (c == 1) return 1;
    if (c == 2) return -1;
    if (c == 3) {
#pragma omp atomic
        g_bad_codes++;
    }
    return 0;
}

int64_t or_unpack(const uint8_t *packed, int64_t rows, int64_t cols, int8_t *w)
{
    int64_t stride = (cols + 3) / 4, bad = 0;
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t i = 0; i < cols; i++) {
            int c = (packed[r * stride + i / 4] >> (2 * (i % 4))) & 3;
            if (c == 3) bad++;
            w[r * cols + i] = (int8_t)(c == 1 ? 1 : (c == 2 ? -1 : 0));
        }
    }
    return bad;
}

/* A ternary weight times a value: pass-through, negate or zero ([MacMini] "What Ternary Actually
 * Means": no multiply is needed). */
static double ternary_times(int t, double v)
{
    if (t == 1) return v;
    if (t == -1) return -v;
    return 0.0;
}

/* One ternary matrix-vector product: each output row is its per-row scale times the sum of
 * pass-through / negated / skipped inputs.  Reading: the scale multiplies after the sum. */
void or_ternary_gemv(const uint8_t *packed, int64_t rows, int64_t cols, const double *scale,
                     const double *x, double *y)
{
    int64_t stride = (cols + 3) / 4;
    for (int64_t r = 0; r < rows; r++) {
        double s = 0.0;
        for (int64_t i = 0; i < cols; i++) s += ternary_times(trit_at(packed + r * stride, i), x[i]);
        y[r] = scale[r] * s;
    }
}

/* ---- base-3 packing: five weights per byte ---------------------------------------------------
 * [Hub] "Ternary Quantization Is More Than Simply Compressing Weights into Three Values": three
 * states need at least log2 3 bits, and a packing may use another aligned form than 2 bits.
 * Reading (tw_oracle.h): byte j = sum_i (w_{5j+i} + 1) 3^i, padding positions count as weight 0,
 * bytes past ceil(cols/5) of a row are 0. */

static int digit_of_value(int8_t w, int64_t *bad)
{
    if (w == -1 || w == 0 || w == 1) return w + 1;
    (*bad)++;
    return 1;
}

int64_t or_pack3(const int8_t *w, int64_t rows, int64_t cols, int64_t row_bytes, uint8_t *packed)
{
    int64_t nb = (cols + 4) / 5, bad = 0;
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t b = 0; b < row_bytes; b++) {
            unsigned v = 0, p3 = 1;
            if (b < nb) {
                for (int i = 0; i < 5; i++) {
                    int64_t c = 5 * b + i;
                    int dg = c < cols ? digit_of_value(w[r * cols + c], &bad) : 1;
                    v += (unsigned)dg * p3;
                    p3 *= 3;
                }
            }
            packed[r * row_bytes + b] = (uint8_t)v;
        }
    }
    return bad;
}

int64_t or_unpack3(const uint8_t *packed, int64_t rows, int64_t cols, int64_t row_bytes, int8_t *w)
{
    int64_t bad = 0;
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t c = 0; c < cols; c++) {
            unsigned v = packed[r * row_bytes + c / 5];
            if (v > 242) {
                if (c % 5 == 0) bad++;
                w[r * cols + c] = 0;
                continue;
            }
            for (int64_t i = 0; i < c % 5; i++) v /= 3;
            w[r * cols + c] = (int8_t)((int)(v % 3) - 1);
        }
    }
    return bad;
}

void or_gemv_i8(const int8_t *w, const float *scale, int64_t rows, int64_t cols, const int8_t *q,
                float sx, float *y)
{
    for (int64_t r = 0; r < rows; r++) {
        int64_t acc = 0;
        for (int64_t i = 0; i < cols; i++) acc += (int64_t)w[r * cols + i] * q[i];
        y[r] = ((float)acc * sx) * scale[r];
    }
}

/* ---- decode attention over a KV cache --------------------------------------------------------
 * [MacMini] "The Architecture: Designed for the Hardware": global and 512-token sliding-window
 * attention layers.  The plain definition: scores, softmax over the cached positions, weighted sum
 * of the values (tw_oracle.h). */
void or_attention_decode(const double *q, const double *k, const double *v, int64_t n, int32_t H,
                         int32_t Hkv, int32_t dh, double *out)
{
    double *s = (double *)malloc(sizeof(double) * (n > 0 ? n : 1));
    int32_t group = H / Hkv;
    double scale = 1.0 / sqrt((double)dh);
    for (int32_t h = 0; h < H; h++) {
        int32_t g = h / group;
        double m = -INFINITY, l = 0.0;
        for (int64_t t = 0; t < n; t++) {
            double d = 0.0;
            for (int32_t i = 0; i < dh; i++) d += q[(int64_t)h * dh + i] * k[(t * Hkv + g) * dh + i];
            s[t] = d * scale;
            if (s[t] > m) m = s[t];
        }
        for (int64_t t = 0; t < n; t++) {
            s[t] = exp(s[t] - m);
            l += s[t];
        }
        for (int32_t i = 0; i < dh; i++) {
            double o = 0.0;
            for (int64_t t = 0; t < n; t++) o += s[t] * v[(t * Hkv + g) * dh + i];
            out[(int64_t)h * dh + i] = o / l;
        }
    }
    free(s);
}

/* ---- approximate output head (clustered vocabulary) ------------------------------------------
 * [MacMini] "The Architecture: Designed for the Hardware": 4-bit centroid scores pick the top
 * clusters; only their tokens get full-precision logits.  Readings in tw_oracle.h. */

static int centroid_value(const uint8_t *row, int32_t i)
{
    int nib = (i & 1) ? (row[i / 2] >> 4) : (row[i / 2] & 15);
    return nib - 8;
}

/* cluster a ranks before cluster b: higher score, or equal score and lower id */
static int cluster_before(const float *score, int32_t a, int32_t b)
{
    if (score[a] != score[b]) return score[a] > score[b];
    return a < b;
}

void or_flash_head(const float *h, int32_t d, const uint8_t *centroids, const float *c_scale,
                   int32_t ncl, const double *wc, const int32_t *member_ids, int32_t cs,
                   int32_t top, int32_t *sel, int32_t *ids, double *logits, float *scores)
{
    int8_t *q = (int8_t *)malloc(d);
    float *sc = (float *)malloc(sizeof(float) * ncl);
    int32_t *order = (int32_t *)malloc(sizeof(int32_t) * ncl);
    float sh;
    /* 1. 4-bit centroid scores against the int8 image of h */
    or_quant_absmax(h, d, q, &sh);
    for (int32_t c = 0; c < ncl; c++) {
        const uint8_t *row = centroids + (int64_t)c * (d / 2);
        int64_t acc = 0;
        for (int32_t i = 0; i < d; i++) acc += (int64_t)centroid_value(row, i) * q[i];
        sc[c] = ((float)acc * sh) * c_scale[c];
        if (scores) scores[c] = sc[c];
    }
    /* 2. the top clusters: a selection by repeated scans for the best remaining cluster */
    for (int32_t c = 0; c < ncl; c++) order[c] = c;
    for (int32_t j = 0; j < top; j++) {
        int32_t best = j;
        for (int32_t c = j + 1; c < ncl; c++)
            if (cluster_before(sc, order[c], order[best])) best = c;
        int32_t t = order[j];
        order[j] = order[best];
        order[best] = t;
        sel[j] = order[j];
    }
    /* 3. full-precision logits of the selected clusters' tokens */
    for (int32_t j = 0; j < top; j++) {
        int64_t c = sel[j];
        for (int32_t m = 0; m < cs; m++) {
            const double *wr = wc + (c * cs + m) * d;
            double acc = 0.0;
            for (int32_t i = 0; i < d; i++) acc += wr[i] * (double)h[i];
            logits[(int64_t)j * cs + m] = acc;
            ids[(int64_t)j * cs + m] = member_ids[c * cs + m];
        }
    }
    free(q);
    free(sc);
    free(order);
}

/* ---- rounding ---------------------------------------------------------------------------- */

uint16_t or_f64_to_bf16(double v)
{
    if (isnan(v)) return 0x7FC0;
    double a = fabs(v);
    double r;
    if (a == 0.0 || isinf(a)) {
        r = a;
    } else {
        int e;
        frexp(a, &e);            /* a = f * 2^e, f in [0.5, 1) */
        int ulp_exp = e - 8;     /* 8 significant bits */
        if (ulp_exp < -133) ulp_exp = -133;   /* bf16 subnormal spacing */
        double q = ldexp(a, -ulp_exp);
        r = ldexp(nearbyint(q), ulp_exp);     /* round half to even, one rounding */
        if (r >= ldexp(1.0, 128)) r = INFINITY;
    }
    float f = (float)(signbit(v) ? -r : r);   /* exact: every bf16 value is an fp32 value */
    uint32_t bits;
    memcpy(&bits, &f, 4);
    return (uint16_t)(bits >> 16);
}

void or_round_bf16_array(const double *v, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; i++) out[i] = or_f64_to_bf16(v[i]);
}

void or_round_f32_array(const double *v, int64_t n, float *out)
{
    for (int64_t i = 0; i < n; i++) out[i] = (float)v[i];
}

static double bf16_value(uint16_t b)
{
    uint32_t bits = (uint32_t)b << 16;
    float f;
    memcpy(&f, &bits, 4);
    return (double)f;
}

/* ---- truth mode -------------------------------------------------------------------------- */

/* FFN input: x itself, or x / sqrt(mean(x^2) + 1e-6) with unit weight when pre-RMSNorm is on. */
static void ffn_input(const or_layer *L, const double *x, double *xn)
{
    int d = L->d_model;
    double scale = 1.0;
    if (L->pre_rmsnorm) {
        double ss = 0.0;
        for (int i = 0; i < d; i++) ss += x[i] * x[i];
        scale = 1.0 / sqrt(ss / d + 1e-6);
    }
    for (int i = 0; i < d; i++) xn[i] = x[i] * scale;
}

/* Router logits l_e = sum_i W_r[e][i] xn_i, then the k largest (ties: lower expert id first),
 * then softmax over those k logits. */
static void route_one(const or_layer *L, const double *xn, int32_t *ids, double *gates,
                      double *logits_out)
{
    int d = L->d_model, E = L->n_experts, k = L->top_k;
    double *l = (double *)malloc(sizeof(double) * E);
    char *taken = (char *)calloc(E, 1);
    for (int e = 0; e < E; e++) {
        double s = 0.0;
        for (int i = 0; i < d; i++) s += L->w_router[(int64_t)e * d + i] * xn[i];
        l[e] = s;
    }
    for (int j = 0; j < k; j++) {
        int best = -1;
        for (int e = 0; e < E; e++)
            if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;
        taken[best] = 1;
        ids[j] = best;
    }
    double top = l[ids[0]], den = 0.0;
    for (int j = 0; j < k; j++) den += exp(l[ids[j]] - top);
    for (int j = 0; j < k; j++) gates[j] = exp(l[ids[j]] - top) / den;
    if (logits_out) memcpy(logits_out, l, sizeof(double) * E);
    free(l);
    free(taken);
}

void or_route(const or_layer *L, const double *x, int64_t n_tokens, int32_t *ids, double *gates,
              double *logits, int32_t n_threads)
{
    int d = L->d_model, E = L->n_experts, k = L->top_k;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads > 0 ? n_threads : 1)
    for (int64_t t = 0; t < n_tokens; t++) {
        double *xn = (double *)malloc(sizeof(double) * d);
        ffn_input(L, x + t * d, xn);
        route_one(L, xn, ids + t * k, gates + t * k, logits ? logits + t * E : NULL);
        free(xn);
    }
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

void or_ffn_token(const or_layer *L, const double *x, const int32_t *ids, const double *gates,
                  double *out)
{
    int d = L->d_model, F = L->d_ff, k = L->top_k;
    int64_t sg = (d + 3) / 4, sd = (F + 3) / 4;
    double *xn = (double *)malloc(sizeof(double) * d);
    double *gate = (double *)malloc(sizeof(double) * F);
    double *up = (double *)malloc(sizeof(double) * F);
    double *h = (double *)malloc(sizeof(double) * F);
    double *y = (double *)malloc(sizeof(double) * d);
    double *mix = (double *)calloc(d, sizeof(double));
    ffn_input(L, x, xn);
    for (int j = 0; j < k; j++) {
        int64_t e = ids[j];
        or_ternary_gemv(L->t_gate + e * F * sg, F, d, L->s_gate + e * F, xn, gate);
        or_ternary_gemv(L->t_up + e * F * sg, F, d, L->s_up + e * F, xn, up);
        for (int r = 0; r < F; r++) h[r] = silu(gate[r]) * up[r];
        or_ternary_gemv(L->t_down + e * d * sd, d, F, L->s_down + e * d, h, y);
        for (int r = 0; r < d; r++) mix[r] += gates[j] * y[r];
    }
    for (int r = 0; r < d; r++) out[r] = x[r] + mix[r];
    free(xn);
    free(gate);
    free(up);
    free(h);
    free(y);
    free(mix);
}

void or_moe_layer(const or_layer *L, const double *x, int64_t n_tokens, double *out,
                  int32_t *ids, double *gates, double *logits, int32_t n_threads)
{
    int d = L->d_model, E = L->n_experts, k = L->top_k;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads > 0 ? n_threads : 1)
    for (int64_t t = 0; t < n_tokens; t++) {
        double *xn = (double *)malloc(sizeof(double) * d);
        ffn_input(L, x + t * d, xn);
        route_one(L, xn, ids + t * k, gates + t * k, logits ? logits + t * E : NULL);
        or_ffn_token(L, x + t * d, ids + t * k, gates + t * k, out + t * d);
        free(xn);
    }
}

void or_decode_stack(const or_layer *layers, int32_t n_layers, const double *x0, int32_t n_steps,
                     double *layer_inputs, double *out, int32_t *ids, double *gates,
                     double *logits)
{
    int d = layers[0].d_model;
    double *cur = (double *)malloc(sizeof(double) * d);
    double *nxt = (double *)malloc(sizeof(double) * d);
    memcpy(cur, x0, sizeof(double) * d);
    for (int32_t t = 0; t < n_steps; t++) {
        for (int32_t l = 0; l < n_layers; l++) {
            const or_layer *L = &layers[l];
            int k = L->top_k, E = L->n_experts;
            int64_t sl = (int64_t)t * n_layers + l;
            int32_t idb[64];
            double gb[64];
            int32_t *pid = ids ? ids + sl * k : idb;
            double *pg = gates ? gates + sl * k : gb;
            if (layer_inputs) memcpy(layer_inputs + sl * d, cur, sizeof(double) * d);
            or_moe_layer(L, cur, 1, nxt, pid, pg, logits ? logits + sl * E : NULL, 1);
            for (int i = 0; i < d; i++) cur[i] = bf16_value(or_f64_to_bf16(nxt[i]));
        }
        memcpy(out + (int64_t)t * d, cur, sizeof(double) * d);
    }
    free(cur);
    free(nxt);
}

/* Dense brute force: unpack every selected expert into dense double matrices W = diag(s) * T and
 * evaluate textbook matrix-vector products. */
void or_dense_ffn_token(const or_layer *L, const double *x, const int32_t *ids,
                        const double *gates, double *out)
{
    int d = L->d_model, F = L->d_ff, k = L->top_k;
    int64_t sg = (d + 3) / 4, sd = (F + 3) / 4;
    double *xn = (double *)malloc(sizeof(double) * d);
    double *Wg = (double *)malloc(sizeof(double) * F * d);
    double *Wu = (double *)malloc(sizeof(double) * F * d);
    double *Wd = (double *)malloc(sizeof(double) * d * F);
    double *h = (double *)malloc(sizeof(double) * F);
    ffn_input(L, x, xn);
    for (int r = 0; r < d; r++) out[r] = x[r];
    for (int j = 0; j < k; j++) {
        int64_t e = ids[j];
        for (int r = 0; r < F; r++)
            for (int i = 0; i < d; i++) {
                Wg[(int64_t)r * d + i] = L->s_gate[e * F + r] * trit_at(L->t_gate + (e * F + r) * sg, i);
                Wu[(int64_t)r * d + i] = L->s_up[e * F + r] * trit_at(L->t_up + (e * F + r) * sg, i);
            }
        for (int r = 0; r < d; r++)
            for (int m = 0; m < F; m++)
                Wd[(int64_t)r * F + m] = L->s_down[e * d + r] * trit_at(L->t_down + (e * d + r) * sd, m);
        for (int r = 0; r < F; r++) {
            double a = 0.0, b = 0.0;
            for (int i = 0; i < d; i++) {
                a += Wg[(int64_t)r * d + i] * xn[i];
                b += Wu[(int64_t)r * d + i] * xn[i];
            }
            h[r] = a * (1.0 / (1.0 + exp(-a))) * b;
        }
        for (int r = 0; r < d; r++) {
            double c = 0.0;
            for (int m = 0; m < F; m++) c += Wd[(int64_t)r * F + m] * h[m];
            out[r] += gates[j] * c;
        }
    }
    free(xn);
    free(Wg);
    free(Wu);
    free(Wd);
    free(h);
}

/* ---- int8 spec mode ------------------------------------------------------------------------
 * Every float step below is one fp32 operation rounded to nearest-even, in the order written.
 * Integer sums are exact: |sum| <= 127 * d < 2^24, so converting one to fp32 is exact too. */

/* exp for the spec mode: Cody-Waite reduction z = n*ln2 + r with ln2 split as C1 + C2 (C1 has
 * its 12 low significand bits clear, so n*C1 is exact for |n| < 2^12), a degree-7 Taylor
 * polynomial for e^r in Horner form with fp32 coefficients 1/m!, then scaling by 2^n.
 * Outside [-80, 80] the result is fixed at 0 or +inf (no subnormal results). */
float or_spec_expf(float z)
{
    if (z > 80.0f) return INFINITY;
    if (z < -80.0f) return 0.0f;
    const float log2e = 1.44269504088896340736f;
    const float c1 = 0.693145751953125f;               /* ln2 with 12 low bits clear */
    const float c2 = (float)(0.6931471805599453094 - 0.693145751953125);
    float n = rintf(z * log2e);
    float r = z - n * c1;
    r = r - n * c2;
    float p = 1.0f / 5040.0f;
    p = p * r + 1.0f / 720.0f;
    p = p * r + 1.0f / 120.0f;
    p = p * r + 1.0f / 24.0f;
    p = p * r + 1.0f / 6.0f;
    p = p * r + 0.5f;
    p = p * r + 1.0f;
    p = p * r + 1.0f;
    return ldexpf(p, (int)n);
}

void or_quant_absmax(const float *v, int64_t n, int8_t *q, float *s)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < n; i++) {
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
        for (int64_t i = 0; i < n; i++) q[i] = 0;
        *s = 0.0f;
        return;
    }
    float inv = 127.0f / amax;
    for (int64_t i = 0; i < n; i++) {
        float t = rintf(v[i] * inv);
        if (t > 127.0f) t = 127.0f;
        if (t < -127.0f) t = -127.0f;
        q[i] = (int8_t)t;
    }
    *s = amax / 127.0f;
}

static int32_t ternary_dot_i8(const uint8_t *row, const int8_t *q, int n)
{
    int32_t s = 0;
    for (int i = 0; i < n; i++) {
        int t = trit_at(row, i);
        if (t == 1) s += q[i];
        else if (t == -1) s -= q[i];
    }
    return s;
}

void or_ffn_token_i8(const or_layer_i8 *L, const float *x, const int32_t *ids, const float *gates,
                     float *out, int8_t *qx_tap, float *sx_tap, int32_t *accg_tap,
                     int32_t *accu_tap, int8_t *qh_tap, float *sh_tap, int32_t *accd_tap,
                     float *y_tap)
{
    int d = L->d_model, F = L->d_ff, k = L->top_k;
    int64_t sg = (d + 3) / 4, sd = (F + 3) / 4;
    int8_t *qx = (int8_t *)malloc(d);
    int8_t *qh = (int8_t *)malloc(F);
    float *h = (float *)malloc(sizeof(float) * F);
    float *y = (float *)malloc(sizeof(float) * (int64_t)k * d);
    float sx, sh;
    or_quant_absmax(x, d, qx, &sx);
    if (qx_tap) memcpy(qx_tap, qx, d);
    if (sx_tap) *sx_tap = sx;
    for (int j = 0; j < k; j++) {
        int64_t e = ids[j];
        for (int r = 0; r < F; r++) {
            int32_t ag = ternary_dot_i8(L->t_gate + (e * F + r) * sg, qx, d);
            int32_t au = ternary_dot_i8(L->t_up + (e * F + r) * sg, qx, d);
            if (accg_tap) accg_tap[(int64_t)j * F + r] = ag;
            if (accu_tap) accu_tap[(int64_t)j * F + r] = au;
            float gate = ((float)ag * sx) * L->s_gate[e * F + r];
            float up = ((float)au * sx) * L->s_up[e * F + r];
            float den = 1.0f + or_spec_expf(-gate);
            float sig = gate / den;
            h[r] = sig * up;
        }
        or_quant_absmax(h, F, qh, &sh);
        if (qh_tap) memcpy(qh_tap + (int64_t)j * F, qh, F);
        if (sh_tap) sh_tap[j] = sh;
        for (int r = 0; r < d; r++) {
            int32_t ad = ternary_dot_i8(L->t_down + (e * d + r) * sd, qh, F);
            if (accd_tap) accd_tap[(int64_t)j * d + r] = ad;
            y[(int64_t)j * d + r] = ((float)ad * sh) * L->s_down[e * d + r];
        }
    }
    if (y_tap) memcpy(y_tap, y, sizeof(float) * (int64_t)k * d);
    for (int r = 0; r < d; r++) {
        float o = x[r];
        for (int j = 0; j < k; j++) {
            float c = gates[j] * y[(int64_t)j * d + r];
            o = o + c;
        }
        out[r] = o;
    }
    free(qx);
    free(qh);
    free(h);
    free(y);
}

void or_ffn_batch_i8(const or_layer_i8 *L, const float *x, int64_t n_tokens, const int32_t *ids,
                     const float *gates, float *out, int32_t n_threads)
{
    int d = L->d_model, k = L->top_k;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads > 0 ? n_threads : 1)
    for (int64_t t = 0; t < n_tokens; t++)
        or_ffn_token_i8(L, x + t * d, ids + t * k, gates + t * k, out + t * d, NULL, NULL, NULL,
                        NULL, NULL, NULL, NULL, NULL);
}

/* ---- float -> ternary quantisation (per-row absmean) ---------------------------------------
 * The pages describe ternary weights as float weights mapped onto three states with scale factors
 * kept beside them ([Hub] "Ternary Quantization Is More Than Simply Compressing Weights into Three
 * Values"), and contrast models quantised to ternary after training with ones trained ternary
 * ([MacMini] "Why Everyone Else Quantizes After Training").  They give no formula; the reading here
 * is the per-row absmean rule: g = mean_i |w_i| over the row, t_i = clamp(rint(w_i / g), -1, 1)
 * (rint: to nearest, ties to even), and g is the row's scale, so that g * t approximates w.  A row
 * of zeros gives t = 0 and g = 0.
 * The mean is the plain one: |w_i| summed in double (each fp32 value is exact in double), divided
 * by cols in double and rounded once to fp32; q_i = w_i / g is one fp32 division.  No summation
 * order is implied by the pages, so none is imitated here. */

int or_quantize_absmean(const float *w, int64_t rows, int64_t cols, int8_t *t, float *scale)
{
    if (cols <= 0) return cols == 0 ? 0 : -1;
    for (int64_t r = 0; r < rows; r++) {
        const float *row = w + r * cols;
        double sum = 0.0;
        for (int64_t i = 0; i < cols; i++) sum += fabs((double)row[i]);
        float g = (float)(sum / (double)cols);
        int8_t *tr = t + r * cols;
        if (g == 0.0f) {
            for (int64_t i = 0; i < cols; i++) tr[i] = 0;
            scale[r] = 0.0f;
            continue;
        }
        for (int64_t i = 0; i < cols; i++) {
            float q = rintf(row[i] / g);
            if (q > 1.0f) q = 1.0f;
            if (q < -1.0f) q = -1.0f;
            tr[i] = (int8_t)q;
        }
        scale[r] = g;
    }
    return 0;
}
