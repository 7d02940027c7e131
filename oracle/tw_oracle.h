/*
 * tw_oracle.h -- plain CPU oracle for the decode-time ternary mixture-of-experts FFN.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load this library.  The product library never links, loads or calls it, and it
 * shares no code, header, table or constant with the product's HIP sources.
 *
 * Pages cited (titles as printed on them):
 *   [MacMini]  "A 20B AI Model Trained in Ternary Just Hit 218 Tokens/Second on a $599 Mac Mini"
 *   [iPhone20B] "How a 20B Model Hits 120 tok/s on an iPhone"
 *   [Hub]      "iPhone Runs a 20B Model at 120 tok/s"
 *   [Mobile]   "Optimizing 20B MoE Models for Mobile: The Maple-Preview Breakthrough"
 *
 * What the pages fix: weights are exactly -1, 0 or +1, so each product is a negate, a zero or a
 * pass-through ([MacMini] "What Ternary Actually Means"; [Mobile] "The Magic of Ternary
 * Quantization"); four weights share one byte ([MacMini] "What Ternary Actually Means"); the dot
 * products accumulate in FP32 with no dequantised matrix ([MacMini] "The Architecture: Designed for
 * the Hardware"); a router picks 8 of 256 experts per token ([MacMini] "The Architecture";
 * [iPhone20B] opening section).
 *
 * What the pages leave open and is read here (each reading is restated where it is used):
 *   - code values 00 -> 0, 01 -> +1, 10 -> -1; code 11 is never produced and is rejected here;
 *   - weight 4b+j of a row sits in bits 2j..2j+1 of byte b (LSB first); a row is one output
 *     channel, its inputs contiguous, stride ceil(cols/4) bytes, padding code 00;
 *   - one fp32 scale per output row, applied after the ternary sum;
 *   - expert = SiLU-gated: h = SiLU(s_g * (T_g x)) * (s_u * (T_u x)); y = s_d * (T_d h);
 *   - routing: logits l = W_r x (no bias), top-k by (l descending, expert id ascending),
 *     gates = softmax over the k selected logits;
 *   - out = x + sum_j g_j y_{id_j}, j in selection order, one final rounding;
 *   - optional pre-RMSNorm (unit weight, eps 1e-6) on the FFN input for the stacked decode;
 *   - int8 "spec" mode: per-vector absmax quantisation to [-127,127], int32 sums, every float
 *     step one round-to-nearest fp32 operation in a fixed order, and a fixed exp (spec_expf).
 *
 * Modes:
 *   truth (or_*):      exact inputs widened to double; every sum in double; one rounding at the end.
 *   int8 spec (or_*_i8): the fixed fp32 operation sequence; bit-exact target for the int8 path.
 */
#ifndef TW_ORACLE_H
#define TW_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Number of invalid codes (11) met by any oracle routine since the last reset. */
int64_t or_bad_codes(void);
void or_reset_bad_codes(void);

/* ---- packing ------------------------------------------------------------------------------ */
/* Packs rows x cols int8 values into rows x ceil(cols/4) bytes.  Returns the number of inputs
 * outside {-1,0,+1}; each of those is written as code 00. */
int64_t or_pack(const int8_t *w, int64_t rows, int64_t cols, uint8_t *packed);
/* Unpacks to int8.  Returns the number of 11 codes met; each is written as 0. */
int64_t or_unpack(const uint8_t *packed, int64_t rows, int64_t cols, int8_t *w);

/* y_r = scale_r * sum_i T[r][i] * x_i for a packed [rows][ceil(cols/4)] matrix (double). */
void or_ternary_gemv(const uint8_t *packed, int64_t rows, int64_t cols, const double *scale,
                     const double *x, double *y);

/* ---- base-3 packing: five weights per byte ---------------------------------------------------
 * A ternary weight carries log2 3 = 1.585 bits; packings that hardware reads natively spend 2 bits
 * or another aligned form ([Hub] "Ternary Quantization Is More Than Simply Compressing Weights into
 * Three Values"; [MacMini] "What Ternary Actually Means": 1.58 bits per weight).  Five trits fit in
 * a byte because 3^5 = 243 <= 256 (1.6 bits per weight).
 * Reading: byte j of a row holds weights 5j .. 5j+4 as sum_i (w_{5j+i} + 1) 3^i (weight 5j is the
 * least significant trit); positions at or past cols count as weight 0; a row occupies row_bytes
 * bytes (row_bytes >= ceil(cols/5)) and its bytes past ceil(cols/5) are 0.
 * or_pack3 returns the number of inputs outside {-1,0,+1} (each packed as 0); or_unpack3 returns
 * the number of content bytes above 242 (each unpacked as five zeros). */
int64_t or_pack3(const int8_t *w, int64_t rows, int64_t cols, int64_t row_bytes, uint8_t *packed);
int64_t or_unpack3(const uint8_t *packed, int64_t rows, int64_t cols, int64_t row_bytes, int8_t *w);

/* int8 spec of one ternary matrix-vector product on unpacked weights w [rows][cols] in {-1,0,+1}:
 * y_r = ((float) sum_i w[r][i] q_i * sx) * scale_r, the sum exact in integers, then two fp32
 * roundings in that order (the order of the int8 FFN below). */
void or_gemv_i8(const int8_t *w, const float *scale, int64_t rows, int64_t cols, const int8_t *q,
                float sx, float *y);

/* ---- decode attention over a KV cache --------------------------------------------------------
 * The pages' model interleaves sliding-window attention (window 512) with global attention at 3:1
 * (6 global, 18 windowed layers), which bounds the cache of the windowed layers ([MacMini] "The
 * Architecture: Designed for the Hardware"; [iPhone20B] opening section).  Reading: one query token
 * attends, per query head h, over n cached positions of KV head h / (H / Hkv) (grouped-query):
 * out_h = sum_t softmax_t(q_h . k_t / sqrt(dh)) v_t.  A windowed layer keeps its last `window`
 * positions in a ring of `window` slots, so it attends over its min(ctx, window) filled slots; the
 * sum does not depend on the slot order.  q [H][dh], k and v [n][Hkv][dh], out [H][dh]; everything
 * in double, exp from the C library, max-subtracted. */
void or_attention_decode(const double *q, const double *k, const double *v, int64_t n, int32_t H,
                         int32_t Hkv, int32_t dh, double *out);

/* ---- approximate output head (clustered vocabulary) ------------------------------------------
 * [MacMini] "The Architecture: Designed for the Hardware": the output head is the costliest step of
 * decode; the vocabulary (about 151,000 tokens) is split into 4,748 clusters, 4-bit centroid
 * scores pick the 512 most relevant clusters, and only their tokens get full-precision logits.
 * Readings: clusters of cs tokens whose head rows are stored cluster-major, wc [ncl][cs][d], with
 * member_ids [ncl][cs] giving each row's token id; centroids [ncl][d/2] bytes, element 2k in the low
 * nibble of byte k and 2k+1 in the high nibble, each nibble the value + 8 (values -8..7), one fp32
 * scale per centroid.  Scoring: h quantised by absmax to int8 (or_quant_absmax), acc_c = exact
 * sum_i value_c,i q_i, score_c = ((float) acc_c * s_h) * scale_c (two fp32 roundings).  Selection:
 * the `top` clusters by (score descending, cluster id ascending).  Logits: sum_i w[v][i] h_i in
 * double for every token of the selected clusters, in selection order then member order.
 * Outputs: sel [top], ids and logits [top][cs]; scores [ncl] (nullable tap). */
void or_flash_head(const float *h, int32_t d, const uint8_t *centroids, const float *c_scale,
                   int32_t ncl, const double *wc, const int32_t *member_ids, int32_t cs,
                   int32_t top, int32_t *sel, int32_t *ids, double *logits, float *scores);

/* ---- rounding ----------------------------------------------------------------------------- */
/* Round-to-nearest-even of a double straight to bfloat16 (one rounding), returned as raw bits. */
uint16_t or_f64_to_bf16(double v);
void or_round_bf16_array(const double *v, int64_t n, uint16_t *out);
void or_round_f32_array(const double *v, int64_t n, float *out);

/* ---- one layer, truth mode ---------------------------------------------------------------- */
typedef struct {
    int32_t d_model, d_ff, n_experts, top_k;
    int32_t pre_rmsnorm;        /* 1: FFN input is x / sqrt(mean(x^2) + 1e-6) */
    const double *w_router;     /* [E][d] exact values */
    const uint8_t *t_gate;      /* [E][F][ceil(d/4)] packed */
    const uint8_t *t_up;        /* [E][F][ceil(d/4)] packed */
    const uint8_t *t_down;      /* [E][d][ceil(F/4)] packed */
    const double *s_gate;       /* [E][F] */
    const double *s_up;         /* [E][F] */
    const double *s_down;       /* [E][d] */
} or_layer;

/* Router for n_tokens tokens.  x [T][d].  Outputs ids [T][k], gates [T][k];
 * logits [T][E] (nullable) are the FFN-input logits in double. */
void or_route(const or_layer *L, const double *x, int64_t n_tokens,
              int32_t *ids, double *gates, double *logits, int32_t n_threads);

/* Expert FFN plus combine for one token under a given routing: out = x + sum_j g_j y_{ids_j}. */
void or_ffn_token(const or_layer *L, const double *x, const int32_t *ids, const double *gates,
                  double *out);

/* Route + FFN for n_tokens tokens, out [T][d] in double (unrounded). */
void or_moe_layer(const or_layer *L, const double *x, int64_t n_tokens, double *out,
                  int32_t *ids, double *gates, double *logits, int32_t n_threads);

/* Chained decode: n_steps steps through n_layers layers, batch 1.  Each layer's output is
 * rounded to bfloat16 and is the next layer's input; the last layer's output of step t is the
 * input of step t+1.  x0 [d] exact.  layer_inputs [n_steps][n_layers][d] (nullable) receives
 * every layer's (bf16-exact) input; out [n_steps][d] the outputs; ids/gates/logits per
 * (step, layer) are nullable. */
void or_decode_stack(const or_layer *layers, int32_t n_layers, const double *x0, int32_t n_steps,
                     double *layer_inputs, double *out, int32_t *ids, double *gates,
                     double *logits);

/* Dense brute force (self-check): W = diag(s) * T built densely, then textbook products. */
void or_dense_ffn_token(const or_layer *L, const double *x, const int32_t *ids,
                        const double *gates, double *out);

/* ---- float -> ternary quantisation ----------------------------------------------------------
 * Per row: g = mean |w| (summed in double, rounded once to fp32), t = clamp(rint(w / g), -1, 1)
 * with one fp32 division, scale = g; zero rows give t = 0, g = 0.  Returns 0 (-1 if cols < 0). */
int or_quantize_absmean(const float *w, int64_t rows, int64_t cols, int8_t *t, float *scale);

/* ---- int8 spec mode ----------------------------------------------------------------------- */
float or_spec_expf(float z);
/* absmax quantisation of n fp32 values: q in [-127,127], scale s (0 when all inputs are 0). */
void or_quant_absmax(const float *v, int64_t n, int8_t *q, float *s);

typedef struct {
    int32_t d_model, d_ff, n_experts, top_k;
    const uint8_t *t_gate, *t_up, *t_down;   /* as in or_layer */
    const float *s_gate, *s_up, *s_down;     /* fp32 scales */
} or_layer_i8;

/* One token of the int8 path under a given routing (ids, fp32 gates).  x [d] fp32 values.
 * out [d] fp32.  Taps (all nullable): qx [d], sx [1], acc_gate/acc_up [k][F], qh [k][F], sh [k],
 * acc_down [k][d], y [k][d]. */
void or_ffn_token_i8(const or_layer_i8 *L, const float *x, const int32_t *ids, const float *gates,
                     float *out, int8_t *qx, float *sx, int32_t *acc_gate, int32_t *acc_up,
                     int8_t *qh, float *sh, int32_t *acc_down, float *y);

/* n_tokens tokens of the int8 path.  x [T][d], ids/gates [T][k], out [T][d] fp32. */
void or_ffn_batch_i8(const or_layer_i8 *L, const float *x, int64_t n_tokens, const int32_t *ids,
                     const float *gates, float *out, int32_t n_threads);

#ifdef __cplusplus
}
#endif
#endif
