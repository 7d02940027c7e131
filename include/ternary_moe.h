/*
 * ternary_moe.h -- C ABI of libternary_moe.so: the decode-time ternary mixture-of-experts FFN on
 * AMD Instinct MI355X (gfx950).
 *
 * Pages cited (titles as printed):
 *   [MacMini]   "A 20B AI Model Trained in Ternary Just Hit 218 Tokens/Second on a $599 Mac Mini"
 *   [iPhone20B] "How a 20B Model Hits 120 tok/s on an iPhone"
 *   [Hub]       "iPhone Runs a 20B Model at 120 tok/s"
 *
 * What one layer computes, per token x (d_model values):
 *   router logits  l = W_r xn            W_r [E][d], no bias; xn = x, or x / sqrt(mean(x^2)+1e-6)
 *                                         when the layer has a pre-RMSNorm (unit weight)
 *   routing        ids = the top_k experts by (l descending, expert id ascending);
 *                  g_j = softmax over the top_k selected logits  (router choosing a few experts
 *                  per token: [Hub] "MoE Is the Other Half of the Story Behind the 20B Figure";
 *                  8 of 256: [MacMini] "The Architecture: Designed for the Hardware")
 *   per expert e = ids_j:
 *                  gate = s_g[e] * (T_g[e] xn),  up = s_u[e] * (T_u[e] xn)   (ternary GEMV)
 *                  h    = SiLU(gate) * up,        SiLU(z) = z / (1 + e^-z)
 *                  y_j  = s_d[e] * (T_d[e] h)                                  (ternary GEMV)
 *   output         out = x + sum_j g_j y_j  (j in selection order)
 * Every weight is -1, 0 or +1, so each product is a pass-through, a negation or a skip, and sums
 * accumulate without any dequantised weight matrix in memory ([MacMini] "What Ternary Actually
 * Means" and "The Architecture: Designed for the Hardware").  The pages leave the expert's form,
 * the gating function and the scale granularity open; the reading above (SiLU-gated expert, softmax
 * over the selected logits, one fp32 scale per output row) is the one this library implements.
 *
 * Packed ternary layout (four weights per byte, [MacMini] "What Ternary Actually Means"):
 *   code 00 = 0, 01 = +1, 10 = -1 (11 never written; read as 0); weight 4b+j of a row in bits
 *   2j..2j+1 of byte b; a row is one output channel with its inputs contiguous; row stride
 *   ceil(cols/4) bytes; expert-major: T_g, T_u [E][F][d/4], T_d [E][d][F/4].
 *
 * Conventions for every entry point:
 *   - Every pointer argument except `layers`/`layer` themselves is a DEVICE pointer (memory from
 *     hipMalloc or torch CUDA tensors).  The tw_moe_layer structs live in HOST memory; they are read
 *     during the call only, and their values are copied into kernel arguments.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null stream).  They never
 *     synchronize, allocate, free or read device memory on the host, so they can be captured into
 *     a hipGraph.  The caller owns every buffer; the library keeps no pointer after the call returns
 *     (kernels already queued still use them).
 *   - Arguments are checked on the host before any HIP call; a failed check returns an error code
 *     and launches nothing.  Launch failures return TW_E_HIP.  Nothing throws across the ABI.
 *   - A workspace belongs to one in-flight call at a time; two calls in flight on different
 *     streams must use different workspaces.  Its contents need no initialisation.
 *   - Supported shapes: d_model and d_ff powers of two in [64, 4096]; 1 <= top_k <= min(E, 32);
 *     n_experts in [1, 1024].  Packed weights, scales, router weights and the activations of the
 *     routing and batched calls must be 16-byte aligned, workspaces 256-byte aligned (torch
 *     allocations are).  Others return TW_E_UNSUPPORTED.
 */
#ifndef TERNARY_MOE_H
#define TERNARY_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TW_OK = 0,
    TW_E_NULL = -1,         /* a required pointer is NULL */
    TW_E_SHAPE = -2,        /* negative or inconsistent sizes */
    TW_E_DTYPE = -3,        /* unknown dtype / activation mode */
    TW_E_WORKSPACE = -4,    /* workspace smaller than the *_workspace_bytes query */
    TW_E_ALIAS = -5,        /* output overlaps an input it must not overlap */
    TW_E_UNSUPPORTED = -6,  /* valid but outside what the kernels implement */
    TW_E_HIP = -7           /* a HIP launch reported an error */
} tw_status;

typedef enum { TW_F32 = 0, TW_BF16 = 1 } tw_float;      /* element types of float tensors */
typedef enum { TW_ACT_FLOAT = 0, TW_ACT_INT8 = 1 } tw_act;

/* One layer's parameters.  All pointers are device pointers. */
typedef struct {
    int32_t d_model;        /* d */
    int32_t d_ff;           /* F, width of one expert */
    int32_t n_experts;      /* E */
    int32_t top_k;          /* k */
    int32_t router_dtype;   /* tw_float of w_router */
    int32_t pre_rmsnorm;    /* 1: the FFN input is x / sqrt(mean(x^2) + 1e-6); residual un-normed */
    const void *w_router;   /* [E][d] router_dtype, row-major */
    const uint8_t *w_gate;  /* [E][F][d/4] packed codes */
    const uint8_t *w_up;    /* [E][F][d/4] packed codes */
    const uint8_t *w_down;  /* [E][d][F/4] packed codes */
    const float *s_gate;    /* [E][F] per-row scales */
    const float *s_up;      /* [E][F] */
    const float *s_down;    /* [E][d] */
} tw_moe_layer;

/* Human-readable name of a status code (static string, never NULL). */
const char *tw_status_str(tw_status status);

/*
 * ternary_pack -- pack int8 weights with values in {-1, 0, +1} into the 2-bit layout above.
 *   w         [rows][cols] int8, device, row-major.
 *   packed    [rows][ceil(cols/4)] uint8, device, written in full (padding weights get code 00).
 *   bad_count nullable device int32: incremented (atomically) by the number of inputs outside
 *             {-1,0,1}; each such input is packed as 0.  Not cleared by the call.
 *   Errors: TW_E_NULL (w or packed NULL with rows*cols > 0), TW_E_SHAPE (rows or cols < 0),
 *   TW_E_ALIAS (packed overlaps w).  rows == 0 or cols == 0 is a no-op.
 *   Source: four weights per byte, [MacMini] "What Ternary Actually Means".
 */
tw_status ternary_pack(const int8_t *w, int64_t rows, int64_t cols, uint8_t *packed,
                       int32_t *bad_count, void *stream);

/*
 * ternary_quantize -- float weights to the packed ternary layout above with one scale per row, by
 * the per-row absmean rule: g = mean_i |w_i|, t_i = clamp(rint(w_i / g), -1, 1) (rint: nearest,
 * ties to even), scale = g, so that scale * T approximates the row; a row of zeros gives codes 0
 * and scale 0.  The codes and scales are the w_gate/w_up/w_down and s_gate/s_up/s_down operands of
 * tw_moe_layer (row = output channel).
 *   w        [rows][cols] in w_dtype (TW_F32 or TW_BF16), device, row-major.
 *   packed   [rows][cols/4] uint8 output, device; scales [rows] fp32 output, device.
 *   Precision: because g decides integer codes, the sum of |w_i| is taken in one fixed fp32 order
 *   (the row in 8-element chunks; partial p < 256 adds chunks p, p + 256, ... in order; partials
 *   64m..64m+63 by a balanced pairwise tree into s_m; sum = (s_0 + s_1) + (s_2 + s_3)); g = sum /
 *   cols and w_i / g are correctly rounded fp32 divisions.  Equal inputs give equal codes on any
 *   device and in any call.
 *   Errors: TW_E_SHAPE (rows or cols < 0), TW_E_DTYPE, TW_E_NULL, TW_E_UNSUPPORTED (cols not a
 *   multiple of 8 or above 65536; w or packed not 16-byte aligned; scales not 4-byte aligned),
 *   TW_E_ALIAS (any two of w, packed, scales overlap).  rows == 0 or cols == 0 is a no-op.
 *   Source: ternary weights as float weights mapped onto three states with scale factors kept
 *   beside them, [Hub] "Ternary Quantization Is More Than Simply Compressing Weights into Three
 *   Values"; models quantised to ternary after training, [MacMini] "Why Everyone Else Quantizes
 *   After Training".  The pages give no formula; the absmean rule is the reading taken here.
 */
tw_status ternary_quantize(const void *w, int32_t w_dtype, int64_t rows, int64_t cols,
                           uint8_t *packed, float *scales, void *stream);

/*
 * ternary_pack3_row_bytes -- bytes per row of the base-3 layout: ceil(cols/5) rounded up to a
 *   multiple of 16 (416 for 2048 weights, against 512 in the 2-bit layout); -1 if cols < 0.
 * ternary_pack3 -- pack int8 weights with values in {-1, 0, +1} five per byte (3^5 = 243 <= 256,
 *   1.6 bits per weight): byte j of a row holds weights 5j .. 5j+4 as sum_i (w_{5j+i} + 1) 3^i,
 *   weight 5j the least significant trit; positions at or past cols count as weight 0; the bytes of
 *   a row past ceil(cols/5) are 0.
 *   w         [rows][cols] int8, device, row-major.
 *   packed    [rows][ternary_pack3_row_bytes(cols)] uint8, device, written in full.
 *   bad_count nullable device int32: incremented (atomically) by the number of inputs outside
 *             {-1,0,1}; each such input is packed as 0.  Not cleared by the call.
 *   Errors: TW_E_NULL, TW_E_SHAPE (rows or cols < 0, rows * cols above 2^40), TW_E_ALIAS (packed
 *   or bad_count overlapping an input or each other).  rows == 0 or cols == 0 is a no-op.
 *   Source: a ternary weight needs at least log2 3 = 1.585 bits, and the packing may use another
 *   aligned representation than 2 bits, [Hub] "Ternary Quantization Is More Than Simply
 *   Compressing Weights into Three Values"; 1.58 bits per weight, [MacMini] "What Ternary Actually
 *   Means".  The byte layout is the reading taken here.
 */
int64_t ternary_pack3_row_bytes(int64_t cols);
tw_status ternary_pack3(const int8_t *w, int64_t rows, int64_t cols, uint8_t *packed,
                        int32_t *bad_count, void *stream);

/*
 * ternary_gemv_i8 -- one ternary matrix-vector product with int8 activations, from either packed
 * layout: y_r = (float(sum_i W[r][i] q_i) * x_scale) * scales_r, the sum exact in int32, then two
 * fp32 roundings in that order (the order of the int8 batched FFN's gate, up and down values).
 *   codes    layout 2: [rows][cols/4] as written by ternary_pack (cols a multiple of 64, at most
 *            4096); layout 3: [rows][ternary_pack3_row_bytes(cols)] as written by ternary_pack3
 *            (cols at most 5120).  Device, 16-byte aligned.
 *   scales   [rows] fp32, device.   xq [cols] int8 codes, device.   x_scale one fp32, device.
 *   y        [rows] fp32 output, device.
 *   Bytes 243..255 in base-3 codes (never written by ternary_pack3) contribute nothing.
 *   Errors: TW_E_NULL, TW_E_SHAPE (rows or cols < 0), TW_E_DTYPE (layout not 2 or 3),
 *   TW_E_UNSUPPORTED (cols outside the limits above, codes not 16-byte aligned, scales, y or
 *   x_scale not 4-byte aligned), TW_E_ALIAS (y overlapping an input).  rows == 0 is a no-op.
 *   Source: the ternary matrix-vector product of one decode step, in which each weight passes
 *   its input through, negates it or skips it, [MacMini] "What Ternary Actually Means".
 */
tw_status ternary_gemv_i8(const uint8_t *codes, int32_t layout, const float *scales, int64_t rows,
                          int64_t cols, const int8_t *xq, const float *x_scale, float *y,
                          void *stream);

/*
 * attention_decode_workspace_bytes -- workspace bytes of attention_decode for n_heads query heads
 *   of head_dim 128 over n_slots cached positions (0 when the arguments are invalid).
 * attention_decode -- one query token attending over a KV cache:
 *   out_h = sum_t softmax_t(q_h . k_t / sqrt(head_dim)) v_t over the n_slots cached positions t,
 *   query head h reading KV head h / (n_heads / n_kv_heads) (grouped-query attention).
 *   q        [n_heads][head_dim] bf16, device (after any rotary embedding).
 *   k_cache, v_cache  [n_slots][n_kv_heads][head_dim] bf16, device: the filled slots of a layer's
 *            cache.  A global layer holds one slot per position; a sliding-window layer keeps its
 *            last `window` positions in a ring of `window` slots and passes min(positions, window)
 *            slots.  The result does not depend on the slot order.
 *   out      [n_heads][head_dim] fp32 output, device.
 *   workspace  device, 256-byte aligned, at least attention_decode_workspace_bytes bytes.
 *   Sums in fp32; the softmax is max-subtracted per split of 16 slots and the splits are merged
 *   with exp(m_s - M) rescaling.
 *   Limits: head_dim 128; n_heads / n_kv_heads in {1, 2, 4, 8}; n_heads <= 128; 1 <= n_slots <=
 *   2^21.  Errors: TW_E_NULL, TW_E_SHAPE (n_slots < 1 or above 2^21, heads < 1, n_heads not a
 *   multiple of n_kv_heads), TW_E_UNSUPPORTED (limits above, q/k/v not 16-byte aligned, out not
 *   4-byte aligned, workspace not 256-byte aligned), TW_E_WORKSPACE, TW_E_ALIAS (out or workspace
 *   overlapping an input or each other).
 *   Source: interleaved sliding-window (512 tokens) and global attention at 3:1, 6 global and 18
 *   windowed layers, [MacMini] "The Architecture: Designed for the Hardware"; [iPhone20B] opening
 *   section.  Head counts and head size are not given by the pages; 16 query heads over 4 KV heads
 *   of 128 (16 x 128 = d_model 2048) is the shape tested and measured here.
 */
size_t attention_decode_workspace_bytes(int32_t n_heads, int32_t head_dim, int64_t n_slots);
tw_status attention_decode(const void *q, const void *k_cache, const void *v_cache, int64_t n_slots,
                           int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, float *out,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * attention_decode_one_workspace_bytes -- workspace bytes of attention_decode_one (0 when the
 *   arguments are invalid or n_slots is above 1024).
 * attention_decode_one -- the operation of attention_decode in one kernel launch instead of two,
 *   for at most 1024 cached slots (64 splits of 16).  The split workgroups publish their partial
 *   (max, sum, 128 outputs) per query head as 64-bit words, each an fp32 value beside a 32-bit tag
 *   that names the call; one workgroup per query head, last in the grid, waits until its words carry
 *   the call's tag and merges them in attention_decode's order, so the outputs are the same bits as
 *   attention_decode's.  Arguments, layouts and errors as attention_decode, with the workspace size
 *   of attention_decode_one_workspace_bytes and TW_E_UNSUPPORTED above 1024 slots.
 *   Workspace contract (unlike the other calls): zero-filled before its first call (for example by
 *   hipMemsetAsync) and used by no other call; every call that completes writes zeros back over the
 *   words it used.  Calls on one workspace must not overlap.  A wait that runs out (only if a split
 *   workgroup never ran) leaves NaN in that head's output and the head's words in place.
 *   Source: as attention_decode.
 */
size_t attention_decode_one_workspace_bytes(int32_t n_heads, int32_t head_dim, int64_t n_slots);
tw_status attention_decode_one(const void *q, const void *k_cache, const void *v_cache, int64_t n_slots,
                               int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, float *out,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * flash_head_workspace_bytes -- workspace bytes of flash_head for n_clusters clusters (0 if invalid).
 * flash_head -- approximate output head over a clustered vocabulary: 4-bit centroid scores pick
 * the `top` most relevant clusters, and only their tokens get full-precision logits.
 *   h            [d] bf16 hidden state, device.  d in {512, 1024, 2048, 4096}.
 *   centroids    [n_clusters][d/2] uint8, device, 16-byte aligned: element 2k of a centroid in the
 *                low nibble of byte k, 2k+1 in the high nibble, each nibble the value + 8 (values
 *                -8..7).   centroid_scales [n_clusters] fp32, device.
 *   w_clustered  [n_clusters][cluster_size][d] bf16, device, 16-byte aligned: the head's rows in
 *                cluster-major order.   member_ids [n_clusters][cluster_size] int32: the token id
 *                of each of those rows.
 *   sel_clusters [top] int32 output: the selected clusters, by score descending, ties to the lower
 *                cluster id.   token_ids, logits [top][cluster_size] int32 / fp32 outputs: the
 *                selected clusters' tokens in that order and, per cluster, in row order.
 *   Scores: h is quantised by absmax to int8 (q = clamp(rint(h * (127 / amax)), -127, 127),
 *   s_h = amax / 127), acc = exact sum_i value_i q_i, score = (float(acc) * s_h) * scale, in that
 *   order (so equal inputs select equal clusters on any device).  Logits: fp32 sums of bf16 x bf16
 *   products.
 *   Limits: 1 <= n_clusters <= 8192, 1 <= cluster_size <= 1024, 1 <= top <= n_clusters.
 *   Errors: TW_E_NULL, TW_E_SHAPE (sizes out of those ranges), TW_E_UNSUPPORTED (d, alignment:
 *   centroids and w_clustered 16 bytes, h 2, scales/ids/outputs 4, workspace 256), TW_E_WORKSPACE,
 *   TW_E_ALIAS (an output or the workspace overlapping an input or another output).
 *   Source: the approximate output head, [MacMini] "The Architecture: Designed for the Hardware"
 *   (about 151,000 tokens in 4,748 clusters, top 512 clusters by 4-bit centroid scores, full
 *   precision only inside them).  The layouts and the int8 image of h are the readings taken here.
 */
size_t flash_head_workspace_bytes(int32_t n_clusters);
tw_status flash_head(const void *h, int32_t d, const uint8_t *centroids,
                     const float *centroid_scales, int32_t n_clusters, const void *w_clustered,
                     const int32_t *member_ids, int32_t cluster_size, int32_t top,
                     int32_t *sel_clusters, int32_t *token_ids, float *logits, void *workspace,
                     size_t workspace_bytes, void *stream);

/*
 * moe_route_topk -- router logits, top-k selection and softmax gates for n_tokens tokens.
 *   x          [T][d] in x_dtype (TW_F32 or TW_BF16).
 *   w_router   [E][d] in w_dtype.
 *   pre_rmsnorm  1: logits of x / sqrt(mean(x^2) + 1e-6).
 *   logits     [T][E] fp32 output (the logits the selection used).
 *   expert_ids [T][k] int32 output, in selection order (descending logit, ties to the lower id).
 *   gate_w     [T][k] fp32 output, softmax over the k selected logits (sums to 1).
 *   Sums accumulate in fp32.  Errors: TW_E_NULL, TW_E_SHAPE (T < 0, k > E, k < 1), TW_E_DTYPE,
 *   TW_E_UNSUPPORTED (shape limits above), TW_E_ALIAS (an output overlapping another output).
 *   Source: routing of a token to a few experts, [Hub] "MoE Is the Other Half of the Story Behind
 *   the 20B Figure"; 8 of 256 experts per token, [MacMini] "The Architecture: Designed for the
 *   Hardware".
 */
tw_status moe_route_topk(const void *x, int32_t x_dtype, const void *w_router, int32_t w_dtype,
                         int64_t n_tokens, int32_t d_model, int32_t n_experts, int32_t top_k,
                         int32_t pre_rmsnorm, float *logits, int32_t *expert_ids, float *gate_w,
                         void *stream);

/*
 * ternary_moe_ffn_decode -- batch-1 decode through n_layers consecutive layers (the layer above,
 * applied n_layers times; layer i's output is layer i+1's input).
 *   layers     host array of n_layers descriptors (1 <= n_layers <= 64), equal shapes and dtypes.
 *   x_in       [d] in io_dtype; x_out [d] in io_dtype, must not overlap x_in.
 *   io_dtype   TW_F32 or TW_BF16; between layers the residual is rounded to io_dtype, exactly as if
 *              the layers were called one at a time.
 *   workspace  device memory of at least ternary_moe_decode_workspace_bytes(layers, n_layers).
 *   Float arithmetic: ternary sums are exact integer sums of the activations split into int8
 *   digits under a power-of-two scale (2 digits for bf16 I/O, 3 for fp32 I/O), then scaled in
 *   fp32; everything else is fp32.  Errors: as moe_route_topk, plus TW_E_WORKSPACE, TW_E_ALIAS.
 *   Source: one decode step is a sequence of matrix-vector products that stream the active
 *   weights, [MacMini] "What Ternary Actually Means"; 24 layers, [iPhone20B] opening section.
 */
tw_status ternary_moe_ffn_decode(const tw_moe_layer *layers, int32_t n_layers, const void *x_in,
                                 void *x_out, int32_t io_dtype, void *workspace, size_t ws_bytes,
                                 void *stream);
size_t ternary_moe_decode_workspace_bytes(const tw_moe_layer *layers, int32_t n_layers);

/*
 * ternary_moe_decode_error_offset -- byte offset, inside a decode workspace for these layers, of a
 * uint32 health word.  Every ternary_moe_ffn_decode call clears it first (in stream order).  The
 * one-launch stacked decode keeps all its workgroups resident and hands vectors between them
 * through polled words; each wait is bounded (about 2^21 polls), and a wait that runs out, which
 * happens only when the GPU cannot hold every workgroup of the launch at once (for instance while
 * other work occupies its compute units, or while another such decode runs on a second stream:
 * keep these calls on one stream per device), ends the launch early, sets the word nonzero and
 * leaves x_out undefined.  The caller may read it after the call has completed.  Returns 0 for layers that
 * ternary_moe_decode_workspace_bytes rejects (the word never sits at offset 0).
 * Source: not a step of the method; a property of the persistent kernel that serves it.
 */
size_t ternary_moe_decode_error_offset(const tw_moe_layer *layers, int32_t n_layers);

/*
 * ternary_moe_ffn_decode_static -- ternary_moe_ffn_decode without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  The call allocates nothing: its workspace is a scratch array of
 * TW_STATIC_SCRATCH_BYTES (2 MiB) that the library holds in each device's memory from its first
 * call on that device until the process ends; the 24-layer d_model 2048 / 256 experts / width 512
 * / top-8 stack needs about 0.8 MiB of it.  Results equal ternary_moe_ffn_decode's bit for bit (the same
 * kernels run).
 *   layers, n_layers, x_in, x_out, io_dtype, stream: as ternary_moe_ffn_decode.
 *   health     nullable device uint32 (4-byte aligned): receives the call's health word (see
 *              ternary_moe_decode_error_offset) once the call completes in stream order.
 *   Every call on one device shares that device's scratch, which keeps the last call's contents
 *   (the call clears what it needs cleared): calls that overlap on one device race on it, so keep
 *   these calls on one stream per device and do not run two at once.
 *   Errors: as ternary_moe_ffn_decode, plus TW_E_WORKSPACE when the layers need a larger workspace
 *   than TW_STATIC_SCRATCH_BYTES (ternary_moe_decode_workspace_bytes tells), TW_E_UNSUPPORTED
 *   (health misaligned), TW_E_ALIAS (health overlapping x_in or x_out).
 */
#define TW_STATIC_SCRATCH_BYTES (2u << 20)
tw_status ternary_moe_ffn_decode_static(const tw_moe_layer *layers, int32_t n_layers,
                                        const void *x_in, void *x_out, int32_t io_dtype,
                                        uint32_t *health, void *stream);

/*
 * ternary_moe_ffn_batched -- one layer for n_tokens independent tokens, each expert's weights read
 * once per call: (token, slot) pairs are grouped by expert and each expert's rows are applied to
 * all of its tokens.
 *   x_in       [T][d] in in_dtype; x_out [T][d] in out_dtype (must not overlap x_in).
 *   act        TW_ACT_FLOAT: as the decode call.  TW_ACT_INT8: per-token absmax quantisation of x
 *              to int8 in [-127,127] (scale amax/127), int32 sums, h re-quantised the same way per
 *              (token, expert), then the fixed fp32 sequence gate = (acc*s_x)*s_g, h =
 *              (gate/(1+exp(-gate)))*up, y = (acc*s_h)*s_d, out = ((x + g_0 y_0) + g_1 y_1) + ...,
 *              with one rounding per operation and a fixed exp: the result is bit-exact and does
 *              not depend on grouping or launch shape.  int8 with pre_rmsnorm is unsupported.
 *   expert_ids, gate_w  nullable [T][k]: when given, this routing is used as is (both or
 *              neither; a slot whose id is outside [0, E) contributes nothing); when NULL the call
 *              routes itself as moe_route_topk does.
 *   workspace  at least ternary_moe_batched_workspace_bytes(layer, n_tokens, act).
 *   n_tokens == 0 is a no-op.  Errors: as above.
 *   Source: expert layout and scheduling co-designed against scattered reads, [Hub] "MoE Is the
 *   Other Half of the Story Behind the 20B Figure"; prefill versus decode, [Hub] "What Makes
 *   120 tok/s So Fast?".
 */
tw_status ternary_moe_ffn_batched(const tw_moe_layer *layer, int64_t n_tokens, const void *x_in,
                                  int32_t in_dtype, void *x_out, int32_t out_dtype, int32_t act,
                                  const int32_t *expert_ids, const float *gate_w, void *workspace,
                                  size_t ws_bytes, void *stream);
size_t ternary_moe_batched_workspace_bytes(const tw_moe_layer *layer, int64_t n_tokens,
                                           int32_t act);

#ifdef __cplusplus
}
#endif
#endif
