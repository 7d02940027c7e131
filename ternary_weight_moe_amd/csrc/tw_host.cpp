// tw_host.cpp -- the C ABI of libternary_moe.so: argument checks, workspace sizing and status
// strings.  This translation unit includes no HIP header: every check here runs before any HIP
// call, so the error paths are testable on a machine without a GPU.
#include <stdint.h>
#include <string.h>

#include "../../include/ternary_moe.h"
#include "tw_aux.h"
#include "tw_internal.h"

namespace {

bool is_pow2_in(int64_t v, int64_t lo, int64_t hi)
{
    return v >= lo && v <= hi && (v & (v - 1)) == 0;
}

bool valid_float(int32_t t) { return t == TW_F32 || t == TW_BF16; }

size_t fsize(int32_t t) { return t == TW_BF16 ? 2 : 4; }

// [a, a+na) and [b, b+nb) overlap?
bool overlap(const void *a, size_t na, const void *b, size_t nb)
{
    if (!a || !b || na == 0 || nb == 0) return false;
    uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

tw_status check_dims(int64_t d, int64_t F, int64_t E, int64_t k)
{
    if (d <= 0 || F <= 0 || E <= 0 || k <= 0) return TW_E_SHAPE;
    if (k > E) return TW_E_SHAPE;
    if (!is_pow2_in(d, 64, 4096) || !is_pow2_in(F, 64, 4096)) return TW_E_UNSUPPORTED;
    if (E > tw::kMaxExperts || k > tw::kMaxTopK) return TW_E_UNSUPPORTED;
    return TW_OK;
}

tw_status check_layer(const tw_moe_layer *L)
{
    if (!L) return TW_E_NULL;
    tw_status s = check_dims(L->d_model, L->d_ff, L->n_experts, L->top_k);
    if (s != TW_OK) return s;
    if (!valid_float(L->router_dtype)) return TW_E_DTYPE;
    if (L->pre_rmsnorm != 0 && L->pre_rmsnorm != 1) return TW_E_SHAPE;
    if (!L->w_router || !L->w_gate || !L->w_up || !L->w_down || !L->s_gate || !L->s_up ||
        !L->s_down)
        return TW_E_NULL;
    // packed rows, router rows and scales are read 16 bytes at a time
    if (((uintptr_t)L->w_gate | (uintptr_t)L->w_up | (uintptr_t)L->w_down | (uintptr_t)L->w_router |
         (uintptr_t)L->s_gate | (uintptr_t)L->s_up | (uintptr_t)L->s_down) & 15)
        return TW_E_UNSUPPORTED;
    return TW_OK;
}

tw::Dims dims_of(const tw_moe_layer *L)
{
    tw::Dims d{};
    d.d = L->d_model;
    d.F = L->d_ff;
    d.E = L->n_experts;
    d.k = L->top_k;
    d.router_bf16 = L->router_dtype == TW_BF16;
    d.pre_norm = L->pre_rmsnorm;
    return d;
}

tw::LayerPtrs ptrs_of(const tw_moe_layer *L)
{
    tw::LayerPtrs p{};
    p.w_router = L->w_router;
    p.w_gate = L->w_gate;
    p.w_up = L->w_up;
    p.w_down = L->w_down;
    p.s_gate = L->s_gate;
    p.s_up = L->s_up;
    p.s_down = L->s_down;
    return p;
}

}  // namespace

extern "C" {

const char *tw_status_str(tw_status s)
{
    switch (s) {
    case TW_OK: return "ok";
    case TW_E_NULL: return "a required pointer is NULL";
    case TW_E_SHAPE: return "invalid or inconsistent sizes";
    case TW_E_DTYPE: return "unknown dtype or activation mode";
    case TW_E_WORKSPACE: return "workspace too small";
    case TW_E_ALIAS: return "an output overlaps an input";
    case TW_E_UNSUPPORTED: return "shape outside what the kernels implement";
    case TW_E_HIP: return "HIP launch error";
    }
    return "unknown status";
}

tw_status ternary_pack(const int8_t *w, int64_t rows, int64_t cols, uint8_t *packed,
                       int32_t *bad_count, void *stream)
{
    if (rows < 0 || cols < 0) return TW_E_SHAPE;
    if (rows == 0 || cols == 0) return TW_OK;
    if (!w || !packed) return TW_E_NULL;
    if (cols > (int64_t(1) << 40) / rows) return TW_E_SHAPE;
    int64_t stride = (cols + 3) / 4;
    if (overlap(w, size_t(rows * cols), packed, size_t(rows * stride))) return TW_E_ALIAS;
    if (bad_count && (overlap(bad_count, 4, packed, size_t(rows * stride)) ||
                      overlap(bad_count, 4, w, size_t(rows * cols))))
        return TW_E_ALIAS;
    return tw::launch_pack(w, rows, cols, packed, bad_count, stream) ? TW_E_HIP : TW_OK;
}

tw_status ternary_quantize(const void *w, int32_t w_dtype, int64_t rows, int64_t cols,
                           uint8_t *packed, float *scales, void *stream)
{
    if (rows < 0 || cols < 0) return TW_E_SHAPE;
    if (!valid_float(w_dtype)) return TW_E_DTYPE;
    if (rows == 0 || cols == 0) return TW_OK;
    if (!w || !packed || !scales) return TW_E_NULL;
    if (cols % 8 != 0 || cols > 65536) return TW_E_UNSUPPORTED;
    if (rows > (int64_t(1) << 40) / cols) return TW_E_SHAPE;
    if ((((uintptr_t)w | (uintptr_t)packed) & 15) || ((uintptr_t)scales & 3)) return TW_E_UNSUPPORTED;
    const size_t nw = size_t(rows * cols) * fsize(w_dtype), np = size_t(rows * cols / 4),
                 ns = size_t(rows) * 4;
    if (overlap(w, nw, packed, np) || overlap(w, nw, scales, ns) || overlap(packed, np, scales, ns))
        return TW_E_ALIAS;
    return tw::launch_quantize(w, w_dtype == TW_BF16, rows, cols, packed, scales, stream) ? TW_E_HIP
                                                                                          : TW_OK;
}

int64_t ternary_pack3_row_bytes(int64_t cols)
{
    if (cols < 0 || cols > (int64_t(1) << 40)) return -1;
    return tw::pack3_row_bytes(cols);
}

tw_status ternary_pack3(const int8_t *w, int64_t rows, int64_t cols, uint8_t *packed,
                        int32_t *bad_count, void *stream)
{
    if (rows < 0 || cols < 0) return TW_E_SHAPE;
    if (rows == 0 || cols == 0) return TW_OK;
    if (!w || !packed) return TW_E_NULL;
    if (cols > (int64_t(1) << 40) / rows) return TW_E_SHAPE;
    const int64_t rb = tw::pack3_row_bytes(cols);
    if (overlap(w, size_t(rows * cols), packed, size_t(rows * rb))) return TW_E_ALIAS;
    if (bad_count && (overlap(bad_count, 4, packed, size_t(rows * rb)) ||
                      overlap(bad_count, 4, w, size_t(rows * cols))))
        return TW_E_ALIAS;
    return tw::launch_pack3(w, rows, cols, packed, bad_count, stream) ? TW_E_HIP : TW_OK;
}

tw_status ternary_gemv_i8(const uint8_t *codes, int32_t layout, const float *scales, int64_t rows,
                          int64_t cols, const int8_t *xq, const float *x_scale, float *y,
                          void *stream)
{
    if (rows < 0 || cols < 0) return TW_E_SHAPE;
    if (layout != 2 && layout != 3) return TW_E_DTYPE;
    if (rows == 0) return TW_OK;
    if (!codes || !scales || !xq || !x_scale || !y) return TW_E_NULL;
    if (cols == 0 || (layout == 2 && (cols % 64 != 0 || cols > 4096)) ||
        (layout == 3 && cols > 5120))
        return TW_E_UNSUPPORTED;
    if (rows > (int64_t(1) << 40) / cols) return TW_E_SHAPE;
    if (((uintptr_t)codes & 15) || (((uintptr_t)scales | (uintptr_t)y | (uintptr_t)x_scale) & 3))
        return TW_E_UNSUPPORTED;
    const int64_t rb = layout == 3 ? tw::pack3_row_bytes(cols) : cols / 4;
    const size_t ny = size_t(rows) * 4;
    if (overlap(y, ny, codes, size_t(rows * rb)) || overlap(y, ny, scales, size_t(rows) * 4) ||
        overlap(y, ny, xq, size_t(cols)) || overlap(y, ny, x_scale, 4))
        return TW_E_ALIAS;
    return tw::launch_gemv_i8(codes, layout, scales, rows, int(cols), xq, x_scale, y, stream)
               ? TW_E_HIP
               : TW_OK;
}

size_t attention_decode_workspace_bytes(int32_t n_heads, int32_t head_dim, int64_t n_slots)
{
    if (n_heads < 1 || n_heads > 128 || head_dim != tw::kAttnHeadDim || n_slots < 1 ||
        n_slots > (int64_t(1) << 21))
        return 0;
    return tw::attn_ws_bytes(n_slots, n_heads);
}

tw_status attention_decode(const void *q, const void *k_cache, const void *v_cache, int64_t n_slots,
                           int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, float *out,
                           void *workspace, size_t workspace_bytes, void *stream)
{
    if (n_slots < 1 || n_slots > (int64_t(1) << 21) || n_heads < 1 || n_kv_heads < 1 ||
        n_heads % n_kv_heads != 0)
        return TW_E_SHAPE;
    const int G = n_heads / n_kv_heads;
    if (head_dim != tw::kAttnHeadDim || n_heads > 128 || (G != 1 && G != 2 && G != 4 && G != 8))
        return TW_E_UNSUPPORTED;
    if (!q || !k_cache || !v_cache || !out || !workspace) return TW_E_NULL;
    if ((((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache) & 15) || ((uintptr_t)out & 3) ||
        ((uintptr_t)workspace & 255))
        return TW_E_UNSUPPORTED;
    const size_t need = tw::attn_ws_bytes(n_slots, n_heads);
    if (workspace_bytes < need) return TW_E_WORKSPACE;
    const size_t nq = size_t(n_heads) * head_dim * 2, nkv = size_t(n_slots) * n_kv_heads * head_dim * 2,
                 no = size_t(n_heads) * head_dim * 4;
    if (overlap(out, no, q, nq) || overlap(out, no, k_cache, nkv) || overlap(out, no, v_cache, nkv) ||
        overlap(out, no, workspace, need) || overlap(workspace, need, q, nq) ||
        overlap(workspace, need, k_cache, nkv) || overlap(workspace, need, v_cache, nkv))
        return TW_E_ALIAS;
    return tw::launch_attn_decode(q, k_cache, v_cache, n_slots, n_heads, n_kv_heads, out, workspace,
                                  stream)
               ? TW_E_HIP
               : TW_OK;
}

size_t attention_decode_one_workspace_bytes(int32_t n_heads, int32_t head_dim, int64_t n_slots)
{
    if (n_heads < 1 || n_heads > 128 || head_dim != tw::kAttnHeadDim || n_slots < 1 ||
        tw::attn_splits(n_slots) > tw::kAttnOneMaxSplits)
        return 0;
    return tw::attn_one_ws_bytes(n_slots, n_heads);
}

tw_status attention_decode_one(const void *q, const void *k_cache, const void *v_cache, int64_t n_slots,
                               int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, float *out,
                               void *workspace, size_t workspace_bytes, void *stream)
{
    if (n_slots < 1 || n_slots > (int64_t(1) << 21) || n_heads < 1 || n_kv_heads < 1 ||
        n_heads % n_kv_heads != 0)
        return TW_E_SHAPE;
    const int G = n_heads / n_kv_heads;
    if (head_dim != tw::kAttnHeadDim || n_heads > 128 || (G != 1 && G != 2 && G != 4 && G != 8) ||
        tw::attn_splits(n_slots) > tw::kAttnOneMaxSplits)
        return TW_E_UNSUPPORTED;
    if (!q || !k_cache || !v_cache || !out || !workspace) return TW_E_NULL;
    if ((((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache) & 15) || ((uintptr_t)out & 3) ||
        ((uintptr_t)workspace & 255))
        return TW_E_UNSUPPORTED;
    const size_t need = tw::attn_one_ws_bytes(n_slots, n_heads);
    if (workspace_bytes < need) return TW_E_WORKSPACE;
    const size_t nq = size_t(n_heads) * head_dim * 2, nkv = size_t(n_slots) * n_kv_heads * head_dim * 2,
                 no = size_t(n_heads) * head_dim * 4;
    if (overlap(out, no, q, nq) || overlap(out, no, k_cache, nkv) || overlap(out, no, v_cache, nkv) ||
        overlap(out, no, workspace, need) || overlap(workspace, need, q, nq) ||
        overlap(workspace, need, k_cache, nkv) || overlap(workspace, need, v_cache, nkv))
        return TW_E_ALIAS;
    return tw::launch_attn_decode_one(q, k_cache, v_cache, n_slots, n_heads, n_kv_heads, out,
                                      workspace, stream)
               ? TW_E_HIP
               : TW_OK;
}

size_t flash_head_workspace_bytes(int32_t n_clusters)
{
    if (n_clusters < 1 || n_clusters > tw::kHeadMaxClusters) return 0;
    return tw::head_ws_bytes(n_clusters);
}

tw_status flash_head(const void *h, int32_t d, const uint8_t *centroids,
                     const float *centroid_scales, int32_t n_clusters, const void *w_clustered,
                     const int32_t *member_ids, int32_t cluster_size, int32_t top,
                     int32_t *sel_clusters, int32_t *token_ids, float *logits, void *workspace,
                     size_t workspace_bytes, void *stream)
{
    if (d < 1 || n_clusters < 1 || n_clusters > tw::kHeadMaxClusters || cluster_size < 1 ||
        cluster_size > 1024 || top < 1 || top > n_clusters)
        return TW_E_SHAPE;
    if (d != 512 && d != 1024 && d != 2048 && d != 4096) return TW_E_UNSUPPORTED;
    if (!h || !centroids || !centroid_scales || !w_clustered || !member_ids || !sel_clusters ||
        !token_ids || !logits || !workspace)
        return TW_E_NULL;
    if ((((uintptr_t)centroids | (uintptr_t)w_clustered) & 15) || ((uintptr_t)h & 1) ||
        (((uintptr_t)centroid_scales | (uintptr_t)member_ids | (uintptr_t)sel_clusters |
          (uintptr_t)token_ids | (uintptr_t)logits) & 3) ||
        ((uintptr_t)workspace & 255))
        return TW_E_UNSUPPORTED;
    const size_t need = tw::head_ws_bytes(n_clusters);
    if (workspace_bytes < need) return TW_E_WORKSPACE;
    const size_t nsel = size_t(top) * 4, nout = size_t(top) * cluster_size * 4;
    const void *ins[5] = {h, centroids, centroid_scales, w_clustered, member_ids};
    const size_t nin[5] = {size_t(d) * 2, size_t(n_clusters) * d / 2, size_t(n_clusters) * 4,
                           size_t(n_clusters) * cluster_size * d * 2,
                           size_t(n_clusters) * cluster_size * 4};
    const void *outs[4] = {sel_clusters, token_ids, logits, workspace};
    const size_t nouts[4] = {nsel, nout, nout, need};
    for (int o = 0; o < 4; o++) {
        for (int i = 0; i < 5; i++)
            if (overlap(outs[o], nouts[o], ins[i], nin[i])) return TW_E_ALIAS;
        for (int p = o + 1; p < 4; p++)
            if (overlap(outs[o], nouts[o], outs[p], nouts[p])) return TW_E_ALIAS;
    }
    return tw::launch_flash_head(h, d, centroids, centroid_scales, n_clusters, w_clustered,
                                 member_ids, cluster_size, top, sel_clusters, token_ids, logits,
                                 workspace, stream)
               ? TW_E_HIP
               : TW_OK;
}

tw_status moe_route_topk(const void *x, int32_t x_dtype, const void *w_router, int32_t w_dtype,
                         int64_t n_tokens, int32_t d_model, int32_t n_experts, int32_t top_k,
                         int32_t pre_rmsnorm, float *logits, int32_t *expert_ids, float *gate_w,
                         void *stream)
{
    if (n_tokens < 0) return TW_E_SHAPE;
    tw_status s = check_dims(d_model, 64, n_experts, top_k);
    if (s != TW_OK) return s;
    if (!valid_float(x_dtype) || !valid_float(w_dtype)) return TW_E_DTYPE;
    if (pre_rmsnorm != 0 && pre_rmsnorm != 1) return TW_E_SHAPE;
    if (n_tokens == 0) return TW_OK;
    if (!x || !w_router || !logits || !expert_ids || !gate_w) return TW_E_NULL;
    if (((uintptr_t)x | (uintptr_t)w_router) & 15) return TW_E_UNSUPPORTED;   // 16-byte loads
    size_t T = size_t(n_tokens);
    size_t nl = T * n_experts * 4, nk = T * top_k * 4;
    if (overlap(logits, nl, expert_ids, nk) || overlap(logits, nl, gate_w, nk) ||
        overlap(expert_ids, nk, gate_w, nk) || overlap(x, T * d_model * fsize(x_dtype), logits, nl) ||
        overlap(x, T * d_model * fsize(x_dtype), expert_ids, nk) ||
        overlap(x, T * d_model * fsize(x_dtype), gate_w, nk))
        return TW_E_ALIAS;
    tw::Dims dm{d_model, 64, n_experts, top_k, w_dtype == TW_BF16, pre_rmsnorm};
    return tw::launch_route(x, x_dtype == TW_BF16, w_router, w_dtype == TW_BF16, n_tokens, dm,
                            logits, expert_ids, gate_w, stream)
               ? TW_E_HIP
               : TW_OK;
}

size_t ternary_moe_decode_workspace_bytes(const tw_moe_layer *layers, int32_t n_layers)
{
    if (!layers || n_layers < 1 || check_layer(&layers[0]) != TW_OK) return 0;
    return tw::decode_ws_layout(dims_of(&layers[0])).total;
}

size_t ternary_moe_decode_error_offset(const tw_moe_layer *layers, int32_t n_layers)
{
    if (!layers || n_layers < 1 || check_layer(&layers[0]) != TW_OK) return 0;
    return tw::decode_ws_layout(dims_of(&layers[0])).err;
}

static_assert(TW_STATIC_SCRATCH_BYTES == tw::kStaticScratchBytes, "one size for the static scratch");

namespace {

// Checks shared by the two decode entry points (everything but the workspace); fills dm and ptrs.
tw_status check_decode(const tw_moe_layer *layers, int32_t n_layers, const void *x_in,
                       void *x_out, int32_t io_dtype, tw::Dims &dm, tw::LayerPtrs *ptrs)
{
    if (!layers) return TW_E_NULL;
    if (n_layers < 1) return TW_E_SHAPE;
    if (n_layers > tw::kMaxLayers) return TW_E_UNSUPPORTED;
    for (int i = 0; i < n_layers; i++) {
        tw_status s = check_layer(&layers[i]);
        if (s != TW_OK) return s;
        const tw_moe_layer &a = layers[0], &b = layers[i];
        if (a.d_model != b.d_model || a.d_ff != b.d_ff || a.n_experts != b.n_experts ||
            a.top_k != b.top_k || a.router_dtype != b.router_dtype ||
            a.pre_rmsnorm != b.pre_rmsnorm)
            return TW_E_SHAPE;
    }
    if (!valid_float(io_dtype)) return TW_E_DTYPE;
    if (!x_in || !x_out) return TW_E_NULL;
    dm = dims_of(&layers[0]);
    // the down kernel keeps the digit planes of all k expert activations in 64 KiB of LDS
    if (size_t(dm.k) * 3 * dm.F > 65536 - 1024) return TW_E_UNSUPPORTED;
    size_t xb = size_t(dm.d) * fsize(io_dtype);
    if (overlap(x_in, xb, x_out, xb)) return TW_E_ALIAS;
    for (int i = 0; i < n_layers; i++) ptrs[i] = ptrs_of(&layers[i]);
    return TW_OK;
}

}  // namespace

tw_status ternary_moe_ffn_decode(const tw_moe_layer *layers, int32_t n_layers, const void *x_in,
                                 void *x_out, int32_t io_dtype, void *workspace, size_t ws_bytes,
                                 void *stream)
{
    tw::Dims dm{};
    tw::LayerPtrs ptrs[tw::kMaxLayers];
    tw_status s = check_decode(layers, n_layers, x_in, x_out, io_dtype, dm, ptrs);
    if (s != TW_OK) return s;
    if (!workspace) return TW_E_NULL;
    if ((uintptr_t)workspace & 255) return TW_E_UNSUPPORTED;   // its regions are 256-byte aligned
    size_t need = tw::decode_ws_layout(dm).total;
    if (ws_bytes < need) return TW_E_WORKSPACE;
    size_t xb = size_t(dm.d) * fsize(io_dtype);
    if (overlap(workspace, ws_bytes, x_in, xb) || overlap(workspace, ws_bytes, x_out, xb))
        return TW_E_ALIAS;
    return tw::launch_decode(dm, ptrs, n_layers, x_in, x_out, io_dtype == TW_BF16, workspace,
                             stream)
               ? TW_E_HIP
               : TW_OK;
}

tw_status ternary_moe_ffn_decode_static(const tw_moe_layer *layers, int32_t n_layers,
                                        const void *x_in, void *x_out, int32_t io_dtype,
                                        uint32_t *health, void *stream)
{
    tw::Dims dm{};
    tw::LayerPtrs ptrs[tw::kMaxLayers];
    tw_status s = check_decode(layers, n_layers, x_in, x_out, io_dtype, dm, ptrs);
    if (s != TW_OK) return s;
    if (tw::decode_ws_layout(dm).total > tw::kStaticScratchBytes) return TW_E_WORKSPACE;
    if ((uintptr_t)health & 3) return TW_E_UNSUPPORTED;
    size_t xb = size_t(dm.d) * fsize(io_dtype);
    if (overlap(health, 4, x_in, xb) || overlap(health, 4, x_out, xb)) return TW_E_ALIAS;
    return tw::launch_decode_static(dm, ptrs, n_layers, x_in, x_out, io_dtype == TW_BF16, health,
                                    stream)
               ? TW_E_HIP
               : TW_OK;
}

size_t ternary_moe_batched_workspace_bytes(const tw_moe_layer *layer, int64_t n_tokens,
                                           int32_t act)
{
    if (!layer || n_tokens < 0 || check_layer(layer) != TW_OK) return 0;
    if (act != TW_ACT_FLOAT && act != TW_ACT_INT8) return 0;
    int planes = act == TW_ACT_INT8 ? 1 : 3;
    return tw::batched_ws_layout(dims_of(layer), n_tokens, planes).total;
}

tw_status ternary_moe_ffn_batched(const tw_moe_layer *layer, int64_t n_tokens, const void *x_in,
                                  int32_t in_dtype, void *x_out, int32_t out_dtype, int32_t act,
                                  const int32_t *expert_ids, const float *gate_w, void *workspace,
                                  size_t ws_bytes, void *stream)
{
    tw_status s = check_layer(layer);
    if (s != TW_OK) return s;
    if (n_tokens < 0) return TW_E_SHAPE;
    if (!valid_float(in_dtype) || !valid_float(out_dtype)) return TW_E_DTYPE;
    if (act != TW_ACT_FLOAT && act != TW_ACT_INT8) return TW_E_DTYPE;
    if (act == TW_ACT_INT8 && layer->pre_rmsnorm) return TW_E_UNSUPPORTED;
    if ((expert_ids == nullptr) != (gate_w == nullptr)) return TW_E_NULL;
    if (n_tokens > (int64_t(1) << 24)) return TW_E_UNSUPPORTED;
    if (n_tokens == 0) return TW_OK;
    if (!x_in || !x_out || !workspace) return TW_E_NULL;
    if (((uintptr_t)x_in | (uintptr_t)x_out) & 15) return TW_E_UNSUPPORTED;   // 16-byte accesses
    if ((uintptr_t)workspace & 255) return TW_E_UNSUPPORTED;   // its regions are 256-byte aligned
    tw::Dims dm = dims_of(layer);
    int planes = act == TW_ACT_INT8 ? 1 : 3;
    size_t need = tw::batched_ws_layout(dm, n_tokens, planes).total;
    if (ws_bytes < need) return TW_E_WORKSPACE;
    size_t T = size_t(n_tokens);
    size_t xin = T * dm.d * fsize(in_dtype), xout = T * dm.d * fsize(out_dtype);
    if (overlap(x_in, xin, x_out, xout)) return TW_E_ALIAS;
    if (overlap(workspace, ws_bytes, x_in, xin) || overlap(workspace, ws_bytes, x_out, xout))
        return TW_E_ALIAS;
    if (expert_ids && (overlap(x_out, xout, expert_ids, T * dm.k * 4) ||
                       overlap(x_out, xout, gate_w, T * dm.k * 4) ||
                       overlap(workspace, ws_bytes, expert_ids, T * dm.k * 4) ||
                       overlap(workspace, ws_bytes, gate_w, T * dm.k * 4)))
        return TW_E_ALIAS;
    return tw::launch_batched(dm, ptrs_of(layer), n_tokens, x_in, in_dtype == TW_BF16, x_out,
                              out_dtype == TW_BF16, act == TW_ACT_INT8, expert_ids, gate_w,
                              workspace, stream)
               ? TW_E_HIP
               : TW_OK;
}

}  // extern "C"
