// tw_aux.h -- internal interface between the host-side argument checks (tw_host.cpp) and the
// kernels of the base-3 layout (tw_base3.hip) and of decode attention (tw_attn.hip).  Kept apart
// from tw_internal.h so that these calls can change without touching what the FFN kernels include.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "tw_internal.h"

namespace tw {

// Base-3 layout (tw_base3.hip): bytes per row, ceil(cols/5) rounded up to a multiple of 16.
inline int64_t pack3_row_bytes(int64_t cols) { return ((cols + 4) / 5 + 15) / 16 * 16; }
int launch_pack3(const int8_t *w, int64_t rows, int64_t cols, uint8_t *packed, int32_t *bad,
                 void *stream);
// layout 2: ternary_pack's rows (cols / 4 bytes); layout 3: base-3 rows.  At most 64 chunks of 16
// bytes per row.
int launch_gemv_i8(const uint8_t *codes, int layout, const float *scales, int64_t rows, int cols,
                   const int8_t *xq, const float *x_scale, float *y, void *stream);
// Decode attention (tw_attn.hip): head dimension 128, splits of 16 cached positions; the
// workspace holds (max, sum, 128 outputs) per (split, query head).
constexpr int kAttnHeadDim = 128;
constexpr int kAttnChunk = 16;
inline int64_t attn_splits(int64_t n) { return (n + kAttnChunk - 1) / kAttnChunk; }
inline size_t attn_ws_bytes(int64_t n, int H) { return align256(sizeof(float) * size_t(attn_splits(n)) * H * (kAttnHeadDim + 2)); }
int launch_attn_decode(const void *q, const void *k, const void *v, int64_t n, int H, int Hkv,
                       float *out, void *ws, void *stream);
// The one-launch form: at most kAttnOneMaxSplits splits; the workspace holds one 64-bit tagged
// word per (split, query head, value) and is zero-filled between calls.
constexpr int kAttnOneMaxSplits = 64;
inline size_t attn_one_ws_bytes(int64_t n, int H) { return align256(sizeof(uint64_t) * size_t(attn_splits(n)) * H * (kAttnHeadDim + 2)); }
int launch_attn_decode_one(const void *q, const void *k, const void *v, int64_t n, int H, int Hkv,
                           float *out, void *ws, void *stream);
// Approximate output head (tw_head.hip): d in {512, 1024, 2048, 4096}, at most 8192 clusters; the
// workspace holds the clusters' fp32 scores.
constexpr int kHeadMaxD = 4096;
constexpr int kHeadMaxClusters = 8192;
inline size_t head_ws_bytes(int ncl) { return align256(sizeof(float) * size_t(ncl)); }
int launch_flash_head(const void *h, int d, const uint8_t *cent, const float *cscale, int ncl,
                      const void *wc, const int32_t *members, int cs, int top, int32_t *sel,
                      int32_t *ids, float *logits, void *ws, void *stream);

}  // namespace tw
