// tw_internal.h -- internal interface between the host-side argument checks (tw_host.cpp, no HIP
// headers) and the HIP kernels and launchers (tw_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace tw {

// A layer as the kernels see it (device pointers only).
struct LayerPtrs {
    const void *w_router;
    const uint8_t *w_gate, *w_up, *w_down;
    const float *s_gate, *s_up, *s_down;
};

struct Dims {
    int32_t d, F, E, k;
    int32_t router_bf16;   // 1: router weights are bf16, 0: fp32
    int32_t pre_norm;      // 1: pre-RMSNorm on the FFN input
};

constexpr int kMaxLayers = 64;
constexpr int kMaxPersistLayers = 32;   // layers per launch of the one-launch stacked decode
constexpr int kMaxTopK = 32;
constexpr int kMaxExperts = 1024;

// Number of int8 digit planes the float path splits an activation vector into.
inline int float_planes(int io_bf16) { return io_bf16 ? 2 : 3; }

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// ---- decode (batch 1) workspace -------------------------------------------------------------
struct DecodeWs {
    size_t ctrl, logits, ids, gates, xinfo, xdig, h, xbuf, ll, err, ts, total;
};
// Phase timestamps of the one-launch stacked decode, kept only by a library built with
// TW_PHASE_TIMES (a measurement build): per workgroup and layer, kPhaseStamps 64-bit clock values.
constexpr int kPhaseStamps = 10;
constexpr int kPhaseWorkgroups = 256;
// Tagged words of the one-launch stacked decode: two parities of kLlCopies copies of one set of
// (E logits, k*F fp32 h values, d/2 packed bf16 residual pairs).  Every word is stored into each
// copy and each workgroup polls the copy of its own XCD, so that the polls of all 256 workgroups do
// not converge on the same few lines (an all-to-all round of tagged words over 256 workgroups
// measured 2.42 us with one copy, 2.07 with two, 1.90 with four, 1.86 with eight).
// Logit words of the one-launch decode lie kLgStride words apart (each workgroup publishes one; four
// writers per 128-byte line measured faster than sixteen, and than one with sixteen times the
// lines to poll).
constexpr int kLgStride = 4;
constexpr int kLlCopies = 8;
inline size_t persist_set_words(const Dims &dm) { return size_t(dm.E) * kLgStride + size_t(dm.k) * dm.F + dm.d / 2; }
inline size_t persist_words(const Dims &dm) { return 2 * size_t(kLlCopies) * persist_set_words(dm); }
inline DecodeWs decode_ws_layout(const Dims &dm) {
    DecodeWs w{};
    size_t o = 0;
    w.ctrl = o;   o += align256(256);
    w.logits = o; o += align256(sizeof(float) * dm.E);
    w.ids = o;    o += align256(sizeof(int32_t) * kMaxTopK);
    w.gates = o;  o += align256(sizeof(float) * kMaxTopK);
    w.xinfo = o;  o += align256(64);
    w.xdig = o;   o += align256(size_t(3) * dm.d);
    w.h = o;      o += align256(sizeof(float) * size_t(dm.k) * dm.F);
    w.xbuf = o;   o += align256(sizeof(float) * 2 * size_t(dm.d));
    w.ll = o;     o += align256(sizeof(uint64_t) * persist_words(dm));
    w.err = o;    o += align256(sizeof(uint32_t) * 4);
#ifdef TW_PHASE_TIMES
    w.ts = o;     o += align256(sizeof(uint64_t) * kPhaseWorkgroups * kMaxPersistLayers * kPhaseStamps);
#endif
    w.total = o;
    return w;
}

// ---- batched workspace ------------------------------------------------------------------------
struct BatchedWs {
    // y: fp32 y rows (v_dot4 path; float activations on the matrix cores), or with int8 activations
    // on the matrix cores the int32 down sums that do not fit y16; y16 / shp (int8 activations
    // only): 16-bit down sums and each pair's s_h (zero-size otherwise)
    size_t ctrl, logits, ids, gates, tinfo, xdig, counts, offsets, pairs, tiles, tilemeta, h, y, y16, shp, total;
    int64_t spare_row;   // first of kSpareRows y rows behind the last pair: stores of padding
                         // tokens land there (workgroup b uses row spare_row + b % kSpareRows)
};
constexpr int kSpareRows = 256;
constexpr int kTileTokens = 64;     // tokens per tile: large tiles (many tokens per expert)
constexpr int kMinTile = 8;         // fewest tokens per tile of any grouping (sizes the tile lists)
// Upper bound on the (expert, tile) work items of T tokens in tiles of `tt` tokens, rounded up to a
// multiple of 8.
inline int64_t max_tiles(const Dims &dm, int64_t T, int tt)
{
    const int64_t n = (T * dm.k + tt - 1) / tt + dm.E;
    return (n + 7) / 8 * 8;
}
inline BatchedWs batched_ws_layout(const Dims &dm, int64_t T, int planes) {
    BatchedWs w{};
    size_t o = 0;
    size_t pairs = size_t(T) * dm.k;
    w.ctrl = o;    o += align256(256);
    w.logits = o;  o += align256(sizeof(float) * size_t(T) * dm.E);
    w.ids = o;     o += align256(sizeof(int32_t) * pairs);
    w.gates = o;   o += align256(sizeof(float) * pairs);
    w.tinfo = o;   o += align256(sizeof(float) * 2 * size_t(T));
    w.xdig = o;    o += align256(size_t(planes) * size_t(T) * dm.d);
    w.counts = o;  o += align256(sizeof(int32_t) * (dm.E + 1));
    w.offsets = o; o += align256(sizeof(int32_t) * (dm.E + 1));
    w.pairs = o;   o += align256(sizeof(int32_t) * pairs);
    w.tiles = o;   o += align256(sizeof(int32_t) * size_t(max_tiles(dm, T, kMinTile) + 16));
    w.tilemeta = o; o += align256(2 * sizeof(int32_t) * size_t(max_tiles(dm, T, kMinTile) + 16));
    w.h = o;       o += align256(sizeof(float) * pairs * dm.F);
    w.y = o;       o += align256(sizeof(float) * (pairs + kSpareRows) * dm.d);
    w.y16 = o;     o += planes == 1 ? align256(sizeof(int16_t) * (pairs + kSpareRows) * dm.d) : 0;
    w.shp = o;     o += planes == 1 ? align256(sizeof(float) * pairs) : 0;
    w.spare_row = int64_t(pairs);
    w.total = o;
    return w;
}

// ---- launchers (tw_kernels.hip); each returns 0 or a hipError_t value --------------------------
int launch_pack(const int8_t *w, int64_t rows, int64_t cols, uint8_t *packed, int32_t *bad,
                void *stream);
int launch_quantize(const void *w, int w_bf16, int64_t rows, int64_t cols, uint8_t *packed,
                    float *scales, void *stream);
int launch_route(const void *x, int x_bf16, const void *w_router, int w_bf16, int64_t T,
                 const Dims &dm, float *logits, int32_t *ids, float *gates, void *stream);
// One launch per (up to kMaxPersistLayers) layers; returns -1 when the shape or device is not
// served by that path (the caller then uses launch_decode).
int launch_decode_persist(const Dims &dm, const LayerPtrs *layers, int n_layers, const void *x_in,
                          void *x_out, int io_bf16, void *ws, void *stream);
int launch_decode(const Dims &dm, const LayerPtrs *layers, int n_layers, const void *x_in,
                  void *x_out, int io_bf16, void *ws, void *stream);
// The same decode with the library's static scratch (tw_static.hip) as its workspace; health
// (nullable, device) receives the health word after the call.
constexpr size_t kStaticScratchBytes = size_t(2) << 20;
int launch_decode_static(const Dims &dm, const LayerPtrs *layers, int n_layers, const void *x_in,
                         void *x_out, int io_bf16, uint32_t *health, void *stream);
// Grouped MFMA path of the batched FFN (after quantisation/digit planes): planes = 1 (int8
// activations) or 2 (digit planes of bf16 inputs).  sel_ids == nullptr: tiles of `tile` tokens from
// k_group's lists; else the T k expert ids themselves (one workgroup per expert finds its pairs,
// only where grouped_mfma_self holds).
int launch_grouped_mfma(const Dims &dm, const LayerPtrs &layer, int64_t T, int planes, int tile,
                        const BatchedWs &L, uint8_t *ws, const int32_t *sel_ids, void *stream);
// Whether that path serves this shape; *tile receives the tile size to group with.
bool grouped_mfma_serves(const Dims &dm, int64_t T, int planes, int *tile);
// Whether it can take the ids directly (no k_group) at this batch size and tile.
bool grouped_mfma_self(const Dims &dm, int64_t T, int tile);
int launch_batched(const Dims &dm, const LayerPtrs &layer, int64_t T, const void *x_in,
                   int in_bf16, void *x_out, int out_bf16, int int8_act, const int32_t *ids,
                   const float *gates, void *ws, void *stream);

}  // namespace tw
