// tw_attn.hip -- decode attention of one query token over a KV cache (the attention half of a decode
// layer).  The model of the pages interleaves sliding-window attention with a 512-token window and
// global attention at 3:1 (6 global, 18 windowed layers), which bounds the cache of the windowed
// layers ("A 20B AI Model Trained in Ternary Just Hit 218 Tokens/Second on a $599 Mac Mini",
// section "The Architecture: Designed for the Hardware").  A windowed layer keeps its last 512
// positions in a ring of 512 slots and a global layer one slot per position; either way the call
// attends over the filled slots, and the result does not depend on their order.
//
// out_h = sum_t softmax_t(q_h . k_t / sqrt(128)) v_t over n slots, query head h reading KV head
// h / G (G query heads per KV head).  q, k, v bf16 (post-rotary; positions are not the kernel's
// concern), sums and output fp32.
//
// Split over positions (flash-decoding): workgroup (s, g) is one wave over slots 16 s .. 16 s + 15
// of KV head g and all G of its query heads, and issues all of its global loads before any use (one
// memory round trip per workgroup).  Scores: four lanes per slot, each reading a quarter of the key
// row (64 contiguous bytes) against the G query rows in LDS, the quarters summed by DPP.  Softmax
// part: wave max and sum per head.  Values: lane = two dimensions; each slot's value row is one
// coalesced 256-byte read.  The partial (max, sum, 128 outputs) per (split, head) goes to the
// workspace, and a second kernel merges the splits of each head with the usual rescaling by
// exp(m_s - M).  attention_decode_one does the same in one launch (up to 64 splits): the partials
// go out as tagged words and merge workgroups at the end of the grid wait for them (below).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "tw_device.h"
#include "tw_aux.h"
#include "tw_internal.h"

namespace tw {
namespace {

template <int G>
__global__ __launch_bounds__(64) void k_attn_part(const uint16_t *__restrict__ q,
                                                  const uint16_t *__restrict__ k,
                                                  const uint16_t *__restrict__ v, int64_t n,
                                                  int Hkv, float scale, float *__restrict__ ws)
{
    constexpr int DH = kAttnHeadDim, CH = kAttnChunk;
    static_assert(CH == 16 && DH == 128, "four lanes per slot, two dimensions per lane");
    __shared__ float s_q[G][DH];
    __shared__ float s_p[G][CH];
    const int lane = threadIdx.x, g = blockIdx.y;
    const int H = Hkv * G;
    const int64_t sp = blockIdx.x, t0 = sp * CH;
    const int slot = lane >> 2, qd = lane & 3;
    const int64_t t = t0 + slot;
    const bool valid = t < n;
    const int nv = int(n - t0 < CH ? n - t0 : CH);
    // every global load is issued first: the quarter key row of this lane's slot (dimensions
    // 32 qd .. 32 qd + 31), the value pair (dimensions 2 lane, 2 lane + 1) of every slot of the
    // chunk, and the G query rows
    uint4 kr[4];
    const uint4 *kp = reinterpret_cast<const uint4 *>(k + (int64_t(valid ? t : t0) * Hkv + g) * DH + 32 * qd);
#pragma unroll
    for (int c = 0; c < 4; c++) kr[c] = kp[c];
    uint32_t vv[CH];
    const uint16_t *vp = v + (t0 * Hkv + g) * DH + 2 * lane;
#pragma unroll
    for (int u = 0; u < CH; u++)
        vv[u] = u < nv ? *reinterpret_cast<const uint32_t *>(vp + int64_t(u) * Hkv * DH) : 0u;
#pragma unroll
    for (int i = lane; i < G * DH; i += 64) s_q[i / DH][i % DH] = bf16_to_f32(q[int64_t(g) * G * DH + i]);
    __syncthreads();
    float sc[G];
#pragma unroll
    for (int j = 0; j < G; j++) sc[j] = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; c++) {
        const uint32_t w[4] = {kr[c].x, kr[c].y, kr[c].z, kr[c].w};
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const float kv = bf16_to_f32(uint16_t(w[e >> 1] >> (16 * (e & 1))));
#pragma unroll
            for (int j = 0; j < G; j++) sc[j] = sc[j] + s_q[j][32 * qd + 8 * c + e] * kv;
        }
    }
    // the four quarter sums of a slot: (q0 + q1) + (q2 + q3), the same in all four lanes
#pragma unroll
    for (int j = 0; j < G; j++) {
        sc[j] = sc[j] + dpp_f<kDppXor1>(sc[j]);
        sc[j] = sc[j] + dpp_f<kDppXor2>(sc[j]);
    }
    float m[G], l[G];
#pragma unroll
    for (int j = 0; j < G; j++) {
        const float x = valid ? sc[j] * scale : -INFINITY;
        m[j] = wave_max(x);
        const float p = valid ? expf(x - m[j]) : 0.0f;
        l[j] = wave_sum(qd == 0 ? p : 0.0f);
        if (qd == 0) s_p[j][slot] = p;
    }
    __syncthreads();
    float o[G][2];
#pragma unroll
    for (int j = 0; j < G; j++) o[j][0] = o[j][1] = 0.0f;
#pragma unroll
    for (int u = 0; u < CH; u++) {
        if (u < nv) {
            const float v0 = bf16_to_f32(uint16_t(vv[u])), v1 = bf16_to_f32(uint16_t(vv[u] >> 16));
#pragma unroll
            for (int j = 0; j < G; j++) {
                o[j][0] = o[j][0] + s_p[j][u] * v0;
                o[j][1] = o[j][1] + s_p[j][u] * v1;
            }
        }
    }
#pragma unroll
    for (int j = 0; j < G; j++) {
        float *pw = ws + (sp * H + int64_t(g) * G + j) * (DH + 2);
        *reinterpret_cast<float2 *>(pw + 2 * lane) = make_float2(o[j][0], o[j][1]);
        if (lane == 0) {
            pw[DH] = m[j];
            pw[DH + 1] = l[j];
        }
    }
}

// One workgroup of 256 threads per query head.  The splits' (max, sum) pairs are read by all
// threads at once (one memory round trip for up to 256 splits per pass) and reduced in LDS; then
// thread (half, dim) sums the rescaled outputs of every other split, 16 loads in flight, and the
// two halves are added.
__global__ __launch_bounds__(256) void k_attn_merge(const float *__restrict__ ws, int64_t S, int H,
                                                    float *__restrict__ out)
{
    constexpr int DH = kAttnHeadDim, U = 16;
    __shared__ float s_red[4];
    __shared__ float s_o[DH];
    const int h = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
    float mx = -INFINITY;
    for (int64_t s = t; s < S; s += 256) mx = fmaxf(mx, ws[(s * H + h) * (DH + 2) + DH]);
    mx = wave_max(mx);
    if (lane == 0) s_red[wave] = mx;
    __syncthreads();
    const float M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    const int i = t & (DH - 1), half = t >> 7;
    float L = 0.0f, O = 0.0f;
    for (int64_t s0 = half; s0 < S; s0 += 2 * U) {
        float ms[U], ls[U], os[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int64_t s = s0 + 2 * u;
            const float *pw = ws + ((s < S ? s : 0) * H + h) * (DH + 2);   // split 0 always exists
            ms[u] = s < S ? pw[DH] : -INFINITY;
            ls[u] = s < S ? pw[DH + 1] : 0.0f;
            os[u] = s < S ? pw[i] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            const float e = expf(ms[u] - M);
            L = L + e * ls[u];
            O = O + e * os[u];
        }
    }
    __syncthreads();
    if (half == 1) {
        s_o[i] = O;
        if (i == 0) s_red[0] = L;
    }
    __syncthreads();
    if (half == 0) out[int64_t(h) * DH + i] = (O + s_o[i]) / (L + s_red[0]);
}

// ---- one launch: the splits publish tagged words, a merge workgroup per query head waits for them
//
// Each partial value goes to the workspace as one 64-bit word, a 32-bit tag naming the call beside
// the fp32 bits, stored and read with single 64-bit device-scope accesses: a word that carries the
// call's tag holds this call's value, so no fence is needed between the splits and the merge.  The
// merge workgroups come last in the grid: workgroups are dispatched in order, so every split's
// workgroup has been dispatched when a merge workgroup starts waiting, and the splits never wait.
// After merging, each merge workgroup writes zeros over the words it read, so the workspace is
// zero-filled again between calls; stale words from a call that did not complete carry that
// call's tag.

// Splits of 16 slots: wave w of workgroup (KV head g, b) takes split 4 b + w.
template <int G>
__device__ __forceinline__ void attn_one_part(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                                              const uint16_t *__restrict__ v, int64_t n, int Hkv, float scale,
                                              uint64_t *__restrict__ ws, uint32_t tag, int g, int b)
{
    constexpr int DH = kAttnHeadDim, CH = kAttnChunk;
    __shared__ float s_q[G][DH];
    __shared__ float s_p[4][G][CH];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int H = Hkv * G;
    const int64_t S = (n + CH - 1) / CH;
    const int64_t sp = int64_t(4) * b + wave;
    const bool act = sp < S;
    const int64_t t0 = (act ? sp : 0) * CH;
    const int slot = lane >> 2, qd = lane & 3;
    const int64_t tt = t0 + slot;
    const bool valid = act && tt < n;
    const int nv = act ? int(n - t0 < CH ? n - t0 : CH) : 0;
    uint4 kr[4];
    const uint4 *kp = reinterpret_cast<const uint4 *>(k + (int64_t(valid ? tt : t0) * Hkv + g) * DH + 32 * qd);
#pragma unroll
    for (int c = 0; c < 4; c++) kr[c] = kp[c];
    uint32_t vv[CH];
    const uint16_t *vp = v + (t0 * Hkv + g) * DH + 2 * lane;
#pragma unroll
    for (int u = 0; u < CH; u++)
        vv[u] = u < nv ? *reinterpret_cast<const uint32_t *>(vp + int64_t(u) * Hkv * DH) : 0u;
    for (int i = t; i < G * DH; i += 256) s_q[i / DH][i % DH] = bf16_to_f32(q[int64_t(g) * G * DH + i]);
    __syncthreads();
    float sc[G];
#pragma unroll
    for (int j = 0; j < G; j++) sc[j] = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; c++) {
        const uint32_t w[4] = {kr[c].x, kr[c].y, kr[c].z, kr[c].w};
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const float kv = bf16_to_f32(uint16_t(w[e >> 1] >> (16 * (e & 1))));
#pragma unroll
            for (int j = 0; j < G; j++) sc[j] = sc[j] + s_q[j][32 * qd + 8 * c + e] * kv;
        }
    }
#pragma unroll
    for (int j = 0; j < G; j++) {
        sc[j] = sc[j] + dpp_f<kDppXor1>(sc[j]);
        sc[j] = sc[j] + dpp_f<kDppXor2>(sc[j]);
    }
    float m[G], l[G];
#pragma unroll
    for (int j = 0; j < G; j++) {
        const float x = valid ? sc[j] * scale : -INFINITY;
        m[j] = wave_max(x);
        const float p = valid ? expf(x - m[j]) : 0.0f;
        l[j] = wave_sum(qd == 0 ? p : 0.0f);
        if (qd == 0) s_p[wave][j][slot] = p;
    }
    __syncthreads();
    if (!act) return;
    float o[G][2];
#pragma unroll
    for (int j = 0; j < G; j++) o[j][0] = o[j][1] = 0.0f;
#pragma unroll
    for (int u = 0; u < CH; u++) {
        if (u < nv) {
            const float v0 = bf16_to_f32(uint16_t(vv[u])), v1 = bf16_to_f32(uint16_t(vv[u] >> 16));
#pragma unroll
            for (int j = 0; j < G; j++) {
                o[j][0] = o[j][0] + s_p[wave][j][u] * v0;
                o[j][1] = o[j][1] + s_p[wave][j][u] * v1;
            }
        }
    }
#pragma unroll
    for (int j = 0; j < G; j++) {
        uint64_t *pw = ws + (sp * H + int64_t(g) * G + j) * (DH + 2);
        st_tagged(pw + 2 * lane, tag, __float_as_uint(o[j][0]));
        st_tagged(pw + 2 * lane + 1, tag, __float_as_uint(o[j][1]));
        if (lane == 0) {
            st_tagged(pw + DH, tag, __float_as_uint(m[j]));
            st_tagged(pw + DH + 1, tag, __float_as_uint(l[j]));
        }
    }
}

constexpr uint32_t kAttnOneSpin = 1u << 22;

// The merge of query head h: thread (i, half) sums the rescaled outputs of the splits s = half,
// half + 2, ... in increasing order, as k_attn_merge does, so the results are the same bits.
__device__ __forceinline__ void attn_one_merge(uint64_t *__restrict__ ws, int64_t S, int H, int h,
                                               uint32_t tag, float *__restrict__ out)
{
    constexpr int DH = kAttnHeadDim, NO = kAttnOneMaxSplits / 2;
    __shared__ float s_m[kAttnOneMaxSplits], s_l[kAttnOneMaxSplits];
    __shared__ float s_red[4];
    __shared__ float s_o[DH];
    __shared__ int s_bad;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int i = t & (DH - 1), half = t >> 7;
    const int ns = int((S - half + 1) / 2);   // splits of this thread's half
    if (t == 0) s_bad = 0;
    // words of this thread: o[i] of its half's splits, and (t < S) the max and sum of split t
    uint64_t wo[NO], wm = 0, wl = 0;
#pragma unroll
    for (int u = 0; u < NO; u++) wo[u] = 0;
    uint64_t pend = 0;
#pragma unroll
    for (int u = 0; u < NO; u++)
        if (u < ns) pend |= uint64_t(1) << u;
    const bool ml = t < S;
    bool pml = ml;
    const uint64_t *base = ws + int64_t(h) * (DH + 2);
    const int64_t stride = int64_t(H) * (DH + 2);
    uint32_t it = 0;
    for (; (pend || pml) && it < kAttnOneSpin; ++it) {
#pragma unroll
        for (int u = 0; u < NO; u++)
            if ((pend >> u) & 1u) wo[u] = ld_tagged(base + (half + 2 * u) * stride + i);
        if (pml) {
            wm = ld_tagged(base + t * stride + DH);
            wl = ld_tagged(base + t * stride + DH + 1);
        }
#pragma unroll
        for (int u = 0; u < NO; u++)
            if (((pend >> u) & 1u) && uint32_t(wo[u] >> 32) == tag) pend &= ~(uint64_t(1) << u);
        if (pml && uint32_t(wm >> 32) == tag && uint32_t(wl >> 32) == tag) pml = false;
    }
    __syncthreads();
    if (pend || pml) s_bad = 1;
    if (ml) {
        s_m[t] = __uint_as_float(uint32_t(wm));
        s_l[t] = __uint_as_float(uint32_t(wl));
    }
    float mx = ml ? __uint_as_float(uint32_t(wm)) : -INFINITY;
    mx = wave_max(mx);
    if (lane == 0) s_red[wave] = mx;
    __syncthreads();
    const float M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int u = 0; u < NO; u++) {
        if (u < ns) {
            const int s = half + 2 * u;
            const float e = expf(s_m[s] - M);
            L = L + e * s_l[s];
            O = O + e * __uint_as_float(uint32_t(wo[u]));
        }
    }
    // zeros over the words read (the workspace is zero-filled again for the next call)
    if (!s_bad) {
#pragma unroll
        for (int u = 0; u < NO; u++)
            if (u < ns) st_tagged(const_cast<uint64_t *>(base) + (half + 2 * u) * stride + i, 0u, 0u);
        if (ml) {
            st_tagged(const_cast<uint64_t *>(base) + t * stride + DH, 0u, 0u);
            st_tagged(const_cast<uint64_t *>(base) + t * stride + DH + 1, 0u, 0u);
        }
    }
    __syncthreads();
    if (half == 1) {
        s_o[i] = O;
        if (i == 0) s_red[0] = L;
    }
    __syncthreads();
    if (half == 0) out[int64_t(h) * DH + i] = s_bad ? __uint_as_float(0x7fc00000u) : (O + s_o[i]) / (L + s_red[0]);
}

template <int G>
__global__ __launch_bounds__(256) void k_attn_one(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                                                  const uint16_t *__restrict__ v, int64_t n, int Hkv, float scale,
                                                  uint64_t *__restrict__ ws, uint32_t tag, float *__restrict__ out)
{
    const int64_t S = (n + kAttnChunk - 1) / kAttnChunk;
    const int nb = int((S + 3) / 4);   // split workgroups per KV head
    const int bid = blockIdx.x;
    if (bid < nb * Hkv)
        attn_one_part<G>(q, k, v, n, Hkv, scale, ws, tag, bid / nb, bid % nb);
    else
        attn_one_merge(ws, S, Hkv * G, bid - nb * Hkv, tag, out);
}

}  // namespace

int launch_attn_decode_one(const void *q, const void *k, const void *v, int64_t n, int H, int Hkv,
                           float *out, void *ws, void *stream)
{
    static std::atomic<uint32_t> calls{0};
    uint32_t tag = calls.fetch_add(1, std::memory_order_relaxed) + 1;
    if (tag == 0) tag = calls.fetch_add(1, std::memory_order_relaxed) + 1;   // 0 marks a cleared word
    const int G = H / Hkv;
    const int64_t S = attn_splits(n);
    if (S > kAttnOneMaxSplits) return int(hipErrorInvalidValue);
    const float scale = 1.0f / sqrtf(float(kAttnHeadDim));
    hipStream_t st = static_cast<hipStream_t>(stream);
    const unsigned nbk = unsigned((S + 3) / 4 * Hkv + H);
    auto qp = static_cast<const uint16_t *>(q), kp = static_cast<const uint16_t *>(k),
         vp = static_cast<const uint16_t *>(v);
    uint64_t *w = static_cast<uint64_t *>(ws);
    switch (G) {
    case 1: k_attn_one<1><<<nbk, 256, 0, st>>>(qp, kp, vp, n, Hkv, scale, w, tag, out); break;
    case 2: k_attn_one<2><<<nbk, 256, 0, st>>>(qp, kp, vp, n, Hkv, scale, w, tag, out); break;
    case 4: k_attn_one<4><<<nbk, 256, 0, st>>>(qp, kp, vp, n, Hkv, scale, w, tag, out); break;
    case 8: k_attn_one<8><<<nbk, 256, 0, st>>>(qp, kp, vp, n, Hkv, scale, w, tag, out); break;
    default: return int(hipErrorInvalidValue);
    }
    return int(hipGetLastError());
}

int launch_attn_decode(const void *q, const void *k, const void *v, int64_t n, int H, int Hkv,
                       float *out, void *ws, void *stream)
{
    const int G = H / Hkv;
    const int64_t S = attn_splits(n);
    const float scale = 1.0f / sqrtf(float(kAttnHeadDim));
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 grid{unsigned(S), unsigned(Hkv)};
    auto qp = static_cast<const uint16_t *>(q), kp = static_cast<const uint16_t *>(k),
         vp = static_cast<const uint16_t *>(v);
    float *w = static_cast<float *>(ws);
    switch (G) {
    case 1: k_attn_part<1><<<grid, 64, 0, st>>>(qp, kp, vp, n, Hkv, scale, w); break;
    case 2: k_attn_part<2><<<grid, 64, 0, st>>>(qp, kp, vp, n, Hkv, scale, w); break;
    case 4: k_attn_part<4><<<grid, 64, 0, st>>>(qp, kp, vp, n, Hkv, scale, w); break;
    case 8: k_attn_part<8><<<grid, 64, 0, st>>>(qp, kp, vp, n, Hkv, scale, w); break;
    default: return int(hipErrorInvalidValue);
    }
    k_attn_merge<<<unsigned(H), 256, 0, st>>>(w, S, H, out);
    return int(hipGetLastError());
}

}  // namespace tw
