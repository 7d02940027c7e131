// tw_head.hip -- approximate output head over a clustered vocabulary ("A 20B AI Model Trained in
// Ternary Just Hit 218 Tokens/Second on a $599 Mac Mini", section "The Architecture: Designed for
// the Hardware": the vocabulary is split into 4,748 clusters, 4-bit centroid scores pick the 512
// most relevant ones, and only their tokens get full-precision logits).
//
// Three launches on the caller's stream:
//   k_head_score   each wave scores up to eight centroid rows, all their loads issued before h
//                  is quantised to int8 by absmax in the workgroup (the same fp32 steps as the int8
//                  FFN path, so the codes are identical); each lane holds the codes of its
//                  32-input chunks as even/odd int8x4 words, and the offset-binary nibbles
//                  (value + 8) of the centroid are masked into int8x4 words for v_dot4; the exact
//                  sum is corrected by -8 sum(q) and scaled, score = (float(acc) * s_h) * scale
//                  (two fp32 roundings);
//   k_head_rank    every cluster's rank (the clusters with a higher score, or the same score and a
//                  lower id) by one wave per two clusters over all keys in LDS; the clusters of
//                  rank < top write their id at that rank;
//   k_head_logits  one workgroup per selected cluster, four waves; each wave takes rows
//                  wave, wave + 4, ... of the cluster's cluster-major head rows, all loads of a
//                  batch of rows issued first, fp32 dot with h (from LDS), wave sum.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tw_aux.h"
#include "tw_device.h"
#include "tw_internal.h"

namespace tw {
namespace {

// int8 image of h (absmax) into LDS, and its scale; every thread of the workgroup takes part.
template <int NT>
__device__ __forceinline__ float head_quant_h(const uint16_t *__restrict__ h, int d, int8_t *s_q,
                                              float *s_red)
{
    const int t = threadIdx.x;
    constexpr int PER = kHeadMaxD / NT;
    float hv[PER];
#pragma unroll
    for (int m = 0; m < PER; m++) {   // every load issued before the first is used
        const int i = t + NT * m;
        hv[m] = i < d ? bf16_to_f32(h[i]) : 0.0f;
    }
    float am = 0.0f;
#pragma unroll
    for (int m = 0; m < PER; m++) am = fmaxf(am, fabsf(hv[m]));
    am = wave_max(am);
    if ((t & 63) == 0) s_red[t >> 6] = am;
    __syncthreads();
    am = 0.0f;
#pragma unroll
    for (int w = 0; w < NT / 64; w++) am = fmaxf(am, s_red[w]);
    const float inv = 127.0f / am;
#pragma unroll
    for (int m = 0; m < PER; m++) {
        const int i = t + NT * m;
        if (i < d) s_q[i] = am > 0.0f ? int8_quant(hv[m], inv) : int8_t(0);
    }
    __syncthreads();
    return am > 0.0f ? am / 127.0f : 0.0f;
}

// Each wave scores up to kHeadRowsPerWave centroid rows (rows blockIdx.x * 4 + wave + k * gridDim.x
// * 4); all of its row loads are issued first, so they are in flight while h is quantised.
constexpr int kHeadRowsPerWave = 8;

template <int MC>   // MC = d / 2048 rounded up: 16-byte centroid chunks per lane and row
__global__ __launch_bounds__(256) void k_head_score(const uint16_t *__restrict__ h, int d,
                                                    const uint8_t *__restrict__ cent,
                                                    const float *__restrict__ cscale, int ncl,
                                                    float *__restrict__ scores)
{
    __shared__ int8_t s_q[kHeadMaxD];
    __shared__ float s_red[4];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int nch = d / 32;   // 32-input chunks (16 centroid bytes) per row
    uint4 cv[kHeadRowsPerWave][MC];
    float csc[kHeadRowsPerWave];
#pragma unroll
    for (int k = 0; k < kHeadRowsPerWave; k++) {
        const int c0 = blockIdx.x * 4 + wave + k * gridDim.x * 4;
        const uint4 *row = reinterpret_cast<const uint4 *>(cent + int64_t(c0 < ncl ? c0 : 0) * (d / 2));
#pragma unroll
        for (int m = 0; m < MC; m++)
            cv[k][m] = c0 < ncl && lane + 64 * m < nch ? row[lane + 64 * m] : make_uint4(0, 0, 0, 0);
        csc[k] = c0 < ncl && lane == 0 ? cscale[c0] : 0.0f;
    }
    const float sh = head_quant_h<256>(h, d, s_q, s_red);
    // this lane's chunks: even and odd input words, and sum(q)
    uint32_t xe[MC][4], xo[MC][4];
    int32_t sq = 0;
#pragma unroll
    for (int m = 0; m < MC; m++) {
        const int c = lane + 64 * m;
#pragma unroll
        for (int w = 0; w < 4; w++) {
            xe[m][w] = xo[m][w] = 0u;
            if (c < nch) {
                const int b = 32 * c + 8 * w;
                int32_t e[4], o[4];
#pragma unroll
                for (int k = 0; k < 4; k++) {
                    e[k] = s_q[b + 2 * k];
                    o[k] = s_q[b + 2 * k + 1];
                    sq += e[k] + o[k];
                }
                xe[m][w] = (uint32_t(uint8_t(e[0]))) | (uint32_t(uint8_t(e[1])) << 8) |
                           (uint32_t(uint8_t(e[2])) << 16) | (uint32_t(uint8_t(e[3])) << 24);
                xo[m][w] = (uint32_t(uint8_t(o[0]))) | (uint32_t(uint8_t(o[1])) << 8) |
                           (uint32_t(uint8_t(o[2])) << 16) | (uint32_t(uint8_t(o[3])) << 24);
            }
        }
    }
    int32_t sqw[1] = {sq};
    group_reduce<1>(sqw, 64);   // sum(q) over the row, in every lane
#pragma unroll
    for (int k = 0; k < kHeadRowsPerWave; k++) {
        const int c0 = blockIdx.x * 4 + wave + k * gridDim.x * 4;
        if (c0 >= ncl) break;   // uniform over the wave
        int32_t acc[1] = {0};
#pragma unroll
        for (int m = 0; m < MC; m++) {
            const uint32_t wd[4] = {cv[k][m].x, cv[k][m].y, cv[k][m].z, cv[k][m].w};
#pragma unroll
            for (int w = 0; w < 4; w++) {
                acc[0] = __builtin_amdgcn_sdot4(int32_t(wd[w] & 0x0F0F0F0Fu), int32_t(xe[m][w]), acc[0], false);
                acc[0] = __builtin_amdgcn_sdot4(int32_t((wd[w] >> 4) & 0x0F0F0F0Fu), int32_t(xo[m][w]), acc[0], false);
            }
        }
        group_reduce<1>(acc, 64);
        if (lane == 0) scores[c0] = (float(acc[0] - 8 * sqw[0]) * sh) * csc[k];
    }
}

// Orderable key of an fp32 score (larger score, larger key; -0 taken as +0, so equal scores give
// equal keys and the id decides).  Every real key is above 0, the key of the padding.
__device__ __forceinline__ uint32_t score_key(float s)
{
    const uint32_t u = __float_as_uint(s == 0.0f ? 0.0f : s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Rank selection: a cluster's place in the output is the number of clusters that come before it
// (higher score key, or the same key and a lower id).  Each wave counts that for two clusters
// against every cluster's key (the keys of all clusters are first copied
// into LDS as 64-bit composites key << 32 | ~id, so that "comes before" is one unsigned compare and
// every composite is distinct), and the clusters of rank < top write their id to sel[rank].  The
// ranks are exact integer counts, so the selection and its order do not depend on the launch
// shape; no threshold search, no sort and no single-workgroup step.
__global__ __launch_bounds__(256) void k_head_rank(const float *__restrict__ scores, int ncl, int top,
                                                   int32_t *__restrict__ sel)
{
    extern __shared__ uint64_t s_c[];   // ncl composites
    const int t = threadIdx.x;
    constexpr int PER = kHeadMaxClusters / 256;
    float sv[PER];
#pragma unroll
    for (int m = 0; m < PER; m++) {   // every score load issued before the first is used
        const int i = t + 256 * m;
        sv[m] = i < ncl ? scores[i] : 0.0f;
    }
#pragma unroll
    for (int m = 0; m < PER; m++) {
        const int i = t + 256 * m;
        if (i < ncl) s_c[i] = (uint64_t(score_key(sv[m])) << 32) | uint64_t(~uint32_t(i));
    }
    __syncthreads();
    // each wave ranks two clusters: every key read from LDS is compared with both
    const int lane = t & 63;
    const int i0 = (blockIdx.x * 4 + (t >> 6)) * 2, i1 = i0 + 1;
    const uint64_t c0 = i0 < ncl ? s_c[i0] : ~uint64_t(0), c1 = i1 < ncl ? s_c[i1] : ~uint64_t(0);
    int32_t cnt[2] = {0, 0};
#pragma unroll 4
    for (int j = lane; j < ncl; j += 64) {
        const uint64_t cj = s_c[j];
        cnt[0] += int32_t(cj > c0);
        cnt[1] += int32_t(cj > c1);
    }
    group_reduce<2>(cnt, 64);
    if (lane == 0 && i0 < ncl && cnt[0] < top) sel[cnt[0]] = i0;
    if (lane == 1 && i1 < ncl && cnt[1] < top) sel[cnt[1]] = i1;
}

template <int M>   // M = d / 512: 8-input chunks per lane and row
__global__ __launch_bounds__(256) void k_head_logits(const uint16_t *__restrict__ h, int d,
                                                     const uint16_t *__restrict__ wc,
                                                     const int32_t *__restrict__ members, int cs,
                                                     const int32_t *__restrict__ sel,
                                                     int32_t *__restrict__ ids,
                                                     float *__restrict__ logits)
{
    constexpr int RB = 16 / M;   // rows per batch, all of a batch's loads in flight together
    __shared__ float s_h[kHeadMaxD];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int j = blockIdx.x;
    const int64_t c = sel[j];
    {
        constexpr int PER = kHeadMaxD / 256;
        float hv[PER];
#pragma unroll
        for (int m = 0; m < PER; m++) {   // every load issued before the first is used
            const int i = t + 256 * m;
            hv[m] = i < d ? bf16_to_f32(h[i]) : 0.0f;
        }
#pragma unroll
        for (int m = 0; m < PER; m++)
            if (t + 256 * m < d) s_h[t + 256 * m] = hv[m];
    }
    __syncthreads();
    for (int r0 = wave; r0 < cs; r0 += 4 * RB) {
        uint4 buf[RB][M];
#pragma unroll
        for (int b = 0; b < RB; b++) {
            const int r = r0 + 4 * b;
            const uint4 *row = reinterpret_cast<const uint4 *>(wc + (c * cs + (r < cs ? r : 0)) * d);
#pragma unroll
            for (int m = 0; m < M; m++) buf[b][m] = row[lane + 64 * m];
        }
#pragma unroll
        for (int b = 0; b < RB; b++) {
            const int r = r0 + 4 * b;
            float acc = 0.0f;
#pragma unroll
            for (int m = 0; m < M; m++) {
                const uint32_t wd[4] = {buf[b][m].x, buf[b][m].y, buf[b][m].z, buf[b][m].w};
                const int e0 = 8 * (lane + 64 * m);
#pragma unroll
                for (int e = 0; e < 8; e++)
                    acc = acc + bf16_to_f32(uint16_t(wd[e >> 1] >> (16 * (e & 1)))) * s_h[e0 + e];
            }
            acc = wave_sum(acc);
            if (lane == 0 && r < cs) {
                logits[int64_t(j) * cs + r] = acc;
                ids[int64_t(j) * cs + r] = members[c * cs + r];
            }
        }
    }
}

}  // namespace

int launch_flash_head(const void *h, int d, const uint8_t *cent, const float *cscale, int ncl,
                      const void *wc, const int32_t *members, int cs, int top, int32_t *sel,
                      int32_t *ids, float *logits, void *ws, void *stream)
{
    hipStream_t st = static_cast<hipStream_t>(stream);
    auto hp = static_cast<const uint16_t *>(h);
    float *scores = static_cast<float *>(ws);
    // at most kHeadRowsPerWave rows per wave, and about 256 workgroups at the largest sizes
    const int waves = (ncl + kHeadRowsPerWave - 1) / kHeadRowsPerWave;
    const int nb = max((waves + 3) / 4, min((ncl + 3) / 4, 256));
    if (d > 2048)
        k_head_score<2><<<nb, 256, 0, st>>>(hp, d, cent, cscale, ncl, scores);
    else
        k_head_score<1><<<nb, 256, 0, st>>>(hp, d, cent, cscale, ncl, scores);
    k_head_rank<<<(ncl + 7) / 8, 256, size_t(ncl) * sizeof(uint64_t), st>>>(scores, ncl, top, sel);
    auto wp = static_cast<const uint16_t *>(wc);
    switch (d / 512) {
    case 1: k_head_logits<1><<<top, 256, 0, st>>>(hp, d, wp, members, cs, sel, ids, logits); break;
    case 2: k_head_logits<2><<<top, 256, 0, st>>>(hp, d, wp, members, cs, sel, ids, logits); break;
    case 4: k_head_logits<4><<<top, 256, 0, st>>>(hp, d, wp, members, cs, sel, ids, logits); break;
    case 8: k_head_logits<8><<<top, 256, 0, st>>>(hp, d, wp, members, cs, sel, ids, logits); break;
    default: return int(hipErrorInvalidValue);
    }
    return int(hipGetLastError());
}

}  // namespace tw
