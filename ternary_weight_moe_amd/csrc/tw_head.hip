// tw_head.hip -- approximate output head over a clustered vocabulary ("A 20B AI Model Trained in
// Ternary Just Hit 218 Tokens/Second on a $599 Mac Mini", section "The Architecture: Designed for
// the Hardware": the vocabulary is split into 4,748 clusters, 4-bit centroid scores pick the 512
// most relevant ones, and only their tokens get full-precision logits).
//
// Three launches on the caller's stream:
//   k_head_score   one wave per centroid row: h is quantised to int8 by absmax in every workgroup
//                  (the same fp32 steps as the int8 FFN path, so the codes are identical), each
//                  lane holds the codes of its 32-input chunks as even/odd int8x4 words, and the
//                  offset-binary nibbles (value + 8) of the centroid are masked into int8x4 words
//                  for v_dot4; the exact sum is corrected by -8 sum(q) and scaled,
//                  score = (float(acc) * s_h) * scale (two fp32 roundings);
//   k_head_select  one 1024-thread workgroup: the threshold key of the `top`-th cluster by three
//                  radix passes of 11, 11 and 10 bits (LDS histograms), the clusters above it plus the lowest ids
//                  at it, then a bitonic sort in LDS of those `top` (orderable score key, cluster
//                  id) pairs, descending by score and ascending by id;
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
    float am = 0.0f;
    for (int i = t; i < d; i += NT) am = fmaxf(am, fabsf(bf16_to_f32(h[i])));
    am = wave_max(am);
    if ((t & 63) == 0) s_red[t >> 6] = am;
    __syncthreads();
    am = 0.0f;
#pragma unroll
    for (int w = 0; w < NT / 64; w++) am = fmaxf(am, s_red[w]);
    const float inv = 127.0f / am;
    for (int i = t; i < d; i += NT) s_q[i] = am > 0.0f ? int8_quant(bf16_to_f32(h[i]), inv) : int8_t(0);
    __syncthreads();
    return am > 0.0f ? am / 127.0f : 0.0f;
}

__global__ __launch_bounds__(256) void k_head_score(const uint16_t *__restrict__ h, int d,
                                                    const uint8_t *__restrict__ cent,
                                                    const float *__restrict__ cscale, int ncl,
                                                    float *__restrict__ scores)
{
    __shared__ int8_t s_q[kHeadMaxD];
    __shared__ float s_red[4];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int nch = d / 32;   // 32-input chunks (16 centroid bytes) per row
    const float sh = head_quant_h<256>(h, d, s_q, s_red);
    // this lane's chunks (at most kHeadMaxD / 2048 = 2): even and odd input words, and sum(q)
    constexpr int MC = kHeadMaxD / 32 / 64;
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
    for (int c0 = blockIdx.x * 4 + wave; c0 < ncl; c0 += gridDim.x * 4) {
        const uint4 *row = reinterpret_cast<const uint4 *>(cent + int64_t(c0) * (d / 2));
        uint4 cv[MC];
#pragma unroll
        for (int m = 0; m < MC; m++) cv[m] = lane + 64 * m < nch ? row[lane + 64 * m] : make_uint4(0, 0, 0, 0);
        int32_t acc[1] = {0};
#pragma unroll
        for (int m = 0; m < MC; m++) {
            const uint32_t wd[4] = {cv[m].x, cv[m].y, cv[m].z, cv[m].w};
#pragma unroll
            for (int w = 0; w < 4; w++) {
                acc[0] = __builtin_amdgcn_sdot4(int32_t(wd[w] & 0x0F0F0F0Fu), int32_t(xe[m][w]), acc[0], false);
                acc[0] = __builtin_amdgcn_sdot4(int32_t((wd[w] >> 4) & 0x0F0F0F0Fu), int32_t(xo[m][w]), acc[0], false);
            }
        }
        group_reduce<1>(acc, 64);
        if (lane == 0) scores[c0] = (float(acc[0] - 8 * sqw[0]) * sh) * cscale[c0];
    }
}

// Orderable key of an fp32 score (larger score, larger key; -0 taken as +0, so equal scores give
// equal keys and the id decides).  Every real key is above 0, the key of the padding.
__device__ __forceinline__ uint32_t score_key(float s)
{
    const uint32_t u = __float_as_uint(s == 0.0f ? 0.0f : s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(1024) void k_head_select(const float *__restrict__ scores, int ncl,
                                                      int top, int32_t *__restrict__ sel)
{
    constexpr int PER = kHeadMaxClusters / 1024;
    __shared__ uint32_t s_key[kHeadMaxClusters];
    __shared__ uint16_t s_id[kHeadMaxClusters];
    __shared__ int s_hist[2048];
    __shared__ int s_wc[kHeadMaxClusters / 1024][16];
    __shared__ uint32_t s_prefix;
    __shared__ int s_above, s_cnt;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    uint32_t key[PER];
#pragma unroll
    for (int m = 0; m < PER; m++) {
        const int i = t + 1024 * m;
        key[m] = i < ncl ? score_key(scores[i]) : 0u;
    }
    // 1. the threshold key T (count(key > T) < top <= count(key >= T)) by three radix passes of
    //    11, 11 and 10 bits from the top down; `above` counts the keys above the current bucket
    uint32_t prefix = 0, mask = 0;
    int above = 0;
#pragma unroll
    for (int pass = 0; pass < 3; pass++) {
        const int shift = pass == 0 ? 21 : pass == 1 ? 10 : 0, bits = pass == 2 ? 10 : 11;
        const int nbins = 1 << bits, per = nbins / 64;
        for (int i = t; i < nbins; i += 1024) s_hist[i] = 0;
        __syncthreads();
#pragma unroll
        for (int m = 0; m < PER; m++)
            if (t + 1024 * m < ncl && (key[m] & mask) == prefix)
                atomicAdd(&s_hist[(key[m] >> shift) & uint32_t(nbins - 1)], 1);
        __syncthreads();
        if (wave == 0) {
            // lane l holds bins nbins-1-per*l .. down; counts accumulate from the highest bin down
            int tot = 0;
            for (int q = 0; q < per; q++) tot += s_hist[nbins - 1 - per * lane - q];
            int inc = tot;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int v = __shfl_up(inc, off);
                if (lane >= off) inc += v;
            }
            int run = above + inc - tot, found = -1, found_above = 0;
            for (int q = 0; q < per; q++) {
                const int c = s_hist[nbins - 1 - per * lane - q];
                if (found < 0 && run + c >= top) {
                    found = nbins - 1 - per * lane - q;
                    found_above = run;
                }
                run += c;
            }
            const uint64_t bal = __ballot(found >= 0);
            if (lane == __ffsll((unsigned long long)bal) - 1) {
                s_prefix = prefix | (uint32_t(found) << shift);
                s_above = found_above;
            }
        }
        __syncthreads();
        prefix = s_prefix;
        above = s_above;
        mask |= uint32_t(nbins - 1) << shift;
        __syncthreads();
    }
    // 2. the selected clusters: every key above T, and the (top - above) lowest ids with key T
    //    (ranked in id order: row m of 1024 ids before row m + 1, waves in order inside a row),
    //    collected in LDS in any order; one barrier for the per-wave counts of all rows
    const int need = top - above;
    if (t == 0) s_cnt = 0;
    uint64_t eqb[PER];
#pragma unroll
    for (int m = 0; m < PER; m++) {
        const int i = t + 1024 * m;
        eqb[m] = __ballot(i < ncl && key[m] == prefix);
        if (lane == 0) s_wc[m][wave] = __popcll(eqb[m]);
    }
    __syncthreads();
    int eq_before = 0;
#pragma unroll
    for (int m = 0; m < PER; m++) {
        const int i = t + 1024 * m;
        const bool valid = i < ncl;
        const bool gt = valid && key[m] > prefix, eq = valid && key[m] == prefix;
        int before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < 16; w++) {
            before += w < wave ? s_wc[m][w] : 0;
            total += s_wc[m][w];
        }
        const int r = __popcll(eqb[m] & ((uint64_t(1) << lane) - 1));
        if (gt || (eq && eq_before + before + r < need)) {
            const int pos = atomicAdd(&s_cnt, 1);
            s_key[pos] = key[m];
            s_id[pos] = uint16_t(i);
        }
        eq_before += total;
    }
    __syncthreads();
    // 3. bitonic sort of the `top` selected (padded to a power of two N), descending by key, then
    //    lower id first.  Up to 1024 of them: one per thread in registers, partners at distance
    //    below 64 exchanged by lane shuffles, farther ones through LDS (5 barrier stages for 512);
    //    more than 1024: the same network entirely in LDS.
    int N = 1;
    while (N < top) N <<= 1;
    if (N <= 1024) {
        uint32_t kk = t < top ? s_key[t] : 0u;
        uint32_t ii = t < top ? uint32_t(s_id[t]) : 0xFFFFu;
        for (int k = 2; k <= N; k <<= 1) {
            for (int j = k >> 1; j > 0; j >>= 1) {
                uint32_t kp, ip;
                if (j >= 64) {
                    __syncthreads();   // every read of the previous exchange is done
                    if (t < N) {
                        s_key[t] = kk;
                        s_id[t] = uint16_t(ii);
                    }
                    __syncthreads();
                    kp = t < N ? s_key[t ^ j] : 0u;
                    ip = t < N ? uint32_t(s_id[t ^ j]) : 0xFFFFu;
                } else {
                    kp = uint32_t(__shfl_xor(int(kk), j));
                    ip = uint32_t(__shfl_xor(int(ii), j));
                }
                const bool mine_first = kk > kp || (kk == kp && ii < ip);
                const bool keep_first = ((t & j) == 0) == ((t & k) == 0);
                if (keep_first != mine_first) {
                    kk = kp;
                    ii = ip;
                }
            }
        }
        if (t < top) sel[t] = int32_t(ii);
        return;
    }
    for (int i = top + t; i < N; i += 1024) {
        s_key[i] = 0u;
        s_id[i] = 0xFFFF;
    }
    __syncthreads();
    for (int k = 2; k <= N; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = t; i < N; i += 1024) {
                const int l = i ^ j;
                if (l > i) {
                    const uint32_t ki = s_key[i], kl = s_key[l];
                    const uint16_t ii = s_id[i], il = s_id[l];
                    const bool l_first = kl > ki || (kl == ki && il < ii);   // l ranks before i
                    const bool i_first = ki > kl || (ki == kl && ii < il);
                    if (((i & k) == 0) ? l_first : i_first) {
                        s_key[i] = kl;
                        s_key[l] = ki;
                        s_id[i] = il;
                        s_id[l] = ii;
                    }
                }
            }
            __syncthreads();
        }
    }
    for (int i = t; i < top; i += 1024) sel[i] = int32_t(s_id[i]);
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
    for (int i = t; i < d; i += 256) s_h[i] = bf16_to_f32(h[i]);
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
    const int nb = (ncl + 3) / 4 < 1024 ? (ncl + 3) / 4 : 1024;
    k_head_score<<<nb, 256, 0, st>>>(hp, d, cent, cscale, ncl, scores);
    k_head_select<<<1, 1024, 0, st>>>(scores, ncl, top, sel);
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
