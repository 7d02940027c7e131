// tw_prefill.hip -- grouped MFMA path of the batched FFN (gfx950): every call whose shape it is
// instantiated for, from a few tokens per expert (batched decode) to many (prefill-shaped).
//
// The ternary products are int8 contractions and run on the matrix cores:
// v_mfma_i32_16x16x64_i8 multiplies a 16x64 int8 tile of weights (A operand, decoded in registers
// from the 2-bit codes) by a 64x16 int8 tile of activations (B operand, from LDS) into exact 16x16
// int32 sums.  Activations enter as P int8 planes (P = 1: int8 absmax mode; P = 2: the digit planes
// of bf16 inputs, tw_device.h); the activation tile holds MT x P rows (token m, plane pl at row
// m P + pl) and each MFMA takes 16 of them, so with two planes its 16 columns are 8 tokens x 2
// planes and the two lanes of a token combine their sums with one DPP exchange.  Every result is
// bit-identical to the per-pair v_dot4 path and to the batch-1 decode.
//
// One workgroup (8 or 16 waves) takes one (expert e, tile of MT tokens) work item (with 64-token
// tiles, an expert's last tile of at most 32 tokens runs the same steps compiled for 32):
//   1. the tile's MT x P rows of activation digits (d bytes each, 4x4-transposed inside groups of
//      16 as in tw_device.h) are copied into LDS, rows padded by 16 bytes so that the 16 rows read
//      by one MFMA operand fetch spread over the banks;
//   2. gate/up: wave w owns h rows [F/W w, F/W (w+1)) in groups of 16; the group's gate and up code
//      rows stream through a ring of register slots (each lane: one row, 16 bytes per 256 inputs,
//      several units in flight), each code word is decoded into the 16 int8 weights of an MFMA A
//      operand with nine ALU operations (no LDS round trip), and the activation fragments of the
//      next step are read from LDS while the current one is computed; the epilogue forms gate, up
//      and h = SiLU(gate) * up in fp32 in the order of the specification, in registers;
//   3. per token: max |h| over all F rows (registers, lane shuffles, LDS over waves), h re-quantised
//      (int8 absmax) or split into digit planes into LDS;
//   4. down: wave w owns d/W output rows; same scheme with the down codes; four consecutive outputs
//      of a token per lane stored as one vector per (token, slot) pair for the ordered combine:
//      y in fp32, except for int8 activations in 64-token tiles (prefill-shaped calls): there the
//      int32 down sums themselves are stored as int16 (|sum| <= 127 F; a sum outside the int16
//      range is marked and kept in 32-bit rows), and the combine forms y = (sum s_h) s_down from
//      them, which halves the bytes of the y round trip.  Small tiles keep fp32 y: their y traffic
//      is small and the combine's extra scale loads would cost more than it saves.
// K order: lane group g of an MFMA at step (S, s) covers inputs 256 S + 64 g + 16 s .. +16 -- a
// permutation of the inputs shared by both operands, so every int32 sum is the exact dot product.
// Work items are mapped to workgroups so that pairs of consecutive tiles (usually one expert) run on
// the same XCD at about the same time (workgroups b and b + 8 share an XCD): the second tile's code
// bytes then come from that XCD's L2.
// Prefill-shaped int8 calls (many tokens per expert) take k_pf_expert instead: one workgroup per
// expert's tokens (up to 192), described where it is defined.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "tw_device.h"
#include "tw_internal.h"

namespace tw {
namespace {

typedef int32_t v4i __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

// Waves per workgroup: 16 for 16-token tiles of at most two planes (at <= 128 VGPRs, four waves
// per SIMD); 8 otherwise (256 VGPRs: the h values of a 64-token tile stay in registers).
// AHEAD: code units (one 16-row block of gate and up codes over 256 inputs, or one 16-row block of
// down codes) each wave keeps in flight ahead of the one it computes: 4 for the small tiles (3 and 4
// measured the same, 5 slower), 2 for the large ones (4096 int8 tokens: 263.0 us per call against
// 266.2 with 3, 267.7 with 4 (register spills), 285.4 with 1).
template <int MT, int P>
struct PfShape {
    static constexpr int W = MT * P <= 16 ? 16 : 8;
    static constexpr int T = 64 * W;
    static constexpr int AHEAD = MT * P <= 16 ? 4 : 2;
};

// The 16 int8 weights of one 32-bit code word, in the transposed order of the activation digits.
__device__ __forceinline__ v4i decode16(uint32_t w)
{
    int32_t a, b, c, d;
    decode_word(w, a, b, c, d);
    return v4i{a, b, c, d};
}

__device__ __forceinline__ uint32_t word_of(const int4 &v, int s)
{
    return uint32_t(s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w);
}

__device__ __forceinline__ float comp(const float4 &v, int r)
{
    return r == 0 ? v.x : r == 1 ? v.y : r == 2 ? v.z : v.w;
}

// Address of 16-byte chunk c of row r in a tile of rows of `rowb` bytes, each padded by 16 bytes.
__device__ __forceinline__ int tofs(int r, int c, int rowb) { return r * (rowb + 16) + 16 * c; }

// Weights as the A operand, activations as B: the result tile is [weight row][token], so lane l
// holds rows 4 (l / 16) .. +3 of token l % 16.
__device__ __forceinline__ v4i mfma8(const v4i &w, const v4i &x, const v4i &c)
{
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(w, x, c, 0, 0, 0);
}

// The work of one (expert e, tile) item after the tile lookup: meta = (position of the tile's first
// pair in the pair list: k_group's pairs[] or, SELF, the expert's list in LDS, s_list), tokens).
// MT: tokens the body is compiled for (the kernel's tile size, or half of it for an expert's last
// tile when that holds at most half); Y16: the call keeps 16-bit down sums (decided per call, so
// that a half-size tile stores the same form as the full ones).
template <int D, int F, int P, int MT, bool SELF, bool Y16>
__device__ __forceinline__ void pf_work(const Dims &dm, const BatchedWs &L, const LayerPtrs &lp, uint8_t *ws,
                                        int e, int2 meta, const int32_t *s_list, int8_t *sm)
{
    constexpr int W = PfShape<MT, P>::W, NT = PfShape<MT, P>::T;
    constexpr bool INT8 = P == 1;
    constexpr int RS = MT * P / 16;       // row sub-tiles
    constexpr int TPS = 16 / P;           // tokens per row sub-tile
    constexpr int GPW = F / 16 / W;       // h-row groups of 16 per wave
    constexpr int NSD = D / 16 / W;       // down row blocks of 16 per wave
    constexpr int SG = D / 256, SD = F / 256;
    constexpr int NGU = GPW * SG;         // gate/up code units per wave, then NSD down units
    constexpr int kPfAhead = PfShape<MT, P>::AHEAD;
    constexpr int NU = NGU + NSD, RING = kPfAhead + 1;
    static_assert(SD <= 2, "a down unit is at most two 16-byte chunks per lane");
    static_assert(!Y16 || INT8, "16-bit down sums need int8 activations");
    __shared__ int32_t s_pair[MT];
    __shared__ float s_tk[MT][2];         // per token: s_x (int8) or digit shift bits; 1/rms
    __shared__ float s_hk[MT];            // per token: s_h (int8) or digit shift bits of h
    __shared__ float s_amx[MT];
    __shared__ float s_pam[W][MT];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, l16 = lane & 15, g4 = lane >> 4;
    (void)NT;
    // The activation tile has MT * P rows (token m, plane pl at row m P + pl); an MFMA takes 16 of
    // them, so the 16 result columns of sub-tile rs are 16 / P tokens x P planes: column l16 is
    // token rs * TPS + l16 / P, plane l16 % P.  With two planes the two lanes of a token combine
    // their sums with one DPP exchange.

    // Code units of this wave, in the order they are computed.  Unit u < NGU: gate and up chunk
    // u % SG of h-row group u / SG (plus, with the first chunk, the group's gate and up scales);
    // unit NGU + n: the down codes and scales of output row block n.  All loops over units are
    // unrolled, so ring slots and scale registers are static.
    int4 ring[RING][2];
    float4 gsc[GPW][2], dsc[NSD];
    // uniform bases (scalar registers) plus one 32-bit offset per lane
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const uint8_t *gbase = lp.w_gate + (int64_t(e) * F + wv * GPW * 16) * (D / 4);
    const uint8_t *ubase = lp.w_up + (int64_t(e) * F + wv * GPW * 16) * (D / 4);
    const uint8_t *dbase = lp.w_down + (int64_t(e) * D + wv * NSD * 16) * (F / 4);
    const float *gsbase = lp.s_gate + int64_t(e) * F + wv * GPW * 16;
    const float *usbase = lp.s_up + int64_t(e) * F + wv * GPW * 16;
    const float *dsbase = lp.s_down + int64_t(e) * D + wv * NSD * 16;
    const uint32_t gofs = uint32_t(l16 * (D / 4) + 16 * g4), dofs = uint32_t(l16 * (F / 4) + 16 * g4);
    const uint32_t sofs = uint32_t(4 * g4);
    auto issue = [&](int u) {
        if (u >= NU) return;
        int4 (&slot)[2] = ring[u % RING];
        if (u < NGU) {
            const int gi = u / SG, kc = u % SG;
            slot[0] = *reinterpret_cast<const int4 *>(gbase + gi * 16 * (D / 4) + 64 * kc + gofs);
            slot[1] = *reinterpret_cast<const int4 *>(ubase + gi * 16 * (D / 4) + 64 * kc + gofs);
            if (kc == 0) {
                gsc[gi][0] = *reinterpret_cast<const float4 *>(gsbase + gi * 16 + sofs);
                gsc[gi][1] = *reinterpret_cast<const float4 *>(usbase + gi * 16 + sofs);
            }
        } else {
            const int n = u - NGU;
            slot[0] = *reinterpret_cast<const int4 *>(dbase + n * 16 * (F / 4) + dofs);
            if (SD > 1) slot[1] = *reinterpret_cast<const int4 *>(dbase + n * 16 * (F / 4) + 64 + dofs);
            if constexpr (!Y16) dsc[n] = *reinterpret_cast<const float4 *>(dsbase + n * 16 + sofs);
        }
    };
#pragma unroll
    for (int u = 0; u < kPfAhead; u++) issue(u);

    const int32_t *pairs = reinterpret_cast<const int32_t *>(ws + L.pairs);
    const float *tinfo = reinterpret_cast<const float *>(ws + L.tinfo);
    const int8_t *xdig = reinterpret_cast<const int8_t *>(ws + L.xdig);
    float *ybuf = reinterpret_cast<float *>(ws + L.y);
    int16_t *y16 = reinterpret_cast<int16_t *>(ws + L.y16);    // int8 activations: 16-bit sums,
    int32_t *ywide = reinterpret_cast<int32_t *>(ws + L.y);    // the sums that do not fit them,
    float *shp = reinterpret_cast<float *>(ws + L.shp);        // and each pair's s_h
    const int k = dm.k;
    const int pl = l16 % P;                         // this lane's plane in every sub-tile
    const int nv = meta.y;                          // tokens in this tile (1 .. MT)
    const int rsv = (nv + TPS - 1) / TPS;           // row sub-tiles holding any of them
    if constexpr (SELF) __syncthreads();            // the expert's pair list is complete
    if (t < MT) s_pair[t] = t < nv ? (SELF ? s_list[meta.x + t] : pairs[meta.x + t]) : -1;
    __syncthreads();
    // 1. activation tile: row (m, plane) = plane of token m, and each token's scale words; every
    //    load is issued before the first LDS store (padding tokens re-read token 0's row, which
    //    every tile has, and store zeros)
    {
        constexpr int NCH = MT * P * (D / 16), PER = (NCH + NT - 1) / NT;
        const int pr0 = s_pair[0];
        int4 v[PER];
        float tk0 = 0.0f, tk1 = 0.0f;
        if (t < MT) {
            const int pr = s_pair[t] >= 0 ? s_pair[t] : pr0;
            tk0 = tinfo[2 * (pr / k)];
            tk1 = tinfo[2 * (pr / k) + 1];
        }
#pragma unroll
        for (int i = 0; i < PER; i++) {
            const int idx = min(t + i * NT, NCH - 1);
            const int r = idx / (D / 16), c = idx % (D / 16);
            const int pr = s_pair[r / P] >= 0 ? s_pair[r / P] : pr0;
            v[i] = reinterpret_cast<const int4 *>(xdig + (int64_t(pr / k) * P + r % P) * D)[c];
        }
        if (t < MT) {
            s_tk[t][0] = s_pair[t] >= 0 ? tk0 : 0.0f;
            s_tk[t][1] = s_pair[t] >= 0 ? tk1 : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < PER; i++) {
            const int idx = t + i * NT;
            const int r = idx / (D / 16);
            if (idx < NCH)
                *reinterpret_cast<int4 *>(sm + tofs(r, idx % (D / 16), D)) =
                    s_pair[r / P] >= 0 ? v[i] : make_int4(0, 0, 0, 0);
        }
    }
    __syncthreads();

    // 2. gate/up, one unit (4 steps of 64 inputs) at a time, kPfAhead units in flight
    float hreg[GPW][RS][4];
#pragma unroll
    for (int gi = 0; gi < GPW; gi++) {
        v4i accg[RS], accu[RS];
#pragma unroll
        for (int rs = 0; rs < RS; rs++) accg[rs] = accu[rs] = v4i{0, 0, 0, 0};
        // the activation fragments of step q + 1 are read from LDS while step q is computed
        v4i avc[RS], avn[RS];
        auto read_av = [&](int q, v4i (&av)[RS]) {
            const int c = 16 * (q >> 2) + 4 * g4 + (q & 3);
#pragma unroll
            for (int rs = 0; rs < RS; rs++)
                av[rs] = *reinterpret_cast<const v4i *>(sm + tofs(rs * 16 + l16, c, D));
        };
        read_av(0, avc);
#pragma unroll
        for (int kc = 0; kc < SG; kc++) {
            const int u = gi * SG + kc;
            issue(u + kPfAhead);
            const int4 gq = ring[u % RING][0], uq = ring[u % RING][1];
#pragma unroll
            for (int s = 0; s < 4; s++) {
                const int q = 4 * kc + s;
                if (q + 1 < 4 * SG) read_av(q + 1, avn);
                const v4i bg = decode16(word_of(gq, s)), bu = decode16(word_of(uq, s));
#pragma unroll
                for (int rs = 0; rs < RS; rs++) {
                    accg[rs] = mfma8(bg, avc[rs], accg[rs]);
                    accu[rs] = mfma8(bu, avc[rs], accu[rs]);
                }
#pragma unroll
                for (int rs = 0; rs < RS; rs++) avc[rs] = avn[rs];
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // epilogue: lane holds h rows 16 gi' + 4 g4 + r of token rs * TPS + l16 / P
#pragma unroll
        for (int rs = 0; rs < RS; rs++) {
            if (rs > 0 && rs >= rsv) {
#pragma unroll
                for (int r = 0; r < 4; r++) hreg[gi][rs][r] = 0.0f;
                continue;
            }
            const int m = rs * TPS + l16 / P;
            const float tk0 = s_tk[m][0], tk1 = s_tk[m][1];
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const float sgv = comp(gsc[gi][0], r), suv = comp(gsc[gi][1], r);
                float gate, up;
                if constexpr (INT8) {
                    gate = (float(accg[rs][r]) * tk0) * sgv;
                    up = (float(accu[rs][r]) * tk0) * suv;
                } else {
                    const int32_t og = dpp_i<kDppXor1>(accg[rs][r]), ou = dpp_i<kDppXor1>(accu[rs][r]);
                    const int32_t ag[2] = {pl == 0 ? accg[rs][r] : og, pl == 0 ? og : accg[rs][r]};
                    const int32_t au[2] = {pl == 0 ? accu[rs][r] : ou, pl == 0 ? ou : accu[rs][r]};
                    const int sh = __float_as_int(tk0);
                    gate = float_value<2>(ag, sh) * sgv * tk1;
                    up = float_value<2>(au, sh) * suv * tk1;
                }
                hreg[gi][rs][r] = tw_silu(gate) * up;
            }
            __builtin_amdgcn_sched_barrier(0);   // four SiLUs at a time: bounded temporaries
        }
    }

    // 3. per-token max |h| (registers, the four lanes of a token, LDS over waves), then int8
    //    re-quantisation or digit planes of h into LDS (with two planes, each lane of a token
    //    writes its own plane)
#pragma unroll
    for (int rs = 0; rs < RS; rs++) {
        float v = 0.0f;
#pragma unroll
        for (int gi = 0; gi < GPW; gi++)
#pragma unroll
            for (int r = 0; r < 4; r++) v = fmaxf(v, fabsf(hreg[gi][rs][r]));
        v = fmaxf(v, __shfl_xor(v, 16));
        v = fmaxf(v, __shfl_xor(v, 32));
        if (g4 == 0 && pl == 0) s_pam[wave][rs * TPS + l16 / P] = v;
    }
    __syncthreads();   // every wave is done with the activation tile
    if (t < MT) {
        float am = 0.0f;
#pragma unroll
        for (int w = 0; w < W; w++) am = fmaxf(am, s_pam[w][t]);
        s_amx[t] = am;
        if (INT8) {
            s_hk[t] = am > 0.0f ? am / 127.0f : 0.0f;
            if (Y16 && s_pair[t] >= 0) shp[s_pair[t]] = s_hk[t];   // the combine forms y from it
        } else {
            s_hk[t] = __int_as_float(float_digit_shift(am, P));
        }
    }
    __syncthreads();
#pragma unroll
    for (int rs = 0; rs < RS; rs++) {
        const int m = rs * TPS + l16 / P;
        const float am = s_amx[m], hk = s_hk[m];
#pragma unroll
        for (int gi = 0; gi < GPW; gi++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int pos = perm16((wave * GPW + gi) * 16 + 4 * g4 + r);
                int8_t q;
                if constexpr (INT8) {
                    q = am > 0.0f ? int8_quant(hreg[gi][rs][r], 127.0f / am) : int8_t(0);
                } else {
                    int8_t dg[2];
                    float_digits<2>(hreg[gi][rs][r], __float_as_int(hk), dg);
                    q = pl == 0 ? dg[0] : dg[1];
                }
                sm[tofs(m * P + pl, pos >> 4, F) + (pos & 15)] = q;
            }
    }
    __syncthreads();

    // 4. down, one 16-row block per unit; lane holds output rows R0 + 4 g4 .. +3 of token
    //    ms * 16 + l16 and stores them as one 16-byte vector (padding tokens write a spare row
    //    behind the last pair, one per workgroup slot so that few workgroups share one; every store
    //    is unconditional, so the wait for a code unit never has to wait for a store)
    // 16-bit sums: each row sub-tile's store offset (bytes from y16) is formed once, with this
    // wave's first output row, so that a unit's store adds only a constant
    uint32_t yoff[RS];
    if constexpr (Y16) {
#pragma unroll
        for (int rs = 0; rs < RS; rs++) {
            const int m = rs * TPS + l16 / P, pr = s_pair[m];
            const int64_t row = pr >= 0 ? int64_t(pr) : L.spare_row + (blockIdx.x % kSpareRows);
            yoff[rs] = uint32_t(row) * uint32_t(2 * D) + uint32_t(2 * (wave * NSD * 16 + 4 * g4));
        }
    }
#pragma unroll
    for (int n = 0; n < NSD; n++) {
        const int u = NGU + n;
        issue(u + kPfAhead);
        const int R0 = (wave * NSD + n) * 16;
        const int4 q0 = ring[u % RING][0], q1 = ring[u % RING][1];
        v4i acc[RS];
#pragma unroll
        for (int rs = 0; rs < RS; rs++) acc[rs] = v4i{0, 0, 0, 0};
        // h fragments of step i + 1 are read from LDS while step i is computed
        v4i hc[RS], hn[RS];
        auto read_h = [&](int i, v4i (&hv)[RS]) {
            const int c = 16 * (i >> 2) + 4 * g4 + (i & 3);
#pragma unroll
            for (int rs = 0; rs < RS; rs++)
                hv[rs] = *reinterpret_cast<const v4i *>(sm + tofs(rs * 16 + l16, c, F));
        };
        read_h(0, hc);
#pragma unroll
        for (int i = 0; i < 4 * SD; i++) {
            const int S = i >> 2, s = i & 3;
            if (i + 1 < 4 * SD) read_h(i + 1, hn);
            const v4i bd = decode16(word_of(S == 0 ? q0 : q1, s));
#pragma unroll
            for (int rs = 0; rs < RS; rs++) acc[rs] = mfma8(bd, hc[rs], acc[rs]);
#pragma unroll
            for (int rs = 0; rs < RS; rs++) hc[rs] = hn[rs];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int rs = 0; rs < RS; rs++) {
            if (rs > 0 && rs >= rsv) break;
            const int m = rs * TPS + l16 / P, pr = s_pair[m];
            // the second lane of a two-plane token holds the same values: it writes a spare row
            const int64_t row = pr >= 0 && pl == 0 ? int64_t(pr) : L.spare_row + (blockIdx.x % kSpareRows);
            if constexpr (Y16) {
                // 16-bit sums; a sum outside [-32767, 32767] is stored as the marker -32768 (the
                // clamp to [-32768, 32768] maps every such sum to a value whose low 16 bits are
                // 0x8000) and the four int32 sums of this lane go to the 32-bit rows as well
                int32_t c[4];
                bool wide = false;
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int32_t v = acc[rs][r];
                    c[r] = min(max(v, -32768), 32768);
                    wide = wide || uint32_t(v + 32767) > 65534u;
                }
                const uint2 hv = make_uint2((uint32_t(c[0]) & 0xffffu) | (uint32_t(c[1]) << 16),
                                            (uint32_t(c[2]) & 0xffffu) | (uint32_t(c[3]) << 16));
                *reinterpret_cast<uint2 *>(reinterpret_cast<uint8_t *>(y16) + yoff[rs] + 32 * n) = hv;
                if (wide)
                    *reinterpret_cast<int4 *>(ywide + row * D + R0 + 4 * g4) =
                        make_int4(acc[rs][0], acc[rs][1], acc[rs][2], acc[rs][3]);
            } else {
                const float hk = s_hk[m];
                float y[4];
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    if constexpr (INT8) {
                        y[r] = (float(acc[rs][r]) * hk) * comp(dsc[n], r);
                    } else {
                        const int32_t o = dpp_i<kDppXor1>(acc[rs][r]);
                        const int32_t ad[2] = {pl == 0 ? acc[rs][r] : o, pl == 0 ? o : acc[rs][r]};
                        y[r] = float_value<2>(ad, __float_as_int(hk)) * comp(dsc[n], r);
                    }
                }
                *reinterpret_cast<f4 *>(ybuf + row * D + R0 + 4 * g4) = f4{y[0], y[1], y[2], y[3]};
            }
        }
    }
}

// SELF: every workgroup builds the tile list itself from the T k expert ids (at most one id per
// thread): per-expert counts, the tiles of MT tokens per expert in expert order, this workgroup's
// tile, and the tile's pairs (the expert's pairs in ascending order).  The list is the one k_group
// writes (the same tiles in the same order; inside a tile k_group's order may differ, which changes
// nothing), so no grouping kernel runs.  Otherwise the work item comes from k_group's lists.
template <int D, int F, int P, int MT, bool SELF>
__global__ __launch_bounds__((PfShape<MT, P>::T)) void k_pf_ffn(Dims dm, BatchedWs L, LayerPtrs lp, uint8_t *ws, int nb,
                                                               const int32_t *__restrict__ sel_ids, int npairs)
{
    constexpr int W = PfShape<MT, P>::W, NT = PfShape<MT, P>::T;
    static_assert(D % 256 == 0 && F % 256 == 0 && F % (16 * W) == 0 && D % (16 * W) == 0, "shape");
    static_assert((P == 1 || P == 2) && (MT * P) % 16 == 0 && MT <= NT, "tile");
    // int8 activations in large tiles: 16-bit down sums (the combine forms y); else fp32 y
    constexpr bool Y16 = P == 1 && MT >= 64;
    extern __shared__ __attribute__((aligned(16))) int8_t sm[];   // [MT][P] rows of D, later of F
    __shared__ int32_t s_cnt[SELF ? NT : 1];    // SELF: pairs per expert, then the expert's pairs
    __shared__ int32_t s_wcnt[W], s_wtil[W];
    __shared__ int32_t s_sel[2];

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    // workgroups b and b + 8 run on the same XCD: they take consecutive tiles (usually one expert),
    // and every 16 workgroups cover 16 consecutive tiles, so work spreads evenly over the XCDs
    const int b = blockIdx.x;
    const int ti = (b / 16) * 16 + (b % 8) * 2 + ((b / 8) & 1);
    int e;
    int2 meta;   // first pair position (k_group lists) or tile (SELF), tokens of the tile
    if constexpr (SELF) {
        const int E = dm.E;
        const int id = t < npairs ? sel_ids[t] : -1;
        const bool valid = id >= 0 && id < E;
        if (t < E) s_cnt[t] = 0;
        __syncthreads();
        if (valid) atomicAdd(&s_cnt[id], 1);
        __syncthreads();
        // exclusive scan of the tiles per expert (expert t per thread), inside each wave and then
        // over the wave totals
        const int c = t < E ? s_cnt[t] : 0, nt = (c + MT - 1) / MT;
        int it = nt;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int u = __shfl_up(it, off);
            if (lane >= off) it += u;
        }
        if (lane == 63) s_wtil[wave] = it;
        if (t < 2) s_sel[t] = -1;
        __syncthreads();
        int bt = 0;
#pragma unroll
        for (int w = 0; w < W; w++) bt += w < wave ? s_wtil[w] : 0;
        const int tile0 = bt + it - nt;
        if (ti >= tile0 && ti < tile0 + nt) {   // this workgroup's tile belongs to expert t
            s_sel[0] = t;
            s_sel[1] = ti - tile0;
        }
        __syncthreads();
        e = s_sel[0];
        if (e < 0) return;   // past the last tile (uniform over the workgroup)
        const int tl = s_sel[1];
        // the expert's pairs in ascending order: a ballot per wave, then the waves' counts
        const uint64_t hit = __ballot(id == e);
        const int rank = __popcll(hit & ((uint64_t(1) << lane) - 1));
        if (lane == 0) s_wcnt[wave] = __popcll(hit);
        __syncthreads();   // every read of s_cnt is done
        int before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < W; w++) {
            before += w < wave ? s_wcnt[w] : 0;
            total += s_wcnt[w];
        }
        if (id == e) s_cnt[before + rank] = t;
        meta = make_int2(tl * MT, min(MT, total - tl * MT));
    } else {
        const int32_t *tiles = reinterpret_cast<const int32_t *>(ws + L.tiles);
        const int2 *tmeta = reinterpret_cast<const int2 *>(ws + L.tilemeta);
        // ti < nb: inside the tile lists' storage (read before the count is known, then checked)
        const int ntiles = tiles[0], tile = tiles[1 + ti];
        meta = tmeta[ti];
        if (ti >= ntiles) return;
        e = tile & 1023;
    }

    // an expert's last tile with at most half the tokens takes the half-size body (half the matrix
    // operations and epilogues; same code stream)
    if constexpr (!SELF && MT >= 64) {
        if (meta.y <= MT / 2) {
            pf_work<D, F, P, MT / 2, SELF, Y16>(dm, L, lp, ws, e, meta, s_cnt, sm);
            return;
        }
    }
    pf_work<D, F, P, MT, SELF, Y16>(dm, L, lp, ws, e, meta, s_cnt, sm);
}

// ---- prefill-shaped int8 calls: one workgroup per (expert, up to 192 tokens) ------------------
//
// A work item is one of k_group's tiles with tiles of kExMaxTok tokens: with many tokens per expert
// usually one item per expert, so the 256 items of a 256-expert layer run as one round on 256
// compute units.  The item's workgroup streams its expert's codes once and decodes every code word
// once for half of its tokens (up to 6 row sub-tiles of 16 per decoded operand; the 64-token tiles
// decode each expert in every tile):
//   gate/up: four passes of 128 h rows; the item's activation rows stream through LDS in slices of
//     256 inputs (loaded straight from memory into LDS, three buffers); h (fp32) goes to the
//     workspace and max |h| per token is folded into LDS;
//   h: re-read per (token, 16-row group) and re-quantised (int8 absmax over all F rows) into an int8
//     tile in LDS, in the digit-plane byte order;
//   down: the 16-bit sums of pf_work, two output blocks per step.
// Per value the operations and their order are pf_work's (int8 activations), so the results are
// the same bits.
constexpr int kExW = 8, kExT = 64 * kExW;   // waves, threads
constexpr int kExKS = 256;                  // inputs per activation slice
constexpr int kExPD = 3;                    // LDS operand reads in flight ahead of the products
constexpr int kExMaxRS = 12;
constexpr int kExMaxTok = 16 * kExMaxRS;    // 192 tokens per work item

template <int D, int F, int RS>
constexpr size_t ex_lds()
{
    constexpr size_t slices = 3 * size_t(RS) * 16 * kExKS + 1024,
                     htile = (size_t(RS) * 16 * (F + 16) + 1023) / 1024 * 1024 + 2 * 4 * 2 * (F / 256) * 1024 +
                             kExW * 16 * 80;
    return slices > htile ? slices : htile;
}

// One 16-byte load per lane from global memory straight into LDS: the wave's 64 lanes fill the 1024
// bytes at lds (lane l at byte 16 l); lds is wave-uniform.
__device__ __forceinline__ void load_lds16(const void *g, void *lds)
{
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)g,
                                     (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left alone)
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier for LDS hand-offs whose global-to-LDS loads the caller has already waited for
// (wait_vm): this wave's LDS operations are complete, then s_barrier.  __syncthreads() would also
// wait for every load still in flight (the loads straight into LDS make its fence wait for all
// vector memory operations), including the ones requested ahead on purpose.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int D, int F, int RS>
__device__ __forceinline__ void ex_work(const Dims &dm, const BatchedWs &L, const LayerPtrs &lp, uint8_t *ws,
                                        int e, int2 meta, int8_t *sm, int32_t *s_pair, float *s_sx,
                                        uint32_t *s_amax, const float *s_gs, const float *s_us)
{
    // Waves: row group rg = wave % 4 (two blocks of 16 h rows per pass and per down step), token
    // half th = wave / 4 (row sub-tiles th, th + 2, ...).  Every activation operand read from LDS
    // feeds four matrix products (two blocks, gate and up), every h operand two.
    constexpr int HP = 16 * kExW;               // h rows per pass
    constexpr int NPASS = F / HP;
    constexpr int NSL = D / kExKS;              // activation slices per pass
    constexpr int NG = NPASS * NSL;             // slice steps
    constexpr int HS = RS / 2;                  // row sub-tiles per wave
    constexpr int NTK = RS * 16;                // token rows, padded
    constexpr int SLICE = NTK * kExKS;          // one slice buffer: unpadded rows of 256 bytes
    constexpr int NJ = NTK / 4;                 // 1024-byte groups (4 rows) per slice
    constexpr int JPW = (NJ + kExW - 1) / kExW; // groups per wave (at most)
    constexpr int DB = D / 16 / 4;              // output row blocks per row group
    constexpr int NDS = DB / 2;                 // down steps (two blocks each)
    constexpr int SD = F / 256;
    static_assert(RS % 2 == 0 && F % HP == 0 && D % kExKS == 0 && NSL % 2 == 0 && NG >= 2, "shape");
    static_assert(DB % 2 == 0 && NDS % 2 == 0 && SD >= 1 && SD <= 2, "shape");

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, l16 = lane & 15, g4 = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int rg = wv & 3, th = wv >> 2;
    const int k = dm.k, nv = meta.y, rsv = (nv + 15) / 16;
    const int32_t *pairs = reinterpret_cast<const int32_t *>(ws + L.pairs);
    const float *tinfo = reinterpret_cast<const float *>(ws + L.tinfo);
    const int8_t *xdig = reinterpret_cast<const int8_t *>(ws + L.xdig);
    float *hbuf = reinterpret_cast<float *>(ws + L.h);
    int16_t *y16 = reinterpret_cast<int16_t *>(ws + L.y16);
    int32_t *ywide = reinterpret_cast<int32_t *>(ws + L.y);
    float *shp = reinterpret_cast<float *>(ws + L.shp);
    if (t < NTK) {
        const int pr = t < nv ? pairs[meta.x + t] : -1;
        s_pair[t] = pr;
        s_sx[t] = pr >= 0 ? tinfo[2 * (pr / k)] : 0.0f;
        s_amax[t] = 0u;
    }

    // gate/up code units: unit g = pass * NSL + slice holds, for both of the wave's row blocks, the
    // 16 rows of gate and of up over the slice's 256 inputs (one 16-byte chunk per lane each).  Unit
    // g sits in ring slot g % 2; once step g has decoded the slot's last words it requests unit g + 2
    // into the same registers.
    int4 ring[2][4];
    const uint32_t gofs = uint32_t(l16 * (D / 4) + 16 * g4);
    const uint8_t *gbase = lp.w_gate + (int64_t(e) * F + rg * 32) * (D / 4);
    const uint8_t *ubase = lp.w_up + (int64_t(e) * F + rg * 32) * (D / 4);
    auto issue_gu = [&](int u, auto slot_c) __attribute__((always_inline)) {
        constexpr int SLOT = decltype(slot_c)::value;
        u = min(u, NG - 1);   // past the last unit: a harmless re-read (the slot is always refilled)
        const int ps = u / NSL, sl = u % NSL;
        const int64_t o = int64_t(ps) * HP * (D / 4) + 64 * sl + gofs;
#pragma unroll
        for (int bb = 0; bb < 2; bb++) {
            ring[SLOT][2 * bb] = *reinterpret_cast<const int4 *>(gbase + o + bb * 16 * (D / 4));
            ring[SLOT][2 * bb + 1] = *reinterpret_cast<const int4 *>(ubase + o + bb * 16 * (D / 4));
        }
    };
    // activation slices, from memory straight into LDS (three buffers: step g computes slice g from
    // buffer g % 3 while slices g + 1 and g + 2 arrive): chunk q (16 bytes) of row m sits at position
    // q ^ (m % 16) of the row, so that the 16 rows an operand read takes hit 16 different bank
    // groups.  Group j (rows 4 j .. 4 j + 3) is one wave-wide load: lane l fills row 4 j + l / 16,
    // position l % 16.  A padding row holds the item's first token (its results are never stored).
    // Every wave issues JPW loads per slice (a wave with fewer groups re-reads its first group into
    // a spare kilobyte behind the buffers), so that each step has a fixed number of loads in flight.
    uint32_t xoff[JPW];
    auto load_slice = [&](int sl, int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < JPW; i++) {
            const int j = wv + kExW * i;
            const bool real = j < NJ;
            load_lds16(xdig + (real ? xoff[i] : xoff[0]) + kExKS * sl,
                       sm + (real ? buf * SLICE + 1024 * j : 3 * SLICE));
        }
    };
    issue_gu(0, std::integral_constant<int, 0>{});
    issue_gu(1, std::integral_constant<int, 1>{});
    __syncthreads();   // s_pair, s_sx, s_amax and the expert's scales
    {
        const int pr0 = s_pair[0];
#pragma unroll
        for (int i = 0; i < JPW; i++) {
            const int m = min(4 * (wv + kExW * i) + (lane >> 4), NTK - 1), q = (lane & 15) ^ (m & 15);
            const int pr = s_pair[m] >= 0 ? s_pair[m] : pr0;
            xoff[i] = uint32_t(pr / k) * uint32_t(D) + uint32_t(16 * q);
        }
    }
    // the lane's operand reads: chunk 4 g4 + s of rows (2 i + th) * 16 + l16 (row % 16 = l16)
    uint32_t aoff[4];
#pragma unroll
    for (int s = 0; s < 4; s++) aoff[s] = uint32_t((th * 16 + l16) * kExKS + 16 * ((4 * g4 + s) ^ l16));
    load_slice(0, 0);
    load_slice(1 % NSL, 1);
    wait_vm<JPW>();   // slice 0 and the first two code units are in
    lds_barrier();

    int gb = 0;   // buffer of the current step
    v4i wd[2][4];   // decoded weights (gate and up of both blocks) of two input steps
#pragma unroll
    for (int c = 0; c < 4; c++) wd[0][c] = decode16(word_of(ring[0][c], 0));
    for (int ps = 0; ps < NPASS; ps++) {
        v4i accg[2][HS], accu[2][HS];
#pragma unroll
        for (int i = 0; i < HS; i++)
#pragma unroll
            for (int bb = 0; bb < 2; bb++) accg[bb][i] = accu[bb][i] = v4i{0, 0, 0, 0};
        auto slice_step = [&](int sl, auto slot_c) __attribute__((always_inline)) {
            constexpr int SLOT = decltype(slot_c)::value;
            const int g = ps * NSL + sl;
            const int4 (&cq)[4] = ring[SLOT];
            // slice g + 2 into buffer (g + 2) % 3 (past the last step: a harmless re-read into a
            // buffer no step reads again), so that every step issues the same loads
            load_slice((sl + 2) % NSL, gb == 0 ? 2 : gb - 1);
            // fragments n = s * HS + i (input step s, sub-tile 2 i + th), read kExPD ahead of their
            // products.  The weights of input step s + 1 are decoded while the products
            // of step s run (those of step 0 at the end of the previous slice step); once the last
            // words are decoded, unit g + 2 is requested into the same registers.
            const int8_t *abase = sm + gb * SLICE;
            v4i a[kExPD + 1];
            auto aread = [&](int n) __attribute__((always_inline)) {
                return *reinterpret_cast<const v4i *>(abase + (n % HS) * 32 * kExKS + aoff[n / HS]);
            };
#pragma unroll
            for (int n = 0; n < kExPD; n++) a[n] = aread(n);
#pragma unroll
            for (int n = 0; n < 4 * HS; n++) {
                const int s = n / HS, i = n % HS;
                if (n + kExPD < 4 * HS) a[(n + kExPD) % (kExPD + 1)] = aread(n + kExPD);
                __builtin_amdgcn_sched_barrier(0);   // the read stays ahead of this fragment's products
                const v4i(&w)[4] = wd[s & 1];
                const v4i &af = a[n % (kExPD + 1)];
                accg[0][i] = mfma8(w[0], af, accg[0][i]);
                accu[0][i] = mfma8(w[1], af, accu[0][i]);
                accg[1][i] = mfma8(w[2], af, accg[1][i]);
                accu[1][i] = mfma8(w[3], af, accu[1][i]);
                if (i == 0 && s < 3) {
#pragma unroll
                    for (int c = 0; c < 4; c++) wd[(s + 1) & 1][c] = decode16(word_of(cq[c], s + 1));
                    if (s == 2) {
                        __builtin_amdgcn_sched_barrier(0);   // the unit's registers are free again
                        issue_gu(g + 2, slot_c);
                    }
                }
            }
            // input step 0 of the next unit (past the last one: a harmless decode of the re-read)
#pragma unroll
            for (int c = 0; c < 4; c++) wd[0][c] = decode16(word_of(ring[1 - SLOT][c], 0));
            // slice g + 1 is in LDS: everything but this step's requests has arrived
            wait_vm<JPW + 4>();
            lds_barrier();
            gb = gb == 2 ? 0 : gb + 1;
        };
        for (int sl = 0; sl < NSL; sl += 2) {
            slice_step(sl, std::integral_constant<int, 0>{});
            slice_step(sl + 1, std::integral_constant<int, 1>{});
        }
        // epilogue of the pass: h = SiLU(gate) * up (pf_work's operations), stored in fp32; max |h|
        // per token folded into LDS.  Sub-tiles past the item's tokens are skipped.
        const int row0 = ps * HP + rg * 32 + 4 * g4;
        f4 gsc[2], usc[2];
#pragma unroll
        for (int bb = 0; bb < 2; bb++) {
            gsc[bb] = *reinterpret_cast<const f4 *>(s_gs + row0 + 16 * bb);
            usc[bb] = *reinterpret_cast<const f4 *>(s_us + row0 + 16 * bb);
        }
        float mxs[HS];
#pragma unroll
        for (int i = 0; i < HS; i++) mxs[i] = 0.0f;
#pragma unroll
        for (int i = 0; i < HS; i++) {
            if (2 * i + th >= rsv && i > 0) break;
            const int m = (2 * i + th) * 16 + l16;
            const float sx = s_sx[m];
            const int pr = s_pair[m];
            float &mx = mxs[i];
#pragma unroll
            for (int bb = 0; bb < 2; bb++) {
                float hv[4];
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const float gate = (float(accg[bb][i][r]) * sx) * gsc[bb][r];
                    const float up = (float(accu[bb][i][r]) * sx) * usc[bb][r];
                    hv[r] = tw_silu(gate) * up;
                    mx = fmaxf(mx, fabsf(hv[r]));
                }
                if (pr >= 0)
                    *reinterpret_cast<f4 *>(hbuf + int64_t(pr) * F + row0 + 16 * bb) = f4{hv[0], hv[1], hv[2], hv[3]};
                __builtin_amdgcn_sched_barrier(0);   // four SiLUs at a time: bounded temporaries
            }
        }
        // the per-token maxima after all SiLUs (an LDS atomic waits for the loads still in flight)
#pragma unroll
        for (int i = 0; i < HS; i++) {
            const int m = (2 * i + th) * 16 + l16;
            float mx = fmaxf(mxs[i], __shfl_xor(mxs[i], 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            if (g4 == 0 && s_pair[m] >= 0) atomicMax(&s_amax[m], __float_as_uint(mx));
        }
    }

    // down code units: unit j (step j) holds the two 16-row output blocks 2 j, 2 j + 1 of the row
    // group (rows rg * D / 4 + 32 j ..), SD 16-byte chunks per lane and block; unit j sits in slot
    // j % 2, and step j requests unit j + 1 as it starts.  The first is requested before the
    // re-quantisation.
    const uint32_t dofs = uint32_t(l16 * (F / 4) + 16 * g4);
    const uint8_t *dbase = lp.w_down + (int64_t(e) * D + rg * (D / 4)) * (F / 4);
    int4 dring[2][2][SD];
    auto issue_d = [&](int j, auto slot_c) __attribute__((always_inline)) {
        constexpr int SLOT = decltype(slot_c)::value;
        if (j >= NDS) return;
#pragma unroll
        for (int bb = 0; bb < 2; bb++)
#pragma unroll
            for (int S = 0; S < SD; S++)
                dring[SLOT][bb][S] = *reinterpret_cast<const int4 *>(dbase + (2 * j + bb) * 16 * (F / 4) + 64 * S + dofs);
    };
    // the two token halves of a row group use the same down codes: the th = 0 wave loads them and
    // passes them on through LDS (two buffers behind the h tile, lane-linear 16-byte chunks)
    constexpr int CBUF = 4 * 2 * SD * 1024;
    int8_t *const cbase = sm + ((NTK * (F + 16) + 1023) / 1024) * 1024 + (rg * 2 * SD) * 1024 + 16 * lane;
    auto put_d = [&](int j, auto slot_c) __attribute__((always_inline)) {
        constexpr int SLOT = decltype(slot_c)::value;
#pragma unroll
        for (int bb = 0; bb < 2; bb++)
#pragma unroll
            for (int S = 0; S < SD; S++)
                *reinterpret_cast<int4 *>(cbase + (j & 1) * CBUF + (bb * SD + S) * 1024) = dring[SLOT][bb][S];
    };
    auto get_d = [&](int j, auto slot_c) __attribute__((always_inline)) {
        constexpr int SLOT = decltype(slot_c)::value;
#pragma unroll
        for (int bb = 0; bb < 2; bb++)
#pragma unroll
            for (int S = 0; S < SD; S++)
                dring[SLOT][bb][S] = *reinterpret_cast<const int4 *>(cbase + (j & 1) * CBUF + (bb * SD + S) * 1024);
    };
    // the last steps' slice loads (re-reads into buffers no step reads again) must land before the
    // h tile reuses those LDS bytes
    wait_vm<0>();
    if (th == 0) issue_d(0, std::integral_constant<int, 0>{});
    __syncthreads();   // every h store and max of this item is done

    // h: per (token, 16-row group) re-quantised against the token's max |h| into the int8 tile (byte
    // j of a group's 16 rows goes to byte 4 (j % 4) + j / 4, the order of the decoded code words);
    // the loads of QB items are in flight together (a padding row reads the item's first token)
    {
        constexpr int NQ = NTK * (F / 16), QPT = (NQ + kExT - 1) / kExT, QB = 4;
        const int pr0 = s_pair[0];
#pragma unroll
        for (int j0 = 0; j0 < QPT; j0 += QB) {
            f4 v[QB][4];
            int mq[QB], gq[QB], pq[QB];
#pragma unroll
            for (int b = 0; b < QB; b++) {
                const int i = t + kExT * (j0 + b);
                mq[b] = min(i / (F / 16), NTK - 1);
                gq[b] = i % (F / 16);
                pq[b] = j0 + b < QPT && i < NQ ? s_pair[mq[b]] : -2;
                const f4 *hp = reinterpret_cast<const f4 *>(hbuf + int64_t(pq[b] >= 0 ? pq[b] : pr0) * F + 16 * gq[b]);
                if (j0 + b < QPT) {
#pragma unroll
                    for (int c = 0; c < 4; c++) v[b][c] = hp[c];
                }
            }
#pragma unroll
            for (int b = 0; b < QB; b++) {
                if (j0 + b >= QPT || pq[b] == -2) continue;
                int4 packed = make_int4(0, 0, 0, 0);
                if (pq[b] >= 0) {
                    const float am = __uint_as_float(s_amax[mq[b]]);
                    int8_t q[16];
#pragma unroll
                    for (int c = 0; c < 4; c++)
#pragma unroll
                        for (int j = 0; j < 4; j++)
                            q[4 * c + j] = am > 0.0f ? int8_quant(v[b][c][j], 127.0f / am) : int8_t(0);
                    uint32_t d[4];
#pragma unroll
                    for (int dd = 0; dd < 4; dd++)
                        d[dd] = uint32_t(uint8_t(q[dd])) | (uint32_t(uint8_t(q[dd + 4])) << 8) |
                                (uint32_t(uint8_t(q[dd + 8])) << 16) | (uint32_t(uint8_t(q[dd + 12])) << 24);
                    packed = make_int4(int32_t(d[0]), int32_t(d[1]), int32_t(d[2]), int32_t(d[3]));
                }
                *reinterpret_cast<int4 *>(sm + mq[b] * (F + 16) + 16 * gq[b]) = packed;
            }
        }
    }
    if (t < NTK && s_pair[t] >= 0) {
        const float am = __uint_as_float(s_amax[t]);
        shp[s_pair[t]] = am > 0.0f ? am / 127.0f : 0.0f;   // the combine forms y from it
    }
    if (th == 0) put_d(0, std::integral_constant<int, 0>{});
    __syncthreads();
    if (th != 0) get_d(0, std::integral_constant<int, 0>{});

    // down, two 16-row blocks per step (pf_work's sums and 16-bit stores); sub-tiles past the item's
    // tokens store into spare rows
    uint32_t yoff[HS];
#pragma unroll
    for (int i = 0; i < HS; i++) {
        const int pr = s_pair[(2 * i + th) * 16 + l16];
        const int64_t row = pr >= 0 ? int64_t(pr) : L.spare_row + (blockIdx.x % kSpareRows);
        yoff[i] = uint32_t(row) * uint32_t(2 * D) + uint32_t(2 * (rg * (D / 4) + 4 * g4));
    }
    const int8_t *hbase = sm + tofs(th * 16 + l16, 4 * g4, F);
    // 16-bit sums of both blocks of sub-tile 2 i + th of down step j (a sum outside [-32767, 32767]
    // is stored as the marker -32768, and the lane's four sums go to the 32-bit rows as well);
    // padding tokens of a sub-tile that holds real ones write spare rows.  The lane's 8-byte pieces
    // of the two blocks pass through this wave's LDS area (token rows of 80 bytes) so that each lane
    // stores 16 contiguous bytes: rows 8 g4 .. 8 g4 + 7 of the step's 32 (half the store requests).
    int8_t *const wst = sm + ((NTK * (F + 16) + 1023) / 1024) * 1024 + 2 * (4 * 2 * SD * 1024) + wv * (16 * 80);
    auto emit = [&](const v4i &a0, const v4i &a1, int i, int j) __attribute__((always_inline)) {
        if (i > 0 && 2 * i + th >= rsv) return;   // a sub-tile of padding rows only: nothing to keep
#pragma unroll
        for (int bb = 0; bb < 2; bb++) {
            const v4i &v4 = bb == 0 ? a0 : a1;
            int32_t cl[4];
            bool wide = false;
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int32_t v = v4[r];
                cl[r] = min(max(v, -32768), 32768);
                wide = wide || uint32_t(v + 32767) > 65534u;
            }
            *reinterpret_cast<uint2 *>(wst + l16 * 80 + 32 * bb + 8 * g4) =
                make_uint2((uint32_t(cl[0]) & 0xffffu) | (uint32_t(cl[1]) << 16),
                           (uint32_t(cl[2]) & 0xffffu) | (uint32_t(cl[3]) << 16));
            // the same element in the 32-bit rows sits at twice the byte offset
            if (wide)
                *reinterpret_cast<int4 *>(reinterpret_cast<uint8_t *>(ywide) + (2u * yoff[i] + uint32_t(128 * j + 64 * bb))) =
                    make_int4(v4[0], v4[1], v4[2], v4[3]);   // 2 yoff < 2^32: the rows end below 4 GiB
        }
        // this wave's own LDS writes, read back in order: rows 8 g4 .. of token l16
        const uint4 q16 = *reinterpret_cast<const uint4 *>(wst + l16 * 80 + 16 * g4);
        *reinterpret_cast<uint4 *>(reinterpret_cast<uint8_t *>(y16) + (yoff[i] - 8 * g4) + 64 * j + 16 * g4) = q16;
    };
    // step j sums into acc[j % 2]; the sums of step j - 1 are stored piece by piece while the
    // products of step j run (one sub-tile's two blocks after every 4 SD fragments)
    v4i acc[2][2][HS];
    auto down_step = [&](int j, auto slot_c) __attribute__((always_inline)) {
        constexpr int SLOT = decltype(slot_c)::value;
        if (th == 0) issue_d(j + 1, std::integral_constant<int, 1 - SLOT>{});
        const int4 (&cq)[2][SD] = dring[SLOT];
        v4i (&ac)[2][HS] = acc[SLOT];
        const v4i (&ap)[2][HS] = acc[1 - SLOT];
        // fragments n = c * HS + i (h chunk 16 (c / 4) + 4 g4 + c % 4, sub-tile 2 i + th), read
        // kExPD ahead of their products; the two blocks' words of step c are decoded as it starts
        v4i w[2], hv[kExPD + 1];
        auto hread = [&](int n) __attribute__((always_inline)) {
            const int c = n / HS, i = n % HS;
            return *reinterpret_cast<const v4i *>(hbase + i * 32 * (F + 16) + 256 * (c >> 2) + 16 * (c & 3));
        };
#pragma unroll
        for (int n = 0; n < kExPD; n++) hv[n] = hread(n);
#pragma unroll
        for (int n = 0; n < 4 * SD * HS; n++) {
            const int c = n / HS, i = n % HS;
            if (i == 0) {
#pragma unroll
                for (int bb = 0; bb < 2; bb++) w[bb] = decode16(word_of(cq[bb][c >> 2], c & 3));
            }
            if (n + kExPD < 4 * SD * HS) hv[(n + kExPD) % (kExPD + 1)] = hread(n + kExPD);
            __builtin_amdgcn_sched_barrier(0);   // the read stays ahead of this fragment's products
#pragma unroll
            for (int bb = 0; bb < 2; bb++)   // the first product of a sum starts from zero
                ac[bb][i] = mfma8(w[bb], hv[n % (kExPD + 1)], c == 0 ? v4i{0, 0, 0, 0} : ac[bb][i]);
            if (j > 0 && n % (4 * SD) == 4 * SD - 1) {
                const int pi = n / (4 * SD);   // 0 .. HS - 1
                emit(ap[0][pi], ap[1][pi], pi, j - 1);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (j + 1 < NDS) {
            if (th == 0) put_d(j + 1, std::integral_constant<int, 1 - SLOT>{});
            lds_barrier();   // the next step's codes are in LDS
            if (th != 0) get_d(j + 1, std::integral_constant<int, 1 - SLOT>{});
        }
    };
    for (int j = 0; j < NDS; j += 2) {
        down_step(j, std::integral_constant<int, 0>{});
        down_step(j + 1, std::integral_constant<int, 1>{});
    }
    // the last step's sums (NDS is even: they are in acc[1])
#pragma unroll
    for (int i = 0; i < HS; i++) emit(acc[1][0][i], acc[1][1][i], i, NDS - 1);
}

template <int D, int F>
__global__ __launch_bounds__(kExT) void k_pf_expert(Dims dm, BatchedWs L, LayerPtrs lp, uint8_t *ws)
{
    extern __shared__ __attribute__((aligned(16))) int8_t sm[];
    __shared__ int32_t s_pair[kExMaxTok];
    __shared__ float s_sx[kExMaxTok];
    __shared__ uint32_t s_amax[kExMaxTok];
    __shared__ __attribute__((aligned(16))) float s_gs[F];
    __shared__ __attribute__((aligned(16))) float s_us[F];
    const int b = blockIdx.x, t = threadIdx.x;
    const int32_t *tiles = reinterpret_cast<const int32_t *>(ws + L.tiles);
    const int2 *tmeta = reinterpret_cast<const int2 *>(ws + L.tilemeta);
    const int ntiles = tiles[0];
    if (b >= ntiles) return;
    const int e = tiles[1 + b] & 1023;
    const int2 meta = tmeta[b];
    for (int i = t; i < F; i += kExT) {
        s_gs[i] = lp.s_gate[int64_t(e) * F + i];
        s_us[i] = lp.s_up[int64_t(e) * F + i];
    }
    const int rsv = (meta.y + 15) / 16;
    if (rsv <= 4)
        ex_work<D, F, 4>(dm, L, lp, ws, e, meta, sm, s_pair, s_sx, s_amax, s_gs, s_us);
    else if (rsv <= 8)
        ex_work<D, F, 8>(dm, L, lp, ws, e, meta, sm, s_pair, s_sx, s_amax, s_gs, s_us);
    else if (rsv <= 10)
        ex_work<D, F, 10>(dm, L, lp, ws, e, meta, sm, s_pair, s_sx, s_amax, s_gs, s_us);
    else
        ex_work<D, F, 12>(dm, L, lp, ws, e, meta, sm, s_pair, s_sx, s_amax, s_gs, s_us);
}

template <int D, int F>
int ex_run(const Dims &dm, const LayerPtrs &lp, int64_t T, const BatchedWs &L, uint8_t *ws, void *stream)
{
    constexpr size_t lds = ex_lds<D, F, kExMaxRS>();
    static std::atomic<int> attr_set{0};
    if (!attr_set.load(std::memory_order_relaxed)) {
        if (hipFuncSetAttribute(reinterpret_cast<const void *>(k_pf_expert<D, F>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)) != hipSuccess)
            return int(hipErrorInvalidValue);
        attr_set.store(1, std::memory_order_relaxed);
    }
    const int nb = int(max_tiles(dm, T, kExMaxTok));
    k_pf_expert<D, F><<<nb, kExT, lds, static_cast<hipStream_t>(stream)>>>(dm, L, lp, ws);
    return int(hipGetLastError());
}

// One workgroup per tile slot; sel_ids != nullptr: the workgroups build the tile list themselves
// (needs T k and E <= the workgroup size), else they read k_group's.
template <int D, int F, int P, int MT, bool SELF>
int pf_run(const Dims &dm, const LayerPtrs &lp, int64_t T, const BatchedWs &L, uint8_t *ws,
           const int32_t *sel_ids, void *stream)
{
    constexpr size_t lds = size_t(MT) * P * ((D > F ? D : F) + 16);
    static std::atomic<int> attr_set{0};
    if (!attr_set.load(std::memory_order_relaxed)) {
        if (hipFuncSetAttribute(reinterpret_cast<const void *>(k_pf_ffn<D, F, P, MT, SELF>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)) != hipSuccess)
            return int(hipErrorInvalidValue);
        attr_set.store(1, std::memory_order_relaxed);
    }
    const int64_t npairs = T * dm.k;
    if (SELF && (npairs > PfShape<MT, P>::T || dm.E > PfShape<MT, P>::T)) return -1;
    const int nb = int((max_tiles(dm, T, MT) + 15) / 16 * 16);
    k_pf_ffn<D, F, P, MT, SELF><<<nb, PfShape<MT, P>::T, lds, static_cast<hipStream_t>(stream)>>>(
        dm, L, lp, ws, nb, sel_ids, int(npairs));
    return int(hipGetLastError());
}

template <int D, int F>
int pf_dispatch(const Dims &dm, const LayerPtrs &lp, int64_t T, int planes, int tile,
                const BatchedWs &L, uint8_t *ws, const int32_t *sel_ids, void *stream)
{
    if (planes == 1) {
        if (tile == kExMaxTok) return ex_run<D, F>(dm, lp, T, L, ws, stream);
        if (tile == 64) return pf_run<D, F, 1, 64, false>(dm, lp, T, L, ws, nullptr, stream);
        if (sel_ids) return pf_run<D, F, 1, 16, true>(dm, lp, T, L, ws, sel_ids, stream);
        return pf_run<D, F, 1, 16, false>(dm, lp, T, L, ws, nullptr, stream);
    }
    if (tile == 32) return pf_run<D, F, 2, 32, false>(dm, lp, T, L, ws, nullptr, stream);
    if (sel_ids) return pf_run<D, F, 2, 8, true>(dm, lp, T, L, ws, sel_ids, stream);
    return pf_run<D, F, 2, 8, false>(dm, lp, T, L, ws, nullptr, stream);
}

}  // namespace

bool grouped_mfma_serves(const Dims &dm, int64_t T, int planes, int *tile)
{
    const bool shape = (dm.d == 2048 && dm.F == 512) || (dm.d == 1024 && dm.F == 256);
    if (!shape || dm.E > 1024 || planes < 1 || planes > 2) return false;
    // tiles of 64 activation rows when there are at least 32 of them per expert on average (int8:
    // 64 tokens, two planes: 32 tokens), else of 16 rows (16 or 8 tokens)
    const bool big = T * dm.k * planes >= int64_t(32) * dm.E;
    *tile = planes == 1 ? (big ? 64 : 16) : (big ? 32 : 8);
    // int8 activations with at least 96 tokens per expert on average: one work item per expert
    if (planes == 1 && T * dm.k >= int64_t(96) * dm.E) *tile = kExMaxTok;
    return true;
}

bool grouped_mfma_self(const Dims &dm, int64_t T, int tile)
{
    // small tiles (16 activation rows: one 1024-thread workgroup per expert), at most one id per
    // thread
    return (tile == 16 || tile == 8) && T * dm.k <= 1024;
}

int launch_grouped_mfma(const Dims &dm, const LayerPtrs &layer, int64_t T, int planes, int tile,
                        const BatchedWs &L, uint8_t *ws, const int32_t *sel_ids, void *stream)
{
    if (dm.d == 2048 && dm.F == 512)
        return pf_dispatch<2048, 512>(dm, layer, T, planes, tile, L, ws, sel_ids, stream);
    if (dm.d == 1024 && dm.F == 256)
        return pf_dispatch<1024, 256>(dm, layer, T, planes, tile, L, ws, sel_ids, stream);
    return -1;
}

}  // namespace tw
