// tw_prefill.hip -- grouped MFMA path of the batched FFN (gfx950): every call whose shape it is
// instantiated for, from a few tokens per expert (batched decode) to many (prefill-shaped).
//
// The ternary products are int8 contractions and run on the matrix cores:
// v_mfma_i32_16x16x64_i8 multiplies a 16x64 int8 tile of activations by a 64x16 int8 tile of
// weights into exact 16x16 int32 sums.  Activations enter as P int8 planes (P = 1: int8 absmax
// mode; P = 2, 3: the float digit planes of tw_device.h), each contracted on its own, so every
// result is bit-identical to the per-pair v_dot4 path and to the batch-1 decode.
//
// One workgroup (512 threads, 8 waves) takes one (expert e, tile of MT tokens) work item:
//   1. the tile's MT x P planes of activation digits (d bytes each, 4x4-transposed inside groups
//      of 16 as in tw_device.h) are copied into LDS, rows padded by 16 bytes so that the 16 rows
//      read by one MFMA operand fetch spread over the banks;
//   2. gate/up: wave w owns h rows [F/8 w, F/8 (w+1)) in groups of 16; for each group it loads the
//      16 gate and 16 up code rows (each lane: one row, 16 bytes per 256 inputs), decodes 16 codes
//      into the 16 int8 weights of its MFMA B operand with four v_perm_b32 (no LDS round trip), and
//      runs MT/16 token sub-tiles x P planes x (gate, up) MFMAs per 64 inputs; the epilogue forms
//      gate, up and h = SiLU(gate) * up in fp32 in the order of the specification, in registers;
//   3. per token: max |h| over all F rows (registers, DPP inside 16-lane rows, LDS over waves), h
//      re-quantised (int8 absmax) or split into digit planes (float) into LDS;
//   4. down: wave w owns d/8 output rows; same MFMA scheme with the down codes; y in fp32, stored
//      per (token, slot) pair for the ordered combine.
// K order: lane group g of an MFMA at step (S, s) covers inputs 256 S + 64 g + 16 s .. +16 -- a
// permutation of the inputs shared by both operands, so every int32 sum is the exact dot product.
// Work items are mapped to workgroups so that pairs of consecutive tiles (usually one expert) run on
// the same XCD at about the same time (workgroups b and b + 8 share an XCD): the second tile's code
// bytes then come from that XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "tw_device.h"
#include "tw_internal.h"

namespace tw {
namespace {

typedef int32_t v4i __attribute__((ext_vector_type(4)));

// Waves per workgroup: 8 for 64-token tiles; 16 for 16-token tiles (at <= 128 VGPRs, four waves
// per SIMD hide each other's code-row loads).
template <int MT>
struct PfShape {
    static constexpr int W = MT <= 16 ? 16 : 8;
    static constexpr int T = 64 * W;
};

// The 16 int8 weights of one 32-bit code word, in the transposed order of the activation digits.
__device__ __forceinline__ v4i decode16(uint32_t w)
{
    v4i r;
    r.x = lut4(w & kCodeMask);
    r.y = lut4((w >> 2) & kCodeMask);
    r.z = lut4((w >> 4) & kCodeMask);
    r.w = lut4((w >> 6) & kCodeMask);
    return r;
}

__device__ __forceinline__ uint32_t word_of(const int4 &v, int s)
{
    return uint32_t(s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w);
}

// Row maximum over the 16 lanes of each DPP row (every lane of the row receives it).
__device__ __forceinline__ float row16_max(float v)
{
    v = fmaxf(v, dpp_f<kDppXor1>(v));
    v = fmaxf(v, dpp_f<kDppXor2>(v));
    v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_f<kDppMirror>(v));
    return v;
}

// Address of 16-byte chunk c of row r in a tile of rows of `rowb` bytes, each padded by 16 bytes.
__device__ __forceinline__ int tofs(int r, int c, int rowb) { return r * (rowb + 16) + 16 * c; }

__device__ __forceinline__ v4i mfma8(const v4i &a, const v4i &b, const v4i &c)
{
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

template <int D, int F, int P, int MT>
__global__ __launch_bounds__(PfShape<MT>::T) void k_pf_ffn(Dims dm, BatchedWs L, LayerPtrs lp, uint8_t *ws, int nb)
{
    constexpr int kPfW = PfShape<MT>::W, kPfT = PfShape<MT>::T;
    static_assert(D % 256 == 0 && F % 256 == 0 && F % (16 * kPfW) == 0 && D % (16 * kPfW) == 0, "shape");
    static_assert(MT % 16 == 0 && MT <= kPfT, "tile");
    constexpr bool INT8 = P == 1;
    constexpr int MS = MT / 16;           // token sub-tiles
    constexpr int GPW = F / 16 / kPfW;    // h-row groups of 16 per wave
    constexpr int NSD = D / 16 / kPfW;    // down sub-tiles of 16 rows per wave
    constexpr int SG = D / 256, SD = F / 256;
    extern __shared__ __attribute__((aligned(16))) int8_t sm[];   // [MT][P] rows of D, later of F
    __shared__ int32_t s_pair[MT];
    __shared__ float s_tk[MT][2];         // per token: s_x (int8) or digit shift bits; 1/rms
    __shared__ float s_hk[MT];            // per token: s_h (int8) or digit shift bits of h
    __shared__ float s_amx[MT];
    __shared__ float s_pam[kPfW][MT];

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, l16 = lane & 15, g4 = lane >> 4;
    const int32_t *tiles = reinterpret_cast<const int32_t *>(ws + L.tiles);
    // workgroups b and b + 8 run on the same XCD: they take consecutive tiles (usually one expert),
    // and every 16 workgroups cover 16 consecutive tiles, so work spreads evenly over the XCDs
    const int b = blockIdx.x;
    const int ti = (b / 16) * 16 + (b % 8) * 2 + ((b / 8) & 1);
    if (ti >= tiles[0]) return;
    const int tile = tiles[1 + ti], e = tile & 1023, mt = tile >> 10;
    const int32_t *counts = reinterpret_cast<const int32_t *>(ws + L.counts);
    const int32_t *offsets = reinterpret_cast<const int32_t *>(ws + L.offsets);
    const int32_t *pairs = reinterpret_cast<const int32_t *>(ws + L.pairs);
    const float *tinfo = reinterpret_cast<const float *>(ws + L.tinfo);
    const int8_t *xdig = reinterpret_cast<const int8_t *>(ws + L.xdig);
    float *ybuf = reinterpret_cast<float *>(ws + L.y);
    const int nv = min(MT, counts[e] - mt * MT);
    const int p0 = offsets[e] + mt * MT;
    const int k = dm.k;

    if (t < MT) {
        const int pr = t < nv ? pairs[p0 + t] : -1;
        s_pair[t] = pr;
        s_tk[t][0] = pr >= 0 ? tinfo[2 * (pr / k)] : 0.0f;
        s_tk[t][1] = pr >= 0 ? tinfo[2 * (pr / k) + 1] : 0.0f;
    }
    __syncthreads();
    // 1. activation tile: row (m, plane) = plane of token m
    for (int idx = t; idx < MT * P * (D / 16); idx += kPfT) {
        const int r = idx / (D / 16), c = idx % (D / 16), m = r / P, pr = s_pair[m];
        const int4 v = pr >= 0 ? reinterpret_cast<const int4 *>(xdig + (int64_t(pr / k) * P + r % P) * D)[c]
                               : make_int4(0, 0, 0, 0);
        *reinterpret_cast<int4 *>(sm + tofs(r, c, D)) = v;
    }
    __syncthreads();

    // 2. gate/up.  With small tiles (PF) the code rows of group gi+1 are requested before group gi
    //    is computed (two register buffers, fully unrolled so every index is static).
    constexpr bool PF = false;
    float hreg[GPW][MS][4];
    int4 cg[PF ? 2 : 1][SG], cu[PF ? 2 : 1][SG];
    auto load_gu = [&](int gi, int4 (&g)[SG], int4 (&u)[SG]) {
        const int r0 = (wave * GPW + gi) * 16;
        const int4 *grow = reinterpret_cast<const int4 *>(lp.w_gate + (int64_t(e) * F + r0 + l16) * (D / 4));
        const int4 *urow = reinterpret_cast<const int4 *>(lp.w_up + (int64_t(e) * F + r0 + l16) * (D / 4));
#pragma unroll
        for (int S = 0; S < SG; S++) {
            g[S] = grow[4 * S + g4];
            u[S] = urow[4 * S + g4];
        }
    };
    if (PF) load_gu(0, cg[0], cu[0]);
#pragma unroll
    for (int gi = 0; gi < GPW; gi++) {
        const int r0 = (wave * GPW + gi) * 16;
        const int bi = PF ? (gi & 1) : 0;
        if (!PF) load_gu(gi, cg[0], cu[0]);
        if (PF && gi + 1 < GPW) load_gu(gi + 1, cg[bi ^ 1], cu[bi ^ 1]);
        v4i accg[P][MS], accu[P][MS];
#pragma unroll
        for (int pl = 0; pl < P; pl++)
#pragma unroll
            for (int ms = 0; ms < MS; ms++) accg[pl][ms] = accu[pl][ms] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 4 * SG; i++) {
            const int S = i >> 2, s = i & 3;
            const int c = 16 * S + 4 * g4 + s;
            const v4i bg = decode16(word_of(cg[bi][S], s)), bu = decode16(word_of(cu[bi][S], s));
#pragma unroll
            for (int ms = 0; ms < MS; ms++)
#pragma unroll
                for (int pl = 0; pl < P; pl++) {
                    const v4i av = *reinterpret_cast<const v4i *>(sm + tofs((ms * 16 + l16) * P + pl, c, D));
                    accg[pl][ms] = mfma8(av, bg, accg[pl][ms]);
                    accu[pl][ms] = mfma8(av, bu, accu[pl][ms]);
                }
            if (!PF) __builtin_amdgcn_sched_barrier(0);
        }
        const float sgv = lp.s_gate[int64_t(e) * F + r0 + l16], suv = lp.s_up[int64_t(e) * F + r0 + l16];
#pragma unroll
        for (int ms = 0; ms < MS; ms++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int m = ms * 16 + 4 * g4 + r;
                float gate, up;
                if (INT8) {
                    gate = (float(accg[0][ms][r]) * s_tk[m][0]) * sgv;
                    up = (float(accu[0][ms][r]) * s_tk[m][0]) * suv;
                } else {
                    int32_t ag[P], au[P];
#pragma unroll
                    for (int pl = 0; pl < P; pl++) {
                        ag[pl] = accg[pl][ms][r];
                        au[pl] = accu[pl][ms][r];
                    }
                    const int sh = __float_as_int(s_tk[m][0]);
                    gate = float_value<P>(ag, sh) * sgv * s_tk[m][1];
                    up = float_value<P>(au, sh) * suv * s_tk[m][1];
                }
                hreg[gi][ms][r] = tw_silu(gate) * up;
            }
        if (!PF) __builtin_amdgcn_sched_barrier(0);
    }

    // 3. per-token max |h|, then int8 re-quantisation or digit planes of h into LDS
#pragma unroll
    for (int ms = 0; ms < MS; ms++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
            float v = 0.0f;
#pragma unroll
            for (int gi = 0; gi < GPW; gi++) v = fmaxf(v, fabsf(hreg[gi][ms][r]));
            v = row16_max(v);
            if (l16 == 0) s_pam[wave][ms * 16 + 4 * g4 + r] = v;
        }
    __syncthreads();   // every wave is done with the activation tile
    if (t < MT) {
        float am = 0.0f;
#pragma unroll
        for (int w = 0; w < kPfW; w++) am = fmaxf(am, s_pam[w][t]);
        s_amx[t] = am;
        if (INT8)
            s_hk[t] = am > 0.0f ? am / 127.0f : 0.0f;
        else
            s_hk[t] = __int_as_float(float_digit_shift(am, P));
    }
    __syncthreads();
#pragma unroll
    for (int gi = 0; gi < GPW; gi++) {
        const int row = (wave * GPW + gi) * 16 + l16;
        const int pos = perm16(row);
#pragma unroll
        for (int ms = 0; ms < MS; ms++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int m = ms * 16 + 4 * g4 + r;
                if (INT8) {
                    const float am = s_amx[m];
                    const int8_t q = am > 0.0f ? int8_quant(hreg[gi][ms][r], 127.0f / am) : int8_t(0);
                    sm[tofs(m, pos >> 4, F) + (pos & 15)] = q;
                } else {
                    int8_t dg[P];
                    float_digits<P>(hreg[gi][ms][r], __float_as_int(s_hk[m]), dg);
#pragma unroll
                    for (int pl = 0; pl < P; pl++) sm[tofs(m * P + pl, pos >> 4, F) + (pos & 15)] = dg[pl];
                }
            }
    }
    __syncthreads();

    // 4. down (with small tiles, the next sub-tile's code rows are requested before the current
    //    one is computed)
    int4 cdv[PF ? 2 : 1][SD];
    auto load_dn = [&](int nt, int4 (&cd)[SD]) {
        const int R0 = (wave * NSD + nt) * 16;
        const int4 *drow = reinterpret_cast<const int4 *>(lp.w_down + (int64_t(e) * D + R0 + l16) * (F / 4));
#pragma unroll
        for (int S = 0; S < SD; S++) cd[S] = drow[4 * S + g4];
    };
    if (PF) load_dn(0, cdv[0]);
#pragma unroll
    for (int nt = 0; nt < NSD; nt++) {
        const int R0 = (wave * NSD + nt) * 16;
        const int bi = PF ? (nt & 1) : 0;
        if (!PF) load_dn(nt, cdv[0]);
        if (PF && nt + 1 < NSD) load_dn(nt + 1, cdv[bi ^ 1]);
        v4i acc[P][MS];
#pragma unroll
        for (int pl = 0; pl < P; pl++)
#pragma unroll
            for (int ms = 0; ms < MS; ms++) acc[pl][ms] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 4 * SD; i++) {
            const int S = i >> 2, s = i & 3;
            const v4i bd = decode16(word_of(cdv[bi][S], s));
            const int c = 16 * S + 4 * g4 + s;
#pragma unroll
            for (int ms = 0; ms < MS; ms++)
#pragma unroll
                for (int pl = 0; pl < P; pl++) {
                    const v4i av = *reinterpret_cast<const v4i *>(sm + tofs((ms * 16 + l16) * P + pl, c, F));
                    acc[pl][ms] = mfma8(av, bd, acc[pl][ms]);
                }
            if (!PF) __builtin_amdgcn_sched_barrier(0);
        }
        const float sdv = lp.s_down[int64_t(e) * D + R0 + l16];
#pragma unroll
        for (int ms = 0; ms < MS; ms++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int m = ms * 16 + 4 * g4 + r, pr = s_pair[m];
                float y;
                if (INT8) {
                    y = (float(acc[0][ms][r]) * s_hk[m]) * sdv;
                } else {
                    int32_t ad[P];
#pragma unroll
                    for (int pl = 0; pl < P; pl++) ad[pl] = acc[pl][ms][r];
                    y = float_value<P>(ad, __float_as_int(s_hk[m])) * sdv;
                }
                if (pr >= 0) ybuf[int64_t(pr) * D + R0 + l16] = y;
            }
    }
}

template <int D, int F, int P, int MT>
int pf_run(const Dims &dm, const LayerPtrs &lp, int64_t T, const BatchedWs &L, uint8_t *ws,
           void *stream)
{
    constexpr size_t lds = size_t(MT) * P * ((D > F ? D : F) + 16);
    static std::atomic<int> attr_set{0};
    if (!attr_set.load(std::memory_order_relaxed)) {
        if (hipFuncSetAttribute(reinterpret_cast<const void *>(k_pf_ffn<D, F, P, MT>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)) != hipSuccess)
            return int(hipErrorInvalidValue);
        attr_set.store(1, std::memory_order_relaxed);
    }
    const int nb = int((max_tiles(dm, T, MT) + 15) / 16 * 16);
    k_pf_ffn<D, F, P, MT><<<nb, PfShape<MT>::T, lds, static_cast<hipStream_t>(stream)>>>(dm, L, lp, ws, nb);
    return int(hipGetLastError());
}

template <int D, int F>
int pf_dispatch(const Dims &dm, const LayerPtrs &lp, int64_t T, int planes, int tile,
                const BatchedWs &L, uint8_t *ws, void *stream)
{
    if (planes == 1) {
        if (tile == kTileTokens) return pf_run<D, F, 1, kTileTokens>(dm, lp, T, L, ws, stream);
        return pf_run<D, F, 1, kSmallTile>(dm, lp, T, L, ws, stream);
    }
    if (planes == 2) return pf_run<D, F, 2, kSmallTile>(dm, lp, T, L, ws, stream);
    return pf_run<D, F, 3, kSmallTile>(dm, lp, T, L, ws, stream);
}

}  // namespace

bool grouped_mfma_serves(const Dims &dm, int64_t T, int planes, int *tile)
{
    const bool shape = (dm.d == 2048 && dm.F == 512) || (dm.d == 1024 && dm.F == 256);
    if (!shape || dm.E > 1024 || planes < 1 || planes > 3) return false;
    // int8 with at least 32 tokens per expert on average: 64-token tiles; otherwise 16-token tiles
    *tile = (planes == 1 && T * dm.k >= int64_t(32) * dm.E) ? kTileTokens : kSmallTile;
    return true;
}

int launch_grouped_mfma(const Dims &dm, const LayerPtrs &layer, int64_t T, int planes, int tile,
                        const BatchedWs &L, uint8_t *ws, void *stream)
{
    if (dm.d == 2048 && dm.F == 512) return pf_dispatch<2048, 512>(dm, layer, T, planes, tile, L, ws, stream);
    if (dm.d == 1024 && dm.F == 256) return pf_dispatch<1024, 256>(dm, layer, T, planes, tile, L, ws, stream);
    return -1;
}

}  // namespace tw
