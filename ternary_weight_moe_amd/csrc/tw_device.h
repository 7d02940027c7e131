// tw_device.h -- device-side helpers shared by the HIP kernels of libternary_moe.so (gfx950).
//
// Pages cited (titles as printed):
//   [MacMini] "A 20B AI Model Trained in Ternary Just Hit 218 Tokens/Second on a $599 Mac Mini"
//   [Hub]     "iPhone Runs a 20B Model at 120 tok/s"
//
// The ternary dot product.  The pages' kernel masks each 2-bit code and adds, subtracts or skips
// the activation, accumulating in FP32 ([MacMini] "What Ternary Actually Means", "The
// Architecture: Designed for the Hardware").  On gfx950 the cheapest add/subtract/skip is an int8
// dot: one v_perm_b32 turns four 2-bit codes into four int8 weights in {-1,0,+1} (a byte lookup
// with the codes as selectors), and one v_dot4_i32_i8 applies four of them to four int8
// activations with an exact int32 sum.  Activations are therefore split into int8 "digit planes":
//   - int8 activation mode: one plane, q = clamp(rint(v * (127/amax)), +-127), scale amax/127;
//   - float mode: P planes (P = 2 for bf16 I/O, 3 for fp32 I/O) of a fixed-point image
//     X = rint(v * 2^sh) with |X| < 2^(7P), digits of |X| in base 128 carrying the sign of X.
//     The dot is sum_k 128^(P-1-k) acc_k * 2^-sh; its error is the fixed-point rounding of the
//     activations (<= amax * 2^-(7P) per element), far below the bf16 output rounding for P = 2 and
//     of the order of fp32 accumulation error for P = 3.
// Code word layout: a 32-bit word holds weights 0..15 of a 16-weight group (weight i in bits
// 2i..2i+1).  Decoding gives four int8x4 words W_m whose byte b is weight 4b+m; the matching
// activation digits are stored with the same 4x4 transpose inside every group of 16, so that
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tw_internal.h"

namespace tw {
namespace {

constexpr uint32_t kCodeMask = 0x03030303u;
// Byte c of this word is the int8 weight of code c: 00 -> 0, 01 -> +1, 10 -> -1, 11 -> 0.
constexpr uint32_t kCodeLut = 0x00FF0100u;
// The same table for a code left in bits 2-3 of a selector byte (selector 4c): byte permute
// selector 0 picks low byte 0 (0x00), 4 picks high byte 0 (0x01), 8 replicates the sign bit of low
// byte 1 (0xFF), 12 gives 0x00.
constexpr uint32_t kCodeMaskHi = 0x0C0C0C0Cu;
constexpr uint32_t kCodeLutHiLow = 0x00008000u, kCodeLutHiHigh = 0x00000001u;

// ------------------------------------------------------------------------------------------------
// scalar helpers

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;   // NaN
    u += 0x7fffu + ((u >> 16) & 1u);                       // round to nearest, ties to even
    return uint16_t(u >> 16);
}

__device__ __forceinline__ float load_act(const void *p, int64_t i, int bf16)
{
    return bf16 ? bf16_to_f32(static_cast<const uint16_t *>(p)[i]) : static_cast<const float *>(p)[i];
}

__device__ __forceinline__ void store_act(void *p, int64_t i, float v, int bf16)
{
    if (bf16)
        static_cast<uint16_t *>(p)[i] = f32_to_bf16(v);
    else
        static_cast<float *>(p)[i] = v;
}

// ---- cross-lane reductions (DPP inside 16-lane rows, then across rows) ---------------------------
// DPP row permutations used as butterfly steps: each pairs lanes symmetrically, so both lanes of a
// pair compute the same value (a+b = b+a) and every lane of a row ends with the row's result.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i inside each 8 lanes
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i inside each 16 lanes

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ int32_t dpp_i(int32_t v)
{
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}

// Sum over the wave in one fixed order: the butterfly above inside each row, then
// (row0 + row1) + (row2 + row3).  Every lane returns the same value.
__device__ __forceinline__ float wave_sum(float v)
{
    v = v + dpp_f<kDppXor1>(v);
    v = v + dpp_f<kDppXor2>(v);
    v = v + dpp_f<kDppHalfMirror>(v);
    v = v + dpp_f<kDppMirror>(v);
    const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (a + b) + (c + d);
}

__device__ __forceinline__ float wave_max(float v)
{
    v = fmaxf(v, dpp_f<kDppXor1>(v));
    v = fmaxf(v, dpp_f<kDppXor2>(v));
    v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_f<kDppMirror>(v));
    const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// exp used by SiLU and the softmax gates: Cody-Waite reduction z = n ln2 + r with ln2 split in a
// high part whose 12 low significand bits are zero (so n * hi is exact) and a low part, a degree-7
// Taylor polynomial of e^r in Horner form (coefficients 1/m! rounded to fp32), then a scaling by
// 2^n.  Arguments above 80 give +inf and below -80 give 0, so no result is subnormal.  Compiled
// with -ffp-contract=off: every step is one rounded fp32 operation.  Branch-free: the steps run on
// the argument clamped to [-80, 80] (equal to it wherever their result is used) and the special
// cases are selected afterwards.
__device__ __forceinline__ float tw_exp(float z)
{
    const float kLog2e = 1.44269504088896340736f;
    const float kLn2Hi = 0.693145751953125f;
    const float kLn2Lo = 1.42860682030941723212e-6f;
    const float zc = __builtin_fminf(__builtin_fmaxf(z, -80.0f), 80.0f);
    float n = __builtin_rintf(zc * kLog2e);
    float r = zc - n * kLn2Hi;
    r = r - n * kLn2Lo;
    float p = 1.98412698412698412698e-4f;    // 1/7!
    p = p * r + 1.38888888888888888889e-3f;  // 1/6!
    p = p * r + 8.33333333333333333333e-3f;  // 1/5!
    p = p * r + 4.16666666666666666667e-2f;  // 1/4!
    p = p * r + 1.66666666666666666667e-1f;  // 1/3!
    p = p * r + 0.5f;
    p = p * r + 1.0f;
    p = p * r + 1.0f;
    const uint32_t v = __float_as_uint(__builtin_ldexpf(p, int(n)));
    // special cases by masks (sign-extended comparisons), not by branches
    const uint32_t hi = uint32_t(-int32_t(z > 80.0f)), lo = uint32_t(-int32_t(z < -80.0f));
    const uint32_t nan = uint32_t(-int32_t(z != z));
    return __uint_as_float((v & ~(hi | lo | nan)) | (hi & 0x7f800000u) | (nan & __float_as_uint(z)));
}

// SiLU(z) = z / (1 + e^-z), as the division of z by one rounded denominator.
__device__ __forceinline__ float tw_silu(float z) { return z / (1.0f + tw_exp(-z)); }

// Position of element i in the digit-plane layout (4x4 transpose inside every group of 16).
__device__ __forceinline__ int perm16(int i) { return (i & ~15) | ((i & 3) << 2) | ((i >> 2) & 3); }

// ---- digit planes ---------------------------------------------------------------------------

// Shift sh with |v| * 2^sh < 2^(7P) for every |v| <= amax.
__device__ __forceinline__ int float_digit_shift(float amax, int P)
{
    if (!(amax > 0.0f)) return 0;
    int e;
    frexpf(amax, &e);   // amax = f 2^e, f in [0.5, 1)
    return 7 * P - e;
}

template <int P>
__device__ __forceinline__ void float_digits(float v, int sh, int8_t (&dg)[P])
{
    float X = __builtin_rintf(__builtin_ldexpf(v, sh));
    int a = int(fminf(fabsf(X), float((1 << (7 * P)) - 1)));
#pragma unroll
    for (int k = 0; k < P; k++) {
        int dk = (a >> (7 * (P - 1 - k))) & 127;
        dg[k] = int8_t(X < 0.0f ? -dk : dk);
    }
}

// The two digits of s = clamp(rint(v 2^sh), -(2^14 - 1), 2^14 - 1) as a floor split, packed in one
// word: byte 0 holds lo = s mod 128 (0..127), byte 2 holds hi = floor(s / 128) (-128..127), so
// s = 128 hi + lo.  float_digits<2> splits |s| instead and puts the sign on both digits; the planes
// differ but every integer dot against them recombines (128 * sum_hi + sum_lo) to the same exact
// sum, so the results are identical bit for bit.  NaN maps to +(2^14 - 1) in both.
__device__ __forceinline__ uint32_t float_digit_pair(float v, int sh)
{
    const float X = __builtin_rintf(__builtin_ldexpf(v, sh));
    const int a = int(fminf(fabsf(X), 16383.0f));
    const uint32_t s = uint32_t(X < 0.0f ? -a : a);
    return (s & 127u) | ((s << 9) & 0x00ff0000u);
}

// Digit-plane layout: element i of a plane is byte perm16(i), i.e. byte 4k + r of a 16-element group
// is element 4r + k.  Given the digit pairs of the elements 4r + k (r = 0..3) of one group, returns
// the group's dword k of the low-digit plane and of the high-digit plane (the high plane is plane 0
// of float_value<2>, the low plane plane 1).
__device__ __forceinline__ void digit_pair_dwords(const uint32_t (&p)[4], uint32_t &lo, uint32_t &hi)
{
    // v_perm byte selectors: 0..3 pick bytes of the second operand, 4..7 bytes of the first
    const uint32_t m01 = __builtin_amdgcn_perm(p[1], p[0], 0x06020400u);   // lo0 lo1 hi0 hi1
    const uint32_t m23 = __builtin_amdgcn_perm(p[3], p[2], 0x06020400u);   // lo2 lo3 hi2 hi3
    lo = __builtin_amdgcn_perm(m23, m01, 0x05040100u);
    hi = __builtin_amdgcn_perm(m23, m01, 0x07060302u);
}

// int8 activation mode: q = clamp(rint(v * inv), -127, 127) with inv = 127 / amax.
__device__ __forceinline__ int8_t int8_quant(float v, float inv)
{
    float t = __builtin_rintf(v * inv);
    t = fminf(fmaxf(t, -127.0f), 127.0f);
    return int8_t(int(t));
}

// ---- the ternary dot on one 16-byte chunk of codes (64 weights) -------------------------------

__device__ __forceinline__ int32_t lut4(uint32_t sel)
{
    return int32_t(__builtin_amdgcn_perm(0u, kCodeLut, sel));
}

// The four int8x4 weight words of one 32-bit code word: word m holds codes 4j + m (bits 8j + 2m)
// of its bytes j.  Nine ALU operations: the codes in bits 2-3 of a byte are looked up in place.
__device__ __forceinline__ void decode_word(uint32_t w, int32_t &t0, int32_t &t1, int32_t &t2, int32_t &t3)
{
    const uint32_t h = w >> 4;
    t0 = int32_t(__builtin_amdgcn_perm(0u, kCodeLut, w & kCodeMask));
    t1 = int32_t(__builtin_amdgcn_perm(kCodeLutHiHigh, kCodeLutHiLow, w & kCodeMaskHi));
    t2 = int32_t(__builtin_amdgcn_perm(0u, kCodeLut, h & kCodeMask));
    t3 = int32_t(__builtin_amdgcn_perm(kCodeLutHiHigh, kCodeLutHiLow, h & kCodeMaskHi));
}

template <int P>
__device__ __forceinline__ void chunk_dot(const int4 code, const int4 (&dg)[P][4], int32_t (&acc)[P])
{
    const uint32_t w[4] = {uint32_t(code.x), uint32_t(code.y), uint32_t(code.z), uint32_t(code.w)};
#pragma unroll
    for (int q = 0; q < 4; q++) {
        int32_t t0, t1, t2, t3;
        decode_word(w[q], t0, t1, t2, t3);
#pragma unroll
        for (int p = 0; p < P; p++) {
            acc[p] = __builtin_amdgcn_sdot4(t0, dg[p][q].x, acc[p], false);
            acc[p] = __builtin_amdgcn_sdot4(t1, dg[p][q].y, acc[p], false);
            acc[p] = __builtin_amdgcn_sdot4(t2, dg[p][q].z, acc[p], false);
            acc[p] = __builtin_amdgcn_sdot4(t3, dg[p][q].w, acc[p], false);
        }
    }
}

// The same dot with the 16-byte chunk decoded once (wd[4q+m] = the int8x4 word W_m of code word q),
// for chunks applied to several activation vectors.
__device__ __forceinline__ void decode_chunk(const int4 code, int32_t (&wd)[16])
{
    const uint32_t w[4] = {uint32_t(code.x), uint32_t(code.y), uint32_t(code.z), uint32_t(code.w)};
#pragma unroll
    for (int q = 0; q < 4; q++)
        decode_word(w[q], wd[4 * q], wd[4 * q + 1], wd[4 * q + 2], wd[4 * q + 3]);
}

template <int P>
__device__ __forceinline__ void dec_dot(const int32_t (&wd)[16], const int4 (&dg)[P][4], int32_t (&acc)[P])
{
#pragma unroll
    for (int q = 0; q < 4; q++) {
#pragma unroll
        for (int p = 0; p < P; p++) {
            acc[p] = __builtin_amdgcn_sdot4(wd[4 * q + 0], dg[p][q].x, acc[p], false);
            acc[p] = __builtin_amdgcn_sdot4(wd[4 * q + 1], dg[p][q].y, acc[p], false);
            acc[p] = __builtin_amdgcn_sdot4(wd[4 * q + 2], dg[p][q].z, acc[p], false);
            acc[p] = __builtin_amdgcn_sdot4(wd[4 * q + 3], dg[p][q].w, acc[p], false);
        }
    }
}

// Integer sum over the `lanes` consecutive lanes that share one row of weights (lanes a power of
// two <= 64); every lane of the group receives the total (integer sums: any order is exact).
template <int P>
__device__ __forceinline__ void group_reduce(int32_t (&acc)[P], int lanes)
{
#pragma unroll
    for (int p = 0; p < P; p++) {
        int32_t v = acc[p];
        if (lanes > 1) v += dpp_i<kDppXor1>(v);
        if (lanes > 2) v += dpp_i<kDppXor2>(v);
        if (lanes > 4) v += dpp_i<kDppHalfMirror>(v);
        if (lanes > 8) v += dpp_i<kDppMirror>(v);
        if (lanes > 16) v += __shfl_xor(v, 16);
        if (lanes > 32) v += __shfl_xor(v, 32);
        acc[p] = v;
    }
}

// Float-mode value of a row: sum_k 128^(P-1-k) acc_k, scaled by 2^-sh.
template <int P>
__device__ __forceinline__ float float_value(const int32_t (&acc)[P], int sh)
{
    float v = float(acc[0]);
#pragma unroll
    for (int p = 1; p < P; p++) v = v * 128.0f + float(acc[p]);
    return __builtin_ldexpf(v, -sh);
}

// ---- canonical float dot products ------------------------------------------------------------
// Every fp32 dot product that feeds routing (router logits, the sum of squares of the pre-RMSNorm)
// is summed in one fixed order, whichever kernel computes it: the d elements form 8-element chunks;
// chunk c is added (products in order) into partial t = c mod 256, partials accumulating their
// chunks in increasing c; partials 64w..64w+63 are reduced by wave_sum into s_w, and the result is
// (s_0 + s_1) + (s_2 + s_3).  A 256-thread block computes it with one partial per thread; a single
// wave loops over w.  Equal inputs therefore give equal logits in the decode and batched paths.
// w(i) and x(i) return element i as fp32.
template <typename W, typename X>
__device__ __forceinline__ float canon_dot(int d, int lane, W w, X x)
{
    float s[4];
#pragma unroll
    for (int wv = 0; wv < 4; wv++) {
        float acc = 0.0f;
        for (int c = 64 * wv + lane; c < (d >> 3); c += 256) {
#pragma unroll
            for (int j = 0; j < 8; j++) acc = acc + w(8 * c + j) * x(8 * c + j);
        }
        s[wv] = wave_sum(acc);
    }
    return (s[0] + s[1]) + (s[2] + s[3]);
}

// Inverse RMS of the pre-RMSNorm (unit weight, eps 1e-6) from the canonical sum of squares.
__device__ __forceinline__ float inv_rms_of(float ss, int d) { return 1.0f / sqrtf(ss / float(d) + 1e-6f); }

__device__ __forceinline__ float bf16_round(float v) { return bf16_to_f32(f32_to_bf16(v)); }

// ---- tagged 64-bit words -------------------------------------------------------------------
// Workgroups of one launch hand each other small vectors through 64-bit words that carry a 32-bit
// tag next to 32 bits of data, written and read with single 64-bit device-scope atomic accesses:
// a reader that sees the expected tag also sees the data stored with it, so no fence or barrier
// is needed between producer and consumer.
__device__ __forceinline__ void st_tagged(uint64_t *p, uint32_t tag, uint32_t data)
{
    __hip_atomic_store(p, (uint64_t(tag) << 32) | data, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t ld_tagged(const uint64_t *p)
{
    return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

// ---- top-k + softmax by one wave ------------------------------------------------------------
// Selection order: larger logit first; equal logits -> lower expert id first.  A logit is mapped to
// an order-preserving 32-bit key (+0 and -0 share one key).  Lane l holds the experts l, l+64, ...
// sorted by (key descending, id ascending); each round takes the wave maximum of the lane heads,
// then the lowest id among the heads that carry it, and that lane pops its head.
__device__ __forceinline__ uint32_t float_order_key(float v)
{
    const uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float float_of_order_key(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max(v, uint32_t(dpp_i<kDppXor1>(int32_t(v))));
    v = max(v, uint32_t(dpp_i<kDppXor2>(int32_t(v))));
    v = max(v, uint32_t(dpp_i<kDppHalfMirror>(int32_t(v))));
    v = max(v, uint32_t(dpp_i<kDppMirror>(int32_t(v))));
    const uint32_t a = uint32_t(__builtin_amdgcn_readlane(int32_t(v), 0));
    const uint32_t b = uint32_t(__builtin_amdgcn_readlane(int32_t(v), 16));
    const uint32_t c = uint32_t(__builtin_amdgcn_readlane(int32_t(v), 32));
    const uint32_t d = uint32_t(__builtin_amdgcn_readlane(int32_t(v), 48));
    return max(max(a, b), max(c, d));
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v)
{
    v = min(v, uint32_t(dpp_i<kDppXor1>(int32_t(v))));
    v = min(v, uint32_t(dpp_i<kDppXor2>(int32_t(v))));
    v = min(v, uint32_t(dpp_i<kDppHalfMirror>(int32_t(v))));
    v = min(v, uint32_t(dpp_i<kDppMirror>(int32_t(v))));
    const uint32_t a = uint32_t(__builtin_amdgcn_readlane(int32_t(v), 0));
    const uint32_t b = uint32_t(__builtin_amdgcn_readlane(int32_t(v), 16));
    const uint32_t c = uint32_t(__builtin_amdgcn_readlane(int32_t(v), 32));
    const uint32_t d = uint32_t(__builtin_amdgcn_readlane(int32_t(v), 48));
    return min(min(a, b), min(c, d));
}

// Top-k of one wave over logits in registers: lv[s] is the logit of expert lane + 64 s (any value
// where that is >= E).  ids_out / gates_out receive the k ids and gates in selection order;
// GATES = false leaves the selected logits in gates_out (softmax_gates_wave finishes the gates).
template <int KPER, bool GATES = true>
__device__ __forceinline__ void topk_softmax_wave_regs(const float (&lv)[KPER], int E, int k,
                                                       int32_t *ids_out, float *gates_out, int lane)
{
    uint32_t key[KPER];
    uint32_t idv[KPER];
#pragma unroll
    for (int s = 0; s < KPER; s++) {
        idv[s] = uint32_t(lane + 64 * s);
        key[s] = int(idv[s]) < E ? float_order_key(lv[s] + 0.0f) : 0u;   // 0: no candidate
    }
    // sort the lane's candidates: key descending, id ascending (ids already ascending in s)
#pragma unroll
    for (int i = 1; i < KPER; i++)
#pragma unroll
        for (int j = i; j > 0; j--) {
            const bool sw = key[j] > key[j - 1];   // equal keys keep their (ascending id) order
            const uint32_t k0 = key[j - 1], i0 = idv[j - 1];
            key[j - 1] = sw ? key[j] : k0;
            idv[j - 1] = sw ? idv[j] : i0;
            key[j] = sw ? k0 : key[j];
            idv[j] = sw ? i0 : idv[j];
        }
    float my_v = 0.0f;
    int32_t my_id = 0;
    for (int j = 0; j < k; j++) {
        const uint32_t m = wave_max_u32(key[0]);
        // the lane heads carrying the maximum: one lane (the usual case) or a tie on the logit
        const uint64_t holders = __ballot(key[0] == m);
        const uint32_t id = __popcll(holders) == 1
                                ? uint32_t(__builtin_amdgcn_readlane(int32_t(idv[0]), __ffsll((long long)holders) - 1))
                                : wave_min_u32(key[0] == m ? idv[0] : 0xffffffffu);
        if (idv[0] == id && key[0] == m) {
#pragma unroll
            for (int s = 0; s + 1 < KPER; s++) {
                key[s] = key[s + 1];
                idv[s] = idv[s + 1];
            }
            key[KPER - 1] = 0u;
        }
        if (lane == j) {
            my_v = float_of_order_key(m);
            my_id = int32_t(id);
        }
    }
    if (!GATES) {
        // the selected logits (canonical, in selection order) for softmax_gates_wave
        if (lane < k) {
            ids_out[lane] = my_id;
            gates_out[lane] = my_v;
        }
        return;
    }
    // gates: softmax over the selected logits; e^(l_j - l_0) in parallel, the sum in order
    const float v0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_v), 0));
    const float ex = tw_exp(my_v - v0);
    float den = 0.0f;
    for (int j = 0; j < k; j++) den = den + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
    if (lane < k) {
        ids_out[lane] = my_id;
        gates_out[lane] = ex / den;
    }
}

// A shorter form of topk_softmax_wave_regs<KPER, false> for E <= 256.  Each candidate becomes one
// 32-bit composite: the upper 24 bits of its order key, then 255 - id, so that a round is a single
// 32-bit wave maximum with no tie step (composites are distinct).  It runs k rounds and accepts the
// result when the 24-bit parts of the k winners strictly decrease and no other candidate's 24-bit
// part reaches the k-th winner's: a larger key never has a smaller 24-bit part, so then the k
// rounds selected the k largest keys in the exact order, and no candidate outside them has a key as
// large as the k-th.  Returns false when they do not (near-equal
// or equal logits); the caller then runs the exact form.  On success lane j < k holds the id and
// the logit selected in round j.  Measured alone (one wave, 8 of 256): 0.78 us against 0.95 for the
// exact form.
template <int KPER>
__device__ __forceinline__ bool topk_wave_composite(const float (&lv)[KPER], int E, int k, int32_t &my_id,
                                                    float &my_v, int lane)
{
    static_assert(KPER <= 4, "composites carry 8-bit ids");
    uint32_t c[KPER];
#pragma unroll
    for (int s = 0; s < KPER; s++) {
        const uint32_t id = uint32_t(lane + 64 * s);
        c[s] = int(id) < E ? (float_order_key(lv[s] + 0.0f) & 0xffffff00u) | (255u - id) : 0u;
    }
    // the lane's composites in descending order (distinct, so max / min exchanges)
#pragma unroll
    for (int i = 1; i < KPER; i++)
#pragma unroll
        for (int j = i; j > 0; j--) {
            const uint32_t hi = max(c[j - 1], c[j]), lo = min(c[j - 1], c[j]);
            c[j - 1] = hi;
            c[j] = lo;
        }
    uint32_t mine = 0u;   // lane j: the composite selected in round j
    uint32_t prev = 0xffffffffu;
    bool ok = true;
    for (int j = 0; j < k; j++) {
        const uint32_t m = wave_max_u32(c[0]);
        ok = ok && (j == 0 || (m >> 8) < (prev >> 8));
        prev = m;
        mine = lane == j ? m : mine;
        if (c[0] == m) {
#pragma unroll
            for (int s = 0; s + 1 < KPER; s++) c[s] = c[s + 1];
            c[KPER - 1] = 0u;
        }
    }
    // in place of round k + 1: no remaining candidate (each lane's head is its largest) reaches the
    // 24-bit part of the k-th selected one
    ok = ok && __ballot((c[0] >> 8) >= (prev >> 8)) == 0;
    if (!ok) return false;
    // lane j < k: its logit is in lane id % 64, slot id / 64
    const uint32_t id = 255u - (mine & 255u);
    const int src = int(id & 63u) * 4;
    float v = 0.0f;
#pragma unroll
    for (int s = 0; s < KPER; s++) {
        const float f = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(lv[s])));
        v = int(id >> 6) == s ? f : v;
    }
    my_id = int32_t(id);
    my_v = v + 0.0f;
    return true;
}

// The same, the ids and selected logits written to ids_out / vals_out[0 .. k) on success.
template <int KPER>
__device__ __forceinline__ bool topk_wave_composite_to(const float (&lv)[KPER], int E, int k, int32_t *ids_out,
                                                       float *vals_out, int lane)
{
    int32_t id;
    float v;
    if (!topk_wave_composite<KPER>(lv, E, k, id, v, lane)) return false;
    if (lane < k) {
        ids_out[lane] = id;
        vals_out[lane] = v;
    }
    return true;
}

// The same, the logits read from logits[0 .. E).
template <int KPER, bool GATES = true>
__device__ __forceinline__ void topk_softmax_wave_t(const float *logits, int E, int k, int32_t *ids_out,
                                    float *gates_out, int lane)
{
    float lv[KPER];
#pragma unroll
    for (int s = 0; s < KPER; s++) {   // every load issued before the first use (index clamped)
        const int e = lane + 64 * s;
        lv[s] = logits[e < E ? e : E - 1];
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (KPER <= 4) {
        int32_t my_id;
        float my_v;
        if (topk_wave_composite<KPER>(lv, E, k, my_id, my_v, lane)) {
            if (GATES) {   // the gates as topk_softmax_wave_regs forms them
                const float v0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_v), 0));
                const float ex = tw_exp(my_v - v0);
                float den = 0.0f;
                for (int j = 0; j < k; j++) den = den + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
                my_v = ex / den;
            }
            if (lane < k) {
                ids_out[lane] = my_id;
                gates_out[lane] = my_v;
            }
            return;
        }
    }
    topk_softmax_wave_regs<KPER, GATES>(lv, E, k, ids_out, gates_out, lane);
}

// The gates of topk_softmax_wave_t<KPER, false>: g[j] holds the j-th selected logit on entry and
// its gate on return, the same operations in the same order as the fused form.  One wave.
__device__ __forceinline__ void softmax_gates_wave(float *g, int k, int lane)
{
    const float my_v = lane < k ? g[lane] : 0.0f;
    const float v0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_v), 0));
    const float ex = tw_exp(my_v - v0);
    float den = 0.0f;
    for (int j = 0; j < k; j++) den = den + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
    if (lane < k) g[lane] = ex / den;
}

__device__ __forceinline__ void topk_softmax_wave(const float *logits, int E, int k, int32_t *ids_out,
                                                  float *gates_out, int lane)
{
    if (E <= 64) topk_softmax_wave_t<1>(logits, E, k, ids_out, gates_out, lane);
    else if (E <= 128) topk_softmax_wave_t<2>(logits, E, k, ids_out, gates_out, lane);
    else if (E <= 256) topk_softmax_wave_t<4>(logits, E, k, ids_out, gates_out, lane);
    else if (E <= 512) topk_softmax_wave_t<8>(logits, E, k, ids_out, gates_out, lane);
    else topk_softmax_wave_t<16>(logits, E, k, ids_out, gates_out, lane);
}

}  // namespace
}  // namespace tw
