// tw_kernels.hip -- HIP kernels for the ternary MoE FFN on gfx950 (MI355X), and their launchers.
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
// W_m lines up with the activation word A_m without any shuffling at run time.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tw_internal.h"

namespace tw {
namespace {

constexpr uint32_t kCodeMask = 0x03030303u;
// Byte c of this word is the int8 weight of code c: 00 -> 0, 01 -> +1, 10 -> -1, 11 -> 0.
constexpr uint32_t kCodeLut = 0x00FF0100u;

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

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// exp used by SiLU and the softmax gates: Cody-Waite reduction z = n ln2 + r with ln2 split in a
// high part whose 12 low significand bits are zero (so n * hi is exact) and a low part, a degree-7
// Taylor polynomial of e^r in Horner form (coefficients 1/m! rounded to fp32), then a scaling by
// 2^n.  Arguments above 80 give +inf and below -80 give 0, so no result is subnormal.  Compiled
// with -ffp-contract=off: every step is one rounded fp32 operation.
__device__ __forceinline__ float tw_exp(float z)
{
    if (z > 80.0f) return __builtin_inff();
    if (z < -80.0f) return 0.0f;
    const float kLog2e = 1.44269504088896340736f;
    const float kLn2Hi = 0.693145751953125f;
    const float kLn2Lo = 1.42860682030941723212e-6f;
    float n = __builtin_rintf(z * kLog2e);
    float r = z - n * kLn2Hi;
    r = r - n * kLn2Lo;
    float p = 1.98412698412698412698e-4f;    // 1/7!
    p = p * r + 1.38888888888888888889e-3f;  // 1/6!
    p = p * r + 8.33333333333333333333e-3f;  // 1/5!
    p = p * r + 4.16666666666666666667e-2f;  // 1/4!
    p = p * r + 1.66666666666666666667e-1f;  // 1/3!
    p = p * r + 0.5f;
    p = p * r + 1.0f;
    p = p * r + 1.0f;
    return __builtin_ldexpf(p, int(n));
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

template <int P>
__device__ __forceinline__ void chunk_dot(const int4 code, const int4 (&dg)[P][4], int32_t (&acc)[P])
{
    const uint32_t w[4] = {uint32_t(code.x), uint32_t(code.y), uint32_t(code.z), uint32_t(code.w)};
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const int32_t t0 = lut4(w[q] & kCodeMask);
        const int32_t t1 = lut4((w[q] >> 2) & kCodeMask);
        const int32_t t2 = lut4((w[q] >> 4) & kCodeMask);
        const int32_t t3 = lut4((w[q] >> 6) & kCodeMask);
#pragma unroll
        for (int p = 0; p < P; p++) {
            acc[p] = __builtin_amdgcn_sdot4(t0, dg[p][q].x, acc[p], false);
            acc[p] = __builtin_amdgcn_sdot4(t1, dg[p][q].y, acc[p], false);
            acc[p] = __builtin_amdgcn_sdot4(t2, dg[p][q].z, acc[p], false);
            acc[p] = __builtin_amdgcn_sdot4(t3, dg[p][q].w, acc[p], false);
        }
    }
}

// Sum over the `lanes` consecutive lanes that share one row (lanes is a power of two <= 64).
template <int P>
__device__ __forceinline__ void group_reduce(int32_t (&acc)[P], int lanes)
{
    for (int o = lanes >> 1; o > 0; o >>= 1) {
#pragma unroll
        for (int p = 0; p < P; p++) acc[p] += __shfl_xor(acc[p], o);
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

// ---- top-k + softmax by one wave ------------------------------------------------------------
// Selection order: larger logit first; equal logits -> lower expert id first.
__device__ void topk_softmax_wave(const float *logits, int E, int k, int32_t *ids_out,
                                  float *gates_out, int lane)
{
    constexpr int kPer = kMaxExperts / 64;
    float v[kPer];
    uint32_t taken = 0;
#pragma unroll
    for (int s = 0; s < kPer; s++) {
        int e = lane + 64 * s;
        v[s] = e < E ? logits[e] : -__builtin_inff();
        if (e >= E) taken |= 1u << s;
    }
    float sel_v[kMaxTopK];
    int32_t sel_i[kMaxTopK];
    for (int j = 0; j < k; j++) {
        float bv = -__builtin_inff();
        int bi = 0x7fffffff;
#pragma unroll
        for (int s = 0; s < kPer; s++) {
            int e = lane + 64 * s;
            bool free_ = !((taken >> s) & 1u);
            // the first free entry is always taken, so the id is valid even for NaN logits
            if (free_ && (bi == 0x7fffffff || v[s] > bv || (v[s] == bv && e < bi))) {
                bv = v[s];
                bi = e;
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            float ov = __shfl_xor(bv, o);
            int oi = __shfl_xor(bi, o);
            if (oi != 0x7fffffff && (bi == 0x7fffffff || ov > bv || (ov == bv && oi < bi))) {
                bv = ov;
                bi = oi;
            }
        }
        if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
        sel_v[j] = bv;
        sel_i[j] = bi;
    }
    if (lane == 0) {
        float ex[kMaxTopK];
        float den = 0.0f;
        for (int j = 0; j < k; j++) {
            ex[j] = tw_exp(sel_v[j] - sel_v[0]);
            den = den + ex[j];
        }
        for (int j = 0; j < k; j++) {
            ids_out[j] = sel_i[j];
            gates_out[j] = ex[j] / den;
        }
    }
}

// ------------------------------------------------------------------------------------------------
// ternary_pack

__global__ void k_pack16(const int4 *__restrict__ w, int64_t n16, uint32_t *__restrict__ out,
                         int32_t *bad)
{
    int local_bad = 0;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16;
         i += int64_t(gridDim.x) * blockDim.x) {
        const int4 v = w[i];
        const uint32_t word[4] = {uint32_t(v.x), uint32_t(v.y), uint32_t(v.z), uint32_t(v.w)};
        uint32_t res = 0;
#pragma unroll
        for (int q = 0; q < 4; q++) {
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int x = int8_t(word[q] >> (8 * j));
                const uint32_t c = x == 1 ? 1u : (x == -1 ? 2u : 0u);
                local_bad += (x > 1 || x < -1);
                res |= c << (8 * q + 2 * j);
            }
        }
        out[i] = res;
    }
    if (bad) {
        float s = wave_sum(float(local_bad));
        if ((threadIdx.x & 63) == 0 && s > 0.0f) atomicAdd(bad, int32_t(s));
    }
}

__global__ void k_pack_any(const int8_t *__restrict__ w, int64_t rows, int64_t cols,
                           uint8_t *__restrict__ out, int32_t *bad)
{
    const int64_t stride = (cols + 3) / 4, n = rows * stride;
    int local_bad = 0;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * blockDim.x) {
        const int64_t r = i / stride, b = i % stride;
        uint32_t byte = 0;
        for (int j = 0; j < 4; j++) {
            const int64_t c = 4 * b + j;
            if (c < cols) {
                const int x = w[r * cols + c];
                byte |= (x == 1 ? 1u : (x == -1 ? 2u : 0u)) << (2 * j);
                local_bad += (x > 1 || x < -1);
            }
        }
        out[i] = uint8_t(byte);
    }
    if (bad) {
        float s = wave_sum(float(local_bad));
        if ((threadIdx.x & 63) == 0 && s > 0.0f) atomicAdd(bad, int32_t(s));
    }
}

// ------------------------------------------------------------------------------------------------
// Router logits for T tokens: one wave per (token, expert), fp32 sums.  Also the pre-RMSNorm
// factor of the token, folded in as a scalar: W_r (x / rms) = (W_r x) / rms.

__global__ __launch_bounds__(256) void k_router_logits(const void *__restrict__ x, int x_bf16,
                                                       const void *__restrict__ wr, int w_bf16,
                                                       int64_t T, int d, int E, int pre_norm,
                                                       float *__restrict__ logits)
{
    const int lane = threadIdx.x & 63;
    const int64_t gw = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (gw >= T * E) return;
    const int64_t t = gw / E;
    const int e = int(gw % E);
    const int64_t xo = t * d;
    float acc = 0.0f, ss = 0.0f;
    for (int i = lane; i < d; i += 64) {
        const float xv = load_act(x, xo + i, x_bf16);
        const float wv = load_act(wr, int64_t(e) * d + i, w_bf16);
        acc += wv * xv;
        ss += xv * xv;
    }
    acc = wave_sum(acc);
    if (pre_norm) {
        ss = wave_sum(ss);
        acc = acc * (1.0f / sqrtf(ss / float(d) + 1e-6f));
    }
    if (lane == 0) logits[t * E + e] = acc;
}

__global__ __launch_bounds__(256) void k_topk(const float *__restrict__ logits, int64_t T, int E,
                                              int k, int32_t *__restrict__ ids,
                                              float *__restrict__ gates)
{
    const int lane = threadIdx.x & 63;
    const int64_t t = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    topk_softmax_wave(logits + t * E, E, k, ids + t * k, gates + t * k, lane);
}

// ------------------------------------------------------------------------------------------------
// Batch-1 decode, one layer = three kernels: route, gate/up, down + combine.

struct DecodeArgs {
    Dims dm;
    DecodeWs L;
    int io_bf16;
};

__global__ void k_zero_u32(uint32_t *p, int n)
{
    for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

// Router logits (one wave per expert), the pre-RMSNorm factor, and the digit planes of x (block 0).
// The last block to finish selects the top-k and computes the gates.
template <int P>
__global__ __launch_bounds__(256) void k_dec_route(DecodeArgs a, const void *__restrict__ wr,
                                                   const void *__restrict__ x,
                                                   uint8_t *__restrict__ ws)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int d = a.dm.d, E = a.dm.E;
    float *logits = reinterpret_cast<float *>(ws + a.L.logits);
    float ss = 0.0f;
    for (int i = lane; i < d; i += 64) {
        const float v = load_act(x, i, a.io_bf16);
        ss += v * v;
    }
    ss = wave_sum(ss);
    const float inv_rms = a.dm.pre_norm ? 1.0f / sqrtf(ss / float(d) + 1e-6f) : 1.0f;
    const int e = blockIdx.x * 4 + wave;
    if (e < E) {
        float acc = 0.0f;
        for (int i = lane; i < d; i += 64)
            acc += load_act(wr, int64_t(e) * d + i, a.dm.router_bf16) * load_act(x, i, a.io_bf16);
        acc = wave_sum(acc);
        if (lane == 0) logits[e] = acc * inv_rms;
    }
    if (blockIdx.x == 0 && wave == 0) {
        float am = 0.0f;
        for (int i = lane; i < d; i += 64) am = fmaxf(am, fabsf(load_act(x, i, a.io_bf16)));
        am = wave_max(am);
        const int sh = float_digit_shift(am, P);
        int8_t *xd = reinterpret_cast<int8_t *>(ws + a.L.xdig);
        for (int i = lane; i < d; i += 64) {
            int8_t dg[P];
            float_digits<P>(load_act(x, i, a.io_bf16), sh, dg);
#pragma unroll
            for (int p = 0; p < P; p++) xd[p * d + perm16(i)] = dg[p];
        }
        if (lane == 0) {
            int32_t *xi = reinterpret_cast<int32_t *>(ws + a.L.xinfo);
            xi[0] = sh;
            reinterpret_cast<float *>(xi)[1] = inv_rms;
        }
    }
    __shared__ int is_last;
    __syncthreads();
    uint32_t *ctrl = reinterpret_cast<uint32_t *>(ws + a.L.ctrl);
    if (threadIdx.x == 0) {
        __threadfence();
        is_last = atomicAdd(ctrl, 1u) == gridDim.x - 1;
    }
    __syncthreads();
    if (is_last) {
        __threadfence();
        if (wave == 0)
            topk_softmax_wave(logits, E, a.dm.k, reinterpret_cast<int32_t *>(ws + a.L.ids),
                              reinterpret_cast<float *>(ws + a.L.gates), lane);
        if (threadIdx.x == 0) ctrl[0] = 0;
    }
}

constexpr int kDecRowsGU = 16;   // gate rows (and as many up rows) per block
constexpr int kDecRowsDown = 8;  // output rows per block (for all k experts)

template <int P>
__global__ __launch_bounds__(256) void k_dec_gateup(DecodeArgs a, LayerPtrs lp,
                                                    uint8_t *__restrict__ ws)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int d = a.dm.d, F = a.dm.F;
    const int nrb = F / kDecRowsGU;
    const int j = blockIdx.x / nrb, rb = blockIdx.x % nrb;
    const int e = reinterpret_cast<const int32_t *>(ws + a.L.ids)[j];
    const int32_t *xi = reinterpret_cast<const int32_t *>(ws + a.L.xinfo);
    const int sh = xi[0];
    const float inv_rms = reinterpret_cast<const float *>(xi)[1];
    const int lpr = d >> 6;                 // lanes per row (16 bytes = 64 weights per lane)
    const int rpp = 64 / lpr;               // rows per wave pass
    const int sub = lane / lpr, c = lane % lpr;
    const int8_t *xd = reinterpret_cast<const int8_t *>(ws + a.L.xdig);
    int4 dg[P][4];
#pragma unroll
    for (int p = 0; p < P; p++)
#pragma unroll
        for (int q = 0; q < 4; q++) dg[p][q] = reinterpret_cast<const int4 *>(xd + p * d + c * 64)[q];

    __shared__ float sums[2 * kDecRowsGU];
    const int njobs = 2 * kDecRowsGU;
    const int64_t rstride = d / 4;
    for (int base = wave * rpp; base < njobs; base += 4 * rpp) {
        const int job = base + sub;
        const bool valid = job < njobs;
        const int rl = job % kDecRowsGU;
        const bool up = job >= kDecRowsGU;
        const int r = rb * kDecRowsGU + rl;
        const uint8_t *row = (up ? lp.w_up : lp.w_gate) + (int64_t(e) * F + r) * rstride;
        const int4 code = valid ? reinterpret_cast<const int4 *>(row)[c] : make_int4(0, 0, 0, 0);
        int32_t acc[P] = {};
        chunk_dot<P>(code, dg, acc);
        group_reduce<P>(acc, lpr);
        if (c == 0 && valid) {
            const float s = (up ? lp.s_up : lp.s_gate)[int64_t(e) * F + r];
            sums[job] = float_value<P>(acc, sh) * s * inv_rms;
        }
    }
    __syncthreads();
    if (threadIdx.x < kDecRowsGU) {
        const int t = threadIdx.x;
        const float g = sums[t], u = sums[kDecRowsGU + t];
        reinterpret_cast<float *>(ws + a.L.h)[j * F + rb * kDecRowsGU + t] = tw_silu(g) * u;
    }
}

template <int P>
__global__ __launch_bounds__(256) void k_dec_down(DecodeArgs a, LayerPtrs lp,
                                                  const void *__restrict__ x,
                                                  void *__restrict__ out, uint8_t *__restrict__ ws)
{
    extern __shared__ __attribute__((aligned(16))) int8_t smem[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int d = a.dm.d, F = a.dm.F, k = a.dm.k;
    int8_t *hd = smem;                                          // [k][P][F]
    int *shs = reinterpret_cast<int *>(smem + k * P * F);      // [k]
    float *ys = reinterpret_cast<float *>(shs + kMaxTopK);     // [k][RO]
    const float *h = reinterpret_cast<const float *>(ws + a.L.h);
    const int32_t *ids = reinterpret_cast<const int32_t *>(ws + a.L.ids);
    const float *gates = reinterpret_cast<const float *>(ws + a.L.gates);

    for (int j = wave; j < k; j += 4) {
        float am = 0.0f;
        for (int i = lane; i < F; i += 64) am = fmaxf(am, fabsf(h[j * F + i]));
        am = wave_max(am);
        const int sh = float_digit_shift(am, P);
        for (int i = lane; i < F; i += 64) {
            int8_t dg[P];
            float_digits<P>(h[j * F + i], sh, dg);
#pragma unroll
            for (int p = 0; p < P; p++) hd[(j * P + p) * F + perm16(i)] = dg[p];
        }
        if (lane == 0) shs[j] = sh;
    }
    __syncthreads();

    const int lpr = F >> 6, rpp = 64 / lpr;
    const int sub = lane / lpr, c = lane % lpr;
    const int njobs = kDecRowsDown * k;
    const int64_t rstride = F / 4;
    for (int base = wave * rpp; base < njobs; base += 4 * rpp) {
        const int job = base + sub;
        const bool valid = job < njobs;
        const int jj = valid ? job / kDecRowsDown : 0, rl = job % kDecRowsDown;
        const int e = ids[jj];
        const int r = blockIdx.x * kDecRowsDown + rl;
        const uint8_t *row = lp.w_down + (int64_t(e) * d + r) * rstride;
        const int4 code = valid ? reinterpret_cast<const int4 *>(row)[c] : make_int4(0, 0, 0, 0);
        int4 dg[P][4];
#pragma unroll
        for (int p = 0; p < P; p++)
#pragma unroll
            for (int q = 0; q < 4; q++)
                dg[p][q] = reinterpret_cast<const int4 *>(hd + (jj * P + p) * F + c * 64)[q];
        int32_t acc[P] = {};
        chunk_dot<P>(code, dg, acc);
        group_reduce<P>(acc, lpr);
        if (c == 0 && valid)
            ys[jj * kDecRowsDown + rl] = float_value<P>(acc, shs[jj]) * lp.s_down[int64_t(e) * d + r];
    }
    __syncthreads();
    if (threadIdx.x < kDecRowsDown) {
        const int r = blockIdx.x * kDecRowsDown + threadIdx.x;
        float o = load_act(x, r, a.io_bf16);
        for (int j = 0; j < k; j++) o = o + gates[j] * ys[j * kDecRowsDown + threadIdx.x];
        store_act(out, r, o, a.io_bf16);
    }
}

// ------------------------------------------------------------------------------------------------
// Batched: tokens grouped by expert so that each expert's rows are read once per call.

struct BatchedArgs {
    Dims dm;
    BatchedWs L;
    int64_t T;
    int int8_act;
};

// Digit planes of every token (int8 mode: one plane, scale amax/127; float mode: P planes, shift).
template <int P, bool INT8>
__global__ __launch_bounds__(64) void k_bat_quant_x(BatchedArgs a, const void *__restrict__ x,
                                                    int x_bf16, uint8_t *__restrict__ ws)
{
    const int lane = threadIdx.x;
    const int64_t t = blockIdx.x;
    const int d = a.dm.d;
    const int64_t xo = t * d;
    float am = 0.0f;
    for (int i = lane; i < d; i += 64) am = fmaxf(am, fabsf(load_act(x, xo + i, x_bf16)));
    am = wave_max(am);
    int8_t *xd = reinterpret_cast<int8_t *>(ws + a.L.xdig) + t * int64_t(P) * d;
    float *ti = reinterpret_cast<float *>(ws + a.L.tinfo) + 2 * t;
    if (INT8) {
        const float inv = am > 0.0f ? 127.0f / am : 0.0f;
        for (int i = lane; i < d; i += 64)
            xd[perm16(i)] = am > 0.0f ? int8_quant(load_act(x, xo + i, x_bf16), inv) : int8_t(0);
        if (lane == 0) ti[0] = am > 0.0f ? am / 127.0f : 0.0f;
    } else {
        const int sh = float_digit_shift(am, P);
        for (int i = lane; i < d; i += 64) {
            int8_t dg[P];
            float_digits<P>(load_act(x, xo + i, x_bf16), sh, dg);
#pragma unroll
            for (int p = 0; p < P; p++) xd[p * d + perm16(i)] = dg[p];
        }
        if (lane == 0) reinterpret_cast<int32_t *>(ti)[0] = sh;
    }
}

// Counting sort of the T*k (token, slot) pairs by expert, stable in pair index: one block, one
// thread per expert scanning all pairs in order.
__global__ __launch_bounds__(1024) void k_group(BatchedArgs a, const int32_t *__restrict__ ids,
                                                uint8_t *__restrict__ ws)
{
    const int E = a.dm.E;
    const int64_t npairs = a.T * a.dm.k;
    int32_t *counts = reinterpret_cast<int32_t *>(ws + a.L.counts);
    int32_t *offsets = reinterpret_cast<int32_t *>(ws + a.L.offsets);
    int32_t *pairs = reinterpret_cast<int32_t *>(ws + a.L.pairs);
    __shared__ int32_t cnt[kMaxExperts + 1];
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int32_t c = 0;
        for (int64_t p = 0; p < npairs; p++) c += ids[p] == e;
        cnt[e] = c;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int32_t run = 0;
        for (int e = 0; e < E; e++) {
            offsets[e] = run;
            counts[e] = cnt[e];
            run += cnt[e];
        }
        offsets[E] = run;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int32_t pos = offsets[e];
        for (int64_t p = 0; p < npairs; p++)
            if (ids[p] == e) pairs[pos++] = int32_t(p);
    }
}

// Gate/up rows of one expert for all its tokens: block = (expert, block of 16 rows).
template <int P, bool INT8>
__global__ __launch_bounds__(256) void k_bat_gateup(BatchedArgs a, LayerPtrs lp,
                                                    uint8_t *__restrict__ ws)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int d = a.dm.d, F = a.dm.F, k = a.dm.k;
    const int nrb = F / kDecRowsGU;
    const int e = blockIdx.x / nrb, rb = blockIdx.x % nrb;
    const int32_t *offsets = reinterpret_cast<const int32_t *>(ws + a.L.offsets);
    const int32_t *pairs = reinterpret_cast<const int32_t *>(ws + a.L.pairs);
    const int p0 = offsets[e], p1 = offsets[e + 1];
    if (p0 == p1) return;
    const int lpr = d >> 6, rpp = 64 / lpr;
    const int sub = lane / lpr, c = lane % lpr;
    const int njobs = 2 * kDecRowsGU;
    const int64_t rstride = d / 4;
    const int8_t *xdig = reinterpret_cast<const int8_t *>(ws + a.L.xdig);
    const float *tinfo = reinterpret_cast<const float *>(ws + a.L.tinfo);
    float *hbuf = reinterpret_cast<float *>(ws + a.L.h);
    __shared__ float sums[2 * kDecRowsGU];
    for (int pi = p0; pi < p1; pi++) {
        const int pair = pairs[pi];
        const int64_t t = pair / k;
        const int8_t *xd = xdig + t * int64_t(P) * d;
        int4 dg[P][4];
#pragma unroll
        for (int p = 0; p < P; p++)
#pragma unroll
            for (int q = 0; q < 4; q++) dg[p][q] = reinterpret_cast<const int4 *>(xd + p * d + c * 64)[q];
        for (int base = wave * rpp; base < njobs; base += 4 * rpp) {
            const int job = base + sub;
            const bool valid = job < njobs;
            const int rl = job % kDecRowsGU;
            const bool up = job >= kDecRowsGU;
            const int r = rb * kDecRowsGU + rl;
            const uint8_t *row = (up ? lp.w_up : lp.w_gate) + (int64_t(e) * F + r) * rstride;
            const int4 code = valid ? reinterpret_cast<const int4 *>(row)[c] : make_int4(0, 0, 0, 0);
            int32_t acc[P] = {};
            chunk_dot<P>(code, dg, acc);
            group_reduce<P>(acc, lpr);
            if (c == 0 && valid) {
                const float s = (up ? lp.s_up : lp.s_gate)[int64_t(e) * F + r];
                float v;
                if (INT8)
                    v = (float(acc[0]) * tinfo[2 * t]) * s;
                else
                    v = float_value<P>(acc, reinterpret_cast<const int32_t *>(tinfo)[2 * t]) * s;
                sums[job] = v;
            }
        }
        __syncthreads();
        if (threadIdx.x < kDecRowsGU) {
            const int tt = threadIdx.x;
            const float g = sums[tt], u = sums[kDecRowsGU + tt];
            hbuf[int64_t(pair) * F + rb * kDecRowsGU + tt] = tw_silu(g) * u;
        }
        __syncthreads();
    }
}

// Down rows of one expert for all its tokens (block = expert, block of 8 rows); h of each pair is
// turned into digit planes in shared memory first (int8 mode: per (token, expert) absmax).
template <int P, bool INT8>
__global__ __launch_bounds__(256) void k_bat_down(BatchedArgs a, LayerPtrs lp,
                                                  uint8_t *__restrict__ ws)
{
    extern __shared__ __attribute__((aligned(16))) int8_t smem[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int d = a.dm.d, F = a.dm.F;
    const int nrb = d / kDecRowsDown;
    const int e = blockIdx.x / nrb, rb = blockIdx.x % nrb;
    const int32_t *offsets = reinterpret_cast<const int32_t *>(ws + a.L.offsets);
    const int32_t *pairs = reinterpret_cast<const int32_t *>(ws + a.L.pairs);
    const int p0 = offsets[e], p1 = offsets[e + 1];
    if (p0 == p1) return;
    const float *hbuf = reinterpret_cast<const float *>(ws + a.L.h);
    float *ybuf = reinterpret_cast<float *>(ws + a.L.y);
    int8_t *hd = smem;                                          // [P][F]
    float *hs = reinterpret_cast<float *>(smem + P * F);        // [1] scale / shift
    const int lpr = F >> 6, rpp = 64 / lpr;
    const int sub = lane / lpr, c = lane % lpr;
    const int njobs = kDecRowsDown;
    const int64_t rstride = F / 4;
    for (int pi = p0; pi < p1; pi++) {
        const int pair = pairs[pi];
        const float *h = hbuf + int64_t(pair) * F;
        if (wave == 0) {
            float am = 0.0f;
            for (int i = lane; i < F; i += 64) am = fmaxf(am, fabsf(h[i]));
            am = wave_max(am);
            if (INT8) {
                const float inv = am > 0.0f ? 127.0f / am : 0.0f;
                for (int i = lane; i < F; i += 64) hd[perm16(i)] = am > 0.0f ? int8_quant(h[i], inv) : int8_t(0);
                if (lane == 0) hs[0] = am > 0.0f ? am / 127.0f : 0.0f;
            } else {
                const int sh = float_digit_shift(am, P);
                for (int i = lane; i < F; i += 64) {
                    int8_t dg[P];
                    float_digits<P>(h[i], sh, dg);
#pragma unroll
                    for (int p = 0; p < P; p++) hd[p * F + perm16(i)] = dg[p];
                }
                if (lane == 0) reinterpret_cast<int32_t *>(hs)[0] = sh;
            }
        }
        __syncthreads();
        for (int base = wave * rpp; base < njobs; base += 4 * rpp) {
            const int job = base + sub;
            const bool valid = job < njobs;
            const int r = rb * kDecRowsDown + (valid ? job : 0);
            const uint8_t *row = lp.w_down + (int64_t(e) * d + r) * rstride;
            const int4 code = valid ? reinterpret_cast<const int4 *>(row)[c] : make_int4(0, 0, 0, 0);
            int4 dg[P][4];
#pragma unroll
            for (int p = 0; p < P; p++)
#pragma unroll
                for (int q = 0; q < 4; q++) dg[p][q] = reinterpret_cast<const int4 *>(hd + p * F + c * 64)[q];
            int32_t acc[P] = {};
            chunk_dot<P>(code, dg, acc);
            group_reduce<P>(acc, lpr);
            if (c == 0 && valid) {
                const float s = lp.s_down[int64_t(e) * d + r];
                float v;
                if (INT8)
                    v = (float(acc[0]) * hs[0]) * s;
                else
                    v = float_value<P>(acc, reinterpret_cast<const int32_t *>(hs)[0]) * s;
                ybuf[int64_t(pair) * d + r] = v;
            }
        }
        __syncthreads();
    }
}

// out[t] = ((x[t] + g_0 y_0) + g_1 y_1) + ..., j in selection order.  Slots whose expert id is
// outside [0, E) contribute nothing (k_group does not place them either).
__global__ __launch_bounds__(256) void k_bat_combine(BatchedArgs a, const void *__restrict__ x,
                                                     int x_bf16, void *__restrict__ out,
                                                     int out_bf16, const int32_t *__restrict__ ids,
                                                     const float *__restrict__ gates,
                                                     uint8_t *__restrict__ ws)
{
    const int d = a.dm.d, k = a.dm.k, E = a.dm.E;
    const int64_t n = a.T * d;
    const float *ybuf = reinterpret_cast<const float *>(ws + a.L.y);
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * blockDim.x) {
        const int64_t t = i / d;
        const int r = int(i % d);
        float o = load_act(x, i, x_bf16);
        for (int j = 0; j < k; j++) {
            const int id = ids[t * k + j];
            if (id < 0 || id >= E) continue;
            const float c = gates[t * k + j] * ybuf[(t * k + j) * d + r];
            o = o + c;
        }
        store_act(out, i, o, out_bf16);
    }
}

inline hipStream_t S(void *s) { return static_cast<hipStream_t>(s); }

int last_error() { return int(hipGetLastError()); }

template <int P>
int decode_p(const Dims &dm, const LayerPtrs *layers, int n, const void *x_in, void *x_out,
             int io_bf16, void *ws, void *stream)
{
    DecodeArgs a{dm, decode_ws_layout(dm), io_bf16};
    uint8_t *w = static_cast<uint8_t *>(ws);
    const size_t eb = io_bf16 ? 2 : 4;
    void *buf[2] = {w + a.L.xbuf, w + a.L.xbuf + size_t(dm.d) * eb};
    k_zero_u32<<<1, 64, 0, S(stream)>>>(reinterpret_cast<uint32_t *>(w + a.L.ctrl), 64);
    const size_t smem_down = size_t(dm.k) * P * dm.F + sizeof(int) * kMaxTopK +
                             sizeof(float) * dm.k * kDecRowsDown;
    for (int l = 0; l < n; l++) {
        const void *src = l == 0 ? x_in : buf[(l - 1) & 1];
        void *dst = l == n - 1 ? x_out : buf[l & 1];
        k_dec_route<P><<<(dm.E + 3) / 4, 256, 0, S(stream)>>>(a, layers[l].w_router, src, w);
        k_dec_gateup<P><<<dm.k * (dm.F / kDecRowsGU), 256, 0, S(stream)>>>(a, layers[l], w);
        k_dec_down<P><<<dm.d / kDecRowsDown, 256, smem_down, S(stream)>>>(a, layers[l], src, dst, w);
    }
    return last_error();
}

template <int P, bool INT8>
int batched_p(const Dims &dm, const LayerPtrs &lp, int64_t T, const void *x_in, int in_bf16,
              void *x_out, int out_bf16, const int32_t *ids, const float *gates, void *ws,
              void *stream)
{
    BatchedArgs a{dm, batched_ws_layout(dm, T, INT8 ? 1 : 3), T, INT8};
    uint8_t *w = static_cast<uint8_t *>(ws);
    if (!ids) {
        float *logits = reinterpret_cast<float *>(w + a.L.logits);
        int32_t *wid = reinterpret_cast<int32_t *>(w + a.L.ids);
        float *wg = reinterpret_cast<float *>(w + a.L.gates);
        const int64_t waves = T * dm.E;
        k_router_logits<<<unsigned((waves + 3) / 4), 256, 0, S(stream)>>>(
            x_in, in_bf16, lp.w_router, dm.router_bf16, T, dm.d, dm.E, dm.pre_norm, logits);
        k_topk<<<unsigned((T + 3) / 4), 256, 0, S(stream)>>>(logits, T, dm.E, dm.k, wid, wg);
        ids = wid;
        gates = wg;
    }
    k_bat_quant_x<P, INT8><<<unsigned(T), 64, 0, S(stream)>>>(a, x_in, in_bf16, w);
    k_group<<<1, 1024, 0, S(stream)>>>(a, ids, w);
    k_bat_gateup<P, INT8><<<dm.E * (dm.F / kDecRowsGU), 256, 0, S(stream)>>>(a, lp, w);
    const size_t smem_down = size_t(P) * dm.F + 16;
    k_bat_down<P, INT8><<<dm.E * (dm.d / kDecRowsDown), 256, smem_down, S(stream)>>>(a, lp, w);
    const int64_t n = T * dm.d;
    const unsigned nb = unsigned(n / 256 + 1 < 65536 ? n / 256 + 1 : 65536);
    k_bat_combine<<<nb, 256, 0, S(stream)>>>(a, x_in, in_bf16, x_out, out_bf16, ids, gates, w);
    return last_error();
}

}  // namespace

int launch_pack(const int8_t *w, int64_t rows, int64_t cols, uint8_t *packed, int32_t *bad,
                void *stream)
{
    const int64_t n = rows * ((cols + 3) / 4);
    if (cols % 16 == 0 && (uintptr_t(w) & 15) == 0 && (uintptr_t(packed) & 3) == 0) {
        const int64_t n16 = rows * cols / 16;
        const unsigned nb = unsigned(n16 / 256 + 1 < 16384 ? n16 / 256 + 1 : 16384);
        k_pack16<<<nb, 256, 0, S(stream)>>>(reinterpret_cast<const int4 *>(w), n16,
                                             reinterpret_cast<uint32_t *>(packed), bad);
    } else {
        const unsigned nb = unsigned(n / 256 + 1 < 16384 ? n / 256 + 1 : 16384);
        k_pack_any<<<nb, 256, 0, S(stream)>>>(w, rows, cols, packed, bad);
    }
    return last_error();
}

int launch_route(const void *x, int x_bf16, const void *w_router, int w_bf16, int64_t T,
                 const Dims &dm, float *logits, int32_t *ids, float *gates, void *stream)
{
    const int64_t waves = T * dm.E;
    k_router_logits<<<unsigned((waves + 3) / 4), 256, 0, S(stream)>>>(
        x, x_bf16, w_router, w_bf16, T, dm.d, dm.E, dm.pre_norm, logits);
    k_topk<<<unsigned((T + 3) / 4), 256, 0, S(stream)>>>(logits, T, dm.E, dm.k, ids, gates);
    return last_error();
}

int launch_decode(const Dims &dm, const LayerPtrs *layers, int n_layers, const void *x_in,
                  void *x_out, int io_bf16, void *ws, void *stream)
{
    if (io_bf16) return decode_p<2>(dm, layers, n_layers, x_in, x_out, io_bf16, ws, stream);
    return decode_p<3>(dm, layers, n_layers, x_in, x_out, io_bf16, ws, stream);
}

int launch_batched(const Dims &dm, const LayerPtrs &layer, int64_t T, const void *x_in,
                   int in_bf16, void *x_out, int out_bf16, int int8_act, const int32_t *ids,
                   const float *gates, void *ws, void *stream)
{
    if (int8_act)
        return batched_p<1, true>(dm, layer, T, x_in, in_bf16, x_out, out_bf16, ids, gates, ws,
                                  stream);
    if (in_bf16)
        return batched_p<2, false>(dm, layer, T, x_in, in_bf16, x_out, out_bf16, ids, gates, ws,
                                   stream);
    return batched_p<3, false>(dm, layer, T, x_in, in_bf16, x_out, out_bf16, ids, gates, ws,
                               stream);
}

}  // namespace tw
