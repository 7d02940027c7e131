// tw_kernels.hip -- HIP kernels for the ternary MoE FFN on gfx950 (MI355X), and their launchers:
// packing, routing, the per-layer batch-1 decode kernels and the expert-grouped batched path.
// The ternary dot product and the activation digit planes are described in tw_device.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tw_device.h"
#include "tw_internal.h"

namespace tw {
namespace {

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
    auto xv = [&](int i) { return load_act(x, xo + i, x_bf16); };
    float acc = canon_dot(d, lane, [&](int i) { return load_act(wr, int64_t(e) * d + i, w_bf16); }, xv);
    if (pre_norm) acc = acc * inv_rms_of(canon_dot(d, lane, xv, xv), d);
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
    auto xv = [&](int i) { return load_act(x, i, a.io_bf16); };
    const float inv_rms = a.dm.pre_norm ? inv_rms_of(canon_dot(d, lane, xv, xv), d) : 1.0f;
    const int e = blockIdx.x * 4 + wave;
    if (e < E) {
        float acc = canon_dot(d, lane, [&](int i) { return load_act(wr, int64_t(e) * d + i, a.dm.router_bf16); }, xv);
        if (a.dm.pre_norm) acc = acc * inv_rms;
        if (lane == 0) logits[e] = acc;
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
        auto xv = [&](int i) { return load_act(x, xo + i, x_bf16); };
        const float inv = a.dm.pre_norm ? inv_rms_of(canon_dot(d, lane, xv, xv), d) : 1.0f;
        if (lane == 0) {
            reinterpret_cast<int32_t *>(ti)[0] = sh;
            ti[1] = inv;
        }
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
                    v = float_value<P>(acc, reinterpret_cast<const int32_t *>(tinfo)[2 * t]) * s *
                        tinfo[2 * t + 1];
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
    const int r = launch_decode_persist(dm, layers, n_layers, x_in, x_out, io_bf16, ws, stream);
    if (r >= 0) return r;
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
