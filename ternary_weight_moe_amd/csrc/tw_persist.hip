// tw_persist.hip -- batch-1 decode through a stack of layers in ONE launch (gfx950, bf16 I/O).
//
// Why one launch.  A decode step is latency-bound: each layer is a chain of all-to-all
// dependencies (residual -> router logits -> top-k -> gate/up rows -> h -> down rows -> residual),
// and a kernel boundary inside a hipGraph costs about 1.5 us on MI355X, three per layer.  Here
// 256 workgroups of 1024 threads (one per compute unit) stay resident for the whole stack and hand each other the
// three small vectors of every layer through tagged 64-bit words (tw_device.h): each word is one
// device-scope atomic store of (tag, data) and is read by polling, so a hand-off costs one memory
// round trip and needs no grid barrier, no fence and no atomic read-modify-write.  Every word is
// stored into eight copies and each workgroup polls the copy of its own XCD (hardware register
// XCC_ID), which spreads the polls of the 256 workgroups over eight sets of lines; any copy holds
// the same values, so which one a workgroup reads never changes a result.
//
// Per layer, workgroup b (of 256) does:
//   1. input   x: layer 0 reads x_in; later layers gather the d/2 words of packed bf16 pairs that
//              the previous layer published (every workgroup needs all of x): each router wave
//              polls the 256 words of its lanes' 8-element chunks and passes them on through LDS.
//   2. router  the workgroup computes the logits of experts b + 256 m (router rows prefetched
//              during the previous layer, one 16-byte chunk per thread) and publishes them; the
//              pre-RMSNorm is a scalar on the logits and on the gate/up sums.
//   3. top-k   in every workgroup one wave gathers all E logits into registers and selects the
//              same top-k (same values, same deterministic selection), so nothing else has to be
//              broadcast.
//   4. loads   the workgroup's share of gate/up rows (2 x k*F/256 rows of d/4 bytes, ~4 MB
//              across the chip for the 2048/512/top-8 layer) is requested at once, with its scales;
//              the gates are formed while it is in flight.  Once it has arrived, the share of down
//              rows (k experts x d/256 output rows of F/4 bytes) is requested: it is needed only
//              after the h hand-off, and keeping it out of the first burst lets the gate/up bytes,
//              which are on the critical path, arrive sooner.  The next layer's router row is
//              requested after the combine, once the down rows are in.
//   5. gate/up the ternary dots (tw_device.h) against the digit planes of x, h = SiLU(gate)*up
//              in fp32, published one value per word.
//   6. down    wave j gathers the F values of expert j's h, takes their max, writes the digit
//              planes to its own LDS region and computes expert j's down rows of the workgroup's
//              outputs (no workgroup barrier until the combine); then out = x + sum_j g_j y_j in
//              selection order, rounded to bf16 and published (or stored to x_out after the last
//              layer).
// Tags are the layer index + 1 and the words alternate between two parities by layer, so a word
// is never overwritten while a reader may still need its previous value (a workgroup can be at
// most one hand-off ahead of any other).  A small kernel zeroes the words before each launch.
//
// Every wait is bounded: a wait that exceeds the spin limit marks the workgroup aborted (its
// remaining waits return at once) and sets a word in the workspace error slot, so the launch
// always ends.  The arithmetic is that of the per-layer kernels (same digit planes, same canonical
// router order, same rounding points), so results equal a chain of single-layer calls bit for bit.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "tw_device.h"
#include "tw_internal.h"

// A measurement build (-DTW_PHASE_TIMES, made by phase_times.py) stores the 100 MHz wall clock at
// the phase boundaries of every layer from thread 0 of every workgroup into the workspace, for a
// per-layer time breakdown; the product build compiles these stores out.
#ifdef TW_PHASE_TIMES
#define TW_STAMP(P) \
    if (t == 0 && a.ts) a.ts[(size_t(b) * kMaxPersistLayers + l) * kPhaseStamps + (P)] = wall_clock64()
#else
#define TW_STAMP(P) ((void)0)
#endif

namespace tw {
namespace {

constexpr int kPB = 256;               // workgroups of a launch (one per compute unit)
constexpr int kPT = 1024;              // threads per workgroup (16 waves)
constexpr int kNW = kPT / 64;          // waves per workgroup
constexpr int kCT = 256;               // threads of the canonical router order (4 waves)
constexpr uint32_t kSpinLimit = 1u << 21;
// Waits before the first poll of a hand-off, in s_sleep units (64 clocks, ~27 ns): the words cannot
// arrive sooner than about a memory round trip after the slowest producer, and early polls from
// every workgroup only add traffic to the memory system that the producers' stores and the expert
// rows go through.  Measured on MI355X (24-layer stack, tokens/s): no waits 252.6 us per token;
// 20 before the h words 232.6 (15: 234.8, 25: 234.0, 40: 243.9); and 10 before the residual words
// 220.3 (5: 223.0, 15: 222.5, 20: 224.7); a wait before the logits or between polls adds nothing.
constexpr int kSleepX = 10;            // before polling the residual words
constexpr int kSleepH = 20;            // before polling the h words
constexpr int kEM = 1;                 // router rows per workgroup: expert b (E <= 256)

struct PLayer {
    const uint16_t *w_router;
    const uint8_t *w_gate, *w_up, *w_down;
    const float *s_gate, *s_up, *s_down;
};

struct PArgs {
    const uint16_t *x_in;
    uint16_t *x_out;
    uint64_t *ll;      // tagged words (2 parities)
    uint32_t *err;     // error slot: nonzero after a wait timed out
    uint64_t *ts;      // phase timestamps (measurement build only)
    int E, n_layers, pre_norm;
    int cont;          // 1: a later launch of one call (reads the health word first)
    PLayer L[kMaxPersistLayers];
};

template <int D, int F, int K>
struct PC {
    static constexpr int Q = K * F / kPB;                    // h rows per workgroup
    static constexpr int LPR = D / 64;                       // lanes per gate/up row (16 B each)
    static constexpr int RPP = kPT / LPR;                    // gate/up rows per pass
    static constexpr int PGU = (2 * Q + RPP - 1) / RPP;      // gate/up passes
    static constexpr int RD = D / kPB;                       // output rows per workgroup
    static constexpr int LPRD = F / 64;                      // lanes per down row
    static constexpr int DL = RD * LPRD;                     // lanes of an expert's down rows
    static constexpr int XW = D / 2;                         // residual words (bf16 pairs)
    static constexpr int HW = K * F;                         // h words (fp32)
    static constexpr int NRC = (D / 8 + kCT - 1) / kCT;      // 8-element chunks per router thread
    static_assert(Q >= 1, "k*F must be a multiple of 256");
    static_assert(RD >= 2 && RD % 2 == 0, "d must be a multiple of 512");
    static_assert(LPR >= 1 && LPR <= 64 && LPRD >= 1 && LPRD <= 64, "row widths 64..4096");
    static_assert(K <= kMaxTopK && K <= 16, "top-k");
    static_assert(HW % kPT == 0 && HW <= 4 * kPT && F % 256 == 0, "k*F in {1024, 2048, 3072, 4096}");
    static_assert(DL <= 64 && K <= kPT / 64, "wave j takes expert j's down rows");
    static_assert(2 * Q <= 64, "one wave loads the scales of the workgroup's gate/up rows");
    static_assert(NRC == 1 && D / 8 % 64 == 0, "router wave w holds chunks 64w .. 64w + 63, words 256w ..");
    static_assert(XW % 64 == 0 && D % kPT == 0, "d a multiple of 1024");
};

// Waits until the words base[first + stride*n] (n < N, index < W) carry `tag`; v receives them.  Words
// that never arrive end the wait after kSpinLimit polls and mark the workgroup aborted; after that
// the workgroup's later waits return at once (the flag is read once per wait, not per poll: a
// per-poll read of it would also wait for every memory read in flight).
template <int N>
__device__ __forceinline__ void wait_words(const uint64_t *base, int first, int stride, int W, uint32_t tag,
                                           uint64_t (&v)[N], volatile int *s_abort, uint32_t *err)
{
    uint32_t pend = 0;
#pragma unroll
    for (int n = 0; n < N; n++)
        if (first + stride * n < W) pend |= 1u << n;
    if (*s_abort) return;
    for (uint32_t it = 0; pend; ++it) {
#pragma unroll
        for (int n = 0; n < N; n++)
            if ((pend >> n) & 1u) v[n] = ld_tagged(base + first + stride * n);
#pragma unroll
        for (int n = 0; n < N; n++)
            if (((pend >> n) & 1u) && uint32_t(v[n] >> 32) == tag) pend &= ~(1u << n);
        if (pend && it > kSpinLimit) {
            *s_abort = 1;
            atomicOr(err, 1u);
            break;
        }
    }
}

// Router rows of the experts b + kPB*m (m < kEM) of this workgroup: router thread t (< kCT)
// holds the 16-byte chunks t + kCT*n (8 bf16 each) of each row.
template <int NRC>
__device__ __forceinline__ void load_router(int4 (&rw)[kEM][NRC], const uint16_t *wr, int b, int E,
                                            int d)
{
#pragma unroll
    for (int m = 0; m < kEM; m++)
#pragma unroll
        for (int n = 0; n < NRC; n++) {
            const int c = threadIdx.x + kCT * n, e = b + kPB * m;
            rw[m][n] = (threadIdx.x < kCT && e < E && c < (d >> 3))
                           ? reinterpret_cast<const int4 *>(wr + size_t(e) * d)[c]
                           : make_int4(0, 0, 0, 0);
        }
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return bf16_to_f32(uint16_t(w & 0xffffu)); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return bf16_to_f32(uint16_t(w >> 16)); }

template <int D, int F, int K>
__global__ __launch_bounds__(kPT) void k_persist(PArgs a)
{
    using C = PC<D, F, K>;
    const int b = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int E = a.E;
    __shared__ __attribute__((aligned(16))) float xs[D];         // layer input x
    __shared__ __attribute__((aligned(16))) int8_t xd[2 * D];    // its digit planes
    __shared__ __attribute__((aligned(16))) int8_t hd[K * 2 * F];// digit planes of h, per expert
    __shared__ float sums[2 * C::Q];
    __shared__ float s_scl[2 * C::Q];   // scales of the workgroup's gate/up rows
    __shared__ float ys[K * C::RD];
    __shared__ float red[4][2 + kEM];
    __shared__ __attribute__((aligned(16))) float hs[C::HW];     // h, in digit-plane byte order
    __shared__ int32_t s_ids[kMaxTopK];
    __shared__ float s_gates[kMaxTopK];
    __shared__ int s_xsh;
    __shared__ float s_inv;
    __shared__ int s_abort;
    // a launch that continues a call (more layers than one launch holds) starts aborted if a wait
    // of an earlier launch ran out: its input is undefined, and the health word already reports it
    // (the first launch of a call does not read the word: it was just cleared)
    if (t == 0) s_abort = a.cont ? *reinterpret_cast<volatile uint32_t *>(a.err) != 0u : 0;

    int4 rw[kEM][C::NRC];
    load_router<C::NRC>(rw, a.L[0].w_router, b, E, D);
    const size_t lls = size_t(E) * kLgStride + C::HW + C::XW;   // words of one copy
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    const size_t own = size_t(xcc & uint32_t(kLlCopies - 1)) * lls;   // the copy this workgroup polls
    const int c_gu = t % C::LPR, c_d = t % C::LPRD;
    __syncthreads();

    for (int l = 0; l < a.n_layers; l++) {
        const PLayer &P = a.L[l];
        const uint32_t tag = uint32_t(l + 1);
        TW_STAMP(0);
        // copy 0 of this layer's parity (stores go to every copy) and the copy read here
        uint64_t *set0 = a.ll + size_t(l & 1) * kLlCopies * lls;
        const uint64_t *lgw = set0 + own, *hw = lgw + E * kLgStride;

        // 1. layer input: layer 0 reads x_in into LDS; later layers are read by the router threads
        //    below, each polling the four words (bf16 pairs) of its own 8-element chunks
        const uint64_t *xprev = a.ll + size_t((l + 1) & 1) * kLlCopies * lls + own + E * kLgStride + C::HW;   // layer l - 1's
        if (l == 0) {
            for (int i = t; i < D; i += kPT) xs[i] = bf16_to_f32(a.x_in[i]);
            __syncthreads();
        }

        // 2. router threads: their 8-element chunks of x (amax, sum of squares, router partials in
        //    the canonical order; from layer 1 on from the polled words, which their wave stores
        //    to LDS, where the digit planes and the combine also read them), wave reductions, then
        //    block totals, logits and digit planes
        if (t < kCT) {
            float am = 0.0f, ss = 0.0f, rp[kEM];
#pragma unroll
            for (int m = 0; m < kEM; m++) rp[m] = 0.0f;
#pragma unroll
            for (int n = 0; n < C::NRC; n++) {
                const int c = t + kCT * n;
                if (c < (D >> 3)) {
                    float xv[8];
                    if (l == 0) {
#pragma unroll
                        for (int j = 0; j < 8; j++) xv[j] = xs[8 * c + j];
                    } else {
                        // router wave w polls the words 256 w + lane + 64 q (q < 4), 4 lines an
                        // instruction, the words its lanes' chunks are made of; they reach the
                        // lanes through LDS, inside the wave (its LDS accesses take effect in
                        // order).  Polling each lane's own 4 words (16 lines an instruction)
                        // took 190.0 us per token, this 187.6
                        uint64_t v[4] = {0, 0, 0, 0};
                        if (n == 0) __builtin_amdgcn_s_sleep(kSleepX);
                        const int w0 = 256 * (t >> 6) + (t & 63);
                        wait_words<4>(xprev, w0, 64, C::XW, tag - 1, v, &s_abort, a.err);
#pragma unroll
                        for (int q = 0; q < 4; q++) {
                            const int k = w0 + 64 * q;
                            if (k < C::XW)
                                *reinterpret_cast<float2 *>(xs + 2 * k) =
                                    make_float2(bf16_lo(uint32_t(v[q])), bf16_hi(uint32_t(v[q])));
                        }
                        const float4 a0 = *reinterpret_cast<const float4 *>(xs + 8 * c);
                        const float4 a1 = *reinterpret_cast<const float4 *>(xs + 8 * c + 4);
                        xv[0] = a0.x; xv[1] = a0.y; xv[2] = a0.z; xv[3] = a0.w;
                        xv[4] = a1.x; xv[5] = a1.y; xv[6] = a1.z; xv[7] = a1.w;
                    }
#pragma unroll
                    for (int j = 0; j < 8; j++) {
                        am = fmaxf(am, fabsf(xv[j]));
                        ss = ss + xv[j] * xv[j];
                    }
#pragma unroll
                    for (int m = 0; m < kEM; m++) {
                        const uint32_t w4[4] = {uint32_t(rw[m][n].x), uint32_t(rw[m][n].y),
                                                uint32_t(rw[m][n].z), uint32_t(rw[m][n].w)};
#pragma unroll
                        for (int j = 0; j < 8; j++) {
                            const float wv = (j & 1) ? bf16_hi(w4[j >> 1]) : bf16_lo(w4[j >> 1]);
                            rp[m] = rp[m] + wv * xv[j];
                        }
                    }
                }
            }
            am = wave_max(am);
            ss = wave_sum(ss);
#pragma unroll
            for (int m = 0; m < kEM; m++) rp[m] = wave_sum(rp[m]);
            if (lane == 0) {
                red[wave][0] = am;
                red[wave][1] = ss;
#pragma unroll
                for (int m = 0; m < kEM; m++) red[wave][2 + m] = rp[m];
            }
        }
        __syncthreads();
        TW_STAMP(1);
        {
            const float am = fmaxf(fmaxf(red[0][0], red[1][0]), fmaxf(red[2][0], red[3][0]));
            const float ss = (red[0][1] + red[1][1]) + (red[2][1] + red[3][1]);
            const float inv = a.pre_norm ? inv_rms_of(ss, D) : 1.0f;
            const int sh = float_digit_shift(am, 2);
            if (t < kEM * kLlCopies && b + kPB * (t / kLlCopies) < E) {   // thread t: copy t % kLlCopies
                const int m = t / kLlCopies;
                float lgt = (red[0][2 + m] + red[1][2 + m]) + (red[2][2 + m] + red[3][2 + m]);
                if (a.pre_norm) lgt = lgt * inv;
                st_tagged(set0 + (t % kLlCopies) * lls + (b + kPB * m) * kLgStride, tag, __float_as_uint(lgt));
            }
            if (t == 0) {
                s_xsh = sh;
                s_inv = inv;
            }
            if (t < D / 4) {   // dword t % 4 of 16-element group t / 4 of both planes
                const int o = 16 * (t >> 2) + (t & 3);
                uint32_t pr[4], lo, hi;
#pragma unroll
                for (int r = 0; r < 4; r++) pr[r] = float_digit_pair(xs[o + 4 * r], sh);
                digit_pair_dwords(pr, lo, hi);
                *reinterpret_cast<uint32_t *>(xd + 4 * t) = hi;        // plane 0: high digits
                *reinterpret_cast<uint32_t *>(xd + D + 4 * t) = lo;
            }
        }

        // 3. routing: in every workgroup wave 0 gathers all E logits (lane l: experts l + 64 s) into
        //    registers and selects the same experts
        if (wave == 0) {
            constexpr int S = kPB / 64;
            uint64_t v[S];
            float lv[S];
#pragma unroll
            for (int q = 0; q < S; q++) v[q] = 0;
            wait_words<S>(lgw, lane * kLgStride, 64 * kLgStride, E * kLgStride, tag, v, &s_abort, a.err);
#pragma unroll
            for (int q = 0; q < S; q++) lv[q] = __uint_as_float(uint32_t(v[q]));
            TW_STAMP(7);
            if (!topk_wave_composite_to<S>(lv, E, K, s_ids, s_gates, lane))
                topk_softmax_wave_regs<S, false>(lv, E, K, s_ids, s_gates, lane);
            TW_STAMP(8);
        }
        __syncthreads();
        TW_STAMP(2);

        // 4. request the gate/up rows of this workgroup's share at once (the down rows follow once
        //    these have arrived and the next router rows after the combine, so that these, on the
        //    critical path, do not share the memory system with them); the gates are formed
        //    meanwhile.  The rows'
        //    scales (two 64-byte runs) come in one instruction of wave 0, not one per wave and row:
        //    a compute unit keeps only so many lines in flight, and the code rows need them (with
        //    a load per wave and row the token took 199.5 us, with one 193.9 us)
        int4 cg[C::PGU];
#pragma unroll
        for (int p = 0; p < C::PGU; p++) {
            const int jb = p * C::RPP + t / C::LPR;
            const bool valid = jb < 2 * C::Q;
            const int i = valid ? (jb >> 1) : 0, kind = jb & 1;
            const int q = b * C::Q + i, j = q / F, r = q % F;
            const int e = min(max(s_ids[j], 0), E - 1);
            const uint8_t *row = (kind ? P.w_up : P.w_gate) + (size_t(e) * F + r) * (D / 4);
            cg[p] = valid ? reinterpret_cast<const int4 *>(row)[c_gu] : make_int4(0, 0, 0, 0);
        }
        float scl = 0.0f;   // wave 0, lane jb < 2Q: the scale of gate/up row jb (jb odd: up)
        if (wave == 0 && lane < 2 * C::Q) {
            const int i = lane >> 1, kind = lane & 1;
            const int q = b * C::Q + i, j = q / F, r = q % F;
            const int e = min(max(s_ids[j], 0), E - 1);
            scl = (kind ? P.s_up : P.s_gate)[size_t(e) * F + r];
        }
        if (wave == 0) softmax_gates_wave(s_gates, K, lane);

        // 5. gate/up dots, h = SiLU(gate) * up in fp32, published one value per word
        int4 cd;   // wave j < k: row lane / (F/64) of expert j's down rows, 64 columns
        float sd;
        {
            int4 dg[2][4];
#pragma unroll
            for (int pl = 0; pl < 2; pl++)
#pragma unroll
                for (int qq = 0; qq < 4; qq++)
                    dg[pl][qq] = reinterpret_cast<const int4 *>(xd + pl * D + c_gu * 64)[qq];
#pragma unroll
            for (int p = 0; p < C::PGU; p++) {
                const int jb = p * C::RPP + t / C::LPR;
                int32_t acc[2] = {0, 0};
                chunk_dot<2>(cg[p], dg, acc);
                group_reduce<2>(acc, C::LPR);
                if (c_gu == 0 && jb < 2 * C::Q) sums[jb] = float_value<2>(acc, s_xsh);
            }
            if (wave == 0 && lane < 2 * C::Q) s_scl[lane] = scl;
            // the down rows of this workgroup's outputs (wave j: expert j)
            {
                const bool valid = wave < K && lane < C::DL;
                const int j = valid ? wave : 0, rl = lane / C::LPRD;
                const int R = b * C::RD + (valid ? rl : 0);
                const int e = min(max(s_ids[j], 0), E - 1);
                const uint8_t *row = P.w_down + (size_t(e) * D + R) * (F / 4);
                cd = valid ? reinterpret_cast<const int4 *>(row)[c_d] : make_int4(0, 0, 0, 0);
                sd = (valid && c_d == 0) ? P.s_down[size_t(e) * D + R] : 0.0f;
            }
        }
        __syncthreads();
        TW_STAMP(3);
        if (t < C::Q * kLlCopies) {   // thread t: value t % Q into copy t / Q
            const int i = t % C::Q;
            // (sum * scale) * inverse RMS, as the other kernels form a gate or up value
            const float gv = sums[2 * i] * s_scl[2 * i] * s_inv;
            const float uv = sums[2 * i + 1] * s_scl[2 * i + 1] * s_inv;
            const float h = tw_silu(gv) * uv;
            st_tagged(set0 + (t / C::Q) * lls + E * kLgStride + b * C::Q + i, tag, __float_as_uint(h));
        }

        // 6. wave j (< k) gathers the F words of expert j's h itself (lane l: elements l + 64 m),
        //    takes the expert's max |h| with one wave reduction, stores h in the digit-plane byte
        //    order to its own LDS region and turns it into both digit planes (four elements of a
        //    dword at a time), then computes expert j's down rows of this workgroup's outputs: no
        //    workgroup barrier until the combine, and an expert goes ahead as soon as its h is
        //    complete (the LDS accesses of one wave take effect in order)
        if (wave < K) {
            constexpr int M = F / 64;
            const int j = wave;
            float *hsj = hs + j * F;
            uint64_t v[M];
#pragma unroll
            for (int m = 0; m < M; m++) v[m] = 0;
            // the wave's down rows are in before it starts to poll: its polls (32 lines a round)
            // would otherwise share the compute unit's lines in flight with them (a token took
            // 192.0 us polling at once after the wait below, 189.2 us waiting for the rows first)
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_sleep(kSleepH);
            wait_words<M>(hw + j * F, lane, 64, F, tag, v, &s_abort, a.err);
            TW_STAMP(4);
            float am = 0.0f;
#pragma unroll
            for (int m = 0; m < M; m++) {
                const float h = __uint_as_float(uint32_t(v[m]));
                hsj[perm16(lane + 64 * m)] = h;
                am = fmaxf(am, fabsf(h));
            }
            const int sh = float_digit_shift(wave_max(am), 2);
#pragma unroll
            for (int u = 0; u < F / 256; u++) {   // dword q of both planes: elements 4q .. 4q + 3
                const int q = lane + 64 * u;
                const float4 hv = *reinterpret_cast<const float4 *>(hsj + 4 * q);
                const uint32_t pr[4] = {float_digit_pair(hv.x, sh), float_digit_pair(hv.y, sh),
                                        float_digit_pair(hv.z, sh), float_digit_pair(hv.w, sh)};
                uint32_t lo, hi;
                digit_pair_dwords(pr, lo, hi);
                *reinterpret_cast<uint32_t *>(hd + (j * 2) * F + 4 * q) = hi;   // plane 0: high
                *reinterpret_cast<uint32_t *>(hd + (j * 2 + 1) * F + 4 * q) = lo;
            }
            int4 dh[2][4];
#pragma unroll
            for (int pl = 0; pl < 2; pl++)
#pragma unroll
                for (int qq = 0; qq < 4; qq++)
                    dh[pl][qq] = reinterpret_cast<const int4 *>(hd + (j * 2 + pl) * F + c_d * 64)[qq];
            int32_t acc[2] = {0, 0};
            chunk_dot<2>(cd, dh, acc);
            group_reduce<2>(acc, C::LPRD);
            if (c_d == 0 && lane < C::DL) ys[j * C::RD + lane / C::LPRD] = float_value<2>(acc, sh) * sd;
        }
        __syncthreads();
        TW_STAMP(5);
        if (t < (C::RD / 2) * kLlCopies) {   // thread t: row pair t % (RD/2) into copy t / (RD/2)
            const int i = t % (C::RD / 2), c = t / (C::RD / 2);
            const int R0 = b * C::RD + 2 * i;
            float o0 = xs[R0], o1 = xs[R0 + 1];
            for (int j = 0; j < K; j++) {
                o0 = o0 + s_gates[j] * ys[j * C::RD + 2 * i];
                o1 = o1 + s_gates[j] * ys[j * C::RD + 2 * i + 1];
            }
            if (l == a.n_layers - 1) {
                if (c == 0) {
                    a.x_out[R0] = f32_to_bf16(o0);
                    a.x_out[R0 + 1] = f32_to_bf16(o1);
                }
            } else {
                st_tagged(set0 + c * lls + E * kLgStride + C::HW + (b * C::RD) / 2 + i, tag, pack_bf16x2(o0, o1));
            }
        }
        // the next layer's router rows, requested once this layer's rows are in: in flight while
        // the residual is gathered (requested with the down rows, a token took 193.6 us; here 192.1)
        if (l + 1 < a.n_layers) load_router<C::NRC>(rw, a.L[l + 1].w_router, b, E, D);
        __syncthreads();
        TW_STAMP(6);
    }
}

// Clears the tagged words before a launch; the health word only before the first launch of a call
// (err == nullptr for the later ones), so that a wait that ran out in an earlier launch stays
// reported.
__global__ void k_persist_zero(uint64_t *ll, int64_t n, uint32_t *err)
{
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * blockDim.x)
        ll[i] = 0;
    if (err && blockIdx.x == 0 && threadIdx.x < 4) err[threadIdx.x] = 0;
}

// Whether all kPB workgroups of an instantiation fit on the current device at once (cached).
template <int D, int F, int K>
bool fits_device()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
    int c = cache[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        int cus = 0, per_cu = 0;
        bool ok = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
                  hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_persist<D, F, K>, kPT, 0) ==
                      hipSuccess &&
                  int64_t(cus) * per_cu >= kPB;
        c = ok ? 1 : -1;
        cache[dev].store(c, std::memory_order_relaxed);
    }
    return c > 0;
}

template <int D, int F, int K>
int persist_run(const Dims &dm, const LayerPtrs *layers, int n, const void *x_in, void *x_out,
                void *ws, void *stream)
{
    for (int i = 0; i < n; i++)   // router rows are read 16 bytes at a time
        if (reinterpret_cast<uintptr_t>(layers[i].w_router) & 15) return -1;
    if (!fits_device<D, F, K>()) return -1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const DecodeWs L = decode_ws_layout(dm);
    uint8_t *w = static_cast<uint8_t *>(ws);
    uint64_t *ll = reinterpret_cast<uint64_t *>(w + L.ll);
    uint32_t *err = reinterpret_cast<uint32_t *>(w + L.err);
    uint16_t *xb[2] = {reinterpret_cast<uint16_t *>(w + L.xbuf),
                       reinterpret_cast<uint16_t *>(w + L.xbuf) + dm.d};
    const int64_t nw = int64_t(persist_words(dm));
    int done = 0, chunk = 0;
    while (done < n) {
        const int m = n - done < kMaxPersistLayers ? n - done : kMaxPersistLayers;
        PArgs a{};
        a.x_in = done == 0 ? static_cast<const uint16_t *>(x_in) : xb[(chunk - 1) & 1];
        a.x_out = done + m == n ? static_cast<uint16_t *>(x_out) : xb[chunk & 1];
        a.ll = ll;
        a.err = err;
        a.ts = L.ts && done == 0 ? reinterpret_cast<uint64_t *>(w + L.ts) : nullptr;   // first launch only
        a.E = dm.E;
        a.n_layers = m;
        a.pre_norm = dm.pre_norm;
        a.cont = chunk > 0;
        for (int i = 0; i < m; i++) {
            const LayerPtrs &p = layers[done + i];
            a.L[i] = PLayer{static_cast<const uint16_t *>(p.w_router), p.w_gate, p.w_up, p.w_down,
                            p.s_gate, p.s_up, p.s_down};
        }
        k_persist_zero<<<int((nw + 2047) / 2048), 256, 0, s>>>(ll, nw, chunk == 0 ? err : nullptr);
        k_persist<D, F, K><<<kPB, kPT, 0, s>>>(a);
        done += m;
        chunk++;
    }
    return int(hipGetLastError());
}

}  // namespace

int launch_decode_persist(const Dims &dm, const LayerPtrs *layers, int n_layers, const void *x_in,
                          void *x_out, int io_bf16, void *ws, void *stream)
{
    if (!io_bf16 || !dm.router_bf16 || dm.E > kPB || dm.E < dm.k) return -1;
    if (dm.d == 2048 && dm.F == 512 && dm.k == 8)
        return persist_run<2048, 512, 8>(dm, layers, n_layers, x_in, x_out, ws, stream);
    if (dm.d == 1024 && dm.F == 256 && dm.k == 4)
        return persist_run<1024, 256, 4>(dm, layers, n_layers, x_in, x_out, ws, stream);
    return -1;
}

}  // namespace tw
