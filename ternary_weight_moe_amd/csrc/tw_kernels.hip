// tw_kernels.hip -- HIP kernels for the ternary MoE FFN on gfx950 (MI355X), and their launchers:
// packing, routing, the per-layer batch-1 decode kernels and the expert-grouped batched path.
// The ternary dot product and the activation digit planes are described in tw_device.h.
#include <hip/hip_runtime.h>

#include <atomic>
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
// ternary_quantize: one wave per row.  Lane l holds the partial sums l + 64 m (m < 4) of |w| in the
// canonical order of canon_dot (chunks l + 64 m, + 256, ... in order, then wave_sum per m and
// (s_0 + s_1) + (s_2 + s_3)), so the row's absmean, and with it every code, is the same in every
// call.  Rows of at most 256 chunks keep their chunks in registers between the sum and the codes;
// longer rows read them again.  Each chunk of 8 weights becomes two bytes of codes.
template <bool BF16>
__device__ __forceinline__ void quant_chunk(const void *row, int c, float (&v)[8])
{
    if (BF16) {
        const int4 q = reinterpret_cast<const int4 *>(row)[c];
        const uint32_t w[4] = {uint32_t(q.x), uint32_t(q.y), uint32_t(q.z), uint32_t(q.w)};
#pragma unroll
        for (int j = 0; j < 8; j++) v[j] = bf16_to_f32(uint16_t(w[j >> 1] >> (16 * (j & 1))));
    } else {
        const float4 *p = reinterpret_cast<const float4 *>(row) + 2 * c;
        const float4 a = p[0], b = p[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
}

// Codes of 8 weights: clamp(rint(w / g), -1, 1) with w / g one rounded fp32 division.  For g of at
// least 2^-125 (so that g / 2 is exact) that is a comparison with g / 2: if g / 2 = M 2^e (M a
// 24-bit integer), the next fp32 value above it, (M + 1) 2^e, gives w / g = 1/2 + 1/(2M) > 1/2 +
// 2^-25, the midpoint between 1/2 and the next fp32 value, so the quotient rounds above 1/2 and
// rint gives 1; w = g / 2 gives exactly 1/2, which rint takes to 0 (ties to even); every w below
// gives a quotient of at most 1/2.  So the code is +1 iff w > g / 2 and -1 iff w < -g / 2, with no
// division.  Smaller g (and g = 0) take the division itself.
__device__ __forceinline__ uint32_t quant_codes8(const float (&v)[8], float g)
{
    uint32_t bits = 0;
    if (g >= 0x1p-125f) {
        const float hg = 0.5f * g;
#pragma unroll
        for (int j = 0; j < 8; j++) bits |= (v[j] > hg ? 1u : (v[j] < -hg ? 2u : 0u)) << (2 * j);
    } else {
#pragma unroll
        for (int j = 0; j < 8; j++) {
            float q = g == 0.0f ? 0.0f : __builtin_rintf(v[j] / g);
            q = fminf(fmaxf(q, -1.0f), 1.0f);
            bits |= (q > 0.0f ? 1u : (q < 0.0f ? 2u : 0u)) << (2 * j);
        }
    }
    return bits;
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_quant_absmean(const void *__restrict__ w, int64_t rows, int cols,
                                                      uint8_t *__restrict__ packed,
                                                      float *__restrict__ scales)
{
    const int lane = threadIdx.x & 63;
    const int nch = cols >> 3;
    const size_t eb = BF16 ? 2 : 4;
    for (int64_t r = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6); r < rows;
         r += int64_t(gridDim.x) * 4) {
        const void *row = static_cast<const uint8_t *>(w) + size_t(r) * cols * eb;
        uint16_t *prow = reinterpret_cast<uint16_t *>(packed + size_t(r) * (cols >> 2));
        float s[4];
        if (nch <= 256) {
            float v[4][8];
#pragma unroll
            for (int m = 0; m < 4; m++) {
                const int c = 64 * m + lane;
                if (c < nch) quant_chunk<BF16>(row, c, v[m]);
            }
#pragma unroll
            for (int m = 0; m < 4; m++) {
                float acc = 0.0f;
                if (64 * m + lane < nch) {
#pragma unroll
                    for (int j = 0; j < 8; j++) acc = acc + fabsf(v[m][j]);
                }
                s[m] = wave_sum(acc);
            }
            const float g = ((s[0] + s[1]) + (s[2] + s[3])) / float(cols);
#pragma unroll
            for (int m = 0; m < 4; m++) {
                const int c = 64 * m + lane;
                if (c < nch) prow[c] = uint16_t(quant_codes8(v[m], g));
            }
            if (lane == 0) scales[r] = g;
        } else {
#pragma unroll
            for (int m = 0; m < 4; m++) {
                float acc = 0.0f;
                for (int c = 64 * m + lane; c < nch; c += 256) {
                    float v[8];
                    quant_chunk<BF16>(row, c, v);
#pragma unroll
                    for (int j = 0; j < 8; j++) acc = acc + fabsf(v[j]);
                }
                s[m] = wave_sum(acc);
            }
            const float g = ((s[0] + s[1]) + (s[2] + s[3])) / float(cols);
            for (int c = lane; c < nch; c += 64) {
                float v[8];
                quant_chunk<BF16>(row, c, v);
                prow[c] = uint16_t(quant_codes8(v, g));
            }
            if (lane == 0) scales[r] = g;
        }
    }
}

// Rows of at most 64 chunks: 16 lanes per row, four rows per wave.  Lane i of a row's 16 holds the
// chunks (= partials; partials beyond the row are 0) i, i + 16, i + 32, i + 48, so that each load
// instruction reads 256 contiguous bytes of the row; the DPP butterfly inside the 16 lanes forms the
// balanced tree over each run of 16 partials and (r0 + r1) + (r2 + r3) finishes the same tree over
// partials 0 .. 63 that wave_sum forms (the other three groups of 64 partials are 0).  With each
// lane holding 4 consecutive chunks instead (every instruction touching all of a row's lines), the
// down matrix of one layer took 132.8 us instead of about 111.
template <bool BF16>
__global__ __launch_bounds__(256) void k_quant_absmean16(const void *__restrict__ w, int64_t rows,
                                                        int cols, uint8_t *__restrict__ packed,
                                                        float *__restrict__ scales)
{
    const int lane = threadIdx.x & 63, li = lane & 15;
    const int nch = cols >> 3;
    const size_t eb = BF16 ? 2 : 4;
    for (int64_t r0 = (int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6)) * 4; r0 < rows;
         r0 += int64_t(gridDim.x) * 16) {
        const int64_t r = r0 + (lane >> 4);
        const bool live = r < rows;
        const void *row = static_cast<const uint8_t *>(w) + size_t(live ? r : 0) * cols * eb;
        float v[4][8], p[4];
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int c = li + 16 * q;
            p[q] = 0.0f;
            if (live && c < nch) {
                quant_chunk<BF16>(row, c, v[q]);
#pragma unroll
                for (int j = 0; j < 8; j++) p[q] = p[q] + fabsf(v[q][j]);
            }
        }
#pragma unroll
        for (int q = 0; q < 4; q++) {   // partials 16q .. 16q + 15, a balanced tree over the lanes
            p[q] = p[q] + dpp_f<kDppXor1>(p[q]);
            p[q] = p[q] + dpp_f<kDppXor2>(p[q]);
            p[q] = p[q] + dpp_f<kDppHalfMirror>(p[q]);
            p[q] = p[q] + dpp_f<kDppMirror>(p[q]);
        }
        const float g = ((p[0] + p[1]) + (p[2] + p[3])) / float(cols);
        if (live) {
            uint16_t *prow = reinterpret_cast<uint16_t *>(packed + size_t(r) * (cols >> 2));
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int c = li + 16 * q;
                if (c < nch) prow[c] = uint16_t(quant_codes8(v[q], g));
            }
            if (li == 0) scales[r] = g;
        }
    }
}

// ------------------------------------------------------------------------------------------------
// Router logits for T tokens (k_route below).  Every logit is summed in the canonical order of
// canon_dot: 256 partials, partial t adding the products of chunks t, t + 256 (8 elements each) in
// order, then a balanced tree over the partials (wave_sum per 64, (w0+w1)+(w2+w3)).  The
// pre-RMSNorm factor comes from the token's sum of squares in the same order, folded in as a
// scalar: W_r (x / rms) = (W_r x) / rms.
constexpr int kRouteTok = 8;   // tokens per workgroup of the router

// The 8 activations of chunk c of row `row` (bf16 or fp32), as fp32.
__device__ __forceinline__ void load_chunk8(const void *x, int64_t row, int d, int c, int bf16, float (&v)[8])
{
    if (bf16) {
        const int4 q = reinterpret_cast<const int4 *>(static_cast<const uint16_t *>(x) + row * d)[c];
        const uint32_t w[4] = {uint32_t(q.x), uint32_t(q.y), uint32_t(q.z), uint32_t(q.w)};
#pragma unroll
        for (int j = 0; j < 8; j++) v[j] = bf16_to_f32(uint16_t(w[j >> 1] >> (16 * (j & 1))));
    } else {
        const int4 *p = reinterpret_cast<const int4 *>(static_cast<const float *>(x) + row * d) + 2 * c;
        const int4 a = p[0], b = p[1];
        v[0] = __int_as_float(a.x); v[1] = __int_as_float(a.y); v[2] = __int_as_float(a.z); v[3] = __int_as_float(a.w);
        v[4] = __int_as_float(b.x); v[5] = __int_as_float(b.y); v[6] = __int_as_float(b.z); v[7] = __int_as_float(b.w);
    }
}

// The 8 int8 values of chunk c (elements 8c .. 8c+7) of one plane, stored in the 4x4-transposed
// layout of tw_device.h: the lanes holding chunks 2i and 2i+1 (adjacent lanes; chunk parity =
// lane parity) fill one 16-byte group together, exchanging half of their bytes, so every lane
// stores 8 contiguous bytes.  Both lanes of a pair must call it.
__device__ __forceinline__ void store_chunk_digits(int8_t *plane, int c, const int8_t (&q)[8])
{
    uint32_t h[4];
#pragma unroll
    for (int s = 0; s < 4; s++) h[s] = uint32_t(uint8_t(q[s])) | (uint32_t(uint8_t(q[4 + s])) << 8);
    const bool odd = c & 1;
    const uint32_t send = odd ? (h[0] | (h[1] << 16)) : (h[2] | (h[3] << 16));
    const uint32_t recv = uint32_t(dpp_i<kDppXor1>(int32_t(send)));
    uint2 o;
    if (!odd) {
        o.x = h[0] | ((recv & 0xffffu) << 16);
        o.y = h[1] | ((recv >> 16) << 16);
    } else {
        o.x = (recv & 0xffffu) | (h[2] << 16);
        o.y = (recv >> 16) | (h[3] << 16);
    }
    *reinterpret_cast<uint2 *>(plane + 16 * (c >> 1) + 8 * (c & 1)) = o;
}

// Digit planes (QP = 2, 3) or int8 absmax codes (QP = 1) of a token whose chunks c = t + 256 i
// this thread (t: its index among the token's 256 threads) holds, given the token's max |x| and
// canonical sum of squares.
template <int QP, int NCH>
__device__ __forceinline__ void quantize_token(const float (&v)[NCH][8], int nch, float am, float ss, int d,
                                               int pre_norm, int8_t *xd, float *ti, int t)
{
    if constexpr (QP == 1) {
        const float inv = am > 0.0f ? 127.0f / am : 0.0f;
#pragma unroll
        for (int i = 0; i < NCH; i++) {
            const int c = t + 256 * i;
            if (c < nch) {
                int8_t q[8];
#pragma unroll
                for (int j = 0; j < 8; j++) q[j] = am > 0.0f ? int8_quant(v[i][j], inv) : int8_t(0);
                store_chunk_digits(xd, c, q);
            }
        }
        if (t == 0) ti[0] = am > 0.0f ? am / 127.0f : 0.0f;
    } else {
        const int sh = float_digit_shift(am, QP);
#pragma unroll
        for (int i = 0; i < NCH; i++) {
            const int c = t + 256 * i;
            if (c < nch) {
                int8_t q[QP][8];
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    int8_t dg[QP];
                    float_digits<QP>(v[i][j], sh, dg);
#pragma unroll
                    for (int p = 0; p < QP; p++) q[p][j] = dg[p];
                }
#pragma unroll
                for (int p = 0; p < QP; p++) store_chunk_digits(xd + p * d, c, q[p]);
            }
        }
        if (t == 0) {
            reinterpret_cast<int32_t *>(ti)[0] = sh;
            ti[1] = pre_norm ? inv_rms_of(ss, d) : 1.0f;
        }
    }
}

// Chunk t + 256 i (8 elements) of rows row0 + r, r < R, of d bf16 or fp32 elements: raw_rows8
// issues the loads (rows past the n valid ones re-read the last valid row: their values are never
// used; the dtype branch is uniform, so the loads form one straight run), cvt_rows8 turns them into
// fp32 after every load of the caller has been issued.  Chunks past the row read as zeros.
template <int R, int NCH>
__device__ __forceinline__ void raw_rows8(const void *base, int bf16, int64_t row0, int n, int d,
                                          int4 (&raw)[R][NCH][2])
{
    const int t = threadIdx.x, nch = d >> 3;
    if (bf16) {
        const uint16_t *b = static_cast<const uint16_t *>(base);
#pragma unroll
        for (int r = 0; r < R; r++)
#pragma unroll
            for (int i = 0; i < NCH; i++) {
                const int c = min(t + 256 * i, nch - 1);
                raw[r][i][0] = reinterpret_cast<const int4 *>(b + (row0 + min(r, n - 1)) * d)[c];
            }
    } else {
        const float *f = static_cast<const float *>(base);
#pragma unroll
        for (int r = 0; r < R; r++)
#pragma unroll
            for (int i = 0; i < NCH; i++) {
                const int c = min(t + 256 * i, nch - 1);
                const int4 *p = reinterpret_cast<const int4 *>(f + (row0 + min(r, n - 1)) * d) + 2 * c;
                raw[r][i][0] = p[0];
                raw[r][i][1] = p[1];
            }
    }
}

template <int R, int NCH>
__device__ __forceinline__ void cvt_rows8(const int4 (&raw)[R][NCH][2], int bf16, int d,
                                          float (&v)[R][NCH][8])
{
    const int t = threadIdx.x, nch = d >> 3;
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
        for (int i = 0; i < NCH; i++) {
            const int4 a = raw[r][i][0], b = raw[r][i][1];
            const bool in = t + 256 * i < nch;
            if (bf16) {
                const uint32_t w[4] = {uint32_t(a.x), uint32_t(a.y), uint32_t(a.z), uint32_t(a.w)};
#pragma unroll
                for (int j = 0; j < 8; j++) v[r][i][j] = in ? bf16_to_f32(uint16_t(w[j >> 1] >> (16 * (j & 1)))) : 0.0f;
            } else {
                const int q[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
                for (int j = 0; j < 8; j++) v[r][i][j] = in ? __int_as_float(q[j]) : 0.0f;
            }
        }
}

// Router logits.  Workgroup (experts 4 f .. 4 f + 3, tokens 8 g .. 8 g + 7), 256 threads: thread t
// holds the 8-element chunks t + 256 i of the 8 tokens and of the 4 router rows (every load issued
// at once) and forms the canonical partial of each (expert, token) pair and each token's sum of
// squares; the partials go to LDS and each wave adds those of two tokens in the canonical tree
// (4 partials per lane, then wave_sum), so the pre-RMSNorm factor multiplies the logits in the same
// wave.  With QP > 0 the workgroups also write the tokens' activation codes (quantize_token) and
// their scale words, token u of a group by expert group u: the router has every chunk of its
// tokens in registers already.
constexpr int kRouteExp = 4;   // 8: a 64-token batched call 1.3 us slower (fewer, busier workgroups)

template <int NCH, int QP>
__global__ __launch_bounds__(256) void k_route(const void *__restrict__ x, int x_bf16,
                                               const void *__restrict__ wr, int w_bf16, int64_t T,
                                               int d, int E, int pre_norm,
                                               float *__restrict__ logits, int8_t *__restrict__ xdig,
                                               float *__restrict__ tinfo)
{
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int e0 = blockIdx.x * kRouteExp;
    const int64_t tb = int64_t(blockIdx.y) * kRouteTok;
    const int nt = int(T - tb < kRouteTok ? T - tb : kRouteTok);
    const int ne = E - e0 < kRouteExp ? E - e0 : kRouteExp;
    const int nch = d >> 3;
    constexpr int NPR = kRouteExp * kRouteTok + kRouteTok;   // pairs + sums of squares
    __shared__ __attribute__((aligned(16))) float part[NPR][256];
    __shared__ float s_am[4][kRouteTok];
    float xv[kRouteTok][NCH][8], wv[kRouteExp][NCH][8];
    {
        int4 rx[kRouteTok][NCH][2], rw[kRouteExp][NCH][2];
        raw_rows8<kRouteTok, NCH>(x, x_bf16, tb, nt, d, rx);
        raw_rows8<kRouteExp, NCH>(wr, w_bf16, e0, ne, d, rw);
        cvt_rows8<kRouteTok, NCH>(rx, x_bf16, d, xv);
        cvt_rows8<kRouteExp, NCH>(rw, w_bf16, d, wv);
    }
#pragma unroll
    for (int u = 0; u < kRouteTok; u++) {
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < NCH; i++)
#pragma unroll
            for (int q = 0; q < 8; q++) ss = ss + xv[u][i][q] * xv[u][i][q];
        part[kRouteExp * kRouteTok + u][t] = ss;
#pragma unroll
        for (int m = 0; m < kRouteExp; m++) {
            float dot = 0.0f;
#pragma unroll
            for (int i = 0; i < NCH; i++)
#pragma unroll
                for (int q = 0; q < 8; q++) dot = dot + wv[m][i][q] * xv[u][i][q];
            part[m * kRouteTok + u][t] = dot;
        }
    }
    // token u's codes are written by expert group u % gridDim.x, so the work spreads over the
    // expert groups (one token each when there are at least 8)
    const bool quant = QP > 0 && int(blockIdx.x) < kRouteTok;
    auto mine = [&](int u) { return u % int(gridDim.x) == int(blockIdx.x); };
    if (quant) {
#pragma unroll
        for (int u = 0; u < kRouteTok; u++) {
            if (!mine(u)) continue;
            float am = 0.0f;
#pragma unroll
            for (int i = 0; i < NCH; i++)
#pragma unroll
                for (int q = 0; q < 8; q++) am = fmaxf(am, fabsf(xv[u][i][q]));
            am = wave_max(am);
            if (lane == 0) s_am[wave][u] = am;
        }
    }
    __syncthreads();
    // wave w: tokens 2w, 2w + 1 -- the sum of squares, then the kRouteExp logits
    float ssv[2];
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const int u = 2 * wave + h;
        auto tree = [&](int r) {
            const float4 f = reinterpret_cast<const float4 *>(part[r])[lane];
            return wave_sum((f.x + f.y) + (f.z + f.w));
        };
        const float ss = tree(kRouteExp * kRouteTok + u);
        ssv[h] = ss;
        const float inv = pre_norm ? inv_rms_of(ss, d) : 1.0f;
        float out = 0.0f;
#pragma unroll
        for (int m = 0; m < kRouteExp; m++) {
            float v = tree(m * kRouteTok + u);
            if (pre_norm) v = v * inv;
            if (lane == m) out = v;
        }
        if (u < nt && lane < ne) logits[(tb + u) * E + e0 + lane] = out;
    }
    if constexpr (QP > 0) {
        if (!quant) return;
        // the token's sum of squares is needed by thread 0 only (its scale word); wave w has those
        // of tokens 2w, 2w + 1, so it is passed through LDS
        __shared__ float s_ss[kRouteTok];
        if (lane == 0) {
            s_ss[2 * wave] = ssv[0];
            s_ss[2 * wave + 1] = ssv[1];
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kRouteTok; u++) {
            if (u >= nt) break;
            if (!mine(u)) continue;
            const float am = fmaxf(fmaxf(s_am[0][u], s_am[1][u]), fmaxf(s_am[2][u], s_am[3][u]));
            quantize_token<QP, NCH>(xv[u], nch, am, s_ss[u], d, pre_norm,
                                    xdig + (tb + u) * int64_t(QP) * d, tinfo + 2 * (tb + u), t);
        }
    }
}

// Top-k and gates of T tokens, one wave per token; KPER = candidates per lane (E <= 64 KPER).
template <int KPER>
__global__ __launch_bounds__(256) void k_topk(const float *__restrict__ logits, int64_t T, int E,
                                              int k, int32_t *__restrict__ ids,
                                              float *__restrict__ gates)
{
    const int lane = threadIdx.x & 63;
    const int64_t t = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    topk_softmax_wave_t<KPER>(logits + t * E, E, k, ids + t * k, gates + t * k, lane);
}

void launch_topk(const float *logits, int64_t T, int E, int k, int32_t *ids, float *gates, void *stream)
{
    const unsigned g = unsigned((T + 3) / 4);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (E <= 64) k_topk<1><<<g, 256, 0, st>>>(logits, T, E, k, ids, gates);
    else if (E <= 128) k_topk<2><<<g, 256, 0, st>>>(logits, T, E, k, ids, gates);
    else if (E <= 256) k_topk<4><<<g, 256, 0, st>>>(logits, T, E, k, ids, gates);
    else if (E <= 512) k_topk<8><<<g, 256, 0, st>>>(logits, T, E, k, ids, gates);
    else k_topk<16><<<g, 256, 0, st>>>(logits, T, E, k, ids, gates);
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

// Digit planes of one token (int8 mode: one plane, scale amax/127; float mode: P planes, shift) by
// 256 threads: thread q of the group holds the 8-element chunks q, q + 256 of the token; red is the
// group's [4][2] LDS scratch.  Contains one workgroup barrier, which every thread of the workgroup
// reaches (tok >= T: no loads, no stores).
template <int P, bool INT8>
__device__ __forceinline__ void quant_token256(const BatchedArgs &a, const void *__restrict__ x, int x_bf16,
                                               uint8_t *__restrict__ ws, int64_t tok, int q, float (*red)[2])
{
    const int lane = q & 63, wave = q >> 6;
    const int d = a.dm.d, nch = d >> 3;
    const bool live = tok < a.T;
    float v[2][8] = {};
    float am = 0.0f, ss = 0.0f;
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int c = q + 256 * i;
        if (live && c < nch) {
            load_chunk8(x, tok, d, c, x_bf16, v[i]);
#pragma unroll
            for (int j = 0; j < 8; j++) {
                am = fmaxf(am, fabsf(v[i][j]));
                ss = ss + v[i][j] * v[i][j];
            }
        }
    }
    am = wave_max(am);
    if (!INT8 && a.dm.pre_norm) ss = wave_sum(ss);
    if (lane == 0) {
        red[wave][0] = am;
        red[wave][1] = ss;
    }
    __syncthreads();
    if (!live) return;
    am = fmaxf(fmaxf(red[0][0], red[1][0]), fmaxf(red[2][0], red[3][0]));
    // the pre-RMSNorm sum of squares in the canonical order (partials t, waves in pairs)
    const float tot = (red[0][1] + red[1][1]) + (red[2][1] + red[3][1]);
    quantize_token<INT8 ? 1 : P, 2>(v, nch, am, tot, d, a.dm.pre_norm,
                                    reinterpret_cast<int8_t *>(ws + a.L.xdig) + tok * int64_t(P) * d,
                                    reinterpret_cast<float *>(ws + a.L.tinfo) + 2 * tok, q);
}

// One workgroup per token.
template <int P, bool INT8>
__global__ __launch_bounds__(256) void k_bat_quant_x(BatchedArgs a, const void *__restrict__ x,
                                                     int x_bf16, uint8_t *__restrict__ ws)
{
    __shared__ float red[4][2];
    quant_token256<P, INT8>(a, x, x_bf16, ws, int64_t(blockIdx.x), int(threadIdx.x), red);
}

// Groups the T*k (token, slot) pairs by expert: counts[e], offsets[E+1] and pairs[] (the pairs of
// expert e at offsets[e]..offsets[e+1]; their order inside a group is not fixed, and no result
// depends on it: every pair is computed on its own), plus the list of (expert, tile of tt tokens)
// work items: tiles[0] = their number, tiles[1 + i] = e | (tile << 10), tilemeta[i] = (position of the
// tile's first pair in pairs[], its number of pairs).
// Workgroups of 1024 threads; counts and placement use LDS atomics.  Workgroup g of G places the
// pairs of the experts [E g / G, E (g + 1) / G) and writes their counts, offsets and tiles; each
// counts every pair, since the offsets and tile numbers of its experts follow from all the experts
// before them.  The ids are read in passes of 32 per thread, all loads of a pass issued before any
// is used (one memory round trip per pass instead of one per id); with a single pass they stay in
// registers for the placement.  Up to kGrpStage pairs the placement is staged in LDS (stage[j] is
// pairs[a0 + j], a0 the range's first position rounded down to a multiple of 4) and written out
// with 16-byte stores (scattered 4-byte stores from one workgroup are limited by its address rate).
constexpr int kGrpPer = 32;                    // ids per thread per pass
constexpr int kGrpPass = 1024 * kGrpPer;       // pairs per pass
constexpr int kGrpStage = kGrpPass;            // pairs staged in LDS (128 KiB, plus 3 for alignment)
constexpr int kGrpWgs = 8;                     // grouping workgroups of k_quant_group

__device__ __forceinline__ void group_pairs(const BatchedArgs &a, const int32_t *__restrict__ ids,
                                            uint8_t *__restrict__ ws, int tt, int32_t *stage, int g, int G)
{
    const int E = a.dm.E, t = threadIdx.x;
    const int e_lo = int(int64_t(E) * g / G), e_hi = int(int64_t(E) * (g + 1) / G);
    const int64_t npairs = a.T * a.dm.k;
    const bool staged = npairs <= kGrpStage;
    int32_t *counts = reinterpret_cast<int32_t *>(ws + a.L.counts);
    int32_t *offsets = reinterpret_cast<int32_t *>(ws + a.L.offsets);
    int32_t *pairs = reinterpret_cast<int32_t *>(ws + a.L.pairs);
    int32_t *tiles = reinterpret_cast<int32_t *>(ws + a.L.tiles);
    int2 *tmeta = reinterpret_cast<int2 *>(ws + a.L.tilemeta);
    __shared__ int32_t cnt[kMaxExperts], cur[kMaxExperts], s_wc[16], s_wt[16], s_lo, s_hi;
    const int64_t npass = (npairs + kGrpPass - 1) / kGrpPass;
    int v[kGrpPer];
    // v[i] = id of pair base + t + 1024 i, or -1 past the end
    auto load = [&](int64_t base) {
#pragma unroll
        for (int i = 0; i < kGrpPer; i++) {
            const int64_t p = base + t + 1024 * i;
            v[i] = p < npairs ? ids[p] : -1;
        }
    };
    for (int e = t; e < E; e += 1024) cnt[e] = 0;
    __syncthreads();
    for (int64_t ps = 0; ps < npass; ps++) {
        load(ps * kGrpPass);
#pragma unroll
        for (int i = 0; i < kGrpPer; i++)
            if (v[i] >= 0 && v[i] < E) atomicAdd(&cnt[v[i]], 1);
    }
    __syncthreads();
    const int c = t < E ? cnt[t] : 0;
    const int nt = (c + tt - 1) / tt;
    // exclusive scans of the counts and tile counts over the experts: inside each wave, then over
    // the 16 wave totals
    const int lane = t & 63, wave = t >> 6;
    int ic = c, it = nt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int uc = __shfl_up(ic, off), ut = __shfl_up(it, off);
        if (lane >= off) {
            ic += uc;
            it += ut;
        }
    }
    if (lane == 63) {
        s_wc[wave] = ic;
        s_wt[wave] = it;
    }
    __syncthreads();
    int bc = 0, bt = 0, placed = 0, ntiles = 0;
#pragma unroll
    for (int w = 0; w < 16; w++) {
        bc += w < wave ? s_wc[w] : 0;
        bt += w < wave ? s_wt[w] : 0;
        placed += s_wc[w];   // pairs with a valid id
        ntiles += s_wt[w];
    }
    const int off_e = bc + ic - c, tile0 = bt + it - nt;
    if (t < E) cur[t] = off_e;
    if (t >= e_lo && t < e_hi) {
        counts[t] = c;
        offsets[t] = off_e;
        for (int i = 0; i < nt; i++) {
            tiles[1 + tile0 + i] = t | (i << 10);
            tmeta[tile0 + i] = make_int2(off_e + i * tt, min(tt, c - i * tt));
        }
    }
    // the range's first and end positions
    if (t < E && t == e_lo) s_lo = off_e;
    if (t < E && t == e_hi) s_hi = off_e;
    if (t == 1023) {
        if (e_lo >= E) s_lo = placed;
        if (e_hi >= E) s_hi = placed;
        if (g == 0) {
            offsets[E] = placed;
            tiles[0] = ntiles;
        }
    }
    __syncthreads();
    const int a0 = s_lo & ~3, p_hi = s_hi;
    for (int64_t ps = 0; ps < npass; ps++) {
        const int64_t base = ps * kGrpPass;
        if (npass > 1) load(base);
#pragma unroll
        for (int i = 0; i < kGrpPer; i++)
            if (v[i] >= e_lo && v[i] < e_hi) {
                const int pos = atomicAdd(&cur[v[i]], 1);
                const int32_t pr = int32_t(base + t + 1024 * i);
                if (staged)
                    stage[pos - a0] = pr;
                else
                    pairs[pos] = pr;
            }
    }
    if (!staged) return;
    __syncthreads();
    // pairs is 256-byte aligned inside the workspace, so pairs + a0 is 16-byte aligned; the stage
    // holds positions s_lo .. p_hi - 1 at indices s_lo - a0 ..
    const int j_lo = s_lo - a0, j_hi = p_hi - a0;
    for (int i = t; 4 * i < j_hi; i += 1024) {
        if (4 * i >= j_lo && 4 * i + 3 < j_hi)
            reinterpret_cast<int4 *>(pairs + a0)[i] = reinterpret_cast<const int4 *>(stage)[i];
        else
            for (int j = max(4 * i, j_lo); j < min(4 * i + 4, j_hi); j++) pairs[a0 + j] = stage[j];
    }
}

__global__ __launch_bounds__(1024) void k_group(BatchedArgs a, const int32_t *__restrict__ ids,
                                                uint8_t *__restrict__ ws, int tt)
{
    extern __shared__ __attribute__((aligned(16))) int32_t stage[];   // [npairs + 3] when staged
    group_pairs(a, ids, ws, tt, stage, 0, 1);
}

// The quantisation of the tokens and the grouping of the pairs in one launch (they are
// independent): workgroups 0 .. kGrpWgs - 1 group (one range of experts each), workgroup kGrpWgs + j
// quantises tokens 4 j .. 4 j + 3, one per 256-thread quarter, so the grouping runs beside the
// quantisation instead of after it.
template <int P, bool INT8>
__global__ __launch_bounds__(1024) void k_quant_group(BatchedArgs a, const void *__restrict__ x, int x_bf16,
                                                      const int32_t *__restrict__ ids,
                                                      uint8_t *__restrict__ ws, int tt)
{
    extern __shared__ __attribute__((aligned(16))) int32_t stage[];   // [npairs + 3] when staged
    __shared__ float red[4][4][2];
    if (blockIdx.x < kGrpWgs) {
        group_pairs(a, ids, ws, tt, stage, int(blockIdx.x), kGrpWgs);
        return;
    }
    const int q = int(threadIdx.x) >> 8;
    quant_token256<P, INT8>(a, x, x_bf16, ws, int64_t(blockIdx.x - kGrpWgs) * 4 + q, int(threadIdx.x) & 255, red[q]);
}

template <int P, bool INT8>
int launch_quant_group(const BatchedArgs &a, const void *x, int x_bf16, const int32_t *ids, uint8_t *ws,
                       int tt, void *stream)
{
    const int64_t npairs = a.T * a.dm.k;
    const size_t lds = npairs <= kGrpStage ? size_t(npairs + 4) * sizeof(int32_t) : 0;
    static std::atomic<int> attr_set{0};
    if (lds > 0 && !attr_set.load(std::memory_order_relaxed)) {
        if (hipFuncSetAttribute(reinterpret_cast<const void *>(k_quant_group<P, INT8>),
                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                int((kGrpStage + 4) * sizeof(int32_t))) != hipSuccess)
            return int(hipErrorInvalidValue);
        attr_set.store(1, std::memory_order_relaxed);
    }
    k_quant_group<P, INT8><<<unsigned(kGrpWgs + (a.T + 3) / 4), 1024, lds, static_cast<hipStream_t>(stream)>>>(
        a, x, x_bf16, ids, ws, tt);
    return 0;
}

// Launches k_group (one workgroup) with the LDS staging area when the pairs fit in it.
int launch_group(const BatchedArgs &a, const int32_t *ids, uint8_t *ws, int tt, void *stream)
{
    const int64_t npairs = a.T * a.dm.k;
    const size_t lds = npairs <= kGrpStage ? size_t(npairs + 4) * sizeof(int32_t) : 0;
    static std::atomic<int> attr_set{0};
    if (lds > 0 && !attr_set.load(std::memory_order_relaxed)) {
        if (hipFuncSetAttribute(reinterpret_cast<const void *>(k_group),
                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                int((kGrpStage + 4) * sizeof(int32_t))) != hipSuccess)
            return int(hipErrorInvalidValue);
        attr_set.store(1, std::memory_order_relaxed);
    }
    k_group<<<1, 1024, lds, static_cast<hipStream_t>(stream)>>>(a, ids, ws, tt);
    return 0;
}

// Batched gate/up and down.  Work items are (expert tile, row block) -- a tile is up to 64 of an
// expert's tokens (k_group) and a row block is 16 h rows (gate/up: 32 code rows of d/4 bytes) or
// 64 output rows (down: 64 code rows of F/4 bytes).  A grid of kBatG workgroups walks the items
// in expert-major order, each workgroup a contiguous range: the code rows of its next item are
// requested before the current item is computed (latency hidden behind the dots), and the
// activation digits of a tile are staged in LDS once for all of the tile's row blocks.  Each code
// byte is read once per call.
constexpr int kBatTok = 16;    // at most this many tokens staged per round
constexpr int kBatG = 512;     // workgroups of the gate/up and down grids
// Tokens per round such that their staged digit planes fit in 64 KiB of LDS.
inline int tokens_per_round(int bytes_per_token)
{
    const int n = 65536 / bytes_per_token;
    return n < 1 ? 1 : (n > kBatTok ? kBatTok : n);
}

// Item metadata of a tile: expert, its tokens in the tile, first pair position.
struct BatTile {
    int e, ntok, p0;
};

__device__ __forceinline__ BatTile bat_tile(const int32_t *tiles, const int32_t *counts,
                                            const int32_t *offsets, int ti)
{
    const int tl = tiles[1 + ti], e = tl & 1023, mt = tl >> 10;
    const int n = counts[e] - mt * kTileTokens;
    return BatTile{e, n < kTileTokens ? n : kTileTokens, offsets[e] + mt * kTileTokens};
}

// NP: passes of code rows per item (>= rows * (cols / 64) / 256).
template <int P, bool INT8, int NP>
__global__ __launch_bounds__(256) void k_bat_gu(BatchedArgs a, LayerPtrs lp, uint8_t *__restrict__ ws,
                                                int tpr)
{
    extern __shared__ __attribute__((aligned(16))) int8_t smem[];   // [tpr][P][d]
    __shared__ float sums[kBatTok][32];
    __shared__ int32_t s_pair[kBatTok];
    __shared__ float s_tok[kBatTok][2];   // per token: s_x (int8) or digit shift bits, 1/rms
    const int t = threadIdx.x;
    const int d = a.dm.d, F = a.dm.F, k = a.dm.k;
    const int nrb = F / 16;
    const int32_t *tiles = reinterpret_cast<const int32_t *>(ws + a.L.tiles);
    const int32_t *counts = reinterpret_cast<const int32_t *>(ws + a.L.counts);
    const int32_t *offsets = reinterpret_cast<const int32_t *>(ws + a.L.offsets);
    const int32_t *pairs = reinterpret_cast<const int32_t *>(ws + a.L.pairs);
    const int8_t *xdig = reinterpret_cast<const int8_t *>(ws + a.L.xdig);
    const float *tinfo = reinterpret_cast<const float *>(ws + a.L.tinfo);
    float *hbuf = reinterpret_cast<float *>(ws + a.L.h);
    const int nitems = tiles[0] * nrb;
    const int i0 = int(int64_t(blockIdx.x) * nitems / gridDim.x);
    const int i1 = int(int64_t(blockIdx.x + 1) * nitems / gridDim.x);
    if (i0 >= i1) return;
    const int lpr = d >> 6, rpp = 256 / lpr, c = t % lpr;
    const int npass = (32 + rpp - 1) / rpp;
    // code rows of item `it` (clamped into the block's range: loads are unconditional, so the
    // compiler can count them and wait only for the ones it needs)
    int ld_ti = -1, ld_e = 0;
    auto load = [&](int it, int4 (&code)[NP], float (&sc)[NP]) {
        it = it < i1 ? it : i1 - 1;
        const int ti = it / nrb;
        if (ti != ld_ti) {
            ld_ti = ti;
            ld_e = tiles[1 + ti] & 1023;
        }
        const int r0 = (it % nrb) * 16;
#pragma unroll
        for (int p = 0; p < NP; p++) {
            const int jb = p * rpp + t / lpr;
            const bool valid = p < npass && jb < 32;
            const int i = valid ? (jb >> 1) : 0, kind = jb & 1;
            const int64_t row = int64_t(ld_e) * F + r0 + i;
            const int4 v = reinterpret_cast<const int4 *>((kind ? lp.w_up : lp.w_gate) + row * (d / 4))[c];
            const float sv = (kind ? lp.s_up : lp.s_gate)[row];
            code[p] = valid ? v : make_int4(0, 0, 0, 0);
            sc[p] = valid ? sv : 0.0f;
        }
    };
    int cur_ti = -1, staged = -1;
    BatTile tl{0, 0, 0};
    auto process = [&](int it, const int4 (&code)[NP], const float (&sc)[NP]) {
        const int ti = it / nrb, r0 = (it % nrb) * 16;
        if (ti != cur_ti) {
            cur_ti = ti;
            tl = bat_tile(tiles, counts, offsets, ti);
        }
        int32_t wd[NP][16];
#pragma unroll
        for (int p = 0; p < NP; p++) decode_chunk(code[p], wd[p]);
        for (int tb = 0; tb < tl.ntok; tb += tpr) {
            const int nt = tl.ntok - tb < tpr ? tl.ntok - tb : tpr;
            if (!(staged == ti && tb == 0)) {
                __syncthreads();
                if (t < nt) {
                    const int pr = pairs[tl.p0 + tb + t];
                    s_pair[t] = pr;
                    s_tok[t][0] = tinfo[2 * (pr / k)];
                    s_tok[t][1] = tinfo[2 * (pr / k) + 1];
                }
                __syncthreads();
                const int cpt = P * d / 16;   // 16-byte chunks per token
                for (int idx = t; idx < nt * cpt; idx += 256) {
                    const int j = idx / cpt, r = idx % cpt;
                    const int64_t tok = s_pair[j] / k;
                    reinterpret_cast<int4 *>(smem + j * P * d)[r] =
                        reinterpret_cast<const int4 *>(xdig + tok * P * d)[r];
                }
                __syncthreads();
                staged = tl.ntok <= tpr ? ti : -1;
            }
            for (int j = 0; j < nt; j++) {
                int4 dg[P][4];
#pragma unroll
                for (int pl = 0; pl < P; pl++)
#pragma unroll
                    for (int q = 0; q < 4; q++)
                        dg[pl][q] = reinterpret_cast<const int4 *>(smem + (j * P + pl) * d + c * 64)[q];
#pragma unroll
                for (int p = 0; p < NP; p++) {
                    if (p < npass) {
                        const int jb = p * rpp + t / lpr;
                        int32_t acc[P] = {};
                        dec_dot<P>(wd[p], dg, acc);
                        group_reduce<P>(acc, lpr);
                        if (c == 0 && jb < 32) {
                            float v;
                            if (INT8)
                                v = (float(acc[0]) * s_tok[j][0]) * sc[p];
                            else
                                v = float_value<P>(acc, __float_as_int(s_tok[j][0])) * sc[p] * s_tok[j][1];
                            sums[j][jb] = v;
                        }
                    }
                }
            }
            __syncthreads();
            for (int idx = t; idx < nt * 16; idx += 256) {
                const int j = idx >> 4, i = idx & 15;
                hbuf[int64_t(s_pair[j]) * F + r0 + i] = tw_silu(sums[j][2 * i]) * sums[j][2 * i + 1];
            }
            __syncthreads();
        }
    };
    int4 ca[NP], cb[NP];
    float sa[NP], sb[NP];
    load(i0, ca, sa);
    for (int it = i0; it < i1; it += 2) {
        load(it + 1, cb, sb);
        process(it, ca, sa);
        if (it + 1 >= i1) break;
        load(it + 2, ca, sa);
        process(it + 1, cb, sb);
    }
}

// Down: item = (expert tile, 64 output rows); per token round, the tokens' h vectors become digit
// planes in LDS (per (token, expert) maximum: int8 absmax, or the float fixed-point shift) once
// per tile when all of its tokens fit, then every token's dots run against the item's codes.
template <int P, bool INT8, int NP>
__global__ __launch_bounds__(256) void k_bat_dn(BatchedArgs a, LayerPtrs lp, uint8_t *__restrict__ ws,
                                                int tpr)
{
    extern __shared__ __attribute__((aligned(16))) int8_t smem[];   // [tpr][P][F] digits
    __shared__ int32_t s_pair[kBatTok];
    __shared__ float s_hs[kBatTok];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int d = a.dm.d, F = a.dm.F;
    const int nrb = d / 64;
    const int32_t *tiles = reinterpret_cast<const int32_t *>(ws + a.L.tiles);
    const int32_t *counts = reinterpret_cast<const int32_t *>(ws + a.L.counts);
    const int32_t *offsets = reinterpret_cast<const int32_t *>(ws + a.L.offsets);
    const int32_t *pairs = reinterpret_cast<const int32_t *>(ws + a.L.pairs);
    const float *hbuf = reinterpret_cast<const float *>(ws + a.L.h);
    float *ybuf = reinterpret_cast<float *>(ws + a.L.y);
    const int nitems = tiles[0] * nrb;
    const int i0 = int(int64_t(blockIdx.x) * nitems / gridDim.x);
    const int i1 = int(int64_t(blockIdx.x + 1) * nitems / gridDim.x);
    if (i0 >= i1) return;
    const int lpr = F >> 6, rpp = 256 / lpr, c = t % lpr;
    const int npass = (64 + rpp - 1) / rpp;
    int ld_ti = -1, ld_e = 0;
    auto load = [&](int it, int4 (&code)[NP], float (&sc)[NP]) {
        it = it < i1 ? it : i1 - 1;
        const int ti = it / nrb;
        if (ti != ld_ti) {
            ld_ti = ti;
            ld_e = tiles[1 + ti] & 1023;
        }
        const int r0 = (it % nrb) * 64;
#pragma unroll
        for (int p = 0; p < NP; p++) {
            const int jd = p * rpp + t / lpr;
            const bool valid = p < npass && jd < 64;
            const int64_t row = int64_t(ld_e) * d + r0 + (valid ? jd : 0);
            const int4 v = reinterpret_cast<const int4 *>(lp.w_down + row * (F / 4))[c];
            const float sv = lp.s_down[row];
            code[p] = valid ? v : make_int4(0, 0, 0, 0);
            sc[p] = valid ? sv : 0.0f;
        }
    };
    int cur_ti = -1, staged = -1;
    BatTile tl{0, 0, 0};
    auto process = [&](int it, const int4 (&code)[NP], const float (&sc)[NP]) {
        const int ti = it / nrb, r0 = (it % nrb) * 64;
        if (ti != cur_ti) {
            cur_ti = ti;
            tl = bat_tile(tiles, counts, offsets, ti);
        }
        int32_t wd[NP][16];
#pragma unroll
        for (int p = 0; p < NP; p++) decode_chunk(code[p], wd[p]);
        for (int tb = 0; tb < tl.ntok; tb += tpr) {
            const int nt = tl.ntok - tb < tpr ? tl.ntok - tb : tpr;
            if (!(staged == ti && tb == 0)) {
                __syncthreads();
                if (t < nt) s_pair[t] = pairs[tl.p0 + tb + t];
                __syncthreads();
                for (int j = wave; j < nt; j += 4) {
                    const float *h = hbuf + int64_t(s_pair[j]) * F;
                    float am = 0.0f;
                    for (int i = lane; i < F; i += 64) am = fmaxf(am, fabsf(h[i]));
                    am = wave_max(am);
                    int8_t *hd = smem + j * P * F;
                    if (INT8) {
                        const float inv = am > 0.0f ? 127.0f / am : 0.0f;
                        for (int i = lane; i < F; i += 64) hd[perm16(i)] = am > 0.0f ? int8_quant(h[i], inv) : int8_t(0);
                        if (lane == 0) s_hs[j] = am > 0.0f ? am / 127.0f : 0.0f;
                    } else {
                        const int sh = float_digit_shift(am, P);
                        for (int i = lane; i < F; i += 64) {
                            int8_t dg[P];
                            float_digits<P>(h[i], sh, dg);
#pragma unroll
                            for (int pl = 0; pl < P; pl++) hd[pl * F + perm16(i)] = dg[pl];
                        }
                        if (lane == 0) reinterpret_cast<int32_t *>(s_hs)[j] = sh;
                    }
                }
                __syncthreads();
                staged = tl.ntok <= tpr ? ti : -1;
            }
            for (int j = 0; j < nt; j++) {
                int4 dh[P][4];
#pragma unroll
                for (int pl = 0; pl < P; pl++)
#pragma unroll
                    for (int q = 0; q < 4; q++)
                        dh[pl][q] = reinterpret_cast<const int4 *>(smem + (j * P + pl) * F + c * 64)[q];
#pragma unroll
                for (int p = 0; p < NP; p++) {
                    if (p < npass) {
                        const int jd = p * rpp + t / lpr;
                        int32_t acc[P] = {};
                        dec_dot<P>(wd[p], dh, acc);
                        group_reduce<P>(acc, lpr);
                        if (c == 0 && jd < 64) {
                            float v;
                            if (INT8)
                                v = (float(acc[0]) * s_hs[j]) * sc[p];
                            else
                                v = float_value<P>(acc, reinterpret_cast<const int32_t *>(s_hs)[j]) * sc[p];
                            ybuf[int64_t(s_pair[j]) * d + r0 + jd] = v;
                        }
                    }
                }
            }
        }
    };
    int4 ca[NP], cb[NP];
    float sa[NP], sb[NP];
    load(i0, ca, sa);
    for (int it = i0; it < i1; it += 2) {
        load(it + 1, cb, sb);
        process(it, ca, sa);
        if (it + 1 >= i1) break;
        load(it + 2, ca, sa);
        process(it + 1, cb, sb);
    }
}

// Rows of 16-bit down sums (int8 activations on the matrix cores): the down sum of a (pair, output)
// is an int32 of at most 127 F in magnitude; it is kept as an int16 when it lies in
// [-32767, 32767] and otherwise as the marker -32768, with the int32 itself in the same position of
// the 32-bit rows.  y = (float(sum) * s_h) * s_down[e][r] is formed here, in the same fp32 operations
// as the v_dot4 and batch-1 paths, from the pair's s_h and the expert's down scales.
struct Y16Rows {
    const int16_t *y16;     // [T k + spare][d]
    const int32_t *ywide;   // [T k + spare][d], read only at markers
    const float *s_h;       // [T k]
    const float *s_down;    // the layer's [E][d]
};

// out[t] = ((x[t] + g_0 y_0) + g_1 y_1) + ..., over the slots j < k in selection order whose expert
// id is in [0, E) (the others contribute nothing: the expert kernels do not compute them either);
// every product and every sum is one fp32 rounding.  One call covers the 8-element chunk c of token
// tok; x and out in bf16 (XB / OB) or fp32; y rows [T k][d] fp32, or 16-bit sums (Y16).  Every load
// of the chunk is issued before the first is used (the residual chunk, the y rows of eight slots,
// their ids and gates, and with Y16 the s_h and down scales); the residual and the y rows are read
// once, with non-temporal loads, so that they do not push the down scales (read by every token)
// out of L2 (4096 int8 tokens: 253.2 -> 250.3 us per call).  The y row of every slot exists
// (unwritten for slots without a valid expert, and then unused).
template <bool XB, bool OB, bool Y16, int KK>
__device__ __forceinline__ void combine_chunk(const void *__restrict__ x, void *__restrict__ out,
                                              const int32_t *__restrict__ ids,
                                              const float *__restrict__ gates,
                                              const float *__restrict__ ybuf, const Y16Rows &yr,
                                              int64_t tok, int c, int d, int k_rt, int E)
{
    typedef float f4 __attribute__((ext_vector_type(4)));
    typedef int i4v __attribute__((ext_vector_type(4)));
    const int k = KK > 0 ? KK : k_rt;   // KK: the slot count known when compiled
    float o[8];
    if constexpr (XB) {
        const i4v q = __builtin_nontemporal_load(reinterpret_cast<const i4v *>(static_cast<const uint16_t *>(x) + tok * d) + c);
        const uint32_t w[4] = {uint32_t(q.x), uint32_t(q.y), uint32_t(q.z), uint32_t(q.w)};
#pragma unroll
        for (int jj = 0; jj < 8; jj++) o[jj] = bf16_to_f32(uint16_t(w[jj >> 1] >> (16 * (jj & 1))));
    } else {
        const f4 *p = reinterpret_cast<const f4 *>(static_cast<const float *>(x) + tok * d) + 2 * c;
        const f4 p0 = __builtin_nontemporal_load(p), p1 = __builtin_nontemporal_load(p + 1);
        o[0] = p0.x; o[1] = p0.y; o[2] = p0.z; o[3] = p0.w;
        o[4] = p1.x; o[5] = p1.y; o[6] = p1.z; o[7] = p1.w;
    }
    for (int j0 = 0; j0 < k; j0 += 8) {
        // per slot: the pair index, expert id, gate (and s_h), loaded before any row
        int64_t pj[8];
        int id[8];
        float g[8], sh[8];
        bool ok[8];
#pragma unroll
        for (int u = 0; u < 8; u++) pj[u] = tok * k + (j0 + u < k ? j0 + u : k - 1);
        // the 16-bit rows first: their addresses need no id, so their loads are in flight while the
        // ids arrive
        [[maybe_unused]] int4 yq[8];
        if constexpr (Y16) {
#pragma unroll
            for (int u = 0; u < 8; u++) {
                const i4v q = __builtin_nontemporal_load(reinterpret_cast<const i4v *>(yr.y16 + pj[u] * d) + c);
                yq[u] = make_int4(q.x, q.y, q.z, q.w);
            }
        }
#pragma unroll
        for (int u = 0; u < 8; u++) {
            id[u] = ids[pj[u]];
            g[u] = gates[pj[u]];
            if constexpr (Y16) sh[u] = yr.s_h[pj[u]];
        }
#pragma unroll
        for (int u = 0; u < 8; u++) ok[u] = j0 + u < k && id[u] >= 0 && id[u] < E;
        float yy[8][8];
        if constexpr (Y16) {
            f4 sd[8][2];
#pragma unroll
            for (int u = 0; u < 8; u++) {
                const f4 *sp = reinterpret_cast<const f4 *>(yr.s_down + int64_t(ok[u] ? id[u] : 0) * d) + 2 * c;
                sd[u][0] = sp[0];
                sd[u][1] = sp[1];
            }
#pragma unroll
            for (int u = 0; u < 8; u++) {
                const uint32_t w[4] = {uint32_t(yq[u].x), uint32_t(yq[u].y), uint32_t(yq[u].z), uint32_t(yq[u].w)};
                int32_t v[8];
                bool marked = false;
#pragma unroll
                for (int q = 0; q < 8; q++) {
                    v[q] = int32_t(int16_t(uint16_t(w[q >> 1] >> (16 * (q & 1)))));
                    marked = marked || v[q] == -32768;
                }
                if (marked && ok[u]) {   // a sum outside the int16 range: the 32-bit row holds it
                    const int4 *wp = reinterpret_cast<const int4 *>(yr.ywide + pj[u] * d + 8 * c);
                    const int4 w0 = wp[0], w1 = wp[1];
                    const int32_t wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
                    for (int q = 0; q < 8; q++) v[q] = v[q] == -32768 ? wv[q] : v[q];
                }
                const float sdv[8] = {sd[u][0].x, sd[u][0].y, sd[u][0].z, sd[u][0].w,
                                      sd[u][1].x, sd[u][1].y, sd[u][1].z, sd[u][1].w};
#pragma unroll
                for (int q = 0; q < 8; q++) yy[u][q] = (float(v[q]) * sh[u]) * sdv[q];
            }
        } else {
            f4 yv[8][2];
#pragma unroll
            for (int u = 0; u < 8; u++) {
                const f4 *yp = reinterpret_cast<const f4 *>(ybuf + pj[u] * d + 8 * c);
                yv[u][0] = __builtin_nontemporal_load(yp);
                yv[u][1] = __builtin_nontemporal_load(yp + 1);
            }
#pragma unroll
            for (int u = 0; u < 8; u++) {
                yy[u][0] = yv[u][0].x; yy[u][1] = yv[u][0].y; yy[u][2] = yv[u][0].z; yy[u][3] = yv[u][0].w;
                yy[u][4] = yv[u][1].x; yy[u][5] = yv[u][1].y; yy[u][6] = yv[u][1].z; yy[u][7] = yv[u][1].w;
            }
        }
#pragma unroll
        for (int u = 0; u < 8; u++) {
            if (ok[u]) {
#pragma unroll
                for (int q = 0; q < 8; q++) o[q] = o[q] + g[u] * yy[u][q];
            }
        }
    }
    if constexpr (OB) {
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; q++)
            w[q] = uint32_t(f32_to_bf16(o[2 * q])) | (uint32_t(f32_to_bf16(o[2 * q + 1])) << 16);
        reinterpret_cast<int4 *>(static_cast<uint16_t *>(out) + tok * d)[c] =
            make_int4(int(w[0]), int(w[1]), int(w[2]), int(w[3]));
    } else {
        f4 *op = reinterpret_cast<f4 *>(static_cast<float *>(out) + tok * d) + 2 * c;
        op[0] = f4{o[0], o[1], o[2], o[3]};
        op[1] = f4{o[4], o[5], o[6], o[7]};
    }
}

// (token, s) covers the 8-element chunks s * blockDim + i of the token, one per thread (a small
// batch takes one-wave workgroups so that its few tokens still spread over the compute units);
// every load of a chunk is issued at once.
template <bool XB, bool OB, bool Y16, int KK>
__global__ __launch_bounds__(256) void k_bat_combine(BatchedArgs a, const void *__restrict__ x,
                                                     void *__restrict__ out,
                                                     const int32_t *__restrict__ ids,
                                                     const float *__restrict__ gates,
                                                     uint8_t *__restrict__ ws, const float *__restrict__ s_down)
{
    const int d = a.dm.d, nch = d >> 3;
    const int c = int(blockIdx.y * blockDim.x + threadIdx.x);
    if (c >= nch) return;
    const Y16Rows yr{reinterpret_cast<const int16_t *>(ws + a.L.y16), reinterpret_cast<const int32_t *>(ws + a.L.y),
                     reinterpret_cast<const float *>(ws + a.L.shp), s_down};
    combine_chunk<XB, OB, Y16, KK>(x, out, ids, gates, reinterpret_cast<const float *>(ws + a.L.y), yr,
                               int64_t(blockIdx.x), c, d, a.dm.k, a.dm.E);
}

// s_down != nullptr: the y rows are 16-bit down sums (grouped MFMA path, int8 activations).
void launch_combine(const BatchedArgs &a, const void *x, int in_bf16, void *out, int out_bf16,
                    const int32_t *ids, const float *gates, uint8_t *ws, const float *s_down,
                    void *stream)
{
    const int nt = a.T >= 1024 ? 256 : 64, nch = a.dm.d >> 3;
    const dim3 g(unsigned(a.T), unsigned((nch + nt - 1) / nt));
    hipStream_t st = static_cast<hipStream_t>(stream);
#define TW_COMB(XB, OB, Y)                                                                        \
    do {                                                                                          \
        if (a.dm.k == 8) k_bat_combine<XB, OB, Y, 8><<<g, nt, 0, st>>>(a, x, out, ids, gates, ws, s_down); \
        else k_bat_combine<XB, OB, Y, 0><<<g, nt, 0, st>>>(a, x, out, ids, gates, ws, s_down);    \
    } while (0)
    if (s_down) {
        if (in_bf16 && out_bf16) TW_COMB(true, true, true);
        else if (in_bf16) TW_COMB(true, false, true);
        else if (out_bf16) TW_COMB(false, true, true);
        else TW_COMB(false, false, true);
    } else {
        if (in_bf16 && out_bf16) TW_COMB(true, true, false);
        else if (in_bf16) TW_COMB(true, false, false);
        else if (out_bf16) TW_COMB(false, true, false);
        else TW_COMB(false, false, false);
    }
#undef TW_COMB
}

inline hipStream_t S(void *s) { return static_cast<hipStream_t>(s); }

// Router logits of T tokens; with quant_planes > 0 the first expert group of workgroups also writes
// the tokens' activation codes (quant_planes = 1: int8 absmax, 2 or 3: digit planes) and scale words.
void launch_router(const void *x, int x_bf16, const void *wr, int w_bf16, int64_t T, const Dims &dm,
                   float *logits, void *stream, int quant_planes = 0, int8_t *xdig = nullptr,
                   float *tinfo = nullptr)
{
    const dim3 grid(unsigned((dm.E + kRouteExp - 1) / kRouteExp), unsigned((T + kRouteTok - 1) / kRouteTok));
#define TW_ROUTE(NCH, QP) k_route<NCH, QP><<<grid, 256, 0, S(stream)>>>(x, x_bf16, wr, w_bf16, T, dm.d, dm.E, dm.pre_norm, logits, xdig, tinfo)
    if (dm.d <= 2048) {
        switch (quant_planes) {
        case 1: TW_ROUTE(1, 1); break;
        case 2: TW_ROUTE(1, 2); break;
        case 3: TW_ROUTE(1, 3); break;
        default: TW_ROUTE(1, 0); break;
        }
    } else {
        switch (quant_planes) {
        case 1: TW_ROUTE(2, 1); break;
        case 2: TW_ROUTE(2, 2); break;
        case 3: TW_ROUTE(2, 3); break;
        default: TW_ROUTE(2, 0); break;
        }
    }
#undef TW_ROUTE
}

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
    k_zero_u32<<<1, 64, 0, S(stream)>>>(reinterpret_cast<uint32_t *>(w + a.L.err), 4);   // health word
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
    const bool routed = ids != nullptr;   // routing passed in: the activation codes are made here
    if (!ids) {
        // routing inside: the router also writes the activation codes
        float *logits = reinterpret_cast<float *>(w + a.L.logits);
        int32_t *wid = reinterpret_cast<int32_t *>(w + a.L.ids);
        float *wg = reinterpret_cast<float *>(w + a.L.gates);
        launch_router(x_in, in_bf16, lp.w_router, dm.router_bf16, T, dm, logits, stream, P,
                      reinterpret_cast<int8_t *>(w + a.L.xdig), reinterpret_cast<float *>(w + a.L.tinfo));
        launch_topk(logits, T, dm.E, dm.k, wid, wg, stream);
        ids = wid;
        gates = wg;
    }
    int tile = kTileTokens;
    const bool mfma = grouped_mfma_serves(dm, T, P, &tile);
    // small batches on the matrix cores: each expert's workgroup finds its own tokens, no grouping
    const bool self = mfma && grouped_mfma_self(dm, T, tile);
    const int tt = mfma ? tile : kTileTokens;
    bool grouped = false;
    if (routed) {
        if (self) {
            k_bat_quant_x<P, INT8><<<unsigned(T), 256, 0, S(stream)>>>(a, x_in, in_bf16, w);
        } else {
            const int r = launch_quant_group<P, INT8>(a, x_in, in_bf16, ids, w, tt, stream);
            if (r != 0) return r;
            grouped = true;
        }
    }
    if (mfma) {
        int r = self || grouped ? 0 : launch_group(a, ids, w, tile, stream);
        if (r != 0) return r;
        r = launch_grouped_mfma(dm, lp, T, P, tile, a.L, w, self ? ids : nullptr, stream);
        if (r != 0) return r;
        // int8 activations in 64-token tiles: the grouped kernel stored 16-bit down sums
        launch_combine(a, x_in, in_bf16, x_out, out_bf16, ids, gates, w,
                       INT8 && tile >= 64 ? lp.s_down : nullptr, stream);
        return last_error();
    }
    const int rg = grouped ? 0 : launch_group(a, ids, w, kTileTokens, stream);
    if (rg != 0) return rg;
    const int tg = tokens_per_round(P * dm.d), td = tokens_per_round(P * dm.F);
    if (dm.d <= 2048)
        k_bat_gu<P, INT8, 4><<<kBatG, 256, size_t(tg) * P * dm.d, S(stream)>>>(a, lp, w, tg);
    else
        k_bat_gu<P, INT8, 8><<<kBatG, 256, size_t(tg) * P * dm.d, S(stream)>>>(a, lp, w, tg);
    if (dm.F <= 512)
        k_bat_dn<P, INT8, 2><<<kBatG, 256, size_t(td) * P * dm.F, S(stream)>>>(a, lp, w, td);
    else
        k_bat_dn<P, INT8, 16><<<kBatG, 256, size_t(td) * P * dm.F, S(stream)>>>(a, lp, w, td);
    launch_combine(a, x_in, in_bf16, x_out, out_bf16, ids, gates, w, nullptr, stream);
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

int launch_quantize(const void *w, int w_bf16, int64_t rows, int64_t cols, uint8_t *packed,
                    float *scales, void *stream)
{
    if (cols <= 512) {   // at most 64 chunks: four rows per wave
        const int64_t nb64 = (rows + 15) / 16;
        const unsigned nb = unsigned(nb64 < 65536 ? nb64 : 65536);
        if (w_bf16)
            k_quant_absmean16<true><<<nb, 256, 0, S(stream)>>>(w, rows, int(cols), packed, scales);
        else
            k_quant_absmean16<false><<<nb, 256, 0, S(stream)>>>(w, rows, int(cols), packed, scales);
        return last_error();
    }
    const int64_t nb64 = (rows + 3) / 4;
    const unsigned nb = unsigned(nb64 < 65536 ? nb64 : 65536);
    if (w_bf16)
        k_quant_absmean<true><<<nb, 256, 0, S(stream)>>>(w, rows, int(cols), packed, scales);
    else
        k_quant_absmean<false><<<nb, 256, 0, S(stream)>>>(w, rows, int(cols), packed, scales);
    return last_error();
}

int launch_route(const void *x, int x_bf16, const void *w_router, int w_bf16, int64_t T,
                 const Dims &dm, float *logits, int32_t *ids, float *gates, void *stream)
{
    launch_router(x, x_bf16, w_router, w_bf16, T, dm, logits, stream);
    launch_topk(logits, T, dm.E, dm.k, ids, gates, stream);
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
