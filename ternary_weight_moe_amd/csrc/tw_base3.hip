// tw_base3.hip -- base-3 packing of ternary weights (five per byte) and an int8 ternary GEMV that
// reads either packed layout, so that the two can be measured against each other on one kernel
// structure.
//
// A ternary weight carries log2 3 = 1.585 bits of information; a layout that hardware reads
// natively spends 2 bits, or uses another aligned form ("iPhone Runs a 20B Model at 120 tok/s",
// section "Ternary Quantization Is More Than Simply Compressing Weights into Three Values").  Five
// trits fit in one byte (3^5 = 243 <= 256): 1.6 bits per weight, a 2048-weight row in 410 bytes
// (416 at a 16-byte row stride) instead of 512.
//
// Layout (base 3): byte j of a row holds weights 5j .. 5j+4 as sum_i (w_{5j+i} + 1) 3^i, weight 5j
// the least significant trit; positions at or past cols count as weight 0; rows are
// ternary_pack3_row_bytes(cols) = ceil(cols/5) rounded up to 16 bytes apart, their bytes past
// ceil(cols/5) are 0.
//
// GEMV: y_r = (float(sum_i W[r][i] q_i) * s_x) * s_r with int8 activation codes q and exact int32
// sums.  One 16-byte chunk of a row per lane; the lanes of a row form a power-of-two group (at most
// 64) and the row's sum is a DPP reduction inside it.  Each lane keeps the activations of its chunk
// in registers for the whole kernel: with the 2-bit layout, 16 int8x4 words in the 4x4-transposed
// order of the code words' decode (tw_device.h); with the base-3 layout, per code byte the word of
// its first four inputs, and per four code bytes the word of their fifth inputs.  A base-3 byte is
// decoded by a lookup in LDS: four tables of 256 eight-byte entries, one per byte position p of a
// 32-bit code word; entry v < 243 holds the int8 weights of trits 0..3 of v in its low word and the
// weight of trit 4 in byte p of its high word, so the fifth weights of four bytes are OR-ed into one
// word and take one v_dot4.  Bytes 243..255 are never written by the packer; their entries are zero.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tw_device.h"
#include "tw_aux.h"
#include "tw_internal.h"

namespace tw {
namespace {

__global__ void k_pack3(const int8_t *__restrict__ w, int64_t rows, int64_t cols, int64_t rb,
                        uint8_t *__restrict__ out, int32_t *bad)
{
    const int64_t nb = (cols + 4) / 5, n = rows * rb;
    int local_bad = 0;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * blockDim.x) {
        const int64_t r = i / rb, b = i % rb;
        uint32_t v = 0;
        if (b < nb) {
            uint32_t p3 = 1;
            for (int j = 0; j < 5; j++) {
                const int64_t c = 5 * b + j;
                const int x = c < cols ? int(w[r * cols + c]) : 0;
                const bool ok = x >= -1 && x <= 1;
                local_bad += !ok;
                v += uint32_t(ok ? x + 1 : 1) * p3;
                p3 *= 3;
            }
        }
        out[i] = uint8_t(v);
    }
    if (bad) {
        const float s = wave_sum(float(local_bad));
        if ((threadIdx.x & 63) == 0 && s > 0.0f) atomicAdd(bad, int32_t(s));
    }
}

constexpr int kGvWaves = 4;     // waves per workgroup
constexpr int kGvUnroll = 8;    // rows per lane group in flight
constexpr int kGvMaxChunks = 64;

__device__ __forceinline__ uint32_t bytes4(int a, int b, int c, int d)
{
    return (uint32_t(uint8_t(a))) | (uint32_t(uint8_t(b)) << 8) | (uint32_t(uint8_t(c)) << 16) |
           (uint32_t(uint8_t(d)) << 24);
}

// FMT 2: the 2-bit layout of ternary_pack; FMT 3: the base-3 layout above.  rb: row stride in
// bytes (a multiple of 16, at most 1024); lg: log2 of the lanes per row.
template <int FMT>
__global__ __launch_bounds__(64 * kGvWaves) void k_gemv_i8(const uint8_t *__restrict__ codes,
                                                            const float *__restrict__ scales,
                                                            int64_t rows, int cols, int rb, int lg,
                                                            const int8_t *__restrict__ xq,
                                                            const float *__restrict__ xs,
                                                            float *__restrict__ y)
{
    // activation words, per chunk in the order the lanes read them (16 words, and for base 3 the
    // 4 words of fifth inputs behind all chunks' first-four words)
    __shared__ uint32_t s_xw[kGvMaxChunks * 20];
    __shared__ uint2 s_lut[FMT == 3 ? 4 * 256 : 1];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int nc = rb >> 4;
    if constexpr (FMT == 3) {
        for (int e = t; e < 4 * 256; e += 64 * kGvWaves) {
            const int p = e >> 8, v = e & 255;
            uint2 ent = make_uint2(0u, 0u);
            if (v < 243) {
                const int d0 = v % 3, d1 = v / 3 % 3, d2 = v / 9 % 3, d3 = v / 27 % 3, d4 = v / 81;
                ent.x = bytes4(d0 - 1, d1 - 1, d2 - 1, d3 - 1);
                ent.y = uint32_t(uint8_t(d4 - 1)) << (8 * p);
            }
            s_lut[e] = ent;
        }
        // group g (code byte g of a row): inputs 5g .. 5g+4, zero past cols
        for (int g = t; g < 16 * nc; g += 64 * kGvWaves) {
            int v[5];
#pragma unroll
            for (int i = 0; i < 5; i++) v[i] = 5 * g + i < cols ? int(xq[5 * g + i]) : 0;
            s_xw[g] = bytes4(v[0], v[1], v[2], v[3]);
            reinterpret_cast<uint8_t *>(s_xw + 16 * kGvMaxChunks)[g] = uint8_t(v[4]);
        }
    } else {
        // chunk j, code word q, decoded word m: inputs 64 j + 16 q + 4 b + m for b = 0..3
        for (int i = t; i < 16 * nc; i += 64 * kGvWaves) {
            const int base = 64 * (i >> 4) + 16 * ((i >> 2) & 3), m = i & 3;
            s_xw[i] = bytes4(xq[base + m], xq[base + 4 + m], xq[base + 8 + m], xq[base + 12 + m]);
        }
    }
    __syncthreads();

    const int lpr = 1 << lg, rpw = 64 >> lg;
    const int j = lane & (lpr - 1), sub = lane >> lg;
    const bool act = j < nc;
    // lanes past the row's chunks hold zero activations (their zero code bytes would decode to
    // weights -1 in base 3)
    const int jj = act ? j : 0;
    uint32_t xw[16], xf[4];
#pragma unroll
    for (int i = 0; i < 16; i++) xw[i] = act ? s_xw[16 * jj + i] : 0u;
#pragma unroll
    for (int i = 0; i < 4; i++) xf[i] = FMT == 3 && act ? s_xw[16 * kGvMaxChunks + 4 * jj + i] : 0u;
    const float sx = xs[0];

    const int64_t per_wave = int64_t(rpw) * kGvUnroll;
    const int64_t step = int64_t(gridDim.x) * kGvWaves * per_wave;
    for (int64_t R = (int64_t(blockIdx.x) * kGvWaves + wave) * per_wave; R < rows; R += step) {
        int4 cv[kGvUnroll];
        float sc[kGvUnroll];
#pragma unroll
        for (int u = 0; u < kGvUnroll; u++) {
            const int64_t r = R + u * rpw + sub;
            cv[u] = act && r < rows ? *reinterpret_cast<const int4 *>(codes + r * rb + 16 * j)
                                    : make_int4(0, 0, 0, 0);
            sc[u] = j == 0 && r < rows ? scales[r] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kGvUnroll; u++) {
            int32_t acc[1] = {0};
            const uint32_t w4[4] = {uint32_t(cv[u].x), uint32_t(cv[u].y), uint32_t(cv[u].z),
                                    uint32_t(cv[u].w)};
#pragma unroll
            for (int q = 0; q < 4; q++) {
                if constexpr (FMT == 3) {
                    uint32_t hi = 0;
#pragma unroll
                    for (int p = 0; p < 4; p++) {
                        const uint2 e = s_lut[256 * p + ((w4[q] >> (8 * p)) & 255u)];
                        acc[0] = __builtin_amdgcn_sdot4(int32_t(e.x), int32_t(xw[4 * q + p]), acc[0], false);
                        hi |= e.y;
                    }
                    acc[0] = __builtin_amdgcn_sdot4(int32_t(hi), int32_t(xf[q]), acc[0], false);
                } else {
                    int32_t t0, t1, t2, t3;
                    decode_word(w4[q], t0, t1, t2, t3);
                    acc[0] = __builtin_amdgcn_sdot4(t0, int32_t(xw[4 * q + 0]), acc[0], false);
                    acc[0] = __builtin_amdgcn_sdot4(t1, int32_t(xw[4 * q + 1]), acc[0], false);
                    acc[0] = __builtin_amdgcn_sdot4(t2, int32_t(xw[4 * q + 2]), acc[0], false);
                    acc[0] = __builtin_amdgcn_sdot4(t3, int32_t(xw[4 * q + 3]), acc[0], false);
                }
            }
            group_reduce<1>(acc, lpr);
            const int64_t r = R + u * rpw + sub;
            if (j == 0 && r < rows) y[r] = (float(acc[0]) * sx) * sc[u];
        }
    }
}

}  // namespace

int launch_pack3(const int8_t *w, int64_t rows, int64_t cols, uint8_t *packed, int32_t *bad,
                 void *stream)
{
    const int64_t n = rows * pack3_row_bytes(cols);
    const unsigned nb = unsigned(n / 256 + 1 < 16384 ? n / 256 + 1 : 16384);
    k_pack3<<<nb, 256, 0, static_cast<hipStream_t>(stream)>>>(w, rows, cols, pack3_row_bytes(cols),
                                                              packed, bad);
    return int(hipGetLastError());
}

int launch_gemv_i8(const uint8_t *codes, int layout, const float *scales, int64_t rows, int cols,
                   const int8_t *xq, const float *x_scale, float *y, void *stream)
{
    const int rb = int(layout == 3 ? pack3_row_bytes(cols) : cols / 4);
    const int nc = rb / 16;
    if (rb % 16 || nc < 1 || nc > kGvMaxChunks) return int(hipErrorInvalidValue);
    int lg = 0;
    while ((1 << lg) < nc) lg++;
    const int64_t per_wave = int64_t(64 >> lg) * kGvUnroll;
    const int64_t nb64 = ((rows + per_wave - 1) / per_wave + kGvWaves - 1) / kGvWaves;
    const unsigned nb = unsigned(nb64 < 1024 ? nb64 : 1024);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (layout == 3)
        k_gemv_i8<3><<<nb, 64 * kGvWaves, 0, st>>>(codes, scales, rows, cols, rb, lg, xq, x_scale, y);
    else
        k_gemv_i8<2><<<nb, 64 * kGvWaves, 0, st>>>(codes, scales, rows, cols, rb, lg, xq, x_scale, y);
    return int(hipGetLastError());
}

}  // namespace tw
