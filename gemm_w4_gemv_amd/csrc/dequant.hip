// Test-only dequantisers.  They expose, bit for bit, the operands the hot
// kernels build from the packed formats, by calling the same device routines:
//   * int4_word_dequant_bf16 is the prefill GEMM's matrix-core B operand
//     (and int4_word_dequant_f32 the FP32 values it rounds);
//   * int4_word_biased_pairs with x_pairs_for_biased are the operands of the
//     GEMV, the decode chain, the two-row GEMV and the small-M GEMM (the
//     biased codes 128 + q as bf16 pairs, and x in the matching pair order);
//   * fp4_word_pairs is the unpack of the FP4 expert GEMV and grouped GEMM.
// Comparing these outputs with an independent reference checks nibble order,
// group indexing, zero point, scale and BF16 rounding of the real code.
#include "w4_device.hpp"
#include "w4_internal.hpp"

namespace w4 {
namespace {

// One thread per packed word (8 weights).
__global__ __launch_bounds__(256) void dequant_int4_kernel(const uint32_t* __restrict__ qw,
                                                           const uint16_t* __restrict__ s,
                                                           const uint16_t* __restrict__ z,
                                                           float* __restrict__ out_f32,
                                                           uint16_t* __restrict__ out_bf16, int K,
                                                           size_t words) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= words) return;
    const int wpr = K / 8;
    const size_t n = i / wpr;
    const int p = (int)(i % wpr);
    const size_t g = n * (K / 128) + p / 16;
    const float sc = f16_to_f32(s[g]);
    const float nzs = -f16_to_f32(z[g]) * sc;  // as the GEMM forms it
    const size_t o = n * K + 8 * (size_t)p;
    if (out_f32) {
        float f[8];
        int4_word_dequant_f32(qw[i], sc, nzs, f);
#pragma unroll
        for (int j = 0; j < 8; ++j) out_f32[o + j] = f[j];
    }
    if (out_bf16) {
        const u32x4_t b = int4_word_dequant_bf16(qw[i], sc, nzs);
        const uint32_t v[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            out_bf16[o + 2 * j] = (uint16_t)(v[j] & 0xFFFFu);
            out_bf16[o + 2 * j + 1] = (uint16_t)(v[j] >> 16);
        }
    }
}

// One thread per packed word: the four biased code pairs the GEMV-path
// kernels dot with x (pair j = (128 + q_{8p+j}, 128 + q_{8p+j+4}) as bf16)
// and, for row 0's thread of each word, the four x pairs they are dotted
// with, in the same order.
__global__ __launch_bounds__(256) void int4_gemv_operands_kernel(const uint32_t* __restrict__ qw,
                                                                 const uint32_t* __restrict__ x,
                                                                 uint32_t* __restrict__ out_codes,
                                                                 uint32_t* __restrict__ out_x, int K,
                                                                 size_t words) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= words) return;
    const uint32_t bias = vgpr_const(kInt4BiasPair);
    uint32_t t[4];
    int4_word_biased_pairs(qw[i], bias, t);
#pragma unroll
    for (int j = 0; j < 4; ++j) out_codes[4 * i + j] = t[j];
    const int wpr = K / 8;
    if (out_x && i < (size_t)wpr) {  // word p of x: its eight bf16 values as four words
        const uint32_t xw[4] = {x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]};
        uint32_t xp[4];
        x_pairs_for_biased(xw, xp);
#pragma unroll
        for (int j = 0; j < 4; ++j) out_x[4 * i + j] = xp[j];
    }
}

// One thread per 4 bytes (8 codes); all 8 codes share one scale (32 per group).
__global__ __launch_bounds__(256) void dequant_fp4_kernel(const uint32_t* __restrict__ qw,
                                                          const uint16_t* __restrict__ s,
                                                          float* __restrict__ out_f32,
                                                          uint16_t* __restrict__ out_bf16, int K,
                                                          size_t words) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= words) return;
    const int wpr = K / 8;
    const size_t n = i / wpr;
    const int p = (int)(i % wpr);
    const float sc = bf16_to_f32(s[n * (K / 32) + p / 4]);
    uint32_t t[4];
    fp4_word_pairs(qw[i], t);
    const size_t o = n * K + 8 * (size_t)p;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const float lo = bf16_to_f32(t[b] & 0xFFFFu) * sc;  // exact: 2 x 8 significant bits
        const float hi = bf16_to_f32(t[b] >> 16) * sc;
        if (out_f32) {
            out_f32[o + 2 * b] = lo;
            out_f32[o + 2 * b + 1] = hi;
        }
        if (out_bf16) {
            out_bf16[o + 2 * b] = f32_to_bf16(lo);
            out_bf16[o + 2 * b + 1] = f32_to_bf16(hi);
        }
    }
}

}  // namespace

hipError_t launch_dequant_int4(const int32_t* qw, const void* s, const void* z, float* out_f32,
                               void* out_bf16, int K, int N, hipStream_t stream) {
    const size_t words = (size_t)N * (K / 8);
    const unsigned blocks = (unsigned)((words + 255) / 256);
    dequant_int4_kernel<<<blocks, 256, 0, stream>>>(
        reinterpret_cast<const uint32_t*>(qw), static_cast<const uint16_t*>(s),
        static_cast<const uint16_t*>(z), out_f32, static_cast<uint16_t*>(out_bf16), K, words);
    return hipGetLastError();
}

hipError_t launch_int4_gemv_operands(const int32_t* qw, const void* x, uint32_t* out_codes, uint32_t* out_x, int K,
                                     int N, hipStream_t stream) {
    const size_t words = (size_t)N * (K / 8);
    const unsigned blocks = (unsigned)((words + 255) / 256);
    int4_gemv_operands_kernel<<<blocks, 256, 0, stream>>>(reinterpret_cast<const uint32_t*>(qw),
                                                           static_cast<const uint32_t*>(x), out_codes, out_x, K,
                                                           words);
    return hipGetLastError();
}

hipError_t launch_dequant_fp4(const uint8_t* qw, const void* s, float* out_f32, void* out_bf16,
                              int K, int N, hipStream_t stream) {
    const size_t words = (size_t)N * (K / 8);
    const unsigned blocks = (unsigned)((words + 255) / 256);
    dequant_fp4_kernel<<<blocks, 256, 0, stream>>>(
        reinterpret_cast<const uint32_t*>(qw), static_cast<const uint16_t*>(s), out_f32,
        static_cast<uint16_t*>(out_bf16), K, words);
    return hipGetLastError();
}

}  // namespace w4
