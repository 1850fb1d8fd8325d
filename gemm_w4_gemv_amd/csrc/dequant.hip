// Test-only dequantisers.  They expose, bit for bit, what the hot kernels
// compute from the packed formats: int4_word_dequant_f32 is the GEMM's
// weight-tile path and fp4_word_pairs is the FP4 GEMV's unpack, so a
// comparison of these outputs with an independent reference checks nibble
// order, group indexing, zero point, scale and BF16 rounding of the real code.
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
    float f[8];
    int4_word_dequant_f32(qw[i], f16_to_f32(s[g]), f16_to_f32(z[g]), f);
    const size_t o = n * K + 8 * (size_t)p;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (out_f32) out_f32[o + j] = f[j];
        if (out_bf16) out_bf16[o + j] = f32_to_bf16(f[j]);
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
