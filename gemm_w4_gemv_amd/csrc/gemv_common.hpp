// INT4 GEMV building blocks shared by the single-GEMV kernel and the
// persistent decode-chain kernel: per-chunk x staging and the per-chunk dot
// product of 32 packed codes with x (see gemv_int4.hip for the design).
#pragma once

#include "w4_device.hpp"

namespace w4 {

// x pairs for one chunk, matching int4_word_biased_pairs, and their FP32 sum.
// ``raw`` holds the chunk's 32 bf16 values x[32c .. 32c + 31] as loaded.
__device__ __forceinline__ float x_chunk_pairs(const u32x4_t raw[4], uint32_t xp[16]) {
    float sum = 0.f;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t xw[4] = {raw[p].x, raw[p].y, raw[p].z, raw[p].w};
        x_pairs_for_biased(xw, &xp[4 * p]);
#pragma unroll
        for (int i = 0; i < 4; ++i) sum += bf16_to_f32(xw[i] & 0xFFFFu) + bf16_to_f32(xw[i] >> 16);
    }
    return sum;
}

// sum over the chunk's 32 codes of (128 + q) * x.
__device__ __forceinline__ float chunk_dot(const u32x4_t w, const uint32_t xp[16], uint32_t bias) {
    const uint32_t words[4] = {w.x, w.y, w.z, w.w};
    float d0 = 0.f, d1 = 0.f;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        uint32_t t[4];
        int4_word_biased_pairs(words[p], bias, t);
        d0 = dot2_bf16(t[0], xp[4 * p + 0], d0);
        d1 = dot2_bf16(t[1], xp[4 * p + 1], d1);
        d0 = dot2_bf16(t[2], xp[4 * p + 2], d0);
        d1 = dot2_bf16(t[3], xp[4 * p + 3], d1);
    }
    return d0 + d1;
}

}  // namespace w4
