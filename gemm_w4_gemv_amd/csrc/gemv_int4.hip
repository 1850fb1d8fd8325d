// Decode GEMV (M = 1) over packed INT4 weights with an FP16 scale and zero per
// 128 along K.
//
// "Lab 5: Gemma4 端到端推理优化", section "INT4 融合 GEMV": the decode linear
// sees a [1, hidden] input; the fused kernel reads the packed weights once,
// unpacks them in registers, applies scale and zero per group and dots with
// the input vector, keeping that vector in registers or shared memory.
//
// gfx950 design.  The kernel is bound by HBM: every weight byte is read once
// with 16-byte (dwordx4) loads and nothing else of size is touched.
//   * A row of K codes is C = K / 32 chunks of 16 bytes.  Lane l of a wave
//     owns chunks l, l + 64, ... of its K-slice, so each load instruction of
//     a wave reads 1 KiB of consecutive memory, and the lane's part of x
//     never changes: it is loaded once and kept in registers as bf16 pairs.
//   * Unpacking uses the bf16 bias trick: 0x4300 | q is the bf16 value
//     128 + q, and one mask pulls two nibbles 16 bits apart, so a word of 8
//     codes becomes 4 bf16 pairs in 7 integer operations, and
//     v_dot2_f32_bf16 multiplies and adds two codes per instruction.
//   * Scale and zero enter once per 32-code chunk (a chunk lies in one
//     group): sum_k (q - z) s x = s (sum_k (128 + q) x - (128 + z) sum_k x),
//     where sum_k x per chunk is precomputed with the x registers.
//   * Each wave carries RPT rows at once (RPT x CPL loads in flight per
//     lane), reduces them across lanes with a halving exchange, and the
//     waves that split one row (long K) combine through LDS in a fixed
//     order.  No atomics: results are bit-reproducible.
#include "gemv_common.hpp"
#include "tune.hpp"
#include "w4_internal.hpp"

namespace w4 {
namespace {

constexpr int kThreads = 256;

// All loads are issued before any of their results is used, from offsets
// clamped into the arrays, so a wave keeps RPT x CPL weight loads in flight
// without branches.  Clamped duplicates are harmless: a chunk past the row
// end gets x = 0 (contributes nothing) and a row past N is never stored.
// Weights are read with buffer loads: the row offset is wave-uniform (SGPR),
// the lane offset 32-bit.
//
// x is staged once per workgroup in LDS (each workgroup's waves share it):
// thread t loads 16-byte pieces t, t + 256, ... of x (coalesced, issued
// before the weights), piece p of chunk c lands at p * kXChunks + c, and
// chunks past the row end are zeros.  Each row's scales and zeros come from
// one load per row (two past 32 groups per K-slice): lane l < 32 loads the
// scale of the slice's group l, lane l >= 32 the zero of group l - 32, and a
// lane gathers its chunk's pair with ds_bpermute.  Loading x per wave and
// two 2-byte values per chunk and row instead read 8 KB of x per wave from
// L2 and issued four scale/zero load instructions per row: each cost 13-15 %
// of the logits GEMV's time.
template <int S, int CPL, int RPT>
__global__ __launch_bounds__(kThreads) void gemv_int4_kernel(
    const u32x4_t* __restrict__ qw, const uint16_t* __restrict__ s, const uint16_t* __restrict__ z,
    const u32x4_t* __restrict__ x, uint16_t* __restrict__ y, int C, int N) {
    constexpr int T = 4 / S;                    // row teams per workgroup
    constexpr int kXChunks = S * CPL * kWave;   // staged chunks (the row, padded)
    constexpr int kPerThread = kXChunks * 4 / kThreads;  // 16-byte pieces each thread stages
    constexpr int kSliceGroups = CPL * kWave / 4;
    constexpr bool kOneSZ = kSliceGroups <= 32;  // scale and zero of a row in one load
    // Staging pays when several row teams share x; with one team (a row cut
    // over all four waves) each wave loads its own slice straight into
    // registers.
    constexpr bool kStageX = T >= 2;
    static_assert(kXChunks * 4 % kThreads == 0, "whole pieces per thread");
    __shared__ u32x4_t xs[kStageX ? 4 * kXChunks : 1];
    __shared__ float part[S][T * RPT];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int slice = wave % S;
    const int team = wave / S;
    const int G = C >> 2;  // groups of 128 per row
    const uint32_t row_bytes = (uint32_t)C * 16u;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(qw, (uint32_t)N * row_bytes);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, row_bytes * 4u);  // C chunks of 64 bytes; past them reads 0
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(s, (uint32_t)N * (uint32_t)G * 2u);
    const __amdgpu_buffer_rsrc_t rz = make_rsrc(z, (uint32_t)N * (uint32_t)G * 2u);

    // x first: its loads complete before the weights', which are issued after it.
    u32x4_t xload[kStageX ? kPerThread : 4 * CPL];
    if constexpr (kStageX) {
#pragma unroll
        for (int j = 0; j < kPerThread; ++j)
            xload[j] = buf_load_b128(rx, (uint32_t)(threadIdx.x + kThreads * j) * 16u, 0u);
    } else {
#pragma unroll
        for (int i = 0; i < CPL; ++i)
#pragma unroll
            for (int p = 0; p < 4; ++p)
                xload[4 * i + p] = buf_load_b128(rx, (uint32_t)(slice * kWave * CPL + i * kWave + lane) * 64u + 16u * p, 0u);
    }

    int c[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) c[i] = min(slice * kWave * CPL + i * kWave + lane, C - 1);

    const int row0 = (blockIdx.x * T + team) * RPT;
    u32x4_t wv[RPT][CPL];
    uint32_t sz0[RPT], sz1[RPT];
    // Scales and zeros before the weights: the rows' math waits for them,
    // and loads complete in issue order, so row r's math can start as soon
    // as row r's weights are in.
    const int g0 = slice * kSliceGroups;
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const uint32_t roff = (uint32_t)min(row0 + r, N - 1) * (uint32_t)G * 2u;
        if constexpr (kOneSZ) {
            const uint32_t goff = (uint32_t)min(g0 + (lane & 31), G - 1) * 2u;
            // Lanes 0-31 read the scale, 32-63 the zero: two buffers, each lane
            // in range for one of them only (the other read returns 0).
            sz0[r] = (uint32_t)buf_load_u16(rs, lane < 32 ? goff : 0x80000000u, roff) |
                     (uint32_t)buf_load_u16(rz, lane < 32 ? 0x80000000u : goff, roff);
        } else {
            const uint32_t goff = (uint32_t)min(g0 + lane, G - 1) * 2u;
            sz0[r] = buf_load_u16(rs, goff, roff);
            sz1[r] = buf_load_u16(rz, goff, roff);
        }
    }
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const uint32_t row = (uint32_t)min(row0 + r, N - 1);
#pragma unroll
        for (int i = 0; i < CPL; ++i)
            wv[r][i] = buf_load_b128<kAuxNontemporal>(rw, (uint32_t)c[i] * 16u, row * row_bytes);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep every load above ahead of the math below

    if constexpr (kStageX) {
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const int q = threadIdx.x + kThreads * j;  // piece p = q % 4 of chunk q / 4
            xs[(q & 3) * kXChunks + (q >> 2)] = xload[j];
        }
        __syncthreads();
    }

    uint32_t xp[CPL][16];
    float sx[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        u32x4_t xraw[4];
        const int cx = slice * kWave * CPL + i * kWave + lane;  // chunks past C read zeros
#pragma unroll
        for (int p = 0; p < 4; ++p) xraw[p] = kStageX ? xs[p * kXChunks + cx] : xload[4 * i + p];
        sx[i] = x_chunk_pairs(xraw, xp[i]);
    }

    const uint32_t bias = vgpr_const(kInt4BiasPair);
    float acc[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        acc[r] = 0.f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int gi = 16 * i + (lane >> 2);  // the chunk's group within the slice
            uint32_t sb, zbits;
            if constexpr (kOneSZ) {
                sb = (uint32_t)__shfl((int)sz0[r], gi, kWave);
                zbits = (uint32_t)__shfl((int)sz0[r], 32 + gi, kWave);
            } else {
                sb = (uint32_t)__shfl((int)sz0[r], gi, kWave);
                zbits = (uint32_t)__shfl((int)sz1[r], gi, kWave);
            }
            const float d = chunk_dot(wv[r][i], xp[i], bias);
            const float zb = f16_to_f32((uint16_t)zbits) + 128.f;
            acc[r] = __builtin_fmaf(f16_to_f32((uint16_t)sb), __builtin_fmaf(-zb, sx[i], d), acc[r]);
        }
    }

    const float total = reduce_rows<RPT>(acc, lane);
    constexpr int kLanesPerRow = kWave / RPT;
    if ((lane % kLanesPerRow) == 0) part[slice][team * RPT + lane / kLanesPerRow] = total;
    __syncthreads();
    if (threadIdx.x < T * RPT) {
        float t = 0.f;
#pragma unroll
        for (int k = 0; k < S; ++k) t += part[k][threadIdx.x];
        const int row = blockIdx.x * (T * RPT) + threadIdx.x;
        if (row < N) y[row] = f32_to_bf16(t);
    }
}

template <int S, int CPL, int RPT>
hipError_t launch_shape(const void* x, const int32_t* qw, const void* s, const void* z, void* y,
                        int C, int N, hipStream_t stream) {
    constexpr int T = 4 / S;
    const int rows_per_block = T * RPT;
    const unsigned blocks = (unsigned)((N + rows_per_block - 1) / rows_per_block);
    gemv_int4_kernel<S, CPL, RPT><<<blocks, kThreads, 0, stream>>>(
        reinterpret_cast<const u32x4_t*>(qw), static_cast<const uint16_t*>(s),
        static_cast<const uint16_t*>(z), static_cast<const u32x4_t*>(x),
        static_cast<uint16_t*>(y), C, N);
    return hipGetLastError();
}

// Rows per wave from the per-shape table (else the rule in tune.hip).
template <int S, int CPL>
hipError_t launch_rpt(const void* x, const int32_t* qw, const void* s, const void* z, void* y,
                      int C, int N, hipStream_t stream) {
    switch (gemv_rows_per_wave(C * 32, N)) {
        case 8: return launch_shape<S, CPL, 8>(x, qw, s, z, y, C, N, stream);
        case 4: return launch_shape<S, CPL, 4>(x, qw, s, z, y, C, N, stream);
        case 2: return launch_shape<S, CPL, 2>(x, qw, s, z, y, C, N, stream);
        default: return launch_shape<S, CPL, 1>(x, qw, s, z, y, C, N, stream);
    }
}

}  // namespace

hipError_t launch_gemv_int4(const void* x, const int32_t* qw, const void* s, const void* z,
                            void* y, int K, int N, hipStream_t stream) {
    const int C = K / 32;
    const RowSplit rs = row_split(C);
    switch (rs.slices * 16 + rs.cpl) {
        case 1 * 16 + 1: return launch_rpt<1, 1>(x, qw, s, z, y, C, N, stream);
        case 1 * 16 + 2: return launch_rpt<1, 2>(x, qw, s, z, y, C, N, stream);
        case 2 * 16 + 2: return launch_rpt<2, 2>(x, qw, s, z, y, C, N, stream);
        case 4 * 16 + 2: return launch_rpt<4, 2>(x, qw, s, z, y, C, N, stream);
        case 4 * 16 + 3: return launch_rpt<4, 3>(x, qw, s, z, y, C, N, stream);
        case 4 * 16 + 4: return launch_rpt<4, 4>(x, qw, s, z, y, C, N, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace w4
