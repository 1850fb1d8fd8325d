// INT4 GEMV over two rows of x at once: the w4_gemm path at M = 2 (two
// decode tokens).
//
// "Lab 5: Gemma4 端到端推理优化", section "INT4 融合 GEMV": the fused kernel
// reads the packed weights once, unpacks them in registers and applies scale
// and zero per group.  With M rows of x the same weight word serves M dot
// products, so this kernel is the M = 1 GEMV (gemv_int4.hip) with every
// unpacked word dotted with each row of x before the next word: the weights
// are still read once with 16-byte loads, and the unpack (7 integer
// operations per word) is shared by the M rows.
//   * Lane l owns chunks l, l + 64, ... of its K-slice for all M rows of x,
//     kept in registers as bf16 pairs with their per-chunk sums (so K is
//     limited to 2 chunks per lane: K <= 16384).
//   * Per weight row and chunk: unpack once, 4 dot2 per word and row of x,
//     then the group's zero and scale as in the GEMV:
//     sum_k (q - z) s x = s (sum_k (128 + q) x - (128 + z) sum_k x).
//   * The RPT x M sums of a wave are reduced across lanes together; waves
//     that split a row combine through LDS in a fixed order.  No atomics.
//   * Measured on the decode shapes: M = 2 takes 11.3 / 11.8 us (K3840 ->
//     N15360 / K15360 -> N3840) against 15.5 / 13.6 us on the 16-row
//     matrix-core path.  Four rows (MX = 4, up to 198 VGPRs, two waves per
//     SIMD) took 16.0 / 16.4 us, slower than that path (15.7 / 14.0), and
//     fewer weight rows per wave to free registers was slower still (2 rows:
//     21-23 us, 1 row: 30-33 us: fewer loads in flight), so M >= 3 stays
//     there.
#include "gemv_common.hpp"
#include "tune.hpp"
#include "w4_internal.hpp"

namespace w4 {
namespace {

constexpr int kThreads = 256;

// sum over the chunk's 32 codes of (128 + q) * x_m for each of MX rows of x,
// the codes unpacked once.
template <int MX>
__device__ __forceinline__ void chunk_dot_rows(const u32x4_t w, const uint32_t (&xp)[MX][16], uint32_t bias,
                                               float (&d)[MX]) {
    const uint32_t words[4] = {w.x, w.y, w.z, w.w};
    float d0[MX], d1[MX];
#pragma unroll
    for (int m = 0; m < MX; ++m) d0[m] = d1[m] = 0.f;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        uint32_t t[4];
        int4_word_biased_pairs(words[p], bias, t);
#pragma unroll
        for (int m = 0; m < MX; ++m) {
            d0[m] = dot2_bf16(t[0], xp[m][4 * p + 0], d0[m]);
            d1[m] = dot2_bf16(t[1], xp[m][4 * p + 1], d1[m]);
            d0[m] = dot2_bf16(t[2], xp[m][4 * p + 2], d0[m]);
            d1[m] = dot2_bf16(t[3], xp[m][4 * p + 3], d1[m]);
        }
    }
#pragma unroll
    for (int m = 0; m < MX; ++m) d[m] = d0[m] + d1[m];
}

// As gemv_int4_kernel, with MX rows of x (rows past M repeat row M - 1 and
// are not stored).
template <int S, int CPL, int RPT, int MX>
__global__ __launch_bounds__(kThreads) void gemv_rows_int4_kernel(
    const u32x4_t* __restrict__ qw, const uint16_t* __restrict__ s, const uint16_t* __restrict__ z,
    const u32x4_t* __restrict__ x, uint16_t* __restrict__ y, int M, int C, int N) {
    constexpr int T = 4 / S;      // row teams per workgroup
    constexpr int R = RPT * MX;   // sums per wave: (weight row, x row)
    // x staged once per workgroup in LDS when row teams share it (piece p of
    // chunk c of x row m at (m * 4 + p) * kXChunks + c, chunks past the row
    // end zeros), else loaded per wave.
    constexpr bool kStageX = T >= 2;
    constexpr int kXChunks = S * CPL * kWave;
    constexpr int kPerThread = MX * kXChunks * 4 / kThreads;
    static_assert(kXChunks * 4 % kThreads == 0, "whole pieces per thread");
    __shared__ float part[S][T * R];
    __shared__ u32x4_t xs[kStageX ? MX * 4 * kXChunks : 1];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int slice = wave % S;
    const int team = wave / S;
    const int G = C >> 2;
    const uint32_t row_bytes = (uint32_t)C * 16u;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(qw, (uint32_t)N * row_bytes);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(s, (uint32_t)N * (uint32_t)G * 2u);
    const __amdgpu_buffer_rsrc_t rz = make_rsrc(z, (uint32_t)N * (uint32_t)G * 2u);

    int c[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) c[i] = min(slice * kWave * CPL + i * kWave + lane, C - 1);

    // x first (small, cache-resident); a row of x is C chunks of 4 x 16 bytes
    // (reads past it return zeros).
    u32x4_t xload[kStageX ? kPerThread : MX * CPL * 4];
    if constexpr (kStageX) {
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const int q = threadIdx.x + kThreads * j;  // piece of x row q / (4 kXChunks)
            const int m = q / (4 * kXChunks), qq = q % (4 * kXChunks);
            const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + (size_t)min(m, M - 1) * (size_t)C * 4u, row_bytes * 4u);
            xload[j] = buf_load_b128(rx, (uint32_t)qq * 16u, 0u);
        }
    } else {
#pragma unroll
        for (int m = 0; m < MX; ++m) {
            const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + (size_t)min(m, M - 1) * (size_t)C * 4u, row_bytes * 4u);
#pragma unroll
            for (int i = 0; i < CPL; ++i)
#pragma unroll
                for (int p = 0; p < 4; ++p)
                    xload[(m * CPL + i) * 4 + p] =
                        buf_load_b128(rx, (uint32_t)(slice * kWave * CPL + i * kWave + lane) * 64u + 16u * p, 0u);
        }
    }

    // Scales and zeros before the weights: loads complete in issue order, so
    // row r's math can start as soon as row r's weights are in.
    const int row0 = (blockIdx.x * T + team) * RPT;
    u32x4_t wv[RPT][CPL];
    uint16_t sraw[RPT][CPL], zraw[RPT][CPL];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const uint32_t row = (uint32_t)min(row0 + r, N - 1);
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const uint32_t goff = (uint32_t)(c[i] >> 2) * 2u;
            sraw[r][i] = buf_load_u16(rs, goff, row * (uint32_t)G * 2u);
            zraw[r][i] = buf_load_u16(rz, goff, row * (uint32_t)G * 2u);
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
            const int q = threadIdx.x + kThreads * j;
            const int m = q / (4 * kXChunks), qq = q % (4 * kXChunks);  // piece qq % 4 of chunk qq / 4
            xs[(m * 4 + (qq & 3)) * kXChunks + (qq >> 2)] = xload[j];
        }
        __syncthreads();
    }

    uint32_t xp[CPL][MX][16];
    float sx[CPL][MX];
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
        for (int m = 0; m < MX; ++m) {
            const int cx = slice * kWave * CPL + i * kWave + lane;  // chunks past C read zeros
            u32x4_t xraw[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) xraw[p] = kStageX ? xs[(m * 4 + p) * kXChunks + cx] : xload[(m * CPL + i) * 4 + p];
            sx[i][m] = x_chunk_pairs(xraw, xp[i][m]);
        }

    const uint32_t bias = vgpr_const(kInt4BiasPair);
    float acc[R];  // acc[r * MX + m]
#pragma unroll
    for (int k = 0; k < R; ++k) acc[k] = 0.f;
#pragma unroll
    for (int r = 0; r < RPT; ++r)
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            float d[MX];
            chunk_dot_rows<MX>(wv[r][i], xp[i], bias, d);
            const float sc = f16_to_f32(sraw[r][i]);
            const float zb = f16_to_f32(zraw[r][i]) + 128.f;
#pragma unroll
            for (int m = 0; m < MX; ++m)
                acc[r * MX + m] = __builtin_fmaf(sc, __builtin_fmaf(-zb, sx[i][m], d[m]), acc[r * MX + m]);
        }

    const float total = reduce_rows<R>(acc, lane);  // lane L: sum L / (kWave / R)
    constexpr int kLanesPerSum = kWave / R;
    if ((lane % kLanesPerSum) == 0) part[slice][team * R + lane / kLanesPerSum] = total;
    __syncthreads();
    if (threadIdx.x < T * R) {
        float t = 0.f;
#pragma unroll
        for (int k = 0; k < S; ++k) t += part[k][threadIdx.x];
        const int f = threadIdx.x;  // team * R + r * MX + m
        const int m = f % MX;
        const int row = (blockIdx.x * T + f / R) * RPT + (f % R) / MX;
        if (row < N && m < M) y[(size_t)m * (size_t)N + row] = f32_to_bf16(t);
    }
}

template <int S, int CPL, int RPT, int MX>
hipError_t launch_shape(const void* x, const int32_t* qw, const void* s, const void* z, void* y, int M,
                        int C, int N, hipStream_t stream) {
    constexpr int T = 4 / S;
    const unsigned blocks = (unsigned)((N + T * RPT - 1) / (T * RPT));
    gemv_rows_int4_kernel<S, CPL, RPT, MX><<<blocks, kThreads, 0, stream>>>(
        reinterpret_cast<const u32x4_t*>(qw), static_cast<const uint16_t*>(s),
        static_cast<const uint16_t*>(z), static_cast<const u32x4_t*>(x), static_cast<uint16_t*>(y), M, C, N);
    return hipGetLastError();
}

// Rows per wave from the per-shape table (else the rule in tune.hip).
template <int S, int CPL, int MX>
hipError_t launch_rpt(const void* x, const int32_t* qw, const void* s, const void* z, void* y, int M, int C,
                      int N, hipStream_t stream) {
    switch (gemv_rows2_rows_per_wave(C * 32, N)) {
        case 8: return launch_shape<S, CPL, 8, MX>(x, qw, s, z, y, M, C, N, stream);
        case 4: return launch_shape<S, CPL, 4, MX>(x, qw, s, z, y, M, C, N, stream);
        case 2: return launch_shape<S, CPL, 2, MX>(x, qw, s, z, y, M, C, N, stream);
        default: return launch_shape<S, CPL, 1, MX>(x, qw, s, z, y, M, C, N, stream);
    }
}

template <int MX>
hipError_t launch_mx(const void* x, const int32_t* qw, const void* s, const void* z, void* y, int M, int C,
                     int N, hipStream_t stream) {
    const RowSplit rs = row_split(C);
    switch (rs.slices * 16 + rs.cpl) {
        case 1 * 16 + 1: return launch_rpt<1, 1, MX>(x, qw, s, z, y, M, C, N, stream);
        case 1 * 16 + 2: return launch_rpt<1, 2, MX>(x, qw, s, z, y, M, C, N, stream);
        case 2 * 16 + 2: return launch_rpt<2, 2, MX>(x, qw, s, z, y, M, C, N, stream);
        case 4 * 16 + 2: return launch_rpt<4, 2, MX>(x, qw, s, z, y, M, C, N, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool gemv_rows_int4_supports(int M, int K) {
    return M == 2 && K % 128 == 0 && K > 0 && row_split(K / 32).cpl <= 2;
}

hipError_t launch_gemv_rows_int4(const void* x, const int32_t* qw, const void* s, const void* z, void* y,
                                 int M, int K, int N, hipStream_t stream) {
    if (!gemv_rows_int4_supports(M, K)) return hipErrorInvalidValue;
    return launch_mx<2>(x, qw, s, z, y, M, K / 32, N, stream);
}

}  // namespace w4
