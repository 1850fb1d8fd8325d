// FP4 (E2M1) expert GEMVs, M = 1 per slot, with a BF16 scale per 32 along K.
//
// "DeepSeek V4 Triton FP4 优化实战", section "深度分析": item 2 -- the fused
// dequant+matmul pairs even columns with the low nibble and odd columns with
// the high nibble, and keeps the dequantised values in registers; item 4 --
// every token runs 2 FC x 6 active experts per layer, all bandwidth-bound.
//
// gfx950 design.  Same streaming structure as the INT4 GEMV: a row is C =
// K / 32 chunks of 16 bytes, and a chunk is exactly one scale group (32
// codes).  v_cvt_scalef32_pk_bf16_fp4 turns one byte (an even/odd k pair)
// into a bf16 pair, which lines up with x's own storage order (x[2i],
// x[2i+1]) in one register, so each byte costs one convert and one
// v_dot2_f32_bf16.  The chunk's BF16 scale multiplies the chunk's sum once.
// blockIdx.y selects the slot; its expert id is read on the device, and an id
// outside the pool turns that slot's outputs into NaN without touching any
// weight.
#include "w4_device.hpp"
#include "tune.hpp"
#include "w4_internal.hpp"


namespace w4 {
namespace {

constexpr int kThreads = 256;

// sum over the chunk's 32 codes of e2m1(code) * x.
__device__ __forceinline__ float chunk_dot(const u32x4_t w, const uint32_t xp[16]) {
    const uint32_t words[4] = {w.x, w.y, w.z, w.w};
    float d0 = 0.f, d1 = 0.f;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        uint32_t t[4];
        fp4_word_pairs(words[p], t);
        d0 = dot2_bf16(t[0], xp[4 * p + 0], d0);
        d1 = dot2_bf16(t[1], xp[4 * p + 1], d1);
        d0 = dot2_bf16(t[2], xp[4 * p + 2], d0);
        d1 = dot2_bf16(t[3], xp[4 * p + 3], d1);
    }
    return d0 + d1;
}

template <int S, int CPL, int RPT>
__global__ __launch_bounds__(kThreads) void moe_gemv_fp4_kernel(
    const u32x4_t* __restrict__ x, long x_stride_vec, const u32x4_t* __restrict__ qw,
    const uint16_t* __restrict__ s, const int32_t* __restrict__ ids, uint16_t* __restrict__ y,
    int C, int N, int num_experts) {
    constexpr int T = 4 / S;
    __shared__ float part[S][T * RPT];

    const int slot = blockIdx.y;
    const int expert = ids[slot];
    if (expert < 0 || expert >= num_experts) {  // uniform across the workgroup
        if (threadIdx.x < T * RPT) {
            const int row = blockIdx.x * (T * RPT) + threadIdx.x;
            if (row < N) y[(size_t)slot * N + row] = 0x7FC0u;  // bf16 quiet NaN
        }
        return;
    }

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int slice = wave % S;
    const int team = wave / S;
    const u32x4_t* xs = x + (size_t)slot * x_stride_vec;
    const uint32_t row_bytes = (uint32_t)C * 16u;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(qw + (size_t)expert * N * C, (uint32_t)N * row_bytes);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(s + (size_t)expert * N * C, (uint32_t)N * (uint32_t)C * 2u);

    // Clamped, branch-free loads (see the INT4 GEMV): x, then weights, then scales.
    int c[CPL];
    bool ok[CPL];
    u32x4_t xraw[CPL][4];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int ci = slice * kWave * CPL + i * kWave + lane;
        ok[i] = ci < C;
        c[i] = ok[i] ? ci : C - 1;
#pragma unroll
        for (int p = 0; p < 4; ++p) xraw[i][p] = xs[4 * c[i] + p];
    }

    const int row0 = (blockIdx.x * T + team) * RPT;
    u32x4_t wv[RPT][CPL];
    uint16_t sraw[RPT][CPL];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const uint32_t row = (uint32_t)min(row0 + r, N - 1);
#pragma unroll
        for (int i = 0; i < CPL; ++i)
            wv[r][i] = buf_load_b128<kAuxNontemporal>(rw, (uint32_t)c[i] * 16u, row * row_bytes);
    }
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const uint32_t row = (uint32_t)min(row0 + r, N - 1);
#pragma unroll
        for (int i = 0; i < CPL; ++i) sraw[r][i] = buf_load_u16(rs, (uint32_t)c[i] * 2u, row * (uint32_t)C * 2u);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep every load above ahead of the math below

    uint32_t xp[CPL][16];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            xp[i][4 * p + 0] = ok[i] ? xraw[i][p].x : 0u;
            xp[i][4 * p + 1] = ok[i] ? xraw[i][p].y : 0u;
            xp[i][4 * p + 2] = ok[i] ? xraw[i][p].z : 0u;
            xp[i][4 * p + 3] = ok[i] ? xraw[i][p].w : 0u;
        }
    }
    float sv[RPT][CPL];
#pragma unroll
    for (int r = 0; r < RPT; ++r)
#pragma unroll
        for (int i = 0; i < CPL; ++i) sv[r][i] = bf16_to_f32(sraw[r][i]);

    float acc[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        acc[r] = 0.f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) acc[r] = __builtin_fmaf(sv[r][i], chunk_dot(wv[r][i], xp[i]), acc[r]);
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
        if (row < N) y[(size_t)slot * N + row] = f32_to_bf16(t);
    }
}

template <int S, int CPL, int RPT>
hipError_t launch_shape(const void* x, int64_t x_stride, const uint8_t* qw, const void* s,
                        const int32_t* ids, void* y, int E, int num_experts, int C, int N,
                        hipStream_t stream) {
    constexpr int T = 4 / S;
    const dim3 grid((unsigned)((N + T * RPT - 1) / (T * RPT)), (unsigned)E);
    moe_gemv_fp4_kernel<S, CPL, RPT><<<grid, kThreads, 0, stream>>>(
        static_cast<const u32x4_t*>(x), (long)(x_stride / 8), reinterpret_cast<const u32x4_t*>(qw),
        static_cast<const uint16_t*>(s), ids, static_cast<uint16_t*>(y), C, N, num_experts);
    return hipGetLastError();
}

// Rows per wave from the per-shape table (else the rule in tune.hip).
template <int S, int CPL>
hipError_t launch_rpt(const void* x, int64_t x_stride, const uint8_t* qw, const void* s,
                      const int32_t* ids, void* y, int E, int num_experts, int C, int N,
                      hipStream_t stream) {
    switch (moe_gemv_rows_per_wave(E, C * 32, N)) {
        case 4: return launch_shape<S, CPL, 4>(x, x_stride, qw, s, ids, y, E, num_experts, C, N, stream);
        case 2: return launch_shape<S, CPL, 2>(x, x_stride, qw, s, ids, y, E, num_experts, C, N, stream);
        default: return launch_shape<S, CPL, 1>(x, x_stride, qw, s, ids, y, E, num_experts, C, N, stream);
    }
}

}  // namespace

hipError_t launch_moe_gemv_fp4(const void* x, int64_t x_stride, const uint8_t* qw, const void* s,
                               const int32_t* ids, void* y, int E, int num_experts, int K, int N,
                               hipStream_t stream) {
    const int C = K / 32;
    const RowSplit rs = row_split(C);
    switch (rs.slices * 16 + rs.cpl) {
        case 1 * 16 + 1: return launch_rpt<1, 1>(x, x_stride, qw, s, ids, y, E, num_experts, C, N, stream);
        case 1 * 16 + 2: return launch_rpt<1, 2>(x, x_stride, qw, s, ids, y, E, num_experts, C, N, stream);
        case 2 * 16 + 2: return launch_rpt<2, 2>(x, x_stride, qw, s, ids, y, E, num_experts, C, N, stream);
        case 4 * 16 + 2: return launch_rpt<4, 2>(x, x_stride, qw, s, ids, y, E, num_experts, C, N, stream);
        case 4 * 16 + 3: return launch_rpt<4, 3>(x, x_stride, qw, s, ids, y, E, num_experts, C, N, stream);
        case 4 * 16 + 4: return launch_rpt<4, 4>(x, x_stride, qw, s, ids, y, E, num_experts, C, N, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace w4
