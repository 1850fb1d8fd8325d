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

// One FC of expert GEMVs: slot e's x at x + e * x_stride_vec (16-byte
// units), weights and scales of the pool, output y [E][N].
struct MoeFc {
    const u32x4_t* x;
    long x_stride_vec;
    const u32x4_t* qw;
    const uint16_t* s;
    uint16_t* y;
    int C, N;
};

// Rows [bx T RPT, (bx + 1) T RPT) of slot ``slot``: the work of one workgroup.
// x is loaded before the expert id is known (it depends on the slot only);
// when several row teams share it, it is staged once per workgroup in LDS
// (thread t loads 16-byte pieces t, t + 256, ...; piece p of chunk c lands
// at p * S * CPL * 64 + c, chunks past the row end read zeros), else each
// wave loads its own slice.
template <int S, int CPL, int RPT>
__device__ __forceinline__ void moe_gemv_rows(const MoeFc& f, const int32_t* __restrict__ ids, int num_experts,
                                              int bx, int slot, float (&part)[S][(4 / S) * RPT], u32x4_t* xs) {
    constexpr int T = 4 / S;
    constexpr bool kStageX = T >= 2;
    constexpr int kXChunks = S * CPL * kWave;
    constexpr int kPerThread = kXChunks * 4 / kThreads;
    static_assert(kXChunks * 4 % kThreads == 0, "whole pieces per thread");
    const u32x4_t* __restrict__ qw = f.qw;
    const uint16_t* __restrict__ s = f.s;
    uint16_t* __restrict__ y = f.y;
    const int C = f.C, N = f.N;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int slice = wave % S;
    const int team = wave / S;
    const uint32_t row_bytes = (uint32_t)C * 16u;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(f.x + (size_t)slot * f.x_stride_vec, row_bytes * 4u);

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

    const int expert = ids[slot];
    if (expert < 0 || expert >= num_experts) {  // uniform across the workgroup
        if (threadIdx.x < T * RPT) {
            const int row = bx * (T * RPT) + threadIdx.x;
            if (row < N) y[(size_t)slot * N + row] = 0x7FC0u;  // bf16 quiet NaN
        }
        return;
    }
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(qw + (size_t)expert * N * C, (uint32_t)N * row_bytes);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(s + (size_t)expert * N * C, (uint32_t)N * (uint32_t)C * 2u);

    // Clamped, branch-free loads (see the INT4 GEMV): scales, then weights.
    int c[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) c[i] = min(slice * kWave * CPL + i * kWave + lane, C - 1);

    // Scales before the weights: loads complete in issue order, so row r's
    // math can start as soon as row r's weights are in.
    const int row0 = (bx * T + team) * RPT;
    u32x4_t wv[RPT][CPL];
    uint16_t sraw[RPT][CPL];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const uint32_t row = (uint32_t)min(row0 + r, N - 1);
#pragma unroll
        for (int i = 0; i < CPL; ++i) sraw[r][i] = buf_load_u16(rs, (uint32_t)c[i] * 2u, row * (uint32_t)C * 2u);
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
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int cx = slice * kWave * CPL + i * kWave + lane;  // chunks past C read zeros
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const u32x4_t v = kStageX ? xs[p * kXChunks + cx] : xload[4 * i + p];
            xp[i][4 * p + 0] = v.x;
            xp[i][4 * p + 1] = v.y;
            xp[i][4 * p + 2] = v.z;
            xp[i][4 * p + 3] = v.w;
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
        const int row = bx * (T * RPT) + threadIdx.x;
        if (row < N) y[(size_t)slot * N + row] = f32_to_bf16(t);
    }
}

template <int S, int CPL, int RPT>
__global__ __launch_bounds__(kThreads) void moe_gemv_fp4_kernel(MoeFc f, const int32_t* __restrict__ ids,
                                                                int num_experts) {
    __shared__ float part[S][(4 / S) * RPT];
    __shared__ u32x4_t xs[(4 / S) >= 2 ? 4 * S * CPL * kWave : 1];
    moe_gemv_rows<S, CPL, RPT>(f, ids, num_experts, blockIdx.x, blockIdx.y, part, xs);
}

// Two FCs over the same slots and expert ids in one launch: workgroups
// [0, b1) of each slot run the first FC, the rest the second.  One launch
// instead of two: the second FC's weights stream while the first's finish,
// with one ramp and one tail.
template <int CPL1, int CPL2, int RPT1, int RPT2>
__global__ __launch_bounds__(kThreads) void moe_gemv2_fp4_kernel(MoeFc f1, MoeFc f2, int b1,
                                                                 const int32_t* __restrict__ ids,
                                                                 int num_experts) {
    constexpr int R = RPT1 > RPT2 ? RPT1 : RPT2;
    __shared__ float part[4 * R];
    __shared__ u32x4_t xs[4 * (CPL1 > CPL2 ? CPL1 : CPL2) * kWave];
    if ((int)blockIdx.x < b1)
        moe_gemv_rows<1, CPL1, RPT1>(f1, ids, num_experts, blockIdx.x, blockIdx.y,
                                     *reinterpret_cast<float(*)[1][4 * RPT1]>(part), xs);
    else
        moe_gemv_rows<1, CPL2, RPT2>(f2, ids, num_experts, blockIdx.x - b1, blockIdx.y,
                                     *reinterpret_cast<float(*)[1][4 * RPT2]>(part), xs);
}

template <int S, int CPL, int RPT>
hipError_t launch_shape(const void* x, int64_t x_stride, const uint8_t* qw, const void* s,
                        const int32_t* ids, void* y, int E, int num_experts, int C, int N,
                        hipStream_t stream) {
    constexpr int T = 4 / S;
    const dim3 grid((unsigned)((N + T * RPT - 1) / (T * RPT)), (unsigned)E);
    const MoeFc f{static_cast<const u32x4_t*>(x), (long)(x_stride / 8), reinterpret_cast<const u32x4_t*>(qw),
                  static_cast<const uint16_t*>(s), static_cast<uint16_t*>(y), C, N};
    moe_gemv_fp4_kernel<S, CPL, RPT><<<grid, kThreads, 0, stream>>>(f, ids, num_experts);
    return hipGetLastError();
}

// Rows per wave from the per-shape table (else the rule in tune.hip).
template <int S, int CPL>
hipError_t launch_rpt(const void* x, int64_t x_stride, const uint8_t* qw, const void* s,
                      const int32_t* ids, void* y, int E, int num_experts, int C, int N,
                      hipStream_t stream) {
    switch (moe_gemv_rows_per_wave(E, C * 32, N)) {
        case 8: return launch_shape<S, CPL, 8>(x, x_stride, qw, s, ids, y, E, num_experts, C, N, stream);
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

namespace {

template <int CPL1, int CPL2, int RPT1, int RPT2>
hipError_t launch_pair(const MoeFc& f1, const MoeFc& f2, const int32_t* ids, int E, int num_experts,
                       hipStream_t stream) {
    const int b1 = (f1.N + 4 * RPT1 - 1) / (4 * RPT1), b2 = (f2.N + 4 * RPT2 - 1) / (4 * RPT2);
    moe_gemv2_fp4_kernel<CPL1, CPL2, RPT1, RPT2><<<dim3((unsigned)(b1 + b2), (unsigned)E), kThreads, 0, stream>>>(
        f1, f2, b1, ids, num_experts);
    return hipGetLastError();
}

template <int RPT1, int RPT2>
hipError_t launch_pair_cpl(const MoeFc& f1, const MoeFc& f2, const int32_t* ids, int E, int num_experts,
                           hipStream_t stream) {
    switch (row_split(f1.C).cpl * 16 + row_split(f2.C).cpl) {
        case 1 * 16 + 1: return launch_pair<1, 1, RPT1, RPT2>(f1, f2, ids, E, num_experts, stream);
        case 1 * 16 + 2: return launch_pair<1, 2, RPT1, RPT2>(f1, f2, ids, E, num_experts, stream);
        case 2 * 16 + 1: return launch_pair<2, 1, RPT1, RPT2>(f1, f2, ids, E, num_experts, stream);
        default: return launch_pair<2, 2, RPT1, RPT2>(f1, f2, ids, E, num_experts, stream);
    }
}

template <int RPT1>
hipError_t launch_pair_rpt(int rpt2, const MoeFc& f1, const MoeFc& f2, const int32_t* ids, int E,
                           int num_experts, hipStream_t stream) {
    switch (rpt2) {
        case 8: return launch_pair_cpl<RPT1, 8>(f1, f2, ids, E, num_experts, stream);
        case 4: return launch_pair_cpl<RPT1, 4>(f1, f2, ids, E, num_experts, stream);
        default: return launch_pair_cpl<RPT1, 2>(f1, f2, ids, E, num_experts, stream);
    }
}

}  // namespace

hipError_t launch_moe_gemv2_fp4(const MoeFcArgs& a, const MoeFcArgs& b, const int32_t* ids, int E, int num_experts,
                                hipStream_t stream) {
    // One launch when both rows fit one wave's slice (K <= 4096) and both
    // shapes take 2, 4 or 8 rows per wave (each FC its own, as in its own
    // launch); else the two FCs one after the other (same results, bit for
    // bit).  The first FC's workgroups come first in the grid, so the
    // launch's tail is the second FC's.
    const int Ca = a.K / 32, Cb = b.K / 32;
    const int pa = moe_gemv_rows_per_wave(E, a.K, a.N), pb = moe_gemv_rows_per_wave(E, b.K, b.N);
    auto pair_rpt = [](int p) { return p == 2 || p == 4 || p == 8; };
    if (row_split(Ca).slices != 1 || row_split(Cb).slices != 1 || !pair_rpt(pa) || !pair_rpt(pb)) {
        hipError_t err = launch_moe_gemv_fp4(a.x, a.x_stride, a.qw, a.s, ids, a.y, E, num_experts, a.K, a.N, stream);
        if (err != hipSuccess) return err;
        return launch_moe_gemv_fp4(b.x, b.x_stride, b.qw, b.s, ids, b.y, E, num_experts, b.K, b.N, stream);
    }
    const MoeFc f1{static_cast<const u32x4_t*>(a.x), (long)(a.x_stride / 8), reinterpret_cast<const u32x4_t*>(a.qw),
                   static_cast<const uint16_t*>(a.s), static_cast<uint16_t*>(a.y), Ca, a.N};
    const MoeFc f2{static_cast<const u32x4_t*>(b.x), (long)(b.x_stride / 8), reinterpret_cast<const u32x4_t*>(b.qw),
                   static_cast<const uint16_t*>(b.s), static_cast<uint16_t*>(b.y), Cb, b.N};
    switch (pa) {
        case 8: return launch_pair_rpt<8>(pb, f1, f2, ids, E, num_experts, stream);
        case 4: return launch_pair_rpt<4>(pb, f1, f2, ids, E, num_experts, stream);
        default: return launch_pair_rpt<2>(pb, f1, f2, ids, E, num_experts, stream);
    }
}

}  // namespace w4
