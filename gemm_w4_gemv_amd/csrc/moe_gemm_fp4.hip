// Grouped FP4 (E2M1) expert GEMM: several tokens per expert.
//
// "DeepSeek V4 Triton FP4 优化实战", section "深度分析": item 2 -- the fused
// FP4 kernel is a matrix product whose weight tile is unpacked in registers
// (even k from the low nibble, odd k from the high nibble), never written out
// as BF16; item 4 -- the tokens of a layer are routed to experts, each
// applying its FCs.  Group e owns rows row_start[e] .. row_start[e+1] - 1 of
// x and applies expert ids[e] to them.
//
// gfx950 design (the structure of the small-M INT4 path):
//   * Grid: (weight-row tiles of 32 or 16 rows) x (slabs of 16 rows of a
//     group) x (groups).  A workgroup whose slab starts past its group's last
//     row exits at once; an expert id outside the pool turns the slab's
//     outputs into NaN without reading any weight.
//   * 4 waves split the K range in steps of 128 k; a wave issues and
//     computes exactly its own steps (a wave-uniform exit at the end of its
//     range).  Per step, lane (i, b) of
//     a column block loads 16 bytes (words 4b..4b+3, 8 codes per word) of
//     weight row i; a 4 x 4 transpose across the four 16-lane rows
//     (v_permlane32_swap, v_permlane16_swap) leaves word 4t + b in register
//     t, the B operand of k-slice t of v_mfma_f32_16x16x32_bf16.
//   * v_cvt_scalef32_pk_bf16_fp4 (scale 1.0) turns each byte into the exact
//     (even k, odd k) bf16 pair, already in x's order.  A k-slice is one
//     scale group of 32, so each slice's MFMA starts from zero and its sum
//     is multiplied by the lane's column scale in FP32 (exact inputs, no
//     rounding before the output).
//   * Activations are loaded 4 rows x 256 bytes per instruction and put in
//     the A layout through a 4 KB LDS tile of the wave's own; the scales of
//     the workgroup's weight rows are staged in LDS once.
//   * The 4 waves' partial sums are added through LDS in a fixed order.
#include <type_traits>

#include "w4.h"
#include "w4_device.hpp"
#include "w4_internal.hpp"

namespace w4 {
namespace {

constexpr int kStep = 128;  // k per step: 4 MFMA k-slices, 4 scale groups
// Four waves per workgroup: four workgroups (four waves per SIMD) share a
// compute unit, so a 6 x 16-row pair of FCs starts 1024 of its 1152
// workgroups at once, and each wave streams a quarter of K.
constexpr int kWaves = 4, kThreads = kWaves * kWave;
constexpr int kMaxSteps = W4_MOE_GEMM_MAX_K / kStep;

__device__ __forceinline__ f32x4_t mfma(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

// Register u of lane row g (g = lane / 16) becomes register g of lane row u.
__device__ __forceinline__ void transpose4x4_rows(u32x4_t& v) {
    auto s02 = __builtin_amdgcn_permlane32_swap(v.x, v.z, false, false);
    auto s13 = __builtin_amdgcn_permlane32_swap(v.y, v.w, false, false);
    auto s01 = __builtin_amdgcn_permlane16_swap(s02[0], s13[0], false, false);
    auto s23 = __builtin_amdgcn_permlane16_swap(s02[1], s13[1], false, false);
    v = u32x4_t{s01[0], s01[1], s23[0], s23[1]};
}

template <int kCB>
struct Slot {
    u32x4_t w[kCB];  // one 16-byte weight piece per column block
    u32x4_t a[4];    // activation chunk (lane % 16) of rows lane / 16 + 4 i
};

// One FC of the grouped GEMM, as w4_moe_gemm takes it.
struct GemmFc {
    const uint16_t* x;  // bf16 [R][K]
    const uint8_t* qw;  // [num_experts][N][K/2]
    const uint16_t* s;  // bf16 [num_experts][N][K/32]
    uint16_t* y;        // bf16 [R][N]
    int K, N;
};

// LDS of one workgroup: the scales of its rows, then each wave's activation
// tile (in the K loop) or partial sums (after it).
template <int kCB>
constexpr int tile_lds_bytes() {
    constexpr int kBN = 16 * kCB;
    constexpr int kSBytes = kBN * kMaxSteps * 4 * 2;      // bf16 scales [kBN][K / 32]
    constexpr int kXBytes = kWaves * 16 * kStep * 2;      // each wave's 16 x 128 activation tile
    constexpr int kRedBytes = kWaves * kCB * kWave * 16;  // each wave's 16 x kBN partial sums
    return kSBytes + (kRedBytes > kXBytes ? kRedBytes : kXBytes);
}

// Weight-row tile bx (16 kCB rows) of FC f for slab blockIdx.y of group
// blockIdx.z.
template <int kCB>
__device__ __forceinline__ void moe_gemm_tile(const GemmFc& f, const int32_t* __restrict__ row_start,
                                              const int32_t* __restrict__ ids, int R, int num_experts, int bx,
                                              char* lds) {
    constexpr int kBN = 16 * kCB;
    constexpr int kSBytes = kBN * kMaxSteps * 4 * 2;
    static_assert(tile_lds_bytes<kCB>() <= 160 * 1024, "LDS budget of one gfx950 workgroup");
    const uint16_t* __restrict__ x = f.x;
    const uint8_t* __restrict__ qw = f.qw;
    const uint16_t* __restrict__ s = f.s;
    uint16_t* __restrict__ y = f.y;
    const int K = f.K, N = f.N;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int li = lane & 15, lb = lane >> 4;
    const int n0 = bx * kBN;
    const int group = blockIdx.z;

    // The group's rows, clamped into x and y: [r0, r1).
    const int r0 = min(max(row_start[group], 0), R);
    const int r1 = min(max(row_start[group + 1], r0), R);
    const int m0 = r0 + 16 * (int)blockIdx.y;
    if (m0 >= r1) return;  // uniform: this slab of the group is empty
    const int expert = ids[group];
    if (expert < 0 || expert >= num_experts) {  // uniform: an id outside the pool
        for (int i = tid; i < kBN * 16; i += kThreads) {
            const int m = m0 + i / kBN, n = n0 + i % kBN;
            if (m < r1 && n < N) y[(size_t)m * N + n] = 0x7FC0u;  // bf16 quiet NaN
        }
        return;
    }

    const int S = K / kStep;
    const int g0 = (int)(((long)wave * S) / kWaves);
    const int g1 = (int)(((long)(wave + 1) * S) / kWaves);
    const uint32_t row_bytes = (uint32_t)K / 2;
    const int G = K / 32;  // scale groups per weight row
    const uint8_t* qe = qw + (size_t)expert * N * row_bytes;
    const uint16_t* se = s + (size_t)expert * N * G;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qe, (uint32_t)N * row_bytes);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)((size_t)R * K * 2));

    // Weights: row n0 + 16 c + i (rows past N read row N - 1, never stored),
    // bytes 16 b .. +15 of the step.  Activations: rows m0 + lane / 16 + 4 i
    // (rows past the group read its last row, never stored).
    uint32_t woff[kCB];
#pragma unroll
    for (int c = 0; c < kCB; ++c) woff[c] = (uint32_t)min(n0 + 16 * c + li, N - 1) * row_bytes + 16u * lb;
    uint32_t aoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) aoff[i] = (uint32_t)(((size_t)min(m0 + (lane >> 4) + 4 * i, r1 - 1) * K + 8 * li) * 2);
    char* xw_lds = lds + kSBytes + wave * (16 * kStep * 2);

    auto issue = [&](int g, Slot<kCB>& T) {
        const uint32_t gg = (uint32_t)g;
#pragma unroll
        for (int c = 0; c < kCB; ++c) T.w[c] = buf_load_b128<kAuxNontemporal>(rq, woff[c], gg * 64u);
#pragma unroll
        for (int t = 0; t < 4; ++t) T.a[t] = buf_load_b128(rx, aoff[t], gg * 256u);
    };

    // Steps of loads in flight per wave: two at 32 rows per workgroup keeps
    // the kernel within 128 VGPRs (four waves per SIMD).
    constexpr int kSlots = kCB == 2 ? 2 : 4;
    Slot<kCB> ring[kSlots];
#pragma unroll
    for (int d = 0; d < kSlots; ++d) {
        if (g0 + d < g1) issue(g0 + d, ring[d]);
        __builtin_amdgcn_sched_barrier(0);
    }

    // Scales of the workgroup's weight rows, [kBN][G] bf16, 8 bytes per load
    // (the expert's block starts 8-byte aligned: K is a multiple of 128).
    // The piece that straddles the end of the expert's scales is read 2 bytes
    // at a time: a buffer load partly out of range reads all zeros.
    {
        const uint32_t s_bytes = (uint32_t)N * (uint32_t)G * 2u;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(se, s_bytes);
        const uint32_t base = (uint32_t)n0 * (uint32_t)G * 2u;
        const int pieces = kBN * G * 2 / 8;
        for (int p = tid; p < pieces; p += kThreads) {
            const uint32_t off = base + (uint32_t)p * 8u;
            u32x2_t v;
            if (off + 8u <= s_bytes) {
                v = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rs, (int)off, 0, 0));
            } else {
                uint32_t h[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) h[j] = buf_load_u16(rs, off + 2u * j, 0u);
                v = u32x2_t{h[0] | h[1] << 16, h[2] | h[3] << 16};
            }
            *reinterpret_cast<u32x2_t*>(lds + p * 8) = v;
        }
    }
    const uint16_t* lds_s = reinterpret_cast<const uint16_t*>(lds);
    __syncthreads();

    f32x4_t acc[kCB];
#pragma unroll
    for (int c = 0; c < kCB; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int g = g0; g < g1; g += kSlots) {
#pragma unroll
        for (int d = 0; d < kSlots; ++d) {
            Slot<kCB>& T = ring[d];
            const int gd = g + d;
            if (gd >= g1) break;  // wave-uniform: the wave's last steps
            // Activations through this wave's LDS tile (row r, chunk c at
            // c ^ r) into the A layout: lane (i, b) of k-slice t takes chunk
            // 4 t + b of row i.
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int r = (lane >> 4) + 4 * t;
                *reinterpret_cast<u32x4_t*>(xw_lds + (r * 16 + (li ^ r)) * 16) = T.a[t];
            }
            u32x4_t a[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) a[t] = *reinterpret_cast<const u32x4_t*>(xw_lds + (li * 16 + ((4 * t + lb) ^ li)) * 16);
            const int gi = gd;
#pragma unroll
            for (int c = 0; c < kCB; ++c) {
                u32x4_t w = T.w[c];
                transpose4x4_rows(w);
                const uint32_t wt[4] = {w.x, w.y, w.z, w.w};
                const int n = 16 * c + li;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    uint32_t bp[4];
                    fp4_word_pairs(wt[t], bp);
                    const f32x4_t p = mfma(a[t], u32x4_t{bp[0], bp[1], bp[2], bp[3]}, f32x4_t{0.f, 0.f, 0.f, 0.f});
                    const float sc = bf16_to_f32(lds_s[n * G + 4 * gi + t]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[c][e] = __builtin_fmaf(sc, p[e], acc[c][e]);
                }
            }
            if (gd + kSlots < g1) issue(gd + kSlots, T);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Cross-wave sum in wave order.  Lane (i, b) of column block c holds
    // rows 4 b + e, column 16 c + i.
    __syncthreads();  // every wave is done with its activation tile
    float* red = reinterpret_cast<float*>(lds + kSBytes);
#pragma unroll
    for (int c = 0; c < kCB; ++c)
        *reinterpret_cast<f32x4_t*>(&red[((wave * kCB + c) * kWave + lane) * 4]) = acc[c];
    __syncthreads();
    if (tid < kCB * kWave) {
        const int c = tid / kWave, l = tid % kWave;
        f32x4_t t = *reinterpret_cast<const f32x4_t*>(&red[(c * kWave + l) * 4]);
#pragma unroll
        for (int w = 1; w < kWaves; ++w) t += *reinterpret_cast<const f32x4_t*>(&red[((w * kCB + c) * kWave + l) * 4]);
        const int n = n0 + 16 * c + (l & 15);
        if (n < N) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = m0 + 4 * (l >> 4) + e;
                if (m < r1) y[(size_t)m * N + n] = f32_to_bf16(t[e]);
            }
        }
    }
}

template <int kCB>
__global__ __launch_bounds__(kThreads) void moe_gemm_fp4_kernel(GemmFc f, const int32_t* __restrict__ row_start,
                                                                const int32_t* __restrict__ ids, int R,
                                                                int num_experts) {
    __shared__ __attribute__((aligned(16))) char lds[tile_lds_bytes<kCB>()];
    moe_gemm_tile<kCB>(f, row_start, ids, R, num_experts, blockIdx.x, lds);
}

// Two FCs over the same groups in one launch: weight-row tiles [0, b1) of
// each slab run the first FC, the rest the second.
template <int kCB1, int kCB2>
__global__ __launch_bounds__(kThreads) void moe_gemm2_fp4_kernel(GemmFc f1, GemmFc f2, int b1,
                                                                 const int32_t* __restrict__ row_start,
                                                                 const int32_t* __restrict__ ids, int R,
                                                                 int num_experts) {
    constexpr int kBytes = tile_lds_bytes<kCB1>() > tile_lds_bytes<kCB2>() ? tile_lds_bytes<kCB1>()
                                                                             : tile_lds_bytes<kCB2>();
    __shared__ __attribute__((aligned(16))) char lds[kBytes];
    if ((int)blockIdx.x < b1) moe_gemm_tile<kCB1>(f1, row_start, ids, R, num_experts, blockIdx.x, lds);
    else moe_gemm_tile<kCB2>(f2, row_start, ids, R, num_experts, blockIdx.x - b1, lds);
}

// 32 weight rows per workgroup (four workgroups per compute unit) when that
// gives at least 240 workgroups for groups of max_rows rows, else 16.
// Measured on 6 experts x 16 rows, FC1 and FC2 in one launch: 20.3 us per
// pair at 32 rows, 25.1 at 16, 23.6 at 64 (183 VGPRs: two workgroups per
// compute unit).
int column_blocks(int N, int slabs, int E) { return (long)((N + 31) / 32) * slabs * E >= 240 ? 2 : 1; }

}  // namespace

hipError_t launch_moe_gemm_fp4(const void* x, const int32_t* row_start, const int32_t* ids, const uint8_t* qw,
                               const void* s, void* y, int R, int E, int max_rows, int num_experts, int K, int N,
                               hipStream_t stream) {
    const GemmFc f{static_cast<const uint16_t*>(x), qw, static_cast<const uint16_t*>(s), static_cast<uint16_t*>(y),
                   K, N};
    const unsigned slabs = (unsigned)((max_rows + 15) / 16);
    auto launch = [&](auto cb) {
        constexpr int kCB = decltype(cb)::value;
        const dim3 grid((unsigned)((N + 16 * kCB - 1) / (16 * kCB)), slabs, (unsigned)E);
        moe_gemm_fp4_kernel<kCB><<<grid, kThreads, 0, stream>>>(f, row_start, ids, R, num_experts);
        return hipGetLastError();
    };
    if (column_blocks(N, (int)slabs, E) == 2) return launch(std::integral_constant<int, 2>{});
    return launch(std::integral_constant<int, 1>{});
}

hipError_t launch_moe_gemm2_fp4(const MoeGemmFcArgs& a, const MoeGemmFcArgs& b, const int32_t* row_start,
                                const int32_t* ids, int R, int E, int max_rows, int num_experts,
                                hipStream_t stream) {
    const GemmFc f1{static_cast<const uint16_t*>(a.x), a.qw, static_cast<const uint16_t*>(a.s),
                    static_cast<uint16_t*>(a.y), a.K, a.N};
    const GemmFc f2{static_cast<const uint16_t*>(b.x), b.qw, static_cast<const uint16_t*>(b.s),
                    static_cast<uint16_t*>(b.y), b.K, b.N};
    const int slabs = (max_rows + 15) / 16;
    // Each FC takes the tile width its own launch would (same bits).
    auto launch = [&](auto cb1, auto cb2) {
        constexpr int kCB1 = decltype(cb1)::value, kCB2 = decltype(cb2)::value;
        const int b1 = (a.N + 16 * kCB1 - 1) / (16 * kCB1), b2 = (b.N + 16 * kCB2 - 1) / (16 * kCB2);
        const dim3 grid((unsigned)(b1 + b2), (unsigned)slabs, (unsigned)E);
        moe_gemm2_fp4_kernel<kCB1, kCB2><<<grid, kThreads, 0, stream>>>(f1, f2, b1, row_start, ids, R, num_experts);
        return hipGetLastError();
    };
    using One = std::integral_constant<int, 1>;
    using Two = std::integral_constant<int, 2>;
    switch (column_blocks(a.N, slabs, E) * 16 + column_blocks(b.N, slabs, E)) {
        case 2 * 16 + 2: return launch(Two{}, Two{});
        case 2 * 16 + 1: return launch(Two{}, One{});
        case 1 * 16 + 2: return launch(One{}, Two{});
        default: return launch(One{}, One{});
    }
}

}  // namespace w4
