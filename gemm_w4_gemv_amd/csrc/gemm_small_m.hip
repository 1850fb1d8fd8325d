// Small-M INT4 GEMM (a few decode tokens at once, M <= 16):
// y[m][n] = bf16( sum_k (q[n][k] - z) s x[m][k] ).
//
// "Lab 5: Gemma4 端到端推理优化": decode (one token) and prefill (many) run
// on different backends ("INT4 融合 GEMV" for M = 1, a matrix-core GEMM for
// prefill).  Between them, a handful of rows still reads every weight once
// and is bound by HBM, like the GEMV, but the per-row work is small enough
// for the matrix cores: one v_mfma_f32_16x16x32_bf16 block covers 16 rows of
// x against 16 weight rows.
//
// gfx950 design:
//   * A workgroup owns 64, 32 or 16 weight rows (1 to 4 MFMA column blocks;
//     the widest that still launches 240 workgroups) and all M (<= 16) x
//     rows; its 8 waves split the K groups, each streaming its own groups
//     with three or four groups of loads in flight and no barrier inside
//     the K loop.  A wave issues and computes exactly its own groups (a
//     wave-uniform exit at the end of its range): with about four groups per
//     wave on a K = 3840 shape, padding the range to whole rounds of the
//     ring cost as many dummy loads and MFMA steps as real ones.
//   * Weights: lane (i, b) of a column block loads 16 bytes (words 4b..4b+3
//     of one group of row i), so a load instruction reads 16 rows x 64
//     contiguous bytes.  A 4 x 4 transpose across the four 16-lane rows
//     (v_permlane32_swap, v_permlane16_swap) leaves word 4t + b in register
//     t: exactly the B operand of k-slice t (k = 32 t + 8 b .. +7).
//     Activations are loaded 4 rows x 256 bytes per instruction, one
//     instruction per 4 rows of x that exist (ceil(M / 4), a template
//     parameter), and put in the matching A layout through a 4 KB LDS tile of
//     the wave's own; the tile's rows past them are never written and only
//     feed output rows past M, which are not stored (an A-layout load would
//     cover 16 rows x 64 bytes per instruction, measured 15 % slower at
//     M = 16 on the K15360 shape, and 7-23 % slower at M = 3..16 together
//     with weights loaded 4 rows x 256 bytes per instruction and re-laid
//     through LDS).
//   * Unpacking uses the bf16 bias trick of the GEMV: 0x4300 | q is exactly
//     128 + q, 7 integer operations per 8 codes, with the activation pairs
//     permuted to match.  Per group, sum_k (q - z) s x
//     = s (sum_k (128 + q) x - (128 + z) sum_k x): the first sum is one MFMA
//     accumulator per column block, the second one more MFMA against a B of
//     ones, and both fold into the running sum with two FMAs per output.
//   * The eight waves' partial sums are added through LDS in a fixed order
//     (no atomics, bit-reproducible).
#include <type_traits>

#include "w4.h"
#include "w4_device.hpp"
#include "tune.hpp"
#include "w4_internal.hpp"

namespace w4 {
namespace {

constexpr int kGroup = 128;
constexpr int kWaves = 8, kThreads = kWaves * kWave;
constexpr int kMaxGroups = W4_GEMM_MAX_K / kGroup;

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

// One group's operands of one lane: a weight chunk per column block and the
// 4 activation chunks of k-slices 0..3.
template <int kCB>
struct Slot {
    u32x4_t w[kCB];
    u32x4_t a[4];
};

// kCB column blocks of 16 weight rows per workgroup; kMQ = ceil(M / 4)
// activation load instructions (4 rows each) per group.
template <int kCB, int kMQ>
__global__ __launch_bounds__(kThreads) void gemm_int4_small_m_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ qw, const uint16_t* __restrict__ s,
    const uint16_t* __restrict__ z, uint16_t* __restrict__ y, int M, int K, int N) {
    constexpr int kBN = 16 * kCB;
    constexpr int kSlots = kCB == 4 ? 3 : 4;  // groups of loads in flight per wave (register budget)
    constexpr int kSZBytes = 2 * kBN * kMaxGroups * 2;    // raw fp16 s then z, [kBN][G] each
    constexpr int kRedBytes = kWaves * kCB * kWave * 16;  // each wave's 16 x kBN partial sums
    constexpr int kXBytes = kWaves * 16 * kGroup * 2;       // each wave's 16 x 128 activation tile
    constexpr int kTail = kRedBytes > kXBytes ? kRedBytes : kXBytes;
    static_assert(kSZBytes + kTail <= 160 * 1024, "LDS budget of one gfx950 workgroup");
    __shared__ __attribute__((aligned(16))) char lds[kSZBytes + kTail];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int li = lane & 15, lb = lane >> 4;
    const int n0 = blockIdx.x * kBN;
    constexpr int m0 = 0;
    const int G = K / kGroup;
    const int g0 = (int)(((long)wave * G) / kWaves);
    const int g1 = (int)(((long)(wave + 1) * G) / kWaves);
    const uint32_t row_bytes = (uint32_t)K / 2;

    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)((size_t)M * K * 2));
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qw, (uint32_t)((size_t)N * row_bytes));

    // Lane offsets.  Weights: row n0 + 16 c + i (rows past N read row N - 1),
    // bytes 16 b .. 16 b + 15 of the group.  Activations: row m0 + i (rows
    // past M read row M - 1, never stored), k = 32 t + 8 b of the group.
    uint32_t woff[kCB];
#pragma unroll
    for (int c = 0; c < kCB; ++c) woff[c] = (uint32_t)min(n0 + 16 * c + li, N - 1) * row_bytes + 16u * lb;
    // Activations: chunk (lane % 16) of rows lane / 16 + 4 i, i.e. 4 rows x
    // 256 bytes per load instruction; reordered through LDS below.
    uint32_t aoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) aoff[i] = (uint32_t)(((size_t)min(m0 + (lane >> 4) + 4 * i, M - 1) * K + 8 * li) * 2);
    char* xw_lds = lds + kSZBytes + wave * (16 * kGroup * 2);

    auto issue = [&](int g, Slot<kCB>& S) {
        const uint32_t gg = (uint32_t)g;
#pragma unroll
        for (int c = 0; c < kCB; ++c) S.w[c] = buf_load_b128<kAuxNontemporal>(rq, woff[c], gg * 64u);
#pragma unroll
        for (int t = 0; t < kMQ; ++t) S.a[t] = buf_load_b128(rx, aoff[t], gg * 256u);
    };

    // The first groups' loads go out before the scale staging below, so
    // their latency overlaps it.
    Slot<kCB> ring[kSlots];
#pragma unroll
    for (int d = 0; d < kSlots; ++d) {
        if (g0 + d < g1) issue(g0 + d, ring[d]);
        __builtin_amdgcn_sched_barrier(0);
    }

    // Scales and zeros of the workgroup's rows, all groups, staged raw (rows
    // past N read 0 and are never stored).  The chunk that straddles the end
    // of the arrays is read 2 bytes at a time: a 16-byte buffer load that is
    // partly out of range reads all zeros.
    {
        const uint32_t sz_bytes = (uint32_t)((size_t)N * G * 2);
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(s, sz_bytes);
        const __amdgpu_buffer_rsrc_t rz = make_rsrc(z, sz_bytes);
        const uint32_t base = (uint32_t)n0 * (uint32_t)G * 2u;  // 16-byte aligned: n0 is a multiple of 16
        const int chunks = kBN * G * 2 / 16;
        for (int c = tid; c < chunks; c += kThreads) {
            const uint32_t off = base + (uint32_t)c * 16u;
            u32x4_t vs, vz;
            if (off + 16u <= sz_bytes) {
                vs = buf_load_b128(rs, off, 0u);
                vz = buf_load_b128(rz, off, 0u);
            } else {
                uint32_t hs[8], hz[8];
#pragma unroll
                for (int h = 0; h < 8; ++h) {
                    hs[h] = buf_load_u16(rs, off + 2u * h, 0u);
                    hz[h] = buf_load_u16(rz, off + 2u * h, 0u);
                }
                vs = u32x4_t{hs[0] | hs[1] << 16, hs[2] | hs[3] << 16, hs[4] | hs[5] << 16, hs[6] | hs[7] << 16};
                vz = u32x4_t{hz[0] | hz[1] << 16, hz[2] | hz[3] << 16, hz[4] | hz[5] << 16, hz[6] | hz[7] << 16};
            }
            *reinterpret_cast<u32x4_t*>(lds + c * 16) = vs;
            *reinterpret_cast<u32x4_t*>(lds + kBN * G * 2 + c * 16) = vz;
        }
    }
    const uint16_t* lds_s = reinterpret_cast<const uint16_t*>(lds);
    const uint16_t* lds_z = lds_s + kBN * G;
    __syncthreads();

    const uint32_t bias = vgpr_const(kInt4BiasPair);
    const u32x4_t ones = u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0
    f32x4_t acc[kCB];
#pragma unroll
    for (int c = 0; c < kCB; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int g = g0; g < g1; g += kSlots) {
#pragma unroll
        for (int d = 0; d < kSlots; ++d) {
            Slot<kCB>& S = ring[d];
            const int gd = g + d;
            if (gd >= g1) break;  // wave-uniform: the wave's last groups
            // Activation pairs (x_j, x_{j+4}) of each 16-byte chunk, matching
            // the biased weight pairs, built as the chunk goes into this wave's
            // LDS tile (row r, chunk c at c ^ r: each lane converts ceil(M / 4)
            // chunks, not the four it reads back); read in the MFMA layout:
            // lane (i, b) of k-slice t takes chunk 4 t + b of row i.  The same
            // A against ones gives sum_k x.  Rows past 4 kMQ are never
            // written; they only feed output rows past M, which are not stored.
#pragma unroll
            for (int t = 0; t < kMQ; ++t) {
                const int r = (lane >> 4) + 4 * t;
                const uint32_t xw[4] = {S.a[t].x, S.a[t].y, S.a[t].z, S.a[t].w};
                uint32_t p[4];
                x_pairs_for_biased(xw, p);
                *reinterpret_cast<u32x4_t*>(xw_lds + (r * 16 + (li ^ r)) * 16) = u32x4_t{p[0], p[1], p[2], p[3]};
            }
            u32x4_t a[4];
#pragma unroll
            for (int t = 0; t < 4; ++t)
                a[t] = *reinterpret_cast<const u32x4_t*>(xw_lds + (li * 16 + ((4 * t + lb) ^ li)) * 16);
            f32x4_t sx = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 4; ++t) sx = mfma(a[t], ones, sx);
            const int gi = gd;
#pragma unroll
            for (int c = 0; c < kCB; ++c) {
                u32x4_t w = S.w[c];
                transpose4x4_rows(w);
                const uint32_t wt[4] = {w.x, w.y, w.z, w.w};
                f32x4_t p = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    uint32_t bp[4];
                    int4_word_biased_pairs(wt[t], bias, bp);
                    p = mfma(a[t], u32x4_t{bp[0], bp[1], bp[2], bp[3]}, p);
                }
                const int n = 16 * c + li;
                const float sc = f16_to_f32(lds_s[n * G + gi]);
                const float szb = sc * (f16_to_f32(lds_z[n * G + gi]) + 128.f);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[c][e] = __builtin_fmaf(sc, p[e], __builtin_fmaf(-szb, sx[e], acc[c][e]));
            }
            if (gd + kSlots < g1) issue(gd + kSlots, S);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Cross-wave sum in wave order.  Lane (i, b) of column block c holds
    // rows 4 b + e, column 16 c + i.
    __syncthreads();  // every wave is done with its activation tile
    float* red = reinterpret_cast<float*>(lds + kSZBytes);
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
                if (m < M) y[(size_t)m * N + n] = f32_to_bf16(t[e]);
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm_int4_small_m(const void* x, const int32_t* qw, const void* s, const void* z, void* y,
                                    int M, int K, int N, hipStream_t stream) {
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const uint32_t* wb = reinterpret_cast<const uint32_t*>(qw);
    const uint16_t* sb = static_cast<const uint16_t*>(s);
    const uint16_t* zb = static_cast<const uint16_t*>(z);
    uint16_t* yb = static_cast<uint16_t*>(y);
    // Weight rows per workgroup (16 per block) from the per-shape table, else
    // the widest tile that still gives 240 workgroups (the rule in tune.hip).
    auto launch_q = [&](auto cb, auto mq) {
        constexpr int kCB = decltype(cb)::value;
        constexpr int kMQ = decltype(mq)::value;
        const dim3 grid((unsigned)((N + 16 * kCB - 1) / (16 * kCB)));
        gemm_int4_small_m_kernel<kCB, kMQ><<<grid, kThreads, 0, stream>>>(xb, wb, sb, zb, yb, M, K, N);
        return hipGetLastError();
    };
    auto launch = [&](auto cb) {
        switch ((M + 3) / 4) {
            case 1: return launch_q(cb, std::integral_constant<int, 1>{});
            case 2: return launch_q(cb, std::integral_constant<int, 2>{});
            case 3: return launch_q(cb, std::integral_constant<int, 3>{});
            default: return launch_q(cb, std::integral_constant<int, 4>{});
        }
    };
    switch (gemm_small_m_blocks(M, K, N)) {
        case 4: return launch(std::integral_constant<int, 4>{});
        case 2: return launch(std::integral_constant<int, 2>{});
        default: return launch(std::integral_constant<int, 1>{});
    }
}

}  // namespace w4
