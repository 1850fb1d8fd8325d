// Prefill GEMM (M rows of activations, built for M = 128) over packed INT4
// weights.
//
// "Lab 5: Gemma4 端到端推理优化", section "Triton 反量化 + cuBLAS": the prefill
// path dequantised the INT4 weight to BF16 and handed it to a tensor-core
// GEMM, writing and re-reading the whole BF16 weight in device memory.  Here
// the dequantised tile only ever exists in LDS: each K-step of 128 (one
// quantisation group) unpacks a 64 x 128 weight tile, computes
// bf16((q - z) * s) with round-to-nearest-even, stores it in LDS, and the
// eight waves of the workgroup feed it to v_mfma_f32_16x16x32_bf16 as the B
// operand.  The activation fragments (A operand) are read straight from
// device memory in the MFMA lane layout (8 consecutive k per lane), so they
// need no LDS.
//
// Tile: 128 (M) x 64 (N) per workgroup; wave w computes rows 32 (w % 4) ..
// +32 and columns 32 (w / 4) .. +32 as 2 x 2 MFMA blocks of 16 x 16.  The
// weight tile is double-buffered in LDS so the next tile's global loads and
// dequantisation overlap the current tile's MFMAs, with one barrier per
// K-step.  When the N x M tiles cannot fill the GPU, K is split; each split
// writes FP32 partials to the caller's workspace and a second kernel adds
// them in split order (deterministic, no atomics).
#include "w4_device.hpp"
#include "w4_internal.hpp"

namespace w4 {
namespace {

constexpr int kBM = 128, kBN = 64, kBK = 128;
constexpr int kThreads = 512;
constexpr int kLdsStride = kBK + 8;  // bf16 elements per LDS row; +16 bytes keeps ds_read_b128 conflict-free
constexpr int kTargetBlocks = 256;   // one workgroup per compute unit of an MI355X

__device__ __forceinline__ void mfma_16x16x32(const u32x4_t& a, const u32x4_t& b, f32x4_t& acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}

template <bool kSplit>
__global__ __launch_bounds__(kThreads) void gemm_int4_mfma_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ qw, const uint16_t* __restrict__ s,
    const uint16_t* __restrict__ z, uint16_t* __restrict__ y, float* __restrict__ ws, int M, int K,
    int N, int splits) {
    __shared__ __attribute__((aligned(16))) uint16_t wt[2][kBN][kLdsStride];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wm = wave & 3, wn = wave >> 2;
    const int n0 = blockIdx.x * kBN;
    const int m0 = blockIdx.y * kBM;
    const int KT = K / kBK;
    const int G = K / kBK;
    const int kt0 = (int)(((long)blockIdx.z * KT) / splits);
    const int kt1 = (int)(((long)(blockIdx.z + 1) * KT) / splits);
    const int words_per_row = K / 8;

    // Weight-tile loader: thread -> (row r, 16 codes at k = 16 part).
    const int lr = tid >> 3, part = tid & 7;
    const bool row_ok = (n0 + lr) < N;
    const uint32_t* wrow = qw + (size_t)(row_ok ? n0 + lr : 0) * words_per_row + 2 * part;
    const uint16_t* srow = s + (size_t)(row_ok ? n0 + lr : 0) * G;
    const uint16_t* zrow = z + (size_t)(row_ok ? n0 + lr : 0) * G;

    // Activation fragments: lane -> row (lane & 15) of each 16-row block, k = 8 (lane >> 4) + 0..7.
    int arow[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int m = m0 + 32 * wm + 16 * i + (lane & 15);
        arow[i] = m < M ? m : M - 1;  // rows past M read a valid row; their results are never stored
    }
    const int acol = 8 * (lane >> 4);

    u32x2_t wreg;
    float sreg, zreg;
    auto load_w = [&](int kt) {
        if (row_ok) {
            wreg = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(wrow + kt * 16));
            sreg = f16_to_f32(srow[kt]);
            zreg = f16_to_f32(zrow[kt]);
        } else {
            wreg = u32x2_t{0u, 0u};
            sreg = 0.f;
            zreg = 0.f;
        }
    };
    auto store_w = [&](int buf) {
        float f[16];
        int4_word_dequant_f32(wreg.x, sreg, zreg, f);
        int4_word_dequant_f32(wreg.y, sreg, zreg, f + 8);
        u32x4_t lo, hi;
        lo.x = pack_bf16x2(f[0], f[1]);
        lo.y = pack_bf16x2(f[2], f[3]);
        lo.z = pack_bf16x2(f[4], f[5]);
        lo.w = pack_bf16x2(f[6], f[7]);
        hi.x = pack_bf16x2(f[8], f[9]);
        hi.y = pack_bf16x2(f[10], f[11]);
        hi.z = pack_bf16x2(f[12], f[13]);
        hi.w = pack_bf16x2(f[14], f[15]);
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(&wt[buf][lr][16 * part]);
        dst[0] = lo;
        dst[1] = hi;
    };
    u32x4_t a[2][4];
    auto load_a = [&](int kt, u32x4_t (&dst)[2][4]) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                dst[i][ks] = *reinterpret_cast<const u32x4_t*>(x + (size_t)arow[i] * K + kt * kBK + 32 * ks + acol);
    };

    f32x4_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    if (kt0 < kt1) {
        load_w(kt0);
        load_a(kt0, a);
        store_w(0);
        __syncthreads();
        for (int kt = kt0; kt < kt1; ++kt) {
            const int buf = (kt - kt0) & 1;
            const bool more = kt + 1 < kt1;
            u32x4_t an[2][4];
            if (more) {
                load_w(kt + 1);
                load_a(kt + 1, an);
            }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                u32x4_t b[2];
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    b[j] = *reinterpret_cast<const u32x4_t*>(&wt[buf][32 * wn + 16 * j + (lane & 15)][32 * ks + acol]);
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) mfma_16x16x32(a[i][ks], b[j], acc[i][j]);
            }
            if (more) {
                store_w(buf ^ 1);
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) a[i][ks] = an[i][ks];
            }
            __syncthreads();
        }
    }

    // Output fragment: lane -> column (lane & 15), rows 4 (lane >> 4) + 0..3.
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + 32 * wn + 16 * j + (lane & 15);
            if (n >= N) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = m0 + 32 * wm + 16 * i + 4 * (lane >> 4) + e;
                if (m >= M) continue;
                if constexpr (kSplit) {
                    ws[((size_t)blockIdx.z * M + m) * N + n] = acc[i][j][e];
                } else {
                    y[(size_t)m * N + n] = f32_to_bf16(acc[i][j][e]);
                }
            }
        }
    }
}

// y = bf16(sum over splits of the FP32 partials), splits added in order.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ ws,
                                                            uint16_t* __restrict__ y, size_t count,
                                                            int splits) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= count) return;
    float t = ws[i];
    for (int k = 1; k < splits; ++k) t += ws[(size_t)k * count + i];
    y[i] = f32_to_bf16(t);
}

int choose_splits(int M, int K, int N) {
    const long tiles = (long)((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
    const int KT = K / kBK;
    int splits = (int)((kTargetBlocks + tiles / 2) / tiles);  // round(target / tiles)
    if (splits < 1) splits = 1;
    if (splits > KT) splits = KT;
    if (splits > 16) splits = 16;
    return splits;
}

}  // namespace

size_t gemm_int4_workspace_bytes(int M, int K, int N) {
    if (M <= 0 || N <= 0 || K <= 0 || K % kBK != 0) return 0;
    const int splits = choose_splits(M, K, N);
    return splits > 1 ? (size_t)splits * (size_t)M * (size_t)N * sizeof(float) : 0;
}

hipError_t launch_gemm_int4(const void* x, const int32_t* qw, const void* s, const void* z,
                            void* y, int M, int K, int N, void* workspace, hipStream_t stream) {
    const int splits = choose_splits(M, K, N);
    const dim3 grid((unsigned)((N + kBN - 1) / kBN), (unsigned)((M + kBM - 1) / kBM), (unsigned)splits);
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const uint32_t* wb = reinterpret_cast<const uint32_t*>(qw);
    const uint16_t* sb = static_cast<const uint16_t*>(s);
    const uint16_t* zb = static_cast<const uint16_t*>(z);
    uint16_t* yb = static_cast<uint16_t*>(y);
    if (splits == 1) {
        gemm_int4_mfma_kernel<false><<<grid, kThreads, 0, stream>>>(xb, wb, sb, zb, yb, nullptr, M, K, N, 1);
        return hipGetLastError();
    }
    float* ws = static_cast<float*>(workspace);
    gemm_int4_mfma_kernel<true><<<grid, kThreads, 0, stream>>>(xb, wb, sb, zb, yb, ws, M, K, N, splits);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const size_t count = (size_t)M * N;
    const unsigned blocks = (unsigned)((count + 255) / 256);
    splitk_reduce_kernel<<<blocks, 256, 0, stream>>>(ws, yb, count, splits);
    return hipGetLastError();
}

}  // namespace w4
