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
// operand.  The activation tile (A operand, 128 x 128 per K-step) is loaded
// once per workgroup with full-line loads and staged in LDS beside it.
//
// Tile: 128 (M) x 64 (N) per workgroup; wave w computes rows 32 (w % 4) ..
// +32 and columns 32 (w / 4) .. +32 as 2 x 2 MFMA blocks of 16 x 16.  The
// activation and dequantised weight tiles are double-buffered in LDS, with
// one barrier per K-step of 128.  Global loads run kDepth K-steps ahead of
// the MFMAs: this thread's 64 bytes of the next kDepth activation tiles and
// its packed weights, scales and zeros of the next kDepth weight tiles live
// in a ring of registers, the loop unrolled kDepth times so every ring slot
// is a fixed register set (up to kDepth - 1 surplus steps at the end compute
// on zeros: loads past the K range use an empty buffer range, which returns
// zeros without touching memory).  The staging of step j + 1 (dequantise,
// LDS stores) is spread between step j's MFMAs.  LDS is what bounds this
// kernel on MI355X: 16 fragment reads per wave and 176 KB per K-step, and a
// 64-lane ds_read_b128 costs about the same time whatever its addresses, so
// the count of LDS read instructions per MFMA sets the pace; removing the
// MFMAs leaves the time unchanged.  All loads are buffer loads (weights
// non-temporal).  When
// the N x M tiles cannot fill the GPU, K is split; each split writes FP32
// partials to the caller's workspace and a second kernel adds them in split
// order (deterministic, no atomics).
#include "w4_device.hpp"
#include "w4_internal.hpp"

namespace w4 {
namespace {

constexpr int kBM = 128, kBN = 64, kBK = 128;
constexpr int kThreads = 512;
constexpr int kDepth = 2;            // K-steps of loads in flight ahead of the MFMAs
constexpr int kTargetBlocks = 256;   // one workgroup per compute unit of an MI355X

// LDS tiles are rows of kBK bf16 (16 chunks of 16 bytes), chunk c of row r
// stored at chunk position c ^ (r % 16): the 16 rows an MFMA fragment read
// touches at one chunk, and the 16 chunks of one row a staging write
// touches, each land on 16 distinct positions, i.e. on all 64 banks once.
__device__ __forceinline__ int lds_elem(int row, int chunk) { return row * kBK + ((chunk ^ (row & 15)) << 3); }

__device__ __forceinline__ void mfma_16x16x32(const u32x4_t& a, const u32x4_t& b, f32x4_t& acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}

// One ring slot: this thread's share of one K-step's activation tile (chunk
// tid % 16 of rows tid / 16 + 32 i) and of its packed weight tile (16 codes
// of one row, with that row's scale and zero).
struct Slot {
    u32x4_t a[4];
    u32x4_t w;  // .x, .y: codes; .z, .w: scale and zero bits
};

template <bool kSplit>
__global__ __launch_bounds__(kThreads) void gemm_int4_mfma_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ qw, const uint16_t* __restrict__ s,
    const uint16_t* __restrict__ z, uint16_t* __restrict__ y, float* __restrict__ ws, int M, int K,
    int N, int splits) {
    __shared__ __attribute__((aligned(16))) uint16_t wt[2][kBN * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t at[2][kBM * kBK];

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
    const int nsteps = kt1 - kt0;
    const int words_per_row = K / 8;

    // Weight-tile loader: thread -> (row r, 16 codes at k = 16 part).  Rows
    // past N read row N - 1 (never stored).
    const int lr = tid >> 3, part = tid & 7;
    const int wr = min(n0 + lr, N - 1);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qw, (uint32_t)((size_t)N * words_per_row * 4));
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(s, (uint32_t)((size_t)N * G * 2));
    const __amdgpu_buffer_rsrc_t rz = make_rsrc(z, (uint32_t)((size_t)N * G * 2));
    const __amdgpu_buffer_rsrc_t rnone = make_rsrc(qw, 0u);
    const uint32_t qoff = (uint32_t)(((size_t)wr * words_per_row + 2 * part) * 4);
    const uint32_t szoff = (uint32_t)((size_t)wr * G * 2);

    // Activation tile loader: chunk tid % 16 of rows tid / 16 + 32 i: each
    // load instruction covers 4 whole rows (8 whole 128-byte lines).  Rows
    // past M read row M - 1; their results are never stored.
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)((size_t)M * K * 2));
    const int ar = tid >> 4, ac = tid & 15;
    uint32_t aoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) aoff[i] = (uint32_t)(((size_t)min(m0 + ar + 32 * i, M - 1) * K + 8 * ac) * 2);

    // Loads of K-step kt0 + j into a slot (an empty range past the split's end).
    auto issue = [&](int j, Slot& S) {
        const bool live = j < nsteps;
        const int kt = kt0 + (live ? j : 0);
        const __amdgpu_buffer_rsrc_t ra = live ? rx : rnone;
        const __amdgpu_buffer_rsrc_t rqq = live ? rq : rnone;
        const __amdgpu_buffer_rsrc_t rss = live ? rs : rnone;
        const __amdgpu_buffer_rsrc_t rzz = live ? rz : rnone;
#pragma unroll
        for (int i = 0; i < 4; ++i) S.a[i] = buf_load_b128(ra, aoff[i], (uint32_t)(kt * kBK) * 2u);
        const u32x2_t q = __builtin_bit_cast(
            u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rqq, (int)qoff, (int)sgpr((uint32_t)kt * 64u), kAuxNontemporal));
        S.w.x = q.x;
        S.w.y = q.y;
        S.w.z = buf_load_u16(rss, szoff, (uint32_t)kt * 2u);
        S.w.w = buf_load_u16(rzz, szoff, (uint32_t)kt * 2u);
    };
    // Staging of one K-step into LDS buffer ``buf``, in four parts that the
    // main loop interleaves with its MFMAs: dequantise this thread's 16 codes
    // (part 0) and store them (1), store its activations (2, 3).
    u32x4_t wlo, whi;
    auto stage = [&](const Slot& S, int buf, int part_no) {
        if (part_no == 0) {
            const float sc = f16_to_f32((uint16_t)S.w.z), zp = f16_to_f32((uint16_t)S.w.w);
            float f[16];
            int4_word_dequant_f32(S.w.x, sc, zp, f);
            int4_word_dequant_f32(S.w.y, sc, zp, f + 8);
            wlo.x = pack_bf16x2(f[0], f[1]);
            wlo.y = pack_bf16x2(f[2], f[3]);
            wlo.z = pack_bf16x2(f[4], f[5]);
            wlo.w = pack_bf16x2(f[6], f[7]);
            whi.x = pack_bf16x2(f[8], f[9]);
            whi.y = pack_bf16x2(f[10], f[11]);
            whi.z = pack_bf16x2(f[12], f[13]);
            whi.w = pack_bf16x2(f[14], f[15]);
        } else if (part_no == 1) {
            *reinterpret_cast<u32x4_t*>(&wt[buf][lds_elem(lr, 2 * part)]) = wlo;
            *reinterpret_cast<u32x4_t*>(&wt[buf][lds_elem(lr, 2 * part + 1)]) = whi;
        } else {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int i = 2 * (part_no - 2) + h;
                *reinterpret_cast<u32x4_t*>(&at[buf][lds_elem(ar + 32 * i, ac)]) = S.a[i];
            }
        }
    };
    auto store_w = [&](const Slot& S, int buf) {
#pragma unroll
        for (int p = 0; p < 4; ++p) stage(S, buf, p);
    };

    f32x4_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Step j (0-based within the split) computes from LDS buffer j & 1; before
    // its barrier it stages step j + 1 (slot (j + 1) % kDepth) into the other
    // buffer, then refills slot j % kDepth with step j + kDepth.
    Slot ring[kDepth];
    if (nsteps > 0) {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) issue(d, ring[d]);
        store_w(ring[0], 0);
        __syncthreads();
        for (int j0 = 0; j0 < nsteps; j0 += kDepth) {
#pragma unroll
            for (int d = 0; d < kDepth; ++d) {
                const int j = j0 + d;
                const int buf = j & 1;
                Slot& S = ring[d];
                const Slot& T = ring[(d + 1) % kDepth];
                // All fragments of the step first, so the LDS reads overlap
                // each other rather than each waiting before its MFMAs.
                u32x4_t a[4][2], b[4][2];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        a[ks][i] = *reinterpret_cast<const u32x4_t*>(
                            &at[buf][lds_elem(32 * wm + 16 * i + (lane & 15), 4 * ks + (lane >> 4))]);
#pragma unroll
                    for (int jj = 0; jj < 2; ++jj)
                        b[ks][jj] = *reinterpret_cast<const u32x4_t*>(
                            &wt[buf][lds_elem(32 * wn + 16 * jj + (lane & 15), 4 * ks + (lane >> 4))]);
                }
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int jj = 0; jj < 2; ++jj) mfma_16x16x32(a[ks][i], b[ks][jj], acc[i][jj]);
                    // Part ks of step j + 1's staging runs while these MFMAs execute.
                    stage(T, buf ^ 1, ks);
                }
                issue(j + kDepth, S);
                __syncthreads();
            }
        }
    }

    // Output fragment: lane -> column (lane & 15), rows 4 (lane >> 4) + 0..3.
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int n = n0 + 32 * wn + 16 * jj + (lane & 15);
            if (n >= N) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = m0 + 32 * wm + 16 * i + 4 * (lane >> 4) + e;
                if (m >= M) continue;
                if constexpr (kSplit) {
                    ws[((size_t)blockIdx.z * M + m) * N + n] = acc[i][jj][e];
                } else {
                    y[(size_t)m * N + n] = f32_to_bf16(acc[i][jj][e]);
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
