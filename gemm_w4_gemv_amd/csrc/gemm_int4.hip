// Prefill GEMM (M rows of activations, built for M = 128) over packed INT4
// weights.
//
// "Lab 5: Gemma4 端到端推理优化", section "Triton 反量化 + cuBLAS": the prefill
// path dequantised the INT4 weight to BF16 and handed it to a tensor-core
// GEMM, writing and re-reading the whole BF16 weight in device memory.  Here
// the weight is dequantised in registers, straight into the B operand of
// v_mfma_f32_16x16x32_bf16, and never exists as BF16 outside them.
//
// Operand layout of v_mfma_f32_16x16x32_bf16 (lane l, i = l % 16, b = l / 16):
// A holds row i, k = 8b .. 8b+7 of a 16 x 32 block; B holds column i, the same
// k.  Eight consecutive k of one weight row are exactly one packed INT4 word
// (bits 4j .. 4j+3 hold k = 8p + j), so lane (i, b) takes one word of row i
// and dequantises it in place: bf16((q - z) * s), the product exact in FP32
// and rounded to nearest even once.
//
// Tile: a workgroup of sixteen waves (four per SIMD) owns 128 (M) x 64 (N)
// outputs and walks its K range one quantisation group (128 k) per step.
// Each step's activation tile (128 x 128 bf16, 32 KB) and packed weight tile
// (64 rows x 64 bytes) are loaded with whole-line loads (each activation load
// instruction covers 4 rows x 256 bytes) into registers two steps ahead, then
// stored in LDS (double-buffered, one barrier per step).  Wave w takes the
// k-slice 32 (w % 4) .. +31 of every group and the 16 output columns
// 16 (w / 4) .. +15: per step it reads 8 A fragments (16 bytes per lane
// each) and one packed word, and computes 128 x 16 outputs over its slices
// (8 MFMA blocks, 32 accumulator registers).  Scales and zeros of the
// workgroup's 64 rows are staged in LDS once, at the start.  At the end the
// four k-slice waves' partial sums of each column block are added in a fixed
// order through LDS.  Measured on MI355X, neither the matrix cores nor LDS
// are saturated (about 28 % and 55 % busy); the waves mostly wait on the
// per-step chain of global load, LDS store, barrier and LDS read, which is
// why four waves per SIMD run faster than one or two with larger tiles.
//
// When the tiles cannot fill the GPU, K is split across workgroups; each
// split writes FP32 partials to the caller's workspace and a second kernel
// adds them in split order (deterministic, no atomics).
#include <mutex>

#include "w4.h"
#include "w4_device.hpp"
#include "tune.hpp"
#include "w4_internal.hpp"

namespace w4 {
namespace {

constexpr int kBM = kGemmTileM, kBN = kGemmTileN, kGroup = 128;
constexpr int kWaves = 16, kThreads = kWaves * kWave;
constexpr int kRB = kBM / 16, kCB = kBN / 16;     // MFMA row and column blocks per tile
constexpr int kNH = kWaves / 4, kCBW = kCB / kNH;  // column parts, column blocks per wave
constexpr int kDepth = 2;                          // steps of global loads in flight in registers
constexpr int kMaxGroups = W4_GEMM_MAX_K / kGroup;

// LDS map (bytes).  During the K loop: two activation tiles, two weight
// tiles, the raw fp16 scales and zeros of the workgroup's rows.  After it:
// the sixteen waves' partial sums, over the tiles.
constexpr int kXTile = kBM * kGroup * 2;            // 32 KB
constexpr int kWTile = kBN * kGroup / 2;            // 4 KB
constexpr int kOffW = 2 * kXTile;
constexpr int kOffSZ = kOffW + 2 * kWTile;
constexpr int kSZBytes = 2 * kBN * kMaxGroups * 2;  // s then z, [64][G] fp16 each
constexpr int kRedBytes = kWaves * kRB * kCBW * kWave * 16;
constexpr int kLdsBytes = (kOffSZ + kSZBytes) > kRedBytes ? (kOffSZ + kSZBytes) : kRedBytes;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget of one gfx950 workgroup");
static_assert(W4_GEMM_MAX_K <= W4_GEMV_MAX_K, "an M = 1 GEMM runs the GEMV kernel");

__device__ __forceinline__ void mfma_16x16x32(const u32x4_t& a, const u32x4_t& b, f32x4_t& acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}

// Activation tile: row r, 16-byte chunk c (k = 8c .. 8c+7) at chunk position
// c ^ (r % 16), so the 16 rows of a fragment read and the 16 chunks of a row
// store each cover all banks once.
__device__ __forceinline__ int x_lds(int r, int c) { return (r * 16 + (c ^ (r & 15))) * 16; }
// Weight tile: row n, word p (0..15) at word 4 ((p / 4) ^ ((n / 4) % 4)) + p % 4.
__device__ __forceinline__ int w_lds(int n, int p) { return (n * 16 + 4 * ((p >> 2) ^ ((n >> 2) & 3)) + (p & 3)) * 4; }

// One register slot: this thread's share of one step's tiles.
constexpr int kXL = kRB * 4 / kWaves;  // activation loads per thread per step
struct Slot {
    u32x4_t a[kXL];  // activation chunk (tid % 16) of rows tid / 16 + (kThreads / 16) i
    uint32_t w;      // weight word (tid % 16) of row tid / 16
};

template <bool kSplit>
__global__ __launch_bounds__(kThreads) void gemm_int4_mfma_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ qw, const uint16_t* __restrict__ s,
    const uint16_t* __restrict__ z, uint16_t* __restrict__ y, float* __restrict__ ws, int M, int K,
    int N, int splits) {
    __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int li = lane & 15, lb = lane >> 4;
    const int wsl = wave & 3, nh = wave >> 2;  // k-slice and N part of this wave
    const int n0 = blockIdx.x * kBN;
    const int m0 = blockIdx.y * kBM;
    const int G = K / kGroup;
    const int g0 = (int)(((long)blockIdx.z * G) / splits);
    const int g1 = (int)(((long)(blockIdx.z + 1) * G) / splits);
    const int nsteps = g1 - g0;
    const uint32_t row_bytes = (uint32_t)K / 2;

    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)((size_t)M * K * 2));
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qw, (uint32_t)((size_t)N * row_bytes));
    const __amdgpu_buffer_rsrc_t rnone = make_rsrc(qw, 0u);

    // Scales and zeros of rows n0 .. n0+63 (all G groups; rows past N read 0
    // and are never stored): contiguous [64 G] fp16 blocks, staged raw.
    {
        const uint32_t sz_bytes = (uint32_t)((size_t)N * G * 2);
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(s, sz_bytes);
        const __amdgpu_buffer_rsrc_t rz = make_rsrc(z, sz_bytes);
        // 16-byte aligned: n0 is a multiple of 64.  The whole offset is the
        // lane offset, which the buffer range check covers.
        const uint32_t base = (uint32_t)n0 * (uint32_t)G * 2u;
        const int chunks = kBN * G * 2 / 16;  // per array
        for (int c = tid; c < chunks; c += kThreads) {
            const uint32_t off = base + (uint32_t)c * 16u;
            u32x4_t vs, vz;
            if (off + 16u <= sz_bytes) {
                vs = buf_load_b128(rs, off, 0u);
                vz = buf_load_b128(rz, off, 0u);
            } else {
                // The chunk that straddles the end of the arrays: a 16-byte load
                // partly out of range reads all zeros, so take it 2 bytes at a
                // time (halves at or past the end read 0).
                uint32_t hs[8], hz[8];
#pragma unroll
                for (int h = 0; h < 8; ++h) {
                    hs[h] = buf_load_u16(rs, off + 2u * h, 0u);
                    hz[h] = buf_load_u16(rz, off + 2u * h, 0u);
                }
                vs = u32x4_t{hs[0] | hs[1] << 16, hs[2] | hs[3] << 16, hs[4] | hs[5] << 16, hs[6] | hs[7] << 16};
                vz = u32x4_t{hz[0] | hz[1] << 16, hz[2] | hz[3] << 16, hz[4] | hz[5] << 16, hz[6] | hz[7] << 16};
            }
            *reinterpret_cast<u32x4_t*>(lds + kOffSZ + c * 16) = vs;
            *reinterpret_cast<u32x4_t*>(lds + kOffSZ + kBN * G * 2 + c * 16) = vz;
        }
    }
    const uint16_t* lds_s = reinterpret_cast<const uint16_t*>(lds + kOffSZ);
    const uint16_t* lds_z = lds_s + kBN * G;

    // Global loaders.  Activations: chunk tid % 16 of rows tid / 16 + 16 i
    // (rows past M read row M - 1, never stored).  Weights: chunk tid % 4 of
    // row tid / 4 (rows past N read row N - 1).
    const int xr = tid >> 4, xc = tid & 15;
    constexpr int kXRows = kThreads / 16;
    uint32_t xoff[kXL];
#pragma unroll
    for (int i = 0; i < kXL; ++i) xoff[i] = (uint32_t)(((size_t)min(m0 + xr + kXRows * i, M - 1) * K + 8 * xc) * 2);
    const int wr = tid >> 4, wc = tid & 15;
    const uint32_t woff = (uint32_t)min(n0 + wr, N - 1) * row_bytes + 4u * wc;

    auto issue = [&](int j, Slot& S) {
        const bool live = j < nsteps;
        const uint32_t g = (uint32_t)(g0 + (live ? j : 0));
        const __amdgpu_buffer_rsrc_t ra = live ? rx : rnone;
        const __amdgpu_buffer_rsrc_t rw = live ? rq : rnone;
        S.w = __builtin_amdgcn_raw_buffer_load_b32(rw, (int)woff, (int)sgpr(g * 64u), kAuxNontemporal);
#pragma unroll
        for (int i = 0; i < kXL; ++i) S.a[i] = buf_load_b128(ra, xoff[i], g * 256u);
    };
    auto store = [&](const Slot& S, int buf) {
        *reinterpret_cast<uint32_t*>(lds + kOffW + buf * kWTile + w_lds(wr, wc)) = S.w;
#pragma unroll
        for (int i = 0; i < kXL; ++i)
            *reinterpret_cast<u32x4_t*>(lds + buf * kXTile + x_lds(xr + kXRows * i, xc)) = S.a[i];
    };

    f32x4_t acc[kRB][kCBW];
#pragma unroll
    for (int r = 0; r < kRB; ++r)
#pragma unroll
        for (int c = 0; c < kCBW; ++c) acc[r][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Step j computes group g0 + j from LDS buffer j & 1.  Before it, the
    // register slot holding step j + 1 was stored into the other buffer and
    // refilled with step j + 1 + kDepth.
    Slot ring[kDepth];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
        issue(d, ring[d]);
        __builtin_amdgcn_sched_barrier(0);
    }
    store(ring[0], 0);
    issue(kDepth, ring[0]);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    for (int j0 = 0; j0 < nsteps; j0 += kDepth) {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            const int j = j0 + d;
            const int buf = j & 1;
            const char* xt = lds + buf * kXTile;
            const char* wt = lds + kOffW + buf * kWTile;
            u32x4_t b[kCBW];
#pragma unroll
            for (int c = 0; c < kCBW; ++c) {
                const int n = 16 * (kCBW * nh + c) + li;
                const uint32_t q = *reinterpret_cast<const uint32_t*>(wt + w_lds(n, 4 * wsl + lb));
                // A surplus step past the range (nsteps not a multiple of
                // kDepth) has zero tiles; its scale and zero stay finite.
                const int gi = g0 + min(j, nsteps - 1);
                const float sc = f16_to_f32(lds_s[n * G + gi]);
                const float zp = f16_to_f32(lds_z[n * G + gi]);
                b[c] = int4_word_dequant_bf16(q, sc, -zp * sc);
            }
#pragma unroll
            for (int r = 0; r < kRB; ++r) {
                const u32x4_t a = *reinterpret_cast<const u32x4_t*>(xt + x_lds(16 * r + li, 4 * wsl + lb));
#pragma unroll
                for (int c = 0; c < kCBW; ++c) mfma_16x16x32(a, b[c], acc[r][c]);
            }
            Slot& T = ring[(d + 1) % kDepth];
            store(T, buf ^ 1);
            issue(j + 1 + kDepth, T);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
        }
    }

    // Cross-wave sum: every wave stores its partials, then thread t adds the
    // four copies of 4-float groups t, t + 256, ... in wave order.
    float* red = reinterpret_cast<float*>(lds);
    constexpr int kPer = kRB * kCBW * kWave * 4;  // floats per wave
#pragma unroll
    for (int r = 0; r < kRB; ++r)
#pragma unroll
        for (int c = 0; c < kCBW; ++c)
            *reinterpret_cast<f32x4_t*>(&red[wave * kPer + ((r * kCBW + c) * kWave + lane) * 4]) = acc[r][c];
    __syncthreads();
#pragma unroll
    for (int i = tid; i < kNH * kPer / 4; i += kThreads) {
        // i = (part * kRB * kCBW + r * kCBW + c) * 64 + l: rows 16 r + 4 (l / 16) + e,
        // column 16 (kCBW part + c) + l % 16; summed over the 4 k-slice waves of the part.
        const int part = i / (kPer / 4), ii = i % (kPer / 4);
        f32x4_t t = *reinterpret_cast<const f32x4_t*>(&red[(4 * part) * kPer + ii * 4]);
#pragma unroll
        for (int w = 1; w < 4; ++w) t += *reinterpret_cast<const f32x4_t*>(&red[(4 * part + w) * kPer + ii * 4]);
        const int l = ii & (kWave - 1), rc = ii / kWave;
        const int r = rc / kCBW, c = kCBW * part + rc % kCBW;
        const int n = n0 + 16 * c + (l & 15);
        if (n >= N) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = m0 + 16 * r + 4 * (l >> 4) + e;
            if (m >= M) continue;
            if constexpr (kSplit) {
                ws[((size_t)blockIdx.z * M + m) * N + n] = t[e];
            } else {
                y[(size_t)m * N + n] = f32_to_bf16(t[e]);
            }
        }
    }
}

// y = bf16(sum over splits of the FP32 partials), splits added in order;
// four consecutive outputs per thread (16-byte partial loads, one 8-byte
// store), the last few one at a time when M * N is not a multiple of four.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ ws,
                                                            uint16_t* __restrict__ y, size_t count,
                                                            int splits) {
    const size_t i = 4 * ((size_t)blockIdx.x * blockDim.x + threadIdx.x);
    if (i >= count) return;
    // (The workspace is 16-byte aligned; y only 2-byte aligned in general.)
    if (i + 4 <= count && (count & 3) == 0 && (reinterpret_cast<uintptr_t>(y) & 7) == 0) {
        f32x4_t t = *reinterpret_cast<const f32x4_t*>(ws + i);
        for (int k = 1; k < splits; ++k) t += *reinterpret_cast<const f32x4_t*>(ws + (size_t)k * count + i);
        *reinterpret_cast<u32x2_t*>(y + i) = u32x2_t{pack_bf16x2(t[0], t[1]), pack_bf16x2(t[2], t[3])};
        return;
    }
    for (size_t e = i; e < i + 4 && e < count; ++e) {
        float t = ws[e];
        for (int k = 1; k < splits; ++k) t += ws[(size_t)k * count + e];
        y[e] = f32_to_bf16(t);
    }
}


}  // namespace

size_t gemm_int4_workspace_bytes(int M, int K, int N) {
    if (M <= kGemmSmallMMax || N <= 0 || K <= 0 || K % kGroup != 0 || K > W4_GEMM_MAX_K) return 0;
    const int splits = gemm_splits(M, K, N);
    return splits > 1 ? (size_t)splits * (size_t)M * (size_t)N * sizeof(float) : 0;
}

hipError_t launch_gemm_int4(const void* x, const int32_t* qw, const void* s, const void* z,
                            void* y, int M, int K, int N, void* workspace, hipStream_t stream) {
    // One row is a GEMV: its kernel streams the weights at a higher rate than
    // the 16-row matrix-core block of the small-M path (K <= W4_GEMM_MAX_K ==
    // W4_GEMV_MAX_K).
    if (M == 1) return launch_gemv_int4(x, qw, s, z, y, K, N, stream);
    // Two rows: still a GEMV, each unpacked word shared by both rows.
    if (gemv_rows_int4_supports(M, K)) return launch_gemv_rows_int4(x, qw, s, z, y, M, K, N, stream);
    if (M <= kGemmSmallMMax) return launch_gemm_int4_small_m(x, qw, s, z, y, M, K, N, stream);
    const int splits = gemm_splits(M, K, N);
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
    const unsigned blocks = (unsigned)((count + 1023) / 1024);
    splitk_reduce_kernel<<<blocks, 256, 0, stream>>>(ws, yb, count, splits);
    return hipGetLastError();
}

// Scratch for w4_gemm_noalloc, the entry point for callers that cannot
// allocate: the split-K partial sums go here instead of into a workspace of
// the caller's.  A __device__ array: every GPU the library runs on holds its
// own copy until the process ends, and every call on that GPU shares it.  In
// host code the array's name is not a device address; its address on the
// current device comes from hipGetSymbolAddress, resolved once per device on
// that device's first call and kept.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t gemm_noalloc_scratch(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* per_device[kMaxDevices] = {};
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!per_device[dev]) {
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        per_device[dev] = p;
    }
    *ptr = per_device[dev];
    return hipSuccess;
}

}  // namespace w4
