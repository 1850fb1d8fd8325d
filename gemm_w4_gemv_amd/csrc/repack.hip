// Import of weights in GPTQ's own layout.
//
// "Lab 5: Gemma4 端到端推理优化", section "量化正确性": the linears are
// quantised with GPTQ (INT4, group 128, asymmetric).  GPTQ keeps the packed
// codes K-major, qweight int32 [K/8][N] (word (p, n) holds the codes of
// k = 8p .. 8p+7 of output n, nibble j for k = 8p + j), with scales and zeros
// [K/128][N].  The kernels here read one weight row's codes contiguously
// (F.linear orientation, [N][K/8]), so a GPTQ checkpoint is repacked once, at
// load: a transpose of 32-bit words (the nibble order inside a word is the
// same in both layouts) and of the 16-bit scales and zeros.
//
// One 64 x 64 tile per workgroup of 256 threads, staged through LDS so that
// both the reads (along a source row) and the writes (along a destination
// row) are whole consecutive runs; the LDS row is padded by one element so
// the column reads of the transposed tile hit distinct banks.
#include "w4_internal.hpp"

namespace w4 {
namespace {

constexpr int kTile = 64, kRowsPerPass = 4;

// dst[c][r] = src[r][c] for a rows x cols matrix of T.
template <typename T>
__global__ __launch_bounds__(kTile * kRowsPerPass) void transpose_kernel(const T* __restrict__ src,
                                                                          T* __restrict__ dst, int rows, int cols) {
    __shared__ T tile[kTile][kTile + 1];
    const int tx = threadIdx.x % kTile, ty = threadIdx.x / kTile;
    const int r0 = blockIdx.y * kTile, c0 = blockIdx.x * kTile;
    for (int i = ty; i < kTile; i += kRowsPerPass) {
        const int r = r0 + i, c = c0 + tx;
        if (r < rows && c < cols) tile[i][tx] = src[(size_t)r * cols + c];
    }
    __syncthreads();
    for (int i = ty; i < kTile; i += kRowsPerPass) {
        const int c = c0 + i, r = r0 + tx;  // destination row c, column r
        if (c < cols && r < rows) dst[(size_t)c * rows + r] = tile[tx][i];
    }
}

template <typename T>
hipError_t transpose(const void* src, void* dst, int rows, int cols, hipStream_t stream) {
    if (rows == 0 || cols == 0) return hipSuccess;
    const dim3 grid((unsigned)((cols + kTile - 1) / kTile), (unsigned)((rows + kTile - 1) / kTile));
    transpose_kernel<T><<<grid, kTile * kRowsPerPass, 0, stream>>>(static_cast<const T*>(src), static_cast<T*>(dst),
                                                                    rows, cols);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_repack_gptq(const int32_t* qw_kn, const void* s_gn, const void* z_gn, int32_t* qw, void* s, void* z,
                              int K, int N, hipStream_t stream) {
    hipError_t err = transpose<uint32_t>(qw_kn, qw, K / 8, N, stream);
    if (err == hipSuccess) err = transpose<uint16_t>(s_gn, s, K / 128, N, stream);
    if (err == hipSuccess) err = transpose<uint16_t>(z_gn, z, K / 128, N, stream);
    return err;
}

}  // namespace w4
