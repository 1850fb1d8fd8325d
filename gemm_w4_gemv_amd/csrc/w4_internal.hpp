// Launchers behind the C ABI.  Arguments are already validated by the caller
// (w4_api.hip); each launcher only picks a launch shape and enqueues kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "w4.h"

namespace w4 {

hipError_t launch_gemv_int4(const void* x, const int32_t* qw, const void* s, const void* z,
                            void* y, int K, int N, hipStream_t stream);

size_t gemm_int4_workspace_bytes(int M, int K, int N);
// Output tile of the prefill GEMM's workgroup (rows of x, weight rows).
constexpr int kGemmTileM = 128, kGemmTileN = 64;
// Small-M path of w4_gemm (M <= kGemmSmallMMax): one matrix-core block of 16
// x rows against the weights, streamed once, no workspace.  Measured on the
// decode shapes (us, small-M path vs the tiled GEMM): M = 16: 16.8 vs 23.0
// (K3840 -> N15360), 18.2 vs 26.5 (K15360 -> N3840); M = 32 (two 16-row
// passes over the weights): 31.1 vs 23.0, 27.8 vs 26.9.
constexpr int kGemmSmallMMax = 16;
hipError_t launch_gemm_int4_small_m(const void* x, const int32_t* qw, const void* s, const void* z,
                                    void* y, int M, int K, int N, hipStream_t stream);
hipError_t launch_gemm_int4(const void* x, const int32_t* qw, const void* s, const void* z,
                            void* y, int M, int K, int N, void* workspace, hipStream_t stream);
// The split-K scratch of w4_gemm_noalloc: its size, and its address on the
// current device (resolved on the device's first call, then kept).
constexpr size_t kNoAllocScratchBytes = W4_GEMM_NOALLOC_SCRATCH_BYTES;
hipError_t gemm_noalloc_scratch(void** ptr);
// Two rows of x as a GEMV: each unpacked weight word is dotted with both
// rows; K <= 16384 (x held in registers).
bool gemv_rows_int4_supports(int M, int K);
hipError_t launch_gemv_rows_int4(const void* x, const int32_t* qw, const void* s, const void* z, void* y,
                                 int M, int K, int N, hipStream_t stream);

hipError_t launch_moe_gemv_fp4(const void* x, int64_t x_stride, const uint8_t* qw,
                               const void* s, const int32_t* ids, void* y, int E,
                               int num_experts, int K, int N, hipStream_t stream);

// One FC of expert GEMVs, as w4_moe_gemv takes it.
struct MoeFcArgs {
    const void* x;
    int64_t x_stride;
    const uint8_t* qw;
    const void* s;
    void* y;
    int K, N;
};
hipError_t launch_moe_gemv2_fp4(const MoeFcArgs& a, const MoeFcArgs& b, const int32_t* ids, int E, int num_experts,
                                hipStream_t stream);

hipError_t launch_moe_gemm_fp4(const void* x, const int32_t* row_start, const int32_t* ids, const uint8_t* qw,
                               const void* s, void* y, int R, int E, int max_rows, int num_experts, int K, int N,
                               hipStream_t stream);
// One FC of the grouped expert GEMM, as w4_moe_gemm takes it.
struct MoeGemmFcArgs {
    const void* x;
    const uint8_t* qw;
    const void* s;
    void* y;
    int K, N;
};
hipError_t launch_moe_gemm2_fp4(const MoeGemmFcArgs& a, const MoeGemmFcArgs& b, const int32_t* row_start,
                                const int32_t* ids, int R, int E, int max_rows, int num_experts,
                                hipStream_t stream);

hipError_t launch_dequant_int4(const int32_t* qw, const void* s, const void* z, float* out_f32,
                               void* out_bf16, int K, int N, hipStream_t stream);
hipError_t launch_int4_gemv_operands(const int32_t* qw, const void* x, uint32_t* out_codes, uint32_t* out_x, int K,
                                     int N, hipStream_t stream);
hipError_t launch_dequant_fp4(const uint8_t* qw, const void* s, float* out_f32, void* out_bf16,
                              int K, int N, hipStream_t stream);

hipError_t launch_repack_gptq(const int32_t* qw_kn, const void* s_gn, const void* z_gn, int32_t* qw, void* s, void* z,
                              int K, int N, hipStream_t stream);

hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, int sink_words, hipStream_t stream);

// Split of the K range of a GEMV row over the four waves of a workgroup.
// A row has C = K / 32 chunks of 16 bytes.  Each lane owns up to ``cpl``
// chunks of one K-slice and keeps their x values in registers; ``slices``
// waves share a row when the row is too long for one wave.
struct RowSplit {
    int slices;  // 1, 2 or 4 waves per row
    int cpl;     // chunks per lane, 1..4
};

inline RowSplit row_split(int chunks) {
    if (chunks <= 128) return {1, (chunks + 63) / 64};
    if (chunks <= 256) return {2, 2};
    return {4, (chunks + 255) / 256};
}

}  // namespace w4
