// C ABI of the fused 4-bit-weight GEMV/GEMM library: host-side validation,
// dispatch to the launchers, HIP-graph capture helpers and error reporting.
// Every check here runs before the first HIP call of an entry point, so an
// invalid call launches nothing and can be tested on a host without a GPU.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "chain.hpp"
#include "tune.hpp"
#include "w4.h"
#include "w4_internal.hpp"

namespace {

thread_local char g_last_error[256] = "no error";

w4_status fail(w4_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
w4_status fail(w4_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

w4_status hip_fail(hipError_t err, const char* what) {
    return fail(W4_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(err), (int)err);
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};
Range range(const void* p, size_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return {a, a + bytes};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo < a.hi && b.lo < b.hi; }

// Shared checks of the INT4 weight operand and K.
w4_status check_int4(const char* fn, const int32_t* qw, const void* s, const void* z, int K, int N,
                     int g, int max_k) {
    if (!qw || !s || !z) return fail(W4_ERR_NULL, "%s: qw, s and z must not be NULL", fn);
    if (g != W4_INT4_GROUP) return fail(W4_ERR_UNSUPPORTED, "%s: group size %d (only 128 is supported)", fn, g);
    if (N < 0) return fail(W4_ERR_SHAPE, "%s: N = %d is negative", fn, N);
    if (K <= 0 || K % g != 0) return fail(W4_ERR_SHAPE, "%s: K = %d is not a positive multiple of %d", fn, K, g);
    if (max_k > 0 && K > max_k) return fail(W4_ERR_SHAPE, "%s: K = %d exceeds the limit %d", fn, K, max_k);
    if (!aligned(qw, 16)) return fail(W4_ERR_ALIGN, "%s: qw must be 16-byte aligned", fn);
    if (!aligned(s, 2) || !aligned(z, 2)) return fail(W4_ERR_ALIGN, "%s: s and z must be 2-byte aligned", fn);
    return W4_OK;
}

}  // namespace

extern "C" {

W4_API int w4_abi_version(void) { return 1; }

W4_API const char* w4_status_string(w4_status status) {
    switch (status) {
        case W4_OK: return "W4_OK";
        case W4_ERR_NULL: return "W4_ERR_NULL";
        case W4_ERR_SHAPE: return "W4_ERR_SHAPE";
        case W4_ERR_UNSUPPORTED: return "W4_ERR_UNSUPPORTED";
        case W4_ERR_ALIGN: return "W4_ERR_ALIGN";
        case W4_ERR_WORKSPACE: return "W4_ERR_WORKSPACE";
        case W4_ERR_ALIAS: return "W4_ERR_ALIAS";
        case W4_ERR_ARG: return "W4_ERR_ARG";
        case W4_ERR_HIP: return "W4_ERR_HIP";
    }
    return "W4_ERR_UNKNOWN";
}

W4_API const char* w4_last_error(void) { return g_last_error; }

W4_API w4_status w4_gemv(const void* x, const int32_t* qw, const void* s, const void* z, void* y,
                         int K, int N, int g, void* stream) {
    const char* fn = "w4_gemv";
    if (!x || !y) return fail(W4_ERR_NULL, "%s: x and y must not be NULL", fn);
    w4_status st = check_int4(fn, qw, s, z, K, N, g, W4_GEMV_MAX_K);
    if (st != W4_OK) return st;
    if (!aligned(x, 16)) return fail(W4_ERR_ALIGN, "%s: x must be 16-byte aligned", fn);
    if (!aligned(y, 2)) return fail(W4_ERR_ALIGN, "%s: y must be 2-byte aligned", fn);
    if ((unsigned long long)N * (unsigned long long)(K / 2) > W4_GEMV_MAX_MATRIX_BYTES)
        return fail(W4_ERR_SHAPE, "%s: N * K / 2 exceeds %llu bytes", fn, W4_GEMV_MAX_MATRIX_BYTES);
    const Range ry = range(y, (size_t)N * 2);
    const size_t sz_bytes = (size_t)N * (K / g) * 2;
    if (overlap(ry, range(x, (size_t)K * 2)) || overlap(ry, range(qw, (size_t)N * K / 2)) ||
        overlap(ry, range(s, sz_bytes)) || overlap(ry, range(z, sz_bytes)))
        return fail(W4_ERR_ALIAS, "%s: y overlaps an input", fn);
    if (N == 0) return W4_OK;
    hipError_t err = w4::launch_gemv_int4(x, qw, s, z, y, K, N, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? W4_OK : hip_fail(err, fn);
}

W4_API size_t w4_gemm_workspace_bytes(int M, int K, int N, int g) {
    if (g != W4_INT4_GROUP) return 0;
    return w4::gemm_int4_workspace_bytes(M, K, N);
}

W4_API w4_status w4_gemm(const void* x, const int32_t* qw, const void* s, const void* z, void* y,
                         int M, int K, int N, int g, void* workspace, size_t workspace_bytes,
                         void* stream) {
    const char* fn = "w4_gemm";
    if (!x || !y) return fail(W4_ERR_NULL, "%s: x and y must not be NULL", fn);
    w4_status st = check_int4(fn, qw, s, z, K, N, g, W4_GEMM_MAX_K);
    if (st != W4_OK) return st;
    if (M < 0) return fail(W4_ERR_SHAPE, "%s: M = %d is negative", fn, M);
    if ((unsigned long long)M * (unsigned long long)K * 2ull > W4_GEMV_MAX_MATRIX_BYTES ||
        (unsigned long long)N * (unsigned long long)(K / 2) > W4_GEMV_MAX_MATRIX_BYTES)
        return fail(W4_ERR_SHAPE, "%s: M * K * 2 or N * K / 2 exceeds %llu bytes", fn, W4_GEMV_MAX_MATRIX_BYTES);
    if (!aligned(x, 16)) return fail(W4_ERR_ALIGN, "%s: x must be 16-byte aligned", fn);
    if (!aligned(y, 2)) return fail(W4_ERR_ALIGN, "%s: y must be 2-byte aligned", fn);
    const size_t need = w4_gemm_workspace_bytes(M, K, N, g);
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(W4_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given%s", fn, need,
                        workspace_bytes, workspace ? "" : " (NULL)");
        if (!aligned(workspace, 16)) return fail(W4_ERR_ALIGN, "%s: workspace must be 16-byte aligned", fn);
    }
    const Range ry = range(y, (size_t)M * N * 2);
    const Range rw = range(workspace, need);
    const size_t sz_bytes = (size_t)N * (K / g) * 2;
    const Range ins[4] = {range(x, (size_t)M * K * 2), range(qw, (size_t)N * K / 2), range(s, sz_bytes),
                          range(z, sz_bytes)};
    for (const Range& r : ins)
        if (overlap(ry, r) || overlap(rw, r)) return fail(W4_ERR_ALIAS, "%s: y or workspace overlaps an input", fn);
    if (overlap(ry, rw)) return fail(W4_ERR_ALIAS, "%s: y overlaps the workspace", fn);
    if (M == 0 || N == 0) return W4_OK;
    hipError_t err = w4::launch_gemm_int4(x, qw, s, z, y, M, K, N, workspace, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? W4_OK : hip_fail(err, fn);
}

W4_API w4_status w4_gemm_noalloc(const void* x, const int32_t* qw, const void* s, const void* z, void* y, int M,
                                 int K, int N, int g, void* stream) {
    const char* fn = "w4_gemm_noalloc";
    if (!x || !y) return fail(W4_ERR_NULL, "%s: x and y must not be NULL", fn);
    w4_status st = check_int4(fn, qw, s, z, K, N, g, W4_GEMM_MAX_K);
    if (st != W4_OK) return st;
    if (M < 0) return fail(W4_ERR_SHAPE, "%s: M = %d is negative", fn, M);
    if ((unsigned long long)M * (unsigned long long)K * 2ull > W4_GEMV_MAX_MATRIX_BYTES ||
        (unsigned long long)N * (unsigned long long)(K / 2) > W4_GEMV_MAX_MATRIX_BYTES)
        return fail(W4_ERR_SHAPE, "%s: M * K * 2 or N * K / 2 exceeds %llu bytes", fn, W4_GEMV_MAX_MATRIX_BYTES);
    if (!aligned(x, 16)) return fail(W4_ERR_ALIGN, "%s: x must be 16-byte aligned", fn);
    if (!aligned(y, 2)) return fail(W4_ERR_ALIGN, "%s: y must be 2-byte aligned", fn);
    const size_t need = w4_gemm_workspace_bytes(M, K, N, g);
    if (need > W4_GEMM_NOALLOC_SCRATCH_BYTES)
        return fail(W4_ERR_WORKSPACE, "%s: M = %d, K = %d, N = %d needs %zu bytes of split-K scratch, above the "
                    "library's %llu", fn, M, K, N, need, (unsigned long long)W4_GEMM_NOALLOC_SCRATCH_BYTES);
    const Range ry = range(y, (size_t)M * N * 2);
    const size_t sz_bytes = (size_t)N * (K / g) * 2;
    const Range ins[4] = {range(x, (size_t)M * K * 2), range(qw, (size_t)N * K / 2), range(s, sz_bytes),
                          range(z, sz_bytes)};
    for (const Range& r : ins)
        if (overlap(ry, r)) return fail(W4_ERR_ALIAS, "%s: y overlaps an input", fn);
    if (M == 0 || N == 0) return W4_OK;
    void* scratch = nullptr;
    if (need > 0) {
        hipError_t err = w4::gemm_noalloc_scratch(&scratch);
        if (err != hipSuccess) return hip_fail(err, fn);
    }
    hipError_t err = w4::launch_gemm_int4(x, qw, s, z, y, M, K, N, scratch, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? W4_OK : hip_fail(err, fn);
}

W4_API int w4_tune_param(int kernel, int M, int K, int N) {
    switch (kernel) {
        case W4_TUNE_GEMV: return w4::gemv_rows_per_wave(K, N);
        case W4_TUNE_GEMV_ROWS2: return w4::gemv_rows2_rows_per_wave(K, N);
        case W4_TUNE_GEMM_SMALL_M: return w4::gemm_small_m_blocks(M, K, N);
        case W4_TUNE_GEMM: return w4::gemm_splits(M, K, N);
        case W4_TUNE_MOE_GEMV: return w4::moe_gemv_rows_per_wave(M, K, N);
        default: return -1;
    }
}

W4_API w4_status w4_tune_force(int kernel, int param) {
    if (kernel < 0 || kernel >= W4_TUNE_KERNELS) return fail(W4_ERR_ARG, "w4_tune_force: unknown kernel %d", kernel);
    if (param != 0 && !w4::tune_param_valid(kernel, param))
        return fail(W4_ERR_ARG, "w4_tune_force: %d is not a launch parameter of kernel %d", param, kernel);
    w4::tune_force(kernel, param);
    return W4_OK;
}

W4_API w4_status w4_repack_gptq(const int32_t* qw_kn, const void* s_gn, const void* z_gn, int32_t* qw, void* s,
                                void* z, int K, int N, int g, void* stream) {
    const char* fn = "w4_repack_gptq";
    if (!qw_kn || !s_gn || !z_gn || !qw || !s || !z) return fail(W4_ERR_NULL, "%s: no pointer may be NULL", fn);
    if (g != W4_INT4_GROUP) return fail(W4_ERR_UNSUPPORTED, "%s: group size %d (only 128 is supported)", fn, g);
    if (N < 0) return fail(W4_ERR_SHAPE, "%s: N = %d is negative", fn, N);
    if (K <= 0 || K % g != 0) return fail(W4_ERR_SHAPE, "%s: K = %d is not a positive multiple of %d", fn, K, g);
    if (!aligned(qw_kn, 4) || !aligned(qw, 4) || !aligned(s_gn, 2) || !aligned(z_gn, 2) || !aligned(s, 2) ||
        !aligned(z, 2))
        return fail(W4_ERR_ALIGN, "%s: packed words must be 4-byte, scales and zeros 2-byte aligned", fn);
    const size_t wb = (size_t)N * K / 2, sb = (size_t)N * (K / g) * 2;
    const Range ins[3] = {range(qw_kn, wb), range(s_gn, sb), range(z_gn, sb)};
    const Range outs[3] = {range(qw, wb), range(s, sb), range(z, sb)};
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 3; ++j)
            if (overlap(outs[i], ins[j])) return fail(W4_ERR_ALIAS, "%s: an output overlaps an input", fn);
        for (int j = 0; j < i; ++j)
            if (overlap(outs[i], outs[j])) return fail(W4_ERR_ALIAS, "%s: two outputs overlap", fn);
    }
    if (N == 0) return W4_OK;
    hipError_t err = w4::launch_repack_gptq(qw_kn, s_gn, z_gn, qw, s, z, K, N, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? W4_OK : hip_fail(err, fn);
}

W4_API w4_status w4_moe_gemv(const void* x, int64_t x_stride, const uint8_t* qw_fp4, const void* s_fp4,
                             const int32_t* expert_ids, void* y, int E, int num_experts, int K, int N,
                             void* stream) {
    const char* fn = "w4_moe_gemv";
    if (!x || !qw_fp4 || !s_fp4 || !expert_ids || !y)
        return fail(W4_ERR_NULL, "%s: x, qw_fp4, s_fp4, expert_ids and y must not be NULL", fn);
    if (E < 0 || N < 0) return fail(W4_ERR_SHAPE, "%s: E = %d, N = %d must not be negative", fn, E, N);
    if (K <= 0 || K % W4_FP4_GROUP != 0 || K > W4_GEMV_MAX_K)
        return fail(W4_ERR_SHAPE, "%s: K = %d must be a positive multiple of 32 up to %d", fn, K, W4_GEMV_MAX_K);
    if (num_experts < 1) return fail(W4_ERR_ARG, "%s: num_experts = %d must be positive", fn, num_experts);
    if ((unsigned long long)N * (unsigned long long)(K / 2) > W4_GEMV_MAX_MATRIX_BYTES)
        return fail(W4_ERR_SHAPE, "%s: N * K / 2 exceeds %llu bytes", fn, W4_GEMV_MAX_MATRIX_BYTES);
    if (x_stride < 0 || x_stride % 8 != 0)
        return fail(W4_ERR_ARG, "%s: x_stride = %lld must be a non-negative multiple of 8", fn, (long long)x_stride);
    if (!aligned(x, 16) || !aligned(qw_fp4, 16))
        return fail(W4_ERR_ALIGN, "%s: x and qw_fp4 must be 16-byte aligned", fn);
    if (!aligned(s_fp4, 2) || !aligned(y, 2) || !aligned(expert_ids, 4))
        return fail(W4_ERR_ALIGN, "%s: s_fp4 and y must be 2-byte, expert_ids 4-byte aligned", fn);
    const Range ry = range(y, (size_t)E * N * 2);
    const size_t x_elems = E > 0 ? (size_t)(E - 1) * (size_t)x_stride + (size_t)K : 0;
    const Range ins[4] = {range(x, x_elems * 2), range(qw_fp4, (size_t)num_experts * N * K / 2),
                          range(s_fp4, (size_t)num_experts * N * (K / 32) * 2), range(expert_ids, (size_t)E * 4)};
    for (const Range& r : ins)
        if (overlap(ry, r)) return fail(W4_ERR_ALIAS, "%s: y overlaps an input", fn);
    if (E == 0 || N == 0) return W4_OK;
    hipError_t err = w4::launch_moe_gemv_fp4(x, x_stride, qw_fp4, s_fp4, expert_ids, y, E, num_experts, K, N,
                                             static_cast<hipStream_t>(stream));
    return err == hipSuccess ? W4_OK : hip_fail(err, fn);
}

W4_API w4_status w4_moe_gemv2(const w4_moe_fc* fc1, const w4_moe_fc* fc2, const int32_t* expert_ids, int E,
                              int num_experts, void* stream) {
    const char* fn = "w4_moe_gemv2";
    if (!fc1 || !fc2 || !expert_ids) return fail(W4_ERR_NULL, "%s: fc1, fc2 and expert_ids must not be NULL", fn);
    if (E < 0) return fail(W4_ERR_SHAPE, "%s: E = %d is negative", fn, E);
    if (num_experts < 1) return fail(W4_ERR_ARG, "%s: num_experts = %d must be positive", fn, num_experts);
    if (!aligned(expert_ids, 4)) return fail(W4_ERR_ALIGN, "%s: expert_ids must be 4-byte aligned", fn);
    const w4_moe_fc* fcs[2] = {fc1, fc2};
    Range ys[2], ins[2][3];
    for (int i = 0; i < 2; ++i) {
        const w4_moe_fc& f = *fcs[i];
        if (!f.x || !f.qw_fp4 || !f.s_fp4 || !f.y)
            return fail(W4_ERR_NULL, "%s: fc%d: x, qw_fp4, s_fp4 and y must not be NULL", fn, i + 1);
        if (f.N < 0) return fail(W4_ERR_SHAPE, "%s: fc%d: N = %d is negative", fn, i + 1, f.N);
        if (f.K <= 0 || f.K % W4_FP4_GROUP != 0 || f.K > W4_GEMV_MAX_K)
            return fail(W4_ERR_SHAPE, "%s: fc%d: K = %d must be a positive multiple of 32 up to %d", fn, i + 1, f.K,
                        W4_GEMV_MAX_K);
        if ((unsigned long long)f.N * (unsigned long long)(f.K / 2) > W4_GEMV_MAX_MATRIX_BYTES)
            return fail(W4_ERR_SHAPE, "%s: fc%d: N * K / 2 exceeds %llu bytes", fn, i + 1, W4_GEMV_MAX_MATRIX_BYTES);
        if (f.x_stride < 0 || f.x_stride % 8 != 0)
            return fail(W4_ERR_ARG, "%s: fc%d: x_stride = %lld must be a non-negative multiple of 8", fn, i + 1,
                        (long long)f.x_stride);
        if (!aligned(f.x, 16) || !aligned(f.qw_fp4, 16))
            return fail(W4_ERR_ALIGN, "%s: fc%d: x and qw_fp4 must be 16-byte aligned", fn, i + 1);
        if (!aligned(f.s_fp4, 2) || !aligned(f.y, 2))
            return fail(W4_ERR_ALIGN, "%s: fc%d: s_fp4 and y must be 2-byte aligned", fn, i + 1);
        ys[i] = range(f.y, (size_t)E * f.N * 2);
        const size_t x_elems = E > 0 ? (size_t)(E - 1) * (size_t)f.x_stride + (size_t)f.K : 0;
        ins[i][0] = range(f.x, x_elems * 2);
        ins[i][1] = range(f.qw_fp4, (size_t)num_experts * f.N * f.K / 2);
        ins[i][2] = range(f.s_fp4, (size_t)num_experts * f.N * (f.K / 32) * 2);
    }
    const Range rid = range(expert_ids, (size_t)E * 4);
    for (int i = 0; i < 2; ++i) {
        if (overlap(ys[i], rid)) return fail(W4_ERR_ALIAS, "%s: fc%d's y overlaps expert_ids", fn, i + 1);
        for (int j = 0; j < 2; ++j)
            for (const Range& r : ins[j])
                if (overlap(ys[i], r))
                    return fail(W4_ERR_ALIAS, "%s: fc%d's y overlaps an input of fc%d (the two FCs run together)",
                                fn, i + 1, j + 1);
    }
    if (overlap(ys[0], ys[1])) return fail(W4_ERR_ALIAS, "%s: the two outputs overlap", fn);
    if (E == 0) return W4_OK;
    if (fc1->N == 0 || fc2->N == 0) {  // one FC only
        const w4_moe_fc& f = fc1->N == 0 ? *fc2 : *fc1;
        if (f.N == 0) return W4_OK;
        hipError_t err = w4::launch_moe_gemv_fp4(f.x, f.x_stride, f.qw_fp4, f.s_fp4, expert_ids, f.y, E, num_experts,
                                                 f.K, f.N, static_cast<hipStream_t>(stream));
        return err == hipSuccess ? W4_OK : hip_fail(err, fn);
    }
    const w4::MoeFcArgs a{fc1->x, fc1->x_stride, fc1->qw_fp4, fc1->s_fp4, fc1->y, fc1->K, fc1->N};
    const w4::MoeFcArgs b{fc2->x, fc2->x_stride, fc2->qw_fp4, fc2->s_fp4, fc2->y, fc2->K, fc2->N};
    hipError_t err = w4::launch_moe_gemv2_fp4(a, b, expert_ids, E, num_experts, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? W4_OK : hip_fail(err, fn);
}

W4_API w4_status w4_moe_gemm(const void* x, const int32_t* row_start, const int32_t* expert_ids,
                             const uint8_t* qw_fp4, const void* s_fp4, void* y, int R, int E, int max_rows,
                             int num_experts, int K, int N, void* stream) {
    const char* fn = "w4_moe_gemm";
    if (!x || !row_start || !expert_ids || !qw_fp4 || !s_fp4 || !y)
        return fail(W4_ERR_NULL, "%s: x, row_start, expert_ids, qw_fp4, s_fp4 and y must not be NULL", fn);
    if (R < 0 || E < 0 || max_rows < 0 || N < 0)
        return fail(W4_ERR_SHAPE, "%s: R = %d, E = %d, max_rows = %d, N = %d must not be negative", fn, R, E,
                    max_rows, N);
    if (K <= 0 || K % 128 != 0 || K > W4_MOE_GEMM_MAX_K)
        return fail(W4_ERR_SHAPE, "%s: K = %d must be a positive multiple of 128 up to %d", fn, K,
                    W4_MOE_GEMM_MAX_K);
    if (num_experts < 1) return fail(W4_ERR_ARG, "%s: num_experts = %d must be positive", fn, num_experts);
    if ((unsigned long long)N * (unsigned long long)(K / 2) > W4_GEMV_MAX_MATRIX_BYTES ||
        (unsigned long long)R * (unsigned long long)K * 2ull > W4_GEMV_MAX_MATRIX_BYTES)
        return fail(W4_ERR_SHAPE, "%s: N * K / 2 or R * K * 2 exceeds %llu bytes", fn, W4_GEMV_MAX_MATRIX_BYTES);
    if (!aligned(x, 16) || !aligned(qw_fp4, 16))
        return fail(W4_ERR_ALIGN, "%s: x and qw_fp4 must be 16-byte aligned", fn);
    if (!aligned(s_fp4, 8) || !aligned(y, 2) || !aligned(row_start, 4) || !aligned(expert_ids, 4))
        return fail(W4_ERR_ALIGN, "%s: s_fp4 must be 8-byte, y 2-byte, row_start and expert_ids 4-byte aligned", fn);
    const Range ry = range(y, (size_t)R * N * 2);
    const Range ins[5] = {range(x, (size_t)R * K * 2), range(qw_fp4, (size_t)num_experts * N * K / 2),
                          range(s_fp4, (size_t)num_experts * N * (K / 32) * 2), range(expert_ids, (size_t)E * 4),
                          range(row_start, (size_t)(E + 1) * 4)};
    for (const Range& r : ins)
        if (overlap(ry, r)) return fail(W4_ERR_ALIAS, "%s: y overlaps an input", fn);
    if (R == 0 || E == 0 || max_rows == 0 || N == 0) return W4_OK;
    hipError_t err = w4::launch_moe_gemm_fp4(x, row_start, expert_ids, qw_fp4, s_fp4, y, R, E, max_rows, num_experts,
                                             K, N, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? W4_OK : hip_fail(err, fn);
}

W4_API w4_status w4_moe_gemm2(const w4_moe_gemm_fc* fc1, const w4_moe_gemm_fc* fc2, const int32_t* row_start,
                              const int32_t* expert_ids, int R, int E, int max_rows, int num_experts,
                              void* stream) {
    const char* fn = "w4_moe_gemm2";
    if (!fc1 || !fc2 || !row_start || !expert_ids)
        return fail(W4_ERR_NULL, "%s: fc1, fc2, row_start and expert_ids must not be NULL", fn);
    if (R < 0 || E < 0 || max_rows < 0)
        return fail(W4_ERR_SHAPE, "%s: R = %d, E = %d, max_rows = %d must not be negative", fn, R, E, max_rows);
    if (num_experts < 1) return fail(W4_ERR_ARG, "%s: num_experts = %d must be positive", fn, num_experts);
    if (!aligned(row_start, 4) || !aligned(expert_ids, 4))
        return fail(W4_ERR_ALIGN, "%s: row_start and expert_ids must be 4-byte aligned", fn);
    const w4_moe_gemm_fc* fcs[2] = {fc1, fc2};
    Range ys[2], ins[2][3];
    for (int i = 0; i < 2; ++i) {
        const w4_moe_gemm_fc& f = *fcs[i];
        if (!f.x || !f.qw_fp4 || !f.s_fp4 || !f.y)
            return fail(W4_ERR_NULL, "%s: fc%d: x, qw_fp4, s_fp4 and y must not be NULL", fn, i + 1);
        if (f.N < 0) return fail(W4_ERR_SHAPE, "%s: fc%d: N = %d is negative", fn, i + 1, f.N);
        if (f.K <= 0 || f.K % 128 != 0 || f.K > W4_MOE_GEMM_MAX_K)
            return fail(W4_ERR_SHAPE, "%s: fc%d: K = %d must be a positive multiple of 128 up to %d", fn, i + 1, f.K,
                        W4_MOE_GEMM_MAX_K);
        if ((unsigned long long)f.N * (unsigned long long)(f.K / 2) > W4_GEMV_MAX_MATRIX_BYTES ||
            (unsigned long long)R * (unsigned long long)f.K * 2ull > W4_GEMV_MAX_MATRIX_BYTES)
            return fail(W4_ERR_SHAPE, "%s: fc%d: N * K / 2 or R * K * 2 exceeds %llu bytes", fn, i + 1,
                        W4_GEMV_MAX_MATRIX_BYTES);
        if (!aligned(f.x, 16) || !aligned(f.qw_fp4, 16))
            return fail(W4_ERR_ALIGN, "%s: fc%d: x and qw_fp4 must be 16-byte aligned", fn, i + 1);
        if (!aligned(f.s_fp4, 8) || !aligned(f.y, 2))
            return fail(W4_ERR_ALIGN, "%s: fc%d: s_fp4 must be 8-byte and y 2-byte aligned", fn, i + 1);
        ys[i] = range(f.y, (size_t)R * f.N * 2);
        ins[i][0] = range(f.x, (size_t)R * f.K * 2);
        ins[i][1] = range(f.qw_fp4, (size_t)num_experts * f.N * f.K / 2);
        ins[i][2] = range(f.s_fp4, (size_t)num_experts * f.N * (f.K / 32) * 2);
    }
    const Range shared[2] = {range(expert_ids, (size_t)E * 4), range(row_start, (size_t)(E + 1) * 4)};
    for (int i = 0; i < 2; ++i) {
        for (const Range& r : shared)
            if (overlap(ys[i], r)) return fail(W4_ERR_ALIAS, "%s: fc%d's y overlaps row_start or expert_ids", fn, i + 1);
        for (int j = 0; j < 2; ++j)
            for (const Range& r : ins[j])
                if (overlap(ys[i], r))
                    return fail(W4_ERR_ALIAS, "%s: fc%d's y overlaps an input of fc%d (the two FCs run together)",
                                fn, i + 1, j + 1);
    }
    if (overlap(ys[0], ys[1])) return fail(W4_ERR_ALIAS, "%s: the two outputs overlap", fn);
    if (R == 0 || E == 0 || max_rows == 0) return W4_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (fc1->N == 0 || fc2->N == 0) {  // one FC only
        const w4_moe_gemm_fc& f = fc1->N == 0 ? *fc2 : *fc1;
        if (f.N == 0) return W4_OK;
        hipError_t err = w4::launch_moe_gemm_fp4(f.x, row_start, expert_ids, f.qw_fp4, f.s_fp4, f.y, R, E, max_rows,
                                                 num_experts, f.K, f.N, st);
        return err == hipSuccess ? W4_OK : hip_fail(err, fn);
    }
    const w4::MoeGemmFcArgs a{fc1->x, fc1->qw_fp4, fc1->s_fp4, fc1->y, fc1->K, fc1->N};
    const w4::MoeGemmFcArgs b{fc2->x, fc2->qw_fp4, fc2->s_fp4, fc2->y, fc2->K, fc2->N};
    hipError_t err = w4::launch_moe_gemm2_fp4(a, b, row_start, expert_ids, R, E, max_rows, num_experts, st);
    return err == hipSuccess ? W4_OK : hip_fail(err, fn);
}

struct w4_graph {
    hipGraph_t graph;
    hipGraphExec_t exec;
};

W4_API w4_status w4_graph_begin(void* stream) {
    if (!stream) return fail(W4_ERR_ARG, "w4_graph_begin: capture needs a non-NULL stream");
    hipError_t err = hipStreamBeginCapture(static_cast<hipStream_t>(stream), hipStreamCaptureModeThreadLocal);
    return err == hipSuccess ? W4_OK : hip_fail(err, "w4_graph_begin");
}

W4_API w4_status w4_graph_end(void* stream, w4_graph_t* graph) {
    if (!graph) return fail(W4_ERR_ARG, "w4_graph_end: graph must not be NULL");
    *graph = nullptr;
    if (!stream) return fail(W4_ERR_ARG, "w4_graph_end: capture needs a non-NULL stream");
    hipGraph_t g = nullptr;
    hipError_t err = hipStreamEndCapture(static_cast<hipStream_t>(stream), &g);
    if (err != hipSuccess) return hip_fail(err, "w4_graph_end (end capture)");
    hipGraphExec_t exec = nullptr;
    err = hipGraphInstantiate(&exec, g, nullptr, nullptr, 0);
    if (err != hipSuccess) {
        (void)hipGraphDestroy(g);
        return hip_fail(err, "w4_graph_end (instantiate)");
    }
    *graph = new w4_graph{g, exec};
    return W4_OK;
}

W4_API w4_status w4_graph_replay(w4_graph_t graph, void* stream) {
    if (!graph) return fail(W4_ERR_ARG, "w4_graph_replay: graph must not be NULL");
    hipError_t err = hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? W4_OK : hip_fail(err, "w4_graph_replay");
}

W4_API void w4_graph_destroy(w4_graph_t graph) {
    if (!graph) return;
    (void)hipGraphExecDestroy(graph->exec);
    (void)hipGraphDestroy(graph->graph);
    delete graph;
}

// ------------------------------------------------------------ decode chains
struct w4_chain {
    w4::ChainLaunch launch;
};

namespace {

// Host analysis of a chain: validation, stages, producers and the
// output copies (mirrors) the workspace must hold.
struct ChainPlan {
    int num_stages = 0;
    std::vector<int> producer;      // GEMV whose output is this GEMV's x, or -1
    std::vector<long> mirror_word;  // offset in values of this GEMV's copy within each half, or -1 (no reader)
    size_t mirror_words = 0;
};

w4_status plan_chain(const char* fn, const w4_gemv_desc* descs, int count, ChainPlan& plan) {
    if (!descs) return fail(W4_ERR_NULL, "%s: descs must not be NULL", fn);
    if (count <= 0) return fail(W4_ERR_ARG, "%s: count = %d must be positive", fn, count);
    std::vector<Range> writes(count), reads(count), weights;
    for (int i = 0; i < count; ++i) {
        const w4_gemv_desc& d = descs[i];
        if (!d.x || !d.y) return fail(W4_ERR_NULL, "%s: descriptor %d: x and y must not be NULL", fn, i);
        w4_status st = check_int4(fn, d.qw, d.s, d.z, d.K, d.N, W4_INT4_GROUP, W4_CHAIN_MAX_K);
        if (st != W4_OK) return st;
        if ((unsigned long long)d.N * (unsigned long long)(d.K / 2) > W4_GEMV_MAX_MATRIX_BYTES)
            return fail(W4_ERR_SHAPE, "%s: descriptor %d: N * K / 2 exceeds %llu bytes", fn, i, W4_GEMV_MAX_MATRIX_BYTES);
        if (!aligned(d.x, 16) || !aligned(d.y, 2)) return fail(W4_ERR_ALIGN, "%s: descriptor %d: x or y misaligned", fn, i);
        if (d.reserved != 0) return fail(W4_ERR_ARG, "%s: descriptor %d: reserved must be 0", fn, i);
        if (d.stage < 0 || (i > 0 && d.stage < descs[i - 1].stage))
            return fail(W4_ERR_ARG, "%s: descriptor %d: stages must be non-negative and non-decreasing", fn, i);
        if (i == 0 || d.stage != descs[i - 1].stage) ++plan.num_stages;
        const size_t sz = (size_t)d.N * (d.K / W4_INT4_GROUP) * 2;
        writes[i] = range(d.y, (size_t)d.N * 2);
        reads[i] = range(d.x, (size_t)d.K * 2);
        weights.push_back(range(d.qw, (size_t)d.N * d.K / 2));
        weights.push_back(range(d.s, sz));
        weights.push_back(range(d.z, sz));
    }
    if (plan.num_stages >= 65535) return fail(W4_ERR_ARG, "%s: %d stages (at most 65534)", fn, plan.num_stages);
    plan.producer.assign(count, -1);
    plan.mirror_word.assign(count, -1);
    for (int i = 0; i < count; ++i) {
        for (const Range& w : weights)
            if (overlap(writes[i], w)) return fail(W4_ERR_ALIAS, "%s: output %d overlaps a weight, scale or zero", fn, i);
        for (int j = 0; j < count; ++j) {
            if (j != i && overlap(writes[i], writes[j])) return fail(W4_ERR_ALIAS, "%s: outputs %d and %d overlap", fn, i, j);
            if (descs[j].stage == descs[i].stage && overlap(writes[i], reads[j]))
                return fail(W4_ERR_ALIAS, "%s: output %d overlaps input %d of the same stage", fn, i, j);
        }
        // An input written by an earlier GEMV must be exactly its output.
        for (int j = 0; j < i; ++j) {
            if (descs[j].stage == descs[i].stage || !overlap(writes[j], reads[i])) continue;
            if (descs[i].x != descs[j].y || descs[i].K != descs[j].N)
                return fail(W4_ERR_UNSUPPORTED, "%s: input %d overlaps output %d without being exactly that output",
                            fn, i, j);
            plan.producer[i] = j;
        }
    }
    // An output that overwrites an earlier GEMV's input must wait for that
    // GEMV's output, through its chain of producers (a GEMV starts only once
    // its producer's output is complete, and that output is computed after
    // every workgroup has read the producer's input).
    for (int j = 0; j < count; ++j)
        for (int i = 0; i < count; ++i) {
            if (descs[i].stage >= descs[j].stage || !overlap(writes[j], reads[i])) continue;
            int p = plan.producer[j];
            while (p >= 0 && p != i) p = plan.producer[p];
            if (p != i)
                return fail(W4_ERR_UNSUPPORTED,
                            "%s: output %d overwrites input %d of an earlier stage without depending on its output",
                            fn, j, i);
        }
    for (int i = 0; i < count; ++i) {
        const int j = plan.producer[i];
        if (j >= 0 && plan.mirror_word[j] < 0) {
            plan.mirror_word[j] = (long)plan.mirror_words;
            plan.mirror_words += ((size_t)descs[j].N + 63) / 64 * 64;
        }
    }
    if (plan.mirror_words > ((size_t)1 << 29))
        return fail(W4_ERR_SHAPE, "%s: the outputs later GEMVs read total %zu values (limit 2^29)", fn,
                    plan.mirror_words);
    return W4_OK;
}

}  // namespace

W4_API size_t w4_chain_workspace_bytes(const w4_gemv_desc* descs, int count) {
    ChainPlan plan;
    if (plan_chain("w4_chain_workspace_bytes", descs, count, plan) != W4_OK) return 0;
    return w4::chain_layout(count, plan.num_stages, plan.mirror_words).total;
}

W4_API w4_status w4_chain_create(const w4_gemv_desc* descs, int count, void* workspace, size_t workspace_bytes,
                                 w4_chain_t* chain) {
    const char* fn = "w4_chain_create";
    if (!chain) return fail(W4_ERR_ARG, "%s: chain must not be NULL", fn);
    *chain = nullptr;
    if (!descs || !workspace) return fail(W4_ERR_NULL, "%s: descs and workspace must not be NULL", fn);
    if (!aligned(workspace, 256)) return fail(W4_ERR_ALIGN, "%s: workspace must be 256-byte aligned", fn);
    ChainPlan plan;
    w4_status pst = plan_chain(fn, descs, count, plan);
    if (pst != W4_OK) return pst;
    const int num_stages = plan.num_stages;
    const w4::ChainLayout lay = w4::chain_layout(count, num_stages, plan.mirror_words);
    if (workspace_bytes < lay.total)
        return fail(W4_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, lay.total, workspace_bytes);
    for (int i = 0; i < count; ++i) {
        const w4_gemv_desc& d = descs[i];
        const Range ws = range(workspace, lay.total);
        if (overlap(ws, range(d.y, (size_t)d.N * 2)) || overlap(ws, range(d.x, (size_t)d.K * 2)) ||
            overlap(ws, range(d.qw, (size_t)d.N * d.K / 2)) ||
            overlap(ws, range(d.s, (size_t)d.N * (d.K / W4_INT4_GROUP) * 2)) ||
            overlap(ws, range(d.z, (size_t)d.N * (d.K / W4_INT4_GROUP) * 2)))
            return fail(W4_ERR_ALIAS, "%s: workspace overlaps an operand of descriptor %d", fn, i);
    }

    // Tables.
    std::vector<w4::ChainStage> stages;
    std::vector<w4::ChainGemv> gemvs(count);
    int x_bytes = 0;
    for (int i = 0; i < count; ++i) {
        const w4_gemv_desc& d = descs[i];
        if (i == 0 || d.stage != descs[i - 1].stage) {
            stages.push_back({i, 0, 0, 0, -1});
            x_bytes = 0;
        }
        w4::ChainStage& st = stages.back();
        w4::ChainGemv& g = gemvs[i];
        g.qw = d.qw;
        g.s = d.s;
        g.z = d.z;
        g.x = d.x;
        g.y = d.y;
        g.C = d.K / 32;
        g.N = d.N;
        g.sp = g.C <= 128 ? 1 : (g.C <= 256 ? 2 : 4);
        g.tile0 = st.tiles;
        g.x_internal = plan.producer[i] >= 0;
        st.x_internal |= g.x_internal;
        // GEMVs of a stage with the same input share one staged copy.
        int same = -1;
        for (int j = st.gemv0; j < i && same < 0; ++j)
            if (descs[j].x == d.x && descs[j].K == d.K) same = j;
        if (same >= 0) {
            g.x_lds = gemvs[same].x_lds;
            g.x_slots = 0;
        } else {
            g.x_lds = x_bytes;
            g.x_slots = w4::chain_x_chunks(g.C) / 64;
            x_bytes += w4::chain_x_lds_bytes(g.C);
        }
        if (x_bytes > w4::kChainXLdsBytes)
            return fail(W4_ERR_SHAPE, "%s: the inputs of stage %d need %d bytes of LDS (limit %d)",
                        fn, d.stage, x_bytes, w4::kChainXLdsBytes);
        const int rows_per_tile = w4::kChainTileRows / g.sp;
        st.tiles += (d.N + rows_per_tile - 1) / rows_per_tile;
        st.ngemv += 1;
    }
    char* base = static_cast<char*>(workspace);
    uint16_t* mirrors = reinterpret_cast<uint16_t*>(base + lay.mirrors);
    for (int i = 0; i < count; ++i) {
        gemvs[i].ym = plan.mirror_word[i] >= 0 ? mirrors + plan.mirror_word[i] : nullptr;
        gemvs[i].xm = plan.producer[i] >= 0 ? mirrors + plan.mirror_word[plan.producer[i]] : nullptr;
        gemvs[i].xm_stage = 0;
    }
    for (int t = 0; t < num_stages; ++t)
        for (int k = 0; k < stages[t].ngemv; ++k) {
            const int i = stages[t].gemv0 + k;
            if (plan.producer[i] < 0) continue;
            const int j = plan.producer[i];
            for (int u = 0; u < num_stages; ++u)
                if (j >= stages[u].gemv0 && j < stages[u].gemv0 + stages[u].ngemv) gemvs[i].xm_stage = u;
            if (gemvs[i].xm_stage > stages[t].x_after) stages[t].x_after = gemvs[i].xm_stage;
        }
    int occ = 0, cus = 0, dev = 0;
    hipError_t err = w4::chain_occupancy(&occ);
    if (err == hipSuccess) err = hipGetDevice(&dev);
    if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return hip_fail(err, "w4_chain_create (device query)");
    if (occ < 1) return fail(W4_ERR_HIP, "%s: the chain kernel cannot be resident (occupancy %d)", fn, occ);
    int workers = cus;  // one workgroup per compute unit, all resident at once
    if (workers > w4::kChainMaxWorkers) workers = w4::kChainMaxWorkers;

    // Zero the counters; both halves of the output copies start empty.
    err = hipMemset(base, 0, lay.stages);
    if (err == hipSuccess && plan.mirror_words) err = hipMemset(base + lay.mirrors, 0xFF, plan.mirror_words * 4);
    if (err == hipSuccess)
        err = hipMemcpy(base + lay.stages, stages.data(), stages.size() * sizeof(w4::ChainStage), hipMemcpyHostToDevice);
    if (err == hipSuccess)
        err = hipMemcpy(base + lay.gemvs, gemvs.data(), gemvs.size() * sizeof(w4::ChainGemv), hipMemcpyHostToDevice);
    if (err == hipSuccess) err = hipDeviceSynchronize();
    if (err != hipSuccess) return hip_fail(err, "w4_chain_create (upload)");

    w4::ChainLaunch L;
    L.stages = reinterpret_cast<const w4::ChainStage*>(base + lay.stages);
    L.gemvs = reinterpret_cast<const w4::ChainGemv*>(base + lay.gemvs);
    L.err = reinterpret_cast<unsigned*>(base + lay.err);
    L.counters = reinterpret_cast<unsigned*>(base + lay.counters);
    L.num_stages = num_stages;
    L.workers = workers;
    L.spin_limit = 1u << 20;
    L.mirrors = mirrors;
    L.mirror_half_bytes = (uint32_t)(plan.mirror_words * 2);
    *chain = new w4_chain{L};
    return W4_OK;
}

W4_API w4_status w4_chain_run(w4_chain_t chain, void* stream) {
    if (!chain) return fail(W4_ERR_ARG, "w4_chain_run: chain must not be NULL");
    hipError_t err = w4::launch_chain(chain->launch, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? W4_OK : hip_fail(err, "w4_chain_run");
}

W4_API w4_status w4_chain_set_spin_limit(w4_chain_t chain, uint32_t spin_limit) {
    if (!chain) return fail(W4_ERR_ARG, "w4_chain_set_spin_limit: chain must not be NULL");
    chain->launch.spin_limit = spin_limit;
    return W4_OK;
}

W4_API w4_status w4_chain_error(w4_chain_t chain, uint32_t* error_word) {
    if (!chain || !error_word) return fail(W4_ERR_ARG, "w4_chain_error: chain and error_word must not be NULL");
    hipError_t err = hipDeviceSynchronize();
    if (err == hipSuccess) err = hipMemcpy(error_word, chain->launch.err, sizeof(uint32_t), hipMemcpyDeviceToHost);
    return err == hipSuccess ? W4_OK : hip_fail(err, "w4_chain_error");
}

W4_API void w4_chain_destroy(w4_chain_t chain) { delete chain; }

W4_API w4_status w4_read_probe(const void* src, size_t bytes, uint32_t* sink, void* stream) {
    const char* fn = "w4_read_probe";
    if (!sink || (!src && bytes)) return fail(W4_ERR_NULL, "%s: sink (and src when bytes > 0) must not be NULL", fn);
    if (bytes % 16 != 0) return fail(W4_ERR_SHAPE, "%s: bytes = %zu is not a multiple of 16", fn, bytes);
    if ((src && !aligned(src, 16)) || !aligned(sink, 4)) return fail(W4_ERR_ALIGN, "%s: src (16) or sink (4) misaligned", fn);
    if (overlap(range(sink, (size_t)W4_READ_PROBE_SINK * 4), range(src, bytes)))
        return fail(W4_ERR_ALIAS, "%s: sink overlaps the source", fn);
    hipError_t err = w4::launch_read_probe(src, bytes, sink, W4_READ_PROBE_SINK, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? W4_OK : hip_fail(err, fn);
}

W4_API w4_status w4_dequant_int4(const int32_t* qw, const void* s, const void* z, float* out_f32,
                                 void* out_bf16, int K, int N, int g, void* stream) {
    const char* fn = "w4_dequant_int4";
    if (!out_f32 && !out_bf16) return fail(W4_ERR_NULL, "%s: out_f32 and out_bf16 are both NULL", fn);
    w4_status st = check_int4(fn, qw, s, z, K, N, g, 0);
    if (st != W4_OK) return st;
    if ((out_f32 && !aligned(out_f32, 4)) || (out_bf16 && !aligned(out_bf16, 2)))
        return fail(W4_ERR_ALIGN, "%s: outputs misaligned", fn);
    const size_t sz_bytes = (size_t)N * (K / g) * 2;
    const Range ins[3] = {range(qw, (size_t)N * K / 2), range(s, sz_bytes), range(z, sz_bytes)};
    const Range outs[2] = {range(out_f32, out_f32 ? (size_t)N * K * 4 : 0),
                           range(out_bf16, out_bf16 ? (size_t)N * K * 2 : 0)};
    for (const Range& o : outs)
        for (const Range& r : ins)
            if (overlap(o, r)) return fail(W4_ERR_ALIAS, "%s: an output overlaps an input", fn);
    if (overlap(outs[0], outs[1])) return fail(W4_ERR_ALIAS, "%s: the two outputs overlap", fn);
    if (N == 0) return W4_OK;
    hipError_t err = w4::launch_dequant_int4(qw, s, z, out_f32, out_bf16, K, N, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? W4_OK : hip_fail(err, fn);
}

W4_API w4_status w4_int4_gemv_operands(const int32_t* qw, const void* x, uint32_t* codes_out, uint32_t* x_out,
                                       int K, int N, void* stream) {
    const char* fn = "w4_int4_gemv_operands";
    if (!qw || !codes_out) return fail(W4_ERR_NULL, "%s: qw and codes_out must not be NULL", fn);
    if (!x != !x_out) return fail(W4_ERR_NULL, "%s: x and x_out must both be given or both be NULL", fn);
    if (N < 0) return fail(W4_ERR_SHAPE, "%s: N = %d is negative", fn, N);
    if (K <= 0 || K % 8 != 0) return fail(W4_ERR_SHAPE, "%s: K = %d is not a positive multiple of 8", fn, K);
    if (!aligned(qw, 4) || !aligned(codes_out, 4) || (x && !aligned(x, 4)) || (x_out && !aligned(x_out, 4)))
        return fail(W4_ERR_ALIGN, "%s: qw, x and the outputs must be 4-byte aligned", fn);
    const Range ins[2] = {range(qw, (size_t)N * K / 2), range(x, x ? (size_t)K * 2 : 0)};
    const Range outs[2] = {range(codes_out, (size_t)N * K * 2), range(x_out, x_out ? (size_t)K * 2 : 0)};
    for (const Range& o : outs)
        for (const Range& r : ins)
            if (overlap(o, r)) return fail(W4_ERR_ALIAS, "%s: an output overlaps an input", fn);
    if (overlap(outs[0], outs[1])) return fail(W4_ERR_ALIAS, "%s: the two outputs overlap", fn);
    if (N == 0) return W4_OK;
    hipError_t err = w4::launch_int4_gemv_operands(qw, x, codes_out, x_out, K, N, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? W4_OK : hip_fail(err, fn);
}

W4_API w4_status w4_dequant_fp4(const uint8_t* qw_fp4, const void* s_fp4, float* out_f32, void* out_bf16,
                                int K, int N, void* stream) {
    const char* fn = "w4_dequant_fp4";
    if (!qw_fp4 || !s_fp4) return fail(W4_ERR_NULL, "%s: qw_fp4 and s_fp4 must not be NULL", fn);
    if (!out_f32 && !out_bf16) return fail(W4_ERR_NULL, "%s: out_f32 and out_bf16 are both NULL", fn);
    if (N < 0) return fail(W4_ERR_SHAPE, "%s: N = %d is negative", fn, N);
    if (K <= 0 || K % W4_FP4_GROUP != 0) return fail(W4_ERR_SHAPE, "%s: K = %d is not a positive multiple of 32", fn, K);
    if (!aligned(qw_fp4, 16) || !aligned(s_fp4, 2)) return fail(W4_ERR_ALIGN, "%s: qw_fp4 (16) or s_fp4 (2) misaligned", fn);
    if ((out_f32 && !aligned(out_f32, 4)) || (out_bf16 && !aligned(out_bf16, 2)))
        return fail(W4_ERR_ALIGN, "%s: outputs misaligned", fn);
    const Range ins[2] = {range(qw_fp4, (size_t)N * K / 2), range(s_fp4, (size_t)N * (K / 32) * 2)};
    const Range outs[2] = {range(out_f32, out_f32 ? (size_t)N * K * 4 : 0),
                           range(out_bf16, out_bf16 ? (size_t)N * K * 2 : 0)};
    for (const Range& o : outs)
        for (const Range& r : ins)
            if (overlap(o, r)) return fail(W4_ERR_ALIAS, "%s: an output overlaps an input", fn);
    if (overlap(outs[0], outs[1])) return fail(W4_ERR_ALIAS, "%s: the two outputs overlap", fn);
    if (N == 0) return W4_OK;
    hipError_t err = w4::launch_dequant_fp4(qw_fp4, s_fp4, out_f32, out_bf16, K, N, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? W4_OK : hip_fail(err, fn);
}

}  // extern "C"
