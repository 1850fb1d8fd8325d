// C ABI of the fused 4-bit-weight GEMV/GEMM library: host-side validation,
// dispatch to the launchers, HIP-graph capture helpers and error reporting.
// Every check here runs before the first HIP call of an entry point, so an
// invalid call launches nothing and can be tested on a host without a GPU.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

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
    w4_status st = check_int4(fn, qw, s, z, K, N, g, 0);
    if (st != W4_OK) return st;
    if (M < 0) return fail(W4_ERR_SHAPE, "%s: M = %d is negative", fn, M);
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
