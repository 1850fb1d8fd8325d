/*
 * w4.h -- C ABI of the fused 4-bit-weight x BF16 GEMV / GEMM library (MI355X, gfx950).
 *
 * The operation.  A linear layer y = x * W^T (``F.linear`` semantics, no bias)
 * whose weight W[N][K] is stored packed in 4 bits and is never expanded to
 * BF16 in device memory:
 *
 *   INT4 (GPTQ-style, asymmetric): W[n][k] = (q[n][k] - z[n][k/128]) * s[n][k/128]
 *     -- "Lab 5: Gemma4 端到端推理优化", sections "量化正确性" (GPTQ INT4,
 *        group 128, asymmetric), "最终配置" (FP16 scale) and "INT4 融合 GEMV"
 *        (fused GEMV: packed INT4 read once, unpacked in registers, per-group
 *        scale/zero applied, dot with the BF16 input; M = 1 decode and an
 *        M = 128 prefill path).
 *   FP4 (E2M1):  W[n][k] = e2m1(c[n][k]) * s[n][k/32]
 *     -- "DeepSeek V4 Triton FP4 优化实战", section "深度分析" item 2 (even k
 *        in the low nibble, odd k in the high nibble) and item 4 (6 active
 *        experts x 2 FC per layer, each at M = 1).
 *
 * Arithmetic: products and sums in FP32; the output is rounded once to BF16,
 * round-to-nearest-even.  Summation order is unspecified but fixed: the same
 * call on the same inputs returns the same bits (no floating-point atomics).
 *
 * Layouts (all row-major, contiguous, little-endian):
 *   x       bf16   [M][K]                activations (M = 1 for the GEMVs)
 *   qw      int32  [N][K/8]              INT4 codes; bits 4j..4j+3 of word p hold k = 8p + j
 *   s, z    fp16   [N][K/128]            INT4 scale and zero point (zero integer-valued, 0..15)
 *   qw_fp4  uint8  [experts][N][K/2]     E2M1 codes; low nibble = even k, high nibble = odd k
 *   s_fp4   bf16   [experts][N][K/32]    FP4 scale (a full BF16 multiplier)
 *   y       bf16   [M][N]                output
 * BF16 and FP16 buffers are passed as pointers to their 16-bit patterns.
 *
 * Conventions shared by every entry point:
 *   - Pointers named as device pointers must point to device memory of the
 *     current HIP device.  The caller owns every buffer, including the GEMM
 *     workspace; the library never allocates, frees or reads device memory
 *     on the host and never synchronises, so every call can be captured into
 *     a HIP graph.
 *   - ``stream`` is a hipStream_t (NULL = the default stream).  Calls are
 *     asynchronous: a return of W4_OK means the work was enqueued.
 *   - Arguments are validated on the host before any HIP call.  On a
 *     validation error nothing is launched and an error status is returned;
 *     w4_last_error() then describes it.
 *   - M = 0 or N = 0 (or E = 0) is an empty problem: W4_OK, nothing launched.
 *   - Outputs must not overlap any input (checked from the address ranges).
 *   - Not checked (would need a device read): zero points integer-valued in
 *     0..15, and finite inputs within range: the INT4 GEMV-path kernels
 *     (w4_gemv, the decode chain, w4_gemm at M <= 16) sum (128 + q) * x over
 *     32 codes in FP32 before applying the zero point, which needs
 *     |x| < about 7e34 (any activation of a real model is far below).  Expert ids outside [0, num_experts) are
 *     checked on the device: that slot's outputs are set to NaN and no
 *     weight is read for it.
 */
#ifndef W4_H
#define W4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define W4_API __attribute__((visibility("default")))
#else
#define W4_API
#endif

typedef enum w4_status {
    W4_OK = 0,
    W4_ERR_NULL = 1,        /* a required pointer is NULL */
    W4_ERR_SHAPE = 2,       /* negative size; K not a positive multiple of the group; K above the limit */
    W4_ERR_UNSUPPORTED = 3, /* group size other than 128 (INT4) */
    W4_ERR_ALIGN = 4,       /* a pointer is not aligned as its entry point requires */
    W4_ERR_WORKSPACE = 5,   /* GEMM workspace NULL or smaller than w4_gemm_workspace_bytes() */
    W4_ERR_ALIAS = 6,       /* an output range overlaps an input range */
    W4_ERR_ARG = 7,         /* other invalid argument (stride, expert count, NULL graph or stream) */
    W4_ERR_HIP = 8          /* the HIP runtime reported an error (see w4_last_error()) */
} w4_status;

/* Largest K accepted by w4_gemv / w4_moe_gemv (registers hold the whole x row slice). */
#define W4_GEMV_MAX_K 32768
/* Largest packed weight matrix (N * K / 2 bytes, per expert for FP4) of one
 * w4_gemv / w4_moe_gemv call: the kernels address it with 32-bit offsets. */
#define W4_GEMV_MAX_MATRIX_BYTES 4294967295ull
/* Largest K accepted by w4_gemm (a workgroup stages the scales and zeros of
 * its 64 weight rows, all K / 128 groups, in LDS).  The activations
 * (M * K * 2 bytes) and the packed weights (N * K / 2 bytes) of one call must
 * each stay within W4_GEMV_MAX_MATRIX_BYTES: 32-bit offsets address them. */
#define W4_GEMM_MAX_K 32768
/* Largest K accepted by w4_moe_gemm (a workgroup stages the scales of its
 * weight rows, all K / 32 groups, in LDS). */
#define W4_MOE_GEMM_MAX_K 8192
#define W4_INT4_GROUP 128
#define W4_FP4_GROUP 32

/* ABI version of this header (bumped on any incompatible change). */
W4_API int w4_abi_version(void);

/* Name of a status code (static string, never NULL). */
W4_API const char* w4_status_string(w4_status status);

/* Description of the most recent error returned on the calling thread (static per thread). */
W4_API const char* w4_last_error(void);

/*
 * w4_gemv -- decode GEMV, M = 1, INT4 weights.
 *   y[n] = bf16( sum_k (q[n][k] - z[n][k/g]) * s[n][k/g] * x[k] ),  n < N
 * "Lab 5: Gemma4 端到端推理优化", section "INT4 融合 GEMV": weights read once,
 * unpacked in registers, the input vector reused from registers or LDS.
 *   x   device bf16 [K], 16-byte aligned      qw  device int32 [N][K/8], 16-byte aligned
 *   s,z device fp16 [N][K/g], 2-byte aligned  y   device bf16 [N], 2-byte aligned
 *   K   multiple of g, 0 < K <= W4_GEMV_MAX_K;  N >= 0;  g must be 128;
 *       N * K / 2 <= W4_GEMV_MAX_MATRIX_BYTES.
 * Errors: W4_ERR_NULL, W4_ERR_SHAPE, W4_ERR_UNSUPPORTED, W4_ERR_ALIGN, W4_ERR_ALIAS, W4_ERR_HIP.
 */
W4_API w4_status w4_gemv(const void* x, const int32_t* qw, const void* s, const void* z,
                         void* y, int K, int N, int g, void* stream);

/*
 * w4_gemm -- prefill GEMM, any M >= 0 (built for M = 128), INT4 weights,
 * 0 < K <= W4_GEMM_MAX_K.
 *   y[m][n] = bf16( sum_k bf16((q[n][k] - z[n][k/g]) * s[n][k/g]) * x[m][k] )
 * "Lab 5: Gemma4 端到端推理优化", sections "Triton 反量化 + cuBLAS" (prefill:
 * dequantised BF16 weights into a tensor-core GEMM) and "INT4 融合 GEMV"
 * (equivalence tested at M = 128).  Here each packed word is dequantised in
 * registers straight into the matrix-core operand (BF16, round-to-nearest-
 * even) and the BF16 weight is never written to device memory.  M = 1 runs
 * w4_gemv's kernel (same result, bit for bit, as w4_gemv); M = 2 with
 * K <= 16384 a GEMV over both rows (weights unpacked once, exact codes).
 * Other M <= 16 (a few decode tokens at once) take a streaming path: one 16-row
 * matrix-core block of x against the exact codes, the group's zero and scale
 * applied to the FP32 block sums, weights read once and no workspace.
 *   x   device bf16 [M][K], 16-byte aligned   qw, s, z as for w4_gemv
 *   y   device bf16 [M][N], 2-byte aligned
 *   workspace  device memory of at least w4_gemm_workspace_bytes(M, K, N, g)
 *              bytes, 16-byte aligned (may be NULL when that size is 0).  It
 *              holds FP32 split-K partial sums; its contents on entry are
 *              ignored and on return are unspecified.  Calls that share one
 *              workspace must be ordered (same stream).
 * Errors: as w4_gemv, plus W4_ERR_WORKSPACE.
 */
W4_API size_t w4_gemm_workspace_bytes(int M, int K, int N, int g);
W4_API w4_status w4_gemm(const void* x, const int32_t* qw, const void* s, const void* z,
                         void* y, int M, int K, int N, int g,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * w4_gemm_noalloc -- w4_gemm for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): same operation, kernels, limits and result, bit for bit, but no
 * workspace argument.  The split-K partial sums go to a scratch array the
 * library holds on each GPU it runs on (W4_GEMM_NOALLOC_SCRATCH_BYTES, kept
 * until the process ends); the call itself allocates nothing.  Shapes whose
 * w4_gemm_workspace_bytes() exceeds that size are rejected (W4_ERR_WORKSPACE).
 * Every call on a GPU shares its scratch: calls that may overlap in time on
 * one GPU (different streams, or several threads) race and must be ordered
 * by the caller.  The scratch holds only values each call writes before it
 * reads them.  The first call on a device looks up the scratch's address.
 * Errors: as w4_gemm.
 */
#define W4_GEMM_NOALLOC_SCRATCH_BYTES (16ull << 20)
W4_API w4_status w4_gemm_noalloc(const void* x, const int32_t* qw, const void* s, const void* z,
                                 void* y, int M, int K, int N, int g, void* stream);

/*
 * w4_moe_gemv -- FP4 expert GEMVs, M = 1 per slot.
 *   y[e][n] = bf16( sum_k e2m1(c[ids[e]][n][k]) * s[ids[e]][n][k/32] * x_e[k] ),  e < E
 *   with x_e = x + e * x_stride (elements); x_stride = 0 shares one vector.
 * "DeepSeek V4 Triton FP4 优化实战", "深度分析" items 2 and 4.
 *   x          device bf16, 16-byte aligned; x_stride >= 0, a multiple of 8
 *   qw_fp4     device uint8 [num_experts][N][K/2], 16-byte aligned
 *   s_fp4      device bf16 [num_experts][N][K/32], 2-byte aligned
 *   expert_ids device int32 [E], 4-byte aligned (read on the device)
 *   y          device bf16 [E][N], 2-byte aligned
 *   K multiple of 32, 0 < K <= W4_GEMV_MAX_K;  E >= 0;  num_experts >= 1;
 *   N * K / 2 <= W4_GEMV_MAX_MATRIX_BYTES.
 * Errors: W4_ERR_NULL, W4_ERR_SHAPE, W4_ERR_ALIGN, W4_ERR_ALIAS, W4_ERR_ARG, W4_ERR_HIP.
 */
W4_API w4_status w4_moe_gemv(const void* x, int64_t x_stride, const uint8_t* qw_fp4,
                             const void* s_fp4, const int32_t* expert_ids, void* y,
                             int E, int num_experts, int K, int N, void* stream);

/*
 * w4_moe_gemv2 -- two FP4 expert FCs over the same E slots and expert ids in
 * one launch: the result of w4_moe_gemv(fc1) and w4_moe_gemv(fc2), bit for
 * bit, for two FCs whose inputs are both ready (neither reads the other's
 * output).  "DeepSeek V4 Triton FP4 优化实战", "深度分析" item 4: every token
 * runs 2 FC on each of its 6 active experts, all bandwidth-bound, so one
 * launch saves a launch's ramp and tail.
 *   w4_moe_fc   { x, x_stride, qw_fp4, s_fp4, y, K, N } -- each field as for
 *               w4_moe_gemv (fc1 and fc2 each have their own expert pool)
 *   expert_ids  device int32 [E], 4-byte aligned, for both FCs (read on the
 *               device; an id outside [0, num_experts) makes that slot's
 *               outputs of both FCs NaN)
 * Neither output may overlap any input of either FC, the ids or the other
 * output.  A FC with N = 0 is skipped.
 * Errors: as w4_moe_gemv.
 */
typedef struct w4_moe_fc {
    const void* x;        /* device bf16, slot e's vector at x + e * x_stride */
    int64_t x_stride;     /* elements; 0 shares one vector */
    const uint8_t* qw_fp4; /* device uint8 [num_experts][N][K/2] */
    const void* s_fp4;    /* device bf16 [num_experts][N][K/32] */
    void* y;              /* device bf16 [E][N] */
    int K;
    int N;
} w4_moe_fc;
W4_API w4_status w4_moe_gemv2(const w4_moe_fc* fc1, const w4_moe_fc* fc2, const int32_t* expert_ids,
                              int E, int num_experts, void* stream);

/*
 * w4_moe_gemm -- grouped FP4 expert GEMM: several tokens per expert (MoE
 * prefill, or a decode batch routed to experts).
 *   for each group e < E, rows r in [row_start[e], row_start[e+1]):
 *   y[r][n] = bf16( sum_k e2m1(c[ids[e]][n][k]) * s[ids[e]][n][k/32] * x[r][k] )
 * "DeepSeek V4 Triton FP4 优化实战", "深度分析" items 2 (the fused FP4 kernel
 * is a matrix product; even k in the low nibble, odd k in the high nibble)
 * and 4 (tokens routed to experts).  The FP4 codes are decoded in registers
 * straight into the matrix-core operand; each group of 32 k is summed
 * exactly in FP32 and scaled in FP32.
 *   x          device bf16 [R][K], 16-byte aligned
 *   row_start  device int32 [E+1], 4-byte aligned (read on the device):
 *              group e owns rows row_start[e] .. row_start[e+1] - 1;
 *              values are clamped into [0, R] and a group's end below its
 *              start counts as empty
 *   expert_ids device int32 [E], 4-byte aligned (read on the device); an id
 *              outside [0, num_experts) makes that group's rows NaN
 *   qw_fp4     device uint8 [num_experts][N][K/2], 16-byte aligned
 *   s_fp4      device bf16 [num_experts][N][K/32], 8-byte aligned
 *   y          device bf16 [R][N], 2-byte aligned; rows in no group are not
 *              written
 *   max_rows   the most rows any group has: rows of a group past its first
 *              max_rows are not written (precondition, not checked)
 *   K multiple of 128, 0 < K <= W4_MOE_GEMM_MAX_K;  R, E, max_rows, N >= 0;
 *   num_experts >= 1;  N * K / 2 and R * K * 2 <= W4_GEMV_MAX_MATRIX_BYTES.
 * Errors: W4_ERR_NULL, W4_ERR_SHAPE, W4_ERR_ALIGN, W4_ERR_ALIAS, W4_ERR_ARG, W4_ERR_HIP.
 */
W4_API w4_status w4_moe_gemm(const void* x, const int32_t* row_start, const int32_t* expert_ids,
                             const uint8_t* qw_fp4, const void* s_fp4, void* y, int R, int E,
                             int max_rows, int num_experts, int K, int N, void* stream);

/*
 * w4_moe_gemm2 -- two grouped FP4 expert GEMMs over the same groups (row
 * ranges and expert ids) in one launch: the result of w4_moe_gemm(fc1) and
 * w4_moe_gemm(fc2), bit for bit, for two FCs whose inputs are both ready
 * (neither reads the other's output, e.g. the gate and up projections of the
 * routed tokens).  "DeepSeek V4 Triton FP4 优化实战", "深度分析" items 2 and 4:
 * each routed token runs 2 FC on its experts; one launch saves a launch's
 * ramp and tail.
 *   w4_moe_gemm_fc { x, qw_fp4, s_fp4, y, K, N } -- each field as for
 *               w4_moe_gemm (fc1 and fc2 each have their own expert pool of
 *               num_experts experts, their own K and N, and x [R][K])
 *   row_start, expert_ids, R, E, max_rows, num_experts: as for w4_moe_gemm,
 *               shared by both FCs
 * Neither output may overlap any input of either FC, row_start, the ids or
 * the other output.  A FC with N = 0 is skipped.
 * Errors: as w4_moe_gemm.
 */
typedef struct w4_moe_gemm_fc {
    const void* x;         /* device bf16 [R][K], 16-byte aligned */
    const uint8_t* qw_fp4; /* device uint8 [num_experts][N][K/2], 16-byte aligned */
    const void* s_fp4;     /* device bf16 [num_experts][N][K/32], 8-byte aligned */
    void* y;               /* device bf16 [R][N], 2-byte aligned */
    int K;
    int N;
} w4_moe_gemm_fc;
W4_API w4_status w4_moe_gemm2(const w4_moe_gemm_fc* fc1, const w4_moe_gemm_fc* fc2, const int32_t* row_start,
                              const int32_t* expert_ids, int R, int E, int max_rows, int num_experts,
                              void* stream);

/*
 * w4_repack_gptq -- import a weight stored in GPTQ's own K-major layout
 * ("Lab 5: Gemma4 端到端推理优化", section "量化正确性": GPTQ INT4, group 128,
 * asymmetric), once, at load time, into the layout every other entry point
 * reads:
 *   qw_kn  device int32 [K/8][N]: word (p, n) holds the codes of k = 8p .. 8p+7
 *          of output n, nibble j (bits 4j .. 4j+3) for k = 8p + j
 *   s_gn, z_gn  device fp16 [K/g][N]
 * into qw int32 [N][K/8], s and z fp16 [N][K/g] (a transpose of words and of
 * 16-bit values; every code keeps its nibble position).  Inputs are not
 * modified; outputs must not overlap inputs or each other.  Packed words
 * 4-byte aligned, scales and zeros 2-byte aligned; K a positive multiple of
 * g = 128; N >= 0.  Asynchronous on ``stream``; capturable.
 * Errors: W4_ERR_NULL, W4_ERR_SHAPE, W4_ERR_UNSUPPORTED, W4_ERR_ALIGN, W4_ERR_ALIAS, W4_ERR_HIP.
 */
W4_API w4_status w4_repack_gptq(const int32_t* qw_kn, const void* s_gn, const void* z_gn, int32_t* qw,
                                void* s, void* z, int K, int N, int g, void* stream);

/*
 * Launch tuning.  Each kernel family has one launch parameter; its value for
 * a call comes from a table of choices measured on an MI355X for the
 * workloads' shapes ("Lab 5: Gemma4 端到端推理优化", section "GEMV 分块测试":
 * the GEMV block shape was chosen per workload by a sweep), else from the
 * launcher's rule.  Every value computes the same operation; summation order
 * (and so the last bits) may differ between values, never between runs.
 *   W4_TUNE_GEMV          w4_gemv, w4_gemm at M = 1: weight rows per wave, 1, 2, 4 or 8
 *   W4_TUNE_GEMV_ROWS2    w4_gemm at M = 2 (K <= 16384): weight rows per wave, 1, 2, 4 or 8
 *   W4_TUNE_GEMM_SMALL_M  w4_gemm at 3 <= M <= 16: weight rows per workgroup / 16, 1, 2 or 4
 *   W4_TUNE_GEMM          w4_gemm at M > 16: K splits, 1 .. 16 (at most K / 128); it sets
 *                         w4_gemm_workspace_bytes()
 *   W4_TUNE_MOE_GEMV      w4_moe_gemv: weight rows per wave, 1, 2, 4 or 8 (M = the slot count E)
 * w4_tune_param returns the parameter a call of shape (M, K, N) would launch
 * with, or -1 for an unknown kernel.  w4_tune_force makes every later call of
 * a kernel family launch with ``param`` (0 restores the table), for tuning
 * sweeps and tests; it is process-wide and must not race with calls.
 * Errors (w4_tune_force): W4_ERR_ARG (unknown kernel or parameter).
 */
#define W4_TUNE_GEMV 0
#define W4_TUNE_GEMV_ROWS2 1
#define W4_TUNE_GEMM_SMALL_M 2
#define W4_TUNE_GEMM 3
#define W4_TUNE_MOE_GEMV 4
#define W4_TUNE_KERNELS 5
W4_API int w4_tune_param(int kernel, int M, int K, int N);
W4_API w4_status w4_tune_force(int kernel, int param);

/*
 * Decode-step graphs.  "Lab 5: Gemma4 端到端推理优化", section "CUDA Graph":
 * the whole decode step is captured once and replayed once per token, which
 * needs static buffers.  w4_graph_begin starts capturing ``stream`` (which
 * must not be NULL); every library call made on that stream by this thread
 * until w4_graph_end is recorded instead of run; w4_graph_end ends the
 * capture and instantiates the graph.  w4_graph_replay enqueues one replay on
 * ``stream``.  The graph keeps the pointers it was captured with: those
 * buffers must stay allocated until w4_graph_destroy.  A failed w4_graph_end
 * leaves *graph NULL.
 * Errors: W4_ERR_ARG (NULL stream or graph), W4_ERR_HIP.
 */
typedef struct w4_graph* w4_graph_t;
W4_API w4_status w4_graph_begin(void* stream);
W4_API w4_status w4_graph_end(void* stream, w4_graph_t* graph);
W4_API w4_status w4_graph_replay(w4_graph_t graph, void* stream);
W4_API void w4_graph_destroy(w4_graph_t graph);

/*
 * Decode chains: a sequence of dependent INT4 GEMVs run by one persistent
 * launch.  "Lab 5: Gemma4 端到端推理优化", sections "CUDA Graph" and "性能分析":
 * after fusing the GEMV, the decode step's remaining cost is per-launch
 * overhead; "在 Triton 中利用 Cutlass 内核命名解锁 FP8 张量核心加速" (last
 * paragraph) names the remedy, a persistent kernel that fuses several GEMMs
 * into one launch.
 *
 * Each descriptor is one w4_gemv (same operands, layouts and limits,
 * N * K / 2 <= W4_GEMV_MAX_MATRIX_BYTES included, plus K <= W4_CHAIN_MAX_K)
 * tagged with a stage number.  Descriptors must be given
 * in non-decreasing stage order.  The result is that of running the stages
 * one after another, each stage's GEMVs in any order: a GEMV may read as x
 * the output y of a GEMV of an earlier stage, and then sees it complete.
 * Such an input must be exactly that output (same pointer, K equal to the
 * producer's N); a partial overlap is W4_ERR_UNSUPPORTED.  Inside the launch
 * a GEMV waits only for the output it reads (its readers poll a BF16 copy
 * of it kept in the workspace, in one of two halves that alternate between
 * runs), so GEMVs that do not depend on each other may overlap in time.  Hence an output may overwrite an earlier stage's
 * input only if its GEMV depends, through its chain of inputs, on that
 * earlier GEMV's output (W4_ERR_UNSUPPORTED otherwise).  An output must not
 * overlap any weight, scale or zero of the chain, any other output, or any
 * input of its own stage (W4_ERR_ALIAS).  The x vectors of one stage must
 * fit the kernel's LDS staging area: the sum over the stage's distinct
 * inputs (GEMVs with the same x share one copy) of 68 * P bytes, with
 * P = 128 for K <= 4096, 256 for K <= 8192 and 512 above, at most 65536
 * (W4_ERR_SHAPE from w4_chain_create otherwise).  The outputs that later
 * GEMVs read may total at most 2^29 values (W4_ERR_SHAPE).
 * At most 65534 stages.
 *
 * w4_chain_workspace_bytes(descs, count) validates the descriptors and
 * returns the workspace size they need (0 if they are invalid; the reason
 * is in w4_last_error).  w4_chain_create validates the descriptors on the
 * host, then (blocking, not capturable) clears the workspace's counters,
 * marks the output copies empty and writes the chain's tables into it; it
 * never allocates
 * device memory.  The workspace (device memory, 256-byte aligned, at least
 * w4_chain_workspace_bytes(descs, count) bytes) belongs to the chain until
 * w4_chain_destroy.  w4_chain_run enqueues one run on ``stream`` (one kernel
 * launch; capturable into a graph).  Runs of one chain must not overlap each
 * other or any other kernel that fills the GPU: the launch keeps one
 * workgroup resident on every compute unit and they wait for each other.
 * Every wait is bounded: a run that cannot make progress ends within about a
 * second and records a non-zero error word; w4_chain_error synchronises the
 * device and returns that word (0 = no error).  After a non-zero error word,
 * create the chain again before running it.
 * Errors: W4_ERR_NULL, W4_ERR_SHAPE, W4_ERR_UNSUPPORTED, W4_ERR_ALIGN,
 * W4_ERR_ALIAS, W4_ERR_ARG (no descriptors, stage order, too many stages),
 * W4_ERR_WORKSPACE, W4_ERR_HIP.
 * (A separate build with -DW4_CHAIN_TIMELINE, made by
 * gemm_w4_gemv_amd/chain_timeline.py for profiling, also exports
 * w4_chain_timeline_read; the product library does not.)
 */
#define W4_CHAIN_MAX_K 16384

typedef struct w4_gemv_desc {
    const void* x;     /* device bf16 [K], 16-byte aligned */
    const int32_t* qw; /* device int32 [N][K/8], 16-byte aligned */
    const void* s;     /* device fp16 [N][K/128] */
    const void* z;     /* device fp16 [N][K/128] */
    void* y;           /* device bf16 [N] */
    int K;
    int N;
    int stage;
    int reserved;      /* must be 0 */
} w4_gemv_desc;

typedef struct w4_chain* w4_chain_t;
W4_API size_t w4_chain_workspace_bytes(const w4_gemv_desc* descs, int count);
W4_API w4_status w4_chain_create(const w4_gemv_desc* descs, int count, void* workspace,
                                 size_t workspace_bytes, w4_chain_t* chain);
W4_API w4_status w4_chain_run(w4_chain_t chain, void* stream);
W4_API w4_status w4_chain_error(w4_chain_t chain, uint32_t* error_word);
W4_API void w4_chain_destroy(w4_chain_t chain);
/*
 * For tests of failure handling: bound every wait of the chain's later runs
 * to ``spin_limit`` polls (default 1 << 20, about a second).  With 0 a run
 * gives up at the first wait that is not already satisfied: it records a
 * non-zero error word, leaves the outputs undefined and still ends normally.
 * Errors: W4_ERR_ARG (chain is NULL).
 */
W4_API w4_status w4_chain_set_spin_limit(w4_chain_t chain, uint32_t spin_limit);

/*
 * Measurement only: read ``bytes`` of device memory at ``src`` once with
 * streaming 16-byte loads, as fast as the GPU allows, and write one XOR
 * digest word per workgroup to ``sink`` (device uint32, W4_READ_PROBE_SINK
 * words, not read by the host).  The achieved rate is the HBM read ceiling
 * that the weight-streaming kernels are compared with.  With bytes = 0 it
 * launches one workgroup that does nothing else, the floor of a launch.
 * src must be 16-byte aligned and bytes a multiple of 16.  Asynchronous on
 * ``stream``; capturable.  Errors: W4_ERR_NULL, W4_ERR_ALIGN, W4_ERR_SHAPE,
 * W4_ERR_ALIAS (sink inside the source), W4_ERR_HIP.
 */
#define W4_READ_PROBE_SINK 4096
W4_API w4_status w4_read_probe(const void* src, size_t bytes, uint32_t* sink, void* stream);

/*
 * Test-only dequantisers.  They call the very device routines the hot
 * kernels use to build their operands, so the packed formats can be compared
 * bit for bit with an independent reference:
 *   w4_dequant_int4: the prefill GEMM's dequantisation ("Lab 5", section
 *                    "Python 反量化基线": the reference path materialises the
 *                    BF16 weight (q - z) * s before F.linear).  out_f32 gets
 *                    every weight's FP32 value as the GEMM computes it
 *                    (exact: at most 15 significant bits), out_bf16 the
 *                    GEMM's matrix-core operand, that value rounded to BF16
 *                    (nearest even).  qw, s, z as for w4_gemv; out_f32 float
 *                    [N][K]; out_bf16 bf16 [N][K]; either may be NULL, not both.
 *   w4_dequant_fp4:  the FP4 kernels' unpack (E2M1 code pairs, even k low),
 *                    times the BF16 scale in FP32, and its BF16 rounding.
 *                    qw_fp4 uint8 [N][K/2], s_fp4 bf16 [N][K/32] (one expert).
 * Errors: as w4_gemv.
 */
W4_API w4_status w4_dequant_int4(const int32_t* qw, const void* s, const void* z,
                                 float* out_f32, void* out_bf16, int K, int N, int g,
                                 void* stream);
W4_API w4_status w4_dequant_fp4(const uint8_t* qw_fp4, const void* s_fp4, float* out_f32,
                                void* out_bf16, int K, int N, void* stream);

/*
 * Test-only: the operands of the GEMV-path kernels (w4_gemv, the decode
 * chain, w4_gemm at M <= 16), from the same device routines.  Those kernels
 * never scale the codes: they dot the biased codes 128 + q, exact in BF16,
 * with x and apply zero and scale to the FP32 group sums,
 * sum_k (q - z) s x = s (sum_k (128 + q) x - (128 + z) sum_k x)
 * ("Lab 5", section "INT4 融合 GEMV": codes unpacked in registers, per-group
 * scale and zero applied in the fused GEMV).
 *   codes_out  uint32 [N][K/8][4]: for word p of row n, pair j (j = 0..3) is
 *              the bf16 pair (128 + q[n][8p+j], 128 + q[n][8p+j+4]), low half first
 *   x_out      uint32 [K/8][4]: pair j of word p is (x[8p+j], x[8p+j+4]), the
 *              x pair each code pair is dotted with; x is bf16 [K]
 *   qw, x and the outputs 4-byte aligned; K a positive multiple of 8;
 *   x and x_out both given or both NULL.
 * Errors: W4_ERR_NULL, W4_ERR_SHAPE, W4_ERR_ALIGN, W4_ERR_ALIAS, W4_ERR_HIP.
 */
W4_API w4_status w4_int4_gemv_operands(const int32_t* qw, const void* x, uint32_t* codes_out,
                                       uint32_t* x_out, int K, int N, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4_H */
