// Per-shape launch parameters: the measured table, the launchers' rules for
// other shapes, and the process-wide override used by the sweep and tests.
//
// "Lab 5: Gemma4 端到端推理优化", section "GEMV 分块测试": the GEMV's block
// shape was chosen per workload by a sweep (BLOCK_N 32 -> 16, BLOCK_PK 512 ->
// 256 -> 128), and section "INT4 融合 GEMV" notes that the choice moved the
// time, not the result.  Here each kernel has one launch parameter and the
// table below holds, for the shapes of the decode step, the logits GEMV, the
// prefill GEMMs, small decode batches and the FP4 expert FCs, the value a
// sweep over every allowed parameter measured fastest on an MI355X.  Every
// parameter computes the same operation (the summation order may differ, so
// results can differ in the last bits between parameters, never between runs).
#include <atomic>

#include "tune.hpp"
#include "w4_internal.hpp"

namespace w4 {
namespace {

struct TuneEntry {
    int kernel, M, K, N, param;  // M = 0 matches any M
};

// Measured table (graph replays over weight copies that walk >= 512 MB, so
// every call streams from HBM; the fastest parameter per shape).
constexpr TuneEntry kTable[] = {
#include "tune_table.inc"
    {-1, 0, 0, 0, 0},  // end
};

std::atomic<int> g_forced[W4_TUNE_KERNELS] = {};

int groups_of(int K) { return K / 128; }

}  // namespace

bool tune_param_valid(int kernel, int param) {
    switch (kernel) {
        case W4_TUNE_GEMV: return param == 1 || param == 2 || param == 4 || param == 8;
        case W4_TUNE_GEMV_ROWS2: return param == 1 || param == 2 || param == 4 || param == 8;
        case W4_TUNE_GEMM_SMALL_M: return param == 1 || param == 2 || param == 4;
        case W4_TUNE_GEMM: return param >= 1 && param <= 16;
        case W4_TUNE_MOE_GEMV: return param == 1 || param == 2 || param == 4 || param == 8;
        default: return false;
    }
}

int tuned_param(int kernel, int M, int K, int N, int rule) {
    const int f = g_forced[kernel].load(std::memory_order_relaxed);
    if (f > 0) return f;
    int any = 0;
    for (const TuneEntry& e : kTable) {
        if (e.kernel != kernel || e.K != K || e.N != N) continue;
        if (e.M == M) return e.param;
        if (e.M == 0) any = e.param;
    }
    return any > 0 ? any : rule;
}

void tune_force(int kernel, int param) { g_forced[kernel].store(param, std::memory_order_relaxed); }

// Rows per wave of the GEMV: the most (8, 4, 2, 1) that still launch 240
// workgroups for a matrix under 16 MB (512 above).  Fewer, larger workgroups
// cost less per launch; more of them keep more loads in flight.
int gemv_rows_per_wave_rule(int K, int N) {
    const int C = K / 32;
    const int T = 4 / row_split(C).slices;
    const long min_blocks = (size_t)N * (size_t)C * 16u < ((size_t)16 << 20) ? 240 : 512;
    for (int rpt = 8; rpt > 1; rpt /= 2)
        if ((N + T * rpt - 1) / (T * rpt) >= min_blocks) return rpt;
    return 1;
}

// The two-row GEMV: the most (8, 4, 2, 1) rows per wave that launch 512 workgroups.
int gemv_rows2_rows_per_wave_rule(int K, int N) {
    const int T = 4 / row_split(K / 32).slices;
    for (int rpt = 8; rpt > 1; rpt /= 2)
        if ((N + T * rpt - 1) / (T * rpt) >= 512) return rpt;
    return 1;
}

// The small-M GEMM: the widest tile (4, 2, 1 blocks of 16 weight rows) that
// still gives 240 workgroups (wider tiles read the activations fewer times).
int gemm_small_m_blocks_rule(int N) {
    if ((N + 63) / 64 >= 240) return 4;
    if ((N + 31) / 32 >= 240) return 2;
    return 1;
}

// The prefill GEMM: split K when its tiles cannot fill the 256 compute units,
// round(256 / tiles) ways, at most 16 and at most one group per split.
int gemm_splits_rule(int M, int K, int N) {
    const long tiles = (long)((M + kGemmTileM - 1) / kGemmTileM) * ((N + kGemmTileN - 1) / kGemmTileN);
    int splits = (int)((256 + tiles / 2) / tiles);
    if (splits < 1) splits = 1;
    if (splits > groups_of(K)) splits = groups_of(K);
    if (splits > 16) splits = 16;
    return splits;
}

// The FP4 expert GEMV: the most (4, 2, 1) rows per wave that launch 512
// workgroups over all slots.
int moe_gemv_rows_per_wave_rule(int E, int K, int N) {
    const int T = 4 / row_split(K / 32).slices;
    for (int rpt = 8; rpt > 1; rpt /= 2)
        if ((long)E * ((N + T * rpt - 1) / (T * rpt)) >= 512) return rpt;
    return 1;
}

int gemv_rows_per_wave(int K, int N) { return tuned_param(W4_TUNE_GEMV, 1, K, N, gemv_rows_per_wave_rule(K, N)); }
int gemv_rows2_rows_per_wave(int K, int N) {
    return tuned_param(W4_TUNE_GEMV_ROWS2, 2, K, N, gemv_rows2_rows_per_wave_rule(K, N));
}
int gemm_small_m_blocks(int M, int K, int N) {
    return tuned_param(W4_TUNE_GEMM_SMALL_M, M, K, N, gemm_small_m_blocks_rule(N));
}
int gemm_splits(int M, int K, int N) {
    int s = tuned_param(W4_TUNE_GEMM, M, K, N, gemm_splits_rule(M, K, N));
    return s > groups_of(K) ? groups_of(K) : s;  // a forced value never exceeds one group per split
}
int moe_gemv_rows_per_wave(int E, int K, int N) {
    return tuned_param(W4_TUNE_MOE_GEMV, E, K, N, moe_gemv_rows_per_wave_rule(E, K, N));
}

}  // namespace w4
