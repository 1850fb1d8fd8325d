// Per-shape launch parameters.  Each launcher has one tunable parameter
// (rows per wave, weight rows per workgroup, K splits); the value comes from
// a table of measured choices for the workloads' shapes, else from the
// launcher's own rule.  A process-wide override (w4_tune_force) serves the
// sweep that measures the table and the tests that run every variant.
#pragma once

#include "w4.h"

namespace w4 {

// Whether ``param`` is a launch parameter the kernel ``kernel`` has (the
// prefill GEMM's K splits also need splits <= K / 128, checked by the caller).
bool tune_param_valid(int kernel, int param);

// The parameter a call of shape (M, K, N) launches with: the forced value if
// one is set, else the table's entry for the shape, else ``rule``.
int tuned_param(int kernel, int M, int K, int N, int rule);

// Every later call of ``kernel`` launches with ``param`` (0: back to the
// table and the rules).  Process-wide; not for calls running concurrently.
void tune_force(int kernel, int param);

// The launchers' rules for shapes outside the table (also what the table's
// unmeasured shapes fall back to).
int gemv_rows_per_wave_rule(int K, int N);
int gemv_rows2_rows_per_wave_rule(int K, int N);
int gemm_small_m_blocks_rule(int N);
int gemm_splits_rule(int M, int K, int N);
int moe_gemv_rows_per_wave_rule(int E, int K, int N);

// The parameter each launcher actually uses (tuned_param with its rule).
int gemv_rows_per_wave(int K, int N);
int gemv_rows2_rows_per_wave(int K, int N);
int gemm_small_m_blocks(int M, int K, int N);
int gemm_splits(int M, int K, int N);
int moe_gemv_rows_per_wave(int E, int K, int N);

}  // namespace w4
