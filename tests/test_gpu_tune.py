"""Every launch parameter of every kernel family, forced through the C ABI's
tuning override, against the FP64 oracle on shapes that span several tiles
and a ragged tail.  Whatever the per-shape table picks, that variant's
parity is covered here (the full-size workloads run the table's own choices
in test_gpu_parity.py).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from parity import check_outputs

pytestmark = pytest.mark.gpu

w4 = pytest.importorskip("gemm_w4_gemv_amd")
from gemm_w4_gemv_amd import host  # noqa: E402


@pytest.fixture(autouse=True)
def _reset():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    for k in w4.TUNE_KERNELS:
        w4.w4_tune_force(k, 0)


def _int4_case(M, K, N, key):
    lin = si.int4_linear(95, key, K, N)
    x_bits = si.bf16_normal(95, key + (1,), (M, K))
    W = oracle.dequant_int4(lin["qw"], lin["s"], lin["z"])
    y_ref = oracle.linear(oracle.bf16_to_f64(x_bits), W)
    return lin, x_bits, y_ref, np.linalg.norm(oracle.bf16_to_f64(x_bits), axis=1), np.abs(W).max(axis=1)


def _run_gemm(lin, x_bits, M, K, N):
    t = host.int4_tensors(lin)
    x = host.bf16_tensor(x_bits)
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    need = w4.w4_gemm_workspace_bytes(M, K, N)
    ws = torch.empty(max(need // 4, 1), dtype=torch.float32, device="cuda") if need else None
    if M == 1:
        w4.w4_gemv(x[0], t["qw"], t["s"], t["z"], y[0])
    else:
        w4.w4_gemm(x, t["qw"], t["s"], t["z"], y, workspace=ws)
    torch.cuda.synchronize()
    return host.bf16_values(y)


@pytest.mark.parametrize("rpt", [1, 2, 4, 8])
@pytest.mark.parametrize("K,N", [(3840, 2051), (8192, 130), (15360, 67)])
def test_gemv_rows_per_wave(rpt, K, N):
    w4.w4_tune_force("gemv", rpt)
    assert w4.w4_tune_param("gemv", 1, K, N) == rpt
    lin, x_bits, y_ref, xn, wmax = _int4_case(1, K, N, (0, K, N))
    check_outputs(_run_gemm(lin, x_bits, 1, K, N), y_ref, xn, wmax, f"gemv rpt={rpt} K={K} N={N}")


@pytest.mark.parametrize("rpt", [1, 2, 4, 8])
@pytest.mark.parametrize("K,N", [(3840, 1000), (15360, 130)])
def test_two_row_gemv_rows_per_wave(rpt, K, N):
    w4.w4_tune_force("gemv_rows2", rpt)
    lin, x_bits, y_ref, xn, wmax = _int4_case(2, K, N, (1, K, N))
    check_outputs(_run_gemm(lin, x_bits, 2, K, N), y_ref, xn, wmax, f"two-row gemv rpt={rpt} K={K} N={N}")


@pytest.mark.parametrize("blocks", [1, 2, 4])
@pytest.mark.parametrize("M,K,N", [(4, 3840, 1000), (16, 15360, 130), (9, 1024, 200)])
def test_small_m_rows_per_workgroup(blocks, M, K, N):
    w4.w4_tune_force("gemm_small_m", blocks)
    lin, x_bits, y_ref, xn, wmax = _int4_case(M, K, N, (2, M, K, N))
    check_outputs(_run_gemm(lin, x_bits, M, K, N), y_ref, xn, wmax, f"small-M blocks={blocks} M={M} K={K} N={N}")


@pytest.mark.parametrize("splits", list(range(1, 17)))
def test_prefill_k_splits(splits):
    M, K, N = 130, 2048, 130  # two row tiles, three ragged column tiles, 16 groups
    w4.w4_tune_force("gemm", splits)
    assert w4.w4_gemm_workspace_bytes(M, K, N) == (splits * M * N * 4 if splits > 1 else 0)
    lin, x_bits, y_ref, xn, wmax = _int4_case(M, K, N, (3,))
    check_outputs(_run_gemm(lin, x_bits, M, K, N), y_ref, xn, wmax, f"prefill splits={splits}")


@pytest.mark.parametrize("rpt", [1, 2, 4, 8])
@pytest.mark.parametrize("K,N,shared", [(4096, 200, True), (2048, 130, False)])
def test_moe_gemv_rows_per_wave(rpt, K, N, shared):
    w4.w4_tune_force("moe_gemv", rpt)
    pool = si.fp4_pool(96, (K, N), 8, K, N)
    ids = np.array([5, 0, 7], dtype=np.int32)
    x_bits = si.bf16_normal(96, (K, N, 1), (K,) if shared else (3, K))
    d = host.fp4_tensors(pool)
    y = torch.empty(3, N, dtype=torch.bfloat16, device="cuda")
    w4.w4_moe_gemv(host.bf16_tensor(x_bits), d["qw"], d["s"], torch.from_numpy(ids).cuda(), y)
    torch.cuda.synchronize()
    y_ref = oracle.moe_gemv_fp4(x_bits, pool["qw"], pool["s"], ids)
    xs = np.broadcast_to(oracle.bf16_to_f64(x_bits), (3, K))
    for e in range(3):
        W = oracle.dequant_fp4(pool["qw"][ids[e]], pool["s"][ids[e]])
        check_outputs(host.bf16_values(y)[e], y_ref[e], np.linalg.norm(xs[e]), np.abs(W).max(axis=1),
                      f"moe rpt={rpt} slot {e}")
