"""w4_gemm_noalloc, the GEMM entry point for callers that cannot allocate,
through the C ABI: its output equals w4_gemm's bit for bit (same kernels;
its split-K partials live in the library's per-GPU scratch instead of a
workspace) and meets the oracle's tolerance, on two calls in a row, the
second smaller, so the scratch's leftovers from the first call cannot leak
into the second.  Then the small-M path (no scratch) and w4_gemm again.
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

# (M, K, N): both split K (7.5 MiB, then 512 KiB of partial sums), then M = 4 (no scratch)
CASES = [(128, 15360, 3840), (128, 2048, 64), (4, 3840, 1000)]


def _gemm_pair(M, K, N, seed):
    lin = si.int4_linear(90, (seed,), K, N)
    x_bits = si.bf16_normal(90, (seed, 1), (M, K))
    t = host.int4_tensors(lin)
    x = host.bf16_tensor(x_bits)
    y_ref_dev = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    y_na = torch.full((M, N), -7.0, dtype=torch.bfloat16, device="cuda")
    need = w4.w4_gemm_workspace_bytes(M, K, N)
    ws = torch.empty(max(need // 4, 1), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    st = w4.lib.w4_gemm(x.data_ptr(), t["qw"].data_ptr(), t["s"].data_ptr(), t["z"].data_ptr(), y_ref_dev.data_ptr(),
                        M, K, N, 128, ws.data_ptr(), ws.numel() * 4, None)
    assert st == 0, w4.w4_last_error()
    st = w4.lib.w4_gemm_noalloc(x.data_ptr(), t["qw"].data_ptr(), t["s"].data_ptr(), t["z"].data_ptr(),
                                y_na.data_ptr(), M, K, N, 128, None)
    assert st == 0, w4.w4_last_error()
    torch.cuda.synchronize()
    return lin, x_bits, need, y_ref_dev, y_na


def test_gemm_noalloc_equals_gemm_two_calls_then_smaller():
    needs = []
    for i, (M, K, N) in enumerate(CASES):
        print(f"w4_gemm_noalloc case {i}: M={M} K={K} N={N}", flush=True)
        lin, x_bits, need, y_gemm, y_na = _gemm_pair(M, K, N, i)
        needs.append(need)
        assert torch.equal(y_na.view(torch.int16), y_gemm.view(torch.int16)), f"case {i}: differs from w4_gemm"
        W = oracle.dequant_int4(lin["qw"], lin["s"], lin["z"])
        y_ref = oracle.linear(oracle.bf16_to_f64(x_bits), W)
        check_outputs(host.bf16_values(y_na), y_ref,
                      np.linalg.norm(oracle.bf16_to_f64(x_bits), axis=1), np.abs(W).max(axis=1), f"noalloc case {i}")
    assert needs[0] > needs[1] > 0 and needs[2] == 0, needs
    assert needs[0] <= w4.GEMM_NOALLOC_SCRATCH_BYTES


def test_gemm_noalloc_repeated_calls_stay_equal():
    """The same call twice more after other work: identical bits each time."""
    M, K, N = CASES[0]
    _, _, _, y_gemm, y_na = _gemm_pair(M, K, N, 0)
    first = y_na.clone()
    for rep in range(2):
        _, _, _, _, y2 = _gemm_pair(M, K, N, 0)
        assert torch.equal(y2.view(torch.int16), first.view(torch.int16)), f"repeat {rep}"
    assert torch.equal(first.view(torch.int16), y_gemm.view(torch.int16))
