"""w4_repack_gptq: GPTQ's K-major layout in, this path's layout out, bit for bit
against the oracle's repack; then the GEMV on the repacked weight against the
oracle's product written from the GPTQ layout's own definition."""
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
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def gptq_weight(K, N, key):
    """A weight in GPTQ's layout: random words [K/8, N], scales and zeros [K/128, N]."""
    lin = si.int4_linear(97, key, K, N)  # only its bits are reused, in the other orientation
    qweight = np.ascontiguousarray(lin["qw"].view(np.uint32).reshape(K // 8, N)).view(np.int32)
    return qweight, np.ascontiguousarray(lin["s"].reshape(K // 128, N)), np.ascontiguousarray(lin["z"].reshape(K // 128, N))


@pytest.mark.parametrize("K,N", [(3840, 2051), (128, 1), (15360, 3840), (4096, 64)])
def test_repack_gptq_bit_exact(K, N):
    qweight, s, z = gptq_weight(K, N, (K, N))
    qw_d, s_d, z_d = w4.w4_repack_gptq(torch.from_numpy(qweight).cuda(), host.f16_tensor(s), host.f16_tensor(z))
    torch.cuda.synchronize()
    qw_r, s_r, z_r = oracle.repack_gptq(qweight, s, z)
    assert np.array_equal(qw_d.cpu().numpy(), qw_r)
    assert np.array_equal(host.bits_of(s_d), s_r) and np.array_equal(host.bits_of(z_d), z_r)


def test_gemv_on_repacked_gptq_weight():
    K, N = 3840, 2051
    qweight, s, z = gptq_weight(K, N, (9,))
    qw_d, s_d, z_d = w4.w4_repack_gptq(torch.from_numpy(qweight).cuda(), host.f16_tensor(s), host.f16_tensor(z))
    x_bits = si.bf16_normal(97, (9, 1), (K,))
    y = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    w4.w4_gemv(host.bf16_tensor(x_bits), qw_d, s_d, z_d, y)
    torch.cuda.synchronize()
    codes = oracle.gptq_codes(qweight).astype(np.float64)
    W = (codes - np.repeat(oracle.f16_to_f64(z).T, 128, axis=1)) * np.repeat(oracle.f16_to_f64(s).T, 128, axis=1)
    x = oracle.bf16_to_f64(x_bits)
    check_outputs(host.bf16_values(y), W @ x, np.linalg.norm(x), np.abs(W).max(axis=1), "gemv on a GPTQ import")
