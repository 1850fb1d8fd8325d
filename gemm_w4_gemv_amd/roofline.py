"""Algorithmic bytes and flops of each operation, and MI355X peak figures.

Algorithmic bytes count every operand once: packed weights, scales (and
zeros), activations and outputs.  The BF16 weight that a materialising
implementation would write and read back is not counted.  Flops are
2 * M * K * N.
"""
from __future__ import annotations

HBM_PEAK_GBPS = 8000.0            # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0    # MI355X dense BF16 matrix peak, 2.5 PFLOP/s
INT4_GROUP = 128
FP4_GROUP = 32


def int4_weight_bytes(K: int, N: int, group: int = INT4_GROUP) -> int:
    """Packed codes (K/2 bytes per row) plus an FP16 scale and FP16 zero per group."""
    return N * K // 2 + 2 * 2 * N * (K // group)


def int4_linear_bytes(K: int, N: int, M: int = 1, group: int = INT4_GROUP) -> int:
    """One INT4 linear: weight bytes + BF16 x [M, K] + BF16 y [M, N]."""
    return int4_weight_bytes(K, N, group) + 2 * M * K + 2 * M * N


def fp4_expert_bytes(K: int, N: int) -> int:
    """One FP4 expert matrix: packed codes plus a BF16 scale per 32."""
    return N * K // 2 + 2 * N * (K // FP4_GROUP)


def moe_bytes(E: int, K: int, N: int, shared_x: bool) -> int:
    """E slots of one FP4 FC: E expert matrices, x once (shared) or per slot, y [E, N]."""
    xb = 2 * K if shared_x else 2 * E * K
    return E * fp4_expert_bytes(K, N) + xb + 2 * E * N


def flops(M: int, K: int, N: int) -> int:
    return 2 * M * K * N
