"""Plain FP64 CPU oracle for the fused 4-bit-weight x BF16 GEMV / GEMM.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, tables or helpers); the only thing both sides
use is ``seeded_inputs``, which draws random bits and holds no arithmetic of
the method.

Sources.  The operation is stated on three pages:

* "Lab 5: Gemma4 端到端推理优化" (Lab 5: Gemma4 end-to-end inference
  optimisation) -- sections "量化正确性" (GPTQ INT4, group 128, asymmetric),
  "Python 反量化基线" (the reference path: unpack INT4, elementwise
  scale/zero, materialise BF16, ``F.linear``), "INT4 融合 GEMV" (fused GEMV
  over packed INT4 with per-group scale/zero; equivalence test with random
  INT4, FP16 scale/zero, BF16 input at M=1 and M=128) and "最终配置"
  (``scale_dtype: float16``, ``group_size: 128``, ``symmetric: false``).
* "DeepSeek V4 Triton FP4 优化实战" (DeepSeek V4 Triton FP4 optimisation in
  practice) -- section "深度分析" item 2 (fused FP4 dequant+matmul: even
  columns use the low nibble, odd columns the high nibble) and item 4 (per
  token, 2 FC x 6 active experts per layer).

Readings where the pages are silent (each is also listed in the design notes):

1. INT4 dequant is ``(q - z) * s`` with an integer zero point stored as FP16.
2. INT4 nibble order: bits ``4j..4j+3`` of word ``p`` hold ``k = 8p + j``
   (lower k in the lower nibble, the same little-endian stream as FP4).
3. Layout follows ``F.linear``: weights ``[N, K]`` logically, K contiguous;
   scales/zeros ``[N, K/group]``.
4. FP4 is OCP MX E2M1 (sign bit 3, exponent bits 2..1 with bias 1, mantissa
   bit 0), scaled by a full BF16 multiply per 32 along K.
5. Output rounding is float -> bfloat16 round-to-nearest-even (the pages'
   reference path is PyTorch, whose bfloat16 cast is RNE).

Everything below is float64 unless stated; matrix products use
``numpy.matmul`` (a library routine) with no blocking or reordering.
"""
from __future__ import annotations

import numpy as np

INT4_GROUP = 128
FP4_GROUP = 32

__all__ = [
    "f16_to_f64", "bf16_to_f64", "int4_codes", "dequant_int4", "e2m1_value",
    "fp4_codes", "dequant_fp4", "linear", "gemv_int4", "gemm_int4",
    "moe_gemv_fp4", "moe_gemm_fp4", "round_bf16", "bf16_bits", "INT4_GROUP", "FP4_GROUP",
    "gptq_codes", "repack_gptq",
]


# ----------------------------------------------------------------- encodings
def f16_to_f64(bits) -> np.ndarray:
    """IEEE binary16 bit patterns -> float64 (numpy's exact widening)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns -> float64: a bfloat16 is the top half of a binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------- INT4
def int4_codes(qw) -> np.ndarray:
    """Unpack ``int32 [N, K/8]`` into 4-bit codes ``uint8 [N, K]``.

    Lab 5, "INT4 融合 GEMV": the kernel reads packed INT4 and unpacks it in
    registers.  Reading 2: nibble ``j`` of word ``p`` is the code of
    ``k = 8p + j``.
    """
    w = np.asarray(qw).view(np.uint32)
    n, kw = w.shape
    shifts = (4 * np.arange(8, dtype=np.uint32))[None, None, :]
    codes = (w[:, :, None] >> shifts) & np.uint32(0xF)
    return codes.reshape(n, kw * 8).astype(np.uint8)


def dequant_int4(qw, s_bits, z_bits, group: int = INT4_GROUP) -> np.ndarray:
    """``W[n, k] = (q[n, k] - z[n, k // group]) * s[n, k // group]`` in float64.

    Lab 5, "量化正确性" and "最终配置": GPTQ INT4, group 128, asymmetric, FP16
    scale; "Python 反量化基线": elementwise scale/zero on the unpacked codes.
    Reading 1: the zero point is subtracted from the code, then scaled.
    """
    q = int4_codes(qw).astype(np.float64)
    s = np.repeat(f16_to_f64(s_bits), group, axis=1)
    z = np.repeat(f16_to_f64(z_bits), group, axis=1)
    assert s.shape == q.shape and z.shape == q.shape, "scale/zero shape does not match K/group"
    return (q - z) * s


def gptq_codes(qweight) -> np.ndarray:
    """Codes ``uint8 [N, K]`` of a weight in GPTQ's own K-major layout.

    Lab 5, "量化正确性": the weights are GPTQ INT4.  GPTQ keeps the packed codes
    K-major, ``qweight int32 [K/8, N]``: word ``(p, n)`` holds the codes of
    ``k = 8p .. 8p+7`` of output ``n``, nibble ``j`` for ``k = 8p + j`` (the same
    nibble order as reading 2); its scales and zeros are ``[K/128, N]``.
    """
    w = np.asarray(qweight).view(np.uint32)
    kw, n = w.shape
    shifts = (4 * np.arange(8, dtype=np.uint32))[None, None, :]
    codes = (w.T[:, :, None] >> shifts) & np.uint32(0xF)  # [N, K/8, 8]
    return codes.reshape(n, kw * 8).astype(np.uint8)


def repack_gptq(qweight, s_gn, z_gn):
    """GPTQ's layout -> this path's ``F.linear`` layout (reading 3): ``qw int32 [N, K/8]``
    with nibble ``j`` of word ``(n, p)`` the code of ``k = 8p + j``, and scales and
    zeros ``[N, K/128]``.  The codes are unpacked by their GPTQ definition and packed
    again by this layout's, each code unchanged."""
    codes = gptq_codes(qweight).astype(np.uint32)
    n, k = codes.shape
    shifts = (4 * np.arange(8, dtype=np.uint32))[None, None, :]
    qw = np.bitwise_or.reduce(codes.reshape(n, k // 8, 8) << shifts, axis=2).astype(np.uint32).view(np.int32)
    return qw, np.ascontiguousarray(np.asarray(s_gn).T), np.ascontiguousarray(np.asarray(z_gn).T)


# ----------------------------------------------------------------------- FP4
def e2m1_value(code) -> np.ndarray:
    """Value of a 4-bit E2M1 code (reading 4, OCP MX element format).

    bit 3: sign; bits 2..1: exponent E (bias 1); bit 0: mantissa m.
    E == 0 is subnormal: 0.5 * m; otherwise 2**(E - 1) * (1 + m / 2).
    """
    c = np.asarray(code, dtype=np.int64)
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    mag = np.where(e == 0, 0.5 * m, np.exp2(e.astype(np.float64) - 1.0) * (1.0 + 0.5 * m))
    return sign * mag


def fp4_codes(qw) -> np.ndarray:
    """Unpack ``uint8 [..., N, K/2]`` into E2M1 codes ``[..., N, K]``.

    DeepSeek V4 Triton FP4, "深度分析" item 2: even K positions use the low
    nibble of a byte, odd positions the high nibble.
    """
    b = np.asarray(qw, dtype=np.uint8)
    lo = b & np.uint8(0xF)
    hi = b >> np.uint8(4)
    out = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def dequant_fp4(qw, s_bits, group: int = FP4_GROUP) -> np.ndarray:
    """``W[..., n, k] = e2m1(code[..., n, k]) * s[..., n, k // 32]`` in float64 (reading 4)."""
    v = e2m1_value(np.arange(16))[fp4_codes(qw)]  # the formula evaluated once per code
    s = np.repeat(bf16_to_f64(s_bits), group, axis=-1)
    assert s.shape == v.shape, "scale shape does not match K/32"
    return v * s


# ------------------------------------------------------------------ products
def linear(x, W) -> np.ndarray:
    """``y[m, n] = sum_k W[n, k] * x[m, k]`` (``F.linear`` semantics, no bias).

    Lab 5, "Python 反量化基线" (materialised weight, then ``F.linear``).
    """
    return np.matmul(np.asarray(x, dtype=np.float64), np.asarray(W, dtype=np.float64).T)


def gemm_int4(x_bits, qw, s_bits, z_bits, group: int = INT4_GROUP) -> np.ndarray:
    """FP64 ``y [M, N]`` for BF16 activations ``x_bits [M, K]`` and an INT4 linear."""
    x = bf16_to_f64(np.atleast_2d(x_bits))
    return linear(x, dequant_int4(qw, s_bits, z_bits, group))


def gemv_int4(x_bits, qw, s_bits, z_bits, group: int = INT4_GROUP, row_chunk: int = 8192) -> np.ndarray:
    """FP64 ``y [N]`` for one BF16 vector ``x_bits [K]`` (M = 1).

    Lab 5, "INT4 融合 GEMV": decode-time linears see a ``[1, hidden]`` input.
    Rows are processed ``row_chunk`` at a time only to bound host memory.
    """
    x_bits = np.asarray(x_bits).reshape(1, -1)
    qw, s_bits, z_bits = np.asarray(qw), np.asarray(s_bits), np.asarray(z_bits)
    n = qw.shape[0]
    out = np.empty(n, dtype=np.float64)
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        out[r0:r1] = gemm_int4(x_bits, qw[r0:r1], s_bits[r0:r1], z_bits[r0:r1], group)[0]
    return out


def moe_gemv_fp4(x_bits, pool_qw, pool_s, ids) -> np.ndarray:
    """FP64 ``y [E, N]``: slot ``e`` applies expert ``ids[e]`` of the pool to ``x_e``.

    DeepSeek V4 Triton FP4, "深度分析" item 4: each token runs 2 FC per layer
    on each of 6 active experts, each at M = 1.  ``x_bits`` is ``[K]`` (one
    vector shared by every slot) or ``[E, K]`` (one vector per slot).
    """
    ids = np.asarray(ids, dtype=np.int64)
    pool_qw, pool_s = np.asarray(pool_qw), np.asarray(pool_s)
    E = ids.shape[0]
    x_bits = np.asarray(x_bits)
    if x_bits.ndim == 1:
        x_bits = np.broadcast_to(x_bits, (E, x_bits.shape[0]))
    ys = []
    for e in range(E):
        W = dequant_fp4(pool_qw[ids[e]], pool_s[ids[e]])
        ys.append(linear(bf16_to_f64(x_bits[e])[None, :], W)[0])
    return np.stack(ys)


def moe_gemm_fp4(x_bits, row_start, ids, pool_qw, pool_s, cols=None) -> np.ndarray:
    """FP64 ``y [R, N]`` of a grouped FP4 expert GEMM (several tokens per expert).

    DeepSeek V4 Triton FP4, "深度分析" item 2: the fused FP4 kernel is a
    matrix product (dequantised tile times a block of activations), and item
    4: the tokens of a layer are routed to experts, each applying its 2 FC.
    Group ``e`` owns rows ``row_start[e] .. row_start[e+1] - 1`` of ``x_bits
    [R, K]`` and applies expert ``ids[e]``: ``y[r] = W_{ids[e]} x[r]``.
    Rows in no group are NaN.  ``cols`` selects output columns (weight rows).
    """
    x = bf16_to_f64(np.atleast_2d(np.asarray(x_bits)))
    row_start = np.asarray(row_start, dtype=np.int64)
    ids = np.asarray(ids, dtype=np.int64)
    pool_qw, pool_s = np.asarray(pool_qw), np.asarray(pool_s)
    N = pool_qw.shape[1] if cols is None else len(cols)
    y = np.full((x.shape[0], N), np.nan)
    for e in range(ids.shape[0]):
        a, b = int(row_start[e]), int(row_start[e + 1])
        if a >= b:
            continue
        qw_e, s_e = pool_qw[ids[e]], pool_s[ids[e]]
        if cols is not None:
            qw_e, s_e = qw_e[cols], s_e[cols]
        y[a:b] = linear(x[a:b], dequant_fp4(qw_e, s_e))
    return y


# ------------------------------------------------------------------ rounding
def round_bf16(v) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even (reading 5).

    A bfloat16 keeps 8 significant bits.  With ``v = f * 2**e`` and
    ``0.5 <= |f| < 1``, the result is ``rint(f * 2**8) * 2**(e - 8)``; numpy's
    ``rint`` rounds halfway cases to even.  Normal bfloat16 range only (the
    workloads' values are far from the subnormal and overflow limits).
    """
    v = np.asarray(v, dtype=np.float64)
    f, e = np.frexp(v)
    return np.ldexp(np.rint(f * 256.0), e - 8)


def bf16_bits(v) -> np.ndarray:
    """bfloat16 bit patterns of ``round_bf16(v)`` (exact: the value fits binary32's top half)."""
    r = round_bf16(v).astype(np.float32)
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
