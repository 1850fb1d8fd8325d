"""Each plausible oracle mistake must fail at least one pin (planted on the CPU only)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import test_oracle_pins as pins

_orig = {name: getattr(oracle, name) for name in oracle.__all__ if callable(getattr(oracle, name))}


def _reversed_nibbles(qw):
    c = _orig["int4_codes"](qw)
    n, k = c.shape
    return c.reshape(n, k // 8, 8)[:, :, ::-1].reshape(n, k)


def _swapped_fp4(qw):
    c = _orig["fp4_codes"](qw)
    out = c.copy()
    out[..., 0::2], out[..., 1::2] = c[..., 1::2], c[..., 0::2]
    return out


def _q_s_minus_z(qw, s_bits, z_bits, group=128):
    q = oracle.int4_codes(qw).astype(np.float64)
    s = np.repeat(oracle.f16_to_f64(s_bits), group, axis=1)
    z = np.repeat(oracle.f16_to_f64(z_bits), group, axis=1)
    return q * s - z


def _no_zero(qw, s_bits, z_bits, group=128):
    q = oracle.int4_codes(qw).astype(np.float64)
    return q * np.repeat(oracle.f16_to_f64(s_bits), group, axis=1)


def _wrong_group(qw, s_bits, z_bits, group=128):
    q = oracle.int4_codes(qw).astype(np.float64)
    idx = np.minimum(np.arange(q.shape[1]) // 64, s_bits.shape[1] - 1)
    s = oracle.f16_to_f64(s_bits)[:, idx]
    z = oracle.f16_to_f64(z_bits)[:, idx]
    return (q - z) * s


def _sign_flip_zero(qw, s_bits, z_bits, group=128):
    q = oracle.int4_codes(qw).astype(np.float64)
    s = np.repeat(oracle.f16_to_f64(s_bits), group, axis=1)
    z = np.repeat(oracle.f16_to_f64(z_bits), group, axis=1)
    return (z - q) * s


def _e2m1_bias0(code):
    c = np.asarray(code, dtype=np.int64)
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    return sign * np.where(e == 0, 0.5 * m, np.exp2(e.astype(np.float64)) * (1.0 + 0.5 * m))


def _linear_untransposed(x, W):
    W = np.asarray(W, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    return np.matmul(x, W.reshape(W.shape[1], W.shape[0]))


def _round_half_up(v):
    v = np.asarray(v, dtype=np.float64)
    f, e = np.frexp(v)
    return np.ldexp(np.floor(f * 256.0 + 0.5), e - 8)


def _moe_ignores_ids(x_bits, pool_qw, pool_s, ids):
    return _orig["moe_gemv_fp4"](x_bits, pool_qw, pool_s, list(range(len(ids))))


def _gemv_chunks_shifted(x_bits, qw, s_bits, z_bits, group=128, row_chunk=8192):
    """Each row chunk after the first computed from the rows one place later (a slip in the chunk bounds)."""
    y = _orig["gemv_int4"](x_bits, qw, s_bits, z_bits, group, row_chunk)
    n = np.asarray(qw).shape[0]
    if n > row_chunk:
        shifted = _orig["gemv_int4"](x_bits, np.roll(qw, -1, axis=0), np.roll(s_bits, -1, axis=0),
                                     np.roll(z_bits, -1, axis=0), group, row_chunk)
        y = y.copy()
        y[row_chunk:] = shifted[row_chunk:]
    return y


def _moe_gemm_group_shifted(x_bits, row_start, ids, pool_qw, pool_s, cols=None):
    rs = list(row_start)
    rs = [rs[0]] + [r + 1 for r in rs[1:-1]] + [rs[-1]]  # every group boundary one row late
    return _orig["moe_gemm_fp4"](x_bits, rs, ids, pool_qw, pool_s, cols)


def _moe_gemm_ids_ignored(x_bits, row_start, ids, pool_qw, pool_s, cols=None):
    return _orig["moe_gemm_fp4"](x_bits, row_start, list(range(len(ids))), pool_qw, pool_s, cols)


def _dequant_fp4_scale_by_k(qw, s_bits, group=32):
    v = oracle.e2m1_value(oracle.fp4_codes(qw))
    s = oracle.bf16_to_f64(s_bits)
    idx = np.minimum(np.arange(v.shape[-1]) // 16, s.shape[-1] - 1)
    return v * s[..., idx]


def _repack_reshaped_not_transposed(qweight, s_gn, z_gn):
    qw = np.ascontiguousarray(np.asarray(qweight).reshape(np.asarray(qweight).shape[::-1]))
    return qw, np.ascontiguousarray(np.asarray(s_gn).T), np.ascontiguousarray(np.asarray(z_gn).T)


def _gptq_codes_nibbles_reversed(qweight):
    c = _orig["gptq_codes"](qweight)
    n, k = c.shape
    return c.reshape(n, k // 8, 8)[:, :, ::-1].reshape(n, k)


MUTANTS = {
    "reversed_int4_nibbles": ("int4_codes", _reversed_nibbles),
    "swapped_fp4_nibbles": ("fp4_codes", _swapped_fp4),
    "q_times_s_minus_z": ("dequant_int4", _q_s_minus_z),
    "zero_point_dropped": ("dequant_int4", _no_zero),
    "int4_group_of_64": ("dequant_int4", _wrong_group),
    "zero_point_sign": ("dequant_int4", _sign_flip_zero),
    "e2m1_exponent_bias": ("e2m1_value", _e2m1_bias0),
    "untransposed_weight": ("linear", _linear_untransposed),
    "bf16_round_half_up": ("round_bf16", _round_half_up),
    "moe_slot_ids_ignored": ("moe_gemv_fp4", _moe_ignores_ids),
    "fp4_group_of_16": ("dequant_fp4", _dequant_fp4_scale_by_k),
    "moe_gemm_group_boundary_off_by_one": ("moe_gemm_fp4", _moe_gemm_group_shifted),
    "moe_gemm_ids_ignored": ("moe_gemm_fp4", _moe_gemm_ids_ignored),
    "gemv_row_chunks_shifted": ("gemv_int4", _gemv_chunks_shifted),
    "gptq_repack_reshaped": ("repack_gptq", _repack_reshaped_not_transposed),
    "gptq_nibbles_reversed": ("gptq_codes", _gptq_codes_nibbles_reversed),
}


def _all_pins():
    calls = []
    for name in dir(pins):
        if not name.startswith("test_"):
            continue
        fn = getattr(pins, name)
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if params:
            argnames = [a.strip() for a in params[0].args[0].split(",")]
            for values in params[0].args[1]:
                calls.append((name, fn, dict(zip(argnames, values))))
        else:
            calls.append((name, fn, {}))
    return calls


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_mutant_is_caught(mutant, monkeypatch):
    attr, fn = MUTANTS[mutant]
    monkeypatch.setattr(oracle, attr, fn)
    caught = []
    for name, pin, kwargs in _all_pins():
        try:
            pin(**kwargs)
        except Exception:  # AssertionError, or a shape error from a broken operand
            caught.append(name)
    assert caught, f"no pin catches mutant {mutant}"
