"""Pins of the FP64 oracle to facts that do not come from the oracle itself.

Every check here is chosen so that a plausible slip in the oracle (a swapped
nibble, a transposed operand, a dropped zero point, a wrong group index, a
sign error, double rounding) fails at least one of them.  CPU only.
"""
from __future__ import annotations

import json
import pathlib
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from seeded_inputs import rng, bf16_normal, int4_linear, fp4_pool

GOLDEN = pathlib.Path(__file__).parent / "golden"


def load(name):
    return json.loads((GOLDEN / name).read_text())


# ---------------------------------------------------------------- helpers
def pack_int4(codes: np.ndarray) -> np.ndarray:
    """Independent packer (Python integers): code of k = 8p + j goes to bits 4j..4j+3."""
    n, k = codes.shape
    out = np.zeros((n, k // 8), dtype=np.uint32)
    for r in range(n):
        for p in range(k // 8):
            word = 0
            for j in range(8):
                word |= int(codes[r, 8 * p + j]) << (4 * j)
            out[r, p] = word
    return out.view(np.int32)


def pack_fp4(codes: np.ndarray) -> np.ndarray:
    """Independent packer: even k -> low nibble, odd k -> high nibble."""
    flat = codes.reshape(-1, codes.shape[-1])
    out = np.zeros((flat.shape[0], flat.shape[1] // 2), dtype=np.uint8)
    for r in range(flat.shape[0]):
        for i in range(flat.shape[1] // 2):
            out[r, i] = int(flat[r, 2 * i]) | (int(flat[r, 2 * i + 1]) << 4)
    return out.reshape(codes.shape[:-1] + (codes.shape[-1] // 2,))


def f16_bits(values) -> np.ndarray:
    return np.asarray(values, dtype=np.float64).astype(np.float16).view(np.uint16)


def bf16_bits_exact(values) -> np.ndarray:
    """bfloat16 bits of values that are exactly representable (asserted)."""
    f = np.asarray(values, dtype=np.float32)
    b = f.view(np.uint32)
    assert np.all(b & 0xFFFF == 0), "value not exactly representable in bfloat16"
    return (b >> 16).astype(np.uint16)


def frac_f16(bits: int) -> Fraction:
    return Fraction(struct.unpack("<e", struct.pack("<H", int(bits)))[0])


def frac_bf16(bits: int) -> Fraction:
    return Fraction(struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0])


# -------------------------------------------------------------- nibble order
def test_int4_nibble_order_literal_words():
    for case in load("int4_nibble_order.json")["cases"]:
        word = np.array([[int(case["word"], 16)]], dtype=np.uint32).view(np.int32)
        assert oracle.int4_codes(word)[0].tolist() == case["codes"], case["word"]


def test_fp4_literal_bytes_and_table():
    g = load("fp4_e2m1.json")
    table = {int(k): v for k, v in g["table"].items()}
    vals = oracle.e2m1_value(np.arange(16))
    for c in range(16):
        assert vals[c] == table[c]
        assert np.signbit(vals[c]) == (c >= 8)  # code 8 is -0.0
    for case in g["bytes"]:
        b = np.array([[int(case["byte"], 16)]], dtype=np.uint8)
        got = oracle.e2m1_value(oracle.fp4_codes(b))[0].tolist()
        assert got == case["values"], case["byte"]
        assert [np.signbit(v) for v in got] == [np.signbit(v) for v in case["values"]]


def test_pack_unpack_round_trip():
    g = rng(1, 1)
    codes = g.integers(0, 16, size=(5, 256)).astype(np.uint8)
    assert np.array_equal(oracle.int4_codes(pack_int4(codes)), codes)
    c4 = g.integers(0, 16, size=(2, 3, 64)).astype(np.uint8)
    assert np.array_equal(oracle.fp4_codes(pack_fp4(c4)), c4)


# ------------------------------------------------------- dequant formula pins
def test_zero8_is_textbook_signed_int4():
    """With z = 8 and s = 1, (q - z) equals the two's-complement int4 value of q ^ 8."""
    g = rng(1, 2)
    codes = g.integers(0, 16, size=(4, 256)).astype(np.uint8)
    qw = pack_int4(codes)
    ones = f16_bits(np.ones((4, 2)))
    eights = f16_bits(np.full((4, 2), 8.0))
    W = oracle.dequant_int4(qw, ones, eights)
    signed = (((codes ^ 8).astype(np.int8) << 4) >> 4).astype(np.float64)  # sign-extend 4 -> 8 bits
    assert np.array_equal(W, signed)


def test_zero8_mirror_negates_output():
    """Codes q' = 16 - q (q in 1..15) with z = 8 negate every weight, hence y."""
    g = rng(1, 3)
    codes = g.integers(1, 16, size=(3, 384)).astype(np.uint8)
    s = f16_bits(g.uniform(0.002, 0.02, size=(3, 3)))
    z = f16_bits(np.full((3, 3), 8.0))
    x = bf16_normal(1, (3, 1), (2, 384))
    y = oracle.gemm_int4(x, pack_int4(codes), s, z)
    y_m = oracle.gemm_int4(x, pack_int4((16 - codes).astype(np.uint8)), s, z)
    assert np.array_equal(y_m, -y)


def test_unit_scale_zero_zero_is_integer_matmul():
    """s = 1, z = 0 reduces to an integer matrix product (numpy int64 matmul)."""
    g = rng(1, 4)
    M, K, N = 3, 512, 7
    codes = g.integers(0, 16, size=(N, K)).astype(np.int64)
    xi = g.integers(-8, 9, size=(M, K)).astype(np.int64)
    y = oracle.gemm_int4(bf16_bits_exact(xi.astype(np.float32)), pack_int4(codes.astype(np.uint8)),
                         f16_bits(np.ones((N, K // 128))), f16_bits(np.zeros((N, K // 128))))
    assert np.array_equal(y, (xi @ codes.T).astype(np.float64))


def test_group_boundaries_one_hot():
    """One-hot x at k in {0, 127, 128, 255}: y[n] = (q[n,k] - z[n,g]) * s[g], g = k // 128."""
    g = rng(1, 5)
    N, K = 5, 256
    codes = g.integers(0, 16, size=(N, K)).astype(np.uint8)
    s_vals = np.array([[1.0, 2.0]] * N)           # s_g = 2**g
    z_vals = np.array([[3.0, 11.0]] * N)          # distinct zero per group
    qw = pack_int4(codes)
    for k in (0, 127, 128, 255):
        x = np.zeros(K, dtype=np.float32)
        x[k] = 1.0
        y = oracle.gemv_int4(bf16_bits_exact(x), qw, f16_bits(s_vals), f16_bits(z_vals))
        grp = k // 128
        expect = (codes[:, k].astype(np.float64) - z_vals[:, grp]) * s_vals[:, grp]
        assert np.array_equal(y, expect), k


def test_single_weight_is_not_transposed():
    """A single non-zero weight at (n0, k0) and one-hot x at k0 light exactly output n0."""
    N, K = 3, 384
    codes = np.full((N, K), 8, dtype=np.uint8)    # z = 8 -> every weight 0 ...
    n0, k0 = 2, 129
    codes[n0, k0] = 13                            # ... except W[n0, k0] = 5 * s
    s = f16_bits(np.full((N, 3), 0.25))
    z = f16_bits(np.full((N, 3), 8.0))
    x = np.zeros(K, dtype=np.float32)
    x[k0] = 1.0
    y = oracle.gemv_int4(bf16_bits_exact(x), pack_int4(codes), s, z)
    assert y.tolist() == [0.0, 0.0, 1.25]


def test_closed_form_int4():
    """x = 1, q = c, z = z0, s = s0 everywhere: y = K (c - z0) s0."""
    N, K = 4, 640
    for c, z0, s0 in [(0, 0, 0.5), (15, 0, 0.0078125), (3, 12, 0.015625), (9, 9, 0.25), (15, 15, 1.0)]:
        qw = np.full((N, K // 8), c * 0x11111111, dtype=np.uint32).view(np.int32)
        y = oracle.gemv_int4(bf16_bits_exact(np.ones(K, dtype=np.float32)), qw,
                             f16_bits(np.full((N, K // 128), s0)), f16_bits(np.full((N, K // 128), float(z0))))
        assert np.array_equal(y, np.full(N, K * (c - z0) * s0)), (c, z0, s0)


@pytest.mark.parametrize("N,row_chunk", [(8192 + 37, 8192), (10, 3)])
def test_gemv_row_chunks_closed_form(N, row_chunk):
    """The GEMV oracle takes its rows in chunks (8192 by default): every row
    past a chunk boundary still gives its own closed form.  Row n holds the
    constant code c_n = n mod 16, zero z_n = (n / 16) mod 16 and scale
    s_n = 2^-(1 + (n / 256) mod 8); with x = 1, y[n] = K (c_n - z_n) s_n."""
    K = 128
    n = np.arange(N)
    c = n % 16
    z = (n // 16) % 16
    sv = 2.0 ** -(1 + (n // 256) % 8)
    qw = np.repeat((c * 0x11111111).astype(np.uint32)[:, None], K // 8, axis=1).view(np.int32)
    y = oracle.gemv_int4(bf16_bits_exact(np.ones(K, dtype=np.float32)), qw, f16_bits(sv[:, None]),
                         f16_bits(z[:, None].astype(np.float64)), row_chunk=row_chunk)
    assert np.array_equal(y, K * (c - z) * sv)


def test_closed_form_fp4():
    """x = 1, every code c, scale s0: y = K * v(c) * s0 with v from the OCP table."""
    table = {int(k): v for k, v in load("fp4_e2m1.json")["table"].items()}
    N, K = 3, 96
    for c in range(16):
        pool = np.full((1, N, K // 2), c | (c << 4), dtype=np.uint8)
        s0 = 0.125
        s = bf16_bits_exact(np.full((1, N, K // 32), s0, dtype=np.float32))
        y = oracle.moe_gemv_fp4(bf16_bits_exact(np.ones(K, dtype=np.float32)), pool, s, [0])
        assert np.array_equal(y[0], np.full(N, K * table[c] * s0)), c


def test_fp4_group_and_parity_one_hot():
    """FP4: one-hot x at k in {0, 1, 31, 32, 63} picks nibble (k even: low) and scale k // 32."""
    g = rng(1, 6)
    N, K = 3, 64
    codes = g.integers(0, 16, size=(1, N, K)).astype(np.uint8)
    pool = pack_fp4(codes)
    svals = np.array([[[0.25, 4.0]] * N], dtype=np.float32)
    table = oracle.e2m1_value(np.arange(16))
    for k in (0, 1, 31, 32, 63):
        x = np.zeros(K, dtype=np.float32)
        x[k] = 1.0
        y = oracle.moe_gemv_fp4(bf16_bits_exact(x), pool, bf16_bits_exact(svals), [0])[0]
        assert np.array_equal(y, table[codes[0, :, k]] * svals[0, :, k // 32]), k


def test_moe_slot_order_and_broadcast():
    """Slot e uses expert ids[e]; a broadcast x equals the same x repeated per slot."""
    E_pool, N, K = 8, 4, 64
    # expert i: every code = 2 (value 1.0), scale = i + 1 -> y = K * (i + 1) for x = 1
    pool = np.full((E_pool, N, K // 2), 0x22, dtype=np.uint8)
    s = bf16_bits_exact(np.broadcast_to(np.arange(1, E_pool + 1, dtype=np.float32)[:, None, None],
                                        (E_pool, N, K // 32)).copy())
    ids = [5, 0, 7, 2]
    ones = bf16_bits_exact(np.ones(K, dtype=np.float32))
    y = oracle.moe_gemv_fp4(ones, pool, s, ids)
    assert y.tolist() == [[K * (i + 1.0)] * N for i in ids]
    y2 = oracle.moe_gemv_fp4(np.stack([ones] * len(ids)), pool, s, ids)
    assert np.array_equal(y, y2)


def test_moe_gemm_groups_by_hand():
    """Grouped FP4 GEMM on a hand-built case: group 0 = rows 0, 1 -> expert 1;
    group 1 = no rows; group 2 = row 2 -> expert 0.  One-hot rows pick single
    weights, whose values follow from the OCP E2M1 table times the scale."""
    table = {int(k): v for k, v in load("fp4_e2m1.json")["table"].items()}
    K, N = 32, 2
    codes = np.zeros((2, N, K), dtype=np.uint8)
    codes[0, :, 5] = [3, 12]     # expert 0, k = 5: 1.5, -2.0
    codes[1, :, 0] = [7, 1]      # expert 1, k = 0: 6.0, 0.5
    codes[1, :, 31] = [10, 4]    # expert 1, k = 31: -1.0, 2.0
    pool = pack_fp4(codes)
    s = bf16_bits_exact(np.array([[[0.5]] * N, [[4.0]] * N], dtype=np.float32))
    x = np.zeros((3, K), dtype=np.float32)
    x[0, 0] = 1.0
    x[1, 31] = 1.0
    x[2, 5] = 1.0
    y = oracle.moe_gemm_fp4(bf16_bits_exact(x), [0, 2, 2, 3], [1, 1, 0], pool, s)
    expect = [[table[7] * 4.0, table[1] * 4.0],
              [table[10] * 4.0, table[4] * 4.0],
              [table[3] * 0.5, table[12] * 0.5]]
    assert y.tolist() == expect == [[24.0, 2.0], [-4.0, 8.0], [0.75, -1.0]]


def test_moe_gemm_rows_match_per_token_gemv():
    """Every row of the grouped GEMM equals the M = 1 expert GEMV of its token
    with its group's expert; rows outside every group stay NaN."""
    g = rng(4, 7)
    P, N, K = 5, 6, 96
    pool = g.integers(0, 256, size=(P, N, K // 2)).astype(np.uint8)
    s = bf16_bits_exact((np.exp2(g.integers(-8, -1, size=(P, N, K // 32)))
                         * g.choice([1.0, 1.25, 1.5, 1.75], size=(P, N, K // 32))).astype(np.float32))
    R = 9
    x = bf16_normal(4, (7, 1), (R, K))
    row_start, ids = [0, 3, 3, 7, 8], [4, 1, 0, 2]   # row 8 in no group
    y = oracle.moe_gemm_fp4(x, row_start, ids, pool, s)
    for e, expert in enumerate(ids):
        for r in range(row_start[e], row_start[e + 1]):
            assert np.allclose(y[r], oracle.moe_gemv_fp4(x[r], pool, s, [expert])[0], rtol=1e-12, atol=1e-300)
    assert np.all(np.isnan(y[8]))
    cols = [5, 0, 3]
    assert np.array_equal(oracle.moe_gemm_fp4(x, row_start, ids, pool, s, cols=cols)[:8], y[:8][:, cols])


# ------------------------------------------------------------ brute force
@pytest.mark.parametrize("K,N,M", [(128, 1, 1), (128, 3, 2), (256, 2, 2), (256, 3, 1)])
def test_bruteforce_exact_fractions_int4(K, N, M):
    """Oracle vs exact rational arithmetic over the exact FP16/BF16 input values."""
    g = rng(2, K, N, M)
    codes = g.integers(0, 16, size=(N, K)).astype(np.uint8)
    s = f16_bits(g.uniform(0.002, 0.02, size=(N, K // 128)))
    z = f16_bits(g.integers(0, 16, size=(N, K // 128)).astype(np.float64))
    x = bf16_normal(2, (K, N, M, 9), (M, K))
    y = oracle.gemm_int4(x, pack_int4(codes), s, z)
    for m in range(M):
        for n in range(N):
            exact = Fraction(0)
            mag = Fraction(0)
            for k in range(K):
                w = (int(codes[n, k]) - frac_f16(z[n, k // 128])) * frac_f16(s[n, k // 128])
                t = w * frac_bf16(x[m, k])
                exact += t
                mag += abs(t)
            # K float64 additions of exact products, each rounding error <= eps * partial magnitude
            bound = float(mag) * K * 2.0 ** -53 + 1e-300
            assert abs(y[m, n] - float(exact)) <= bound, (m, n)


@pytest.mark.parametrize("K,N", [(64, 2), (128, 3)])
def test_bruteforce_exact_fractions_fp4(K, N):
    table = load("fp4_e2m1.json")["table"]
    g = rng(3, K, N)
    codes = g.integers(0, 16, size=(2, N, K)).astype(np.uint8)
    pool = pack_fp4(codes)
    s = bf16_bits_exact(np.exp2(g.integers(-8, -1, size=(2, N, K // 32))).astype(np.float32)
                        * np.float32(1.5))
    x = bf16_normal(3, (K, N, 1), (2, K))
    ids = [1, 0]
    y = oracle.moe_gemv_fp4(x, pool, s, ids)
    for e in range(2):
        for n in range(N):
            exact = Fraction(0)
            mag = Fraction(0)
            for k in range(K):
                v = Fraction(table[str(int(codes[ids[e], n, k]))])
                t = v * frac_bf16(s[ids[e], n, k // 32]) * frac_bf16(x[e, k])
                exact += t
                mag += abs(t)
            assert abs(y[e, n] - float(exact)) <= float(mag) * K * 2.0 ** -53 + 1e-300


# -------------------------------------------------------------- rounding
def test_bf16_rne_matches_torch_cast():
    g = rng(4, 0)
    v = np.concatenate([g.standard_normal(500_000), g.uniform(-1e4, 1e4, 250_000),
                        np.exp2(g.uniform(-60, 60, 250_000)) * g.choice([-1, 1], 250_000)]).astype(np.float32)
    ours = oracle.bf16_bits(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_rne_ties():
    one = 1.0
    assert oracle.round_bf16(one + 2.0 ** -8) == 1.0                      # tie -> even (down)
    assert oracle.round_bf16(one + 3 * 2.0 ** -8) == one + 2.0 ** -6      # tie -> even (up)
    assert oracle.round_bf16(-(one + 3 * 2.0 ** -8)) == -(one + 2.0 ** -6)
    assert oracle.round_bf16(one + 2.0 ** -8 + 2.0 ** -30) == one + 2.0 ** -7  # above the tie
    assert oracle.bf16_bits(np.array([1.0]))[0] == 0x3F80


def test_fp16_decode_and_dequant_exact_in_fp32():
    """(q - z) * s is exact in binary32 for every code, zero and FP16 scale in range."""
    lin = int4_linear(5, (0,), 256, 64)
    W = oracle.dequant_int4(lin["qw"], lin["s"], lin["z"])
    assert np.array_equal(W.astype(np.float32).astype(np.float64), W)
    pool = fp4_pool(5, (1,), 2, 64, 8)
    W4 = oracle.dequant_fp4(pool["qw"], pool["s"])
    assert np.array_equal(W4.astype(np.float32).astype(np.float64), W4)
    assert oracle.f16_to_f64(np.array([0x3C00, 0xC000, 0x1A8E], dtype=np.uint16)).tolist()[:2] == [1.0, -2.0]


def test_generator_distributions():
    """The seeded generators produce the stated ranges (codes uniform over 16)."""
    lin = int4_linear(0, (9,), 3840, 64)
    q = oracle.int4_codes(lin["qw"])
    counts = np.bincount(q.ravel(), minlength=16)
    assert counts.min() > 0.9 * q.size / 16 and counts.max() < 1.1 * q.size / 16
    s = oracle.f16_to_f64(lin["s"])
    z = oracle.f16_to_f64(lin["z"])
    assert s.min() >= 0.0019 and s.max() <= 0.0201
    assert set(np.unique(z).tolist()) <= set(range(16))
    pool = fp4_pool(0, (9,), 4, 4096, 16)
    sv = oracle.bf16_to_f64(pool["s"])
    assert sv.min() >= 2.0 ** -8 * 0.99 and sv.max() <= 2.0 ** -2 * 1.01


# ------------------------------------------------------------ GPTQ layout
def test_gptq_layout_literal_words():
    """GPTQ's K-major words: column n's codes run down the word rows.  Column 0
    holds 0..7 then F..8, column 1 holds 8..F then 7..0, so the repacked rows
    are those literal words side by side."""
    qweight = np.array([[0x76543210, 0xFEDCBA98],
                        [0x89ABCDEF, 0x01234567]], dtype=np.uint32).view(np.int32)
    codes = oracle.gptq_codes(qweight)
    assert codes.tolist() == [list(range(8)) + list(range(15, 7, -1)),
                              list(range(8, 16)) + list(range(7, -1, -1))]
    s = f16_bits([[0.5, 0.25]])
    z = f16_bits([[3.0, 9.0]])
    qw, s2, z2 = oracle.repack_gptq(qweight, s, z)
    assert qw.view(np.uint32).tolist() == [[0x76543210, 0x89ABCDEF], [0xFEDCBA98, 0x01234567]]
    assert s2.tolist() == [[s[0, 0]], [s[0, 1]]] and z2.tolist() == [[z[0, 0]], [z[0, 1]]]


def test_gptq_repack_keeps_every_code_and_the_product():
    """Random GPTQ-layout weights: the repacked codes are the GPTQ codes (checked
    against an independent packer, Python integers), and the product is the one
    written from the GPTQ layout's definition."""
    K, N = 256, 5
    g = rng(41, 0)
    codes = g.integers(0, 16, (N, K))
    qweight = np.zeros((K // 8, N), dtype=np.uint32)
    for n in range(N):
        for k in range(K):
            qweight[k // 8, n] |= int(codes[n, k]) << (4 * (k % 8))
    qweight = qweight.view(np.int32)
    s = f16_bits(g.uniform(0.002, 0.02, (K // 128, N)))
    z = f16_bits(g.integers(0, 16, (K // 128, N)).astype(np.float64))
    assert np.array_equal(oracle.gptq_codes(qweight), codes)
    qw, s2, z2 = oracle.repack_gptq(qweight, s, z)
    assert np.array_equal(qw, pack_int4(codes.astype(np.uint8)))
    x = bf16_normal(41, (1,), (K,))
    W = (codes - np.repeat(oracle.f16_to_f64(z).T, 128, axis=1)) * np.repeat(oracle.f16_to_f64(s).T, 128, axis=1)
    assert np.allclose(oracle.gemv_int4(x, qw, s2, z2), W @ oracle.bf16_to_f64(x), rtol=0, atol=1e-12)
