"""GPU parity of every entry point against the FP64 oracle, through the C ABI.

Small shapes are compared in full; the full-size workloads (3840 x 3840
GEMV, the 336-linear decode step captured in a graph exactly as the bench
times it, the M = 128 prefill shapes, the 262144-row logits GEMV and the
six-expert FP4 MoE pair) are compared in full where the oracle is quick and
on sampled rows otherwise.  Dequantised tiles must match bit for bit.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from parity import check_outputs

pytestmark = pytest.mark.gpu

w4 = pytest.importorskip("gemm_w4_gemv_amd")
from gemm_w4_gemv_amd import host  # noqa: E402
from gemm_w4_gemv_amd.decode import DecodeStep  # noqa: E402

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def run_gemv(lin_np, x_bits):
    t = host.int4_tensors(lin_np)
    x = host.bf16_tensor(x_bits)
    y = torch.empty(t["qw"].shape[0], dtype=torch.bfloat16, device=DEV)
    w4.w4_gemv(x, t["qw"], t["s"], t["z"], y)
    torch.cuda.synchronize()
    return host.bf16_values(y)


def int4_ref(lin_np, x_bits, rows=None):
    """Oracle output and the per-row max |W| of the selected rows."""
    qw, s, z = lin_np["qw"], lin_np["s"], lin_np["z"]
    if rows is not None:
        qw, s, z = qw[rows], s[rows], z[rows]
    W = oracle.dequant_int4(qw, s, z)
    y = oracle.linear(oracle.bf16_to_f64(np.atleast_2d(x_bits)), W)
    return y, np.abs(W).max(axis=1)


def xnorm(x_bits):
    return np.linalg.norm(oracle.bf16_to_f64(np.atleast_2d(x_bits)), axis=1)


# ------------------------------------------------------------ dequant tiles
@pytest.mark.parametrize("N,K", [(37, 256), (64, 3840), (3, 15360), (130, 4096), (1, 128)])
def test_dequant_int4_bit_exact(N, K):
    lin = si.int4_linear(11, (N, K), K, N)
    t = host.int4_tensors(lin)
    f32 = torch.empty(N, K, dtype=torch.float32, device=DEV)
    b16 = torch.empty(N, K, dtype=torch.bfloat16, device=DEV)
    w4.w4_dequant_int4(t["qw"], t["s"], t["z"], f32, b16)
    torch.cuda.synchronize()
    W = oracle.dequant_int4(lin["qw"], lin["s"], lin["z"])
    got = f32.cpu().numpy()
    assert np.array_equal(got.astype(np.float64), W)
    assert np.array_equal(got.view(np.uint32), W.astype(np.float32).view(np.uint32))  # same zero signs too
    assert np.array_equal(host.bits_of(b16), oracle.bf16_bits(W))


@pytest.mark.parametrize("N,K", [(37, 256), (5, 3840), (2, 15360), (1, 8)])
def test_int4_gemv_operands_bit_exact(N, K):
    """The operands of the GEMV, the chain, the two-row GEMV and the small-M
    GEMM, from their own device routines: biased code pairs bf16(128 + q) in
    the oracle's nibble order, and x pairs holding the same two k."""
    lin = si.int4_linear(13, (N, K), K, N) if K % 128 == 0 else {
        "qw": si.rng(13, N, K).integers(0, 2 ** 32, (N, K // 8), dtype=np.uint64).astype(np.uint32).view(np.int32)}
    x_bits = si.bf16_normal(13, (1, N, K), (K,))
    qw = torch.from_numpy(np.ascontiguousarray(lin["qw"]).view(np.int32)).to(DEV)
    codes = torch.empty(N, K // 8, 4, dtype=torch.int32, device=DEV)
    xo = torch.empty(K // 8, 4, dtype=torch.int32, device=DEV)
    w4.w4_int4_gemv_operands(qw, codes, host.bf16_tensor(x_bits), xo)
    torch.cuda.synchronize()
    q = oracle.int4_codes(lin["qw"]).astype(np.float64).reshape(N, K // 8, 8)
    lo = oracle.bf16_bits(128.0 + q[:, :, 0:4]).astype(np.uint32)
    hi = oracle.bf16_bits(128.0 + q[:, :, 4:8]).astype(np.uint32)
    assert np.array_equal(codes.cpu().numpy().view(np.uint32), lo | (hi << 16))
    xb = np.asarray(x_bits, dtype=np.uint16).reshape(K // 8, 8).astype(np.uint32)
    assert np.array_equal(xo.cpu().numpy().view(np.uint32), xb[:, 0:4] | (xb[:, 4:8] << 16))


@pytest.mark.parametrize("N,K", [(33, 64), (128, 4096), (7, 2048), (2, 32)])
def test_dequant_fp4_bit_exact(N, K):
    pool = si.fp4_pool(12, (N, K), 1, K, N)
    qw = torch.from_numpy(pool["qw"][0]).to(DEV)
    s = host.bf16_tensor(pool["s"][0])
    f32 = torch.empty(N, K, dtype=torch.float32, device=DEV)
    b16 = torch.empty(N, K, dtype=torch.bfloat16, device=DEV)
    w4.w4_dequant_fp4(qw, s, f32, b16)
    torch.cuda.synchronize()
    W = oracle.dequant_fp4(pool["qw"][0], pool["s"][0])
    got = f32.cpu().numpy().astype(np.float64)
    assert np.array_equal(got, W)  # +0 == -0: the sign of a zero code cannot change a sum
    bits, ref = host.bits_of(b16), oracle.bf16_bits(W)
    nz = W != 0
    assert np.array_equal(bits[nz], ref[nz])
    assert np.all((bits[~nz] & 0x7FFF) == 0)


# --------------------------------------------------------------- INT4 GEMV
GEMV_SHAPES = [
    (128, 1), (128, 7), (256, 33), (384, 5),      # one group .. a few, tiny N
    (3840, 3840),                                 # the single-GEMV workload
    (4096, 130), (3840, 2051),                    # q/o row length, ragged N
    (8192, 64), (8320, 17),                       # two waves per row, and a ragged slice
    (15360, 67),                                  # four waves per row (down projection)
    (20480, 40), (32768, 9),                      # three and four chunks per lane (K limit)
]


@pytest.mark.parametrize("K,N", GEMV_SHAPES)
def test_gemv_parity(K, N):
    print(f"gemv K={K} N={N}", flush=True)
    lin, x = si.single_gemv(K, N, seed=3)
    y = run_gemv(lin, x)
    y_ref, wmax = int4_ref(lin, x)
    check_outputs(y, y_ref[0], xnorm(x), wmax, f"gemv K={K} N={N}")


def test_gemv_single_workload_seed0():
    """The 3840 x 3840 single GEMV with its own seed-0 inputs, every output."""
    lin, x = si.single_gemv()
    y = run_gemv(lin, x)
    y_ref, wmax = int4_ref(lin, x)
    check_outputs(y, y_ref[0], xnorm(x), wmax, "single gemv")


def test_gemv_logits_sampled():
    """K3840 -> N262144 at full size; oracle on 3000 sampled rows plus both ends."""
    lin, x = si.logits()
    y = run_gemv(lin, x)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(262144 - 8, 262144),
                                     si.rng(5, 1).choice(262144, 3000, replace=False)]))
    y_ref, wmax = int4_ref(lin, x, rows)
    check_outputs(y[rows], y_ref[0], xnorm(x), wmax, "logits")


def test_gemv_deterministic_and_guarded():
    """Two calls give identical bits; memory around the output is untouched."""
    lin, x_bits = si.single_gemv(3840, 1000, seed=4)
    t = host.int4_tensors(lin)
    x = host.bf16_tensor(x_bits)
    pad = 64
    buf = torch.full((1000 + 2 * pad,), 7.0, dtype=torch.bfloat16, device=DEV)
    y = buf[pad:pad + 1000]
    w4.w4_gemv(x, t["qw"], t["s"], t["z"], y)
    first = y.clone()
    w4.w4_gemv(x, t["qw"], t["s"], t["z"], y)
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), y.view(torch.int16))
    assert torch.all(buf[:pad] == 7.0) and torch.all(buf[pad + 1000:] == 7.0)


def test_gemv_empty_is_noop():
    """N = 0 returns W4_OK and launches nothing (the output buffer keeps its contents)."""
    t = host.int4_tensors(si.int4_linear(1, (0,), 256, 4))
    x = host.bf16_tensor(si.bf16_normal(1, (0,), (256,)))
    y = torch.full((8,), 1.0, dtype=torch.bfloat16, device=DEV)
    assert w4.lib.w4_gemv(x.data_ptr(), t["qw"].data_ptr(), t["s"].data_ptr(), t["z"].data_ptr(),
                          y.data_ptr(), 256, 0, 128, None) == 0
    torch.cuda.synchronize()
    assert torch.all(y == 1.0)


# ---------------------------------------------------------- decode-step graph
@pytest.fixture(scope="module")
def decode_step_data():
    """The decode step's 336 linears (device tensors, each with its own seeded
    input) built as the bench builds them, and their host bits for the oracle."""
    from gemm_w4_gemv_amd.decode import decode_linears
    lins = decode_linears()
    host_in = [si.decode_linear(t["layer"], t["index"]) for t in lins]
    yield lins, host_in
    del lins, host_in
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_decode_step_graph_full_size(decode_step_data):
    """All 336 linears of the decode step, captured and replayed as 336 launches.

    Graph replays equal the eager chain bit for bit (replays interleaved with
    other work), and every one of the 336 outputs matches the oracle on
    sampled rows.
    """
    lins, host_in = decode_step_data
    for t in lins:
        t["y"].zero_()
    step = DecodeStep(lins)
    torch.cuda.synchronize()  # the zero fills above ran on the default stream
    step.run_eager()
    torch.cuda.synchronize()
    eager = [t["y"].clone() for t in lins]
    for t in lins:
        t["y"].zero_()
    step.capture()
    for rep in range(3):
        step.replay()
        step.stream.synchronize()
        for t, e in zip(lins, eager):
            assert torch.equal(t["y"].view(torch.int16), e.view(torch.int16)), f"replay {rep} differs"
        for t in lins:  # eager work between replays
            t["y"].fill_(3.0)
        torch.cuda.synchronize()
    step.replay()
    step.stream.synchronize()
    g = si.rng(6, 0)
    for (lin_np, x_bits), t in zip(host_in, lins):
        N = t["N"]
        rows = np.unique(np.concatenate([[0, N - 1], g.choice(N, 24, replace=False)]))
        y = host.bf16_values(t["y"])[rows]
        y_ref, wmax = int4_ref(lin_np, x_bits, rows)
        check_outputs(y, y_ref[0], xnorm(x_bits), wmax, f"layer {t['layer']} {t['name']}")
    step.destroy()


# ------------------------------------------------------------- prefill GEMM
def run_gemm(lin_np, x_bits):
    t = host.int4_tensors(lin_np)
    x = host.bf16_tensor(x_bits)
    M, K = x.shape
    N = t["qw"].shape[0]
    y = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    nbytes = w4.w4_gemm_workspace_bytes(M, K, N)
    ws = torch.empty(max(nbytes, 16) // 4 + 4, dtype=torch.float32, device=DEV) if nbytes else None
    w4.w4_gemm(x, t["qw"], t["s"], t["z"], y, workspace=ws)
    torch.cuda.synchronize()
    return host.bf16_values(y), (nbytes > 0)


@pytest.mark.parametrize("shape_index", [0, 1])
def test_gemm_prefill_full(shape_index):
    """M = 128 prefill at both full shapes, every output (the K15360 shape splits K)."""
    lin, x = si.prefill(shape_index)
    y, split = run_gemm(lin, x)
    assert split == (shape_index == 1)
    y_ref, wmax = int4_ref(lin, x)
    check_outputs(y, y_ref, xnorm(x), wmax, f"prefill {si.PREFILL_SHAPES[shape_index]}")


@pytest.mark.parametrize("M,K,N", [
    (1, 128, 64), (5, 384, 100), (128, 256, 64), (200, 256, 130), (129, 640, 63),
    (128, 1024, 16),     # one tile: K split eight ways
    (64, 15360, 192),    # split K with a ragged N
    (16, 4096, 3840),
])
def test_gemm_parity(M, K, N):
    print(f"gemm M={M} K={K} N={N}", flush=True)
    lin = si.int4_linear(21, (M, K, N), K, N)
    x = si.bf16_normal(21, (M, K, N, 7), (M, K))
    y, _ = run_gemm(lin, x)
    y_ref, wmax = int4_ref(lin, x)
    check_outputs(y, y_ref, xnorm(x), wmax, f"gemm M={M} K={K} N={N}")


@pytest.mark.parametrize("M", [16, 128])
def test_gemm_deterministic(M):
    """Both paths (the small-M path at M = 16, the tiled GEMM with split K at M = 128)."""
    lin, x_bits = si.prefill(1, M=M)
    a, _ = run_gemm(lin, x_bits)
    b, _ = run_gemm(lin, x_bits)
    assert np.array_equal(a.view(np.uint64), b.view(np.uint64))


@pytest.mark.parametrize("M,K,N", [
    (2, 3840, 15360),    # 64-row tiles (the gate / up shape)
    (8, 15360, 3840),    # 16-row tiles, 15 groups per wave (the down shape)
    (16, 1024, 7680),    # 32-row tiles, all 16 rows
    (13, 640, 1000),     # 5 groups for 8 waves (some waves idle), ragged N
    (16, 256, 130),      # 2 groups
    (3, 4096, 262144),   # logits-sized N, 64-row tiles
    (4, 15360, 3840),    # the down shape at M = 4
    (2, 15360, 3840),    # two-row GEMV (M = 2, K <= 16384), four waves per row
    (2, 640, 1000),      # two-row GEMV, one chunk per lane, ragged N
    (2, 8192, 130),      # two-row GEMV, two waves per row
    (2, 16512, 100),     # M = 2 with K past the two-row GEMV's limit: the matrix-core block
])
def test_gemm_small_m(M, K, N):
    """The small-M paths of w4_gemm (2 <= M <= 16): sampled rows against the oracle."""
    print(f"gemm small M={M} K={K} N={N}", flush=True)
    lin = si.int4_linear(23, (M, K, N), K, N)
    x = si.bf16_normal(23, (M, K, N, 7), (M, K))
    assert w4.w4_gemm_workspace_bytes(M, K, N) == 0
    y, _ = run_gemm(lin, x)
    g = np.random.default_rng(1)
    rows = np.unique(np.concatenate([[0, N - 1], np.arange(min(N, 96)), g.choice(N, min(N, 160), replace=False)]))
    y_ref, wmax = int4_ref(lin, x, rows)
    check_outputs(y[:, rows], y_ref, xnorm(x), wmax, f"gemm small M={M} K={K} N={N}")


@pytest.mark.parametrize("K,N", [(3840, 15360), (15360, 3840), (640, 1000), (32768, 64)])
def test_gemm_single_row_is_the_gemv(K, N):
    """w4_gemm at M = 1 gives exactly w4_gemv's output, and that matches the oracle."""
    print(f"gemm M=1 K={K} N={N}", flush=True)
    lin = si.int4_linear(26, (K, N), K, N)
    x = si.bf16_normal(26, (K, N, 7), (1, K))
    assert w4.w4_gemm_workspace_bytes(1, K, N) == 0
    y, _ = run_gemm(lin, x)
    t = host.int4_tensors(lin)
    yv = torch.empty(N, dtype=torch.bfloat16, device=DEV)
    w4.w4_gemv(host.bf16_tensor(x[0]), t["qw"], t["s"], t["z"], yv)
    torch.cuda.synchronize()
    assert np.array_equal(host.bf16_values(yv).view(np.uint64), y[0].view(np.uint64))  # bit for bit
    y_ref, wmax = int4_ref(lin, x)
    check_outputs(y, y_ref, xnorm(x), wmax, f"gemm M=1 K={K} N={N}")


@pytest.mark.parametrize("M", [17, 32])
def test_gemm_just_past_small_m(M):
    """M = 17 and 32 take the tiled GEMM (split K on this shape): every output."""
    K, N = 1024, 3840
    lin = si.int4_linear(24, (M,), K, N)
    x = si.bf16_normal(24, (M, 7), (M, K))
    assert w4.w4_gemm_workspace_bytes(M, K, N) > 0
    y, split = run_gemm(lin, x)
    y_ref, wmax = int4_ref(lin, x)
    check_outputs(y, y_ref, xnorm(x), wmax, f"gemm M={M} K={K} N={N}")


# ------------------------------------------------------------------- FP4 MoE
@pytest.fixture(scope="module")
def moe():
    pools = si.moe_pools()
    dev = [host.fp4_tensors(p) for p in pools]
    return pools, dev


def moe_run(dev_pool, x_bits, ids, shared):
    x = host.bf16_tensor(x_bits)
    idt = torch.from_numpy(np.asarray(ids, dtype=np.int32)).to(DEV)
    N = dev_pool["qw"].shape[1]
    y = torch.empty(len(ids), N, dtype=torch.bfloat16, device=DEV)
    w4.w4_moe_gemv(x, dev_pool["qw"], dev_pool["s"], idt, y)
    return y


def test_moe_full_workload(moe):
    """Six experts x 2 FC at full size: 120 tokens' id sets plus hand-picked ones, every output.

    The oracle output of every (x, expert) pair is computed once; each id set
    is then checked against the rows of its experts (layer-by-layer numeric
    comparison over many expert combinations, as the DeepSeek V4 FP4 page
    recommends in "实践启示" item 2).
    """
    pools, dev = moe
    ids0, x1, x2 = si.moe_inputs(0)
    refs = []
    for fc, (K, N) in enumerate(si.MOE_FC):
        xs = oracle.bf16_to_f64(np.atleast_2d(x1 if fc == 0 else x2))
        y_all = np.empty((si.MOE_POOL, xs.shape[0], N))
        wmax = np.empty((si.MOE_POOL, N))
        for e in range(si.MOE_POOL):
            W = oracle.dequant_fp4(pools[fc]["qw"][e], pools[fc]["s"][e])
            y_all[e] = oracle.linear(xs, W)
            wmax[e] = np.abs(W).max(axis=1)
        refs.append((y_all, wmax, np.linalg.norm(xs, axis=1)))
    id_sets = [si.moe_inputs(t)[0] for t in range(120)]
    id_sets += [np.array([0, 63, 1, 62, 31, 32]), np.array([5, 5, 5, 9, 9, 0]), np.array([63] * 6)]
    for ids in id_sets:
        for fc in range(2):
            y_all, wmax, xn = refs[fc]
            y = host.bf16_values(moe_run(dev[fc], x1 if fc == 0 else x2, ids, fc == 0))
            torch.cuda.synchronize()
            for e, eid in enumerate(ids):
                xi = 0 if fc == 0 else e
                check_outputs(y[e], y_all[eid, xi], xn[xi], wmax[eid], f"fc{fc + 1} slot {e} expert {eid}")


def test_moe_pair_in_one_launch(moe):
    """w4_moe_gemv2: FC1 (shared x) and FC2 (one x per slot) of the full-size
    workload in one launch equal the two separate w4_moe_gemv calls bit for
    bit over 40 tokens' id sets (and so the oracle, checked above), with an
    out-of-pool id turning that slot of both FCs into NaN."""
    pools, dev = moe
    _, x1b, x2b = si.moe_inputs(0)
    x1, x2 = host.bf16_tensor(x1b), host.bf16_tensor(x2b)
    (K1, N1), (K2, N2) = si.MOE_FC
    id_sets = [si.moe_inputs(t)[0] for t in range(40)] + [np.array([3, 64, 7, -1, 0, 63])]
    for t, ids in enumerate(id_sets):
        idt = torch.from_numpy(np.asarray(ids, dtype=np.int32)).to(DEV)
        y1 = torch.full((len(ids), N1), 5.0, dtype=torch.bfloat16, device=DEV)
        y2 = torch.full((len(ids), N2), 5.0, dtype=torch.bfloat16, device=DEV)
        w4.w4_moe_gemv2((x1, dev[0]["qw"], dev[0]["s"], y1), (x2, dev[1]["qw"], dev[1]["s"], y2), idt)
        r1 = torch.empty_like(y1)
        r2 = torch.empty_like(y2)
        w4.w4_moe_gemv(x1, dev[0]["qw"], dev[0]["s"], idt, r1)
        w4.w4_moe_gemv(x2, dev[1]["qw"], dev[1]["s"], idt, r2)
        torch.cuda.synchronize()
        for y, r, name in ((y1, r1, "fc1"), (y2, r2, "fc2")):
            assert same_bits_or_both_nan(y, r), f"token {t} {name}: one launch differs from two"
        if t == len(id_sets) - 1:
            bad = torch.tensor([(e < 0 or e >= si.MOE_POOL) for e in ids], device=DEV)
            for y in (y1, y2):
                assert torch.all(torch.isnan(y.float()[bad])) and torch.all(torch.isfinite(y.float()[~bad]))


def test_moe_invalid_id_gives_nan_and_others_unaffected(moe):
    pools, dev = moe
    _, x1, _ = si.moe_inputs(1)
    ok = host.bf16_values(moe_run(dev[0], x1, [3, 4, 5], True))
    bad = host.bf16_values(moe_run(dev[0], x1, [3, 64, -1], True))
    torch.cuda.synchronize()
    assert np.array_equal(ok[0], bad[0])
    assert np.all(np.isnan(bad[1])) and np.all(np.isnan(bad[2]))


def test_moe_small_shapes_and_determinism():
    for (E, K, N) in [(1, 32, 1), (3, 96, 10), (6, 8192, 33), (2, 15360, 5)]:
        print(f"moe E={E} K={K} N={N}", flush=True)
        pool = si.fp4_pool(31, (E, K, N), 4, K, N)
        d = host.fp4_tensors(pool)
        ids = np.arange(E, dtype=np.int32)[::-1] % 4
        x = si.bf16_normal(31, (E, K, N, 7), (E, K))
        y1 = moe_run(d, x, ids, False)
        y2 = moe_run(d, x, ids, False)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
        y_ref = oracle.moe_gemv_fp4(x, pool["qw"], pool["s"], ids)
        W = oracle.dequant_fp4(pool["qw"], pool["s"])
        for e in range(E):
            check_outputs(host.bf16_values(y1)[e], y_ref[e], xnorm(x[e]), np.abs(W[ids[e]]).max(axis=1),
                          f"moe E={E} K={K} N={N} slot {e}")


# ------------------------------------------------------ persistent decode chain
def test_chain_decode_step_full_size(decode_step_data):
    """The 336 GEMVs, each reading its own input, as one persistent chain launch inside a graph."""
    lins, host_in = decode_step_data
    for t in lins:
        t["y"].zero_()
    step = DecodeStep(lins, mode="chain")
    torch.cuda.synchronize()
    step.run_eager()
    step.stream.synchronize()
    assert step.chain.error() == 0
    eager = [t["y"].clone() for t in lins]
    step.capture()
    for rep in range(3):
        for t in lins:
            t["y"].zero_()
        torch.cuda.synchronize()
        step.replay()
        step.stream.synchronize()
        for t, e in zip(lins, eager):
            assert torch.equal(t["y"].view(torch.int16), e.view(torch.int16)), f"replay {rep} differs"
    assert step.chain.error() == 0
    g = si.rng(7, 0)
    for (lin_np, x_bits), t in zip(host_in, lins):
        N = t["N"]
        rows = np.unique(np.concatenate([[0, N - 1], g.choice(N, 24, replace=False)]))
        y = host.bf16_values(t["y"])[rows]
        y_ref, wmax = int4_ref(lin_np, x_bits, rows)
        check_outputs(y, y_ref[0], xnorm(x_bits), wmax, f"chain layer {t['layer']} {t['name']}")
    step.destroy()


def same_bits_or_both_nan(a, b):
    """Two bf16 tensors hold the same bits wherever either is not NaN (NaN payloads may differ)."""
    both_nan = torch.isnan(a.float()) & torch.isnan(b.float())
    return bool(torch.all((a.view(torch.int16) == b.view(torch.int16)) | both_nan))


# Layers whose linked outputs are all finite: the values grow about 1000x per
# layer (no norms or activations on this path).  Layer 11's o outputs reach
# 1e36, past the input range of the GEMV kernels' FP32 chunk sums of
# (128 + q) x (|x| below about 7e34), so layer 11's gate is not finite.
LINKED_FINITE_LAYERS = 11
# Linears compared with the oracle's own chain: layer 0 and layer 1's q, k, v.
LINKED_ORACLE_CHAIN_LINEARS = 10


def test_chain_linked_decode_step_full_size(decode_step_data):
    """The timed step itself: 336 GEMVs linked as a decoder reads them (o <- q,
    gate/up <- o, down <- gate, next q/k/v <- down), 288 stages, one chain
    launch replayed from a graph, exactly as bench.py builds it.

    * error word 0, and three replays (outputs zeroed before each) identical bit for bit;
    * every one of the 192 dependent boundaries delivered its producer's
      complete output: the same GEMVs run without dependencies (grouped
      schedule), each fed a copy of the input it read, give the same bits
      for all 336 outputs (tile math depends only on the staged x);
    * layers 0..10 (77 linears, every output finite) match the oracle on
      every output, on the very input each GEMV read;
    * the first ten linears (layer 0, then layer 1's q, k, v: all four kinds
      of boundary, down -> q, q -> o, o -> gate/up, gate -> down) also match
      the oracle's own chain, run in order with each intermediate rounded to
      BF16 as the chain stores it.  Further on, the chain (no norms) amplifies
      one-ulp BF16 differences of its inputs by itself: an FP32 evaluation of
      the oracle's own formula drifts 1.5e-3 from the FP64 chain by layer 1's
      down and 4.7e-3 by layer 2's gate, so there the per-input check above is
      the element-by-element one; the drift is printed.
    """
    from gemm_w4_gemv_amd.decode import DECODER_INPUT, decoder_stages, linked_copy
    own, host_in = decode_step_data
    lins = linked_copy(own)
    assert len({t["stage"] for t in lins}) == 288
    assert sum(t["x"] is not own[0]["x"] for t in lins) == 333  # all but layer 0's q, k, v read an output
    step = DecodeStep(lins, mode="chain")
    step.capture()
    outs = None
    for rep in range(3):
        for t in lins:
            t["y"].zero_()
        torch.cuda.synchronize()
        step.replay()
        step.stream.synchronize()
        assert step.chain.error() == 0, f"replay {rep}: error word"
        cur = [t["y"].clone() for t in lins]
        if outs is None:
            outs = cur
        else:
            for i, (a, b) in enumerate(zip(cur, outs)):
                assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"replay {rep} output {i} differs"
    step.destroy()

    # the same GEMVs with no dependencies, each reading a copy of what it read
    clones = [dict(t, x=lt["x"].clone(), y=torch.zeros_like(t["y"]),
                   stage=decoder_stages([t["name"]], [t["layer"]], grouped=True)[0]) for t, lt in zip(own, lins)]
    ind = DecodeStep(clones, mode="chain")
    torch.cuda.synchronize()
    ind.run_eager()
    ind.stream.synchronize()
    assert ind.chain.error() == 0
    for i, (c, o) in enumerate(zip(clones, outs)):
        assert same_bits_or_both_nan(c["y"], o), f"linear {i} (layer {c['layer']} {c['name']}): linked output differs"
    x_read = [host.bits_of(c["x"]) for c in clones[:7 * LINKED_FINITE_LAYERS]]
    ind.destroy()
    del clones

    ref_out = {}
    for i in range(7 * LINKED_FINITE_LAYERS):
        t = own[i]
        layer, name = t["layer"], t["name"]
        lin_np = host_in[i][0]
        src = DECODER_INPUT[name]
        if src == "h":
            x_ref = host_in[0][1] if layer == 0 else ref_out[(layer - 1, "down")]
        else:
            x_ref = ref_out[(layer, src)]
        W = oracle.dequant_int4(lin_np["qw"], lin_np["s"], lin_np["z"])
        y2 = oracle.linear(oracle.bf16_to_f64(np.stack([x_read[i], x_ref])), W)
        wmax = np.abs(W).max(axis=1)
        del W
        y = host.bf16_values(outs[i])
        check_outputs(y, y2[0], xnorm(x_read[i]), wmax, f"linked layer {layer} {name}, oracle on the input read")
        drift = np.linalg.norm(y - y2[1]) / np.linalg.norm(y2[1])
        print(f"linked layer {layer} {name}: relative RMSE against the oracle chain {drift:.2e}", flush=True)
        if i < LINKED_ORACLE_CHAIN_LINEARS:
            check_outputs(y, y2[1], xnorm(x_ref), wmax, f"linked layer {layer} {name}, oracle chain")
        ref_out[(layer, name)] = oracle.bf16_bits(y2[1])


def test_chain_data_dependent():
    """Each stage reads the previous stage's output: q -> o -> gate -> down -> q -> o.

    Outputs are zeroed before every run, so a stage that read its input
    before the previous stage finished writing it would see zeros.  The
    oracle runs the same chain, rounding each intermediate to BF16 as the
    chain stores it.
    """
    shapes = [(3840, 4096), (4096, 3840), (3840, 15360), (15360, 3840), (3840, 4096), (4096, 3840)]
    x0_bits = si.bf16_normal(8, (0,), (3840,))
    gemvs, lin_nps = [], []
    x_dev = host.bf16_tensor(x0_bits)
    for i, (K, N) in enumerate(shapes):
        lin_np = si.int4_linear(8, (1, i), K, N)
        t = host.int4_tensors(lin_np)
        t["x"] = x_dev
        t["y"] = torch.zeros(N, dtype=torch.bfloat16, device=DEV)
        t["stage"] = i
        x_dev = t["y"]
        gemvs.append(t)
        lin_nps.append(lin_np)
    # oracle chain
    refs, x_bits = [], x0_bits
    for lin_np in lin_nps:
        y_ref, wmax = int4_ref(lin_np, x_bits)
        refs.append((y_ref[0], wmax, xnorm(x_bits)))
        x_bits = oracle.bf16_bits(y_ref[0])
    step = DecodeStep(gemvs, mode="chain")
    step.capture()
    for rep in range(4):
        for t in gemvs:
            t["y"].zero_()
        torch.cuda.synchronize()
        step.replay()
        step.stream.synchronize()
        for i, (t, (y_ref, wmax, xn)) in enumerate(zip(gemvs, refs)):
            check_outputs(host.bf16_values(t["y"]), y_ref, xn, wmax, f"dependent stage {i} replay {rep}")
    assert step.chain.error() == 0
    step.destroy()


def test_chain_nan_outputs_and_alternating_copies():
    """A producer whose outputs are NaN does not stall the GEMV that reads them,
    and consecutive runs keep their output copies apart.

    An input holding the all-ones BF16 pattern (a NaN, the same bits as the
    copies' empty mark) makes every output of the first GEMV NaN; the second
    GEMV reads them through the copy and must see them as written.  Runs use
    the two halves of the copies in turn, and the inputs go finite, finite,
    NaN, NaN, finite, finite, so every run finds in its half what the run two
    before wrote, of the other kind, unless that half was marked empty again.
    """
    lin0 = si.int4_linear(9, (0,), 256, 128)
    lin1 = si.int4_linear(9, (1,), 128, 64)
    x_fin = si.bf16_normal(9, (2,), (256,))
    x_nan = x_fin.copy()
    x_nan[[3, 100]] = 0xFFFF
    t0, t1 = host.int4_tensors(lin0), host.int4_tensors(lin1)
    t0["x"] = host.bf16_tensor(x_fin)
    t0["y"] = torch.zeros(128, dtype=torch.bfloat16, device=DEV)
    t1["x"] = t0["y"]
    t1["y"] = torch.zeros(64, dtype=torch.bfloat16, device=DEV)
    t0["stage"], t1["stage"] = 0, 1
    y0_ref, w0 = int4_ref(lin0, x_fin)
    y1_ref, w1 = int4_ref(lin1, oracle.bf16_bits(y0_ref[0]))
    step = DecodeStep([t0, t1], mode="chain")
    for run, bad in enumerate([False, False, True, True, False, False]):
        print(f"chain NaN/copies run {run} nan_input={bad}", flush=True)
        t0["x"].copy_(host.bf16_tensor(x_nan if bad else x_fin))
        t0["y"].zero_()
        t1["y"].zero_()
        torch.cuda.synchronize()
        step.run_eager()
        step.stream.synchronize()
        assert step.chain.error() == 0, f"run {run}"
        y0, y1 = host.bf16_values(t0["y"]), host.bf16_values(t1["y"])
        if bad:
            assert np.all(np.isnan(y0)) and np.all(np.isnan(y1)), f"run {run}"
        else:
            check_outputs(y0, y0_ref[0], xnorm(x_fin), w0, f"NaN/copies run {run} first GEMV")
            check_outputs(y1, y1_ref[0], xnorm(oracle.bf16_bits(y0_ref[0])), w1, f"NaN/copies run {run} second GEMV")
    step.destroy()


@pytest.mark.parametrize("grouped", [False, True], ids=["six_stages_per_layer", "grouped_four_stages"])
def test_chain_two_decoder_layers(grouped):
    """Two full decoder layers wired as a decoder reads them, as the timed decode step is
    (both stage schedules: k, v and up in stages of their own, or grouped with q and gate).

    q, k and v of layer 0 read one input; o reads q's output, gate and up
    read o's, down reads gate's, layer 1's q, k and v read layer 0's down
    output.  GEMVs that do not depend on each other may overlap in the
    kernel; every one of the 14 outputs is compared in full with the oracle
    run in the same order (each intermediate rounded to BF16 as stored).
    The outputs are zeroed before every replay, and the tagged copies keep
    the previous replay's values, so a reader that took a stale copy fails.
    """
    from gemm_w4_gemv_amd.decode import decoder_stages, link_decoder_inputs
    shapes = {n: (K, N) for n, K, N in si.DECODE_LAYER}
    x0_bits = si.bf16_normal(9, (0,), (3840,))
    h0 = host.bf16_tensor(x0_bits)
    gemvs, lin_nps = [], []
    for layer in range(2):
        for idx, (name, K, N) in enumerate(si.DECODE_LAYER):
            lin_np = si.int4_linear(9, (1, layer, idx), K, N)
            t = host.int4_tensors(lin_np)
            t["x"] = h0
            t["y"] = torch.zeros(N, dtype=torch.bfloat16, device=DEV)
            t["name"], t["layer"], t["stage"] = name, layer, decoder_stages([name], [layer], grouped)[0]
            gemvs.append(t)
            lin_nps.append(lin_np)
    link_decoder_inputs(gemvs)
    # oracle in layer order with the same wiring
    outs, refs = {}, []
    for t, lin_np in zip(gemvs, lin_nps):
        src = {"q": "h", "k": "h", "v": "h", "o": "q", "gate": "o", "up": "o", "down": "gate"}[t["name"]]
        if src == "h":
            xb = x0_bits if t["layer"] == 0 else outs[(t["layer"] - 1, "down")]
        else:
            xb = outs[(t["layer"], src)]
        assert xb.shape[0] == shapes[t["name"]][0]
        y_ref, wmax = int4_ref(lin_np, xb)
        refs.append((y_ref[0], wmax, xnorm(xb)))
        outs[(t["layer"], t["name"])] = oracle.bf16_bits(y_ref[0])
    step = DecodeStep(gemvs, mode="chain")
    step.capture()
    for rep in range(3):
        for t in gemvs:
            t["y"].zero_()
        torch.cuda.synchronize()
        step.replay()
        step.stream.synchronize()
        for t, (y_ref, wmax, xn) in zip(gemvs, refs):
            check_outputs(host.bf16_values(t["y"]), y_ref, xn, wmax,
                          f"layer {t['layer']} {t['name']} replay {rep}")
    assert step.chain.error() == 0
    step.destroy()


def test_chain_mixed_shapes():
    """Stages mixing K classes (one, two and four waves per row), ragged N and tiny stages."""
    plan = [[(128, 1), (1024, 7)], [(8192, 100)], [(4096, 1000), (15360, 3), (256, 33)], [(16384, 9)],
            [(3840, 2)], [(512, 4096), (2048, 77)],
            # rows of 260 and 384 chunks: four segments, the last one all padding
            [(8320, 6), (640, 5)], [(12288, 3)]]
    gemvs, refs = [], []
    for st, group in enumerate(plan):
        for j, (K, N) in enumerate(group):
            lin_np, x_bits = si.single_gemv(K, N, seed=40 + st * 8 + j)
            t = host.int4_tensors(lin_np)
            t["x"] = host.bf16_tensor(x_bits)
            t["y"] = torch.zeros(N, dtype=torch.bfloat16, device=DEV)
            t["stage"] = st * 3  # stage numbers need not be consecutive
            gemvs.append(t)
            y_ref, wmax = int4_ref(lin_np, x_bits)
            refs.append((y_ref[0], wmax, xnorm(x_bits), f"stage {st} K={K} N={N}"))
    step = DecodeStep(gemvs, mode="chain")
    for rep in range(2):
        step.run_eager()
        step.stream.synchronize()
        for t, (y_ref, wmax, xn, what) in zip(gemvs, refs):
            check_outputs(host.bf16_values(t["y"]), y_ref, xn, wmax, what)
    assert step.chain.error() == 0
    step.destroy()


def test_chain_many_gemvs_per_stage():
    """Stages of many GEMVs (a tile's GEMV is found by binary search, then by a forward scan):
    40 GEMVs sharing three inputs in one stage, tiny and ragged N, then 24 GEMVs that read
    outputs of the first stage."""
    rng = np.random.default_rng(5)
    xs = {K: si.bf16_normal(60, (K,), (K,)) for K in (128, 1024, 3840)}
    xs_dev = {K: host.bf16_tensor(b) for K, b in xs.items()}
    gemvs, refs, first = [], [], []
    for j in range(40):
        K = (128, 1024, 3840)[j % 3]
        N = int(rng.choice([1, 3, 5, 64, 128, 333, 1024]))
        lin_np, _ = si.single_gemv(K, N, seed=300 + j)
        t = host.int4_tensors(lin_np)
        t["x"], t["y"], t["stage"] = xs_dev[K], torch.zeros(N, dtype=torch.bfloat16, device=DEV), 0
        y_ref, wmax = int4_ref(lin_np, xs[K])
        gemvs.append(t)
        refs.append((y_ref[0], wmax, xnorm(xs[K]), f"stage 0 gemv {j} K={K} N={N}"))
        first.append((t, oracle.bf16_bits(y_ref[0])))
    # second stage: each GEMV reads one first-stage output whose length is a valid K
    # at most six distinct inputs: their staged copies share one stage's LDS budget
    sources = [(t, yb) for t, yb in first if t["y"].numel() in (128, 1024)][:6]
    assert sources
    for j in range(24):
        src, y_bits = sources[j % len(sources)]
        K = src["y"].numel()
        N = int(rng.choice([2, 64, 257]))
        lin_np, _ = si.single_gemv(K, N, seed=400 + j)
        t = host.int4_tensors(lin_np)
        t["x"], t["y"], t["stage"] = src["y"], torch.zeros(N, dtype=torch.bfloat16, device=DEV), 1
        y_ref, wmax = int4_ref(lin_np, y_bits)
        gemvs.append(t)
        refs.append((y_ref[0], wmax, xnorm(y_bits), f"stage 1 gemv {j} K={K} N={N}"))
    step = DecodeStep(gemvs, mode="chain")
    for rep in range(2):
        for t in gemvs:
            t["y"].zero_()
        torch.cuda.synchronize()
        step.run_eager()
        step.stream.synchronize()
        for t, (y_ref, wmax, xn, what) in zip(gemvs, refs):
            check_outputs(host.bf16_values(t["y"]), y_ref, xn, wmax, f"{what} run {rep}")
    assert step.chain.error() == 0
    step.destroy()


def test_chain_wait_limit_reports_error_and_recovers():
    """Failure handling, forced from the host: with a spin limit of 0 the first wait that is not
    already satisfied gives up, so the run records a non-zero error word and still ends (every
    wave leaves its loop); a chain planned again on the same workspace then runs correctly.
    Stage 0 has more tiles than the GPU has compute waves, so every workgroup's stage-1 staging
    must wait for it."""
    lin0, x_bits = si.single_gemv(3840, 15360, seed=71)
    lin1 = si.int4_linear(72, (1,), 15360, 512)
    t0, t1 = host.int4_tensors(lin0), host.int4_tensors(lin1)
    t0["x"], t0["y"], t0["stage"] = host.bf16_tensor(x_bits), torch.zeros(15360, dtype=torch.bfloat16, device=DEV), 0
    t1["x"], t1["y"], t1["stage"] = t0["y"], torch.zeros(512, dtype=torch.bfloat16, device=DEV), 1
    gemvs = [t0, t1]
    nbytes = w4.w4_chain_workspace_bytes(gemvs)
    ws = torch.zeros(nbytes + 256, dtype=torch.uint8, device=DEV)
    off = (-ws.data_ptr()) % 256
    chain = w4.w4_chain_create(gemvs, ws[off:off + nbytes])
    chain.set_spin_limit(0)
    chain.run()
    torch.cuda.synchronize()
    assert chain.error() != 0
    chain.destroy()
    chain = w4.w4_chain_create(gemvs, ws[off:off + nbytes])
    for t in gemvs:
        t["y"].zero_()
    chain.run()
    torch.cuda.synchronize()
    assert chain.error() == 0
    y0_ref, w0max = int4_ref(lin0, x_bits)
    check_outputs(host.bf16_values(t0["y"]), y0_ref[0], xnorm(x_bits), w0max, "stage 0 after recovery")
    y0_bits = oracle.bf16_bits(y0_ref[0])
    y1_ref, w1max = int4_ref(lin1, y0_bits)
    check_outputs(host.bf16_values(t1["y"]), y1_ref[0], xnorm(y0_bits), w1max, "stage 1 after recovery")
    chain.destroy()


def test_read_probe_reads_every_word():
    """The read probe folds every 32-bit word of the range into its workgroup digests exactly once:
    the XOR of the digests equals the XOR of the words (ragged sizes and one past the sink's width)."""
    gen = torch.Generator().manual_seed(11)
    for nbytes in (16, 4096 + 48, 3 * 256 * 16 * 4096 + 32):
        words = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, generator=gen)
        src = words.to(DEV)
        sink = torch.zeros(w4.READ_PROBE_SINK, dtype=torch.int32, device=DEV)
        w4.w4_read_probe(src, sink)
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        want = np.bitwise_xor.reduce(words.numpy().view(np.uint32))
        assert got == want, f"{nbytes} bytes"


# ------------------------------------------------------- FP4 grouped expert GEMM
def run_moe_gemm(dev_pool, x_bits, row_start, ids, max_rows, fill=None):
    R, _ = x_bits.shape
    N = dev_pool["qw"].shape[1]
    y = torch.empty(R, N, dtype=torch.bfloat16, device=DEV)
    if fill is not None:
        y.view(torch.int16).fill_(fill)
    w4.w4_moe_gemm(host.bf16_tensor(x_bits), torch.tensor(row_start, dtype=torch.int32, device=DEV),
                   torch.tensor(ids, dtype=torch.int32, device=DEV), dev_pool["qw"], dev_pool["s"], y, max_rows)
    torch.cuda.synchronize()
    return y


def check_moe_groups(y, x_bits, pool, row_start, ids, cols=None):
    y_ref = oracle.moe_gemm_fp4(x_bits, row_start, ids, pool["qw"], pool["s"], cols=cols)
    for e, expert in enumerate(ids):
        a, b = row_start[e], row_start[e + 1]
        if a >= b:
            continue
        qw_e, s_e = pool["qw"][expert], pool["s"][expert]
        if cols is not None:
            qw_e, s_e = qw_e[cols], s_e[cols]
        wmax = np.abs(oracle.dequant_fp4(qw_e, s_e)).max(axis=1)
        check_outputs(y[a:b], y_ref[a:b], xnorm(x_bits[a:b]), wmax, f"moe_gemm group {e} (expert {expert})")


@pytest.mark.parametrize("fc", [0, 1])
def test_moe_gemm_prefill_groups(fc):
    """Both FC shapes of the 64-expert pools: 6 groups of 3, 0, 16, 5, 1 and 9 rows
    (one empty, one full slab); every output of FC1, 512 sampled columns of FC2."""
    K, N = si.MOE_FC[fc]
    pool = si.moe_pools()[fc]
    dev_pool = host.fp4_tensors(pool)
    sizes = [3, 0, 16, 5, 1, 9]
    row_start = np.concatenate([[0], np.cumsum(sizes)]).tolist()
    ids = si.expert_ids(si.SEED, (50, fc)).tolist()
    x = si.bf16_normal(si.SEED, (50, fc, 7), (row_start[-1], K))
    print(f"moe_gemm fc={fc} K={K} N={N} rows={sizes} ids={ids}", flush=True)
    y = host.bf16_values(run_moe_gemm(dev_pool, x, row_start, ids, max(sizes)))
    cols = None if fc == 0 else np.sort(np.random.default_rng(5).choice(N, 512, replace=False))
    check_moe_groups(y if cols is None else y[:, cols], x, pool, row_start, ids, cols)


def test_moe_gemm_multi_slab_invalid_id_and_untouched_rows():
    """Groups of 40 and 17 rows (three and two slabs of 16), an id outside the pool
    (its rows NaN), rows in no group left as they were; run twice, same bits."""
    P, K, N = 8, 384, 100
    pool = si.fp4_pool(51, (1,), P, K, N)
    dev_pool = host.fp4_tensors(pool)
    row_start = [0, 40, 40, 57, 60]          # groups: 40 rows, empty, 17 rows, 3 rows (bad id); rows 60, 61 in none
    ids = [6, 2, 1, 9]
    x = si.bf16_normal(51, (2,), (62, K))
    print("moe_gemm multi-slab", flush=True)
    y1 = run_moe_gemm(dev_pool, x, row_start, ids, 40, fill=0x1234)
    y2 = run_moe_gemm(dev_pool, x, row_start, ids, 40, fill=0x1234)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    bits = host.bits_of(y1)
    assert np.all(bits[60:] == 0x1234)
    yv = host.bf16_values(y1)
    assert np.all(np.isnan(yv[57:60]))
    check_moe_groups(yv, x, pool, row_start[:4], ids[:3])


@pytest.mark.parametrize("K", [128, 384, 640])
def test_moe_gemm_fewer_steps_than_waves(K):
    """K split over the workgroup's waves in steps of 128 k with fewer steps than
    waves (1 or 3) or a ragged split (5): waves with no steps add nothing."""
    P, N = 5, 80
    pool = si.fp4_pool(54, (K,), P, K, N)
    dev_pool = host.fp4_tensors(pool)
    row_start, ids = [0, 7, 7, 30], [4, 1, 0]  # 7 rows, an empty group, 23 rows (two slabs)
    x = si.bf16_normal(54, (K, 2), (30, K))
    print(f"moe_gemm K={K}", flush=True)
    y = host.bf16_values(run_moe_gemm(dev_pool, x, row_start, ids, 23))
    check_moe_groups(y, x, pool, row_start, ids)


def test_moe_gemm2_pair_equals_two_launches():
    """w4_moe_gemm2: both FC shapes of the 64-expert pools over the same groups
    (6 groups of 16 rows, as bench.py times them, then ragged groups with an empty
    one and an id outside the pool) in one launch equal two w4_moe_gemm calls bit
    for bit, NaNs included; FC1's outputs are checked against the oracle."""
    pools = si.moe_pools()
    dev = [host.fp4_tensors(p) for p in pools]
    (K1, N1), (K2, N2) = si.MOE_FC
    for case, (sizes, ids) in enumerate([([16] * 6, si.expert_ids(si.SEED, (53, 0)).tolist()),
                                         ([5, 0, 16, 2, 9, 1], [7, 3, 70, 0, 63, 12])]):
        row_start = np.concatenate([[0], np.cumsum(sizes)]).tolist()
        R, mr = row_start[-1], max(sizes)
        print(f"moe_gemm2 case {case}: rows={sizes} ids={ids}", flush=True)
        x1 = si.bf16_normal(si.SEED, (53, case, 1), (R, K1))
        x2 = si.bf16_normal(si.SEED, (53, case, 2), (R, K2))
        rs = torch.tensor(row_start, dtype=torch.int32, device=DEV)
        idt = torch.tensor(ids, dtype=torch.int32, device=DEV)
        xt1, xt2 = host.bf16_tensor(x1), host.bf16_tensor(x2)
        y1 = torch.full((R, N1), 0.5, dtype=torch.bfloat16, device=DEV)
        y2 = torch.full((R, N2), 0.5, dtype=torch.bfloat16, device=DEV)
        w4.w4_moe_gemm2((xt1, dev[0]["qw"], dev[0]["s"], y1), (xt2, dev[1]["qw"], dev[1]["s"], y2), rs, idt, mr)
        r1, r2 = torch.full_like(y1, 0.5), torch.full_like(y2, 0.5)
        w4.w4_moe_gemm(xt1, rs, idt, dev[0]["qw"], dev[0]["s"], r1, mr)
        w4.w4_moe_gemm(xt2, rs, idt, dev[1]["qw"], dev[1]["s"], r2, mr)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), r1.view(torch.int16)), f"case {case}: FC1 differs from its own launch"
        assert torch.equal(y2.view(torch.int16), r2.view(torch.int16)), f"case {case}: FC2 differs from its own launch"
        valid = [e for e, i in enumerate(ids) if 0 <= i < si.MOE_POOL]
        yv1 = host.bf16_values(y1)
        for e in range(len(ids)):
            if e not in valid:
                assert np.all(np.isnan(yv1[row_start[e]:row_start[e + 1]]))
        keep = [e for e in valid]
        rs_v = [0]
        rows = []
        for e in keep:
            rows.extend(range(row_start[e], row_start[e + 1]))
            rs_v.append(len(rows))
        check_moe_groups(yv1[rows], x1[rows], pools[0], rs_v, [ids[e] for e in keep])
    # a FC with N = 0 touches none of its buffers: the pair equals the other FC's own
    # launch (torch hands out NULL for empty tensors, so the C-ABI is called directly)
    y1.fill_(0.5)
    y2.fill_(0.25)
    ptr = lambda t: t.data_ptr()
    f1 = w4.MoeGemmFc(ptr(xt1), ptr(dev[0]["qw"]), ptr(dev[0]["s"]), ptr(y1), K1, N1)
    f0 = w4.MoeGemmFc(ptr(xt2), ptr(dev[1]["qw"]), ptr(dev[1]["s"]), ptr(y2), K2, 0)
    stream = torch.cuda.current_stream().cuda_stream
    assert w4.lib.w4_moe_gemm2(ctypes.byref(f1), ctypes.byref(f0), ptr(rs), ptr(idt), R, len(ids), mr,
                               si.MOE_POOL, stream) == 0
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), r1.view(torch.int16)), "FC1 alone differs from its own launch"
    assert torch.all(y2 == 0.25), "the FC with N = 0 wrote its output"


def test_moe_gemm_row_table_clamped():
    """Group bounds outside [0, R] are clamped on the device: a start below 0 reads
    as 0, an end past R as R, and an end below its start as an empty group."""
    P, K, N = 4, 256, 48
    pool = si.fp4_pool(52, (1,), P, K, N)
    dev_pool = host.fp4_tensors(pool)
    R = 20
    x = si.bf16_normal(52, (2,), (R, K))
    print("moe_gemm clamped row table", flush=True)
    y = run_moe_gemm(dev_pool, x, [-5, 6, 6, 1000, 3], [3, 1, 0, 2], 16, fill=0x1234)
    yv = host.bf16_values(y)
    # effective groups: rows 0..5 -> expert 3; empty; rows 6..19 -> expert 0; empty (end below start)
    check_moe_groups(yv, x, pool, [0, 6, 6, 20], [3, 1, 0])


def test_graph_replays_of_gemm_paths_equal_eager():
    """The tiled GEMM (split K), the small-M GEMM, the grouped FP4 GEMM and the
    grouped pair (w4_moe_gemm2) captured in one HIP graph: five replays, with eager
    work and synchronisations between them and the outputs cleared before each, all
    equal the eager results bit for bit."""
    stream = torch.cuda.Stream()
    lin = si.int4_linear(25, (1,), 2048, 192)
    t = host.int4_tensors(lin)
    xb = host.bf16_tensor(si.bf16_normal(25, (2,), (128, 2048)))
    xs = host.bf16_tensor(si.bf16_normal(25, (3,), (5, 2048)))
    yb = torch.empty(128, 192, dtype=torch.bfloat16, device=DEV)
    ys = torch.empty(5, 192, dtype=torch.bfloat16, device=DEV)
    nbytes = w4.w4_gemm_workspace_bytes(128, 2048, 192)
    assert nbytes > 0
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device=DEV)
    pool = host.fp4_tensors(si.fp4_pool(25, (4,), 6, 512, 80))
    xm = host.bf16_tensor(si.bf16_normal(25, (5,), (30, 512)))
    ym = torch.empty(30, 80, dtype=torch.bfloat16, device=DEV)
    rs = torch.tensor([0, 7, 7, 23, 30], dtype=torch.int32, device=DEV)
    ids = torch.tensor([5, 0, 2, 3], dtype=torch.int32, device=DEV)
    pool2 = host.fp4_tensors(si.fp4_pool(25, (6,), 6, 256, 144))
    xm2 = host.bf16_tensor(si.bf16_normal(25, (7,), (30, 256)))
    yp1 = torch.empty(30, 80, dtype=torch.bfloat16, device=DEV)
    yp2 = torch.empty(30, 144, dtype=torch.bfloat16, device=DEV)

    def body():
        w4.w4_gemm(xb, t["qw"], t["s"], t["z"], yb, workspace=ws, stream=stream)
        w4.w4_gemm(xs, t["qw"], t["s"], t["z"], ys, stream=stream)
        w4.w4_moe_gemm(xm, rs, ids, pool["qw"], pool["s"], ym, 16, stream=stream)
        w4.w4_moe_gemm2((xm, pool["qw"], pool["s"], yp1), (xm2, pool2["qw"], pool2["s"], yp2), rs, ids, 16,
                        stream=stream)

    outs = (yb, ys, ym, yp1, yp2)
    with torch.cuda.stream(stream):
        body()
    stream.synchronize()
    ref = [y.clone() for y in outs]
    assert torch.equal(yp1.view(torch.int16), ym.view(torch.int16))  # the pair's FC1 is w4_moe_gemm's call
    torch.cuda.synchronize()
    w4.w4_graph_begin(stream)
    try:
        body()
    finally:
        g = w4.w4_graph_end(stream)
    try:
        for rep in range(5):
            for y in outs:
                y.zero_()
            torch.cuda.synchronize()
            g.replay(stream)
            stream.synchronize()
            for y, r in zip(outs, ref):
                assert torch.equal(y.view(torch.int16), r.view(torch.int16)), f"replay {rep}"
            junk = torch.randn(1 << 20, device=DEV) * 2  # unrelated eager work between replays
            torch.cuda.synchronize()
            del junk
    finally:
        g.destroy()


@pytest.mark.parametrize("M,K,N", [
    (128, 32768, 64),    # the largest K: scales and zeros of 256 groups staged in LDS, K split
    (4, 32768, 80),      # the same K through the small-M path
    (130, 32768, 70),    # two row tiles, ragged N
])
def test_gemm_max_k(M, K, N):
    print(f"gemm max K M={M} K={K} N={N}", flush=True)
    lin = si.int4_linear(26, (M, K, N), K, N)
    x = si.bf16_normal(26, (M, K, N, 7), (M, K))
    y, _ = run_gemm(lin, x)
    y_ref, wmax = int4_ref(lin, x)
    check_outputs(y, y_ref, xnorm(x), wmax, f"gemm M={M} K={K} N={N}")


def test_moe_gemm_max_k():
    """The largest K of w4_moe_gemm (8192: scales of 256 groups per row staged in LDS)."""
    P, K, N = 3, 8192, 40
    pool = si.fp4_pool(53, (1,), P, K, N)
    dev_pool = host.fp4_tensors(pool)
    x = si.bf16_normal(53, (2,), (21, K))
    row_start, ids = [0, 9, 21], [2, 0]
    print("moe_gemm max K", flush=True)
    y = host.bf16_values(run_moe_gemm(dev_pool, x, row_start, ids, 12))
    check_moe_groups(y, x, pool, row_start, ids)
