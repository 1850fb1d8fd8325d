"""The C ABI: the library loads, exports every symbol the header declares, and
rejects invalid arguments with the documented status before any HIP call.

CPU only.  The pointers passed here are fake addresses; every call is built
to fail validation (or to be an empty problem), so nothing is ever launched.
"""
from __future__ import annotations

import ctypes
import json
import pathlib
import re

import pytest

import gemm_w4_gemv_amd as w4
from gemm_w4_gemv_amd import roofline

ROOT = pathlib.Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "w4.h"
lib = w4.lib

OK, NULL, SHAPE, UNSUP, ALIGN, WS, ALIAS, ARG = 0, 1, 2, 3, 4, 5, 6, 7

# fake, distinct, 256-aligned addresses (never dereferenced)
X, QW, S, Z, Y, WSP, IDS = (0x7F0000000000 + i * 0x10000000 for i in range(7))


def declared_functions():
    text = HEADER.read_text()
    return sorted(set(re.findall(r"W4_API\s+[\w\s\*]+?\b(w4_\w+)\s*\(", text)))


def test_header_symbols_exported_and_bound():
    names = declared_functions()
    assert len(names) == 28, names
    for name in names:
        assert hasattr(lib, name), f"libw4.so does not export {name}"
        assert name in w4.SIGNATURES, f"binding has no signature for {name}"
    assert set(w4.SIGNATURES) == set(names)


def test_abi_version_and_status_strings():
    assert lib.w4_abi_version() == 1
    for code, name in w4.STATUS.items():
        assert w4.w4_status_string(code) == name
    assert w4.w4_status_string(99) == "W4_ERR_UNKNOWN"


def test_header_constants_match_binding():
    text = HEADER.read_text()
    assert f"W4_GEMV_MAX_K {w4.GEMV_MAX_K}" in text
    assert f"W4_INT4_GROUP {w4.INT4_GROUP}" in text
    assert f"W4_FP4_GROUP {w4.FP4_GROUP}" in text


def gemv(x=X, qw=QW, s=S, z=Z, y=Y, K=3840, N=3840, g=128):
    return lib.w4_gemv(x, qw, s, z, y, K, N, g, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(x=None), NULL), (dict(qw=None), NULL), (dict(s=None), NULL), (dict(z=None), NULL), (dict(y=None), NULL),
    (dict(K=100), SHAPE), (dict(K=0), SHAPE), (dict(K=-128), SHAPE), (dict(N=-1), SHAPE),
    (dict(K=32768 + 128), SHAPE), (dict(K=32768, N=262144 + 1), SHAPE),
    (dict(g=64), UNSUP), (dict(g=32), UNSUP),
    (dict(qw=QW + 8), ALIGN), (dict(x=X + 2), ALIGN), (dict(s=S + 1), ALIGN), (dict(y=Y + 1), ALIGN),
    (dict(y=QW + 1024), ALIAS), (dict(y=X), ALIAS), (dict(y=S + 2), ALIAS),
])
def test_gemv_validation(kwargs, status):
    assert gemv(**kwargs) == status
    assert "w4_gemv" in w4.w4_last_error()


def test_gemv_empty_problem_launches_nothing():
    assert gemv(N=0) == OK


def test_gemm_validation():
    need = lib.w4_gemm_workspace_bytes(128, 15360, 3840, 128)
    assert need > 0
    args = lambda **k: (k.get("x", X), QW, S, Z, k.get("y", Y), k.get("M", 128), k.get("K", 15360),
                        k.get("N", 3840), k.get("g", 128), k.get("ws", WSP), k.get("wsb", need), None)
    assert lib.w4_gemm(*args(ws=None)) == WS
    assert lib.w4_gemm(*args(wsb=need - 1)) == WS
    assert lib.w4_gemm(*args(ws=WSP + 4)) == ALIGN
    assert lib.w4_gemm(*args(M=-1)) == SHAPE
    assert lib.w4_gemm(*args(K=15360 + 64)) == SHAPE
    assert lib.w4_gemm(*args(K=32768 + 128)) == SHAPE     # past W4_GEMM_MAX_K
    assert lib.w4_gemm(*args(M=65537, K=32768)) == SHAPE  # activations past 32-bit offsets
    assert lib.w4_gemm(*args(g=256)) == UNSUP
    assert lib.w4_gemm(*args(ws=Y)) == ALIAS          # workspace overlaps y
    assert lib.w4_gemm(*args(ws=QW)) == ALIAS         # workspace overlaps the weights
    assert lib.w4_gemm(*args(M=0)) == OK              # empty problem
    assert "w4_gemm" in w4.w4_last_error() or True


def test_gemm_workspace_sizes():
    # 128 x 15360 output: 240 tiles of 128 x 64 fill the GPU without a K split
    assert lib.w4_gemm_workspace_bytes(128, 3840, 15360, 128) == 0
    # 128 x 3840 output: 60 tiles, K is split four ways
    assert lib.w4_gemm_workspace_bytes(128, 15360, 3840, 128) == 4 * 128 * 3840 * 4
    assert lib.w4_gemm_workspace_bytes(128, 15360, 3840, 64) == 0
    assert lib.w4_gemm_workspace_bytes(0, 15360, 3840, 128) == 0


def test_moe_validation():
    def call(**k):
        return lib.w4_moe_gemv(k.get("x", X), k.get("stride", 0), k.get("qw", QW), S, k.get("ids", IDS),
                               k.get("y", Y), k.get("E", 6), k.get("ne", 64), k.get("K", 4096), k.get("N", 2048), None)
    assert call(ids=None) == NULL
    assert call(ne=0) == ARG
    assert call(stride=3) == ARG
    assert call(stride=-8) == ARG
    assert call(K=48) == SHAPE
    assert call(E=-1) == SHAPE
    assert call(qw=QW + 4) == ALIGN
    assert call(ids=IDS + 2) == ALIGN
    assert call(y=IDS) == ALIAS
    assert call(E=0) == OK


def test_moe_gemm_validation():
    RS = IDS + 0x1000

    def call(**k):
        return lib.w4_moe_gemm(k.get("x", X), k.get("rs", RS), k.get("ids", IDS), k.get("qw", QW), k.get("s", S),
                               k.get("y", Y), k.get("R", 96), k.get("E", 6), k.get("mr", 16), k.get("ne", 64),
                               k.get("K", 4096), k.get("N", 2048), None)
    assert call(rs=None) == NULL
    assert call(ids=None) == NULL
    assert call(ne=0) == ARG
    assert call(K=4096 + 32) == SHAPE          # not a multiple of 128
    assert call(K=8192 + 128) == SHAPE         # past W4_MOE_GEMM_MAX_K
    assert call(R=-1) == SHAPE
    assert call(mr=-1) == SHAPE
    assert call(R=(1 << 31) // 4096) == SHAPE  # activations past 32-bit offsets
    assert call(qw=QW + 8) == ALIGN
    assert call(s=S + 4) == ALIGN              # scales need 8-byte alignment
    assert call(rs=RS + 2) == ALIGN
    assert call(y=RS) == ALIAS
    assert call(y=X + 64) == ALIAS
    assert call(E=0) == OK and call(R=0) == OK and call(mr=0) == OK and call(N=0) == OK
    assert "w4_moe_gemm" in w4.w4_last_error()


def test_graph_and_dequant_validation():
    h = ctypes.c_void_p()
    assert lib.w4_graph_begin(None) == ARG
    assert lib.w4_graph_end(None, ctypes.byref(h)) == ARG and h.value is None
    assert lib.w4_graph_end(X, None) == ARG
    assert lib.w4_graph_replay(None, X) == ARG
    lib.w4_graph_destroy(None)  # no-op
    assert lib.w4_dequant_int4(QW, S, Z, None, None, 256, 4, 128, None) == NULL
    assert lib.w4_dequant_int4(QW, S, Z, Y, None, 200, 4, 128, None) == SHAPE
    assert lib.w4_dequant_fp4(QW, S, None, None, 64, 4, None) == NULL
    assert lib.w4_dequant_fp4(QW, S, Y, None, 48, 4, None) == SHAPE
    op = lib.w4_int4_gemv_operands
    assert op(None, None, Y, None, 256, 4, None) == NULL
    assert op(QW, X, Y, None, 256, 4, None) == NULL  # x without x_out
    assert op(QW, None, Y, WSP, 256, 4, None) == NULL  # x_out without x
    assert op(QW, None, Y, None, 12, 4, None) == SHAPE
    assert op(QW, None, Y, None, 256, -1, None) == SHAPE
    assert op(QW + 2, None, Y, None, 256, 4, None) == ALIGN
    assert op(QW, X, QW + 64, WSP, 256, 4, None) == ALIAS  # codes_out over the weights
    assert op(QW, X, Y, Y + 64, 256, 4, None) == ALIAS  # the two outputs overlap
    assert op(QW, X, Y, WSP, 256, 0, None) == OK  # empty: nothing launched


def test_gemm_noalloc_validation():
    na = lib.w4_gemm_noalloc
    assert na(None, QW, S, Z, Y, 128, 3840, 64, 128, None) == NULL
    assert na(X, QW, S, Z, Y, 128, 200, 64, 128, None) == SHAPE
    assert na(X, QW, S, Z, Y, -1, 256, 64, 128, None) == SHAPE
    assert na(X, QW, S, Z, Y, 128, 256, 64, 64, None) == UNSUP
    assert na(X + 8, QW, S, Z, Y, 128, 256, 64, 128, None) == ALIGN
    assert na(X, QW, S, Z, X + 64, 128, 256, 64, 128, None) == ALIAS
    assert na(X, QW, S, Z, Y, 0, 256, 64, 128, None) == OK  # empty: nothing launched, no scratch looked up
    assert f"W4_GEMM_NOALLOC_SCRATCH_BYTES ({w4.GEMM_NOALLOC_SCRATCH_BYTES >> 20}ull << 20)" in HEADER.read_text()


def test_chain_spin_limit_validation():
    assert lib.w4_chain_set_spin_limit(None, 0) == ARG


def test_read_probe_validation():
    assert lib.w4_read_probe(X, 1024, None, None) == NULL
    assert lib.w4_read_probe(None, 1024, Y, None) == NULL
    assert lib.w4_read_probe(X, 1000, Y, None) == SHAPE
    assert lib.w4_read_probe(X + 8, 1024, Y, None) == ALIGN
    assert lib.w4_read_probe(X, 1024, Y + 2, None) == ALIGN
    assert lib.w4_read_probe(X, 1 << 20, X + 4096, None) == ALIAS


def test_byte_model_against_pages():
    """Decode-step storage of 4-bit codes + FP16 scale/zero per 128, vs the pages' total."""
    g = json.loads((ROOT / "tests" / "golden" / "w4a16_bytes.json").read_text())
    from seeded_inputs import DECODE_LAYER, DECODE_LAYERS
    total = DECODE_LAYERS * sum(roofline.int4_weight_bytes(K, N) for _, K, N in DECODE_LAYER)
    assert total == g["expected_bytes_here"]
    assert abs(total - g["pages_bytes"]) / g["pages_bytes"] < g["max_relative_gap"]
    # the alternatives fit the pages' figure worse: scale only, or zeros packed in 4 bits
    scale_only = DECODE_LAYERS * sum(N * K // 2 + 2 * N * (K // 128) for _, K, N in DECODE_LAYER)
    packed_zero = DECODE_LAYERS * sum(N * K // 2 + 2 * N * (K // 128) + N * (K // 128) // 2
                                      for _, K, N in DECODE_LAYER)
    gap = lambda v: abs(v - g["pages_bytes"])
    assert gap(total) < gap(scale_only) and gap(total) < gap(packed_zero)
    assert round(g["pages_bytes"] / 2 ** 30, 3) == g["pages_gib"]


def test_chain_validation():
    def desc(**k):
        d = dict(x=X, qw=QW, s=S, z=Z, y=Y, K=3840, N=4096, stage=0, reserved=0)
        d.update(k)
        return w4.GemvDesc(d["x"], d["qw"], d["s"], d["z"], d["y"], d["K"], d["N"], d["stage"], d["reserved"])

    def create(descs, ws=WSP, nbytes=1 << 20):
        arr = (w4.GemvDesc * len(descs))(*descs)
        h = ctypes.c_void_p()
        st = lib.w4_chain_create(arr, len(descs), ws, nbytes, ctypes.byref(h))
        assert h.value is None
        return st

    def ws_bytes(descs):
        arr = (w4.GemvDesc * max(len(descs), 1))(*descs)
        return lib.w4_chain_workspace_bytes(ctypes.cast(arr, ctypes.c_void_p), len(descs))

    one = ws_bytes([desc()])
    assert one > 128 * 1024
    assert ws_bytes([]) == 0
    assert ws_bytes([desc(K=100)]) == 0                        # invalid descriptors
    # q (stage 0) -> o (stage 1) reading q's output exactly: the workspace
    # also holds two BF16 copies of q's 4096 outputs (one per run parity)
    q = desc(K=3840, N=4096, y=Y)
    o = desc(x=Y, K=4096, N=3840, y=Y + 65536, stage=1)
    assert ws_bytes([q, o]) >= ws_bytes([q, desc(N=3840, y=Y + 65536, stage=1)]) + 4096 * 4
    assert create([desc()], ws=None) == NULL
    assert create([desc(K=16384 + 128)]) == SHAPE          # the chain's K limit
    assert create([desc(K=16384, N=1 << 20)]) == SHAPE     # N * K / 2 over the 32-bit offsets' range
    assert ws_bytes([desc(K=16384, N=(1 << 19) - 1, qw=0x7E0000000000)]) > 0   # just under it (weights far from the rest)
    assert create([desc(K=100)]) == SHAPE
    assert create([desc(x=X + 8)]) == ALIGN
    assert create([desc()], ws=WSP + 128) == ALIGN           # workspace needs 256-byte alignment
    assert create([desc(reserved=1)]) == ARG
    assert create([desc(stage=1), desc(stage=0, y=Y + 65536)]) == ARG   # stages must not decrease
    assert create([desc(stage=-1)]) == ARG
    assert create([desc(), desc(y=Y + 2)]) == ALIAS          # two outputs overlap
    assert create([desc(y=QW + 64)]) == ALIAS                 # output over a weight
    assert create([desc(), desc(x=Y, y=Y + 65536)]) == ALIAS  # same-stage read of an output
    assert create([desc()], nbytes=64) == WS
    # an input written by an earlier stage must be exactly that output
    assert create([desc(N=4096, y=Y), desc(x=Y + 64, K=3840, N=3840, y=Y + 65536, stage=1)]) == UNSUP
    assert create([desc(N=4096, y=Y), desc(x=Y, K=3840, N=3840, y=Y + 65536, stage=1)]) == UNSUP  # K != N
    # a later output over an earlier input needs a path of inputs back to that GEMV's output
    a0 = desc(x=X, K=3840, N=3840, y=Y, stage=0)
    b1 = desc(x=Y + 65536, K=3840, N=3840, y=X, stage=1)      # overwrites a0's input, does not read a0's output
    assert create([a0, b1]) == UNSUP
    assert ws_bytes([a0, b1]) == 0
    c1 = desc(x=Y, K=3840, N=3840, y=X, stage=1)              # reads a0's output: allowed
    assert ws_bytes([a0, c1]) > 0
    h = ctypes.c_void_p()
    assert lib.w4_chain_create(None, 1, WSP, 1 << 20, ctypes.byref(h)) == NULL
    assert lib.w4_chain_create((w4.GemvDesc * 1)(desc()), 0, WSP, 1 << 20, ctypes.byref(h)) == ARG
    assert lib.w4_chain_run(None, None) == ARG
    lib.w4_chain_destroy(None)


# ------------------------------------------------------------- launch tuning
TABLE = ROOT / "gemm_w4_gemv_amd" / "csrc" / "tune_table.inc"
TUNE_IDS = {"W4_TUNE_GEMV": 0, "W4_TUNE_GEMV_ROWS2": 1, "W4_TUNE_GEMM_SMALL_M": 2, "W4_TUNE_GEMM": 3,
            "W4_TUNE_MOE_GEMV": 4}


def table_entries():
    rows = re.findall(r"\{(W4_TUNE_\w+),\s*(\d+),\s*(\d+),\s*(\d+),\s*(\d+)\}", TABLE.read_text())
    return [(TUNE_IDS[k], int(m), int(kk), int(n), int(p)) for k, m, kk, n, p in rows]


def test_tune_ids_match_header():
    text = HEADER.read_text()
    for name, i in TUNE_IDS.items():
        assert f"#define {name} {i}" in text
    assert sorted(w4.TUNE_KERNELS.values()) == sorted(TUNE_IDS.values())


def test_tune_table_drives_the_launchers():
    """Every measured entry is what the launchers use for its shape."""
    entries = table_entries()
    assert entries, "the tuning table is empty"
    for kernel, M, K, N, param in entries:
        assert lib.w4_tune_param(kernel, M if M else 1, K, N) == param, (kernel, M, K, N)


def test_tune_rules_outside_the_table():
    # the rules: GEMV rows per wave, small-M width, prefill K splits, FP4 GEMV rows per wave
    assert lib.w4_tune_param(0, 1, 256, 7) == 1
    assert lib.w4_tune_param(0, 1, 4096, 1 << 20) == 8
    assert lib.w4_tune_param(2, 4, 256, 130) == 1
    assert lib.w4_tune_param(2, 4, 256, 64 * 240) == 4
    assert lib.w4_tune_param(3, 128, 2048, 64) == 16  # one tile: 16 splits (= K / 128)
    assert lib.w4_tune_param(3, 128, 256, 64) == 2   # at most one group per split
    assert lib.w4_tune_param(3, 1024, 3840, 1 << 14) == 1
    assert lib.w4_tune_param(4, 6, 256, 1 << 16) == 8
    assert lib.w4_tune_param(4, 6, 256, 1 << 11) == 4
    assert lib.w4_tune_param(9, 1, 256, 64) == -1


def test_tune_force_and_reset():
    assert lib.w4_tune_force(5, 1) == ARG
    assert lib.w4_tune_force(-1, 1) == ARG
    assert lib.w4_tune_force(0, 3) == ARG
    assert lib.w4_tune_force(3, 17) == ARG
    before = lib.w4_tune_param(3, 128, 2048, 64)
    try:
        assert lib.w4_tune_force(3, 5) == OK
        assert lib.w4_tune_param(3, 128, 2048, 64) == 5
        assert lib.w4_tune_param(3, 128, 256, 64) == 2  # still at most one group per split
        assert lib.w4_gemm_workspace_bytes(128, 2048, 64, 128) == 5 * 128 * 64 * 4
        assert lib.w4_tune_force(0, 8) == OK
        assert lib.w4_tune_param(0, 1, 3840, 3840) == 8
    finally:
        assert lib.w4_tune_force(3, 0) == OK
        assert lib.w4_tune_force(0, 0) == OK
    assert lib.w4_tune_param(3, 128, 2048, 64) == before


def test_repack_gptq_validation():
    rp = lib.w4_repack_gptq
    assert rp(None, S, Z, QW, WSP, Y, 256, 64, 128, None) == NULL
    assert rp(X, S, Z, QW, WSP, Y, 200, 64, 128, None) == SHAPE
    assert rp(X, S, Z, QW, WSP, Y, 256, -1, 128, None) == SHAPE
    assert rp(X, S, Z, QW, WSP, Y, 256, 64, 64, None) == UNSUP
    assert rp(X + 2, S, Z, QW, WSP, Y, 256, 64, 128, None) == ALIGN
    assert rp(X, S, Z, X + 64, WSP, Y, 256, 64, 128, None) == ALIAS  # qw over qw_kn
    assert rp(X, S, Z, QW, QW + 64, Y, 256, 64, 128, None) == ALIAS  # s over qw
    assert rp(X, S, Z, QW, WSP, Y, 256, 0, 128, None) == OK  # empty: nothing launched


def test_moe_gemm2_validation():
    RS = IDS + 0x1000

    def fc(x=X, qw=QW, s=S, y=Y, K=4096, N=2048):
        return w4.MoeGemmFc(x, qw, s, y, K, N)
    g2 = lib.w4_moe_gemm2
    ok1 = fc()
    ok2 = fc(x=X + 0x1000000, qw=QW + 0x1000000, s=S + 0x1000000, y=Y + 0x1000000, K=2048, N=4096)

    def call(f1=ok1, f2=ok2, rs=RS, ids=IDS, R=96, E=6, mr=16, ne=64):
        return g2(ctypes.byref(f1) if f1 is not None else None, ctypes.byref(f2) if f2 is not None else None,
                  rs, ids, R, E, mr, ne, None)
    assert call(f2=None) == NULL
    assert call(rs=None) == NULL and call(ids=None) == NULL
    assert call(f1=fc(s=None)) == NULL
    assert call(f2=fc(K=2048 + 32)) == SHAPE       # not a multiple of 128
    assert call(f1=fc(K=8192 + 128)) == SHAPE      # past W4_MOE_GEMM_MAX_K
    assert call(f1=fc(N=-1)) == SHAPE and call(R=-1) == SHAPE and call(mr=-1) == SHAPE
    assert call(ne=0) == ARG
    assert call(f1=fc(qw=QW + 8)) == ALIGN
    assert call(f2=fc(s=S + 4, K=2048, N=4096)) == ALIGN  # scales need 8-byte alignment
    assert call(rs=RS + 2) == ALIGN
    # an output over the other FC's input, over row_start, or over the other output
    assert call(f2=fc(x=X + 0x1000000, qw=QW + 0x1000000, s=S + 0x1000000, y=X + 64, K=2048, N=4096)) == ALIAS
    assert call(f1=fc(y=RS)) == ALIAS
    assert call(f2=fc(x=X + 0x1000000, qw=QW + 0x1000000, s=S + 0x1000000, y=Y + 64, K=2048, N=4096)) == ALIAS
    assert call(E=0) == OK and call(R=0) == OK and call(mr=0) == OK  # empty: nothing launched
    assert "w4_moe_gemm2" in w4.w4_last_error()


def test_moe_gemv2_validation():
    def fc(x=X, stride=0, qw=QW, s=S, y=Y, K=256, N=64):
        return w4.MoeFc(x, stride, qw, s, y, K, N)
    g2 = lib.w4_moe_gemv2
    ok1, ok2 = fc(), fc(x=X + 0x1000000, qw=QW + 0x1000000, s=S + 0x1000000, y=Y + 0x1000000)
    assert g2(ctypes.byref(ok1), None, IDS, 6, 64, None) == NULL
    assert g2(ctypes.byref(ok1), ctypes.byref(ok2), None, 6, 64, None) == NULL
    bad = fc(K=48)
    assert g2(ctypes.byref(ok1), ctypes.byref(bad), IDS, 6, 64, None) == SHAPE
    bad = fc(stride=3)
    assert g2(ctypes.byref(bad), ctypes.byref(ok2), IDS, 6, 64, None) == ARG
    bad = fc(qw=QW + 8)
    assert g2(ctypes.byref(bad), ctypes.byref(ok2), IDS, 6, 64, None) == ALIGN
    assert g2(ctypes.byref(ok1), ctypes.byref(ok2), IDS, 6, 0, None) == ARG
    # fc2's output over fc1's input: the two run together
    bad = fc(x=X + 0x1000000, qw=QW + 0x1000000, s=S + 0x1000000, y=X + 64)
    assert g2(ctypes.byref(ok1), ctypes.byref(bad), IDS, 6, 64, None) == ALIAS
    same_y = fc(x=X + 0x1000000, qw=QW + 0x1000000, s=S + 0x1000000, y=Y + 64)
    assert g2(ctypes.byref(ok1), ctypes.byref(same_y), IDS, 6, 64, None) == ALIAS
    assert g2(ctypes.byref(ok1), ctypes.byref(ok2), IDS, 0, 64, None) == OK  # empty: nothing launched
