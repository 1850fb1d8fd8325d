"""Python binding of ``libw4.so``, the fused 4-bit-weight x BF16 GEMV/GEMM library.

Argument marshalling only: each function takes torch tensors that already
live in device memory, checks their dtypes and shapes, and passes raw
pointers, sizes and the current HIP stream to the C entry point of the same
name (declared in ``include/w4.h``).  Every step of the computation runs in
the library's HIP kernels; there is no fallback.  If the shared library is
not built, importing this package raises ImportError.

Tensor formats (see ``include/w4.h``):
    x     bfloat16 [M, K] (or [K])       qw      int32 [N, K/8]
    s, z  float16  [N, K/128]            qw_fp4  uint8 [experts, N, K/2]
    s_fp4 bfloat16 [experts, N, K/32]    y       bfloat16 [M, N] (or [N])
"""
from __future__ import annotations

import ctypes
import os
import pathlib

import torch

__all__ = [
    "W4Error", "lib", "LIB_PATH", "w4_abi_version", "w4_status_string", "w4_last_error",
    "w4_gemv", "w4_gemm", "w4_gemm_workspace_bytes", "w4_moe_gemv", "w4_moe_gemv2", "w4_moe_gemm", "w4_moe_gemm2",
    "w4_graph_begin", "w4_graph_end", "w4_graph_replay", "w4_graph_destroy", "W4Graph",
    "w4_dequant_int4", "w4_dequant_fp4", "w4_int4_gemv_operands", "INT4_GROUP", "FP4_GROUP", "GEMV_MAX_K",
    "GemvDesc", "W4Chain", "w4_chain_workspace_bytes", "w4_chain_create", "w4_chain_run",
    "w4_chain_error", "w4_chain_destroy", "CHAIN_MAX_K", "w4_read_probe", "READ_PROBE_SINK",
    "w4_tune_param", "w4_tune_force", "TUNE_KERNELS", "w4_gemm_noalloc", "w4_repack_gptq",
]

# W4_LIBRARY names another build of the same library (the chain-timeline build
# of chain_timeline.py); by default the libw4.so next to this file.
LIB_PATH = pathlib.Path(os.environ.get("W4_LIBRARY") or pathlib.Path(__file__).resolve().with_name("libw4.so"))
INT4_GROUP = 128
FP4_GROUP = 32
GEMV_MAX_K = 32768
GEMM_NOALLOC_SCRATCH_BYTES = 16 << 20
# launch-tuning kernel families (W4_TUNE_*), name -> id
TUNE_KERNELS = {"gemv": 0, "gemv_rows2": 1, "gemm_small_m": 2, "gemm": 3, "moe_gemv": 4}
CHAIN_MAX_K = 16384

STATUS = {0: "W4_OK", 1: "W4_ERR_NULL", 2: "W4_ERR_SHAPE", 3: "W4_ERR_UNSUPPORTED", 4: "W4_ERR_ALIGN",
          5: "W4_ERR_WORKSPACE", 6: "W4_ERR_ALIAS", 7: "W4_ERR_ARG", 8: "W4_ERR_HIP"}

_vp = ctypes.c_void_p
_i32 = ctypes.c_int
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t



class GemvDesc(ctypes.Structure):
    """struct w4_gemv_desc (include/w4.h)."""
    _fields_ = [("x", ctypes.c_void_p), ("qw", ctypes.c_void_p), ("s", ctypes.c_void_p), ("z", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("K", ctypes.c_int), ("N", ctypes.c_int), ("stage", ctypes.c_int),
                ("reserved", ctypes.c_int)]


class MoeFc(ctypes.Structure):
    """struct w4_moe_fc (include/w4.h)."""
    _fields_ = [("x", ctypes.c_void_p), ("x_stride", ctypes.c_int64), ("qw_fp4", ctypes.c_void_p),
                ("s_fp4", ctypes.c_void_p), ("y", ctypes.c_void_p), ("K", ctypes.c_int), ("N", ctypes.c_int)]


class MoeGemmFc(ctypes.Structure):
    """struct w4_moe_gemm_fc (include/w4.h)."""
    _fields_ = [("x", ctypes.c_void_p), ("qw_fp4", ctypes.c_void_p), ("s_fp4", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("K", ctypes.c_int), ("N", ctypes.c_int)]


# name -> (restype, argtypes), mirroring include/w4.h
SIGNATURES = {
    "w4_abi_version": (_i32, []),
    "w4_status_string": (ctypes.c_char_p, [_i32]),
    "w4_last_error": (ctypes.c_char_p, []),
    "w4_gemv": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp]),
    "w4_gemm_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "w4_gemm": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _sz, _vp]),
    "w4_gemm_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp]),
    "w4_moe_gemv": (_i32, [_vp, _i64, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp]),
    "w4_moe_gemv2": (_i32, [ctypes.POINTER(MoeFc), ctypes.POINTER(MoeFc), _vp, _i32, _i32, _vp]),
    "w4_moe_gemm": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp]),
    "w4_moe_gemm2": (_i32, [ctypes.POINTER(MoeGemmFc), ctypes.POINTER(MoeGemmFc), _vp, _vp, _i32, _i32, _i32, _i32,
                            _vp]),
    "w4_graph_begin": (_i32, [_vp]),
    "w4_graph_end": (_i32, [_vp, ctypes.POINTER(_vp)]),
    "w4_graph_replay": (_i32, [_vp, _vp]),
    "w4_graph_destroy": (None, [_vp]),
    "w4_chain_workspace_bytes": (_sz, [_vp, _i32]),
    "w4_chain_create": (_i32, [ctypes.POINTER(GemvDesc), _i32, _vp, _sz, ctypes.POINTER(_vp)]),
    "w4_chain_run": (_i32, [_vp, _vp]),
    "w4_chain_error": (_i32, [_vp, ctypes.POINTER(ctypes.c_uint32)]),
    "w4_chain_destroy": (None, [_vp]),
    "w4_chain_set_spin_limit": (_i32, [_vp, ctypes.c_uint32]),
    "w4_dequant_int4": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp]),
    "w4_dequant_fp4": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _vp]),
    "w4_int4_gemv_operands": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _vp]),
    "w4_read_probe": (_i32, [_vp, _sz, _vp, _vp]),
    "w4_tune_param": (_i32, [_i32, _i32, _i32, _i32]),
    "w4_repack_gptq": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp]),
    "w4_tune_force": (_i32, [_i32, _i32]),
}

READ_PROBE_SINK = 4096


def _load() -> ctypes.CDLL:
    if not LIB_PATH.exists():
        raise ImportError(f"{LIB_PATH} is not built: run `python gemm_w4_gemv_amd/build.py` "
                          "(or __graft_entry__.build()) first")
    handle = ctypes.CDLL(str(LIB_PATH))
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    return handle


lib = _load()


class W4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        self.name = STATUS.get(status, f"status {status}")
        detail = lib.w4_last_error().decode(errors="replace")
        super().__init__(f"{where}: {self.name}: {detail}")


def _check(status: int, where: str) -> None:
    if status != 0:
        raise W4Error(status, where)


def w4_abi_version() -> int:
    return lib.w4_abi_version()


def w4_status_string(status: int) -> str:
    return lib.w4_status_string(status).decode()


def w4_last_error() -> str:
    return lib.w4_last_error().decode(errors="replace")


# ---------------------------------------------------------------- marshalling
def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev(t: torch.Tensor, name: str, dtypes) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


_BF16 = (torch.bfloat16,)
_F16 = (torch.float16,)
_I32 = (torch.int32,)
_U8 = (torch.uint8,)


def _int4_weight(qw, s, z, K, group):
    N = qw.shape[0]
    if qw.dim() != 2 or qw.shape[1] * 8 != K:
        raise ValueError(f"qw must be int32 [N, K/8] with K = {K}; got {tuple(qw.shape)}")
    G = K // group if group > 0 else 0
    for name, t in (("s", s), ("z", z)):
        if tuple(t.shape) != (N, G):
            raise ValueError(f"{name} must be [N, K/{group}] = {(N, G)}; got {tuple(t.shape)}")
    return N, _dev(qw, "qw", _I32), _dev(s, "s", _F16), _dev(z, "z", _F16)


def w4_gemv(x, qw, s, z, y, group: int = INT4_GROUP, stream=None) -> torch.Tensor:
    """``y[n] = bf16(sum_k (q - z) s x)`` for one BF16 vector ``x [K]`` (M = 1)."""
    K = x.numel()
    N, pq, ps, pz = _int4_weight(qw, s, z, K, group)
    if y.numel() != N:
        raise ValueError(f"y must hold N = {N} values; got {tuple(y.shape)}")
    _check(lib.w4_gemv(_dev(x, "x", _BF16), pq, ps, pz, _dev(y, "y", _BF16), K, N, group, _stream(stream)),
           "w4_gemv")
    return y


def w4_gemm_workspace_bytes(M: int, K: int, N: int, group: int = INT4_GROUP) -> int:
    return lib.w4_gemm_workspace_bytes(M, K, N, group)


def w4_gemm(x, qw, s, z, y, workspace=None, group: int = INT4_GROUP, stream=None) -> torch.Tensor:
    """``y [M, N] = x [M, K] @ bf16(dequant(W)).T`` with FP32 accumulation."""
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    M, K = x.shape
    N, pq, ps, pz = _int4_weight(qw, s, z, K, group)
    if tuple(y.shape) != (M, N):
        raise ValueError(f"y must be [M, N] = {(M, N)}; got {tuple(y.shape)}")
    if workspace is None:
        pw, nbytes = None, 0
    else:
        pw, nbytes = _dev(workspace, "workspace", (workspace.dtype,)), workspace.numel() * workspace.element_size()
    _check(lib.w4_gemm(_dev(x, "x", _BF16), pq, ps, pz, _dev(y, "y", _BF16), M, K, N, group, pw, nbytes,
                       _stream(stream)), "w4_gemm")
    return y


def w4_moe_gemm(x, row_start, expert_ids, qw_fp4, s_fp4, y, max_rows: int, stream=None) -> torch.Tensor:
    """Group ``e`` applies FP4 expert ``expert_ids[e]`` to rows ``row_start[e] .. row_start[e+1]-1`` of ``x``."""
    if qw_fp4.dim() != 3:
        raise ValueError("qw_fp4 must be [experts, N, K/2]")
    num_experts, N, half_k = qw_fp4.shape
    K = 2 * half_k
    if tuple(s_fp4.shape) != (num_experts, N, K // FP4_GROUP):
        raise ValueError(f"s_fp4 must be [experts, N, K/32]; got {tuple(s_fp4.shape)}")
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"x must be [R, K] with K = {K}; got {tuple(x.shape)}")
    R = x.shape[0]
    E = expert_ids.numel()
    if row_start.numel() != E + 1:
        raise ValueError(f"row_start must have E + 1 = {E + 1} entries")
    if tuple(y.shape) != (R, N):
        raise ValueError(f"y must be [R, N] = {(R, N)}; got {tuple(y.shape)}")
    _check(lib.w4_moe_gemm(_dev(x, "x", _BF16), _dev(row_start, "row_start", _I32),
                           _dev(expert_ids, "expert_ids", _I32), _dev(qw_fp4, "qw_fp4", _U8),
                           _dev(s_fp4, "s_fp4", _BF16), _dev(y, "y", _BF16), R, E, int(max_rows), num_experts, K, N,
                           _stream(stream)), "w4_moe_gemm")
    return y


def _moe_gemm_fc(x, qw_fp4, s_fp4, y, R):
    if qw_fp4.dim() != 3:
        raise ValueError("qw_fp4 must be [experts, N, K/2]")
    num_experts, N, half_k = qw_fp4.shape
    K = 2 * half_k
    if tuple(s_fp4.shape) != (num_experts, N, K // FP4_GROUP):
        raise ValueError(f"s_fp4 must be [experts, N, K/32]; got {tuple(s_fp4.shape)}")
    if tuple(x.shape) != (R, K):
        raise ValueError(f"x must be [R, K] = {(R, K)}; got {tuple(x.shape)}")
    if tuple(y.shape) != (R, N):
        raise ValueError(f"y must be [R, N] = {(R, N)}; got {tuple(y.shape)}")
    fc = MoeGemmFc(_dev(x, "x", _BF16), _dev(qw_fp4, "qw_fp4", _U8), _dev(s_fp4, "s_fp4", _BF16), _dev(y, "y", _BF16),
                   K, N)
    return fc, num_experts


def w4_moe_gemm2(fc1, fc2, row_start, expert_ids, max_rows: int, stream=None):
    """Two grouped FP4 expert GEMMs over the same groups in one launch; ``fc1`` and ``fc2`` are
    ``(x, qw_fp4, s_fp4, y)`` as for ``w4_moe_gemm`` (their inputs must not depend on each other)."""
    R = fc1[0].shape[0]
    E = expert_ids.numel()
    if row_start.numel() != E + 1:
        raise ValueError(f"row_start must have E + 1 = {E + 1} entries")
    f1, n1 = _moe_gemm_fc(*fc1, R)
    f2, n2 = _moe_gemm_fc(*fc2, R)
    if n1 != n2:
        raise ValueError("both expert pools must hold the same number of experts")
    _check(lib.w4_moe_gemm2(ctypes.byref(f1), ctypes.byref(f2), _dev(row_start, "row_start", _I32),
                            _dev(expert_ids, "expert_ids", _I32), R, E, int(max_rows), n1, _stream(stream)),
           "w4_moe_gemm2")
    return fc1[3], fc2[3]


def w4_moe_gemv(x, qw_fp4, s_fp4, expert_ids, y, stream=None) -> torch.Tensor:
    """Slot ``e`` applies FP4 expert ``expert_ids[e]`` to ``x`` ([K], shared) or ``x[e]`` ([E, K])."""
    if qw_fp4.dim() != 3:
        raise ValueError("qw_fp4 must be [experts, N, K/2]")
    num_experts, N, half_k = qw_fp4.shape
    K = 2 * half_k
    if tuple(s_fp4.shape) != (num_experts, N, K // FP4_GROUP):
        raise ValueError(f"s_fp4 must be [experts, N, K/32]; got {tuple(s_fp4.shape)}")
    E = expert_ids.numel()
    if x.dim() == 1:
        stride = 0
        if x.numel() != K:
            raise ValueError(f"x must have K = {K} values")
    else:
        if x.dim() != 2 or x.shape[1] != K or x.shape[0] < E:
            raise ValueError(f"x must be [E, K] = {(E, K)}; got {tuple(x.shape)}")
        stride = K
    if tuple(y.shape) != (E, N):
        raise ValueError(f"y must be [E, N] = {(E, N)}; got {tuple(y.shape)}")
    _check(lib.w4_moe_gemv(_dev(x, "x", _BF16), stride, _dev(qw_fp4, "qw_fp4", _U8), _dev(s_fp4, "s_fp4", _BF16),
                           _dev(expert_ids, "expert_ids", _I32), _dev(y, "y", _BF16), E, num_experts, K, N,
                           _stream(stream)), "w4_moe_gemv")
    return y


def _moe_fc(x, qw_fp4, s_fp4, y, E):
    if qw_fp4.dim() != 3:
        raise ValueError("qw_fp4 must be [experts, N, K/2]")
    num_experts, N, half_k = qw_fp4.shape
    K = 2 * half_k
    if tuple(s_fp4.shape) != (num_experts, N, K // FP4_GROUP):
        raise ValueError(f"s_fp4 must be [experts, N, K/32]; got {tuple(s_fp4.shape)}")
    if x.dim() == 1:
        stride = 0
        if x.numel() != K:
            raise ValueError(f"x must have K = {K} values")
    else:
        if x.dim() != 2 or x.shape[1] != K or x.shape[0] < E:
            raise ValueError(f"x must be [E, K] = {(E, K)}; got {tuple(x.shape)}")
        stride = K
    if tuple(y.shape) != (E, N):
        raise ValueError(f"y must be [E, N] = {(E, N)}; got {tuple(y.shape)}")
    fc = MoeFc(_dev(x, "x", _BF16), stride, _dev(qw_fp4, "qw_fp4", _U8), _dev(s_fp4, "s_fp4", _BF16),
               _dev(y, "y", _BF16), K, N)
    return fc, num_experts


def w4_moe_gemv2(fc1, fc2, expert_ids, stream=None):
    """Two FP4 expert FCs over the same slots in one launch; ``fc1`` and ``fc2`` are
    ``(x, qw_fp4, s_fp4, y)`` as for ``w4_moe_gemv`` (their inputs must not depend on each other)."""
    E = expert_ids.numel()
    f1, n1 = _moe_fc(*fc1, E)
    f2, n2 = _moe_fc(*fc2, E)
    if n1 != n2:
        raise ValueError("both expert pools must hold the same number of experts")
    _check(lib.w4_moe_gemv2(ctypes.byref(f1), ctypes.byref(f2), _dev(expert_ids, "expert_ids", _I32), E, n1,
                            _stream(stream)), "w4_moe_gemv2")
    return fc1[3], fc2[3]


class W4Graph:
    """An instantiated HIP graph owned by the library (w4_graph_t)."""

    def __init__(self, handle: int):
        self.handle = handle

    def replay(self, stream=None) -> None:
        w4_graph_replay(self, stream)

    def destroy(self) -> None:
        if self.handle:
            lib.w4_graph_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def w4_graph_begin(stream) -> None:
    _check(lib.w4_graph_begin(_stream(stream)), "w4_graph_begin")


def w4_graph_end(stream) -> W4Graph:
    h = _vp()
    _check(lib.w4_graph_end(_stream(stream), ctypes.byref(h)), "w4_graph_end")
    return W4Graph(h.value)


def w4_graph_replay(graph: W4Graph, stream=None) -> None:
    _check(lib.w4_graph_replay(graph.handle, _stream(stream)), "w4_graph_replay")


def w4_graph_destroy(graph: W4Graph) -> None:
    graph.destroy()


def _chain_descs(gemvs):
    descs = (GemvDesc * len(gemvs))()
    for i, g in enumerate(gemvs):
        K = g["x"].numel()
        N, pq, ps, pz = _int4_weight(g["qw"], g["s"], g["z"], K, INT4_GROUP)
        if g["y"].numel() != N:
            raise ValueError(f"gemv {i}: y must hold N = {N} values")
        descs[i] = GemvDesc(_dev(g["x"], "x", _BF16), pq, ps, pz, _dev(g["y"], "y", _BF16), K, N, int(g["stage"]), 0)
    return descs


def w4_chain_workspace_bytes(gemvs) -> int:
    """Workspace bytes the chain of ``gemvs`` (as for w4_chain_create) needs."""
    descs = _chain_descs(gemvs)
    n = lib.w4_chain_workspace_bytes(ctypes.cast(descs, _vp), len(gemvs))
    if n == 0:  # invalid descriptors; w4_last_error says why
        raise W4Error(7, "w4_chain_workspace_bytes")
    return n


class W4Chain:
    """A planned decode chain (w4_chain_t); keeps its descriptors' tensors alive."""

    def __init__(self, handle: int, keep):
        self.handle = handle
        self._keep = keep

    def run(self, stream=None) -> None:
        w4_chain_run(self, stream)

    def error(self) -> int:
        return w4_chain_error(self)

    def set_spin_limit(self, spin_limit: int) -> None:
        """For tests of failure handling: bound every wait of later runs to ``spin_limit`` polls."""
        _check(lib.w4_chain_set_spin_limit(self.handle, int(spin_limit)), "w4_chain_set_spin_limit")

    def destroy(self) -> None:
        if self.handle:
            lib.w4_chain_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def w4_chain_create(gemvs, workspace: torch.Tensor) -> W4Chain:
    """Plan a chain.  ``gemvs``: sequence of dicts with device tensors ``x`` (bf16 [K]),
    ``qw`` (int32 [N, K/8]), ``s``, ``z`` (fp16 [N, K/128]), ``y`` (bf16 [N]) and an int
    ``stage`` (non-decreasing).  ``workspace``: device tensor of at least
    w4_chain_workspace_bytes(gemvs) bytes."""
    descs = _chain_descs(gemvs)
    nbytes = workspace.numel() * workspace.element_size()
    h = _vp()
    _check(lib.w4_chain_create(descs, len(gemvs), _dev(workspace, "workspace", (workspace.dtype,)), nbytes,
                               ctypes.byref(h)), "w4_chain_create")
    return W4Chain(h.value, (list(gemvs), workspace))


def w4_chain_run(chain: W4Chain, stream=None) -> None:
    _check(lib.w4_chain_run(chain.handle, _stream(stream)), "w4_chain_run")


def w4_chain_error(chain: W4Chain) -> int:
    word = ctypes.c_uint32(0)
    _check(lib.w4_chain_error(chain.handle, ctypes.byref(word)), "w4_chain_error")
    return word.value


def w4_chain_destroy(chain: W4Chain) -> None:
    chain.destroy()


def w4_dequant_int4(qw, s, z, out_f32=None, out_bf16=None, group: int = INT4_GROUP, stream=None) -> None:
    """Test-only: FP32 values and/or BF16 matrix-core operand of an INT4 weight, from the prefill GEMM's routine."""
    N, K = qw.shape[0], qw.shape[1] * 8
    _, pq, ps, pz = _int4_weight(qw, s, z, K, group)
    pf = _dev(out_f32, "out_f32", (torch.float32,)) if out_f32 is not None else None
    pb = _dev(out_bf16, "out_bf16", _BF16) if out_bf16 is not None else None
    for t in (out_f32, out_bf16):
        if t is not None and tuple(t.shape) != (N, K):
            raise ValueError(f"outputs must be [N, K] = {(N, K)}")
    _check(lib.w4_dequant_int4(pq, ps, pz, pf, pb, K, N, group, _stream(stream)), "w4_dequant_int4")


def w4_int4_gemv_operands(qw, codes_out, x=None, x_out=None, stream=None) -> None:
    """Test-only: the biased code pairs (int32 ``[N, K/8, 4]``) and, with ``x``, the matching x
    pairs (int32 ``[K/8, 4]``) that the GEMV-path kernels dot, from their own routines."""
    if not (isinstance(qw, torch.Tensor) and qw.dtype == torch.int32 and qw.dim() == 2):
        raise ValueError("qw must be an int32 [N, K/8] tensor")
    N, K = qw.shape[0], qw.shape[1] * 8
    if tuple(codes_out.shape) != (N, K // 8, 4):
        raise ValueError(f"codes_out must be [N, K/8, 4] = {(N, K // 8, 4)}")
    if (x is None) != (x_out is None):
        raise ValueError("x and x_out go together")
    px = pxo = None
    if x is not None:
        if tuple(x.shape) != (K,) or tuple(x_out.shape) != (K // 8, 4):
            raise ValueError("x must be [K] and x_out [K/8, 4]")
        px, pxo = _dev(x, "x", _BF16), _dev(x_out, "x_out", (torch.int32,))
    _check(lib.w4_int4_gemv_operands(_dev(qw, "qw", (torch.int32,)), px, _dev(codes_out, "codes_out", (torch.int32,)),
                                     pxo, K, N, _stream(stream)), "w4_int4_gemv_operands")


def w4_dequant_fp4(qw_fp4, s_fp4, out_f32=None, out_bf16=None, stream=None) -> None:
    """Test-only: FP32 and/or BF16 image of one FP4 expert ``[N, K/2]``, from the GEMV's unpack code."""
    N, K = qw_fp4.shape[0], qw_fp4.shape[1] * 2
    if tuple(s_fp4.shape) != (N, K // FP4_GROUP):
        raise ValueError("s_fp4 must be [N, K/32]")
    pf = _dev(out_f32, "out_f32", (torch.float32,)) if out_f32 is not None else None
    pb = _dev(out_bf16, "out_bf16", _BF16) if out_bf16 is not None else None
    for t in (out_f32, out_bf16):
        if t is not None and tuple(t.shape) != (N, K):
            raise ValueError(f"outputs must be [N, K] = {(N, K)}")
    _check(lib.w4_dequant_fp4(_dev(qw_fp4, "qw_fp4", _U8), _dev(s_fp4, "s_fp4", _BF16), pf, pb, K, N,
                              _stream(stream)), "w4_dequant_fp4")


def w4_read_probe(src, sink, nbytes: int | None = None, stream=None) -> None:
    """Measurement only: stream ``nbytes`` (default: all) of ``src`` once; one digest word per workgroup into ``sink``.

    ``sink`` is a device uint32 tensor of at least READ_PROBE_SINK words.  With
    nbytes = 0 the call is one empty launch.
    """
    if not (isinstance(src, torch.Tensor) and src.is_cuda and src.is_contiguous()):
        raise ValueError("src must be a contiguous device tensor")
    if not (isinstance(sink, torch.Tensor) and sink.is_cuda and sink.dtype == torch.int32 and sink.numel() >= READ_PROBE_SINK):
        raise ValueError(f"sink must be a device int32 tensor of at least {READ_PROBE_SINK} words")
    total = src.numel() * src.element_size()
    n = total if nbytes is None else int(nbytes)
    if n < 0 or n > total:
        raise ValueError(f"nbytes must lie in [0, {total}]")
    _check(lib.w4_read_probe(src.data_ptr(), n, sink.data_ptr(), _stream(stream)), "w4_read_probe")


def w4_tune_param(kernel: str, M: int, K: int, N: int) -> int:
    """The launch parameter a call of shape (M, K, N) of a kernel family uses (table, else rule)."""
    return int(lib.w4_tune_param(TUNE_KERNELS[kernel], M, K, N))


def w4_tune_force(kernel: str, param: int) -> None:
    """Make every later call of a kernel family launch with ``param`` (0: back to the table)."""
    _check(lib.w4_tune_force(TUNE_KERNELS[kernel], int(param)), "w4_tune_force")


def w4_gemm_noalloc(x, qw, s, z, y, group: int = INT4_GROUP, stream=None) -> torch.Tensor:
    """``w4_gemm`` for callers that cannot allocate: split-K partials in the library's per-GPU scratch."""
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    M, K = x.shape
    N, pq, ps, pz = _int4_weight(qw, s, z, K, group)
    if tuple(y.shape) != (M, N):
        raise ValueError(f"y must be [M, N] = {(M, N)}")
    _check(lib.w4_gemm_noalloc(_dev(x, "x", _BF16), pq, ps, pz, _dev(y, "y", _BF16), M, K, N, group,
                               _stream(stream)), "w4_gemm_noalloc")
    return y


def w4_repack_gptq(qweight, s_gn, z_gn, group: int = INT4_GROUP, stream=None):
    """GPTQ's K-major layout (int32 ``[K/8, N]``, fp16 ``[K/128, N]``) -> new device tensors
    ``qw [N, K/8]``, ``s``, ``z [N, K/128]`` in the layout the other entry points read."""
    if not (isinstance(qweight, torch.Tensor) and qweight.dtype == torch.int32 and qweight.dim() == 2):
        raise ValueError("qweight must be an int32 [K/8, N] tensor")
    K, N = qweight.shape[0] * 8, qweight.shape[1]
    for name, t in (("s_gn", s_gn), ("z_gn", z_gn)):
        if tuple(t.shape) != (K // group, N):
            raise ValueError(f"{name} must be [K/{group}, N] = {(K // group, N)}")
    qw = torch.empty(N, K // 8, dtype=torch.int32, device=qweight.device)
    s = torch.empty(N, K // group, dtype=torch.float16, device=qweight.device)
    z = torch.empty_like(s)
    _check(lib.w4_repack_gptq(_dev(qweight, "qweight", _I32), _dev(s_gn, "s_gn", _F16), _dev(z_gn, "z_gn", _F16),
                              qw.data_ptr(), s.data_ptr(), z.data_ptr(), K, N, group, _stream(stream)), "w4_repack_gptq")
    return qw, s, z
