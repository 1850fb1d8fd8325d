"""Seeded synthetic inputs shared by the FP64 oracle, the GPU tests and the bench.

This module only draws random numbers and stores them in the bit formats the
library consumes. It holds none of the method's arithmetic: no nibble
unpacking, no dequantisation, no products. Packed weights are drawn as raw
random bytes, which makes every 4-bit code independent and uniform over its 16
values without choosing any packing order here.

Bit formats (all little-endian, row-major, contiguous):

* INT4 linear (N outputs, K inputs, group g):
    ``qw``  int32  [N, K/8]   eight 4-bit codes per word, K contiguous
    ``s``   uint16 [N, K/g]   IEEE binary16 bits, uniform in [0.002, 0.02]
    ``z``   uint16 [N, K/g]   IEEE binary16 bits, integer uniform in 0..15
* FP4 expert pool (num_experts, N, K):
    ``qw``  uint8  [num_experts, N, K/2]  two E2M1 codes per byte
    ``s``   uint16 [num_experts, N, K/32] bfloat16 bits of 2**u, u ~ U(-8, -2)
* Activations: uint16 bfloat16 bits of N(0, 1) draws.

Distributions follow the five workloads of the fused 4-bit GEMV/GEMM study
(single 3840x3840 GEMV; a 48-layer x 7-linear decode step; M=128 prefill; the
262144-row logits GEMV; a six-expert FP4 MoE pair).  Float-to-bfloat16 and
float-to-binary16 conversions are done by torch / numpy casts (round to
nearest even), i.e. library routines, not code of this project.

Seeds: every tensor comes from ``numpy.random.default_rng(SeedSequence(seed,
spawn_key=key))`` so that any single tensor of a large workload can be
regenerated on its own, e.g. by the oracle for a sampled check.
"""
from __future__ import annotations

import numpy as np
import torch

INT4_GROUP = 128
FP4_GROUP = 32

# Decode-step chain: per layer, (name, K, N) in launch order.
HIDDEN = 3840
DECODE_LAYER = (
    ("q", 3840, 4096),
    ("k", 3840, 2048),
    ("v", 3840, 2048),
    ("o", 4096, 3840),
    ("gate", 3840, 15360),
    ("up", 3840, 15360),
    ("down", 15360, 3840),
)
DECODE_LAYERS = 48
PREFILL_M = 128
PREFILL_SHAPES = ((3840, 15360), (15360, 3840))  # (K, N)
LOGITS_SHAPE = (3840, 262144)  # (K, N)
MOE_SLOTS = 6
MOE_POOL = 64
MOE_FC = ((4096, 2048), (2048, 4096))  # FC1 (K, N), FC2 (K, N)


def rng(seed: int, *key: int) -> np.random.Generator:
    """Generator for one tensor, addressed by (seed, key...)."""
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=tuple(int(k) for k in key)))


def random_words(g: np.random.Generator, shape, dtype) -> np.ndarray:
    """Uniform random bits in an array of ``dtype`` (every bit independent)."""
    shape = tuple(int(d) for d in shape)
    n = int(np.prod(shape)) * np.dtype(dtype).itemsize
    return np.frombuffer(g.bytes(n), dtype=dtype).reshape(shape).copy()


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns via torch's cast (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def to_f16_bits(a: np.ndarray) -> np.ndarray:
    """float64/float32 -> IEEE binary16 bit patterns via numpy's cast."""
    return np.asarray(a).astype(np.float16).view(np.uint16)


def bf16_normal(seed: int, key, shape) -> np.ndarray:
    """bfloat16 bits of standard-normal draws."""
    g = rng(seed, *key)
    return to_bf16_bits(g.standard_normal(tuple(shape), dtype=np.float32))


def int4_linear(seed: int, key, K: int, N: int, group: int = INT4_GROUP,
                scale_range=(0.002, 0.02), zero_range=(0, 16)) -> dict:
    """Packed INT4 weights with FP16 scale and FP16 integer zero per group.

    Returns dict(qw=int32[N,K/8], s=uint16[N,K/group], z=uint16[N,K/group]).
    """
    assert K % 8 == 0 and K % group == 0
    key = tuple(key)
    qw = random_words(rng(seed, *key, 0), (N, K // 8), np.uint32).view(np.int32)
    ng = K // group
    s = to_f16_bits(rng(seed, *key, 1).uniform(scale_range[0], scale_range[1], size=(N, ng)))
    z = to_f16_bits(rng(seed, *key, 2).integers(zero_range[0], zero_range[1], size=(N, ng)).astype(np.float64))
    return {"qw": qw, "s": s, "z": z}


def fp4_pool(seed: int, key, num_experts: int, K: int, N: int) -> dict:
    """Packed E2M1 expert pool with a bfloat16 scale per 32 along K.

    Returns dict(qw=uint8[E,N,K/2], s=uint16[E,N,K/32]); s = bf16(2**u), u ~ U(-8,-2).
    """
    assert K % FP4_GROUP == 0
    key = tuple(key)
    qw = random_words(rng(seed, *key, 0), (num_experts, N, K // 2), np.uint8)
    u = rng(seed, *key, 1).uniform(-8.0, -2.0, size=(num_experts, N, K // FP4_GROUP))
    s = to_bf16_bits(np.exp2(u).astype(np.float32))
    return {"qw": qw, "s": s}


def expert_ids(seed: int, key, slots: int = MOE_SLOTS, pool: int = MOE_POOL) -> np.ndarray:
    """``slots`` distinct expert ids drawn uniformly from ``range(pool)`` (int32)."""
    return rng(seed, *key).choice(pool, size=slots, replace=False).astype(np.int32)


def decode_step_specs():
    """(layer, index, name, K, N) for every linear of the decode step, in launch order."""
    out = []
    for layer in range(DECODE_LAYERS):
        for i, (name, K, N) in enumerate(DECODE_LAYER):
            out.append((layer, i, name, K, N))
    return out


# --------------------------------------------------------------- workloads
# Keys: (workload, a, b, ...).  Weight tensors append 0/1/2 (codes, scale,
# zero) inside int4_linear / fp4_pool; activations use a trailing 7.
SEED = 0
W_SINGLE, W_DECODE, W_PREFILL, W_LOGITS, W_MOE = 0, 1, 2, 3, 4


def single_gemv(K: int = 3840, N: int = 3840, seed: int = SEED):
    """Single INT4 GEMV (3840 x 3840 by default): (weights, x bits [K])."""
    return int4_linear(seed, (W_SINGLE, K, N), K, N), bf16_normal(seed, (W_SINGLE, K, N, 7), (K,))


def decode_linear(layer: int, index: int, seed: int = SEED):
    """Linear ``index`` (0..6 = q, k, v, o, gate, up, down) of decode layer ``layer``."""
    _, K, N = DECODE_LAYER[index]
    return int4_linear(seed, (W_DECODE, layer, index), K, N), bf16_normal(seed, (W_DECODE, layer, index, 7), (K,))


def prefill(shape_index: int, M: int = PREFILL_M, seed: int = SEED):
    """Prefill GEMM ``shape_index`` (0: K3840->N15360, 1: K15360->N3840): (weights, x bits [M, K])."""
    K, N = PREFILL_SHAPES[shape_index]
    return (int4_linear(seed, (W_PREFILL, shape_index), K, N),
            bf16_normal(seed, (W_PREFILL, shape_index, 7), (M, K)))


def logits(seed: int = SEED):
    """Logits GEMV, K3840 -> N262144: (weights, x bits [K])."""
    K, N = LOGITS_SHAPE
    return int4_linear(seed, (W_LOGITS,), K, N), bf16_normal(seed, (W_LOGITS, 7), (K,))


def moe_pools(seed: int = SEED):
    """Two FP4 expert pools (FC1: K4096->N2048, FC2: K2048->N4096) of MOE_POOL experts."""
    return [fp4_pool(seed, (W_MOE, fc), MOE_POOL, K, N) for fc, (K, N) in enumerate(MOE_FC)]


def moe_inputs(token: int, seed: int = SEED):
    """Token ``token``: (expert ids [6], FC1 x [K1] shared by all slots, FC2 x [6, K2] one per slot)."""
    ids = expert_ids(seed, (W_MOE, 9, token))
    x1 = bf16_normal(seed, (W_MOE, 0, token, 7), (MOE_FC[0][0],))
    x2 = bf16_normal(seed, (W_MOE, 1, token, 7), (MOE_SLOTS, MOE_FC[1][0]))
    return ids, x1, x2
