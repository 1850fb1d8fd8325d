"""Host-side plumbing: move packed bit arrays (numpy) into device tensors of the
dtypes the binding expects.  No arithmetic of the method happens here."""
from __future__ import annotations

import numpy as np
import torch


def bf16_tensor(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 bfloat16 bit patterns -> torch.bfloat16 tensor on ``device``."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(device)


def f16_tensor(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 binary16 bit patterns -> torch.float16 tensor on ``device``."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.float16)
    return t.to(device)


def int4_tensors(lin: dict, device="cuda") -> dict:
    """{'qw', 's', 'z'} numpy bits -> device tensors (int32, float16, float16)."""
    return {
        "qw": torch.from_numpy(np.ascontiguousarray(lin["qw"]).view(np.int32)).to(device),
        "s": f16_tensor(lin["s"], device),
        "z": f16_tensor(lin["z"], device),
    }


def fp4_tensors(pool: dict, device="cuda") -> dict:
    """{'qw', 's'} numpy bits -> device tensors (uint8, bfloat16)."""
    return {
        "qw": torch.from_numpy(np.ascontiguousarray(pool["qw"])).to(device),
        "s": bf16_tensor(pool["s"], device),
    }


def bits_of(t: torch.Tensor) -> np.ndarray:
    """Device bfloat16/float16 tensor -> uint16 bit patterns on the host."""
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def bf16_values(t: torch.Tensor) -> np.ndarray:
    """Device bfloat16 tensor -> float64 values on the host (exact widening)."""
    return t.detach().float().cpu().numpy().astype(np.float64)
