"""Host <-> device marshalling helpers for the GPU parity tests (no arithmetic)."""
from __future__ import annotations

import numpy as np
import torch

DEV = "cuda"


def gpu_available() -> bool:
    return torch.cuda.is_available()


def bf16_to_dev(bits: np.ndarray) -> torch.Tensor:
    """BF16 bit patterns (uint16) -> torch.bfloat16 device tensor (same bits)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(DEV)


def bf16_from_dev(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def from_dev(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def log(msg: str) -> None:
    print(msg, flush=True)
