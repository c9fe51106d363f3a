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


def check_inv_rms(r_gpu: np.ndarray, r_ref: np.ndarray, cols: int) -> float:
    """RMSNorm's r: the order of its reduction is not fixed, so the device value
    must lie within (ceil(log2 K) + 4) * 2^-24 * r of the oracle's (which sums
    exact squares in fp64 and rounds once). Returns the largest error seen, in
    units of 2^-24 * r."""
    r_gpu = np.asarray(r_gpu, np.float64)
    r_ref = np.asarray(r_ref, np.float64)
    bound = (int(np.ceil(np.log2(cols))) + 4) * 2.0 ** -24
    rel = np.abs(r_gpu - r_ref) / np.where(r_ref > 0, r_ref, 1.0)
    assert np.all(np.isfinite(r_gpu)) and np.all(rel <= bound), \
        f"inv_rms off by {rel.max() / 2.0 ** -24:.2f} x 2^-24 (bound {bound / 2.0 ** -24:.0f})"
    return float(rel.max() / 2.0 ** -24)


def check_ln_mean(mu_gpu: np.ndarray, mu_ref: np.ndarray, x_f32: np.ndarray) -> float:
    """LayerNorm's mean: within (ceil(log2 K) + 4) * 2^-24 * mean|x| of the
    oracle's (the sum's order is not fixed). Returns the largest error in
    units of 2^-24 * mean|x|."""
    K = x_f32.shape[1]
    scale = np.mean(np.abs(x_f32.astype(np.float64)), axis=1)
    bound = (int(np.ceil(np.log2(K))) + 4) * 2.0 ** -24
    err = np.abs(np.asarray(mu_gpu, np.float64) - np.asarray(mu_ref, np.float64))
    rel = err / np.where(scale > 0, scale, 1.0)
    assert np.all(np.isfinite(mu_gpu)) and np.all(rel <= bound), \
        f"mean off by {rel.max() / 2.0 ** -24:.2f} x 2^-24 mean|x|"
    return float(rel.max() / 2.0 ** -24)
