"""Seeded synthetic inputs for the W8A8 INT8 Linear workloads.

This module only draws random numbers and rounds them to BF16 bit patterns.
It holds none of the W8A8 arithmetic (no quantisation, no GEMM, no norm), so
both the CPU oracle and the HIP path can take their inputs from it without
sharing any of the method's code.

Every matrix is generated in blocks of ``CHUNK_ROWS`` rows, each block from
its own ``torch.Generator`` seeded with ``(seed, tensor tag, block index)``.
That makes any row of any workload reproducible on its own, which is what the
sampled full-size parity checks use: they regenerate only the rows the oracle
needs.

The shapes and value distributions are those of the five workloads:

* ``tiny``      X [64,256] ~N(0,1); W [128,256] ~N(0,0.02)
* ``square``    X [4096,4096] ~N(0,1), 41 (=1% of K) column indices scaled x20
                before BF16 rounding; W [4096,4096] ~N(0,0.02)
* ``up_proj``   X [28672,4096] ~N(0,1) (16 latent frames x 32x56 tokens);
                gamma [4096] ~N(1,0.1); eps 1e-6; W [16384,4096] ~N(0,0.02)
* ``down_proj`` X [32760,13824] = BF16(GELU_erf(z)), z ~N(0,1)
                (21 latent frames x 30x52 tokens); W [5120,13824] ~N(0,0.01)
* ``blockwise_small`` / ``blockwise_large``  X [1000 | 32760, 5120] ~N(0,1);
                W [5120,5120] ~N(0,0.02)
* ``ln_up_proj`` the up_proj shapes with a LayerNorm prologue instead of the
                RMSNorm: no affine, eps 1e-6, adaLN modulation scale and shift
                [4096] ~N(0,0.2); X ~N(0,1); W ~N(0,0.02)
* ``up_proj_gelu`` the up_proj shapes as an FFN up projection: bias [16384]
                ~N(0,0.1), GELU on the output
* ``small_m``   X [256,13824] = BF16(GELU_erf(z)) (a short sequence against
                the down projection's weight); W [5120,13824] ~N(0,0.01)
* ``m1000``     X [1000,5120] ~N(0,1) (a thousand tokens); W [5120,5120]
                ~N(0,0.02): the post-scale GEMM at the blockwise_small shape
"""
from __future__ import annotations

import dataclasses
import numpy as np
import torch

CHUNK_ROWS = 1024

_TAGS = {"x": 1, "w": 2, "gamma": 3, "outlier": 4, "mod_scale": 5, "mod_shift": 6, "bias": 7}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    seed: int
    x_kind: str          # "normal" | "gelu"
    x_std: float
    w_std: float
    outlier_frac: float = 0.0   # fraction of K columns scaled by outlier_mul
    outlier_mul: float = 1.0
    norm: bool = False          # RMSNorm prologue in front of the quant
    gamma_mean: float = 1.0
    gamma_std: float = 0.1
    eps: float = 1e-6
    blockwise: bool = False     # 1x128 activation / 128x128 weight scales
    layernorm: bool = False     # LayerNorm + adaLN modulation prologue (no affine)
    mod_std: float = 0.2
    bias_std: float = 0.0       # > 0: a Linear bias [N] ~N(0, bias_std)
    gelu: bool = False          # GELU (erf form) on the Linear output

    @property
    def gemm_ops(self) -> int:
        return 2 * self.M * self.N * self.K


WORKLOADS = {
    "tiny": Workload("tiny", 64, 128, 256, 1001, "normal", 1.0, 0.02),
    "square": Workload("square", 4096, 4096, 4096, 1002, "normal", 1.0, 0.02,
                       outlier_frac=0.01, outlier_mul=20.0),
    "up_proj": Workload("up_proj", 28672, 16384, 4096, 1003, "normal", 1.0, 0.02,
                        norm=True),
    "down_proj": Workload("down_proj", 32760, 5120, 13824, 1004, "gelu", 1.0, 0.01),
    "blockwise_small": Workload("blockwise_small", 1000, 5120, 5120, 1005, "normal",
                                1.0, 0.02, blockwise=True),
    "blockwise_large": Workload("blockwise_large", 32760, 5120, 5120, 1006, "normal",
                                1.0, 0.02, blockwise=True),
    "ln_up_proj": Workload("ln_up_proj", 28672, 16384, 4096, 1007, "normal", 1.0, 0.02,
                           layernorm=True),
    "up_proj_gelu": Workload("up_proj_gelu", 28672, 16384, 4096, 1008, "normal", 1.0, 0.02,
                             norm=True, bias_std=0.1, gelu=True),
    "small_m": Workload("small_m", 256, 5120, 13824, 1009, "gelu", 1.0, 0.01),
    "m1000": Workload("m1000", 1000, 5120, 5120, 1010, "normal", 1.0, 0.02),
}


def _gen(seed: int, tag: str, chunk: int) -> torch.Generator:
    return torch.Generator().manual_seed(seed * 1_000_003 + _TAGS[tag] * 65_537 + chunk)


def _to_bf16_bits(t: torch.Tensor) -> np.ndarray:
    """fp32 tensor -> BF16 bit patterns (uint16), torch's round-to-nearest-even."""
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def outlier_columns(wl: Workload) -> np.ndarray:
    """Indices of the K columns that carry the x``outlier_mul`` outliers."""
    n = int(round(wl.outlier_frac * wl.K))
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    perm = torch.randperm(wl.K, generator=_gen(wl.seed, "outlier", 0))
    return np.sort(perm[:n].numpy())


def _matrix_rows(wl: Workload, tag: str, n_rows: int, n_cols: int, std: float,
                 kind: str, rows: np.ndarray | None) -> np.ndarray:
    if rows is None:
        rows = np.arange(n_rows)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, n_cols), dtype=np.uint16)
    if rows.size == 0:
        return out
    ocols = outlier_columns(wl) if (tag == "x" and wl.outlier_frac > 0) else None
    chunks = np.unique(rows // CHUNK_ROWS)
    for c in chunks:
        r0 = int(c) * CHUNK_ROWS
        r1 = min(r0 + CHUNK_ROWS, n_rows)
        z = torch.randn(r1 - r0, n_cols, generator=_gen(wl.seed, tag, int(c)),
                        dtype=torch.float32)
        if kind == "gelu":
            z = torch.nn.functional.gelu(z, approximate="none")
        else:
            z = z * std
        if ocols is not None and ocols.size:
            z[:, torch.from_numpy(ocols)] *= wl.outlier_mul
        bits = _to_bf16_bits(z)
        sel = np.nonzero((rows >= r0) & (rows < r1))[0]
        out[sel] = bits[rows[sel] - r0]
    return out


def x_bits(wl: Workload, rows: np.ndarray | None = None) -> np.ndarray:
    """Activation X [M, K] as BF16 bits (or only the given rows)."""
    return _matrix_rows(wl, "x", wl.M, wl.K, wl.x_std, wl.x_kind, rows)


def w_bits(wl: Workload, rows: np.ndarray | None = None) -> np.ndarray:
    """Weight W [N, K] (nn.Linear layout) as BF16 bits (or only the given rows)."""
    return _matrix_rows(wl, "w", wl.N, wl.K, wl.w_std, "normal", rows)


def gamma_bits(wl: Workload) -> np.ndarray:
    """RMSNorm gain [K] ~ N(gamma_mean, gamma_std) as BF16 bits."""
    z = torch.randn(wl.K, generator=_gen(wl.seed, "gamma", 0), dtype=torch.float32)
    return _to_bf16_bits(z * wl.gamma_std + wl.gamma_mean)


def mod_bits(wl: Workload, which: str) -> np.ndarray:
    """adaLN modulation vector [K] ("mod_scale" or "mod_shift") ~ N(0, mod_std) as BF16 bits."""
    z = torch.randn(wl.K, generator=_gen(wl.seed, which, 0), dtype=torch.float32)
    return _to_bf16_bits(z * wl.mod_std)


def bias_bits(wl: Workload) -> np.ndarray:
    """Linear bias [N] ~ N(0, bias_std) as BF16 bits."""
    z = torch.randn(wl.N, generator=_gen(wl.seed, "bias", 0), dtype=torch.float32)
    return _to_bf16_bits(z * wl.bias_std)


def random_bits(shape, seed: int, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    """Generic seeded BF16 matrix for ad-hoc shapes in the tests."""
    z = torch.randn(*shape, generator=torch.Generator().manual_seed(seed),
                    dtype=torch.float32)
    return _to_bf16_bits(z * std + mean)


def random_int8(shape, seed: int, lo: int = -127, hi: int = 127) -> np.ndarray:
    """Seeded INT8 codes, uniform in [lo, hi]."""
    g = torch.Generator().manual_seed(seed)
    return torch.randint(lo, hi + 1, shape, generator=g, dtype=torch.int32).numpy().astype(np.int8)


def random_scales(shape, seed: int, lo: float = 1e-3, hi: float = 1e-1) -> np.ndarray:
    """Seeded positive fp32 scales, log-uniform in [lo, hi]."""
    g = torch.Generator().manual_seed(seed)
    u = torch.rand(*shape, generator=g, dtype=torch.float64).numpy()
    return np.exp(np.log(lo) + u * (np.log(hi) - np.log(lo))).astype(np.float32)
