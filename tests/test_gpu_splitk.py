"""Split-K post-scale GEMM on the GPU, against the oracle.

"TurboDiffusion Integration Notes", section "Differences From TurboDiffusion",
paragraph under the table: one INT32 accumulation over all of K, scales in the
epilogue. When a shape's tiles cannot fill the chip the library cuts K into
parts, adds their INT32 partial sums exactly and applies the same fp32
epilogue, so the output must equal the oracle's post-scale of the exact sums
bit for bit (no ulp allowance here), with and without a bias.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
import w8a8_int8_quantized_token_amd as w8
from tests.gpu_util import bf16_from_dev, bf16_to_dev, log, to_dev

pytestmark = pytest.mark.gpu

# (M, N, K): small M against wide N and long K, where the library's cost model
# splits K (parts in the comments, for 256 compute units): ragged and whole
# tiles, parts of equal and unequal stage counts, one-stage parts
SPLIT_SHAPES = [((129, 5120, 13824), 132),    # 9 parts of 12 stages
                ((64, 1024, 4096), 134),      # 16 parts of 2
                ((33, 128, 8192), 137),       # 64 parts of 1
                ((1, 5120, 5120), 138),       # 10 parts of 4
                ((100, 2048, 3200), 139),     # 9 parts of 2 or 3 stages
                ((300, 768, 5248), 140),      # 11 parts of 3 or 4; full-tile mode
                ((77, 384, 11136), 145),      # 44 parts of 1 or 2
                ((512, 1280, 8192), 146),     # 8 parts of 8; full-tile mode
                # not split (the tiles fill the chip, or the partial sums cost
                # more than they save): the single pass, same bar
                ((1000, 5120, 5120), 131), ((257, 640, 1024), 133)]


@pytest.mark.parametrize("with_bias", [False, True])
@pytest.mark.parametrize("shape,seed", SPLIT_SHAPES)
def test_splitk_postscale_exact(shape, seed, with_bias):
    M, N, K = shape
    log(f"split-K post-scale {shape} bias={with_bias}")
    qa = W.random_int8((M, K), seed)
    qw = W.random_int8((N, K), seed + 1)
    if M > 1:
        qa[1] = 127                      # a row at the INT32 extreme against +-127 weights
        qw[: min(N, 4)] = 127
    sa = W.random_scales((M,), seed + 2)
    sw = W.random_scales((N,), seed + 3, lo=1e-5, hi=1e-3)
    b = W.random_bits((N,), seed + 4, std=0.5) if with_bias else None
    out = w8.w8a8_gemm_postscale(to_dev(qa), to_dev(qw), to_dev(sa), to_dev(sw),
                                 bias=None if b is None else bf16_to_dev(b))
    torch.cuda.synchronize()
    acc = O.gemm_i32(qa, qw)
    ref = O.postscale_bf16(acc, sa, sw) if b is None else O.postscale_bias_bf16(acc, sa, sw, b)
    got = bf16_from_dev(out)
    d = O.bf16_ulp_distance(got, ref)
    log(f"  max ulp {int(d.max())}")
    assert np.array_equal(got, ref)


def test_splitk_strided_output_and_repeat():
    M, N, K = 200, 1024, 3072                   # 8 parts of 3 stages
    log("split-K with a strided output, twice in a row")
    qa = W.random_int8((M, K), 141)
    qw = W.random_int8((N, K), 142)
    sa = W.random_scales((M,), 143)
    sw = W.random_scales((N,), 144, lo=1e-5, hi=1e-3)
    ref = O.postscale_bf16(O.gemm_i32(qa, qw), sa, sw)
    full = torch.full((M, N + 128), -3.0, dtype=torch.bfloat16, device="cuda")
    args = (to_dev(qa), to_dev(qw), to_dev(sa), to_dev(sw))
    for _ in range(2):
        w8.w8a8_gemm_postscale(*args, out=full[:, :N])
        torch.cuda.synchronize()
        assert np.array_equal(bf16_from_dev(full[:, :N]), ref)
        assert torch.all(full[:, N:] == -3.0)
