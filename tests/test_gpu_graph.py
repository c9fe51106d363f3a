"""The per-call path (per-token quant, then the post-scale GEMM) captured in a
HIP graph and replayed: single pass and split-K (whose stream-ordered
workspace becomes an allocation node of the graph). Every replay, with eager
work and synchronisation between replays and a changed input, must match the
eager results bit for bit."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
import w8a8_int8_quantized_token_amd as w8
from tests.gpu_util import bf16_from_dev, bf16_to_dev, log, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape,seed", [((1000, 384, 512), 191),      # single pass
                                        ((129, 5120, 13824), 192)])   # split over K
def test_graph_replays_match_eager(shape, seed):
    M, N, K = shape
    log(f"graph capture of quant + post-scale GEMM {shape} (split-K parts "
        f"{w8.splitk_parts(M, N, K)})")
    qw, sw = w8.w8a8_quant_rows(bf16_to_dev(W.random_bits((N, K), seed, std=0.02)))
    xs = [bf16_to_dev(W.random_bits((M, K), seed + 1 + i)) for i in range(2)]

    def step(x, out):
        qa, sa = w8.w8a8_quant_rows(x)
        return w8.w8a8_gemm_postscale(qa, qw, sa, sw, out=out)

    eager = []
    for x in xs:
        eager.append(bf16_from_dev(step(x, torch.empty((M, N), dtype=torch.bfloat16,
                                                       device="cuda"))))
    assert not np.array_equal(eager[0], eager[1])

    x_static = xs[0].clone()
    out_static = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up on the capture stream
        step(x_static, out_static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(x_static, out_static)
    torch.cuda.synchronize()
    for r in range(4):
        i = r % 2
        x_static.copy_(xs[i])
        junk = to_dev(np.arange(1024, dtype=np.float32)).sum()   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = bf16_from_dev(out_static)
        log(f"  replay {r} (input {i}): {int(np.count_nonzero(got != eager[i]))} mismatches")
        assert np.array_equal(got, eager[i])
        del junk
