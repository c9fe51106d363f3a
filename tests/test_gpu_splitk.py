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

# (M, N, K): small M against wide N and long K. The library's cost model
# (for 256 compute units) splits K for some of them and runs others as one
# pass (on 128 x 160 tiles, or on 256 x 256 tiles where those fill the chip);
# every result must equal the oracle's either way. Ragged and whole tiles,
# parts of equal and unequal stage counts.
SPLIT_SHAPES = [((129, 5120, 13824), 132),    # 9 parts of 12 stages
                ((64, 1024, 4096), 134),
                ((33, 128, 8192), 137),       # 8 parts of 8
                ((1, 5120, 5120), 138),
                ((100, 2048, 3200), 139),
                ((300, 768, 5248), 140),
                ((77, 384, 11136), 145),      # 10 parts of 8 or 9
                ((512, 1280, 8192), 146),     # 8 parts of 8; full-tile mode
                ((1000, 5120, 5120), 131), ((257, 640, 1024), 133)]


def test_split_shapes_cover_both_paths():
    # the list above must keep exercising split-K and the single pass
    parts = [w8.splitk_parts(*shape) for shape, _ in SPLIT_SHAPES]
    assert sum(p > 1 for p in parts) >= 4 and sum(p == 1 for p in parts) >= 3, parts


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


# parts forced to 64, capped by the 128-byte K stages: one-stage parts, parts
# of one or two stages, and as many parts as stages
FORCED = [((33, 128, 8192), 171, 64), ((77, 384, 11136), 172, 64),
          ((300, 768, 5248), 173, 41), ((256, 512, 2048), 174, 16)]


@pytest.mark.parametrize("shape,seed,parts", FORCED)
def test_splitk_forced_parts_exact(shape, seed, parts):
    """Many small parts, which the cost model does not pick: one-stage parts,
    parts of unequal length, full-tile mode, with bias and GELU epilogues, the
    part count passed explicitly and the workspace given by the caller."""
    M, N, K = shape
    log(f"split-K forced to {parts} parts: {shape}")
    assert w8.postscale_workspace_size(M, N, K, parts) == parts * M * N * 4
    qa = W.random_int8((M, K), seed)
    qw = W.random_int8((N, K), seed + 1)
    qa[1] = 127
    qw[:4] = 127
    sa = W.random_scales((M,), seed + 2)
    sw = W.random_scales((N,), seed + 3, lo=1e-5, hi=1e-3)
    b = W.random_bits((N,), seed + 4, std=0.5)
    ws = torch.empty((parts * M * N * 4,), dtype=torch.uint8, device="cuda")
    acc = O.gemm_i32(qa, qw)
    for bias, gelu in ((None, False), (b, False), (b, True)):
        out = w8.w8a8_gemm_postscale(to_dev(qa), to_dev(qw), to_dev(sa), to_dev(sw),
                                     bias=None if bias is None else bf16_to_dev(bias),
                                     gelu=gelu, parts=parts, workspace=ws)
        torch.cuda.synchronize()
        if gelu:
            ref = O.postscale_gelu_bf16(acc, sa, sw, bias)
        elif bias is None:
            ref = O.postscale_bf16(acc, sa, sw)
        else:
            ref = O.postscale_bias_bf16(acc, sa, sw, bias)
        got = bf16_from_dev(out)
        log(f"  bias={bias is not None} gelu={gelu}: {int(np.count_nonzero(got != ref))} mismatches")
        assert np.array_equal(got, ref)


def test_splitk_workspace_rules_on_device():
    """A workspace one byte short, or a forced split without one, is refused
    before anything runs; the output keeps its contents."""
    M, N, K = 64, 256, 1024
    qa, qw = to_dev(W.random_int8((M, K), 175)), to_dev(W.random_int8((N, K), 176))
    sa, sw = to_dev(W.random_scales((M,), 177)), to_dev(W.random_scales((N,), 178))
    out = torch.full((M, N), 5.0, dtype=torch.bfloat16, device="cuda")
    short = torch.empty((4 * M * N * 4 - 1,), dtype=torch.uint8, device="cuda")
    with pytest.raises(w8.W8A8Error, match="workspace"):
        w8.w8a8_gemm_postscale(qa, qw, sa, sw, out=out, parts=4, workspace=short)
    st = w8.lib().w8a8_gemm_postscale_ex(qa.data_ptr(), K, qw.data_ptr(), K, sa.data_ptr(),
                                         sw.data_ptr(), None, 0, out.data_ptr(), N, M, N, K, 4,
                                         None, 0, torch.cuda.current_stream().cuda_stream)
    assert st == w8.W8A8_ERR_INVALID_ARGUMENT and b"workspace" in w8.lib().w8a8_last_error()
    torch.cuda.synchronize()
    assert torch.all(out == 5.0)


def test_concurrent_streams_exact():
    """Split-K and single-pass GEMMs issued on two side streams at once, many
    times over: each split call gets its own workspace from torch's allocator
    on its stream, so concurrent calls never share partial sums. Every result
    is checked against the oracle; the streams keep the default priority."""
    log("concurrent split-K / single-pass GEMMs on two streams")
    cases = []
    for (M, N, K), seed in (((129, 5120, 13824), 181), ((64, 1024, 4096), 182),
                            ((512, 1280, 8192), 183), ((1000, 384, 512), 184)):
        qa = W.random_int8((M, K), seed)
        qw = W.random_int8((N, K), seed + 1)
        sa = W.random_scales((M,), seed + 2)
        sw = W.random_scales((N,), seed + 3, lo=1e-5, hi=1e-3)
        ref = O.postscale_bf16(O.gemm_i32(qa, qw), sa, sw)
        cases.append(((to_dev(qa), to_dev(qw), to_dev(sa), to_dev(sw)), ref))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    outs = []
    for it in range(6):
        for c, (args, ref) in enumerate(cases):
            st = streams[(it + c) % 2]
            with torch.cuda.stream(st):
                out = torch.empty(ref.shape, dtype=torch.bfloat16, device="cuda")
                w8.w8a8_gemm_postscale(*args, out=out, stream=st)
            outs.append((out, ref, st))
    torch.cuda.synchronize()
    bad = 0
    for out, ref, _ in outs:
        bad += int(np.count_nonzero(bf16_from_dev(out) != ref))
    log(f"  {len(outs)} calls, {bad} mismatching outputs")
    assert bad == 0
