"""The no-allocation post-scale entry point against the workspace one.

w8a8_gemm_postscale_noalloc is w8a8_gemm_postscale_ex with the split-K partial
sums in the library's fixed 64 MiB device array instead of a caller
workspace. Called through the raw C ABI, its output must equal the workspace
entry point's bit for bit (and the oracle's), on two calls in a row, the
second with a smaller input, so the second reads the array the first left
behind; explicit splits that do not fit the array are rejected before any
launch.
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

MIB64 = 64 << 20


def _operands(M, N, K, seed):
    qa = W.random_int8((M, K), seed)
    qw = W.random_int8((N, K), seed + 1)
    sa = W.random_scales((M,), seed + 2)
    sw = W.random_scales((N,), seed + 3, lo=1e-5, hi=1e-3)
    b = W.random_bits((N,), seed + 4, std=0.5)
    return qa, qw, sa, sw, b


def _noalloc_raw(qa, qw, sa, sw, bias, gelu, out, parts):
    M, K = qa.shape
    N = qw.shape[0]
    return w8.lib().w8a8_gemm_postscale_noalloc(
        qa.data_ptr(), K, qw.data_ptr(), K, sa.data_ptr(), sw.data_ptr(),
        None if bias is None else bias.data_ptr(), w8.W8A8_EPILOGUE_GELU if gelu else 0,
        out.data_ptr(), N, M, N, K, parts, torch.cuda.current_stream().cuda_stream)


# (M, N, K, parts): the library's choice on a split shape (8 parts of
# 256 x 5120 partial sums, 42 MB), then a smaller one; forced parts; the
# single pass
CASES = [
    ((256, 5120, 13824), 0, (129, 5120, 13824), 0),
    ((300, 768, 5248), 41, (77, 384, 11136), 64),
    ((512, 1280, 8192), 8, (33, 128, 8192), 1),
    ((1000, 1024, 2048), 1, (64, 1024, 4096), 0),
]


@pytest.mark.parametrize("first,p1,second,p2", CASES)
@pytest.mark.parametrize("bias_gelu", [(False, False), (True, False), (True, True)])
def test_noalloc_matches_workspace_entry(first, p1, second, p2, bias_gelu):
    with_bias, gelu = bias_gelu
    for (M, N, K), parts, seed in ((first, p1, 901), (second, p2, 911)):
        run = parts if parts > 0 else w8.splitk_parts(M, N, K)
        log(f"no-alloc {M}x{N}x{K} parts={parts} (runs {run}) bias={with_bias} gelu={gelu}")
        assert run * M * N * 4 <= MIB64 or run == 1
        qa, qw, sa, sw, b = _operands(M, N, K, seed)
        d = [to_dev(qa), to_dev(qw), to_dev(sa), to_dev(sw)]
        bias = bf16_to_dev(b) if with_bias else None
        ref_dev = w8.w8a8_gemm_postscale(*d, bias=bias, gelu=gelu, parts=run)
        out = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
        st = _noalloc_raw(*d, bias, gelu, out, parts)
        assert st == w8.W8A8_OK, w8.lib().w8a8_last_error()
        torch.cuda.synchronize()
        got = bf16_from_dev(out)
        assert np.array_equal(got, bf16_from_dev(ref_dev))
        acc = O.gemm_i32(qa, qw)
        bb = b if with_bias else None
        if gelu:
            ref = O.postscale_gelu_bf16(acc, sa, sw, bb)
        elif with_bias:
            ref = O.postscale_bias_bf16(acc, sa, sw, bb)
        else:
            ref = O.postscale_bf16(acc, sa, sw)
        assert np.array_equal(got, ref)


def test_noalloc_rejects_splits_beyond_the_scratch():
    # 2048 x 4096 partial sums are 32 MiB per part: 3 parts do not fit 64 MiB
    M, N, K = 2048, 4096, 4096
    qa, qw, sa, sw, _ = _operands(M, N, K, 921)
    d = [to_dev(qa), to_dev(qw), to_dev(sa), to_dev(sw)]
    out = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    st = _noalloc_raw(*d, None, False, out, 3)
    assert st == w8.W8A8_ERR_INVALID_ARGUMENT
    assert b"scratch" in w8.lib().w8a8_last_error()
    # the library's own choice stays within the array (here: the single pass)
    assert _noalloc_raw(*d, None, False, out, 0) == w8.W8A8_OK
    torch.cuda.synchronize()
    assert np.array_equal(bf16_from_dev(out), O.postscale_bf16(O.gemm_i32(qa, qw), sa, sw))
