"""The up projection with its FFN activation (GELU, erf form) on the GPU,
against the oracle (R13: GELU of the BF16 post-scale output, rounded once).

The device evaluates GELU from fp32 erfcf (a table of it in the fused
epilogue, erfcf itself in the split-K pass) and rounds to BF16. Over every
finite BF16 input that equals the correctly rounded value (the first two
tests, which cover GELU's whole input domain on both paths), so every GELU
output below is required bit for bit; then the rest of the feed-forward chain (per-token
quantisation of the GELU output, the down projection) is checked exactly.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
import w8a8_int8_quantized_token_amd as w8
from tests.gpu_util import bf16_from_dev, bf16_to_dev, from_dev, log, to_dev

pytestmark = pytest.mark.gpu


def exact_report(got, ref, what):
    d = O.bf16_ulp_distance(got, ref)
    log(f"  {what}: max ulp {int(d.max()) if d.size else 0} over {d.size}")
    assert np.array_equal(got, ref)


def test_gelu_every_bf16_value():
    """acc = 1 everywhere and w_scale = 1, so row m's output is GELU of the
    BF16 value a_scale[m]: one row per BF16 bit pattern, the non-finite ones
    included (y/2 * erfc(-y / sqrt(2)) gives +inf for +inf and NaN for -inf
    and NaN)."""
    log("GELU epilogue over all 65536 BF16 patterns")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = O.bf16_to_f32(bits)
    finite = np.isfinite(vals)
    sa = vals.astype(np.float32)
    M, N, K = 65536, 128, 128
    qa = np.zeros((M, K), np.int8)
    qa[:, 0] = 1
    qw = np.zeros((N, K), np.int8)
    qw[:, 0] = 1
    sw = np.ones(N, np.float32)
    out = w8.w8a8_gemm_postscale(to_dev(qa), to_dev(qw), to_dev(sa), to_dev(sw), gelu=True)
    torch.cuda.synchronize()
    got = bf16_from_dev(out)
    assert np.all(got == got[:, :1])                       # every column the same
    exact_report(got[finite, 0], O.gelu_bf16(bits[finite]), "GELU of every finite BF16 value")
    g = O.bf16_to_f32(got[:, 0])
    assert g[0x7F80] == np.inf                             # +inf
    assert np.isnan(g[0xFF80])                             # -inf
    nan_in = np.isnan(vals)
    assert nan_in.sum() == 254 and np.all(np.isnan(g[nan_in]))


def test_gelu_every_bf16_value_split_k():
    """The same over the split-K path, whose reduce pass computes GELU with
    erfcf itself: forced to 2 parts."""
    log("GELU in the split-K reduce pass over all 65536 BF16 patterns")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = O.bf16_to_f32(bits)
    finite = np.isfinite(vals)
    M, N, K = 65536, 128, 256
    qa = np.zeros((M, K), np.int8)
    qa[:, 0] = 1
    qw = np.zeros((N, K), np.int8)
    qw[:, 0] = 1
    out = w8.w8a8_gemm_postscale(to_dev(qa), to_dev(qw), to_dev(vals.astype(np.float32)),
                                 to_dev(np.ones(N, np.float32)), gelu=True, parts=2)
    torch.cuda.synchronize()
    got = bf16_from_dev(out)
    assert np.all(got == got[:, :1])
    bad = int(np.count_nonzero(got[finite, 0] != O.gelu_bf16(bits[finite])))
    g = O.bf16_to_f32(got[:, 0])
    log(f"  split-K GELU mismatches {bad}")
    assert bad == 0
    assert g[0x7F80] == np.inf and np.isnan(g[0xFF80]) and np.all(np.isnan(g[np.isnan(vals)]))


SHAPES = [((64, 128, 256), 151), ((1000, 384, 512), 152), ((257, 640, 1024), 153),
          ((2048, 4096, 1024), 154), ((300, 1152, 640), 155),
          ((129, 5120, 13824), 156),          # split over K
          ((4100, 1280, 384), 157)]


@pytest.mark.parametrize("with_bias", [False, True])
@pytest.mark.parametrize("shape,seed", SHAPES)
def test_gemm_postscale_gelu(shape, seed, with_bias):
    M, N, K = shape
    log(f"post-scale + GELU {shape} bias={with_bias}")
    qa = W.random_int8((M, K), seed)
    qw = W.random_int8((N, K), seed + 1)
    sa = W.random_scales((M,), seed + 2)
    sw = W.random_scales((N,), seed + 3, lo=1e-5, hi=1e-3)
    b = W.random_bits((N,), seed + 4, std=2.0) if with_bias else None
    out = w8.w8a8_gemm_postscale(to_dev(qa), to_dev(qw), to_dev(sa), to_dev(sw),
                                 bias=None if b is None else bf16_to_dev(b), gelu=True)
    torch.cuda.synchronize()
    ref = O.postscale_gelu_bf16(O.gemm_i32(qa, qw), sa, sw, b)
    exact_report(bf16_from_dev(out), ref, "post-scale + GELU vs oracle")


@pytest.mark.parametrize("shape,seed", [((600, 1280, 384), 158),    # 256 x 256 tiles, full-tile mode
                                        ((70, 128, 256), 159),      # one clamped tile
                                        ((1000, 5120, 1024), 160)]) # 128 x 160 tiles
def test_gemm_postscale_gelu_strided_output(shape, seed):
    """Bias + GELU into a column slice of a wider buffer: the stores follow
    the output's row stride and the columns past N keep their contents."""
    M, N, K = shape
    log(f"post-scale + bias + GELU into a strided output {shape}")
    assert w8.lib().w8a8_gemm_tile_channels(M, N, K, 0) == (160 if M == 1000 else 256)
    qa = W.random_int8((M, K), seed)
    qw = W.random_int8((N, K), seed + 1)
    sa = W.random_scales((M,), seed + 2)
    sw = W.random_scales((N,), seed + 3, lo=1e-5, hi=1e-3)
    b = W.random_bits((N,), seed + 4, std=2.0)
    full = torch.full((M, N + 64), -7.0, dtype=torch.bfloat16, device="cuda")
    w8.w8a8_gemm_postscale(to_dev(qa), to_dev(qw), to_dev(sa), to_dev(sw), bias=bf16_to_dev(b),
                           gelu=True, out=full[:, :N])
    torch.cuda.synchronize()
    ref = O.postscale_gelu_bf16(O.gemm_i32(qa, qw), sa, sw, b)
    exact_report(bf16_from_dev(full[:, :N]), ref, "strided post-scale + bias + GELU vs oracle")
    assert torch.all(full[:, N:] == -7.0)


def test_ffn_chain_up_gelu_quant_down():
    """x -> per-token quant -> up projection + GELU -> per-token quant -> down
    projection; each step checked from the device's own inputs."""
    M, D, H = 1000, 512, 2048
    log(f"FFN chain M={M} D={D} H={H}")
    x = W.random_bits((M, D), 161)
    w1 = W.random_bits((H, D), 162, std=0.05)
    b1 = W.random_bits((H,), 163, std=0.5)
    w2 = W.random_bits((D, H), 164, std=0.02)
    q1, s1 = w8.w8a8_quant_rows(bf16_to_dev(w1))
    q2, s2 = w8.w8a8_quant_rows(bf16_to_dev(w2))
    qx, sx = w8.w8a8_quant_rows(bf16_to_dev(x))
    h = w8.w8a8_gemm_postscale(qx, q1, sx, s1, bias=bf16_to_dev(b1), gelu=True)
    qh, sh = w8.w8a8_quant_rows(h)
    y = w8.w8a8_gemm_postscale(qh, q2, sh, s2)
    torch.cuda.synchronize()
    qx_o, sx_o = O.quantize_rows(x)
    q1_o, s1_o = O.quantize_rows(w1)
    q2_o, s2_o = O.quantize_rows(w2)
    assert np.array_equal(from_dev(qx), qx_o) and np.array_equal(from_dev(q1), q1_o)
    h_ref = O.postscale_gelu_bf16(O.gemm_i32(qx_o, q1_o), sx_o, s1_o, b1)
    h_got = bf16_from_dev(h)
    exact_report(h_got, h_ref, "GELU output")
    qh_o, sh_o = O.quantize_rows(h_got)                     # from the device's h
    assert np.array_equal(from_dev(qh), qh_o)
    assert np.array_equal(from_dev(sh).view(np.uint32), sh_o.view(np.uint32))
    y_ref = O.postscale_bf16(O.gemm_i32(qh_o, q2_o), sh_o, s2_o)
    assert np.array_equal(bf16_from_dev(y), y_ref)
