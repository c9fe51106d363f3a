"""Full-size parity: the workloads at their real sizes, through the C ABI, in
the same launch configuration bench.py times.

The device computes everything (weight quant at init, the per-call
activation quant or RMSNorm+quant, the GEMM). The oracle checks:
  * weight codes and scales: every element;
  * activation codes and scales: every element where the oracle finishes in
    a few seconds, else a seeded sample of rows plus every row of the ragged
    last tile;
  * GEMM output: the sampled rows (every row when M is small), recomputed by
    the oracle from the oracle's own codes (which were just shown equal to the
    device's), bit for bit.

The GEMM is called exactly as bench.py calls it: the post-scale family
through w8a8_gemm_postscale with the workload's bias and GELU and the
library's own choice of K parts (small_m splits K; the others run the single
pass in full-tile mode).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
import w8a8_int8_quantized_token_amd as w8
from tests.gpu_util import bf16_from_dev, bf16_to_dev, check_inv_rms, check_ln_mean, from_dev, log

pytestmark = pytest.mark.gpu

FULL_CHECK_ELEMS = 150_000_000      # compare every activation code below this size
N_SAMPLE = 192


def sample_rows(M: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    tail = np.arange(max(0, M - 300), M)                # covers the ragged last 256-row tile
    pick = rng.choice(M, size=min(N_SAMPLE, M), replace=False)
    return np.unique(np.concatenate([pick, tail, [0]]))


def exact_check(got, ref, what):
    d = O.bf16_ulp_distance(got, ref)
    log(f"  {what}: max ulp {int(d.max())}, differing {int(np.sum(d != 0))} of {d.size}")
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("name", ["square", "up_proj", "down_proj", "blockwise_small",
                                  "blockwise_large", "ln_up_proj", "up_proj_gelu", "small_m",
                                  "m1000"])
def test_workload_full_size(name):
    wl = W.WORKLOADS[name]
    M, N, K = wl.M, wl.N, wl.K
    log(f"full-size {name}: M={M} N={N} K={K}")
    x = W.x_bits(wl)
    wb = W.w_bits(wl)
    xd, wd = bf16_to_dev(x), bf16_to_dev(wb)

    # ---- init-time weight quant, checked in full --------------------------
    if wl.blockwise:
        qw, sw = w8.w8a8_quant_rows(wd, 128, 128)
        qw_o, sw_o = O.quantize_groups(wb, 128, 128)
    else:
        qw, sw = w8.w8a8_quant_rows(wd)
        qw_o, sw_o = O.quantize_rows(wb)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(qw), qw_o), "weight codes"
    assert np.array_equal(from_dev(sw).reshape(sw_o.shape).view(np.uint32), sw_o.view(np.uint32))
    del wd

    # ---- per-call path ----------------------------------------------------
    r = None
    if wl.norm:
        g = W.gamma_bits(wl)
        qa, sa, r = w8.w8a8_rmsnorm_quant(xd, bf16_to_dev(g), wl.eps)
    elif wl.layernorm:
        msc, msh = W.mod_bits(wl, "mod_scale"), W.mod_bits(wl, "mod_shift")
        qa, sa, mu, r = w8.w8a8_layernorm_quant(xd, wl.eps, mod_scale=bf16_to_dev(msc),
                                                mod_shift=bf16_to_dev(msh))
    elif wl.blockwise:
        qa, sa = w8.w8a8_quant_rows(xd, 1, 128)
    else:
        qa, sa = w8.w8a8_quant_rows(xd)
    bias = W.bias_bits(wl) if wl.bias_std > 0 else None
    if wl.blockwise:
        out = w8.w8a8_gemm_blockwise(qa, qw, sa, sw)
    else:
        parts = w8.splitk_parts(M, N, K)
        log(f"  post-scale GEMM: bias={bias is not None} gelu={wl.gelu} K parts {parts} "
            f"tile channels {w8.tile_channels(M, N, K)}")
        if name == "small_m":
            assert parts > 1
        out = w8.w8a8_gemm_postscale(qa, qw, sa, sw, bias=None if bias is None else bf16_to_dev(bias),
                                     gelu=wl.gelu)
    torch.cuda.synchronize()
    del xd

    rows = np.arange(M) if M * K <= FULL_CHECK_ELEMS else sample_rows(M, 7 + M)
    log(f"  checking {rows.size} of {M} activation rows")
    qa_h = from_dev(qa)[rows]
    sa_h = from_dev(sa).reshape(M, -1)[rows]
    xs = x[rows]
    if wl.norm:
        rg = from_dev(r)[rows]
        rref = O.rmsnorm_inv_rms(xs, wl.eps)
        check_inv_rms(rg, rref, K)
        qa_o, sa_o, _ = O.rmsnorm_quant(xs, g, wl.eps, r=rg)
    elif wl.layernorm:
        mg, rg = from_dev(mu)[rows], from_dev(r)[rows]
        mu_ref, r_ref = O.layernorm_stats(xs, wl.eps)
        check_ln_mean(mg, mu_ref, O.bf16_to_f32(xs))
        check_inv_rms(rg, r_ref, K)
        qa_o, sa_o, _, _ = O.layernorm_quant(xs, wl.eps, scale_bits=msc, shift_bits=msh,
                                             mu=mg, r=rg)
    elif wl.blockwise:
        qa_o, sa_o = O.quantize_groups(xs, 1, 128)
    else:
        qa_o, sa_o = O.quantize_rows(xs)
    assert np.array_equal(qa_h, qa_o), "activation codes"
    assert np.array_equal(sa_h.reshape(sa_o.shape).view(np.uint32), sa_o.view(np.uint32))

    # ---- GEMM on sampled rows --------------------------------------------
    if rows.size == M:
        grows = np.arange(M) if M <= 1024 else sample_rows(M, 11 + M)
        sel = grows
    else:
        grows = rows
        sel = np.arange(rows.size)
    got = bf16_from_dev(out)[grows]
    if wl.blockwise:
        ref = O.gemm_blockwise_bf16(qa_o[sel], sa_o.reshape(rows.size, -1)[sel], qw_o, sw_o)
    else:
        acc = O.gemm_i32(qa_o[sel], qw_o)
        sa_sel = sa_o.reshape(-1)[sel]
        if wl.gelu:
            ref = O.postscale_gelu_bf16(acc, sa_sel, sw_o, bias)
        elif bias is not None:
            ref = O.postscale_bias_bf16(acc, sa_sel, sw_o, bias)
        else:
            ref = O.postscale_bf16(acc, sa_sel, sw_o)
    exact_check(got, ref, f"{name} output on {grows.size} rows")
