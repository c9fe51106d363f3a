"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: INT8 codes, fp32 scales, INT32 accumulators and BF16 outputs
bit-exact. The BF16 outputs may by the pages' tolerance differ by 1 BF16 ulp,
but the kernels perform the oracle's fp32 operations in the oracle's order
(post-scale: two RN products then one RN rounding to BF16; blockwise: one fma
per K block in ascending order), so the results must be identical; the ulp
distance is still logged. RMSNorm's r (an fp32 reduction whose order is not fixed)
must be within (ceil(log2 K) + 4) * 2^-24 * r of the oracle's, and everything
downstream of r is compared bit for bit given the device's r.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
import w8a8_int8_quantized_token_amd as w8
from tests.gpu_util import (bf16_from_dev, bf16_to_dev, check_inv_rms, check_ln_mean, from_dev,
                            log, to_dev)

pytestmark = pytest.mark.gpu


def sync():
    torch.cuda.synchronize()


def special_rows(cols: int, seed: int) -> np.ndarray:
    """Rows that exercise the quantiser's edge cases."""
    rows = [np.zeros(cols, np.uint16)]                                   # all zero
    r = np.zeros(cols, np.uint16)
    r[cols // 3] = 0xC040                                                # single -3.0
    rows.append(r)
    rows.append(W.random_bits((cols,), seed, std=1e-33))                 # tiny: IEEE-divide path
    rows.append(W.random_bits((cols,), seed + 1, std=1e35))              # huge
    r = W.random_bits((cols,), seed + 2)
    r[0] = 0x42FE                                                        # absmax 127 -> scale 1
    r[1:6] = [0x3F00, 0x3FC0, 0x4020, 0xC020, 0x42FD]                    # 0.5 1.5 2.5 -2.5 126.5
    rows.append(np.where(np.abs(O.bf16_to_f32(r)) <= 127, r, 0).astype(np.uint16))
    r = np.zeros(cols, np.uint16)
    r[0], r[1] = 0x3E90, 0x3E10                                          # 0.28125, 0.140625
    rows.append(r)
    rows.append(np.full(cols, 0x0001, np.uint16))                        # smallest subnormal
    return np.stack(rows)


def check_quant(x_bits: np.ndarray, group=(1, None), ldx_pad=0, ldq_pad=0):
    rows, cols = x_bits.shape
    gr, gc = group
    gc_ = cols if gc is None else gc
    # device buffers with optional padding of the leading dimension
    xd_full = torch.zeros((rows, cols + ldx_pad), dtype=torch.bfloat16, device="cuda")
    xd_full[:, :cols] = bf16_to_dev(x_bits)
    xd = xd_full[:, :cols]
    qd_full = torch.full((rows + 2, cols + ldq_pad), 77, dtype=torch.int8, device="cuda")
    qd = qd_full[:rows, :cols]
    q, s = w8.w8a8_quant_rows(xd, gr, gc_, q=qd)
    sync()
    if gr == 1 and gc_ == cols:
        qo, so = O.quantize_rows(x_bits)
    else:
        qo, so = O.quantize_groups(x_bits, gr, gc_)
    qg = from_dev(q)
    sg = from_dev(s).reshape(so.shape)
    assert np.array_equal(qg, qo), f"codes differ at {np.argwhere(qg != qo)[:5]}"
    assert np.array_equal(sg.view(np.uint32), so.view(np.uint32)), "scales differ"
    # guard rows and padding untouched
    assert torch.all(qd_full[rows:] == 77)
    if ldq_pad:
        assert torch.all(qd_full[:rows, cols:] == 77)


# Up to 2048 rows of at least 8192 columns (1024 with (1, 128) groups) run
# several waves per row (the row's vectors spread over 2 to 16 waves, 4 to 1
# per lane; exact or with predicated lanes); other inputs one wave per row.
@pytest.mark.parametrize("shape,seed", [((64, 256), 1), ((3, 8), 2), ((1000, 5120), 3),
                                        ((129, 13824), 4), ((7, 20480), 5), ((333, 4096), 6),
                                        ((16, 1032), 7), ((100, 8200), 8), ((50, 12800), 9),
                                        ((2048, 8192), 10), ((2049, 8192), 12), ((5, 32768), 13)])
def test_quant_rows_per_token(shape, seed):
    log(f"quant_rows per-token {shape}")
    x = W.random_bits(shape, seed, std=1.0)
    if shape[0] >= 8:
        sp = special_rows(shape[1], seed + 100)
        x[: sp.shape[0]] = sp
    check_quant(x)


def test_quant_rows_workload_inputs():
    for name in ("tiny", "square"):
        wl = W.WORKLOADS[name]
        log(f"quant_rows workload {name}")
        check_quant(W.x_bits(wl))
        check_quant(W.w_bits(wl))


def test_quant_rows_strided():
    log("quant_rows strided")
    x = W.random_bits((300, 1024), 11)
    check_quant(x, ldx_pad=64, ldq_pad=16)
    check_quant(x, group=(1, 128), ldx_pad=8, ldq_pad=48)


@pytest.mark.parametrize("shape,group,seed", [((1000, 5120), (1, 128), 21), ((37, 384), (1, 128), 22),
                                              ((200, 384), (128, 128), 23),
                                              ((5120, 1024), (128, 128), 24),
                                              ((3, 20480), (1, 128), 25), ((1, 128), (1, 128), 26),
                                              ((40, 3200), (1, 128), 27), ((300, 1024), (1, 128), 28)])
def test_quant_groups(shape, group, seed):
    log(f"quant_rows group {group} {shape}")
    x = W.random_bits(shape, seed)
    x[:, 128:256] = W.random_bits((shape[0], 128), seed + 1, std=30.0) if shape[1] >= 256 else x[:, 128:256]
    if shape[0] >= 8 and shape[1] >= 256:
        x[2, :128] = 0
        x[3, 128:256] = W.random_bits((128,), seed + 2, std=1e-33)
    check_quant(x, group=group)


def test_quant_empty_rows():
    log("quant_rows rows=0")
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda")
    q, s = w8.w8a8_quant_rows(x)
    sync()
    assert q.shape == (0, 256)


@pytest.mark.slow
def test_quant_exhaustive_bf16_pairs():
    """Every (absmax, x) pair of finite BF16 values, both signs of x (about
    1.07e9 pairs), through the device quantiser and the oracle."""
    K = 4096
    per_row = K - 1
    amax_all = np.arange(1, 0x7F80, dtype=np.uint32)
    start = 0
    n_checked = 0
    while start < amax_all.size:
        rows = []
        b = start
        budget = 8192
        while b < amax_all.size and len(rows) < budget:
            ab = int(amax_all[b])
            cand = np.arange(1, ab + 1, dtype=np.uint32)
            cand = np.concatenate([cand, cand | 0x8000])
            n = -(-cand.size // per_row)
            pad = np.zeros(n * per_row, np.uint32)
            pad[: cand.size] = cand
            blk = np.empty((n, K), np.uint16)
            blk[:, 0] = ab
            blk[:, 1:] = pad.reshape(n, per_row)
            rows.append(blk)
            b += 1
        x = np.concatenate(rows)
        log(f"exhaustive amax bits [{start + 1:#06x}, {b:#06x}] rows={x.shape[0]}")
        check_quant(x)
        n_checked += x.shape[0] * per_row
        start = b
    assert n_checked > 1e9


def test_rmsnorm_quant():
    # full rows of 1, 3, 4, 5, 6 and 8 vectors per lane (the fp32-resident
    # kernel), 27 and 32 (packed rows), ragged rows, few rows and more rows than
    # the persistent grid covers in one pass
    for shape, seed in (((64, 256), 31), ((2048, 4096), 32), ((100, 13824), 33), ((5, 16384), 34),
                        ((3, 8), 35), ((777, 2048), 36), ((3, 512), 37), ((40000, 512), 38),
                        ((70, 1536), 39), ((50, 2560), 40), ((300, 3072), 41), ((33, 1000), 42),
                        ((5000, 4096), 43)):
        log(f"rmsnorm_quant {shape}")
        x = W.random_bits(shape, seed)
        if shape[0] >= 8:
            x[0] = 0                                                  # r = 1/sqrt(eps)
            x[1] = 0x4040                                             # constant 3.0
            x[2] = W.random_bits((shape[1],), seed + 1, std=1e-3)     # eps matters
            x[3] = W.random_bits((shape[1],), seed + 2, std=300.0)
            x[4] = W.random_bits((shape[1],), seed + 4, std=1e25)     # squares overflow fp32
            x[5] = W.random_bits((shape[1],), seed + 5, std=1e-22)    # squares below fp32 normals
        g = W.random_bits((shape[1],), seed + 3, std=0.1, mean=1.0)
        for gamma, eps in ((g, 1e-6), (np.zeros_like(g), 1e-6), (g, 0.0)):
            xs = x if eps > 0 else x[1:]                              # eps 0: no all-zero row
            q, s, r = w8.w8a8_rmsnorm_quant(bf16_to_dev(xs), bf16_to_dev(gamma), eps)
            sync()
            rg = from_dev(r)
            err = check_inv_rms(rg, O.rmsnorm_inv_rms(xs, eps), shape[1])
            log(f"  eps {eps}: inv_rms max error {err:.2f} x 2^-24 r")
            qo, so, _ = O.rmsnorm_quant(xs, gamma, eps, r=rg)
            assert np.array_equal(from_dev(q), qo)
            assert np.array_equal(from_dev(s).view(np.uint32), so.view(np.uint32))


def test_rmsnorm_quant_no_inv_rms_and_stride():
    log("rmsnorm_quant strided, no inv_rms")
    x = W.random_bits((64, 4096), 41)
    g = W.random_bits((4096,), 42, std=0.1, mean=1.0)
    xd_full = torch.zeros((64, 4096 + 64), dtype=torch.bfloat16, device="cuda")
    xd_full[:, :4096] = bf16_to_dev(x)
    q, s, r = w8.w8a8_rmsnorm_quant(xd_full[:, :4096], bf16_to_dev(g), 1e-6, inv_rms=False)
    q2, s2, r2 = w8.w8a8_rmsnorm_quant(bf16_to_dev(x), bf16_to_dev(g), 1e-6)
    sync()
    assert r is None
    assert torch.equal(q, q2) and torch.equal(s, s2)


def layernorm_rows(shape, seed):
    x = W.random_bits(shape, seed)
    rows, K = shape
    if rows >= 8:
        x[0] = 0                                                     # zero row
        x[1] = 0x4040                                                # constant 3.0
        x[2] = W.random_bits((K,), seed + 1, std=1.0, mean=50.0)     # mean dominates
        x[3] = W.random_bits((K,), seed + 2, std=1e-3)               # eps matters
        x[4] = W.random_bits((K,), seed + 3, std=1e25)               # squares overflow fp32
        x[5] = W.random_bits((K,), seed + 4, std=1e-22)              # squares below normals
    return x


@pytest.mark.parametrize("shape,seed", [((64, 256), 81), ((2048, 4096), 82), ((100, 5120), 83),
                                        ((5, 8192), 84), ((3, 8), 85), ((777, 2048), 86),
                                        ((40, 1000), 87), ((9, 6144), 88), ((300, 3072), 89),
                                        ((20000, 256), 90), ((5000, 4096), 91), ((60, 2560), 92),
                                        ((50, 1536), 93), ((3000, 5120), 94), ((7, 4800), 95)])
def test_layernorm_quant(shape, seed):
    log(f"layernorm_quant {shape}")
    x = layernorm_rows(shape, seed)
    K = shape[1]
    g = W.random_bits((K,), seed + 10, std=0.1, mean=1.0)
    b = W.random_bits((K,), seed + 11, std=0.1)
    sc = W.random_bits((K,), seed + 12, std=0.2)
    sh = W.random_bits((K,), seed + 13, std=0.2)
    for opts in (dict(), dict(g=g, b=b), dict(g=g, b=b, sc=sc, sh=sh), dict(sc=sc, sh=sh)):
        for eps in (1e-6, 1e-5, 0.0):
            # eps 0: no zero-variance row (its r would be infinite)
            xs = x if eps > 0 or shape[0] < 8 else x[2:]
            xf = O.bf16_to_f32(xs)
            dev = {k: bf16_to_dev(v) for k, v in opts.items()}
            q, s, mu, r = w8.w8a8_layernorm_quant(bf16_to_dev(xs), eps, dev.get("g"), dev.get("b"),
                                                  dev.get("sc"), dev.get("sh"))
            sync()
            mg, rg = from_dev(mu), from_dev(r)
            mu_ref, r_ref = O.layernorm_stats(xs, eps)
            em = check_ln_mean(mg, mu_ref, xf)
            er = check_inv_rms(rg, r_ref, K)
            qo, so, _, _ = O.layernorm_quant(xs, eps, opts.get("g"), opts.get("b"), opts.get("sc"),
                                             opts.get("sh"), mu=mg, r=rg)
            assert np.array_equal(from_dev(q), qo), f"codes {sorted(opts)} eps {eps}"
            assert np.array_equal(from_dev(s).view(np.uint32), so.view(np.uint32))
        log(f"  {sorted(opts)}: mean error {em:.2f}, r error {er:.2f} (x 2^-24)")


def test_layernorm_quant_long_rows_unsupported():
    x = torch.zeros((2, 8200), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(w8.W8A8Unsupported):
        w8.w8a8_layernorm_quant(x, 1e-6)


def test_layernorm_quant_strided_no_stats():
    log("layernorm_quant strided, no stats")
    x = W.random_bits((64, 4096), 91)
    sc = W.random_bits((4096,), 92, std=0.2)
    xd_full = torch.zeros((64, 4096 + 64), dtype=torch.bfloat16, device="cuda")
    xd_full[:, :4096] = bf16_to_dev(x)
    q_full = torch.full((64, 4096 + 128), 77, dtype=torch.int8, device="cuda")
    q, s, mu, r = w8.w8a8_layernorm_quant(xd_full[:, :4096], 1e-6, mod_scale=bf16_to_dev(sc),
                                          q=q_full[:, :4096], stats=False)
    q2, s2, _, _ = w8.w8a8_layernorm_quant(bf16_to_dev(x), 1e-6, mod_scale=bf16_to_dev(sc))
    sync()
    assert mu is None and r is None
    assert torch.equal(q, q2) and torch.equal(s, s2)
    assert torch.all(q_full[:, 4096:] == 77)


GEMM_SHAPES = [((64, 128, 256), 51), ((1, 128, 128), 52), ((1000, 384, 512), 53),
               ((257, 640, 1024), 54), ((4096, 4096, 4096), 55), ((129, 5120, 13824), 56),
               ((300, 256, 128), 57), ((513, 1152, 640), 58),
               # more tiles than CUs: several tiles per persistent workgroup
               ((4096, 16384, 256), 59), ((8292, 4096, 128), 60), ((2000, 3200, 384), 66),
               # one whole tile; one row short of it (clamped loads)
               ((256, 256, 256), 80), ((255, 4096, 512), 81),
               # fewer than 16 tokens: clamped rows on one or both sides of the
               # store's swap between lanes 8 rows apart
               ((7, 256, 256), 82), ((9, 384, 128), 83), ((15, 1280, 384), 84)]


@pytest.mark.parametrize("shape,seed", GEMM_SHAPES)
def test_gemm_i32(shape, seed):
    M, N, K = shape
    log(f"gemm_i32 {shape}")
    qa = W.random_int8((M, K), seed)
    qw = W.random_int8((N, K), seed + 1)
    if M >= 2 and N >= 2:
        qa[0] = 127
        qw[0] = -127
        qw[1] = 127
    out = w8.w8a8_gemm_i32(to_dev(qa), to_dev(qw))
    sync()
    ref = O.gemm_i32(qa, qw)
    assert np.array_equal(from_dev(out), ref)


def exact_check(got_bits, ref_bits, what):
    d = O.bf16_ulp_distance(got_bits, ref_bits)
    log(f"  {what}: max ulp {int(d.max()) if d.size else 0}, differing {int(np.sum(d != 0))}"
        f" of {d.size}")
    assert np.array_equal(got_bits, ref_bits)
    return d


@pytest.mark.parametrize("shape,seed", GEMM_SHAPES)
def test_gemm_postscale(shape, seed):
    M, N, K = shape
    log(f"gemm_postscale {shape}")
    qa = W.random_int8((M, K), seed)
    qw = W.random_int8((N, K), seed + 1)
    sa = W.random_scales((M,), seed + 2)
    sw = W.random_scales((N,), seed + 3, lo=1e-5, hi=1e-3)
    if M > 3:
        sa[3] = 0.0
    out = w8.w8a8_gemm_postscale(to_dev(qa), to_dev(qw), to_dev(sa), to_dev(sw))
    sync()
    ref = O.postscale_bf16(O.gemm_i32(qa, qw), sa, sw)
    exact_check(bf16_from_dev(out), ref, "postscale vs oracle")


BLOCKWISE_SHAPES = [((64, 128, 256), 61), ((1000, 5120, 5120), 62), ((300, 256, 384), 63),
                    ((1, 128, 128), 64), ((257, 640, 1024), 65),
                    # more tiles than CUs, ragged M, N % 256 == 128
                    ((8292, 1152, 256), 67), ((4100, 4096, 384), 68), ((129, 384, 13824), 69),
                    # 128 x 160 tiles (few tokens, long K): N % 160 = 0, 32 and 96
                    ((300, 2560, 8192), 70), ((200, 1152, 8192), 71), ((100, 4096, 8192), 72)]


def test_parity_shapes_cover_both_tilings():
    # the shape lists must keep exercising both the 256-channel and the
    # 128 x 160 kernels (the library picks by a cost model, for 256 CUs here)
    post = [w8.tile_channels(*s) for s, _ in GEMM_SHAPES if w8.splitk_parts(*s) == 1]
    block = [w8.tile_channels(*s, blockwise=True) for s, _ in BLOCKWISE_SHAPES]
    assert post.count(160) >= 3 and post.count(256) >= 3, post
    assert block.count(160) >= 3 and block.count(256) >= 3, block


@pytest.mark.parametrize("shape,seed", BLOCKWISE_SHAPES)
def test_gemm_blockwise(shape, seed):
    M, N, K = shape
    log(f"gemm_blockwise {shape}")
    qa = W.random_int8((M, K), seed)
    qw = W.random_int8((N, K), seed + 1)
    sa = W.random_scales((M, K // 128), seed + 2)
    sw = W.random_scales((N // 128, K // 128), seed + 3, lo=1e-5, hi=1e-3)
    if M > 5 and K >= 256:
        sa[5, 1] = 0.0          # one zero block scale inside a row
        sa[4, :] = 0.0          # an all-zero row
    out = w8.w8a8_gemm_blockwise(to_dev(qa), to_dev(qw), to_dev(sa), to_dev(sw))
    sync()
    ref = O.gemm_blockwise_bf16(qa, sa, qw, sw)
    exact_check(bf16_from_dev(out), ref, "blockwise vs oracle")


def test_gemm_blockwise_strides_and_guard():
    log("gemm_blockwise strided operands / guard")
    M, N, K = 200, 384, 512
    qa = W.random_int8((M, K), 75)
    qw = W.random_int8((N, K), 76)
    sa = W.random_scales((M, K // 128), 77)
    sw = W.random_scales((N // 128, K // 128), 78, lo=1e-5, hi=1e-3)
    a_full = torch.zeros((M, K + 256), dtype=torch.int8, device="cuda")
    a_full[:, :K] = to_dev(qa)
    w_full = torch.zeros((N, K + 128), dtype=torch.int8, device="cuda")
    w_full[:, :K] = to_dev(qw)
    out_full = torch.full((M + 8, N + 64), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    out = out_full[:M, :N]
    w8.w8a8_gemm_blockwise(a_full[:, :K], w_full[:, :K], to_dev(sa), to_dev(sw), out=out)
    sync()
    ref = O.gemm_blockwise_bf16(qa, sa, qw, sw)
    exact_check(bf16_from_dev(out), ref, "strided blockwise vs oracle")
    guard = bf16_from_dev(out_full)
    assert np.all(guard[M:] == 0xFFFF) and np.all(guard[:M, N:] == 0xFFFF)


def test_gemm_guard_rows_and_strides():
    log("gemm guard rows / strides / M=0")
    M, N, K = 100, 256, 384
    qa = W.random_int8((M, K), 71)
    qw = W.random_int8((N, K), 72)
    sa = W.random_scales((M,), 73)
    sw = W.random_scales((N,), 74)
    a_full = torch.zeros((M, K + 128), dtype=torch.int8, device="cuda")
    a_full[:, :K] = to_dev(qa)
    out_full = torch.full((M + 8, N + 64), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    out = out_full[:M, :N]
    w8.w8a8_gemm_postscale(a_full[:, :K], to_dev(qw), to_dev(sa), to_dev(sw), out=out)
    sync()
    ref = O.postscale_bf16(O.gemm_i32(qa, qw), sa, sw)
    assert np.array_equal(bf16_from_dev(out), ref)
    guard = bf16_from_dev(out_full)
    assert np.all(guard[M:] == 0xFFFF) and np.all(guard[:M, N:] == 0xFFFF)
    # M = 0 is a no-op
    empty = w8.w8a8_gemm_postscale(torch.zeros((0, K), dtype=torch.int8, device="cuda"),
                                   to_dev(qw), to_dev(sa[:0].copy()), to_dev(sw))
    sync()
    assert empty.shape == (0, N)


def test_unsupported_shape_raises():
    qa = torch.zeros((4, 200), dtype=torch.int8, device="cuda")
    with pytest.raises(w8.W8A8Unsupported):
        w8.w8a8_gemm_i32(qa, qa)


def test_tiny_linear_end_to_end():
    log("tiny W8A8 linear end to end")
    wl = W.WORKLOADS["tiny"]
    x, wb = W.x_bits(wl), W.w_bits(wl)
    qw, sw = w8.w8a8_quant_rows(bf16_to_dev(wb))
    qa, sa = w8.w8a8_quant_rows(bf16_to_dev(x))
    out = w8.w8a8_gemm_postscale(qa, qw, sa, sw)
    sync()
    ref, qa_o, sa_o, qw_o, sw_o, acc = O.w8a8_linear(x, wb)
    assert np.array_equal(from_dev(qa), qa_o) and np.array_equal(from_dev(qw), qw_o)
    exact_check(bf16_from_dev(out), ref, "tiny linear")


def test_max_k_int32_extremes():
    """K = W8A8_MAX_K (133120, the largest multiple of 128 with 127^2 K < 2^31):
    rows of +127 and -127 against rows of +127 and -127 reach the INT32
    extremes +-2147123200 exactly, through the INT32 export (one pass over the
    whole K) and the post-scale path (split over K at this size)."""
    M, N, K = 16, 128, w8.W8A8_MAX_K
    log(f"K = W8A8_MAX_K: {M}x{N}x{K}, split-K parts {w8.splitk_parts(M, N, K)}")
    qa = W.random_int8((M, K), 201)
    qw = W.random_int8((N, K), 202)
    qa[0], qa[1] = 127, -127
    qw[0], qw[1] = 127, -127
    sa = W.random_scales((M,), 203)
    sw = W.random_scales((N,), 204, lo=1e-5, hi=1e-3)
    ref = O.gemm_i32(qa, qw)
    assert ref[0, 0] == 127 * 127 * K and ref[1, 0] == -127 * 127 * K and ref[1, 1] == 127 * 127 * K
    got = from_dev(w8.w8a8_gemm_i32(to_dev(qa), to_dev(qw)))
    sync()
    assert np.array_equal(got, ref)
    out = w8.w8a8_gemm_postscale(to_dev(qa), to_dev(qw), to_dev(sa), to_dev(sw))
    sync()
    assert np.array_equal(bf16_from_dev(out), O.postscale_bf16(ref, sa, sw))
