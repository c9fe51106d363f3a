"""Int8Linear and the bias epilogue on the GPU, against the oracle.

"TurboDiffusion Integration Notes", section "Reused Components", W8A8 Linear
bullet: the Linear is replaced by an INT8 one that quantises the activation per
token on each call, with the weight quantised once. Its bias joins the fp32
post-scale epilogue (the oracle's postscale_bias_bf16) in the oracle's order
of fp32 operations, so the output is checked bit for bit like every other
post-scale output.
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

BIAS_SHAPES = [((64, 128, 256), 71), ((1, 128, 128), 72), ((1000, 384, 512), 73),
               ((257, 640, 1024), 74), ((129, 5120, 13824), 75), ((300, 256, 128), 76),
               # more tiles than CUs, N % 256 == 128, ragged M
               ((4096, 16384, 256), 77), ((8292, 4224, 128), 78), ((2000, 3200, 384), 79)]


def exact_check(got_bits, ref_bits, what):
    d = O.bf16_ulp_distance(got_bits, ref_bits)
    log(f"  {what}: max ulp {int(d.max()) if d.size else 0}, differing {int(np.sum(d != 0))}"
        f" of {d.size}")
    assert np.array_equal(got_bits, ref_bits)


def bias_bits(N: int, seed: int) -> np.ndarray:
    b = W.random_bits((N,), seed, std=0.5)
    specials = np.array([0x0000, 0x8000, 0x7F7F, 0x3F80, 0xBF80, 0x0001], np.uint16)
    b[:min(N, specials.size)] = specials[:min(N, specials.size)]      # +-0, max, +-1, denormal
    return b


@pytest.mark.parametrize("shape,seed", BIAS_SHAPES)
def test_gemm_postscale_bias(shape, seed):
    M, N, K = shape
    log(f"gemm_postscale_bias {shape}")
    qa = W.random_int8((M, K), seed)
    qw = W.random_int8((N, K), seed + 1)
    sa = W.random_scales((M,), seed + 2)
    sw = W.random_scales((N,), seed + 3, lo=1e-5, hi=1e-3)
    if M > 3:
        sa[3] = 0.0                       # output row = bias exactly
    b = bias_bits(N, seed + 4)
    out = w8.w8a8_gemm_postscale(to_dev(qa), to_dev(qw), to_dev(sa), to_dev(sw),
                                 bias=bf16_to_dev(b))
    torch.cuda.synchronize()
    got = bf16_from_dev(out)
    ref = O.postscale_bias_bf16(O.gemm_i32(qa, qw), sa, sw, b)
    exact_check(got, ref, "postscale+bias vs oracle")
    if M > 3:                             # 0 * s + b == b (as values: -0 + +0 is +0)
        assert np.array_equal(O.bf16_to_f32(got[3]), O.bf16_to_f32(b))


def test_gemm_postscale_bias_strided_and_guard():
    M, N, K = 300, 384, 512
    log("gemm_postscale_bias strided output, guard columns")
    qa = W.random_int8((M, K), 81)
    qw = W.random_int8((N, K), 82)
    sa = W.random_scales((M,), 83)
    sw = W.random_scales((N,), 84, lo=1e-5, hi=1e-3)
    b = bias_bits(N, 85)
    full = torch.full((M, N + 64), 1.5, dtype=torch.bfloat16, device="cuda")
    out = full[:, :N]
    w8.w8a8_gemm_postscale(to_dev(qa), to_dev(qw), to_dev(sa), to_dev(sw), out=out,
                           bias=bf16_to_dev(b))
    torch.cuda.synchronize()
    ref = O.postscale_bias_bf16(O.gemm_i32(qa, qw), sa, sw, b)
    exact_check(bf16_from_dev(out), ref, "strided postscale+bias")
    assert torch.all(full[:, N:] == 1.5)


@pytest.mark.parametrize("with_bias", [False, True])
def test_int8_linear_matches_oracle(with_bias):
    wl = W.WORKLOADS["tiny"]
    log(f"Int8Linear tiny workload, bias={with_bias}")
    x, wb = W.x_bits(wl), W.w_bits(wl)
    b = bias_bits(wl.N, 91) if with_bias else None
    lin = w8.Int8Linear(bf16_to_dev(wb), None if b is None else bf16_to_dev(b))
    assert lin.int8
    out = lin(bf16_to_dev(x))
    torch.cuda.synchronize()
    ref, qa_o, sa_o, qw_o, sw_o, _ = O.w8a8_linear(x, wb, b)
    assert np.array_equal(from_dev(lin.qweight), qw_o)
    assert np.array_equal(from_dev(lin.weight_scale).view(np.uint32), sw_o.view(np.uint32))
    exact_check(bf16_from_dev(out), ref, "Int8Linear vs oracle")


def test_int8_linear_batched_input_shape():
    log("Int8Linear on a [B, S, K] input")
    B, S, K, N = 3, 77, 512, 384
    xb = W.random_bits((B, S, K), 101)
    wb = W.random_bits((N, K), 102, std=0.02)
    b = bias_bits(N, 103)
    lin = w8.Int8Linear(bf16_to_dev(wb), bf16_to_dev(b))
    out = lin(bf16_to_dev(xb))
    torch.cuda.synchronize()
    assert out.shape == (B, S, N) and out.dtype == torch.bfloat16
    ref = O.w8a8_linear(xb.reshape(B * S, K), wb, b)[0]
    exact_check(bf16_from_dev(out).reshape(B * S, N), ref, "batched Int8Linear")
    empty = lin(torch.empty((0, K), dtype=torch.bfloat16, device="cuda"))
    assert empty.shape == (0, N)


def test_int8_linear_falls_back_on_unsupported_shapes():
    log("Int8Linear BF16 fallback for K % 128 != 0 and N % 128 != 0")
    for (N, K), seed in (((256, 200), 111), ((100, 256), 112)):
        wb = bf16_to_dev(W.random_bits((N, K), seed, std=0.05))
        bb = bf16_to_dev(W.random_bits((N,), seed + 1))
        lin = w8.Int8Linear(wb, bb)
        assert not lin.int8 and lin.qweight is None
        x = bf16_to_dev(W.random_bits((33, K), seed + 2))
        assert torch.equal(lin(x), torch.nn.functional.linear(x, wb, bb))


def test_replace_linear_with_int8():
    log("replace_linear_with_int8 on a small block")
    torch.manual_seed(5)
    block = torch.nn.Sequential(
        torch.nn.Linear(256, 512), torch.nn.GELU(),
        torch.nn.Sequential(torch.nn.Linear(512, 256, bias=False)),
        torch.nn.Linear(256, 100)).to(device="cuda", dtype=torch.bfloat16)
    ref_layers = [block[0], block[2][0], block[3]]
    n = w8.replace_linear_with_int8(block, select=lambda name, m: m.out_features % 128 == 0)
    assert n == 2
    assert isinstance(block[0], w8.Int8Linear) and isinstance(block[2][0], w8.Int8Linear)
    assert isinstance(block[3], torch.nn.Linear)
    x = bf16_to_dev(W.random_bits((65, 256), 121))
    with torch.no_grad():
        h = block[0](x)
        wb = bf16_from_dev(ref_layers[0].weight)
        bb = bf16_from_dev(ref_layers[0].bias)
        ref = O.w8a8_linear(bf16_from_dev(x), wb, bb)[0]
        exact_check(bf16_from_dev(h), ref, "replaced first layer")
        y = block(x)
    assert y.shape == (65, 100) and torch.isfinite(y.float()).all()


def test_int8_linear_gelu_activation():
    log("Int8Linear(activation='gelu') against the oracle, and its BF16 fallback")
    M, K, N = 300, 512, 1280
    x = W.random_bits((M, K), 171)
    wb = W.random_bits((N, K), 172, std=0.05)
    b = bias_bits(N, 173)
    lin = w8.Int8Linear(bf16_to_dev(wb), bf16_to_dev(b), activation="gelu")
    out = lin(bf16_to_dev(x))
    torch.cuda.synchronize()
    _, qa_o, sa_o, qw_o, sw_o, acc = O.w8a8_linear(x, wb, b)
    ref = O.postscale_gelu_bf16(acc, sa_o, sw_o, b)
    assert np.array_equal(bf16_from_dev(out), ref)
    fb = w8.Int8Linear(bf16_to_dev(W.random_bits((100, 256), 174)), activation="gelu")
    assert not fb.int8
    xs = bf16_to_dev(W.random_bits((7, 256), 175))
    assert torch.equal(fb(xs), torch.nn.functional.gelu(torch.nn.functional.linear(xs, fb.weight)))


# ---- NormInt8Linear: a norm fused with the Int8Linear's activation quant ----

def _norm_linear(norm, K, N, seed, affine=True):
    w = W.random_bits((N, K), seed, std=0.02)
    b = W.random_bits((N,), seed + 1, std=0.1)
    g = W.random_bits((K,), seed + 2, std=0.1, mean=1.0)
    beta = W.random_bits((K,), seed + 3, std=0.1) if (affine and norm == "layernorm") else None
    lin = w8.Int8Linear(bf16_to_dev(w), bf16_to_dev(b))
    gamma = g if (affine or norm == "rmsnorm") else None
    mod = w8.NormInt8Linear(lin, norm, None if gamma is None else bf16_to_dev(gamma),
                            None if beta is None else bf16_to_dev(beta), eps=1e-6)
    return mod, w, b, gamma, beta


@pytest.mark.parametrize("norm,affine,modulated", [("rmsnorm", True, False),
                                                   ("layernorm", True, True),
                                                   ("layernorm", False, True),
                                                   ("layernorm", True, False)])
def test_norm_int8_linear_matches_oracle(norm, affine, modulated):
    # the fused path: codes from the device's statistics, then the exact
    # GEMM and the bias epilogue, all bit for bit
    K, N = 512, 384
    log(f"NormInt8Linear {norm} affine={affine} modulated={modulated}")
    mod, w, b, g, beta = _norm_linear(norm, K, N, 301, affine)
    x = W.random_bits((2, 50, K), 305, std=1.5, mean=0.2)
    sc = W.random_bits((K,), 306, std=0.2) if modulated else None
    sh = W.random_bits((K,), 307, std=0.2) if modulated else None
    xd = bf16_to_dev(x)
    out = mod(xd, None if sc is None else bf16_to_dev(sc), None if sh is None else bf16_to_dev(sh))
    x2 = x.reshape(-1, K)
    if norm == "rmsnorm":
        _, _, r = w8.w8a8_rmsnorm_quant(bf16_to_dev(x2), bf16_to_dev(g), 1e-6)
        torch.cuda.synchronize()
        qa, sa, _ = O.rmsnorm_quant(x2, g, 1e-6, r=from_dev(r))
    else:
        _, _, mu, r = w8.w8a8_layernorm_quant(
            bf16_to_dev(x2), 1e-6, *[None if t is None else bf16_to_dev(t) for t in (g, beta, sc, sh)])
        torch.cuda.synchronize()
        qa, sa, _, _ = O.layernorm_quant(x2, 1e-6, g, beta, sc, sh, mu=from_dev(mu), r=from_dev(r))
    qw, sw = O.quantize_rows(w)
    ref = O.postscale_bias_bf16(O.gemm_i32(qa, qw), sa, sw, b)
    assert out.shape == (2, 50, N)
    exact_check(bf16_from_dev(out).reshape(-1, N), ref, f"{norm} module")


def test_norm_int8_linear_torch_norm_where_the_fused_kernel_does_not_fit():
    # LayerNorm rows longer than the fused kernels take (K = 8320): the norm
    # and modulation run as torch operations, then the Int8Linear quantises
    # their BF16 output; against the oracle with its own statistics
    K, N = 8320, 256
    log("NormInt8Linear layernorm at K = 8320 (torch norm, INT8 Linear)")
    mod, w, b, g, beta = _norm_linear("layernorm", K, N, 311)
    x = W.random_bits((40, K), 315, std=1.0)
    sc = W.random_bits((K,), 316, std=0.2)
    sh = W.random_bits((K,), 317, std=0.2)
    out = mod(bf16_to_dev(x), bf16_to_dev(sc), bf16_to_dev(sh))
    mu, r = O.layernorm_stats(x, 1e-6)
    y = O.modulate_bf16(O.layernorm_bf16(x, mu, r, g, beta), sc, sh)
    qa, sa = O.quantize_rows(y)
    qw, sw = O.quantize_rows(w)
    ref = O.postscale_bias_bf16(O.gemm_i32(qa, qw), sa, sw, b)
    exact_check(bf16_from_dev(out), ref, "torch norm + INT8 Linear")


def test_norm_int8_linear_bf16_fallback_and_argument_errors():
    # a weight the INT8 GEMM does not take (K = 200): torch's RMSNorm steps,
    # then torch's BF16 Linear
    K, N = 200, 128
    mod, w, b, g, _ = _norm_linear("rmsnorm", K, N, 321)
    assert not mod.linear.int8
    x = W.random_bits((30, K), 325)
    out = mod(bf16_to_dev(x))
    y = O.rmsnorm_bf16(x, g, O.rmsnorm_inv_rms(x, 1e-6))
    ref = torch.nn.functional.linear(bf16_to_dev(y), bf16_to_dev(w), bf16_to_dev(b))
    assert torch.equal(out, ref)
    lin = w8.Int8Linear(bf16_to_dev(w), bf16_to_dev(b))
    with pytest.raises(w8.W8A8Error):
        w8.NormInt8Linear(lin, "rmsnorm")                       # RMSNorm needs its gain
    with pytest.raises(w8.W8A8Error):
        w8.NormInt8Linear(lin, "batchnorm")
    with pytest.raises(w8.W8A8Error):
        mod(bf16_to_dev(x), mod_scale=bf16_to_dev(g))          # modulation follows LayerNorm only
    with pytest.raises(w8.W8A8Error):
        mod(bf16_to_dev(x).float())
