"""Host-side checks of the C ABI (no GPU needed, nothing is launched).

The library must load, export every entry point include/w8a8.h declares, and
reject invalid or unsupported arguments on the host with the documented
status, before anything reaches a GPU. Every call here fails validation, so
the fake pointers are never dereferenced.
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest
import torch

import w8a8_int8_quantized_token_amd as w8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w8a8.h")

OK, INVALID, UNSUPPORTED = 0, 1, 2
P = 0x10000          # fake, 64 KiB-aligned "device" addresses (never touched)
Q = 0x40000000
S = 0x50000000
O = 0x60000000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w8a8_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == {"w8a8_quant_rows", "w8a8_rmsnorm_quant", "w8a8_layernorm_quant",
                          "w8a8_gemm_postscale", "w8a8_gemm_postscale_bias",
                          "w8a8_gemm_postscale_gelu",
                          "w8a8_gemm_blockwise", "w8a8_gemm_i32", "w8a8_status_string",
                          "w8a8_last_error", "w8a8_version", "w8a8_gemm_splitk_parts",
                          "w8a8_gemm_postscale_ex", "w8a8_gemm_postscale_workspace_size",
                          "w8a8_gemm_postscale_noalloc", "w8a8_gemm_tile_channels"}
    raw = ctypes.CDLL(w8.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    assert set(names) == set(w8.EXPORTED_SYMBOLS)


def test_status_strings():
    lib = w8.lib()
    assert lib.w8a8_status_string(0) == b"ok"
    assert b"unsupported" in lib.w8a8_status_string(2)
    assert lib.w8a8_status_string(99) == b"unknown status"
    assert w8.w8a8_version().startswith("w8a8-gfx950")


def quant(x=P, rows=64, cols=256, ldx=256, gr=1, gc=256, q=Q, ldq=256, s=S):
    return w8.lib().w8a8_quant_rows(x, rows, cols, ldx, gr, gc, q, ldq, s, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(x=None), INVALID),
    (dict(q=None), INVALID),
    (dict(s=None), INVALID),
    (dict(rows=-1), INVALID),
    (dict(ldx=128), INVALID),
    (dict(ldq=128), INVALID),
    (dict(cols=0, gc=0), UNSUPPORTED),
    (dict(cols=100, ldx=104, ldq=112, gc=100), UNSUPPORTED),        # cols % 8
    (dict(gr=2, gc=256), UNSUPPORTED),                              # unsupported group
    (dict(gr=1, gc=64), UNSUPPORTED),
    (dict(cols=264, ldx=264, ldq=272, gc=128), UNSUPPORTED),        # 128-group, cols % 128
    (dict(x=P + 8), UNSUPPORTED),                                   # misaligned
    (dict(q=Q + 4), UNSUPPORTED),
    (dict(ldx=260), UNSUPPORTED),
    (dict(ldq=260), UNSUPPORTED),
    (dict(s=S + 2), UNSUPPORTED),
    (dict(q=P + 1024), INVALID),                                    # q overlaps x
    (dict(s=P + 4096), INVALID),                                    # scale overlaps x
])
def test_quant_rows_rejects(kwargs, status):
    assert quant(**kwargs) == status
    assert w8.lib().w8a8_last_error() != b""


def rms(x=P, gamma=0x30000000, eps=1e-6, rows=8, cols=256, ldx=256, q=Q, ldq=256, s=S,
        inv=0x70000000):
    return w8.lib().w8a8_rmsnorm_quant(x, gamma, eps, rows, cols, ldx, q, ldq, s, inv, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(gamma=None), INVALID),
    (dict(eps=float("nan")), INVALID),
    (dict(eps=float("inf")), INVALID),
    (dict(eps=-1.0), INVALID),
    (dict(gamma=0x30000008), UNSUPPORTED),
    (dict(inv=0x70000002), UNSUPPORTED),
    (dict(cols=16392, ldx=16392, ldq=16400), UNSUPPORTED),          # longer than supported
    (dict(inv=S), INVALID),                                         # inv_rms aliases scale
])
def test_rmsnorm_quant_rejects(kwargs, status):
    assert rms(**kwargs) == status


def test_last_error_is_per_thread():
    # the description of a failed call belongs to the calling thread: another
    # thread starts with none and its own failures leave this one's untouched
    import threading
    assert quant(x=None) == INVALID
    mine = w8.lib().w8a8_last_error()
    assert mine != b""
    seen = {}

    def other():
        seen["before"] = w8.lib().w8a8_last_error()
        seen["status"] = rms(gamma=None)
        seen["after"] = w8.lib().w8a8_last_error()

    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert seen["before"] == b"" and seen["status"] == INVALID
    assert seen["after"] != b"" and seen["after"] != mine
    assert w8.lib().w8a8_last_error() == mine


def ln(x=P, gamma=0x30000000, beta=0x30100000, sc=0x30200000, sh=0x30300000, eps=1e-6, rows=8,
       cols=256, ldx=256, q=Q, ldq=256, s=S, mean=0x70000000, rstd=0x70100000):
    return w8.lib().w8a8_layernorm_quant(x, gamma, beta, sc, sh, eps, rows, cols, ldx, q, ldq, s,
                                         mean, rstd, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(x=None), INVALID),
    (dict(s=None), INVALID),
    (dict(eps=float("nan")), INVALID),
    (dict(eps=-1.0), INVALID),
    (dict(gamma=0x30000008), UNSUPPORTED),
    (dict(beta=0x30100004), UNSUPPORTED),
    (dict(sc=0x30200002), UNSUPPORTED),
    (dict(sh=0x30300008), UNSUPPORTED),
    (dict(mean=0x70000002), UNSUPPORTED),
    (dict(cols=8200, ldx=8200, ldq=8200), UNSUPPORTED),             # longer than supported
    (dict(mean=S), INVALID),                                        # mean aliases scale
    (dict(rstd=Q + 64), INVALID),                                   # rstd inside q
    (dict(q=0x30300000 - 256), INVALID),                            # q overlaps mod_shift
    (dict(mean=0x70000000, rstd=0x70000000 + 16), INVALID),         # mean and rstd overlap
])
def test_layernorm_quant_rejects(kwargs, status):
    assert ln(**kwargs) == status
    assert w8.lib().w8a8_last_error() != b""


def test_layernorm_quant_optional_vectors_may_be_null():
    # with every optional pointer null the call only fails for its real error
    assert ln(gamma=None, beta=None, sc=None, sh=None, mean=None, rstd=None, eps=-1.0) == INVALID


def gemm(fn="w8a8_gemm_postscale", a=P, lda=256, w=Q, ldw=256, sa=S, sw=S + 0x100000,
         out=O, ldo=128, M=64, N=128, K=256):
    f = getattr(w8.lib(), fn)
    if fn in ("w8a8_gemm_postscale_bias", "w8a8_gemm_postscale_gelu"):
        return f(a, lda, w, ldw, sa, sw, S + 0x200000, out, ldo, M, N, K, None)
    if fn == "w8a8_gemm_i32":
        return f(a, lda, w, ldw, out, ldo, M, N, K, None)
    if fn == "w8a8_gemm_postscale_ex":
        return f(a, lda, w, ldw, sa, sw, None, 0, out, ldo, M, N, K, 1, None, 0, None)
    return f(a, lda, w, ldw, sa, sw, out, ldo, M, N, K, None)


GEMM_CASES = [
    (dict(a=None), INVALID),
    (dict(w=None), INVALID),
    (dict(out=None), INVALID),
    (dict(M=-1), INVALID),
    (dict(lda=128), INVALID),
    (dict(ldo=64), INVALID),
    (dict(K=0, lda=256, ldw=256), UNSUPPORTED),
    (dict(K=200, lda=208, ldw=208), UNSUPPORTED),                   # K % 128
    (dict(N=192, ldo=192), UNSUPPORTED),                            # N % 128
    (dict(K=133248, lda=133248, ldw=133248), UNSUPPORTED),          # INT32 overflow bound
    (dict(a=P + 8), UNSUPPORTED),
    (dict(w=Q + 4), UNSUPPORTED),
    (dict(out=O + 2), UNSUPPORTED),
    (dict(lda=264), UNSUPPORTED),
    (dict(ldo=132), UNSUPPORTED),
    (dict(lda=1 << 23), UNSUPPORTED),                               # 256 rows >= 2^31 bytes
    (dict(ldo=1 << 22), UNSUPPORTED),                               # 256 output rows >= 2^31 bytes
    (dict(out=P), INVALID),                                         # out aliases a
]


@pytest.mark.parametrize("kwargs,status", GEMM_CASES)
@pytest.mark.parametrize("fn", ["w8a8_gemm_postscale", "w8a8_gemm_postscale_bias",
                                "w8a8_gemm_postscale_gelu", "w8a8_gemm_postscale_ex",
                                "w8a8_gemm_blockwise"])
def test_gemm_rejects(fn, kwargs, status):
    assert gemm(fn, **kwargs) == status


@pytest.mark.parametrize("kwargs,status", GEMM_CASES[:5] + [
    (dict(K=200, lda=208, ldw=208), UNSUPPORTED), (dict(ldo=130), UNSUPPORTED)])
def test_gemm_i32_rejects(kwargs, status):
    assert gemm("w8a8_gemm_i32", **kwargs) == status


def test_gemm_null_scales():
    assert gemm(sa=None) == INVALID
    assert gemm("w8a8_gemm_blockwise", sw=None) == INVALID
    assert gemm(sa=S + 2) == UNSUPPORTED


def bias_gemm(bias, out=O, M=64, N=128):
    return w8.lib().w8a8_gemm_postscale_bias(P, 256, Q, 256, S, S + 0x100000, bias, out, N,
                                             M, N, 256, None)


def test_gemm_bias_rejects():
    assert bias_gemm(None) == INVALID
    assert bias_gemm(S + 0x200008) == UNSUPPORTED                    # bias not 16-byte aligned
    assert bias_gemm(O + 0x1000) == INVALID                          # bias inside the output
    assert bias_gemm(O - 0x100, N=256) == INVALID                    # bias runs into the output
    assert bias_gemm(None, M=0) == OK                                # empty call: a no-op


def gelu_gemm(bias, out=O, M=64, N=128):
    return w8.lib().w8a8_gemm_postscale_gelu(P, 256, Q, 256, S, S + 0x100000, bias, out, N,
                                             M, N, 256, None)


def test_gemm_gelu_rejects():
    assert gelu_gemm(S + 0x200008) == UNSUPPORTED                    # bias not 16-byte aligned
    assert gelu_gemm(O + 0x1000) == INVALID                          # bias inside the output
    assert gelu_gemm(None, out=S) == INVALID                         # output over a scale
    assert gelu_gemm(None, M=0) == OK                                # empty call: a no-op
    assert w8.lib().w8a8_gemm_postscale_gelu(P, 256, Q, 256, None, S, None, O, 128, 64, 128,
                                             256, None) == INVALID   # null scale


def test_empty_calls_are_noops():
    lib = w8.lib()
    assert lib.w8a8_quant_rows(None, 0, 256, 256, 1, 256, None, 256, None, None) == OK
    assert lib.w8a8_rmsnorm_quant(None, None, 1e-6, 0, 256, 256, None, 256, None, None, None) == OK
    assert lib.w8a8_layernorm_quant(None, None, None, None, None, 1e-6, 0, 256, 256, None, 256,
                                    None, None, None, None) == OK
    assert lib.w8a8_gemm_postscale(None, 256, Q, 256, None, S, None, 128, 0, 128, 256, None) == OK
    assert lib.w8a8_gemm_blockwise(None, 256, Q, 256, None, S, None, 128, 0, 128, 256, None) == OK
    assert lib.w8a8_gemm_i32(None, 256, None, 256, None, 128, 0, 128, 256, None) == OK
    # shape rules still apply to empty calls
    assert lib.w8a8_gemm_i32(None, 256, None, 256, None, 128, 0, 128, 200, None) == UNSUPPORTED


def test_max_k_constant():
    # 127^2 * K must fit INT32; W8A8_MAX_K is the largest multiple of 128 that does
    assert 127 * 127 * w8.W8A8_MAX_K <= 2**31 - 1
    assert 127 * 127 * (w8.W8A8_MAX_K + 128) > 2**31 - 1
    assert w8.W8A8_MAX_K % 128 == 0
    assert "#define W8A8_MAX_K 133120" in open(HEADER).read()


def test_binding_rejects_host_tensors():
    x = torch.zeros(4, 256, dtype=torch.bfloat16)
    with pytest.raises(w8.W8A8Error):
        w8.w8a8_quant_rows(x)
    a = torch.zeros(4, 256, dtype=torch.int8)
    with pytest.raises(w8.W8A8Error):
        w8.w8a8_gemm_i32(a, a)


def test_int8_linear_rejects_cpu_weights():
    with pytest.raises(w8.W8A8Error):
        w8.Int8Linear(torch.zeros(128, 256, dtype=torch.bfloat16))
    assert w8.linear.int8_shape_supported(128, 256)
    assert not w8.linear.int8_shape_supported(100, 256)
    assert not w8.linear.int8_shape_supported(128, 200)
    assert not w8.linear.int8_shape_supported(128, w8.W8A8_MAX_K + 128)


def test_splitk_parts_query():
    # no GPU here: the model runs with its 256-unit default
    assert w8.splitk_parts(28672, 16384, 4096) == 1          # tiles fill the chip
    assert w8.splitk_parts(1000, 5120, 5120) == 1            # partial sums would cost more
    assert w8.splitk_parts(129, 5120, 13824) > 1
    # the cost model's measured calls (MI355X, GPU time of graph-replayed
    # calls): split where that was faster than the better single pass
    # (129 x 5120 x 13824: 31 us in 8 parts against 48 us on 128 x 160
    # tiles), not where one pass on 128 x 160 tiles was (512 x 4096 x 4096:
    # 19.6 us against 28.8 us in 4 parts)
    assert w8.splitk_parts(512, 4096, 4096) == 1
    assert w8.splitk_parts(1024, 4096, 4096) == 1 and w8.splitk_parts(256, 16384, 4096) == 1
    assert 4 <= w8.splitk_parts(256, 5120, 13824) <= 16
    assert w8.splitk_parts(0, 128, 256) == 1 and w8.splitk_parts(4, 128, 0) == 1
    for M, N, K in ((1, 256, 2048), (256, 5120, 13824), (33, 128, 8192)):
        p = w8.splitk_parts(M, N, K)
        assert 1 <= p <= K // 128 and p * M * N * 4 <= 1 << 30


def test_tile_channels_query():
    # no GPU here: the model runs with its 256-unit default. Few tokens take
    # 128 x 160 tiles (measured: 1000 x 5120 x 5120 in 28.8 against 50 us),
    # shapes whose 256 x 256 tiles fill the chip keep them
    assert w8.tile_channels(1000, 5120, 5120) == 160
    assert w8.tile_channels(1000, 5120, 5120, blockwise=True) == 160
    assert w8.tile_channels(512, 4096, 4096) == 160
    assert w8.tile_channels(28672, 16384, 4096) == 256
    assert w8.tile_channels(32760, 5120, 13824) == 256
    assert w8.tile_channels(4096, 4096, 4096) == 256
    assert w8.tile_channels(2048, 5120, 5120) == 256            # two rounds of 128 x 160 tiles
    assert w8.tile_channels(4096, 5120, 5120, blockwise=True) == 256
    assert w8.tile_channels(0, 128, 128) == 256
    assert w8.tile_channels(64, 100, 256) == -1 and w8.tile_channels(64, 128, 200) == -1
    assert w8.lib().w8a8_gemm_tile_channels(64, 128, 256, 2) == -1


def test_workspace_size_query():
    # parts = 0: the library's choice (no GPU here: the 256-unit default)
    for M, N, K in ((256, 5120, 13824), (129, 5120, 13824), (28672, 16384, 4096)):
        p = w8.splitk_parts(M, N, K)
        assert w8.postscale_workspace_size(M, N, K) == (p * M * N * 4 if p > 1 else 0)
    # forced parts, the single pass, and arguments the entry point would reject
    assert w8.postscale_workspace_size(256, 5120, 13824, 3) == 3 * 256 * 5120 * 4
    assert w8.postscale_workspace_size(256, 5120, 13824, 1) == 0
    assert w8.postscale_workspace_size(0, 5120, 13824, 4) == 0
    assert w8.postscale_workspace_size(64, 128, 256, 2) == 2 * 64 * 128 * 4
    assert w8.postscale_workspace_size(64, 128, 256, 3) == -1          # more parts than stages
    assert w8.postscale_workspace_size(64, 128, 256 * 64, 65) == -1    # more than 64 parts
    assert w8.postscale_workspace_size(64, 128, 256, -1) == -1
    assert w8.postscale_workspace_size(64, 100, 256, 0) == -1          # N % 128
    assert w8.postscale_workspace_size(64, 128, 200, 0) == -1          # K % 128
    assert w8.postscale_workspace_size(-1, 128, 256, 0) == -1


WS = 0x70000000          # fake workspace address


def ex(parts=2, ws=WS, ws_bytes=1 << 20, flags=0, bias=None, out=O, M=64, N=128, K=256):
    return w8.lib().w8a8_gemm_postscale_ex(P, 256, Q, 256, S, S + 0x100000, bias, flags, out, N,
                                           M, N, K, parts, ws, ws_bytes, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(flags=2), INVALID),                               # unknown epilogue flag
    (dict(parts=-1), INVALID),
    (dict(parts=65, K=65 * 128), INVALID),                  # more than 64 parts
    (dict(parts=3), INVALID),                               # more parts than K stages (2)
    (dict(ws=None, ws_bytes=0), INVALID),                   # forced split without workspace
    (dict(ws_bytes=2 * 64 * 128 * 4 - 4), INVALID),         # workspace too small
    (dict(ws_bytes=-1), INVALID),
    (dict(ws=WS + 8), UNSUPPORTED),                         # workspace not 16-byte aligned
    (dict(ws=O + 0x100), INVALID),                          # workspace inside the output
    (dict(ws=Q - 0x100), INVALID),                          # workspace runs into w
    (dict(ws=S - 0x100), INVALID),                          # workspace runs into a_scale
    (dict(bias=S + 0x200008), UNSUPPORTED),                 # bias not 16-byte aligned
])
def test_postscale_ex_rejects(kwargs, status):
    assert ex(**kwargs) == status
    assert w8.lib().w8a8_last_error() != b""


def test_postscale_ex_empty_call_is_noop():
    # zero rows: nothing to split, no workspace needed
    assert ex(parts=2, ws=None, ws_bytes=0, M=0) == OK
    assert ex(parts=3, M=0) == INVALID          # the parts rule still applies


# The binding checks every buffer against the call's shape before anything
# reaches the library (which sees bare pointers). Host tensors reach the
# shape checks first, so these run without a GPU.

def _bf(*shape):
    return torch.zeros(*shape, dtype=torch.bfloat16)


def _i8(*shape):
    return torch.zeros(*shape, dtype=torch.int8)


def _f32(*shape):
    return torch.zeros(*shape, dtype=torch.float32)


@pytest.mark.parametrize("call,what", [
    (lambda: w8.w8a8_quant_rows(_bf(4, 256), q=_i8(3, 256)), "q must have shape"),
    (lambda: w8.w8a8_quant_rows(_bf(4, 256), q=_i8(4, 128)), "q must have shape"),
    (lambda: w8.w8a8_quant_rows(_bf(4, 256), scale=_f32(3)), "scale must be contiguous with 4"),
    (lambda: w8.w8a8_quant_rows(_bf(4, 256), 1, 128, scale=_f32(4)), "with 8 elements"),
    (lambda: w8.w8a8_quant_rows(_bf(200, 256), 128, 128, scale=_f32(2)), "with 4 elements"),
    (lambda: w8.w8a8_quant_rows(_bf(4, 256), scale=_bf(4)), "scale must be a torch.float32"),
    (lambda: w8.w8a8_rmsnorm_quant(_bf(4, 256), _bf(255)), "gamma"),
    (lambda: w8.w8a8_rmsnorm_quant(_bf(4, 256), _bf(256), inv_rms=_f32(3)), "inv_rms"),
    (lambda: w8.w8a8_rmsnorm_quant(_bf(4, 256), _bf(256), scale=_f32(5)), "scale"),
    (lambda: w8.w8a8_layernorm_quant(_bf(4, 256), mean=_f32(3)), "mean"),
    (lambda: w8.w8a8_layernorm_quant(_bf(4, 256), rstd=_f32(2)), "rstd"),
    (lambda: w8.w8a8_layernorm_quant(_bf(4, 256), mod_shift=_bf(128)), "mod_shift"),
    (lambda: w8.w8a8_layernorm_quant(_bf(4, 256), q=_i8(4, 255)), "q must have shape"),
    (lambda: w8.w8a8_gemm_postscale(_i8(64, 256), _i8(128, 256), _f32(64), _f32(128),
                                    out=_bf(63, 128)), "out must have shape (64, 128)"),
    (lambda: w8.w8a8_gemm_postscale(_i8(64, 256), _i8(128, 256), _f32(64), _f32(128),
                                    out=_bf(64, 256)[:, :127]), "out must have shape"),
    (lambda: w8.w8a8_gemm_postscale(_i8(64, 256), _i8(128, 256), _f32(63), _f32(128)),
     "a_scale must be contiguous with 64"),
    (lambda: w8.w8a8_gemm_postscale(_i8(64, 256), _i8(128, 256), _f32(64), _f32(127)),
     "w_scale must be contiguous with 128"),
    (lambda: w8.w8a8_gemm_postscale(_i8(64, 256), _i8(128, 256), _f32(64), _bf(128)),
     "w_scale must be a torch.float32"),
    (lambda: w8.w8a8_gemm_postscale(_i8(64, 256), _i8(128, 256), _f32(64), _f32(128),
                                    bias=_bf(64)), "bias"),
    (lambda: w8.w8a8_gemm_postscale(_i8(64, 256), _i8(128, 128), _f32(64), _f32(128)),
     "K mismatch"),
    (lambda: w8.w8a8_gemm_blockwise(_i8(64, 256), _i8(128, 256), _f32(64, 1), _f32(1, 2)),
     "a_scale must be contiguous with 128"),
    (lambda: w8.w8a8_gemm_blockwise(_i8(64, 256), _i8(128, 256), _f32(64, 2), _f32(1, 1)),
     "w_scale must be contiguous with 2"),
    (lambda: w8.w8a8_gemm_blockwise(_i8(64, 256), _i8(128, 256), _f32(64, 2), _f32(1, 2),
                                    out=_bf(64, 64)), "out must have shape"),
    (lambda: w8.w8a8_gemm_i32(_i8(64, 256), _i8(128, 256), out=torch.zeros(64, 64, dtype=torch.int32)),
     "out must have shape"),
])
def test_binding_rejects_undersized_buffers(call, what):
    with pytest.raises(w8.W8A8Error) as e:
        call()
    assert what in str(e.value), str(e.value)


def test_binding_rejects_host_tensors_after_shape_checks():
    # right shapes on the host: the device check is what fails
    with pytest.raises(w8.W8A8Error, match="device tensor"):
        w8.w8a8_gemm_postscale(_i8(64, 256), _i8(128, 256), _f32(64), _f32(128))
    with pytest.raises(w8.W8A8Error, match="device tensor"):
        w8.w8a8_rmsnorm_quant(_bf(4, 256), _bf(256))


def test_probe_library_loads_and_rejects_bad_arguments():
    # the main-loop ceiling probe is a library of its own (not part of the C ABI);
    # bad arguments are refused before anything touches a device
    import ctypes
    path = os.path.join(ROOT, "w8a8_int8_quantized_token_amd", "libw8a8_probe.so")
    lib = ctypes.CDLL(path)
    f = lib.w8a8_probe_mainloop
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                  ctypes.c_int64, ctypes.c_void_p]
    assert f(None, 2 << 20, 8, 1, None, 1 << 20, None) == 1          # null buffers
    assert f(1 << 20, (2 << 20) - 1, 8, 1, 1 << 20, 1 << 20, None) == 1   # buffer too small
    assert f(1 << 20, 2 << 20, 0, 1, 1 << 20, 1 << 20, None) == 1    # no stages
    assert f(1 << 20, 2 << 20, 8, 2, 1 << 20, 1 << 20, None) == 1    # refill not 0/1


def test_bench_refuses_several_gpus():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr
