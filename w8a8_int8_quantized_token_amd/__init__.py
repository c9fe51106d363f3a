"""Python binding of the MI355X (gfx950) W8A8 INT8 Linear library.

Thin ctypes marshalling over ``libw8a8.so`` (declared in include/w8a8.h):
every function below has the name of the C entry point it calls, takes torch
tensors that already live in device memory, passes their data pointers, sizes
and strides plus torch's current HIP stream, and raises on a non-zero status.
All arithmetic happens in the HIP kernels; torch only supplies device memory
and the stream. If the library is missing, importing this package fails.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "W8A8Error", "W8A8Unsupported", "lib", "LIB_PATH", "EXPORTED_SYMBOLS",
    "w8a8_quant_rows", "w8a8_rmsnorm_quant", "w8a8_layernorm_quant", "w8a8_gemm_postscale",
    "w8a8_gemm_blockwise", "w8a8_gemm_i32", "w8a8_version", "splitk_parts",
    "w8a8_gemm_postscale_noalloc", "tile_channels",
    "postscale_workspace_size", "Int8Linear", "NormInt8Linear",
    "replace_linear_with_int8",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libw8a8.so")

W8A8_OK = 0
W8A8_ERR_INVALID_ARGUMENT = 1
W8A8_ERR_UNSUPPORTED_SHAPE = 2
W8A8_ERR_HIP = 3
W8A8_MAX_K = 133120
W8A8_EPILOGUE_GELU = 1


class W8A8Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class W8A8Unsupported(W8A8Error):
    """The shape is outside what the INT8 kernels cover; use a BF16 Linear."""


if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m w8a8_int8_quantized_token_amd.build` "
        "(or __graft_entry__.build()). There is no fallback path.")

_lib = ctypes.CDLL(LIB_PATH)

_i64 = ctypes.c_int64
_p = ctypes.c_void_p
_st = ctypes.c_int

_SIGS = {
    "w8a8_quant_rows": [_p, _i64, _i64, _i64, _i64, _i64, _p, _i64, _p, _p],
    "w8a8_rmsnorm_quant": [_p, _p, ctypes.c_float, _i64, _i64, _i64, _p, _i64, _p, _p, _p],
    "w8a8_layernorm_quant": [_p, _p, _p, _p, _p, ctypes.c_float, _i64, _i64, _i64, _p, _i64, _p,
                             _p, _p, _p],
    "w8a8_gemm_postscale": [_p, _i64, _p, _i64, _p, _p, _p, _i64, _i64, _i64, _i64, _p],
    "w8a8_gemm_postscale_bias": [_p, _i64, _p, _i64, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _p],
    "w8a8_gemm_postscale_gelu": [_p, _i64, _p, _i64, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _p],
    "w8a8_gemm_blockwise": [_p, _i64, _p, _i64, _p, _p, _p, _i64, _i64, _i64, _i64, _p],
    "w8a8_gemm_i32": [_p, _i64, _p, _i64, _p, _i64, _i64, _i64, _i64, _p],
    "w8a8_gemm_postscale_ex": [_p, _i64, _p, _i64, _p, _p, _p, ctypes.c_int32, _p, _i64, _i64,
                               _i64, _i64, ctypes.c_int32, _p, _i64, _p],
    "w8a8_gemm_postscale_noalloc": [_p, _i64, _p, _i64, _p, _p, _p, ctypes.c_int32, _p, _i64,
                                    _i64, _i64, _i64, ctypes.c_int32, _p],
}
for _name, _args in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _st
_lib.w8a8_status_string.argtypes = [_st]
_lib.w8a8_status_string.restype = ctypes.c_char_p
_lib.w8a8_last_error.argtypes = []
_lib.w8a8_last_error.restype = ctypes.c_char_p
_lib.w8a8_version.argtypes = []
_lib.w8a8_version.restype = ctypes.c_char_p
_lib.w8a8_gemm_splitk_parts.argtypes = [_i64, _i64, _i64]
_lib.w8a8_gemm_splitk_parts.restype = ctypes.c_int32
_lib.w8a8_gemm_postscale_workspace_size.argtypes = [_i64, _i64, _i64, ctypes.c_int32]
_lib.w8a8_gemm_postscale_workspace_size.restype = _i64
_lib.w8a8_gemm_tile_channels.argtypes = [_i64, _i64, _i64, ctypes.c_int32]
_lib.w8a8_gemm_tile_channels.restype = ctypes.c_int32

EXPORTED_SYMBOLS = tuple(_SIGS) + ("w8a8_status_string", "w8a8_last_error", "w8a8_version",
                                   "w8a8_gemm_splitk_parts", "w8a8_gemm_postscale_workspace_size",
                                   "w8a8_gemm_tile_channels")


def lib() -> ctypes.CDLL:
    """The loaded C library (raw ctypes handle, for tests of the ABI itself)."""
    return _lib


def w8a8_version() -> str:
    return _lib.w8a8_version().decode()


def tile_channels(M: int, N: int, K: int, blockwise: bool = False) -> int:
    """Output-channel width of the tiles a single pass uses on the current
    device: 256 (persistent kernels) or 160 (128 x 160 tiles); -1 if rejected."""
    return int(_lib.w8a8_gemm_tile_channels(M, N, K, 1 if blockwise else 0))


def splitk_parts(M: int, N: int, K: int) -> int:
    """K parts the post-scale GEMMs use for this shape on the current device."""
    return int(_lib.w8a8_gemm_splitk_parts(M, N, K))


def _check(status: int, name: str) -> None:
    if status == W8A8_OK:
        return
    msg = f"{name}: {_lib.w8a8_status_string(status).decode()}: {_lib.w8a8_last_error().decode()}"
    if status == W8A8_ERR_UNSUPPORTED_SHAPE:
        raise W8A8Unsupported(status, msg)
    raise W8A8Error(status, msg)


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


# Buffer checks. The C ABI receives bare pointers and cannot see how large a
# buffer is, so this layer checks every tensor's dtype, layout and size
# against the call's shape (shape checks first, so that they are reported
# even for tensors on the wrong device), then that all of them live on the
# device the call runs on.

def _bad(msg: str):
    raise W8A8Error(W8A8_ERR_INVALID_ARGUMENT, msg)


def _mat(t: torch.Tensor, dtype: torch.dtype, name: str, rows: int | None = None,
         cols: int | None = None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        _bad(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        _bad(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        _bad(f"{name} must be a row-major 2-D matrix")
    if (rows is not None and t.shape[0] != rows) or (cols is not None and t.shape[1] != cols):
        _bad(f"{name} must have shape ({rows}, {cols}), got {tuple(t.shape)}")
    return t


def _vec(t: torch.Tensor, dtype: torch.dtype, n: int, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or t.dtype != dtype:
        _bad(f"{name} must be a {dtype} tensor")
    if t.numel() != n or not t.is_contiguous():
        _bad(f"{name} must be contiguous with {n} elements, got {tuple(t.shape)}")
    return t


def _on_device(device: torch.device, **tensors) -> None:
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            _bad(f"{name} must be a device tensor")
        if t.device != device:
            _bad(f"{name} is on {t.device}, the call runs on {device}")


def _ld(t: torch.Tensor) -> int:
    return t.stride(0) if t.shape[0] > 1 else max(t.shape[1], t.stride(0))


def _scale_elems(rows: int, cols: int, group_rows: int, group_cols: int) -> int | None:
    """Scales a (group_rows, group_cols) quantisation of [rows, cols] writes, or
    None for a group the library rejects anyway (nothing is launched then)."""
    if group_rows <= 0 or group_cols <= 0 or cols % group_cols:
        return None
    return -(-rows // group_rows) * (cols // group_cols)


def w8a8_quant_rows(x: torch.Tensor, group_rows: int = 1, group_cols: int | None = None,
                    q: torch.Tensor | None = None, scale: torch.Tensor | None = None,
                    stream=None):
    """Symmetric absmax INT8 quantisation of a BF16 [rows, cols] matrix.

    group (1, cols) (default): one scale per row; (1, 128): per 128-wide
    block of each row; (128, 128): per 128x128 block. Returns (q, scale).
    """
    _mat(x, torch.bfloat16, "x")
    rows, cols = x.shape
    gc = cols if group_cols is None else group_cols
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.int8, device=x.device)
    n_sc = _scale_elems(rows, cols, group_rows, gc)
    if scale is None:
        n_gr = -(-rows // group_rows) if group_rows > 0 else 0
        shape = (n_gr,) if (group_rows == 1 and gc == cols) else (n_gr, cols // gc if gc > 0 else 0)
        scale = torch.empty(shape, dtype=torch.float32, device=x.device)
    _mat(q, torch.int8, "q", rows, cols)
    if n_sc is not None:
        _vec(scale, torch.float32, n_sc, "scale")
    _on_device(x.device, x=x, q=q, scale=scale)
    st = _lib.w8a8_quant_rows(_ptr(x), rows, cols, _ld(x), group_rows, gc, _ptr(q), _ld(q),
                              _ptr(scale), _stream(stream))
    _check(st, "w8a8_quant_rows")
    return q, scale


def w8a8_rmsnorm_quant(x: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-6,
                       q: torch.Tensor | None = None, scale: torch.Tensor | None = None,
                       inv_rms: torch.Tensor | bool | None = True, stream=None):
    """RMSNorm (gain gamma, no bias) fused with per-token INT8 quantisation.
    Returns (q, scale, inv_rms) (inv_rms is None when not requested)."""
    _mat(x, torch.bfloat16, "x")
    rows, cols = x.shape
    _vec(gamma, torch.bfloat16, cols, "gamma")
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.int8, device=x.device)
    if scale is None:
        scale = torch.empty((rows,), dtype=torch.float32, device=x.device)
    if inv_rms is True:
        inv_rms = torch.empty((rows,), dtype=torch.float32, device=x.device)
    elif inv_rms is False:
        inv_rms = None
    _mat(q, torch.int8, "q", rows, cols)
    _vec(scale, torch.float32, rows, "scale")
    if inv_rms is not None:
        _vec(inv_rms, torch.float32, rows, "inv_rms")
    _on_device(x.device, x=x, gamma=gamma, q=q, scale=scale, inv_rms=inv_rms)
    st = _lib.w8a8_rmsnorm_quant(_ptr(x), _ptr(gamma), float(eps), rows, cols, _ld(x), _ptr(q),
                                 _ld(q), _ptr(scale), _ptr(inv_rms), _stream(stream))
    _check(st, "w8a8_rmsnorm_quant")
    return q, scale, inv_rms


def w8a8_layernorm_quant(x: torch.Tensor, eps: float = 1e-6, gamma: torch.Tensor | None = None,
                         beta: torch.Tensor | None = None, mod_scale: torch.Tensor | None = None,
                         mod_shift: torch.Tensor | None = None, q: torch.Tensor | None = None,
                         scale: torch.Tensor | None = None, stats: bool = True,
                         mean: torch.Tensor | None = None, rstd: torch.Tensor | None = None,
                         stream=None):
    """LayerNorm (optional gamma/beta) and adaLN modulation z = y*(1+mod_scale)+mod_shift
    (each optional), fused with per-token INT8 quantisation.
    Returns (q, scale, mean, rstd) (mean and rstd are None when stats is False;
    given mean/rstd tensors are written in place)."""
    _mat(x, torch.bfloat16, "x")
    rows, cols = x.shape
    for t, name in ((gamma, "gamma"), (beta, "beta"), (mod_scale, "mod_scale"),
                    (mod_shift, "mod_shift")):
        if t is not None:
            _vec(t, torch.bfloat16, cols, name)
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.int8, device=x.device)
    if scale is None:
        scale = torch.empty((rows,), dtype=torch.float32, device=x.device)
    if stats:
        mean = torch.empty((rows,), dtype=torch.float32, device=x.device) if mean is None else mean
        rstd = torch.empty((rows,), dtype=torch.float32, device=x.device) if rstd is None else rstd
        _vec(mean, torch.float32, rows, "mean")
        _vec(rstd, torch.float32, rows, "rstd")
    else:
        mean = rstd = None
    _mat(q, torch.int8, "q", rows, cols)
    _vec(scale, torch.float32, rows, "scale")
    _on_device(x.device, x=x, gamma=gamma, beta=beta, mod_scale=mod_scale, mod_shift=mod_shift,
               q=q, scale=scale, mean=mean, rstd=rstd)
    st = _lib.w8a8_layernorm_quant(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(mod_scale),
                                   _ptr(mod_shift), float(eps), rows, cols, _ld(x), _ptr(q),
                                   _ld(q), _ptr(scale), _ptr(mean), _ptr(rstd), _stream(stream))
    _check(st, "w8a8_layernorm_quant")
    return q, scale, mean, rstd


def _gemm_args(a, w, out, out_dtype):
    _mat(a, torch.int8, "a")
    _mat(w, torch.int8, "w")
    M, K = a.shape
    N, K2 = w.shape
    if K != K2:
        _bad(f"K mismatch: a has {K}, w has {K2}")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    _mat(out, out_dtype, "out", M, N)
    return M, N, K, out


def postscale_workspace_size(M: int, N: int, K: int, parts: int = 0) -> int:
    """Bytes of split-K workspace the post-scale GEMM needs for this shape with
    `parts` (0 = the library's choice): 0 for a single pass, -1 if the library
    would reject the arguments."""
    return int(_lib.w8a8_gemm_postscale_workspace_size(M, N, K, parts))


def w8a8_gemm_postscale(a: torch.Tensor, w: torch.Tensor, a_scale: torch.Tensor,
                        w_scale: torch.Tensor, out: torch.Tensor | None = None, stream=None,
                        bias: torch.Tensor | None = None, gelu: bool = False, parts: int = 0,
                        workspace: torch.Tensor | None = None):
    """out[M,N] (BF16) = bf16(acc * a_scale[m] * w_scale[n] (+ bias[n])), acc the
    exact INT32 sum over K of a[m,k] * w[n,k]; with gelu=True, the GELU (erf
    form) of that BF16 output. Calls w8a8_gemm_postscale_ex: with parts=0 the
    library chooses how many K parts to split into (few tokens, long K), 1 is
    the single pass, n forces n parts. The split-K workspace is `workspace`
    (a device tensor of at least the bytes postscale_workspace_size reports),
    or one allocated here from torch's allocator on the call's stream."""
    M, N, K, out = _gemm_args(a, w, out, torch.bfloat16)
    _vec(a_scale, torch.float32, M, "a_scale")
    _vec(w_scale, torch.float32, N, "w_scale")
    if bias is not None:
        _vec(bias, torch.bfloat16, N, "bias")
    _on_device(a.device, a=a, w=w, out=out, a_scale=a_scale, w_scale=w_scale, bias=bias,
               workspace=workspace)
    need = postscale_workspace_size(M, N, K, parts) if M > 0 else 0
    if workspace is None and need > 0:
        workspace = torch.empty((need,), dtype=torch.uint8, device=a.device)
        if stream is not None:
            # the allocator may hand this block out again once `stream`'s work
            # that uses it is done, not merely the current stream's
            sobj = stream if isinstance(stream, torch.cuda.Stream) else \
                torch.cuda.ExternalStream(int(stream), device=a.device)
            workspace.record_stream(sobj)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if workspace is not None and not workspace.is_contiguous():
        _bad("workspace must be contiguous")
    st = _lib.w8a8_gemm_postscale_ex(_ptr(a), _ld(a), _ptr(w), _ld(w), _ptr(a_scale),
                                     _ptr(w_scale), _ptr(bias), W8A8_EPILOGUE_GELU if gelu else 0,
                                     _ptr(out), _ld(out), M, N, K, int(parts), _ptr(workspace),
                                     ws_bytes, _stream(stream))
    _check(st, "w8a8_gemm_postscale_ex")
    return out


def w8a8_gemm_postscale_noalloc(a: torch.Tensor, w: torch.Tensor, a_scale: torch.Tensor,
                                w_scale: torch.Tensor, out: torch.Tensor, stream=None,
                                bias: torch.Tensor | None = None, gelu: bool = False,
                                parts: int = 0):
    """The post-scale GEMM family without any allocation: split-K partial sums
    go to the library's fixed 64 MiB device array (calls that overlap on one
    GPU race on it). `out` must be given."""
    if out is None:
        _bad("out must be given (this call allocates nothing)")
    M, N, K, out = _gemm_args(a, w, out, torch.bfloat16)
    _vec(a_scale, torch.float32, M, "a_scale")
    _vec(w_scale, torch.float32, N, "w_scale")
    if bias is not None:
        _vec(bias, torch.bfloat16, N, "bias")
    _on_device(a.device, a=a, w=w, out=out, a_scale=a_scale, w_scale=w_scale, bias=bias)
    st = _lib.w8a8_gemm_postscale_noalloc(_ptr(a), _ld(a), _ptr(w), _ld(w), _ptr(a_scale),
                                          _ptr(w_scale), _ptr(bias),
                                          W8A8_EPILOGUE_GELU if gelu else 0, _ptr(out), _ld(out),
                                          M, N, K, int(parts), _stream(stream))
    _check(st, "w8a8_gemm_postscale_noalloc")
    return out


def w8a8_gemm_blockwise(a: torch.Tensor, w: torch.Tensor, a_scale: torch.Tensor,
                        w_scale: torch.Tensor, out: torch.Tensor | None = None, stream=None):
    """Blockwise-scaled GEMM: a_scale [M, K/128], w_scale [N/128, K/128]."""
    M, N, K, out = _gemm_args(a, w, out, torch.bfloat16)
    if K % 128 == 0 and N % 128 == 0:         # other shapes: the library rejects them
        _vec(a_scale, torch.float32, M * (K // 128), "a_scale")
        _vec(w_scale, torch.float32, (N // 128) * (K // 128), "w_scale")
    _on_device(a.device, a=a, w=w, out=out, a_scale=a_scale, w_scale=w_scale)
    st = _lib.w8a8_gemm_blockwise(_ptr(a), _ld(a), _ptr(w), _ld(w), _ptr(a_scale), _ptr(w_scale),
                                  _ptr(out), _ld(out), M, N, K, _stream(stream))
    _check(st, "w8a8_gemm_blockwise")
    return out


def w8a8_gemm_i32(a: torch.Tensor, w: torch.Tensor, out: torch.Tensor | None = None, stream=None):
    """The post-scale GEMM's INT32 accumulators, out[m,n] = sum_k a[m,k] * w[n,k]."""
    M, N, K, out = _gemm_args(a, w, out, torch.int32)
    _on_device(a.device, a=a, w=w, out=out)
    st = _lib.w8a8_gemm_i32(_ptr(a), _ld(a), _ptr(w), _ld(w), _ptr(out), _ld(out), M, N, K,
                            _stream(stream))
    _check(st, "w8a8_gemm_i32")
    return out


from .linear import Int8Linear, NormInt8Linear, replace_linear_with_int8  # noqa: E402  (needs the binding above)
