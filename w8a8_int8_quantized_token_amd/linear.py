"""Int8Linear: the W8A8 Linear as a torch module.

"TurboDiffusion Integration Notes", section "Reused Components", W8A8 Linear
bullet: selected Linear layers become INT8 once, when the model is set up,
their activations are quantised dynamically before every call, and shapes the
INT8 kernels do not cover keep using the native Linear. The module therefore
keeps the BF16 weight (for those shapes), quantises it per output channel once
at construction, and on every call quantises the activation per token and runs
the INT8 GEMM with the scales (and the bias) applied in its epilogue.

Every INT8 step is a call into libw8a8; when the library reports
W8A8_ERR_UNSUPPORTED_SHAPE the call runs torch's BF16 Linear on the same
device instead. There is no CPU path: CPU tensors are an error.
"""
from __future__ import annotations

import torch

from . import W8A8Error, W8A8Unsupported, W8A8_ERR_INVALID_ARGUMENT, W8A8_MAX_K
from . import (w8a8_gemm_postscale, w8a8_layernorm_quant, w8a8_quant_rows,
               w8a8_rmsnorm_quant)


def int8_shape_supported(out_features: int, in_features: int) -> bool:
    """Whether the INT8 GEMM takes a [out_features, in_features] weight: K a
    multiple of 128 up to W8A8_MAX_K, N a multiple of 128."""
    return (in_features % 128 == 0 and 128 <= in_features <= W8A8_MAX_K
            and out_features % 128 == 0 and out_features > 0)


class Int8Linear(torch.nn.Module):
    """y = x W^T (+ b) with W quantised per output channel at construction and
    x quantised per token on every call (BF16 in, BF16 out). With
    activation="gelu" the layer is an FFN up projection: y = GELU(x W^T (+ b))
    (erf form) on the BF16 Linear output, fused into the GEMM's epilogue."""

    def __init__(self, weight: torch.Tensor, bias: torch.Tensor | None = None,
                 activation: str | None = None):
        super().__init__()
        if activation not in (None, "gelu"):
            raise W8A8Error(W8A8_ERR_INVALID_ARGUMENT, f"unknown activation {activation!r}")
        self.activation = activation
        if not isinstance(weight, torch.Tensor) or weight.device.type != "cuda":
            raise W8A8Error(W8A8_ERR_INVALID_ARGUMENT, "Int8Linear needs a weight on a GPU")
        weight = weight.detach().to(torch.bfloat16).contiguous()
        self.out_features, self.in_features = weight.shape
        self.register_buffer("weight", weight)
        self.register_buffer("bias", None if bias is None else
                             bias.detach().to(device=weight.device, dtype=torch.bfloat16)
                             .contiguous())
        self.int8 = int8_shape_supported(self.out_features, self.in_features)
        qw = sw = None
        if self.int8:
            try:
                qw, sw = w8a8_quant_rows(weight)
            except W8A8Unsupported:
                self.int8 = False
        self.register_buffer("qweight", qw)
        self.register_buffer("weight_scale", sw)

    @classmethod
    def from_linear(cls, linear: torch.nn.Linear, activation: str | None = None) -> "Int8Linear":
        return cls(linear.weight, linear.bias, activation)

    def extra_repr(self) -> str:
        return (f"in_features={self.in_features}, out_features={self.out_features}, "
                f"bias={self.bias is not None}, activation={self.activation}, int8={self.int8}")

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if x.device.type != "cuda":
            raise W8A8Error(W8A8_ERR_INVALID_ARGUMENT, "Int8Linear runs on the GPU only")
        if x.dtype != torch.bfloat16:
            raise W8A8Error(W8A8_ERR_INVALID_ARGUMENT, "Int8Linear takes BF16 activations")
        if self.int8:
            x2 = x.reshape(-1, self.in_features)
            if not x2.is_contiguous():
                x2 = x2.contiguous()
            try:
                qa, sa = w8a8_quant_rows(x2)
                out = w8a8_gemm_postscale(qa, self.qweight, sa, self.weight_scale,
                                          bias=self.bias, gelu=self.activation == "gelu")
                return out.reshape(*x.shape[:-1], self.out_features)
            except W8A8Unsupported:
                pass
        y = torch.nn.functional.linear(x, self.weight, self.bias)
        return torch.nn.functional.gelu(y) if self.activation == "gelu" else y


class NormInt8Linear(torch.nn.Module):
    """A norm followed by an Int8Linear, with the norm fused into the
    Linear's per-token activation quant.

    "Reused Components", FastNorm and W8A8 Linear bullets: the norms and the
    Linear are separate reused modules; here the normalised BF16 row is
    quantised where it is formed and never reaches memory, which gives the
    same codes as the norm module (BF16 out) followed by the Int8Linear.

    norm="rmsnorm": y = bf16((x r) g), r = 1 / sqrt(mean x^2 + eps), g the
    gain (`weight`, required). norm="layernorm": y = bf16(((x - mu) r) g + b)
    with `weight` and `bias` optional, then, if forward() gets them, the adaLN
    modulation bf16(bf16(y bf16(1 + mod_scale)) + mod_shift). Where the fused
    kernels do not take the shape, the same steps run as torch operations on
    the GPU, in fp32 with the statistics in fp64, each BF16 rounding where the
    fused kernels round, and `linear` then runs on their BF16 output as usual.
    """

    def __init__(self, linear: Int8Linear, norm: str, weight: torch.Tensor | None = None,
                 bias: torch.Tensor | None = None, eps: float = 1e-6):
        super().__init__()
        if not isinstance(linear, Int8Linear):
            raise W8A8Error(W8A8_ERR_INVALID_ARGUMENT, "NormInt8Linear wraps an Int8Linear")
        if norm not in ("rmsnorm", "layernorm"):
            raise W8A8Error(W8A8_ERR_INVALID_ARGUMENT, f"unknown norm {norm!r}")
        if norm == "rmsnorm" and (weight is None or bias is not None):
            raise W8A8Error(W8A8_ERR_INVALID_ARGUMENT, "RMSNorm takes a gain and no bias")
        self.linear = linear
        self.norm = norm
        self.eps = float(eps)
        dev = linear.weight.device
        k = linear.in_features
        for name, t in (("norm_weight", weight), ("norm_bias", bias)):
            if t is not None and t.numel() != k:
                raise W8A8Error(W8A8_ERR_INVALID_ARGUMENT, f"{name} must have {k} elements")
            self.register_buffer(name, None if t is None else
                                 t.detach().to(device=dev, dtype=torch.bfloat16).reshape(k)
                                 .contiguous())

    def extra_repr(self) -> str:
        return f"norm={self.norm}, eps={self.eps}"

    def _norm_torch(self, x: torch.Tensor, mod_scale, mod_shift) -> torch.Tensor:
        xf = x.float()
        eps = torch.tensor(self.eps, dtype=torch.float32).item()   # the fp32 eps
        if self.norm == "rmsnorm":
            r = (1.0 / torch.sqrt(xf.double().square().mean(-1, keepdim=True) + eps)).float()
            return ((xf * r) * self.norm_weight.float()).bfloat16()
        xd = xf.double()
        mu = xd.mean(-1, keepdim=True)
        r = (1.0 / torch.sqrt((xd - mu).square().mean(-1, keepdim=True) + eps)).float()
        u = (xf - mu.float()) * r
        if self.norm_weight is not None:
            u = u * self.norm_weight.float()
        if self.norm_bias is not None:
            u = u + self.norm_bias.float()
        y = u.bfloat16()
        if mod_scale is not None:
            y = (y.float() * (1.0 + mod_scale.float()).bfloat16().float()).bfloat16()
        if mod_shift is not None:
            y = (y.float() + mod_shift.float()).bfloat16()
        return y

    def forward(self, x: torch.Tensor, mod_scale: torch.Tensor | None = None,
                mod_shift: torch.Tensor | None = None) -> torch.Tensor:
        if x.device.type != "cuda":
            raise W8A8Error(W8A8_ERR_INVALID_ARGUMENT, "NormInt8Linear runs on the GPU only")
        if x.dtype != torch.bfloat16:
            raise W8A8Error(W8A8_ERR_INVALID_ARGUMENT, "NormInt8Linear takes BF16 activations")
        if self.norm == "rmsnorm" and (mod_scale is not None or mod_shift is not None):
            raise W8A8Error(W8A8_ERR_INVALID_ARGUMENT, "the modulation follows a LayerNorm")
        lin = self.linear
        k = lin.in_features
        mods = [None if t is None else t.to(torch.bfloat16).reshape(k).contiguous()
                for t in (mod_scale, mod_shift)]
        if lin.int8:
            x2 = x.reshape(-1, k)
            if not x2.is_contiguous():
                x2 = x2.contiguous()
            try:
                if self.norm == "rmsnorm":
                    qa, sa, _ = w8a8_rmsnorm_quant(x2, self.norm_weight, self.eps, inv_rms=False)
                else:
                    qa, sa, _, _ = w8a8_layernorm_quant(x2, self.eps, self.norm_weight,
                                                        self.norm_bias, mods[0], mods[1],
                                                        stats=False)
                out = w8a8_gemm_postscale(qa, lin.qweight, sa, lin.weight_scale, bias=lin.bias,
                                          gelu=lin.activation == "gelu")
                return out.reshape(*x.shape[:-1], lin.out_features)
            except W8A8Unsupported:
                pass
        return lin(self._norm_torch(x, mods[0], mods[1]))


def replace_linear_with_int8(module: torch.nn.Module, select=None) -> int:
    """Swap the nn.Linear layers under `module` (those `select(name, layer)`
    accepts, all by default) for Int8Linear, in place. Returns how many were
    swapped. This is the model-side switch that turns the W8A8 path on."""
    count = 0
    for name, child in list(module.named_children()):
        if isinstance(child, torch.nn.Linear) and (select is None or select(name, child)):
            setattr(module, name, Int8Linear.from_linear(child))
            count += 1
        else:
            count += replace_linear_with_int8(child, select)
    return count
