"""MXFP4 quantization-aware training on top of the C-ABI kernels.

The pieces the amct PR builds around its QDQ operator (fake_quant.py and
linear.py of "feat: add MXFP4 QAT fake-quant Linear (with STE)"), here as thin
wrappers whose arithmetic all runs in libmxfp4's HIP kernels:

- ``mxfp4_fake_quant``: differentiable fake quantization; the forward pass is
  the row-wise QDQ over the last dimension (``mxfp4_qdq_fwd``), the backward
  pass the straight-through estimator -- plain (gradient unchanged) or
  clipped (``mxfp4_ste_bwd`` zeroes the gradient where the forward saturated).
- ``MXFP4FakeQuantizer``: a stateless module around it (no parameters or
  buffers, so a model's state_dict is unchanged).
- ``MXFP4QATConfig``: weight / input quantization switches, block size,
  scale factor, clipped STE and the scale rule.
- ``MXFP4QATLinear``: ``nn.Linear`` computing ``F.linear(Q(x), Q(W), b)``
  (the bias is not quantized); ``convert_to_mxfp4_qat`` swaps the Linear
  layers of a model in place (substring ``skip_names``; idempotent).

There is no CPU path: tensors must be on the GPU and bf16 or fp32.
"""
from __future__ import annotations

import dataclasses

import torch
import torch.nn.functional as F
from torch import nn

from . import ROW, mxfp4_qdq_fwd, mxfp4_ste_bwd

__all__ = ["mxfp4_fake_quant", "MXFP4FakeQuantizer", "MXFP4QATConfig", "MXFP4QATLinear",
           "convert_to_mxfp4_qat"]

_RULES = ("floor", "amct")


def _validate(block_size: int, scale_factor: float, rule: str) -> None:
    if block_size not in (32, 128):
        raise ValueError(f"block_size must be 32 or 128, got {block_size}")
    if not scale_factor > 0:
        raise ValueError(f"scale_factor must be positive, got {scale_factor}")
    if rule not in _RULES:
        raise ValueError(f"rule must be one of {_RULES}, got {rule!r}")


class _FakeQuantSTE(torch.autograd.Function):
    """QDQ forward (+ clip bitmap when clipping); STE backward."""

    @staticmethod
    def forward(ctx, x, block_size, scale_factor, clip_grad, rule):
        if x.dim() == 0:
            raise ValueError("x must have at least 1 dimension")
        xc = x.contiguous()
        cols = xc.shape[-1]
        rows = xc.numel() // cols if cols else 0
        y = torch.empty_like(xc)
        mask = None
        if clip_grad:
            mask = torch.empty((rows, -(-cols // 32)), dtype=torch.int32, device=xc.device)
        mxfp4_qdq_fwd(xc, ROW, y_row=y, mask_row=mask, block=block_size, rule=rule,
                      scale_factor=scale_factor)
        ctx.clip_grad = clip_grad
        ctx.block_size = block_size
        if clip_grad:
            ctx.save_for_backward(mask)
        return y

    @staticmethod
    def backward(ctx, grad_output):
        if not ctx.clip_grad:
            return grad_output, None, None, None, None       # plain STE: identity
        (mask,) = ctx.saved_tensors
        g = grad_output.contiguous()
        grad_in = torch.empty_like(g)
        mxfp4_ste_bwd(g, mask, grad_in, layout=ROW, block=ctx.block_size)
        return grad_in, None, None, None, None


def mxfp4_fake_quant(x: torch.Tensor, block_size: int = 32, scale_factor: float = 6.0,
                     clip_grad: bool = False, rule: str = "floor") -> torch.Tensor:
    """Differentiable MXFP4 fake quantization over the last dimension.

    Same shape, dtype and device as ``x``; the gradient flows back unchanged
    (``clip_grad=False``) or is zeroed where ``|x| > 6 * scale``."""
    _validate(block_size, scale_factor, rule)
    return _FakeQuantSTE.apply(x, block_size, scale_factor, clip_grad, rule)


class MXFP4FakeQuantizer(nn.Module):
    """Stateless module around :func:`mxfp4_fake_quant`."""

    def __init__(self, block_size: int = 32, scale_factor: float = 6.0, clip_grad: bool = False,
                 rule: str = "floor") -> None:
        super().__init__()
        _validate(block_size, scale_factor, rule)
        self.block_size = block_size
        self.scale_factor = scale_factor
        self.clip_grad = clip_grad
        self.rule = rule

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return mxfp4_fake_quant(x, self.block_size, self.scale_factor, self.clip_grad, self.rule)

    def extra_repr(self) -> str:
        return (f"block_size={self.block_size}, scale_factor={self.scale_factor}, "
                f"clip_grad={self.clip_grad}, rule={self.rule!r}")


@dataclasses.dataclass
class MXFP4QATConfig:
    """Settings shared by every converted layer (defaults: W4A16, plain STE)."""

    quantize_weight: bool = True
    quantize_input: bool = False
    block_size: int = 32
    scale_factor: float = 6.0
    clip_grad: bool = False
    rule: str = "floor"

    def __post_init__(self) -> None:
        _validate(self.block_size, self.scale_factor, self.rule)

    def make_quantizer(self) -> MXFP4FakeQuantizer:
        return MXFP4FakeQuantizer(self.block_size, self.scale_factor, self.clip_grad, self.rule)


class MXFP4QATLinear(nn.Linear):
    """``nn.Linear`` whose weight (and optionally input) is MXFP4 fake-quantized;
    ``state_dict`` is identical to the float layer's."""

    def __init__(self, in_features: int, out_features: int, bias: bool = True, device=None,
                 dtype=None, config: MXFP4QATConfig | None = None) -> None:
        super().__init__(in_features, out_features, bias, device=device, dtype=dtype)
        self.config = config if config is not None else MXFP4QATConfig()
        self.weight_quantizer = self.config.make_quantizer() if self.config.quantize_weight else None
        self.input_quantizer = self.config.make_quantizer() if self.config.quantize_input else None

    @classmethod
    def from_linear(cls, linear: nn.Linear, config: MXFP4QATConfig | None = None) -> "MXFP4QATLinear":
        """Wrap an existing Linear, adopting its Parameter objects (no copy)."""
        q = cls(linear.in_features, linear.out_features, bias=linear.bias is not None,
                device="meta", dtype=linear.weight.dtype, config=config)
        q.weight = linear.weight
        if linear.bias is not None:
            q.bias = linear.bias
        return q

    def forward(self, input: torch.Tensor) -> torch.Tensor:
        if self.input_quantizer is not None:
            input = self.input_quantizer(input)
        weight = self.weight
        if self.weight_quantizer is not None:
            weight = self.weight_quantizer(weight)
        return F.linear(input, weight, self.bias)


def convert_to_mxfp4_qat(module: nn.Module, config: MXFP4QATConfig | None = None,
                         skip_names: tuple[str, ...] = ()) -> nn.Module:
    """Replace every ``nn.Linear`` below ``module`` in place (a dotted path
    containing any of ``skip_names`` is left, with its subtree, as is);
    already converted layers are kept, so converting twice is a no-op."""

    def walk(mod: nn.Module, prefix: str) -> None:
        for name, child in list(mod.named_children()):
            path = f"{prefix}{name}"
            if any(s in path for s in skip_names):
                continue
            if isinstance(child, MXFP4QATLinear):
                continue
            if isinstance(child, nn.Linear):
                setattr(mod, name, MXFP4QATLinear.from_linear(child, config))
            else:
                walk(child, f"{path}.")

    walk(module, "")
    return module
