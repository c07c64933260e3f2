"""MXFP4 quantization-aware training over the C-ABI kernels.

What the amct PR "feat: add MXFP4 QAT fake-quant Linear (with STE)" offers
around its QDQ operator (README section "1. MXFP4 and STE"): a differentiable
fake quantization whose backward is the straight-through estimator (plain or
clipped), and a Linear layer that computes F.linear(Q(x), Q(W), b) with a
float master weight, keeps a state_dict identical to the float layer's, and is
swapped into a model in place (named layers can be left in float, converting
twice changes nothing).  Here every step runs in libmxfp4's HIP kernels:

- ``MXFP4Spec``: how one tensor is fake-quantized (block, scale rule, scale
  factor, clipped or plain STE); calling it quantizes a tensor.
- ``QATPolicy``: which operands of a linear layer are quantized (weight,
  activation), each with its own spec or None.
- ``QATLinear``: an ``nn.Linear`` whose forward applies the policy;
  ``QATLinear.wrap`` turns an existing Linear into one in place of it, sharing
  its Parameter objects.
- ``quantize_model``: swaps every Linear of a model (outside the excluded
  paths) for a QATLinear.

The names of the PR's interface (``mxfp4_fake_quant``, ``MXFP4FakeQuantizer``,
``MXFP4QATConfig``, ``MXFP4QATLinear``, ``convert_to_mxfp4_qat``) are kept as
thin entry points onto these, with the PR's argument names, for code written
against it.

There is no CPU path: tensors must be on the GPU and bf16 or fp32.  Blocks run
along the last dimension (row-wise), as the PR blocks a tensor.
"""
from __future__ import annotations

import dataclasses
from typing import Iterable, Optional

import torch
import torch.nn.functional as F
from torch import nn

from . import ROW, mxfp4_qdq_fwd, mxfp4_qdq_fwd_rows_batch, mxfp4_ste_bwd, mxfp4_ste_bwd_rows_batch

__all__ = ["MXFP4Spec", "QATPolicy", "QATLinear", "FakeQuant", "fake_quant", "quantize_model",
           "mxfp4_fake_quant", "MXFP4FakeQuantizer", "MXFP4QATConfig", "MXFP4QATLinear",
           "convert_to_mxfp4_qat"]


@dataclasses.dataclass(frozen=True)
class MXFP4Spec:
    """One tensor's fake quantization: blocks of ``block`` elements along the
    last dimension, the E8M0 scale rule (``"floor"``: 2^(floor(log2 amax) - 2);
    ``"amct"``: the PR's rounded log2 of amax / scale_factor), and the
    backward: the plain STE (gradient unchanged) or, with ``clipped``, the
    clipped STE (zero where |x| > 6 * scale)."""

    block: int = 32
    rule: str = "floor"
    scale_factor: float = 6.0
    clipped: bool = False

    def __post_init__(self):
        if self.block not in (32, 128):
            raise ValueError(f"block must be 32 or 128, got {self.block}")
        if self.rule not in ("floor", "amct"):
            raise ValueError(f"rule must be 'floor' or 'amct', got {self.rule!r}")
        if not self.scale_factor > 0:
            raise ValueError(f"scale_factor must be positive, got {self.scale_factor}")

    def __call__(self, t: torch.Tensor) -> torch.Tensor:
        return _FakeQuantSTE.apply(t, self)


class _FakeQuantSTE(torch.autograd.Function):
    """QDQ forward (+ clip bitmap when clipping); STE backward."""

    @staticmethod
    def forward(ctx, x, spec: MXFP4Spec):
        if x.dim() == 0:
            raise ValueError("x must have at least 1 dimension")
        xc = x.contiguous()
        cols = xc.shape[-1]
        rows = xc.numel() // cols if cols else 0
        y = torch.empty_like(xc)
        mask = None
        if spec.clipped:
            mask = torch.empty((rows, -(-cols // 32)), dtype=torch.int32, device=xc.device)
        mxfp4_qdq_fwd(xc, ROW, y_row=y, mask_row=mask, block=spec.block, rule=spec.rule,
                      scale_factor=spec.scale_factor)
        ctx.spec = spec
        if spec.clipped:
            ctx.save_for_backward(mask)
        return y

    @staticmethod
    def backward(ctx, grad_output):
        if not ctx.spec.clipped:
            return grad_output, None                       # plain STE: identity
        (mask,) = ctx.saved_tensors
        g = grad_output.contiguous()
        grad_in = torch.empty_like(g)
        mxfp4_ste_bwd(g, mask, grad_in, layout=ROW, block=ctx.spec.block)
        return grad_in, None


class _FakeQuantPairSTE(torch.autograd.Function):
    """Two tensors under specs that share block, rule and scale factor (the
    layer's input and weight): one batched forward launch, one batched STE
    launch for the clipped ones."""

    @staticmethod
    def forward(ctx, a, b, sa: MXFP4Spec, sb: MXFP4Spec):
        ts = [a.contiguous(), b.contiguous()]
        ys = [torch.empty_like(t) for t in ts]
        masks = []
        for t, sp in zip(ts, (sa, sb)):
            if sp.clipped:
                cols = t.shape[-1]
                rows = t.numel() // cols if cols else 0
                masks.append(torch.empty((rows, -(-cols // 32)), dtype=torch.int32, device=t.device))
            else:
                masks.append(None)
        mxfp4_qdq_fwd_rows_batch(ts, ys, masks, block=sa.block, rule=sa.rule, scale_factor=sa.scale_factor)
        ctx.block = sa.block
        ctx.clipped = (sa.clipped, sb.clipped)
        ctx.save_for_backward(*[m for m in masks if m is not None])
        return ys[0], ys[1]

    @staticmethod
    def backward(ctx, ga, gb):
        saved = list(ctx.saved_tensors)
        masks = [saved.pop(0) if c else None for c in ctx.clipped]
        outs, gs, gis, ms = [ga, gb], [], [], []
        for i, (g, m) in enumerate(zip((ga, gb), masks)):
            if g is None or m is None:
                continue                               # plain STE (or no gradient): unchanged
            g = g.contiguous()
            gi = torch.empty_like(g)
            gs.append(g)
            gis.append(gi)
            ms.append(m)
            outs[i] = gi
        if gs:
            mxfp4_ste_bwd_rows_batch(gs, ms, gis, block=ctx.block)
        return outs[0], outs[1], None, None


def _pairable(a: torch.Tensor, b: torch.Tensor, sa: MXFP4Spec, sb: MXFP4Spec) -> bool:
    return (a.dtype == b.dtype and a.dtype in (torch.bfloat16, torch.float32) and a.dim() > 0 and b.dim() > 0
            and (sa.block, sa.rule, sa.scale_factor) == (sb.block, sb.rule, sb.scale_factor))


def fake_quant(x: torch.Tensor, spec: MXFP4Spec = MXFP4Spec()) -> torch.Tensor:
    """Differentiable MXFP4 fake quantization of ``x`` (same shape, dtype and
    device) under ``spec``."""
    return spec(x)


class FakeQuant(nn.Module):
    """A spec as a module: no parameters and no buffers, so a model that holds
    one keeps the float model's state_dict."""

    def __init__(self, spec: MXFP4Spec = MXFP4Spec()):
        super().__init__()
        self.spec = spec

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return self.spec(x)

    def extra_repr(self) -> str:
        s = self.spec
        return f"block={s.block}, rule={s.rule!r}, scale_factor={s.scale_factor}, clipped={s.clipped}"


@dataclasses.dataclass(frozen=True)
class QATPolicy:
    """Which operands of a linear layer are fake-quantized: ``weight`` and
    ``activation`` (the layer input) each take a spec, or None to stay in
    float.  The bias is never quantized."""

    weight: Optional[MXFP4Spec] = MXFP4Spec()
    activation: Optional[MXFP4Spec] = None

    @classmethod
    def w4a16(cls, **spec) -> "QATPolicy":
        """Weights in MXFP4, activations in float."""
        return cls(weight=MXFP4Spec(**spec), activation=None)

    @classmethod
    def w4a4(cls, **spec) -> "QATPolicy":
        """Weights and activations in MXFP4 with the same spec."""
        s = MXFP4Spec(**spec)
        return cls(weight=s, activation=s)


class QATLinear(nn.Linear):
    """``nn.Linear`` computing ``F.linear(A(x), W(weight), bias)`` where A and W
    are the policy's specs (identity where a spec is None).  The float weight
    stays the trained parameter; its state_dict keys and tensors are those of
    an ``nn.Linear``."""

    def __init__(self, in_features: int, out_features: int, bias: bool = True, *,
                 policy: Optional[QATPolicy] = None, device=None, dtype=None):
        super().__init__(in_features, out_features, bias, device=device, dtype=dtype)
        self.policy = QATPolicy() if policy is None else policy

    @classmethod
    def wrap(cls, linear: nn.Linear, policy: Optional[QATPolicy] = None) -> "QATLinear":
        """A QATLinear that holds ``linear``'s own Parameter objects (nothing is
        allocated or copied, so optimizer state keyed on them stays valid)."""
        q = cls.__new__(cls)
        nn.Module.__init__(q)
        q.in_features, q.out_features = linear.in_features, linear.out_features
        q.register_parameter("weight", linear.weight)
        q.register_parameter("bias", linear.bias)
        q.policy = QATPolicy() if policy is None else policy
        q.train(linear.training)
        return q

    from_linear = wrap  # the PR's name

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        p = self.policy
        if p.activation is not None and p.weight is not None and _pairable(x, self.weight, p.activation, p.weight):
            xq, wq = _FakeQuantPairSTE.apply(x, self.weight, p.activation, p.weight)  # one launch each way
        else:
            xq = x if p.activation is None else p.activation(x)
            wq = self.weight if p.weight is None else p.weight(self.weight)
        return F.linear(xq, wq, self.bias)

    def extra_repr(self) -> str:
        return f"{super().extra_repr()}, policy={self.policy}"


def quantize_model(model: nn.Module, policy: Optional[QATPolicy] = None,
                   exclude: Iterable[str] = ()) -> nn.Module:
    """Swap every ``nn.Linear`` (subclasses included) of ``model`` for a
    QATLinear sharing its parameters, in place; returns ``model``.  A module
    whose dotted path contains one of the ``exclude`` strings is left as it
    is, with everything below it.  QATLinear layers are left as they are, so
    converting again changes nothing; a Linear reachable under several paths
    becomes one QATLinear."""
    exclude = tuple(exclude)
    policy = QATPolicy() if policy is None else policy
    done = {}                       # id(original Linear) -> its QATLinear
    replaced = []                   # paths already swapped (their subtrees go with them)
    for path, mod in list(model.named_modules(remove_duplicate=False)):
        if not path or isinstance(mod, QATLinear) or not isinstance(mod, nn.Linear):
            continue
        if any(s in path for s in exclude) or any(path.startswith(r + ".") for r in replaced):
            continue
        parent_path, _, leaf = path.rpartition(".")
        parent = model.get_submodule(parent_path) if parent_path else model
        if id(mod) not in done:
            done[id(mod)] = QATLinear.wrap(mod, policy)
        setattr(parent, leaf, done[id(mod)])
        replaced.append(path)
    return model


# ---------------------------------------------------------------------------
# The PR's interface names, onto the pieces above.

def mxfp4_fake_quant(x: torch.Tensor, block_size: int = 32, scale_factor: float = 6.0,
                     clip_grad: bool = False, rule: str = "floor") -> torch.Tensor:
    """Fake-quantize ``x`` over its last dimension; the gradient flows back
    unchanged, or zeroed where the forward clipped (``clip_grad``)."""
    return MXFP4Spec(block_size, rule, scale_factor, clip_grad)(x)


def MXFP4FakeQuantizer(block_size: int = 32, scale_factor: float = 6.0, clip_grad: bool = False,
                       rule: str = "floor") -> FakeQuant:
    """The PR's stateless quantizer module: a FakeQuant of that spec."""
    return FakeQuant(MXFP4Spec(block_size, rule, scale_factor, clip_grad))


def MXFP4QATConfig(quantize_weight: bool = True, quantize_input: bool = False, block_size: int = 32,
                   scale_factor: float = 6.0, clip_grad: bool = False, rule: str = "floor") -> QATPolicy:
    """The PR's settings (W4A16 by default) as a QATPolicy: one spec shared by
    the quantized operands."""
    spec = MXFP4Spec(block_size, rule, scale_factor, clip_grad)
    return QATPolicy(weight=spec if quantize_weight else None, activation=spec if quantize_input else None)


MXFP4QATLinear = QATLinear


def convert_to_mxfp4_qat(module: nn.Module, config: Optional[QATPolicy] = None,
                         skip_names: Iterable[str] = ()) -> nn.Module:
    """quantize_model with the PR's argument names."""
    return quantize_model(module, config, exclude=skip_names)
