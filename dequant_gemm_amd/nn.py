"""NF4Linear: a frozen NF4-quantized linear layer with autograd over the fused GEMMs.

"Zenbit" page, section "What's inside": the fused NF4 dense layer takes an
activation and a quantized weight; its custom backward forms the gradient with
respect to the activation only (the quantized weight is frozen, no weight
gradient).  "bitsandbytes" page, 4-bit/LoRA paragraph: the 4-bit base weights
stay frozen while adapters train.

Forward:  y = x W^T by ``nf4_matmul_fwd`` (W^ formed on chip, never in memory).
Backward: dx = dy W^ by ``nf4_matmul_bwd_dx``; the weight gets no gradient.

Every product runs in libnf4's kernels.  The layer takes bf16 activations of
any leading shape [..., in_features] and returns [..., out_features] in
``out_dtype`` (bf16 by default: one round-to-nearest-even of the fp32
accumulator inside the kernel; fp32 on request).  The gradient it returns for
x is bf16 like x, rounded once inside the kernel.  An incoming fp32 gradient
is rounded to bf16 (torch's round-to-nearest-even conversion) before the
backward GEMM, whose operands are bf16.  Layers with a bias are not supported:
the decoder linears this path serves have none.
"""
from __future__ import annotations

from typing import Optional

import torch

from ._lib import (LORA_MAX_RANK, LORA_RANK_STEP, QTensor, nf4_adapter_matmul, nf4_matmul_bwd_dx, nf4_matmul_bwd_dx_lora,
                   nf4_matmul_fwd, nf4_matmul_fwd_lora, nf4_quantize)


class _NF4Matmul(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x: torch.Tensor, q: QTensor, out_dtype: torch.dtype):
        lead = x.shape[:-1]
        x2 = x.reshape(-1, q.cols)
        if not x2.is_contiguous():
            x2 = x2.contiguous()
        y = nf4_matmul_fwd(x2, q, out_dtype)
        ctx.q = q
        ctx.lead = lead
        return y.reshape(*lead, q.rows)

    @staticmethod
    def backward(ctx, gy: torch.Tensor):
        q = ctx.q
        g2 = gy.reshape(-1, q.rows)
        if g2.dtype != torch.bfloat16:
            g2 = g2.to(torch.bfloat16)
        if not g2.is_contiguous():
            g2 = g2.contiguous()
        dx = nf4_matmul_bwd_dx(g2, q, torch.bfloat16)
        return dx.reshape(*ctx.lead, q.cols), None, None


def nf4_linear(x: torch.Tensor, q: QTensor, out_dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """y = x W^T for bf16 x [..., q.cols]; differentiable in x (the weight is frozen)."""
    if x.dtype != torch.bfloat16:
        raise TypeError(f"x must be bfloat16 (got {x.dtype})")
    if x.shape[-1] != q.cols:
        raise ValueError(f"x has {x.shape[-1]} features, the weight expects {q.cols}")
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out_dtype must be torch.bfloat16 or torch.float32")
    return _NF4Matmul.apply(x, q, out_dtype)


class NF4Linear(torch.nn.Module):
    """A bias-free linear layer whose frozen weight is stored NF4-quantized.

    Build it from a dense weight with :meth:`from_weight` or :meth:`from_linear`
    (quantized on the device by ``nf4_quantize``), or around an existing
    :class:`QTensor`.
    """

    def __init__(self, qweight: QTensor, out_dtype: torch.dtype = torch.bfloat16):
        super().__init__()
        if out_dtype not in (torch.bfloat16, torch.float32):
            raise TypeError("out_dtype must be torch.bfloat16 or torch.float32")
        self.qweight = qweight
        self.out_dtype = out_dtype

    @property
    def in_features(self) -> int:
        return self.qweight.cols

    @property
    def out_features(self) -> int:
        return self.qweight.rows

    @classmethod
    def from_weight(cls, weight: torch.Tensor, double_quant: bool = True,
                    out_dtype: torch.dtype = torch.bfloat16, quant_type: str = "nf4") -> "NF4Linear":
        """Quantizes a [out_features, in_features] bf16/fp32 device weight (NF4, or FP4)."""
        if weight.dtype not in (torch.bfloat16, torch.float32):
            raise TypeError("weight must be bfloat16 or float32")
        if weight.dim() != 2:
            raise ValueError("weight must be 2-D [out_features, in_features]")
        w = weight.detach()
        if not w.is_contiguous():
            w = w.contiguous()
        return cls(nf4_quantize(w, double_quant=double_quant, quant_type=quant_type), out_dtype)

    @classmethod
    def from_linear(cls, linear: torch.nn.Linear, double_quant: bool = True,
                    out_dtype: torch.dtype = torch.bfloat16, quant_type: str = "nf4") -> "NF4Linear":
        if linear.bias is not None:
            raise ValueError("NF4Linear has no bias; the layer to convert has one")
        return cls.from_weight(linear.weight, double_quant, out_dtype, quant_type)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return nf4_linear(x, self.qweight, self.out_dtype)

    def extra_repr(self) -> str:
        return (f"in_features={self.in_features}, out_features={self.out_features}, "
                f"quant_type={self.qweight.quant_type}, double_quant={self.qweight.double_quant}, "
                f"out_dtype={self.out_dtype}")


class _NF4LoraMatmul(torch.autograd.Function):
    """y = x W^T + s (x A^T) B^T with the adapter term added inside the fused GEMM.

    Every product runs in libnf4: the down projection U = bf16(s x A^T)
    (nf4_adapter_matmul), the fused forward adding U B^T; in the backward
    V = bf16(s dy B), the fused input gradient adding V A, and the adapter's
    gradients dA = V^T x and dB = dy^T U (nf4_adapter_matmul, bf16 outputs).
    torch supplies memory and the stream.
    """

    @staticmethod
    def forward(ctx, x, lora_a, lora_b, q: QTensor, scaling: float, out_dtype: torch.dtype):
        lead = x.shape[:-1]
        x2 = x.reshape(-1, q.cols)
        if not x2.is_contiguous():
            x2 = x2.contiguous()
        u = nf4_adapter_matmul(x2, lora_a, trans_b=True, alpha=scaling, out_dtype=torch.bfloat16)   # [M, r]
        y = nf4_matmul_fwd_lora(x2, q, u, lora_b.contiguous(), out_dtype)
        ctx.save_for_backward(x2, lora_a, lora_b, u)
        ctx.q, ctx.lead, ctx.scaling = q, lead, scaling
        return y.reshape(*lead, q.rows)

    @staticmethod
    def backward(ctx, gy):
        x2, lora_a, lora_b, u = ctx.saved_tensors
        q, s = ctx.q, ctx.scaling
        g2 = gy.reshape(-1, q.rows)
        gb = g2 if g2.dtype == torch.bfloat16 else g2.to(torch.bfloat16)
        if not gb.is_contiguous():
            gb = gb.contiguous()
        v = nf4_adapter_matmul(gb, lora_b.contiguous(), alpha=s, out_dtype=torch.bfloat16)         # [M, r]
        dx = nf4_matmul_bwd_dx_lora(gb, q, v, lora_a.t().contiguous(), torch.bfloat16)
        d_a = nf4_adapter_matmul(v, x2, trans_a=True, out_dtype=lora_a.dtype)                        # [r, K]
        d_b = nf4_adapter_matmul(gb, u, trans_a=True, out_dtype=lora_b.dtype)                        # [N, r]
        return dx.reshape(*ctx.lead, q.cols), d_a, d_b, None, None, None


class NF4LoraLinear(torch.nn.Module):
    """A frozen NF4 linear layer plus a trainable low-rank adapter (QLoRA's layer).

    y = x W^T + (alpha / r) (x A^T) B^T with A [r, in_features] and B
    [out_features, r] trainable bf16 parameters; B starts at zero, so the layer
    starts equal to the frozen one.  The adapter term runs inside the fused
    NF4 GEMM (forward and input gradient).  The rank must be a multiple of 16
    (at most 1024).
    """

    def __init__(self, qweight: QTensor, r: int, alpha: float = None,
                 out_dtype: torch.dtype = torch.bfloat16, seed: int = 0):
        super().__init__()
        if r < LORA_RANK_STEP or r > LORA_MAX_RANK or r % LORA_RANK_STEP:
            raise ValueError(f"rank must be a multiple of {LORA_RANK_STEP} in [{LORA_RANK_STEP}, {LORA_MAX_RANK}]")
        if out_dtype not in (torch.bfloat16, torch.float32):
            raise TypeError("out_dtype must be torch.bfloat16 or torch.float32")
        self.qweight = qweight
        self.r = r
        self.scaling = float(alpha if alpha is not None else r) / r
        self.out_dtype = out_dtype
        dev = qweight.device
        g = torch.Generator(device="cpu").manual_seed(seed)
        bound = 1.0 / (qweight.cols ** 0.5)                   # uniform init of A, as nn.Linear's weight
        a = (torch.rand(r, qweight.cols, generator=g) * 2 - 1) * bound
        self.lora_a = torch.nn.Parameter(a.to(torch.bfloat16).to(dev))
        self.lora_b = torch.nn.Parameter(torch.zeros(qweight.rows, r, dtype=torch.bfloat16, device=dev))

    @classmethod
    def from_weight(cls, weight: torch.Tensor, r: int, alpha: float = None, double_quant: bool = True,
                    out_dtype: torch.dtype = torch.bfloat16, seed: int = 0,
                    quant_type: str = "nf4") -> "NF4LoraLinear":
        w = weight.detach()
        return cls(nf4_quantize(w if w.is_contiguous() else w.contiguous(), double_quant=double_quant,
                                quant_type=quant_type), r, alpha, out_dtype, seed)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if x.dtype != torch.bfloat16:
            raise TypeError(f"x must be bfloat16 (got {x.dtype})")
        if x.shape[-1] != self.qweight.cols:
            raise ValueError(f"x has {x.shape[-1]} features, the weight expects {self.qweight.cols}")
        return _NF4LoraMatmul.apply(x, self.lora_a, self.lora_b, self.qweight, self.scaling, self.out_dtype)

    def extra_repr(self) -> str:
        return (f"in_features={self.qweight.cols}, out_features={self.qweight.rows}, r={self.r}, "
                f"scaling={self.scaling}, out_dtype={self.out_dtype}")


def quantize_linears(module: torch.nn.Module, double_quant: bool = True,
                     out_dtype: torch.dtype = torch.bfloat16,
                     skip: Optional[set] = None, quant_type: str = "nf4") -> torch.nn.Module:
    """Replaces every bias-free ``nn.Linear`` below ``module`` by an NF4Linear, in place.

    ``skip`` holds qualified child names to leave dense; ``quant_type`` is "nf4"
    or "fp4".  Returns ``module``.
    """
    skip = skip or set()
    for name, child in list(module.named_modules()):
        for cname, c in list(child.named_children()):
            full = f"{name}.{cname}" if name else cname
            if isinstance(c, torch.nn.Linear) and c.bias is None and full not in skip:
                setattr(child, cname, NF4Linear.from_linear(c, double_quant, out_dtype, quant_type))
    return module
