"""Quantization-aware training op: INT4 fake quant with a straight-through
estimator ("INT4 QAT end-to-end for RL" §2.1; "Quantization basics: from
FP32 to INT4", the STE passage).

Forward: W_fq = bf16(q * s) with s = bf16(amax / 7) per 32-element group
and q = clamp(rint_even(w / s), -8, 7), computed by ``w4_fake_quant`` (the
library's HIP kernel, through the C ABI).  Backward: the straight-through
estimator treats the rounding as the identity, so dL/dW = dL/dW_fq.  With
s = amax / 7 no weight of a group lies outside [-7 s, 7 s], so the clipped
variant of the estimator (zero gradient where w was clamped) never masks
anything and equals the identity.

The master weight stays bf16; only the forward sees the quantization grid,
so training and INT4 inference use the same values (fake quant equals the
dequantized packed weight bit for bit).
"""

import torch

from . import w4_fake_quant

__all__ = ["FakeInt4STE", "fake_quant_ste"]


class FakeInt4STE(torch.autograd.Function):
    """y = fake_quant(W) forward, dy/dW = identity backward."""

    @staticmethod
    def forward(ctx, W):
        return w4_fake_quant(W.contiguous())

    @staticmethod
    def backward(ctx, grad_out):
        return grad_out


def fake_quant_ste(W):
    """Fake-quantized bf16 weight [N, K] (K % 32 == 0) whose gradient flows
    straight through to W."""
    return FakeInt4STE.apply(W)
