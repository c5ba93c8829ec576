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

``qat_linear`` is the layer form: y = x * fake_quant(W)^T.  Because the
dequantized packed weight equals the fake-quantized one bit for bit, its
forward packs W (``w4_quantize_pack``) and runs the W4A16 product on the
codes ("INT4 QAT end-to-end for RL" §4) instead of writing W_fq and reading
it back: 3.125 bytes of weight traffic per element (read W, write and read
0.5625 bytes of codes and scales) instead of 6 (read W, write W_fq, read
W_fq).  The backward is the straight-through estimator.  The input
gradient dX = dY * W_fq runs in the library: ``w4_dequant_t`` writes W_fq^T
from the packed codes the forward made (bit-exact with fake quant) and
``w4_bf16_gemm_nt`` multiplies (N % 8 == 0).  The weight gradient
dW = dY^T * X runs in the library too: ``w4_bf16_transpose`` writes dY^T and
X^T with the token dimension padded to a multiple of 8 (zeros), and
``w4_bf16_gemm_nt`` contracts over it.
"""

import torch

from . import (w4_bf16_gemm_nt, w4_bf16_transpose, w4_dequant_t, w4_fake_quant, w4_quantize_pack,
               w4a16_gemm)

__all__ = ["FakeInt4STE", "fake_quant_ste", "Int4QATLinear", "qat_linear"]


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


class Int4QATLinear(torch.autograd.Function):
    """y = x * fake_quant(W)^T through the packed INT4 product; straight-through
    backward to the bf16 master weight."""

    @staticmethod
    def forward(ctx, X, W):
        N, K = W.shape
        if X.shape[-1] != K:
            raise ValueError(f"X has {X.shape[-1]} features, W expects {K}")
        W = W.contiguous()
        X2 = X.reshape(-1, K).contiguous()
        Wq, S = w4_quantize_pack(W)
        Y = w4a16_gemm(X2, Wq, S)
        ctx.save_for_backward(X2, Wq, S)
        ctx.x_shape = X.shape
        return Y.reshape(*X.shape[:-1], N)

    @staticmethod
    def backward(ctx, grad_out):
        X2, Wq, S = ctx.saved_tensors
        N = Wq.shape[0]
        dY = grad_out.reshape(-1, N).to(torch.bfloat16).contiguous()
        dX = dW = None
        if ctx.needs_input_grad[0]:
            if N % 8:
                raise ValueError(f"the QAT input gradient needs N % 8 == 0 (N = {N})")
            dX = w4_bf16_gemm_nt(dY, w4_dequant_t(Wq, S)).reshape(ctx.x_shape)
        if ctx.needs_input_grad[1]:
            Mp = (dY.shape[0] + 7) // 8 * 8
            dW = w4_bf16_gemm_nt(w4_bf16_transpose(dY, Mp), w4_bf16_transpose(X2, Mp))
        return dX, dW


def qat_linear(X, W):
    """QAT linear layer without bias: X bf16 [..., K], W bf16 [N, K]
    (K % 32 == 0) -> bf16 [..., N] = X * fake_quant(W)^T."""
    return Int4QATLinear.apply(X, W)
