"""GPU: the QAT ops (fake quant forward, straight-through backward).

Forward: bit-exact against the oracle's fake quant.  Backward: the
straight-through estimator passes the upstream gradient unchanged to the
bf16 master weight (grad_W == grad_out bit for bit), also through a small
linear layer whose loss depends on the fake-quantized weight.  The QAT
linear layer (forward through the packed INT4 product): forward within
|y - y_ref| <= 2e-2 + 1e-2 |y_ref| of the fp64 product with the oracle's
fake-quantized weight, and both gradients of the straight-through estimator
against fp64 references.
"""

import numpy as np
import pytest
import torch

import synth
from gpu_util import dev, down_bits, say, up_bits
from int4_weight_only_amd.qat import fake_quant_ste
from oracle import bf16, gemm, quant

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,K,seed", [(512, 512, 0), (96, 160, 7), (1, 32, 3)])
def test_forward_matches_oracle(N, K, seed):
    say(f"qat forward N={N} K={K}")
    Wb = synth.bits(synth.weights(N, K, seed))
    W = up_bits(Wb).requires_grad_(True)
    Y = fake_quant_ste(W)
    np.testing.assert_array_equal(down_bits(Y.detach()), quant.fake_quant(Wb))


@pytest.mark.parametrize("N,K", [(256, 512), (64, 96)])
def test_backward_is_identity(N, K):
    say(f"qat backward N={N} K={K}")
    W = synth.weights(N, K, 11).to(dev()).requires_grad_(True)
    G = synth.activations(N, K, 12).to(dev())
    Y = fake_quant_ste(W)
    Y.backward(G)
    torch.cuda.synchronize()
    assert W.grad is not None and W.grad.dtype == torch.bfloat16
    np.testing.assert_array_equal(synth.bits(W.grad), synth.bits(G))


def test_gradient_through_a_linear_layer():
    """loss = sum(X @ fq(W)^T * R): dloss/dW = R^T @ X exactly as for an
    unquantized weight (the estimator hides the rounding)."""
    say("qat linear layer")
    M, N, K = 8, 64, 128
    W = synth.weights(N, K, 21).to(dev()).float().requires_grad_(True)
    X = synth.activations(M, K, 22).to(dev()).float()
    R = synth.activations(M, N, 23).to(dev()).float()
    Wq = fake_quant_ste(W.to(torch.bfloat16)).float()
    loss = ((X @ Wq.t()) * R).sum()
    loss.backward()
    torch.cuda.synchronize()
    # the gradient reaches W through one bf16 cast; the two fp32 products may
    # round differently, so allow one bf16 step
    expect = (R.t().cpu().double() @ X.cpu().double()).numpy()
    np.testing.assert_allclose(W.grad.cpu().numpy(), expect, rtol=2 ** -7, atol=1e-3)
    # and the forward used the quantization grid
    ref = quant.fake_quant(synth.bits(W.detach().to(torch.bfloat16).cpu()))
    np.testing.assert_array_equal(synth.bits(Wq.detach().to(torch.bfloat16)), ref)


# ------------------------------------------------------------ QAT linear --

ATOL, RTOL = 2e-2, 1e-2


@pytest.mark.parametrize("shape,N,K", [((1, 544), 96, 544), ((16, 256), 200, 256),
                                       ((33, 512), 64, 512), ((2, 150, 160), 48, 160)])
def test_qat_linear_forward_matches_oracle(shape, N, K):
    """Forward = X * fake_quant(W)^T, the fake-quantized weight from the
    oracle's own quantizer, fp64 product; decode (M <= 32) and tiled (M > 32)
    products both run."""
    from int4_weight_only_amd.qat import qat_linear
    say(f"qat_linear forward X{shape} N={N} K={K}")
    Wb = synth.bits(synth.weights(N, K, 31))
    Xb = synth.bits(synth.activations(int(np.prod(shape[:-1])), K, 32)).reshape(*shape)
    Y = qat_linear(up_bits(Xb), up_bits(Wb))
    assert tuple(Y.shape) == tuple(shape[:-1]) + (N,)
    wfq = bf16.to_f32(quant.fake_quant(Wb)).astype(np.float64)
    ref = bf16.to_f32(Xb.reshape(-1, K)).astype(np.float64) @ wfq.T
    ok, a, r = gemm.within_tolerance(down_bits(Y).reshape(-1, N), ref, ATOL, RTOL)
    assert ok, (a, r)


@pytest.mark.parametrize("M", [40, 37, 300])
def test_qat_linear_backward_is_straight_through(M):
    """dX = dY * fake_quant(W) and dW = dY^T * X (the estimator passes the
    gradient of the quantized weight to the master weight); M = 37 pads the
    token dimension of the weight gradient's transposed operands."""
    from int4_weight_only_amd.qat import qat_linear
    say(f"qat_linear backward M={M}")
    N, K = 64, 128
    Wb = synth.bits(synth.weights(N, K, 41))
    Xb = synth.bits(synth.activations(M, K, 42))
    Gb = synth.bits(synth.activations(M, N, 43))
    W = up_bits(Wb).requires_grad_(True)
    X = up_bits(Xb).requires_grad_(True)
    Y = qat_linear(X, W)
    Y.backward(up_bits(Gb))
    torch.cuda.synchronize()
    g = bf16.to_f32(Gb).astype(np.float64)
    x = bf16.to_f32(Xb).astype(np.float64)
    wfq = bf16.to_f32(quant.fake_quant(Wb)).astype(np.float64)
    for got, ref, name in ((X.grad, g @ wfq, "dX"), (W.grad, g.T @ x, "dW")):
        assert got.dtype == torch.bfloat16
        ok, a, r = gemm.within_tolerance(down_bits(got), ref, ATOL, RTOL)
        assert ok, (name, a, r)


# ------------------------------------------------- input-gradient kernels --

@pytest.mark.parametrize("asym", [False, True])
@pytest.mark.parametrize("N,K", [(1, 32), (63, 96), (64, 128), (200, 544), (1000, 4096)])
def test_dequant_t_bit_exact(asym, N, K):
    """w4_dequant_t = the oracle's dequantized weight, transposed, bit for bit
    (N not a multiple of 8 takes the element-store tail)."""
    import int4_weight_only_amd as w4
    from oracle import quant_asym
    say(f"dequant_t asym={asym} N={N} K={K}")
    Wb = synth.bits(synth.weights(N, K, 50 + N))
    if asym:
        Wq, S, Z = quant_asym.quantize_pack_asym(Wb)
        ref = quant_asym.dequant_asym(quant_asym.unpack_unsigned(Wq), S, Z)
        got = w4.w4_dequant_t(torch.from_numpy(Wq).to(dev()), up_bits(S),
                              torch.from_numpy(Z).to(dev()))
    else:
        Wq, S = quant.quantize_pack(Wb)
        ref = quant.dequant(quant.unpack(Wq), S)
        got = w4.w4_dequant_t(torch.from_numpy(Wq).to(dev()), up_bits(S))
    np.testing.assert_array_equal(down_bits(got), np.ascontiguousarray(ref.T))


@pytest.mark.parametrize("M,N,K", [(1, 1, 8), (5, 7, 24), (130, 257, 96), (64, 128, 4096),
                                   (300, 200, 14336), (4096, 4096, 14336)])
def test_bf16_gemm_nt_matches_oracle(M, N, K):
    """C = A B^T against the fp64 product of the same bf16 operands; the
    last shape is the input gradient of the prefill layer (dY [4096, 14336]
    times W'^T [4096, 14336])."""
    import int4_weight_only_amd as w4
    say(f"bf16_gemm_nt M={M} N={N} K={K}")
    Ab = synth.bits(synth.activations(M, K, 60))
    Bb = synth.bits(synth.weights(N, K, 61))
    C = down_bits(w4.w4_bf16_gemm_nt(up_bits(Ab), up_bits(Bb)))
    ref = bf16.to_f32(Ab).astype(np.float64) @ bf16.to_f32(Bb).astype(np.float64).T
    ok, a, r = gemm.within_tolerance(C, ref, ATOL, RTOL)
    assert ok, (a, r)


@pytest.mark.parametrize("R,C,RP,offset", [(1, 1, 1, 0), (37, 64, 40, 0), (64, 64, 64, 0),
                                          (130, 200, 136, 0), (4096, 4096, 4096, 0),
                                          (45, 19, 45, 0), (33, 40, 48, 1), (0, 16, 8, 0)])
def test_bf16_transpose_bit_exact(R, C, RP, offset):
    """AT[c, r] = A[r, c], zero columns r >= R; 16-byte paths (C and RP
    multiples of 8, aligned buffers) and the element-wise path (ragged C, or
    buffers one element off)."""
    import int4_weight_only_amd as w4
    say(f"transpose R={R} C={C} RP={RP} offset={offset}")
    Ab = synth.bits(synth.activations(max(R, 1), C, 62))[:R]
    flat = torch.zeros(R * C + offset, dtype=torch.bfloat16, device=dev())
    A = flat[offset:].view(R, C)
    if R:
        A.copy_(up_bits(np.ascontiguousarray(Ab)).view(R, C))
    out = torch.full((C * RP + offset,), 3.0, dtype=torch.bfloat16, device=dev())
    w4.w4_bf16_transpose(A, RP, out=out[offset:])
    got = down_bits(out[offset:]).reshape(C, RP)
    ref = np.zeros((C, RP), dtype=np.uint16)
    ref[:, :R] = np.asarray(Ab).reshape(R, C).T
    np.testing.assert_array_equal(got, ref)


def test_qat_linear_input_gradient_needs_n_multiple_of_8():
    from int4_weight_only_amd.qat import qat_linear
    say("qat_linear N % 8 != 0")
    W = synth.weights(36, 64, 70).to(dev()).requires_grad_(True)
    X = synth.activations(4, 64, 71).to(dev()).requires_grad_(True)
    Y = qat_linear(X, W)
    with pytest.raises(ValueError, match="N % 8"):
        Y.backward(torch.ones_like(Y))
