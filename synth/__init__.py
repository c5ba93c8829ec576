"""Seeded synthetic inputs and the workload table.

This module holds no arithmetic of the quantization method: it only draws
seeded random tensors (torch generators, so the same code serves CPU tests
and on-device generation of multi-gigabyte expert weights) and lists the
workload shapes.  Both the oracle-side tests and the HIP-side callers use
it; neither side's arithmetic lives here.

Recipe (all draws are float32 normal samples, cast to bfloat16 by torch):

* weights:     N(0, 0.02^2)  shape [N, K] (expert weights: one stream per
  expert and matrix)
* activations: N(0, 1)       shape [M, K]
* router logits: N(0, 1)     shape [T, E]; for the skewed prefill layer,
  8 hot experts (the first 8 entries of a seeded permutation of E) receive
  +3.0 on T // 10 tokens drawn without replacement.

Each tensor gets its own generator seeded from (workload seed, stream id),
so any single tensor -- one expert's weight, say -- can be regenerated
without drawing the others.
"""

import numpy as np
import torch

WEIGHT_SIGMA = 0.02

# stream ids
S_W = 1
S_X = 2
S_LOGITS = 3
S_SKEW = 4
S_GATE_UP = 1000      # + expert index
S_DOWN = 200000       # + expert index

WORKLOADS = {
    "dense_small": dict(kind="dense", N=512, K=512, M=[4], seed=0),
    "decode": dict(kind="dense", N=12288, K=4096, M=[1, 8, 16, 32], seed=1),
    "prefill": dict(kind="dense", N=14336, K=4096, M=[4096], seed=2),
    "moe_qwen": dict(kind="moe", T=256, E=128, k=8, H=4096, I=1536, seed=3,
                     skew=None),
    "moe_kimi": dict(kind="moe", T=4096, E=384, k=8, H=7168, I=2048, seed=4,
                     skew=dict(hot=8, frac_div=10, bias=3.0)),
}


def stream_seed(seed, stream):
    """Distinct 63-bit seed per (workload seed, stream id)."""
    return (int(seed) * 1_000_003 + int(stream) * 7_919 + 0x5EED) % (1 << 63)


def generator(seed, stream, device="cpu"):
    g = torch.Generator(device=device)
    g.manual_seed(stream_seed(seed, stream))
    return g


def normal_bf16(shape, sigma, seed, stream, device="cpu"):
    """bf16 tensor of N(0, sigma^2) draws (float32 sample, cast by torch)."""
    g = generator(seed, stream, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(sigma)
    return x.to(torch.bfloat16)


def weights(N, K, seed, stream=S_W, device="cpu"):
    return normal_bf16((N, K), WEIGHT_SIGMA, seed, stream, device)


def activations(M, K, seed, stream=S_X, device="cpu"):
    return normal_bf16((M, K), 1.0, seed, stream, device)


def activations_wide(M, K, seed, gain=1.0, outlier_frac=0.0, outlier_gain=1.0,
                     stream=S_X, device="cpu"):
    """N(0, 1) activations times a power-of-two ``gain`` (exact in bf16),
    with a seeded ``outlier_frac`` of the K channels times a further
    power-of-two ``outlier_gain`` (the few large channels of real hidden
    states).  Returns (bf16 tensor, sorted outlier channel indices)."""
    x = activations(M, K, seed, stream, device)
    if gain != 1.0:
        x = x * gain
    g = generator(seed, stream + 500, "cpu")
    n_out = int(round(outlier_frac * K))
    ch = torch.sort(torch.randperm(K, generator=g)[:n_out]).values
    if n_out:
        x[:, ch.to(x.device)] *= outlier_gain
    return x, ch.numpy()


def expert_gate_up(e, I, H, seed, device="cpu"):
    return normal_bf16((2 * I, H), WEIGHT_SIGMA, seed, S_GATE_UP + e, device)


def expert_down(e, I, H, seed, device="cpu"):
    return normal_bf16((H, I), WEIGHT_SIGMA, seed, S_DOWN + e, device)


def _skew_draw(T, E, seed, skew):
    gs = generator(seed, S_SKEW, "cpu")
    hot = torch.randperm(E, generator=gs)[: skew["hot"]]
    biased = torch.randperm(T, generator=gs)[: T // skew["frac_div"]]
    return hot, biased


def hot_experts(T, E, seed, skew):
    """The experts the skew biases (sorted), as router_logits draws them."""
    return sorted(int(e) for e in _skew_draw(T, E, seed, skew)[0])


def router_logits(T, E, seed, skew=None, device="cpu"):
    """float32 [T, E] logits; optional hot-expert skew (see module doc)."""
    g = generator(seed, S_LOGITS, "cpu")
    lg = torch.randn((T, E), generator=g, dtype=torch.float32)
    if skew is not None:
        hot, biased = _skew_draw(T, E, seed, skew)
        lg[biased.unsqueeze(1), hot.unsqueeze(0)] += skew["bias"]
    return lg.to(device)


def random_ids(T, k, E, seed, device="cpu"):
    """Top-k style expert ids: k distinct experts per token, uniform."""
    g = generator(seed, S_LOGITS + 17, "cpu")
    ids = torch.argsort(torch.rand((T, E), generator=g), dim=1)[:, :k]
    return ids.to(torch.int32).contiguous().to(device)


def bits(t):
    """bf16 torch tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(b, device="cpu"):
    """numpy uint16 bit patterns -> bf16 torch tensor."""
    arr = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(device)
