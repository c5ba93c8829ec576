"""Helpers shared by the GPU parity tests (host-side marshalling only).

Inputs come from ``synth`` (seeded generators, no method arithmetic);
expected values come only from ``oracle``; the library is reached through
the Python binding over the C ABI.
"""

import numpy as np
import torch

import synth

CANARY = 0x7FC1          # a quiet-NaN bf16 pattern no kernel ever writes


def dev():
    return torch.device("cuda", 0)


def up_bits(b):
    """numpy uint16 bf16 bits -> bf16 tensor on the GPU."""
    return synth.from_bits(b, dev())


def up(a):
    """numpy array (int32 / float32) -> tensor on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def down_bits(t):
    torch.cuda.synchronize()
    return synth.bits(t)


def down(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def canary_bf16(shape):
    """bf16 GPU tensor filled with the canary pattern."""
    t = torch.full(shape, CANARY, dtype=torch.int16, device=dev())
    return t.view(torch.bfloat16)


def say(msg):
    """Name the case before a GPU step (flushed, so a crash still shows it)."""
    print(msg, flush=True)
