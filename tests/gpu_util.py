"""Helpers shared by the GPU parity tests (inputs from the seeded generators)."""

import numpy as np
import torch

from synth.workloads import bf16_to_bits, normal_bf16

DEV = "cuda"


def gen(shape, sigma, seed):
    """Seeded bf16 tensor generated on the CPU, then copied to the GPU."""
    t = normal_bf16(shape, sigma, seed, "cpu")
    return t.to(DEV), bf16_to_bits(t)


def channel_varied(shape, sigma, seed, axis):
    """bf16 weights whose channels differ in magnitude by up to e^+-3 (per-channel scales matter)."""
    t = normal_bf16(shape, sigma, seed, "cpu").float()
    g = torch.Generator().manual_seed(seed + 1000)
    mshape = [1] * len(shape)
    mshape[0] = shape[0]
    mshape[axis] = shape[axis]
    mult = torch.exp(torch.rand(mshape, generator=g) * 6 - 3)
    t = (t * mult).to(torch.bfloat16)
    return t.to(DEV), bf16_to_bits(t)


def gs_tensor(sizes):
    return torch.tensor(np.asarray(sizes, np.int32), device=DEV)


def sync():
    torch.cuda.synchronize()
