"""Parity metrics between the HIP library's outputs and the oracle's.

Floating-point outputs (the reading of "max relative error 1e-3 after identical
quantization"): per group, max |Y - R| / max |R| <= tol, where R is the oracle's
fp32-accumulated result and Y the library's f32 output.  A group whose reference is
all zero must be exactly zero.  bf16 outputs cannot meet 1e-3 against an fp32
reference (half a bf16 ulp is up to 2^-8 relative), so for them every element must be
RNE_bf16(R) or one of its two bf16 neighbours.
Codes and scales: byte-exact.
"""

import numpy as np
import torch

from oracle.fp8 import f32_to_bf16_bits

TOL = 1e-3


def to_np(t):
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def group_rel_err(Y, R, row_ranges):
    """max over groups of max|Y-R| / max|R| (rows of each group); zero groups must match exactly."""
    worst = 0.0
    for lo, hi in row_ranges:
        if hi <= lo:
            continue
        y, r = Y[lo:hi].astype(np.float64), R[lo:hi].astype(np.float64)
        den = np.abs(r).max()
        if den == 0:
            assert np.all(y == 0), "reference group is zero but output is not"
            continue
        worst = max(worst, float(np.abs(y - r).max() / den))
    return worst


def slab_rel_err(Y, R):
    """tgmm: the same metric per [K, N] slab."""
    return group_rel_err(Y, R, [(g, g + 1) for g in range(Y.shape[0])])


def _ordered(bits):
    """bf16 bits -> integers in value order (so adjacent values differ by 1)."""
    b = bits.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)


def assert_bf16_close(Ybits, R, ranges=None, tol=TOL, min_exact=0.95):
    """bf16 outputs: every element lies between RNE_bf16(R - d) and RNE_bf16(R + d), with
    d = tol * max|R| of its group (the fp32 contract followed by one monotone rounding),
    and most elements equal RNE_bf16(R) exactly.  Returns the fraction not exactly equal."""
    Y = _ordered(np.asarray(Ybits, np.uint16))
    R = np.asarray(R, np.float32)
    if ranges is None:
        ranges = [(0, R.shape[0])]
    exact = np.zeros(R.shape, bool)
    for lo, hi in ranges:
        if hi <= lo:
            continue
        r = R[lo:hi]
        d = np.float32(tol) * np.abs(r).max()
        lo_b = _ordered(f32_to_bf16_bits((r.astype(np.float64) - d).astype(np.float32)))
        hi_b = _ordered(f32_to_bf16_bits((r.astype(np.float64) + d).astype(np.float32)))
        y = Y[lo:hi]
        assert ((y >= lo_b) & (y <= hi_b)).all(), "bf16 output outside the rounded tolerance band"
        exact[lo:hi] = y == _ordered(f32_to_bf16_bits(r))
    frac = float(1.0 - exact.mean())
    assert 1.0 - frac >= min_exact, f"only {1 - frac:.4f} of bf16 outputs equal RNE(oracle)"
    return frac


def group_row_ranges(group_sizes):
    off = np.concatenate([[0], np.cumsum(np.asarray(group_sizes, np.int64))])
    return [(int(off[g]), int(off[g + 1])) for g in range(len(off) - 1)]
