"""Parity metrics between the HIP library's outputs and the oracle's.

Floating-point outputs (the reading of "max relative error 1e-3 after identical
quantization"): per group, max |Y - R| / max |R| <= tol, where R is the oracle's
fp32-accumulated result and Y the library's f32 output.  A group whose reference is
all zero must be exactly zero.  Beside that metric, f32 outputs are also held element
by element to an error bound of their sums (assert_rounding_bound): the fp32 roundings of
both sides plus the truncation that gfx950's FP8 matrix instructions apply inside each
instruction (measured, see MFMA_TRUNC), which a wrong term in a single output would
break unless it is smaller than that bound.
bf16 outputs cannot meet 1e-3 against an fp32 reference (half a bf16 ulp is up to 2^-8
relative), so for them (assert_bf16_close) every element must lie between
RNE_bf16(R - d) and RNE_bf16(R + d), d = tol * max|R| of its group, and at least 95% of
the elements must equal RNE_bf16(R) exactly.
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


U = 2.0 ** -24  # unit roundoff of float32
# gfx950's FP8 MFMA does not add its 64 products in fp32: it sums each aligned group of 8
# contraction elements after truncating every product toward zero 13 bits below the
# group's largest product (tests/test_gpu_mfma_accumulation.py pins this with designed
# inputs).  The other 7 products of a group then lose less than 2^-13 of the largest
# each, so an instruction's sum is off by less than 7 * 2^-13 * sum |a||b| over its terms.
MFMA_TRUNC = 7.0 * 2.0 ** -13


def magnitudes(codes):
    """fp8 codes of |value|: the sign bit cleared (finite codes stay finite)."""
    return np.asarray(codes, np.uint8) & np.uint8(0x7F)


def assert_rounding_bound(Y, R, absR, n_terms):
    """f32 outputs, element by element:
    |Y - R| <= (MFMA_TRUNC + 2 (n + 8) u) absR + 4 u |R| + 2^-126.

    absR holds the same product computed on the codes' magnitudes (sum |a| |b| times the
    positive scales); n_terms is the contraction length (broadcast against Y: for tgmm the
    rows of each group).  Y and R sum the same exact products in two fp32 orders (the
    oracle's sequential sum; the MFMA's 64-term instructions, the rescaling between tgmm's
    row blocks), each within (n + 8) u absR of the exact sum, Y's instructions add their
    truncation (MFMA_TRUNC absR at most), and both round the scale products of the
    epilogue twice; 2^-126 absorbs subnormal results."""
    Y = np.asarray(Y, np.float64)
    R = np.asarray(R, np.float64)
    A = np.asarray(absR, np.float64)
    n = np.asarray(n_terms, np.float64)
    bound = (MFMA_TRUNC + 2.0 * (n + 8.0) * U) * A + 4.0 * U * np.abs(R) + 2.0 ** -126
    excess = np.abs(Y - R) - bound
    bad = excess > 0
    assert not bad.any(), (f"{int(bad.sum())} of {bad.size} outputs outside their rounding "
                           f"bound (worst excess {float(excess.max()):.3e})")


def group_row_ranges(group_sizes):
    off = np.concatenate([[0], np.cumsum(np.asarray(group_sizes, np.int64))])
    return [(int(off[g]), int(off[g + 1])) for g in range(len(off) - 1)]


def fp8_order(codes):
    """fp8 codes -> integers in value order (sign-magnitude; +0 and -0 both map to 0)."""
    c = np.asarray(codes).astype(np.int64)
    return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)


def swiglu_h_bound(R, absR, K, I, mfma=True):
    """(h, dh): the float64 SwiGLU of the oracle's fp32 products R [M, 2I] and a bound on
    how far a correct evaluation of it can lie from h.  absR holds sum |a||b| s_A s_B
    of every product (the oracle's product of the codes' magnitudes).  Each product may
    differ from R by the rounding of two fp32 sums of K terms (the oracle's in its order,
    the library's in MFMA blocks of 64: at most K + 7 K / 64 roundings), the truncation
    inside the MFMA instructions (MFMA_TRUNC, when the products come from them) and the
    two scale multiplies; silu is 1.1-Lipschitz; the fp32 evaluation of silu(g) * u adds a
    few ulp."""
    from oracle.swiglu import silu

    R = np.asarray(R, np.float64)
    absR = np.asarray(absR, np.float64)
    gamma = (K + 7 * K / 64 + 4) * 2.0 ** -24 + (MFMA_TRUNC if mfma else 0.0)
    g, u = R[:, :I], R[:, I:2 * I]
    dg, du = gamma * absR[:, :I], gamma * absR[:, I:2 * I]
    h = silu(g) * u
    dh = 1.1 * dg * (np.abs(u) + du) + np.abs(silu(g)) * du + 8 * 2.0 ** -24 * np.abs(h)
    return h, dh


def assert_fp8_codes_in_band(codes, h, dh, s, fmt, ref_codes, min_exact=0.95):
    """Every code lies between the codes of (h - dh) / s and (h + dh) / s (quantized as the
    oracle does, widened by an fp32 rounding), and most equal the oracle's codes.  s is
    one scale or one per element (a zero scale quantizes with inverse 0).  Returns
    (fraction not equal to ref_codes, fraction of elements whose band spans two codes)."""
    from oracle.fp8 import encode_fp8
    from oracle.quant import qmax_of

    s32 = np.asarray(s, np.float32)
    with np.errstate(divide="ignore"):
        inv = np.where(s32 == 0, 0.0, (np.float32(1.0) / s32).astype(np.float64))
    q = qmax_of(fmt)

    def code_of(y):
        y = np.clip(y, -q, q).astype(np.float32)
        return fp8_order(encode_fp8(y, fmt))

    lo = (h - dh) * inv
    hi = (h + dh) * inv
    lo_c = code_of(lo - 2.0 ** -22 * np.abs(lo))
    hi_c = code_of(hi + 2.0 ** -22 * np.abs(hi))
    c = fp8_order(codes)
    bad = (c < lo_c) | (c > hi_c)
    assert not bad.any(), f"{int(bad.sum())} fp8 codes outside their rounding band"
    exact = float(np.mean(c == fp8_order(ref_codes)))
    assert exact >= min_exact, f"only {exact:.4f} of the codes equal the oracle's"
    return 1.0 - exact, float(np.mean(lo_c != hi_c))
