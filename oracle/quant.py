"""Quantizers of the FP8 grouped matmul (oracle; test infrastructure).

What is computed, and where the pages fix it:

* Static per-tensor symmetric lhs scaling ("add static LHS scaling support for GMM v2
  FWD", PR #4735, Description and the review thread on the lhs docstring): the lhs
  arrives unquantized, the kernel forms clip(lhs / scale) in fp8 and the product is
  multiplied back by the scale.  The scale is a per-tensor [1,1] value extracted from
  a fixed calibration range; only symmetric ranges (min == -max) are accepted.
* Dynamic per-block abs-max lhs scaling (same page, review thread on
  ``block_scale_inv``): the inverse scale is zero where the block scale is zero, and
  the block is multiplied by the inverse scale before the cast to fp8.
* Pre-quantized weights with per-channel scales ("FP8 Megablox for batch split",
  PR #3770, Description (1); "Support quantization for tokamax gmm v2", PR #4451,
  review thread on per-channel scales).

Readings where the pages leave a step open (each is also listed in the design notes):

* Division by the scale is carried out as a multiplication by the float32 inverse
  RNE(1/s), for static and dynamic alike, so both recipes share one formula.
* The value is clamped to +-qmax in float32 *before* rounding to fp8 (the "clip").
* The dynamic scale is s = RNE_f32(amax / qmax); the inverse is 0 when s == 0 and
  also when 1/s overflows float32 (an under-flowing block, which would otherwise
  give 0 * inf = NaN).
* A dynamic block is 128 consecutive rows by the full row width, aligned to row 0 of
  the tensor, independent of the expert grouping.
"""

import numpy as np

from .fp8 import FORMATS, bf16_bits_to_f32, encode_fp8

_F32_MIN_NORMAL = np.float32(np.finfo(np.float32).tiny)


def qmax_of(fmt):
    return np.float32(FORMATS[fmt]["qmax"])


def static_scale_from_bound(lo, hi, fmt):
    """Per-tensor scale from a fixed symmetric calibration range [lo, hi] = [-b, b].

    s = RNE_f32(b / qmax).  An asymmetric range is rejected, as the pages reject
    min != -max for the in-kernel static scale (PR #4735 review thread).
    Parity: pinned (closed form: bound 4 with e4m3 gives fp32(4/448)).
    """
    lo, hi = np.float32(lo), np.float32(hi)
    if not (np.isfinite(lo) and np.isfinite(hi)) or lo != -hi or hi <= 0:
        raise ValueError("static scale needs a finite symmetric range with min == -max > 0")
    return np.float32(hi / qmax_of(fmt))


def static_inv(s):
    """float32 inverse of a validated static scale: RNE_f32(1/s).

    The scale must be finite, positive and normal (the pages guard against
    underflow and scales close to zero, PR #4735 review summary).
    Parity: pinned (closed form at s = fp32(4/448)).
    """
    s = np.float32(s)
    if not np.isfinite(s) or s < _F32_MIN_NORMAL:
        raise ValueError("static scale must be finite, positive and a normal float32")
    return np.float32(np.float32(1.0) / s)


def dynamic_scale_from_amax(amax, fmt):
    """(s, inv) for abs-max values: s = RNE(amax/qmax); inv = 0 if s == 0 or 1/s overflows.

    Parity: pinned (closed forms; exhaustive invariant amax*inv within clamp range).
    """
    amax = np.asarray(amax, dtype=np.float32)
    with np.errstate(divide="ignore", over="ignore"):
        s = (amax / qmax_of(fmt)).astype(np.float32)
        inv = (np.float32(1.0) / s).astype(np.float32)
    inv = np.where((s == 0) | ~np.isfinite(inv), np.float32(0.0), inv).astype(np.float32)
    return s, inv


def quantize_with_inv(x_f32, inv_per_row, fmt):
    """codes[r, c] = encode(clip(RNE_f32(x[r, c] * inv[r]), -qmax, qmax)).

    Parity: pinned (via encode_fp8's pins and the hand-derived static examples).
    """
    x = np.asarray(x_f32, dtype=np.float32)
    inv = np.asarray(inv_per_row, dtype=np.float32).reshape(-1, *([1] * (x.ndim - 1)))
    y = (x * inv).astype(np.float32)
    q = qmax_of(fmt)
    y = np.minimum(np.maximum(y, -q), q)
    return encode_fp8(y, fmt)


def quantize_static(x_bits, s, fmt):
    """bf16 bits [R, C] with a per-tensor scale -> (codes [R, C], inv)."""
    inv = static_inv(s)
    x = bf16_bits_to_f32(x_bits)
    return quantize_with_inv(x, np.full(x.shape[0], inv, np.float32), fmt), inv


def block_amax(x_bits, block_rows=128):
    """Abs-max of each block of ``block_rows`` rows (all columns); the last block may be short."""
    x = np.abs(bf16_bits_to_f32(x_bits))
    R = x.shape[0]
    nb = -(-R // block_rows)
    amax = np.zeros(nb, np.float32)
    for b in range(nb):
        blk = x[b * block_rows:(b + 1) * block_rows]
        amax[b] = blk.max() if blk.size else np.float32(0.0)
    return amax


def quantize_rowblock(x_bits, fmt, block_rows=128):
    """Dynamic per-block quantization of bf16 bits [R, C].

    Returns (codes [R, C], scales [nb], inv [nb]), nb = ceil(R / block_rows).
    Parity: pinned (codes through encode_fp8; scales through the closed forms and the
    static/dynamic equivalence when the block abs-max equals the static bound).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    amax = block_amax(x_bits, block_rows)
    s, inv = dynamic_scale_from_amax(amax, fmt)
    R = x_bits.shape[0]
    row_inv = np.repeat(inv, block_rows)[:R]
    codes = quantize_with_inv(bf16_bits_to_f32(x_bits), row_inv, fmt)
    return codes, s, inv


def quantize_rhs_per_channel(w_bits, fmt, channel_axis):
    """Per-channel weight quantization of bf16 bits [G, K, N].

    channel_axis == "n": one scale per (g, n), abs-max over k -> scales [G, N]
        (the output channels of the forward product).
    channel_axis == "k": one scale per (g, k), abs-max over n -> scales [G, K]
        (the output channels of the dlhs product, which contracts over n).
    Codes keep the [G, K, N] layout.  Parity: pinned (brute-force per channel).
    """
    w = bf16_bits_to_f32(np.asarray(w_bits, dtype=np.uint16))
    red = 1 if channel_axis == "n" else 2 if channel_axis == "k" else None
    if red is None:
        raise ValueError("channel_axis must be 'n' or 'k'")
    amax = np.abs(w).max(axis=red)
    s, inv = dynamic_scale_from_amax(amax, fmt)
    inv_b = inv[:, None, :] if red == 1 else inv[:, :, None]
    y = (w * inv_b).astype(np.float32)
    q = qmax_of(fmt)
    y = np.minimum(np.maximum(y, -q), q)
    return encode_fp8(y, fmt), s.astype(np.float32)
