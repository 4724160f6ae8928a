"""SwiGLU of the merged gate|up projection, forward and backward (oracle; test
infrastructure).

"FP8 Megablox for batch split" (PR #3770), Description (2) merges the gate and up
projections W0 | W1 along N, so one grouped product yields x = [g | u] ([M, 2I]); the
feed-forward block then applies h = silu(g) * u before the down projection.  The
definitions, written out in float64 and rounded once to float32:

  silu(v)  = v / (1 + exp(-v)) = v * sigmoid(v)
  h        = silu(g) * u
  dL/dg    = dL/dh * u * sigmoid(g) * (1 + g * (1 - sigmoid(g)))     (d silu / dv)
  dL/du    = dL/dh * silu(g)

With h emitted as fp8 codes for the down projection (its lhs, quantized with a fixed
per-tensor scale as in "add static LHS scaling support for GMM v2 FWD", Description), the
codes are those of the static quantization O2/O3 applied to the float32 h:
code = encode(clip(RNE_f32(h * RNE_f32(1/s)), -qmax, qmax)).
With dynamic scales instead, h takes the sub-channel layout that the same page's review
thread on the lhs docstring names ([M, num_blocks] scales): per row and block of bk
channels, s = RNE(amax / qmax) over the block's float32 |h|, inverse 0 when s is 0 or
1/s overflows, and the codes as above with that block's inverse (the dynamic recipe O4
with the abs-max taken over the block).

Parity: pinned by closed forms (sigmoid(ln 3) = 3/4), the identity silu(v) - silu(-v) = v,
the large-|v| limits, and central finite differences of the forward for the backward;
the fp8 codes of h by a brute-force nearest search over all 256 codes, saturation and
signed zeros; the sub-channel codes by a hand-worked example, by agreement with the
static codes under each block's own scale, and by all-zero blocks
(``tests/test_oracle_swiglu.py``).
"""

import numpy as np

from .fp8 import encode_fp8
from .quant import dynamic_scale_from_amax, qmax_of, quantize_with_inv, static_inv


def silu(v):
    """v / (1 + exp(-v)) in float64 (exp(-v) overflowing to inf gives -0.0 / 0.0)."""
    v = np.asarray(v, np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def sigmoid(v):
    v = np.asarray(v, np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-v))


def swiglu_ref(x, I):
    """x [M, 2I] (the merged product, any float dtype) -> h [M, I] float32."""
    x = np.asarray(x, np.float64)
    g, u = x[:, :I], x[:, I:2 * I]
    return (silu(g) * u).astype(np.float32)


def swiglu_bwd_ref(dh, gu, I):
    """dh [M, I] and gu = [g | u] [M, 2I] (float values) -> d_gu [M, 2I] float32."""
    dh = np.asarray(dh, np.float64)
    gu = np.asarray(gu, np.float64)
    g, u = gu[:, :I], gu[:, I:2 * I]
    s = sigmoid(g)
    dg = dh * u * s * (1.0 + g * (1.0 - s))
    du = dh * g * s
    return np.concatenate([dg, du], axis=1).astype(np.float32)


def swiglu_fp8_ref(x, I, s, fmt):
    """x [M, 2I] (the merged product) -> (codes uint8 [M, I], h float32 [M, I]): h as in
    swiglu_ref, then its static fp8 quantization under the per-tensor scale s."""
    h = swiglu_ref(x, I)
    inv = static_inv(s)
    return quantize_with_inv(h, np.full(h.shape[0], inv, np.float32), fmt), h


def swiglu_fp8_subchannel_ref(x, I, fmt, bk=128):
    """x [M, 2I] (the merged product) -> (codes uint8 [M, I], scales float32 [M, I/bk],
    h float32 [M, I]): h as in swiglu_ref, then one dynamic scale per row and block of bk
    channels of the float32 h."""
    h = swiglu_ref(x, I)
    M = h.shape[0]
    assert I % bk == 0
    amax = np.abs(h).reshape(M, I // bk, bk).max(axis=2).astype(np.float32)
    s, inv = dynamic_scale_from_amax(amax, fmt)
    y = (h * np.repeat(inv, bk, axis=1)).astype(np.float32)
    q = qmax_of(fmt)
    codes = encode_fp8(np.minimum(np.maximum(y, -q), q), fmt)
    return codes, s.astype(np.float32), h
