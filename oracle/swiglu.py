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

Parity: pinned by closed forms (sigmoid(ln 3) = 3/4), the identity silu(v) - silu(-v) = v,
the large-|v| limits, and central finite differences of the forward for the backward;
the fp8 codes of h by a brute-force nearest search over all 256 codes, saturation and
signed zeros (``tests/test_oracle_swiglu.py``).
"""

import numpy as np

from .quant import quantize_with_inv, static_inv


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
