"""FP8 and bfloat16 codecs, written from the format definitions (oracle; test infrastructure).

The pages name the formats only as e4m3 / e5m2 fp8 recipes ("FP8 Megablox for batch
split", Description (1)).  The reading taken here is the OCP 8-bit floating-point
formats, because the static scale of the tiny workload (4.0/448) presupposes a largest
finite e4m3 value of 448:

  E4M3FN  sign | 4 exponent bits (bias 7)  | 3 mantissa bits; largest finite 448,
          smallest subnormal 2^-9, no infinities, NaN = S.1111.111.
  E5M2    sign | 5 exponent bits (bias 15) | 2 mantissa bits; largest finite 57344,
          smallest subnormal 2^-16, infinities S.11111.00, NaN S.11111.{01,10,11}.

``encode_fp8`` takes already-clamped finite float32 values and rounds to nearest,
ties to even, with gradual underflow and the sign of zero kept.  Every operation
below is exact in float64 (power-of-two scalings of float32 values), so the only
rounding is the single explicit round-half-even step.

bfloat16 is the upper half of a float32; ``f32_to_bf16_bits`` rounds to nearest even.
"""

import numpy as np

# name -> (exponent bits, mantissa bits, bias, largest finite value, has infinities)
FORMATS = {
    "e4m3": dict(ebits=4, mbits=3, bias=7, qmax=448.0, has_inf=False),
    "e5m2": dict(ebits=5, mbits=2, bias=15, qmax=57344.0, has_inf=True),
}


def _fmt(fmt):
    if fmt not in FORMATS:
        raise ValueError(f"unknown fp8 format {fmt!r}")
    return FORMATS[fmt]


def encode_fp8(y, fmt):
    """float32 array (finite, |y| <= qmax) -> uint8 codes, round-to-nearest-even.

    Parity: pinned (round trip over every code; equality with torch's CPU float8
    cast at every rounding midpoint and its float32 neighbours; hand-derived codes).
    """
    f = _fmt(fmt)
    mbits, bias = f["mbits"], f["bias"]
    y = np.asarray(y, dtype=np.float32)
    if not np.all(np.isfinite(y)):
        raise ValueError("encode_fp8 expects finite inputs")
    if np.any(np.abs(y) > f["qmax"]):
        raise ValueError("encode_fp8 expects inputs already clamped to +-qmax")
    sign = np.signbit(y).astype(np.uint16) << 7
    a = np.abs(y.astype(np.float64))
    emin = 1 - bias  # exponent of the smallest normal number
    # floor(log2(a)) from the exact binary exponent; a == 0 is handled by r == 0 below.
    _, e2 = np.frexp(a)
    e = np.maximum(e2.astype(np.int64) - 1, emin)
    quantum = np.ldexp(1.0, e - mbits)  # spacing of representable values around a
    r = np.rint(a / quantum)  # exact quotient, then round half to even
    # A carry out of the mantissa moves the value to the next binade.
    carry = r >= (1 << (mbits + 1))
    e = np.where(carry, e + 1, e)
    r = np.where(carry, r / 2, r)
    normal = r >= (1 << mbits)
    exp_field = np.where(normal, e + bias, 0).astype(np.uint16)
    man = np.where(normal, r - (1 << mbits), r).astype(np.uint16)
    code = sign | (exp_field << mbits) | man
    return code.astype(np.uint8)


def decode_fp8(code, fmt):
    """uint8 codes -> float32 values (exact).  NaN codes give NaN, e5m2 inf codes give inf.

    Parity: pinned (equality with torch's CPU float8 -> float32 conversion for all 256
    codes; the OCP extremes 448 / 57344 and smallest subnormals 2^-9 / 2^-16).
    """
    f = _fmt(fmt)
    mbits, bias, ebits = f["mbits"], f["bias"], f["ebits"]
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp_field = (c >> mbits) & ((1 << ebits) - 1)
    man = c & ((1 << mbits) - 1)
    emin = 1 - bias
    sub = np.ldexp(man.astype(np.float64), emin - mbits)
    nrm = np.ldexp((man + (1 << mbits)).astype(np.float64), exp_field - bias - mbits)
    val = sign * np.where(exp_field == 0, sub, nrm)
    top = exp_field == (1 << ebits) - 1
    if f["has_inf"]:
        val = np.where(top & (man == 0), sign * np.inf, val)
        val = np.where(top & (man != 0), np.nan, val)
    else:
        val = np.where(top & (man == (1 << mbits) - 1), np.nan, val)
    return val.astype(np.float32)


def bf16_bits_to_f32(bits):
    """uint16 bfloat16 bit patterns -> float32 (exact: the bits are the upper half)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def f32_to_bf16_bits(x):
    """float32 -> uint16 bfloat16 bits, round to nearest, ties to even.  NaN stays NaN.

    Parity: pinned (equality with torch's CPU .to(torch.bfloat16)).
    """
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    hi = u >> 16
    lo = u & 0xFFFF
    up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & 1) == 1))
    r = (hi + up.astype(np.uint64)) & 0xFFFF
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    r = np.where(nan, (hi | 0x40) & 0xFFFF, r)
    return r.astype(np.uint16)


def bf16_round(x):
    """float32 -> float32 holding the nearest-even bfloat16 value."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))
