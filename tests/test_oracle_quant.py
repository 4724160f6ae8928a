"""Pins of the oracle's quantizers: hand-derived codes, closed forms and invariants."""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle.fp8 import bf16_bits_to_f32, decode_fp8
from oracle.quant import (
    dynamic_scale_from_amax,
    quantize_rhs_per_channel,
    quantize_rowblock,
    quantize_static,
    quantize_with_inv,
    static_inv,
    static_scale_from_bound,
)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32bits(x):
    return int(np.float32(x).view(np.uint32))


def nearest_f32(q: Fraction):
    """The float32 nearest to an exact rational (ties to even), found by bracketing."""
    c = np.float32(float(q))  # within one float32 ulp of q
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    best = min(cands, key=lambda v: (abs(Fraction(float(v)) - q), int(np.float32(v).view(np.uint32)) & 1))
    return np.float32(best)


def load_static_golden():
    rows, meta = [], {}
    with open(os.path.join(GOLDEN, "static_e4m3_s4over448.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            if parts[0] in ("s_bits", "inv_bits"):
                meta[parts[0]] = int(parts[1], 16)
            else:
                rows.append((int(parts[0], 16), int(parts[1], 16)))
    return meta, rows


def test_static_scale_and_inverse_hand_derived():
    meta, _ = load_static_golden()
    s = static_scale_from_bound(-4.0, 4.0, "e4m3")
    assert f32bits(s) == meta["s_bits"]
    assert f32bits(static_inv(s)) == meta["inv_bits"]
    # independent exact-rational check of both roundings
    assert s == nearest_f32(Fraction(4, 448))
    assert static_inv(s) == nearest_f32(1 / Fraction(float(s)))


def test_static_codes_hand_derived():
    meta, rows = load_static_golden()
    s = np.float32(np.uint32(meta["s_bits"]).view(np.float32))
    bits = np.array([[r[0] for r in rows]], np.uint16)
    codes, inv = quantize_static(bits, s, "e4m3")
    assert f32bits(inv) == meta["inv_bits"]
    assert codes[0].tolist() == [r[1] for r in rows]


def test_static_scale_validation():
    with pytest.raises(ValueError):
        static_scale_from_bound(-3.0, 4.0, "e4m3")  # asymmetric range
    with pytest.raises(ValueError):
        static_scale_from_bound(0.0, 0.0, "e4m3")
    for bad in (0.0, -1.0, np.inf, np.nan, 1e-40):  # 1e-40 is a float32 subnormal
        with pytest.raises(ValueError):
            static_inv(bad)


def test_dynamic_scale_closed_forms():
    s, inv = dynamic_scale_from_amax(np.float32([448.0, 0.0, 57344.0]), "e4m3")
    assert s[0] == 1.0 and inv[0] == 1.0
    assert s[1] == 0.0 and inv[1] == 0.0  # zero block -> zero inverse
    assert s[2] == 128.0 and inv[2] == 1.0 / 128
    s, inv = dynamic_scale_from_amax(np.float32([57344.0]), "e5m2")
    assert s[0] == 1.0 and inv[0] == 1.0
    s, inv = dynamic_scale_from_amax(np.float32([3.0]), "e4m3")
    assert s[0] == nearest_f32(Fraction(3, 448))
    assert inv[0] == nearest_f32(1 / Fraction(float(s[0])))
    # an underflowing block: 1/s overflows float32 -> inverse forced to zero
    s, inv = dynamic_scale_from_amax(np.float32([1e-38]), "e4m3")
    assert s[0] > 0 and inv[0] == 0.0


@pytest.mark.parametrize("fmt,qcode", [("e4m3", 0x7E), ("e5m2", 0x7B)])
def test_dynamic_scale_maps_block_max_to_qmax_for_every_bf16(fmt, qcode):
    # every positive finite bf16 abs-max: the block maximum lands on the largest code
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    amax = bf16_bits_to_f32(bits)
    s, inv = dynamic_scale_from_amax(amax, fmt)
    live = inv > 0
    assert live.mean() > 0.9
    # the public quantizer on one-element blocks holding the block maximum itself
    codes = quantize_with_inv(amax[live], inv[live], fmt)
    assert (codes == qcode).all()
    # dequantized block max within half a quantum of the true max
    deq = decode_fp8(np.full(live.sum(), qcode, np.uint8), fmt) * s[live]
    rel = np.abs(deq.astype(np.float64) - amax[live]) / amax[live]
    assert rel.max() < 2.0 ** -20
    # inverse is zero exactly for the under-flowing range
    dead = bits[~live]
    assert bf16_bits_to_f32(dead).max() < 2e-33


def test_static_equals_dynamic_when_block_max_is_the_bound():
    rng = np.random.default_rng(3)
    x = rng.uniform(-3.9, 3.9, (300, 64)).astype(np.float32)
    x[::128, 5] = 4.0  # every 128-row block reaches the bound exactly
    x[7, 9] = -4.0
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    s = static_scale_from_bound(-4.0, 4.0, "e4m3")
    cs, _ = quantize_static(bits, s, "e4m3")
    cd, sd, _ = quantize_rowblock(bits, "e4m3")
    assert (sd == s).all()
    assert (cs == cd).all()


def test_rowblock_geometry_brute_force():
    rng = np.random.default_rng(4)
    R, C = 300, 40  # 3 blocks, last one 44 rows
    x = (rng.standard_normal((R, C)) * np.exp(rng.uniform(-8, 8, (R, 1)))).astype(np.float32)
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    codes, s, inv = quantize_rowblock(bits, "e5m2")
    assert s.shape == (3,)
    xf = bf16_bits_to_f32(bits)
    for b, (lo, hi) in enumerate([(0, 128), (128, 256), (256, 300)]):
        amax = max(abs(float(v)) for v in xf[lo:hi].ravel())
        assert s[b] == nearest_f32(Fraction(amax) / 57344)
        # reconstruction within half a quantum (relative 2^-3) or the subnormal floor
        deq = torch.from_numpy(codes[lo:hi]).view(torch.float8_e5m2).to(torch.float64).numpy() * float(s[b])
        err = np.abs(deq - xf[lo:hi])
        assert (err <= np.maximum(np.abs(xf[lo:hi]) * 2.0 ** -3, float(s[b]) * 2.0 ** -17) * 1.0001).all()


@pytest.mark.parametrize("axis", ["n", "k"])
def test_rhs_per_channel_brute_force(axis):
    rng = np.random.default_rng(5)
    G, K, N = 3, 16, 24
    w = (rng.standard_normal((G, K, N)) * 0.02 * np.exp(rng.uniform(-3, 3, (G, 1, N)))).astype(np.float32)
    bits = torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    codes, s = quantize_rhs_per_channel(bits, "e4m3", axis)
    wf = bf16_bits_to_f32(bits)
    deq = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for g in range(G):
        for ch in range(N if axis == "n" else K):
            col = wf[g, :, ch] if axis == "n" else wf[g, ch, :]
            cc = deq[g, :, ch] if axis == "n" else deq[g, ch, :]
            sc = s[g, ch]
            amax = max(abs(float(v)) for v in col)
            assert sc == nearest_f32(Fraction(amax) / 448)
            assert abs(cc[np.argmax(np.abs(col))]) == 448.0  # channel max -> largest code
            err = np.abs(cc * float(sc) - col)
            assert (err <= np.maximum(np.abs(col) * 2.0 ** -4, float(sc) * 2.0 ** -10) * 1.0001).all()
