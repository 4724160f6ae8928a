"""Pins of the oracle's FP8 / bf16 codecs against the format definitions and torch's casts."""

import numpy as np
import pytest
import torch

from oracle.fp8 import bf16_bits_to_f32, decode_fp8, encode_fp8, f32_to_bf16_bits

TORCH_DT = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
QMAX = {"e4m3": 448.0, "e5m2": 57344.0}


def torch_encode(y, fmt):
    """torch's CPU cast (round to nearest even) of already-clamped float32 values."""
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32))
    return t.to(TORCH_DT[fmt]).view(torch.uint8).numpy()


def torch_decode(codes, fmt):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(TORCH_DT[fmt]).to(torch.float32).numpy()


def finite_codes(fmt):
    c = np.arange(256, dtype=np.uint8)
    v = torch_decode(c, fmt)
    return c[np.isfinite(v)]


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_decode_matches_torch_all_codes(fmt):
    c = np.arange(256, dtype=np.uint8)
    ours, ref = decode_fp8(c, fmt), torch_decode(c, fmt)
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all(), c[~same]
    # the two extremes that pin the OCP flavour (an FNUZ e4m3 would top out at 240)
    assert decode_fp8(np.uint8(0x7E), "e4m3") == 448.0
    assert np.isnan(decode_fp8(np.uint8(0x7F), "e4m3"))
    assert decode_fp8(np.uint8(0x7B), "e5m2") == 57344.0
    assert decode_fp8(np.uint8(0x7C), "e5m2") == np.inf


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_round_trip_every_finite_code(fmt):
    c = finite_codes(fmt)
    assert (encode_fp8(decode_fp8(c, fmt), fmt) == c).all()


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_encode_matches_torch_at_every_midpoint(fmt):
    c = finite_codes(fmt)
    v = np.unique(decode_fp8(c, fmt).astype(np.float32))
    v = v[v >= 0]
    mids = ((v[:-1].astype(np.float64) + v[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (v[:-1].astype(np.float64) + v[1:]) / 2)  # exact
    probes = np.concatenate([
        v, mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0)),
        np.array([np.float32(v[1]) / 4, np.float32(v[1]) / 2 * np.float32(1.0000001)], np.float32),
    ]).astype(np.float32)
    probes = probes[np.abs(probes) <= QMAX[fmt]]
    probes = np.concatenate([probes, -probes])
    assert (encode_fp8(probes, fmt) == torch_encode(probes, fmt)).all()


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_encode_matches_torch_random_magnitudes(fmt):
    rng = np.random.default_rng(0)
    e = rng.uniform(-30, np.log2(QMAX[fmt]), 200000)
    y = (np.exp2(e) * rng.choice([-1.0, 1.0], e.size)).astype(np.float32)
    y = np.clip(y, -QMAX[fmt], QMAX[fmt]).astype(np.float32)
    assert (encode_fp8(y, fmt) == torch_encode(y, fmt)).all()


def test_format_table_constants():
    # OCP 8-bit float tables: extremes, smallest normals and subnormals, signed zero
    assert encode_fp8(np.float32(448.0), "e4m3") == 0x7E
    assert encode_fp8(np.float32(57344.0), "e5m2") == 0x7B
    assert encode_fp8(np.float32(2.0 ** -9), "e4m3") == 0x01
    assert encode_fp8(np.float32(2.0 ** -16), "e5m2") == 0x01
    assert encode_fp8(np.float32(2.0 ** -6), "e4m3") == 0x08
    assert encode_fp8(np.float32(2.0 ** -14), "e5m2") == 0x04
    assert encode_fp8(np.float32(-0.0), "e4m3") == 0x80
    assert encode_fp8(np.float32(-1e-30), "e5m2") == 0x80
    assert encode_fp8(np.float32(1.0), "e4m3") == 0x38
    assert encode_fp8(np.float32(1.0), "e5m2") == 0x3C
    # ties to even at half the smallest subnormal (-> 0) and at 1.5x it (-> 2 quanta)
    assert encode_fp8(np.float32(2.0 ** -10), "e4m3") == 0x00
    assert encode_fp8(np.float32(3 * 2.0 ** -10), "e4m3") == 0x02
    with pytest.raises(ValueError):
        encode_fp8(np.float32(449.0), "e4m3")


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    u = rng.integers(0, 2 ** 32, 500000, dtype=np.uint64).astype(np.uint32)
    # add exact ties and near-ties
    ties = (rng.integers(0, 2 ** 16, 20000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    u = np.concatenate([u, ties, ties + 1, ties - 1]).astype(np.uint32)
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (f32_to_bf16_bits(x) == ref).all()
    back = torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    assert (bf16_bits_to_f32(ref) == back).all()
