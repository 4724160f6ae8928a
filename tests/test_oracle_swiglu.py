"""Pins of the SwiGLU oracle against closed forms, identities and finite differences."""

import math

import numpy as np
import pytest

from oracle.swiglu import (silu, swiglu_bwd_ref, swiglu_fp8_ref, swiglu_fp8_subchannel_ref,
                           swiglu_ref)


def test_silu_closed_forms_and_limits():
    assert silu(0.0) == 0.0
    # sigmoid(ln 3) = 1 / (1 + 1/3) = 3/4
    assert abs(silu(math.log(3.0)) - 0.75 * math.log(3.0)) < 1e-15
    # sigmoid(-ln 3) = 1/4
    assert abs(silu(-math.log(3.0)) + 0.25 * math.log(3.0)) < 1e-15
    assert silu(60.0) == 60.0 * (1.0 / (1.0 + math.exp(-60.0)))
    assert abs(silu(60.0) - 60.0) < 1e-20
    assert 0.0 > silu(-60.0) > -1e-24
    assert silu(-1000.0) == 0.0  # exp overflows to inf: -1000 / inf


def test_silu_odd_part_identity():
    # silu(v) - silu(-v) = v (sigmoid(v) + sigmoid(-v) = 1)
    v = np.random.default_rng(1).normal(0.0, 4.0, 10000)
    assert np.max(np.abs(silu(v) - silu(-v) - v) / np.maximum(np.abs(v), 1e-300)) < 1e-14


def test_swiglu_at_closed_form_points():
    g = np.array([[0.0, math.log(3.0), -math.log(3.0), 50.0]])
    u = np.array([[7.0, 2.0, 4.0, -0.5]])
    h = swiglu_ref(np.concatenate([g, u], axis=1), 4)
    want = np.array([[0.0, 1.5 * math.log(3.0), -math.log(3.0), -25.0]], np.float32)
    assert np.array_equal(h, want)


def test_backward_is_the_derivative_of_the_forward():
    # central differences of h = silu(g) u in float64, against dL/dg and dL/du with dh
    rng = np.random.default_rng(2)
    M, I = 64, 32
    g = rng.normal(0.0, 3.0, (M, I))
    u = rng.normal(0.0, 1.0, (M, I))
    dh = rng.normal(0.0, 1.0, (M, I))
    eps = 1e-6
    num_dg = dh * (silu(g + eps) * u - silu(g - eps) * u) / (2 * eps)
    num_du = dh * (silu(g) * (u + eps) - silu(g) * (u - eps)) / (2 * eps)
    d = swiglu_bwd_ref(dh, np.concatenate([g, u], axis=1), I).astype(np.float64)
    scale = np.max(np.abs(num_dg))
    assert np.max(np.abs(d[:, :I] - num_dg)) < 1e-6 * scale
    assert np.max(np.abs(d[:, I:] - num_du)) < 1e-6 * np.max(np.abs(num_du))


def test_backward_at_a_closed_form_point():
    # g = ln 3: sigmoid = 3/4, d silu/dg = 3/4 (1 + ln3 / 4)
    l3 = math.log(3.0)
    d = swiglu_bwd_ref(np.array([[2.0]]), np.array([[l3, 5.0]]), 1)
    assert abs(d[0, 0] - np.float32(2.0 * 5.0 * 0.75 * (1 + l3 / 4))) <= 1e-6 * abs(d[0, 0])
    assert abs(d[0, 1] - np.float32(2.0 * 0.75 * l3)) <= 1e-6 * abs(d[0, 1])


def _nearest_code(y, fmt):
    """Brute force: the finite code nearest to y, ties to the even code (mantissa LSB 0)."""
    from oracle.fp8 import decode_fp8

    codes = np.arange(256, dtype=np.uint8)
    vals = decode_fp8(codes, fmt).astype(np.float64)
    ok = np.isfinite(vals)
    codes, vals = codes[ok], vals[ok]
    out = np.empty(y.shape, np.uint8)
    for i, v in np.ndenumerate(y):
        d = np.abs(vals - v)
        best = codes[d == d.min()]
        if len(best) > 1:  # a tie (or +0 / -0): the even code, keeping the sign of v
            best = best[(best & 1) == 0]
            if len(best) > 1:
                best = best[(best >= 0x80) == bool(np.signbit(v))]
        out[i] = best[0]
    return out


@pytest.mark.parametrize("fmt,qmax", [("e4m3", 448.0), ("e5m2", 57344.0)])
def test_swiglu_fp8_codes_are_the_nearest_fp8_of_h_over_s(fmt, qmax):
    rng = np.random.default_rng(7)
    M, I = 24, 16
    x = rng.normal(0.0, 2.0, (M, 2 * I)).astype(np.float32)
    x[0, :4] = [0.0, -0.0, -30.0, 80.0]  # h = 0, -0 * u, a tiny negative, a large value
    s = np.float32(0.01)
    codes, h = swiglu_fp8_ref(x, I, s, fmt)
    assert np.array_equal(h, swiglu_ref(x, I))
    inv = np.float64(np.float32(1.0) / s)
    # RNE_f32 of the exact product of two float32 values, then the clip to +-qmax
    y = np.clip((h.astype(np.float64) * inv).astype(np.float32).astype(np.float64), -qmax, qmax)
    assert np.array_equal(codes, _nearest_code(y, fmt))
    # saturation: a scale that puts every |h| above qmax gives only the two extreme codes
    big, _ = swiglu_fp8_ref(np.full((2, 2 * I), 5.0, np.float32), I, 1e-6, fmt)
    assert np.all(big == (0x7E if fmt == "e4m3" else 0x7B))
    neg = np.concatenate([np.full((2, I), 5.0), np.full((2, I), -5.0)], axis=1)
    small, _ = swiglu_fp8_ref(neg.astype(np.float32), I, 1e-6, fmt)
    assert np.all(small == (0xFE if fmt == "e4m3" else 0xFB))
    # signed zero: silu(-200) * 1 underflows to -0.0 and stays -0
    z, hz = swiglu_fp8_ref(np.array([[-200.0, 1.0]], np.float32), 1, 1.0, fmt)
    assert hz[0, 0] == 0 and np.signbit(hz[0, 0]) and z[0, 0] == 0x80


def test_fp8_band_check_accepts_the_oracle_and_catches_a_one_step_error():
    """The GPU test's band for h's codes: the oracle's own codes pass, the band (a worst-case
    bound on the fp32 sums; without the MFMA truncation term, since both sides here are
    fp32 evaluations) spans two codes for a minority of elements, and a code moved by one
    step where the band holds one code fails."""
    from oracle.gmm import gmm_fwd_ref
    from oracle.quant import quantize_rhs_per_channel, quantize_rowblock
    from tests.parity import assert_fp8_codes_in_band, fp8_order, swiglu_h_bound

    rng = np.random.default_rng(11)
    sizes = [70, 0, 186]
    M, K, I = sum(sizes), 256, 64
    xb = (rng.normal(0, 1, (M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    wb = (rng.normal(0, 0.02, (3, K, 2 * I)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    a, sa, _ = quantize_rowblock(xb, "e4m3")
    b, sb = quantize_rhs_per_channel(wb, "e4m3", "n")
    rs = np.repeat(sa, 128)[:M]
    R = gmm_fwd_ref(a, "e4m3", rs, b, "e4m3", sb, sizes)
    absR = gmm_fwd_ref(a & 0x7F, "e4m3", rs, b & 0x7F, "e4m3", sb, sizes)
    s = np.float32(np.abs(swiglu_ref(R, I)).max() / 448.0)
    codes, _ = swiglu_fp8_ref(R, I, s, "e4m3")
    h, dh = swiglu_h_bound(R, absR, K, I, mfma=False)
    diff, amb = assert_fp8_codes_in_band(codes, h, dh, s, "e4m3", codes, min_exact=1.0)
    assert diff == 0 and amb < 0.1
    # one code moved one step further from zero, at 50 elements in turn: most are caught
    cand = np.flatnonzero((np.abs(fp8_order(codes)) > 8) & (np.abs(fp8_order(codes)) < 100))
    caught = 0
    for i in cand[:50]:
        bad = codes.copy()
        bad.flat[i] = codes.flat[i] + 1
        try:
            assert_fp8_codes_in_band(bad, h, dh, s, "e4m3", codes, min_exact=0.0)
        except AssertionError:
            caught += 1
    assert caught >= 40, caught


def test_subchannel_codes_hand_worked():
    """g = 20 makes silu(g) round to 20.0 in float32, so h = 20 u exactly for these u: the
    first block of row 0 holds 20, 10, -5 and zeros, its scale is RNE(20 / 448) and its
    codes are e4m3 448, 224 and -112; the second block is all zero: scale 0, codes 0."""
    I, bk = 256, 128
    x = np.zeros((2, 2 * I), np.float32)
    x[0, :I] = 20.0
    x[0, I:I + 3] = [1.0, 0.5, -0.25]
    x[1, :I] = np.linspace(-3.0, 3.0, I)
    x[1, I:] = np.linspace(1.0, -2.0, I)
    codes, scales, h = swiglu_fp8_subchannel_ref(x, I, "e4m3", bk)
    assert scales.shape == (2, 2) and scales.dtype == np.float32
    assert h[0, 0] == 20.0 and h[0, 1] == 10.0 and h[0, 2] == -5.0
    assert scales[0, 0] == np.float32(0.044642857142857144)  # 20 / 448 rounded to float32
    assert list(codes[0, :4]) == [0x7E, 0x76, 0xEE, 0x00]
    assert np.all(codes[0, 4:bk] == 0)
    assert scales[0, 1] == 0.0 and np.all(codes[0, bk:] == 0)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_subchannel_codes_are_the_static_codes_of_each_block(fmt):
    """Each (row, block) of the dynamic sub-channel recipe equals the static recipe (pinned
    above by a brute-force nearest-code search) applied to that block with its own scale,
    and that scale is the block's largest |h| over qmax, rounded to float32."""
    rng = np.random.default_rng(21)
    M, I, bk = 6, 384, 128
    x = rng.normal(0.0, 2.0, (M, 2 * I)).astype(np.float32)
    x[2, :bk] = 0.0  # a block of h = 0: scale 0
    codes, scales, h = swiglu_fp8_subchannel_ref(x, I, fmt, bk)
    qmax = 448.0 if fmt == "e4m3" else 57344.0
    for r in range(M):
        for b in range(I // bk):
            cols = slice(b * bk, (b + 1) * bk)
            amax = np.float32(np.abs(swiglu_ref(x[r:r + 1], I)[0, cols]).max())
            assert scales[r, b] == np.float32(amax / np.float32(qmax))
            if scales[r, b] == 0:
                assert np.all(codes[r, cols] == 0) or np.all((codes[r, cols] & 0x7F) == 0)
                continue
            xb = np.concatenate([x[r:r + 1, :I][:, cols], x[r:r + 1, I:][:, cols]], axis=1)
            ref, _ = swiglu_fp8_ref(xb, bk, scales[r, b], fmt)
            assert np.array_equal(codes[r, cols], ref[0])
