"""Pins of the block-wise-scale oracle: exact rationals on tiny inputs, the one-block
reduction to the per-channel forward, block-constant scales factoring out, and the
block abs-max of both quantizers by brute force."""

from fractions import Fraction

import numpy as np
import pytest

from oracle.blockwise import (gmm_dlhs_blockwise_ref, gmm_fwd_blockwise_ref, quantize_rhs_blockwise,
                              quantize_rhs_blockwise_dlhs, quantize_subchannel)
from oracle.fp8 import bf16_bits_to_f32
from oracle.gmm import gmm_dlhs_ref, gmm_fwd_ref
from oracle.quant import quantize_rhs_per_channel, quantize_with_inv
from tests.test_oracle_gmm import gamma, random_codes, random_scales, tdec


def bits(rng, shape, sigma):
    return (rng.normal(0, sigma, shape).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("bk", [4, 8])
def test_blockwise_forward_brute_force(bk):
    rng = np.random.default_rng(30)
    M, G, K, N = 7, 3, 16, 5
    gs = np.array([3, 0, 4], np.int32)
    aq = random_codes(rng, (M, K), "e4m3")
    bq = random_codes(rng, (G, K, N), "e4m3")
    sa = random_scales(rng, (M, K // bk))
    sb = random_scales(rng, (G, K // bk, N))
    R = gmm_fwd_blockwise_ref(aq, "e4m3", sa, bq, "e4m3", sb, gs, bk)
    A, B = tdec(aq, "e4m3"), tdec(bq, "e4m3")
    gid = np.repeat(np.arange(G), gs)
    for m in range(M):
        for n in range(N):
            g = gid[m]
            ex = Fraction(0)
            ab = Fraction(0)
            for kb in range(K // bk):
                sc = Fraction(float(sa[m, kb])) * Fraction(float(sb[g, kb, n]))
                terms = [Fraction(A[m, k]) * Fraction(B[g, k, n]) for k in range(kb * bk, (kb + 1) * bk)]
                ex += sum(terms) * sc
                ab += sum(abs(t) for t in terms) * sc
            err = abs(Fraction(float(R[m, n])) - ex)
            # each block: its float32 sum, two scale roundings, one float32 addition
            lim = ab * Fraction(1.01 * gamma(bk + 3 + K // bk)) + Fraction(2.0 ** -140)
            assert err <= lim, (m, n, float(err), float(lim))


def test_one_block_is_the_per_channel_forward():
    rng = np.random.default_rng(31)
    M, G, K, N = 300, 4, 256, 96
    gs = np.array([100, 0, 150, 50], np.int32)
    xb, wb = bits(rng, (M, K), 1.0), bits(rng, (G, K, N), 0.02)
    aq, sa = quantize_subchannel(xb, "e4m3", K)
    bq, sb = quantize_rhs_blockwise(wb, "e4m3", K)
    bq2, sb2 = quantize_rhs_per_channel(wb, "e4m3", "n")
    assert np.array_equal(bq, bq2) and np.array_equal(sb[:, 0, :], sb2)
    R = gmm_fwd_blockwise_ref(aq, "e4m3", sa, bq, "e4m3", sb, gs, K)
    R2 = gmm_fwd_ref(aq, "e4m3", sa[:, 0], bq2, "e4m3", sb2, gs)
    assert np.array_equal(R, R2)


def test_block_constant_scales_factor_out():
    # scales equal across blocks: the same sum up to the float32 rounding of the blocks
    rng = np.random.default_rng(32)
    M, G, K, N, bk = 64, 2, 512, 32, 128
    gs = np.array([40, 24], np.int32)
    aq = random_codes(rng, (M, K), "e4m3")
    bq = random_codes(rng, (G, K, N), "e4m3")
    ra = random_scales(rng, M)
    rb = random_scales(rng, (G, N))
    sa = np.repeat(ra[:, None], K // bk, axis=1)
    sb = np.repeat(rb[:, None, :], K // bk, axis=1)
    R = gmm_fwd_blockwise_ref(aq, "e4m3", sa, bq, "e4m3", sb, gs, bk).astype(np.float64)
    R1 = gmm_fwd_ref(aq, "e4m3", ra, bq, "e4m3", rb, gs).astype(np.float64)
    A, B = tdec(aq, "e4m3"), tdec(bq, "e4m3")
    gid = np.repeat(np.arange(G), gs)
    absum = np.stack([np.abs(A[m]) @ np.abs(B[gid[m]]) for m in range(M)]) * ra[:, None] * rb[gid]
    assert np.all(np.abs(R - R1) <= absum * 2 * gamma(K + 8))


@pytest.mark.parametrize("bk", [128, 256])
def test_quantizers_block_absmax_brute_force(bk):
    rng = np.random.default_rng(33)
    M, K, G, N = 40, 512, 2, 24
    xb = bits(rng, (M, K), 1.0)
    xb[3, :bk] = 0  # an all-zero block: scale 0, inverse 0, codes 0
    codes, s = quantize_subchannel(xb, "e4m3", bk)
    x = bf16_bits_to_f32(xb)
    for m in range(M):
        for kb in range(K // bk):
            blk = x[m, kb * bk:(kb + 1) * bk]
            amax = np.float32(np.abs(blk).max())
            assert s[m, kb] == np.float32(amax / np.float32(448.0))
            inv = np.float32(0) if s[m, kb] == 0 else np.float32(np.float32(1) / s[m, kb])
            want = quantize_with_inv(blk[None, :], np.array([inv], np.float32), "e4m3")[0]
            assert np.array_equal(codes[m, kb * bk:(kb + 1) * bk], want)
    assert s[3, 0] == 0 and not codes[3, :bk].any()
    wb = bits(rng, (G, K, N), 0.02)
    wq, ws = quantize_rhs_blockwise(wb, "e5m2", bk)
    w = bf16_bits_to_f32(wb)
    for g in range(G):
        for kb in range(K // bk):
            for n in range(N):
                amax = np.float32(np.abs(w[g, kb * bk:(kb + 1) * bk, n]).max())
                assert ws[g, kb, n] == np.float32(amax / np.float32(57344.0))
    # the largest element of every block maps to +-qmax
    assert np.all(np.isin((codes & 0x7F).reshape(M, K // bk, bk).max(axis=2), [0x7E, 0x00]))


def test_fold_by_unit_and_power_of_two_scales():
    """Folding scales of 1 is the plain dynamic quantization; folding 2^e multiplies exactly,
    so the codes stay and the block scales gain the factor 2^e exactly."""
    from oracle.blockwise import quantize_folded
    from oracle.quant import quantize_rowblock

    rng = np.random.default_rng(34)
    M, N, G = 300, 256, 3
    gs = np.array([100, 0, 200], np.int32)
    gb = bits(rng, (M, N), 1e-3)
    c1, s1 = quantize_folded(gb, np.ones((G, N), np.float32), gs, "e5m2")
    c0, s0, _ = quantize_rowblock(gb, "e5m2")
    assert np.array_equal(c1, c0) and np.array_equal(s1, s0)
    c2, s2 = quantize_folded(gb, np.full((G, N), 2.0 ** 7, np.float32), gs, "e5m2")
    assert np.array_equal(c2, c0) and np.array_equal(s2, s0 * np.float32(2.0 ** 7))


def test_folded_dlhs_matches_the_definition():
    """dlhs through the fold (one weight copy, per-n forward scales) against the float64
    sum_n grad[m, n] W[g, k, n] s[g, n], within the e5m2 and e4m3 rounding of the operands."""
    from oracle.blockwise import quantize_folded
    from oracle.gmm import gmm_dlhs_ref, row_scales

    rng = np.random.default_rng(35)
    M, N, K, G = 256, 512, 128, 2
    gs = np.array([150, 106], np.int32)
    gb = bits(rng, (M, N), 1e-3)
    wb = bits(rng, (G, K, N), 0.02)
    wq, ws = quantize_rhs_per_channel(wb, "e4m3", "n")  # the forward copy: s[g, n]
    codes, s = quantize_folded(gb, ws, gs, "e5m2")
    R = gmm_dlhs_ref(codes, "e5m2", row_scales(s, M), wq, "e4m3", np.ones((G, K), np.float32), gs)
    x = bf16_bits_to_f32(gb).astype(np.float64)
    W = tdec(wq, "e4m3") * ws[:, None, :].astype(np.float64)
    gid = np.repeat(np.arange(G), gs)
    exact = np.stack([W[gid[m]] @ x[m] for m in range(M)])
    absum = np.stack([np.abs(W[gid[m]]) @ np.abs(x[m]) for m in range(M)])
    # e5m2 relative rounding 2^-3 per gradient element (plus its subnormal floor)
    assert np.all(np.abs(R - exact) <= absum * 2.0 ** -3 + 1e-12)
    assert np.abs(R - exact).max() < 0.1 * np.abs(exact).max()


@pytest.mark.parametrize("bk", [4, 8])
def test_blockwise_dlhs_brute_force(bk):
    """dlhs[m, k] against exact rationals: the sum over n of grad[m, n] w[g, k, n], each
    block of bk columns n scaled by sG[m, nb] sW[g, k, nb]."""
    rng = np.random.default_rng(33)
    M, G, K, N = 7, 3, 5, 16
    gs = np.array([3, 0, 4], np.int32)
    gq = random_codes(rng, (M, N), "e5m2")
    wq = random_codes(rng, (G, K, N), "e4m3")
    sg = random_scales(rng, (M, N // bk))
    sw = random_scales(rng, (G, K, N // bk))
    R = gmm_dlhs_blockwise_ref(gq, "e5m2", sg, wq, "e4m3", sw, gs, bk)
    A, W = tdec(gq, "e5m2"), tdec(wq, "e4m3")
    gid = np.repeat(np.arange(G), gs)
    for m in range(M):
        for k in range(K):
            g = gid[m]
            ex = Fraction(0)
            ab = Fraction(0)
            for nb in range(N // bk):
                sc = Fraction(float(sg[m, nb])) * Fraction(float(sw[g, k, nb]))
                terms = [Fraction(A[m, n]) * Fraction(W[g, k, n]) for n in range(nb * bk, (nb + 1) * bk)]
                ex += sum(terms) * sc
                ab += sum(abs(t) for t in terms) * sc
            err = abs(Fraction(float(R[m, k])) - ex)
            lim = ab * Fraction(1.01 * gamma(bk + 3 + N // bk)) + Fraction(2.0 ** -140)
            assert err <= lim, (m, k, float(err), float(lim))


def test_one_block_dlhs_is_the_per_channel_dlhs():
    """With one block (bk = N) the weight's dlhs copy is the per-output-channel-k
    quantization and the block-wise dlhs is the per-channel dlhs, bit for bit."""
    rng = np.random.default_rng(34)
    M, G, K, N = 300, 4, 96, 256
    gs = np.array([100, 0, 150, 50], np.int32)
    gb, wb = bits(rng, (M, N), 1e-3), bits(rng, (G, K, N), 0.02)
    gq, sg = quantize_subchannel(gb, "e5m2", N)
    wq, sw = quantize_rhs_blockwise_dlhs(wb, "e4m3", N)
    wq2, sw2 = quantize_rhs_per_channel(wb, "e4m3", "k")
    assert np.array_equal(wq, wq2) and np.array_equal(sw[:, :, 0], sw2)
    R = gmm_dlhs_blockwise_ref(gq, "e5m2", sg, wq, "e4m3", sw, gs, N)
    R2 = gmm_dlhs_ref(gq, "e5m2", sg[:, 0], wq2, "e4m3", sw2, gs)
    assert np.array_equal(R, R2)
