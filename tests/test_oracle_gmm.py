"""Pins of the oracle's grouped products: exact-rational brute force and invariants.

Decoding here goes through torch's float8 dtypes (a library routine independent of the
oracle's codec), and the reference sums are exact rationals or float64.
"""

import itertools
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle.ops as ops
from oracle.gmm import gmm_dlhs_ref, gmm_fwd_ref, group_offsets, row_scales, tgmm_ref
from oracle.quant import quantize_rhs_per_channel, static_scale_from_bound
from synth.workloads import bf16_to_bits, normal_bf16

TORCH_DT = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
U = 2.0 ** -24


def tdec(codes, fmt):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(TORCH_DT[fmt]).to(torch.float64).numpy()


def gamma(n):
    return n * U / (1 - n * U)


def random_codes(rng, shape, fmt):
    """Uniform over the finite codes of the format (both signs, subnormals included)."""
    c = np.arange(256, dtype=np.uint8)
    fin = c[np.isfinite(tdec(c, fmt))]
    return rng.choice(fin, size=shape).astype(np.uint8)


def random_scales(rng, shape):
    return np.exp2(rng.uniform(-12, 2, shape)).astype(np.float32)


def compositions(M, G):
    for cuts in itertools.combinations(range(M + G - 1), G - 1):
        prev, sizes = -1, []
        for c in cuts + (M + G - 1,):
            sizes.append(c - prev - 1)
            prev = c
        yield np.array(sizes, np.int32)


def check_bound(R, exact, absum, extra_rel=3 * U):
    """|R - exact| <= gamma-style bound; exact/absum are Fraction arrays (object dtype)."""
    for r, e, a in zip(np.ravel(R), np.ravel(exact), np.ravel(absum)):
        err = abs(Fraction(float(r)) - e)
        lim = a * Fraction(1.01 * gamma(64)) + abs(e) * Fraction(extra_rel) + Fraction(2.0 ** -140)
        assert err <= lim, (float(r), float(e), float(err), float(lim))


def brute_fwd(aq, afmt, sa_row, bq, bfmt, sb, gs, transpose_b=False):
    """Exact rationals: out[m, n] = s_a[m] s_b[g, n] sum_k a[m, k] b[g, k, n]."""
    A, B = tdec(aq, afmt), tdec(bq, bfmt)
    if transpose_b:  # dlhs: contract over the last axis of b, scale per b row
        B = np.transpose(B, (0, 2, 1))
    M, K = A.shape
    Nn = B.shape[2]
    gid = np.repeat(np.arange(len(gs)), gs)
    ex = np.empty((M, Nn), object)
    ab = np.empty((M, Nn), object)
    for m in range(M):
        g = gid[m]
        for n in range(Nn):
            terms = [Fraction(A[m, k]) * Fraction(B[g, k, n]) for k in range(K)]
            sc = Fraction(float(sa_row[m])) * Fraction(float(sb[g, n]))
            ex[m, n] = sum(terms) * sc
            ab[m, n] = sum(abs(t) for t in terms) * sc
    return ex, ab


def brute_tgmm(aq, afmt, sa_blk, gq, gfmt, sg_blk, gs, block_rows):
    A, Gm = tdec(aq, afmt), tdec(gq, gfmt)
    M, K = A.shape
    N = Gm.shape[1]
    off = np.concatenate([[0], np.cumsum(gs)])
    ex = np.empty((len(gs), K, N), object)
    ab = np.empty((len(gs), K, N), object)
    for g in range(len(gs)):
        for k in range(K):
            for n in range(N):
                terms = [Fraction(A[m, k]) * Fraction(Gm[m, n]) * Fraction(float(sa_blk[m // block_rows]))
                         * Fraction(float(sg_blk[m // block_rows])) for m in range(off[g], off[g + 1])]
                ex[g, k, n] = sum(terms, Fraction(0))
                ab[g, k, n] = sum((abs(t) for t in terms), Fraction(0))
    return ex, ab


@pytest.mark.parametrize("afmt,bfmt", [("e4m3", "e4m3"), ("e5m2", "e4m3")])
def test_fwd_and_dlhs_every_composition_brute_force(afmt, bfmt):
    rng = np.random.default_rng(10)
    M, G, K, N = 9, 3, 16, 4
    for gs in compositions(M, G):
        aq = random_codes(rng, (M, K), afmt)
        sa = random_scales(rng, M)
        bq = random_codes(rng, (G, K, N), bfmt)
        sb = random_scales(rng, (G, N))
        R = gmm_fwd_ref(aq, afmt, sa, bq, bfmt, sb, gs)
        ex, ab = brute_fwd(aq, afmt, sa, bq, bfmt, sb, gs)
        check_bound(R, ex, ab)
        # dlhs: grad [M, N'] against the same rhs contracted over its last axis
        gq = random_codes(rng, (M, N), afmt)
        sk = random_scales(rng, (G, K))
        R = gmm_dlhs_ref(gq, afmt, sa, bq, bfmt, sk, gs)
        ex, ab = brute_fwd(gq, afmt, sa, bq, bfmt, sk, gs, transpose_b=True)
        check_bound(R, ex, ab)


@pytest.mark.parametrize("block_rows", [4, 128])
def test_tgmm_every_composition_brute_force(block_rows):
    rng = np.random.default_rng(11)
    M, G, K, N = 9, 3, 4, 5
    nb = -(-M // block_rows)
    for gs in compositions(M, G):
        aq = random_codes(rng, (M, K), "e4m3")
        gq = random_codes(rng, (M, N), "e5m2")
        sa, sg = random_scales(rng, nb), random_scales(rng, nb)
        R = tgmm_ref(aq, "e4m3", sa, gq, "e5m2", sg, gs, block_rows)
        ex, ab = brute_tgmm(aq, "e4m3", sa, gq, "e5m2", sg, gs, block_rows)
        check_bound(R, ex, ab, extra_rel=8 * U)
        for g in np.flatnonzero(gs == 0):  # empty expert: +0.0 slab, sign bit clear
            assert (R[g].view(np.uint32) == 0).all()


def bits_of(t):
    return bf16_to_bits(t)


@pytest.fixture(scope="module")
def medium():
    """A medium ragged problem with an empty expert in the middle."""
    G, M, K, N = 5, 700, 256, 384
    gs = np.array([130, 0, 301, 1, 268], np.int32)
    lhs = bits_of(normal_bf16((M, K), 1.0, 21))
    w = bits_of(normal_bf16((G, K, N), 0.02, 22))
    grad = bits_of(normal_bf16((M, N), 1e-3, 23))
    return dict(G=G, M=M, K=K, N=N, gs=gs, lhs=lhs, w=w, grad=grad)


def test_fwd_equals_float64_loop_over_experts(medium):
    d = medium
    wq, ws = quantize_rhs_per_channel(d["w"], "e4m3", "n")
    R, aq, sa = ops.fwd(d["lhs"], wq, ws, d["gs"], "e4m3", "dynamic")
    A = tdec(aq, "e4m3") * row_scales(sa, d["M"])[:, None]
    off = group_offsets(d["gs"], d["M"])
    for g in range(d["G"]):
        r0, r1 = off[g], off[g + 1]
        B = tdec(wq[g], "e4m3") * ws[g][None, :].astype(np.float64)
        ref = A[r0:r1] @ B
        absref = np.abs(A[r0:r1]) @ np.abs(B)
        assert (np.abs(R[r0:r1] - ref) <= absref * gamma(d["K"]) + np.abs(ref) * 3 * U + 1e-30).all()


def test_tgmm_equals_sum_of_row_outer_products(medium):
    d = medium
    R, sa, sg = ops.tgmm(d["lhs"], d["grad"], d["gs"])
    from oracle.quant import quantize_rowblock

    aq, _, _ = quantize_rowblock(d["lhs"], "e4m3")
    gq, _, _ = quantize_rowblock(d["grad"], "e5m2")
    A = tdec(aq, "e4m3") * row_scales(sa, d["M"])[:, None]
    Gm = tdec(gq, "e5m2") * row_scales(sg, d["M"])[:, None]
    off = group_offsets(d["gs"], d["M"])
    for g in range(d["G"]):
        ref = np.zeros((d["K"], d["N"]))
        absref = np.zeros((d["K"], d["N"]))
        for m in range(off[g], off[g + 1]):
            ref += np.outer(A[m], Gm[m])
            absref += np.abs(np.outer(A[m], Gm[m]))
        assert (np.abs(R[g] - ref) <= absref * gamma(d["M"] + 8) + 1e-30).all()
        if off[g] == off[g + 1]:
            assert (R[g].view(np.uint32) == 0).all()


def test_merged_gate_up_equals_two_calls(medium):
    d = medium
    half = d["N"] // 2
    w0, w1 = d["w"][:, :, :half], d["w"][:, :, half:]
    wq, ws = quantize_rhs_per_channel(np.concatenate([w0, w1], axis=2), "e4m3", "n")
    wq0, ws0 = quantize_rhs_per_channel(np.ascontiguousarray(w0), "e4m3", "n")
    wq1, ws1 = quantize_rhs_per_channel(np.ascontiguousarray(w1), "e4m3", "n")
    assert (wq[:, :, :half] == wq0).all() and (wq[:, :, half:] == wq1).all()
    s = static_scale_from_bound(-4.0, 4.0, "e4m3")
    Rm, _, _ = ops.fwd(d["lhs"], wq, ws, d["gs"], "e4m3", "static", s)
    R0, _, _ = ops.fwd(d["lhs"], wq0, ws0, d["gs"], "e4m3", "static", s)
    R1, _, _ = ops.fwd(d["lhs"], wq1, ws1, d["gs"], "e4m3", "static", s)
    assert np.array_equal(Rm, np.concatenate([R0, R1], axis=1))


def test_expert_permutation_permutes_outputs(medium):
    d = medium
    wq, ws = quantize_rhs_per_channel(d["w"], "e4m3", "n")
    s = static_scale_from_bound(-4.0, 4.0, "e4m3")
    R, _, _ = ops.fwd(d["lhs"], wq, ws, d["gs"], "e4m3", "static", s)
    perm = np.array([3, 0, 4, 2, 1])
    off = group_offsets(d["gs"], d["M"])
    rows = np.concatenate([np.arange(off[p], off[p + 1]) for p in perm])
    Rp, _, _ = ops.fwd(d["lhs"][rows], wq[perm], ws[perm], d["gs"][perm], "e4m3", "static", s)
    assert np.array_equal(Rp, R[rows])


def test_dlhs_equals_forward_of_transposed_problem(medium):
    d = medium
    wq, wsk = quantize_rhs_per_channel(d["w"], "e4m3", "k")
    R, gq, sg = ops.dlhs(d["grad"], wq, wsk, d["gs"])
    wt = np.ascontiguousarray(np.transpose(wq, (0, 2, 1)))
    Rt = gmm_fwd_ref(gq, "e5m2", row_scales(sg, d["M"]), wt, "e4m3", wsk, d["gs"])
    # same sums, possibly in another float32 order: within a few ulps of the largest value
    assert np.abs(R - Rt).max() <= np.abs(Rt).max() * 1e-6


def test_quantized_result_within_bound_of_bf16_result(medium):
    d = medium
    wq, ws = quantize_rhs_per_channel(d["w"], "e4m3", "n")
    R, aq, sa = ops.fwd(d["lhs"], wq, ws, d["gs"], "e4m3", "dynamic")
    from oracle.fp8 import bf16_bits_to_f32

    X = bf16_bits_to_f32(d["lhs"]).astype(np.float64)
    W = bf16_bits_to_f32(d["w"]).astype(np.float64)
    Xh = tdec(aq, "e4m3") * row_scales(sa, d["M"])[:, None]
    Wh = tdec(wq, "e4m3") * ws[:, None, :].astype(np.float64)
    off = group_offsets(d["gs"], d["M"])
    for g in range(d["G"]):
        r0, r1 = off[g], off[g + 1]
        if r0 == r1:
            continue
        ref = X[r0:r1] @ W[g]
        dx, dw = np.abs(Xh[r0:r1] - X[r0:r1]), np.abs(Wh[g] - W[g])
        # per-element quantization error is at most half a quantum
        assert (dx <= np.maximum(np.abs(X[r0:r1]) * 2.0 ** -4, 1e-30) * 1.0001 + row_scales(sa, d["M"])[r0:r1, None] * 2.0 ** -10).all()
        lim = dx @ np.abs(W[g]) + np.abs(X[r0:r1]) @ dw + dx @ dw
        lim += (np.abs(Xh[r0:r1]) @ np.abs(Wh[g])) * gamma(d["K"] + 3)
        assert (np.abs(R[r0:r1] - ref) <= lim * 1.0001 + 1e-30).all()
        # and the bound is not vacuous: typical relative error of an fp8 product is a few %
        assert np.abs(R[r0:r1] - ref).max() < 0.2 * np.abs(ref).max()


def test_group_sizes_validation():
    with pytest.raises(ValueError):
        group_offsets([3, -1, 2])
    with pytest.raises(ValueError):
        group_offsets([3, 1, 2], M=7)
    assert group_offsets([0, 0, 5], 5).tolist() == [0, 0, 0, 5]


def test_local_windows_tile_the_plain_products(medium):
    """Local-expert windows: the full window is the plain product; windows that tile the
    experts (each zero outside its rows) add up to it exactly; tgmm windows are its slabs."""
    from oracle.gmm import gmm_dlhs_local_ref, gmm_fwd_local_ref, tgmm_local_ref
    from oracle.quant import quantize_rowblock

    d = medium
    M, G = d["M"], d["G"]
    wq, ws = quantize_rhs_per_channel(d["w"], "e4m3", "n")
    wk, sk = quantize_rhs_per_channel(d["w"], "e4m3", "k")
    aq, sa, _ = quantize_rowblock(d["lhs"], "e4m3")
    gq, sg, _ = quantize_rowblock(d["grad"], "e5m2")
    ra, rg = row_scales(sa, M), row_scales(sg, M)
    plain_f = gmm_fwd_ref(aq, "e4m3", ra, wq, "e4m3", ws, d["gs"])
    plain_d = gmm_dlhs_ref(gq, "e5m2", rg, wk, "e4m3", sk, d["gs"])
    plain_t = tgmm_ref(aq, "e4m3", sa, gq, "e5m2", sg, d["gs"])
    assert np.array_equal(gmm_fwd_local_ref(aq, "e4m3", ra, wq, "e4m3", ws, d["gs"], 0), plain_f)
    for cuts in ([0, 2, 5], [0, 1, 2, 3, 4, 5], [0, 3, 5]):
        sum_f = np.zeros_like(plain_f)
        sum_d = np.zeros_like(plain_d)
        slabs = []
        off = group_offsets(d["gs"], M)
        for a, b in zip(cuts[:-1], cuts[1:]):
            f = gmm_fwd_local_ref(aq, "e4m3", ra, wq[a:b], "e4m3", ws[a:b], d["gs"], a)
            dl = gmm_dlhs_local_ref(gq, "e5m2", rg, wk[a:b], "e4m3", sk[a:b], d["gs"], a)
            outside = np.ones(M, bool)
            outside[off[a]:off[b]] = False
            assert not f[outside].any() and not dl[outside].any()
            sum_f += f
            sum_d += dl
            slabs.append(tgmm_local_ref(aq, "e4m3", sa, gq, "e5m2", sg, d["gs"], a, b - a))
        assert np.array_equal(sum_f, plain_f) and np.array_equal(sum_d, plain_d)
        assert np.array_equal(np.concatenate(slabs), plain_t)
