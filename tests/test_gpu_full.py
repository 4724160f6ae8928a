"""Full-size GPU parity at the benchmark workloads' shapes, on sampled outputs.

Each product runs through the library as bench.py launches it: device-resident bf16
inputs from the seeded generators, block scales from the abs-max prepass handed in as
given scales, bf16 outputs (and once more with f32 outputs for the 1e-3 metric).  The
oracle then recomputes a sample of the outputs from the same bf16 inputs: the dynamic
block scales from whole 128-row blocks, the codes only for the sampled rows (and, for
the weights, only the sampled channels), the grouped products over the sample.  Scales
and sampled codes are compared byte for byte.
"""

import numpy as np
import pytest
import torch

from oracle.fp8 import bf16_bits_to_f32
from oracle.gmm import gmm_dlhs_ref, gmm_fwd_ref, tgmm_ref
from oracle.quant import (block_amax, dynamic_scale_from_amax, quantize_rhs_per_channel,
                          quantize_with_inv, static_inv)
from synth.workloads import WORKLOADS, bf16_to_bits, normal_bf16
from tests.gpu_util import DEV, gs_tensor, sync
from tests.parity import (TOL, assert_bf16_close, assert_rounding_bound, group_rel_err,
                          group_row_ranges, magnitudes, to_np)

pytestmark = pytest.mark.gpu

S_4_448 = float(np.float32(4.0) / np.float32(448.0))


def sample_rows(sizes, rng, per_group=3):
    """First and last row of every group, rows on both sides of a 128-row block boundary
    inside it, and a few random rows."""
    off = np.concatenate([[0], np.cumsum(sizes)])
    rows = set()
    for g in range(len(sizes)):
        a, b = int(off[g]), int(off[g + 1])
        if b == a:
            continue
        rows.update({a, b - 1})
        rows.update(int(r) for r in rng.integers(a, b, size=per_group))
        edge = (a // 128 + 1) * 128
        if edge < b:
            rows.update({edge - 1, edge})
    return np.array(sorted(rows), np.int64)


def sample_cols(n, rng, count=64):
    """Both ends, both sides of the gate|up seam at n/2, and random columns."""
    cols = {0, n - 1, n // 2 - 1, n // 2}
    cols.update(int(c) for c in rng.integers(0, n, size=count))
    return np.array(sorted(cols), np.int64)


def sampled_sizes(rows, sizes):
    off = np.concatenate([[0], np.cumsum(sizes)])
    return np.array([int(((rows >= off[g]) & (rows < off[g + 1])).sum())
                     for g in range(len(sizes))], np.int32)


def dynamic_block_scales(x_bits, fmt):
    return dynamic_scale_from_amax(block_amax(x_bits, 128), fmt)


def check_sampled(Ybf, Y32, R, sub_sizes, absR=None, n_terms=None):
    ranges = group_row_ranges(sub_sizes)
    err = group_rel_err(Y32, R, ranges)
    print(f"sampled max group relative error {err:.3e} over {R.size} outputs", flush=True)
    assert err <= TOL, err
    if absR is not None:
        assert_rounding_bound(Y32, R, absR, n_terms)
    assert_bf16_close(Ybf, R, ranges)


def test_mixtral_gate_up_forward(lib):
    wl = WORKLOADS["mixtral_gate_up"]
    G, M, K, N = wl.G, wl.M, wl.K, wl.N
    sizes = wl.group_sizes()
    seed = wl.seed * 100
    x = normal_bf16((M, K), 1.0, seed, DEV)
    w = normal_bf16((G, K, N), 0.02, seed + 1, DEV)
    gs = gs_tensor(sizes)
    wq, ws = lib.gmm_quantize_rhs(w, "e4m3", 0, "nk")
    s = lib.gmm_dynamic_scales(x, "e4m3")
    out = lib.gmm_fwd(x, wq, ws, gs, lhs_scaling="dynamic_given", lhs_scales=s)
    out32 = lib.gmm_fwd(x, wq, ws, gs, lhs_scaling="dynamic_given", lhs_scales=s,
                        out_dtype=torch.float32)
    sync()
    rng = np.random.default_rng(2)
    rows, cols = sample_rows(sizes, rng), sample_cols(N, rng)
    xb = bf16_to_bits(x)
    s_ref, inv_ref = dynamic_block_scales(xb, "e4m3")
    assert np.array_equal(to_np(s).view(np.uint32), s_ref.view(np.uint32))
    a_codes = quantize_with_inv(bf16_bits_to_f32(xb[rows]), inv_ref[rows // 128], "e4m3")
    b_codes, b_s = quantize_rhs_per_channel(bf16_to_bits(w[:, :, cols]), "e4m3", "n")
    ci = torch.as_tensor(cols, device=DEV)
    assert np.array_equal(to_np(ws[:, ci]).view(np.uint32), b_s.view(np.uint32))
    assert np.array_equal(np.transpose(to_np(wq[:, ci, :]), (0, 2, 1)), b_codes)
    sub = sampled_sizes(rows, sizes)
    R = gmm_fwd_ref(a_codes, "e4m3", s_ref[rows // 128], b_codes, "e4m3", b_s, sub)
    absR = gmm_fwd_ref(magnitudes(a_codes), "e4m3", s_ref[rows // 128], magnitudes(b_codes),
                       "e4m3", b_s, sub)
    ri = torch.as_tensor(rows, device=DEV)
    check_sampled(to_np(out[ri][:, ci]), to_np(out32[ri][:, ci]), R, sub, absR, K)


@pytest.fixture(scope="module")
def deepseek():
    """The DeepSeek-style local-expert tensors, generated once for the module."""
    wl = WORKLOADS["deepseek_local"]
    G, M, K, N = wl.G, wl.M, wl.K, wl.N
    seed = wl.seed * 100
    sizes = wl.group_sizes()
    assert sizes[0] == 0 and sizes[17] == 0
    x = normal_bf16((M, K), 1.0, seed, DEV)
    w = normal_bf16((G, K, N), 0.02, seed + 1, DEV)
    grad = normal_bf16((M, N), 1e-3, seed + 2, DEV)
    return wl, sizes, x, w, grad


def test_deepseek_local_forward_static(lib, deepseek):
    wl, sizes, x, w, _ = deepseek
    N = wl.N
    gs = gs_tensor(sizes)
    wq, ws = lib.gmm_quantize_rhs(w, "e4m3", 0, "nk")
    out = lib.gmm_fwd(x, wq, ws, gs, lhs_scaling="static", static_scale=S_4_448)
    out32 = lib.gmm_fwd(x, wq, ws, gs, lhs_scaling="static", static_scale=S_4_448,
                        out_dtype=torch.float32)
    sync()
    rng = np.random.default_rng(3)
    rows, cols = sample_rows(sizes, rng), sample_cols(N, rng)
    inv = static_inv(np.float32(S_4_448))
    a_codes = quantize_with_inv(bf16_bits_to_f32(bf16_to_bits(x[torch.as_tensor(rows, device=DEV)])),
                                np.full(len(rows), inv, np.float32), "e4m3")
    b_codes, b_s = quantize_rhs_per_channel(bf16_to_bits(w[:, :, cols]), "e4m3", "n")
    sub = sampled_sizes(rows, sizes)
    R = gmm_fwd_ref(a_codes, "e4m3", np.full(len(rows), S_4_448, np.float32), b_codes, "e4m3",
                    b_s, sub)
    absR = gmm_fwd_ref(magnitudes(a_codes), "e4m3", np.full(len(rows), S_4_448, np.float32),
                       magnitudes(b_codes), "e4m3", b_s, sub)
    ri, ci = torch.as_tensor(rows, device=DEV), torch.as_tensor(cols, device=DEV)
    check_sampled(to_np(out[ri][:, ci]), to_np(out32[ri][:, ci]), R, sub, absR, a_codes.shape[1])


@pytest.mark.parametrize("route", ["hybrid", "fused"])
def test_deepseek_local_dlhs(lib, deepseek, route):
    wl, sizes, _, w, grad = deepseek
    K = wl.K
    gs = gs_tensor(sizes)
    wk, sk = lib.gmm_quantize_rhs(w, "e4m3", 1, "kn")
    if route == "hybrid":  # as the benchmark step: quantize once, then the fp8-A product
        gq, sg = lib.gmm_quantize(grad, "e5m2", "dynamic")
        a, kw = gq, dict(grad_format="e5m2", grad_scaling="dynamic", grad_scales=sg)
    else:
        sg = lib.gmm_dynamic_scales(grad, "e5m2")
        a, kw = grad, dict(grad_format="e5m2", grad_scaling="dynamic_given", grad_scales=sg)
    out = lib.gmm_dlhs(a, wk, sk, gs, **kw)
    out32 = lib.gmm_dlhs(a, wk, sk, gs, out_dtype=torch.float32, **kw)
    sync()
    rng = np.random.default_rng(4)
    rows, kcols = sample_rows(sizes, rng), sample_cols(K, rng)
    gb = bf16_to_bits(grad)
    s_ref, inv_ref = dynamic_block_scales(gb, "e5m2")
    assert np.array_equal(to_np(sg).view(np.uint32), s_ref.view(np.uint32))
    g_codes = quantize_with_inv(bf16_bits_to_f32(gb[rows]), inv_ref[rows // 128], "e5m2")
    if route == "hybrid":
        assert np.array_equal(to_np(gq[torch.as_tensor(rows, device=DEV)]), g_codes)
    b_codes, b_s = quantize_rhs_per_channel(bf16_to_bits(w[:, kcols, :]), "e4m3", "k")
    ki = torch.as_tensor(kcols, device=DEV)
    assert np.array_equal(to_np(sk[:, ki]).view(np.uint32), b_s.view(np.uint32))
    assert np.array_equal(to_np(wk[:, ki, :]), b_codes)
    sub = sampled_sizes(rows, sizes)
    R = gmm_dlhs_ref(g_codes, "e5m2", s_ref[rows // 128], b_codes, "e4m3", b_s, sub)
    absR = gmm_dlhs_ref(magnitudes(g_codes), "e5m2", s_ref[rows // 128], magnitudes(b_codes),
                        "e4m3", b_s, sub)
    ri = torch.as_tensor(rows, device=DEV)
    check_sampled(to_np(out[ri][:, ki]), to_np(out32[ri][:, ki]), R, sub, absR, g_codes.shape[1])


def test_deepseek_local_tgmm(lib, deepseek):
    wl, sizes, x, _, grad = deepseek
    G, K, N = wl.G, wl.K, wl.N
    gs = gs_tensor(sizes)
    sa = lib.gmm_dynamic_scales(x, "e4m3")
    sg = lib.gmm_dynamic_scales(grad, "e5m2")
    kw = dict(lhs_scaling="dynamic_given", lhs_scales=sa, grad_scaling="dynamic_given",
              grad_scales=sg)
    out = lib.tgmm_drhs(x, grad, gs, **kw)
    out32 = lib.tgmm_drhs(x, grad, gs, out_dtype=torch.float32, **kw)
    sync()
    rng = np.random.default_rng(5)
    ks, ns = sample_cols(K, rng, 32), sample_cols(N, rng, 32)
    xb, gb = bf16_to_bits(x), bf16_to_bits(grad)
    sa_ref, ia = dynamic_block_scales(xb, "e4m3")
    sg_ref, ig = dynamic_block_scales(gb, "e5m2")
    assert np.array_equal(to_np(sa).view(np.uint32), sa_ref.view(np.uint32))
    assert np.array_equal(to_np(sg).view(np.uint32), sg_ref.view(np.uint32))
    rb = np.arange(wl.M) // 128
    a_codes = quantize_with_inv(bf16_bits_to_f32(xb[:, ks]), ia[rb], "e4m3")
    g_codes = quantize_with_inv(bf16_bits_to_f32(gb[:, ns]), ig[rb], "e5m2")
    R = tgmm_ref(a_codes, "e4m3", sa_ref, g_codes, "e5m2", sg_ref, np.asarray(sizes))
    ki, ni = torch.as_tensor(ks, device=DEV), torch.as_tensor(ns, device=DEV)
    Ybf = to_np(out[:, ki][:, :, ni])
    Y32 = to_np(out32[:, ki][:, :, ni])
    for g in (0, 17):  # the empty experts: whole slabs of +0.0
        assert (to_np(out32[g]).view(np.uint32) == 0).all()
        assert (to_np(out[g]) == 0).all()
    ranges = [(g, g + 1) for g in range(G)]
    err = group_rel_err(Y32, R, ranges)
    print(f"sampled max slab relative error {err:.3e}", flush=True)
    assert err <= TOL, err
    absR = tgmm_ref(magnitudes(a_codes), "e4m3", sa_ref, magnitudes(g_codes), "e5m2", sg_ref,
                    np.asarray(sizes))
    assert_rounding_bound(Y32, R, absR, np.asarray(sizes)[:, None, None])
    assert_bf16_close(Ybf, R, ranges)


# ---- the MoE SwiGLU feed-forward chain, forward and backward -------------------------

def _check_fwd(lib, lhs, scaling, s_gpu, w_bits_cols, wq, ws, cols, sizes, out, out32, rng,
               w_layout="nk"):
    """One forward product against the oracle on sampled rows x the sampled columns."""
    rows = sample_rows(sizes, rng)
    lb = bf16_to_bits(lhs)
    if scaling == "static":
        inv = static_inv(np.float32(S_4_448))
        s_row = np.full(len(rows), S_4_448, np.float32)
        a_codes = quantize_with_inv(bf16_bits_to_f32(lb[rows]), np.full(len(rows), inv, np.float32), "e4m3")
    else:
        s_ref, inv_ref = dynamic_block_scales(lb, "e4m3")
        assert np.array_equal(to_np(s_gpu).view(np.uint32), s_ref.view(np.uint32))
        s_row = s_ref[rows // 128]
        a_codes = quantize_with_inv(bf16_bits_to_f32(lb[rows]), inv_ref[rows // 128], "e4m3")
    b_codes, b_s = quantize_rhs_per_channel(w_bits_cols, "e4m3", "n")
    ci = torch.as_tensor(cols, device=DEV)
    assert np.array_equal(to_np(ws[:, ci]).view(np.uint32), b_s.view(np.uint32))
    assert np.array_equal(np.transpose(to_np(wq[:, ci, :]), (0, 2, 1)), b_codes)
    sub = sampled_sizes(rows, sizes)
    R = gmm_fwd_ref(a_codes, "e4m3", s_row, b_codes, "e4m3", b_s, sub)
    absR = gmm_fwd_ref(magnitudes(a_codes), "e4m3", s_row, magnitudes(b_codes), "e4m3", b_s, sub)
    ri = torch.as_tensor(rows, device=DEV)
    check_sampled(to_np(out[ri][:, ci]), to_np(out32[ri][:, ci]), R, sub, absR, a_codes.shape[1])


def _check_dlhs(grad, s_gpu, w_bits_krows, wk, sk, kcols, sizes, out, out32, rng):
    rows = sample_rows(sizes, rng)
    gb = bf16_to_bits(grad)
    s_ref, inv_ref = dynamic_block_scales(gb, "e5m2")
    assert np.array_equal(to_np(s_gpu).view(np.uint32), s_ref.view(np.uint32))
    g_codes = quantize_with_inv(bf16_bits_to_f32(gb[rows]), inv_ref[rows // 128], "e5m2")
    b_codes, b_s = quantize_rhs_per_channel(w_bits_krows, "e4m3", "k")
    ki = torch.as_tensor(kcols, device=DEV)
    assert np.array_equal(to_np(sk[:, ki]).view(np.uint32), b_s.view(np.uint32))
    assert np.array_equal(to_np(wk[:, ki, :]), b_codes)
    sub = sampled_sizes(rows, sizes)
    R = gmm_dlhs_ref(g_codes, "e5m2", s_ref[rows // 128], b_codes, "e4m3", b_s, sub)
    absR = gmm_dlhs_ref(magnitudes(g_codes), "e5m2", s_ref[rows // 128], magnitudes(b_codes),
                        "e4m3", b_s, sub)
    ri = torch.as_tensor(rows, device=DEV)
    check_sampled(to_np(out[ri][:, ki]), to_np(out32[ri][:, ki]), R, sub, absR, g_codes.shape[1])


def _check_tgmm(lhs, grad, sa, sg, sizes, out, out32, rng):
    M, K = lhs.shape
    N = grad.shape[1]
    ks, ns = sample_cols(K, rng, 24), sample_cols(N, rng, 24)
    lb, gb = bf16_to_bits(lhs), bf16_to_bits(grad)
    sa_ref, ia = dynamic_block_scales(lb, "e4m3")
    sg_ref, ig = dynamic_block_scales(gb, "e5m2")
    assert np.array_equal(to_np(sa).view(np.uint32), sa_ref.view(np.uint32))
    assert np.array_equal(to_np(sg).view(np.uint32), sg_ref.view(np.uint32))
    rb = np.arange(M) // 128
    a_codes = quantize_with_inv(bf16_bits_to_f32(lb[:, ks]), ia[rb], "e4m3")
    g_codes = quantize_with_inv(bf16_bits_to_f32(gb[:, ns]), ig[rb], "e5m2")
    R = tgmm_ref(a_codes, "e4m3", sa_ref, g_codes, "e5m2", sg_ref, np.asarray(sizes))
    absR = tgmm_ref(magnitudes(a_codes), "e4m3", sa_ref, magnitudes(g_codes), "e5m2", sg_ref,
                    np.asarray(sizes))
    ki, ni = torch.as_tensor(ks, device=DEV), torch.as_tensor(ns, device=DEV)
    ranges = [(g, g + 1) for g in range(len(sizes))]
    err = group_rel_err(to_np(out32[:, ki][:, :, ni]), R, ranges)
    print(f"sampled max slab relative error {err:.3e}", flush=True)
    assert err <= TOL, err
    assert_rounding_bound(to_np(out32[:, ki][:, :, ni]), R, absR, np.asarray(sizes)[:, None, None])
    assert_bf16_close(to_np(out[:, ki][:, :, ni]), R, ranges)


def test_mixtral_gate_up_step(lib):
    """The benchmark step at full size, launched as bench.py launches it: lhs and grad each
    quantized once (dynamic 128-row blocks), fwd and dlhs on those codes, tgmm on both
    codes.  Sampled codes byte for byte, sampled outputs of all three products against
    the oracle recomputed from the bf16 inputs."""
    wl = WORKLOADS["mixtral_gate_up"]
    G, M, K, N = wl.G, wl.M, wl.K, wl.N
    sizes = wl.group_sizes()
    seed = wl.seed * 100
    x = normal_bf16((M, K), 1.0, seed, DEV)
    w = normal_bf16((G, K, N), 0.02, seed + 1, DEV)
    grad = normal_bf16((M, N), 1e-3, seed + 2, DEV)
    gs = gs_tensor(sizes)
    wq, ws = lib.gmm_quantize_rhs(w, "e4m3", 0, "nk")
    wk, sk = lib.gmm_quantize_rhs(w, "e4m3", 1, "kn")
    xq, sx = lib.gmm_quantize(x, "e4m3", "dynamic")
    gq, sg = lib.gmm_quantize(grad, "e5m2", "dynamic")
    fk = dict(lhs_scaling="dynamic", lhs_scales=sx)
    out = lib.gmm_fwd(xq, wq, ws, gs, **fk)
    out32 = lib.gmm_fwd(xq, wq, ws, gs, out_dtype=torch.float32, **fk)
    dk = dict(grad_scaling="dynamic", grad_scales=sg)
    dl = lib.gmm_dlhs(gq, wk, sk, gs, **dk)
    dl32 = lib.gmm_dlhs(gq, wk, sk, gs, out_dtype=torch.float32, **dk)
    tk = dict(lhs_scales=sx, grad_scales=sg)
    dw = lib.tgmm_drhs(xq, gq, gs, **tk)
    dw32 = lib.tgmm_drhs(xq, gq, gs, out_dtype=torch.float32, **tk)
    sync()
    rng = np.random.default_rng(7)
    rows = sample_rows(sizes, rng)
    ri = torch.as_tensor(rows, device=DEV)
    for t, codes, fmt in ((x, xq, "e4m3"), (grad, gq, "e5m2")):
        b = bf16_to_bits(t)
        _, inv = dynamic_block_scales(b, fmt)
        ref = quantize_with_inv(bf16_bits_to_f32(b[rows]), inv[rows // 128], fmt)
        assert np.array_equal(to_np(codes[ri]), ref)
    cols = sample_cols(N, rng)
    _check_fwd(lib, x, "dynamic", sx, bf16_to_bits(w[:, :, cols]), wq, ws, cols, sizes, out,
               out32, rng)
    kc = sample_cols(K, rng)
    _check_dlhs(grad, sg, bf16_to_bits(w[:, kc, :]), wk, sk, kc, sizes, dl, dl32, rng)
    _check_tgmm(x, grad, sx, sg, sizes, dw, dw32, rng)


def test_moe_swiglu_fused_forward(lib, swiglu):
    """gmm_fwd_swiglu at the full SwiGLU block shape: sampled rows x sampled channel pairs
    of h against the oracle's product and SwiGLU, and the product half against gmm_fwd;
    gmm_fwd_swiglu_fp8's codes of h on the same samples."""
    wl, sizes, x, w_gu = swiglu[:4]
    I = wl.extra["intermediate"]
    gs = gs_tensor(sizes)
    wq, ws = lib.gmm_quantize_rhs(w_gu, "e4m3", 0, "nk")
    xq, sx = lib.gmm_quantize(x, "e4m3", "dynamic")
    h, gu = lib.gmm_fwd_swiglu(xq, wq, ws, gs, lhs_scales=sx, out_dtype=torch.float32, gu=True)
    plain = lib.gmm_fwd(xq, wq, ws, gs, lhs_scales=sx, out_dtype=torch.float32)
    sync()
    assert torch.equal(gu.view(torch.int32), plain.view(torch.int32))
    rng = np.random.default_rng(8)
    rows = sample_rows(sizes, rng)
    cols = sample_cols(I, rng, 24)
    both = np.concatenate([cols, I + cols])
    xb = bf16_to_bits(x)
    s_ref, inv_ref = dynamic_block_scales(xb, "e4m3")
    a_codes = quantize_with_inv(bf16_bits_to_f32(xb[rows]), inv_ref[rows // 128], "e4m3")
    bi = torch.as_tensor(both, device=DEV)
    b_codes, b_s = quantize_rhs_per_channel(bf16_to_bits(w_gu[:, :, bi]), "e4m3", "n")
    sub = sampled_sizes(rows, sizes)
    R = gmm_fwd_ref(a_codes, "e4m3", s_ref[rows // 128], b_codes, "e4m3", b_s, sub)
    from oracle.swiglu import swiglu_ref
    Rh = swiglu_ref(R, len(cols))
    ri, ci = torch.as_tensor(rows, device=DEV), torch.as_tensor(cols, device=DEV)
    err = group_rel_err(to_np(h[ri][:, ci]), Rh, group_row_ranges(sub))
    print(f"sampled max group relative error of h {err:.3e}", flush=True)
    assert err <= TOL, err
    # h as e4m3 codes of a static scale (the largest sampled |h| at qmax): the sampled codes
    # lie in the rounding band of the oracle's h
    from oracle.swiglu import swiglu_fp8_ref
    from tests.parity import assert_fp8_codes_in_band, swiglu_h_bound

    s_h = np.float32(np.abs(Rh).max() / 448.0)
    hq = lib.gmm_fwd_swiglu_fp8(xq, wq, ws, gs, float(s_h), lhs_scales=sx)
    sync()
    ref_codes, _ = swiglu_fp8_ref(R, len(cols), s_h, "e4m3")
    absR = gmm_fwd_ref(a_codes & 0x7F, "e4m3", s_ref[rows // 128], b_codes & 0x7F, "e4m3", b_s, sub)
    hb, dh = swiglu_h_bound(R, absR, x.shape[1], len(cols))
    diff, amb = assert_fp8_codes_in_band(to_np(hq[ri][:, ci]), hb, dh, s_h, "e4m3", ref_codes,
                                         min_exact=0.99)
    print(f"sampled fp8 h codes differing from the oracle's {diff:.2e} (bands spanning two "
          f"codes {amb:.2e})", flush=True)


@pytest.fixture(scope="module")
def swiglu():
    wl = WORKLOADS["moe_swiglu"]
    G, M, H = wl.G, wl.M, wl.K
    inter = wl.extra["intermediate"]
    seed = wl.seed * 100
    sizes = wl.group_sizes()
    x = normal_bf16((M, H), 1.0, seed, DEV)
    w_gu = normal_bf16((G, H, 2 * inter), 0.02, seed + 1, DEV)
    w_down = normal_bf16((G, inter, H), 0.02, seed + 2, DEV)
    grad_y = normal_bf16((M, H), 1e-3, seed + 3, DEV)
    # the down projection's input and the gate|up gradient, seeded like the rest (each
    # product gets inputs of its own, none produced by another product of the library)
    h = normal_bf16((M, inter), 1.0, seed + 4, DEV)
    d_gu = normal_bf16((M, 2 * inter), 1e-3, seed + 5, DEV)
    return wl, sizes, x, w_gu, w_down, grad_y, h, d_gu


@pytest.mark.parametrize("scaling", ["static", "dynamic"])
@pytest.mark.parametrize("mode", ["pure", "hybrid"])
def test_moe_swiglu_chain(lib, swiglu, mode, scaling):
    """The six products of the MoE SwiGLU block at full size, for pure / hybrid and static
    / dynamic lhs scaling: gate|up and down forward, the dlhs of both, the tgmm of both.
    Each runs on seeded inputs of its shape (x, the down projection's input h, the
    output gradient, the gate|up gradient), so the oracle never sees a value the
    library produced; each is checked on sampled rows and columns."""
    wl, sizes, x, w_gu, w_down, grad_y, h, d_gu = swiglu
    inter = wl.extra["intermediate"]
    gs = gs_tensor(sizes)
    rng = np.random.default_rng(6)
    fwd_kw = (dict(lhs_scaling="static", static_scale=S_4_448) if scaling == "static"
              else dict(lhs_scaling="dynamic"))

    def fwd(lhs, wq, ws):
        out, s = lib.gmm_fwd(lhs, wq, ws, gs, return_scales=True, **fwd_kw)
        out32 = lib.gmm_fwd(lhs, wq, ws, gs, out_dtype=torch.float32, **fwd_kw)
        return out, out32, s

    def dlhs(grad, wk, sk):
        if mode == "hybrid":
            gq, sg = lib.gmm_quantize(grad, "e5m2", "dynamic")
            a, kw = gq, dict(grad_scaling="dynamic", grad_scales=sg)
        else:
            a, kw = grad, dict(grad_scaling="dynamic")
        out, sg = lib.gmm_dlhs(a, wk, sk, gs, return_scales=True, **kw)
        out32 = lib.gmm_dlhs(a, wk, sk, gs, out_dtype=torch.float32, **kw)
        return out, out32, sg

    # forward
    wgu_q, wgu_s = lib.gmm_quantize_rhs(w_gu, "e4m3", 0, "nk")
    wdn_q, wdn_s = lib.gmm_quantize_rhs(w_down, "e4m3", 0, "nk")
    gu, gu32, s_x = fwd(x, wgu_q, wgu_s)
    y, y32, s_h = fwd(h, wdn_q, wdn_s)
    # backward
    wgu_k, wgu_sk = lib.gmm_quantize_rhs(w_gu, "e4m3", 1, "kn")
    wdn_k, wdn_sk = lib.gmm_quantize_rhs(w_down, "e4m3", 1, "kn")
    dh, dh32, s_gy = dlhs(grad_y, wdn_k, wdn_sk)
    dx, dx32, s_dgu = dlhs(d_gu, wgu_k, wgu_sk)
    tk = dict(lhs_scaling="dynamic", grad_scaling="dynamic", return_scales=True)
    dwd, sa_h, sg_y = lib.tgmm_drhs(h, grad_y, gs, **tk)
    dwd32 = lib.tgmm_drhs(h, grad_y, gs, out_dtype=torch.float32, lhs_scaling="dynamic",
                          grad_scaling="dynamic")
    dwg, sa_x, sg_dgu = lib.tgmm_drhs(x, d_gu, gs, **tk)
    dwg32 = lib.tgmm_drhs(x, d_gu, gs, out_dtype=torch.float32, lhs_scaling="dynamic",
                          grad_scaling="dynamic")
    sync()

    H = wl.K
    cols = sample_cols(2 * inter, rng)
    _check_fwd(lib, x, scaling, s_x, bf16_to_bits(w_gu[:, :, cols]), wgu_q, wgu_s, cols, sizes,
               gu, gu32, rng)
    cols = sample_cols(H, rng)
    _check_fwd(lib, h, scaling, s_h, bf16_to_bits(w_down[:, :, cols]), wdn_q, wdn_s, cols, sizes,
               y, y32, rng)
    kc = sample_cols(inter, rng)
    _check_dlhs(grad_y, s_gy, bf16_to_bits(w_down[:, kc, :]), wdn_k, wdn_sk, kc, sizes, dh, dh32, rng)
    kc = sample_cols(H, rng)
    _check_dlhs(d_gu, s_dgu, bf16_to_bits(w_gu[:, kc, :]), wgu_k, wgu_sk, kc, sizes, dx, dx32, rng)
    _check_tgmm(h, grad_y, sa_h, sg_y, sizes, dwd, dwd32, rng)
    _check_tgmm(x, d_gu, sa_x, sg_dgu, sizes, dwg, dwg32, rng)
