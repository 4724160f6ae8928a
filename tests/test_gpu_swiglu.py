"""GPU parity of the SwiGLU steps: the merged gate|up forward with SwiGLU in its epilogue
(gmm_fwd_swiglu), the elementwise backward (gmm_swiglu_bwd) and the backward in the
epilogue of the down projection's dlhs (gmm_dlhs_swiglu_bwd)."""

import numpy as np
import pytest
import torch

import oracle.ops as ops
from oracle.fp8 import bf16_bits_to_f32, decode_fp8, f32_to_bf16_bits
from oracle.gmm import gmm_fwd_ref, row_scales
from oracle.quant import qmax_of, quantize_rhs_per_channel
from oracle.ops import dlhs as dlhs_oracle
from oracle.swiglu import swiglu_bwd_ref, swiglu_fp8_ref, swiglu_ref
from tests.gpu_util import gen, gs_tensor
from tests.parity import (TOL, assert_bf16_close, assert_fp8_codes_in_band, group_rel_err,
                          group_row_ranges, swiglu_h_bound, to_np)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("lhs_kind", ["codes", "bf16"])
def test_fused_swiglu_forward(lib, lhs_kind):
    # ragged groups with empty ones, I = 384 (3 channel-pair tiles), K tail of 256
    sizes = [0, 300, 5, 0, 457, 130]
    G, M, K, I = len(sizes), sum(sizes), 256, 384
    x, xb = gen((M, K), 1.0, 501)
    w, wb = gen((G, K, 2 * I), 0.02, 502)  # merged [W0 | W1] along N
    wq, ws = lib.gmm_quantize_rhs(w, "e4m3", 0, "nk")
    gs = gs_tensor(sizes)
    if lhs_kind == "codes":
        xq, sx = lib.gmm_quantize(x, "e4m3", "dynamic")
        lhs, kw = xq, dict(lhs_scales=sx)
    else:
        lhs, kw = x, {}
    a_codes, s_blk = ops.quantize_operand(xb, "e4m3", "dynamic")
    b_codes, b_s = quantize_rhs_per_channel(wb, "e4m3", "n")
    R = gmm_fwd_ref(a_codes, "e4m3", row_scales(s_blk, M), b_codes, "e4m3", b_s, sizes)
    Rh = swiglu_ref(R, I)
    ranges = group_row_ranges(sizes)
    for dt, view in ((torch.float32, torch.int32), (torch.bfloat16, torch.int16)):
        h, gu = lib.gmm_fwd_swiglu(lhs, wq, ws, gs, out_dtype=dt, gu=True, **kw)
        # the product half is exactly what gmm_fwd stores (GPU against GPU)
        plain = lib.gmm_fwd(lhs, wq, ws, gs, out_dtype=dt, **kw)
        assert torch.equal(gu.view(view), plain.view(view))
        if dt == torch.float32:
            err = group_rel_err(to_np(h), Rh, ranges)
            print(f"{lhs_kind}: max group relative error of h {err:.3e}")
            assert err <= TOL, err
        else:
            assert_bf16_close(to_np(h), Rh, ranges)
    # h alone (no gu) gives the same h
    h2 = lib.gmm_fwd_swiglu(lhs, wq, ws, gs, out_dtype=torch.float32, **kw)
    h1, _ = lib.gmm_fwd_swiglu(lhs, wq, ws, gs, out_dtype=torch.float32, gu=True, **kw)
    assert torch.equal(h1.view(torch.int32), h2.view(torch.int32))


def test_fused_swiglu_forward_saturated_gates(lib):
    """Gate values spread over about +-130: e^-g overflows fp32 for g below about -88 and
    underflows for large g, where the sigmoid saturates to 0 and 1; h stays finite and
    within the parity metric of the float64 definition."""
    sizes = [0, 300, 133, 457]
    G, M, K, I = len(sizes), sum(sizes), 256, 256
    x, xb = gen((M, K), 100.0, 531)
    w, wb = gen((G, K, 2 * I), 0.02, 532)
    wq, ws = lib.gmm_quantize_rhs(w, "e4m3", 0, "nk")
    gs = gs_tensor(sizes)
    a_codes, s_blk = ops.quantize_operand(xb, "e4m3", "dynamic")
    b_codes, b_s = quantize_rhs_per_channel(wb, "e4m3", "n")
    R = gmm_fwd_ref(a_codes, "e4m3", row_scales(s_blk, M), b_codes, "e4m3", b_s, sizes)
    assert R[:, :I].min() < -100 and R[:, :I].max() > 100  # both saturations occur
    h = to_np(lib.gmm_fwd_swiglu(x, wq, ws, gs, out_dtype=torch.float32))
    assert np.isfinite(h).all()
    err = group_rel_err(h, swiglu_ref(R, I), group_row_ranges(sizes))
    print(f"max group relative error of h {err:.3e}")
    assert err <= TOL, err


def test_swiglu_backward(lib):
    M, I = 777, 384
    dh, dhb = gen((M, I), 1e-3, 511)
    gu, gub = gen((M, 2 * I), 2.0, 512)
    # saturated sigmoids too: g = +-60 and -100 (exp(100) overflows in fp32)
    gu[:3, :4] = torch.tensor([60.0, -60.0, -100.0, 0.0], dtype=torch.bfloat16, device=gu.device)
    gub = gu.to("cpu").view(torch.int16).numpy().view(np.uint16)
    d = lib.gmm_swiglu_bwd(dh, gu)
    R = swiglu_bwd_ref(bf16_bits_to_f32(dhb), bf16_bits_to_f32(gub), I)
    Y = bf16_bits_to_f32(to_np(d))
    assert np.all(np.abs(Y - R) <= np.abs(R) * 2.0 ** -7 + 1e-37)  # within one bf16 ulp
    exact = np.mean(to_np(d) == f32_to_bf16_bits(R))
    print(f"bf16 outputs equal to RNE of the exact value: {exact:.5f}")
    assert exact >= 0.99


@pytest.mark.parametrize("grad_kind", ["codes", "bf16"])
def test_dlhs_swiglu_bwd(lib, grad_kind):
    """gmm_dlhs_swiglu_bwd: the same bits as gmm_dlhs (bf16 dh) followed by gmm_swiglu_bwd,
    and within the parity metric of the SwiGLU backward of the oracle's dh.  Ragged groups
    with empty and one-row ones over several 256-row tiles; I = 384, so the last 256-column
    tile is half outside the output."""
    sizes = [0, 300, 5, 0, 457, 130, 1]
    G, M, H, I = len(sizes), sum(sizes), 512, 384
    gy, gyb = gen((M, H), 1e-3, 541)
    wd, wdb = gen((G, I, H), 0.02, 542)  # down projection [G, I, hidden]
    gu, gub = gen((M, 2 * I), 2.0, 543)
    wk, wks = lib.gmm_quantize_rhs(wd, "e4m3", 1, "kn")
    gs = gs_tensor(sizes)
    if grad_kind == "codes":
        gq, sg = lib.gmm_quantize(gy, "e5m2", "dynamic")
        grad, kw = gq, dict(grad_scales=sg)
    else:
        grad, kw = gy, {}
    dh = lib.gmm_dlhs(grad, wk, wks, gs, **kw)
    two_calls = lib.gmm_swiglu_bwd(dh, gu)
    d = lib.gmm_dlhs_swiglu_bwd(grad, wk, wks, gs, gu, **kw)
    assert torch.equal(d.view(torch.int16), two_calls.view(torch.int16))
    # into a given output, twice: the same bits
    out = torch.full_like(d, float("nan"))
    lib.gmm_dlhs_swiglu_bwd(grad, wk, wks, gs, gu, out=out, **kw)
    assert torch.equal(out.view(torch.int16), two_calls.view(torch.int16))
    with pytest.raises(ValueError):
        lib.gmm_dlhs_swiglu_bwd(grad, wk, wks, gs, gu[:, :I].contiguous(), **kw)
    # d_gu's dynamic block scales from the same epilogue: the prepass's values, bit for bit
    for fmt in ("e5m2", "e4m3"):
        d2, sc = lib.gmm_dlhs_swiglu_bwd(grad, wk, wks, gs, gu, d_gu_format=fmt, **kw)
        assert torch.equal(d2.view(torch.int16), two_calls.view(torch.int16))
        want = lib.gmm_dynamic_scales(two_calls, fmt)
        assert torch.equal(sc.view(torch.int32), want.view(torch.int32)), fmt
    # oracle: dh from the oracle's dlhs, rounded to bf16 as the method hands it on, then
    # the SwiGLU backward.  Both sides round dh to bf16; where the two fp32 sums lie on
    # either side of a rounding boundary the dh differ by one bf16 ulp (2^-8 relative),
    # which scales that row's d_gu values alike, and the GPU rounds d_gu once more
    # (2^-9): so each element is held to 2^-7 of itself plus the parity metric's
    # 1e-3 of its group's largest value (the fp32 sums' own difference).
    c_ref, s_ref = quantize_rhs_per_channel(wdb, "e4m3", "k")
    R_dh, _, _ = dlhs_oracle(gyb, c_ref, s_ref, sizes, "e5m2", "dynamic")
    dh_ref = bf16_bits_to_f32(f32_to_bf16_bits(R_dh))
    R = swiglu_bwd_ref(dh_ref, bf16_bits_to_f32(gub), I).astype(np.float64)
    Y = bf16_bits_to_f32(to_np(d)).astype(np.float64)
    worst = 0.0
    for lo, hi in group_row_ranges(sizes):
        if hi <= lo:
            continue
        r, y = R[lo:hi], Y[lo:hi]
        bound = 2.0 ** -7 * np.abs(r) + TOL * np.abs(r).max()
        worst = max(worst, float((np.abs(y - r) / bound).max()))
    exact = float(np.mean(to_np(d) == f32_to_bf16_bits(R.astype(np.float32))))
    print(f"{grad_kind}: worst error / bound {worst:.3f}; d_gu equal to RNE(oracle): {exact:.5f}")
    assert worst <= 1.0
    assert exact >= 0.95


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fused_swiglu_forward_fp8_h(lib, fmt):
    """gmm_fwd_swiglu_fp8: h as fp8 codes of a static scale, then the down projection on
    those codes.  Codes lie within the rounding band of the oracle's h (the products'
    fp32 sums may round differently) and nearly all equal the oracle's; the down output
    matches the oracle's, allowing one code step where the band spans two codes."""
    sizes = [0, 300, 5, 0, 457, 130]
    G, M, K, I = len(sizes), sum(sizes), 256, 384
    x, xb = gen((M, K), 1.0, 521)
    w, wb = gen((G, K, 2 * I), 0.02, 522)
    wd, wdb = gen((G, I, K), 0.02, 523)  # down projection [G, I, hidden]
    gs = gs_tensor(sizes)
    wq, ws = lib.gmm_quantize_rhs(w, "e4m3", 0, "nk")
    wdq, wds = lib.gmm_quantize_rhs(wd, "e4m3", 0, "nk")
    xq, sx = lib.gmm_quantize(x, "e4m3", "dynamic")
    a_codes, s_blk = ops.quantize_operand(xb, "e4m3", "dynamic")
    b_codes, b_s = quantize_rhs_per_channel(wb, "e4m3", "n")
    sa = row_scales(s_blk, M)
    R = gmm_fwd_ref(a_codes, "e4m3", sa, b_codes, "e4m3", b_s, sizes)
    absR = gmm_fwd_ref(a_codes & 0x7F, "e4m3", sa, b_codes & 0x7F, "e4m3", b_s, sizes)
    # a scale that puts the largest |h| at twice qmax: the top values saturate
    s = np.float32(np.abs(swiglu_ref(R, I)).max() / (2 * qmax_of(fmt)))
    ref_codes, _ = swiglu_fp8_ref(R, I, s, fmt)
    h_codes, gu = lib.gmm_fwd_swiglu_fp8(xq, wq, ws, gs, float(s), h_format=fmt, lhs_scales=sx,
                                         gu=True)
    assert h_codes.dtype == torch.uint8 and tuple(h_codes.shape) == (M, I)
    plain = lib.gmm_fwd(xq, wq, ws, gs, lhs_scales=sx)
    assert torch.equal(gu.view(torch.int16), plain.view(torch.int16))
    h_only = lib.gmm_fwd_swiglu_fp8(xq, wq, ws, gs, float(s), h_format=fmt, lhs_scales=sx)
    assert torch.equal(h_only, h_codes)
    codes = to_np(h_codes)
    h, dh = swiglu_h_bound(R, absR, K, I)
    diff, amb = assert_fp8_codes_in_band(codes, h, dh, s, fmt, ref_codes, min_exact=0.99)
    print(f"{fmt}: codes differing from the oracle's {diff:.2e}, bands spanning two codes {amb:.2e}")
    assert np.mean(np.abs(swiglu_ref(R, I)) / s >= qmax_of(fmt)) > 0  # saturation exercised
    # the down projection on the codes, against the oracle's on its own codes
    y = lib.gmm_fwd(h_codes, wdq, wds, gs, lhs_format=fmt, lhs_scaling="static",
                    static_scale=float(s), out_dtype=torch.float32)
    bd, bds = quantize_rhs_per_channel(wdb, "e4m3", "n")
    Ry = gmm_fwd_ref(ref_codes, fmt, np.full(M, s, np.float32), bd, "e4m3", bds, sizes)
    # one code step of slack wherever the GPU code differs from the oracle's
    step = np.abs(decode_fp8(codes, fmt).astype(np.float64) -
                  decode_fp8(ref_codes, fmt).astype(np.float64)) * s
    wabs = np.abs(decode_fp8(bd, "e4m3").astype(np.float64)) * bds[:, None, :]
    Y = to_np(y).astype(np.float64)
    for g, (lo, hi) in enumerate(group_row_ranges(sizes)):
        if hi == lo:
            continue
        allow = TOL * np.abs(Ry[lo:hi]).max() + step[lo:hi] @ wabs[g] * (1 + 1e-6)
        assert np.all(np.abs(Y[lo:hi] - Ry[lo:hi]) <= allow), g
