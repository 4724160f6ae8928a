"""GPU parity of gmm_fwd_swiglu_fp8_subchannel: h of the merged gate|up forward as fp8
codes under dynamic scales per row and 128-channel block, taken in the product's
epilogue, and the down projection on them through gmm_fwd_blockwise (bk = 128).

The kernel's h differs from the oracle's by the rounding of the products' sums and of
the SwiGLU (the band of swiglu_h_bound), so its block abs-max, and with it the rounded
scale, is usually a few ulps off the oracle's: the scales are held to that band, the
codes to the band of h under the kernel's own scales and, nearly all, to the oracle's h
quantized under those scales, and the down projection, given the kernel's codes and
scales, to the oracle's on the same inputs."""

import numpy as np
import pytest
import torch

import oracle.ops as ops
from oracle.blockwise import gmm_fwd_blockwise_ref, quantize_rhs_blockwise
from oracle.fp8 import encode_fp8
from oracle.gmm import gmm_fwd_ref, row_scales
from oracle.quant import qmax_of, quantize_rhs_per_channel
from oracle.swiglu import swiglu_fp8_subchannel_ref
from tests.gpu_util import gen, gs_tensor, sync
from tests.parity import (TOL, U, assert_fp8_codes_in_band, assert_rounding_bound,
                          group_rel_err, group_row_ranges, magnitudes, swiglu_h_bound, to_np)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_swiglu_fp8_subchannel_and_down_projection(lib, fmt):
    sizes = [0, 300, 5, 0, 457, 130]
    G, M, K, I, H = len(sizes), sum(sizes), 256, 384, 512
    x, xb = gen((M, K), 1.0, 531)
    w, wb = gen((G, K, 2 * I), 0.02, 532)
    wd, wdb = gen((G, I, H), 0.02, 533)  # down projection [G, I, hidden]
    gs = gs_tensor(sizes)
    wq, ws = lib.gmm_quantize_rhs(w, "e4m3", 0, "nk")
    xq, sx = lib.gmm_quantize(x, "e4m3", "dynamic")
    h_codes, h_scales, gu = lib.gmm_fwd_swiglu_fp8_subchannel(xq, wq, ws, gs, h_format=fmt,
                                                              lhs_scales=sx, gu=True)
    plain = lib.gmm_fwd(xq, wq, ws, gs, lhs_scales=sx)
    sync()
    assert tuple(h_codes.shape) == (M, I) and tuple(h_scales.shape) == (M, I // 128)
    assert torch.equal(gu.view(torch.int16), plain.view(torch.int16))
    # the oracle's products, h, codes and scales
    a_codes, s_blk = ops.quantize_operand(xb, "e4m3", "dynamic")
    b_codes, b_s = quantize_rhs_per_channel(wb, "e4m3", "n")
    sa = row_scales(s_blk, M)
    R = gmm_fwd_ref(a_codes, "e4m3", sa, b_codes, "e4m3", b_s, sizes)
    absR = gmm_fwd_ref(magnitudes(a_codes), "e4m3", sa, magnitudes(b_codes), "e4m3", b_s, sizes)
    _, _, h_ref = swiglu_fp8_subchannel_ref(R, I, fmt)
    h, dh = swiglu_h_bound(R, absR, K, I)
    live = np.concatenate([np.arange(lo, hi) for lo, hi in group_row_ranges(sizes)])
    codes, scales = to_np(h_codes)[live], to_np(h_scales)[live]
    h, dh, h_ref = h[live], dh[live], h_ref[live]
    # scales: the block abs-max of a kernel h inside the band, over qmax, rounded
    qmax = qmax_of(fmt)
    habs = np.abs(h).reshape(len(live), I // 128, 128)
    band = dh.reshape(len(live), I // 128, 128)
    lo = np.max(np.maximum(habs - band, 0.0), axis=2) / qmax
    hi = np.max(habs + band, axis=2) / qmax
    assert np.all((scales >= lo * (1 - 2 * U)) & (scales <= hi * (1 + 2 * U)))
    assert np.all(scales[:, :][habs.max(axis=2) > 0] > 0)
    # codes: in the band of h under the kernel's own scales, and nearly all equal to the
    # oracle's h quantized under those scales (the recipe of swiglu_fp8_subchannel_ref)
    s_el = np.repeat(scales, 128, axis=1)
    with np.errstate(divide="ignore"):
        inv = np.where(s_el == 0, np.float32(0), np.float32(1.0) / s_el).astype(np.float32)
    ref_codes = encode_fp8(np.clip((h_ref * inv).astype(np.float32), -qmax, qmax), fmt)
    diff, amb = assert_fp8_codes_in_band(codes, h, dh, s_el, fmt, ref_codes, min_exact=0.99)
    print(f"{fmt}: codes differing from the oracle's h under the kernel's scales {diff:.2e} "
          f"(bands spanning two codes {amb:.2e})", flush=True)
    # the down projection on the kernel's codes and scales, block-wise (bk = 128)
    wdq, wds = lib.gmm_quantize_rhs_blockwise(wd, 128, "e4m3", "nk")
    y = lib.gmm_fwd_blockwise(h_codes, h_scales, wdq, wds, gs, 128, lhs_format=fmt,
                              out_dtype=torch.float32)
    sync()
    bd, bds = quantize_rhs_blockwise(wdb, "e4m3", 128)
    assert np.array_equal(to_np(wds).view(np.uint32), bds.view(np.uint32))
    hs_all = to_np(h_scales)
    hc_all = to_np(h_codes)
    Ry = gmm_fwd_blockwise_ref(hc_all, fmt, hs_all, bd, "e4m3", bds, sizes, 128)
    absY = gmm_fwd_blockwise_ref(magnitudes(hc_all), fmt, hs_all, magnitudes(bd), "e4m3", bds,
                                 sizes, 128)
    Y = to_np(y)
    ranges = group_row_ranges(sizes)
    assert group_rel_err(Y, Ry, ranges) <= TOL
    Yl, Rl, Al = Y[live], Ry[live], absY[live]
    assert_rounding_bound(Yl, Rl, Al, I)
