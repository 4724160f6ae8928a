"""GPU parity of gmm_fwd_swiglu_fp8_subchannel: h of the merged gate|up forward as fp8
codes under dynamic scales per row and 128-channel block, taken in the product's
epilogue, and the down projection on them through gmm_fwd_blockwise (bk = 128).

The kernel's h differs from the oracle's by the rounding of the products' sums and of
the SwiGLU (the band of swiglu_h_bound), so its block abs-max, and with it the rounded
scale, is usually a few ulps off the oracle's: the scales are held to that band, the
codes to the band of h under the kernel's own scales and, nearly all, to the oracle's h
quantized under those scales.  The down projection on the kernel's codes is held to the
oracle's on the oracle's own codes and scales, within the rounding bound plus the
difference of the two dequantized h carried through |w|."""

import numpy as np
import pytest
import torch

import oracle.ops as ops
from oracle.blockwise import gmm_fwd_blockwise_ref, quantize_rhs_blockwise
from oracle.fp8 import decode_fp8, encode_fp8
from oracle.gmm import gmm_fwd_ref, row_scales
from oracle.quant import qmax_of, quantize_rhs_per_channel
from oracle.swiglu import swiglu_fp8_subchannel_ref
from tests.gpu_util import gen, gs_tensor, sync
from tests.parity import (MFMA_TRUNC, U, assert_fp8_codes_in_band, group_row_ranges,
                          magnitudes, swiglu_h_bound, to_np)

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
    # the down projection (block-wise, bk = 128) on the kernel's codes and scales, against
    # the oracle's on its own codes and scales, with the difference of the two dequantized
    # h (where codes or scales differ) carried through |w| as slack
    wdq, wds = lib.gmm_quantize_rhs_blockwise(wd, 128, "e4m3", "nk")
    y = lib.gmm_fwd_blockwise(h_codes, h_scales, wdq, wds, gs, 128, lhs_format=fmt,
                              out_dtype=torch.float32)
    sync()
    bd, bds = quantize_rhs_blockwise(wdb, "e4m3", 128)
    assert np.array_equal(to_np(wds).view(np.uint32), bds.view(np.uint32))
    c_ref, s_ref, _ = swiglu_fp8_subchannel_ref(R, I, fmt)
    Ry = gmm_fwd_blockwise_ref(c_ref, fmt, s_ref, bd, "e4m3", bds, sizes, 128)
    absY = gmm_fwd_blockwise_ref(magnitudes(c_ref), fmt, s_ref, magnitudes(bd), "e4m3", bds,
                                 sizes, 128)
    deq = lambda c, sc: decode_fp8(c, fmt).astype(np.float64) * np.repeat(sc, 128, axis=1)
    step = np.abs(deq(to_np(h_codes), to_np(h_scales)) - deq(c_ref, s_ref))
    wabs = np.abs(decode_fp8(bd, "e4m3").astype(np.float64)) * np.repeat(bds, 128, axis=1)
    Y = to_np(y).astype(np.float64)
    ranges = group_row_ranges(sizes)
    for g, (lo, hi) in enumerate(ranges):
        if hi == lo:
            continue
        allow = ((MFMA_TRUNC + 2.0 * (I + 8.0) * U) * absY[lo:hi] + 4.0 * U * np.abs(Ry[lo:hi])
                 + 2.0 ** -126 + step[lo:hi] @ wabs[g] * (1 + 1e-6))
        assert np.all(np.abs(Y[lo:hi] - Ry[lo:hi]) <= allow), g


def test_swiglu_subchannel_full_size_sampled(lib):
    """gmm_fwd_swiglu_fp8_subchannel at the SwiGLU block shape (G=64, M=65536, K=2048,
    I=1408) as the benchmark launches it (e4m3 lhs codes with dynamic 128-row scales, e4m3
    h): sampled rows of 8 experts and 3 of the 11 channel blocks of h, whose scales need
    the block's 128 gate and 128 up columns only, against the oracle (scales and codes in
    their bands, the codes of the oracle's h under the kernel's scales nearly all equal)."""
    from oracle.fp8 import bf16_bits_to_f32
    from oracle.quant import quantize_with_inv
    from synth.workloads import WORKLOADS, bf16_to_bits, normal_bf16
    from tests.gpu_util import DEV
    from tests.test_gpu_full import dynamic_block_scales, sample_rows

    wl = WORKLOADS["moe_swiglu"]
    G, M, K, I = wl.G, wl.M, wl.K, wl.extra["intermediate"]
    sizes = np.asarray(wl.group_sizes())
    seed = wl.seed * 100 + 40
    x = normal_bf16((M, K), 1.0, seed, DEV)
    w = normal_bf16((G, K, 2 * I), 0.02, seed + 1, DEV)
    gs = gs_tensor(sizes)
    wq, ws = lib.gmm_quantize_rhs(w, "e4m3", 0, "nk")
    xq, sx = lib.gmm_quantize(x, "e4m3", "dynamic")
    h_codes, h_scales = lib.gmm_fwd_swiglu_fp8_subchannel(xq, wq, ws, gs, h_format="e4m3",
                                                          lhs_scales=sx)
    sync()
    # experts: the largest, the smallest non-empty and six more spread over the order
    order = np.argsort(-sizes, kind="stable")
    nonempty = [int(g) for g in order if sizes[g] > 0]
    sel = sorted(set(nonempty[i] for i in np.linspace(0, len(nonempty) - 1, 8).astype(int)))
    rng = np.random.default_rng(23)
    off = np.concatenate([[0], np.cumsum(sizes)])
    all_rows = sample_rows(list(sizes), rng)
    rows = np.array([r for r in all_rows if any(off[g] <= r < off[g + 1] for g in sel)], np.int64)
    sub = np.array([int(((rows >= off[g]) & (rows < off[g + 1])).sum()) for g in sel], np.int32)
    blocks = [0, I // 256, I // 128 - 1]  # first, middle and last 128-channel blocks
    ch = np.concatenate([np.arange(128 * b, 128 * b + 128) for b in blocks])
    cols = np.concatenate([ch, I + ch])  # gate then up columns of those channels
    # the oracle: lhs codes of the sampled rows with their blocks' dynamic scales over
    # the whole tensor, the per-channel codes of the sampled experts' columns, the
    # products, h and its bands
    xb = bf16_to_bits(x)
    s_blk, inv_blk = dynamic_block_scales(xb, "e4m3")
    assert np.array_equal(to_np(sx).view(np.uint32), s_blk.view(np.uint32))
    a_codes = quantize_with_inv(bf16_bits_to_f32(xb[rows]), inv_blk[rows // 128], "e4m3")
    sa = s_blk[rows // 128]
    gi, ci = torch.as_tensor(sel, device=DEV), torch.as_tensor(cols, device=DEV)
    b_codes, b_s = quantize_rhs_per_channel(bf16_to_bits(w[gi][:, :, ci]), "e4m3", "n")
    R = gmm_fwd_ref(a_codes, "e4m3", sa, b_codes, "e4m3", b_s, sub)
    absR = gmm_fwd_ref(magnitudes(a_codes), "e4m3", sa, magnitudes(b_codes), "e4m3", b_s, sub)
    Is = len(ch)
    h, dh = swiglu_h_bound(R, absR, K, Is)
    _, _, h_ref = swiglu_fp8_subchannel_ref(R, Is, "e4m3")
    ri = torch.as_tensor(rows, device=DEV)
    codes = to_np(h_codes[ri])[:, ch]
    scales = to_np(h_scales[ri])[:, blocks]
    qmax = qmax_of("e4m3")
    habs = np.abs(h).reshape(len(rows), len(blocks), 128)
    band = dh.reshape(len(rows), len(blocks), 128)
    lo = np.max(np.maximum(habs - band, 0.0), axis=2) / qmax
    hi = np.max(habs + band, axis=2) / qmax
    assert np.all((scales >= lo * (1 - 2 * U)) & (scales <= hi * (1 + 2 * U)))
    s_el = np.repeat(scales, 128, axis=1)
    with np.errstate(divide="ignore"):
        inv = np.where(s_el == 0, np.float32(0), np.float32(1.0) / s_el).astype(np.float32)
    ref_codes = encode_fp8(np.clip((h_ref * inv).astype(np.float32), -qmax, qmax), "e4m3")
    diff, amb = assert_fp8_codes_in_band(codes, h, dh, s_el, "e4m3", ref_codes, min_exact=0.99)
    print(f"{len(rows)} rows of {len(sel)} experts: codes differing from the oracle's h under "
          f"the kernel's scales {diff:.2e} (bands spanning two codes {amb:.2e})", flush=True)

