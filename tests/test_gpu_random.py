"""Seeded random sweep of the three products against the oracle: group counts, group sizes
(empty groups anywhere, one-row groups), K and N tails, both weight layouts, static and
dynamic recipes, bf16 operands quantized in the call and fp8 codes quantized before, the
in-kernel (fused) and quantize-once routes, f32 outputs held to the per-group metric."""

import numpy as np
import pytest
import torch

import oracle.ops as ops
from oracle.quant import quantize_rhs_per_channel
from tests.gpu_util import gen, gs_tensor, sync
from oracle.gmm import gmm_dlhs_ref, gmm_fwd_ref, row_scales, tgmm_ref
from tests.parity import (TOL, assert_rounding_bound, group_rel_err, group_row_ranges,
                          magnitudes, slab_rel_err, to_np)

pytestmark = pytest.mark.gpu

S = float(np.float32(4.0) / np.float32(448.0))


def draw(i):
    """Configuration i: (sizes, K, N, layout, scaling, kind, fused)."""
    rng = np.random.default_rng(1000 + i)
    G = int(rng.integers(1, 13))
    M = int(rng.integers(0, 1300))
    w = rng.random(G) ** 3 + 1e-3
    sizes = rng.multinomial(M, w / w.sum()) if M else np.zeros(G, np.int64)
    sizes[rng.random(G) < 0.2] = 0  # some experts empty
    if G > 1 and M and rng.random() < 0.5:
        sizes[int(rng.integers(0, G))] = 1  # a one-row expert
    K = int(rng.choice([128, 256, 384, 640]))
    N = int(rng.choice([128, 256, 384, 768]))
    layout = str(rng.choice(["nk", "kn"]))
    scaling = str(rng.choice(["static", "dynamic"]))
    kind = str(rng.choice(["bf16", "codes"]))
    fused = bool(rng.random() < 0.3)
    return [int(v) for v in sizes], K, N, layout, scaling, kind, fused


@pytest.mark.parametrize("i", range(64))
def test_random_fwd_dlhs_tgmm(lib, i):
    sizes, K, N, layout, scaling, kind, fused = draw(i)
    G, M = len(sizes), sum(sizes)
    print(f"config {i}: G={G} M={M} K={K} N={N} {layout} {scaling} {kind} fused={fused} sizes={sizes}",
          flush=True)
    x, xb = gen((M, K), 1.0, 2000 + i)
    w, wb = gen((G, K, N), 0.02, 3000 + i)
    gr, grb = gen((M, N), 1e-3, 4000 + i)
    gs = gs_tensor(sizes)
    ranges = group_row_ranges(sizes)
    kw = dict(lhs_scaling=scaling, static_scale=S if scaling == "static" else None)
    gkw = dict(grad_scaling=scaling, static_scale=S if scaling == "static" else None)

    # forward
    wq, ws = lib.gmm_quantize_rhs(w, "e4m3", 0, layout)
    c_ref, s_ref = quantize_rhs_per_channel(wb, "e4m3", "n")
    if kind == "codes" and M:
        xq, sx = lib.gmm_quantize(x, "e4m3", scaling, static_scale=kw["static_scale"])
        lhs = xq
        if scaling == "dynamic":
            kw["lhs_scales"] = sx
    else:
        lhs = x
    out = lib.gmm_fwd(lhs, wq, ws, gs, rhs_layout=layout, out_dtype=torch.float32,
                      fused=fused and kind == "bf16", **kw)
    R, a_codes, a_s = ops.fwd(xb, c_ref, s_ref, np.asarray(sizes), "e4m3", scaling,
                              np.float32(S), "e4m3", "f32")
    if M:
        assert group_rel_err(to_np(out), R, ranges) <= TOL
        absR = gmm_fwd_ref(magnitudes(a_codes), "e4m3", row_scales(a_s, M), magnitudes(c_ref),
                           "e4m3", s_ref, np.asarray(sizes))
        assert_rounding_bound(to_np(out), R, absR, K)

    # dlhs (the rhs quantized per k)
    wk, sk = lib.gmm_quantize_rhs(w, "e4m3", 1, "kn" if layout == "nk" else "nk")
    ck_ref, sk_ref = quantize_rhs_per_channel(wb, "e4m3", "k")
    if kind == "codes" and M:
        gq, sg = lib.gmm_quantize(gr, "e5m2", scaling, static_scale=gkw["static_scale"])
        grad = gq
        if scaling == "dynamic":
            gkw["grad_scales"] = sg
    else:
        grad = gr
    dl = lib.gmm_dlhs(grad, wk, sk, gs, rhs_layout="kn" if layout == "nk" else "nk",
                      out_dtype=torch.float32, fused=fused and kind == "bf16", **gkw)
    Rd, g_codes, g_s = ops.dlhs(grb, ck_ref, sk_ref, np.asarray(sizes), "e5m2", scaling,
                                np.float32(S), "e4m3", "f32")
    if M:
        assert group_rel_err(to_np(dl), Rd, group_row_ranges(sizes)) <= TOL
        absD = gmm_dlhs_ref(magnitudes(g_codes), "e5m2", row_scales(g_s, M), magnitudes(ck_ref),
                            "e4m3", sk_ref, np.asarray(sizes))
        assert_rounding_bound(to_np(dl), Rd, absD, N)

    # tgmm (bf16 operands, or the codes just made)
    if kind == "codes" and M:
        tk = dict(lhs_scaling=scaling, grad_scaling=scaling)
        if scaling == "static":
            tk.update(lhs_static_scale=S, grad_static_scale=S)
        else:
            tk.update(lhs_scales=sx, grad_scales=sg)
        dr = lib.tgmm_drhs(xq, gq, gs, out_dtype=torch.float32, **tk)
    else:
        tk = dict(lhs_scaling=scaling, grad_scaling=scaling)
        if scaling == "static":
            tk.update(lhs_static_scale=S, grad_static_scale=S)
        dr = lib.tgmm_drhs(x, gr, gs, out_dtype=torch.float32, **tk)
    sync()
    Rt, _, _ = ops.tgmm(xb, grb, np.asarray(sizes), "e4m3", scaling, np.float32(S), "e5m2",
                        scaling, np.float32(S), "f32")
    assert slab_rel_err(to_np(dr), Rt) <= TOL
    if M:
        absT = tgmm_ref(magnitudes(a_codes), "e4m3", a_s, magnitudes(g_codes), "e5m2", g_s,
                        np.asarray(sizes))
        assert_rounding_bound(to_np(dr), Rt, absT, np.asarray(sizes)[:, None, None])
    for g in range(G):  # empty experts: +0.0 slabs
        if sizes[g] == 0:
            assert (to_np(dr)[g].view(np.uint32) == 0).all()


@pytest.mark.parametrize("i", range(16))
def test_random_windows(lib, i):
    """Random local-expert windows of random groupings: fwd, dlhs and tgmm (dynamic bf16
    operands) against the oracle's windows; rows outside the window are zero."""
    from oracle.gmm import gmm_dlhs_local_ref, gmm_fwd_local_ref, group_offsets, tgmm_local_ref

    rng = np.random.default_rng(5000 + i)
    G = int(rng.integers(2, 20))
    sizes = [int(v) for v in rng.multinomial(int(rng.integers(1, 1500)), np.ones(G) / G)]
    sizes = [0 if rng.random() < 0.2 else v for v in sizes]
    M = sum(sizes)
    a = int(rng.integers(0, G))
    b = int(rng.integers(1, G - a + 1))
    K, N = int(rng.choice([128, 384])), int(rng.choice([256, 640]))
    print(f"window config {i}: G={G} sizes={sizes} window=({a}, {b}) K={K} N={N}", flush=True)
    x, xb = gen((M, K), 1.0, 6000 + i)
    w, wb = gen((G, K, N), 0.02, 7000 + i)
    gr, grb = gen((M, N), 1e-3, 8000 + i)
    gs = gs_tensor(sizes)
    wq, ws = lib.gmm_quantize_rhs(w[a:a + b].contiguous(), "e4m3", 0, "nk")
    out = lib.gmm_fwd_local(x, wq, ws, gs, a, out_dtype=torch.float32)
    wk, sk = lib.gmm_quantize_rhs(w[a:a + b].contiguous(), "e4m3", 1, "kn")
    dl = lib.gmm_dlhs_local(gr, wk, sk, gs, a, out_dtype=torch.float32)
    dr = lib.tgmm_drhs_local(x, gr, gs, a, b, out_dtype=torch.float32)
    sync()
    aq, sa = ops.quantize_operand(xb, "e4m3", "dynamic")
    gq, sg = ops.quantize_operand(grb, "e5m2", "dynamic")
    c_ref, s_ref = quantize_rhs_per_channel(wb[a:a + b], "e4m3", "n")
    ck_ref, sk_ref = quantize_rhs_per_channel(wb[a:a + b], "e4m3", "k")
    off = group_offsets(sizes)
    win = [(int(off[g]), int(off[g + 1])) for g in range(a, a + b)]
    outside = np.ones(M, bool)
    outside[off[a]:off[a + b]] = False
    R = gmm_fwd_local_ref(aq, "e4m3", np.repeat(sa, 128)[:M], c_ref, "e4m3", s_ref, sizes, a)
    Y = to_np(out)
    assert not Y[outside].any() and group_rel_err(Y, R, win) <= TOL
    Rd = gmm_dlhs_local_ref(gq, "e5m2", np.repeat(sg, 128)[:M], ck_ref, "e4m3", sk_ref, sizes, a)
    D = to_np(dl)
    assert not D[outside].any() and group_rel_err(D, Rd, win) <= TOL
    Rt = tgmm_local_ref(aq, "e4m3", sa, gq, "e5m2", sg, sizes, a, b)
    assert slab_rel_err(to_np(dr), Rt) <= TOL


@pytest.mark.parametrize("i", range(12))
def test_random_blockwise(lib, i):
    """Random shapes and block sizes of the block-wise forward against the oracle."""
    from oracle.blockwise import gmm_fwd_blockwise_ref, quantize_rhs_blockwise, quantize_subchannel

    rng = np.random.default_rng(9000 + i)
    G = int(rng.integers(1, 9))
    sizes = [int(v) for v in rng.multinomial(int(rng.integers(0, 900)), np.ones(G) / G)]
    M = sum(sizes)
    bk = int(rng.choice([128, 256, 512]))
    K = bk * int(rng.integers(1, 5))
    N = 128 * int(rng.integers(1, 5))
    fmt = str(rng.choice(["e4m3", "e5m2"]))
    print(f"block-wise config {i}: sizes={sizes} K={K} N={N} bk={bk} {fmt}", flush=True)
    x, xb = gen((M, K), 1.0, 9100 + i)
    w, wb = gen((G, K, N), 0.02, 9200 + i)
    codes, s = lib.gmm_quantize_subchannel(x, bk, fmt)
    wq, ws = lib.gmm_quantize_rhs_blockwise(w, bk)
    out = lib.gmm_fwd_blockwise(codes, s, wq, ws, gs_tensor(sizes), bk, lhs_format=fmt,
                                out_dtype=torch.float32)
    sync()
    if M == 0:
        return
    c_ref, s_ref = quantize_subchannel(xb, fmt, bk)
    wc_ref, ws_ref = quantize_rhs_blockwise(wb, "e4m3", bk)
    R = gmm_fwd_blockwise_ref(c_ref, fmt, s_ref, wc_ref, "e4m3", ws_ref, sizes, bk)
    assert group_rel_err(to_np(out), R, group_row_ranges(sizes)) <= TOL


@pytest.mark.parametrize("i", range(16))
def test_random_routing(lib, i):
    """Random routings: permute (indices, group sizes, gathered rows) and the weighted
    combine, bit for bit against the oracle."""
    from oracle.fp8 import bf16_bits_to_f32
    from oracle.route import gather_rows_ref, permute_ref, unpermute_ref

    rng = np.random.default_rng(9500 + i)
    T = int(rng.integers(0, 3000))
    k = int(rng.integers(1, 17))
    G = int(rng.integers(1, 300))
    H = 8 * int(rng.integers(1, 300))
    ids = rng.integers(-1, G + 2, (T, k)).astype(np.int32)  # repeats and dropped ids
    print(f"routing config {i}: T={T} k={k} G={G} H={H}", flush=True)
    x, xb = gen((T, H), 1.0, 9600 + i)
    idt = torch.as_tensor(ids, device=x.device)
    xp, gs, ros, sor = lib.gmm_permute(idt, G, x)
    wts = rng.random((T, k)).astype(np.float32)
    y, yb = gen((T * k, H), 1.0, 9700 + i)
    out = lib.gmm_unpermute(y, ros, torch.as_tensor(wts, device=x.device))
    sync()
    gs_r, ros_r, sor_r = permute_ref(ids, G)
    assert np.array_equal(to_np(gs), gs_r) and np.array_equal(to_np(ros), ros_r)
    assert np.array_equal(to_np(sor), sor_r)
    assert np.array_equal(to_np(xp), gather_rows_ref(xb, sor_r, k))
    _, bits = unpermute_ref(bf16_bits_to_f32(yb), ros_r, wts)
    assert np.array_equal(to_np(out), bits)
