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
from tests.parity import TOL, group_rel_err, group_row_ranges, slab_rel_err, to_np

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
    R, _, _ = ops.fwd(xb, c_ref, s_ref, np.asarray(sizes), "e4m3", scaling,
                             np.float32(S), "e4m3", "f32")
    if M:
        assert group_rel_err(to_np(out), R, ranges) <= TOL

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
    Rd, _, _ = ops.dlhs(grb, ck_ref, sk_ref, np.asarray(sizes), "e5m2", scaling,
                                np.float32(S), "e4m3", "f32")
    if M:
        assert group_rel_err(to_np(dl), Rd, group_row_ranges(sizes)) <= TOL

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
    for g in range(G):  # empty experts: +0.0 slabs
        if sizes[g] == 0:
            assert (to_np(dr)[g].view(np.uint32) == 0).all()
