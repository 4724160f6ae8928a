"""The Python binding rejects buffers whose shapes differ from what the call reads or
writes, before anything is enqueued (the C ABI sees only pointers)."""

import numpy as np
import pytest
import torch

from tests.gpu_util import DEV, gs_tensor

pytestmark = pytest.mark.gpu

S = float(np.float32(4.0) / np.float32(448.0))


def _fwd_inputs(M=300, K=256, N=384, G=3):
    x = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((G, N, K), dtype=torch.uint8, device=DEV)
    ws = torch.ones((G, N), dtype=torch.float32, device=DEV)
    gs = gs_tensor([100, 0, 200])
    return x, w, ws, gs


def test_gemm_rejects_bad_shapes(lib):
    x, w, ws, gs = _fwd_inputs()
    kw = dict(lhs_scaling="static", static_scale=S)
    with pytest.raises(ValueError, match="out"):
        lib.gmm_fwd(x, w, ws, gs, out=torch.empty((299, 384), dtype=torch.bfloat16, device=DEV), **kw)
    with pytest.raises(ValueError, match="out"):
        lib.gmm_fwd(x, w, ws, gs, out=torch.empty((300, 256), dtype=torch.bfloat16, device=DEV), **kw)
    with pytest.raises(ValueError, match="rhs_scales"):
        lib.gmm_fwd(x, w, ws[:, :256].contiguous(), gs, **kw)
    with pytest.raises(ValueError, match="rhs_scales"):
        lib.gmm_fwd(x, w, ws[:2].contiguous(), gs, **kw)
    with pytest.raises(ValueError, match="group_sizes"):
        lib.gmm_fwd(x, w, ws, gs_tensor([100, 200]), **kw)
    with pytest.raises(ValueError, match="group_sizes"):
        lib.gmm_fwd(x, w, ws, gs_tensor([100, 0, 100, 100]), **kw)
    # block scales of a dynamic recipe: at least ceil(M / 128) of them
    with pytest.raises(ValueError, match="block scales"):
        lib.gmm_fwd(x, w, ws, gs, lhs_scaling="dynamic",
                    lhs_scales=torch.ones(2, dtype=torch.float32, device=DEV))
    xq = torch.zeros((300, 256), dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError, match="block scales"):
        lib.gmm_fwd(xq, w, ws, gs, lhs_scaling="dynamic",
                    lhs_scales=torch.ones(2, dtype=torch.float32, device=DEV))
    # dlhs: rhs_scales per output channel k, out [M, K]
    g = torch.zeros((300, 384), dtype=torch.bfloat16, device=DEV)
    wk = torch.zeros((3, 256, 384), dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError, match="rhs_scales"):
        lib.gmm_dlhs(g, wk, ws, gs, grad_scaling="static", static_scale=S)
    with pytest.raises(ValueError, match="out"):
        lib.gmm_dlhs(g, wk, torch.ones((3, 256), dtype=torch.float32, device=DEV), gs,
                     grad_scaling="static", static_scale=S,
                     out=torch.empty((300, 384), dtype=torch.bfloat16, device=DEV))


def test_local_window_rejects_bad_offsets(lib):
    x, w, ws, gs = _fwd_inputs()
    gs5 = gs_tensor([10, 100, 0, 190, 0])
    with pytest.raises(ValueError, match="window"):
        lib.gmm_fwd_local(x, w, ws, gs5, 3, lhs_scaling="static", static_scale=S)
    with pytest.raises(ValueError, match="window"):
        lib.gmm_fwd_local(x, w, ws, gs5, -1, lhs_scaling="static", static_scale=S)


def test_tgmm_rejects_bad_shapes(lib):
    x = torch.zeros((300, 256), dtype=torch.bfloat16, device=DEV)
    g = torch.zeros((300, 128), dtype=torch.bfloat16, device=DEV)
    gs = gs_tensor([100, 0, 200])
    with pytest.raises(ValueError, match="out"):
        lib.tgmm_drhs(x, g, gs, out=torch.empty((2, 256, 128), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError, match="out"):
        lib.tgmm_drhs(x, g, gs, out=torch.empty((3, 128, 256), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError, match="block scales"):
        lib.tgmm_drhs(x, g, gs, lhs_scales=torch.empty(1, dtype=torch.float32, device=DEV))
    with pytest.raises(ValueError, match="block scales"):
        lib.tgmm_drhs(x, g, gs, grad_scaling="dynamic_given",
                      grad_scales=torch.ones(2, dtype=torch.float32, device=DEV))
    with pytest.raises(ValueError, match="window"):
        lib.tgmm_drhs_local(x, g, gs, 2, 2)


def test_swiglu_and_blockwise_reject_bad_shapes(lib):
    M, K, I, G = 256, 256, 128, 2
    x = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((G, 2 * I, K), dtype=torch.uint8, device=DEV)
    ws = torch.ones((G, 2 * I), dtype=torch.float32, device=DEV)
    gs = gs_tensor([100, 156])
    kw = dict(lhs_scaling="static", static_scale=S)
    with pytest.raises(ValueError, match="out"):
        lib.gmm_fwd_swiglu(x, w, ws, gs, out=torch.empty((M, 2 * I), dtype=torch.bfloat16, device=DEV), **kw)
    with pytest.raises(ValueError, match="rhs_scales"):
        lib.gmm_fwd_swiglu(x, w, ws[:, :I].contiguous(), gs, **kw)
    with pytest.raises(ValueError, match="group_sizes"):
        lib.gmm_fwd_swiglu(x, w, ws, gs_tensor([256]), **kw)
    dh = torch.zeros((M, I), dtype=torch.bfloat16, device=DEV)
    gu = torch.zeros((M, 2 * I), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError, match="out"):
        lib.gmm_swiglu_bwd(dh, gu, out=torch.empty((M, I), dtype=torch.bfloat16, device=DEV))
    # block-wise forward: scales [M, K / bk] and [G, K / bk, N]
    xq = torch.zeros((M, K), dtype=torch.uint8, device=DEV)
    wq = torch.zeros((G, 256, K), dtype=torch.uint8, device=DEV)
    sa = torch.ones((M, K // 128), dtype=torch.float32, device=DEV)
    sb = torch.ones((G, K // 128, 256), dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError, match="lhs_scales"):
        lib.gmm_fwd_blockwise(xq, sa[:, :1].contiguous(), wq, sb, gs, 128)
    with pytest.raises(ValueError, match="rhs_scales"):
        lib.gmm_fwd_blockwise(xq, sa, wq, sb[:, :1].contiguous(), gs, 128)
    with pytest.raises(ValueError, match="out"):
        lib.gmm_fwd_blockwise(xq, sa, wq, sb, gs, 128,
                              out=torch.empty((M, 128), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError, match="group_sizes"):
        lib.gmm_fwd_blockwise(xq, sa, wq, sb, gs_tensor([256]), 128)


def test_quantize_and_unpermute_reject_bad_shapes(lib):
    x = torch.zeros((300, 256), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError, match="block scales"):
        lib.gmm_quantize(x, "e4m3", "dynamic_given", scales=torch.ones(2, dtype=torch.float32, device=DEV))
    y = torch.zeros((8, 128), dtype=torch.bfloat16, device=DEV)
    ros = torch.zeros((4, 2), dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError, match="out"):
        lib.gmm_unpermute(y, ros, out=torch.empty((8, 128), dtype=torch.bfloat16, device=DEV))
