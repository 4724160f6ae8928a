"""gmm_fwd_noalloc, the forward that allocates nothing (its scratch is a device array of
the library), against gmm_fwd with a workspace: the same codes, scales and outputs, bit for
bit, on two calls in a row (the second smaller, so that scratch left by the first cannot
leak into it), with and without the block scales handed back."""

import numpy as np
import pytest
import torch

from tests.gpu_util import gen, gs_tensor, sync

pytestmark = pytest.mark.gpu

S_4_448 = float(np.float32(4.0) / np.float32(448.0))


def _problem(lib, sizes, K, N, seed):
    M, G = int(sum(sizes)), len(sizes)
    x, _ = gen((M, K), 1.0, seed)
    w, _ = gen((G, K, N), 0.02, seed + 1)
    wq, ws = lib.gmm_quantize_rhs(w, "e4m3", 0, "nk")
    return x, wq, ws, gs_tensor(sizes)


def _same(a, b):
    view = torch.int32 if a.dtype == torch.float32 else torch.int16
    return torch.equal(a.view(view), b.view(view))


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_noalloc_equals_gmm_fwd_two_calls(lib, out_dtype):
    # call 1: 1000 rows, an empty group in the middle, 4 output tiles (gmm_fwd quantizes
    # the lhs once into its workspace; the allocation-free call quantizes in-kernel)
    x, wq, ws, gs = _problem(lib, [300, 0, 700], 256, 1024, 901)
    ref, s_ref = lib.gmm_fwd(x, wq, ws, gs, out_dtype=out_dtype, return_scales=True)
    s = torch.full_like(s_ref, float("nan"))
    out = torch.full_like(ref, float("nan"))
    lib.gmm_fwd_noalloc(x, wq, ws, gs, out_dtype=out_dtype, lhs_scales=s, out=out)
    sync()
    assert _same(out, ref)
    assert torch.equal(s.view(torch.int32), s_ref.view(torch.int32))
    # call 2: fewer rows and columns, scales left in the library's scratch
    x2, wq2, ws2, gs2 = _problem(lib, [50, 0, 150, 3], 128, 256, 902)
    ref2 = lib.gmm_fwd(x2, wq2, ws2, gs2, out_dtype=out_dtype)
    out2 = lib.gmm_fwd_noalloc(x2, wq2, ws2, gs2, out_dtype=out_dtype)
    sync()
    assert _same(out2, ref2)
    # and the first problem again after the smaller one
    out3 = lib.gmm_fwd_noalloc(x, wq, ws, gs, out_dtype=out_dtype)
    sync()
    assert _same(out3, ref)


def test_noalloc_static_and_codes_recipes(lib):
    x, wq, ws, gs = _problem(lib, [128, 0, 372], 256, 512, 903)
    ref = lib.gmm_fwd(x, wq, ws, gs, lhs_scaling="static", static_scale=S_4_448)
    out = lib.gmm_fwd_noalloc(x, wq, ws, gs, lhs_scaling="static", static_scale=S_4_448)
    xq, sx = lib.gmm_quantize(x, "e4m3", "dynamic")
    ref_q = lib.gmm_fwd(xq, wq, ws, gs, lhs_scales=sx)
    out_q = lib.gmm_fwd_noalloc(xq, wq, ws, gs, lhs_scales=sx)
    sync()
    assert _same(out, ref)
    assert _same(out_q, ref_q)


def test_noalloc_rejects_more_rows_than_its_scratch(lib):
    import ctypes

    import fp8_grouped_gemm_ragged_amd as g

    op = g.Operand(g.KIND_BF16, g.E4M3, g.DYNAMIC, 0.0)
    M = (1 << 20) + 1  # GMM_NOALLOC_MAX_ROWS + 1: rejected before anything is read
    st = g.load().gmm_fwd_noalloc(ctypes.byref(op), g.E4M3, g.RHS_NK, g.OUT_BF16, M, 128, 128, 1,
                                  ctypes.c_void_p(256), None, ctypes.c_void_p(512),
                                  ctypes.c_void_p(768), ctypes.c_void_p(1024),
                                  ctypes.c_void_p(1280), None)
    assert st == 5  # GMM_ERR_WORKSPACE
