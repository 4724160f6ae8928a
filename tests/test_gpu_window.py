"""GPU parity of the local-expert window (gmm_fwd_local, gmm_dlhs_local, tgmm_drhs_local)
against the oracle: rows of the window's experts as the plain products compute them, the
other rows zero, tgmm slabs of the local experts; windows that start and end anywhere,
hold empty experts or only an empty expert."""

import numpy as np
import pytest
import torch

import oracle.ops as ops
from oracle.gmm import gmm_dlhs_local_ref, gmm_fwd_local_ref, group_offsets, row_scales, tgmm_local_ref
from oracle.quant import quantize_rhs_per_channel
from tests.gpu_util import gen, gs_tensor, sync
from tests.parity import TOL, assert_bf16_close, group_rel_err, slab_rel_err, to_np

pytestmark = pytest.mark.gpu

SIZES = [130, 0, 301, 1, 268, 0, 77, 500]
WINDOWS = [(0, 8), (2, 3), (7, 1), (1, 1), (5, 2), (0, 1)]


@pytest.fixture(scope="module")
def problem():
    G, M, K, N = len(SIZES), sum(SIZES), 256, 384
    x, xb = gen((M, K), 1.0, 601)
    w, wb = gen((G, K, N), 0.02, 602)
    grad, gb = gen((M, N), 1e-3, 603)
    return dict(G=G, M=M, K=K, N=N, x=x, xb=xb, w=w, wb=wb, grad=grad, gb=gb)


def window_ranges(a, b):
    off = group_offsets(SIZES)
    return [(int(off[g]), int(off[g + 1])) for g in range(a, a + b)]


def outside_rows(M, a, b):
    off = group_offsets(SIZES)
    mask = np.ones(M, bool)
    mask[off[a]:off[a + b]] = False
    return mask


@pytest.mark.parametrize("a,b", WINDOWS)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_fwd_local(lib, problem, a, b, out_dtype):
    d = problem
    codes, scales = lib.gmm_quantize_rhs(d["w"], "e4m3", 0, "nk")
    out = lib.gmm_fwd_local(d["x"], codes[a:a + b].contiguous(), scales[a:a + b].contiguous(),
                            gs_tensor(SIZES), a, out_dtype=out_dtype)
    sync()
    c_ref, s_ref = quantize_rhs_per_channel(d["wb"], "e4m3", "n")
    aq, s_blk = ops.quantize_operand(d["xb"], "e4m3", "dynamic")
    R = gmm_fwd_local_ref(aq, "e4m3", row_scales(s_blk, d["M"]), c_ref[a:a + b], "e4m3",
                          s_ref[a:a + b], SIZES, a)
    Y = to_np(out)
    assert not Y[outside_rows(d["M"], a, b)].any()
    if out_dtype == torch.float32:
        assert group_rel_err(Y, R, window_ranges(a, b)) <= TOL
    else:
        ranges = window_ranges(a, b)
        lo, hi = ranges[0][0], ranges[-1][1]
        if hi > lo:  # the window's rows only
            assert_bf16_close(Y[lo:hi], R[lo:hi], [(r0 - lo, r1 - lo) for r0, r1 in ranges])


@pytest.mark.parametrize("a,b", WINDOWS)
def test_dlhs_local(lib, problem, a, b):
    d = problem
    codes, scales = lib.gmm_quantize_rhs(d["w"], "e4m3", 1, "kn")
    out = lib.gmm_dlhs_local(d["grad"], codes[a:a + b].contiguous(), scales[a:a + b].contiguous(),
                             gs_tensor(SIZES), a, out_dtype=torch.float32)
    sync()
    c_ref, s_ref = quantize_rhs_per_channel(d["wb"], "e4m3", "k")
    gq, s_blk = ops.quantize_operand(d["gb"], "e5m2", "dynamic")
    R = gmm_dlhs_local_ref(gq, "e5m2", row_scales(s_blk, d["M"]), c_ref[a:a + b], "e4m3",
                           s_ref[a:a + b], SIZES, a)
    Y = to_np(out)
    assert not Y[outside_rows(d["M"], a, b)].any()
    assert group_rel_err(Y, R, window_ranges(a, b)) <= TOL


@pytest.mark.parametrize("a,b", WINDOWS)
def test_tgmm_local(lib, problem, a, b):
    d = problem
    out = lib.tgmm_drhs_local(d["x"], d["grad"], gs_tensor(SIZES), a, b,
                              out_dtype=torch.float32)
    sync()
    assert tuple(out.shape) == (b, d["K"], d["N"])
    aq, sa = ops.quantize_operand(d["xb"], "e4m3", "dynamic")
    gq, sg = ops.quantize_operand(d["gb"], "e5m2", "dynamic")
    R = tgmm_local_ref(aq, "e4m3", sa, gq, "e5m2", sg, SIZES, a, b)
    assert slab_rel_err(to_np(out), R) <= TOL
    for j in range(b):  # empty local experts: +0.0 slabs
        if SIZES[a + j] == 0:
            assert (to_np(out)[j].view(np.uint32) == 0).all()


@pytest.mark.parametrize("a,b", [(2, 3), (7, 1)])
def test_tgmm_local_bf16_is_the_rounded_f32(lib, problem, a, b):
    """The window's bf16 slabs are the RNE of its f32 slabs, bit for bit."""
    from oracle.fp8 import f32_to_bf16_bits

    d = problem
    o32 = lib.tgmm_drhs_local(d["x"], d["grad"], gs_tensor(SIZES), a, b, out_dtype=torch.float32)
    o16 = lib.tgmm_drhs_local(d["x"], d["grad"], gs_tensor(SIZES), a, b)
    sync()
    assert np.array_equal(to_np(o16), f32_to_bf16_bits(to_np(o32)))
