"""GPU parity of tgmm_drhs against the oracle."""

import numpy as np
import pytest
import torch

import oracle.ops as ops
from tests.gpu_util import DEV, gen, gs_tensor, sync
from tests.parity import TOL, assert_bf16_close, slab_rel_err, to_np

pytestmark = pytest.mark.gpu

S_4_448 = float(np.float32(4.0) / np.float32(448.0))


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("lhs_scaling", ["dynamic", "static"])
def test_tgmm_ragged_medium(lib, out_dtype, lhs_scaling):
    # group boundaries off the 128-row grid, an empty group first and in the middle,
    # a group inside a single block and one spanning several blocks; K tail 640 = 2.5 x 256
    sizes = [0, 300, 5, 0, 457, 130]
    M, K, N = sum(sizes), 640, 384
    x, xb = gen((M, K), 1.0, 201)
    gr, gb = gen((M, N), 1e-3, 202)
    out, sa, sg = lib.tgmm_drhs(x, gr, gs_tensor(sizes), lhs_scaling=lhs_scaling,
                                lhs_static_scale=S_4_448, out_dtype=out_dtype,
                                return_scales=True)
    R, sa_ref, sg_ref = ops.tgmm(xb, gb, np.asarray(sizes), "e4m3", lhs_scaling,
                                 np.float32(S_4_448), "e5m2", "dynamic")
    if lhs_scaling == "dynamic":
        assert np.array_equal(to_np(sa).view(np.uint32), sa_ref.view(np.uint32))
    assert np.array_equal(to_np(sg).view(np.uint32), sg_ref.view(np.uint32))
    Y = to_np(out)
    for g in np.flatnonzero(np.asarray(sizes) == 0):
        assert (Y[g].view(np.uint32 if out_dtype == torch.float32 else np.uint16) == 0).all()
    if out_dtype == torch.float32:
        err = slab_rel_err(Y, R)
        print(f"max slab relative error {err:.3e}")
        assert err <= TOL, err
    else:
        assert_bf16_close(Y, R, [(g, g + 1) for g in range(len(sizes))])


def test_tgmm_all_groups_empty_writes_zeros(lib):
    K, N = 256, 128
    x = torch.empty((0, K), dtype=torch.bfloat16, device=DEV)
    gr = torch.empty((0, N), dtype=torch.bfloat16, device=DEV)
    out = torch.full((3, K, N), float("nan"), dtype=torch.float32, device=DEV)
    lib.tgmm_drhs(x, gr, gs_tensor([0, 0, 0]), out_dtype=torch.float32, out=out)
    sync()
    assert (out.view(torch.int32) == 0).all()


def test_tgmm_single_row_groups(lib):
    sizes = [1, 1, 0, 1]
    M, K, N = 3, 256, 128
    x, xb = gen((M, K), 1.0, 211)
    gr, gb = gen((M, N), 1e-3, 212)
    out = lib.tgmm_drhs(x, gr, gs_tensor(sizes), out_dtype=torch.float32)
    R, _, _ = ops.tgmm(xb, gb, np.asarray(sizes))
    assert slab_rel_err(to_np(out), R) <= TOL


def test_tgmm_given_scales_equal_in_call_scales(lib):
    sizes = [200, 0, 313]
    M, K, N = sum(sizes), 256, 256
    x, _ = gen((M, K), 1.0, 221)
    gr, _ = gen((M, N), 1e-3, 222)
    gs = gs_tensor(sizes)
    a, sa, sg = lib.tgmm_drhs(x, gr, gs, out_dtype=torch.float32, return_scales=True)
    b = lib.tgmm_drhs(x, gr, gs, lhs_scaling="dynamic_given", lhs_scales=lib.gmm_dynamic_scales(x, "e4m3"),
                      grad_scaling="dynamic_given", grad_scales=lib.gmm_dynamic_scales(gr, "e5m2"),
                      out_dtype=torch.float32)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def _block_scaled(shape, sigma, seed, factors):
    """Seeded bf16 [M, C] whose 128-row block b is multiplied by factors[b] (0: all zero)."""
    from synth.workloads import bf16_to_bits, normal_bf16

    t = normal_bf16(shape, sigma, seed, "cpu").float()
    for b, f in enumerate(factors):
        t[b * 128:(b + 1) * 128] *= f
    t = t.to(torch.bfloat16)
    return t.to(DEV), bf16_to_bits(t)


@pytest.mark.parametrize("sizes", [[200, 0, 250, 190], [640]])
def test_tgmm_blocks_that_add_nothing(lib, sizes):
    # block 1: grad all zero (scale 0); block 2: scale product underflows to 0 while the
    # codes are not zero; block 3: grad scale subnormal, so its inverse is not finite;
    # blocks 0 and 4 ordinary.  In the method such blocks add nothing, and the blocks
    # around them still add theirs with their own scale products.
    M, K, N = 640, 256, 256
    x, xb = _block_scaled((M, K), 1.0, 231, [1, 1, 1e-30, 1, 1])
    gr, gb = _block_scaled((M, N), 1e-3, 232, [1, 0, 1e-17, 1e-36, 1])
    out = torch.full((len(sizes), K, N), float("nan"), dtype=torch.float32, device=DEV)
    _, sa, sg = lib.tgmm_drhs(x, gr, gs_tensor(sizes), out_dtype=torch.float32, out=out,
                              return_scales=True)
    R, sa_ref, sg_ref = ops.tgmm(xb, gb, np.asarray(sizes))
    assert np.array_equal(to_np(sa).view(np.uint32), sa_ref.view(np.uint32))
    assert np.array_equal(to_np(sg).view(np.uint32), sg_ref.view(np.uint32))
    prod = sa_ref.astype(np.float32) * sg_ref.astype(np.float32)
    assert prod[1] == 0 and prod[2] == 0 and prod[0] > 0 and prod[4] > 0  # the cases hold
    Y = to_np(out)
    assert np.isfinite(Y).all()
    err = slab_rel_err(Y, R)
    print(f"max slab relative error {err:.3e}")
    assert err <= TOL, err
    for g in range(len(sizes)):
        if not np.abs(R[g]).max() > 0:
            assert (Y[g].view(np.uint32) == 0).all()


@pytest.mark.parametrize("sizes", [[512], [100, 412], [300, 0, 212]])
def test_tgmm_wide_scale_range_groups(lib, sizes):
    # block 1's scale product is ~1e-36 of block 0's: a group holding both keeps exact
    # per-block promotion (accumulators rescaled block to block would overflow), while
    # the other groups of the call take the rescaled path
    M, K, N = 512, 256, 256
    x, xb = _block_scaled((M, K), 1.0, 241, [1, 1e-18, 1, 1])
    gr, gb = _block_scaled((M, N), 1e-3, 242, [1, 1e-18, 1, 1])
    for out_dtype in (torch.float32, torch.bfloat16):
        out = torch.full((len(sizes), K, N), float("nan"), dtype=out_dtype, device=DEV)
        lib.tgmm_drhs(x, gr, gs_tensor(sizes), out_dtype=out_dtype, out=out)
        R, _, _ = ops.tgmm(xb, gb, np.asarray(sizes))
        Y = to_np(out)
        if out_dtype == torch.float32:
            assert np.isfinite(Y).all()
            err = slab_rel_err(Y, R)
            print(f"max slab relative error {err:.3e}")
            assert err <= TOL, err
        else:
            assert_bf16_close(Y, R, [(g, g + 1) for g in range(len(sizes))])
