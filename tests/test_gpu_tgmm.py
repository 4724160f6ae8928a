"""GPU parity of tgmm_drhs against the oracle."""

import numpy as np
import pytest
import torch

import oracle.ops as ops
from tests.gpu_util import DEV, gen, gs_tensor, sync
from oracle.gmm import tgmm_ref
from tests.parity import (TOL, assert_bf16_close, assert_rounding_bound, magnitudes,
                          slab_rel_err, to_np)

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
        a_codes, _ = ops.quantize_operand(xb, "e4m3", lhs_scaling, np.float32(S_4_448))
        g_codes, _ = ops.quantize_operand(gb, "e5m2", "dynamic")
        absR = tgmm_ref(magnitudes(a_codes), "e4m3", sa_ref, magnitudes(g_codes), "e5m2", sg_ref,
                        np.asarray(sizes))
        assert_rounding_bound(Y, R, absR, np.asarray(sizes)[:, None, None])
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


def _codes_operand(which, name, M, C, fmt, seed, lo, hi, scaling="dynamic"):
    """(tensor for the call, call kwargs, oracle codes, oracle per-block scales).

    Codes operands are seeded random finite fp8 codes with seeded per-block scales (or one
    static scale); bf16 operands are seeded normals that both sides quantize themselves."""
    from synth.workloads import log_uniform_scales, random_fp8_codes

    nb = -(-M // 128)
    if which:
        codes = random_fp8_codes((M, C), fmt, seed)
        t = torch.from_numpy(codes).to(DEV)
        if scaling == "static":
            s = float(log_uniform_scales(1, lo, hi, seed + 1)[0])
            return t, {f"{name}_scaling": "static", f"{name}_static_scale": s}, codes, \
                np.full(nb, np.float32(s), np.float32)
        s = log_uniform_scales(nb, lo, hi, seed + 1)
        return t, {f"{name}_scaling": "dynamic", f"{name}_scales": torch.from_numpy(s).to(DEV)}, codes, s
    x, xb = gen((M, C), 1.0 if name == "lhs" else 1e-3, seed)
    codes, s = ops.quantize_operand(xb, fmt, "dynamic")
    return x, {}, codes, s


@pytest.mark.parametrize("which", ["lhs", "grad", "both", "both_static"])
def test_tgmm_codes_operands(lib, which):
    # operands handed over as fp8 codes quantized beforehand (with their scales): the call
    # only transposes them; ragged groups with empty ones and a K tail, as above
    from oracle.gmm import tgmm_ref

    sizes = [0, 300, 5, 0, 457, 130]
    M, K, N = sum(sizes), 640, 384
    st = "static" if which == "both_static" else "dynamic"
    lhs, lkw, ac, sa = _codes_operand(which != "grad", "lhs", M, K, "e4m3", 301, -3, -1, st)
    grad, gkw, gc, sg = _codes_operand(which != "lhs", "grad", M, N, "e5m2", 303, -8, -6, st)
    for out_dtype in (torch.float32, torch.bfloat16):
        out = lib.tgmm_drhs(lhs, grad, gs_tensor(sizes), out_dtype=out_dtype, **lkw, **gkw)
        R = tgmm_ref(ac, "e4m3", sa, gc, "e5m2", sg, np.asarray(sizes), 128, "f32")
        Y = to_np(out)
        for g in np.flatnonzero(np.asarray(sizes) == 0):
            assert (Y[g].view(np.uint32 if out_dtype == torch.float32 else np.uint16) == 0).all()
        if out_dtype == torch.float32:
            err = slab_rel_err(Y, R)
            print(f"{which}: max slab relative error {err:.3e}")
            assert err <= TOL, err
        else:
            assert_bf16_close(Y, R, [(g, g + 1) for g in range(len(sizes))])


def test_tgmm_codes_route_equals_bf16_route(lib):
    # the codes gmm_quantize makes for a tensor, handed to tgmm with their scales, give
    # the same bits as tgmm quantizing the bf16 tensor itself (GPU against GPU)
    sizes = [200, 0, 313, 129, 6]
    M, K, N = sum(sizes), 512, 384
    x, _ = gen((M, K), 1.0, 311)
    gr, _ = gen((M, N), 1e-3, 312)
    gs = gs_tensor(sizes)
    xq, sx = lib.gmm_quantize(x, "e4m3", "dynamic")
    gq, sgr = lib.gmm_quantize(gr, "e5m2", "dynamic")
    for out_dtype, view in ((torch.float32, torch.int32), (torch.bfloat16, torch.int16)):
        a = lib.tgmm_drhs(x, gr, gs, out_dtype=out_dtype)
        b = lib.tgmm_drhs(xq, gq, gs, lhs_scales=sx, grad_scales=sgr, out_dtype=out_dtype)
        c = lib.tgmm_drhs(x, gq, gs, grad_scales=sgr, out_dtype=out_dtype)
        assert torch.equal(a.view(view), b.view(view))
        assert torch.equal(a.view(view), c.view(view))


@pytest.mark.parametrize("sizes", [[200, 0, 250, 190], [640]])
def test_tgmm_codes_zero_and_subnormal_scale_blocks(lib, sizes):
    # codes are used as given: a block adds nothing only when its scale product is 0
    # (block 1: grad scale 0; block 3: the product underflows).  Block 2 has a subnormal
    # grad scale and nonzero codes: it adds its (tiny) product, and its group's scale
    # products then span more than 2^60, so that group takes the exact promotion.
    from oracle.gmm import tgmm_ref
    from synth.workloads import log_uniform_scales, random_fp8_codes

    M, K, N = 640, 256, 256
    ac = random_fp8_codes((M, K), "e4m3", 321)
    gc = random_fp8_codes((M, N), "e5m2", 322)
    sa = log_uniform_scales(5, -3, -1, 323)
    sg = log_uniform_scales(5, -8, -6, 324)
    sa[3] = np.float32(1e-30)
    sg[1] = np.float32(0.0)
    sg[2] = np.float32(1e-40)
    sg[3] = np.float32(1e-20)
    prod = sa * sg
    assert prod[1] == 0 and prod[3] == 0 and 0 < prod[2] < np.finfo(np.float32).tiny
    out = torch.full((len(sizes), K, N), float("nan"), dtype=torch.float32, device=DEV)
    lib.tgmm_drhs(torch.from_numpy(ac).to(DEV), torch.from_numpy(gc).to(DEV), gs_tensor(sizes),
                  lhs_scales=torch.from_numpy(sa).to(DEV), grad_scales=torch.from_numpy(sg).to(DEV),
                  out_dtype=torch.float32, out=out)
    R = tgmm_ref(ac, "e4m3", sa, gc, "e5m2", sg, np.asarray(sizes), 128, "f32")
    Y = to_np(out)
    assert np.isfinite(Y).all()
    err = slab_rel_err(Y, R)
    print(f"max slab relative error {err:.3e}")
    assert err <= TOL, err
