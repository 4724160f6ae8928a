"""GPU parity of gmm_fwd and gmm_dlhs against the oracle (same bf16 inputs, own quantization)."""

import numpy as np
import pytest
import torch

import oracle.ops as ops
from oracle.gmm import gmm_dlhs_ref, gmm_fwd_ref, row_scales
from oracle.quant import quantize_rhs_per_channel
from synth.workloads import WORKLOADS
from tests.gpu_util import DEV, channel_varied, gen, gs_tensor, sync
from tests.parity import (
    TOL,
    assert_bf16_close,
    assert_rounding_bound,
    group_rel_err,
    group_row_ranges,
    magnitudes,
    to_np,
)

pytestmark = pytest.mark.gpu

S_4_448 = float(np.float32(4.0) / np.float32(448.0))


def quantized_weight(lib, w, axis, layout):
    codes, scales = lib.gmm_quantize_rhs(w, "e4m3", axis, layout)
    return codes, scales


def run_fwd(lib, x, xbits, w, wbits, sizes, scaling, layout, out_dtype, s=S_4_448):
    codes, scales = quantized_weight(lib, w, 0, layout)
    c_ref, s_ref = quantize_rhs_per_channel(wbits, "e4m3", "n")
    assert np.array_equal(to_np(scales).view(np.uint32), s_ref.view(np.uint32))
    out, sc = lib.gmm_fwd(x, codes, scales, gs_tensor(sizes), lhs_format="e4m3",
                          lhs_scaling=scaling, static_scale=s, rhs_layout=layout,
                          out_dtype=out_dtype, return_scales=True)
    R, a_codes, s_blk = ops.fwd(xbits, c_ref, s_ref, np.asarray(sizes), "e4m3", scaling,
                                np.float32(s), "e4m3", "f32")
    if scaling == "dynamic":
        assert np.array_equal(to_np(sc).view(np.uint32), s_blk.view(np.uint32))
    if out_dtype == torch.float32 and xbits.shape[0]:
        absR = gmm_fwd_ref(magnitudes(a_codes), "e4m3", row_scales(s_blk, xbits.shape[0]),
                           magnitudes(c_ref), "e4m3", s_ref, np.asarray(sizes))
        assert_rounding_bound(to_np(out), R, absR, xbits.shape[1])
    return to_np(out), R


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_fwd_tiny_workload(lib, out_dtype):
    wl = WORKLOADS["tiny"]
    sizes = wl.group_sizes()
    assert sizes[1] == 0 and sizes.sum() == wl.M
    x, xb = gen((wl.M, wl.K), 1.0, 101)
    w, wb = gen((wl.G, wl.K, wl.N), 0.02, 102)
    Y, R = run_fwd(lib, x, xb, w, wb, sizes, "static", "nk", out_dtype)
    if out_dtype == torch.float32:
        assert group_rel_err(Y, R, group_row_ranges(sizes)) <= TOL
    else:
        assert_bf16_close(Y, R, group_row_ranges(sizes))


@pytest.mark.parametrize("layout", ["nk", "kn"])
@pytest.mark.parametrize("scaling", ["static", "dynamic"])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_fwd_ragged_medium(lib, layout, scaling, out_dtype):
    # several M-tiles per group, ragged group ends, empty groups first and in the middle,
    # and an N tail (640 = 2.5 tiles of 256)
    sizes = [0, 700, 1, 0, 299, 500]
    M, K, N = sum(sizes), 512, 640
    x, xb = gen((M, K), 1.0, 111)
    w, wb = channel_varied((len(sizes), K, N), 0.02, 112, 2)
    Y, R = run_fwd(lib, x, xb, w, wb, sizes, scaling, layout, out_dtype)
    if out_dtype == torch.float32:
        err = group_rel_err(Y, R, group_row_ranges(sizes))
        print(f"max group relative error {err:.3e}")
        assert err <= TOL, err
    else:
        assert_bf16_close(Y, R, group_row_ranges(sizes))


@pytest.mark.parametrize("layout", ["kn", "nk"])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_dlhs_ragged_medium(lib, layout, out_dtype):
    sizes = [257, 0, 511, 128, 104]
    M, K, N = sum(sizes), 640, 384
    gr, gb = gen((M, N), 1e-3, 121)
    w, wb = channel_varied((len(sizes), K, N), 0.02, 122, 1)
    codes, scales = lib.gmm_quantize_rhs(w, "e4m3", 1, layout)
    c_ref, s_ref = quantize_rhs_per_channel(wb, "e4m3", "k")
    assert np.array_equal(to_np(scales).view(np.uint32), s_ref.view(np.uint32))
    out, sc = lib.gmm_dlhs(gr, codes, scales, gs_tensor(sizes), grad_format="e5m2",
                           grad_scaling="dynamic", rhs_layout=layout, out_dtype=out_dtype,
                           return_scales=True)
    R, g_codes, s_blk = ops.dlhs(gb, c_ref, s_ref, np.asarray(sizes))
    assert np.array_equal(to_np(sc).view(np.uint32), s_blk.view(np.uint32))
    Y = to_np(out)
    if out_dtype == torch.float32:
        err = group_rel_err(Y, R, group_row_ranges(sizes))
        print(f"max group relative error {err:.3e}")
        assert err <= TOL, err
        absR = gmm_dlhs_ref(magnitudes(g_codes), "e5m2", row_scales(s_blk, M), magnitudes(c_ref),
                            "e4m3", s_ref, np.asarray(sizes))
        assert_rounding_bound(Y, R, absR, N)
    else:
        assert_bf16_close(Y, R, group_row_ranges(sizes))


def test_hybrid_dlhs_equals_fused(lib):
    """Pre-quantized grad (stand-alone quantizer) through the fp8-A kernel gives the same
    bits as the fused in-kernel quantization."""
    sizes = [300, 212, 0, 500]
    M, K, N = sum(sizes), 384, 512
    gr, _ = gen((M, N), 1e-3, 131)
    w, _ = channel_varied((len(sizes), K, N), 0.02, 132, 1)
    codes, scales = lib.gmm_quantize_rhs(w, "e4m3", 1, "kn")
    gs = gs_tensor(sizes)
    fused = lib.gmm_dlhs(gr, codes, scales, gs, out_dtype=torch.float32)
    gq, gsc = lib.gmm_quantize(gr, "e5m2", "dynamic")
    hybrid = lib.gmm_dlhs(gq, codes, scales, gs, grad_scales=gsc, out_dtype=torch.float32)
    assert torch.equal(fused.view(torch.int32), hybrid.view(torch.int32))


def test_prequantized_static_forward_equals_fused(lib):
    sizes = [129, 383]
    M, K, N = sum(sizes), 256, 256
    x, _ = gen((M, K), 1.0, 141)
    w, _ = gen((2, K, N), 0.02, 142)
    codes, scales = lib.gmm_quantize_rhs(w, "e4m3", 0, "nk")
    gs = gs_tensor(sizes)
    fused = lib.gmm_fwd(x, codes, scales, gs, lhs_scaling="static", static_scale=S_4_448,
                        out_dtype=torch.float32)
    xq, _ = lib.gmm_quantize(x, "e4m3", "static", S_4_448)
    pre = lib.gmm_fwd(xq, codes, scales, gs, lhs_scaling="static", static_scale=S_4_448,
                      out_dtype=torch.float32)
    assert torch.equal(fused.view(torch.int32), pre.view(torch.int32))


def test_merged_gate_up_equals_two_calls(lib):
    sizes = [200, 0, 350]
    M, K, Nh = sum(sizes), 256, 384
    x, _ = gen((M, K), 1.0, 151)
    w0, _ = gen((3, K, Nh), 0.02, 152)
    w1, _ = gen((3, K, Nh), 0.02, 153)
    gs = gs_tensor(sizes)
    c, s = lib.gmm_quantize_rhs(torch.cat([w0, w1], dim=2).contiguous(), "e4m3", 0, "nk")
    c0, s0 = lib.gmm_quantize_rhs(w0, "e4m3", 0, "nk")
    c1, s1 = lib.gmm_quantize_rhs(w1, "e4m3", 0, "nk")
    merged = lib.gmm_fwd(x, c, s, gs, out_dtype=torch.float32)
    a = lib.gmm_fwd(x, c0, s0, gs, out_dtype=torch.float32)
    b = lib.gmm_fwd(x, c1, s1, gs, out_dtype=torch.float32)
    assert torch.equal(merged.view(torch.int32), torch.cat([a, b], 1).view(torch.int32))


def test_rows_written_exactly_once_with_canaries(lib):
    sizes = [0, 300, 0, 45, 211]
    M, K, N = sum(sizes), 256, 384
    x, _ = gen((M, K), 1.0, 161)
    w, _ = gen((5, K, N), 0.02, 162)
    codes, scales = lib.gmm_quantize_rhs(w, "e4m3", 0, "nk")
    pad = 64
    buf = torch.full(((M + 2 * pad) * N,), float("nan"), dtype=torch.float32, device=DEV)
    out = buf[pad * N:(pad + M) * N].view(M, N)
    lib.gmm_fwd(x, codes, scales, gs_tensor(sizes), out_dtype=torch.float32, out=out)
    sync()
    assert not torch.isnan(out).any()
    assert torch.isnan(buf[:pad * N]).all() and torch.isnan(buf[(pad + M) * N:]).all()


def test_sizes_outside_the_contract_stay_inside_the_output(lib):
    # group sizes that break the contract (one near INT_MAX, a negative one, a sum past M)
    # are clamped by the schedulers: every kernel still writes only inside its output
    # (NaN canaries on both sides stay), whatever it writes there
    M, K, N, G = 556, 256, 384, 5
    sizes = [300, 2147483000, 45, -5, 211]
    x, _ = gen((M, K), 1.0, 163)
    gr, _ = gen((M, N), 1e-3, 164)
    w, _ = gen((G, K, N), 0.02, 165)
    codes, scales = lib.gmm_quantize_rhs(w, "e4m3", 0, "nk")
    wk, sk = lib.gmm_quantize_rhs(w, "e4m3", 1, "kn")
    gs = gs_tensor(sizes)
    pad = 64

    def canaried(rows, cols):
        buf = torch.full(((rows + 2 * pad) * cols,), float("nan"), dtype=torch.float32, device=DEV)
        return buf, buf[pad * cols:(pad + rows) * cols].view(rows, cols)

    def intact(buf, rows, cols):
        return bool(torch.isnan(buf[:pad * cols]).all() and torch.isnan(buf[(pad + rows) * cols:]).all())

    b1, o1 = canaried(M, N)
    lib.gmm_fwd(x, codes, scales, gs, lhs_scaling="static", static_scale=S_4_448,
                out_dtype=torch.float32, out=o1)
    b2, o2 = canaried(M, K)
    lib.gmm_dlhs(gr, wk, sk, gs, out_dtype=torch.float32, out=o2)
    xq, sx = lib.gmm_quantize_subchannel(x, 128)
    wb, wbs = lib.gmm_quantize_rhs_blockwise(w, 128)
    b3, o3 = canaried(M, N)
    lib.gmm_fwd_blockwise(xq, sx, wb, wbs, gs, 128, out_dtype=torch.float32, out=o3)
    b4, o4 = canaried(G * K, N)
    lib.tgmm_drhs(x, gr, gs, out_dtype=torch.float32, out=o4.view(G, K, N))
    sync()
    assert intact(b1, M, N) and intact(b2, M, K) and intact(b3, M, N) and intact(b4, G * K, N)


def compositions(M, G):
    import itertools

    for cuts in itertools.combinations(range(M + G - 1), G - 1):
        prev, sizes = -1, []
        for c in cuts + (M + G - 1,):
            sizes.append(c - prev - 1)
            prev = c
        yield sizes


def test_every_composition_of_nine_rows(lib):
    K, N = 128, 128
    x, xb = gen((9, K), 1.0, 171)
    w, wb = gen((3, K, N), 0.02, 172)
    codes, scales = lib.gmm_quantize_rhs(w, "e4m3", 0, "nk")
    c_ref, s_ref = quantize_rhs_per_channel(wb, "e4m3", "n")
    n = 0
    for sizes in compositions(9, 3):
        out = lib.gmm_fwd(x, codes, scales, gs_tensor(sizes), lhs_scaling="dynamic",
                          out_dtype=torch.float32)
        R, _, _ = ops.fwd(xb, c_ref, s_ref, np.asarray(sizes), "e4m3", "dynamic")
        assert group_rel_err(to_np(out), R, group_row_ranges(sizes)) <= TOL, sizes
        n += 1
    assert n == 55


def test_empty_and_single_group_edge_cases(lib):
    K, N = 128, 256
    x, xb = gen((1, K), 1.0, 181)
    w, wb = gen((2, K, N), 0.02, 182)
    codes, scales = lib.gmm_quantize_rhs(w, "e4m3", 0, "kn")
    c_ref, s_ref = quantize_rhs_per_channel(wb, "e4m3", "n")
    for sizes in ([1, 0], [0, 1]):
        out = lib.gmm_fwd(x, codes, scales, gs_tensor(sizes), rhs_layout="kn", out_dtype=torch.float32)
        R, _, _ = ops.fwd(xb, c_ref, s_ref, np.asarray(sizes), "e4m3", "dynamic")
        assert group_rel_err(to_np(out), R, group_row_ranges(sizes)) <= TOL
    # M == 0: nothing to do, no error
    empty = torch.empty((0, K), dtype=torch.bfloat16, device=DEV)
    out = lib.gmm_fwd(empty, codes, scales, gs_tensor([0, 0]), rhs_layout="kn")
    assert out.shape == (0, N)


def test_given_scales_equal_in_call_scales(lib):
    """Block scales computed once (gmm_dynamic_scales) and passed in give the same bits."""
    sizes = [130, 0, 400, 90]
    M, K, N = sum(sizes), 384, 256
    x, xb = gen((M, K), 1.0, 191)
    w, _ = gen((4, K, N), 0.02, 192)
    codes, scales = lib.gmm_quantize_rhs(w, "e4m3", 0, "nk")
    gs = gs_tensor(sizes)
    s = lib.gmm_dynamic_scales(x, "e4m3")
    a, sa = lib.gmm_fwd(x, codes, scales, gs, out_dtype=torch.float32, return_scales=True)
    b = lib.gmm_fwd(x, codes, scales, gs, lhs_scaling="dynamic_given", lhs_scales=s,
                    out_dtype=torch.float32)
    assert torch.equal(s.view(torch.int32), sa.view(torch.int32))
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


QO_SIZES = [300, 0, 1, 511, 212]  # 1024 rows; 1152 output columns = 4.5 tiles of 256


@pytest.mark.parametrize("scaling", ["static", "dynamic", "dynamic_given"])
@pytest.mark.parametrize("layout", ["nk", "kn"])
def test_fwd_quantize_once_route(lib, scaling, layout):
    """A wide output makes the call quantize the bf16 lhs once into its workspace and run
    the fp8-A kernel: the same bits as the in-kernel quantization, and oracle parity."""
    sizes = QO_SIZES
    M, K, N = sum(sizes), 384, 1152
    x, xb = gen((M, K), 1.0, 251)
    w, wb = channel_varied((len(sizes), K, N), 0.02, 252, 2)
    codes, scales = lib.gmm_quantize_rhs(w, "e4m3", 0, layout)
    gs = gs_tensor(sizes)
    kw = dict(lhs_scaling=scaling, static_scale=S_4_448, rhs_layout=layout, out_dtype=torch.float32)
    if scaling == "dynamic_given":
        kw["lhs_scales"] = lib.gmm_dynamic_scales(x, "e4m3")
    once = lib.gmm_fwd(x, codes, scales, gs, **kw)
    fused = lib.gmm_fwd(x, codes, scales, gs, fused=True, **kw)
    assert torch.equal(once.view(torch.int32), fused.view(torch.int32))
    c_ref, s_ref = quantize_rhs_per_channel(wb, "e4m3", "n")
    rec = "static" if scaling == "static" else "dynamic"
    R, _, _ = ops.fwd(xb, c_ref, s_ref, sizes, "e4m3", rec, np.float32(S_4_448))
    err = group_rel_err(to_np(once), R, group_row_ranges(sizes))
    assert err <= TOL, err


@pytest.mark.parametrize("layout", ["kn", "nk"])
def test_dlhs_quantize_once_route(lib, layout):
    sizes = QO_SIZES
    M, K, N = sum(sizes), 1152, 640
    gr, gb = gen((M, N), 1e-3, 261)
    w, wb = channel_varied((len(sizes), K, N), 0.02, 262, 1)
    codes, scales = lib.gmm_quantize_rhs(w, "e4m3", 1, layout)
    gs = gs_tensor(sizes)
    once, s1 = lib.gmm_dlhs(gr, codes, scales, gs, rhs_layout=layout, out_dtype=torch.float32,
                            return_scales=True)
    fused = lib.gmm_dlhs(gr, codes, scales, gs, rhs_layout=layout, out_dtype=torch.float32,
                         fused=True)
    assert torch.equal(once.view(torch.int32), fused.view(torch.int32))
    c_ref, s_ref = quantize_rhs_per_channel(wb, "e4m3", "k")
    R, _, sg = ops.dlhs(gb, c_ref, s_ref, sizes)
    assert np.array_equal(to_np(s1).view(np.uint32), sg.view(np.uint32))
    err = group_rel_err(to_np(once), R, group_row_ranges(sizes))
    assert err <= TOL, err


def test_quantize_once_route_writes_the_codes_into_the_workspace(lib):
    """The route really taken: after the call the workspace holds the lhs codes, equal to
    the stand-alone quantizer's."""
    import ctypes

    sizes = QO_SIZES
    M, K, N = sum(sizes), 256, 1024
    x, _ = gen((M, K), 1.0, 271)
    w, _ = gen((len(sizes), K, N), 0.02, 272)
    codes, scales = lib.gmm_quantize_rhs(w, "e4m3", 0, "nk")
    gs = gs_tensor(sizes)
    n = lib.gmm_workspace_size(lib.OP_FWD, "e4m3", "static", M, K, N, static_scale=S_4_448)
    assert n == M * K
    ws = torch.full((n,), 0xAB, dtype=torch.uint8, device=DEV)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    op = lib.Operand(lib.KIND_BF16, lib.E4M3, lib.STATIC, S_4_448)
    c = lambda t: ctypes.c_void_p(t.data_ptr())
    st = lib.load().gmm_fwd(ctypes.byref(op), lib.E4M3, lib.RHS_NK, lib.OUT_BF16, M, K, N,
                            len(sizes), c(x), None, c(codes), c(scales), c(gs), c(out), c(ws), n,
                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    xq, _ = lib.gmm_quantize(x, "e4m3", "static", S_4_448)
    sync()
    assert torch.equal(ws.view(M, K), xq)
    ref = lib.gmm_fwd(x, codes, scales, gs, lhs_scaling="static", static_scale=S_4_448, fused=True)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("op", ["fwd", "dlhs"])
def test_more_tiles_than_cus_is_bit_identical(lib, op):
    """More output tiles than the device has compute units (a full round of workgroups
    and a short last one): the fp8-codes route is bit for bit equal to the in-kernel
    quantization route."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sizes = [256 * 3 + 100, 0, 256 + 7]          # 4 + 0 + 2 = 6 M-tiles of 256 rows
    n_nt = -(-(cus + cus // 8) // 6)             # about 9/8 of the CUs in tiles
    M = sum(sizes)
    gs = gs_tensor(sizes)
    if op == "fwd":
        K, N = 256, 256 * n_nt
        x, _ = gen((M, K), 1.0, 171)
        w, _ = channel_varied((len(sizes), K, N), 0.02, 172, 0)
        codes, scales = lib.gmm_quantize_rhs(w, "e4m3", 0, "nk")
        ref, sc = lib.gmm_fwd(x, codes, scales, gs, out_dtype=torch.float32, return_scales=True,
                              fused=True)
        xq, _ = lib.gmm_quantize(x, "e4m3", "dynamic_given", scales=sc)
        got = lib.gmm_fwd(xq, codes, scales, gs, lhs_scaling="dynamic_given", lhs_scales=sc,
                          out_dtype=torch.float32)
    else:
        K, N = 256 * n_nt, 256                   # dlhs output tiles are 256 columns of K
        gr, _ = gen((M, N), 1e-3, 173)
        w, _ = channel_varied((len(sizes), K, N), 0.02, 174, 1)
        codes, scales = lib.gmm_quantize_rhs(w, "e4m3", 1, "kn")
        ref = lib.gmm_dlhs(gr, codes, scales, gs, out_dtype=torch.float32, fused=True)
        gq, gsc = lib.gmm_quantize(gr, "e5m2", "dynamic")
        got = lib.gmm_dlhs(gq, codes, scales, gs, grad_scales=gsc, out_dtype=torch.float32)
    sync()
    assert torch.equal(ref.view(torch.int32), got.view(torch.int32))
