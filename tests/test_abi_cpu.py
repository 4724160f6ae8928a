"""The C-ABI library without a GPU: it loads, exports every declared symbol, its host-only
functions work, and every validation error is reported before any work is enqueued."""

import ctypes
import os
import re

import numpy as np
import pytest

import fp8_grouped_gemm_ragged_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gmm_fp8.h")

pytestmark = pytest.mark.skipif(not os.path.exists(g.library_path()),
                                reason="libgmm_fp8.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", src, flags=re.M)))


def test_every_declared_symbol_is_exported():
    lib = g.load()
    names = declared_functions()
    assert {"gmm_fwd", "gmm_dlhs", "tgmm_drhs", "gmm_quantize", "gmm_quantize_rhs"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(g.EXPORTED)


def test_host_helpers():
    assert "gfx950" in g.gmm_version()
    assert g.gmm_status_string(0) == "ok"
    s = g.gmm_static_scale_from_bound(-4.0, 4.0, "e4m3")
    assert np.float32(s).view(np.uint32) == 0x3C124925  # RNE_f32(4/448), hand-derived
    assert g.gmm_static_scale_from_bound(-57344.0, 57344.0, "e5m2") == 1.0
    for lo, hi in [(-3.0, 4.0), (0.0, 0.0), (4.0, -4.0), (-np.inf, np.inf), (-1e-40, 1e-40)]:
        with pytest.raises(g.GmmError) as e:
            g.gmm_static_scale_from_bound(lo, hi, "e4m3")
        assert e.value.status == 3  # GMM_ERR_SCALE


def test_workspace_sizes():
    assert g.gmm_workspace_size(g.OP_FWD, "e4m3", "static", 1000) == 0
    # a bf16 operand of a wide output (>= 4 tiles of 256, or unknown) gets room for its codes
    assert g.gmm_workspace_size(g.OP_FWD, "e4m3", "static", 1000, 512) == 512000
    assert g.gmm_workspace_size(g.OP_FWD, "e4m3", "static", 1000, 512, 1024) == 512000
    assert g.gmm_workspace_size(g.OP_DLHS, "e5m2", "static", 1000, 640, 769) == 640000
    assert g.gmm_workspace_size(g.OP_FWD, "e4m3", "static", 1000, 512, 768) == 0  # 3 tiles
    assert g.gmm_workspace_size(g.OP_FWD_FUSED, "e4m3", "static", 1000, 512) == 0
    assert g.gmm_workspace_size(g.OP_FWD, "e4m3", "static", 1000, 512, a_kind=g.KIND_FP8) == 0
    d = g.gmm_workspace_size(g.OP_QUANTIZE, "e4m3", "dynamic", 1000, 512)
    assert g.gmm_workspace_size(g.OP_DLHS_FUSED, "e4m3", "dynamic", 1000, 512) == d
    assert g.gmm_workspace_size(g.OP_FWD, "e4m3", "dynamic", 1000, 512) == d + 512000
    with pytest.raises(g.GmmError):
        g.gmm_workspace_size(9, "e4m3", "static", 1000)
    n = g.gmm_workspace_size(g.OP_FWD, "e4m3", "dynamic", 1000)
    nb = 8
    assert n >= nb * (8 + 2) * 4 and n % 256 == 0
    t = g.gmm_workspace_size(g.OP_TGMM, "e4m3", "dynamic", 1000, 256, 384, b_fmt="e5m2",
                             b_scaling="dynamic", groups=5)
    plan = 256  # 5 G + 2 words, aligned
    sc = 256  # one float per 128-row block, aligned
    ratio = 256  # ceil(1000/128) + 2 G floats, aligned
    codes = 256000 + 384000  # row-major codes of both bf16 operands, each aligned to 256
    assert t == 2 * n + plan + sc + ratio + codes
    s = g.gmm_workspace_size(g.OP_TGMM, "e4m3", "static", 1000, 256, 384, b_scaling="static",
                             static_scale=0.5, groups=5)
    assert s == plan + sc + ratio + codes
    # operands handed over as codes need no room for codes
    c = g.gmm_workspace_size(g.OP_TGMM, "e4m3", "static", 1000, 256, 384, b_scaling="static",
                             static_scale=0.5, groups=5, a_kind=g.KIND_FP8)
    assert c == plan + sc + ratio + 384000


# ---- validation: fake but aligned device pointers; nothing is dereferenced -------------
FAKE = 0x7F0000000000


def ptr(i):
    return ctypes.c_void_p(FAKE + i * (1 << 32))


def op(kind=0, fmt=0, scaling=1, s=0.0):
    return g.Operand(kind, fmt, scaling, s)


def call_fwd(o=None, rhs_format=0, layout=1, out_dtype=0, M=256, K=256, N=256, G=4, lhs=1,
             lhs_scales=2, rhs=3, rhs_scales=4, gs=5, out=6, ws=7, ws_bytes=1 << 20):
    lib = g.load()
    o = o or op()
    P = lambda i: None if i is None else (ptr(i) if isinstance(i, int) else i)
    return lib.gmm_fwd(ctypes.byref(o), rhs_format, layout, out_dtype, M, K, N, G, P(lhs),
                       P(lhs_scales), P(rhs), P(rhs_scales), P(gs), P(out), P(ws), ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(K=100), 2), (dict(N=64), 2), (dict(K=0), 2), (dict(M=-1), 2), (dict(G=0), 2),
    (dict(G=1025), 2), (dict(K=1 << 23), 2),
    (dict(rhs_format=1), 4), (dict(layout=7), 4), (dict(out_dtype=5), 4),
    (dict(o=op(kind=3)), 4), (dict(o=op(fmt=2)), 4), (dict(o=op(scaling=9)), 4),
    (dict(o=op(scaling=0, s=0.0)), 3), (dict(o=op(scaling=0, s=-1.0)), 3),
    (dict(o=op(scaling=0, s=float("nan"))), 3), (dict(o=op(scaling=0, s=1e-40)), 3),
    (dict(rhs=None), 1), (dict(gs=None), 1), (dict(lhs=None), 1), (dict(out=None), 1),
    (dict(rhs_scales=None), 1), (dict(o=op(kind=1, scaling=1), lhs_scales=None), 1),
    (dict(ws=None), 5), (dict(ws_bytes=16), 5),
    (dict(lhs=ctypes.c_void_p(FAKE + 8)), 6),
    (dict(out=1), 9), (dict(ws=6, out=6), 9),
])
def test_fwd_validation_errors(kw, status):
    assert call_fwd(**kw) == status


def test_fwd_empty_problem_is_ok_without_gpu():
    # M == 0: validated, nothing to enqueue
    assert call_fwd(M=0) == 0


def test_dlhs_and_tgmm_validation():
    lib = g.load()
    o = op(fmt=1)
    assert lib.gmm_dlhs(ctypes.byref(o), 0, 0, 0, 256, 200, 256, 2, ptr(1), ptr(2), ptr(3),
                        ptr(4), ptr(5), ptr(6), ptr(7), 1 << 20, None) == 2
    a, b = op(fmt=0), op(fmt=1)
    # fp8 codes are accepted; their dynamic block scales are then an input
    pre = op(kind=1)
    assert lib.tgmm_drhs(ctypes.byref(pre), ctypes.byref(b), 0, 256, 256, 256, 2, ptr(1), None,
                         ptr(3), ptr(4), ptr(5), ptr(6), ptr(7), 1 << 20, None) == 1
    assert lib.tgmm_drhs(ctypes.byref(pre), ctypes.byref(b), 0, 256, 256, 256, 2, ptr(1), ptr(2),
                         ptr(3), ptr(4), ptr(5), ptr(6), ptr(7), 64, None) == 5
    # aliasing is judged with the operand's element size: 1 byte for codes, 2 for bf16
    lhs = ptr(1).value
    near = lambda d: ctypes.c_void_p(lhs + d)
    assert lib.tgmm_drhs(ctypes.byref(pre), ctypes.byref(b), 0, 256, 256, 256, 2, ptr(1), ptr(2),
                         ptr(3), ptr(4), ptr(5), near(256 * 256 - 16), ptr(7), 1 << 26, None) == 9
    assert lib.tgmm_drhs(ctypes.byref(a), ctypes.byref(b), 0, 256, 256, 256, 2, ptr(1), ptr(2),
                         ptr(3), ptr(4), ptr(5), near(256 * 256), ptr(7), 1 << 26, None) == 9
    # scales inside the workspace are rejected (the call overwrites its workspace)
    assert lib.tgmm_drhs(ctypes.byref(pre), ctypes.byref(b), 0, 256, 256, 256, 2, ptr(1), ptr(7),
                         ptr(3), ptr(4), ptr(5), ptr(6), ptr(7), 1 << 26, None) == 9
    assert lib.tgmm_drhs(ctypes.byref(a), ctypes.byref(b), 0, 256, 256, 256, 2, ptr(1), ptr(2),
                         ptr(3), ptr(4), ptr(5), ptr(6), ptr(7), 64, None) == 5
    assert lib.tgmm_drhs(ctypes.byref(a), ctypes.byref(b), 0, 256, 256, 256, 2, ptr(1), ptr(2),
                         ptr(3), ptr(4), ptr(5), ptr(1), ptr(7), 1 << 20, None) == 9  # drhs aliases lhs
    assert lib.tgmm_drhs(ctypes.byref(a), ctypes.byref(b), 0, 256, 256, 256, 2, ptr(1), ptr(2),
                         ptr(3), ptr(4), None, ptr(6), ptr(7), 1 << 20, None) == 1


def test_size_limits():
    lib = g.load()
    a, b = op(fmt=0, scaling=0, s=1.0), op(fmt=1, scaling=0, s=1.0)
    # tgmm: M below 2^31 rows
    assert lib.tgmm_drhs(ctypes.byref(a), ctypes.byref(b), 0, 1 << 31, 256, 256, 2, ptr(1), None,
                         ptr(3), None, ptr(5), ptr(6), ptr(7), 1 << 50, None) == 2
    # gmm: fewer than 2^31 output tiles
    assert call_fwd(M=(1 << 31) - 1, K=128, N=(1 << 22), G=1, o=op(scaling=0, s=1.0)) == 2


def test_given_scales_validation():
    lib = g.load()
    given = op(scaling=2)
    # DYNAMIC_GIVEN: scales are an input (NULL rejected) and the in-kernel route needs no
    # workspace; the quantize-once route needs room for the codes only
    assert call_fwd(o=given, lhs_scales=None) == 1
    assert call_fwd(o=given, ws=None, ws_bytes=0, M=0) == 0
    n = ctypes.c_size_t()
    assert lib.gmm_workspace_size(3, ctypes.byref(given), ctypes.byref(given), 1000, 256, 0, 1, ctypes.byref(n)) == 0
    assert n.value == 0
    assert lib.gmm_workspace_size(0, ctypes.byref(given), ctypes.byref(given), 1000, 256, 0, 1, ctypes.byref(n)) == 0
    assert n.value == 256000
    a, b = op(fmt=0, scaling=2), op(fmt=1, scaling=2)
    assert lib.tgmm_drhs(ctypes.byref(a), ctypes.byref(b), 0, 256, 256, 256, 2, ptr(1), None,
                         ptr(3), ptr(4), ptr(5), ptr(6), None, 0, None) == 1
    assert lib.gmm_dynamic_scales(0, 100, 12, ptr(1), ptr(2), ptr(3), 1 << 20, None) == 2
    assert lib.gmm_dynamic_scales(2, 100, 16, ptr(1), ptr(2), ptr(3), 1 << 20, None) == 4
    assert lib.gmm_dynamic_scales(0, 100, 16, ptr(1), ptr(2), None, 0, None) == 5
    assert lib.gmm_dynamic_scales(0, 0, 16, None, None, None, 0, None) == 0


def test_quantize_validation():
    lib = g.load()
    o = op()
    assert lib.gmm_quantize(ctypes.byref(o), 100, 12, ptr(1), ptr(2), ptr(3), ptr(4), 1 << 20, None) == 2
    assert lib.gmm_quantize(ctypes.byref(op(kind=1)), 100, 16, ptr(1), ptr(2), ptr(3), ptr(4), 1 << 20, None) == 4
    assert lib.gmm_quantize(ctypes.byref(o), 100, 16, ptr(1), ptr(2), ptr(3), None, 0, None) == 5
    assert lib.gmm_quantize_rhs(0, 2, 0, 2, 128, 128, ptr(1), ptr(2), ptr(3), None) == 4
    assert lib.gmm_quantize_rhs(0, 0, 0, 2, 100, 128, ptr(1), ptr(2), ptr(3), None) == 2
    assert lib.gmm_quantize_rhs(0, 0, 0, 2, 128, 128, None, ptr(2), ptr(3), None) == 1


def test_swiglu_validation():
    lib = g.load()
    o = op(kind=1)  # dynamic fp8 codes: block scales are an input
    hop = op(kind=1, fmt=0, scaling=0, s=0.25)

    def fwd_fp8(h=hop, layout=1, M=256, K=256, I=256, gu=None, h_codes=8, gu_dtype=0):
        return lib.gmm_fwd_swiglu_fp8(ctypes.byref(o), 0, layout, gu_dtype, M, K, I, 4, ptr(1),
                                      ptr(2), ptr(3), ptr(4), ptr(5),
                                      None if gu is None else ptr(gu),
                                      None if h is None else ctypes.byref(h),
                                      None if h_codes is None else ptr(h_codes), ptr(7), 1 << 20,
                                      None)

    assert fwd_fp8(M=0) == 0  # validated, nothing to enqueue
    assert fwd_fp8(h=None) == 1
    assert fwd_fp8(h_codes=None) == 1
    assert fwd_fp8(h=op(kind=0, scaling=0, s=0.25)) == 4  # h must be fp8 codes
    assert fwd_fp8(h=op(kind=1, scaling=1)) == 4  # only a static scale fits one pass
    assert fwd_fp8(h=op(kind=1, fmt=2, scaling=0, s=0.25)) == 4
    for bad in (0.0, -1.0, float("inf"), 1e-40):
        assert fwd_fp8(h=op(kind=1, scaling=0, s=bad)) == 3
    assert fwd_fp8(layout=0) == 4  # [G, K, 2I] weights: not on the SwiGLU route
    assert fwd_fp8(I=192) == 2  # 2I must be a multiple of 256
    assert fwd_fp8(gu_dtype=3) == 4
    assert fwd_fp8(h_codes=1) == 9  # h codes over the lhs
    assert fwd_fp8(gu=8) == 9  # the product over h
    assert lib.gmm_fwd_swiglu(ctypes.byref(o), 0, 1, 0, 256, 256, 256, 4, ptr(1), ptr(2), ptr(3),
                              ptr(4), ptr(5), None, None, ptr(7), 1 << 20, None) == 1
    assert lib.gmm_swiglu_bwd(256, 192, ptr(1), ptr(2), ptr(3), None) == 2
    assert lib.gmm_swiglu_bwd(256, 256, ptr(1), None, ptr(3), None) == 1
    assert lib.gmm_swiglu_bwd(256, 256, ptr(1), ptr(2), ptr(2), None) == 9
    assert lib.gmm_swiglu_bwd(0, 256, None, None, None, None) == 0

    def dlhs_bwd(layout=0, M=256, I=256, N=256, gu=8, d_gu=9, ws=7, fmt=1, sc=None):
        P = lambda i: None if i is None else ptr(i)
        return lib.gmm_dlhs_swiglu_bwd(ctypes.byref(op(kind=1, fmt=1)), 0, layout, M, I, N, 4,
                                       ptr(1), ptr(2), ptr(3), ptr(4), ptr(5), P(gu), P(d_gu),
                                       fmt, P(sc), P(ws), 1 << 20, None)

    assert dlhs_bwd(M=0, gu=None, d_gu=None) == 0  # validated, nothing to enqueue
    assert dlhs_bwd(layout=5) == 4
    assert dlhs_bwd(I=0) == 2 and dlhs_bwd(I=192) == 2  # I a positive multiple of 128
    assert dlhs_bwd(I=(1 << 21) + 128) == 2
    assert dlhs_bwd(gu=None) == 1 and dlhs_bwd(d_gu=None) == 1
    assert dlhs_bwd(d_gu=8) == 9  # d_gu over gu
    assert dlhs_bwd(d_gu=1) == 9  # d_gu over the grad codes
    assert dlhs_bwd(d_gu=2) == 9  # d_gu over the grad scales
    assert dlhs_bwd(sc=10, fmt=2) == 4  # d_gu's scales in e4m3 or e5m2 only
    assert dlhs_bwd(sc=9) == 9 and dlhs_bwd(sc=8) == 9  # the scales over d_gu, over gu
    assert dlhs_bwd(sc=2) == 9 and dlhs_bwd(sc=4) == 9  # over the grad scales, rhs_scales


def test_route_validation():
    lib = g.load()
    assert lib.gmm_permute_workspace_size(1000, 8, 64) == ((8000 + 255) // 256 * 65 * 4 + 255) // 256 * 256 + 32000

    def perm(T=100, k=2, G=8, ids=1, rb=64, x=2, xp=3, gs=4, ros=5, sor=6, ws=7, wsb=1 << 20):
        P = lambda i: None if i is None else ptr(i)
        return lib.gmm_permute(T, k, G, P(ids), rb, P(x), P(xp), P(gs), P(ros), P(sor), P(ws), wsb, None)

    assert perm(T=-1) == 2 and perm(k=0) == 2 and perm(k=65) == 2 and perm(G=0) == 2
    assert perm(G=1025) == 2 and perm(T=1 << 30, k=4) == 2
    assert perm(rb=24) == 2 and perm(rb=0) == 2
    assert perm(ids=None) == 1 and perm(gs=None) == 1 and perm(sor=None) == 1
    assert perm(x=None) == 1  # x and x_perm come together
    assert perm(ws=None) == 5 and perm(wsb=16) == 5
    assert perm(xp=2) == 9 and perm(ros=6) == 9 and perm(ws=1) == 9
    assert lib.gmm_permute(100, 2, 8, ctypes.c_void_p(FAKE + 4), 64, ptr(2), ptr(3), ptr(4), ptr(5),
                           ptr(6), ptr(7), 1 << 20, None) == 6

    def unperm(T=100, k=2, H=64, y=1, ros=2, w=3, out=4):
        P = lambda i: None if i is None else ptr(i)
        return lib.gmm_unpermute(T, k, H, P(y), P(ros), P(w), P(out), None)

    assert unperm(H=12) == 2 and unperm(k=0) == 2 and unperm(T=-1) == 2
    assert unperm(y=None) == 1 and unperm(out=None) == 1 and unperm(ros=None) == 1
    assert unperm(out=1) == 9 and unperm(out=3) == 9
    assert unperm(T=0) == 0


def test_local_window_validation():
    lib = g.load()
    o = op(scaling=0, s=1.0)

    def fwd_local(G_total=8, off=2, G_local=3, M=256):
        return lib.gmm_fwd_local(ctypes.byref(o), 0, 1, 0, M, 256, 256, G_total, off, G_local,
                                 ptr(1), None, ptr(3), ptr(4), ptr(5), ptr(6), ptr(7), 1 << 20,
                                 None)

    assert fwd_local(M=0) == 0
    assert fwd_local(off=-1) == 2 and fwd_local(G_local=0) == 2 and fwd_local(off=6) == 2
    assert fwd_local(G_total=1025, off=0, G_local=1) == 2
    assert lib.gmm_dlhs_local(ctypes.byref(o), 0, 0, 0, 0, 256, 256, 8, 5, 4, ptr(1), None, ptr(3),
                              ptr(4), ptr(5), ptr(6), ptr(7), 1 << 20, None) == 2
    a, b = op(fmt=0, scaling=0, s=1.0), op(fmt=1, scaling=0, s=1.0)
    assert lib.tgmm_drhs_local(ctypes.byref(a), ctypes.byref(b), 0, 256, 256, 256, 8, 7, 2, ptr(1),
                               None, ptr(3), None, ptr(5), ptr(6), ptr(7), 1 << 26, None) == 2
    assert lib.tgmm_drhs_local(ctypes.byref(a), ctypes.byref(b), 0, 256, 256, 256, 8, 0, 0, ptr(1),
                               None, ptr(3), None, ptr(5), ptr(6), ptr(7), 1 << 26, None) == 2


def test_blockwise_validation():
    lib = g.load()

    def fwd(fmt=0, odt=0, M=256, K=512, N=256, G=4, bk=128, lhs=1, sl=2, rhs=3, sr=4, gs=5, out=6):
        P = lambda i: None if i is None else ptr(i)
        return lib.gmm_fwd_blockwise(fmt, odt, M, K, N, G, bk, P(lhs), P(sl), P(rhs), P(sr), P(gs),
                                     P(out), None)

    assert fwd(M=0) == 0
    assert fwd(bk=64) == 2 and fwd(bk=384) == 2 and fwd(K=640, bk=256) == 2 and fwd(N=200) == 2
    assert fwd(fmt=2) == 4 and fwd(odt=3) == 4
    assert fwd(sl=None) == 1 and fwd(sr=None) == 1 and fwd(gs=None) == 1 and fwd(out=None) == 1
    assert fwd(out=1) == 9 and fwd(out=4) == 9
    assert lib.gmm_quantize_subchannel(0, 100, 512, 96, ptr(1), ptr(2), ptr(3), None) == 2
    assert lib.gmm_quantize_subchannel(0, 100, 640, 512, ptr(1), ptr(2), ptr(3), None) == 2
    assert lib.gmm_quantize_subchannel(0, 100, 512, 1024, ptr(1), ptr(2), ptr(3), None) == 2
    assert lib.gmm_quantize_subchannel(0, 100, 512, 128, ptr(1), None, ptr(3), None) == 1
    assert lib.gmm_quantize_subchannel(0, 100, 512, 128, ptr(1), ptr(1), ptr(3), None) == 9
    assert lib.gmm_quantize_subchannel(0, 0, 512, 128, None, None, None, None) == 0
    assert lib.gmm_quantize_rhs_blockwise(0, 1, 2, 512, 256, 192, ptr(1), ptr(2), ptr(3), None) == 2
    assert lib.gmm_quantize_rhs_blockwise(0, 5, 2, 512, 256, 128, ptr(1), ptr(2), ptr(3), None) == 4
    assert lib.gmm_quantize_rhs_blockwise(0, 1, 2, 512, 256, 128, ptr(1), ptr(2), ptr(2), None) == 9


def test_folded_quantizer_validation():
    lib = g.load()

    def fold(fmt=1, M=256, N=256, G=4, grad=1, cs=2, gs=3, codes=4, sc=5, ws=6, wsb=1 << 20):
        P = lambda i: None if i is None else ptr(i)
        return lib.gmm_quantize_folded(fmt, M, N, G, P(grad), P(cs), P(gs), P(codes), P(sc), P(ws),
                                       wsb, None)

    assert fold(M=0) == 0
    assert fold(N=200) == 2 and fold(G=0) == 2 and fold(fmt=3) == 4
    assert fold(cs=None) == 1 and fold(codes=None) == 1
    assert fold(ws=None) == 5 and fold(wsb=8) == 5
    assert fold(codes=1) == 9 and fold(sc=4) == 9 and fold(ws=2) == 9


def test_split_workspace_for_dlhs_only():
    """gmm_dlhs's workspace holds the tail split's 256 partial tiles (64 MiB) once a call can
    have more than 256 output tiles and a contraction of 54 steps of 128 or more (a cut
    into 8 slices then saves 48 steps); gmm_fwd's never does."""
    M, G, C = 4352, 4, 54 * 128
    fwd = g.gmm_workspace_size(g.OP_FWD, "e4m3", "dynamic", M, C, 4096, a_kind=g.KIND_FP8,
                               groups=G)
    dl = g.gmm_workspace_size(g.OP_DLHS, "e5m2", "dynamic", M, C, 4096, a_kind=g.KIND_FP8,
                              groups=G)
    dlf = g.gmm_workspace_size(g.OP_DLHS_FUSED, "e5m2", "dynamic", M, C, 4096, groups=G)
    assert fwd == 0 and dl == 256 * 256 * 256 * 4
    assert dlf == dl + g.gmm_workspace_size(g.OP_QUANTIZE, "e5m2", "dynamic", M, C)
    # too few tiles (one round) or too short a contraction: no split
    assert g.gmm_workspace_size(g.OP_DLHS, "e5m2", "dynamic", 1000, C, 4096,
                                a_kind=g.KIND_FP8, groups=G) == 0
    assert g.gmm_workspace_size(g.OP_DLHS, "e5m2", "dynamic", M, C - 128, 4096,
                                a_kind=g.KIND_FP8, groups=G) == 0
