"""The tail split of gmm_dlhs: with its workspace, a call whose last round of 256 x 256
tiles leaves CUs idle cuts those tiles along the contraction and adds the slices' fp32
partial sums in a fixed order.  The shape here has 32 output-tile columns (K = 8192) and
9 tile rows (group boundaries included): 288 tiles, 36 per XCD, a last round of 4, cut
into 8 slices of the 64-step contraction (N = 8192) each.
gmm_fwd never splits: it gets no split workspace and stays bit-identical to the SwiGLU
forward's product half.

Checked: the split output against the oracle (per-group metric and elementwise bound),
against the same call without the workspace (the two may differ by fp32 summation order
only, and with lhs codes spanning many binades they do), and bit-identical between the
fused and the quantize-once routes, which take the same split."""

import ctypes

import numpy as np
import pytest
import torch

import fp8_grouped_gemm_ragged_amd as g
from oracle.gmm import gmm_dlhs_ref, row_scales
from oracle.quant import quantize_rhs_per_channel
from synth.workloads import log_uniform_scales, random_fp8_codes
from tests.gpu_util import DEV, gen, gs_tensor, sync
from tests.parity import (TOL, U, assert_rounding_bound, group_rel_err, group_row_ranges,
                          magnitudes, to_np)

pytestmark = pytest.mark.gpu

SIZES = [1100, 1000]  # 2100 rows, 9 M-tiles of 256 with the group boundary
M = sum(SIZES)


def _raw(lib, grad_codes, scales, w, w_scales, out, workspace, gs):
    """gmm_dlhs through the C ABI with the workspace given (or none: the unsplit call)."""
    op = g.Operand(g.KIND_FP8, g.E5M2, g.DYNAMIC, 0.0)
    Mr, N = grad_codes.shape
    G, K = w.shape[0], out.shape[1]
    ptr = workspace.data_ptr() if workspace is not None else None
    nbytes = workspace.numel() if workspace is not None else 0
    st = lib.gmm_dlhs(ctypes.byref(op), g.E4M3, g.RHS_KN, g.OUT_F32, Mr, K, N, G,
                      grad_codes.data_ptr(), scales.data_ptr(), w.data_ptr(), w_scales.data_ptr(),
                      gs.data_ptr(), out.data_ptr(), ptr, nbytes, None)
    assert st == 0, g.gmm_status_string(st)


def _workspace(lib, rows, contraction, cols):
    op = g.Operand(g.KIND_FP8, g.E5M2, g.DYNAMIC, 0.0)
    n = g._SZ()
    assert lib.gmm_workspace_size(g.OP_DLHS, ctypes.byref(op), ctypes.byref(op), rows,
                                  contraction, cols, len(SIZES), ctypes.byref(n)) == 0
    assert n.value >= 256 * 256 * 256 * 4  # the split's slots
    return torch.empty(n.value, dtype=torch.uint8, device=DEV)


def test_split_against_oracle_and_unsplit(lib):
    K, N = 8192, 8192
    raw = g.load()
    gs = gs_tensor(SIZES)
    # grad codes drawn over all finite encodings: their products span so many binades that
    # the order of the fp32 additions shows in the sums (with normal data the MFMA's
    # truncated group sums are coarse enough for fp32 to add them exactly in any order)
    s_blk = log_uniform_scales((M + 127) // 128, -3.0, 0.0, 603)
    codes = random_fp8_codes((M, N), "e5m2", 611)
    w, wb = gen((len(SIZES), K, N), 0.02, 612)
    wq, ws = lib.gmm_quantize_rhs(w, "e4m3", 1, "kn")
    # the oracle on 512 sampled output columns k (the whole contraction each; each k has its
    # own channel scale, so the sampled rows of the weight quantize as in the whole)
    kc = np.sort(np.random.default_rng(5).choice(K, 512, replace=False))
    cr, sr = quantize_rhs_per_channel(wb[:, kc, :], "e4m3", "k")
    a = torch.from_numpy(codes).to(DEV)
    sa = torch.from_numpy(s_blk).to(DEV)
    split = torch.full((M, K), float("nan"), dtype=torch.float32, device=DEV)
    plain = torch.full((M, K), float("nan"), dtype=torch.float32, device=DEV)
    _raw(raw, a, sa, wq, ws, split, _workspace(raw, M, N, K), gs)
    _raw(raw, a, sa, wq, ws, plain, None, gs)
    sync()
    Ys, Yp = to_np(split), to_np(plain)
    assert np.isfinite(Ys).all() and np.isfinite(Yp).all()
    R = gmm_dlhs_ref(codes, "e5m2", row_scales(s_blk, M), cr, "e4m3", sr, np.asarray(SIZES))
    absR = gmm_dlhs_ref(magnitudes(codes), "e5m2", row_scales(s_blk, M), magnitudes(cr), "e4m3",
                        sr, np.asarray(SIZES))
    ranges = group_row_ranges(SIZES)
    for Y in (Ys[:, kc], Yp[:, kc]):
        assert group_rel_err(Y, R, ranges) <= TOL
        assert_rounding_bound(Y, R, absR, N)
    # the split regroups the fp32 additions of the last round's tiles only: the two
    # differ by at most the rounding of their sums, and somewhere they do differ
    diff = np.abs(Ys.astype(np.float64) - Yp.astype(np.float64))[:, kc]
    assert (diff <= 2.0 * (N / 64 + 8) * U * absR + 2.0 ** -126).all()
    assert (diff > 0).any(), "no tile was split"
    print(f"outputs changed by the split {np.mean(diff > 0):.3f}", flush=True)


def test_split_routes_bit_identical(lib):
    """The fused dlhs (bf16 grad quantized in the kernel) and the hybrid one (codes
    quantized once) take the same split and give the same bits."""
    K, N = 8192, 8192
    grad, _ = gen((M, N), 1e-3, 621)
    w, _ = gen((len(SIZES), K, N), 0.02, 622)
    wk, sk = lib.gmm_quantize_rhs(w, "e4m3", 1, "kn")
    gs = gs_tensor(SIZES)
    fused = lib.gmm_dlhs(grad, wk, sk, gs, grad_scaling="dynamic", fused=True,
                         out_dtype=torch.float32)
    gq, sg = lib.gmm_quantize(grad, "e5m2", "dynamic")
    hybrid = lib.gmm_dlhs(gq, wk, sk, gs, grad_scaling="dynamic", grad_scales=sg,
                          out_dtype=torch.float32)
    sync()
    assert torch.equal(fused.view(torch.int32), hybrid.view(torch.int32))
