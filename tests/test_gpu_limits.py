"""GPU parity at the limits of the shape contract: the most groups, the longest
contraction (K = 2^22 for fwd and tgmm, N = 2^22 for dlhs), the widest output (N = 2^22),
and the most rows (a 16.8 million-row forward, and tgmm at its row limit).  Static scales
keep the oracle's work to the sampled outputs: only sampled slices leave the GPU."""

import numpy as np
import pytest
import torch

from oracle.fp8 import bf16_bits_to_f32
from oracle.gmm import gmm_dlhs_ref, gmm_fwd_ref, tgmm_ref
from oracle.quant import quantize_rhs_per_channel, quantize_with_inv, static_inv
from synth.workloads import bf16_to_bits, multinomial_sizes, normal_bf16
from tests.gpu_util import DEV, gs_tensor, sync
from tests.parity import TOL, group_rel_err, group_row_ranges, slab_rel_err, to_np

pytestmark = pytest.mark.gpu

S_LHS = float(np.float32(4.0) / np.float32(448.0))       # static lhs scale, bound 4
S_GRAD = float(np.float32(0.01) / np.float32(57344.0))   # static grad scale, bound 0.01


def _codes(t_bits, s, fmt):
    """Static-scale codes of bf16 bits (the oracle's quantizer)."""
    inv = static_inv(np.float32(s))
    return quantize_with_inv(bf16_bits_to_f32(t_bits), np.full(t_bits.shape[0], inv, np.float32), fmt)


def _rows_of(sizes, rng, per_group=4):
    off = np.concatenate([[0], np.cumsum(sizes)])
    rows = set()
    for g in range(len(sizes)):
        a, b = int(off[g]), int(off[g + 1])
        if b > a:
            rows.update({a, b - 1})
            rows.update(int(r) for r in rng.integers(a, b, size=per_group))
    return np.array(sorted(rows), np.int64)


def _sub_sizes(rows, sizes):
    off = np.concatenate([[0], np.cumsum(sizes)])
    return np.array([int(((rows >= off[g]) & (rows < off[g + 1])).sum()) for g in range(len(sizes))], np.int32)


def test_most_groups(lib):
    # G = 1024: 224 experts hold rows (multinomial), the other 800 are empty, so empty
    # and tiny groups alternate all through the tile order
    G, K, N = 1024, 128, 256
    live = set(np.random.default_rng(31).choice(G, size=224, replace=False).tolist())
    sizes = multinomial_sizes(20000, G, 32, empty=[g for g in range(G) if g not in live])
    M = int(sizes.sum())
    print(f"most groups: G={G} M={M}", flush=True)
    x = normal_bf16((M, K), 1.0, 33, DEV)
    w = normal_bf16((G, K, N), 0.02, 34, DEV)
    gr = normal_bf16((M, N), 1e-3, 35, DEV)
    gs = gs_tensor(sizes)
    wq, ws = lib.gmm_quantize_rhs(w, "e4m3", 0, "nk")
    wk, sk = lib.gmm_quantize_rhs(w, "e4m3", 1, "kn")
    out = lib.gmm_fwd(x, wq, ws, gs, lhs_scaling="static", static_scale=S_LHS, out_dtype=torch.float32)
    dl = lib.gmm_dlhs(gr, wk, sk, gs, grad_scaling="static", static_scale=S_GRAD, out_dtype=torch.float32)
    dw = lib.tgmm_drhs(x, gr, gs, lhs_scaling="static", lhs_static_scale=S_LHS,
                       grad_scaling="static", grad_static_scale=S_GRAD, out_dtype=torch.float32)
    sync()
    xb, gb, wb = bf16_to_bits(x), bf16_to_bits(gr), bf16_to_bits(w)
    a_codes, g_codes = _codes(xb, S_LHS, "e4m3"), _codes(gb, S_GRAD, "e5m2")
    ranges = group_row_ranges(sizes)
    bq, bs = quantize_rhs_per_channel(wb, "e4m3", "n")
    R = gmm_fwd_ref(a_codes, "e4m3", np.full(M, S_LHS, np.float32), bq, "e4m3", bs, sizes)
    assert group_rel_err(to_np(out), R, ranges) <= TOL
    bq, bs = quantize_rhs_per_channel(wb, "e4m3", "k")
    R = gmm_dlhs_ref(g_codes, "e5m2", np.full(M, S_GRAD, np.float32), bq, "e4m3", bs, sizes)
    assert group_rel_err(to_np(dl), R, ranges) <= TOL
    nb = -(-M // 128)
    R = tgmm_ref(a_codes, "e4m3", np.full(nb, S_LHS, np.float32), g_codes, "e5m2",
                 np.full(nb, S_GRAD, np.float32), sizes)
    Y = to_np(dw)
    for g in np.flatnonzero(sizes == 0):
        assert (Y[g].view(np.uint32) == 0).all()
    assert slab_rel_err(Y, R) <= TOL


@pytest.mark.parametrize("op", ["fwd", "dlhs", "tgmm"])
def test_longest_contraction(lib, op):
    # fwd contracts over K = 2^22 and dlhs over N = 2^22; tgmm gets K = 2^22 output rows
    # per slab (its contraction is the 16 rows).  Two groups of 10 and 6 rows.
    sizes = np.array([10, 6], np.int32)
    M, L, W = 16, 1 << 22, 128  # rows, the long dimension, the short one
    rng = np.random.default_rng(41)
    gs = gs_tensor(sizes)
    ranges = group_row_ranges(sizes)
    print(f"longest contraction: {op} M={M} long={L}", flush=True)
    if op == "fwd":
        x = normal_bf16((M, L), 1.0, 42, DEV)
        w = normal_bf16((2, L, W), 0.02, 43, DEV)
        wq, ws = lib.gmm_quantize_rhs(w, "e4m3", 0, "nk")
        out = lib.gmm_fwd(x, wq, ws, gs, lhs_scaling="static", static_scale=S_LHS, out_dtype=torch.float32)
        sync()
        cols = np.sort(rng.choice(W, size=8, replace=False))
        ci = torch.as_tensor(cols, device=DEV)
        bq, bs = quantize_rhs_per_channel(bf16_to_bits(w[:, :, ci]), "e4m3", "n")
        R = gmm_fwd_ref(_codes(bf16_to_bits(x), S_LHS, "e4m3"), "e4m3", np.full(M, S_LHS, np.float32),
                        bq, "e4m3", bs, sizes)
        assert group_rel_err(to_np(out[:, ci]), R, ranges) <= TOL
    elif op == "dlhs":
        gr = normal_bf16((M, L), 1e-3, 44, DEV)
        w = normal_bf16((2, W, L), 0.02, 45, DEV)
        wk, sk = lib.gmm_quantize_rhs(w, "e4m3", 1, "kn")
        out = lib.gmm_dlhs(gr, wk, sk, gs, grad_scaling="static", static_scale=S_GRAD, out_dtype=torch.float32)
        sync()
        kc = np.sort(rng.choice(W, size=8, replace=False))
        ki = torch.as_tensor(kc, device=DEV)
        bq, bs = quantize_rhs_per_channel(bf16_to_bits(w[:, ki, :]), "e4m3", "k")
        R = gmm_dlhs_ref(_codes(bf16_to_bits(gr), S_GRAD, "e5m2"), "e5m2", np.full(M, S_GRAD, np.float32),
                         bq, "e4m3", bs, sizes)
        assert group_rel_err(to_np(out[:, ki]), R, ranges) <= TOL
    else:  # tgmm: K = 2^22 output rows per slab
        x = normal_bf16((M, L), 1.0, 46, DEV)
        gr = normal_bf16((M, W), 1e-3, 47, DEV)
        dw = lib.tgmm_drhs(x, gr, gs, lhs_scaling="static", lhs_static_scale=S_LHS,
                           grad_scaling="static", grad_static_scale=S_GRAD, out_dtype=torch.float32)
        sync()
        ks = np.sort(np.concatenate([[0, L - 1], rng.choice(L, size=14, replace=False)]))
        ki = torch.as_tensor(ks, device=DEV)
        R = tgmm_ref(_codes(bf16_to_bits(x[:, ki]), S_LHS, "e4m3"), "e4m3", np.full(1, S_LHS, np.float32),
                     _codes(bf16_to_bits(gr), S_GRAD, "e5m2"), "e5m2", np.full(1, S_GRAD, np.float32), sizes)
        assert slab_rel_err(to_np(dw[:, ki, :]), R) <= TOL


def test_widest_output(lib):
    # N = 2^22 output columns (16384 column tiles), two groups
    sizes = np.array([10, 6], np.int32)
    M, K, N = 16, 128, 1 << 22
    print(f"widest output: N={N}", flush=True)
    x = normal_bf16((M, K), 1.0, 51, DEV)
    w = normal_bf16((2, K, N), 0.02, 52, DEV)
    wq, ws = lib.gmm_quantize_rhs(w, "e4m3", 0, "nk")
    out = lib.gmm_fwd(x, wq, ws, gs_tensor(sizes), lhs_scaling="static", static_scale=S_LHS,
                      out_dtype=torch.float32)
    sync()
    rng = np.random.default_rng(53)
    cols = np.sort(np.concatenate([[0, N - 1], rng.choice(N, size=62, replace=False)]))
    ci = torch.as_tensor(cols, device=DEV)
    bq, bs = quantize_rhs_per_channel(bf16_to_bits(w[:, :, ci]), "e4m3", "n")
    R = gmm_fwd_ref(_codes(bf16_to_bits(x), S_LHS, "e4m3"), "e4m3", np.full(M, S_LHS, np.float32),
                    bq, "e4m3", bs, sizes)
    assert group_rel_err(to_np(out[:, ci]), R, group_row_ranges(sizes)) <= TOL


def test_most_rows_forward(lib):
    # 2^24 rows (65536 row tiles), groups of 2^23, 5 and the rest
    M, K, N = 1 << 24, 128, 128
    sizes = np.array([1 << 23, 5, (1 << 24) - (1 << 23) - 5], np.int32)
    print(f"most rows forward: M={M}", flush=True)
    x = normal_bf16((M, K), 1.0, 61, DEV)
    w = normal_bf16((3, K, N), 0.02, 62, DEV)
    wq, ws = lib.gmm_quantize_rhs(w, "e4m3", 0, "nk")
    out = lib.gmm_fwd(x, wq, ws, gs_tensor(sizes), lhs_scaling="static", static_scale=S_LHS,
                      out_dtype=torch.float32)
    sync()
    rows = _rows_of(sizes, np.random.default_rng(63))
    ri = torch.as_tensor(rows, device=DEV)
    bq, bs = quantize_rhs_per_channel(bf16_to_bits(w), "e4m3", "n")
    sub = _sub_sizes(rows, sizes)
    R = gmm_fwd_ref(_codes(bf16_to_bits(x[ri]), S_LHS, "e4m3"), "e4m3",
                    np.full(len(rows), S_LHS, np.float32), bq, "e4m3", bs, sub)
    assert group_rel_err(to_np(out[ri]), R, group_row_ranges(sub)) <= TOL


def test_tgmm_tall(lib):
    # 16.7 million rows in two groups: the row offsets of the operands pass 2^32 bytes
    # (M * K = 2^32 - 2^15 for the lhs), which every 128-row step rebases away
    G = 2
    M = (131071 - G) * 128
    sizes = np.array([M // 2 + 77, M - M // 2 - 77], np.int32)
    K, N = 256, 128
    print(f"tall tgmm: M={M}", flush=True)
    x = normal_bf16((M, K), 1.0, 71, DEV)
    gr = normal_bf16((M, N), 1e-3, 72, DEV)
    dw = lib.tgmm_drhs(x, gr, gs_tensor(sizes), lhs_scaling="static", lhs_static_scale=S_LHS,
                       grad_scaling="static", grad_static_scale=S_GRAD, out_dtype=torch.float32)
    sync()
    rng = np.random.default_rng(73)
    ks = np.sort(rng.choice(K, size=6, replace=False))
    ns = np.sort(rng.choice(N, size=6, replace=False))
    ki, ni = torch.as_tensor(ks, device=DEV), torch.as_tensor(ns, device=DEV)
    nb = -(-M // 128)
    R = tgmm_ref(_codes(bf16_to_bits(x[:, ki]), S_LHS, "e4m3"), "e4m3", np.full(nb, S_LHS, np.float32),
                 _codes(bf16_to_bits(gr[:, ni]), S_GRAD, "e5m2"), "e5m2", np.full(nb, S_GRAD, np.float32),
                 sizes)
    assert slab_rel_err(to_np(dw[:, ki][:, :, ni]), R) <= TOL
