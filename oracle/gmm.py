"""Grouped (ragged) products on fp8 codes (oracle; test infrastructure).

The operations, as the pages define them:

* gmm forward ("FP8 Megablox for batch split", PR #3770, Description (1); "Support
  quantization for tokamax gmm v2", PR #4451, "What this does": fwd_gmm2): rows of
  lhs [M, K] are sorted by expert and split by ``group_sizes``; group g owns rows
  [off_g, off_g + m_g) and multiplies them by rhs[g] [K, N].
* gmm dlhs (PR #4451, the dlhs call in the review of ops.py): the lhs gradient is a
  gmm of grad [M, N] against rhs transposed, out [M, K].
* tgmm drhs (PR #4451, "What this does": drhs_tgmm2): the weight gradient of group g
  is lhs_g^T grad_g, a [K, N] slab; the result is [G, K, N].

Each product is the plain definition on dequantized operands: value = code * scale.
Products of two fp8 values are exact in float32; the sums are float32 sums (numpy's
float32 matmul), which is the fp32 accumulation the method specifies.  Scales that
are constant along the contraction factor out of the sum and are applied after it,
in the order (acc * s_row) * s_col; in tgmm the scales vary along the contraction
(one per 128-row block), so each block's partial sum is scaled by s_lhs[c] * s_grad[c]
before it is added.  Empty groups contribute no rows (gmm, dlhs) or an all-zero slab
(tgmm).

Local-expert window ("FP8 Megablox for batch split", the referencing commit's
Description item 3: the group_offset of the ragged products): with G_local experts from
group_offset on, group_sizes still lists every expert and the rows stay sorted by
expert; only the rows of the local experts are multiplied (by the local rhs), the other
output rows are zero, and tgmm yields the local experts' slabs.

Parity: pinned by brute force with exact rationals on tiny inputs, by float64 dense
loops over experts, by sums of per-row outer products and by the invariants listed in
``tests/test_oracle_gmm.py``; the windows by the full window (the plain products) and
by disjoint windows that tile the experts adding up to the plain products.
"""

import numpy as np

from .fp8 import decode_fp8, f32_to_bf16_bits


def group_offsets(group_sizes, M=None):
    """off_0 = 0, off_{g+1} = off_g + m_g; requires m_g >= 0 and (if given) sum == M."""
    gs = np.asarray(group_sizes, dtype=np.int64)
    if np.any(gs < 0):
        raise ValueError("group sizes must be non-negative")
    off = np.zeros(gs.size + 1, np.int64)
    off[1:] = np.cumsum(gs)
    if M is not None and off[-1] != M:
        raise ValueError(f"group sizes sum to {off[-1]}, expected {M}")
    return off


def _finish(R, out_dtype):
    R = np.asarray(R, dtype=np.float32)
    if out_dtype == "f32":
        return R
    if out_dtype == "bf16":
        return f32_to_bf16_bits(R)
    raise ValueError("out_dtype must be 'f32' or 'bf16'")


def gmm_fwd_ref(a_codes, a_fmt, a_scale_row, b_codes, b_fmt, b_scale, group_sizes,
                out_dtype="f32"):
    """out[m, n] = RNE((sum_k dq(a[m, k]) dq(b[g, k, n]) ) * s_a[m] * s_b[g, n]) for m in group g.

    a_codes [M, K] uint8, a_scale_row [M] float32 (the lhs dequant scale of every row),
    b_codes [G, K, N] uint8, b_scale [G, N] float32.  Returns f32 [M, N] or bf16 bits.
    """
    M, K = a_codes.shape
    G, Kb, N = b_codes.shape
    assert Kb == K and b_scale.shape == (G, N)
    off = group_offsets(group_sizes, M)
    out = np.zeros((M, N), np.float32)
    s_a = np.asarray(a_scale_row, np.float32)
    for g in range(G):
        r0, r1 = off[g], off[g + 1]
        if r0 == r1:
            continue
        A = decode_fp8(a_codes[r0:r1], a_fmt)
        B = decode_fp8(b_codes[g], b_fmt)
        acc = np.matmul(A, B)  # float32 operands: float32 accumulation
        out[r0:r1] = (acc * s_a[r0:r1, None]).astype(np.float32) * b_scale[g][None, :]
    return _finish(out, out_dtype)


def gmm_dlhs_ref(g_codes, g_fmt, g_scale_row, b_codes, b_fmt, b_scale_k, group_sizes,
                 out_dtype="f32"):
    """dlhs[m, k] = RNE((sum_n dq(grad[m, n]) dq(b[g, k, n])) * s_grad[m] * s_b[g, k]).

    The rhs is the same [G, K, N] tensor as in the forward, contracted over n (the
    gmm against rhs transposed); its scales are per dlhs output channel k: [G, K].
    """
    M, N = g_codes.shape
    G, K, Nb = b_codes.shape
    assert Nb == N and b_scale_k.shape == (G, K)
    off = group_offsets(group_sizes, M)
    out = np.zeros((M, K), np.float32)
    s_g = np.asarray(g_scale_row, np.float32)
    for g in range(G):
        r0, r1 = off[g], off[g + 1]
        if r0 == r1:
            continue
        A = decode_fp8(g_codes[r0:r1], g_fmt)
        B = decode_fp8(b_codes[g], b_fmt)
        acc = np.matmul(A, B.T)
        out[r0:r1] = (acc * s_g[r0:r1, None]).astype(np.float32) * b_scale_k[g][None, :]
    return _finish(out, out_dtype)


def tgmm_ref(a_codes, a_fmt, a_scale_blk, g_codes, g_fmt, g_scale_blk, group_sizes,
             block_rows=128, out_dtype="f32"):
    """drhs[g, k, n] = sum_c RNE(partial_c[k, n] * RNE(s_a[c] * s_grad[c])).

    partial_c = sum over rows m of group g inside row block c of dq(a[m, k]) dq(grad[m, n]).
    a_scale_blk / g_scale_blk hold one scale per ``block_rows``-row block (a static
    per-tensor scale is passed as a constant array).  Empty groups give +0.0 slabs.
    """
    M, K = a_codes.shape
    Mg, N = g_codes.shape
    assert Mg == M
    off = group_offsets(group_sizes, M)
    G = len(off) - 1
    out = np.zeros((G, K, N), np.float32)
    sa = np.asarray(a_scale_blk, np.float32)
    sg = np.asarray(g_scale_blk, np.float32)
    for g in range(G):
        r0, r1 = off[g], off[g + 1]
        if r0 == r1:
            continue
        acc = np.zeros((K, N), np.float32)
        for c in range(r0 // block_rows, (r1 - 1) // block_rows + 1):
            lo, hi = max(r0, c * block_rows), min(r1, (c + 1) * block_rows)
            A = decode_fp8(a_codes[lo:hi], a_fmt)
            B = decode_fp8(g_codes[lo:hi], g_fmt)
            partial = np.matmul(A.T, B)
            sc = np.float32(sa[c] * sg[c])
            acc = (acc + (partial * sc).astype(np.float32)).astype(np.float32)
        out[g] = acc
    return _finish(out, out_dtype)


def row_scales(scales_blk, M, block_rows=128):
    """Expand one scale per row block to one scale per row."""
    return np.repeat(np.asarray(scales_blk, np.float32), block_rows)[:M]


def _window_rows(group_sizes, group_offset, G_local):
    off = group_offsets(group_sizes)
    sizes = np.asarray(group_sizes, np.int64)[group_offset:group_offset + G_local]
    return int(off[group_offset]), int(off[group_offset + G_local]), sizes


def gmm_fwd_local_ref(a_codes, a_fmt, a_scale_row, b_codes_local, b_fmt, b_scale_local,
                      group_sizes, group_offset, out_dtype="f32"):
    """gmm_fwd_ref over the window of len(b_codes_local) experts from group_offset on;
    rows of the other experts are zero."""
    lo, hi, sizes = _window_rows(group_sizes, group_offset, b_codes_local.shape[0])
    out = np.zeros((a_codes.shape[0], b_codes_local.shape[2]), np.float32)
    out[lo:hi] = gmm_fwd_ref(a_codes[lo:hi], a_fmt, np.asarray(a_scale_row)[lo:hi],
                             b_codes_local, b_fmt, b_scale_local, sizes)
    return _finish(out, out_dtype)


def gmm_dlhs_local_ref(g_codes, g_fmt, g_scale_row, b_codes_local, b_fmt, b_scale_k_local,
                       group_sizes, group_offset, out_dtype="f32"):
    """gmm_dlhs_ref over the window (as gmm_fwd_local_ref); out [M, K]."""
    lo, hi, sizes = _window_rows(group_sizes, group_offset, b_codes_local.shape[0])
    out = np.zeros((g_codes.shape[0], b_codes_local.shape[1]), np.float32)
    out[lo:hi] = gmm_dlhs_ref(g_codes[lo:hi], g_fmt, np.asarray(g_scale_row)[lo:hi],
                              b_codes_local, b_fmt, b_scale_k_local, sizes)
    return _finish(out, out_dtype)


def tgmm_local_ref(a_codes, a_fmt, a_scale_blk, g_codes, g_fmt, g_scale_blk, group_sizes,
                   group_offset, G_local, block_rows=128, out_dtype="f32"):
    """The slabs group_offset .. group_offset + G_local - 1 of tgmm_ref (the 128-row scale
    blocks stay aligned to the global row index)."""
    full = tgmm_ref(a_codes, a_fmt, a_scale_blk, g_codes, g_fmt, g_scale_blk, group_sizes,
                    block_rows, "f32")
    return _finish(full[group_offset:group_offset + G_local], out_dtype)
