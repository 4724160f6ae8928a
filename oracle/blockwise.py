"""Block-wise scales of the forward grouped matmul (oracle; test infrastructure).

Two scale layouts that the pages raise as extensions of the per-channel / per-tensor
recipes:

* block-wise weight scales, a 3-D scale [G, K/bk, N] ("Support quantization for tokamax
  gmm v2", review thread on the ops diff: a 3-D rhs scale is block-wise quantization);
* sub-channel lhs scales [M, K/bk] ("add static LHS scaling support for GMM v2 FWD",
  review thread on the lhs docstring: the scale's shape sets the granularity, extensible
  from per-tensor [1, 1] to [M, num_blocks]).

With bk contraction elements per block, block kb covers k in [kb bk, (kb + 1) bk).
The scales now vary along the contraction, so each block's partial sum is scaled before
it is added (the promotion the tgmm already applies to its 128-row blocks):

  partial_kb[m, n] = sum_{k in block kb} dq(a[m, k]) dq(b[g, k, n])      (float32)
  out[m, n]        = sum_kb RNE(RNE(partial_kb[m, n] * sA[m, kb]) * sB[g, kb, n])

summed in float32 from +0 in increasing kb.  With one block (bk = K) this is the
per-channel forward of ``gmm.gmm_fwd_ref`` exactly.  The quantizers follow the dynamic
recipe of ``quant`` (s = RNE(amax / qmax), inverse 0 when s is 0 or 1/s overflows,
clamp then round) with the abs-max taken over each block: a row's bk elements for the
lhs, a column's bk elements of one expert for the weights.

The dlhs can also run on the forward's weight copy, whose per-channel scales s[g, n]
lie on the dlhs contraction: they are folded into the gradient before it is quantized
(``quantize_folded``), and the product then takes unit output-channel scales.  With
block-wise scales the dlhs is the same block-wise product on the transposed weight: the
gradient gets sub-channel scales [M, N/bk] and the weight's dlhs copy one scale per
expert, output channel k and block of bk columns n ([G, K, N/bk]).

Parity: pinned by brute force with exact rationals on tiny inputs, by the one-block
reduction to the per-channel forward, by block-constant scales factoring out, and by the
quantizers' brute-force block abs-max; the fold by unit and power-of-two scales
(identical codes, scales multiplied exactly) and by the folded dlhs against the float64
definition within the quantization bound; the block-wise dlhs by brute force with exact
rationals and by its one-block reduction to the per-channel dlhs
(``tests/test_oracle_blockwise.py``).
"""

import numpy as np

from .fp8 import bf16_bits_to_f32, decode_fp8, encode_fp8
from .gmm import _finish, group_offsets
from .quant import dynamic_scale_from_amax, qmax_of


def _quantize(x_f32, inv, fmt):
    y = (np.asarray(x_f32, np.float32) * np.asarray(inv, np.float32)).astype(np.float32)
    q = qmax_of(fmt)
    return encode_fp8(np.minimum(np.maximum(y, -q), q), fmt)


def quantize_subchannel(x_bits, fmt, bk):
    """bf16 bits [M, K] -> (codes [M, K], scales [M, K/bk]): one dynamic scale per row and
    block of bk columns."""
    x = bf16_bits_to_f32(np.asarray(x_bits, np.uint16))
    M, K = x.shape
    assert K % bk == 0
    amax = np.abs(x).reshape(M, K // bk, bk).max(axis=2)
    s, inv = dynamic_scale_from_amax(amax, fmt)
    codes = _quantize(x, np.repeat(inv, bk, axis=1), fmt)
    return codes, s.astype(np.float32)


def quantize_rhs_blockwise(w_bits, fmt, bk):
    """bf16 bits [G, K, N] -> (codes [G, K, N], scales [G, K/bk, N]): one dynamic scale per
    expert, block of bk contraction rows and output column."""
    w = bf16_bits_to_f32(np.asarray(w_bits, np.uint16))
    G, K, N = w.shape
    assert K % bk == 0
    amax = np.abs(w).reshape(G, K // bk, bk, N).max(axis=2)
    s, inv = dynamic_scale_from_amax(amax, fmt)
    codes = _quantize(w, np.repeat(inv, bk, axis=1), fmt)
    return codes, s.astype(np.float32)


def gmm_fwd_blockwise_ref(a_codes, a_fmt, a_scale_kb, b_codes, b_fmt, b_scale_kb, group_sizes,
                          bk, out_dtype="f32"):
    """out[m, n] = sum_kb RNE(RNE(partial_kb * sA[m, kb]) * sB[g, kb, n]) for m in group g.

    a_codes [M, K], a_scale_kb [M, K/bk]; b_codes [G, K, N], b_scale_kb [G, K/bk, N]."""
    M, K = a_codes.shape
    G, Kb, N = b_codes.shape
    nkb = K // bk
    assert Kb == K and K % bk == 0
    assert a_scale_kb.shape == (M, nkb) and b_scale_kb.shape == (G, nkb, N)
    off = group_offsets(group_sizes, M)
    out = np.zeros((M, N), np.float32)
    sa = np.asarray(a_scale_kb, np.float32)
    sb = np.asarray(b_scale_kb, np.float32)
    for g in range(G):
        r0, r1 = off[g], off[g + 1]
        if r0 == r1:
            continue
        A = decode_fp8(a_codes[r0:r1], a_fmt)
        B = decode_fp8(b_codes[g], b_fmt)
        acc = np.zeros((r1 - r0, N), np.float32)
        for kb in range(nkb):
            ks = slice(kb * bk, (kb + 1) * bk)
            partial = np.matmul(A[:, ks], B[ks])  # float32 sums of exact products
            v = (partial * sa[r0:r1, kb][:, None]).astype(np.float32) * sb[g, kb][None, :]
            acc = (acc + v.astype(np.float32)).astype(np.float32)
        out[r0:r1] = acc
    return _finish(out, out_dtype)


def quantize_rhs_blockwise_dlhs(w_bits, fmt, bk):
    """bf16 bits [G, K, N] -> (codes [G, K, N], scales [G, K, N/bk]): the weight copy of the
    block-wise dlhs, whose contraction is n: one dynamic scale per expert, output channel
    k and block of bk columns n (the sub-channel recipe on the rows of w)."""
    w = np.asarray(w_bits, np.uint16)
    G, K, N = w.shape
    codes, s = quantize_subchannel(w.reshape(G * K, N), fmt, bk)
    return codes.reshape(G, K, N), s.reshape(G, K, N // bk)


def gmm_dlhs_blockwise_ref(g_codes, g_fmt, g_scale_kb, w_codes, w_fmt, w_scale_kb, group_sizes,
                           bk, out_dtype="f32"):
    """dlhs[m, k] = sum_nb RNE(RNE(partial_nb[m, k] * sG[m, nb]) * sW[g, k, nb]) for m in
    group g, partial_nb[m, k] = sum_{n in block nb} dq(grad[m, n]) dq(w[g, k, n]): the gmm
    against the transposed weight, with scales that vary along its contraction n.

    g_codes [M, N], g_scale_kb [M, N/bk]; w_codes [G, K, N], w_scale_kb [G, K, N/bk]."""
    return gmm_fwd_blockwise_ref(g_codes, g_fmt, g_scale_kb, np.transpose(w_codes, (0, 2, 1)),
                                 w_fmt, np.transpose(w_scale_kb, (0, 2, 1)), group_sizes, bk,
                                 out_dtype)


def quantize_folded(grad_bits, col_scales, group_sizes, fmt, block_rows=128):
    """The dlhs variant that folds the forward's per-channel weight scales into the
    gradient: y[m, n] = RNE_f32(grad[m, n] * s_fwd[g(m), n]) for the group g(m) of row m,
    then the dynamic 128-row-block recipe on y (abs-max over the block's full width,
    s = RNE(amax / qmax), inverse 0 when s is 0 or 1/s overflows, clamp then round).
    Returns (codes [M, N], scales [ceil(M / block_rows)]).  The dlhs on these codes uses
    the forward's codes with unit output-channel scales."""
    x = bf16_bits_to_f32(np.asarray(grad_bits, np.uint16))
    M, N = x.shape
    off = group_offsets(group_sizes, M)
    gid = np.repeat(np.arange(len(group_sizes)), np.diff(off))
    y = (x * np.asarray(col_scales, np.float32)[gid]).astype(np.float32)
    nb = -(-M // block_rows)
    amax = np.zeros(nb, np.float32)
    for b in range(nb):
        blk = y[b * block_rows:(b + 1) * block_rows]
        amax[b] = np.abs(blk).max() if blk.size else 0.0
    s, inv = dynamic_scale_from_amax(amax, fmt)
    codes = _quantize(y, np.repeat(inv, block_rows)[:M, None], fmt)
    return codes, s.astype(np.float32)
