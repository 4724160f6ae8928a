"""Recipe-level oracle entry points: quantize the bf16 operands, then run the grouped product.

These mirror the three library calls (forward, dlhs, drhs) one for one so that a test
can feed both sides the same bf16 inputs.  The lhs of every product is quantized here
exactly as the kernel is specified to do it in-flight: static per-tensor (scale s,
inverse RNE(1/s)) or dynamic per 128-row block (scale RNE(amax/qmax)).  A
pre-quantized lhs (codes + scales handed in) is also accepted, which is the case of
an activation that was quantized ahead of the product ("add static LHS scaling
support for GMM v2 FWD", PR #4735, the three lhs cases of the follow-up commits).
Test infrastructure only.
"""

import numpy as np

from .gmm import gmm_dlhs_ref, gmm_fwd_ref, row_scales, tgmm_ref
from .quant import quantize_rowblock, quantize_static, static_inv

BLOCK_ROWS = 128


def quantize_operand(x_bits, fmt, scaling, static_scale=None):
    """-> (codes [R, C], per-block scales [nb]) for 'static' or 'dynamic' scaling."""
    R = x_bits.shape[0]
    nb = -(-R // BLOCK_ROWS)
    if scaling == "static":
        codes, _ = quantize_static(x_bits, static_scale, fmt)
        return codes, np.full(nb, np.float32(static_scale), np.float32)
    if scaling == "dynamic":
        codes, s, _ = quantize_rowblock(x_bits, fmt, BLOCK_ROWS)
        return codes, s
    raise ValueError("scaling must be 'static' or 'dynamic'")


def fwd(lhs_bits, rhs_codes, rhs_scale, group_sizes, a_fmt="e4m3", a_scaling="dynamic",
        static_scale=None, b_fmt="e4m3", out_dtype="f32"):
    """gmm forward on a bf16 lhs -> (out, lhs codes, lhs block scales)."""
    codes, s_blk = quantize_operand(lhs_bits, a_fmt, a_scaling, static_scale)
    out = gmm_fwd_ref(codes, a_fmt, row_scales(s_blk, codes.shape[0]), rhs_codes, b_fmt,
                      rhs_scale, group_sizes, out_dtype)
    return out, codes, s_blk


def dlhs(grad_bits, rhs_codes, rhs_scale_k, group_sizes, a_fmt="e5m2", a_scaling="dynamic",
         static_scale=None, b_fmt="e4m3", out_dtype="f32"):
    """gmm dlhs on a bf16 grad -> (dlhs, grad codes, grad block scales)."""
    codes, s_blk = quantize_operand(grad_bits, a_fmt, a_scaling, static_scale)
    out = gmm_dlhs_ref(codes, a_fmt, row_scales(s_blk, codes.shape[0]), rhs_codes, b_fmt,
                       rhs_scale_k, group_sizes, out_dtype)
    return out, codes, s_blk


def tgmm(lhs_bits, grad_bits, group_sizes, a_fmt="e4m3", a_scaling="dynamic",
         a_static_scale=None, g_fmt="e5m2", g_scaling="dynamic", g_static_scale=None,
         out_dtype="f32"):
    """tgmm drhs on bf16 lhs and grad -> (drhs [G, K, N], lhs scales, grad scales)."""
    a_codes, sa = quantize_operand(lhs_bits, a_fmt, a_scaling, a_static_scale)
    g_codes, sg = quantize_operand(grad_bits, g_fmt, g_scaling, g_static_scale)
    out = tgmm_ref(a_codes, a_fmt, sa, g_codes, g_fmt, sg, group_sizes, BLOCK_ROWS, out_dtype)
    return out, sa, sg


def static_inverse(s):
    """RNE(1/s) for a validated static scale (re-exported for the tests)."""
    return static_inv(s)
