"""GPU parity of the SwiGLU steps: the merged gate|up forward with SwiGLU in its epilogue
(gmm_fwd_swiglu) and the elementwise backward (gmm_swiglu_bwd)."""

import numpy as np
import pytest
import torch

import oracle.ops as ops
from oracle.fp8 import bf16_bits_to_f32, f32_to_bf16_bits
from oracle.gmm import gmm_fwd_ref, row_scales
from oracle.quant import quantize_rhs_per_channel
from oracle.swiglu import swiglu_bwd_ref, swiglu_ref
from tests.gpu_util import gen, gs_tensor
from tests.parity import TOL, assert_bf16_close, group_rel_err, group_row_ranges, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("lhs_kind", ["codes", "bf16"])
def test_fused_swiglu_forward(lib, lhs_kind):
    # ragged groups with empty ones, I = 384 (3 channel-pair tiles), K tail of 256
    sizes = [0, 300, 5, 0, 457, 130]
    G, M, K, I = len(sizes), sum(sizes), 256, 384
    x, xb = gen((M, K), 1.0, 501)
    w, wb = gen((G, K, 2 * I), 0.02, 502)  # merged [W0 | W1] along N
    wq, ws = lib.gmm_quantize_rhs(w, "e4m3", 0, "nk")
    gs = gs_tensor(sizes)
    if lhs_kind == "codes":
        xq, sx = lib.gmm_quantize(x, "e4m3", "dynamic")
        lhs, kw = xq, dict(lhs_scales=sx)
    else:
        lhs, kw = x, {}
    a_codes, s_blk = ops.quantize_operand(xb, "e4m3", "dynamic")
    b_codes, b_s = quantize_rhs_per_channel(wb, "e4m3", "n")
    R = gmm_fwd_ref(a_codes, "e4m3", row_scales(s_blk, M), b_codes, "e4m3", b_s, sizes)
    Rh = swiglu_ref(R, I)
    ranges = group_row_ranges(sizes)
    for dt, view in ((torch.float32, torch.int32), (torch.bfloat16, torch.int16)):
        h, gu = lib.gmm_fwd_swiglu(lhs, wq, ws, gs, out_dtype=dt, gu=True, **kw)
        # the product half is exactly what gmm_fwd stores (GPU against GPU)
        plain = lib.gmm_fwd(lhs, wq, ws, gs, out_dtype=dt, **kw)
        assert torch.equal(gu.view(view), plain.view(view))
        if dt == torch.float32:
            err = group_rel_err(to_np(h), Rh, ranges)
            print(f"{lhs_kind}: max group relative error of h {err:.3e}")
            assert err <= TOL, err
        else:
            assert_bf16_close(to_np(h), Rh, ranges)
    # h alone (no gu) gives the same h
    h2 = lib.gmm_fwd_swiglu(lhs, wq, ws, gs, out_dtype=torch.float32, **kw)
    h1, _ = lib.gmm_fwd_swiglu(lhs, wq, ws, gs, out_dtype=torch.float32, gu=True, **kw)
    assert torch.equal(h1.view(torch.int32), h2.view(torch.int32))


def test_swiglu_backward(lib):
    M, I = 777, 384
    dh, dhb = gen((M, I), 1e-3, 511)
    gu, gub = gen((M, 2 * I), 2.0, 512)
    # saturated sigmoids too: g = +-60 and -100 (exp(100) overflows in fp32)
    gu[:3, :4] = torch.tensor([60.0, -60.0, -100.0, 0.0], dtype=torch.bfloat16, device=gu.device)
    gub = gu.to("cpu").view(torch.int16).numpy().view(np.uint16)
    d = lib.gmm_swiglu_bwd(dh, gu)
    R = swiglu_bwd_ref(bf16_bits_to_f32(dhb), bf16_bits_to_f32(gub), I)
    Y = bf16_bits_to_f32(to_np(d))
    assert np.all(np.abs(Y - R) <= np.abs(R) * 2.0 ** -7 + 1e-37)  # within one bf16 ulp
    exact = np.mean(to_np(d) == f32_to_bf16_bits(R))
    print(f"bf16 outputs equal to RNE of the exact value: {exact:.5f}")
    assert exact >= 0.99
