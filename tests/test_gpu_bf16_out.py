"""The bf16 outputs of every product are the f32 outputs of the same call rounded to
nearest even: the two output dtypes share every step up to the final conversion, so this
holds bit for bit at any size, subnormal results included."""

import numpy as np
import pytest
import torch

from oracle.fp8 import f32_to_bf16_bits
from tests.gpu_util import gen, gs_tensor
from tests.parity import to_np

pytestmark = pytest.mark.gpu

F32_TINY = np.float32(1.1754944e-38)

# sigma of (lhs, weights, dlhs grad, tgmm grad).  "subnormal": fwd and dlhs outputs near
# 1e-40 (1e-8 x 1e-33 summed), and a tgmm scale product that is itself subnormal
# (about 2e-11 x 8e-35), so its outputs are too.
SIGMAS = {"normal": (1.0, 0.02, 1e-3, 1e-3), "subnormal": (1e-8, 1e-33, 1e-8, 1e-30)}


@pytest.mark.parametrize("magnitude", ["normal", "subnormal"])
def test_bf16_outputs_are_rne_of_f32_outputs(lib, magnitude):
    xs, wsig, gds, gts = SIGMAS[magnitude]
    sizes = [300, 0, 213, 1]
    M, K, N = sum(sizes), 384, 512
    x, _ = gen((M, K), xs, 411)
    w, _ = gen((len(sizes), K, N), wsig, 412)
    gd, _ = gen((M, N), gds, 413)
    gt, _ = gen((M, N), gts, 414)
    gs = gs_tensor(sizes)
    wq, ws = lib.gmm_quantize_rhs(w, "e4m3", 0, "nk")
    wk, sk = lib.gmm_quantize_rhs(w, "e4m3", 1, "kn")
    xq, sx = lib.gmm_quantize(x, "e4m3", "dynamic")
    gdq, sgd = lib.gmm_quantize(gd, "e5m2", "dynamic")
    gtq, sgt = lib.gmm_quantize(gt, "e5m2", "dynamic")
    calls = {
        # in-kernel quantization of a bf16 lhs, and fp8 codes, in both weight layouts
        "fwd fused": lambda dt: lib.gmm_fwd(x, wq, ws, gs, out_dtype=dt),
        "fwd fused, [G,K,N] weights": lambda dt: lib.gmm_fwd(x, wk, ws, gs, rhs_layout="kn", out_dtype=dt),
        "fwd codes": lambda dt: lib.gmm_fwd(xq, wq, ws, gs, lhs_scales=sx, out_dtype=dt),
        "fwd codes, [G,K,N] weights": lambda dt: lib.gmm_fwd(xq, wk, ws, gs, lhs_scales=sx,
                                                             rhs_layout="kn", out_dtype=dt),
        "dlhs codes": lambda dt: lib.gmm_dlhs(gdq, wk, sk, gs, grad_scales=sgd, out_dtype=dt),
        "tgmm codes": lambda dt: lib.tgmm_drhs(xq, gtq, gs, lhs_scales=sx, grad_scales=sgt,
                                               out_dtype=dt),
        "tgmm bf16": lambda dt: lib.tgmm_drhs(x, gt, gs, out_dtype=dt),
    }
    for name, f in calls.items():
        Y = to_np(f(torch.float32))
        Ybf = to_np(f(torch.bfloat16))
        assert np.array_equal(Ybf, f32_to_bf16_bits(Y)), name
        if magnitude == "subnormal":
            assert ((Y != 0) & (np.abs(Y) < F32_TINY)).any(), f"{name}: no subnormal result"
