"""GPU: quantization codes and scales are byte-identical to the oracle's."""

import numpy as np
import pytest
import torch

from oracle.fp8 import bf16_bits_to_f32, decode_fp8
from oracle.gmm import gmm_fwd_ref, row_scales
from oracle.quant import (
    dynamic_scale_from_amax,
    quantize_rhs_per_channel,
    quantize_rowblock,
    quantize_static,
)
from tests.gpu_util import DEV, channel_varied, gen, gs_tensor
from tests.parity import to_np

pytestmark = pytest.mark.gpu

S_4_448 = float(np.float32(4.0) / np.float32(448.0))


def all_finite_bf16():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = bf16_bits_to_f32(bits)
    bits = bits[np.isfinite(f)]
    assert bits.size == 65280
    return bits.reshape(510, 128)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("s", [S_4_448, 1.0, 2.0 ** -10, 3.0, 1e-3, 0.37, 1e4, 2.0 ** 20, 7.1e-30])
def test_static_quantize_every_bf16(lib, fmt, s):
    bits = all_finite_bf16()
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    codes, _ = lib.gmm_quantize(x, fmt, "static", s)
    ref, _ = quantize_static(bits, np.float32(s), fmt)
    got = to_np(codes)
    bad = np.flatnonzero(got.ravel() != ref.ravel())
    assert bad.size == 0, (bits.ravel()[bad[:8]], got.ravel()[bad[:8]], ref.ravel()[bad[:8]])


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_dynamic_scales_every_bf16_absmax(lib, fmt):
    # one 128-row block per positive finite bf16 magnitude; its only non-zero element is
    # +-that magnitude, so the block abs-max runs through every bf16 value
    amax_bits = np.arange(1, 0x7F80, dtype=np.uint16)
    nb, C = amax_bits.size, 8
    X = np.zeros((nb * 128, C), np.uint16)
    b = np.arange(nb)
    sign = np.where(b % 2 == 1, 0x8000, 0).astype(np.uint16)
    X[b * 128 + (b % 128), b % C] = amax_bits | sign
    x = torch.from_numpy(X.view(np.int16)).view(torch.bfloat16).to(DEV)
    codes, scales = lib.gmm_quantize(x, fmt, "dynamic")
    s_ref, _ = dynamic_scale_from_amax(bf16_bits_to_f32(amax_bits), fmt)
    got_s = to_np(scales)
    assert np.array_equal(got_s.view(np.uint32), s_ref.view(np.uint32))
    c_ref, s_ref2, _ = quantize_rowblock(X, fmt)
    assert np.array_equal(s_ref2.view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(to_np(codes), c_ref)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_dynamic_quantize_real_tensor_ragged_rows(lib, fmt):
    x, bits = gen((1000, 384), 1.0 if fmt == "e4m3" else 1e-3, 31)
    codes, scales = lib.gmm_quantize(x, fmt, "dynamic")
    c_ref, s_ref, _ = quantize_rowblock(bits, fmt)
    assert np.array_equal(to_np(scales).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(to_np(codes), c_ref)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("layout", ["kn", "nk"])
def test_rhs_per_channel(lib, fmt, axis, layout):
    G, K, N = 3, 256, 384
    w, bits = channel_varied((G, K, N), 0.02, 41, 2 if axis == 0 else 1)
    codes, scales = lib.gmm_quantize_rhs(w, fmt, axis, layout)
    c_ref, s_ref = quantize_rhs_per_channel(bits, fmt, "n" if axis == 0 else "k")
    assert np.array_equal(to_np(scales).view(np.uint32), s_ref.view(np.uint32))
    got = to_np(codes)
    if layout == "nk":
        got = np.transpose(got, (0, 2, 1))
    assert np.array_equal(got, c_ref)


@pytest.mark.parametrize("scaling", ["static", "dynamic"])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fused_kernel_codes_through_identity_rhs(lib, scaling, fmt):
    """With rhs = identity (code 1.0, scale 1) the f32 forward output is dq(code) * s_row
    exactly, which exposes the codes the fused kernel formed in registers."""
    M, K = 700, 256
    sizes = [300, 0, 400]
    x, bits = gen((M, K), 1.0, 51)
    eye = np.zeros((3, K, K), np.uint8)
    for gi in range(3):
        eye[gi][np.arange(K), np.arange(K)] = 0x38  # e4m3 code of 1.0
    rhs = torch.from_numpy(eye).to(DEV)
    ones = torch.ones((3, K), dtype=torch.float32, device=DEV)
    s = S_4_448 if fmt == "e4m3" else 1.0 / 57344 * 4
    out, sc = lib.gmm_fwd(x, rhs, ones, gs_tensor(sizes), lhs_format=fmt, lhs_scaling=scaling,
                          static_scale=s, rhs_layout="nk", out_dtype=torch.float32,
                          return_scales=True)
    if scaling == "static":
        codes, _ = quantize_static(bits, np.float32(s), fmt)
        srow = np.full(M, np.float32(s), np.float32)
    else:
        codes, sblk, _ = quantize_rowblock(bits, fmt)
        srow = row_scales(sblk, M)
        assert np.array_equal(to_np(sc).view(np.uint32), sblk.view(np.uint32))
    ref = (decode_fp8(codes, fmt) * srow[:, None]).astype(np.float32)
    got = to_np(out)
    assert np.array_equal(got, ref)  # by value: a -0 code sums to +0 with the zero products
    # the oracle's own grouped product on this exact problem agrees bit for bit
    R = gmm_fwd_ref(codes, fmt, srow, eye, "e4m3", np.ones((3, K), np.float32), np.array(sizes))
    assert np.array_equal(got.view(np.uint32), R.view(np.uint32))
