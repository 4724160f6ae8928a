"""GPU parity of the block-wise scales: gmm_quantize_subchannel and
gmm_quantize_rhs_blockwise byte for byte, gmm_fwd_blockwise against the oracle's
per-block promotion (ragged groups, empty ones, several block sizes), its one-block case
against gmm_fwd, and a sampled check at the Mixtral gate|up shape."""

import numpy as np
import pytest
import torch

from oracle.blockwise import gmm_fwd_blockwise_ref, quantize_rhs_blockwise, quantize_subchannel
from synth.workloads import bf16_to_bits, normal_bf16
from tests.gpu_util import DEV, gen, gs_tensor, sync
from tests.parity import TOL, assert_bf16_close, group_rel_err, group_row_ranges, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("bk", [128, 256, 512])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_quantizers_match_oracle(lib, bk, fmt):
    M, K, G, N = 300, 1024, 3, 256
    x_cpu = normal_bf16((M, K), 1.0, 701, "cpu")
    x_cpu[5, :bk] = 0  # an all-zero block
    x, xb = x_cpu.to(DEV), bf16_to_bits(x_cpu)
    codes, s = lib.gmm_quantize_subchannel(x, bk, fmt)
    w, wb = gen((G, K, N), 0.02, 702)
    wq, ws = lib.gmm_quantize_rhs_blockwise(w, bk, fmt, "kn")
    wq_nk, ws2 = lib.gmm_quantize_rhs_blockwise(w, bk, fmt, "nk")
    sync()
    c_ref, s_ref = quantize_subchannel(xb, fmt, bk)
    assert np.array_equal(to_np(codes), c_ref)
    assert np.array_equal(to_np(s).view(np.uint32), s_ref.view(np.uint32))
    wc_ref, ws_ref = quantize_rhs_blockwise(wb, fmt, bk)
    assert np.array_equal(to_np(wq), wc_ref)
    assert np.array_equal(to_np(wq_nk), np.transpose(wc_ref, (0, 2, 1)))
    assert np.array_equal(to_np(ws).view(np.uint32), ws_ref.view(np.uint32))
    assert np.array_equal(to_np(ws2).view(np.uint32), ws_ref.view(np.uint32))


@pytest.mark.parametrize("bk", [128, 256, 512])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_fwd_blockwise_ragged(lib, bk, out_dtype):
    sizes = [0, 260, 1, 0, 129, 300]
    G, M, K, N = len(sizes), sum(sizes), 1024, 384
    x, xb = gen((M, K), 1.0, 711)
    w, wb = gen((G, K, N), 0.02, 712)
    codes, s = lib.gmm_quantize_subchannel(x, bk)
    wq, ws = lib.gmm_quantize_rhs_blockwise(w, bk)
    out = lib.gmm_fwd_blockwise(codes, s, wq, ws, gs_tensor(sizes), bk, out_dtype=out_dtype)
    sync()
    c_ref, s_ref = quantize_subchannel(xb, "e4m3", bk)
    wc_ref, ws_ref = quantize_rhs_blockwise(wb, "e4m3", bk)
    R = gmm_fwd_blockwise_ref(c_ref, "e4m3", s_ref, wc_ref, "e4m3", ws_ref, sizes, bk)
    ranges = group_row_ranges(sizes)
    if out_dtype == torch.float32:
        err = group_rel_err(to_np(out), R, ranges)
        print(f"bk {bk}: max group relative error {err:.3e}")
        assert err <= TOL, err
    else:
        assert_bf16_close(to_np(out), R, ranges)


def test_fwd_blockwise_scales_vary_by_block(lib):
    """Weights whose blocks differ in magnitude by up to 2^20 (scales that a per-channel
    recipe could not share), e5m2 lhs codes."""
    sizes = [200, 56]
    G, M, K, N, bk = 2, 256, 1024, 256, 128
    x, xb = gen((M, K), 1.0, 721)
    w32 = torch.randn((G, K, N), generator=torch.Generator().manual_seed(722)) * 0.02
    w32 *= torch.exp2(torch.arange(K // bk).repeat_interleave(bk).float() * 2.5 - 10)[None, :, None]
    w_cpu = w32.to(torch.bfloat16)
    w = w_cpu.to(x.device)
    codes, s = lib.gmm_quantize_subchannel(x, bk, "e5m2")
    wq, ws = lib.gmm_quantize_rhs_blockwise(w, bk)
    out = lib.gmm_fwd_blockwise(codes, s, wq, ws, gs_tensor(sizes), bk, lhs_format="e5m2",
                                out_dtype=torch.float32)
    sync()
    c_ref, s_ref = quantize_subchannel(xb, "e5m2", bk)
    wc_ref, ws_ref = quantize_rhs_blockwise(to_np(w_cpu), "e4m3", bk)
    R = gmm_fwd_blockwise_ref(c_ref, "e5m2", s_ref, wc_ref, "e4m3", ws_ref, sizes, bk)
    assert group_rel_err(to_np(out), R, group_row_ranges(sizes)) <= TOL


def test_one_block_matches_gmm_fwd(lib):
    """bk = K: one scale per row and per channel, the per-channel forward on the same codes
    and scales (two kernels, so within the fp32 metric)."""
    sizes = [100, 0, 412]
    G, M, K, N = 3, 512, 512, 256
    x, _ = gen((M, K), 1.0, 731)
    w, _ = gen((G, K, N), 0.02, 732)
    codes, s = lib.gmm_quantize_subchannel(x, K)
    wq, ws = lib.gmm_quantize_rhs_blockwise(w, K)
    out = lib.gmm_fwd_blockwise(codes, s, wq, ws, gs_tensor(sizes), K, out_dtype=torch.float32)
    wq2, ws2 = lib.gmm_quantize_rhs(w, "e4m3", 0, "nk")
    assert torch.equal(wq, wq2) and torch.equal(ws[:, 0, :], ws2)
    # the per-channel forward with these per-row scales: scale each row's output after
    ref = lib.gmm_fwd(codes, wq2, ws2, gs_tensor(sizes), lhs_scaling="static", static_scale=1.0,
                      out_dtype=torch.float32)
    sync()
    R = to_np(ref).astype(np.float64) * to_np(s)[:, :1].astype(np.float64)
    assert group_rel_err(to_np(out), R, group_row_ranges(sizes)) <= TOL


def test_blockwise_mixtral_full_size_sampled(lib):
    """gmm_fwd_blockwise at the Mixtral gate|up shape with bk = 128, as the benchmark
    launches it: sampled rows x sampled columns against the oracle (every scale depends
    on its own row or column only, so the samples are quantized independently)."""
    from synth.workloads import WORKLOADS
    from tests.test_gpu_full import sample_cols, sample_rows, sampled_sizes

    wl = WORKLOADS["mixtral_gate_up"]
    G, M, K, N, bk = wl.G, wl.M, wl.K, wl.N, 128
    sizes = wl.group_sizes()
    x = normal_bf16((M, K), 1.0, wl.seed * 100 + 11, DEV)
    w = normal_bf16((G, K, N), 0.02, wl.seed * 100 + 12, DEV)
    codes, s = lib.gmm_quantize_subchannel(x, bk)
    wq, ws = lib.gmm_quantize_rhs_blockwise(w, bk)
    out = lib.gmm_fwd_blockwise(codes, s, wq, ws, gs_tensor(sizes), bk, out_dtype=torch.float32)
    sync()
    rng = np.random.default_rng(17)
    rows = sample_rows(sizes, rng)
    cols = sample_cols(N, rng, 48)
    ri, ci = torch.as_tensor(rows, device=DEV), torch.as_tensor(cols, device=DEV)
    c_ref, s_ref = quantize_subchannel(bf16_to_bits(x[ri]), "e4m3", bk)
    wc_ref, ws_ref = quantize_rhs_blockwise(bf16_to_bits(w[:, :, ci]), "e4m3", bk)
    sub = sampled_sizes(rows, sizes)
    R = gmm_fwd_blockwise_ref(c_ref, "e4m3", s_ref, wc_ref, "e4m3", ws_ref, sub, bk)
    err = group_rel_err(to_np(out[ri][:, ci]), R, group_row_ranges(sub))
    print(f"sampled max group relative error {err:.3e}", flush=True)
    assert err <= TOL, err


@pytest.mark.parametrize("sizes", [[300, 0, 212, 1], [640]])
def test_folded_dlhs(lib, sizes):
    """The one-weight-copy dlhs: the gradient folded with the forward's per-channel scales
    (codes and scales byte for byte), then gmm_dlhs on the forward's codes with unit
    output-channel scales, against the oracle."""
    from oracle.blockwise import quantize_folded
    from oracle.gmm import gmm_dlhs_ref, row_scales
    from oracle.quant import quantize_rhs_per_channel

    G, M, K, N = len(sizes), sum(sizes), 256, 512
    gr, grb = gen((M, N), 1e-3, 741)
    w, wb = gen((G, K, N), 0.02, 742)
    gs = gs_tensor(sizes)
    wq, ws = lib.gmm_quantize_rhs(w, "e4m3", 0, "kn")  # the forward copy: [G, K, N], s[g, n]
    codes, s = lib.gmm_quantize_folded(gr, ws, gs)
    ones = torch.ones((G, K), dtype=torch.float32, device=gr.device)
    out = lib.gmm_dlhs(codes, wq, ones, gs, grad_scaling="dynamic", grad_scales=s,
                       rhs_layout="kn", out_dtype=torch.float32)
    sync()
    wq_ref, ws_ref = quantize_rhs_per_channel(wb, "e4m3", "n")
    c_ref, s_ref = quantize_folded(grb, ws_ref, sizes, "e5m2")
    assert np.array_equal(to_np(codes), c_ref)
    assert np.array_equal(to_np(s).view(np.uint32), s_ref.view(np.uint32))
    R = gmm_dlhs_ref(c_ref, "e5m2", row_scales(s_ref, M), wq_ref, "e4m3",
                     np.ones((G, K), np.float32), sizes)
    assert group_rel_err(to_np(out), R, group_row_ranges(sizes)) <= TOL


@pytest.mark.parametrize("bk", [128, 256])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_dlhs_blockwise_ragged(lib, bk, out_dtype):
    """gmm_dlhs_blockwise: the gradient's sub-channel codes and the weight's dlhs copy
    (one scale per expert, output channel k and n-block) byte for byte, then the product
    against the oracle's block-wise dlhs (f32: per-group metric and elementwise bound)."""
    from oracle.blockwise import gmm_dlhs_blockwise_ref, quantize_rhs_blockwise_dlhs
    from tests.parity import assert_rounding_bound, magnitudes

    sizes = [0, 260, 1, 0, 129, 300]
    G, M, K, N = len(sizes), sum(sizes), 384, 1024
    gr, grb = gen((M, N), 1e-3, 721)
    w, wb = gen((G, K, N), 0.02, 722)
    codes, s = lib.gmm_quantize_subchannel(gr, bk, "e5m2")
    wq, ws = lib.gmm_quantize_rhs_blockwise_dlhs(w, bk)
    out = lib.gmm_dlhs_blockwise(codes, s, wq, ws, gs_tensor(sizes), bk, out_dtype=out_dtype)
    sync()
    c_ref, s_ref = quantize_subchannel(grb, "e5m2", bk)
    wc_ref, ws_ref = quantize_rhs_blockwise_dlhs(wb, "e4m3", bk)
    assert np.array_equal(to_np(codes), c_ref)
    assert np.array_equal(to_np(s).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(to_np(wq), wc_ref)
    assert np.array_equal(to_np(ws).view(np.uint32), ws_ref.view(np.uint32))
    R = gmm_dlhs_blockwise_ref(c_ref, "e5m2", s_ref, wc_ref, "e4m3", ws_ref, sizes, bk)
    ranges = group_row_ranges(sizes)
    if out_dtype == torch.float32:
        err = group_rel_err(to_np(out), R, ranges)
        print(f"dlhs bk {bk}: max group relative error {err:.3e}")
        assert err <= TOL, err
        absR = gmm_dlhs_blockwise_ref(magnitudes(c_ref), "e5m2", s_ref, magnitudes(wc_ref),
                                      "e4m3", ws_ref, sizes, bk)
        assert_rounding_bound(to_np(out), R, absR, N)
    else:
        assert_bf16_close(to_np(out), R, ranges)


def test_dlhs_blockwise_mixtral_full_size_sampled(lib):
    """gmm_dlhs_blockwise at the Mixtral gate|up shape with bk = 512, as the benchmark
    launches it: the gradient's sub-channel codes and the weight's dlhs copy, then the
    product on sampled rows x sampled output channels k against the oracle (a row's grad
    scales depend on that row only, and the dlhs copy's scales of channel k on row k of
    each expert's weight only, so the samples quantize as in the whole)."""
    from synth.workloads import WORKLOADS
    from oracle.blockwise import gmm_dlhs_blockwise_ref, quantize_rhs_blockwise_dlhs
    from tests.parity import assert_rounding_bound, magnitudes
    from tests.test_gpu_full import sample_cols, sample_rows, sampled_sizes

    wl = WORKLOADS["mixtral_gate_up"]
    G, M, K, N, bk = wl.G, wl.M, wl.K, wl.N, 512
    sizes = wl.group_sizes()
    grad = normal_bf16((M, N), 1e-3, wl.seed * 100 + 13, DEV)
    w = normal_bf16((G, K, N), 0.02, wl.seed * 100 + 12, DEV)
    gq, gsc = lib.gmm_quantize_subchannel(grad, bk, "e5m2")
    wq, ws = lib.gmm_quantize_rhs_blockwise_dlhs(w, bk)
    out = lib.gmm_dlhs_blockwise(gq, gsc, wq, ws, gs_tensor(sizes), bk, out_dtype=torch.float32)
    sync()
    rng = np.random.default_rng(19)
    rows = sample_rows(sizes, rng)
    kc = sample_cols(K, rng, 40)
    ri, ki = torch.as_tensor(rows, device=DEV), torch.as_tensor(kc, device=DEV)
    c_ref, s_ref = quantize_subchannel(bf16_to_bits(grad[ri]), "e5m2", bk)
    assert np.array_equal(to_np(gq[ri]), c_ref)
    assert np.array_equal(to_np(gsc[ri]).view(np.uint32), s_ref.view(np.uint32))
    wc_ref, ws_ref = quantize_rhs_blockwise_dlhs(bf16_to_bits(w[:, ki, :]), "e4m3", bk)
    assert np.array_equal(to_np(ws[:, ki, :]).view(np.uint32), ws_ref.view(np.uint32))
    sub = sampled_sizes(rows, sizes)
    R = gmm_dlhs_blockwise_ref(c_ref, "e5m2", s_ref, wc_ref, "e4m3", ws_ref, sub, bk)
    absR = gmm_dlhs_blockwise_ref(magnitudes(c_ref), "e5m2", s_ref, magnitudes(wc_ref), "e4m3",
                                  ws_ref, sub, bk)
    Y = to_np(out[ri][:, ki])
    err = group_rel_err(Y, R, group_row_ranges(sub))
    print(f"sampled max group relative error {err:.3e}", flush=True)
    assert err <= TOL, err
    assert_rounding_bound(Y, R, absR, N)

