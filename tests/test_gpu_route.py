"""GPU parity of the token routing around the grouped products: gmm_permute (stable sort
by expert, group sizes, row gather of bf16 values or fp8 codes) and gmm_unpermute (the
weighted combine), bit for bit against the oracle, and a permute -> gmm_fwd -> unpermute
chain."""

import numpy as np
import pytest
import torch

from oracle.fp8 import bf16_bits_to_f32, bf16_round
from oracle.gmm import gmm_fwd_ref
from oracle.quant import quantize_rhs_per_channel, quantize_static
from oracle.route import gather_rows_ref, permute_ref, unpermute_ref
from synth.workloads import topk_expert_ids
from tests.gpu_util import DEV, gen, sync
from tests.parity import to_np

pytestmark = pytest.mark.gpu


def ids_tensor(ids):
    return torch.as_tensor(np.ascontiguousarray(ids, np.int32), device=DEV)


@pytest.mark.parametrize("T,k,G,drop,H", [
    (0, 2, 8, 0.0, 64),          # no tokens: every expert empty
    (1, 1, 1, 0.0, 8),           # one slot
    (1000, 2, 8, 0.0, 2048),     # top-2 over 8 experts
    (777, 8, 64, 0.05, 1408),    # top-8 with dropped choices, a ragged last chunk
    (3000, 6, 1024, 0.1, 72),    # the largest expert count
    (300, 4, 3, 0.9, 256),       # mostly dropped
    (500, 3, 5, 0.2, 16),        # odd top-k, 32-byte rows
    (40, 64, 128, 0.0, 64),      # the largest top-k
])
def test_permute_matches_oracle(lib, T, k, G, drop, H):
    if G < k:  # fewer experts than choices: repeats allowed (random ids, some out of range)
        ids = np.random.default_rng(T).integers(-1, G + 1, (T, k)).astype(np.int32)
    else:
        ids = topk_expert_ids(T, k, G, 1.1, 900 + T, drop) if T else np.zeros((0, k), np.int32)
    x, xb = gen((T, H), 1.0, 901)
    xp, gs, ros, sor = lib.gmm_permute(ids_tensor(ids), G, x)
    sync()
    gs_r, ros_r, sor_r = permute_ref(ids, G)
    assert np.array_equal(to_np(gs), gs_r)
    assert np.array_equal(to_np(ros), ros_r)
    assert np.array_equal(to_np(sor), sor_r)
    assert np.array_equal(to_np(xp), gather_rows_ref(xb, sor_r, k))
    # fp8 codes of a static scale move the same way (quantize before the sort; their rows
    # must be whole 16-byte pieces)
    if T and H % 16 == 0:
        codes, _ = quantize_static(xb, 4.0 / 448.0, "e4m3")
        cp, gs2, _, _ = lib.gmm_permute(ids_tensor(ids), G, torch.as_tensor(codes, device=DEV))
        sync()
        assert np.array_equal(to_np(gs2), gs_r)
        assert np.array_equal(to_np(cp), gather_rows_ref(codes, sor_r, k))


@pytest.mark.parametrize("weighted", [True, False])
@pytest.mark.parametrize("k", [1, 3, 4, 6])
def test_unpermute_matches_oracle(lib, weighted, k):
    T, G, H = 1500, 16, 2048
    ids = topk_expert_ids(T, k, G, 1.2, 910, 0.1)
    _, ros, _ = lib.gmm_permute(ids_tensor(ids), G)
    _, ros_r, _ = permute_ref(ids, G)
    y, yb = gen((T * k, H), 1.0, 911)
    w = np.random.default_rng(912).random((T, k)).astype(np.float32) if weighted else None
    out = lib.gmm_unpermute(y, ros, None if w is None else torch.as_tensor(w, device=DEV))
    sync()
    _, bits = unpermute_ref(bf16_bits_to_f32(yb), ros_r, w)
    assert np.array_equal(to_np(out), bits)


def test_route_gmm_chain(lib):
    """permute -> gmm_fwd (static e4m3 lhs, per-channel weights) -> unpermute; the output
    lies within the rounding of the oracle's chain (each gmm output may be one bf16 ulp
    from the oracle's, the combine weighs them)."""
    T, k, G, K, N = 2000, 4, 16, 256, 384
    ids = topk_expert_ids(T, k, G, 1.2, 920, 0.02)
    x, xb = gen((T, K), 1.0, 921)
    w, wb = gen((G, K, N), 0.02, 922)
    cw = np.random.default_rng(923).random((T, k)).astype(np.float32)
    wq, ws = lib.gmm_quantize_rhs(w, "e4m3", 0, "nk")
    s = 4.0 / 448.0
    xp, gs, ros, _ = lib.gmm_permute(ids_tensor(ids), G, x)
    # the dropped slots' rows follow the routed ones: one more group, with zero weights
    M = T * k
    tail = torch.zeros(1, dtype=torch.int32, device=DEV)
    gs_all = torch.cat([gs, tail])
    gs_all[G] = M - gs.sum()
    wq_all = torch.cat([wq, torch.zeros_like(wq[:1])])
    ws_all = torch.cat([ws, torch.ones_like(ws[:1])])
    y = lib.gmm_fwd(xp, wq_all, ws_all, gs_all, lhs_scaling="static", static_scale=s)
    out = lib.gmm_unpermute(y, ros, torch.as_tensor(cw, device=DEV))
    sync()
    gs_r, ros_r, sor_r = permute_ref(ids, G)
    n = int(gs_r.sum())
    a_codes, _ = quantize_static(gather_rows_ref(xb, sor_r[:n], k), s, "e4m3")
    b_codes, b_s = quantize_rhs_per_channel(wb, "e4m3", "n")
    R = gmm_fwd_ref(a_codes, "e4m3", np.full(n, s, np.float32), b_codes, "e4m3", b_s, gs_r)
    yr = bf16_round(np.asarray(R, np.float32))
    ref, _ = unpermute_ref(yr, ros_r, cw)
    live = ros_r >= 0
    slack = np.zeros_like(ref, dtype=np.float64)
    for j in range(k):
        r = np.where(live[:, j], ros_r[:, j], 0)
        slack += live[:, j, None] * np.abs(cw[:, j, None]) * np.abs(yr[r]).astype(np.float64) * 2.0 ** -7
    got = bf16_bits_to_f32(to_np(out)).astype(np.float64)
    assert np.all(np.abs(got - ref) <= slack + np.abs(ref) * 2.0 ** -8 + 1e-30)


def test_route_full_size(lib):
    """The SwiGLU block's routing at full size: 8192 tokens x top-8 of 64 experts (Zipf 1.3
    popularity), hidden 2048, bf16 rows; permute and the weighted combine bit for bit."""
    T, k, G, H = 8192, 8, 64, 2048
    ids = topk_expert_ids(T, k, G, 1.3, 5)
    x, xb = gen((T, H), 1.0, 930)
    xp, gs, ros, sor = lib.gmm_permute(ids_tensor(ids), G, x)
    sync()
    gs_r, ros_r, sor_r = permute_ref(ids, G)
    assert np.array_equal(to_np(gs), gs_r) and np.array_equal(to_np(ros), ros_r)
    assert np.array_equal(to_np(sor), sor_r)
    assert np.array_equal(to_np(xp), gather_rows_ref(xb, sor_r, k))
    w = np.random.default_rng(931).random((T, k)).astype(np.float32)
    out = lib.gmm_unpermute(xp, ros, torch.as_tensor(w, device=DEV))
    sync()
    _, bits = unpermute_ref(bf16_bits_to_f32(gather_rows_ref(xb, sor_r, k)), ros_r, w)
    assert np.array_equal(to_np(out), bits)
