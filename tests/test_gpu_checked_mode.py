"""Checked mode: with GMM_CHECK=1 every product copies group_sizes to the host, waits, and
returns GMM_ERR_GROUP_SIZES (7) for a negative size or sizes that do not sum to M, before
anything is enqueued; valid sizes run as usual."""

import numpy as np
import pytest
import torch

from tests.gpu_util import gen, gs_tensor, sync

pytestmark = pytest.mark.gpu

S = float(np.float32(4.0) / np.float32(448.0))


@pytest.fixture
def checked(monkeypatch):
    monkeypatch.setenv("GMM_CHECK", "1")


def _inputs(lib, M=300, K=256, N=256, G=3):
    x, _ = gen((M, K), 1.0, 951)
    gr, _ = gen((M, N), 1e-3, 952)
    w, _ = gen((G, K, N), 0.02, 953)
    wq, ws = lib.gmm_quantize_rhs(w, "e4m3", 0, "nk")
    wk, sk = lib.gmm_quantize_rhs(w, "e4m3", 1, "kn")
    return x, gr, wq, ws, wk, sk


@pytest.mark.parametrize("sizes", [[100, -1, 201], [100, 100, 99], [100, 100, 101], [301, 0, -1]])
def test_checked_mode_rejects_bad_group_sizes(lib, checked, sizes):
    x, gr, wq, ws, wk, sk = _inputs(lib)
    gs = gs_tensor(sizes)
    out = torch.full((300, 256), float("nan"), dtype=torch.float32, device=x.device)
    for call in (lambda: lib.gmm_fwd(x, wq, ws, gs, lhs_scaling="static", static_scale=S,
                                     out_dtype=torch.float32, out=out),
                 lambda: lib.gmm_dlhs(gr, wk, sk, gs, out_dtype=torch.float32, out=out),
                 lambda: lib.tgmm_drhs(x, gr, gs, out_dtype=torch.float32)):
        with pytest.raises(lib.GmmError) as e:
            call()
        assert e.value.status == 7  # GMM_ERR_GROUP_SIZES
    sync()
    assert torch.isnan(out).all()  # nothing was launched


def test_checked_mode_accepts_valid_sizes(lib, checked):
    x, gr, wq, ws, wk, sk = _inputs(lib)
    gs = gs_tensor([100, 0, 200])
    a = lib.gmm_fwd(x, wq, ws, gs, lhs_scaling="static", static_scale=S, out_dtype=torch.float32)
    t = lib.tgmm_drhs(x, gr, gs, out_dtype=torch.float32)
    sync()
    assert torch.isfinite(a).all() and torch.isfinite(t).all()
