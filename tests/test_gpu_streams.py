"""GPU: the two backward products on two streams (as the benchmark step runs them) write
the same bytes as on one stream: they share only read-only inputs (the grad codes and
scales), and every call enqueues its kernels on the stream it is given."""

import pytest
import torch

from tests.gpu_util import channel_varied, gen, gs_tensor, sync

pytestmark = pytest.mark.gpu


def test_backward_on_two_streams_equals_one_stream(lib):
    sizes = [700, 0, 1300, 513]
    M, K, N = sum(sizes), 512, 1024
    x, _ = gen((M, K), 1.0, 401)
    gr, _ = gen((M, N), 1e-3, 402)
    w, _ = channel_varied((len(sizes), K, N), 0.02, 403, 1)
    wk, sk = lib.gmm_quantize_rhs(w, "e4m3", 1, "kn")
    gs = gs_tensor(sizes)
    xq, sx = lib.gmm_quantize(x, "e4m3", "dynamic")
    gq, sg = lib.gmm_quantize(gr, "e5m2", "dynamic")
    d1 = lib.gmm_dlhs(gq, wk, sk, gs, grad_scales=sg)
    t1 = lib.tgmm_drhs(xq, gq, gs, lhs_scales=sx, grad_scales=sg)
    sync()
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    fork = torch.cuda.Event()
    fork.record(main)
    side.wait_event(fork)
    d2 = lib.gmm_dlhs(gq, wk, sk, gs, grad_scales=sg)
    with torch.cuda.stream(side):
        t2 = lib.tgmm_drhs(xq, gq, gs, lhs_scales=sx, grad_scales=sg)
        join = torch.cuda.Event()
        join.record(side)
    main.wait_event(join)
    sync()
    assert torch.equal(d1.view(torch.int16), d2.view(torch.int16))
    assert torch.equal(t1.view(torch.int16), t2.view(torch.int16))
