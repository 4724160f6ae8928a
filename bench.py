"""Benchmark of the FP8 grouped (ragged) matmul hot path on one MI355X.

One step is the whole path over one batch of an MoE expert layer, inputs resident in HBM
(default workload: the Mixtral-shaped merged gate|up layer, G=8 experts, K=4096,
N=2x14336=28672, M=16384 rows = 8192 tokens x top-2, Zipf(1.1) routing):

  1. quantize lhs once           e4m3 codes [M, K]: dynamic 128-row block scales (abs-max
                                  prepass + codes), or a static per-tensor scale 4/448 when
                                  the workload's forward recipe is static (no prepass)
  2. gmm_fwd   out[M, N]       = q(lhs) . rhs[g]          (the codes of step 1)
  3. quantize grad once          e5m2 codes [M, N] + 128-row block scales
  4. gmm_dlhs  dlhs[M, K]      = q(grad) . rhs[g]^T       (hybrid: the codes of step 3)
  5. tgmm_drhs drhs[G, K, N]   = q(lhs)_g^T . q(grad)_g   (the codes of steps 1 and 3)

value = 3 * 2*M*K*N / step time (TFLOP/s), the step on one HIP stream; the per-op figures
come from the same steps, every call timed with HIP events on that stream, and each
product gets the workspace gmm_workspace_size reports (for dlhs: its tail split).  The
slowest product is reported against the dense FP8 MFMA peak (5.0 PFLOP/s).  The step with
steps 4 and 5 (independent of each other) on two streams is timed beside it.

Also reported (each timed with HIP events on the current stream):
  * protocol: per op and for the whole step, the median and the minimum of `--reps` runs
    after 5 warm-up runs, warm, and cold (a 512 MiB device write between runs flushes the
    4 MB L2 of every XCD and the 256 MB last-level cache);
  * static_vs_dynamic: the workload's forward with a static per-tensor lhs scale and with
    dynamic 128-row block scales, both with the lhs quantized by the call and on
    pre-quantized codes (the pages say static scaling is slightly faster);
  * ffn_chain: the MoE SwiGLU feed-forward block (G=64, M=65536, hidden 2048,
    intermediate 1408), forward and backward as one timed chain, in pure mode (every
    product quantizes its own bf16 operands) and hybrid mode (each gradient quantized once,
    its codes feeding dlhs and tgmm), each with static and dynamic forward lhs scaling,
    and the hybrid static chain with the SwiGLU backward in the down dlhs's epilogue;
  * the SwiGLU, routing and block-wise blocks, and the CPU oracle on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--workload NAME]
       [--no-cpu-baseline] [--no-overlap] [--no-extras] [--no-clock] [--reps 50]
       python bench.py --crossover | --dense-only [--workload NAME] [--reps N]
"""

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 GMM TFLOP/s (fwd/dlhs/drhs) and % of MI355X FP8 MFMA peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
COUNTER_FILE = os.path.join(ROOT, "profiles", "mfma_counters.json")
FP8_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 MFMA
HBM_PEAK_GBS = 8000.0
STATIC_SCALE = float(np.float32(4.0) / np.float32(448.0))  # the pages' bound 4 over e4m3's 448


def kernel_source_hash():
    """sha256 (first 16 hex) over the HIP sources, as recorded with the counter summaries."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fp8_grouped_gemm_ragged_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp")):
            h.update(f.encode())
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def _summary(path, workload):
    """A committed counter summary for this workload, or None when there is none or the
    kernels changed since it was taken."""
    try:
        with open(path) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash():
        return None
    return t.get("workloads", {}).get(workload)


def measured_traffic(op, workload):
    """L2-to-fabric bytes per launch of `op` (FETCH_SIZE + WRITE_SIZE, scaled by a copy of
    known size) from the committed summary, or None."""
    t = _summary(TRAFFIC_FILE, workload)
    entry = t.get("ops", {}).get(op) if t else None
    return int(entry["traffic_bytes"]) if entry else None


def measured_counters(workload):
    """Per-op MFMA-busy fractions and L2 hit rates from the committed counter summary."""
    t = _summary(COUNTER_FILE, workload)
    return t.get("ops") if t else None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="mixtral_gate_up")
    p.add_argument("--reps", type=int, default=50, help="timed runs per op for median / min")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-overlap", action="store_true",
                   help="skip the extra timing of the step with dlhs and tgmm on two streams")
    p.add_argument("--no-extras", action="store_true",
                   help="only the timed steps: no protocol, static/dynamic, FFN chain or blocks")
    p.add_argument("--no-clock", action="store_true", help="skip the GFX clock reading")
    p.add_argument("--crossover", action="store_true",
                   help="only the fused-vs-quantize-once table of the forward (crossover_block)")
    p.add_argument("--dense-only", action="store_true",
                   help="only the vendor dense FP8 GEMM at the workload's shape (dense_ceiling), "
                        "--reps timed calls: the comparison run for counter profiles")
    p.add_argument("--cpu-sample-rows", type=int, default=1024)
    p.add_argument("--cpu-sample-cols", type=int, default=2048, help="at most 4096")
    p.add_argument("--copy-calibration", action="store_true",
                   help="copy 1 GiB device-to-device once before the steps (a known-size "
                        "transfer for scaling HBM byte counters)")
    return p.parse_args()


def _median_min(ts):
    ts = sorted(ts)
    return {"median_ms": round(float(np.median(ts)), 4), "min_ms": round(float(ts[0]), 4)}


def event_times(fn, reps, warmup=5, cold=None):
    """ms of each of `reps` calls of fn() (HIP events on the current stream around each),
    after `warmup` untimed calls; with `cold` (a uint8 tensor) every timed call follows a
    full write of it."""
    import torch

    for _ in range(warmup):
        fn()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    torch.cuda.synchronize()
    for i, (e0, e1) in enumerate(evs):
        if cold is not None:
            cold.fill_(i & 0xFF)
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in evs]


class Step:
    """Pre-allocated buffers and direct C-ABI calls for one pass of the path."""

    def __init__(self, g, wl, seed):
        import torch

        from synth.workloads import normal_bf16

        self.g, self.torch, self.wl = g, torch, wl
        lib = g.load()
        self.lib = lib
        dev = "cuda"
        G, M, K, N = wl.G, wl.M, wl.K, wl.N
        self.G, self.M, self.K, self.N = G, M, K, N
        self.static = wl.lhs_scaling == "static"
        self.sizes = wl.group_sizes()
        self.gs = torch.tensor(self.sizes, dtype=torch.int32, device=dev)
        self.lhs = normal_bf16((M, K), 1.0, seed, dev)
        self.grad = normal_bf16((M, N), 1e-3, seed + 2, dev)
        w = normal_bf16((G, K, N), 0.02, seed + 1, dev)
        # weights arrive pre-quantized: forward copy per output channel n stored [G, N, K]
        # (contraction contiguous), dlhs copy per output channel k stored [G, K, N]
        self.w_fwd, self.s_fwd = g.gmm_quantize_rhs(w, "e4m3", 0, "nk")
        self.w_dlhs, self.s_dlhs = g.gmm_quantize_rhs(w, "e4m3", 1, "kn")
        self.w_sample = w[:, :, :4096].to("cpu")  # for the CPU baseline sample only
        del w
        self.out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        self.dlhs = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        self.drhs = torch.empty((G, K, N), dtype=torch.bfloat16, device=dev)
        nb = (M + 127) // 128
        self.s_lhs = torch.empty(nb, dtype=torch.float32, device=dev)
        self.s_grad = torch.empty(nb, dtype=torch.float32, device=dev)
        self.grad_q = torch.empty((M, N), dtype=torch.uint8, device=dev)
        self.lhs_q = torch.empty((M, K), dtype=torch.uint8, device=dev)
        # quantizer workspace (the abs-max prepass), sized for the wider operand
        op = g.Operand(g.KIND_BF16, g.E4M3, g.DYNAMIC, 0.0)
        n = g._SZ()
        self._chk(lib.gmm_workspace_size(g.OP_QUANTIZE, ctypes.byref(op), ctypes.byref(op), M,
                                         max(K, N), 0, 1, ctypes.byref(n)))
        self.ws = torch.empty(max(n.value, 256), dtype=torch.uint8, device=dev)
        self.ws_n = n.value
        # each tensor is quantized once and its codes feed every product that uses it: lhs
        # codes -> fwd and tgmm (the workload's forward recipe), grad codes -> dlhs and tgmm
        lmode, ls = (g.STATIC, STATIC_SCALE) if self.static else (g.DYNAMIC, 0.0)
        self.op_lq = g.Operand(g.KIND_BF16, g.E4M3, lmode, ls)      # lhs quantizer recipe
        self.op_l8 = g.Operand(g.KIND_FP8, g.E4M3, lmode, ls)       # its codes
        self.op_gq = g.Operand(g.KIND_BF16, g.E5M2, g.DYNAMIC, 0.0)  # grad quantizer recipe
        self.op_g8 = g.Operand(g.KIND_FP8, g.E5M2, g.DYNAMIC, 0.0)   # its codes
        self._chk(lib.gmm_workspace_size(g.OP_TGMM, ctypes.byref(self.op_l8), ctypes.byref(self.op_g8),
                                         M, K, N, G, ctypes.byref(n)))
        self.ws_t = torch.empty(max(n.value, 256), dtype=torch.uint8, device=dev)
        self.ws_t_n = n.value
        # the products' own workspace: on large calls, the tail split's partial sums
        self._chk(lib.gmm_workspace_size(g.OP_FWD, ctypes.byref(self.op_l8), ctypes.byref(self.op_l8),
                                         M, K, N, G, ctypes.byref(n)))
        self.ws_f = torch.empty(max(n.value, 256), dtype=torch.uint8, device=dev)
        self.ws_f_n = n.value
        self._chk(lib.gmm_workspace_size(g.OP_DLHS, ctypes.byref(self.op_g8), ctypes.byref(self.op_g8),
                                         M, N, K, G, ctypes.byref(n)))
        self.ws_d = torch.empty(max(n.value, 256), dtype=torch.uint8, device=dev)
        self.ws_d_n = n.value
        self.r_lq, self.r_l8 = ctypes.byref(self.op_lq), ctypes.byref(self.op_l8)
        self.r_gq, self.r_g8 = ctypes.byref(self.op_gq), ctypes.byref(self.op_g8)
        P = lambda t: t.data_ptr()
        self.p = {k: P(getattr(self, k)) for k in
                  ("lhs", "grad", "lhs_q", "grad_q", "w_fwd", "s_fwd", "w_dlhs", "s_dlhs", "out", "dlhs",
                   "drhs", "s_lhs", "s_grad", "ws", "ws_t", "ws_f", "ws_d", "gs")}
        # a static lhs has no block scales
        self.p_sl = None if self.static else self.p["s_lhs"]
        torch.cuda.synchronize()

    # the five calls of a step, each on stream s
    def q_lhs(self, s):
        self._chk(self.lib.gmm_quantize(self.r_lq, self.M, self.K, self.p["lhs"], self.p["lhs_q"],
                                        self.p_sl, self.p["ws"], self.ws_n, s))

    def fwd(self, s):
        g, p = self.g, self.p
        self._chk(self.lib.gmm_fwd(self.r_l8, g.E4M3, g.RHS_NK, g.OUT_BF16, self.M, self.K, self.N,
                                   self.G, p["lhs_q"], self.p_sl, p["w_fwd"], p["s_fwd"], p["gs"],
                                   p["out"], p["ws_f"], self.ws_f_n, s))

    def q_grad(self, s):
        self._chk(self.lib.gmm_quantize(self.r_gq, self.M, self.N, self.p["grad"], self.p["grad_q"],
                                        self.p["s_grad"], self.p["ws"], self.ws_n, s))

    def dlhs_(self, s):
        g, p = self.g, self.p
        self._chk(self.lib.gmm_dlhs(self.r_g8, g.E4M3, g.RHS_KN, g.OUT_BF16, self.M, self.K, self.N,
                                    self.G, p["grad_q"], p["s_grad"], p["w_dlhs"], p["s_dlhs"],
                                    p["gs"], p["dlhs"], p["ws_d"], self.ws_d_n, s))

    def tgmm(self, s):
        p = self.p
        self._chk(self.lib.tgmm_drhs(self.r_l8, self.r_g8, self.g.OUT_BF16, self.M, self.K, self.N,
                                     self.G, p["lhs_q"], self.p_sl, p["grad_q"], p["s_grad"],
                                     p["gs"], p["drhs"], p["ws_t"], self.ws_t_n, s))

    def run(self, stream, ev=None):
        """Enqueue one step; ev (6 events) brackets: lhs quantize, fwd, grad quantize, dlhs,
        tgmm."""
        rec = (lambda i: ev[i].record()) if ev is not None else (lambda i: None)
        for i, op in enumerate((self.q_lhs, self.fwd, self.q_grad, self.dlhs_, self.tgmm)):
            rec(i)
            op(stream)
        rec(5)

    def run_overlapped(self, s, s2, e_fork, e_join):
        """Enqueue one step with the backward products on two streams: after the grad
        quantizer, dlhs runs on `s` and tgmm on `s2` (torch streams; default priority), so
        that tgmm's workgroups take the CUs dlhs leaves idle in its short last round of
        tiles.  The two read the same grad codes and write separate outputs."""
        sp = s.cuda_stream
        self.q_lhs(sp)
        self.fwd(sp)
        self.q_grad(sp)
        e_fork.record(s)
        s2.wait_event(e_fork)
        self.dlhs_(sp)
        self.tgmm(s2.cuda_stream)
        e_join.record(s2)
        s.wait_event(e_join)

    def _chk(self, status):
        if status != 0:
            raise RuntimeError(f"library call failed: {self.g.gmm_status_string(status)}")


def protocol(step, reps):
    """Median and minimum of `reps` runs per op and per step (one stream), warm and cold."""
    import torch

    s = torch.cuda.current_stream().cuda_stream
    cold = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    ops = {"quantize_lhs": step.q_lhs, "gmm_fwd": step.fwd, "quantize_grad": step.q_grad,
           "gmm_dlhs": step.dlhs_, "tgmm_drhs": step.tgmm}
    ops["step"] = lambda st: step.run(st)
    res = {}
    for name, fn in ops.items():
        r = reps if name != "step" else max(reps // 2, 10)
        warm = event_times(lambda: fn(s), r)
        cld = event_times(lambda: fn(s), r, warmup=1, cold=cold)
        e = _median_min(warm)
        c = _median_min(cld)
        e.update({"cold_median_ms": c["median_ms"], "cold_min_ms": c["min_ms"], "runs": r})
        res[name] = e
    del cold
    torch.cuda.empty_cache()
    return res


def static_vs_dynamic(g, step, reps):
    """The workload's forward with a static per-tensor lhs scale (4/448) and with dynamic
    128-row block scales: (a) the bf16 lhs handed to gmm_fwd, which quantizes it itself
    (dynamic: abs-max prepass first), and (b) gmm_quantize, then gmm_fwd on the codes.
    Medians of `reps` runs."""
    import torch

    lhs, w, ws, gs = step.lhs, step.w_fwd, step.s_fwd, step.gs
    out = step.out
    res = {}
    for mode in ("static", "dynamic"):
        kw = dict(lhs_scaling="static", static_scale=STATIC_SCALE) if mode == "static" else {}
        t_call = event_times(lambda: g.gmm_fwd(lhs, w, ws, gs, out=out, **kw), reps)
        codes = {}

        def two_calls():
            if mode == "static":
                q, _ = g.gmm_quantize(lhs, "e4m3", "static", static_scale=STATIC_SCALE)
                g.gmm_fwd(q, w, ws, gs, out=out, **kw)
            else:
                q, sc = g.gmm_quantize(lhs, "e4m3", "dynamic")
                g.gmm_fwd(q, w, ws, gs, out=out, lhs_scales=sc)

        t_two = event_times(two_calls, reps)
        res[mode] = {"gmm_fwd_bf16_lhs": _median_min(t_call), "quantize_then_fwd": _median_min(t_two)}
        del codes
    a = res["static"]["gmm_fwd_bf16_lhs"]["median_ms"]
    b = res["dynamic"]["gmm_fwd_bf16_lhs"]["median_ms"]
    res["static_over_dynamic"] = round(a / b, 4)
    res["note"] = ("same shape and inputs; the dynamic recipe adds the abs-max prepass over the "
                   "lhs (2 M K bytes) and per-row-block scales in the epilogue")
    torch.cuda.empty_cache()
    return res


def dense_ceiling(wl, reps):
    """Context only: the vendor library's dense FP8 GEMM (torch._scaled_mm, hipBLASLt) at the
    workload's M x K x N with one group, e4m3 operands and unit scales, bf16 out: what a
    tuned dense FP8 GEMM reaches on this chip at the same shape.  Nothing of the path uses
    it.  None when the call is unavailable."""
    import torch

    M, K, N = wl.M, wl.K, wl.N
    try:
        gen = torch.Generator(device="cuda").manual_seed(17)
        a = (torch.randn((M, K), device="cuda", generator=gen) * 0.5).to(torch.float8_e4m3fn)
        b = (torch.randn((N, K), device="cuda", generator=gen) * 0.5).to(torch.float8_e4m3fn).t()
        one = torch.tensor(1.0, device="cuda")
        ts = event_times(lambda: torch._scaled_mm(a, b, scale_a=one, scale_b=one,
                                                  out_dtype=torch.bfloat16), reps)
    except Exception as e:  # pragma: no cover
        return {"error": repr(e)[:200]}
    r = _median_min(ts)
    r["TFLOP/s"] = round(2.0 * M * K * N / r["median_ms"] / 1e9, 1)
    r["frac_peak"] = round(r["TFLOP/s"] / FP8_PEAK_TFLOPS, 4)
    r["what"] = ("torch._scaled_mm (hipBLASLt), dense [M, K] x [K, N] e4m3, random data, "
                 "bf16 out; context for the grouped products, not part of the path")
    del a, b
    torch.cuda.empty_cache()
    return r


def ffn_chain(g, reps=10):
    """The MoE SwiGLU feed-forward block (moe_swiglu shape: G=64, M=65536, hidden 2048,
    intermediate 1408), forward and backward as one chain, timed per op and in total:

      gate|up gmm with SwiGLU in its epilogue (h, and gu for the backward), the down gmm on
      h, dlhs of the down weight (dh), the SwiGLU backward (d_gu), dlhs of the gate|up
      weight (dx), tgmm of both weights.

    pure: every product takes bf16 operands and quantizes them itself.  hybrid: each
    gradient (grad_y, d_gu) is quantized once (e5m2, dynamic) and its codes feed both its
    dlhs and its tgmm.  static: the forward lhs (x, h) uses the static scale 4/448 (h comes
    out of the gate|up epilogue as e4m3 codes); dynamic: 128-row block scales.  Last, the
    hybrid static chain once more with gmm_dlhs_swiglu_bwd in place of the down dlhs and
    the SwiGLU backward (no dh)."""
    import torch

    from synth.workloads import WORKLOADS, normal_bf16

    wl = WORKLOADS["moe_swiglu"]
    G, M, H, I = wl.G, wl.M, wl.K, wl.extra["intermediate"]
    seed = wl.seed * 100
    dev = "cuda"
    gs = torch.tensor(wl.group_sizes(), dtype=torch.int32, device=dev)
    x = normal_bf16((M, H), 1.0, seed, dev)
    w_gu = normal_bf16((G, H, 2 * I), 0.02, seed + 1, dev)
    w_dn = normal_bf16((G, I, H), 0.02, seed + 2, dev)
    grad_y = normal_bf16((M, H), 1e-3, seed + 3, dev)
    wgu_q, wgu_s = g.gmm_quantize_rhs(w_gu, "e4m3", 0, "nk")
    wgu_k, wgu_sk = g.gmm_quantize_rhs(w_gu, "e4m3", 1, "kn")
    wdn_q, wdn_s = g.gmm_quantize_rhs(w_dn, "e4m3", 0, "nk")
    wdn_k, wdn_sk = g.gmm_quantize_rhs(w_dn, "e4m3", 1, "kn")
    del w_gu, w_dn
    bf = torch.bfloat16
    h = torch.empty((M, I), dtype=bf, device=dev)
    hq = torch.empty((M, I), dtype=torch.uint8, device=dev)
    y = torch.empty((M, H), dtype=bf, device=dev)
    dh = torch.empty((M, I), dtype=bf, device=dev)
    d_gu = torch.empty((M, 2 * I), dtype=bf, device=dev)
    dx = torch.empty((M, H), dtype=bf, device=dev)
    dwd = torch.empty((G, I, H), dtype=bf, device=dev)
    dwg = torch.empty((G, H, 2 * I), dtype=bf, device=dev)
    S = STATIC_SCALE
    names = ["fwd_gate_up_swiglu", "fwd_down", "dlhs_down", "swiglu_bwd", "dlhs_gate_up",
             "tgmm_down", "tgmm_gate_up"]

    def chain(mode, scaling, ev=None, fused_bwd=False):
        rec = (lambda i: ev[i].record()) if ev is not None else (lambda i: None)
        rec(0)
        if scaling == "static":
            _, gu = g.gmm_fwd_swiglu_fp8(x, wgu_q, wgu_s, gs, S, lhs_scaling="static",
                                         static_scale=S, out=hq, gu=True)
            rec(1)
            g.gmm_fwd(hq, wdn_q, wdn_s, gs, lhs_scaling="static", static_scale=S, out=y)
            h_lhs, h_kw = hq, dict(lhs_scaling="static", lhs_static_scale=S)
            x_kw = dict(lhs_scaling="static", lhs_static_scale=S)
        else:
            _, gu = g.gmm_fwd_swiglu(x, wgu_q, wgu_s, gs, out=h, gu=True)
            rec(1)
            g.gmm_fwd(h, wdn_q, wdn_s, gs, out=y)
            h_lhs, h_kw, x_kw = h, {}, {}
        rec(2)
        if mode == "hybrid":
            gyq, sgy = g.gmm_quantize(grad_y, "e5m2", "dynamic")
            if fused_bwd:
                # the SwiGLU backward in the down projection's dlhs epilogue (no dh), which
                # also gathers d_gu's block scales (its quantizer then has no prepass)
                _, sdg = g.gmm_dlhs_swiglu_bwd(gyq, wdn_k, wdn_sk, gs, gu, grad_scales=sgy,
                                               out=d_gu, d_gu_format="e5m2")
                rec(3)
                rec(4)
                dgq, _ = g.gmm_quantize(d_gu, "e5m2", "dynamic_given", scales=sdg)
            else:
                g.gmm_dlhs(gyq, wdn_k, wdn_sk, gs, grad_scales=sgy, out=dh)
                rec(3)
                g.gmm_swiglu_bwd(dh, gu, out=d_gu)
                rec(4)
                dgq, sdg = g.gmm_quantize(d_gu, "e5m2", "dynamic")
            g.gmm_dlhs(dgq, wgu_k, wgu_sk, gs, grad_scales=sdg, out=dx)
            rec(5)
            g.tgmm_drhs(h_lhs, gyq, gs, grad_scales=sgy, out=dwd, **h_kw)
            rec(6)
            g.tgmm_drhs(x, dgq, gs, grad_scales=sdg, out=dwg, **x_kw)
        else:
            g.gmm_dlhs(grad_y, wdn_k, wdn_sk, gs, out=dh)
            rec(3)
            g.gmm_swiglu_bwd(dh, gu, out=d_gu)
            rec(4)
            g.gmm_dlhs(d_gu, wgu_k, wgu_sk, gs, out=dx)
            rec(5)
            g.tgmm_drhs(h_lhs, grad_y, gs, out=dwd, **h_kw)
            rec(6)
            g.tgmm_drhs(x, d_gu, gs, out=dwg, **x_kw)
        rec(7)

    two = 2.0 * M * H * I
    flops = {"fwd_gate_up_swiglu": 2 * two, "fwd_down": two, "dlhs_down": two, "swiglu_bwd": 0.0,
             "dlhs_gate_up": 2 * two, "tgmm_down": two, "tgmm_gate_up": 2 * two}
    # algorithmic bytes of the fused path (bf16 operands read, fp8 weights, bf16 outputs)
    nbytes = {"fwd_down": 2 * M * I + G * I * H + 2 * M * H,
              "dlhs_down": 2 * M * H + G * I * H + 2 * M * I,
              "swiglu_bwd": 10 * M * I,
              "tgmm_down": 2 * M * I + 2 * M * H + 2 * G * I * H,
              "tgmm_gate_up": 2 * M * H + 4 * M * I + 4 * G * H * I}
    total_flop = 18.0 * M * H * I
    res = {"workload": wl.name, "G": G, "M": M, "hidden": H, "intermediate": I,
           "flop_per_chain": total_flop, "runs": reps}
    for mode in ("pure", "hybrid"):
        for scaling in ("static", "dynamic"):
            for _ in range(3):
                chain(mode, scaling)
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(8)] for _ in range(reps)]
            torch.cuda.synchronize()
            for i in range(reps):
                chain(mode, scaling, evs[i])
            torch.cuda.synchronize()
            tot = [e[0].elapsed_time(e[7]) for e in evs]
            per = {}
            for j, n in enumerate(names):
                t = float(np.median([e[j].elapsed_time(e[j + 1]) for e in evs]))
                d = {"ms": round(t, 4)}
                if flops[n]:
                    d["TFLOP/s"] = round(flops[n] / t / 1e9, 1)
                    d["frac_peak"] = round(flops[n] / t / 1e9 / FP8_PEAK_TFLOPS, 4)
                if n in nbytes:
                    d["GB/s"] = round(nbytes[n] / t / 1e6, 1)
                    d["frac_hbm"] = round(nbytes[n] / t / 1e6 / HBM_PEAK_GBS, 4)
                per[n] = d
            mt = _median_min(tot)
            res[f"{mode}_{scaling}"] = {"chain": mt,
                                        "TFLOP/s": round(total_flop / mt["median_ms"] / 1e9, 1),
                                        "ops": per}
    # the hybrid static chain again with the SwiGLU backward in the down dlhs's epilogue
    for _ in range(3):
        chain("hybrid", "static", fused_bwd=True)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(8)] for _ in range(reps)]
    torch.cuda.synchronize()
    for i in range(reps):
        chain("hybrid", "static", evs[i], fused_bwd=True)
    torch.cuda.synchronize()
    mt = _median_min([e[0].elapsed_time(e[7]) for e in evs])
    t_fb = float(np.median([e[2].elapsed_time(e[4]) for e in evs]))
    t_two = (res["hybrid_static"]["ops"]["dlhs_down"]["ms"] +
             res["hybrid_static"]["ops"]["swiglu_bwd"]["ms"])
    res["hybrid_static_fused_bwd"] = {
        "chain": mt, "TFLOP/s": round(total_flop / mt["median_ms"] / 1e9, 1),
        "dlhs_down_swiglu_bwd_ms": round(t_fb, 4),
        "two_calls_ms": round(t_two, 4),
        "what": "gmm_dlhs_swiglu_bwd with d_gu's block scales (grad quantizer included) in "
                "place of gmm_dlhs + gmm_swiglu_bwd, and d_gu quantized on those scales "
                "(no prepass); same d_gu bits and codes"}
    res["hybrid_over_pure"] = {s: round(res[f"hybrid_{s}"]["chain"]["median_ms"] /
                                        res[f"pure_{s}"]["chain"]["median_ms"], 4)
                               for s in ("static", "dynamic")}
    res["static_over_dynamic"] = {m: round(res[f"{m}_static"]["chain"]["median_ms"] /
                                           res[f"{m}_dynamic"]["chain"]["median_ms"], 4)
                                  for m in ("pure", "hybrid")}
    res["note"] = ("hybrid timings include the stand-alone gradient quantizers inside the dlhs "
                   "ops; GB/s on algorithmic bytes of the fused path for the ops the roofline "
                   "calls HBM-bound")
    del x, grad_y, wgu_q, wgu_s, wgu_k, wgu_sk, wdn_q, wdn_s, wdn_k, wdn_sk
    del h, hq, y, dh, d_gu, dx, dwd, dwg
    torch.cuda.empty_cache()
    return res


def gfx_clock_during(run, seconds=1.0):
    """Run `run` back to back for `seconds` while amdsmi samples the GFX clock of every XCD;
    return the mean in MHz over the samples taken once the clock had left idle (the first
    readings of the metrics table can be stale), or None when amdsmi is unavailable."""
    import threading

    import torch

    try:
        import amdsmi

        amdsmi.amdsmi_init()
        handle = amdsmi.amdsmi_get_processor_handles()[0]
    except Exception:
        return None
    samples, stop = [], threading.Event()

    def sample():
        while not stop.is_set():
            try:
                m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
                clks = m.get("current_gfxclks")
                # entries of XCDs the table does not fill read 0 (or 0xFFFF): keep clocks
                ok = lambda c: isinstance(c, (int, float)) and 100 <= c < 5000
                vals = [c for c in clks if ok(c)] if isinstance(clks, list) else []
                if not vals and ok(m.get("current_gfxclk")):
                    vals = [m["current_gfxclk"]]
                if vals:
                    samples.append(sum(vals) / len(vals))
            except Exception:
                pass
            stop.wait(0.01)

    th = threading.Thread(target=sample, daemon=True)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        run()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:
        pass
    busy = [x for x in samples if x >= 500.0]  # below the lowest DPM level: idle or stale
    return round(sum(busy) / len(busy), 1) if busy else None


def swiglu_block(g, reps=10):
    """The SwiGLU steps of an MoE feed-forward block at the moe_swiglu shape (G=64,
    M=65536, hidden 2048, intermediate 1408): gmm_fwd_swiglu (merged gate|up product with
    SwiGLU in its epilogue) against gmm_fwd alone, the same with h written as static-scale
    e4m3 codes, the down projection on those codes against the same on the bf16 h, h as
    codes with dynamic scales per row and 128 channels (against bf16 h then the
    sub-channel quantizer) with the block-wise down projection on them, and
    gmm_swiglu_bwd, each timed with HIP events on the current stream; synthetic inputs as
    the workload's."""
    import torch

    from synth.workloads import WORKLOADS, normal_bf16

    wl = WORKLOADS["moe_swiglu"]
    G, M, K, I = wl.G, wl.M, wl.K, wl.extra["intermediate"]
    gs = torch.tensor(wl.group_sizes(), dtype=torch.int32, device="cuda")
    x = normal_bf16((M, K), 1.0, wl.seed * 100, "cuda")
    w = normal_bf16((G, K, 2 * I), 0.02, wl.seed * 100 + 1, "cuda")
    wq, ws = g.gmm_quantize_rhs(w, "e4m3", 0, "nk")
    del w
    xq, sx = g.gmm_quantize(x, "e4m3", "dynamic")
    wd = normal_bf16((G, I, K), 0.02, wl.seed * 100 + 2, "cuda")
    wdq, wds = g.gmm_quantize_rhs(wd, "e4m3", 0, "nk")
    wdbq, wdbs = g.gmm_quantize_rhs_blockwise(wd, 128, "e4m3", "nk")
    del wd
    dh = normal_bf16((M, I), 1e-3, wl.seed * 100 + 3, "cuda")
    h = torch.empty((M, I), dtype=torch.bfloat16, device="cuda")
    hq = torch.empty((M, I), dtype=torch.uint8, device="cuda")
    y = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    gu = torch.empty((M, 2 * I), dtype=torch.bfloat16, device="cuda")
    d_gu = torch.empty_like(gu)

    def timed(fn):
        return float(np.median(event_times(fn, reps, warmup=3)))

    t_plain = timed(lambda: g.gmm_fwd(xq, wq, ws, gs, lhs_scales=sx, out=gu))
    t_fused = timed(lambda: g.gmm_fwd_swiglu(xq, wq, ws, gs, lhs_scales=sx, out=h))
    s_h = STATIC_SCALE  # a static scale for h (its value does not change the work)
    t_fp8 = timed(lambda: g.gmm_fwd_swiglu_fp8(xq, wq, ws, gs, s_h, lhs_scales=sx, out=hq))
    down = dict(lhs_scaling="static", static_scale=s_h, out=y)
    t_down_codes = timed(lambda: g.gmm_fwd(hq, wdq, wds, gs, **down))
    t_down_bf16 = timed(lambda: g.gmm_fwd(h, wdq, wds, gs, **down))
    # h with dynamic scales per row and 128 channels, from the epilogue, and the
    # block-wise down projection on it; against SwiGLU to bf16 h then the quantizer
    hs = torch.empty((M, I // 128), dtype=torch.float32, device="cuda")
    t_fp8_dyn = timed(lambda: g.gmm_fwd_swiglu_fp8_subchannel(xq, wq, ws, gs, lhs_scales=sx,
                                                              out=hq, h_scales=hs))
    t_down_dyn = timed(lambda: g.gmm_fwd_blockwise(hq, hs, wdbq, wdbs, gs, 128, out=y))
    t_unfused_dyn = timed(lambda: (g.gmm_fwd_swiglu(xq, wq, ws, gs, lhs_scales=sx, out=h),
                                   g.gmm_quantize_subchannel(h, 128)))
    g.gmm_fwd(xq, wq, ws, gs, lhs_scales=sx, out=gu)
    t_bwd = timed(lambda: g.gmm_swiglu_bwd(dh, gu, out=d_gu))
    flop = 2.0 * M * K * 2 * I
    bwd_bytes = 10.0 * M * I  # reads dh (2 B) and gu (4 B), writes d_gu (4 B) per channel
    res = {
        "workload": wl.name, "G": G, "M": M, "K": K, "I": I,
        "fwd_swiglu": {"ms": round(t_fused, 4), "TFLOP/s": round(flop / t_fused / 1e9, 1),
                       "frac_peak": round(flop / t_fused / 1e9 / FP8_PEAK_TFLOPS, 4)},
        "fwd_product_only_ms": round(t_plain, 4),
        "fwd_swiglu_fp8_h_ms": round(t_fp8, 4),
        "down_on_h_codes_ms": round(t_down_codes, 4),
        "down_on_bf16_h_ms": round(t_down_bf16, 4),
        "fwd_swiglu_fp8_h_subchannel_ms": round(t_fp8_dyn, 4),
        "fwd_swiglu_bf16_h_then_quantize_subchannel_ms": round(t_unfused_dyn, 4),
        "down_blockwise_on_subchannel_h_ms": round(t_down_dyn, 4),
        "swiglu_bwd": {"ms": round(t_bwd, 4), "GB/s": round(bwd_bytes / t_bwd / 1e6, 1),
                       "frac_hbm": round(bwd_bytes / t_bwd / 1e6 / HBM_PEAK_GBS, 4)},
        "note": "fwd_swiglu writes h [M, I] only; the unfused path would add a bf16 [M, 2I] "
                "write and read around an elementwise SwiGLU",
    }
    del x, xq, wq, ws, wdq, wds, wdbq, wdbs, dh, h, hq, hs, y, gu, d_gu
    torch.cuda.empty_cache()
    return res


def route_block(g, reps=10):
    """Token routing at the moe_swiglu shape (8192 tokens x top-8 of 64 experts, Zipf(1.3)
    popularity, hidden 2048): gmm_permute of bf16 rows and of e4m3 codes, and the weighted
    gmm_unpermute, each against HBM peak on its algorithmic bytes (x read once, every
    permuted row written once, the index arrays)."""
    import torch

    from synth.workloads import WORKLOADS, normal_bf16, topk_expert_ids

    wl = WORKLOADS["moe_swiglu"]
    G, H, k = wl.G, wl.K, 8
    T = wl.M // k
    ids = torch.as_tensor(topk_expert_ids(T, k, G, wl.zipf_s, wl.seed), device="cuda")
    x = normal_bf16((T, H), 1.0, wl.seed * 100 + 7, "cuda")
    codes, _ = g.gmm_quantize(x, "e4m3", "static", static_scale=STATIC_SCALE)
    xp, gs, ros, sor = g.gmm_permute(ids, G, x)
    cp = torch.empty((T * k, H), dtype=torch.uint8, device="cuda")
    w = torch.rand((T, k), device="cuda")
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")

    def timed(fn):
        return float(np.median(event_times(fn, reps, warmup=3)))

    t_perm = timed(lambda: g.gmm_permute(ids, G, x, xp))
    t_perm8 = timed(lambda: g.gmm_permute(ids, G, codes, cp))
    t_idx = timed(lambda: g.gmm_permute(ids, G))
    t_comb = timed(lambda: g.gmm_unpermute(xp, ros, w, out))
    n = T * k
    idx_bytes = 12.0 * n
    perm_b = T * H * 2.0 + n * H * 2.0 + idx_bytes
    perm8_b = T * H * 1.0 + n * H * 1.0 + idx_bytes
    comb_b = n * H * 2.0 + T * H * 2.0 + 8.0 * n

    def rate(b, t):
        return {"ms": round(t, 4), "GB/s": round(b / t / 1e6, 1),
                "frac_hbm": round(b / t / 1e6 / HBM_PEAK_GBS, 4)}

    res = {"workload": wl.name, "tokens": T, "top_k": k, "G": G, "hidden": H,
           "permute_bf16": rate(perm_b, t_perm), "permute_e4m3": rate(perm8_b, t_perm8),
           "permute_index_only_ms": round(t_idx, 4), "unpermute": rate(comb_b, t_comb)}
    del ids, x, codes, xp, gs, ros, sor, cp, w, out
    torch.cuda.empty_cache()
    return res


def blockwise_block(g, reps=10):
    """The forward with block-wise scales at the Mixtral gate|up shape (G=8, M=16384,
    K=4096, N=28672): gmm_fwd_blockwise on sub-channel e4m3 lhs codes ([M, K/bk] scales)
    and block-scaled e4m3 weights ([G, K/bk, N] scales) for bk 128 and 512, against the
    fp8 MFMA peak; the lhs quantization timed apart; the one-weight-copy dlhs (the
    gradient folded with the forward's scales, then the fp8-A dlhs on the forward's
    codes); and the dlhs with block-wise scales (bk 512).  HIP events on the current
    stream."""
    import torch

    from synth.workloads import WORKLOADS, normal_bf16

    wl = WORKLOADS["mixtral_gate_up"]
    G, M, K, N = wl.G, wl.M, wl.K, wl.N
    gs = torch.tensor(wl.group_sizes(), dtype=torch.int32, device="cuda")
    x = normal_bf16((M, K), 1.0, wl.seed * 100 + 11, "cuda")
    w = normal_bf16((G, K, N), 0.02, wl.seed * 100 + 12, "cuda")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def timed(fn):
        return float(np.median(event_times(fn, reps, warmup=3)))

    flop = 2.0 * M * K * N
    res = {"workload": wl.name, "G": G, "M": M, "K": K, "N": N}
    for bk in (128, 512):
        codes, s = g.gmm_quantize_subchannel(x, bk)
        wq, ws = g.gmm_quantize_rhs_blockwise(w, bk)
        t = timed(lambda: g.gmm_fwd_blockwise(codes, s, wq, ws, gs, bk, out=out))
        tq = timed(lambda: g.gmm_quantize_subchannel(x, bk))
        res[f"bk{bk}"] = {"ms": round(t, 4), "TFLOP/s": round(flop / t / 1e9, 1),
                          "frac_peak": round(flop / t / 1e9 / FP8_PEAK_TFLOPS, 4),
                          "lhs_quantize_ms": round(tq, 4)}
        del codes, s, wq, ws
    # the one-weight-copy dlhs: the gradient folded with the forward's per-channel scales,
    # then the fp8-A dlhs on the forward's codes ([G, K, N]) with unit output scales
    grad = normal_bf16((M, N), 1e-3, wl.seed * 100 + 13, "cuda")
    wq, ws = g.gmm_quantize_rhs(w, "e4m3", 0, "kn")
    ones = torch.ones((G, K), dtype=torch.float32, device="cuda")
    dl = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    codes, s = g.gmm_quantize_folded(grad, ws, gs)
    tq = timed(lambda: g.gmm_quantize_folded(grad, ws, gs))
    td = timed(lambda: g.gmm_dlhs(codes, wq, ones, gs, grad_scaling="dynamic", grad_scales=s,
                                  rhs_layout="kn", out=dl))
    res["folded_dlhs"] = {"quantize_ms": round(tq, 4), "dlhs_ms": round(td, 4),
                          "dlhs_TFLOP/s": round(flop / td / 1e9, 1)}
    del wq, ws, ones, codes, s
    # the dlhs with block-wise scales along its contraction n (bk 512): sub-channel grad
    # codes and the weight's dlhs copy with one scale per expert, channel k and n-block
    gq, gsc = g.gmm_quantize_subchannel(grad, 512, "e5m2")
    wq, ws = g.gmm_quantize_rhs_blockwise_dlhs(w, 512)
    tb = timed(lambda: g.gmm_dlhs_blockwise(gq, gsc, wq, ws, gs, 512, out=dl))
    res["dlhs_bk512"] = {"ms": round(tb, 4), "TFLOP/s": round(flop / tb / 1e9, 1),
                         "frac_peak": round(flop / tb / 1e9 / FP8_PEAK_TFLOPS, 4)}
    del x, w, out, grad, wq, ws, dl, gq, gsc
    torch.cuda.empty_cache()
    return res


def crossover_block(g, reps=10):
    """Where quantizing a bf16 lhs once beats the in-kernel ("fused") quantization: the
    forward at a growing number of 256-column output tiles, dynamic lhs scaling, on the
    Mixtral rows (G=8, M=16384, K=4096) and the 64-expert SwiGLU rows (G=64, M=65536,
    K=2048).  Per width: the fused call alone (fused=True: every output tile quantizes
    its rows in the kernel), gmm_quantize then the fp8-codes forward, and the call with
    its full workspace (the library's own choice: quantize once from 4 tiles on).  HIP
    events on the current stream, median of `reps`."""
    import torch

    from synth.workloads import WORKLOADS, normal_bf16

    def timed(fn):
        return float(np.median(event_times(fn, reps, warmup=3)))

    res = {}
    for name in ("mixtral_gate_up", "moe_swiglu"):
        wl = WORKLOADS[name]
        G, M, K = wl.G, wl.M, wl.K
        gs = torch.tensor(wl.group_sizes(), dtype=torch.int32, device="cuda")
        x = normal_bf16((M, K), 1.0, wl.seed * 100 + 21, "cuda")
        rows = []
        for tiles in (1, 2, 3, 4, 6, 8, 16):
            N = 256 * tiles
            w = normal_bf16((G, K, N), 0.02, wl.seed * 100 + 22, "cuda")
            wq, ws = g.gmm_quantize_rhs(w, "e4m3", 0, "nk")
            out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            t_fused = timed(lambda: g.gmm_fwd(x, wq, ws, gs, fused=True, out=out))
            t_lib = timed(lambda: g.gmm_fwd(x, wq, ws, gs, out=out))
            codes, sc = g.gmm_quantize(x, "e4m3", "dynamic")
            t_q = timed(lambda: g.gmm_quantize(x, "e4m3", "dynamic"))
            t_f8 = timed(lambda: g.gmm_fwd(codes, wq, ws, gs, lhs_scaling="dynamic",
                                           lhs_scales=sc, out=out))
            rows.append({"tiles": tiles, "N": N, "fused_ms": round(t_fused, 4),
                         "quantize_ms": round(t_q, 4), "fp8_ms": round(t_f8, 4),
                         "quantize_then_fp8_ms": round(t_q + t_f8, 4),
                         "library_ms": round(t_lib, 4),
                         "fused_over_quantize_once": round(t_fused / (t_q + t_f8), 3)})
            del w, wq, ws, out, codes, sc
        res[name] = {"G": G, "M": M, "K": K, "rows": rows}
        del x
        torch.cuda.empty_cache()
    return res


def cpu_baseline(step, rows, cols):
    """Time the CPU oracle on a bounded sample: the first `rows` rows (with their group
    split), all K, the first `cols` columns of the merged weight; fwd + dlhs + tgmm."""
    import torch

    import oracle.ops as ops
    from oracle.quant import quantize_rhs_per_channel

    try:
        from threadpoolctl import threadpool_info

        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    M, K = rows, step.K
    off = np.concatenate([[0], np.cumsum(step.sizes)])
    sizes = np.clip(np.minimum(off[1:], M) - np.minimum(off[:-1], M), 0, None).astype(np.int32)
    bits = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)
    lhs = bits(step.lhs[:M].to("cpu"))
    grad = bits(step.grad[:M, :cols].to("cpu"))
    w = bits(step.w_sample[:, :, :cols].contiguous())
    lmode = "static" if step.static else "dynamic"
    s = np.float32(STATIC_SCALE) if step.static else None
    t0 = time.perf_counter()
    wq_n, ws_n = quantize_rhs_per_channel(w, "e4m3", "n")
    wq_k, ws_k = quantize_rhs_per_channel(w, "e4m3", "k")
    ops.fwd(lhs, wq_n, ws_n, sizes, "e4m3", lmode, s, "e4m3", "bf16")
    ops.dlhs(grad, wq_k, ws_k, sizes, "e5m2", "dynamic", None, "e4m3", "bf16")
    ops.tgmm(lhs, grad, sizes, "e4m3", lmode, s, out_dtype="bf16")
    dt = time.perf_counter() - t0
    flops = 3 * 2.0 * M * K * cols
    return {
        "value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(blas_threads),
        "kind": "oracle", "seconds": round(dt, 2),
        "sample": f"first {M} rows (their group split), K={K}, first {cols} of N columns; "
                  f"weight quantization + fwd + dlhs + tgmm, bf16 outputs; "
                  f"{len(os.sched_getaffinity(0))} host cores visible",
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path runs "
              "on a single MI355X and the library has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import fp8_grouped_gemm_ragged_amd as g
    from synth.workloads import WORKLOADS

    if args.crossover:
        print(json.dumps({"crossover_block": crossover_block(g)}), flush=True)
        return
    wl = WORKLOADS[args.workload]
    if args.dense_only:
        print(json.dumps({"dense_ceiling": dense_ceiling(wl, args.reps)}), flush=True)
        return
    step = Step(g, wl, seed=wl.seed * 100)
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream
    for _ in range(args.warmup):
        step.run(s)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step.run(s, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    names = ["quantize_lhs", "gmm_fwd", "quantize_grad", "gmm_dlhs", "tgmm_drhs"]
    per = {n: float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(args.steps)]))
           for j, n in enumerate(names)}
    ms_serial = wall * 1000.0 / args.steps
    # The step on one stream gives value and ms_per_step.  The same steps with dlhs and tgmm
    # on two streams are timed beside it (context: with its tail split, dlhs no longer
    # leaves CUs idle for tgmm to take).
    ms_step = ms_serial
    ms_two = None
    if not args.no_overlap:
        s2 = torch.cuda.Stream()
        forks = [(torch.cuda.Event(), torch.cuda.Event()) for _ in range(args.steps)]
        for _ in range(args.warmup):
            step.run_overlapped(stream, s2, *forks[0])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step.run_overlapped(stream, s2, *forks[i])
        torch.cuda.synchronize()
        ms_two = (time.perf_counter() - t0) * 1000.0 / args.steps
    # the GFX clock the chip holds under this load (FP8 MFMA work draws enough power to
    # keep it well below the 2.4 GHz the published peak assumes)
    clock_mhz = None if args.no_clock else gfx_clock_during(lambda: [step.run(s) for _ in range(8)])
    flop_op = 2.0 * wl.M * wl.K * wl.N
    value = 3 * flop_op / (ms_step / 1000.0) / 1e12
    ops = {n: {"ms": round(per[n], 4), "TFLOP/s": round(flop_op / (per[n] / 1000) / 1e12, 1),
               "frac_peak": round(flop_op / (per[n] / 1000) / 1e12 / FP8_PEAK_TFLOPS, 4)}
           for n in ("gmm_fwd", "gmm_dlhs", "tgmm_drhs")}
    dom = max(ops, key=lambda n: per[n])
    ach = flop_op / (per[dom] / 1000.0) / 1e12
    kern = {"gmm_fwd": "gmm_kernel<e4m3,e4m3,fp8 A,contraction-contiguous B>",
            "gmm_dlhs": "gmm_kernel<e5m2,e4m3,fp8 A,contraction-contiguous B>",
            "tgmm_drhs": "tgmm_plan_kernel + tgmm_main_kernel<e4m3,e5m2> + tgmm_promote_kernel "
                         "(exits at once: no wide-range group)"}[dom]
    lhs_desc = ("bf16 -> e4m3 static per-tensor 4/448" if step.static
                else "bf16 -> e4m3 dynamic 128-row blocks")
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": wl.name, "G": wl.G, "M": wl.M, "K": wl.K, "N": wl.N,
                   "routing": f"zipf{wl.zipf_s}" if wl.routing == "zipf" else wl.routing,
                   "group_sizes": [int(x) for x in wl.group_sizes()],
                   "lhs": lhs_desc, "grad": "bf16 -> e5m2 dynamic 128-row blocks",
                   "rhs": "e4m3 per-channel", "out": "bf16",
                   "step": "lhs quantize + fwd + grad quantize + hybrid dlhs + tgmm; each tensor "
                           "quantized once, its codes used by every product"},
        "schedule": "one HIP stream: value, ms_per_step, ops, prep_ms and roofline come from "
                    "the same timed steps",
        "two_stream_ms_per_step": None if ms_two is None else round(ms_two, 4),
        "ops": ops,
        "prep_ms": {"lhs_quantize": round(per["quantize_lhs"], 4),
                    "grad_quantize": round(per["quantize_grad"], 4)},
        "roofline": {"kernel": kern, "op": dom, "bound": "mfma", "achieved": round(ach, 1),
                     "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / FP8_PEAK_TFLOPS, 4),
                     "clock_mhz": clock_mhz,
                     "peak_at_clock": round(256 * 8192 * clock_mhz / 1e6, 1) if clock_mhz else None,
                     "frac_at_clock": round(ach / (256 * 8192 * clock_mhz / 1e6), 4) if clock_mhz else None,
                     "clock_note": "mean GFX clock over the XCDs (amdsmi current_gfxclks) during 1 s "
                                   "of back-to-back steps after the timed region; peak_at_clock = "
                                   "256 CUs x 8192 FP8 FLOP/clk x clock",
                     "traffic": measured_traffic(dom, wl.name),
                     "traffic_unit": "L2-to-fabric bytes per launch (FETCH_SIZE + WRITE_SIZE, "
                                     "scaled by a 1 GiB copy; last-level-cache hits count as "
                                     "fabric traffic); null once the kernel sources changed"},
        "counters": measured_counters(wl.name),
    }
    if not args.no_extras:
        line["protocol"] = protocol(step, args.reps)
        line["static_vs_dynamic"] = static_vs_dynamic(g, step, max(args.reps // 2, 10))
        line["dense_fp8_ceiling"] = dense_ceiling(wl, max(args.reps // 2, 10))
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(step, args.cpu_sample_rows, args.cpu_sample_cols)
    del step
    torch.cuda.empty_cache()
    if not args.no_extras:
        line["ffn_chain"] = ffn_chain(g)
        line["swiglu_block"] = swiglu_block(g)
        line["route_block"] = route_block(g)
        line["blockwise_block"] = blockwise_block(g)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
