"""Workload shapes, routing-count generators and seeded bf16 tensor generators.

Recipe (all seeded; seed = workload index unless a test passes its own):

* routing (``topk_expert_ids``): every token draws k distinct experts without
  replacement, with Zipf(s) popularity over a seeded permutation of the expert ids.

* ``group_sizes`` (int32 [G], rows sorted by expert, sum = M):
  - tiny: multinomial(M, uniform) over 3 experts, placed in experts {0, 2, 3} so the
    empty expert 1 sits between two non-empty ones;
  - Zipf(s) popularity: expected counts M * i^-s / sum_j j^-s for rank i = 1..G,
    rounded by largest remainder so they sum to M, then assigned to expert ids by a
    seeded permutation;
  - near-uniform with forced empty experts: the listed experts get 0 rows, the rest
    share M by multinomial(M, uniform).
* tensors: float32 N(0, 1) from ``torch.Generator(device).manual_seed(seed)`` times
  sigma, rounded to bfloat16 by torch's cast.  Activations use sigma 1, weights 0.02,
  output gradients 1e-3.
"""

from dataclasses import dataclass, field

import numpy as np


def zipf_sizes(M, G, s, seed):
    """Largest-remainder rounding of Zipf(s) expected counts, permuted over experts."""
    w = 1.0 / np.arange(1, G + 1, dtype=np.float64) ** s
    expected = M * w / w.sum()
    base = np.floor(expected).astype(np.int64)
    rem = int(M - base.sum())
    order = np.argsort(-(expected - base), kind="stable")
    base[order[:rem]] += 1
    perm = np.random.default_rng(seed).permutation(G)
    sizes = np.zeros(G, np.int64)
    sizes[perm] = base
    return sizes.astype(np.int32)


def multinomial_sizes(M, G, seed, empty=()):
    """Experts in ``empty`` get no rows; the others share M by multinomial(M, uniform)."""
    rng = np.random.default_rng(seed)
    live = [g for g in range(G) if g not in set(empty)]
    draw = rng.multinomial(M, [1.0 / len(live)] * len(live))
    sizes = np.zeros(G, np.int64)
    sizes[live] = draw
    return sizes.astype(np.int32)


@dataclass(frozen=True)
class Workload:
    name: str
    G: int
    M: int
    K: int
    N: int
    routing: str            # "multinomial" or "zipf"
    zipf_s: float = 0.0
    empty: tuple = ()
    seed: int = 0
    lhs_scaling: str = "dynamic"   # forward lhs recipe of the workload
    notes: str = ""
    extra: dict = field(default_factory=dict)

    def group_sizes(self, seed=None):
        seed = self.seed if seed is None else seed
        if self.routing == "zipf":
            return zipf_sizes(self.M, self.G, self.zipf_s, seed)
        return multinomial_sizes(self.M, self.G, seed, self.empty)

    def flops(self):
        return 2.0 * self.M * self.K * self.N


WORKLOADS = {
    # Tiny forward gmm: static per-tensor lhs scale 4/448, expert 1 empty.
    "tiny": Workload("tiny", G=4, M=512, K=128, N=256, routing="multinomial", empty=(1,),
                     seed=1, lhs_scaling="static"),
    # Mixtral-shaped merged gate|up: K=4096, N=2x14336, 8192 tokens x top-2, Zipf(1.1).
    "mixtral_gate_up": Workload("mixtral_gate_up", G=8, M=16384, K=4096, N=28672,
                                routing="zipf", zipf_s=1.1, seed=2, lhs_scaling="dynamic"),
    # DeepSeek-style local experts: K=7168, N=2x2048, 32 experts, experts 0 and 17 empty.
    "deepseek_local": Workload("deepseek_local", G=32, M=32768, K=7168, N=4096,
                               routing="multinomial", empty=(0, 17), seed=3,
                               lhs_scaling="static"),
    # MoE SwiGLU FFN: hidden 2048, intermediate 1408 (merged N=2816), 64 experts,
    # 8192 tokens x top-8, Zipf(1.3).
    "moe_swiglu": Workload("moe_swiglu", G=64, M=65536, K=2048, N=2816, routing="zipf",
                           zipf_s=1.3, seed=5, lhs_scaling="dynamic",
                           extra=dict(intermediate=1408)),
}


def group_sizes_for(name, seed=None):
    return WORKLOADS[name].group_sizes(seed)


def normal_bf16(shape, sigma, seed, device="cpu"):
    """bf16 tensor of N(0, sigma^2) samples from a seeded torch generator on ``device``."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=gen, device=device, dtype=torch.float32)
    x.mul_(float(sigma))
    return x.to(torch.bfloat16)


def bf16_to_bits(t):
    """torch bf16 tensor -> numpy uint16 bit patterns (a view of the same bytes)."""
    import torch

    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def random_fp8_codes(shape, fmt, seed):
    """numpy uint8 fp8 codes drawn uniformly from the finite encodings of ``fmt``, seeded.

    e4m3 (fn): every byte but 0x7f and 0xff (the NaN encodings), which become 0x7e / 0xfe.
    e5m2: every byte whose exponent field (bits 2..6) is not all ones; those get bit 2
    cleared.  Stands in for an operand that was quantized before the call."""
    rng = np.random.default_rng(int(seed))
    c = rng.integers(0, 256, size=tuple(shape), dtype=np.uint16).astype(np.uint8)
    if fmt == "e4m3":
        bad = (c & 0x7F) == 0x7F
        c[bad] ^= np.uint8(0x01)
    elif fmt == "e5m2":
        bad = (c & 0x7C) == 0x7C
        c[bad] &= np.uint8(0xFB)
    else:
        raise ValueError(fmt)
    return c


def log_uniform_scales(n, lo, hi, seed):
    """numpy float32 [n] with log10 uniform in [lo, hi), seeded (per-block scales)."""
    rng = np.random.default_rng(int(seed))
    return (10.0 ** rng.uniform(lo, hi, size=n)).astype(np.float32)


def topk_expert_ids(T, k, G, s, seed, drop=0.0):
    """int32 [T, k]: each token's k distinct experts, drawn without replacement with
    Zipf(s) popularity (rank i weighted i^-s, ranks assigned to expert ids by a seeded
    permutation), in drawn order.  A fraction ``drop`` of the slots, chosen at random,
    is set to -1 (a dropped choice)."""
    rng = np.random.default_rng(int(seed))
    w = 1.0 / np.arange(1, G + 1, dtype=np.float64) ** s
    p = np.zeros(G)
    p[rng.permutation(G)] = w / w.sum()
    # Gumbel top-k: the k largest of log p + Gumbel noise, a draw without replacement
    keys = np.log(p)[None, :] + rng.gumbel(size=(T, G))
    ids = np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int32)
    if drop > 0:
        ids[rng.random((T, k)) < drop] = -1
    return ids
