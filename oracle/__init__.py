"""CPU oracle for the FP8 grouped (ragged) matmul: TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct NumPy implementation of what the
GPU path computes.  It exists to check the HIP library, never to stand in for it:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code, header, table or helper with the
HIP package ``fp8_grouped_gemm_ragged_amd`` and imports nothing from it.

Modules
-------
fp8    OCP E4M3FN / E5M2 and bfloat16 codecs, written from the format definitions.
quant  in-kernel lhs quantization (static per-tensor, dynamic per-128-row block) and
       the per-channel weight quantization used to prepare the pre-quantized rhs.
gmm    the three grouped products: gmm forward, gmm dlhs and the transposed tgmm, and
       their local-expert windows.
swiglu SwiGLU of the merged gate|up product, forward and backward.
route  token routing around the products: the stable sort by expert, the row gather and
       the weighted combine.
blockwise  block-wise weight scales [G, K/bk, N] and sub-channel lhs scales [M, K/bk]: the
       forward with a per-block promotion, and both quantizers.

Sources (the MaxText pull-request pages this method is taken from):
  * "FP8 Megablox for batch split" (PR #3770), Description (1) and (2): fp8 recipes
    in gmm forward and backward, manually quantized weights, merged W0|W1.
  * "Support quantization for tokamax gmm v2" (PR #4451), "What this does" and the
    review thread on per-channel / block-wise rhs scales.
  * "add static LHS scaling support for GMM v2 FWD" (PR #4735), Description, the
    review threads on the lhs docstring (clip(lhs/scale), multiplied back by the
    scale, per-tensor [1,1]) and on block_scale_inv (zero when the scale is zero).

Parity status of every function is listed in its docstring; all are pinned by the
``-m "not gpu"`` tests in ``tests/test_oracle_*.py``.
"""

from .fp8 import (  # noqa: F401
    FORMATS,
    bf16_bits_to_f32,
    decode_fp8,
    encode_fp8,
    f32_to_bf16_bits,
)
from .quant import (  # noqa: F401
    dynamic_scale_from_amax,
    quantize_rhs_per_channel,
    quantize_rowblock,
    quantize_static,
    quantize_with_inv,
    static_inv,
    static_scale_from_bound,
)
from .gmm import (  # noqa: F401
    group_offsets,
    gmm_dlhs_local_ref,
    gmm_dlhs_ref,
    gmm_fwd_local_ref,
    gmm_fwd_ref,
    tgmm_local_ref,
    tgmm_ref,
)
from .route import gather_rows_ref, permute_ref, unpermute_ref  # noqa: F401
from .blockwise import (  # noqa: F401
    gmm_fwd_blockwise_ref,
    quantize_folded,
    quantize_rhs_blockwise,
    quantize_subchannel,
)
from .swiglu import silu, swiglu_bwd_ref, swiglu_fp8_ref, swiglu_ref  # noqa: F401
