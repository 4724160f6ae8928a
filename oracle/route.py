"""Token routing on either side of the grouped products (oracle; test infrastructure).

The MoE layer sorts token copies by expert before the grouped matmul and gathers the
expert outputs back afterwards (the later commits of "add static LHS scaling support for
GMM v2 FWD": permute()/unpermute() around the gmms, activations quantized before the sort
so it moves fp8; the expert outputs reduced over each token's top-k).  Written from those
definitions:

  slot s = t * k + j        the j-th expert choice of token t (expert_ids [T, k])
  permuted order            the slots with an id in [0, G), by expert; slots of one
                            expert in increasing s (a stable sort); then the dropped
                            slots (any other id), in increasing s
  group_sizes[e]            the number of slots routed to expert e
  x_perm[r]                 x[slot_of_row[r] // k]
  out[t]                    sum over j of w[t, j] * y[row_of_slot[t, j]], dropped slots
                            skipped, in float32 from +0 in increasing j (each product and
                            sum rounded to nearest), then rounded to bfloat16

Parity: pinned by a hand-worked routing example, the brute-force definition (for every
expert, the slots holding its id in increasing order) on small random inputs, the
permutation and group-size invariants, an identity round trip (k = 1, weights 1), and the
weighted sum against an exact float64 sum within its rounding bound
(``tests/test_oracle_route.py``).
"""

import numpy as np

from .fp8 import f32_to_bf16_bits


def permute_ref(expert_ids, G):
    """expert_ids int [T, k] -> (group_sizes int32 [G], row_of_slot int32 [T, k] (-1 for a
    dropped slot), slot_of_row int32 [T * k] (the routed slots, then the dropped ones))."""
    ids = np.asarray(expert_ids, np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    routed = (flat >= 0) & (flat < G)
    # a stable sort with the dropped slots keyed past every expert
    order = np.argsort(np.where(routed, flat, G), kind="stable")
    n = int(routed.sum())
    slot_of_row = order.astype(np.int32)
    row_of_slot = np.full(T * k, -1, np.int32)
    row_of_slot[slot_of_row[:n]] = np.arange(n, dtype=np.int32)
    group_sizes = np.bincount(flat[routed], minlength=G).astype(np.int32)
    return group_sizes, row_of_slot.reshape(T, k), slot_of_row


def gather_rows_ref(x, slot_of_row, k):
    """x [T, ...] -> x_perm [len(slot_of_row), ...] with x_perm[r] = x[slot_of_row[r] // k]."""
    return np.asarray(x)[np.asarray(slot_of_row, np.int64) // k]


def unpermute_ref(y_f32, row_of_slot, weights=None):
    """y [rows, H] float32 values, row_of_slot [T, k] -> (out float32 [T, H] before the bf16
    rounding, its bfloat16 bits)."""
    y = np.asarray(y_f32, np.float32)
    ros = np.asarray(row_of_slot, np.int64)
    T, k = ros.shape
    out = np.zeros((T, y.shape[1]), np.float32)
    w = np.ones((T, k), np.float32) if weights is None else np.asarray(weights, np.float32)
    for j in range(k):
        r = ros[:, j]
        live = r >= 0
        prod = np.zeros_like(out)
        prod[live] = w[live, j][:, None] * y[r[live]]  # float32 products, rounded to nearest
        out[live] = out[live] + prod[live]  # float32 sums, in increasing j
    return out, f32_to_bf16_bits(out)
