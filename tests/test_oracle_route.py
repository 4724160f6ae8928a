"""Pins of the routing oracle (permute / unpermute) against a hand-worked example, the
brute-force definition, invariants, a round trip and exact sums."""

import numpy as np

from oracle.fp8 import bf16_bits_to_f32
from oracle.route import gather_rows_ref, permute_ref, unpermute_ref


def test_hand_worked_example():
    # T = 4 tokens, k = 2 choices, G = 3 experts; -1 and 5 are dropped.
    # slots 0..7 hold ids 2 0 | 1 2 | 0 -1 | 2 5
    # expert 0: slots 1, 4 -> rows 0, 1; expert 1: slot 2 -> row 2;
    # expert 2: slots 0, 3, 6 -> rows 3, 4, 5; the dropped slots 5, 7 -> rows 6, 7
    ids = np.array([[2, 0], [1, 2], [0, -1], [2, 5]])
    gs, ros, sor = permute_ref(ids, 3)
    assert gs.tolist() == [2, 1, 3]
    assert sor.tolist() == [1, 4, 2, 0, 3, 6, 5, 7]
    assert ros.tolist() == [[3, 0], [2, 4], [1, -1], [5, -1]]
    x = np.arange(4)[:, None] * np.ones((1, 8), np.int64)
    assert gather_rows_ref(x, sor, 2)[:, 0].tolist() == [0, 2, 1, 0, 1, 3, 2, 3]


def test_brute_force_definition():
    rng = np.random.default_rng(3)
    for T, k, G in [(1, 1, 1), (7, 3, 4), (40, 8, 16), (33, 2, 70)]:
        ids = rng.integers(-2, G + 2, (T, k))
        gs, ros, sor = permute_ref(ids, G)
        rows = []
        for e in range(G):
            mine = [s for s in range(T * k) if ids[s // k, s % k] == e]
            assert gs[e] == len(mine)
            rows += mine
        dropped = [s for s in range(T * k) if not 0 <= ids[s // k, s % k] < G]
        assert sor.tolist() == rows + dropped
        for s in range(T * k):
            e = ids[s // k, s % k]
            want = rows.index(s) if 0 <= e < G else -1
            assert ros[s // k, s % k] == want


def test_invariants():
    rng = np.random.default_rng(4)
    T, k, G = 500, 6, 32
    ids = rng.integers(0, G, (T, k))
    gs, ros, sor = permute_ref(ids, G)
    assert gs.sum() == T * k and len(sor) == T * k
    assert np.array_equal(np.sort(sor), np.arange(T * k))
    assert np.array_equal(ros.reshape(-1)[sor], np.arange(T * k))
    off = np.concatenate([[0], np.cumsum(gs)])
    flat = ids.reshape(-1)
    for e in range(G):
        blk = sor[off[e]:off[e + 1]]
        assert np.all(flat[blk] == e) and np.all(np.diff(blk) > 0)


def test_round_trip_is_the_identity():
    rng = np.random.default_rng(5)
    T, G, H = 300, 9, 64
    ids = rng.integers(0, G, (T, 1))
    xb = (rng.normal(0, 1, (T, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    _, ros, sor = permute_ref(ids, G)
    xp = gather_rows_ref(xb, sor, 1)
    _, bits = unpermute_ref(bf16_bits_to_f32(xp), ros)
    assert np.array_equal(bits, xb)


def test_weighted_sum_order_and_bound():
    # the sum runs from +0 in increasing j: 1 + 2^-24 + 2^-24 stays 1 (each tie rounds to
    # even), while adding the two small terms first would give 1 + 2^-23
    y = np.array([[1.0], [2.0 ** -24], [2.0 ** -24]], np.float32)
    out, _ = unpermute_ref(y, np.array([[0, 1, 2]]))
    assert out[0, 0] == 1.0
    out, _ = unpermute_ref(y, np.array([[1, 2, 0]]))
    assert out[0, 0] == np.float32(1.0 + 2.0 ** -23)
    # a dropped slot contributes nothing; all dropped gives +0
    out, _ = unpermute_ref(y, np.array([[-1, 0, -1], [-1, -1, -1]]), np.full((2, 3), 3.0, np.float32))
    assert out[0, 0] == 3.0 and out[1, 0] == 0.0 and not np.signbit(out[1, 0])
    # random weights: within the float32 rounding bound of the exact sum
    rng = np.random.default_rng(6)
    T, k, H = 64, 8, 32
    yv = rng.normal(0, 1, (T * k, H)).astype(np.float32)
    w = rng.random((T, k)).astype(np.float32)
    ros = rng.permutation(T * k).reshape(T, k).astype(np.int32)
    out, bits = unpermute_ref(yv, ros, w)
    exact = np.einsum("tj,tjh->th", w.astype(np.float64), yv.astype(np.float64)[ros])
    bound = (2 * k) * 2.0 ** -24 * np.einsum("tj,tjh->th", np.abs(w), np.abs(yv)[ros].astype(np.float64))
    assert np.all(np.abs(out - exact) <= bound)
    assert np.all(np.abs(bf16_bits_to_f32(bits) - out) <= np.abs(out) * 2.0 ** -8)
