"""Pins of the stochastic-length oracle: its Philox-4x64-10 against numpy's
independent Philox bit generator, the selection rule against hand-worked
cases (ties included), and the sampler's properties (sizes, order, subset,
identity below the cap, determinism, uniform inclusion)."""
import numpy as np
import pytest

from oracle import stochastic_length as sl


def test_philox_matches_numpy_bit_generator():
    rng = np.random.default_rng(0)
    for _ in range(20):
        ctr = [int(v) for v in rng.integers(1, 2 ** 63, size=4, dtype=np.int64)]
        key = [int(v) for v in rng.integers(0, 2 ** 63, size=2, dtype=np.int64)]
        # numpy's Philox increments its 256-bit counter before each block
        prev = np.array([ctr[0] - 1] + ctr[1:], dtype=np.uint64)
        bg = np.random.Philox(counter=prev, key=np.array(key, dtype=np.uint64))
        ref = [int(v) for v in bg.random_raw(4)]
        assert list(sl.philox4x64(ctr, key)) == ref


def test_selection_rule_hand_cases():
    u = np.array([5, 1, 3, 1, 9, 0], dtype=np.uint64)
    assert list(sl.select_from_keys(u, 1)) == [5]
    assert list(sl.select_from_keys(u, 2)) == [1, 5]          # key 0, then the first key-1 index
    assert list(sl.select_from_keys(u, 3)) == [1, 3, 5]       # both key-1 events
    assert list(sl.select_from_keys(u, 4)) == [1, 2, 3, 5]
    assert list(sl.select_from_keys(u, 6)) == [0, 1, 2, 3, 4, 5]
    ties = np.array([7, 7, 7, 7], dtype=np.uint64)
    assert list(sl.select_from_keys(ties, 2)) == [0, 1]


def test_select_sizes_order_subset_and_identity_below_cap():
    offsets = np.array([0, 3, 3, 40, 45, 145], dtype=np.int64)
    out_off, idx = sl.select(offsets, 10, seed=11, step=2)
    L = np.diff(offsets)
    assert list(np.diff(out_off)) == [min(10, int(x)) for x in L]
    for b in range(len(L)):
        rows = idx[out_off[b]:out_off[b + 1]]
        assert np.all(np.diff(rows) > 0)                        # order kept
        assert np.all((rows >= offsets[b]) & (rows < offsets[b + 1]))
        if L[b] <= 10:
            assert list(rows) == list(range(offsets[b], offsets[b + 1]))
    # per-sequence caps
    out_off2, _ = sl.select(offsets, [1, 1, 50, 2, 3], seed=11, step=2)
    assert list(np.diff(out_off2)) == [1, 0, 37, 2, 3]


def test_select_is_deterministic_and_depends_on_seed_step_and_sequence():
    offsets = np.array([0, 200, 400], dtype=np.int64)
    a = sl.select(offsets, 20, seed=5, step=1)[1]
    assert np.array_equal(a, sl.select(offsets, 20, seed=5, step=1)[1])
    assert not np.array_equal(a, sl.select(offsets, 20, seed=6, step=1)[1])
    assert not np.array_equal(a, sl.select(offsets, 20, seed=5, step=2)[1])
    # the two sequences (same length) draw different subsets
    assert not np.array_equal(a[:20], a[20:] - 200)


def test_inclusion_is_uniform():
    """Each of L = 12 events is kept with probability cap / L = 1/3 (3000
    draws over the step counter: binomial std 0.0086; 4.6 std allowed)."""
    L, cap, n = 12, 4, 3000
    counts = np.zeros(L)
    for step in range(n):
        keep = sl.select_from_keys(sl.event_keys(L, 0, 1234, step), cap)
        counts[keep] += 1
    freq = counts / n
    assert np.all(np.abs(freq - cap / L) < 0.04), freq
