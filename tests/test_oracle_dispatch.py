"""Pins for the oracle's dispatch: counts, offsets, permutation.

Checked against numpy's stable argsort and bincount (library routines the
oracle does not use) and against the invariants the method fixes: counts sum
to N*k, the permutation is a bijection, each expert's segment holds exactly
its flat slots in increasing order."""
import numpy as np
import pytest

import oracle


def _random_routing(rng, N, E, k):
    return np.stack([np.sort(rng.choice(E, k, replace=False)) for _ in range(N)]).astype(np.int32)


@pytest.mark.parametrize("N,E,k", [(1, 4, 2), (3, 8, 3), (64, 16, 4), (200, 37, 5), (50, 8, 8)])
def test_counts_perm_against_library(N, E, k):
    rng = np.random.default_rng(N + E + k)
    idx = _random_routing(rng, N, E, k)
    counts, offsets, perm, inv = oracle.counts_perm(idx, E)
    flat = idx.ravel()
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and offsets[-1] == N * k and np.all(np.diff(offsets) == counts)
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))
    assert np.array_equal(np.sort(perm), np.arange(N * k))
    assert np.array_equal(inv[perm], np.arange(N * k))
    assert np.array_equal(perm[inv], np.arange(N * k))
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.array_equal(seg, np.flatnonzero(flat == e))


def test_empty_and_extreme_segments():
    # one expert taking every token, others empty
    N, E, k = 10, 6, 2
    idx = np.stack([[1, 4]] * N).astype(np.int32)
    counts, offsets, perm, inv = oracle.counts_perm(idx, E)
    assert counts.tolist() == [0, N, 0, 0, N, 0]
    assert perm[:N].tolist() == list(range(0, 2 * N, 2))
    assert perm[N:].tolist() == list(range(1, 2 * N, 2))
    # no tokens
    counts, offsets, perm, inv = oracle.counts_perm(np.zeros((0, 3), np.int32), 5)
    assert counts.tolist() == [0] * 5 and offsets.tolist() == [0] * 6 and perm.size == 0


def test_out_of_range_expert_rejected():
    with pytest.raises(RuntimeError):
        oracle.counts_perm(np.array([[0, 9]], np.int32), 4)
