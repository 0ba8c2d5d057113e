"""Pins of the oracle's static balancing plan (oracle/route_ref.py,
balance_plan): a hand-worked example, the closed forms of what every rank
keeps and receives, and the minimality of the moved entries."""
import numpy as np
import pytest

import oracle as O


def test_hand_worked_example():
    # 2 ranks own experts {0,1} and {2,3}; 10 entries, 5 per rank
    dest, rc = O.balance_plan(np.array([5, 3, 1, 1]), 2)
    assert dest.tolist() == [0, 0, 0, 0, 0, 1, 1, 1, 1, 1]
    assert rc.tolist() == [[5, 0, 0, 0], [0, 3, 1, 1]]


def test_balanced_loads_move_nothing():
    counts = np.array([3, 1, 2, 2, 0, 4, 1, 3])      # 4 per rank of 2 experts
    dest, rc = O.balance_plan(counts, 4)
    owner = np.repeat(np.arange(4), [4, 4, 4, 4])
    assert dest.tolist() == owner.tolist()
    assert rc.tolist() == [[3, 1, 0, 0, 0, 0, 0, 0], [0, 0, 2, 2, 0, 0, 0, 0],
                           [0, 0, 0, 0, 0, 4, 0, 0], [0, 0, 0, 0, 0, 0, 1, 3]]


@pytest.mark.parametrize("n_ranks,seed", [(2, 1), (8, 2), (8, 3), (16, 4)])
def test_plan_properties(n_ranks, seed):
    rng = np.random.default_rng(seed)
    E = 64 * n_ranks // 2
    counts = rng.zipf(1.6, E).clip(max=60)
    n = int(counts.sum())
    dest, rc = O.balance_plan(counts, n_ranks)
    per = E // n_ranks
    target = np.array([n // n_ranks + (r < n % n_ranks) for r in range(n_ranks)])
    load = counts.reshape(n_ranks, per).sum(axis=1)
    # every rank processes exactly its target; every expert's entries are all placed
    assert np.bincount(dest, minlength=n_ranks).tolist() == target.tolist()
    assert rc.sum(axis=1).tolist() == target.tolist()
    assert rc.sum(axis=0).tolist() == counts.tolist()
    # owners keep min(load, target) of their own entries, and only the
    # overloaded ranks' excess moves: the fewest moves any such plan can make
    own = np.array([rc[r, r * per:(r + 1) * per].sum() for r in range(n_ranks)])
    assert own.tolist() == np.minimum(load, target).tolist()
    moved = n - own.sum()
    assert moved == np.maximum(load - target, 0).sum()
    # dest agrees with rank_counts entry by entry, in expert-major order
    ids = np.repeat(np.arange(E), counts)
    back = np.zeros_like(rc)
    np.add.at(back, (dest, ids), 1)
    assert np.array_equal(back, rc)
