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


# Hand-worked plan with two overloaded and two short ranks (4 ranks, 2
# experts each). Loads 7, 1, 5, 2 over n = 15 entries; targets 4, 4, 4, 3.
# Rank 0 keeps e0's 4 entries, its surplus is e1's 3 entries; rank 2 keeps
# e4's 2 and the first 2 of e5, its surplus is e5's last entry. The surplus
# sequence in rank order (e1, e1, e1, e5) fills the short ranks in rank order:
# rank 1 is short by 3, rank 3 by 1.
HAND_COUNTS = np.array([4, 3, 1, 0, 2, 3, 1, 1])
HAND_DEST = [0, 0, 0, 0, 1, 1, 1, 1, 2, 2, 2, 2, 3, 3, 3]
HAND_RC = [[4, 0, 0, 0, 0, 0, 0, 0],
           [0, 3, 1, 0, 0, 0, 0, 0],
           [0, 0, 0, 0, 2, 2, 0, 0],
           [0, 0, 0, 0, 0, 1, 1, 1]]


def test_hand_worked_two_overloaded_two_short():
    dest, rc = O.balance_plan(HAND_COUNTS, 4)
    assert dest.tolist() == HAND_DEST
    assert rc.tolist() == HAND_RC


def _plan_variant(counts, n_ranks, reverse_takers=False, surplus_from_head=False):
    """The oracle's plan with one planted change of order (test-only copy)."""
    counts = [int(c) for c in counts]
    E = len(counts)
    per = E // n_ranks
    n = sum(counts)
    target = [n // n_ranks + (1 if r < n % n_ranks else 0) for r in range(n_ranks)]
    load = [sum(counts[r * per:(r + 1) * per]) for r in range(n_ranks)]
    keep = [min(load[r], target[r]) for r in range(n_ranks)]
    takers = [r for r in range(n_ranks) for _ in range(target[r] - keep[r])]
    if reverse_takers:
        takers = takers[::-1]
    dest, moved = [], 0
    for r in range(n_ranks):
        own = 0
        for e in range(r * per, (r + 1) * per):
            for _ in range(counts[e]):
                kept = (own >= load[r] - keep[r]) if surplus_from_head else (own < keep[r])
                if kept:
                    dest.append(r)
                else:
                    dest.append(takers[moved])
                    moved += 1
                own += 1
    return dest


def test_unplanted_variant_matches_the_oracle():
    assert _plan_variant(HAND_COUNTS, 4) == HAND_DEST


def test_planted_reversed_taker_order_is_caught():
    assert _plan_variant(HAND_COUNTS, 4, reverse_takers=True) != HAND_DEST


def test_planted_surplus_from_the_head_is_caught():
    assert _plan_variant(HAND_COUNTS, 4, surplus_from_head=True) != HAND_DEST
