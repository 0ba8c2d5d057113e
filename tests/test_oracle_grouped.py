"""Pins of the oracle's grouped-GEMM layout (oracle/route_ref.py,
grouped_layout): a hand-worked example, the closed forms of the padded
offsets, and the permutation-order property checked entry by entry."""
import numpy as np
import pytest

import oracle as O


def test_hand_worked_example():
    # ids 0..3 with 3, 0, 5, 1 entries; tile of 4 rows
    counts = np.array([3, 0, 5, 1], np.int32)
    perm = np.array([10, 2, 7, 4, 5, 6, 8, 9, 11], np.int32)
    rows = O.grouped_layout_rows(9, 4, 4)
    assert rows == 9 + 4 * 3
    po, mi, re = O.grouped_layout(counts, perm, 4, rows)
    assert po.tolist() == [0, 4, 4, 12, 16]
    assert mi.tolist() == [0, 0, 0, -1, 2, 2, 2, 2, 2, -1, -1, -1, 3, -1, -1, -1] + [-1] * 5
    assert re.tolist() == [10, 2, 7, -1, 4, 5, 6, 8, 9, -1, -1, -1, 11, -1, -1, -1] + [-1] * 5


def test_tile_one_is_the_permutation():
    rng = np.random.default_rng(7)
    ids = rng.integers(0, 12, size=(20, 3)).astype(np.int32)
    counts = O.expert_counts(ids, 12)
    perm, _ = O.expert_major_permutation(ids, 12)
    po, mi, re = O.grouped_layout(counts, perm, 1, 60)
    assert po.tolist() == O.exclusive_offsets(counts).tolist()
    assert re.tolist() == perm.tolist()
    assert mi.tolist() == np.sort(ids.ravel(), kind="stable").tolist()


@pytest.mark.parametrize("tile", [2, 8, 128])
def test_padded_layout_properties(tile):
    rng = np.random.default_rng(tile)
    T, K, E = 37, 4, 20
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    counts = O.expert_counts(ids, E)
    perm, _ = O.expert_major_permutation(ids, E)
    rows = O.grouped_layout_rows(T * K, E, tile)
    po, mi, re = O.grouped_layout(counts, perm, tile, rows)
    # closed form of the padded offsets
    want = np.concatenate([[0], np.cumsum([-(-int(c) // tile) * tile for c in counts])])
    assert po.tolist() == want.tolist()
    assert po[-1] <= rows and all(int(v) % tile == 0 for v in po)
    # every entry f sits in its id's block, in ascending f, exactly once
    flat = ids.ravel()
    seen = np.zeros(T * K, bool)
    for e in range(E):
        block = list(range(int(po[e]), int(po[e + 1])))
        real = [r for r in block if mi[r] == e]
        assert len(real) == counts[e]
        assert real == block[:len(real)]                      # real rows first
        fs = [int(re[r]) for r in real]
        assert fs == sorted(fs)                              # stable order
        assert all(flat[f] == e for f in fs)
        seen[fs] = True
        assert all(mi[r] == -1 and re[r] == -1 for r in block[len(real):])
    assert seen.all()
    assert (mi[int(po[-1]):] == -1).all() and (re[int(po[-1]):] == -1).all()
