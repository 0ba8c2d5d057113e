"""Pins of the oracle's grouped top-k (group scores, group choice, expert
top-k and slot order) by brute force and by reduction to a stable sort."""
import itertools

import numpy as np
import pytest

import oracle as O

def _brute_force_row(sp, n_groups, topk_group, top_k, group_topn):
    """Selection from the definition, by exhaustive enumeration.

    Group score: the largest fl32 sum over all `group_topn`-subsets of the
    group (fl32 addition is monotone, so this is the sum of the top values).
    Kept groups: the subset whose (score, -g) keys, sorted, are
    lexicographically largest. Experts: the K-subset of the kept candidates
    whose sorted (sp, -e) keys are lexicographically largest, in that order.
    """
    E = sp.shape[0]
    eg = E // n_groups
    gs = []
    for g in range(n_groups):
        members = range(g * eg, (g + 1) * eg)
        best = None
        for sub in itertools.combinations(members, group_topn):
            vals = sorted((float(sp[e]) for e in sub), reverse=True)
            acc = np.float32(vals[0])
            for v in vals[1:]:
                acc = np.float32(acc + np.float32(v))
            best = acc if best is None or acc > best else best
        gs.append(float(best))
    best_groups = None
    for sub in itertools.combinations(range(n_groups), topk_group):
        key = sorted(((gs[g], -g) for g in sub), reverse=True)
        if best_groups is None or key > best_groups[0]:
            best_groups = (key, sub)
    cand = [e for g in best_groups[1] for e in range(g * eg, (g + 1) * eg)]
    best = None
    for sub in itertools.combinations(cand, top_k):
        key = sorted(((float(sp[e]), -e) for e in sub), reverse=True)
        if best is None or key > best:
            best = key
    return [-ne for _, ne in best]

def _oracle_row(sp, n_groups, topk_group, top_k, group_topn):
    gs = O.group_scores(sp, n_groups, group_topn)
    groups = O.kept_groups(gs, topk_group)
    return O.topk_experts(sp, groups, n_groups, top_k)

def _alphabet_rows(n, E, seed):
    """Rows of biased scores drawn from a tiny alphabet so ties are dense."""
    rng = np.random.default_rng(seed)
    s = O.sigmoid_rn32(rng.choice(np.array([-1.0, 0.0, 1.0], np.float32), size=(n, E)))
    b = rng.choice(np.array([0.0, 0.25], np.float32), size=(n, E)).astype(np.float32)
    return (s + b).astype(np.float32)

SHAPES = [  # (E, n_groups, topk_group, top_k, group_topn)
    (12, 4, 2, 3, 2),
    (12, 4, 2, 3, 1),
    (12, 3, 2, 4, 2),
    (8, 4, 2, 3, 2),
    (10, 1, 1, 4, 2),
]

@pytest.mark.parametrize("shape", SHAPES)
def test_grouped_topk_matches_brute_force(shape):
    E, G, TG, K, N = shape
    rows = _alphabet_rows(600, E, seed=E * 100 + G * 10 + K)
    for sp in rows:
        assert _oracle_row(sp, G, TG, K, N) == _brute_force_row(sp, G, TG, K, N), sp

def test_grouped_topk_brute_force_continuous_values():
    rng = np.random.default_rng(5)
    for _ in range(300):
        sp = (rng.standard_normal(12) * 0.3).astype(np.float32)
        assert _oracle_row(sp, 4, 2, 3, 2) == _brute_force_row(sp, 4, 2, 3, 2)

@pytest.mark.parametrize("G,TG", [(1, 1), (8, 8), (4, 4)])
def test_all_groups_kept_is_a_stable_sort(G, TG):
    rng = np.random.default_rng(11)
    for _ in range(40):
        sp = rng.choice(np.linspace(0, 1, 9).astype(np.float32), size=896).astype(np.float32)
        want = np.argsort(-sp.astype(np.float64), kind="stable")[:16].tolist()
        assert _oracle_row(sp, G, TG, 16, 2) == want

def test_full_pipeline_matches_brute_force_on_tiny_inputs():
    rng = np.random.default_rng(21)
    T, E = 300, 12
    logits = rng.choice(np.array([-1.0, 0.0, 1.0, 2.0], np.float32), size=(T, E))
    bias = rng.choice(np.array([0.0, 0.25, -0.25], np.float32), size=E).astype(np.float32)
    ids, s_sel, w = O.route_tokens(logits, bias, n_groups=4, topk_group=2, top_k=3, group_topn=2)
    s = O.sigmoid_rn32(logits)
    sp = (s + bias[None, :]).astype(np.float32)
    for t in range(T):
        assert ids[t].tolist() == _brute_force_row(sp[t], 4, 2, 3, 2)
        assert np.array_equal(s_sel[t], s[t, ids[t]])

def test_ties_go_to_lower_expert_id():
    sp = np.full(896, 0.5, np.float32)
    assert _oracle_row(sp, 8, 4, 16, 2) == list(range(16))
    sp[700] = sp[3] = np.float32(0.75)
    got = _oracle_row(sp, 8, 4, 16, 2)
    assert got[:2] == [3, 700]

# --- planted mistakes: each plausible error must fail the brute-force pin ---

def _count_mismatches(row_fn, shape, n=300, seed=3):
    E, G, TG, K, N = shape
    rows = _alphabet_rows(n, E, seed)
    return sum(row_fn(sp, G, TG, K, N) != _brute_force_row(sp, G, TG, K, N) for sp in rows)

def test_planted_group_score_top1_is_caught():
    def mutant(sp, G, TG, K, N):
        gs = O.group_scores(sp, G, 1)  # dropped second term
        return O.topk_experts(sp, O.kept_groups(gs, TG), G, K)
    assert _count_mismatches(mutant, (12, 4, 2, 3, 2)) > 0

def test_planted_tie_to_higher_id_is_caught():
    def mutant(sp, G, TG, K, N):
        groups = O.kept_groups(O.group_scores(sp, G, N), TG)
        eg = sp.shape[0] // G
        cand = [e for g in groups for e in range(g * eg, (g + 1) * eg)]
        cand.sort(key=lambda e: (-float(sp[e]), -e))  # wrong tie sign
        return cand[:K]
    assert _count_mismatches(mutant, (12, 4, 2, 3, 2)) > 0

def test_planted_group_tie_to_higher_index_is_caught():
    def mutant(sp, G, TG, K, N):
        gs = O.group_scores(sp, G, N)
        order = sorted(range(G), key=lambda g: (-float(gs[g]), -g))
        return O.topk_experts(sp, sorted(order[:TG]), G, K)
    assert _count_mismatches(mutant, (12, 4, 2, 3, 2)) > 0

def test_planted_group_of_wrong_stride_is_caught():
    def mutant(sp, G, TG, K, N):
        # groups taken as strided (e % G) instead of contiguous runs
        perm = np.concatenate([np.arange(g, sp.shape[0], G) for g in range(G)])
        gs = O.group_scores(sp[perm], G, N)
        groups = O.kept_groups(gs, TG)
        eg = sp.shape[0] // G
        cand = [int(perm[i]) for g in groups for i in range(g * eg, (g + 1) * eg)]
        cand.sort(key=lambda e: (-float(sp[e]), e))
        return cand[:K]
    assert _count_mismatches(mutant, (12, 4, 2, 3, 2)) > 0

def test_brute_force_detects_rank_by_unbiased_score():
    """Selecting on s instead of s + b changes results on these inputs."""
    rng = np.random.default_rng(8)
    logits = rng.standard_normal((200, 12)).astype(np.float32)
    bias = rng.choice(np.array([0.0, 0.3], np.float32), size=12).astype(np.float32)
    ids, _, _ = O.route_tokens(logits, bias, 4, 2, 3, 2)
    s = O.sigmoid_rn32(logits)
    unbiased = [_brute_force_row(s[t], 4, 2, 3, 2) for t in range(200)]
    assert any(ids[t].tolist() != unbiased[t] for t in range(200))
    sp = (s + bias[None, :]).astype(np.float32)
    assert all(ids[t].tolist() == _brute_force_row(sp[t], 4, 2, 3, 2) for t in range(200))

def test_group_scores_reject_nondividing_shape():
    with pytest.raises(ValueError):
        O.route_tokens(np.zeros((1, 10), np.float32), np.zeros(10, np.float32), n_groups=4)

def test_biased_scores_are_fp32_sums():
    s = np.array([[0.5, 0.25]], np.float32)
    b = np.array([2.0 ** -25, 2.0 ** -26], np.float32)
    sp = O.biased_scores(s, b)
    # 0.5 + 2^-25 is a tie between 0.5 and 0.5 + 2^-24: to even -> 0.5
    assert sp[0, 0] == np.float32(0.5)
    assert sp[0, 1] == np.float32(0.25)
