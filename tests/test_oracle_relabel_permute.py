"""Pins of the oracle's relabel, pack, weights, counts, offsets and
permutation: the value the pages print, the invariants they state, library
routines and closed forms."""
import math
import os

import mpmath
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "relabel_printed.txt")


def _golden_rows():
    rows = []
    with open(GOLDEN) as fh:
        for line in fh:
            if line.strip() and not line.startswith("#"):
                rows.append([int(v) for v in line.split()])
    return rows


def test_printed_ep8_local_problem_size():
    for E, K, ep, cnt, e_local in _golden_rows():
        assert E // ep == cnt
        for rank in range(ep):
            assert O.local_num_experts(E, K, rank * cnt, cnt) == e_local


@pytest.mark.parametrize("ep,want", [(2, 464), (4, 240), (8, 128), (16, 72)])
def test_local_problem_size_rule(ep, want):
    cnt = 896 // ep
    assert O.local_num_experts(896, 16, 0, cnt) == want
    assert want % 4 == 0 and want >= cnt + 16 and want - (cnt + 16) < 4


def test_range_that_does_not_apply_keeps_global_ids():
    assert O.local_num_experts(896, 16, 0, 0) == 0          # off
    assert O.local_num_experts(896, 16, 0, 896) == 0        # whole bank
    assert O.local_num_experts(896, 16, 0, 884) == 0        # 900 >= 896: no shrink
    assert O.local_num_experts(896, 16, 12, 877) == 0       # 896 >= 896: no shrink
    assert O.local_num_experts(896, 16, 0, 876) == 892      # still shrinks


@pytest.mark.parametrize("off,cnt", [(-1, 10), (890, 10), (0, 897), (5, -1)])
def test_range_outside_bank_is_an_error(off, cnt):
    with pytest.raises(ValueError):
        O.local_num_experts(896, 16, off, cnt)


def _check_local_vs_global(logits, bias, off, cnt):
    g = O.route_ref(logits, bias)
    loc = O.route_ref(logits, bias, local_expert_offset=off, num_local_experts=cnt)
    K = 16
    e_out = int(loc["num_experts_out"])
    assert e_out == O.local_num_experts(896, K, off, cnt)
    # global ids and weights are unchanged, and so is the weight field
    assert np.array_equal(g["topk_ids"], loc["topk_ids"])
    assert np.array_equal(g["topk_weights"], loc["topk_weights"])
    assert np.array_equal(g["packed"] & 0xFFFF, loc["packed"] & 0xFFFF)
    ids_out = loc["packed"] >> 16
    assert np.array_equal(ids_out, loc["ids_out"])
    T = logits.shape[0]
    for t in range(T):
        row = ids_out[t]
        assert len(set(row.tolist())) == K  # unique per row
        for k in range(K):
            e = int(g["topk_ids"][t, k])
            if off <= e < off + cnt:
                assert row[k] == e - off
            else:
                assert row[k] == cnt + k
    assert ids_out.max() < e_out
    # the same (token, local expert, weight) entries in the same order
    def entries(res, lo, hi, shift):
        ids = res["packed"] >> 16
        out = []
        for f in res["perm"]:
            t, k = divmod(int(f), K)
            e = int(ids[t, k])
            if lo <= e < hi:
                out.append((t, e + shift, int(res["packed"][t, k] & 0xFFFF)))
        return out
    assert entries(loc, 0, cnt, off) == entries(g, off, off + cnt, 0)


@pytest.mark.parametrize("ep", [2, 4, 8, 16])
@pytest.mark.parametrize("which", ["first", "middle", "last"])
def test_relabel_invariants_over_ep_and_ranks(ep, which):
    cnt = 896 // ep
    rank = {"first": 0, "middle": ep // 2, "last": ep - 1}[which]
    for T in (1, 7, 64):
        c = W.random_case(T, seed=1000 * ep + 10 * rank + T)
        _check_local_vs_global(c.logits, c.bias, rank * cnt, cnt)


def test_relabel_invariants_on_decode_sweep_with_twins():
    for rank in (0, 3, 7):
        c = W.decode_sweep(64, rank)
        _check_local_vs_global(c.logits, c.bias, c.off, c.cnt)


def test_counts_offsets_perm_match_library_routines():
    rng = np.random.default_rng(3)
    for e_out in (128, 896):
        ids = np.stack([rng.permutation(e_out)[:16] for _ in range(50)]).astype(np.int32)
        counts = O.expert_counts(ids, e_out)
        assert np.array_equal(counts, np.bincount(ids.ravel(), minlength=e_out))
        offs = O.exclusive_offsets(counts)
        assert np.array_equal(offs, np.concatenate([[0], np.cumsum(counts)]))
        perm, inv = O.expert_major_permutation(ids, e_out)
        assert np.array_equal(perm, np.argsort(ids.ravel(), kind="stable"))
        assert np.array_equal(inv[perm], np.arange(ids.size))


def test_permutation_empty_and_single():
    ids = np.zeros((0, 16), np.int32)
    perm, inv = O.expert_major_permutation(ids, 128)
    assert perm.size == 0 and inv.size == 0
    assert O.exclusive_offsets(O.expert_counts(ids, 128)).tolist() == [0] * 129


def test_planted_unstable_order_is_caught():
    ids = np.array([[3, 1], [1, 3], [3, 0]], np.int32)
    flat = ids.ravel()
    mutant = np.argsort(flat, kind="stable")[::-1]
    mutant = np.concatenate([np.sort(mutant[flat[mutant] == e])[::-1] for e in range(4)])
    assert not np.array_equal(mutant, O.expert_major_permutation(ids, 4)[0])


def test_bf16_rne_matches_torch_conversion():
    rng = np.random.default_rng(4)
    w = np.concatenate([
        rng.random(20000).astype(np.float32),
        np.array([1.0, 0.5, 2.0 ** -20, 1e-38, 1.00390625, 1.01171875], np.float32),
        # exact ties between two bf16 values, both parities
        (np.arange(0x3F000000, 0x3F000000 + 4096, dtype=np.uint32) | np.uint32(0x8000)).view(np.float32),
    ])
    want = torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_rne_bits(w), want.astype(np.uint32))


def test_pack_fields():
    ids = np.array([[0, 127, 895]], np.int32)
    w = np.array([[1.0, 0.5, 0.0625]], np.float32)
    p = O.pack(ids, w)
    assert (p >> 16).tolist() == [[0, 127, 895]]
    assert (p & 0xFFFF).tolist() == [[0x3F80, 0x3F00, 0x3D80]]
    assert np.all(p >= 0)


def test_weights_are_the_renormalised_unbiased_sigmoid():
    mpmath.mp.dps = 40
    c = W.tiny_global()
    r = O.route_ref(c.logits, c.bias)
    for t in range(c.logits.shape[0]):
        ids = r["topk_ids"][t]
        w = r["topk_weights"][t].astype(np.float64)
        sig = [1 / (1 + mpmath.exp(-mpmath.mpf(float(c.logits[t, e])))) for e in ids]
        tot = sum(sig)
        for k in range(16):
            exact = float(sig[k] / tot)
            assert abs(w[k] - exact) <= 2 * 2.0 ** -24 * exact
        assert np.all(w > 0)
        assert abs(math.fsum(w) - 1.0) <= 16 * 2.0 ** -24
        p = r["packed"][t]
        assert np.all((p & 0xFFFF) <= 0x3F80)


def test_planted_biased_weight_is_caught():
    c = W.long_prefill(T=4)
    r = O.route_ref(c.logits, c.bias)
    s = O.sigmoid_rn32(c.logits)
    sp = (s + c.bias[None, :]).astype(np.float32)
    t = 0
    ids = r["topk_ids"][t]
    wrong = O.renormalised_weights(sp[t, ids])
    assert not np.allclose(wrong, r["topk_weights"][t], rtol=1e-6, atol=0)
