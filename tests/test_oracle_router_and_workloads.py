"""Pins of the router-GEMM reference and checks of the seeded workloads."""
from fractions import Fraction

import numpy as np
import torch

import oracle as O
import workloads as W


def _bf16_fraction(bits):
    bits = int(bits)
    sign = -1 if bits & 0x8000 else 1
    exp = (bits >> 7) & 0xFF
    man = bits & 0x7F
    if exp == 0:
        return sign * Fraction(man, 1 << 7) * Fraction(1, 1 << 126)
    return sign * (1 + Fraction(man, 1 << 7)) * (Fraction(2) ** (exp - 127))


def test_router_reference_matches_exact_rational_dot():
    rng = np.random.default_rng(2)
    hidden = rng.integers(0, 1 << 16, size=(3, 64), dtype=np.uint32).astype(np.uint16)
    weight = rng.integers(0, 1 << 16, size=(5, 64), dtype=np.uint32).astype(np.uint16)
    # keep finite values only (exponent field != 0xFF)
    hidden[(hidden >> 7 & 0xFF) == 0xFF] = 0x3F80
    weight[(weight >> 7 & 0xFF) == 0xFF] = 0x3F80
    hidden &= np.uint16(0xC7FF)  # limit the exponent range: exact in binary64
    weight &= np.uint16(0xC7FF)
    ref = O.router_logits_ref(hidden, weight)
    for t in range(3):
        for e in range(5):
            exact = sum(_bf16_fraction(a) * _bf16_fraction(b) for a, b in zip(hidden[t], weight[e]))
            assert abs(Fraction(ref[t, e]) - exact) <= abs(exact) * Fraction(1, 1 << 45) + Fraction(1, 1 << 200)


def test_router_reference_bound_covers_an_fp32_accumulation():
    c = W.router_case(4)
    ref = O.router_logits_ref(c.hidden, c.weight)
    bound = O.router_logits_bound(c.hidden, c.weight)
    h = torch.from_numpy(c.hidden.view(np.int16)).view(torch.bfloat16).float()
    w = torch.from_numpy(c.weight.view(np.int16)).view(torch.bfloat16).float()
    f32 = (h @ w.T).numpy().astype(np.float64)
    assert np.all(np.abs(f32 - ref) <= bound)
    # logit scale of the workload: std ~ sqrt(7168) * 0.02 ~ 1.69
    assert 1.2 < ref.std() < 2.2


def test_workloads_are_seeded_and_shaped():
    a, b = W.tiny_global(), W.tiny_global()
    assert a.logits.shape == (8, 896) and a.logits.dtype == np.float32
    assert np.array_equal(a.logits, b.logits) and np.array_equal(a.bias, b.bias)
    c1 = W.decode_local()
    assert (c1.T, c1.off, c1.cnt) == (16, 336, 112)
    lp = W.long_prefill(T=64)
    assert lp.logits.shape == (64, 896) and (lp.off, lp.cnt) == (0, 112)
    v1 = W.long_prefill(T=64, variant=1)
    assert not np.array_equal(lp.logits, v1.logits)


def test_decode_sweep_twins_are_exact_duplicates():
    c = W.decode_sweep(24, 5)
    for src, dst in W.TWIN_PAIRS:
        assert np.array_equal(c.logits[:, src], c.logits[:, dst])
        assert c.bias[src] == c.bias[dst]


def test_decode_sweep_ties_decide_real_routes():
    """The twins tie exactly in sp; check that ties land inside the top-k
    (both twins chosen, lower id first) and on its boundary (both twins'
    groups kept but only one chosen: it must be the lower id)."""
    both = straddle = 0
    for T in W.DECODE_SWEEP_T:
        c = W.decode_sweep(T, 0)
        r = O.route_ref(c.logits, c.bias)
        sp = O.biased_scores(O.sigmoid_rn32(c.logits), c.bias)
        for t in range(T):
            row = r["topk_ids"][t].tolist()
            kept = O.kept_groups(O.group_scores(sp[t], 8, 2), 4)
            for src, dst in W.TWIN_PAIRS:
                lo, hi = min(src, dst), max(src, dst)
                if lo in row and hi in row:
                    both += 1
                    assert row.index(lo) < row.index(hi)
                elif (lo in row) != (hi in row) and lo // 112 in kept and hi // 112 in kept:
                    straddle += 1
                    assert lo in row
    assert both > 0 and straddle > 0, (both, straddle)


def test_long_prefill_skew_is_about_ten_times_mean():
    c = W.long_prefill(T=2048)
    r = O.route_ref(c.logits, c.bias)
    load = np.bincount(r["topk_ids"].ravel(), minlength=896)
    ratio = load.max() / load.mean()
    assert 7.0 < ratio < 14.0, ratio
