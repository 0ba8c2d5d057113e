"""GPU parity of the static balancing plan (moe_balance_plan) against the
oracle's balance_plan, on the global counts of routing calls over every
workload size and several rank counts."""
import functools

import numpy as np
import pytest
import torch

import moe_expert_routing_amd as M
import oracle as O
import workloads as W
from gpu_util import say, to_dev

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

CASES = {
    "tiny8": lambda: W.tiny_global(8),
    "random1000": lambda: W.random_case(1000, seed=41),
    "random4099": lambda: W.random_case(4099, seed=42),
    "prefill32k": lambda: W.long_prefill(32768),   # Zipf-skewed: heavy surplus
}


@functools.lru_cache(maxsize=None)
@functools.lru_cache(maxsize=None)
def _case_and_oracle(name):
    c = CASES[name]()
    return c, O.route_ref(c.logits, c.bias)          # global ids


def _case(name):
    c, want = _case_and_oracle(name)
    out = M.route(to_dev(c.logits), to_dev(c.bias))
    torch.cuda.synchronize()
    got_counts = out["counts"].cpu().numpy()
    assert np.array_equal(got_counts, want["counts"]), "routing counts differ"
    return c, want, out


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("n_ranks", [1, 2, 7, 8, 16, 32, 64])
def test_balance_plan_matches_oracle(name, n_ranks):
    c, want, out = _case(name)
    n = int(want["perm"].shape[0])
    say(f"case balance plan {name} ranks={n_ranks}")
    plan = M.balance_plan(out["counts"], n_ranks, n)
    torch.cuda.synchronize()
    dest, rc = O.balance_plan(want["counts"], n_ranks)
    assert np.array_equal(plan["rank_counts"].cpu().numpy(), rc), "rank_counts differ"
    gd = plan["dest"].cpu().numpy()
    bad = np.nonzero(gd != dest)[0]
    assert bad.size == 0, f"dest differs at {bad[:5].tolist()}"


def test_balance_plan_empty():
    counts = torch.zeros(896, dtype=torch.int32, device="cuda")
    plan = M.balance_plan(counts, 8, 0)
    torch.cuda.synchronize()
    assert (plan["rank_counts"] == 0).all()
