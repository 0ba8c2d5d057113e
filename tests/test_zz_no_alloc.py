"""The allocation-free entry point moe_route_local_noalloc against
moe_route_local, through the C ABI: two calls in a row on the library's
static scratch, the second with a smaller input, each compared with the
workspace entry point on the same inputs (every output bit-identical: both
run the same kernels) and with the oracle."""
import numpy as np
import pytest
import torch

import moe_expert_routing_amd as M
import workloads as W
from gpu_util import DEV, assert_parity, oracle_case, say, to_dev, to_numpy

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

NAMES = ("topk_ids", "topk_weights", "packed", "counts", "offsets", "perm", "inv_perm")


def _both(case):
    logits, bias = to_dev(case.logits), to_dev(case.bias)
    kw = dict(n_groups=case.n_groups, topk_group=case.topk_group, top_k=case.top_k,
              group_topn=case.group_topn)
    ref = to_numpy(M.route_local(logits, bias, case.off, case.cnt, **kw))
    got = to_numpy(M.route_local_noalloc(logits, bias, case.off, case.cnt, **kw))
    torch.cuda.synchronize()
    return got, ref


def _check(case, with_oracle=True):
    say(f"case noalloc {case.name} T={case.logits.shape[0]} off={case.off} cnt={case.cnt}")
    got, ref = _both(case)
    assert int(got["num_experts_out"]) == int(ref["num_experts_out"])
    for k in NAMES:
        assert got[k].shape == ref[k].shape, k
        assert np.array_equal(got[k].view(np.uint32), ref[k].view(np.uint32)), \
            f"{case.name}: {k} differs from moe_route_local"
    if with_oracle:
        assert_parity(got, oracle_case(case), case.name)


def test_prefill_then_smaller_prefill():
    _check(W.long_prefill(), with_oracle=False)   # 32,768 tokens, rank 0 of 8
    _check(W.random_case(1000, seed=31, off=0, cnt=0))


def test_decode_then_smaller_decode():
    _check(W.random_case(64, seed=32, off=336, cnt=112))
    _check(W.random_case(8, seed=33, off=336, cnt=112))


def test_prefill_then_decode_then_empty():
    _check(W.random_case(4099, seed=34, off=784, cnt=112))
    _check(W.random_case(17, seed=35, off=0, cnt=0))
    _check(W.random_case(0, seed=36, off=0, cnt=0), with_oracle=False)


def test_other_shape_one_token_per_wave_path():
    c = W.random_case(777, seed=37, off=0, cnt=0, e=256, n_groups=8, topk_group=4,
                      top_k=8)
    _check(c)
    _check(W.random_case(65, seed=38, off=0, cnt=0, e=256, n_groups=8, topk_group=4,
                         top_k=8))


def test_largest_accepted_then_one_beyond_is_rejected():
    # 896 experts, global ids: the static scratch holds at most 69,888 tokens
    c = W.random_case(69_888, seed=39, off=0, cnt=0)
    _check(c, with_oracle=False)
    T = 69_888 + 1
    logits = torch.zeros((T, 896), dtype=torch.float32, device=DEV)
    bias = torch.zeros(896, dtype=torch.float32, device=DEV)
    say(f"case noalloc rejected T={T}")
    with pytest.raises(M.MoeRouteError, match="static 16 MiB"):
        M.route_local_noalloc(logits, bias)
    _check(W.random_case(64, seed=40, off=0, cnt=0))   # later calls still work


@pytest.mark.parametrize("T", [16, 4099])
def test_captured_in_a_graph(T):
    # The callers this entry point is for capture it in HIP graphs: each replay
    # (with eager routing and overwritten outputs in between) gives the
    # workspace entry point's result.
    c = W.random_case(T, seed=41 + T, off=336, cnt=112)
    say(f"case noalloc graph replays T={T}")
    logits, bias = to_dev(c.logits), to_dev(c.bias)
    ref = to_numpy(M.route_local(logits, bias, c.off, c.cnt))
    out = M.alloc_outputs(T, 16, int(ref["num_experts_out"]), DEV)
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        M.route_local_noalloc(logits, bias, c.off, c.cnt, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        M.route_local_noalloc(logits, bias, c.off, c.cnt, out=out)
    other = W.random_case(100, seed=5)
    for rep in range(3):
        for k in NAMES:
            out[k].fill_(-1)
        M.route_local(to_dev(other.logits), to_dev(other.bias))  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        got = to_numpy(out)
        for k in NAMES:
            assert np.array_equal(got[k].view(np.uint32), ref[k].view(np.uint32)), \
                f"replay {rep}: {k} differs from moe_route_local"
