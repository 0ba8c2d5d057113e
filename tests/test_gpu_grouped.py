"""GPU parity of the grouped-GEMM layout (moe_grouped_layout) against the
oracle's layout, on the routing outputs of every workload shape: the GPU's
counts and perm are bit-exact with the oracle's (checked first), so the
layouts must be identical, row by row."""
import functools

import numpy as np
import pytest
import torch

import moe_expert_routing_amd as M
import oracle as O
import workloads as W
from gpu_util import DEV, assert_parity, oracle_case, say, to_dev

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

CASES = {
    "tiny8": lambda: W.tiny_global(8),
    "local16": lambda: W.decode_local(16),
    "sweep64": lambda: W.decode_sweep(64, 3),
    "ragged1000": lambda: W.random_case(1000, seed=31, off=224, cnt=112),
    "global4099": lambda: W.random_case(4099, seed=32),
    "prefill32k": lambda: W.long_prefill(32768),
}


@functools.lru_cache(maxsize=None)
def _case_and_oracle(name):
    c = CASES[name]()
    return c, oracle_case(c)


def _route(c):
    out = M.route_local(to_dev(c.logits), to_dev(c.bias), c.off, c.cnt)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("tile", [1, 3, 64, 128, 4096])
def test_grouped_layout_matches_oracle(name, tile):
    c, want = _case_and_oracle(name)
    say(f"case grouped layout {name} tile={tile}")
    out = _route(c)
    got = {k: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v) for k, v in out.items()}
    assert_parity(got, want, c.name)
    lay = M.grouped_layout(out["counts"], out["perm"], tile)
    torch.cuda.synchronize()
    rows = lay["m_indices"].shape[0]
    assert rows == O.grouped_layout_rows(want["perm"].shape[0], want["counts"].shape[0], tile)
    po, mi, re = O.grouped_layout(want["counts"], want["perm"], tile, rows)
    assert np.array_equal(lay["padded_offsets"].cpu().numpy(), po), "padded offsets"
    assert np.array_equal(lay["m_indices"].cpu().numpy(), mi), "m_indices"
    assert np.array_equal(lay["row_entry"].cpu().numpy(), re), "row_entry"


def test_grouped_layout_without_entries_and_spare_rows():
    """row_entry omitted; more rows than the bound: the spare rows are -1."""
    c = W.decode_local(16)
    out = _route(c)
    want = oracle_case(c)
    bound = M.grouped_layout_rows(16 * 16, 128, 32)
    lay = M.grouped_layout(out["counts"], out["perm"], 32, rows=bound + 1000,
                           with_entries=False)
    torch.cuda.synchronize()
    po, mi, _ = O.grouped_layout(want["counts"], want["perm"], 32, bound + 1000)
    assert "row_entry" not in lay
    assert np.array_equal(lay["padded_offsets"].cpu().numpy(), po)
    assert np.array_equal(lay["m_indices"].cpu().numpy(), mi)


def test_grouped_layout_empty_routing():
    counts = torch.zeros(128, dtype=torch.int32, device=DEV)
    perm = torch.zeros(0, dtype=torch.int32, device=DEV)
    lay = M.grouped_layout(counts, perm, 128)
    torch.cuda.synchronize()
    assert lay["padded_offsets"].cpu().tolist() == [0] * 129
    assert lay["m_indices"].shape[0] == 128 * 127
    assert (lay["m_indices"] == -1).all() and (lay["row_entry"] == -1).all()


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("tile", [1, 3, 128, 4096])
def test_route_with_fused_layout(name, tile):
    # moe_route_local_grouped: the routing outputs as moe_route_local's and
    # the layout as moe_grouped_layout's (and the oracle's), row by row;
    # above 64 tokens the scatter writes the layout itself. Spare rows past
    # the bound are -1 too.
    c, want = _case_and_oracle(name)
    say(f"case route + fused layout {name} tile={tile}")
    T = c.logits.shape[0]
    rows = M.grouped_layout_rows(T * c.top_k, int(want["num_experts_out"]), tile) + 5
    out = M.route_local_grouped(to_dev(c.logits), to_dev(c.bias), c.off, c.cnt, tile_m=tile,
                                rows=rows)
    torch.cuda.synchronize()
    got = {k: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v) for k, v in out.items()}
    assert_parity(got, want, name)
    po, mi, re = O.grouped_layout(want["counts"], want["perm"], tile, rows)
    assert np.array_equal(got["padded_offsets"], po), "padded_offsets differ"
    bad = np.nonzero(got["m_indices"] != mi)[0]
    assert bad.size == 0, f"m_indices differ at rows {bad[:5].tolist()}"
    bad = np.nonzero(got["row_entry"] != re)[0]
    assert bad.size == 0, f"row_entry differs at rows {bad[:5].tolist()}"



@pytest.mark.parametrize("case", ["t65_without_entries", "other_shape_t777", "global_t200"])
def test_route_with_fused_layout_edges(case):
    # 65 tokens: the first size above the one-launch routing, where the scatter
    # writes the layout; row_entry omitted there. 256 experts, top 8: the
    # one-token-per-wave route kernel before the same scatter. Global ids at
    # 200 tokens (E' = 896).
    if case == "t65_without_entries":
        c, tile, entries = W.random_case(65, seed=61, off=336, cnt=112), 32, False
    elif case == "other_shape_t777":
        c = W.random_case(777, seed=62, e=256, n_groups=8, topk_group=4, top_k=8)
        tile, entries = 64, True
    else:
        c, tile, entries = W.random_case(200, seed=63), 7, True
    want = oracle_case(c)
    say(f"case route + fused layout {case} tile={tile}")
    T = c.logits.shape[0]
    rows = M.grouped_layout_rows(T * c.top_k, int(want["num_experts_out"]), tile) + 3
    out = M.route_local_grouped(to_dev(c.logits), to_dev(c.bias), c.off, c.cnt, tile_m=tile,
                                rows=rows, with_entries=entries, n_groups=c.n_groups,
                                topk_group=c.topk_group, top_k=c.top_k,
                                group_topn=c.group_topn)
    torch.cuda.synchronize()
    got = {k: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v) for k, v in out.items()}
    assert_parity(got, want, case)
    po, mi, re = O.grouped_layout(want["counts"], want["perm"], tile, rows)
    assert np.array_equal(got["padded_offsets"], po), "padded_offsets differ"
    assert np.array_equal(got["m_indices"], mi), "m_indices differ"
    if entries:
        assert np.array_equal(got["row_entry"], re), "row_entry differs"
    else:
        assert "row_entry" not in got


def test_route_with_fused_layout_empty():
    # no tokens: zero padded offsets, every row -1
    logits = torch.zeros((0, 896), dtype=torch.float32, device=DEV)
    bias = torch.zeros(896, dtype=torch.float32, device=DEV)
    say("case route + fused layout empty")
    out = M.route_local_grouped(logits, bias, 336, 112, tile_m=16)
    torch.cuda.synchronize()
    assert out["padded_offsets"].cpu().tolist() == [0] * 129
    assert out["m_indices"].shape[0] == 128 * 15
    assert (out["m_indices"] == -1).all() and (out["row_entry"] == -1).all()
    assert (out["counts"] == 0).all() and (out["offsets"] == 0).all()
