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

