"""Helpers of the GPU parity tests: run the HIP path through the C ABI and
compare it with the oracle at the required tolerances:
ids, global ids, counts, offsets, perm, inv and the id field of packed
bit-exact; weights within 1e-6 relative (exactly 0 where the oracle's is 0);
the bf16 field within 1 ulp."""
import sys

import numpy as np
import torch

import moe_expert_routing_amd as M
import oracle as O

DEV = torch.device("cuda:0")


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def run_case(case, check_ws=True):
    """Route a workloads.RouteCase on the GPU; returns numpy outputs."""
    logits = to_dev(case.logits)
    bias = to_dev(case.bias)
    out = M.route_local(logits, bias, case.off, case.cnt, n_groups=case.n_groups,
                        topk_group=case.topk_group, top_k=case.top_k,
                        group_topn=case.group_topn)
    torch.cuda.synchronize()
    if check_ws:
        assert_workspace_zero()
    return to_numpy(out)


def assert_workspace_zero():
    """Every call must leave the workspace's control block zeroed."""
    ws = M.cached_workspace(DEV)
    assert ws is not None, "no default workspace on the current stream"
    assert int(ws[:256].count_nonzero()) == 0, "control block not left zeroed"


def to_numpy(out):
    res = {}
    for k, v in out.items():
        res[k] = v.cpu().numpy() if isinstance(v, torch.Tensor) else v
    return res


def oracle_case(case, logits=None):
    lg = case.logits if logits is None else logits
    return O.route_ref(lg, case.bias, n_groups=case.n_groups, topk_group=case.topk_group,
                       top_k=case.top_k, group_topn=case.group_topn,
                       local_expert_offset=case.off, num_local_experts=case.cnt)


def assert_parity(got, want, label=""):
    ids_g, ids_w = got["topk_ids"], want["topk_ids"]
    assert ids_g.shape == ids_w.shape, (label, ids_g.shape, ids_w.shape)
    bad_rows = np.nonzero(np.any(ids_g != ids_w, axis=1))[0]
    assert bad_rows.size == 0, (
        f"{label}: topk_ids differ in {bad_rows.size} rows, first {bad_rows[:5].tolist()}: "
        f"gpu {ids_g[bad_rows[0]].tolist()} oracle {ids_w[bad_rows[0]].tolist()}")
    wg = got["topk_weights"].astype(np.float64)
    ww = want["topk_weights"].astype(np.float64)
    nz = ww != 0.0
    if np.any(nz):
        rel = np.abs(wg[nz] - ww[nz]) / np.abs(ww[nz])
        assert rel.max() <= 1e-6, f"{label}: weight rel err {rel.max():.3g}"
    assert np.all(wg[~nz] == 0.0), f"{label}: weights of zero scores must be 0"
    pg, pw = got["packed"].astype(np.int64), want["packed"].astype(np.int64)
    assert np.array_equal(pg >> 16, pw >> 16), f"{label}: packed ids differ"
    if pg.size:
        assert np.abs((pg & 0xFFFF) - (pw & 0xFFFF)).max() <= 1, f"{label}: bf16 field > 1 ulp"
    assert int(got["num_experts_out"]) == int(want["num_experts_out"]), label
    for k in ("counts", "offsets", "perm", "inv_perm"):
        assert np.array_equal(got[k], want[k]), f"{label}: {k} differs"
