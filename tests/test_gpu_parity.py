"""GPU parity of the HIP routing path against the CPU oracle, through the C
ABI, on every workload and on edge cases."""
import numpy as np
import pytest
import torch

import moe_expert_routing_amd as M
import oracle as O
import workloads as W
from gpu_util import (DEV, assert_parity, assert_workspace_zero, oracle_case, run_case, say,
                      to_dev, to_numpy)

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]


# --------------------------------------------------------------------------
# sigmoid (diagnostic entry point): bit-exact against the oracle
# --------------------------------------------------------------------------

def _hard_sigmoid_inputs(n_keep=4000):
    """Inputs whose binary64 sigmoid lies closest to a binary32 rounding
    boundary (found by a strided sweep), plus saturation and subnormal
    regions."""
    u = np.arange(0, 1 << 23, dtype=np.uint32) * np.uint32(509) + np.uint32(0x3C000000)
    x = u.view(np.float32)
    x = np.concatenate([x, -x])
    x = x[np.isfinite(x) & (np.abs(x) < 60)]
    d = 1.0 / (1.0 + np.exp(-x.astype(np.float64)))
    f = d.astype(np.float32)
    ulp = np.nextafter(f, np.float32(np.inf)).astype(np.float64) - f.astype(np.float64)
    frac = np.abs(np.abs(d - f.astype(np.float64)) / ulp - 0.5)
    hard = x[np.argsort(frac)[:n_keep]]
    extra = np.concatenate([
        np.linspace(-115, -80, 3001, dtype=np.float32),
        np.linspace(15, 45, 1001, dtype=np.float32),
        np.array([0.0, -0.0, 1e-30, -1e-30, 3e38, -3e38, 40.0, -110.0], np.float32),
    ])
    return np.concatenate([hard, extra]).astype(np.float32)


@pytest.mark.parametrize("mode", [0, 1])
def test_sigmoid_bit_exact(mode):
    rng = np.random.default_rng(77)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32),
                        (8 * rng.standard_normal(50000)).astype(np.float32),
                        _hard_sigmoid_inputs()])
    say(f"sigmoid mode={mode} n={x.size}")
    y = M.sigmoid_rn32(to_dev(x), mode=mode).cpu().numpy()
    want = O.sigmoid_rn32(x)
    bad = np.nonzero(y.view(np.uint32) != want.view(np.uint32))[0]
    assert bad.size == 0, [(float(x[i]), float(y[i]), float(want[i])) for i in bad[:5]]


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------

def test_tiny_global_8_tokens():
    c = W.tiny_global()
    say("case tiny_global T=8")
    assert_parity(run_case(c), oracle_case(c), c.name)


def test_decode_local_16_tokens_rank3():
    c = W.decode_local()
    say("case decode_local T=16 off=336 cnt=112")
    got, want = run_case(c), oracle_case(c)
    assert int(want["num_experts_out"]) == 128
    assert_parity(got, want, c.name)


@pytest.mark.parametrize("T", W.DECODE_SWEEP_T)
def test_decode_sweep_all_ranks_with_ties(T):
    for rank in range(W.EP):
        c = W.decode_sweep(T, rank)
        say(f"case {c.name}")
        assert_parity(run_case(c), oracle_case(c), c.name)


def test_long_prefill_32k_full():
    c = W.long_prefill()
    say("case long_prefill T=32768 off=0 cnt=112 (full oracle comparison)")
    got = run_case(c)
    want = oracle_case(c)
    assert_parity(got, want, c.name)
    load = np.bincount(want["topk_ids"].ravel(), minlength=896)
    assert load.max() / load.mean() > 7.0


@pytest.mark.parametrize("off,cnt", [(0, 112), (0, 0)])
def test_long_prefill_beyond_one_wave_round(off, cnt):
    # 49,189 tokens: more route blocks than the row kernel keeps resident at
    # once (1024 at 32,768 tokens), and a last block holding 5 tokens
    T = 49189
    base = W.long_prefill(T, variant=1)
    c = W.RouteCase(f"long_prefill_T{T}_off{off}_cnt{cnt}", base.logits, base.bias, off=off,
                    cnt=cnt)
    say(f"case long_prefill T={T} off={off} cnt={cnt} (full oracle comparison)")
    assert_parity(run_case(c), oracle_case(c), c.name)


@pytest.mark.parametrize("T", [1, 64, 100, 129, 1000, 4096])
def test_router_gemm_then_route(T):
    c = W.router_case(T)
    say(f"case router_gemm T={T}")
    hid = to_dev(c.hidden.view(np.int16))
    wt = to_dev(c.weight.view(np.int16))
    out = M.router_gemm_route(hid, wt, to_dev(c.bias))
    torch.cuda.synchronize()
    assert_workspace_zero()
    logits = out["logits"].cpu().numpy()
    ref = O.router_logits_ref(c.hidden, c.weight)
    bound = O.router_logits_bound(c.hidden, c.weight)
    err = np.abs(logits.astype(np.float64) - ref)
    assert np.all(err <= bound), f"max err {err.max():.3g} vs bound {bound.min():.3g}"
    got = {k: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v) for k, v in out.items()}
    want = O.route_ref(logits, c.bias)  # routing parity on the GPU's own logits
    assert_parity(got, want, c.name)


@pytest.mark.parametrize("T,E,H,G,TG,K", [
    (1, 256, 2048, 8, 4, 8),      # decode tiles, 4 expert tiles
    (100, 256, 2048, 8, 4, 8),    # two token tiles of the decode shape
    (300, 256, 2048, 8, 4, 8),    # prefill tiles, 2 expert tiles, split K
    (64, 1024, 1024, 16, 4, 16),  # 16 expert tiles
    (129, 1024, 1024, 16, 4, 16),
    (2000, 128, 512, 8, 4, 4),    # one expert tile, 16 token tiles
])
def test_router_gemm_other_shapes(T, E, H, G, TG, K):
    c = W.router_case(T, e=E, h=H)
    say(f"case router_gemm T={T} E={E} H={H}")
    out = M.router_gemm_route(to_dev(c.hidden.view(np.int16)), to_dev(c.weight.view(np.int16)),
                              to_dev(c.bias), n_groups=G, topk_group=TG, top_k=K)
    torch.cuda.synchronize()
    assert_workspace_zero()
    logits = out["logits"].cpu().numpy()
    ref = O.router_logits_ref(c.hidden, c.weight)
    bound = O.router_logits_bound(c.hidden, c.weight)
    err = np.abs(logits.astype(np.float64) - ref)
    assert np.all(err <= bound), f"max err {err.max():.3g}"
    got = {k: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v) for k, v in out.items()}
    want = O.route_ref(logits, c.bias, n_groups=G, topk_group=TG, top_k=K)
    assert_parity(got, want, c.name)


def test_router_gemm_decode_calls_in_a_row():
    # Decode-sized GEMMs split K and sum the partials in a fixed order: calls
    # of other sizes in between (other splits, other partial layouts in the
    # same workspace) leave the control block zero, and a repeated call gives
    # the same logits bit for bit.
    first = {}
    for T in (64, 8, 100, 1, 64, 8, 100):
        c = W.router_case(T)
        say(f"case router_gemm in a row T={T}")
        out = M.router_gemm_route(to_dev(c.hidden.view(np.int16)), to_dev(c.weight.view(np.int16)),
                                  to_dev(c.bias))
        torch.cuda.synchronize()
        assert_workspace_zero()
        logits = out["logits"].cpu().numpy()
        if T in first:
            assert np.array_equal(logits, first[T]), f"T={T}: logits differ between calls"
            continue
        ref = O.router_logits_ref(c.hidden, c.weight)
        bound = O.router_logits_bound(c.hidden, c.weight)
        err = np.abs(logits.astype(np.float64) - ref)
        assert np.all(err <= bound), f"T={T}: max err {err.max():.3g}"
        first[T] = logits


# --------------------------------------------------------------------------
# edge cases
# --------------------------------------------------------------------------

def test_zero_tokens():
    c = W.random_case(0, seed=1, off=336, cnt=112)
    say("case T=0")
    got = run_case(c)
    assert got["counts"].tolist() == [0] * 128
    assert got["offsets"].tolist() == [0] * 129
    assert got["perm"].size == 0


@pytest.mark.parametrize("T", [1, 2, 3, 63, 64, 65, 127, 129, 1000, 4099])
def test_ragged_token_counts_cross_both_paths(T):
    for off, cnt in ((0, 0), (448, 112)):
        c = W.random_case(T, seed=500 + T, off=off, cnt=cnt)
        say(f"case ragged T={T} off={off} cnt={cnt}")
        assert_parity(run_case(c), oracle_case(c), c.name)


@pytest.mark.parametrize("ep", [2, 4, 16])
@pytest.mark.parametrize("which", ["first", "middle", "last"])
def test_rank_ranges(ep, which):
    cnt = 896 // ep
    rank = {"first": 0, "middle": ep // 2, "last": ep - 1}[which]
    for T in (1, 24, 64, 200):
        c = W.random_case(T, seed=7000 + 100 * ep + 10 * rank + T, off=rank * cnt, cnt=cnt)
        say(f"case ep={ep} rank={rank} T={T}")
        assert_parity(run_case(c), oracle_case(c), c.name)


def test_range_that_does_not_apply_keeps_global_ids():
    c = W.random_case(40, seed=91, off=0, cnt=884)  # round_up(900, 4) >= 896
    say("case range not applying")
    got = run_case(c)
    assert int(got["num_experts_out"]) == 896
    assert_parity(got, oracle_case(c), c.name)


@pytest.mark.parametrize("E,G,TG,K,N", [
    (896, 1, 1, 16, 2),     # plain top-k
    (896, 8, 8, 16, 2),     # every group kept
    (896, 8, 4, 16, 1),     # group score = group max
    (896, 8, 2, 8, 2),
    (896, 8, 1, 16, 2),     # one group kept, top-16 (one token per wave: 12 TG < K + 1)
    (896, 8, 1, 8, 2),      # one group kept on the row path: the top 9 from one quad's pools
    (896, 8, 4, 1, 2),      # top-1: two tournament rounds, weight 1
    (896, 8, 1, 11, 2),     # the largest top-k the row path takes with one kept group
    (896, 8, 4, 32, 2),     # top-32: one token per wave; 160 entries in one decode block
    (256, 8, 4, 8, 2),
    (1024, 16, 4, 32, 2),
    (128, 64, 8, 4, 2),
    (512, 4, 1, 32, 1),
])
def test_other_parameters(E, G, TG, K, N):
    for T in (5, 130):
        c = W.random_case(T, seed=E + G + TG + K + N + T, e=E, n_groups=G, topk_group=TG,
                          top_k=K, group_topn=N)
        say(f"case E={E} G={G} TG={TG} K={K} N={N} T={T}")
        assert_parity(run_case(c), oracle_case(c), c.name)


def test_extreme_logits_and_dense_ties():
    rng = np.random.default_rng(3)
    T = 96
    logits = rng.choice(np.array([-120, -100, -95, -90, -88, -30, -1, 0, 1, 2, 30, 50],
                                 np.float32), size=(T, 896)).astype(np.float32)
    logits[:8] = 0.0  # every score ties: lower ids win
    c = W.RouteCase("extreme", logits, np.zeros(896, np.float32), off=112, cnt=112)
    say("case extreme logits")
    assert_parity(run_case(c), oracle_case(c), c.name)
    c2 = W.RouteCase("extreme_bias", logits, (0.01 * rng.standard_normal(896)).astype(np.float32))
    assert_parity(run_case(c2), oracle_case(c2), c2.name)


def test_two_streams_route_concurrently():
    # Calls on two streams of one device, not synchronised with each other:
    # each stream has its own default workspace (the 16-token decode's
    # ticket, the 4099-token prefill's tile counts), so every call returns
    # exactly what the same call returns alone.
    ca = W.decode_local(16)
    cb = W.random_case(4099, seed=77, off=448, cnt=112)
    say("case two streams: decode T=16 and prefill T=4099")
    alone_a, alone_b = run_case(ca), run_case(cb)
    la, ba, lb, bb = to_dev(ca.logits), to_dev(ca.bias), to_dev(cb.logits), to_dev(cb.bias)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    torch.cuda.synchronize()
    outs = []
    for _ in range(8):
        with torch.cuda.stream(sa):
            outs.append(("a", M.route_local(la, ba, ca.off, ca.cnt)))
        with torch.cuda.stream(sb):
            outs.append(("b", M.route_local(lb, bb, cb.off, cb.cnt)))
    torch.cuda.synchronize()
    for which, out in outs:
        got, want = to_numpy(out), (alone_a if which == "a" else alone_b)
        for k in ("topk_ids", "topk_weights", "packed", "counts", "offsets", "perm", "inv_perm"):
            assert np.array_equal(got[k], want[k]), f"stream {which}: {k} differs"


@pytest.mark.parametrize("T", [8, 16, 4099])
def test_graph_replays_match_eager(T):
    # One routing call captured in a HIP graph (one-block decode, multi-block
    # decode with its ticket, prefill with its tile counts), replayed with
    # eager work in between: the outputs are overwritten and another routing
    # call runs before every replay, and each replay gives the eager result.
    c = W.random_case(T, seed=90 + T, off=336, cnt=112)
    other = W.random_case(100, seed=5)
    say(f"case graph replays T={T}")
    lg, bs = to_dev(c.logits), to_dev(c.bias)
    e_out = M.local_num_experts(896, 16, c.off, c.cnt)
    eager = to_numpy(M.route_local(lg, bs, c.off, c.cnt))
    out = M.alloc_outputs(T, 16, e_out, DEV)
    ws = torch.zeros(M.lib().moe_route_workspace_bytes(T, e_out, 16), dtype=torch.uint8,
                     device=DEV)
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        M.route_local(lg, bs, c.off, c.cnt, out=out, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        M.route_local(lg, bs, c.off, c.cnt, out=out, ws=ws)
    keys = ("topk_ids", "topk_weights", "packed", "counts", "offsets", "perm", "inv_perm")
    for rep in range(4):
        for k in keys:
            out[k].fill_(-1)
        run_case(other)  # eager routing between replays
        g.replay()
        torch.cuda.synchronize()
        got = to_numpy(out)
        for k in keys:
            assert np.array_equal(got[k], eager[k]), f"replay {rep}: {k} differs"
    assert int(ws[:256].count_nonzero()) == 0, "control block not left zeroed"


def test_deterministic_across_calls():
    c = W.long_prefill(T=8192)
    say("case determinism T=8192")
    a = run_case(c)
    b = run_case(c)
    for k in ("topk_ids", "topk_weights", "packed", "counts", "offsets", "perm", "inv_perm"):
        assert np.array_equal(a[k], b[k]), k


def test_decode_and_prefill_paths_agree():
    """The single-launch decode path and the tiled prefill path select the
    same experts in the same slots; their weights agree within the weight
    tolerance (each is within 1e-6 of the oracle's; the prefill path may take
    them from its certified approximate scores)."""
    c = W.long_prefill(T=256)
    say("case decode-vs-prefill")
    big = run_case(c)
    small_case = W.RouteCase("first64", c.logits[:64], c.bias, off=c.off, cnt=c.cnt)
    small = run_case(small_case)
    assert np.array_equal(big["topk_ids"][:64], small["topk_ids"])
    assert np.array_equal(big["packed"][:64] >> 16, small["packed"] >> 16)
    bf = np.abs((big["packed"][:64] & 0xFFFF).astype(np.int64) - (small["packed"] & 0xFFFF))
    assert bf.max() <= 1
    wb, ws = big["topk_weights"][:64].astype(np.float64), small["topk_weights"].astype(np.float64)
    assert (np.abs(wb - ws) / ws).max() <= 2e-6
    assert_parity(small, oracle_case(small_case), "decode path")
    assert_parity(big, oracle_case(c), "prefill path")


def test_global_and_local_entries_reach_the_gemm_in_the_same_order():
    """The pages' invariant: the same (token, local expert, weight) entries in
    the same order under global and rank-local ids."""
    c = W.long_prefill(T=3000)
    off, cnt = 336, 112
    say("case global-vs-local order")
    g = run_case(W.RouteCase("g", c.logits, c.bias))
    loc = run_case(W.RouteCase("l", c.logits, c.bias, off=off, cnt=cnt))
    K = 16

    def entries(res, lo, hi, shift):
        ids = res["packed"] >> 16
        sel = []
        for f in res["perm"]:
            t, k = divmod(int(f), K)
            e = int(ids[t, k])
            if lo <= e < hi:
                sel.append((t, e + shift, int(res["packed"][t, k] & 0xFFFF)))
        return sel
    assert entries(loc, 0, cnt, off) == entries(g, off, off + cnt, 0)
    assert np.array_equal(g["topk_ids"], loc["topk_ids"])
    assert np.array_equal(g["packed"] & 0xFFFF, loc["packed"] & 0xFFFF)


# --------------------------------------------------------------------------
# decode edges: negative bias offsets and scores that underflow to zero
# --------------------------------------------------------------------------

def _underflow_case(T, rank, offset, seed):
    """N(0,1) logits with a bias moved by `offset`; every 4th row (from row
    1) keeps 8 experts and pushes the others to logits <= -104, whose
    sigmoid rounds to 0 so that their biased score is the bias alone (<= 0
    here); every 4th row from row 3 keeps only one expert. The selection
    then takes experts with s = 0 (weight 0)."""
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, 896), dtype=np.float32)
    bias = (np.float32(0.01) * rng.standard_normal(896, dtype=np.float32) +
            np.float32(offset)).astype(np.float32)
    for t in range(T):
        if t % 4 in (1, 3):
            keep = rng.choice(896, size=8 if t % 4 == 1 else 1, replace=False)
            row = (-104.0 - 16.0 * rng.random(896)).astype(np.float32)
            row[keep] = logits[t, keep]
            logits[t] = row
    return W.RouteCase(f"underflow_T{T}_r{rank}_b{offset}", logits, bias,
                       off=112 * rank, cnt=112)


def _tied_underflow_case(T, rank, offset):
    """Every expert's bias equal to `offset` and every logit <= -104 except
    one expert per row: all other biased scores tie exactly at the bias, so
    the top-k is decided by expert id alone; the kept expert takes weight 1."""
    logits = np.full((T, 896), -110.0, np.float32)
    logits[np.arange(T), (np.arange(T) * 131 + 7) % 896] = 0.25
    return W.RouteCase(f"tied_underflow_T{T}_r{rank}_b{offset}", logits,
                       np.full(896, offset, np.float32), off=112 * rank, cnt=112)


@pytest.mark.parametrize("offset", [-0.3, -0.9, -3.0])
@pytest.mark.parametrize("T", [1, 8, 16, 64])
def test_decode_negative_bias_and_underflow(T, offset):
    ranks = range(8) if T == 16 else (0, 3, 7)
    for rank in ranks:
        c = _underflow_case(T, rank, offset, seed=900 + 10 * T + rank)
        say(f"case {c.name}")
        got, want = run_case(c), oracle_case(c)
        assert_parity(got, want, c.name)
        M.exact_path_tokens(reset=True)
        c2 = _tied_underflow_case(T, rank, offset)
        say(f"case {c2.name}")
        got2, want2 = run_case(c2), oracle_case(c2)
        assert_parity(got2, want2, c2.name)
        exact = M.exact_path_tokens(reset=True)
        assert exact >= T, (c2.name, exact)  # exact ties: the exact pipeline decides
        assert np.all(np.sort(got2["topk_weights"], axis=1)[:, -1] == 1.0)


def test_wave_kernel_on_the_896_shape_with_8_byte_aligned_logits():
    """Logits 8 but not 16 bytes aligned: the 896-expert, 8-group shape runs
    the one-token-per-wave kernel (its float4 loads need 16-byte rows).
    Near-tie rows show which kernel decided: the wave kernel rescores its
    candidates, the four-tokens-per-wave kernel would refine its rows."""
    c = _near_tie_case(T=1000, seed=13)
    buf = torch.empty(1000 * 896 + 4, dtype=torch.float32, device=DEV)
    base = (16 - buf.data_ptr() % 16) // 4 % 4       # first 16-byte aligned element
    view = buf[base + 2: base + 2 + 1000 * 896].view(1000, 896)
    assert view.data_ptr() % 16 == 8
    view.copy_(torch.from_numpy(c.logits))
    for path in (M.PATH_REFINED, M.PATH_RESCORED):
        M.path_tokens(path, reset=True)
    say("case T=1000 896/8 logits at an 8-byte offset")
    out = M.route_local(view, to_dev(c.bias), c.off, c.cnt)
    torch.cuda.synchronize()
    got = {k: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v) for k, v in out.items()}
    assert_parity(got, oracle_case(c), "offset logits")
    refined = M.path_tokens(M.PATH_REFINED, reset=True)
    rescored = M.path_tokens(M.PATH_RESCORED, reset=True)
    say(f"refined {refined}, rescored {rescored}")
    assert refined == 0 and rescored > 0


# --------------------------------------------------------------------------
# the fast path's error bound and its fallback
# --------------------------------------------------------------------------

def _kernel_fast_sig_err():
    import os
    import re
    src = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                       "moe_expert_routing_amd", "csrc", "route_wave.hpp")
    m = re.search(r"FAST_SIG_ERR\s*=\s*0x1p-(\d+)f", open(src).read())
    return 2.0 ** -int(m.group(1))


def test_fast_sigmoid_error_bound_exhaustive():
    """Every finite binary32 input: |fast approximation - exact| must stay
    below half the bound the kernels certify their selections against (the
    approximation only ranks; scores that decide and weights are exact)."""
    bound = _kernel_fast_sig_err()
    worst, worst_x = 0.0, None
    chunk = 1 << 26
    say(f"fast sigmoid sweep of 2^32 inputs, bound {bound:.3g}")
    for c in range((1 << 32) // chunk):
        bits = torch.arange(c * chunk, (c + 1) * chunk, dtype=torch.int64, device=DEV)
        bits = torch.where(bits >= (1 << 31), bits - (1 << 32), bits).to(torch.int32)
        x = bits.view(torch.float32)
        x = torch.where(torch.isfinite(x), x, torch.zeros_like(x))
        exact = M.sigmoid_rn32(x, mode=0).double()
        fast = M.sigmoid_rn32(x, mode=2).double()
        err = (fast - exact).abs()
        i = int(torch.argmax(err))
        if float(err[i]) > worst:
            worst, worst_x = float(err[i]), float(x[i])
    say(f"worst |fast - exact| = {worst:.4g} at x = {worst_x}")
    assert worst <= bound / 2, (worst, worst_x)


def test_both_paths_are_exercised():
    """Random decode tokens take the fast path; rows whose scores all tie
    take the exact path; both give the oracle's answer."""
    c = W.random_case(64, seed=4242, off=112, cnt=112)
    M.exact_path_tokens(reset=True)
    assert_parity(run_case(c), oracle_case(c), "random64")
    n_random = M.exact_path_tokens(reset=True)
    logits = np.zeros((16, 896), np.float32)
    c2 = W.RouteCase("all_tied", logits, np.zeros(896, np.float32))
    assert_parity(run_case(c2), oracle_case(c2), "all_tied")
    n_tied = M.exact_path_tokens(reset=True)
    say(f"exact-path tokens: random {n_random}/64, all-tied {n_tied}/16")
    assert n_random <= 2 and n_tied == 16


# --------------------------------------------------------------------------
# the four-tokens-per-wave prefill path: its exact refinement and the
# one-token-per-wave reroute, forced by near-ties, exact ties and full ties
# --------------------------------------------------------------------------

def _near_tie_case(T=256, seed=9):
    """Rows whose best non-winner is moved to within a few ulp of the 16th
    winner (odd rows) or whose 5th group is moved to within a few ulp of the
    4th group's score (even rows): both fall inside the fast path's error
    band, so the exact refinement has to decide."""
    c = W.random_case(T, seed=seed)
    logits, bias = c.logits.copy(), c.bias
    s = O.sigmoid_rn32(logits)
    for t in range(T):
        sp = O.biased_scores(s[t:t + 1], bias)[0]
        gs = O.group_scores(sp, 8, 2)
        groups = O.kept_groups(gs, 4)
        if t % 2:
            ids = O.topk_experts(sp, groups, 8, 17)
            i, j = ids[15], ids[16]
            target = float(sp[i]) - float(bias[j])
        else:
            order = np.argsort(-gs, kind="stable")
            g5 = int(order[4])
            grp = sp[g5 * 112:(g5 + 1) * 112]
            top = np.argsort(-grp, kind="stable")
            j = g5 * 112 + int(top[0])
            target = float(gs[order[3]]) - float(grp[top[1]]) - float(bias[j])
        if 0.0 < target < 1.0:
            logits[t, j] = np.float32(np.log(target) - np.log1p(-target))
    return W.RouteCase("near_ties", logits, bias, off=224, cnt=112)


def test_decode_rescores_near_ties():
    """Decode tokens whose best non-winner sits within a few ulp of the 16th
    winner (odd rows) fail the certificate on approximate candidate scores,
    and their candidates are scored again exactly; tokens whose 5th group
    sits within a few ulp of the 4th (even rows) get exact group scores from
    their pools. Both give the oracle's answer."""
    c = _near_tie_case(T=64, seed=11)
    for path in (M.PATH_EXACT, M.PATH_RESCORED):
        M.path_tokens(path, reset=True)
    say("case near ties T=64 (decode)")
    assert_parity(run_case(c), oracle_case(c), c.name)
    rescored = M.path_tokens(M.PATH_RESCORED, reset=True)
    exact = M.path_tokens(M.PATH_EXACT, reset=True)
    say(f"rescored {rescored}, exact pipeline {exact}")
    assert rescored >= 48, (rescored, exact)


def test_prefill_rows_refine_near_ties():
    c = _near_tie_case()
    for path in (M.PATH_EXACT, M.PATH_REFINED, M.PATH_REROUTED):
        M.path_tokens(path, reset=True)
    say("case near ties T=256")
    assert_parity(run_case(c), oracle_case(c), c.name)
    refined = M.path_tokens(M.PATH_REFINED, reset=True)
    rerouted = M.path_tokens(M.PATH_REROUTED, reset=True)
    say(f"refined {refined}, rerouted {rerouted}")
    assert refined >= 64, refined


@pytest.mark.parametrize("rank", [0, 5])
def test_prefill_rows_with_exact_ties(rank):
    c = W.decode_sweep(256, rank)
    M.path_tokens(M.PATH_REFINED, reset=True)
    say(f"case exact ties T=256 rank={rank}")
    assert_parity(run_case(c), oracle_case(c), c.name)
    assert M.path_tokens(M.PATH_REFINED, reset=True) > 0


def test_prefill_rows_all_tied_reroute():
    logits = np.zeros((100, 896), np.float32)
    logits[50:] = 0.5
    c = W.RouteCase("all_tied_prefill", logits, np.zeros(896, np.float32))
    M.path_tokens(M.PATH_REROUTED, reset=True)
    say("case all tied T=100")
    assert_parity(run_case(c), oracle_case(c), c.name)
    assert M.path_tokens(M.PATH_REROUTED, reset=True) == 100


@pytest.mark.parametrize("offset,all_rerouted", [
    (0.45, False), (-0.45, False), (1.5, False), (-0.9, False), (600.0, True)])
def test_prefill_rows_key_windows(offset, all_rerouted):
    """Biases near both edges of the narrow key window (b + 1/2), inside the
    wide one (b + 3), and outside both, where every row goes through the exact
    per-token pipeline; the result is the oracle's in every case."""
    c = W.random_case(200, seed=31)
    bias = (c.bias + np.float32(offset)).astype(np.float32)
    case = W.RouteCase(f"bias_offset_{offset}", c.logits, bias)
    M.path_tokens(M.PATH_REROUTED, reset=True)
    say(f"case bias offset {offset} T=200")
    assert_parity(run_case(case), oracle_case(case), case.name)
    rerouted = M.path_tokens(M.PATH_REROUTED, reset=True)
    assert (rerouted == 200) if all_rerouted else (rerouted < 200), rerouted


@pytest.mark.parametrize("kind", ["reroute", "refine"])
def test_prefill_many_blocks_with_slow_rows(kind):
    """More route blocks (3075 of 16 tokens) than the GPU holds at once, a
    ragged last block, and rows that leave the fast path scattered over all
    of them: fully tied rows (routed again one token per wave) or rows with
    exact twins near the 16th place (refined). Everything matches the
    oracle."""
    T = 16 * 3074 + 5
    rng = np.random.default_rng(20261207)
    logits = rng.standard_normal((T, 896), dtype=np.float32)
    if kind == "reroute":
        bias = np.zeros(896, np.float32)
        logits[::409] = np.float32(0.5)
        path = M.PATH_REROUTED
    else:
        src = W.decode_sweep(256, 0)
        bias = src.bias
        rows = np.arange(1, T, 97)
        logits[rows] = src.logits[rows % 256]
        path = M.PATH_REFINED
    c = W.RouteCase(f"many_tiles_{kind}", logits, bias, off=0, cnt=112)
    M.path_tokens(path, reset=True)
    say(f"case many tiles per block T={T} kind={kind}")
    assert_parity(run_case(c), oracle_case(c), c.name)
    n = M.path_tokens(path, reset=True)
    say(f"{kind}: {n} tokens off the fast path")
    assert n > 0
