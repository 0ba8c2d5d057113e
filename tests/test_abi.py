"""C-ABI checks that need no GPU: the built library loads, exports every
function include/moe_route.h declares, and validates arguments on the host
(negative status, nothing launched)."""
import ctypes
import os
import re

import pytest

import moe_expert_routing_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_route.h")

OK, ERR_NULL, ERR_SHAPE, ERR_RANGE, ERR_UNSUP, ERR_WS, ERR_HIP = 0, -1, -2, -3, -4, -5, -6


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(M.LIB_PATH):
        pytest.skip("library not built")
    return M.lib()


def test_every_declared_symbol_is_exported(L):
    names = _declared_functions()
    assert "moe_route" in names and "moe_route_local" in names and "moe_router_gemm_route" in names
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(M.EXPORTS), "binding and header disagree"


def test_abi_version_and_status_strings(L):
    assert L.moe_route_abi_version() == 101
    for code in (OK, ERR_NULL, ERR_SHAPE, ERR_RANGE, ERR_UNSUP, ERR_WS, ERR_HIP):
        assert L.moe_route_status_string(code)
    assert L.moe_route_status_string(-99) == b"unknown status"


@pytest.mark.parametrize("off,cnt,want", [
    (0, 112, 128), (336, 112, 128), (784, 112, 128), (0, 448, 464), (448, 448, 464),
    (0, 224, 240), (0, 56, 72), (0, 0, 0), (0, 896, 0), (0, 884, 0), (0, 876, 892),
])
def test_local_num_experts_matches_rule(L, off, cnt, want):
    assert L.moe_route_local_num_experts(896, 16, off, cnt) == want


@pytest.mark.parametrize("off,cnt", [(-1, 10), (890, 10), (0, 897), (3, -2)])
def test_local_num_experts_range_errors(L, off, cnt):
    assert L.moe_route_local_num_experts(896, 16, off, cnt) == ERR_RANGE


def test_workspace_sizes(L):
    small = L.moe_route_workspace_bytes(64, 896, 16)
    assert small == 256  # decode path: control block only
    big = L.moe_route_workspace_bytes(32768, 128, 16)
    # control block + per-block id counts (4 tokens per block at most) + ranks
    assert big == 256 + 128 * (32768 // 4) * 4 + 32768 * 16
    assert L.moe_route_workspace_bytes(-1, 896, 16) == 0
    g = L.moe_router_gemm_route_workspace_bytes(64, 7168, 896, 896, 16)
    assert g > 256  # decode GEMM stages split-K partials


def _params(E=896, G=8, TG=4, K=16, N=2):
    return M.RouteParams(E, G, TG, K, N)


FAKE = 0x10000  # never dereferenced: every case below fails host validation


def _outs(**kw):
    d = dict(topk_ids=FAKE, topk_weights=FAKE, packed=FAKE, counts=FAKE, offsets=FAKE,
             perm=FAKE, inv_perm=None)
    d.update(kw)
    return M.RouteOutputs(**d)


def _route_local(L, prm, T=8, off=0, cnt=0, outs=None, ws=FAKE, ws_bytes=1 << 20, logits=FAKE,
                 bias=FAKE):
    o = outs or _outs()
    return L.moe_route_local(logits, bias, T, ctypes.byref(prm), off, cnt, ctypes.byref(o), ws,
                             ws_bytes, None)


@pytest.mark.parametrize("prm,want", [
    (_params(E=900), ERR_SHAPE),              # E % G != 0
    (_params(E=896 + 128 * 2), ERR_UNSUP),    # > 1024 experts
    (_params(E=832, G=8), ERR_UNSUP),         # E % 128 != 0 (832 = 8 * 104)
    (_params(G=6, E=768), ERR_UNSUP),         # G not a power of two
    (_params(TG=9), ERR_SHAPE),               # topk_group > n_groups
    (_params(K=33), ERR_UNSUP),               # top_k above the envelope
    (_params(K=0), ERR_SHAPE),
    (_params(N=3), ERR_UNSUP),                # group score of 3 terms
    (_params(TG=1, K=113), ERR_SHAPE),        # K > candidates of the kept groups
])
def test_parameter_validation(L, prm, want):
    assert _route_local(L, prm) == want


def test_null_and_shape_validation(L):
    prm = _params()
    assert _route_local(L, prm, T=-1) == ERR_SHAPE
    assert _route_local(L, prm, logits=None) == ERR_NULL
    assert _route_local(L, prm, bias=None) == ERR_NULL
    assert _route_local(L, prm, outs=_outs(perm=None)) == ERR_NULL
    assert _route_local(L, prm, outs=_outs(counts=None)) == ERR_NULL
    assert _route_local(L, prm, ws=None) == ERR_WS
    assert _route_local(L, prm, T=100, ws_bytes=256) == ERR_WS
    assert _route_local(L, prm, off=890, cnt=10) == ERR_RANGE
    assert _route_local(L, prm, off=-1, cnt=4) == ERR_RANGE
    assert _route_local(L, prm, logits=FAKE + 4) == ERR_SHAPE  # misaligned rows
    # entries t * top_k + k and their positions are int32: 2^27 tokens x 16
    assert _route_local(L, prm, T=1 << 27, ws_bytes=1 << 62) == ERR_SHAPE
    assert _route_local(L, prm, T=(1 << 27) - 1, ws_bytes=1 << 20) == ERR_WS
    assert L.moe_route(FAKE, FAKE, 8, None, ctypes.byref(_outs()), FAKE, 1 << 20, None) == ERR_NULL


def test_noalloc_validation(L):
    prm = _params()
    def call(T=8, off=0, cnt=0, p=prm, outs=None, logits=FAKE):
        o = outs or _outs()
        return L.moe_route_local_noalloc(logits, FAKE, T, ctypes.byref(p), off, cnt,
                                         ctypes.byref(o), None)
    assert call(T=-1) == ERR_SHAPE
    assert call(logits=None) == ERR_NULL
    assert call(outs=_outs(counts=None)) == ERR_NULL
    assert call(off=890, cnt=10) == ERR_RANGE
    assert call(p=_params(N=3)) == ERR_UNSUP
    # the static scratch (16 MiB) holds 69,888 tokens at 896 global ids on the
    # four-tokens-per-wave path; one more token is refused before any launch
    assert call(T=69_889) == ERR_WS
    assert call(T=69_889, logits=FAKE + 8) == ERR_WS      # one-token-per-wave tiles: larger
    assert call(T=400_000, off=0, cnt=112) == ERR_WS       # E' = 128


def test_router_gemm_validation(L):
    prm = _params()
    o = _outs()
    def call(T=8, H=7168, hidden=FAKE, weight=FAKE, logits=FAKE, ws_bytes=1 << 26, off=0, cnt=0,
             p=prm):
        return L.moe_router_gemm_route(hidden, weight, T, H, FAKE, logits, ctypes.byref(p), off,
                                       cnt, ctypes.byref(o), FAKE, ws_bytes, None)
    assert call(H=7160) == ERR_UNSUP          # H not a multiple of 64
    assert call(hidden=None) == ERR_NULL
    assert call(logits=None) == ERR_NULL
    assert call(ws_bytes=16) == ERR_WS
    assert call(off=890, cnt=10) == ERR_RANGE
    assert call(p=_params(N=3)) == ERR_UNSUP  # routing args checked before any launch
    assert call(hidden=FAKE + 2) == ERR_SHAPE
    assert call(logits=FAKE + 8) == ERR_SHAPE   # logits 16-byte aligned


def test_route_quant_validation(L):
    prm = _params()
    o = _outs()
    def call(T=8, hidden=FAKE, H=7168, q=FAKE, sc=FAKE, off=0, cnt=0, p=prm, ws_bytes=1 << 20):
        return L.moe_route_quant_local(FAKE, FAKE, T, ctypes.byref(p), off, cnt, hidden, H, q, sc,
                                       ctypes.byref(o), FAKE, ws_bytes, None)
    assert call(H=7160) == ERR_SHAPE         # not a multiple of 32
    assert call(H=0) == ERR_SHAPE
    assert call(hidden=None) == ERR_NULL
    assert call(q=None) == ERR_NULL
    assert call(sc=None) == ERR_NULL
    assert call(hidden=FAKE + 8) == ERR_SHAPE  # 16-byte alignment
    assert call(q=FAKE + 4) == ERR_SHAPE
    assert call(p=_params(N=3)) == ERR_UNSUP   # routing arguments checked as by moe_route_local
    assert call(off=890, cnt=10) == ERR_RANGE
    assert call(ws_bytes=16) == ERR_WS


def test_balance_plan_validation(L):
    def call(counts=FAKE, E=896, N=8, n=128, dest=FAKE, rc=FAKE):
        return L.moe_balance_plan(counts, E, N, n, dest, rc, None)
    assert call(N=0) == ERR_SHAPE
    assert call(N=65) == ERR_SHAPE
    assert call(E=900) == ERR_SHAPE          # not a multiple of the rank count
    assert call(E=2048, N=8) == ERR_SHAPE    # above 1024 experts
    assert call(n=-1) == ERR_SHAPE
    assert call(counts=None) == ERR_NULL
    assert call(rc=None) == ERR_NULL
    assert call(dest=None) == ERR_NULL


def test_grouped_layout_validation(L):
    assert L.moe_grouped_layout_rows(100, 128, 64) == 100 + 128 * 63
    assert L.moe_grouped_layout_rows(0, 896, 1) == 0
    assert L.moe_grouped_layout_rows(-1, 128, 64) == ERR_SHAPE
    assert L.moe_grouped_layout_rows(10, 0, 64) == ERR_SHAPE
    assert L.moe_grouped_layout_rows(10, 1025, 64) == ERR_SHAPE
    assert L.moe_grouped_layout_rows(10, 128, 0) == ERR_SHAPE
    assert L.moe_grouped_layout_rows(10, 128, 4097) == ERR_SHAPE
    assert L.moe_grouped_layout_rows((1 << 30) + 1, 128, 64) == ERR_SHAPE
    def call(counts=FAKE, perm=FAKE, E=128, n=100, tile=64, po=FAKE, mi=FAKE, re=FAKE, rows=None):
        rows = 100 + 128 * 63 if rows is None else rows
        return L.moe_grouped_layout(counts, perm, E, n, tile, po, mi, re, rows, None)
    assert call(counts=None) == ERR_NULL
    assert call(perm=None) == ERR_NULL
    assert call(po=None) == ERR_NULL
    assert call(mi=None) == ERR_NULL
    assert call(rows=100 + 128 * 63 - 1) == ERR_SHAPE
    assert call(tile=0) == ERR_SHAPE
    assert call(E=0) == ERR_SHAPE


def test_route_grouped_validation(L):
    # the routing checks first, then the layout's; all before any launch
    prm = _params()
    n = 8 * 16
    need = n + 896 * 63  # global ids: E' = 896

    def call(prm=prm, T=8, tile=64, po=FAKE, mi=FAKE, re=FAKE, rows=need, ws_bytes=1 << 20,
             logits=FAKE):
        return L.moe_route_local_grouped(logits, FAKE, T, ctypes.byref(prm), 0, 0,
                                         ctypes.byref(_outs()), tile, po, mi, re, rows, FAKE,
                                         ws_bytes, None)
    assert call(prm=_params(K=33)) == ERR_UNSUP
    assert call(logits=None) == ERR_NULL
    assert call(T=100, ws_bytes=256) == ERR_WS
    assert call(tile=0) == ERR_SHAPE
    assert call(tile=4097) == ERR_SHAPE
    assert call(po=None) == ERR_NULL
    assert call(mi=None) == ERR_NULL
    assert call(rows=need - 1) == ERR_SHAPE


def test_sigmoid_validation(L):
    assert L.moe_sigmoid_rn32(FAKE, FAKE, -1, 0, None) == ERR_SHAPE
    assert L.moe_sigmoid_rn32(None, FAKE, 5, 0, None) == ERR_NULL
    assert L.moe_sigmoid_rn32(FAKE, FAKE, 5, 3, None) == ERR_UNSUP  # invalid mode: no launch
    assert L.moe_sigmoid_rn32(FAKE, FAKE, 0, 0, None) == OK


def test_binding_fails_loudly_without_gpu_tensors():
    import torch
    with pytest.raises(M.MoeRouteError):
        M.route(torch.zeros(4, 896), torch.zeros(896))


def test_binding_noalloc_limit_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define MOE_ROUTE_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m is not None
    assert int(m.group(1)) << int(m.group(2)) == M.NOALLOC_SCRATCH_BYTES
