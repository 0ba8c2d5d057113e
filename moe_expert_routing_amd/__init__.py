"""Python binding of libmoe_route.so: the MI355X routed-MoE routing step.

Argument marshalling only. Every step of the routing runs in the HIP
kernels behind the C ABI of ``include/moe_route.h``; this module passes
``tensor.data_ptr()`` values and the current HIP stream, allocates output
tensors and a cached workspace when the caller gives none, and turns a
negative status into an exception. There is no CPU fallback: without the
built library every call raises.

Calls (same names as the C ABI):
    route(logits, bias, ...)                       -> moe_route
    route_local(logits, bias, off, cnt, ...)       -> moe_route_local
    route_local_noalloc(logits, bias, off, cnt)    -> moe_route_local_noalloc
    router_gemm_route(hidden, weight, bias, ...)   -> moe_router_gemm_route
    local_num_experts(E, K, off, cnt)              -> moe_route_local_num_experts
    route_quant_local(logits, bias, hidden, ...)   -> moe_route_quant_local
    grouped_layout(counts, perm, tile_m, ...)      -> moe_grouped_layout
    route_local_grouped(logits, bias, off, cnt, tile_m=...) -> moe_route_local_grouped
    balance_plan(counts, n_ranks, n_entries)       -> moe_balance_plan
    grouped_layout_rows(n_entries, E', tile_m)     -> moe_grouped_layout_rows
    sigmoid_rn32(x, mode=0)                        -> moe_sigmoid_rn32 (diagnostic)
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_lib", "libmoe_route.so")

MAX_FUSED_TOKENS = 64
NOALLOC_SCRATCH_BYTES = 16 << 20  # MOE_ROUTE_NOALLOC_SCRATCH_BYTES

_c_i32 = ctypes.c_int32
_c_vp = ctypes.c_void_p


class RouteParams(ctypes.Structure):
    _fields_ = [("num_experts", _c_i32), ("n_groups", _c_i32), ("topk_group", _c_i32),
                ("top_k", _c_i32), ("group_topn", _c_i32)]


class RouteOutputs(ctypes.Structure):
    _fields_ = [("topk_ids", _c_vp), ("topk_weights", _c_vp), ("packed", _c_vp),
                ("counts", _c_vp), ("offsets", _c_vp), ("perm", _c_vp), ("inv_perm", _c_vp)]


EXPORTS = {
    "moe_route_abi_version": (_c_i32, []),
    "moe_route_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_route_local_num_experts": (_c_i32, [_c_i32, _c_i32, _c_i32, _c_i32]),
    "moe_route_workspace_bytes": (ctypes.c_size_t, [_c_i32, _c_i32, _c_i32]),
    "moe_route": (ctypes.c_int, [_c_vp, _c_vp, _c_i32, ctypes.POINTER(RouteParams),
                                 ctypes.POINTER(RouteOutputs), _c_vp, ctypes.c_size_t, _c_vp]),
    "moe_route_local": (ctypes.c_int, [_c_vp, _c_vp, _c_i32, ctypes.POINTER(RouteParams),
                                       _c_i32, _c_i32, ctypes.POINTER(RouteOutputs), _c_vp,
                                       ctypes.c_size_t, _c_vp]),
    "moe_route_local_noalloc": (ctypes.c_int, [_c_vp, _c_vp, _c_i32, ctypes.POINTER(RouteParams),
                                               _c_i32, _c_i32, ctypes.POINTER(RouteOutputs),
                                               _c_vp]),
    "moe_route_local_grouped": (ctypes.c_int, [_c_vp, _c_vp, _c_i32, ctypes.POINTER(RouteParams),
                                               _c_i32, _c_i32, ctypes.POINTER(RouteOutputs),
                                               _c_i32, _c_vp, _c_vp, _c_vp, ctypes.c_int64,
                                               _c_vp, ctypes.c_size_t, _c_vp]),
    "moe_router_gemm_route_workspace_bytes": (ctypes.c_size_t,
                                              [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32]),
    "moe_router_gemm_route": (ctypes.c_int, [_c_vp, _c_vp, _c_i32, _c_i32, _c_vp, _c_vp,
                                             ctypes.POINTER(RouteParams), _c_i32, _c_i32,
                                             ctypes.POINTER(RouteOutputs), _c_vp,
                                             ctypes.c_size_t, _c_vp]),
    "moe_sigmoid_rn32": (ctypes.c_int, [_c_vp, _c_vp, ctypes.c_int64, _c_i32, _c_vp]),
    "moe_route_set_kernel_events": (ctypes.c_int, [_c_vp, _c_vp]),
    "moe_route_exact_path_tokens": (ctypes.c_int64, [_c_i32]),
    "moe_route_path_tokens": (ctypes.c_int64, [_c_i32, _c_i32]),
    "moe_grouped_layout_rows": (ctypes.c_int64, [ctypes.c_int64, _c_i32, _c_i32]),
    "moe_balance_plan": (ctypes.c_int, [_c_vp, _c_i32, _c_i32, ctypes.c_int64, _c_vp, _c_vp,
                                        _c_vp]),
    "moe_route_quant_local": (ctypes.c_int, [_c_vp, _c_vp, _c_i32, ctypes.POINTER(RouteParams),
                                             _c_i32, _c_i32, _c_vp, _c_i32, _c_vp, _c_vp,
                                             ctypes.POINTER(RouteOutputs), _c_vp,
                                             ctypes.c_size_t, _c_vp]),
    "moe_grouped_layout": (ctypes.c_int, [_c_vp, _c_vp, _c_i32, ctypes.c_int64, _c_i32, _c_vp,
                                          _c_vp, _c_vp, ctypes.c_int64, _c_vp]),
}

_LIB = None


class MoeRouteError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """Load the built HIP library (raises if it was not built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise MoeRouteError(
                f"{LIB_PATH} is missing: build it with `python -m moe_expert_routing_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def _check(status: int, what: str) -> None:
    if status != 0:
        msg = lib().moe_route_status_string(status).decode()
        raise MoeRouteError(f"{what} failed: {msg} ({status})")


_E_OUT: Dict[tuple, int] = {}


def local_num_experts(num_experts: int, top_k: int, local_expert_offset: int,
                      num_local_experts: int) -> int:
    key = (num_experts, top_k, local_expert_offset, num_local_experts)
    v = _E_OUT.get(key)
    if v is None:
        v = int(lib().moe_route_local_num_experts(*key))
        if v < 0:
            _check(v, "moe_route_local_num_experts")
        _E_OUT[key] = v
    return v


_RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(device: torch.device) -> int:
    """The current HIP stream of `device` as an integer handle."""
    idx = device.index
    if _RAW_STREAM is not None and idx is not None:
        return _RAW_STREAM(idx)
    return torch.cuda.current_stream(device).cuda_stream


# Default workspaces, one per (device, stream): calls that may run at the same
# time must not share one (the decode ticket and the prefill tile counts live
# there), and a workspace is only ever replaced on the stream it was
# allocated and used on, so the caching allocator's stream tracking holds.
_WORKSPACES: Dict[tuple, torch.Tensor] = {}


def _new_workspace(nbytes: int, device: torch.device) -> torch.Tensor:
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def workspace(device: torch.device, nbytes: int, stream: Optional[int] = None) -> torch.Tensor:
    """A zero-initialised byte buffer of at least nbytes, cached per (device,
    stream); `stream` defaults to the device's current stream. Its control
    block is zero when allocated and every call leaves it zero."""
    idx = device.index if device.index is not None else torch.cuda.current_device()
    if stream is None:
        stream = _stream_handle(torch.device("cuda", idx))
    key = (idx, int(stream))
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = _new_workspace(max(nbytes, 1 << 16), device)
        _WORKSPACES[key] = ws
    return ws


def cached_workspace(device: torch.device, stream: Optional[int] = None):
    """The default workspace of (device, stream) if one was made, else None."""
    idx = device.index if device.index is not None else torch.cuda.current_device()
    if stream is None:
        stream = _stream_handle(torch.device("cuda", idx))
    return _WORKSPACES.get((idx, int(stream)))


def alloc_outputs(T: int, top_k: int, e_out: int, device: torch.device,
                  with_inv: bool = True) -> Dict[str, torch.Tensor]:
    i32 = dict(dtype=torch.int32, device=device)
    out = {
        "topk_ids": torch.empty((T, top_k), **i32),
        "topk_weights": torch.empty((T, top_k), dtype=torch.float32, device=device),
        "packed": torch.empty((T, top_k), **i32),
        "counts": torch.empty((e_out,), **i32),
        "offsets": torch.empty((e_out + 1,), **i32),
        "perm": torch.empty((T * top_k,), **i32),
        "inv_perm": torch.empty((T * top_k,), **i32) if with_inv else None,
    }
    return out


_OUTPUT_NAMES = ("topk_ids", "topk_weights", "packed", "counts", "offsets", "perm", "inv_perm")
_PRM_CACHE: Dict[tuple, tuple] = {}  # params struct (and its byref) per shape


def _outputs_struct(out: Dict[str, torch.Tensor]) -> RouteOutputs:
    def p(name):
        t = out.get(name)
        return t.data_ptr() if t is not None and t.numel() > 0 else None
    return RouteOutputs(*(p(n) for n in _OUTPUT_NAMES))


def _params_ref(E, n_groups, topk_group, top_k, group_topn):
    key = (E, n_groups, topk_group, top_k, group_topn)
    hit = _PRM_CACHE.get(key)
    if hit is None:
        prm = RouteParams(*key)
        hit = _PRM_CACHE[key] = (prm, ctypes.byref(prm))
    return hit


def _require(t: torch.Tensor, name: str, dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise MoeRouteError(f"{name} must be a GPU tensor")
    if t.dtype != dtype or t.dim() != ndim or not t.is_contiguous():
        raise MoeRouteError(f"{name} must be a contiguous {ndim}-d {dtype} tensor")


def _params(E, n_groups, topk_group, top_k, group_topn) -> RouteParams:
    return RouteParams(E, n_groups, topk_group, top_k, group_topn)


def route_local(logits: torch.Tensor, bias: torch.Tensor, local_expert_offset: int = 0,
                num_local_experts: int = 0, *, n_groups: int = 8, topk_group: int = 4,
                top_k: int = 16, group_topn: int = 2,
                out: Optional[Dict[str, torch.Tensor]] = None,
                ws: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """moe_route_local over torch tensors; returns the output tensors."""
    _require(logits, "logits", torch.float32, 2)
    _require(bias, "bias", torch.float32, 1)
    T, E = logits.shape
    if bias.shape[0] != E:
        raise MoeRouteError("bias must have num_experts elements")
    e_loc = local_num_experts(E, top_k, local_expert_offset, num_local_experts)
    e_out = e_loc if e_loc > 0 else E
    dev = logits.device
    if out is None:
        out = alloc_outputs(T, top_k, e_out, dev)
    sh = _stream_handle(dev)
    if ws is None:  # a caller's workspace is checked by the library itself
        ws = workspace(dev, lib().moe_route_workspace_bytes(T, e_out, top_k), sh)
    prm = _params_ref(E, n_groups, topk_group, top_k, group_topn)
    o = _outputs_struct(out)
    st = lib().moe_route_local(logits.data_ptr(), bias.data_ptr(), T, prm[1],
                               local_expert_offset, num_local_experts, ctypes.byref(o),
                               ws.data_ptr(), ws.numel(), sh)
    if st:
        _check(st, "moe_route_local")
    out["num_experts_out"] = e_out
    return out


def route_local_noalloc(logits: torch.Tensor, bias: torch.Tensor, local_expert_offset: int = 0,
                        num_local_experts: int = 0, *, n_groups: int = 8, topk_group: int = 4,
                        top_k: int = 16, group_topn: int = 2,
                        out: Optional[Dict[str, torch.Tensor]] = None
                        ) -> Dict[str, torch.Tensor]:
    """moe_route_local_noalloc: route_local on the library's static scratch
    (no workspace). With `out` given, the call allocates nothing."""
    _require(logits, "logits", torch.float32, 2)
    _require(bias, "bias", torch.float32, 1)
    T, E = logits.shape
    if bias.shape[0] != E:
        raise MoeRouteError("bias must have num_experts elements")
    e_loc = local_num_experts(E, top_k, local_expert_offset, num_local_experts)
    e_out = e_loc if e_loc > 0 else E
    dev = logits.device
    if out is None:
        out = alloc_outputs(T, top_k, e_out, dev)
    prm = _params_ref(E, n_groups, topk_group, top_k, group_topn)
    o = _outputs_struct(out)
    with torch.cuda.device(dev):
        st = lib().moe_route_local_noalloc(logits.data_ptr(), bias.data_ptr(), T, prm[1],
                                           local_expert_offset, num_local_experts,
                                           ctypes.byref(o), _stream_handle(dev))
    if st == -5:
        raise MoeRouteError(
            f"moe_route_local_noalloc failed: {T} tokens with {e_out} output ids need more "
            f"scratch than the library's static {NOALLOC_SCRATCH_BYTES >> 20} MiB (-5)")
    if st:
        _check(st, "moe_route_local_noalloc")
    out["num_experts_out"] = e_out
    return out


def route_quant_local(logits: torch.Tensor, bias: torch.Tensor, hidden: torch.Tensor,
                      local_expert_offset: int = 0, num_local_experts: int = 0, *,
                      n_groups: int = 8, topk_group: int = 4, top_k: int = 16,
                      group_topn: int = 2, out: Optional[Dict[str, torch.Tensor]] = None,
                      ws: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """moe_route_quant_local: routing as route_local plus the MXFP8
    activations act_q (uint8 E4M3 codes [T, H]) and act_scale (uint8 E8M0
    codes [T, H/32]). hidden: bf16 (or 16-bit bit patterns) [T, H]."""
    _require(logits, "logits", torch.float32, 2)
    _require(bias, "bias", torch.float32, 1)
    if not hidden.is_cuda or hidden.dim() != 2 or not hidden.is_contiguous() or \
            hidden.element_size() != 2:
        raise MoeRouteError("hidden must be a contiguous 2-d 16-bit GPU tensor")
    T, E = logits.shape
    H = hidden.shape[1]
    if hidden.shape[0] != T or bias.shape[0] != E:
        raise MoeRouteError("inconsistent shapes")
    e_loc = local_num_experts(E, top_k, local_expert_offset, num_local_experts)
    e_out = e_loc if e_loc > 0 else E
    dev = logits.device
    if out is None:
        out = alloc_outputs(T, top_k, e_out, dev)
    if "act_q" not in out:
        out["act_q"] = torch.empty((T, H), dtype=torch.uint8, device=dev)
        out["act_scale"] = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
    sh = _stream_handle(dev)
    if ws is None:
        ws = workspace(dev, lib().moe_route_workspace_bytes(T, e_out, top_k), sh)
    prm = _params_ref(E, n_groups, topk_group, top_k, group_topn)
    o = _outputs_struct(out)
    st = lib().moe_route_quant_local(logits.data_ptr(), bias.data_ptr(), T, prm[1],
                                     local_expert_offset, num_local_experts, hidden.data_ptr(),
                                     H, out["act_q"].data_ptr(), out["act_scale"].data_ptr(),
                                     ctypes.byref(o), ws.data_ptr(), ws.numel(), sh)
    if st:
        _check(st, "moe_route_quant_local")
    out["num_experts_out"] = e_out
    return out


def route(logits: torch.Tensor, bias: torch.Tensor, *, n_groups: int = 8, topk_group: int = 4,
          top_k: int = 16, group_topn: int = 2, out: Optional[Dict[str, torch.Tensor]] = None,
          ws: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """moe_route (global ids) over torch tensors."""
    _require(logits, "logits", torch.float32, 2)
    _require(bias, "bias", torch.float32, 1)
    T, E = logits.shape
    dev = logits.device
    if out is None:
        out = alloc_outputs(T, top_k, E, dev)
    sh = _stream_handle(dev)
    if ws is None:  # a caller's workspace is checked by the library itself
        ws = workspace(dev, lib().moe_route_workspace_bytes(T, E, top_k), sh)
    prm = _params_ref(E, n_groups, topk_group, top_k, group_topn)
    o = _outputs_struct(out)
    st = lib().moe_route(logits.data_ptr(), bias.data_ptr(), T, prm[1], ctypes.byref(o),
                         ws.data_ptr(), ws.numel(), sh)
    _check(st, "moe_route")
    out["num_experts_out"] = E
    return out


def router_gemm_route(hidden: torch.Tensor, weight: torch.Tensor, bias: torch.Tensor,
                      local_expert_offset: int = 0, num_local_experts: int = 0, *,
                      n_groups: int = 8, topk_group: int = 4, top_k: int = 16,
                      group_topn: int = 2, logits: Optional[torch.Tensor] = None,
                      out: Optional[Dict[str, torch.Tensor]] = None,
                      ws: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """moe_router_gemm_route: bf16 hidden [T, H] . bf16 weight [E, H]^T -> fp32
    logits, then routing. hidden/weight may be bfloat16 or int16/uint16 bit
    patterns."""
    for t, n in ((hidden, "hidden"), (weight, "weight")):
        if not t.is_cuda or t.dim() != 2 or not t.is_contiguous() or t.element_size() != 2:
            raise MoeRouteError(f"{n} must be a contiguous 2-d 16-bit GPU tensor")
    _require(bias, "bias", torch.float32, 1)
    T, H = hidden.shape
    E = weight.shape[0]
    if weight.shape[1] != H or bias.shape[0] != E:
        raise MoeRouteError("inconsistent router GEMM shapes")
    dev = hidden.device
    e_loc = local_num_experts(E, top_k, local_expert_offset, num_local_experts)
    e_out = e_loc if e_loc > 0 else E
    if logits is None:
        logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    _require(logits, "logits", torch.float32, 2)
    if out is None:
        out = alloc_outputs(T, top_k, e_out, dev)
    need = lib().moe_router_gemm_route_workspace_bytes(T, H, E, e_out, top_k)
    sh = _stream_handle(dev)
    if ws is None:
        ws = workspace(dev, need, sh)
    prm = _params(E, n_groups, topk_group, top_k, group_topn)
    o = _outputs_struct(out)
    st = lib().moe_router_gemm_route(hidden.data_ptr(), weight.data_ptr(), T, H,
                                      bias.data_ptr(), logits.data_ptr(), ctypes.byref(prm),
                                      local_expert_offset, num_local_experts, ctypes.byref(o),
                                      ws.data_ptr(), ws.numel(), sh)
    _check(st, "moe_router_gemm_route")
    out["logits"] = logits
    out["num_experts_out"] = e_out
    return out


def set_kernel_events(before: Optional[int], after: Optional[int]) -> None:
    """Benchmark hook: record two hipEvent_t handles around the route kernel
    of every later call (None, None turns it off)."""
    _check(lib().moe_route_set_kernel_events(before, after), "moe_route_set_kernel_events")


def exact_path_tokens(reset: bool = False) -> int:
    """Diagnostic: tokens routed through the exact path since the last reset."""
    v = lib().moe_route_exact_path_tokens(1 if reset else 0)
    if v < 0:
        _check(int(v), "moe_route_exact_path_tokens")
    return int(v)


PATH_EXACT, PATH_REFINED, PATH_REROUTED, PATH_RESCORED = 0, 1, 2, 3


def path_tokens(path: int, reset: bool = False) -> int:
    """Diagnostic: tokens that took a kernel path since the last reset
    (PATH_EXACT, PATH_REFINED, PATH_REROUTED or PATH_RESCORED; see
    moe_route_path_tokens)."""
    v = lib().moe_route_path_tokens(path, 1 if reset else 0)
    if v < 0:
        _check(int(v), "moe_route_path_tokens")
    return int(v)


def grouped_layout_rows(n_entries: int, num_experts_out: int, tile_m: int) -> int:
    v = lib().moe_grouped_layout_rows(n_entries, num_experts_out, tile_m)
    if v < 0:
        _check(int(v), "moe_grouped_layout_rows")
    return int(v)


def grouped_layout(counts: torch.Tensor, perm: torch.Tensor, tile_m: int, *,
                   rows: Optional[int] = None, with_entries: bool = True,
                   out: Optional[Dict[str, torch.Tensor]] = None) -> Dict[str, torch.Tensor]:
    """moe_grouped_layout over a routing call's counts [E'] and perm [T*K]:
    padded_offsets [E'+1], m_indices [rows] and (with_entries) row_entry
    [rows]. rows defaults to the bound moe_grouped_layout_rows."""
    _require(counts, "counts", torch.int32, 1)
    _require(perm, "perm", torch.int32, 1)
    e_out, n = counts.shape[0], perm.shape[0]
    need = grouped_layout_rows(n, e_out, tile_m)
    rows = need if rows is None else rows
    dev = counts.device
    if out is None:
        out = {"padded_offsets": torch.empty(e_out + 1, dtype=torch.int32, device=dev),
               "m_indices": torch.empty(rows, dtype=torch.int32, device=dev)}
        if with_entries:
            out["row_entry"] = torch.empty(rows, dtype=torch.int32, device=dev)
    re = out.get("row_entry")
    st = lib().moe_grouped_layout(counts.data_ptr(), perm.data_ptr() if n else None, e_out, n,
                                  tile_m, out["padded_offsets"].data_ptr(),
                                  out["m_indices"].data_ptr() if rows else None,
                                  re.data_ptr() if re is not None and rows else None, rows,
                                  _stream_handle(dev))
    if st:
        _check(st, "moe_grouped_layout")
    return out


def route_local_grouped(logits: torch.Tensor, bias: torch.Tensor, local_expert_offset: int = 0,
                        num_local_experts: int = 0, *, tile_m: int, n_groups: int = 8,
                        topk_group: int = 4, top_k: int = 16, group_topn: int = 2,
                        rows: Optional[int] = None, with_entries: bool = True,
                        out: Optional[Dict[str, torch.Tensor]] = None,
                        ws: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """moe_route_local_grouped: route_local's outputs plus padded_offsets,
    m_indices and (with_entries) row_entry of the grouped-GEMM layout. rows
    defaults to the bound moe_grouped_layout_rows."""
    _require(logits, "logits", torch.float32, 2)
    _require(bias, "bias", torch.float32, 1)
    T, E = logits.shape
    if bias.shape[0] != E:
        raise MoeRouteError("bias must have num_experts elements")
    e_loc = local_num_experts(E, top_k, local_expert_offset, num_local_experts)
    e_out = e_loc if e_loc > 0 else E
    dev = logits.device
    need = grouped_layout_rows(T * top_k, e_out, tile_m)
    rows = need if rows is None else rows
    if out is None:
        out = alloc_outputs(T, top_k, e_out, dev)
        out["padded_offsets"] = torch.empty(e_out + 1, dtype=torch.int32, device=dev)
        out["m_indices"] = torch.empty(rows, dtype=torch.int32, device=dev)
        if with_entries:
            out["row_entry"] = torch.empty(rows, dtype=torch.int32, device=dev)
    sh = _stream_handle(dev)
    if ws is None:  # a caller's workspace is checked by the library itself
        ws = workspace(dev, lib().moe_route_workspace_bytes(T, e_out, top_k), sh)
    prm = _params_ref(E, n_groups, topk_group, top_k, group_topn)
    o = _outputs_struct(out)
    re = out.get("row_entry")
    st = lib().moe_route_local_grouped(logits.data_ptr(), bias.data_ptr(), T, prm[1],
                                       local_expert_offset, num_local_experts, ctypes.byref(o),
                                       tile_m, out["padded_offsets"].data_ptr(),
                                       out["m_indices"].data_ptr() if rows else None,
                                       re.data_ptr() if re is not None and rows else None, rows,
                                       ws.data_ptr(), ws.numel(), sh)
    if st:
        _check(st, "moe_route_local_grouped")
    out["num_experts_out"] = e_out
    return out


def balance_plan(counts: torch.Tensor, n_ranks: int, n_entries: int, *,
                 out: Optional[Dict[str, torch.Tensor]] = None) -> Dict[str, torch.Tensor]:
    """moe_balance_plan over a routing call's global counts [E]: dest
    [n_entries] (rank of each entry of perm) and rank_counts [n_ranks, E]."""
    _require(counts, "counts", torch.int32, 1)
    E = counts.shape[0]
    dev = counts.device
    if out is None:
        out = {"dest": torch.empty(n_entries, dtype=torch.int32, device=dev),
               "rank_counts": torch.empty((n_ranks, E), dtype=torch.int32, device=dev)}
    st = lib().moe_balance_plan(counts.data_ptr(), E, n_ranks, n_entries,
                                out["dest"].data_ptr() if n_entries else None,
                                out["rank_counts"].data_ptr(), _stream_handle(dev))
    if st:
        _check(st, "moe_balance_plan")
    return out


def sigmoid_rn32(x: torch.Tensor, mode: int = 0) -> torch.Tensor:
    """Diagnostic: the kernels' correctly rounded sigmoid over a 1-d tensor."""
    _require(x, "x", torch.float32, 1)
    y = torch.empty_like(x)
    st = lib().moe_sigmoid_rn32(x.data_ptr(), y.data_ptr(), x.numel(), mode,
                                _stream_handle(x.device))
    _check(st, "moe_sigmoid_rn32")
    return y
