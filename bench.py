#!/usr/bin/env python3
"""Benchmark of the MI355X routing library (one GPU).

A step is one call of the whole routing path (sigmoid, bias, grouped top-k,
weights, pack/relabel, counts, offsets, permutation) on the long-prefill
workload: 32768 tokens x 896 fp32 logits, Zipf-skewed bias, rank range
[0, 112) -> 128 output ids. Inputs rotate over three seeded sets (3 x 117 MB
of logits) so they cannot be served from the 256 MB last-level cache.

Also reported: the grouped-GEMM layout of the step's entries (us per call),
a static balancing plan over 8 expert-owning ranks (us per call),
the fused route + MXFP8 activation quantisation at decode (H = 7168),
decode latency (us per call at 8, 16 and 64 tokens, eager and
replayed from a HIP graph), the router GEMM + route at 64 and 4096 tokens,
the roofline of the route kernel (timed live with HIP events on the launch
stream), and the CPU oracle timed on a bounded sample of the same workload.

Prints ONE JSON line on stdout.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import itertools
import json
import os
import platform
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routing µs/call at 8/16/64 tokens; routed tokens/s + HBM GB/s at 32K tokens"
HBM_PEAK_GBPS = 8000.0
BYTES_PER_TOKEN_PATH = 3904     # logits 3584 + ids, weights, packed, perm, inv (5 x 64)
BYTES_PER_TOKEN_ROUTE_KERNEL = 3776  # logits 3584 + ids, weights, packed (3 x 64)
COPY_BYTES = 512 << 20
PROFILE_PMC = os.path.join(ROOT, "profiles", "pmc_route_rows_long_prefill_32768.txt")
PROFILE_BUSY = os.path.join(ROOT, "profiles", "pmc_valu_busy_lds_conflicts_bench_default.txt")
# sources the routing kernels are built from (the router GEMM is not among them)
ROUTE_SOURCES = ("internal.hpp", "moe_route.hip", "rn_sigmoid.hpp", "route_rows.hpp",
                 "route_wave.hpp")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--decode-calls", type=int, default=1000)
    ap.add_argument("--oracle-seconds", type=float, default=12.0)
    ap.add_argument("--skip-oracle", action="store_true")
    ap.add_argument("--oracle-child", action="store_true", help=argparse.SUPPRESS)
    return ap.parse_args()


ORACLE_THREAD_ENV = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")


def oracle_child(seconds: float) -> None:
    """The CPU oracle timed on the host (run as a child process with one BLAS
    / OpenMP thread, before the parent touches the GPU): routed tokens/s on
    the long-prefill workload (chunks of 1024 tokens, each a full oracle call
    with the permutation, for up to `seconds`), and the best of three calls
    on the tiny, decode-local and decode-sweep workloads."""
    import numpy as np  # noqa: F401  (imported under the one-thread environment)

    import oracle as O
    import workloads as W

    def call(c):
        O.route_ref(c.logits, c.bias, n_groups=c.n_groups, topk_group=c.topk_group,
                    top_k=c.top_k, group_topn=c.group_topn, local_expert_offset=c.off,
                    num_local_experts=c.cnt)

    def best_us(c, reps=3):
        best = float("inf")
        for _ in range(reps):
            t0 = time.perf_counter()
            call(c)
            best = min(best, time.perf_counter() - t0)
        return round(best * 1e6, 1)

    per_workload = {"tiny_global_8": best_us(W.tiny_global(8)),
                    "decode_local_16_rank3": best_us(W.decode_local(16))}
    per_workload["decode_sweep_rank3"] = {f"T{T}": best_us(W.decode_sweep(T, 3))
                                          for T in W.DECODE_SWEEP_T}
    T = 32768
    c0 = W.long_prefill(T)
    chunk, done = 1024, 0
    t_start = time.perf_counter()
    while done < T and time.perf_counter() - t_start < seconds:
        O.route_ref(c0.logits[done:done + chunk], c0.bias, local_expert_offset=c0.off,
                    num_local_experts=c0.cnt)
        done += chunk
    el = time.perf_counter() - t_start
    print(json.dumps({"tokens": done, "of": T, "chunk": chunk, "seconds": el,
                      "workloads_us_per_call_best_of_3": per_workload}), flush=True)


def run_oracle_child(seconds: float):
    """Starts oracle_child in a child process (one thread) and returns its
    result, or None when it fails."""
    import subprocess
    env = dict(os.environ)
    for k in ORACLE_THREAD_ENV:
        env[k] = "1"
    cmd = [sys.executable, os.path.abspath(__file__), "--oracle-child",
           "--oracle-seconds", str(seconds)]
    try:
        res = subprocess.run(cmd, env=env, capture_output=True, text=True,
                             timeout=seconds + 300)
    except subprocess.TimeoutExpired:
        log("bench: the oracle child timed out")
        return None
    if res.returncode != 0:
        log(f"bench: the oracle child failed ({res.returncode}): {res.stderr[-500:]}")
        return None
    return json.loads(res.stdout.strip().splitlines()[-1])


def cpu_model() -> str:
    """The host CPU's model name (Linux), or an empty string."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def source_digest() -> str:
    """Digest of the routing sources' code: comments and blank space are
    dropped first, so that a documentation edit does not retire a profile
    taken on the same kernels."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "moe_expert_routing_amd", "csrc")
    for name in ROUTE_SOURCES:
        with open(os.path.join(csrc, name), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(name.encode() + " ".join(text.split()).encode())
    return h.hexdigest()[:16]


def read_profile(path: str, digest: str) -> dict:
    """key = value lines of a committed rocprofv3 summary, if it was taken on
    the current kernel sources (else an empty dict)."""
    if not os.path.exists(path):
        return {}
    kv = {}
    with open(path) as fh:
        for line in fh:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    return kv if kv.get("source_digest") == digest else {}


def read_traffic(digest: str):
    """HBM bytes per launch of the route kernel from the committed rocprofv3
    --pmc summary, if it was taken on the current kernel sources."""
    try:
        return float(read_profile(PROFILE_PMC, digest)["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def read_busy(digest: str) -> dict:
    """VALU-busy and LDS bank-conflict percentages per kernel from the
    committed rocprofv3 --pmc summary (VALUBusy, LDSBankConflict), if it was
    taken on the current kernel sources."""
    out = {}
    for k, v in read_profile(PROFILE_BUSY, digest).items():
        if k.endswith("_pct"):
            try:
                out[k] = float(v)
            except ValueError:
                pass
    return out


class HipEvents:
    """Raw hipEvent_t handles through the HIP runtime (for the kernel hook)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        ev = ctypes.c_void_p()
        assert self.hip.hipEventCreate(ctypes.byref(ev)) == 0
        return ev.value

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, ev):
        self.hip.hipEventDestroy(ev)


def main():
    args = parse()
    if args.oracle_child:
        oracle_child(args.oracle_seconds)
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(this library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    # the CPU oracle first, in a child process, before anything here touches
    # the GPU
    oracle_res = None
    if not args.skip_oracle:
        log(f"bench: oracle on the host, one thread (up to {args.oracle_seconds:.0f} s of "
            "long-prefill tokens, plus the small workloads)")
        oracle_res = run_oracle_child(args.oracle_seconds)

    import numpy as np
    import torch

    import moe_expert_routing_amd as M
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    M.lib()  # fail loudly if the HIP library is missing
    torch.cuda.set_device(dev)

    # ------------------------------------------------------------------
    # long prefill: 32768 tokens, 3 rotating input sets
    # ------------------------------------------------------------------
    T = 32768
    log("bench: generating the long-prefill inputs (3 sets)")
    cases = [W.long_prefill(T, variant=v) for v in range(3)]
    lg = [torch.from_numpy(c.logits).to(dev) for c in cases]
    bs = [torch.from_numpy(c.bias).to(dev) for c in cases]
    off, cnt = cases[0].off, cases[0].cnt
    e_out = M.local_num_experts(W.E, W.K, off, cnt)
    out = M.alloc_outputs(T, W.K, e_out, dev)
    ws = M.workspace(dev, M.lib().moe_route_workspace_bytes(T, e_out, W.K))

    def step(i):
        M.route_local(lg[i % 3], bs[i % 3], off, cnt, out=out, ws=ws)

    log(f"bench: warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    log(f"bench: timing {args.steps} steps")
    torch.cuda.synchronize()
    t0.record()
    for i in range(args.steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms_per_step = total_ms / args.steps

    # the route kernel alone: HIP events recorded right before and after its
    # launch on the launch stream, in a separate pass (the two extra event
    # packets per step would otherwise inflate the step time above)
    he = HipEvents()
    pairs = [(he.create(), he.create()) for _ in range(args.steps)]
    for i in range(args.steps):
        M.set_kernel_events(*pairs[i])
        step(i)
    torch.cuda.synchronize()
    M.set_kernel_events(None, None)
    kern_ms = [he.elapsed_ms(a, b) for a, b in pairs]
    for a, b in pairs:
        he.destroy(a)
        he.destroy(b)
    kern_avg_ms = sum(kern_ms) / len(kern_ms)
    tokens_per_s = T / (ms_per_step * 1e-3)
    path_gbps = BYTES_PER_TOKEN_PATH * T / (ms_per_step * 1e-3) / 1e9
    kern_gbps = BYTES_PER_TOKEN_ROUTE_KERNEL * T / (kern_avg_ms * 1e-3) / 1e9
    digest = source_digest()
    traffic = read_traffic(digest)
    busy = read_busy(digest)
    log(f"bench: {ms_per_step * 1e3:.1f} us/step, route kernel {kern_avg_ms * 1e3:.1f} us")

    # which kernel path the tokens of one step took
    for path in (M.PATH_EXACT, M.PATH_REFINED, M.PATH_REROUTED, M.PATH_RESCORED):
        M.path_tokens(path, reset=True)
    step(0)
    torch.cuda.synchronize()
    paths = {"tokens": T, "exact_refinement": M.path_tokens(M.PATH_REFINED, reset=True),
             "rerouted_one_token_per_wave": M.path_tokens(M.PATH_REROUTED, reset=True),
             "exact_pipeline": M.path_tokens(M.PATH_EXACT, reset=True),
             "rescored_one_token_per_wave": M.path_tokens(M.PATH_RESCORED, reset=True)}

    # ------------------------------------------------------------------
    # plain device copy of 512 MiB (HBM reference bandwidth; the same copy
    # calibrates the FETCH_SIZE / WRITE_SIZE counters)
    # ------------------------------------------------------------------
    log("bench: device copy of 512 MiB")
    csrc_buf = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    cdst_buf = torch.empty_like(csrc_buf)
    copy_ms = []
    for rep in range(6):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        cdst_buf.copy_(csrc_buf)
        b.record()
        torch.cuda.synchronize()
        if rep:
            copy_ms.append(a.elapsed_time(b))
    copy_gbps = 2 * COPY_BYTES / (statistics.median(copy_ms) * 1e-3) / 1e9
    del csrc_buf, cdst_buf

    # ------------------------------------------------------------------
    # decode latency
    # ------------------------------------------------------------------
    def time_calls(fn, n, reps=5):
        vals = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record()
            for _ in range(n):
                fn()
            b.record()
            torch.cuda.synchronize()
            vals.append(a.elapsed_time(b) * 1e3 / n)
        return statistics.median(vals)

    def time_graph(fn, n, reps=5):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for _ in range(3):
                fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        per_graph = 100
        with torch.cuda.graph(g):
            for _ in range(per_graph):
                fn()
        torch.cuda.synchronize()
        return time_calls(g.replay, max(1, n // per_graph), reps) / per_graph

    def empty_launch():
        torch.cuda._sleep(0)

    floor = {"eager": round(time_calls(empty_launch, args.decode_calls), 2),
             "hipgraph": round(time_graph(empty_launch, args.decode_calls), 2)}
    decode = {}
    decode_graph = {}
    decode_cases = {8: W.tiny_global(8), 16: W.decode_local(16), 64: W.decode_sweep(64, 0)}
    for Td, c in decode_cases.items():
        log(f"bench: decode T={Td}")
        dl = torch.from_numpy(c.logits).to(dev)
        db = torch.from_numpy(c.bias).to(dev)
        eo = M.local_num_experts(W.E, W.K, c.off, c.cnt) or W.E
        dout = M.alloc_outputs(Td, W.K, eo, dev)
        dws = torch.zeros(1 << 16, dtype=torch.uint8, device=dev)
        fn = (lambda dl=dl, db=db, c=c, dout=dout, dws=dws:
              M.route_local(dl, db, c.off, c.cnt, out=dout, ws=dws))
        fn()
        decode[f"T{Td}"] = round(time_calls(fn, args.decode_calls), 2)
        try:
            decode_graph[f"T{Td}"] = round(time_graph(fn, args.decode_calls), 2)
        except Exception as exc:  # graph capture is optional for the report
            decode_graph[f"T{Td}"] = f"unavailable: {type(exc).__name__}"

    # fused route + MXFP8 activation quantisation at decode (H = 7168), one
    # launch: us per call, eager and from a HIP graph
    decode_quant, decode_quant_graph = {}, {}
    for Td, c in decode_cases.items():
        log(f"bench: decode route+quant T={Td}")
        rng = np.random.default_rng(Td)
        hb = torch.from_numpy((rng.standard_normal((Td, W.H)).astype(np.float32).view(np.uint32)
                               >> 16).astype(np.uint16).view(np.int16)).to(dev)
        dl = torch.from_numpy(c.logits).to(dev)
        db = torch.from_numpy(c.bias).to(dev)
        eo = M.local_num_experts(W.E, W.K, c.off, c.cnt) or W.E
        qout = M.alloc_outputs(Td, W.K, eo, dev)
        qws = torch.zeros(1 << 16, dtype=torch.uint8, device=dev)
        qfn = (lambda dl=dl, db=db, hb=hb, c=c, qout=qout, qws=qws:
               M.route_quant_local(dl, db, hb, c.off, c.cnt, out=qout, ws=qws))
        qfn()
        decode_quant[f"T{Td}"] = round(time_calls(qfn, args.decode_calls), 2)
        decode_quant_graph[f"T{Td}"] = round(time_graph(qfn, args.decode_calls), 2)

    # the decode sweep (5..64 tokens, rank range [336, 448) -> 128 local ids,
    # exact twins among the logits): us per call from a HIP graph
    decode_sweep_graph = {}
    for Td in W.DECODE_SWEEP_T:
        c = W.decode_sweep(Td, 3)
        log(f"bench: decode sweep T={Td}")
        dl = torch.from_numpy(c.logits).to(dev)
        db = torch.from_numpy(c.bias).to(dev)
        eo = M.local_num_experts(W.E, W.K, c.off, c.cnt) or W.E
        sout = M.alloc_outputs(Td, W.K, eo, dev)
        sws = torch.zeros(1 << 16, dtype=torch.uint8, device=dev)
        sfn = (lambda dl=dl, db=db, c=c, sout=sout, sws=sws:
               M.route_local(dl, db, c.off, c.cnt, out=sout, ws=sws))
        sfn()
        decode_sweep_graph[f"T{Td}"] = round(time_graph(sfn, args.decode_calls), 2)

    # ------------------------------------------------------------------
    # grouped-GEMM layout of the long-prefill step's entries (tile 128): us
    # per call (eager and replayed from a HIP graph) and GB/s over its
    # algorithmic bytes (counts, perm, padded offsets, m_indices and
    # row_entry over the bound row count)
    # ------------------------------------------------------------------
    log("bench: grouped-GEMM layout")
    grouped = {}
    for tile in (128,):
        lay = M.grouped_layout(out["counts"], out["perm"], tile)
        rows = lay["m_indices"].shape[0]
        n_ent = out["perm"].shape[0]
        gl_bytes = 4 * e_out + 4 * n_ent + 4 * (e_out + 1) + 8 * rows
        gl_fn = (lambda tile=tile, lay=lay:
                 M.grouped_layout(out["counts"], out["perm"], tile, out=lay))
        gl_fn()
        gl_us = time_calls(gl_fn, 200)
        gl_graph_us = time_graph(gl_fn, 200)
        # the routing with the layout written by its own scatter
        # (moe_route_local_grouped), against the routing then the layout call;
        # the calls rotate over the 3 input sets like the timed steps (one set
        # alone would stay in the last-level cache)
        fused = M.route_local_grouped(lg[0], bs[0], off, cnt, tile_m=tile, rows=rows)
        ctr = itertools.count()

        def rt_fn():
            i = next(ctr) % 3
            M.route_local(lg[i], bs[i], off, cnt, out=out, ws=ws)

        def two_fn(tile=tile, lay=lay):
            rt_fn()
            M.grouped_layout(out["counts"], out["perm"], tile, out=lay)

        def fu_fn(tile=tile, fused=fused):
            i = next(ctr) % 3
            M.route_local_grouped(lg[i], bs[i], off, cnt, tile_m=tile, rows=rows, out=fused,
                                  ws=ws)
        fu_fn()
        grouped[f"tile{tile}"] = {"us_per_call": round(gl_us, 2),
                                  "us_per_call_hipgraph": round(gl_graph_us, 2), "rows": rows,
                                  "gbps_hipgraph": round(gl_bytes / (gl_graph_us * 1e-6) / 1e9, 1),
                                  "route_then_layout_us_per_call_hipgraph":
                                      round(time_graph(two_fn, 50), 2),
                                  "route_with_fused_layout_us_per_call_hipgraph":
                                      round(time_graph(fu_fn, 50), 2),
                                  "route_alone_us_per_call_hipgraph":
                                      round(time_graph(rt_fn, 50), 2)}

    # static balancing plan over 8 expert-owning ranks from the global counts
    # of the long-prefill input (routed once with global ids, untimed)
    log("bench: balancing plan")
    gout = M.route(lg[0], bs[0])
    n_ent = T * W.K
    plan = M.balance_plan(gout["counts"], 8, n_ent)
    pl_fn = lambda: M.balance_plan(gout["counts"], 8, n_ent, out=plan)
    pl_fn()
    torch.cuda.synchronize()
    rc = plan["rank_counts"].cpu().numpy()
    per = W.E // 8
    own = sum(int(rc[r, r * per:(r + 1) * per].sum()) for r in range(8))
    balance = {"ranks": 8, "entries": n_ent, "moved_entries": n_ent - own,
               "us_per_call": round(time_calls(pl_fn, 200), 2),
               "us_per_call_hipgraph": round(time_graph(pl_fn, 200), 2)}
    del gout

    # ------------------------------------------------------------------
    # router GEMM + route
    # ------------------------------------------------------------------
    gemm = {}
    for Tg in (64, 4096):
        log(f"bench: router GEMM + route T={Tg}")
        c = W.router_case(Tg)
        hid = torch.from_numpy(c.hidden.view(np.int16)).to(dev)
        wt = torch.from_numpy(c.weight.view(np.int16)).to(dev)
        gb = torch.from_numpy(c.bias).to(dev)
        glog = torch.empty((Tg, W.E), dtype=torch.float32, device=dev)
        gout = M.alloc_outputs(Tg, W.K, W.E, dev)
        gws = M.workspace(dev, M.lib().moe_router_gemm_route_workspace_bytes(Tg, W.H, W.E, W.E,
                                                                              W.K))
        fn = (lambda hid=hid, wt=wt, gb=gb, glog=glog, gout=gout, gws=gws:
              M.router_gemm_route(hid, wt, gb, logits=glog, out=gout, ws=gws))
        fn()
        us = time_calls(fn, 200 if Tg == 64 else 50)
        flops = 2.0 * Tg * W.E * W.H
        # context: the same product through the vendor library (hipBLASLt via
        # torch.mm, bf16 operands, fp32 output), GEMM only, no routing
        hb, wb = hid.view(torch.bfloat16), wt.view(torch.bfloat16).t()
        lib_fn = lambda hb=hb, wb=wb: torch.mm(hb, wb, out_dtype=torch.float32)
        try:
            lib_fn()
            lib_us = round(time_calls(lib_fn, 200 if Tg == 64 else 50), 2)
        except (RuntimeError, TypeError) as exc:  # a torch without fp32-output mm
            log(f"bench: library GEMM not timed ({exc})")
            lib_us = None
        gemm[f"T{Tg}"] = {"us_per_call": round(us, 2),
                          "tflops_incl_route": round(flops / (us * 1e-6) / 1e12, 2),
                          "library_gemm_only_us_per_call": lib_us}

    # ------------------------------------------------------------------
    # CPU oracle on a bounded sample of the same workload
    # ------------------------------------------------------------------
    cpu = None
    if oracle_res is not None:
        done, el = oracle_res["tokens"], oracle_res["seconds"]
        cpu = {"value": round(done / el, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"first {done} of the {T} long-prefill tokens, routed in chunks of "
                         f"{oracle_res['chunk']} tokens (each chunk a full oracle call incl. "
                         f"permutation), {el:.1f} s of Python+numpy in a child process with "
                         f"{', '.join(k + '=1' for k in ORACLE_THREAD_ENV)}, on "
                         f"{cpu_model() or platform.processor() or platform.machine()}, "
                         f"{os.cpu_count()} host cores present",
               "threads": 1,
               "small_workloads_us_per_call_best_of_3":
                   oracle_res["workloads_us_per_call_best_of_3"]}

    frac = kern_gbps / HBM_PEAK_GBPS
    res = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "long_prefill_32768x896_zipf_bias_range_0_112",
                   "tokens": T, "num_experts": W.E, "n_groups": W.G, "topk_group": W.TG,
                   "top_k": W.K, "local_expert_offset": off, "num_local_experts": cnt,
                   "num_experts_out": e_out, "input_sets_rotated": 3},
        "hbm_gbps_algorithmic_path": round(path_gbps, 1),
        "token_paths_per_step": paths,
        "copy_gbps_512MiB": round(copy_gbps, 1),
        "decode_us_per_call": decode,
        "empty_kernel_us_per_call": floor,
        "decode_us_per_call_hipgraph": decode_graph,
        "decode_sweep_rank_local_us_per_call_hipgraph": decode_sweep_graph,
        "router_gemm_route": gemm,
        "grouped_layout_32768": grouped,
        "balance_plan_32768": balance,
        "decode_route_quant_mxfp8_us_per_call": decode_quant,
        "decode_route_quant_mxfp8_us_per_call_hipgraph": decode_quant_graph,
        "roofline": {"bound": "hbm", "kernel": "route_rows_kernel",
                     "achieved": round(kern_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(frac, 4),
                     "kernel_us_avg": round(kern_avg_ms * 1e3, 2),
                     "bytes_per_token": BYTES_PER_TOKEN_ROUTE_KERNEL,
                     "frac_of_copy": round(kern_gbps / copy_gbps, 4),
                     "traffic": (round(traffic, 0) if traffic is not None else None),
                     "source_digest": digest,
                     "valu_busy_pct": busy.get("route_rows_valu_busy_pct"),
                     "lds_bank_conflict_pct": busy.get("route_rows_lds_bank_conflict_pct")},
        "counters_from_profiles": busy or None,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
