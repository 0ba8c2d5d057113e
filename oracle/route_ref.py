"""Plain CPU oracle of the routed-MoE routing step.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or run anything in this
package. The product path (the HIP library and its Python binding) never
does, and shares no code with it: the only module both sides use is
``workloads`` (seeded random inputs, no routing arithmetic).

What it computes, in the pages' order:

* a sigmoid router with a correction bias and a grouped top-k
  ("[ROCm][Perf] Kimi-K3: token-sharded residual stream for long prefills",
  the author's reply on shard-routed test coverage in the review thread);
* 896 experts and top_k 16 ("[kimi-k3] Rank-local expert ids for the EP
  routed MoE (upstream #45544)", commit message: the 896-expert, top-16
  routing specialisation);
* packed routed entries, expert id in the high half and the bf16 weight in
  the low half (same commit message, the passage on the fused route+quant
  launch);
* the rank-local relabel of the pack epilogue: experts of the rank's range
  become 0..count-1, any other expert in top-k slot k becomes count + k, and
  the local problem size is num_experts = round_up(count + top_k, 4) (same
  passage; 128 at EP8, also in the PR description's "What" line);
* per-expert counts, exclusive offsets and the expert-major permutation that
  feeds the expert GEMMs, with the same (token, local expert, weight) entries
  in the same order as under global ids (same commit message).

The pages leave open the group count and score, the tie rules, the sigmoid's
rounding and the renormalisation. This oracle takes the plainest readings:

* sigmoid: the correctly rounded binary32 value of 1 / (1 + e^-x);
* biased score sp = fl32(s + b), used for selection only;
* group score: fl32 sum of the group's top `group_topn` biased scores, taken
  with multiplicity, largest first;
* groups ranked by (score desc, group index asc); experts by (sp desc,
  expert id asc); slot k is the k-th expert in that order;
* weights: the unbiased s of the selected experts divided by their sum,
  evaluated in binary64 (exact sum via math.fsum) and rounded to binary32;
* bf16: round-to-nearest-even of the binary32 weight;
* within one expert, entries are ordered by ascending flat index t*top_k+k;
* grouped-GEMM layout (a consumer of counts and perm): each id's entries in
  permutation order from its tile-padded offset, padding rows marked -1;
* activations of the fused route + quant launch: OCP MXFP8 (E4M3 elements,
  one E8M0 scale per 32 elements), round to nearest even, saturating;
* a static balancing plan over N expert-owning ranks: owners keep up to
  their share of the entries, the surplus fills the short ranks in order.

Every function below has a pin in ``tests/test_oracle_*.py`` (brute force,
library routines, closed forms, mpmath, and the value the pages print).
No part of this oracle is "parity unpinned".
"""
from __future__ import annotations

import math
from decimal import Decimal, localcontext
from typing import Dict, Tuple

import numpy as np

# Relative distance to a binary32 rounding boundary below which the binary64
# evaluation of the sigmoid is not trusted (its own error is below 2^-50).
ZIV_REL = 2.0 ** -40

# ----------------------------------------------------------------------------
# a1: sigmoid, correctly rounded to binary32
# ----------------------------------------------------------------------------


def _sigmoid_decimal(x: float) -> Decimal:
    """1 / (1 + e^-x) with 60 significant decimal digits (x is exact)."""
    with localcontext() as ctx:
        ctx.prec = 60
        xd = Decimal(x)
        return Decimal(1) / (Decimal(1) + (-xd).exp())


def sigmoid_rn32(x: np.ndarray) -> np.ndarray:
    """s = RN32(1 / (1 + e^-x)) for every binary32 x (finite).

    Evaluates in binary64; where the binary64 value lies within ZIV_REL of a
    binary32 rounding boundary it re-evaluates with 60-digit decimal
    arithmetic and rounds against the exact boundary. Subnormal results are
    kept.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    xd = x.astype(np.float64)
    with np.errstate(over="ignore"):
        d = 1.0 / (1.0 + np.exp(-xd))
    f = d.astype(np.float32)
    up = np.nextafter(f, np.float32(np.inf))
    dn = np.nextafter(f, np.float32(-np.inf))
    fd = f.astype(np.float64)
    m_up = (fd + up.astype(np.float64)) * 0.5
    m_dn = (fd + dn.astype(np.float64)) * 0.5
    thr = ZIV_REL * d
    risky = (np.abs(d - m_up) <= thr) | (np.abs(d - m_dn) <= thr)
    out = f.copy()
    for idx in zip(*np.nonzero(risky)):
        exact = _sigmoid_decimal(float(x[idx]))
        if exact > Decimal(float(m_up[idx])):
            out[idx] = up[idx]
        elif exact < Decimal(float(m_dn[idx])):
            out[idx] = dn[idx]
        else:
            out[idx] = f[idx]
    return out


def sigmoid_rn32_fallback_count(x: np.ndarray) -> int:
    """How many elements of x need the decimal re-evaluation (diagnostic)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    xd = x.astype(np.float64)
    with np.errstate(over="ignore"):
        d = 1.0 / (1.0 + np.exp(-xd))
    f = d.astype(np.float32)
    fd = f.astype(np.float64)
    m_up = (fd + np.nextafter(f, np.float32(np.inf)).astype(np.float64)) * 0.5
    m_dn = (fd + np.nextafter(f, np.float32(-np.inf)).astype(np.float64)) * 0.5
    thr = ZIV_REL * d
    return int(np.count_nonzero((np.abs(d - m_up) <= thr) | (np.abs(d - m_dn) <= thr)))


# ----------------------------------------------------------------------------
# a2: correction bias
# ----------------------------------------------------------------------------


def biased_scores(s: np.ndarray, bias: np.ndarray) -> np.ndarray:
    """sp[t, e] = fl32(s[t, e] + bias[e]); selection only, never the weight."""
    return (s.astype(np.float32) + bias.astype(np.float32)[None, :]).astype(np.float32)


# ----------------------------------------------------------------------------
# a3-a5: grouped top-k of one token
# ----------------------------------------------------------------------------


def group_scores(sp_row: np.ndarray, n_groups: int, group_topn: int) -> np.ndarray:
    """Per group of E/n_groups consecutive experts: fl32 sum of its top
    `group_topn` biased scores (with multiplicity), added largest first."""
    eg = sp_row.shape[0] // n_groups
    out = np.empty(n_groups, dtype=np.float32)
    for g in range(n_groups):
        vals = np.sort(sp_row[g * eg:(g + 1) * eg])[::-1][:group_topn]
        acc = np.float32(vals[0])
        for v in vals[1:]:
            acc = np.float32(acc + np.float32(v))
        out[g] = acc
    return out


def kept_groups(gs: np.ndarray, topk_group: int) -> list:
    """The `topk_group` groups with the largest score; ties to the lower index."""
    order = sorted(range(gs.shape[0]), key=lambda g: (-float(gs[g]), g))
    return sorted(order[:topk_group])


def topk_experts(sp_row: np.ndarray, groups: list, n_groups: int, top_k: int) -> list:
    """Top `top_k` experts of the kept groups by (sp desc, id asc), in order."""
    eg = sp_row.shape[0] // n_groups
    cand = [e for g in groups for e in range(g * eg, (g + 1) * eg)]
    cand.sort(key=lambda e: (-float(sp_row[e]), e))
    return cand[:top_k]


# ----------------------------------------------------------------------------
# a6: renormalised weights
# ----------------------------------------------------------------------------


def renormalised_weights(s_sel: np.ndarray) -> np.ndarray:
    """w_k = s_k / sum_j s_j in binary64 (exact sum), rounded to binary32."""
    vals = [float(v) for v in s_sel]
    total = math.fsum(vals)
    assert total > 0.0, "sum of selected sigmoid scores must be positive"
    return np.array([v / total for v in vals], dtype=np.float64).astype(np.float32)


# ----------------------------------------------------------------------------
# a7: rank-local relabel and packing
# ----------------------------------------------------------------------------


def local_num_experts(num_experts: int, top_k: int, local_expert_offset: int,
                      num_local_experts: int) -> int:
    """Local id space size round_up(count + top_k, 4) when the rank range is a
    proper sub-range that shrinks the routing problem, else 0 (global ids).

    Raises ValueError for a range outside [0, num_experts)."""
    off, cnt = local_expert_offset, num_local_experts
    if off < 0 or cnt < 0 or off + cnt > num_experts:
        raise ValueError("expert range outside [0, num_experts)")
    if cnt == 0 or cnt >= num_experts:
        return 0
    e_out = ((cnt + top_k + 3) // 4) * 4
    return e_out if e_out < num_experts else 0


def relabel(ids: np.ndarray, local_expert_offset: int, num_local_experts: int,
            applies: bool) -> np.ndarray:
    """id' = id - off for the rank's experts, count + k for any other expert
    in slot k; global ids unchanged when the range does not apply."""
    if not applies:
        return ids.copy()
    off, cnt = local_expert_offset, num_local_experts
    out = np.empty_like(ids)
    T, K = ids.shape
    for t in range(T):
        for k in range(K):
            e = int(ids[t, k])
            out[t, k] = e - off if off <= e < off + cnt else cnt + k
    return out


def bf16_rne_bits(w: np.ndarray) -> np.ndarray:
    """bf16 bit pattern of binary32 w, round to nearest, ties to even
    (finite inputs)."""
    u = np.ascontiguousarray(w, dtype=np.float32).view(np.uint32).astype(np.uint64)
    h = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return (h & np.uint64(0xFFFF)).astype(np.uint32)


def pack(ids_out: np.ndarray, w: np.ndarray) -> np.ndarray:
    """packed = (id' << 16) | bf16_bits(w) as int32."""
    h = bf16_rne_bits(w)
    return ((ids_out.astype(np.int64) << 16) | h.astype(np.int64)).astype(np.int32)


# ----------------------------------------------------------------------------
# a8-a10: counts, offsets, expert-major permutation
# ----------------------------------------------------------------------------


def expert_counts(ids_out: np.ndarray, e_out: int) -> np.ndarray:
    counts = np.zeros(e_out, dtype=np.int64)
    for v in ids_out.ravel():
        counts[int(v)] += 1
    return counts.astype(np.int32)


def exclusive_offsets(counts: np.ndarray) -> np.ndarray:
    offs = np.zeros(counts.shape[0] + 1, dtype=np.int64)
    acc = 0
    for i, c in enumerate(counts):
        offs[i] = acc
        acc += int(c)
    offs[-1] = acc
    return offs.astype(np.int32)


def expert_major_permutation(ids_out: np.ndarray, e_out: int) -> Tuple[np.ndarray, np.ndarray]:
    """perm[p] = flat index f = t*K + k of the p-th entry in expert-major
    order, ascending f within each expert; inv[perm[p]] = p."""
    flat = ids_out.ravel()
    buckets = [[] for _ in range(e_out)]
    for f, v in enumerate(flat):
        buckets[int(v)].append(f)
    perm = np.array([f for b in buckets for f in b], dtype=np.int32)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.shape[0], dtype=np.int32)
    return perm, inv


# ----------------------------------------------------------------------------
# Grouped-GEMM layout (the next consumer of counts and perm)
# ----------------------------------------------------------------------------
# The pages say only that an expert-parallel backend builds the per-row
# expert index array of a grouped GEMM from the routing ("Add MoonEP
# expert-parallel arm of the Kimi-K3 B300 agentic sweep", the review summary
# of the patch: its prepare/finalize step). The plainest reading
# of such a layout, taken here: the entries of output id e occupy rows
# padded_offsets[e] .. padded_offsets[e] + counts[e] - 1 in permutation
# order, then padding rows up to padded_offsets[e+1] = padded_offsets[e] +
# round_up(counts[e], tile_m); each row's expert index is e, or -1 on a
# padding row; each row's entry is the flat index f = t*K + k it holds, or -1.
# Rows past padded_offsets[E'] (up to the caller's row count) are -1.


def grouped_layout_rows(n_entries: int, e_out: int, tile_m: int) -> int:
    """Upper bound on the padded row count: every id wastes < tile_m rows."""
    return n_entries + e_out * (tile_m - 1)


def grouped_layout(counts: np.ndarray, perm: np.ndarray, tile_m: int,
                   rows: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    counts = [int(c) for c in counts]
    e_out = len(counts)
    padded = np.zeros(e_out + 1, dtype=np.int64)
    for e in range(e_out):
        padded[e + 1] = padded[e] + -(-counts[e] // tile_m) * tile_m
    m_indices = np.full(rows, -1, dtype=np.int64)
    row_entry = np.full(rows, -1, dtype=np.int64)
    p = 0  # position in perm: entries of id e are perm[p .. p + counts[e])
    for e in range(e_out):
        for j in range(counts[e]):
            r = int(padded[e]) + j
            m_indices[r] = e
            row_entry[r] = int(perm[p + j])
        p += counts[e]
    return padded.astype(np.int32), m_indices.astype(np.int32), row_entry.astype(np.int32)


# ----------------------------------------------------------------------------
# Static per-rank balancing plan
# ----------------------------------------------------------------------------
# The pages give only the goal: the expert-parallel dispatch holds every
# rank at exactly S*K routed entries by reassigning the surplus of
# overloaded expert owners ("Add MoonEP expert-parallel arm of the Kimi-K3
# B300 agentic sweep", PR description: what MoonEP does). The plan taken
# here, over the expert-major order of one routing call with global ids
# (experts owned in contiguous ranges of E / N by ranks 0..N-1):
#   target[r] = n // N (+1 for the first n % N ranks), n = T*K entries;
#   rank r keeps the first min(load[r], target[r]) of its own entries;
#   the rest of every overloaded rank, in rank order, is the surplus
#   sequence; the ranks short of their target take consecutive runs of it,
#   in rank order, until each holds exactly its target.
# No plan can move fewer entries (every overloaded rank must lose its
# excess), and the order inside each expert is kept.


def balance_plan(counts: np.ndarray, n_ranks: int) -> Tuple[np.ndarray, np.ndarray]:
    """dest[p]: rank of the p-th entry in expert-major order; rank_counts
    [n_ranks, E]: entries of expert e each rank processes."""
    counts = [int(c) for c in counts]
    E = len(counts)
    per = E // n_ranks
    n = sum(counts)
    target = [n // n_ranks + (1 if r < n % n_ranks else 0) for r in range(n_ranks)]
    load = [sum(counts[r * per:(r + 1) * per]) for r in range(n_ranks)]
    keep = [min(load[r], target[r]) for r in range(n_ranks)]
    deficit = [target[r] - keep[r] for r in range(n_ranks)]
    # ranks short of their target, one slot per missing entry, in rank order
    takers = [r for r in range(n_ranks) for _ in range(deficit[r])]
    dest = np.zeros(n, dtype=np.int64)
    rank_counts = np.zeros((n_ranks, E), dtype=np.int64)
    p = 0            # position in expert-major order
    moved = 0        # entries of the surplus sequence assigned so far
    for r in range(n_ranks):
        own = 0      # entries of rank r seen so far
        for e in range(r * per, (r + 1) * per):
            for _ in range(counts[e]):
                if own < keep[r]:
                    d = r
                else:
                    d = takers[moved]
                    moved += 1
                dest[p] = d
                rank_counts[d, e] += 1
                own += 1
                p += 1
    return dest.astype(np.int32), rank_counts.astype(np.int32)


# ----------------------------------------------------------------------------
# Activation quantisation of the fused route + quant launch (MXFP8)
# ----------------------------------------------------------------------------
# The pages name a fused route + quant launch for decode batches of up to 64
# tokens whose routed MoE runs MXFP4 expert weights ("[kimi-k3] Rank-local
# expert ids for the EP routed MoE (upstream #45544)", commit message), but
# not the activation format. Reading taken: OCP MXFP8 with E4M3 elements,
# one E8M0 scale per 32 consecutive elements of a token's hidden row:
#   shared = floor(log2(amax)) - 8   (8 = the largest E4M3 exponent),
#            at least -127; a block of zeros gets shared = -127;
#   scale code = shared + 127 (E8M0: the scale is 2^shared);
#   element = E4M3 code of v / 2^shared, rounded to nearest (ties to even)
#             and saturated at +-448 (E4M3 without infinities, max 448).

MX_BLOCK = 32
E4M3_MAX = 448.0


def e4m3_code(q: float) -> int:
    """OCP E4M3 code of the real q: round to nearest, ties to even, saturate
    at +-448; the sign of zero is kept."""
    neg = math.copysign(1.0, q) < 0
    a = abs(q)
    if a >= E4M3_MAX:
        code = 0x7E
    else:
        # quantum of a's binade (exponent at least -6: the subnormal step is 2^-9)
        e = max(math.frexp(a)[1] - 1, -6) if a > 0 else -6
        quantum = 2.0 ** (e - 3)
        k = a / quantum                    # exact: a is a binary64 multiple of 2^-200
        n = math.floor(k)
        frac = k - n
        if frac > 0.5 or (frac == 0.5 and n % 2 == 1):
            n += 1
        r = n * quantum                    # the rounded magnitude, <= 448
        if r == 0:
            code = 0
        elif r < 2.0 ** -6:                # subnormal: mantissa = r / 2^-9
            code = int(round(r / 2.0 ** -9))
        else:
            ee = math.frexp(r)[1] - 1      # binade of the rounded value
            mant = int(round((r / 2.0 ** ee - 1.0) * 8))
            code = ((ee + 7) << 3) | mant
    return code | (0x80 if neg else 0)


def e4m3_value(code: int) -> float:
    """Real value of an E4M3 code (0x7F / 0xFF, the NaN codes, excluded)."""
    sign = -1.0 if code & 0x80 else 1.0
    ef, mf = (code >> 3) & 0xF, code & 7
    if ef == 0:
        return sign * mf * 2.0 ** -9
    return sign * (1.0 + mf / 8.0) * 2.0 ** (ef - 7)


def mxfp8_quantize(hidden_bits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """bf16 hidden [T, H] (bit patterns, H a multiple of 32) -> E4M3 codes
    uint8 [T, H] and E8M0 scale codes uint8 [T, H / 32]."""
    v = bf16_bits_to_f64(hidden_bits)
    T, H = v.shape
    codes = np.zeros((T, H), dtype=np.uint8)
    scales = np.zeros((T, H // MX_BLOCK), dtype=np.uint8)
    for t in range(T):
        for b in range(H // MX_BLOCK):
            blk = v[t, b * MX_BLOCK:(b + 1) * MX_BLOCK]
            amax = float(np.max(np.abs(blk)))
            shared = max(math.frexp(amax)[1] - 1 - 8, -127) if amax > 0 else -127
            scales[t, b] = shared + 127
            for i, x in enumerate(blk):
                codes[t, b * MX_BLOCK + i] = e4m3_code(math.ldexp(float(x), -shared))
    return codes, scales


# ----------------------------------------------------------------------------
# The whole step
# ----------------------------------------------------------------------------


def route_tokens(logits: np.ndarray, bias: np.ndarray, n_groups: int = 8,
                 topk_group: int = 4, top_k: int = 16, group_topn: int = 2):
    """a1-a6 for every row: (global ids int32 [T,K], s of those ids, weights)."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    if E % n_groups != 0:
        raise ValueError("num_experts must be a multiple of n_groups")
    s = sigmoid_rn32(logits)
    sp = biased_scores(s, bias)
    ids = np.zeros((T, top_k), dtype=np.int32)
    s_sel = np.zeros((T, top_k), dtype=np.float32)
    w = np.zeros((T, top_k), dtype=np.float32)
    for t in range(T):
        gs = group_scores(sp[t], n_groups, group_topn)
        groups = kept_groups(gs, topk_group)
        sel = topk_experts(sp[t], groups, n_groups, top_k)
        ids[t] = sel
        s_sel[t] = s[t, sel]
        w[t] = renormalised_weights(s_sel[t])
    return ids, s_sel, w


def route_ref(logits: np.ndarray, bias: np.ndarray, n_groups: int = 8,
              topk_group: int = 4, top_k: int = 16, group_topn: int = 2,
              local_expert_offset: int = 0, num_local_experts: int = 0) -> Dict[str, np.ndarray]:
    """The full routing step; returns every output the library writes."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    e_local = local_num_experts(E, top_k, local_expert_offset, num_local_experts)
    applies = e_local > 0
    e_out = e_local if applies else E
    ids, _, w = route_tokens(logits, bias, n_groups, topk_group, top_k, group_topn)
    ids_out = relabel(ids, local_expert_offset, num_local_experts, applies)
    packed = pack(ids_out, w)
    counts = expert_counts(ids_out, e_out)
    offsets = exclusive_offsets(counts)
    perm, inv = expert_major_permutation(ids_out, e_out)
    return {"topk_ids": ids, "topk_weights": w, "packed": packed, "ids_out": ids_out,
            "counts": counts, "offsets": offsets, "perm": perm, "inv_perm": inv,
            "num_experts_out": np.int32(e_out)}


# ----------------------------------------------------------------------------
# a0: router GEMM (logits = hidden . W^T), bf16 operands
# ----------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (the high half of a binary32)."""
    u = (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16))
    return u.view(np.float32).astype(np.float64)


def router_logits_ref(hidden_bits: np.ndarray, weight_bits: np.ndarray) -> np.ndarray:
    """logits[t, e] = sum_h hidden[t, h] * W[e, h] in binary64 (bf16 inputs)."""
    return bf16_bits_to_f64(hidden_bits) @ bf16_bits_to_f64(weight_bits).T


def router_logits_bound(hidden_bits: np.ndarray, weight_bits: np.ndarray) -> np.ndarray:
    """Error bound of any binary32 accumulation order of the exact bf16
    products, plus the final rounding: gamma_{H}(2^-24) * sum |a||b| + u|ref|."""
    a = np.abs(bf16_bits_to_f64(hidden_bits))
    b = np.abs(bf16_bits_to_f64(weight_bits))
    n = a.shape[1]
    u = 2.0 ** -24
    gamma = n * u / (1.0 - n * u)
    ref = np.abs(router_logits_ref(hidden_bits, weight_bits))
    return gamma * (a @ b.T) + u * ref
