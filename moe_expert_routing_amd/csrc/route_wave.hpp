// route_wave.hpp - one wavefront routes one token (gfx950, wave64).
//
// The method (a sigmoid router with a correction bias and a grouped top-k:
// "[ROCm][Perf] Kimi-K3: token-sharded residual stream for long prefills",
// author's reply on shard-routed test coverage; packed ids and the
// rank-local pack epilogue: "[kimi-k3] Rank-local expert ids for the EP
// routed MoE (upstream #45544)", commit message):
//   s  = RN32(sigma(logit))                 exact binary32 (rn_sigmoid.hpp)
//   sp = fl32(s + bias)                      selection key only
//   group score = fl32 sum of the group's top `group_topn` sp
//   keep the topk_group best groups          ties -> lower group index
//   top_k experts of the kept groups         by (sp desc, id asc)
//   w_k = s_k / sum_j s_j                    binary64, rounded to binary32
//   packed = (id' << 16) | bf16_rne(w)       id' = rank-local id if relabelled
//
// How the selection is made exact and fast (select_token):
//  1. Every score is approximated with the hardware exp2/rcp (error <=
//     FAST_SIG_ERR, checked over all binary32 inputs by a GPU test) and
//     turned into a 32-bit key (value bits with the slot in the low 4 bits).
//  2. The group choice is accepted only when the score margin between the
//     kept and the dropped groups exceeds the error bound.
//  3. A threshold, found by bisection on the kept lanes' top-5 keys, picks
//     a candidate set (<= 64) holding every possible winner; the candidates
//     are scored again (same approximation) and ranked by (sp~, id).
//  4. The result is accepted only when the top_k-th score beats the largest
//     score any non-candidate can have and adjacent ranks are apart by more
//     than the error (or are exact twins). Otherwise the candidates are
//     scored EXACTLY and ranked by exact (sp, id), and the result is accepted
//     when the exact top_k-th score beats that bound.
//  5. Weights: from the winners' approximate scores when their tested error
//     bound keeps every weight within 0.9e-6 of the exact one, otherwise from
//     the winners' exact scores.
// A token that fails a check runs the same pipeline on exact scores (only
// the key truncation is left to bound), and if that cannot decide either
// (near-ties within 16 ulp at the threshold), route_token_exact: exact
// scores, exact group scores, top_k by wave argmax.
//
// Lane layout. Lane l belongs to group g = l / LPG (LPG = 64 / G lanes per
// group) and holds 2*NP experts of that group as NP float2 pairs:
//   e(i, j) = g*Eg + 2*(l % LPG) + 2*LPG*i + j,   i < NP, j < 2,
// so every load instruction of the wave reads 8-byte pieces that tile whole
// 64-byte segments, and group reductions stay inside LPG adjacent lanes.
// Slot q = 2i + j: within a lane, expert ids increase with the slot.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rn_sigmoid.hpp"

namespace moe {

constexpr int kMaxTopK = 32;

struct RouteParams {
  int E;          // experts
  int G;          // groups
  int TG;         // groups kept
  int K;          // top_k
  int topn;       // group score terms (1 or 2)
  int lpg;        // lanes per group, 64 / G
  int lpg_log2;
  int eg;         // experts per group
  int off, cnt;   // rank range
  int local;      // 1 when the rank-local relabel applies
  int e_out;      // output id space
};

// Tokens that took the exact path (diagnostic, moe_route_exact_path_tokens).
__device__ unsigned long long g_exact_path_tokens = 0ull;
// Tokens of the fast path whose candidates were scored again exactly.
__device__ unsigned long long g_rescored_tokens = 0ull;

// Lanes per group: a compile-time constant (LPG > 0) or the runtime value
// (LPG = 0). The common shapes get constant loops and lane indices.
template <int LPG>
__device__ __forceinline__ int lpg_of(const RouteParams &p) { return LPG ? LPG : p.lpg; }
template <int LPG>
__device__ __forceinline__ int lpg_log2_of(const RouteParams &p) {
  return LPG ? (LPG == 1 ? 0 : LPG == 2 ? 1 : LPG == 4 ? 2 : LPG == 8 ? 3 : LPG == 16 ? 4 : LPG == 32 ? 5 : 6)
             : p.lpg_log2;
}
template <int LPG>
__device__ __forceinline__ int groups_of(const RouteParams &p) { return LPG ? 64 / LPG : p.G; }

// Per-wave LDS scratch of the fast path.
struct WaveScratch {
  uint32_t cand[64];              // candidate expert ids
  unsigned long long key[64];     // candidate keys (score, id)
  uint4 res[kMaxTopK + 1];        // by rank: (id, logit bits, bias bits, score bits)
};

// ---------------------------------------------------------------------------
// Cross-lane helpers (gfx9 DPP controls)
// ---------------------------------------------------------------------------
constexpr int DPP_XOR1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141; // lane i <-> 7-i within 8
constexpr int DPP_MIRROR = 0x140;      // lane i <-> 15-i within 16

// No old value is needed (full masks, bound_ctrl set): the permutations read
// an in-range lane, and a row shift (row_shr) reads zero where no lane lies
// that far down in the row.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = dpp<CTRL>((uint32_t)u), hi = dpp<CTRL>((uint32_t)(u >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t umin(uint32_t a, uint32_t b) { return a < b ? a : b; }
__device__ __forceinline__ uint32_t umed3(uint32_t a, uint32_t b, uint32_t c) {
  return umax(umin(a, b), umin(umax(a, b), c));
}

__device__ __forceinline__ uint32_t readlane_u32(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

// Maximum / minimum over the 64 lanes (wave-uniform result).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = umax(v, dpp<DPP_XOR1>(v));
  v = umax(v, dpp<DPP_XOR2>(v));
  v = umax(v, dpp<DPP_HALF_MIRROR>(v));
  v = umax(v, dpp<DPP_MIRROR>(v));
  return umax(umax(readlane_u32(v, 0), readlane_u32(v, 16)),
              umax(readlane_u32(v, 32), readlane_u32(v, 48)));
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = umin(v, dpp<DPP_XOR1>(v));
  v = umin(v, dpp<DPP_XOR2>(v));
  v = umin(v, dpp<DPP_HALF_MIRROR>(v));
  v = umin(v, dpp<DPP_MIRROR>(v));
  return umin(umin(readlane_u32(v, 0), readlane_u32(v, 16)),
              umin(readlane_u32(v, 32), readlane_u32(v, 48)));
}

// Merge the top-2 (with multiplicity) of two disjoint sets.
__device__ __forceinline__ void top2_merge(uint32_t &a1, uint32_t &a2, uint32_t b1, uint32_t b2) {
  const uint32_t n2 = umax(umin(a1, b1), umax(a2, b2));
  a1 = umax(a1, b1);
  a2 = n2;
}

// Top-2 over each aligned run of `lpg` lanes (all lanes of the run get it).
__device__ __forceinline__ void group_top2(uint32_t &m1, uint32_t &m2, int lpg) {
  if (lpg >= 2) top2_merge(m1, m2, dpp<DPP_XOR1>(m1), dpp<DPP_XOR1>(m2));
  if (lpg >= 4) top2_merge(m1, m2, dpp<DPP_XOR2>(m1), dpp<DPP_XOR2>(m2));
  if (lpg >= 8) top2_merge(m1, m2, dpp<DPP_HALF_MIRROR>(m1), dpp<DPP_HALF_MIRROR>(m2));
  if (lpg >= 16) top2_merge(m1, m2, dpp<DPP_MIRROR>(m1), dpp<DPP_MIRROR>(m2));
  if (lpg >= 32) top2_merge(m1, m2, __shfl_xor(m1, 16), __shfl_xor(m2, 16));
  if (lpg >= 64) top2_merge(m1, m2, __shfl_xor(m1, 32), __shfl_xor(m2, 32));
}

__device__ __forceinline__ int mbcnt(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// LDS written by some lanes of the wave is read by others: LDS instructions
// of one wavefront execute in order; keep the compiler from reordering.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Monotone map of finite binary32 values to unsigned integers.
__device__ __forceinline__ uint32_t ord_f32(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t bf16_rne_bits(float w) {
  const uint32_t u = __float_as_uint(w);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// ---------------------------------------------------------------------------
// Approximate scores
// ---------------------------------------------------------------------------
// Bound on |fast_sigmoid(x) - RN32(sigma(x))| over all finite binary32 x.
constexpr float FAST_SIG_ERR = 0x1p-22f;
// The bound the exhaustive GPU test of fast_sigmoid asserts over every finite
// binary32 input: |fast_sigmoid(x) - RN32(sigma(x))| <= FAST_SIG_ERR / 2. It
// bounds the unbiased scores the row path derives from its keys for the
// weights (selection certificates keep the factor-two margin).
constexpr float FAST_SIG_ERR_TESTED = 0.5f * FAST_SIG_ERR;

// Unit in the last place of a positive normal binary32 value.
__device__ __forceinline__ float ulp32(float v) {
  return __uint_as_float((__float_as_uint(v) & 0x7F800000u) - (23u << 23));
}

__device__ __forceinline__ float fast_sigmoid(float x) {
  const float e = __builtin_amdgcn_exp2f(x * -1.44269504088896340736f);
  return __builtin_amdgcn_rcpf(1.0f + e);
}

// Approximate key: the bits of max(sp~, 0) with the low 4 bits replaced by
// (15 - slot). Keys order by value (to 16 ulp), then by lower expert id
// within a lane. key_value() gives the value part.
__device__ __forceinline__ uint32_t approx_key(float sp, int slot) {
  const int b = __float_as_int(sp);
  return ((uint32_t)(b > 0 ? b : 0) & 0xFFFFFFF0u) | (uint32_t)(15 - slot);
}
__device__ __forceinline__ float key_value(uint32_t k) { return __uint_as_float(k & 0xFFFFFFF0u); }

// |key_value(key_e) - sp_e| <= err_bound(key_value(key_e)) for every expert
// whose key is not clamped: the approximation error, two binary32 roundings
// (of s~ + b and of s + b) and the 15-ulp truncation, with margin.
__device__ __forceinline__ float err_bound(float v) { return 1.01f * FAST_SIG_ERR + 0x1p-18f * v; }
// Same for a group score v = fl32(v1 + v2): per term the truncation
// (< 15/16 * 2^-19 * v_i) and the two roundings (2^-23 * v_i), plus the
// roundings of the approximate and the exact sum (2^-23 * v), stay below
// 2 * FAST_SIG_ERR + 17/16 * 2^-19 * v; 2^-18 * v leaves a margin.
__device__ __forceinline__ float group_err_bound(float v) {
  return 2.02f * FAST_SIG_ERR + 0x1p-18f * v;
}

template <int NP, int LPG>
__device__ __forceinline__ void load_lane_layout(const float *__restrict__ v, const RouteParams &p,
                                                 int lane, float (&out)[2 * NP]) {
  const int lpg = lpg_of<LPG>(p);
  const int g = lane >> lpg_log2_of<LPG>(p);
  const int sub = lane & (lpg - 1);
  const float *base = v + g * (LPG ? 2 * NP * LPG : p.eg) + 2 * sub;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const float2 q = *reinterpret_cast<const float2 *>(base + 2 * lpg * i);
    out[2 * i] = q.x;
    out[2 * i + 1] = q.y;
  }
}

__device__ __forceinline__ int slot_expert(int e0, int lpg, int q) {
  return e0 + 2 * lpg * (q >> 1) + (q & 1);
}

// ---------------------------------------------------------------------------
// Candidate pipeline
// ---------------------------------------------------------------------------
// Descending compare-exchange (wave-uniform operands run on the scalar unit).
__device__ __forceinline__ void ce_desc(uint32_t &a, uint32_t &b) {
  const uint32_t hi = umax(a, b), lo = umin(a, b);
  a = hi;
  b = lo;
}

// Sorts 8 values in descending order (19 comparators, depth 6).
__device__ __forceinline__ void sort8_desc(uint32_t (&v)[8]) {
  ce_desc(v[0], v[2]); ce_desc(v[1], v[3]); ce_desc(v[4], v[6]); ce_desc(v[5], v[7]);
  ce_desc(v[0], v[4]); ce_desc(v[1], v[5]); ce_desc(v[2], v[6]); ce_desc(v[3], v[7]);
  ce_desc(v[0], v[1]); ce_desc(v[2], v[3]); ce_desc(v[4], v[5]); ce_desc(v[6], v[7]);
  ce_desc(v[2], v[4]); ce_desc(v[3], v[5]);
  ce_desc(v[1], v[4]); ce_desc(v[3], v[6]);
  ce_desc(v[1], v[2]); ce_desc(v[3], v[4]); ce_desc(v[5], v[6]);
}

// |sp~ - sp| for an approximate score of magnitude v: the approximation
// error plus two binary32 roundings (of s~ + b and of s + b), with margin.
__device__ __forceinline__ float score_err(float v) {
  return 1.01f * FAST_SIG_ERR + 0x1p-22f * fabsf(v);
}

// Exact group choice for a token whose approximate group scores leave the
// kept/dropped boundary within the error. A group's exact top-`topn` scores
// are among its experts whose approximate key value reaches
// thr = (approximate topn-th value) - 2 * err_bound(approximate top value):
// every expert below thr scores, exactly, below the exact scores of the
// group's approximate top-topn. Each lane holds its 5 best keys; when its
// 5th reaches thr the pool may not hold every such expert and the function
// returns false. Otherwise those pool entries (at most 4 per lane; logits
// and biases read again, from cache) are scored exactly, each group's exact score is the fl32 sum of its exact top
// `topn`, and kept = the TG best groups (ties -> lower group index).
__device__ __forceinline__ bool exact_group_choice(const float *__restrict__ row,
                                                   const float *__restrict__ bias_g, uint32_t p1,
                                                   uint32_t p2, uint32_t p3, uint32_t p4,
                                                   uint32_t p5, uint32_t g1, uint32_t g2,
                                                   const RouteParams &p, int lane, int e0, int lpg,
                                                   int lpg_log2, int G, bool &kept) {
  const float thr = key_value(p.topn == 2 ? g2 : g1) - 2.0f * err_bound(key_value(g1));
  if (__ballot(key_value(p5) >= thr)) return false;
  const uint32_t pool[4] = {p1, p2, p3, p4};
  uint32_t e1 = 0u, e2 = 0u;  // the lane's exact top-2 (ord_f32; 0 = none)
#pragma unroll
  for (int i = 0; i < 4; i += 2) {
    const bool u0 = key_value(pool[i]) >= thr, u1 = key_value(pool[i + 1]) >= thr;
    if (!__ballot(u0 || u1)) break;  // pools are sorted: later entries are lower
    // thr > 0 here, so a selected entry is a filled pool entry: valid slot
    const int d0 = slot_expert(e0, lpg, 15 - (int)(pool[i] & 15u));
    const int d1 = slot_expert(e0, lpg, 15 - (int)(pool[i + 1] & 15u));
    const float x0 = u0 ? row[d0] : 0.0f, b0 = u0 ? bias_g[d0] : 0.0f;
    const float x1 = u1 ? row[d1] : 0.0f, b1 = u1 ? bias_g[d1] : 0.0f;
    const float s0 = sigmoid_rn32(x0), s1 = sigmoid_rn32(x1);
    const uint32_t k0 = u0 ? ord_f32(s0 + b0) : 0u;
    const uint32_t k1 = u1 ? ord_f32(s1 + b1) : 0u;
    top2_merge(e1, e2, umax(k0, k1), umin(k0, k1));
  }
  group_top2(e1, e2, lpg);
  auto val = [](uint32_t k) {  // inverse of ord_f32 (k != 0)
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
  };
  const float gs = (p.topn == 2) ? val(e1) + val(e2) : val(e1);
  const int g = lane >> lpg_log2;
  int rank = 0;
  for (int gg = 0; gg < G; ++gg) {
    const float o = __uint_as_float(readlane_u32(__float_as_uint(gs), gg << lpg_log2));
    rank += ((o > gs) || (o == gs && gg < g)) ? 1 : 0;
  }
  kept = rank < p.TG;
  return true;
}

// Ranks the m candidates (lanes 0..m-1 hold expert eid, logit cx, bias cb
// and score sc) by (score desc, id asc) and stores ranks 0..K in L->res.
__device__ __forceinline__ void rank_candidates(WaveScratch *L, int lane, int m, int K,
                                                uint32_t eid, float cx, float cb, float sc) {
  const bool is_cand = lane < m;
  const uint64_t ck = ((uint64_t)ord_f32(sc) << 32) | (uint64_t)(~eid);
  if (is_cand) L->key[lane] = ck;
  // pad to a multiple of 4, and up to 32 (zero keys rank below every candidate)
  if (lane >= m && lane < max((m + 3) & ~3, 32)) L->key[lane] = 0ull;
  wave_lds_sync();
  int r = 0;
  if (m <= 32) {
    // the usual case: all 32 keys read at once (one LDS round trip)
    uint64_t kk[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) kk[j] = L->key[j];
#pragma unroll
    for (int j = 0; j < 32; ++j) r += kk[j] > ck ? 1 : 0;
  } else if (is_cand) {
    for (int j = 0; j < m; j += 4) {
      const uint64_t k0 = L->key[j], k1 = L->key[j + 1], k2 = L->key[j + 2], k3 = L->key[j + 3];
      r += (k0 > ck ? 1 : 0) + (k1 > ck ? 1 : 0) + (k2 > ck ? 1 : 0) + (k3 > ck ? 1 : 0);
    }
  }
  if (is_cand && r <= K)
    L->res[r] = make_uint4(eid, __float_as_uint(cx), __float_as_uint(cb), __float_as_uint(sc));
  wave_lds_sync();
}

// Selects the top_k experts of one token. The scores that pick the groups
// and the candidates are the fast approximations (EXACT = false) or the
// exact scores (EXACT = true). Returns true, with (id, exact s) of slot
// k = lane in lanes 0..K-1, only when the result is proven equal to the
// exact selection.
template <int NP, int LPG, bool EXACT>
__device__ __forceinline__ bool select_token(const float *__restrict__ row,
                                             const float *__restrict__ bias_g,
                                             const float (&x)[2 * NP], const float (&bias)[2 * NP],
                                             const RouteParams &p, int lane, WaveScratch *L,
                                             int &my_id, float &my_s) {
  constexpr int M = 2 * NP;
  const int lpg = lpg_of<LPG>(p), lpg_log2 = lpg_log2_of<LPG>(p), G = groups_of<LPG>(p);
  const int g = lane >> lpg_log2;
  const int e0 = g * (LPG ? M * LPG : p.eg) + 2 * (lane & (lpg - 1));

  bool rescored = false;  // some scores were recomputed exactly (fast path)

  // ---- streaming: scores -> keys -> the lane's top-5 keys ------------------
  uint32_t p1 = 0u, p2 = 0u, p3 = 0u, p4 = 0u, p5 = 0u;
  float x1 = -__builtin_inff(), x2 = -__builtin_inff();  // exact top-2 (EXACT)
#pragma unroll
  for (int q = 0; q < M; ++q) {
    float sc;
    if (EXACT) {
      sc = sigmoid_rn32(x[q]) + bias[q];
      x2 = fmaxf(x2, fminf(x1, sc));
      x1 = fmaxf(x1, sc);
      __builtin_amdgcn_sched_barrier(0);
    } else {
      sc = fast_sigmoid(x[q]) + bias[q];
    }
    const uint32_t k = approx_key(sc, q);
    p5 = umed3(p4, p5, k);
    p4 = umed3(p3, p4, k);
    p3 = umed3(p2, p3, k);
    p2 = umed3(p1, p2, k);
    p1 = umax(p1, k);
  }

  // ---- groups ---------------------------------------------------------------
  bool kept;
  uint32_t hi_key;  // one above the largest kept key
  if (!EXACT && G <= 8) {
    uint32_t g1 = p1, g2 = p2;
    group_top2(g1, g2, lpg);
    const uint32_t glast = (p.topn == 2) ? g2 : g1;
    const float gs = (p.topn == 2) ? key_value(g1) + key_value(g2) : key_value(g1);  // >= 0
    // every group's score and top key, on the scalar unit
    uint32_t sv[8], top[8];
#pragma unroll
    for (int gg = 0; gg < 8; ++gg) {
      const int src = (gg < G ? gg : 0) << lpg_log2;
      sv[gg] = gg < G ? readlane_u32(__float_as_uint(gs), src) : 0u;
      top[gg] = readlane_u32(g1, src);
    }
    uint32_t srt[8];
#pragma unroll
    for (int gg = 0; gg < 8; ++gg) srt[gg] = sv[gg];
    sort8_desc(srt);
    uint32_t keep_thr = srt[0], drop_max = 0u;
#pragma unroll
    for (int i = 1; i < 8; ++i) {
      if (i == p.TG - 1) keep_thr = srt[i];
      if (i == p.TG) drop_max = srt[i];
    }
    bool near_tie = false;
    if (p.TG < G) {
      const float kmin = __uint_as_float(keep_thr), dmax = __uint_as_float(drop_max);
      near_tie = !(kmin - group_err_bound(kmin) > dmax + group_err_bound(dmax));
    }
    if (!near_tie) {
      hi_key = 0u;
#pragma unroll
      for (int gg = 0; gg < 8; ++gg)
        if (gg < G && sv[gg] >= keep_thr) hi_key = umax(hi_key, top[gg]);
      hi_key += 1u;
      kept = __float_as_uint(gs) >= keep_thr;
    } else {
      // Kept and dropped groups within the error: exact group scores.
      if (!exact_group_choice(row, bias_g, p1, p2, p3, p4, p5, g1, g2, p, lane, e0, lpg, lpg_log2,
                              G, kept))
        return false;
      rescored = true;
      hi_key = wave_max_u32(kept ? p1 : 0u) + 1u;
    }
    // the kept groups' scores must rest on unclamped (positive) values
    if (__ballot(kept && (glast & 0xFFFFFFF0u) == 0u)) return false;
  } else {
    // exact group scores (EXACT), or approximate ones with many groups
    float m1 = EXACT ? x1 : key_value(p1), m2 = EXACT ? x2 : key_value(p2);
    for (int d = 1; d < lpg; d <<= 1) {
      const float o1 = __shfl_xor(m1, d);
      const float o2 = __shfl_xor(m2, d);
      const float n2 = fmaxf(fminf(m1, o1), fmaxf(m2, o2));
      m1 = fmaxf(m1, o1);
      m2 = n2;
    }
    const float gs = (p.topn == 2) ? (m1 + m2) : m1;
    int rank = 0;
    for (int gg = 0; gg < G; ++gg) {
      const float o = __uint_as_float(readlane_u32(__float_as_uint(gs), gg << lpg_log2));
      rank += ((o > gs) || (EXACT && o == gs && gg < g)) ? 1 : 0;
    }
    kept = rank < p.TG;
    if (!EXACT) {
      if (p.TG < G) {
        if (__popcll(__ballot(kept)) != (unsigned)(p.TG * lpg)) return false;
        const uint32_t gsb = __float_as_uint(gs);
        const float kmin = __uint_as_float(wave_min_u32(kept ? gsb : 0x7F7FFFFFu));
        const float dmax = __uint_as_float(wave_max_u32(kept ? 0u : gsb));
        if (!(kmin - group_err_bound(kmin) > dmax + group_err_bound(dmax))) return false;
      }
      if (__ballot(kept && (((p.topn == 2) ? m2 : m1) <= 0.0f))) return false;
    }
    hi_key = wave_max_u32(kept ? p1 : 0u) + 1u;
  }

  // ---- threshold: bisection (value space) on the kept lanes' top-5 --------
  const uint32_t q1 = kept ? p1 : 0u, q2 = kept ? p2 : 0u, q3 = kept ? p3 : 0u,
                 q4 = kept ? p4 : 0u, q5 = kept ? p5 : 0u;
  const int need = p.K + 2;
  uint32_t lo = 1u;
  const int c0 = __popcll(__ballot(q1 >= 1u)) + __popcll(__ballot(q2 >= 1u)) +
                 __popcll(__ballot(q3 >= 1u)) + __popcll(__ballot(q4 >= 1u)) +
                 __popcll(__ballot(q5 >= 1u));
  if (c0 >= need) {
    uint32_t hi = hi_key;
    while (hi - lo > 1u) {
      uint32_t mid = __float_as_uint(0.5f * (key_value(lo) + key_value(hi)));
      if (mid <= lo || mid >= hi) mid = lo + ((hi - lo) >> 1);
      const int c = __popcll(__ballot(q1 >= mid)) + __popcll(__ballot(q2 >= mid)) +
                    __popcll(__ballot(q3 >= mid)) + __popcll(__ballot(q4 >= mid)) +
                    __popcll(__ballot(q5 >= mid));
      if (c >= need) {
        lo = mid;
        if (c <= 28) break;
      } else {
        hi = mid;
      }
    }
  }
  const uint32_t theta = lo;

  // ---- compaction: candidate expert ids ------------------------------------
  int m = 0;
  if (__ballot(q5 >= theta) == 0ull) {
    // no lane has more than 4 keys >= theta: the pool holds them all
    const uint32_t pool[4] = {q1, q2, q3, q4};
    int base[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      base[i] = m;
      m += __popcll(__ballot(pool[i] >= theta));
    }
    if (m > 64) return false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool pr = pool[i] >= theta;
      const uint64_t bm = __ballot(pr);
      if (pr) L->cand[base[i] + mbcnt(bm)] = (uint32_t)slot_expert(e0, lpg, 15 - (int)(pool[i] & 15u));
    }
  } else {
    // re-scan every slot (keys recomputed)
    int base[M];
#pragma unroll
    for (int q = 0; q < M; ++q) {
      const float sc = (EXACT ? sigmoid_rn32(x[q]) : fast_sigmoid(x[q])) + bias[q];
      const uint32_t k = kept ? approx_key(sc, q) : 0u;
      base[q] = m;
      m += __popcll(__ballot(k >= theta));
    }
    if (m > 64) return false;
#pragma unroll
    for (int q = 0; q < M; ++q) {
      const float sc = (EXACT ? sigmoid_rn32(x[q]) : fast_sigmoid(x[q])) + bias[q];
      const bool pr = kept && approx_key(sc, q) >= theta;
      const uint64_t bm = __ballot(pr);
      if (pr) L->cand[base[q] + mbcnt(bm)] = (uint32_t)slot_expert(e0, lpg, q);
    }
  }
  if (m < p.K) return false;
  wave_lds_sync();

  // ---- candidates: scores and ranks by (score desc, id asc) ---------------
  const bool is_cand = lane < m;
  uint32_t eid = 0u;
  float cx = 0.0f, cb = 0.0f;
  if (is_cand) {
    eid = L->cand[lane];
    cx = row[eid];
    cb = bias_g[eid];
  }
  rank_candidates(L, lane, m, p.K, eid, cx, cb,
                  (EXACT ? sigmoid_rn32(cx) : fast_sigmoid(cx)) + cb);

  // ---- certificate -----------------------------------------------------------
  // slot k = lane for lanes 0..K-1; rank K is the best non-winner
  const bool has_next = m > p.K;
  uint4 rr = make_uint4(0u, 0u, 0u, 0u), nr = make_uint4(0u, 0u, 0u, 0u);
  if (lane < p.K) {
    rr = L->res[lane];
    if (lane < p.K - 1 || has_next) nr = L->res[lane + 1];
  }
  // the K-th score must beat every non-candidate (keys below theta)
  const float tau = key_value(theta);
  float kth = __uint_as_float(readlane_u32(rr.w, p.K - 1));
  if (EXACT) {
    if (!(kth > tau + 0x1p-19f * tau)) return false;
  } else {
    bool ok = kth - score_err(kth) > tau + score_err(tau) + 0x1p-19f * tau;
    if (ok) {
      // adjacent winners (and the K-th vs the best non-winner) must be apart
      // by more than the error, or be exact twins (same logit and bias)
      const bool check = lane < p.K && (lane < p.K - 1 || has_next);
      const float rv = __uint_as_float(rr.w), nv = __uint_as_float(nr.w);
      const bool sep = (rv - score_err(rv)) > (nv + score_err(nv));
      const bool twin = (rr.y == nr.y) && (rr.z == nr.z);
      ok = !__ballot(check && !(sep || twin));
    }
    if (!ok) {
      // Near-ties among the candidates: score them exactly and rank again.
      // The candidate set still holds every possible winner when the exact
      // K-th score beats the largest exact score a non-candidate can have.
      rescored = true;
      rank_candidates(L, lane, m, p.K, eid, cx, cb, sigmoid_rn32(cx) + cb);
      if (lane < p.K) rr = L->res[lane];
      kth = __uint_as_float(readlane_u32(rr.w, p.K - 1));
      if (!(kth > tau + score_err(tau) + 0x1p-19f * tau)) return false;
    }
  }
  if (!EXACT && rescored && lane == 0) atomicAdd(&g_rescored_tokens, 1ull);
  const float wx = __uint_as_float(rr.y);
  my_id = (int)rr.x;
  // Weights (w_k = s_k / sum s in binary64, rounded to binary32). From the
  // fast scores when their error bound keeps every weight within 0.9e-6
  // relative: |fast - RN32(sigma)| <= FAST_SIG_ERR_TESTED (tested on every
  // binary32 input) and |RN32(sigma) - sigma| <= ulp(fast) (half an ulp of
  // RN32(sigma), which is at most twice fast's), so with e_k their sum, w_k
  // moves by at most e_k/(s_k - e_k) + sum e/(sum s - sum e) relative, and the
  // final rounding adds 2^-23 (2^-40 covers the binary64 arithmetic here).
  // Otherwise from the exact scores.
  if (!EXACT) {
    const bool in = lane < p.K;
    const float sf = in ? fast_sigmoid(wx) : 0.0f;
    const double s = sf;
    const double e = in ? (double)FAST_SIG_ERR_TESTED + (double)ulp32(fmaxf(sf, 0x1p-126f)) : 0.0;
    double S = s, Se = e;  // sums over lanes 0..K-1 (K <= 32), as in the epilogue
    S += dpp_f64<DPP_XOR1>(S);
    Se += dpp_f64<DPP_XOR1>(Se);
    S += dpp_f64<DPP_XOR2>(S);
    Se += dpp_f64<DPP_XOR2>(Se);
    S += dpp_f64<DPP_HALF_MIRROR>(S);
    Se += dpp_f64<DPP_HALF_MIRROR>(Se);
    S += dpp_f64<DPP_MIRROR>(S);
    Se += dpp_f64<DPP_MIRROR>(Se);
    if (p.K > 16) {
      S += __shfl_xor(S, 16);
      Se += __shfl_xor(Se, 16);
    }
    const double A = s - e, B = S - Se;
    const bool ok = !in || (s > 2.0 * e && S > 2.0 * Se &&
                            e * B + Se * A + (0x1p-23 + 0x1p-40) * (A * B) <= 0.9e-6 * (A * B));
    if (__ballot(!ok) == 0ull) {
      my_s = sf;
      return true;
    }
  }
  my_s = (lane < p.K) ? sigmoid_rn32(wx) : 0.0f;
  return true;
}

// ---------------------------------------------------------------------------
// Exact path (every score exact; top-k by wave argmax).
// ---------------------------------------------------------------------------
template <int NP, int LPG>
__device__ __forceinline__ void route_token_exact(const float *__restrict__ row,
                                               const float (&x)[2 * NP],
                                               const float (&bias)[2 * NP],
                                               const RouteParams &p, int lane, int &my_id,
                                               float &my_s) {
  constexpr int M = 2 * NP;
  const int lpg = lpg_of<LPG>(p), lpg_log2 = lpg_log2_of<LPG>(p), G = groups_of<LPG>(p);
  const int g = lane >> lpg_log2;
  const int e0 = g * (LPG ? M * LPG : p.eg) + 2 * (lane & (lpg - 1));

  float sp[M];
#pragma unroll
  for (int q = 0; q < M; ++q) sp[q] = sigmoid_rn32(x[q]) + bias[q];

  float m1 = -__builtin_inff(), m2 = -__builtin_inff();
#pragma unroll
  for (int q = 0; q < M; ++q) {
    m2 = fmaxf(m2, fminf(m1, sp[q]));
    m1 = fmaxf(m1, sp[q]);
  }
  for (int d = 1; d < lpg; d <<= 1) {
    const float o1 = __shfl_xor(m1, d);
    const float o2 = __shfl_xor(m2, d);
    const float n2 = fmaxf(fminf(m1, o1), fmaxf(m2, o2));
    m1 = fmaxf(m1, o1);
    m2 = n2;
  }
  const float gs = (p.topn == 2) ? (m1 + m2) : m1;
  int rank = 0;
  for (int gg = 0; gg < G; ++gg) {
    const float o = __shfl(gs, gg << lpg_log2);
    rank += (o > gs) || (o == gs && gg < g);
  }
  const bool kept = rank < p.TG;

  // top-k by wave argmax over (sp desc, id asc); keys are built on the fly
  // from sp and the slot, and a per-lane bitmask marks slots already taken
  uint32_t taken = kept ? 0u : 0xFFFFFFFFu;
  my_id = 0;
  for (int r = 0; r < p.K; ++r) {
    uint64_t best = 0;
#pragma unroll
    for (int q = 0; q < M; ++q) {
      const uint32_t e = (uint32_t)slot_expert(e0, lpg, q);
      const uint64_t k = ((uint64_t)ord_f32(sp[q]) << 32) | (uint64_t)(~e);
      best = ((taken >> q) & 1u) ? best : umax64(best, k);
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) best = umax64(best, __shfl_xor(best, d));
    const uint32_t win = ~(uint32_t)best;
    if (lane == r) my_id = (int)win;
#pragma unroll
    for (int q = 0; q < M; ++q)
      if ((uint32_t)slot_expert(e0, lpg, q) == win) taken |= 1u << q;
  }
  my_s = (lane < p.K) ? sigmoid_rn32(row[my_id]) : 0.0f;
}

// ---------------------------------------------------------------------------
// Epilogue: weights, relabel, pack, store. Lanes 0..K-1 hold (id, s) of
// slot k = lane. Returns the output id of the lane's slot (-1 for k >= K).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int route_epilogue(int my_id, float my_s, const RouteParams &p,
                                              int lane, int64_t t, int32_t *__restrict__ ids,
                                              float *__restrict__ wts,
                                              int32_t *__restrict__ packed) {
  double sum = (lane < p.K) ? (double)my_s : 0.0;
  sum += dpp_f64<DPP_XOR1>(sum);
  sum += dpp_f64<DPP_XOR2>(sum);
  sum += dpp_f64<DPP_HALF_MIRROR>(sum);
  sum += dpp_f64<DPP_MIRROR>(sum);            // lanes 0..15 hold the row sum
  if (p.K > 16) sum += __shfl_xor(sum, 16);   // rows 0 and 1
  int idp = -1;
  if (lane < p.K) {
    const float w = (float)((double)my_s / sum);
    idp = my_id;
    if (p.local) idp = (my_id >= p.off && my_id < p.off + p.cnt) ? my_id - p.off : p.cnt + lane;
    const size_t o = (size_t)t * p.K + lane;
    ids[o] = my_id;
    wts[o] = w;
    packed[o] = (int32_t)(((uint32_t)idp << 16) | bf16_rne_bits(w));
  }
  return idp;
}

// Routes token t whose logits are in x (lane layout; row = the token's row).
template <int NP, int LPG>
__device__ __forceinline__ int route_token(const float *__restrict__ row,
                                           const float (&x)[2 * NP], const float (&bias)[2 * NP],
                                           const float *__restrict__ bias_g, const RouteParams &p,
                                           int lane, int64_t t, WaveScratch *L,
                                           int32_t *__restrict__ ids, float *__restrict__ wts,
                                           int32_t *__restrict__ packed,
                                           bool fast_first = true) {
  // Lane-derived values (expert ids of the slots, ...) are cheap to
  // recompute; an opaque copy of the lane index keeps the compiler from
  // hoisting them out of the caller's token loop into dozens of registers.
  int ln = lane;
  asm volatile("" : "+v"(ln));
  int my_id = 0;
  float my_s = 0.0f;
  if (!fast_first || !select_token<NP, LPG, false>(row, bias_g, x, bias, p, ln, L, my_id, my_s)) {
    if (ln == 0) atomicAdd(&g_exact_path_tokens, 1ull);
    if (!select_token<NP, LPG, true>(row, bias_g, x, bias, p, ln, L, my_id, my_s))
      route_token_exact<NP, LPG>(row, x, bias, p, ln, my_id, my_s);
  }
  return route_epilogue(my_id, my_s, p, ln, t, ids, wts, packed);
}

// Routes token t with the plain exact pipeline only (exact scores, exact
// group scores, top_k by wave argmax): the fallback of the four-tokens-per-
// wave path, kept small so that it costs that path few registers.
template <int NP, int LPG>
__device__ __forceinline__ int route_token_plain(const float *__restrict__ row,
                                                 const float (&x)[2 * NP],
                                                 const float (&bias)[2 * NP],
                                                 const RouteParams &p, int lane, int64_t t,
                                                 int32_t *__restrict__ ids,
                                                 float *__restrict__ wts,
                                                 int32_t *__restrict__ packed) {
  int ln = lane;
  asm volatile("" : "+v"(ln));
  int my_id = 0;
  float my_s = 0.0f;
  if (ln == 0) atomicAdd(&g_exact_path_tokens, 1ull);
  route_token_exact<NP, LPG>(row, x, bias, p, ln, my_id, my_s);
  return route_epilogue(my_id, my_s, p, ln, t, ids, wts, packed);
}

}  // namespace moe
