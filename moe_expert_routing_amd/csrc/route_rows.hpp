// route_rows.hpp - four tokens per wavefront, one 16-lane DPP row per token,
// for the 896-expert, 8-group shape (gfx950, wave64).
//
// Same method and the same exact result as route_wave.hpp (sigmoid router
// with a correction bias and a grouped top-k: "[ROCm][Perf] Kimi-K3:
// token-sharded residual stream for long prefills", author's reply on
// shard-routed test coverage; packed ids and the rank-local pack epilogue:
// "[kimi-k3] Rank-local expert ids for the EP routed MoE (upstream #45544)",
// commit message). Routing four tokens with one instruction stream shares
// every cross-lane step between them, and all cross-lane traffic stays inside
// a DPP row, so the selection needs no scalar-unit work per token.
//
// Lane layout. Lane l: row r = l / 16 (token t0 + r), u = l % 16, group
// g = u / 2, sub = u % 2. The lane holds the 56 experts
//   e(q) = 112 g + 4 sub + 8 (q / 4) + (q % 4),   slot q < 56,
// read as 14 float4 loads; within a lane, expert ids increase with the slot.
//
// Keys. v = fl32(s~ + fl32(b + 3)) with s~ the hardware exp2/rcp sigmoid.
// Whenever b >= -1, v lies in [2, 512), a range in which the top 6 bits of
// the binary32 pattern are constant, so
//   key = (bits(v) << 6) | (63 - q)
// orders by v at full binary32 resolution, then by lower slot. |v - (sp +
// 3)| <= row_err(v) (sp the exact biased score); see row_err.
//
// Selection.
//  1. Each lane keeps its top-10 keys (v_max_u32 + nine v_med3_u32 per key).
//  2. Group score from the lane pair's top-2; group ranks by comparing
//     unique integer group keys around the row (row_ror); the choice is
//     certified by the margin between the kept and the dropped groups.
//  3. top_k + 1 rounds of row-maximum extraction over the kept lanes' pool
//     heads: the first top_k are the winners, the last bounds every other
//     expert of the kept groups from above.
//  4. The winners are scored exactly (RN32 sigmoid, fl32 bias add) and
//     ranked by (sp desc, id asc); the result is accepted when the weakest
//     winner's exact score beats that bound, exactly top_k + 1 keys were
//     taken (no equal keys) and no lane used up its pool.
// A row that fails a check is routed again by the one-token-per-wave exact
// pipeline of route_wave.hpp.
#pragma once

#include "route_wave.hpp"

namespace moe {
namespace rows {

// Tokens that went through the exact refinement (diagnostic counter).
__device__ unsigned long long g_refined_tokens = 0ull;

constexpr int E = 896;
constexpr int G = 8;
constexpr int EG = 112;
constexpr int LANES = 16;     // lanes per token (one DPP row)
constexpr int NQ = 14;        // float4 loads per lane
constexpr int SLOTS = 4 * NQ; // experts per lane
constexpr int POOL = 10;      // keys kept per lane
constexpr int MAX_K = 16;     // top_k handled by this path
constexpr int BIAS_GSTRIDE = 120;  // LDS floats per group: b128 reads hit 64 distinct banks
constexpr float BIAS_SHIFT = 3.0f;

constexpr int DPP_ROR2 = 0x122, DPP_ROR4 = 0x124, DPP_ROR6 = 0x126, DPP_ROR8 = 0x128,
              DPP_ROR10 = 0x12A, DPP_ROR12 = 0x12C, DPP_ROR14 = 0x12E;

constexpr int MAX_CAND = 32;  // exact candidates per row in the refinement

// Per-wave LDS of the row path, by row: winner / candidate ids, exact keys
// and scores, the final (id, s) by slot.
struct RowScratch {
  int32_t id[4][MAX_K];
  int32_t cnt[4][LANES];
  int32_t cand[4][MAX_CAND];
  unsigned long long ekey[4][MAX_CAND];
  float sval[4][MAX_CAND];
  uint2 slot[4][MAX_K];
  float kth[4];
};

// |v - (sp + 3)| for a key value v, sp = RN32(RN32(sigma(x)) + b): the fast
// sigmoid error (<= FAST_SIG_ERR) and three binary32 roundings (of b + 3,
// of s~ + (b + 3), of the exact s + b), each at most 2^-24 v, with margin.
__device__ __forceinline__ float row_err(float v) { return 1.01f * FAST_SIG_ERR + 0x1p-22f * v; }
// Same for a group score of up to two key values plus its own rounding and
// the rounding of the exact group score.
__device__ __forceinline__ float row_group_err(float v) {
  return 2.02f * FAST_SIG_ERR + 0x1p-21f * v;
}

__device__ __forceinline__ float key_v(uint32_t k) { return __uint_as_float((k >> 6) | 0x40000000u); }

// Expert id of a key held by the lane whose first expert is `base`.
__device__ __forceinline__ int key_expert(uint32_t k, int base) {
  const int q = 63 - (int)(k & 63u);
  return base + q + (q & ~3);
}

// Inverse of ord_f32.
__device__ __forceinline__ float ord_inv(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  return ((uint64_t)dpp<CTRL>((uint32_t)(v >> 32)) << 32) | dpp<CTRL>((uint32_t)v);
}

// Number of the other 7 groups of the row whose key is larger (keys unique).
template <typename KT>
__device__ __forceinline__ int group_rank(KT gk) {
  int n = 0;
  if constexpr (sizeof(KT) == 8) {
    n += dpp_u64<DPP_ROR2>(gk) > gk ? 1 : 0;
    n += dpp_u64<DPP_ROR4>(gk) > gk ? 1 : 0;
    n += dpp_u64<DPP_ROR6>(gk) > gk ? 1 : 0;
    n += dpp_u64<DPP_ROR8>(gk) > gk ? 1 : 0;
    n += dpp_u64<DPP_ROR10>(gk) > gk ? 1 : 0;
    n += dpp_u64<DPP_ROR12>(gk) > gk ? 1 : 0;
    n += dpp_u64<DPP_ROR14>(gk) > gk ? 1 : 0;
  } else {
    n += dpp<DPP_ROR2>(gk) > gk ? 1 : 0;
    n += dpp<DPP_ROR4>(gk) > gk ? 1 : 0;
    n += dpp<DPP_ROR6>(gk) > gk ? 1 : 0;
    n += dpp<DPP_ROR8>(gk) > gk ? 1 : 0;
    n += dpp<DPP_ROR10>(gk) > gk ? 1 : 0;
    n += dpp<DPP_ROR12>(gk) > gk ? 1 : 0;
    n += dpp<DPP_ROR14>(gk) > gk ? 1 : 0;
  }
  return n;
}

__device__ __forceinline__ uint32_t row_max(uint32_t v) {
  v = umax(v, dpp<DPP_XOR1>(v));
  v = umax(v, dpp<DPP_XOR2>(v));
  v = umax(v, dpp<DPP_HALF_MIRROR>(v));
  return umax(v, dpp<DPP_MIRROR>(v));
}
__device__ __forceinline__ uint32_t row_min(uint32_t v) {
  v = umin(v, dpp<DPP_XOR1>(v));
  v = umin(v, dpp<DPP_XOR2>(v));
  v = umin(v, dpp<DPP_HALF_MIRROR>(v));
  return umin(v, dpp<DPP_MIRROR>(v));
}
__device__ __forceinline__ uint32_t row_sum(uint32_t v) {
  v += dpp<DPP_XOR1>(v);
  v += dpp<DPP_XOR2>(v);
  v += dpp<DPP_HALF_MIRROR>(v);
  return v + dpp<DPP_MIRROR>(v);
}
__device__ __forceinline__ double row_sum_f64(double v) {
  v += dpp_f64<DPP_XOR1>(v);
  v += dpp_f64<DPP_XOR2>(v);
  v += dpp_f64<DPP_HALF_MIRROR>(v);
  return v + dpp_f64<DPP_MIRROR>(v);
}

// Stages fl32(b + 3) in the row layout (block of `threads` threads); returns
// false (block-uniform) when some bias lies outside [-1, 500), where the key
// encoding does not hold. `bad` is an LDS word.
template <int THREADS>
__device__ __forceinline__ bool stage_bias(const float *__restrict__ bias, float *lds, int *bad) {
  if (threadIdx.x == 0) *bad = 0;
  __syncthreads();
  bool ok = true;
#pragma unroll
  for (int k = 0; k < (E + THREADS - 1) / THREADS; ++k) {
    const int e = threadIdx.x + k * THREADS;
    if (e < E) {
      const float bb = bias[e] + BIAS_SHIFT;
      ok = ok && (bb >= 2.0f) && (bb < 503.0f);
      lds[(e / EG) * BIAS_GSTRIDE + (e % EG)] = bb;
    }
  }
  if (!ok) *bad = 1;
  __syncthreads();
  return *bad == 0;
}

// Row epilogue: lane u of a row whose `out` is set holds slot u's (id, s)
// in sl (lanes u >= K hold nothing). Weights, relabel, pack and stores use
// the same arithmetic in the same order as route_epilogue, so all paths give
// identical bits.
__device__ __forceinline__ void row_outputs(bool out, uint2 sl, const RouteParams &p, int u,
                                            int64_t t, int32_t *__restrict__ ids,
                                            float *__restrict__ wts,
                                            int32_t *__restrict__ packed) {
  const double sum = row_sum_f64(out ? (double)__uint_as_float(sl.y) : 0.0);
  if (out) {
    const int id = (int)sl.x;
    const float w = (float)((double)__uint_as_float(sl.y) / sum);
    int idp = id;
    if (p.local) idp = (id >= p.off && id < p.off + p.cnt) ? id - p.off : p.cnt + u;
    const size_t o = (size_t)t * p.K + u;
    ids[o] = id;
    wts[o] = w;
    packed[o] = (int32_t)(((uint32_t)idp << 16) | bf16_rne_bits(w));
  }
}

// Number of pool entries (sorted by key) whose value is >= thr.
__device__ __forceinline__ int pool_count_ge(const uint32_t (&pool)[POOL], double thr) {
  int c = 0;
#pragma unroll
  for (int i = 0; i < POOL; ++i) c += ((double)key_v(pool[i]) >= thr) ? 1 : 0;
  return c;
}

// Exact refinement of the rows with `need` set (call with the whole wave).
// Exact group scores from every pool entry that can hold a group's top
// scores, then the exact top_k from every kept-pool entry within twice the
// key error of the (top_k+1)-th extracted key; both steps decide from exact
// scores, so they can only fail when a lane's pool is too short or the
// candidates exceed MAX_CAND. Returns true (row-uniform) when the row has
// been written.
__device__ __forceinline__ bool refine_rows(const float *__restrict__ row,
                                         const float *__restrict__ bias_g,
                                         const uint32_t (&pool)[POOL], uint32_t m1, uint32_t m2,
                                         bool need, const RouteParams &p, int r, int u, int g,
                                         int base, int64_t t, RowScratch *L,
                                         int32_t *__restrict__ ids, float *__restrict__ wts,
                                         int32_t *__restrict__ packed) {
  const int K = p.K;
  bool fail = false;
  if (need && u == 0) atomicAdd(&g_refined_tokens, 1ull);

  // ---- exact group scores ------------------------------------------------------
  // An expert whose key value is below thr1 is beaten, even exactly, by the
  // two experts holding the group's approximate top-2 keys.
  const float v1 = key_v(m1);
  const double thr1 = (double)(p.topn == 2 ? key_v(m2) : v1) - 2.0 * (double)row_err(v1);
  const int c1 = need ? pool_count_ge(pool, thr1) : 0;
  fail = fail || row_max(c1 >= POOL ? 1u : 0u) != 0u;
  uint32_t t1 = 0u, t2 = 0u;  // exact top-2 of the lane's candidates (ord keys)
#pragma unroll
  for (int i = 0; i < POOL; ++i) {
    if (!__ballot(i < c1)) break;
    if (i < c1) {
      const int e = key_expert(pool[i], base);
      const uint32_t o = ord_f32(sigmoid_rn32(row[e]) + bias_g[e]);
      t2 = umax(t2, umin(t1, o));
      t1 = umax(t1, o);
    }
  }
  top2_merge(t1, t2, dpp<DPP_XOR1>(t1), dpp<DPP_XOR1>(t2));
  const float gsx = (p.topn == 2) ? ord_inv(t1) + ord_inv(t2) : ord_inv(t1);
  const uint64_t gkx = ((uint64_t)ord_f32(gsx) << 3) | (uint64_t)(7 - g);
  const bool kept = group_rank(gkx) < p.TG;

  // ---- extraction over the exactly kept groups ----------------------------------
  uint32_t q[POOL];
#pragma unroll
  for (int i = 0; i < POOL; ++i) q[i] = pool[i];
  q[0] = kept ? q[0] : 0u;
  uint32_t M = 0u;
  for (int rd = 0; rd <= K; ++rd) {
    M = row_max(q[0]);
    const bool win = q[0] == M;
#pragma unroll
    for (int i = 0; i < POOL - 1; ++i) q[i] = win ? q[i + 1] : q[i];
  }

  // ---- exact top_k from the candidates within the error band ----------------------
  const float vm = key_v(M);
  const double thb = (double)vm - 2.0 * (double)row_err(vm);
  const int c2 = (need && kept) ? pool_count_ge(pool, thb) : 0;
  fail = fail || row_max(c2 >= POOL ? 1u : 0u) != 0u;
  const int m = (int)row_sum((uint32_t)c2);
  fail = fail || m > MAX_CAND || m < K;
  L->cnt[r][u] = c2;
  wave_lds_sync();
  int excl = 0;
#pragma unroll
  for (int j = 0; j < LANES; ++j) excl += (j < u) ? L->cnt[r][j] : 0;
#pragma unroll
  for (int i = 0; i < POOL; ++i) {
    if (!__ballot(i < c2)) break;
    if (i < c2 && excl + i < MAX_CAND) L->cand[r][excl + i] = key_expert(pool[i], base);
  }
  wave_lds_sync();
  const bool ok_m = need && !fail;
  uint64_t ek[2] = {0ull, 0ull};
  float es[2] = {0.0f, 0.0f};
  int eid[2] = {0, 0};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int j = u + LANES * h;
    if (ok_m && j < m) {
      eid[h] = L->cand[r][j];
      es[h] = sigmoid_rn32(row[eid[h]]);
      const float sp = es[h] + bias_g[eid[h]];
      ek[h] = ((uint64_t)ord_f32(sp) << 32) | (uint64_t)(~(uint32_t)eid[h]);
      L->ekey[r][j] = ek[h];
    }
  }
  wave_lds_sync();
  const int mmax = (int)wave_max_u32(ok_m ? (uint32_t)m : 0u);
  int rk[2] = {0, 0};
  for (int j = 0; j < mmax; ++j) {
    const uint64_t o = (ok_m && j < m) ? L->ekey[r][j] : 0ull;
    rk[0] += o > ek[0] ? 1 : 0;
    rk[1] += o > ek[1] ? 1 : 0;
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int j = u + LANES * h;
    if (ok_m && j < m && rk[h] < K) {
      L->slot[r][rk[h]] = make_uint2((uint32_t)eid[h], __float_as_uint(es[h]));
      if (rk[h] == K - 1) L->kth[r] = ord_inv((uint32_t)(ek[h] >> 32));
    }
  }
  wave_lds_sync();
  // every expert outside the candidates has key value < thb, so an exact
  // score below thb - 3 + row_err(thb); the K-th winner must beat it (it
  // does whenever the arithmetic above is right; kept as a guard)
  const double bound = thb - 3.0 + (1.01 * (double)FAST_SIG_ERR + 0x1p-22 * thb);
  const bool ok = ok_m && (double)L->kth[r] > bound;
  uint2 sl = make_uint2(0u, 0u);
  if (ok && u < K) sl = L->slot[r][u];
  row_outputs(ok && u < K, sl, p, u, t, ids, wts, packed);
  return ok;
}

// Routes tokens t0 .. t0+3 (rows beyond T are computed on token T-1 and
// discarded). Returns a 4-bit mask of the rows that must be routed again by
// the one-token-per-wave path; every other valid row has been written.
__device__ __forceinline__ uint32_t route_rows4(const float *__restrict__ logits,
                                                const float *__restrict__ bias_g,
                                                const float *__restrict__ bias_lds, int T,
                                                int64_t t0, const RouteParams &p, int lane,
                                                RowScratch *L, int32_t *__restrict__ ids,
                                                float *__restrict__ wts,
                                                int32_t *__restrict__ packed) {
  int ln = lane;
  asm volatile("" : "+v"(ln));
  const int r = ln >> 4, u = ln & 15, g = u >> 1, sub = u & 1;
  const int64_t t = t0 + r;
  const bool valid = t < T;
  const float *row = logits + (size_t)(valid ? t : (int64_t)T - 1) * E;
  const int base = g * EG + 4 * sub;
  const float4 *xp = reinterpret_cast<const float4 *>(row + base);
  const float4 *bp = reinterpret_cast<const float4 *>(bias_lds + g * BIAS_GSTRIDE + 4 * sub);

  // ---- streaming: keys -> the lane's top-7 ----------------------------------
  // Loads run PREFETCH float4 ahead of their use.
  uint32_t p1 = 0u, p2 = 0u, p3 = 0u, p4 = 0u, p5 = 0u, p6 = 0u, p7 = 0u, p8 = 0u, p9 = 0u,
           p10 = 0u;
  constexpr int PREFETCH = 3;
  float4 xq[PREFETCH];
#pragma unroll
  for (int i = 0; i < PREFETCH; ++i) xq[i] = xp[2 * i];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const float4 xv = xq[i % PREFETCH];
    if (i + PREFETCH < NQ) xq[i % PREFETCH] = xp[2 * (i + PREFETCH)];
    const float4 bv = bp[2 * i];
    const float xs[4] = {xv.x, xv.y, xv.z, xv.w};
    const float bs[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float v = fast_sigmoid(xs[j]) + bs[j];
      const uint32_t k = (__float_as_uint(v) << 6) | (uint32_t)(63 - (4 * i + j));
      p10 = umed3(p9, p10, k);
      p9 = umed3(p8, p9, k);
      p8 = umed3(p7, p8, k);
      p7 = umed3(p6, p7, k);
      p6 = umed3(p5, p6, k);
      p5 = umed3(p4, p5, k);
      p4 = umed3(p3, p4, k);
      p3 = umed3(p2, p3, k);
      p2 = umed3(p1, p2, k);
      p1 = umax(p1, k);
    }
    // materialise the pool here: otherwise the compiler sinks the lower
    // pool levels to the end and keeps every intermediate key alive
    asm volatile("" : "+v"(p1), "+v"(p2), "+v"(p3), "+v"(p4), "+v"(p5), "+v"(p6), "+v"(p7),
                 "+v"(p8), "+v"(p9), "+v"(p10));
  }

  // ---- groups ---------------------------------------------------------------
  const uint32_t o1 = dpp<DPP_XOR1>(p1), o2 = dpp<DPP_XOR1>(p2);
  const uint32_t m1 = umax(p1, o1);
  const uint32_t m2 = umax(umax(umin(p1, o1), p2), o2);
  const float gs = (p.topn == 2) ? key_v(m1) + key_v(m2) : key_v(m1);  // in [2, 1030)
  // unique group key: score bits (the top 3 bits are constant), then lower group
  const uint32_t gk = (__float_as_uint(gs) << 3) | (uint32_t)(7 - g);
  const bool kept = group_rank(gk) < p.TG;
  // certified when the weakest kept group beats the strongest dropped one
  // by more than both error bounds
  const uint32_t gsb = __float_as_uint(gs);
  const float kmin = __uint_as_float(row_min(kept ? gsb : 0x7F7FFFFFu));
  const float dmax = __uint_as_float(row_max(kept ? 0u : gsb));
  bool fail = !(kmin - row_group_err(kmin) > dmax + row_group_err(dmax));

  // ---- extraction: top_k + 1 rounds of row maximum ---------------------------
  const uint32_t pool[POOL] = {p1, p2, p3, p4, p5, p6, p7, p8, p9, p10};
  p1 = kept ? p1 : 0u;  // dropped lanes never win (real keys are > 0 unless v == 2)
  const uint32_t s1 = p1, s2 = p2, s3 = p3, s4 = p4, s5 = p5, s6 = p6, s7 = p7, s8 = p8, s9 = p9;
  uint32_t rounds = 0u;  // bit (K - round) set when this lane won that round
  uint32_t M = 0u;       // after the loop: the (K+1)-th key, the best non-winner
  const int K = p.K;
  for (int rd = 0; rd <= K; ++rd) {
    M = row_max(p1);
    const bool win = p1 == M;
    rounds = rounds + rounds + (win ? 1u : 0u);
    p1 = win ? p2 : p1;
    p2 = win ? p3 : p2;
    p3 = win ? p4 : p3;
    p4 = win ? p5 : p4;
    p5 = win ? p6 : p5;
    p6 = win ? p7 : p6;
    p7 = win ? p8 : p7;
    p8 = win ? p9 : p8;
    p9 = win ? p10 : p9;
  }
  const int pops = __popc(rounds);
  const uint32_t total = row_sum((uint32_t)pops);
  // exactly K+1 entries taken (no equal keys) and no lane used up its pool
  fail = fail || total != (uint32_t)(K + 1) || pops >= POOL;

  // ---- winners (the first K extracted) to LDS: expert ids ----------------------
  uint32_t rem = rounds >> 1;  // drop round K (the best non-winner)
#pragma unroll
  for (int i = 0; i < POOL - 1; ++i) {
    if (!__ballot(rem != 0u)) break;
    if (rem != 0u) {
      const uint32_t key = i == 0 ? s1 : i == 1 ? s2 : i == 2 ? s3 : i == 3 ? s4 : i == 4 ? s5
                         : i == 5 ? s6 : i == 6 ? s7 : i == 7 ? s8 : s9;
      const int hb = 31 - __clz(rem);  // earliest remaining round
      rem ^= 1u << hb;
      const int q = 63 - (int)(key & 63u);
      L->id[r][K - 1 - hb] = base + q + (q & ~3);
    }
  }
  wave_lds_sync();

  // ---- exact scores of the winners; exact order by (sp desc, id asc) ---------------
  const uint32_t pre_fail = row_max((fail && valid) ? 1u : 0u);
  const bool act = pre_fail == 0u && valid && u < K;
  int my_id = 0;
  float my_s = 0.0f, my_sp = 0.0f;
  if (act) {
    my_id = L->id[r][u];
    my_s = sigmoid_rn32(row[my_id]);
    my_sp = my_s + bias_g[my_id];
    L->ekey[r][u] = ((uint64_t)ord_f32(my_sp) << 32) | (uint64_t)(~(uint32_t)my_id);
  }
  // every expert outside the winners has a key below M: its exact score is at
  // most key_v(M) - 3 + row_err(key_v(M)); the weakest winner must beat that
  const float vm = key_v(M);
  const double bound = (double)vm - 3.0 + (double)row_err(vm);
  const uint32_t weakest = row_min(act ? ord_f32(my_sp) : 0xFFFFFFFFu);
  const float wsp = __uint_as_float((weakest & 0x80000000u) ? (weakest & 0x7FFFFFFFu) : ~weakest);
  const bool boundary_ok = (double)wsp > bound;
  wave_lds_sync();
  int rank = 0;
  if (act) {
    const uint64_t mk = L->ekey[r][u];
    for (int j = 0; j < K; ++j) rank += L->ekey[r][j] > mk ? 1 : 0;
  }
  const uint32_t row_fail = pre_fail | ((valid && !boundary_ok && pre_fail == 0u) ? 1u : 0u);

  // ---- epilogue: lane u takes slot u (the winner of exact rank u); weights,
  // relabel, pack, store with the same arithmetic, in the same order, as the
  // one-token-per-wave epilogue, so both paths give identical bits
  if (row_fail == 0u && act) L->slot[r][rank] = make_uint2((uint32_t)my_id, __float_as_uint(my_s));
  wave_lds_sync();
  const bool out = row_fail == 0u && act;
  uint2 sl = make_uint2(0u, 0u);
  if (out) sl = L->slot[r][u];
  row_outputs(out, sl, p, u, t, ids, wts, packed);

  // ---- rows whose certificate failed: exact refinement -------------------------
  bool done = row_fail == 0u;
  const bool need = !done && valid;
  if (__ballot(need)) {
    wave_lds_sync();
    done = refine_rows(row, bias_g, pool, m1, m2, need, p, r, u, g, base, t, L, ids, wts, packed) ||
           done;
  }
  // rows to route again
  const uint64_t fb = __ballot(!done && valid && u == 0);
  return (uint32_t)((fb & 1ull) | ((fb >> 15) & 2ull) | ((fb >> 30) & 4ull) | ((fb >> 45) & 8ull));
}

}  // namespace rows
}  // namespace moe
