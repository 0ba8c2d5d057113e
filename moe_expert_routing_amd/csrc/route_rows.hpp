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
// a DPP row, so the selection needs almost no scalar-unit work.
//
// Lane layout. Lane l: row r = l / 16 (token t0 + r), u = l % 16, quad
// c = u / 4, sub = u % 4. In pass 0 the lane reads group c, in pass 1 group
// c + 4; its slot q = 28 pass + 4 i + j (i < 7, j < 4) is expert
//   e(q) = 112 (c + 4 pass) + 4 sub + 16 i + j,
// so the four lanes of a group read 64 contiguous bytes per load, and expert
// ids increase with the slot.
//
// Keys. v = fl32(s~ + fl32(b + B)) with s~ the hardware exp2/rcp sigmoid and a
// constant shift B that puts v in a window of eight binades whose binary32
// patterns share their top 6 bits (a window that starts at a multiple of
// 2^26), so
//   key = (bits(v) << 6) | (63 - q)
// orders by v at full binary32 resolution, then by lower slot (lower id).
// Two windows (KeyWindow): B = 1/2, v in [2^-7, 2), for biases in
// [-0.49, 0.49], which keeps the top scores (v in [1, 2)) at a resolution of
// 2^-23; otherwise B = 3, v in [2, 512), for biases in [-1, 500). Each block
// picks one from the biases it stages.
// |v - (sp + B)| <= row_err(v, B) (sp the exact biased score).
//
// Selection.
//  1. Each lane keeps its top-8 keys of each pass (v_max_u32 + seven
//     v_med3_u32 per key).
//  2. Group scores from the quad's top-2 of each pass; group ranks by
//     comparing unique integer group keys around the row (row_ror); the
//     choice is certified by the margin between the kept and the dropped
//     groups.
//  3. Tournament: each lane writes its two pass pools to LDS; top_k + 1
//     rounds of the row maximum over the heads of the lanes' kept pools, each
//     advancing the winning lane's pointer, give the winners in order, and
//     the last maximum M bounds every other expert of the kept groups. It
//     must take exactly top_k + 1 keys (no equal keys) and use up no pool.
//  4. Certificate from the keys: when each winner's value beats the next
//     one's by more than both errors, the round order is the exact
//     (sp desc, id asc) order and no other expert reaches the K-th score;
//     when, in addition, the scores read off the keys keep every weight
//     within 0.9e-6 of the exact one, the row is written from the keys.
//     Otherwise the winners are scored exactly (RN32 sigmoid, fl32 bias add)
//     and ranked, and that stands when the weakest one beats M's bound.
// A row that fails a check is settled by an exact refinement in the same
// layout (exact group scores, exact scores of every candidate in the error
// band); only a row the refinement cannot decide either (ties denser than
// the pools) is routed again by the one-token-per-wave exact pipeline of
// route_wave.hpp.
#pragma once

#include "route_wave.hpp"

namespace moe {
namespace rows {

// Tokens that went through the exact refinement (diagnostic counter).
__device__ unsigned long long g_refined_tokens = 0ull;

constexpr int E = 896;
constexpr int G = 8;
constexpr int EG = 112;
constexpr int LANES = 16;   // lanes per token (one DPP row)
constexpr int NQP = 7;      // float4 loads per lane and pass
constexpr int PP = 8;       // keys kept per lane and pass
constexpr int PPS = PP;     // keys the streaming keeps
constexpr int POOL = 10;    // merged keys of the kept groups per lane
constexpr int MAX_K = 16;   // top_k handled by this path
constexpr int MAX_CAND = 32;  // exact candidates per row in the refinement
// Key windows: the shift B, the first bit pattern of the window and the range
// that fl32(b + B) must stay in (so that v = s~ + fl32(b + B) stays inside).
template <int W> struct KeyWindow;
template <> struct KeyWindow<0> {  // v in [2^-7, 2)
  static constexpr float shift = 0.5f;
  static constexpr uint32_t base = 0x3C000000u;  // bits(2^-7) = 15 * 2^26
  static constexpr float lo = 0x1p-7f, hi = 0.99f;
};
template <> struct KeyWindow<1> {  // v in [2, 512)
  static constexpr float shift = 3.0f;
  static constexpr uint32_t base = 0x40000000u;  // bits(2) = 16 * 2^26
  static constexpr float lo = 2.0f, hi = 503.0f;
};
constexpr int PREFETCH = 7;   // float4 loads in flight per lane (one pass)
constexpr int NSTORE = 8;     // pool entries per pass the tournament reads from LDS

constexpr int DPP_ROR4 = 0x124, DPP_ROR8 = 0x128, DPP_ROR12 = 0x12C;

// Per-wave LDS of the row path. The tournament's pools (each lane's first
// NSTORE keys of each pass, then a zero sentinel; [pass][i][lane], so the
// lanes of a wave always read 64 different banks) are dead once the winners
// are known, and share their space with the exact stage's candidate ids
// and final (id, s) by slot.
struct RowScratch {
  uint2 win[4][MAX_K];  // winner of tournament round k: (key, lane in the row)
  uint2 sink[64];       // the tournament's stores of lanes that did not win a round
  union {
    uint32_t pool[2][NSTORE + 1][64];
    struct {
      int32_t cand[4][MAX_CAND];
      uint2 slot[4][MAX_K];
      float kth[4];
    };
  };
};

// |v - (sp + B)| for a key value v, sp = RN32(RN32(sigma(x)) + b), sh = B > 0:
// the fast sigmoid error (<= FAST_SIG_ERR) and three binary32 roundings, of
// b + B and of s~ + (b + B) (each at most 2^-24 v) and of the exact s + b
// (at most 2^-24 |sp| <= 2^-24 (v + sh)), with margin.
__device__ __forceinline__ float row_err(float v, float sh) {
  return 1.01f * FAST_SIG_ERR + 0x1p-24f * (3.03f * v + 1.01f * sh);
}
// Same for a group score g = fl32(v1 + v2) of up to two key values: both key
// errors, the rounding of g (2^-24 g) and that of the exact group score
// (2^-24 |gs| <= 2^-24 (g + 2 sh)), with margin.
__device__ __forceinline__ float row_group_err(float g, float sh) {
  return 2.02f * FAST_SIG_ERR + 0x1p-24f * (5.1f * g + 4.1f * sh);
}

template <int W>
__device__ __forceinline__ float key_v(uint32_t k) {
  return __uint_as_float((k >> 6) | KeyWindow<W>::base);
}

// Expert id of a key held by the lane (quad c, sub).
__device__ __forceinline__ int key_expert(uint32_t k, int c, int sub) {
  const int q = 63 - (int)(k & 63u);
  const int pass = q >= 28 ? 1 : 0;
  const int qq = q - 28 * pass;
  return (c + 4 * pass) * EG + 4 * sub + 16 * (qq >> 2) + (qq & 3);
}

// Inverse of ord_f32.
__device__ __forceinline__ float ord_inv(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
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

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  return ((uint64_t)dpp<CTRL>((uint32_t)(v >> 32)) << 32) | dpp<CTRL>((uint32_t)v);
}

// Sum of v over the lanes before this one in its row: a Hillis-Steele scan by
// row shifts (row_shr:n; a lane with no source n lanes down reads zero).
__device__ __forceinline__ uint32_t row_exclusive_sum(uint32_t v) {
  uint32_t s = v;
  s += dpp<0x111>(s);
  s += dpp<0x112>(s);
  s += dpp<0x114>(s);
  s += dpp<0x118>(s);
  return s - v;
}

// Adds to rk_i the number of keys larger than k_i among ks[] of the other
// lanes of the row (row_ror:D for D = 1..15; every lane's keys are unique or
// zero, and zero never counts).
template <int N, int D = 1>
__device__ __forceinline__ void rank_in_row(const uint64_t (&ks)[N], int (&rk)[N]) {
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const uint64_t o = dpp_u64<0x120 + D>(ks[j]);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      rk[i] += o > ks[i] ? 1 : 0;
      // a running count, not a sum tree over every rotation: the selection's
      // register peak is here
      asm volatile("" : "+v"(rk[i]));
    }
  }
  if constexpr (D + 1 < LANES) rank_in_row<N, D + 1>(ks, rk);
}

// Ranks of the lane's two groups (keys a: group c, b: group c + 4) among
// the row's 8 groups: the number of larger keys (keys are unique).
template <typename KT>
__device__ __forceinline__ void group_ranks(KT a, KT b, int &ra, int &rb) {
  KT o[6];
  if constexpr (sizeof(KT) == 8) {
    o[0] = dpp_u64<DPP_ROR4>(a); o[1] = dpp_u64<DPP_ROR8>(a); o[2] = dpp_u64<DPP_ROR12>(a);
    o[3] = dpp_u64<DPP_ROR4>(b); o[4] = dpp_u64<DPP_ROR8>(b); o[5] = dpp_u64<DPP_ROR12>(b);
  } else {
    o[0] = dpp<DPP_ROR4>(a); o[1] = dpp<DPP_ROR8>(a); o[2] = dpp<DPP_ROR12>(a);
    o[3] = dpp<DPP_ROR4>(b); o[4] = dpp<DPP_ROR8>(b); o[5] = dpp<DPP_ROR12>(b);
  }
  ra = b > a ? 1 : 0;
  rb = a > b ? 1 : 0;
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    ra += o[i] > a ? 1 : 0;
    rb += o[i] > b ? 1 : 0;
  }
}

// Stages fl32(b + B) (in expert order) for a block of THREADS threads, for
// the key window that every bias fits (0 preferred). Returns that window, or
// -1 (block-uniform) when some bias fits neither (or is not finite); then
// nothing is staged. `bad` holds one LDS word per wave. Every load is issued
// before the first is used (clamped indices, no branches), so the staging
// costs one memory round trip.
template <int THREADS>
__device__ __forceinline__ int stage_bias(const float *__restrict__ bias, float *lds, int *bad) {
  constexpr int N = (E + THREADS - 1) / THREADS;
  float bb[N];
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const int e = (int)threadIdx.x + k * THREADS;
    bb[k] = bias[e < E ? e : E - 1];
  }
  bool ok0 = true, ok1 = true;
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const float v0 = bb[k] + KeyWindow<0>::shift, v1 = bb[k] + KeyWindow<1>::shift;
    ok0 = ok0 && (v0 >= KeyWindow<0>::lo) && (v0 <= KeyWindow<0>::hi);
    ok1 = ok1 && (v1 >= KeyWindow<1>::lo) && (v1 < KeyWindow<1>::hi);
  }
  const bool bad0 = __ballot(!ok0) != 0ull, bad1 = __ballot(!ok1) != 0ull;
  if ((threadIdx.x & 63) == 0) bad[threadIdx.x >> 6] = (bad0 ? 1 : 0) | (bad1 ? 2 : 0);
  __syncthreads();
  int any = 0;
#pragma unroll
  for (int w = 0; w < THREADS / 64; ++w) any |= bad[w];
  const int window = (any & 1) == 0 ? 0 : ((any & 2) == 0 ? 1 : -1);
  if (window >= 0) {
    const float sh = window == 0 ? KeyWindow<0>::shift : KeyWindow<1>::shift;
#pragma unroll
    for (int k = 0; k < N; ++k) {
      const int e = (int)threadIdx.x + k * THREADS;
      if (e < E) lds[e] = bb[k] + sh;
    }
  }
  __syncthreads();
  return window;
}

// float4 n (n < 14) of a lane: pass n / 7, load n % 7 (float4 units from the
// lane's first expert of the row).
__host__ __device__ constexpr int lane_off(int n) { return (n / NQP) * EG + 4 * (n % NQP); }

// Issues the lane's first PREFETCH float4 loads of the token at `row`.
__device__ __forceinline__ void first_loads(const float *__restrict__ row, int c, int sub,
                                            float4 (&xq)[PREFETCH]) {
  const float4 *xp = reinterpret_cast<const float4 *>(row + c * EG + 4 * sub);
#pragma unroll
  for (int n = 0; n < PREFETCH; ++n) xq[n] = xp[lane_off(n)];
}

// Streams the lane's 56 experts of the token at `row`: keys into the sorted
// top-8 of each pass (a: pass 0, b: pass 1). xq holds the first PREFETCH
// loads (first_loads); the rest are issued here as those are consumed.
__device__ __forceinline__ void stream_pools(const float *__restrict__ row,
                                             const float *__restrict__ bias_lds, int c, int sub,
                                             float4 (&xq)[PREFETCH], uint32_t (&a)[PP],
                                             uint32_t (&b)[PP]) {
  const float4 *xp = reinterpret_cast<const float4 *>(row + c * EG + 4 * sub);
  const float4 *bp = reinterpret_cast<const float4 *>(bias_lds + c * EG + 4 * sub);
  auto off = [](int n) { return lane_off(n); };
#pragma unroll
  for (int i = 0; i < PP; ++i) a[i] = b[i] = 0u;
#pragma unroll
  for (int n = 0; n < 2 * NQP; ++n) {
    const float4 xv = xq[n % PREFETCH];
    if (n + PREFETCH < 2 * NQP) xq[n % PREFETCH] = xp[off(n + PREFETCH)];
    const float4 bv = bp[off(n)];
    const float xs[4] = {xv.x, xv.y, xv.z, xv.w};
    const float bs[4] = {bv.x, bv.y, bv.z, bv.w};
    uint32_t(&pl)[PP] = n < NQP ? a : b;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float v = fast_sigmoid(xs[j]) + bs[j];
      const uint32_t k = (__float_as_uint(v) << 6) | (uint32_t)(63 - (4 * n + j));
#pragma unroll
      for (int i = PPS - 1; i > 0; --i) pl[i] = umed3(pl[i - 1], pl[i], k);
      pl[0] = umax(pl[0], k);
    }
    // materialise the pool here: otherwise the compiler sinks the lower
    // pool levels to the end and keeps every intermediate key alive
    asm volatile("" : "+v"(pl[0]), "+v"(pl[1]), "+v"(pl[2]), "+v"(pl[3]), "+v"(pl[4]),
                 "+v"(pl[5]), "+v"(pl[6]), "+v"(pl[7]));
  }
}

// Approximate group stage: the quad's top-2 of each pass, group scores,
// kept flags, and whether the choice is certified.
template <int W>
__device__ __forceinline__ bool approx_groups(const uint32_t (&a)[PP], const uint32_t (&b)[PP],
                                              const RouteParams &p, int c, bool &kept_a,
                                              bool &kept_b) {
  constexpr float sh = KeyWindow<W>::shift;
  uint32_t a1 = a[0], a2 = a[1], b1 = b[0], b2 = b[1];
  top2_merge(a1, a2, dpp<DPP_XOR1>(a1), dpp<DPP_XOR1>(a2));
  top2_merge(a1, a2, dpp<DPP_XOR2>(a1), dpp<DPP_XOR2>(a2));
  top2_merge(b1, b2, dpp<DPP_XOR1>(b1), dpp<DPP_XOR1>(b2));
  top2_merge(b1, b2, dpp<DPP_XOR2>(b1), dpp<DPP_XOR2>(b2));
  const float ga = (p.topn == 2) ? key_v<W>(a1) + key_v<W>(a2) : key_v<W>(a1);
  const float gb = (p.topn == 2) ? key_v<W>(b1) + key_v<W>(b2) : key_v<W>(b1);
  // unique group keys: score bits above the window start (below 9 * 2^23, a
  // window and one binade more, so three bits to spare), then lower group
  const uint32_t ka = ((__float_as_uint(ga) - KeyWindow<W>::base) << 3) | (uint32_t)(7 - c);
  const uint32_t kb = ((__float_as_uint(gb) - KeyWindow<W>::base) << 3) | (uint32_t)(3 - c);
  int ra, rb;
  group_ranks(ka, kb, ra, rb);
  kept_a = ra < p.TG;
  kept_b = rb < p.TG;
  // certified when the weakest kept group beats the strongest dropped one
  // by more than both error bounds
  const uint32_t ba = __float_as_uint(ga), bb = __float_as_uint(gb);
  const float kmin = __uint_as_float(
      row_min(umin(kept_a ? ba : 0x7F7FFFFFu, kept_b ? bb : 0x7F7FFFFFu)));
  const float dmax = __uint_as_float(row_max(umax(kept_a ? 0u : ba, kept_b ? 0u : bb)));
  return kmin - row_group_err(kmin, sh) > dmax + row_group_err(dmax, sh);
}

// Descending compare-exchange.
__device__ __forceinline__ void cx(uint32_t &x, uint32_t &y) {
  const uint32_t h = umax(x, y), l = umin(x, y);
  x = h;
  y = l;
}

// Sorted top-POOL of the kept pools: a bitonic merge of a (descending) with
// b (descending), keeping the first ten.
__device__ __forceinline__ void merge_kept(const uint32_t (&a)[PP], const uint32_t (&b)[PP],
                                           bool kept_a, bool kept_b, uint32_t (&m)[POOL]) {
  uint32_t h[PP], l[PP];
#pragma unroll
  for (int i = 0; i < PP; ++i) {
    const uint32_t x = kept_a ? a[i] : 0u, y = kept_b ? b[PP - 1 - i] : 0u;
    h[i] = umax(x, y);  // the top 8 of the union, a bitonic sequence
    l[i] = umin(x, y);  // the rest, bitonic, all below h
  }
  cx(h[0], h[4]); cx(h[1], h[5]); cx(h[2], h[6]); cx(h[3], h[7]);
  cx(h[0], h[2]); cx(h[1], h[3]); cx(h[4], h[6]); cx(h[5], h[7]);
  cx(h[0], h[1]); cx(h[2], h[3]); cx(h[4], h[5]); cx(h[6], h[7]);
  cx(l[0], l[4]); cx(l[1], l[5]); cx(l[2], l[6]); cx(l[3], l[7]);
  cx(l[0], l[2]); cx(l[1], l[3]);
  cx(l[0], l[1]);
#pragma unroll
  for (int i = 0; i < PP; ++i) m[i] = h[i];
  m[8] = l[0];
  m[9] = l[1];
}

// top_k + 1 rounds of row maximum over the heads of m (sorted, descending),
// each popping the winning lane's head; returns the last maximum (the
// (top_k+1)-th key).
__device__ __forceinline__ uint32_t extract(const uint32_t (&m)[POOL], int K) {
  uint32_t q[POOL];
#pragma unroll
  for (int i = 0; i < POOL; ++i) q[i] = m[i];
  uint32_t M = 0u;
  for (int rd = 0; rd <= K; ++rd) {
    M = row_max(q[0]);
    const bool won = q[0] == M;
#pragma unroll
    for (int i = 0; i < POOL - 1; ++i) q[i] = won ? q[i + 1] : q[i];
  }
  return M;
}

// LDS byte address of a shared-memory object, and a load from one.
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) uint64_t lds_u64;
__device__ __forceinline__ uint32_t lds_addr(uint32_t *p) {
  return (uint32_t)(uintptr_t)(lds_u32 *)p;
}
__device__ __forceinline__ uint32_t lds_load(uint32_t addr) {
  return *(const lds_u32 *)(uintptr_t)addr;
}

// top_k + 1 rounds of row maximum over the lanes' heads, each lane taking
// the larger head of its two kept pass pools. The pools sit in LDS
// (pool[pass][i][lane], first NSTORE keys, then zero), so a pop advances a
// byte pointer instead of shifting registers; a dropped pass starts at the
// zero sentinel. The lane that wins round rd < K writes (its key, u) to
// win[rd]; ia / ib return the entries taken from each pass. Keys are never
// zero (the slot field is at least 8), so a pointer stops at its sentinel.
// Returns the last maximum (the (top_k+1)-th key).
__device__ __forceinline__ uint32_t tournament(const uint32_t (&a)[PP], const uint32_t (&b)[PP],
                                               bool kept_a, bool kept_b, int K,
                                               uint32_t (*pool)[NSTORE + 1][64], int lane,
                                               uint2 *win, uint2 *sink_row, int u, int &ia,
                                               int &ib) {
#pragma unroll
  for (int i = 0; i < NSTORE; ++i) {
    pool[0][i][lane] = a[i];
    pool[1][i][lane] = b[i];
  }
  pool[0][NSTORE][lane] = 0u;
  pool[1][NSTORE][lane] = 0u;
  // (each lane reads back only its own entries: LDS accesses of a wave stay
  // in order)
  constexpr uint32_t STRIDE = 64 * sizeof(uint32_t);
  const uint32_t pa0 = lds_addr(&pool[0][kept_a ? 0 : NSTORE][lane]);
  const uint32_t pb0 = lds_addr(&pool[1][kept_b ? 0 : NSTORE][lane]);
  uint32_t pa = pa0, pb = pb0;
  uint32_t ha = kept_a ? a[0] : 0u, hb = kept_b ? b[0] : 0u;
  const uint32_t win0 = (uint32_t)(uintptr_t)(lds_u64 *)win;
  const uint32_t sink = (uint32_t)(uintptr_t)(lds_u64 *)&sink_row[lane];
  uint32_t M = 0u;
  for (int rd = 0; rd <= K; ++rd) {
    M = row_max(umax(ha, hb));
    // (a zero head is a sentinel: it never advances, even in a degenerate row
    // whose stored keys all tie and run out before K + 1 rounds)
    const bool ta = ha == M && ha != 0u, tb = hb == M && hb != 0u;
    // every lane stores (no branch): the round's winner to slot rd, the
    // other lanes (and every lane in the last round) to their own sink word
    *(lds_u64 *)(uintptr_t)(((ta || tb) && rd < K) ? win0 + 8u * (uint32_t)rd : sink) =
        ((uint64_t)(uint32_t)u << 32) | M;
    pa = ta ? pa + STRIDE : pa;
    pb = tb ? pb + STRIDE : pb;
    ha = lds_load(pa);
    hb = lds_load(pb);
  }
  ia = (kept_a ? 0 : NSTORE) + (int)((pa - pa0) / STRIDE);
  ib = (kept_b ? 0 : NSTORE) + (int)((pb - pb0) / STRIDE);
  return M;
}

// Row epilogue: lane u of a row whose `out` is set holds slot u's (id, s)
// in sl (lanes u >= K hold nothing). Weights, relabel, pack and stores use
// the same arithmetic in the same order as route_epilogue, so all paths give
// identical bits.
__device__ __forceinline__ void row_outputs(bool out, uint2 sl, const RouteParams &p, int u,
                                            int64_t t, int32_t *__restrict__ ids,
                                            float *__restrict__ wts,
                                            int32_t *__restrict__ packed, int32_t *lid) {
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
    lid[u] = idp;
  }
}

// Row epilogue from binary64 scores: lane u of a row whose `out` is set
// holds slot u's expert and score s, `sum` the row's sum of the K scores.
__device__ __forceinline__ void row_store(bool out, int id, double s, double sum,
                                          const RouteParams &p, int u, int64_t t,
                                          int32_t *__restrict__ ids, float *__restrict__ wts,
                                          int32_t *__restrict__ packed, int32_t *lid) {
  if (out) {
    const float w = (float)(s / sum);
    int idp = id;
    if (p.local) idp = (id >= p.off && id < p.off + p.cnt) ? id - p.off : p.cnt + u;
    const size_t o = (size_t)t * p.K + u;
    ids[o] = id;
    wts[o] = w;
    packed[o] = (int32_t)(((uint32_t)idp << 16) | bf16_rne_bits(w));
    lid[u] = idp;
  }
}


// Number of pool entries (sorted by key) whose value is >= thr.
template <int W>
__device__ __forceinline__ int pool_count_ge(const uint32_t (&pl)[PP], double thr) {
  int n = 0;
#pragma unroll
  for (int i = 0; i < PP; ++i) n += ((double)key_v<W>(pl[i]) >= thr) ? 1 : 0;
  return n;
}

// Exact score (ord key) of expert e.
__device__ __forceinline__ uint32_t exact_key(float x, float b) {
  return ord_f32(sigmoid_rn32(x) + b);
}

// Exact top-2 (ord keys, with multiplicity) of the first na entries of pool
// a and the first nb of pool b, each merged over the quad (the group's four
// lanes). The logits and biases of the first EXACT_PRELOAD entries of both
// pools are loaded together, before any is used, so the usual case costs one
// memory round trip; entries beyond them (rare) follow one by one.
constexpr int EXACT_PRELOAD = 2;
__device__ __forceinline__ void exact_top2_pair(const float *__restrict__ row,
                                                const float *__restrict__ bias_g,
                                                const uint32_t (&a)[PP], int na,
                                                const uint32_t (&b)[PP], int nb, int c, int sub,
                                                uint32_t &ta1, uint32_t &ta2, uint32_t &tb1,
                                                uint32_t &tb2) {
  ta1 = ta2 = tb1 = tb2 = 0u;
  float xa[EXACT_PRELOAD], ya[EXACT_PRELOAD], xb[EXACT_PRELOAD], yb[EXACT_PRELOAD];
#pragma unroll
  for (int i = 0; i < EXACT_PRELOAD; ++i) {  // in-range ids only: expert 0 past n
    const int ea = i < na ? key_expert(a[i], c, sub) : 0;
    const int eb = i < nb ? key_expert(b[i], c, sub) : 0;
    xa[i] = row[ea];
    ya[i] = bias_g[ea];
    xb[i] = row[eb];
    yb[i] = bias_g[eb];
  }
#pragma unroll
  for (int i = 0; i < EXACT_PRELOAD; ++i) {
    if (i < na) {
      const uint32_t o = exact_key(xa[i], ya[i]);
      ta2 = umax(ta2, umin(ta1, o));
      ta1 = umax(ta1, o);
    }
    if (i < nb) {
      const uint32_t o = exact_key(xb[i], yb[i]);
      tb2 = umax(tb2, umin(tb1, o));
      tb1 = umax(tb1, o);
    }
  }
#pragma unroll
  for (int i = EXACT_PRELOAD; i < PP; ++i) {
    if (!__ballot(i < na || i < nb)) break;
    if (i < na) {
      const int e = key_expert(a[i], c, sub);
      const uint32_t o = exact_key(row[e], bias_g[e]);
      ta2 = umax(ta2, umin(ta1, o));
      ta1 = umax(ta1, o);
    }
    if (i < nb) {
      const int e = key_expert(b[i], c, sub);
      const uint32_t o = exact_key(row[e], bias_g[e]);
      tb2 = umax(tb2, umin(tb1, o));
      tb1 = umax(tb1, o);
    }
  }
  top2_merge(ta1, ta2, dpp<DPP_XOR1>(ta1), dpp<DPP_XOR1>(ta2));
  top2_merge(ta1, ta2, dpp<DPP_XOR2>(ta1), dpp<DPP_XOR2>(ta2));
  top2_merge(tb1, tb2, dpp<DPP_XOR1>(tb1), dpp<DPP_XOR1>(tb2));
  top2_merge(tb1, tb2, dpp<DPP_XOR2>(tb1), dpp<DPP_XOR2>(tb2));
}

// Exact refinement of the rows with `need` set (call with the whole wave).
// A row whose group choice the main path could not certify first gets exact
// group scores, from every pool entry that can hold a group's top scores,
// and, when the exactly kept groups differ from the main path's, a new
// extraction over them; the other rows keep the main path's kept groups and
// (top_k+1)-th key M. Then the exact top_k comes from every kept-pool entry
// within twice the key error of M. Both steps
// decide on exact scores, so they only fail when a pool is too short or the
// candidates exceed MAX_CAND. Returns true (row-uniform) when the row has
// been written.
template <int W>
__device__ __forceinline__ bool refine_rows(const float *__restrict__ row,
                                            const float *__restrict__ bias_g,
                                            const uint32_t (&a)[PP], const uint32_t (&b)[PP],
                                            bool need, bool groups_ok, bool kept_a_in,
                                            bool kept_b_in, uint32_t M_in, const RouteParams &p,
                                            int r, int u, int64_t t, RowScratch *L,
                                            int32_t (*tids)[MAX_K],
                                            int32_t *__restrict__ ids, float *__restrict__ wts,
                                            int32_t *__restrict__ packed) {
  const int K = p.K;
  const int c = u >> 2, sub = u & 3;
  constexpr float sh = KeyWindow<W>::shift;
  if (need && u == 0) atomicAdd(&g_refined_tokens, 1ull);
  bool fail = false;
  bool kept_a = kept_a_in, kept_b = kept_b_in;
  uint32_t M = M_in;
  const bool regroup = need && !groups_ok;
  if (__ballot(regroup)) {
    // ---- exact group scores ----------------------------------------------------
    // An expert whose key value is below thr is beaten, even exactly, by the
    // two experts holding its group's approximate top-2 keys.
    uint32_t a1 = a[0], a2 = a[1], b1 = b[0], b2 = b[1];
    top2_merge(a1, a2, dpp<DPP_XOR1>(a1), dpp<DPP_XOR1>(a2));
    top2_merge(a1, a2, dpp<DPP_XOR2>(a1), dpp<DPP_XOR2>(a2));
    top2_merge(b1, b2, dpp<DPP_XOR1>(b1), dpp<DPP_XOR1>(b2));
    top2_merge(b1, b2, dpp<DPP_XOR2>(b1), dpp<DPP_XOR2>(b2));
    const double thra =
        (double)key_v<W>(p.topn == 2 ? a2 : a1) - 2.0 * (double)row_err(key_v<W>(a1), sh);
    const double thrb =
        (double)key_v<W>(p.topn == 2 ? b2 : b1) - 2.0 * (double)row_err(key_v<W>(b1), sh);
    const int na = regroup ? pool_count_ge<W>(a, thra) : 0;
    const int nb = regroup ? pool_count_ge<W>(b, thrb) : 0;
    fail = row_max((na >= PPS || nb >= PPS) ? 1u : 0u) != 0u;
    uint32_t ta1, ta2, tb1, tb2;
    exact_top2_pair(row, bias_g, a, na, b, nb, c, sub, ta1, ta2, tb1, tb2);
    const float gxa = (p.topn == 2) ? ord_inv(ta1) + ord_inv(ta2) : ord_inv(ta1);
    const float gxb = (p.topn == 2) ? ord_inv(tb1) + ord_inv(tb2) : ord_inv(tb1);
    int ra, rb;
    group_ranks(((uint64_t)ord_f32(gxa) << 3) | (uint64_t)(7 - c),
                ((uint64_t)ord_f32(gxb) << 3) | (uint64_t)(3 - c), ra, rb);
    // ---- extraction over the exactly kept groups ------------------------------
    // only for rows whose exactly kept groups differ from the tournament's:
    // over the same groups its last maximum M already is the (top_k+1)-th key
    const bool xa = ra < p.TG, xb = rb < p.TG;
    const bool moved =
        regroup && row_max((xa != kept_a_in || xb != kept_b_in) ? 1u : 0u) != 0u;  // row-uniform
    if (__ballot(moved)) {
      uint32_t m[POOL];
      merge_kept(a, b, xa, xb, m);
      const uint32_t Mx = extract(m, K);
      if (moved) M = Mx;
    }
    if (regroup) {
      kept_a = xa;
      kept_b = xb;
    }
  }

  // ---- exact top_k from the candidates within the error band ----------------------
  const float vm = key_v<W>(M);
  const double thb = (double)vm - 2.0 * (double)row_err(vm, sh);
  const int ca = (need && kept_a) ? pool_count_ge<W>(a, thb) : 0;
  const int cb = (need && kept_b) ? pool_count_ge<W>(b, thb) : 0;
  fail = fail || row_max((ca >= PPS || cb >= PPS) ? 1u : 0u) != 0u;
  const int c2 = ca + cb;
  const int mc = (int)row_sum((uint32_t)c2);
  fail = fail || mc > MAX_CAND || mc < K;
  const int excl = (int)row_exclusive_sum((uint32_t)c2);
#pragma unroll
  for (int i = 0; i < PP; ++i) {
    if (!__ballot(i < ca || i < cb)) break;
    if (i < ca && excl + i < MAX_CAND) L->cand[r][excl + i] = key_expert(a[i], c, sub);
    if (i < cb && excl + ca + i < MAX_CAND)
      L->cand[r][excl + ca + i] = key_expert(b[i], c, sub);
  }
  wave_lds_sync();
  const bool ok_m = need && !fail;
  // candidates u and u + 16 of the row, scored together
  const bool v0 = ok_m && u < mc, v1 = ok_m && u + LANES < mc;
  const int e0 = v0 ? L->cand[r][u] : 0, e1 = v1 ? L->cand[r][u + LANES] : 0;
  float s0, s1;
  sigmoid_rn32_x2(row[e0], row[e1], s0, s1);
  const uint64_t k0 = v0 ? ((uint64_t)ord_f32(s0 + bias_g[e0]) << 32) | (uint64_t)(~(uint32_t)e0)
                         : 0ull;
  const uint64_t k1 = v1 ? ((uint64_t)ord_f32(s1 + bias_g[e1]) << 32) | (uint64_t)(~(uint32_t)e1)
                         : 0ull;
  // ranks by counting the row's larger keys: the lane's other key, then
  // every other lane's two (keys of absent candidates are zero)
  const uint64_t ks[2] = {k0, k1};
  int rk[2] = {k1 > k0 ? 1 : 0, k0 > k1 ? 1 : 0};
  rank_in_row(ks, rk);
  const int rk0 = rk[0], rk1 = rk[1];
  if (v0 && rk0 < K) {
    L->slot[r][rk0] = make_uint2((uint32_t)e0, __float_as_uint(s0));
    if (rk0 == K - 1) L->kth[r] = ord_inv((uint32_t)(k0 >> 32));
  }
  if (v1 && rk1 < K) {
    L->slot[r][rk1] = make_uint2((uint32_t)e1, __float_as_uint(s1));
    if (rk1 == K - 1) L->kth[r] = ord_inv((uint32_t)(k1 >> 32));
  }
  wave_lds_sync();
  // every expert outside the candidates has key value < thb, so an exact
  // score below thb - B + row_err(thb); the K-th winner must beat it (it
  // does whenever the arithmetic above is right; kept as a guard)
  const double bound = thb - (double)sh + (double)row_err((float)thb, sh) * 1.01;
  const bool ok = ok_m && (double)L->kth[r] > bound;
  uint2 sl = make_uint2(0u, 0u);
  if (ok && u < K) sl = L->slot[r][u];
  row_outputs(ok && u < K, sl, p, u, t, ids, wts, packed, tids[r]);
  return ok;
}

// Routes tokens t0 .. t0+3 (rows beyond T are computed on token T-1 and
// discarded); bias_lds holds fl32(b + B) of key window W from stage_bias.
// Returns a 4-bit mask of the rows that must be routed again by the
// one-token-per-wave path; every other valid row has been written.
template <int W>
__device__ __forceinline__ uint32_t route_rows4_post(const uint32_t (&a)[PP],
                                                     const uint32_t (&b)[PP],
                                                     const float *__restrict__ logits,
                                                     const float *__restrict__ bias_g,
                                                     const float *__restrict__ bias_lds, int T,
                                                     int64_t t0, const RouteParams &p, int lane,
                                                     RowScratch *L, int32_t (*tids)[MAX_K],
                                                     int32_t *__restrict__ ids,
                                                     float *__restrict__ wts,
                                                     int32_t *__restrict__ packed) {
  int ln = lane;
  asm volatile("" : "+v"(ln));
  const int r = ln >> 4, u = ln & 15, c = u >> 2;
  const int64_t t = t0 + r;
  const bool valid = t < T;
  const float *row = logits + (size_t)(valid ? t : (int64_t)T - 1) * E;
  const int K = p.K;
  // Issue priority by phase (s_setprio): waves still streaming their rows go
  // first, so every row's loads are in flight early; the selection runs at
  // 1, the stores at 0; a wave that must refine a row goes first again, so
  // that its extra work does not trail the rest of the grid.
  __builtin_amdgcn_s_setprio(1);
  bool kept_a, kept_b;
  const bool groups_ok = approx_groups<W>(a, b, p, c, kept_a, kept_b);  // row-uniform
  bool fail = !groups_ok;
  int ia, ib;
  const uint32_t M =
      tournament(a, b, kept_a, kept_b, K, L->pool, ln, L->win[r], L->sink, u, ia, ib);
  const int pops = (kept_a ? ia : 0) + (kept_b ? ib : 0);
  // a pass whose pool was taken whole may hide further keys above M
  fail = fail || (kept_a && ia == PP) || (kept_b && ib == PP);
  // exactly K+1 entries taken (no equal keys)
  fail = fail || row_sum((uint32_t)pops) != (uint32_t)(K + 1);
  wave_lds_sync();

  // ---- slot order, boundary and weights from the approximate keys -------------------
  // Lane u < K takes the winner of round u; rounds pop keys in descending
  // order. |v - (sp + B)| <= row_err(v) for every key value v, so when
  //  * every winner's value beats the next one's (the K-th winner's: M's) by
  //    more than both errors, the exact (sp desc, id asc) order is the round
  //    order and no other expert reaches the K-th exact score;
  // the slots are certified. Weights: the key holds v = fl32(s~ + fl32(b+B)),
  // so v - fl32(b+B) (exact in binary64) is within e = FAST_SIG_ERR_TESTED +
  // ulp(v)/2 of the exact score s; w = s_k / sum s then moves by at most
  // e_k/(s_k - e_k) + sum e/(sum s - sum e) relative, and two binary32
  // roundings. A row is finished here when that stays within 0.9e-6 for every
  // slot (inside the 1e-6 tolerance on weights); otherwise its winners are
  // scored exactly below.
  const uint32_t pre_fail = row_max((fail && valid) ? 1u : 0u);
  const bool act = pre_fail == 0u && valid && u < K;
  constexpr float sh = KeyWindow<W>::shift;
  int my_id = 0;
  double my_s = 0.0, my_e = 0.0;
  bool ok = true;
  if (act) {
    const uint2 w = L->win[r][u];  // winner of round u: key and the lane holding it
    // (every round of a row that took K + 1 keys had a winner, so w is this
    // row's; the clamp only keeps the index inside the row)
    my_id = min(key_expert(w.x, (int)(w.y >> 2) & 3, (int)(w.y & 3)), E - 1);
    const float v = key_v<W>(w.x);
    const float vn = u + 1 < K ? key_v<W>(L->win[r][u + 1].x) : key_v<W>(M);
    ok = (double)v - (double)row_err(v, sh) > (double)vn + (double)row_err(vn, sh);
    my_s = (double)v - (double)bias_lds[my_id];
    my_e = (double)FAST_SIG_ERR_TESTED + 0.5 * (double)ulp32(v);
  }
  const double S = row_sum_f64(my_s), Se = row_sum_f64(my_e);
  // e_k / (s_k - e_k) + Se / (S - Se) + 2^-23 + 2^-40 <= 0.9e-6, multiplied
  // through by the two positive denominators (the 2^-40 term also covers the
  // binary64 rounding of this check)
  if (act) {
    const double A = my_s - my_e, B = S - Se;
    ok = ok && my_s > 2.0 * my_e && S > 2.0 * Se &&
         my_e * B + Se * A + (0x1p-23 + 0x1p-40) * (A * B) <= 0.9e-6 * (A * B);
  }
  const bool approx_ok = pre_fail == 0u && row_min((act && !ok) ? 0u : 1u) != 0u;  // row-uniform
  __builtin_amdgcn_s_setprio(0);
  row_store(approx_ok && act, my_id, my_s, S, p, u, t, ids, wts, packed, tids[r]);
  bool done = approx_ok || !valid;

  // ---- rows the keys cannot settle: exact scores of the same winners ----------------
  const bool need_exact = valid && pre_fail == 0u && !approx_ok;  // row-uniform
  if (__ballot(need_exact)) {
    const bool ex = need_exact && u < K;
    float es = 0.0f, esp = 0.0f;
    uint64_t ek[1] = {0ull};  // (exact score, lower id first); zero off the winners
    if (ex) {
      es = sigmoid_rn32(row[my_id]);
      esp = es + bias_g[my_id];
      ek[0] = ((uint64_t)ord_f32(esp) << 32) | (uint64_t)(~(uint32_t)my_id);
    }
    // every expert outside the winners has a key below M: its exact score is
    // at most key_v(M) - B + row_err(key_v(M)); the weakest winner must beat it
    const float vm = key_v<W>(M);
    const double bound = (double)vm - (double)sh + (double)row_err(vm, sh);
    const uint32_t weakest = row_min(ex ? ord_f32(esp) : 0xFFFFFFFFu);
    const bool boundary_ok = (double)ord_inv(weakest) > bound;
    int rk[1] = {0};
    rank_in_row(ek, rk);
    const int rank = rk[0];
    const bool exact_ok = need_exact && boundary_ok;
    if (exact_ok && ex) L->slot[r][rank] = make_uint2((uint32_t)my_id, __float_as_uint(es));
    wave_lds_sync();
    uint2 sl = make_uint2(0u, 0u);
    if (exact_ok && u < K) sl = L->slot[r][u];
    row_outputs(exact_ok && u < K, sl, p, u, t, ids, wts, packed, tids[r]);
    done = done || exact_ok;
  }

  // ---- rows whose certificate failed: exact refinement -------------------------
  const bool need = !done && valid;
  if (__ballot(need)) {
    __builtin_amdgcn_s_setprio(3);
    wave_lds_sync();
    done = refine_rows<W>(row, bias_g, a, b, need, groups_ok, kept_a, kept_b, M, p, r, u, t, L, tids,
                          ids,
                       wts, packed) ||
           done;
  }
  // rows to route again
  const uint64_t fb = __ballot(!done && valid && u == 0);
  return (uint32_t)((fb & 1ull) | ((fb >> 15) & 2ull) | ((fb >> 30) & 4ull) | ((fb >> 45) & 8ull));
}

}  // namespace rows
}  // namespace moe
