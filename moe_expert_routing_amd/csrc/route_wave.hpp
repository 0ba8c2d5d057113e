// route_wave.hpp - one wavefront routes one token (gfx950, wave64).
//
// Steps, in the order of the method (a sigmoid router with a correction bias
// and a grouped top-k: "[ROCm][Perf] Kimi-K3: token-sharded residual stream
// for long prefills", author's reply on shard-routed test coverage; packed
// ids and the rank-local pack epilogue: "[kimi-k3] Rank-local expert ids for
// the EP routed MoE (upstream #45544)", commit message):
//   s  = RN32(sigma(logit))                 (exact, rn_sigmoid.hpp)
//   sp = fl32(s + bias)                      selection key only
//   group score = fl32 sum of the group's top `group_topn` sp
//   keep the topk_group best groups          ties -> lower group index
//   top_k experts of the kept groups         by (sp desc, id asc)
//   w_k = s_k / sum_j s_j                    binary64, rounded to binary32
//   packed = (id' << 16) | bf16_rne(w)       id' = rank-local id if relabelled
//
// Lane layout. Lane l belongs to group g = l / LPG (LPG = 64 / G lanes per
// group) and holds 2*NP experts of that group as NP float2 pairs:
//   e(i, j) = g*Eg + 2*(l % LPG) + 2*LPG*i + j,   i < NP, j < 2,
// so every load instruction of the wave reads 8-byte pieces that tile whole
// 64-byte segments, and group reductions stay inside LPG adjacent lanes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rn_sigmoid.hpp"

namespace moe {

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

// Bias in the lane layout (loaded once per wave, reused for every token).
template <int NP>
__device__ __forceinline__ void load_lane_layout(const float *__restrict__ v, const RouteParams &p,
                                                 int lane, float (&out)[2 * NP]) {
  const int g = lane >> p.lpg_log2;
  const int sub = lane & (p.lpg - 1);
  const float *base = v + g * p.eg + 2 * sub;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const float2 q = *reinterpret_cast<const float2 *>(base + 2 * p.lpg * i);
    out[2 * i] = q.x;
    out[2 * i + 1] = q.y;
  }
}

// Routes token t (row = logits + t*E). Lanes 0..K-1 write slot k = lane of
// topk_ids / topk_weights / packed and return the output id id'; other lanes
// return -1. Must be called by all 64 lanes of the wave.
template <int NP>
__device__ __forceinline__ int route_token_wave(const float *__restrict__ row,
                                                const float (&bias)[2 * NP],
                                                const RouteParams &p, int lane, int64_t t,
                                                int32_t *__restrict__ ids,
                                                float *__restrict__ wts,
                                                int32_t *__restrict__ packed) {
  constexpr int M = 2 * NP;
  float x[M];
  load_lane_layout<NP>(row, p, lane, x);
  const int g = lane >> p.lpg_log2;
  const int e0 = g * p.eg + 2 * (lane & (p.lpg - 1));

  float sp[M];
#pragma unroll
  for (int j = 0; j < M; ++j) sp[j] = sigmoid_rn32(x[j]) + bias[j];

  // Top two biased scores of the group, with multiplicity.
  float m1 = -__builtin_inff(), m2 = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < M; ++j) {
    m2 = fmaxf(m2, fminf(m1, sp[j]));
    m1 = fmaxf(m1, sp[j]);
  }
  for (int d = 1; d < p.lpg; d <<= 1) {
    const float q1 = __shfl_xor(m1, d);
    const float q2 = __shfl_xor(m2, d);
    const float n2 = fmaxf(fminf(m1, q1), fmaxf(m2, q2));
    m1 = fmaxf(m1, q1);
    m2 = n2;
  }
  const float gs = (p.topn == 2) ? (m1 + m2) : m1;

  // Rank of this lane's group: groups with a larger score, or an equal score
  // and a lower index, come first.
  int rank = 0;
  for (int gg = 0; gg < p.G; ++gg) {
    const float o = __shfl(gs, gg << p.lpg_log2);
    rank += (o > gs) || (o == gs && gg < g);
  }
  const bool kept = rank < p.TG;

  // Key: ordered sp in the high word, ~id in the low word, so the maximum
  // key is the best (sp desc, id asc) candidate. Dropped groups get 0.
  uint64_t key[M];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t e = (uint32_t)(e0 + 2 * p.lpg * i + j);
      key[2 * i + j] = kept ? (((uint64_t)ord_f32(sp[2 * i + j]) << 32) | (uint64_t)(~e)) : 0ull;
    }
  }
  int my_id = 0;
  for (int r = 0; r < p.K; ++r) {
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < M; ++j) best = umax64(best, key[j]);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) best = umax64(best, __shfl_xor(best, d));
    if (lane == r) my_id = (int)(~(uint32_t)best);
#pragma unroll
    for (int j = 0; j < M; ++j) key[j] = (key[j] == best) ? 0ull : key[j];
  }

  // Weights: unbiased s of the selected experts over their binary64 sum.
  float s_sel = 0.0f;
  if (lane < p.K) s_sel = sigmoid_rn32(row[my_id]);
  double sum = (lane < p.K) ? (double)s_sel : 0.0;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) sum += __shfl_xor(sum, d);

  int idp = -1;
  if (lane < p.K) {
    const float w = (float)((double)s_sel / sum);
    idp = my_id;
    if (p.local) idp = (my_id >= p.off && my_id < p.off + p.cnt) ? my_id - p.off : p.cnt + lane;
    const size_t o = (size_t)t * p.K + lane;
    ids[o] = my_id;
    wts[o] = w;
    packed[o] = (int32_t)(((uint32_t)idp << 16) | bf16_rne_bits(w));
  }
  return idp;
}

}  // namespace moe
