// moe_route.hip - routing kernels for gfx950 and the C ABI of include/moe_route.h.
//
// Paths (both give identical results):
//  * decode, T <= 64: ONE launch. Blocks of 4 waves route one token per wave
//    and publish their outputs; the last block to arrive (ticket in the
//    workspace control block) builds counts, offsets and the permutation from
//    per-expert 64-bit token masks in LDS.
//  * prefill, T > 64: four launches.
//      route_tokens: one token per wave, waves independent (no barriers), so
//                    the per-token latency is hidden by occupancy alone.
//      tile_count:   tiles of 64 tokens: a 64-bit token mask per output id in
//                    LDS gives the tile histogram hist[e'][tile] and each
//                    entry's rank among the tile's entries of the same id.
//      tile_prefix:  per output id, exclusive scan of hist[e'][:] over tiles;
//                    total -> counts[e'].
//      scatter:      offsets = exclusive scan of counts; each entry goes to
//                    offsets[e'] + hist[e'][tile] + rank_in_tile.
// Within one token the output ids are distinct (top-k ids are distinct and
// the relabelled ids are unique per row), so "ascending flat index within an
// expert" is "ascending token", and a token's position among the entries of
// an id is a popcount of the id's token mask below it.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "../../include/moe_route.h"
#include "internal.hpp"
#include "route_rows.hpp"
#include "route_wave.hpp"

static_assert(moe::kMaxTopK == MOE_ROUTE_MAX_TOPK, "top-k capacity");

namespace moe {

constexpr int WAVES_PER_BLOCK = 4;
constexpr int BLOCK = 64 * WAVES_PER_BLOCK;
constexpr size_t CONTROL_BYTES = 256;
// Prefill tiles of the permutation: 64 tokens (token masks are 64-bit).
constexpr int TILE_TOKENS = 64;

// Exclusive scan of in[0..n) (n <= 1024, any memory) into out[0..n] in LDS,
// out[n] = total. All BLOCK threads must call it.
__device__ void block_exclusive_scan(const int32_t *in, int n, int32_t *out, int32_t *wave_tot) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  int v[4];
  int s = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int idx = tid * 4 + k;
    v[k] = idx < n ? in[idx] : 0;
    s += v[k];
  }
  int incl = s;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wave_tot[wv] = incl;
  __syncthreads();
  int wave_off = 0;
  for (int w = 0; w < wv; ++w) wave_off += wave_tot[w];
  int run = wave_off + incl - s;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int idx = tid * 4 + k;
    if (idx < n) out[idx] = run;
    run += v[k];
  }
  if (tid == BLOCK - 1) out[n] = wave_off + incl;
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Decode path: one launch for T <= 64.
// ---------------------------------------------------------------------------
template <int NP, int LPG>
__global__ __launch_bounds__(BLOCK) void route_decode_kernel(
    const float *__restrict__ logits, const float *__restrict__ bias, int T, RouteParams p,
    int32_t *__restrict__ ids, float *__restrict__ wts, int32_t *__restrict__ packed,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets, int32_t *__restrict__ perm,
    int32_t *__restrict__ inv, uint32_t *__restrict__ ticket) {
  __shared__ unsigned long long mask[MOE_ROUTE_MAX_EXPERTS];
  __shared__ int32_t offs[MOE_ROUTE_MAX_EXPERTS + 1];
  __shared__ int32_t wave_tot[WAVES_PER_BLOCK];
  __shared__ WaveScratch scratch[WAVES_PER_BLOCK];
  __shared__ int is_last;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int t = blockIdx.x * WAVES_PER_BLOCK + wave;
  if (t < T) {
    const float *row = logits + (size_t)t * p.E;
    float b[2 * NP], x[2 * NP];
    load_lane_layout<NP, LPG>(row, p, lane, x);
    load_lane_layout<NP, LPG>(bias, p, lane, b);
    route_token<NP, LPG>(row, x, b, bias, p, lane, t, &scratch[wave], ids, wts, packed);
  }
  // Publish this block's outputs, then take a ticket.
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) is_last = (atomicAdd(ticket, 1u) == gridDim.x - 1u);
  __syncthreads();
  if (!is_last) return;
  __threadfence();

  const int n = T * p.K;
  for (int i = threadIdx.x; i < p.e_out; i += BLOCK) mask[i] = 0ull;
  __syncthreads();
  for (int f = threadIdx.x; f < n; f += BLOCK) {
    const int e = packed[f] >> 16;
    atomicOr(&mask[e], 1ull << (f / p.K));
  }
  __syncthreads();
  for (int i = threadIdx.x; i < p.e_out; i += BLOCK) {
    const int c = __popcll(mask[i]);
    offs[i] = c;
    counts[i] = c;
  }
  __syncthreads();
  block_exclusive_scan(offs, p.e_out, offs, wave_tot);  // in place: reads precede writes
  for (int i = threadIdx.x; i <= p.e_out; i += BLOCK) offsets[i] = offs[i];
  for (int f = threadIdx.x; f < n; f += BLOCK) {
    const int e = packed[f] >> 16;
    const int tok = f / p.K;
    const int pos = offs[e] + __popcll(mask[e] & ((1ull << tok) - 1ull));
    perm[pos] = f;
    if (inv) inv[f] = pos;
  }
  if (threadIdx.x == 0) *ticket = 0u;  // leave the control block zeroed
}

// ---------------------------------------------------------------------------
// Prefill path, kernel 1: route tiles of 64 tokens.
// ---------------------------------------------------------------------------
template <int NP, int LPG>
__global__ __launch_bounds__(BLOCK) void route_tokens_kernel(
    const float *__restrict__ logits, const float *__restrict__ bias, int T, RouteParams p,
    int32_t *__restrict__ ids, float *__restrict__ wts, int32_t *__restrict__ packed) {
  __shared__ WaveScratch scratch[WAVES_PER_BLOCK];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int t = blockIdx.x * WAVES_PER_BLOCK + wave;
  if (t >= T) return;
  const float *row = logits + (size_t)t * p.E;
  float b[2 * NP], x[2 * NP];
  load_lane_layout<NP, LPG>(row, p, lane, x);
  load_lane_layout<NP, LPG>(bias, p, lane, b);
  route_token<NP, LPG>(row, x, b, bias, p, lane, t, &scratch[wave], ids, wts, packed);
}

// Prefill path, kernel 1 for the 896-expert, 8-group shape: four tokens per
// wave (route_rows.hpp); rows that fail their certificate are routed again
// one token per wave.
__device__ unsigned long long g_row_fallback_tokens = 0ull;

__global__ __launch_bounds__(BLOCK, 8) void route_rows_kernel(
    const float *__restrict__ logits, const float *__restrict__ bias, int T, RouteParams p,
    int32_t *__restrict__ ids, float *__restrict__ wts, int32_t *__restrict__ packed) {
  __shared__ float bias_lds[rows::E];
  __shared__ union {
    rows::RowScratch r;
    WaveScratch w;
  } scratch[WAVES_PER_BLOCK];
  __shared__ int bad_bias;
  const bool ok = rows::stage_bias<BLOCK>(bias, bias_lds, &bad_bias);  // all threads, before any exit
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int64_t t0 = ((int64_t)blockIdx.x * WAVES_PER_BLOCK + wave) * 4;
  if (t0 >= T) return;
  uint32_t redo = 0xFu;
  if (ok)
    redo = rows::route_rows4(logits, bias, bias_lds, T, t0, p, lane, &scratch[wave].r, ids, wts,
                             packed);
  redo = (uint32_t)__builtin_amdgcn_readfirstlane((int)redo);
  while (redo) {
    const int r = __builtin_ctz(redo);
    redo &= redo - 1u;
    const int64_t t = t0 + r;
    if (t >= T) break;
    if (lane == 0) atomicAdd(&g_row_fallback_tokens, 1ull);
    const float *row = logits + (size_t)t * p.E;
    float b[14], x[14];
    load_lane_layout<7, 8>(row, p, lane, x);
    load_lane_layout<7, 8>(bias, p, lane, b);
    route_token<7, 8>(row, x, b, bias, p, lane, t, &scratch[wave].w, ids, wts, packed,
                      /*fast_first=*/false);
  }
}

// Prefill path, kernel 1b: per tile of TILE_TOKENS tokens, a 64-bit token
// mask per output id (in LDS) gives the tile histogram hist[e'][tile] and
// each entry's rank among the tile's entries of the same id.
__global__ __launch_bounds__(BLOCK) void tile_count_kernel(const int32_t *__restrict__ packed,
                                                           int T, int K, int e_out,
                                                           int32_t *__restrict__ hist, int ntiles,
                                                           int32_t *__restrict__ tile_rank) {
  __shared__ unsigned long long mask[MOE_ROUTE_MAX_EXPERTS];
  const int tile = blockIdx.x;
  const int nt = min(TILE_TOKENS, T - tile * TILE_TOKENS);
  const int n = nt * K;
  const int32_t *pk = packed + (size_t)tile * TILE_TOKENS * K;
  for (int i = threadIdx.x; i < e_out; i += BLOCK) mask[i] = 0ull;
  __syncthreads();
  for (int q = threadIdx.x; q < n; q += BLOCK) atomicOr(&mask[pk[q] >> 16], 1ull << (q / K));
  __syncthreads();
  for (int i = threadIdx.x; i < e_out; i += BLOCK)
    hist[(size_t)i * ntiles + tile] = __popcll(mask[i]);
  int32_t *tr = tile_rank + (size_t)tile * TILE_TOKENS * K;
  for (int q = threadIdx.x; q < n; q += BLOCK)
    tr[q] = __popcll(mask[pk[q] >> 16] & ((1ull << (q / K)) - 1ull));
}

// Prefill path, kernel 2: per output id, exclusive scan over tiles (in
// place) and the id's total -> counts. One block per id; each thread scans a
// contiguous run of PREFIX_RUN tiles, so a wave reads 2 KB contiguously.
constexpr int PREFIX_RUN = 8;
__global__ __launch_bounds__(BLOCK) void tile_prefix_kernel(int32_t *__restrict__ hist, int ntiles,
                                                            int32_t *__restrict__ counts) {
  __shared__ int32_t wave_tot[WAVES_PER_BLOCK];
  int32_t *row = hist + (size_t)blockIdx.x * ntiles;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int carry = 0;
  for (int base = 0; base < ntiles; base += BLOCK * PREFIX_RUN) {
    const int beg = base + tid * PREFIX_RUN;
    int v[PREFIX_RUN];
    int s = 0;
#pragma unroll
    for (int k = 0; k < PREFIX_RUN; ++k) {
      v[k] = (beg + k < ntiles) ? row[beg + k] : 0;
      s += v[k];
    }
    int incl = s;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d);
      if (lane >= d) incl += o;
    }
    if (lane == 63) wave_tot[wv] = incl;
    __syncthreads();
    int off = carry;
    int total = 0;
#pragma unroll
    for (int w = 0; w < WAVES_PER_BLOCK; ++w) {
      if (w < wv) off += wave_tot[w];
      total += wave_tot[w];
    }
    int run = off + incl - s;
#pragma unroll
    for (int k = 0; k < PREFIX_RUN; ++k) {
      if (beg + k < ntiles) row[beg + k] = run;
      run += v[k];
    }
    carry += total;
    __syncthreads();
  }
  if (tid == 0) counts[blockIdx.x] = carry;
}

// Prefill path, kernel 3: scatter every entry to its expert-major position.
__global__ __launch_bounds__(BLOCK) void scatter_kernel(
    const int32_t *__restrict__ packed, const int32_t *__restrict__ tile_rank,
    const int32_t *__restrict__ hist, int ntiles, const int32_t *__restrict__ counts, int e_out,
    int64_t n, int K, int tile_tokens, int32_t *__restrict__ offsets,
    int32_t *__restrict__ perm, int32_t *__restrict__ inv) {
  __shared__ int32_t offs[MOE_ROUTE_MAX_EXPERTS + 1];
  __shared__ int32_t wave_tot[WAVES_PER_BLOCK];
  block_exclusive_scan(counts, e_out, offs, wave_tot);
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= e_out; i += BLOCK) offsets[i] = offs[i];
  for (int64_t f = (int64_t)blockIdx.x * BLOCK + threadIdx.x; f < n;
       f += (int64_t)gridDim.x * BLOCK) {
    const int e = packed[f] >> 16;
    const int tile = (int)((f / K) / tile_tokens);
    const int pos = offs[e] + hist[(size_t)e * ntiles + tile] + tile_rank[f];
    perm[pos] = (int32_t)f;
    if (inv) inv[f] = pos;
  }
}

// Diagnostic sigmoid kernel.
__global__ void sigmoid_kernel(const float *__restrict__ x, float *__restrict__ y, int64_t n,
                               int mode) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    y[i] = mode == 1 ? sigmoid_rn32_dd(x[i]) : (mode == 2 ? fast_sigmoid(x[i]) : sigmoid_rn32(x[i]));
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static int ilog2_exact(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return (1 << l) == v ? l : -1;
}

static int validate_params(const moe_route_params *prm) {
  if (!prm) return MOE_ERR_NULL;
  const int E = prm->num_experts, G = prm->n_groups, TG = prm->topk_group, K = prm->top_k,
            N = prm->group_topn;
  if (E <= 0 || G <= 0 || TG <= 0 || K <= 0 || N <= 0) return MOE_ERR_SHAPE;
  if (E % G != 0 || TG > G || N > E / G || K > TG * (E / G)) return MOE_ERR_SHAPE;
  if (E > MOE_ROUTE_MAX_EXPERTS || E % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (G > 64 || ilog2_exact(G) < 0) return MOE_ERR_UNSUPPORTED;
  if (K > MOE_ROUTE_MAX_TOPK || N > 2) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

static int ntiles_for(int T) { return (T + TILE_TOKENS - 1) / TILE_TOKENS; }

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

static int cu_count();

// Benchmark hook (moe_route_set_kernel_events).
static hipEvent_t g_ev_before = nullptr, g_ev_after = nullptr;

static size_t route_ws_bytes(int T, int e_out, int K) {
  size_t b = CONTROL_BYTES;
  if (T > MOE_ROUTE_MAX_FUSED_TOKENS) {
    b += align256((size_t)e_out * ntiles_for(T) * sizeof(int32_t));
    b += align256((size_t)T * K * sizeof(int32_t));
  }
  return b;
}

// The four-tokens-per-wave path: 896 experts in 8 groups, top_k <= 16, and
// kept lanes whose pools (6 usable keys each) can hold top_k + 1 entries;
// float4 loads need 16-byte aligned rows.
static bool rows_path_applies(const RouteParams &rp, const float *logits) {
  return rp.E == rows::E && rp.G == rows::G && rp.K <= rows::MAX_K &&
         12 * rp.TG >= rp.K + 1 && ((uintptr_t)logits % 16) == 0;
}

template <int NP, int LPG>
static hipError_t launch_route(const float *logits, const float *bias, int T, const RouteParams &rp,
                               const moe_route_outputs *o, char *ws, hipStream_t st) {
  if (T <= MOE_ROUTE_MAX_FUSED_TOKENS) {
    const int grid = T > 0 ? (T + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK : 1;
    if (g_ev_before) hipEventRecord(g_ev_before, st);
    route_decode_kernel<NP, LPG><<<grid, BLOCK, 0, st>>>(logits, bias, T, rp, o->topk_ids,
                                                     o->topk_weights, o->packed, o->counts,
                                                     o->offsets, o->perm, o->inv_perm,
                                                     reinterpret_cast<uint32_t *>(ws));
    if (g_ev_after) hipEventRecord(g_ev_after, st);
    return hipGetLastError();
  }
  const int ntiles = ntiles_for(T);
  int32_t *hist = reinterpret_cast<int32_t *>(ws + CONTROL_BYTES);
  int32_t *tile_rank = reinterpret_cast<int32_t *>(
      ws + CONTROL_BYTES + align256((size_t)rp.e_out * ntiles * sizeof(int32_t)));
  const int cus = cu_count();
  if (g_ev_before) hipEventRecord(g_ev_before, st);
  if (LPG == 8 && NP == 7 && rows_path_applies(rp, logits)) {
    const int nblk = (T + 4 * WAVES_PER_BLOCK - 1) / (4 * WAVES_PER_BLOCK);
    route_rows_kernel<<<nblk, BLOCK, 0, st>>>(logits, bias, T, rp, o->topk_ids, o->topk_weights,
                                              o->packed);
  } else {
    const int nblk = (T + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK;
    route_tokens_kernel<NP, LPG><<<nblk, BLOCK, 0, st>>>(logits, bias, T, rp, o->topk_ids,
                                                     o->topk_weights, o->packed);
  }
  if (g_ev_after) hipEventRecord(g_ev_after, st);
  tile_count_kernel<<<ntiles, BLOCK, 0, st>>>(o->packed, T, rp.K, rp.e_out, hist, ntiles,
                                              tile_rank);
  tile_prefix_kernel<<<rp.e_out, BLOCK, 0, st>>>(hist, ntiles, o->counts);
  const int64_t n = (int64_t)T * rp.K;
  int64_t g3 = (n + BLOCK * 4 - 1) / (BLOCK * 4);
  if (g3 > 8 * cus) g3 = 8 * cus;
  scatter_kernel<<<(int)g3, BLOCK, 0, st>>>(o->packed, tile_rank, hist, ntiles, o->counts,
                                            rp.e_out, n, rp.K, TILE_TOKENS, o->offsets,
                                            o->perm, o->inv_perm);
  return hipGetLastError();
}

int validate_route_call(const float *logits, const float *bias, int32_t T,
                        const moe_route_params *prm, int32_t off, int32_t cnt,
                        const moe_route_outputs *o, const void *workspace, size_t ws_bytes,
                        int *e_out) {
  int st = validate_params(prm);
  if (st != MOE_OK) return st;
  if (!o) return MOE_ERR_NULL;
  if (T < 0) return MOE_ERR_SHAPE;
  if (!o->counts || !o->offsets) return MOE_ERR_NULL;
  if (T > 0 && (!logits || !bias || !o->topk_ids || !o->topk_weights || !o->packed || !o->perm))
    return MOE_ERR_NULL;
  const int32_t e_local = moe_route_local_num_experts(prm->num_experts, prm->top_k, off, cnt);
  if (e_local < 0) return e_local;
  const int eo = e_local > 0 ? e_local : prm->num_experts;
  if (!workspace) return MOE_ERR_WORKSPACE;
  if (ws_bytes < route_ws_bytes(T, eo, prm->top_k)) return MOE_ERR_WORKSPACE;
  if ((uintptr_t)workspace % 8 != 0) return MOE_ERR_WORKSPACE;
  if ((uintptr_t)logits % 8 != 0 || (uintptr_t)bias % 8 != 0) return MOE_ERR_SHAPE;
  if (e_out) *e_out = eo;
  return MOE_OK;
}

static int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int cus = 0;
    hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    cached[dev] = cus > 0 ? cus : 256;
  }
  return cached[dev];
}

static int route_impl(const float *logits, const float *bias, int32_t T,
                      const moe_route_params *prm, int32_t off, int32_t cnt,
                      const moe_route_outputs *o, void *workspace, size_t ws_bytes,
                      void *stream) {
  int e_out = 0;
  const int st = validate_route_call(logits, bias, T, prm, off, cnt, o, workspace, ws_bytes,
                                     &e_out);
  if (st != MOE_OK) return st;
  RouteParams rp;
  rp.E = prm->num_experts;
  rp.G = prm->n_groups;
  rp.TG = prm->topk_group;
  rp.K = prm->top_k;
  rp.topn = prm->group_topn;
  rp.lpg = 64 / rp.G;
  rp.lpg_log2 = ilog2_exact(rp.lpg);
  rp.eg = rp.E / rp.G;
  rp.off = off;
  rp.cnt = cnt;
  rp.local = e_out != rp.E ? 1 : 0;
  rp.e_out = e_out;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char *ws = reinterpret_cast<char *>(workspace);
  hipError_t err;
  // the 896-expert, 8-group shape gets constant lanes per group
  if (rp.E == 896 && rp.lpg == 8) {
    err = launch_route<7, 8>(logits, bias, T, rp, o, ws, s);
    return err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
  }
  switch (rp.E / 128) {
    case 1: err = launch_route<1, 0>(logits, bias, T, rp, o, ws, s); break;
    case 2: err = launch_route<2, 0>(logits, bias, T, rp, o, ws, s); break;
    case 3: err = launch_route<3, 0>(logits, bias, T, rp, o, ws, s); break;
    case 4: err = launch_route<4, 0>(logits, bias, T, rp, o, ws, s); break;
    case 5: err = launch_route<5, 0>(logits, bias, T, rp, o, ws, s); break;
    case 6: err = launch_route<6, 0>(logits, bias, T, rp, o, ws, s); break;
    case 7: err = launch_route<7, 0>(logits, bias, T, rp, o, ws, s); break;
    case 8: err = launch_route<8, 0>(logits, bias, T, rp, o, ws, s); break;
    default: return MOE_ERR_UNSUPPORTED;
  }
  return err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe

extern "C" {

int32_t moe_route_abi_version(void) { return 100; }

const char *moe_route_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "invalid or inconsistent shape";
    case MOE_ERR_RANGE: return "expert range outside [0, num_experts)";
    case MOE_ERR_UNSUPPORTED: return "parameters outside the kernels' envelope";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int32_t moe_route_local_num_experts(int32_t num_experts, int32_t top_k,
                                    int32_t local_expert_offset, int32_t num_local_experts) {
  if (num_experts <= 0 || top_k <= 0) return MOE_ERR_SHAPE;
  const int64_t off = local_expert_offset, cnt = num_local_experts;
  if (off < 0 || cnt < 0 || off + cnt > num_experts) return MOE_ERR_RANGE;
  if (cnt == 0 || cnt >= num_experts) return 0;
  const int64_t e_out = ((cnt + top_k + 3) / 4) * 4;
  return e_out < num_experts ? (int32_t)e_out : 0;
}

size_t moe_route_workspace_bytes(int32_t num_tokens, int32_t num_experts_out, int32_t top_k) {
  if (num_tokens < 0 || num_experts_out <= 0 || top_k <= 0) return 0;
  return moe::route_ws_bytes(num_tokens, num_experts_out, top_k);
}

int moe_route(const float *logits, const float *bias, int32_t num_tokens,
              const moe_route_params *params, const moe_route_outputs *out, void *workspace,
              size_t workspace_bytes, void *stream) {
  return moe::route_impl(logits, bias, num_tokens, params, 0, 0, out, workspace,
                         workspace_bytes, stream);
}

int moe_route_local(const float *logits, const float *bias, int32_t num_tokens,
                    const moe_route_params *params, int32_t local_expert_offset,
                    int32_t num_local_experts, const moe_route_outputs *out, void *workspace,
                    size_t workspace_bytes, void *stream) {
  return moe::route_impl(logits, bias, num_tokens, params, local_expert_offset,
                         num_local_experts, out, workspace, workspace_bytes, stream);
}

int64_t moe_route_exact_path_tokens(int32_t reset) {
  unsigned long long v = 0;
  if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(moe::g_exact_path_tokens), sizeof(v)) != hipSuccess)
    return MOE_ERR_HIP;
  if (reset) {
    const unsigned long long z = 0;
    if (hipMemcpyToSymbol(HIP_SYMBOL(moe::g_exact_path_tokens), &z, sizeof(z)) != hipSuccess)
      return MOE_ERR_HIP;
  }
  return (int64_t)v;
}

int64_t moe_route_path_tokens(int32_t path, int32_t reset) {
  unsigned long long *sym = nullptr;
  switch (path) {
    case 0: return moe_route_exact_path_tokens(reset);
    case 1: sym = &moe::rows::g_refined_tokens; break;
    case 2: sym = &moe::g_row_fallback_tokens; break;
    default: return MOE_ERR_UNSUPPORTED;
  }
  unsigned long long v = 0ull;
  if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(*sym), sizeof(v)) != hipSuccess) return MOE_ERR_HIP;
  if (reset) {
    const unsigned long long z = 0ull;
    if (hipMemcpyToSymbol(HIP_SYMBOL(*sym), &z, sizeof(z)) != hipSuccess) return MOE_ERR_HIP;
  }
  return (int64_t)v;
}

int moe_route_set_kernel_events(void *before, void *after) {
  if ((before == nullptr) != (after == nullptr)) return MOE_ERR_NULL;
  moe::g_ev_before = reinterpret_cast<hipEvent_t>(before);
  moe::g_ev_after = reinterpret_cast<hipEvent_t>(after);
  return MOE_OK;
}

int moe_sigmoid_rn32(const float *x, float *y, int64_t n, int32_t mode, void *stream) {
  if (n < 0) return MOE_ERR_SHAPE;
  if (n == 0) return MOE_OK;
  if (!x || !y) return MOE_ERR_NULL;
  if (mode < 0 || mode > 2) return MOE_ERR_UNSUPPORTED;
  int64_t grid = (n + 255) / 256;
  if (grid > 65536) grid = 65536;
  moe::sigmoid_kernel<<<(int)grid, 256, 0, reinterpret_cast<hipStream_t>(stream)>>>(x, y, n, mode);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
