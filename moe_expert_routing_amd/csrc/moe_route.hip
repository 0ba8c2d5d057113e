// moe_route.hip - routing kernels for gfx950 and the C ABI of include/moe_route.h.
//
// Paths (all give identical results):
//  * decode, T <= 64: ONE launch, one token per wave. Up to 8 tokens one
//    block of 8 waves routes them all and builds counts, offsets and the
//    permutation after its own barrier; above, blocks of 4 waves publish
//    their output ids and the last block to arrive (an acquire-release
//    ticket in the workspace control block) builds them. Both use per-expert
//    64-bit token masks in LDS. With moe_route_quant_local, more blocks of
//    the same launch quantise the activations to MXFP8.
//  * prefill, T > 64: three launches.
//      route:   four tokens per wave (896 experts in 8 groups, route_rows.hpp)
//               or one token per wave (other shapes); at the end of every
//               block, per count tile (16 or 4 tokens) and output id the
//               tile's entry count -> hist[e'][tile], and per entry its rank
//               among the tile's entries of that id -> rank8.
//      prefix:  per output id, exclusive scan of hist[e'][:] over the tiles;
//               total -> counts[e'].
//      scatter: offsets = exclusive scan of counts; each entry goes to
//               offsets[e'] + hist[e'][tile] + rank8[f].
// Consumers of one call's counts and perm, one launch each: the grouped-GEMM
// layout (moe_grouped_layout) and the static balancing plan over expert-
// owning ranks (moe_balance_plan).
// Within one token the output ids are distinct (top-k ids are distinct and
// the relabelled ids are unique per row), so "ascending flat index within an
// expert" is "ascending token", and a token's position among the entries of
// an id is a popcount of the id's token mask below it.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/moe_route.h"
#include "internal.hpp"
#include "route_rows.hpp"
#include "route_wave.hpp"

static_assert(moe::kMaxTopK == MOE_ROUTE_MAX_TOPK, "top-k capacity");

namespace moe {

constexpr int WAVES_PER_BLOCK = 4;
constexpr int BLOCK = 64 * WAVES_PER_BLOCK;
constexpr size_t CONTROL_BYTES = 256;
// Inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4, 8 within each
// row of 16 lanes, then row 0's total into row 1 and row 2's into row 3
// (row_bcast:15), then rows 0-1's total into rows 2-3 (row_bcast:31).
// A lane with no source, or in a row the mask leaves out, adds 0.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// accesses, not for its global loads still in flight (a __syncthreads()
// waits for every outstanding load).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Exclusive scan of in[0..n) (n <= 1024) into out[0..n] in LDS, out[n] =
// total, by a block of THREADS threads (each takes 1024 / THREADS inputs), in
// two steps so that a caller can issue other loads between them: scan_load
// reads this thread's inputs; scan_store scans and writes. All THREADS
// threads must call both; wave_tot holds THREADS / 64 words.
// The loads take clamped indices and are unconditional, so all of them are
// in flight together (a guarded load becomes a branch that waits on its own).
template <int THREADS = BLOCK>
__device__ __forceinline__ void scan_load(const int32_t *in, int n, int (&v)[1024 / THREADS]) {
  constexpr int PER = 1024 / THREADS;
  if (n <= 0) {
#pragma unroll
    for (int k = 0; k < PER; ++k) v[k] = 0;
    return;
  }
  int x[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int idx = threadIdx.x * PER + k;
    x[k] = in[idx < n ? idx : n - 1];
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) v[k] = ((int)threadIdx.x * PER + k < n) ? x[k] : 0;
}
template <int THREADS = BLOCK>
__device__ __forceinline__ void scan_store(const int (&v)[1024 / THREADS], int n, int32_t *out,
                                           int32_t *wave_tot) {
  constexpr int PER = 1024 / THREADS;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  int s = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) s += v[k];
  const int incl = wave_inclusive_scan(s);
  if (lane == 63) wave_tot[wv] = incl;
  lds_barrier();
  int wave_off = 0;
  for (int w = 0; w < wv; ++w) wave_off += wave_tot[w];
  int run = wave_off + incl - s;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int idx = tid * PER + k;
    if (idx < n) out[idx] = run;
    run += v[k];
  }
  if (tid == THREADS - 1) out[n] = wave_off + incl;
  lds_barrier();
}

// ---------------------------------------------------------------------------
// Prefill permutation, part 1 (end of every prefill route block, all BLOCK
// threads, after the block's outputs are written): per output id, the
// block's entry count -> hist[e'][block]; per entry, its rank among the
// block's entries of the same id (token order) -> rank8[f]. Plain stores of
// every value, so the workspace needs no initial contents. A block covers at
// most 32 tokens (32-bit token masks in LDS).
// ---------------------------------------------------------------------------
// Column of count tile `tile` in its id's row of hist. Count tiles are the
// token groups that one route block counts together; a route block covers
// 2^lg consecutive tiles. The hardware sends route block b to XCD b % 8, so
// the columns of one XCD's blocks are made contiguous: every 64-byte line of
// a row is written by the blocks of one XCD, through one L2, and leaves it
// whole. Rows are hist_stride(ntiles, lg) words long.
__host__ __device__ __forceinline__ int hist_stride(int ntiles, int lg = 0) {
  const int nb = (ntiles + (1 << lg) - 1) >> lg;
  return ((nb + 7) >> 3) << (3 + lg);
}
__device__ __forceinline__ int hist_col(int tile, int ntiles, int lg = 0) {
  const int b = tile >> lg, i = tile & ((1 << lg) - 1);
  const int nb = (ntiles + (1 << lg) - 1) >> lg;
  return ((((b & 7) * ((nb + 7) >> 3)) + (b >> 3)) << lg) + i;
}

template <int THREADS>
__device__ void block_counts(const int32_t *__restrict__ packed, int K, int e_out, int64_t t_begin,
                             int ntok, int blk, int nblk, int32_t *__restrict__ hist,
                             uint8_t *__restrict__ rank8, uint32_t *lds_mask) {
  constexpr int PER = (32 * MOE_ROUTE_MAX_TOPK + THREADS - 1) / THREADS;
  const int tid = threadIdx.x;
  __syncthreads();  // every wave done (lds_mask may share LDS with routing scratch)
  for (int e = tid; e < e_out; e += THREADS) lds_mask[e] = 0u;
  __syncthreads();  // also orders this block's output stores before the reads below
  const int n = ntok * K;  // >= 1
  const int32_t *pk = packed + t_begin * K;
  int ev[PER], tv[PER];
#pragma unroll
  for (int h = 0; h < PER; ++h) {  // clamped, unconditional loads: one round trip
    const int i = tid + h * THREADS;
    ev[h] = pk[i < n ? i : n - 1] >> 16;
  }
#pragma unroll
  for (int h = 0; h < PER; ++h) {
    const int i = tid + h * THREADS;
    if (i < n) {
      tv[h] = i / K;
      atomicOr(&lds_mask[ev[h]], 1u << tv[h]);
    }
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < PER; ++h) {
    const int i = tid + h * THREADS;
    if (i < n) rank8[t_begin * K + i] = (uint8_t)__popc(lds_mask[ev[h]] & ((1u << tv[h]) - 1u));
  }
  const int col = hist_col(blk, nblk), stride = hist_stride(nblk);
  for (int e = tid; e < e_out; e += THREADS) hist[(size_t)e * stride + col] = __popc(lds_mask[e]);
}

// ---------------------------------------------------------------------------
// Activation quantisation of the fused route + quant launch: OCP MXFP8, E4M3
// elements with one E8M0 scale per 32 consecutive elements of a hidden row.
//   shared = max(floor(log2(amax)) - 8, -127)  (-127 for a block of zeros),
//   scale code = shared + 127, element = E4M3(v * 2^-shared), round to
//   nearest even, saturating at +-448.
// ---------------------------------------------------------------------------
struct QuantArgs {
  const uint16_t *hidden;  // bf16 [T, H]; nullptr = no quantisation
  uint8_t *q;              // E4M3 codes [T, H]
  uint8_t *scale;          // E8M0 codes [T, H / 32]
  int64_t nchunks;         // T * H / 8: 8-element chunks, 4 per scale block
};

constexpr int QUANT_CHUNKS_PER_BLOCK = BLOCK;  // one 16-byte chunk per thread

// E4M3 code of q (binary32), round to nearest even, saturating.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float q) {
  const uint32_t b = __float_as_uint(q);
  const uint32_t sg = (b >> 24) & 0x80u;
  const uint32_t ab = b & 0x7FFFFFFFu;
  if (ab >= 0x43E00000u) return sg | 0x7Eu;      // |q| >= 448
  if (ab < 0x3C800000u) {                         // |q| < 2^-6: multiples of 2^-9
    const float n = __builtin_rintf(__uint_as_float(ab) * 512.0f);  // exact product, 0..8
    return sg | (uint32_t)n;                      // 8 is 2^-6, the code 0x08
  }
  const uint32_t e = (ab >> 23) - 120u;           // E4M3 biased exponent, 1..15
  const uint32_t m = ab & 0x7FFFFFu;
  const uint32_t r = (m + 0x7FFFFu + ((m >> 20) & 1u)) >> 20;  // 23 -> 3 bits, to even
  const uint32_t code = (e << 3) + r;             // r = 8 carries into the exponent
  return sg | (code > 0x7Eu ? 0x7Eu : code);
}

// Chunk c (8 elements, 16 bytes) per thread; the 4 lanes of a scale block
// are adjacent (chunk indices 4k..4k+3 fall in lanes 4k'..4k'+3 of a wave
// because every block starts at a multiple of 4 chunks and a wave's chunks
// are consecutive).
__device__ __forceinline__ void mx_quant_chunk(const QuantArgs &qa, int64_t c) {
  const bool valid = c < qa.nchunks;
  uint4 raw = make_uint4(0u, 0u, 0u, 0u);
  if (valid) raw = reinterpret_cast<const uint4 *>(qa.hidden)[c];
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  uint32_t amax = 0u;  // largest |bf16| bit pattern of the lane
#pragma unroll
  for (int i = 0; i < 4; ++i) amax = umax(amax, umax(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  amax = umax(amax, dpp<DPP_XOR1>(amax));
  amax = umax(amax, dpp<DPP_XOR2>(amax));
  const int ef = (int)(amax >> 7);  // bf16 exponent field of the block maximum
  const int shared = (amax == 0u || ef == 0) ? -127 : max(ef - 135, -127);
  if (!valid) return;
  uint32_t out[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t h = (w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
    const float v = __builtin_amdgcn_ldexpf(__uint_as_float(h << 16), -shared);
    out[i >> 2] |= e4m3_rne_sat(v) << (8 * (i & 3));
  }
  reinterpret_cast<uint2 *>(qa.q)[c] = make_uint2(out[0], out[1]);
  if ((c & 3) == 0) qa.scale[c >> 2] = (uint8_t)(shared + 127);
}

// Standalone quantisation (the prefill path of the fused entry point).
__global__ __launch_bounds__(BLOCK) void mx_quant_kernel(QuantArgs qa) {
  mx_quant_chunk(qa, (int64_t)blockIdx.x * QUANT_CHUNKS_PER_BLOCK + threadIdx.x);
}

// ---------------------------------------------------------------------------
// Decode path: one launch for T <= 64, NW waves (one token each) per block.
// With one routing block (T <= NW) the block builds the permutation right
// after its own barrier, from its output ids kept in LDS. With several, every
// block also writes its output ids into perm, and after a workgroup barrier
// (its waves' stores happen before) thread 0 takes a ticket with a
// device-scope acquire-release atomic; the block that takes the last ticket
// reads every block's ids back from perm and builds the permutation over
// them. The release half orders each block's id stores before its ticket,
// the acquire half orders the last block's loads after every ticket before
// its own, so the last block sees all ids (on gfx950 the compiler brackets
// the atomic with an L2 write-back and an L2 invalidate). The last block
// resets the ticket, so every call leaves it zero. Blocks past the routing
// blocks quantise the activations.
// ---------------------------------------------------------------------------
constexpr int DECODE_ONE_BLOCK_WAVES = 8;  // T <= 8: one routing block

template <int NP, int LPG, int NW>
__global__ __launch_bounds__(64 * NW) void route_decode_kernel(
    const float *__restrict__ logits, const float *__restrict__ bias, int T, RouteParams p,
    int32_t *__restrict__ ids, float *__restrict__ wts, int32_t *__restrict__ packed,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *perm,  // (also the other blocks' ids: read and written across blocks)
    int32_t *__restrict__ inv, uint32_t *__restrict__ ticket, QuantArgs qa) {
  constexpr int THREADS = 64 * NW;
  // the one-block kernel is launched for T <= NW only
  constexpr bool MULTI = NW != DECODE_ONE_BLOCK_WAVES;
  const int nroute = T > 0 ? (T + NW - 1) / NW : 1;
  if ((int)blockIdx.x >= nroute) {
    mx_quant_chunk(qa, (int64_t)(blockIdx.x - nroute) * THREADS + threadIdx.x);
    return;
  }
  __shared__ unsigned long long mask[MOE_ROUTE_MAX_EXPERTS];
  __shared__ int32_t offs[MOE_ROUTE_MAX_EXPERTS + 1];
  __shared__ int32_t wave_tot[NW];
  __shared__ WaveScratch scratch[NW];
  __shared__ int32_t own_ids[MULTI ? 1 : DECODE_ONE_BLOCK_WAVES * MOE_ROUTE_MAX_TOPK];
  __shared__ int is_last;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int t = blockIdx.x * NW + wave;
  // Thread i owns ids [IPT i, IPT i + IPT) in the permutation below. Their
  // token masks are cleared now, in every routing block (LDS is per block;
  // the block that builds the permutation is only known later), and the
  // barrier after the routing orders the clearing before the first OR.
  constexpr int IPT = MOE_ROUTE_MAX_EXPERTS / THREADS;
  static_assert(IPT * THREADS == MOE_ROUTE_MAX_EXPERTS, "whole ids per thread");
#pragma unroll
  for (int j = 0; j < IPT; ++j) mask[IPT * threadIdx.x + j] = 0ull;
  if (t < T) {
    const float *row = logits + (size_t)t * p.E;
    float b[2 * NP], x[2 * NP];
    load_lane_layout<NP, LPG>(row, p, lane, x);
    load_lane_layout<NP, LPG>(bias, p, lane, b);
    const int idp =
        route_token<NP, LPG>(row, x, b, bias, p, lane, t, &scratch[wave], ids, wts, packed);
    // the last block reads the output ids from perm, where they stay until
    // it writes the permutation there
    if (MULTI && nroute > 1 && lane < p.K) perm[t * p.K + lane] = idp;
    if (!MULTI && lane < p.K) own_ids[t * p.K + lane] = idp;  // the one block's ids, in LDS
  }
  if (MULTI && nroute > 1) {
    // the block's id stores, then its ticket (release: those stores become
    // visible to the device first; acquire: the last block's loads below see
    // every other block's)
    __syncthreads();
    if (threadIdx.x == 0)
      is_last = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
                (uint32_t)nroute - 1u;
    __syncthreads();
    if (!is_last) return;
  } else {
    __syncthreads();  // the only routing block: its own outputs, nothing to wait for
  }

  // Every entry's output id, read once: PER loads per thread issued back to
  // back (indices past the end read the last entry and are not used).
  constexpr int PER = (MOE_ROUTE_MAX_FUSED_TOKENS * MOE_ROUTE_MAX_TOPK + THREADS - 1) / THREADS;
  static_assert(MOE_ROUTE_MAX_FUSED_TOKENS * MOE_ROUTE_MAX_TOPK <= 2048, "entry range");
  const int n = T * p.K;
  // token of entry f = f / K as a multiply-high (exact for f < 2048, K <= 32)
  const uint32_t kinv = 0xFFFFFFFFu / (uint32_t)p.K + 1u;
  int ev[PER], tv[PER];
#pragma unroll
  for (int h = 0; h < PER; ++h) ev[h] = 0;
  if (n > 0) {
#pragma unroll
    for (int h = 0; h < PER; ++h) {
      const int f = min((int)threadIdx.x + h * THREADS, n - 1);
      if constexpr (MULTI)
        ev[h] = nroute > 1 ? perm[f] : packed[f] >> 16;
      else
        ev[h] = own_ids[f];
    }
  }
  // (every id is read into ev, and used, before the barriers below, so
  // before perm is written)
#pragma unroll
  for (int h = 0; h < PER; ++h) {
    const int f = min((int)threadIdx.x + h * THREADS, max(n - 1, 0));
    tv[h] = p.K == 1 ? f : (int)__umulhi((uint32_t)f, kinv);
  }
#pragma unroll
  for (int h = 0; h < PER; ++h)
    if ((int)threadIdx.x + h * THREADS < n) atomicOr(&mask[ev[h]], 1ull << tv[h]);
  __syncthreads();
  // counts and exclusive offsets of the thread's ids: a wave scan of the
  // threads' sums, then the earlier waves' totals
  int c[IPT], sum = 0;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const int e = IPT * (int)threadIdx.x + j;
    c[j] = e < p.e_out ? __popcll(mask[e]) : 0;
    sum += c[j];
  }
  const int incl = wave_inclusive_scan(sum);
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int run = incl - sum;
#pragma unroll
  for (int w = 0; w < NW; ++w) run += w < wave ? wave_tot[w] : 0;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const int e = IPT * (int)threadIdx.x + j;
    if (e < p.e_out) {
      offs[e] = run;
      counts[e] = c[j];
      offsets[e] = run;
    }
    run += c[j];
  }
  if (threadIdx.x == 0) offsets[p.e_out] = n;
  __syncthreads();
  // LDS reads for every slot (clamped entries are valid ids), stores for
  // the real entries
#pragma unroll
  for (int h = 0; h < PER; ++h) {
    const int f = threadIdx.x + h * THREADS;
    const int pos = offs[ev[h]] + __popcll(mask[ev[h]] & ((1ull << tv[h]) - 1ull));
    if (f < n) {
      perm[pos] = f;
      if (inv) inv[f] = pos;
    }
  }
  if (MULTI && nroute > 1 && threadIdx.x == 0) *ticket = 0u;  // leave the control block zeroed
}

// ---------------------------------------------------------------------------
// Prefill path, kernel 1 (any shape): one token per wave, then the block's
// share of the tile counts (prefill_tile_counts).
// ---------------------------------------------------------------------------
struct PrefillCounts {
  int32_t *hist;      // [e_out][route blocks]
  uint8_t *rank8;     // [T * K]
};

template <int NP, int LPG>
__global__ __launch_bounds__(BLOCK) void route_tokens_kernel(
    const float *__restrict__ logits, const float *__restrict__ bias, int T, RouteParams p,
    int32_t *__restrict__ ids, float *__restrict__ wts, int32_t *__restrict__ packed,
    PrefillCounts pc) {
  // routing scratch, reused for the tile counts once every wave is done
  __shared__ union {
    WaveScratch wave[WAVES_PER_BLOCK];
    uint32_t mask[MOE_ROUTE_MAX_EXPERTS];
  } lds;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int64_t tb = (int64_t)blockIdx.x * WAVES_PER_BLOCK;
  const int64_t t = tb + wave;
  if (t < T) {
    const float *row = logits + (size_t)t * p.E;
    float b[2 * NP], x[2 * NP];
    load_lane_layout<NP, LPG>(row, p, lane, x);
    load_lane_layout<NP, LPG>(bias, p, lane, b);
    route_token<NP, LPG>(row, x, b, bias, p, lane, t, &lds.wave[wave], ids, wts, packed);
  }
  block_counts<BLOCK>(packed, p.K, p.e_out, tb, (int)min((int64_t)WAVES_PER_BLOCK, T - tb),
                     blockIdx.x, gridDim.x, pc.hist, pc.rank8, lds.mask);
}

// Prefill path, kernel 1 for the 896-expert, 8-group shape: four tokens per
// wave (route_rows.hpp), two count tiles of 16 tokens per block, software-
// pipelined in every wave: the first pass of the wave's next tile is
// requested before the current tile's selection runs, so the selection of
// one tile overlaps the memory latency of the next (the whole grid no longer
// streams first and selects last). Rows that fail their certificate are
// routed again one token per wave. Then each tile's counts.
__device__ unsigned long long g_row_fallback_tokens = 0ull;

constexpr int ROWS_WAVES = 4;
constexpr int ROWS_BLOCK = 64 * ROWS_WAVES;
constexpr int ROWS_TILE_TOKENS = 4 * ROWS_WAVES;  // tokens per count tile
constexpr int ROWS_TILES_LG = 1;                  // 2 tiles per block
constexpr int ROWS_TILES = 1 << ROWS_TILES_LG;
constexpr int ROWS_TOKENS_PER_BLOCK = ROWS_TILE_TOKENS * ROWS_TILES;
static_assert(ROWS_TILE_TOKENS <= 32 && WAVES_PER_BLOCK <= 32, "32-bit token masks");
static_assert(ROWS_TILE_TOKENS * rows::MAX_K <= ROWS_BLOCK, "one entry per thread");

struct RowsLds {
  rows::RowScratch wave[ROWS_WAVES];
  int32_t ids[ROWS_TILES][ROWS_WAVES][4][rows::MAX_K];  // output ids by tile, wave, row, slot
};

// The wave's rows of its tiles (tile i: tokens tb + 16 i + 4 wave + r), in
// key window W. Returns 4 bits per tile of rows to route again.
template <int W>
__device__ __forceinline__ uint32_t route_tiles(const float *__restrict__ logits,
                                                const float *__restrict__ bias,
                                                const float *__restrict__ bias_lds, int T,
                                                int64_t tb, int wave, const RouteParams &p,
                                                int lane, RowsLds &L, int32_t *__restrict__ ids,
                                                float *__restrict__ wts,
                                                int32_t *__restrict__ packed) {
  const int r = lane >> 4, c = (lane & 15) >> 2, sub = lane & 3;
  auto tile_t0 = [&](int i) { return tb + (int64_t)ROWS_TILE_TOKENS * i + 4 * wave; };
  auto row_of = [&](int i) {
    const int64_t t = tile_t0(i) + r;
    return logits + (size_t)(t < T ? t : (int64_t)T - 1) * rows::E;
  };
  uint32_t redo = 0u;
  float4 xq[rows::PREFETCH];
  rows::first_loads(row_of(0), c, sub, xq);
#pragma unroll 1
  for (int i = 0; i < ROWS_TILES; ++i) {
    uint32_t a[rows::PP], b[rows::PP];
    __builtin_amdgcn_s_setprio(3);
    rows::stream_pools(row_of(i), bias_lds, c, sub, xq, a, b);
    const bool next = i + 1 < ROWS_TILES && tile_t0(i + 1) < T;  // wave-uniform
    if (next) rows::first_loads(row_of(i + 1), c, sub, xq);
    __builtin_amdgcn_sched_barrier(0);
    redo |= rows::route_rows4_post<W>(a, b, logits, bias, bias_lds, T, tile_t0(i), p, lane,
                                      &L.wave[wave], L.ids[i][wave], ids, wts, packed)
            << (4 * i);
    if (!next) break;
  }
  return redo;
}

__global__ __launch_bounds__(ROWS_BLOCK, 4) void route_rows_kernel(
    const float *__restrict__ logits, const float *__restrict__ bias, int T, RouteParams p,
    int32_t *__restrict__ ids, float *__restrict__ wts, int32_t *__restrict__ packed,
    PrefillCounts pc) {
  __shared__ __align__(16) float bias_lds[rows::E];  // fl32(b + B) of the block's key window
  __shared__ RowsLds L;
  __shared__ int bad_bias[ROWS_WAVES];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int64_t tb = (int64_t)blockIdx.x * ROWS_TOKENS_PER_BLOCK;
  // the whole kernel starts at the streaming issue priority (see route_rows4_post)
  __builtin_amdgcn_s_setprio(3);
  const int window = rows::stage_bias<ROWS_BLOCK>(bias, bias_lds, bad_bias);
  uint32_t redo = 0u;
  if (tb + 4 * wave < T) {
    if (window == 0)
      redo = route_tiles<0>(logits, bias, bias_lds, T, tb, wave, p, lane, L, ids, wts, packed);
    else if (window == 1)
      redo = route_tiles<1>(logits, bias, bias_lds, T, tb, wave, p, lane, L, ids, wts, packed);
    else
      redo = (1u << (4 * ROWS_TILES)) - 1u;  // a bias outside both windows
  }
  redo = (uint32_t)__builtin_amdgcn_readfirstlane((int)redo);
  while (redo) {
    const int q = __builtin_ctz(redo), i = q >> 2, r = q & 3;
    redo &= redo - 1u;
    const int64_t t = tb + (int64_t)ROWS_TILE_TOKENS * i + 4 * wave + r;
    if (t >= T) continue;
    if (lane == 0) atomicAdd(&g_row_fallback_tokens, 1ull);
    const float *row = logits + (size_t)t * p.E;
    float b[14], x[14];
    load_lane_layout<7, 8>(row, p, lane, x);
    load_lane_layout<7, 8>(bias, p, lane, b);
    const int idp = route_token_plain<7, 8>(row, x, b, p, lane, t, ids, wts, packed);
    if (lane < p.K) L.ids[i][wave][r][lane] = idp;
  }
  // Each tile's counts, from the output ids the waves left in LDS; the token
  // masks take the bias staging's LDS, free once every wave is done
  // (E' <= 896 words).
  uint32_t *mask = reinterpret_cast<uint32_t *>(bias_lds);
  const int ntiles = (T + ROWS_TILE_TOKENS - 1) / ROWS_TILE_TOKENS;
#pragma unroll 1
  for (int i = 0; i < ROWS_TILES; ++i) {
    const int64_t t0 = tb + (int64_t)ROWS_TILE_TOKENS * i;
    if (t0 >= T) break;  // block-uniform
    __syncthreads();
    for (int e = threadIdx.x; e < p.e_out; e += ROWS_BLOCK) mask[e] = 0u;
    __syncthreads();
    const int ntok = (int)min((int64_t)ROWS_TILE_TOKENS, T - t0);
    const int n = ntok * p.K;  // <= 256 = ROWS_BLOCK
    const int f = threadIdx.x;
    int ev = 0, tk = 0;
    if (f < n) {
      tk = f / p.K;
      ev = L.ids[i][tk >> 2][tk & 3][f - tk * p.K];
      ev = (unsigned)ev < (unsigned)p.e_out ? ev : 0;  // (every id is in range; guard only)
      atomicOr(&mask[ev], 1u << tk);
    }
    __syncthreads();
    if (f < n) pc.rank8[t0 * p.K + f] = (uint8_t)__popc(mask[ev] & ((1u << tk) - 1u));
    const int tile = (int)blockIdx.x * ROWS_TILES + i;
    const int col = hist_col(tile, ntiles, ROWS_TILES_LG), stride = hist_stride(ntiles, ROWS_TILES_LG);
    for (int e = threadIdx.x; e < p.e_out; e += ROWS_BLOCK)
      pc.hist[(size_t)e * stride + col] = __popc(mask[e]);
  }
}

// Prefill permutation, part 2: one block per output id: exclusive scan of
// hist[e'][0..nblk) in place (entries of e' in earlier route blocks) and the
// id's total -> counts[e'].
constexpr int SCAN_PER_THREAD = 8;

__global__ __launch_bounds__(BLOCK) void block_prefix_kernel(int32_t *__restrict__ hist, int nblk,
                                                             int lg, int32_t *__restrict__ counts) {
  __shared__ int32_t wave_tot[WAVES_PER_BLOCK];
  int32_t *row = hist + (size_t)blockIdx.x * hist_stride(nblk, lg);  // tile t at row[hist_col(t)]
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int carry = 0;
  for (int base = 0; base < nblk; base += BLOCK * SCAN_PER_THREAD) {
    const int beg = base + tid * SCAN_PER_THREAD;
    int v[SCAN_PER_THREAD];
    int sum = 0;
#pragma unroll
    for (int k = 0; k < SCAN_PER_THREAD; ++k) {
      v[k] = (beg + k < nblk) ? row[hist_col(beg + k, nblk, lg)] : 0;
      sum += v[k];
    }
    const int incl = wave_inclusive_scan(sum);
    if (lane == 63) wave_tot[wv] = incl;
    __syncthreads();
    int off = carry, total = 0;
#pragma unroll
    for (int w = 0; w < WAVES_PER_BLOCK; ++w) {
      if (w < wv) off += wave_tot[w];
      total += wave_tot[w];
    }
    int run = off + incl - sum;
#pragma unroll
    for (int k = 0; k < SCAN_PER_THREAD; ++k) {
      if (beg + k < nblk) row[hist_col(beg + k, nblk, lg)] = run;
      run += v[k];
    }
    carry += total;
    __syncthreads();
  }
  if (tid == 0) counts[blockIdx.x] = carry;
}

// Prefill permutation, part 3: offsets = exclusive scan of counts (every
// block forms it in LDS; block 0 writes it out), then every entry f goes to
// offsets[e'] + hist[e'][its route block] + rank8[f]. A thread takes
// SCATTER_PER_THREAD entries and issues each round of loads for all of them
// before using any.
constexpr int SCATTER_PER_THREAD = 4;
constexpr int SCATTER_TAB = 2048;  // LDS words for the chunk's route-block prefixes

// Grouped-GEMM layout of the same call, written by the scatter itself
// (moe_route_local_grouped): the rows of id e are padded[e] .. padded[e+1]-1,
// padded = exclusive scan of round_up(counts, tile_m); m_idx[row] = e for the
// first counts[e] of them and -1 for the rest and for rows past padded[E'];
// row_entry[row] = the flat entry at that position of perm, -1 where m_idx
// is. tile_m = 0: no layout.
struct LayoutArgs {
  int tile_m = 0;
  int32_t *padded = nullptr;     // [E'+1]
  int32_t *m_idx = nullptr;      // [rows]
  int32_t *row_entry = nullptr;  // [rows], or nullptr
  int64_t rows = 0;
};

__global__ __launch_bounds__(BLOCK) void scatter_kernel(
    const int32_t *__restrict__ packed, const int32_t *__restrict__ hist,
    const uint8_t *__restrict__ rank8, const int32_t *__restrict__ counts, int e_out, int nblk,
    int lg, int tokens_per_blk, int K, int64_t n, int32_t *__restrict__ offsets,
    int32_t *__restrict__ perm, int32_t *__restrict__ inv, LayoutArgs la) {
  __shared__ int32_t offs[MOE_ROUTE_MAX_EXPERTS + 1];
  __shared__ int32_t pad[MOE_ROUTE_MAX_EXPERTS + 1];  // padded offsets (layout only)
  __shared__ int32_t wave_tot[WAVES_PER_BLOCK];
  __shared__ int32_t tab[SCATTER_TAB];
  // consecutive entry chunks go to blocks on one XCD (block b runs on XCD
  // b % 8), so the perm lines they share are written through one L2
  const int nb = (int)gridDim.x, b = (int)blockIdx.x;
  const int chunk = (nb % 8 == 0) ? (b % 8) * (nb / 8) + b / 8 : b;
  // entry indices fit in 32 bits (n < 2^31, checked on the host); an entry's
  // route block is f / (K * tokens_per_blk)
  const int nn = (int)n;
  const uint32_t kt = (uint32_t)(K * tokens_per_blk);
  const int fb = chunk * BLOCK * SCATTER_PER_THREAD;  // the chunk's first entry (< n)
  const int fe = min(fb + BLOCK * SCATTER_PER_THREAD, nn) - 1;
  // the route blocks the chunk spans; when their prefixes for every id fit
  // in LDS they are loaded together with the entries (one round trip),
  // otherwise each entry's prefix is read after its id
  const int rb0 = (int)((uint32_t)fb / kt);
  const int nrb = (int)((uint32_t)fe / kt) - rb0 + 1;
  const bool tabled = nrb * e_out <= SCATTER_TAB;  // block-uniform
  const int stride = hist_stride(nblk, lg);
  // Every load of the first round (counts, the entries, the table) is issued
  // before any is used: clamped indices, no branches between them.
  int cx[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) cx[k] = counts[min((int)threadIdx.x * 4 + k, e_out - 1)];
  int ev[SCATTER_PER_THREAD], rv[SCATTER_PER_THREAD];
#pragma unroll
  for (int k = 0; k < SCATTER_PER_THREAD; ++k) {
    const int f = min(fb + (int)threadIdx.x + k * BLOCK, fe);
    ev[k] = packed[f];
    rv[k] = rank8[f];
  }
  constexpr int TAB_PER = SCATTER_TAB / BLOCK;
  // (loaded whether or not the table is used: in-range entries either way)
  const int ntab = min(nrb * e_out, SCATTER_TAB);
  int tv[TAB_PER];
#pragma unroll
  for (int h = 0; h < TAB_PER; ++h) {
    const int i = min((int)threadIdx.x + h * BLOCK, ntab - 1);
    const int rb = i / e_out;  // (route block rb0 + rb, id i - rb e_out)
    tv[h] = hist[(size_t)(i - rb * e_out) * stride + hist_col(rb0 + rb, nblk, lg)];
  }
  int cv[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) cv[k] = ((int)threadIdx.x * 4 + k < e_out) ? cx[k] : 0;
#pragma unroll
  for (int k = 0; k < SCATTER_PER_THREAD; ++k) ev[k] >>= 16;
#pragma unroll
  for (int h = 0; h < TAB_PER; ++h)
    if ((int)threadIdx.x + h * BLOCK < ntab) tab[threadIdx.x + h * BLOCK] = tv[h];
  int hv[SCATTER_PER_THREAD];
#pragma unroll
  for (int k = 0; k < SCATTER_PER_THREAD; ++k) hv[k] = 0;
  if (!tabled) {
#pragma unroll
    for (int k = 0; k < SCATTER_PER_THREAD; ++k) {
      const int f = min(fb + (int)threadIdx.x + k * BLOCK, fe);
      hv[k] = hist[(size_t)ev[k] * stride + hist_col((int)((uint32_t)f / kt), nblk, lg)];
    }
  }
  scan_store(cv, e_out, offs, wave_tot);  // its barriers also publish tab
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= e_out; i += BLOCK) offsets[i] = offs[i];
  const bool layout = la.tile_m > 0;  // block-uniform
  if (layout) {
    int pv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) pv[k] = (cv[k] + la.tile_m - 1) / la.tile_m * la.tile_m;
    scan_store(pv, e_out, pad, wave_tot);
    if (blockIdx.x == 0)
      for (int i = threadIdx.x; i <= e_out; i += BLOCK) la.padded[i] = pad[i];
  }
#pragma unroll
  for (int k = 0; k < SCATTER_PER_THREAD; ++k) {
    const int f = fb + (int)threadIdx.x + k * BLOCK;
    if (f <= fe) {
      const int h = tabled ? tab[((int)((uint32_t)f / kt) - rb0) * e_out + ev[k]] : hv[k];
      const int32_t pos = offs[ev[k]] + h + rv[k];
      perm[pos] = f;
      if (inv) inv[f] = pos;
      if (layout && la.row_entry) la.row_entry[pad[ev[k]] + h + rv[k]] = f;
    }
  }
  if (layout) {
    // this block's share of the layout rows, four consecutive rows per
    // thread: the id of each (one binary search over pad for the first, then
    // steps), and row_entry = -1 for the padding and spare rows (the entry
    // rows' row_entry was written above)
    const int64_t groups = (la.rows + 3) / 4;
    const int64_t per = (groups + nb - 1) / nb;
    const int64_t gend = min(groups, (int64_t)(b + 1) * per);
    for (int64_t g = (int64_t)b * per + threadIdx.x; g < gend; g += BLOCK) {
      const int64_t r0 = 4 * g;
      int lo = 0, hi = e_out + 1;  // the largest e with pad[e] <= r0 (pad[0] = 0)
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((int64_t)pad[mid] <= r0) lo = mid;
        else hi = mid;
      }
      int32_t mi[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int64_t r = r0 + k;
        while (lo < e_out && (int64_t)pad[lo + 1] <= r) ++lo;
        mi[k] = (lo < e_out && r - pad[lo] < (int64_t)(offs[lo + 1] - offs[lo])) ? lo : -1;
      }
      if (r0 + 4 <= la.rows && ((uintptr_t)(la.m_idx + r0) & 15) == 0) {
        *reinterpret_cast<int4 *>(la.m_idx + r0) = make_int4(mi[0], mi[1], mi[2], mi[3]);
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (r0 + k < la.rows) la.m_idx[r0 + k] = mi[k];
      }
      if (la.row_entry) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (r0 + k < la.rows && mi[k] < 0) la.row_entry[r0 + k] = -1;
      }
    }
  }
}

// Grouped-GEMM layout from a routing call's counts and perm: the entries of
// id e fill rows padded[e] .. padded[e] + counts[e] - 1 in permutation order,
// then padding rows up to padded[e+1] = padded[e] + round_up(counts[e],
// tile_m). Every block forms both scans of counts in LDS (E' <= 1024);
// block 0 writes the padded offsets; each thread fills LAYOUT_PER_THREAD
// consecutive rows (one 16-byte store per array when aligned), finding the
// first row's id by binary search over the padded offsets. Reads
// of perm and writes of rows are bounds-checked, so counts that do not
// match perm give wrong rows but no access outside the arrays.
constexpr int LAYOUT_PER_THREAD = 4;  // the int4 stores below assume 4

__global__ __launch_bounds__(BLOCK) void grouped_layout_kernel(
    const int32_t *__restrict__ counts, const int32_t *__restrict__ perm, int e_out,
    int64_t n_entries, int tile_m, int32_t *__restrict__ padded_offsets,
    int32_t *__restrict__ m_indices, int32_t *__restrict__ row_entry, int64_t rows) {
  __shared__ int32_t offs[MOE_ROUTE_MAX_EXPERTS + 1];
  __shared__ int32_t pad[MOE_ROUTE_MAX_EXPERTS + 1];
  __shared__ int32_t wave_tot[WAVES_PER_BLOCK];
  int cv[4], pv[4];
  scan_load(counts, e_out, cv);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    cv[k] = max(cv[k], 0);
    pv[k] = (cv[k] + tile_m - 1) / tile_m * tile_m;
  }
  scan_store(cv, e_out, offs, wave_tot);
  scan_store(pv, e_out, pad, wave_tot);
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= e_out; i += BLOCK) padded_offsets[i] = pad[i];
  // this thread's LAYOUT_PER_THREAD consecutive rows: one binary search for
  // the first (the largest e with pad[e] <= r; pad[0] = 0), then step
  const int64_t r0 = ((int64_t)blockIdx.x * BLOCK + threadIdx.x) * LAYOUT_PER_THREAD;
  if (r0 >= rows) return;
  int lo = 0, hi = e_out + 1;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)pad[mid] <= r0) lo = mid;
    else hi = mid;
  }
  int32_t mi[LAYOUT_PER_THREAD], ent[LAYOUT_PER_THREAD];
#pragma unroll
  for (int k = 0; k < LAYOUT_PER_THREAD; ++k) {
    const int64_t r = r0 + k;
    while (lo < e_out && (int64_t)pad[lo + 1] <= r) ++lo;
    mi[k] = -1;
    ent[k] = -1;
    if (lo < e_out) {
      const int64_t j = r - pad[lo];
      if (j < (int64_t)(offs[lo + 1] - offs[lo])) {
        const int64_t idx = offs[lo] + j;
        mi[k] = lo;
        ent[k] = (idx >= 0 && idx < n_entries) ? perm[idx] : -1;
      }
    }
  }
  if (r0 + LAYOUT_PER_THREAD <= rows && ((uintptr_t)(m_indices + r0) & 15) == 0 &&
      (!row_entry || ((uintptr_t)(row_entry + r0) & 15) == 0)) {
    *reinterpret_cast<int4 *>(m_indices + r0) = make_int4(mi[0], mi[1], mi[2], mi[3]);
    if (row_entry)
      *reinterpret_cast<int4 *>(row_entry + r0) = make_int4(ent[0], ent[1], ent[2], ent[3]);
  } else {
#pragma unroll
    for (int k = 0; k < LAYOUT_PER_THREAD; ++k) {
      if (r0 + k >= rows) break;
      m_indices[r0 + k] = mi[k];
      if (row_entry) row_entry[r0 + k] = ent[k];
    }
  }
}

// Static per-rank balancing plan over N ranks that own the experts in
// contiguous ranges of E / N, from one routing call's global counts: rank r
// keeps the first min(load[r], target[r]) of its own entries (expert-major
// order), the rest of every overloaded rank forms one surplus sequence in
// rank order, and the ranks short of their target take consecutive runs of
// it in rank order; target[r] = n / N, +1 for the first n % N ranks. Every
// block forms the scans in LDS; each thread writes 4 consecutive entries'
// ranks; block 0 writes rank_counts [N][E] from interval overlaps.
constexpr int PLAN_MAX_RANKS = 64;
constexpr int PLAN_PER_THREAD = 4;  // the int4 stores below assume 4

__global__ __launch_bounds__(BLOCK) void balance_plan_kernel(const int32_t *__restrict__ counts,
                                                             int E, int n_ranks, int64_t n,
                                                             int32_t *__restrict__ dest,
                                                             int32_t *__restrict__ rank_counts) {
  __shared__ int32_t offs[MOE_ROUTE_MAX_EXPERTS + 1];
  __shared__ int32_t wave_tot[WAVES_PER_BLOCK];
  __shared__ int32_t A[PLAN_MAX_RANKS + 1], keep[PLAN_MAX_RANKS];
  __shared__ int32_t SP[PLAN_MAX_RANKS + 1], DP[PLAN_MAX_RANKS + 1];
  int cv[4];
  scan_load(counts, E, cv);
#pragma unroll
  for (int k = 0; k < 4; ++k) cv[k] = max(cv[k], 0);
  scan_store(cv, E, offs, wave_tot);
  const int per = E / n_ranks;
  if (threadIdx.x < 64) {  // one wave: per-rank keep, surplus and deficit, scanned
    const int r = threadIdx.x;
    int kp = 0, sur = 0, def = 0;
    if (r < n_ranks) {
      const int a = offs[r * per];
      const int load = offs[(r + 1) * per] - a;
      const int tgt = (int)(n / n_ranks) + (r < (int)(n % n_ranks) ? 1 : 0);
      kp = min(load, tgt);
      sur = load - kp;
      def = tgt - kp;
      A[r] = a;
      keep[r] = kp;
    }
    const int si = wave_inclusive_scan(sur), di = wave_inclusive_scan(def);
    if (r < n_ranks) {
      SP[r + 1] = si;
      DP[r + 1] = di;
    }
    if (r == 0) {
      SP[0] = 0;
      DP[0] = 0;
      A[n_ranks] = offs[E];
    }
  }
  lds_barrier();
  if (blockIdx.x == 0) {
    for (int e = threadIdx.x; e < E; e += BLOCK) {
      const int r = e / per;
      const int a = offs[e] - A[r], b = offs[e + 1] - A[r];  // e's entries among rank r's
      const int kept = max(min(b, keep[r]) - a, 0);
      const int s0 = SP[r] + max(a, keep[r]) - keep[r], s1 = SP[r] + b - keep[r];
      for (int q = 0; q < n_ranks; ++q) {
        int c = max(min(s1, DP[q + 1]) - max(s0, DP[q]), 0);  // surplus run taken by q
        if (q == r) c += kept;
        rank_counts[(size_t)q * E + e] = c;
      }
    }
  }
  const int64_t p0 = ((int64_t)blockIdx.x * BLOCK + threadIdx.x) * PLAN_PER_THREAD;
  if (p0 >= n) return;
  int d[PLAN_PER_THREAD];
#pragma unroll
  for (int k = 0; k < PLAN_PER_THREAD; ++k) {
    const int64_t p = p0 + k;
    // the owner: the largest r with A[r] <= p (ranks without entries skipped)
    int lo = 0, hi = n_ranks + 1;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((int64_t)A[mid] <= p) lo = mid;
      else hi = mid;
    }
    const int r = min(lo, n_ranks - 1);
    const int own = (int)(p - A[r]);
    if (own < keep[r]) {
      d[k] = r;
    } else {
      const int sidx = SP[r] + own - keep[r];  // index in the surplus sequence
      int l2 = 0, h2 = n_ranks + 1;
      while (h2 - l2 > 1) {
        const int mid = (l2 + h2) >> 1;
        if (DP[mid] <= sidx) l2 = mid;
        else h2 = mid;
      }
      d[k] = min(l2, n_ranks - 1);
    }
  }
  if (p0 + PLAN_PER_THREAD <= n && ((uintptr_t)(dest + p0) & 15) == 0) {
    *reinterpret_cast<int4 *>(dest + p0) = make_int4(d[0], d[1], d[2], d[3]);
  } else {
#pragma unroll
    for (int k = 0; k < PLAN_PER_THREAD; ++k)
      if (p0 + k < n) dest[p0 + k] = d[k];
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

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Benchmark hook (moe_route_set_kernel_events).
static hipEvent_t g_ev_before = nullptr, g_ev_after = nullptr;

// The four-tokens-per-wave path: 896 experts in 8 groups, top_k <= 16, and
// kept lanes whose pools (6 usable keys each) can hold top_k + 1 entries;
// float4 loads need 16-byte aligned rows.
static bool rows_path_applies(const RouteParams &rp, const float *logits) {
  return rp.E == rows::E && rp.G == rows::G && rp.K <= rows::MAX_K &&
         12 * rp.TG >= rp.K + 1 && ((uintptr_t)logits % 16) == 0;
}

// Workspace layout of one call: the control block, then for the prefill path
// the per-count-tile id counts hist[e'][tile] and the entries' in-tile ranks.
// Count tiles hold 16 tokens on the four-tokens-per-wave path (two tiles per
// route block), 4 on the one-token-per-wave path (one per block).
struct WsLayout {
  int tpb = 0, lg = 0, ntiles = 0;  // tokens per tile, log2 tiles per block, tiles
  size_t hist = 0, rank8 = 0;       // byte offsets in the workspace
  size_t bytes = CONTROL_BYTES;     // total
};

static WsLayout ws_layout(int T, int e_out, int K, bool rows_path) {
  WsLayout w;
  if (T <= MOE_ROUTE_MAX_FUSED_TOKENS) return w;
  w.tpb = rows_path ? ROWS_TILE_TOKENS : WAVES_PER_BLOCK;
  w.lg = rows_path ? ROWS_TILES_LG : 0;
  w.ntiles = (T + w.tpb - 1) / w.tpb;
  w.hist = CONTROL_BYTES;
  w.rank8 = w.hist + align256((size_t)hist_stride(w.ntiles, w.lg) * e_out * sizeof(int32_t));
  w.bytes = w.rank8 + align256((size_t)T * K);
  return w;
}

// Bytes a caller's workspace must hold: the layout of the path with the
// smallest count tiles (one token per wave), which bounds every path's.
static size_t route_ws_bytes(int T, int e_out, int K) {
  return ws_layout(T, e_out, K, false).bytes;
}

template <int NP, int LPG>
static hipError_t launch_route(const float *logits, const float *bias, int T, const RouteParams &rp,
                               const moe_route_outputs *o, char *ws, hipStream_t st,
                               const QuantArgs &qa, const LayoutArgs &la) {
  const int qblocks =
      qa.hidden ? (int)((qa.nchunks + QUANT_CHUNKS_PER_BLOCK - 1) / QUANT_CHUNKS_PER_BLOCK) : 0;
  if (T <= MOE_ROUTE_MAX_FUSED_TOKENS) {
    // one launch: routing blocks, then the quantisation blocks
    auto launch = [&](auto kernel, int nw) {
      const int threads = 64 * nw;
      const int qb =
          qa.hidden ? (int)((qa.nchunks + threads - 1) / threads) : 0;
      const int grid = (T > 0 ? (T + nw - 1) / nw : 1) + qb;
      hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(threads), 0, st, g_ev_before, g_ev_after, 0,
                            logits, bias, T, rp, o->topk_ids, o->topk_weights, o->packed,
                            o->counts, o->offsets, o->perm, o->inv_perm,
                            reinterpret_cast<uint32_t *>(ws), qa);
    };
    if (T <= DECODE_ONE_BLOCK_WAVES)
      launch(route_decode_kernel<NP, LPG, DECODE_ONE_BLOCK_WAVES>, DECODE_ONE_BLOCK_WAVES);
    else
      launch(route_decode_kernel<NP, LPG, WAVES_PER_BLOCK>, WAVES_PER_BLOCK);
    return hipGetLastError();
  }
  if (qblocks > 0) mx_quant_kernel<<<qblocks, BLOCK, 0, st>>>(qa);
  const bool rows_path = LPG == 8 && NP == 7 && rows_path_applies(rp, logits);
  const WsLayout wl = ws_layout(T, rp.e_out, rp.K, rows_path);
  const int tpb = wl.tpb, lg = wl.lg, nblk = wl.ntiles;
  PrefillCounts pc;
  pc.hist = reinterpret_cast<int32_t *>(ws + wl.hist);
  pc.rank8 = reinterpret_cast<uint8_t *>(ws + wl.rank8);
  // the benchmark hook's events are recorded by the launch itself
  if (rows_path) {
    const int grid = (T + ROWS_TOKENS_PER_BLOCK - 1) / ROWS_TOKENS_PER_BLOCK;
    hipExtLaunchKernelGGL(route_rows_kernel, dim3(grid), dim3(ROWS_BLOCK), 0, st, g_ev_before,
                          g_ev_after, 0, logits, bias, T, rp, o->topk_ids, o->topk_weights,
                          o->packed, pc);
  } else {
    hipExtLaunchKernelGGL(route_tokens_kernel<NP, LPG>, dim3(nblk), dim3(BLOCK), 0, st,
                          g_ev_before, g_ev_after, 0, logits, bias, T, rp, o->topk_ids,
                          o->topk_weights, o->packed, pc);
  }
  block_prefix_kernel<<<rp.e_out, BLOCK, 0, st>>>(pc.hist, nblk, lg, o->counts);
  const int64_t n = (int64_t)T * rp.K;
  const int64_t g3 = (n + BLOCK * SCATTER_PER_THREAD - 1) / (BLOCK * SCATTER_PER_THREAD);
  scatter_kernel<<<(int)g3, BLOCK, 0, st>>>(o->packed, pc.hist, pc.rank8, o->counts, rp.e_out,
                                            nblk, lg, tpb, rp.K, n, o->offsets, o->perm,
                                            o->inv_perm, la);
  return hipGetLastError();
}

// Every check of a routing call except the workspace's.
static int validate_route_args(const float *logits, const float *bias, int32_t T,
                               const moe_route_params *prm, int32_t off, int32_t cnt,
                               const moe_route_outputs *o, int *e_out) {
  int st = validate_params(prm);
  if (st != MOE_OK) return st;
  if (!o) return MOE_ERR_NULL;
  if (T < 0) return MOE_ERR_SHAPE;
  // entries f = t * top_k + k and their positions are int32
  if ((int64_t)T * prm->top_k > (int64_t)INT32_MAX) return MOE_ERR_SHAPE;
  if (!o->counts || !o->offsets) return MOE_ERR_NULL;
  if (T > 0 && (!logits || !bias || !o->topk_ids || !o->topk_weights || !o->packed || !o->perm))
    return MOE_ERR_NULL;
  const int32_t e_local = moe_route_local_num_experts(prm->num_experts, prm->top_k, off, cnt);
  if (e_local < 0) return e_local;
  if ((uintptr_t)logits % 8 != 0 || (uintptr_t)bias % 8 != 0) return MOE_ERR_SHAPE;
  *e_out = e_local > 0 ? e_local : prm->num_experts;
  return MOE_OK;
}

int validate_route_call(const float *logits, const float *bias, int32_t T,
                        const moe_route_params *prm, int32_t off, int32_t cnt,
                        const moe_route_outputs *o, const void *workspace, size_t ws_bytes,
                        int *e_out) {
  int eo = 0;
  const int st = validate_route_args(logits, bias, T, prm, off, cnt, o, &eo);
  if (st != MOE_OK) return st;
  if (!workspace) return MOE_ERR_WORKSPACE;
  if (ws_bytes < route_ws_bytes(T, eo, prm->top_k)) return MOE_ERR_WORKSPACE;
  if ((uintptr_t)workspace % 8 != 0) return MOE_ERR_WORKSPACE;
  if (e_out) *e_out = eo;
  return MOE_OK;
}


static RouteParams route_params(const moe_route_params *prm, int32_t off, int32_t cnt,
                                int e_out) {
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
  return rp;
}

// Launches a validated call on workspace `ws`.
static int route_launch(const float *logits, const float *bias, int32_t T, const RouteParams &rp,
                        const moe_route_outputs *o, char *ws, hipStream_t s,
                        const QuantArgs &qa, const LayoutArgs &la = LayoutArgs{}) {
  hipError_t err;
  // the 896-expert, 8-group shape gets constant lanes per group
  if (rp.E == 896 && rp.lpg == 8) {
    err = launch_route<7, 8>(logits, bias, T, rp, o, ws, s, qa, la);
    return err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
  }
  switch (rp.E / 128) {
    case 1: err = launch_route<1, 0>(logits, bias, T, rp, o, ws, s, qa, la); break;
    case 2: err = launch_route<2, 0>(logits, bias, T, rp, o, ws, s, qa, la); break;
    case 3: err = launch_route<3, 0>(logits, bias, T, rp, o, ws, s, qa, la); break;
    case 4: err = launch_route<4, 0>(logits, bias, T, rp, o, ws, s, qa, la); break;
    case 5: err = launch_route<5, 0>(logits, bias, T, rp, o, ws, s, qa, la); break;
    case 6: err = launch_route<6, 0>(logits, bias, T, rp, o, ws, s, qa, la); break;
    case 7: err = launch_route<7, 0>(logits, bias, T, rp, o, ws, s, qa, la); break;
    case 8: err = launch_route<8, 0>(logits, bias, T, rp, o, ws, s, qa, la); break;
    default: return MOE_ERR_UNSUPPORTED;
  }
  return err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

static int route_impl(const float *logits, const float *bias, int32_t T,
                      const moe_route_params *prm, int32_t off, int32_t cnt,
                      const moe_route_outputs *o, void *workspace, size_t ws_bytes,
                      void *stream, const QuantArgs &qa = QuantArgs{nullptr, nullptr, nullptr, 0}) {
  int e_out = 0;
  const int st = validate_route_call(logits, bias, T, prm, off, cnt, o, workspace, ws_bytes,
                                     &e_out);
  if (st != MOE_OK) return st;
  return route_launch(logits, bias, T, route_params(prm, off, cnt, e_out), o,
                      reinterpret_cast<char *>(workspace), reinterpret_cast<hipStream_t>(stream),
                      qa);
}

// moe_route_local_grouped: the routing call and the grouped-GEMM layout of
// its entries. Above the decode cap the scatter writes the layout as it
// places the entries (no layout launch); at decode sizes the layout kernel
// follows the single routing launch.
static int route_grouped_impl(const float *logits, const float *bias, int32_t T,
                              const moe_route_params *prm, int32_t off, int32_t cnt,
                              const moe_route_outputs *o, int32_t tile_m,
                              int32_t *padded_offsets, int32_t *m_indices, int32_t *row_entry,
                              int64_t rows, void *workspace, size_t ws_bytes, void *stream) {
  int e_out = 0;
  const int st = validate_route_call(logits, bias, T, prm, off, cnt, o, workspace, ws_bytes,
                                     &e_out);
  if (st != MOE_OK) return st;
  const int64_t n = (int64_t)T * prm->top_k;
  const int64_t need = moe_grouped_layout_rows(n, e_out, tile_m);
  if (need < 0) return (int)need;
  if (!padded_offsets) return MOE_ERR_NULL;
  if (rows < need) return MOE_ERR_SHAPE;
  if (rows > 0 && !m_indices) return MOE_ERR_NULL;
  const RouteParams rp = route_params(prm, off, cnt, e_out);
  char *ws = reinterpret_cast<char *>(workspace);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const QuantArgs no_quant{nullptr, nullptr, nullptr, 0};
  if (T > MOE_ROUTE_MAX_FUSED_TOKENS) {
    LayoutArgs la;
    la.tile_m = tile_m;
    la.padded = padded_offsets;
    la.m_idx = m_indices;
    la.row_entry = row_entry;
    la.rows = rows;
    return route_launch(logits, bias, T, rp, o, ws, s, no_quant, la);
  }
  const int r = route_launch(logits, bias, T, rp, o, ws, s, no_quant);
  if (r != MOE_OK) return r;
  return moe_grouped_layout(o->counts, o->perm, e_out, n, tile_m, padded_offsets, m_indices,
                            row_entry, rows, stream);
}

// ---------------------------------------------------------------------------
// Allocation-free routing (moe_route_local_noalloc): the workspace is a
// static device array, one copy per GPU, held until the process ends. Host
// code never passes the array's name to a kernel (on the host it is only a
// stand-in for the symbol): its device address is looked up once per device
// with that device current and kept in noalloc_ptr[device].
// ---------------------------------------------------------------------------
constexpr size_t NOALLOC_BYTES = MOE_ROUTE_NOALLOC_SCRATCH_BYTES;
constexpr int NOALLOC_MAX_DEVICES = 64;
static_assert(NOALLOC_BYTES % 256 == 0 && NOALLOC_BYTES >= CONTROL_BYTES, "scratch size");

static __device__ __align__(256) uint8_t scratch[NOALLOC_BYTES];

static std::mutex noalloc_mu;
static char *noalloc_ptr[NOALLOC_MAX_DEVICES];

__global__ void clear_words_kernel(uint32_t *__restrict__ p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

// The current device's scratch address; the first call on a device looks it
// up and clears the control block on `st` (a fill kernel, so that a caller
// may capture the call in a graph).
static int noalloc_scratch(hipStream_t st, char **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(noalloc_mu);
  if (noalloc_ptr[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return MOE_ERR_HIP;
    clear_words_kernel<<<1, 64, 0, st>>>(reinterpret_cast<uint32_t *>(p),
                                         (int)(CONTROL_BYTES / sizeof(uint32_t)));
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
    noalloc_ptr[dev] = reinterpret_cast<char *>(p);
  }
  *out = noalloc_ptr[dev];
  return MOE_OK;
}

static int route_noalloc(const float *logits, const float *bias, int32_t T,
                         const moe_route_params *prm, int32_t off, int32_t cnt,
                         const moe_route_outputs *o, void *stream) {
  int e_out = 0;
  int st = validate_route_args(logits, bias, T, prm, off, cnt, o, &e_out);
  if (st != MOE_OK) return st;
  const RouteParams rp = route_params(prm, off, cnt, e_out);
  if (ws_layout(T, e_out, rp.K, rows_path_applies(rp, logits)).bytes > NOALLOC_BYTES)
    return MOE_ERR_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char *ws = nullptr;
  st = noalloc_scratch(s, &ws);
  if (st != MOE_OK) return st;
  return route_launch(logits, bias, T, rp, o, ws, s,
                      QuantArgs{nullptr, nullptr, nullptr, 0});
}

}  // namespace moe

extern "C" {

int32_t moe_route_abi_version(void) { return 101; }

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

int moe_route_local_grouped(const float *logits, const float *bias, int32_t num_tokens,
                            const moe_route_params *params, int32_t local_expert_offset,
                            int32_t num_local_experts, const moe_route_outputs *out,
                            int32_t tile_m, int32_t *padded_offsets, int32_t *m_indices,
                            int32_t *row_entry, int64_t rows, void *workspace,
                            size_t workspace_bytes, void *stream) {
  return moe::route_grouped_impl(logits, bias, num_tokens, params, local_expert_offset,
                                 num_local_experts, out, tile_m, padded_offsets, m_indices,
                                 row_entry, rows, workspace, workspace_bytes, stream);
}

int moe_route_local_noalloc(const float *logits, const float *bias, int32_t num_tokens,
                            const moe_route_params *params, int32_t local_expert_offset,
                            int32_t num_local_experts, const moe_route_outputs *out,
                            void *stream) {
  return moe::route_noalloc(logits, bias, num_tokens, params, local_expert_offset,
                            num_local_experts, out, stream);
}

int moe_route_quant_local(const float *logits, const float *bias, int32_t num_tokens,
                          const moe_route_params *params, int32_t local_expert_offset,
                          int32_t num_local_experts, const uint16_t *hidden_bf16,
                          int32_t hidden, uint8_t *act_q, uint8_t *act_scale,
                          const moe_route_outputs *out, void *workspace, size_t workspace_bytes,
                          void *stream) {
  if (hidden <= 0 || hidden % 32 != 0) return MOE_ERR_SHAPE;
  if (num_tokens > 0 && (!hidden_bf16 || !act_q || !act_scale)) return MOE_ERR_NULL;
  if (((uintptr_t)hidden_bf16 | (uintptr_t)act_q) % 16 != 0) return MOE_ERR_SHAPE;
  const int64_t nchunks = (int64_t)(num_tokens > 0 ? num_tokens : 0) * hidden / 8;
  if ((nchunks + moe::QUANT_CHUNKS_PER_BLOCK - 1) / moe::QUANT_CHUNKS_PER_BLOCK > INT32_MAX / 2)
    return MOE_ERR_SHAPE;
  const moe::QuantArgs qa{num_tokens > 0 ? hidden_bf16 : nullptr, act_q, act_scale, nchunks};
  return moe::route_impl(logits, bias, num_tokens, params, local_expert_offset,
                         num_local_experts, out, workspace, workspace_bytes, stream, qa);
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
    case 3: sym = &moe::g_rescored_tokens; break;
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

int64_t moe_grouped_layout_rows(int64_t n_entries, int32_t num_experts_out, int32_t tile_m) {
  if (n_entries < 0 || n_entries > MOE_GROUPED_MAX_ENTRIES) return MOE_ERR_SHAPE;
  if (num_experts_out < 1 || num_experts_out > MOE_ROUTE_MAX_EXPERTS) return MOE_ERR_SHAPE;
  if (tile_m < 1 || tile_m > MOE_GROUPED_MAX_TILE) return MOE_ERR_SHAPE;
  return n_entries + (int64_t)num_experts_out * (tile_m - 1);
}

int moe_grouped_layout(const int32_t *counts, const int32_t *perm, int32_t num_experts_out,
                       int64_t n_entries, int32_t tile_m, int32_t *padded_offsets,
                       int32_t *m_indices, int32_t *row_entry, int64_t rows, void *stream) {
  const int64_t need = moe_grouped_layout_rows(n_entries, num_experts_out, tile_m);
  if (need < 0) return (int)need;
  if (!counts || !padded_offsets || (n_entries > 0 && !perm)) return MOE_ERR_NULL;
  if (rows < need) return MOE_ERR_SHAPE;
  if (rows > 0 && !m_indices) return MOE_ERR_NULL;
  const int64_t per_block = (int64_t)moe::BLOCK * moe::LAYOUT_PER_THREAD;
  const int64_t grid = rows > 0 ? (rows + per_block - 1) / per_block : 1;
  if (grid > INT32_MAX) return MOE_ERR_SHAPE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  moe::grouped_layout_kernel<<<(int)grid, moe::BLOCK, 0, st>>>(
      counts, perm, num_experts_out, n_entries, tile_m, padded_offsets, m_indices, row_entry,
      rows);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_balance_plan(const int32_t *counts, int32_t num_experts, int32_t n_ranks,
                     int64_t n_entries, int32_t *dest, int32_t *rank_counts, void *stream) {
  if (n_ranks < 1 || n_ranks > moe::PLAN_MAX_RANKS) return MOE_ERR_SHAPE;
  if (num_experts < 1 || num_experts > MOE_ROUTE_MAX_EXPERTS || num_experts % n_ranks != 0)
    return MOE_ERR_SHAPE;
  if (n_entries < 0 || n_entries > MOE_GROUPED_MAX_ENTRIES) return MOE_ERR_SHAPE;
  if (!counts || !rank_counts || (n_entries > 0 && !dest)) return MOE_ERR_NULL;
  const int64_t per_block = (int64_t)moe::BLOCK * moe::PLAN_PER_THREAD;
  const int64_t grid = n_entries > 0 ? (n_entries + per_block - 1) / per_block : 1;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  moe::balance_plan_kernel<<<(int)grid, moe::BLOCK, 0, st>>>(counts, num_experts, n_ranks,
                                                             n_entries, dest, rank_counts);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
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
