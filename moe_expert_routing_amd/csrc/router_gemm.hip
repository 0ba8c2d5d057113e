// router_gemm.hip - router GEMM (logits = hidden . W^T) on the gfx950 matrix
// cores, then routing through moe_route_local.
//
// The router is a [num_experts, hidden] bf16 matrix replicated on every rank
// ("feat(kimi): tensor- and expert-parallel sharding for the K3.1 decoder",
// memory table: router 0.59 B parameters = 896 x 7168 x 92 layers). Both
// operands keep the hidden dimension contiguous, so each lane's MFMA operand
// is one 16-byte run of 8 bf16 along K.
//
// Kernel. A block of 4 or 8 waves computes a TM (tokens) x TN (experts)
// tile on the matrix cores; each wave owns a WM x WN sub-tile. K advances in stages
// of 64: each stage's A and B tiles go from global memory straight into LDS
// (global_load_lds_dwordx4, no register staging), NS stage buffers deep, so
// NS - 1 stages are in flight while one is consumed; the next stage's
// operand fragments are read from LDS while the current stage's MFMAs run.
// An LDS row holds 64 bf16 = 8 chunks of 16 bytes; chunk c of row r sits at
// position c ^ (r & 7), which makes every 8-lane group of a fragment read
// (8 rows, one chunk) hit 8 different bank quads.
//
// Shapes (v_mfma_f32_16x16x32_bf16, 4 stage buffers). Decode (T <= 128),
// bound by reading W once: 64 x 64 tiles, 4 waves of 32 x 32. Prefill:
// 128 x 128 tiles, 8 waves: each 64 x 64 wave tile is shared by two waves,
// one taking the first K step of every stage and one the second, summed
// through LDS at the end (two waves per SIMD, so that one wave's MFMAs run
// while the other waits on LDS or the barrier, and the LDS fragment reads
// per MFMA stay those of 64 x 64 tiles). (Measured on MI355X: 32x32x16 MFMA
// tiles, 4 waves of 64 x 64, 8 waves of 32 x 64, deeper or shallower stage
// rings, and operands loaded straight into registers without LDS were all
// slower here.) When
// the tiles do not fill the chip, K is split into S equal ranges; each
// writes its own fp32 partial and a second kernel sums the S partials in a
// fixed order, so the result does not depend on timing. Blocks are numbered
// so that the blocks the hardware places on one XCD (every 8th block) share
// operand rows in that XCD's L2. Logits are written, never accumulated into
// existing memory.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_route.h"
#include "internal.hpp"

namespace moe_gemm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void *lds_ptr_t;
typedef __attribute__((address_space(1))) void *gbl_ptr_t;

constexpr int TK = 64;          // K per stage (bf16): one 128-byte LDS row
constexpr int THREADS = 256;    // 4 waves
constexpr int MAX_SPLITS = 16;
constexpr int DECODE_MAX_T = 128;

template <int TM_, int TN_, int WM_, int WN_, int MF_, int NS_, int NW_ = 4, int KS_ = 1>
struct Tile {
  static constexpr int TM = TM_, TN = TN_, WM = WM_, WN = WN_;
  static constexpr int NW = NW_;    // waves per block
  static constexpr int KS = KS_;    // waves sharing one wave tile, each on part of every stage's K
  static constexpr int NTHREADS = 64 * NW;
  static constexpr int MF = MF_;    // MFMA tile: 16 (16x16x32) or 32 (32x32x16)
  static constexpr int NS = NS_;    // LDS stage buffers
  static constexpr int KMF = MF == 16 ? 32 : 16;  // K per MFMA
  static constexpr int KSTEPS = TK / KMF;
  static constexpr int KSW = KSTEPS / KS;  // MFMA K steps per wave and stage
  static_assert(KSW * KS == KSTEPS, "whole K steps per wave");
  static constexpr int WAVES_N = TN / WN;
  static constexpr int NWT = NW / KS;      // wave tiles per block
  static_assert((TM / WM) * (TN / WN) * KS == NW, "every wave tile on KS waves");
  static_assert(WM % MF == 0 && WN % MF == 0, "whole MFMA tiles");
  static constexpr int FM = WM / MF, FN = WN / MF;  // MFMA tiles per wave
  static constexpr int A_BYTES = TM * TK * 2, B_BYTES = TN * TK * 2;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  // one load instruction fills 8 LDS rows (64 lanes x 16 bytes)
  static constexpr int A_LOADS = TM / (8 * NW), B_LOADS = TN / (8 * NW);  // per wave per stage
  static_assert(A_LOADS * 8 * NW == TM && B_LOADS * 8 * NW == TN, "whole loads");
  static constexpr int LOADS = A_LOADS + B_LOADS;
  static_assert((NS - 2) * LOADS <= 63, "vmcnt range");
};
using DecodeTile = Tile<64, 64, 32, 32, 16, 4>;
using PrefillTile = Tile<128, 128, 64, 64, 16, 4, 8, 2>;

template <int MF>
struct MfmaAcc;
template <>
struct MfmaAcc<16> {
  typedef f32x4 type;
};
template <>
struct MfmaAcc<32> {
  typedef f32x16 type;
};

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// s_waitcnt vmcnt(n) for a run-time n in [0, MAXN] with the count encoded as
// an immediate.
template <int N>
__device__ __forceinline__ void wait_vmcnt_imm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
template <int STEP, int MAXK>
__device__ __forceinline__ void wait_vmcnt_steps(int k) {
  if constexpr (MAXK > 0) {
    if (k >= MAXK) {
      wait_vmcnt_imm<MAXK * STEP>();
      return;
    }
    wait_vmcnt_steps<STEP, MAXK - 1>(k);
  } else {
    wait_vmcnt_imm<0>();
  }
}

// Workgroup barrier that orders LDS accesses for the compiler without
// waiting for the stage loads still in flight (a __syncthreads() would wait
// for every outstanding load). Each wave first waits for its own LDS reads,
// so that no fragment read of a buffer is still pending when another wave's
// loads start refilling it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Tile index of this block: the hardware sends block b to XCD b % 8, so the
// blocks of one XCD take a contiguous run of tiles (same token rows, every
// expert tile) when the tile count is a multiple of 8.
__device__ __forceinline__ int tile_of_block(int b, int ntiles) {
  if (ntiles % 8 != 0) return b;
  return (b % 8) * (ntiles / 8) + b / 8;
}

template <class C>
__global__ __launch_bounds__(C::NTHREADS, 1) void router_gemm_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, float *__restrict__ Cout,
    int T, int E, int H, int k_per_split, int m_tiles, int n_tiles) {
  typedef typename MfmaAcc<C::MF>::type Acc;
  constexpr int NS = C::NS, MF = C::MF;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * C::STAGE_BYTES];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tile = tile_of_block(blockIdx.x, (int)gridDim.x);
  const int split = tile / (m_tiles * n_tiles);
  const int mt = (tile / n_tiles) % m_tiles, nt = tile % n_tiles;
  const int m0 = mt * C::TM, n0 = nt * C::TN, kbeg = split * k_per_split;
  const int nk = k_per_split / TK;
  float *Cs = Cout + (size_t)split * T * E;

  // Load q of this wave fills LDS rows R..R+7, R = (wave * LOADS_X + q) * 8;
  // lane i writes row R + i/8 at position i%8, which holds global chunk
  // (i%8) ^ (i/8). Rows past the last token read the last token's row.
  const int lr = lane >> 3, lchunk = (lane & 7) ^ lr;
  const uint16_t *a_src[C::A_LOADS];
  const uint16_t *b_src[C::B_LOADS];
#pragma unroll
  for (int q = 0; q < C::A_LOADS; ++q) {
    const int gm = min(m0 + (wave * C::A_LOADS + q) * 8 + lr, T - 1);
    a_src[q] = A + (size_t)gm * H + kbeg + lchunk * 8;
  }
#pragma unroll
  for (int q = 0; q < C::B_LOADS; ++q)
    b_src[q] = B + (size_t)(n0 + (wave * C::B_LOADS + q) * 8 + lr) * H + kbeg + lchunk * 8;

  auto issue = [&](int s) {
    uint8_t *base = smem + (s % NS) * C::STAGE_BYTES;
#pragma unroll
    for (int q = 0; q < C::A_LOADS; ++q)
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(a_src[q] + s * TK),
                                       (lds_ptr_t)(base + (wave * C::A_LOADS + q) * 1024), 16, 0,
                                       0);
#pragma unroll
    for (int q = 0; q < C::B_LOADS; ++q)
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(b_src[q] + s * TK),
                                       (lds_ptr_t)(base + C::A_BYTES +
                                                   (wave * C::B_LOADS + q) * 1024),
                                       16, 0, 0);
  };

  Acc acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int v = 0; v < (int)(sizeof(Acc) / sizeof(float)); ++v) acc[i][j][v] = 0.f;

  // wave tile wt, its part kh of each stage's K steps
  const int wt = wave % C::NWT, kh = wave / C::NWT;
  const int wm = (wt / C::WAVES_N) * C::WM, wn = (wt % C::WAVES_N) * C::WN;
  // operand lane layout: row lane % MF of the MFMA tile, K run lane / MF
  const int fr = lane % MF, fq = lane / MF;

  // Fragments of one stage in registers, two sets: the next stage's
  // fragments are read from LDS while the current stage's MFMAs run.
  bf16x8 fa[2][C::KSW][C::FM], fb[2][C::KSW][C::FN];
  auto read_frags = [&](int s, int set) {
    const uint8_t *As = smem + (s % NS) * C::STAGE_BYTES;
    const uint8_t *Bs = As + C::A_BYTES;
#pragma unroll
    for (int ks = 0; ks < C::KSW; ++ks) {
      const int pos = (((kh * C::KSW + ks) * (C::KMF / 8) + fq) ^ (fr & 7)) * 16;
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
        fa[set][ks][i] = *reinterpret_cast<const bf16x8 *>(As + (wm + MF * i + fr) * 128 + pos);
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
        fb[set][ks][j] = *reinterpret_cast<const bf16x8 *>(Bs + (wn + MF * j + fr) * 128 + pos);
    }
  };
  // Marks a register set's fragments as settled. stage_ready's wait (inside
  // inline asm, which the compiler's wait insertion cannot see) has already
  // drained their LDS reads; without this the compiler waits for every LDS
  // read in flight before the set's first MFMA, including the next stage's
  // fragment reads issued just before, so those could not overlap the MFMAs.
  auto settle = [&](int set) {
#pragma unroll
    for (int ks = 0; ks < C::KSW; ++ks) {
#pragma unroll
      for (int i = 0; i < C::FM; ++i) asm volatile("" : "+v"(fa[set][ks][i]));
#pragma unroll
      for (int j = 0; j < C::FN; ++j) asm volatile("" : "+v"(fb[set][ks][j]));
    }
  };
  auto mfmas = [&](int set) {
#pragma unroll
    for (int ks = 0; ks < C::KSW; ++ks)
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) acc[i][j] = mfma(fa[set][ks][i], fb[set][ks][j], acc[i][j]);
  };
  // Wait until stage s has landed (only the later stages' loads may still be
  // pending), then a barrier: every wave's part of stage s is in LDS, and
  // every wave has finished reading the buffer the next issue overwrites.
  auto stage_ready = [&](int s) {
    wait_vmcnt_steps<C::LOADS, NS - 2>(min(NS - 2, nk - 1 - s));
    stage_barrier();
    if (s + NS - 1 < nk) issue(s + NS - 1);
  };

#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) issue(s);
  stage_ready(0);
  read_frags(0, 0);
  // two stages per trip, so the register sets have constant indices
  int s = 0;
  for (; s + 1 < nk; s += 2) {
    stage_ready(s + 1);
    settle(0);
    read_frags(s + 1, 1);
    mfmas(0);
    if (s + 2 < nk) stage_ready(s + 2);
    settle(1);  // on both paths, so that the merge below carries no wait
    if (s + 2 < nk) read_frags(s + 2, 0);
    mfmas(1);
  }
  if (s < nk) mfmas(0);  // odd stage count: the last stage is in set 0

  if constexpr (C::KS == 2) {
    // The two waves of a wave tile summed in a fixed order (kh 0 + kh 1),
    // through the stage buffers: same accumulator layout in both, so each
    // lane adds the value at its own index.
    static_assert(C::NWT * C::FM * C::FN * (int)sizeof(Acc) * 64 <= NS * C::STAGE_BYTES,
                  "partials fit in the stage buffers");
    constexpr int NV = (int)(sizeof(Acc) / sizeof(float));
    float *red = reinterpret_cast<float *>(smem) + wt * (C::FM * C::FN * NV * 64);
    __syncthreads();  // every wave is done with the stage buffers
    if (kh == 1) {
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
          for (int v = 0; v < NV; ++v) red[((i * C::FN + j) * NV + v) * 64 + lane] = acc[i][j][v];
    }
    __syncthreads();
    if (kh == 1) return;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[i][j][v] += red[((i * C::FN + j) * NV + v) * 64 + lane];
  }

  // D of one MFMA tile: 16x16: row 4*(lane/16) + v, column lane % 16;
  // 32x32: row 8*(v/4) + 4*(lane/32) + v%4, column lane % 32.
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int v = 0; v < (int)(sizeof(Acc) / sizeof(float)); ++v) {
        const int r = MF == 16 ? 4 * fq + v : 8 * (v / 4) + 4 * fq + (v % 4);
        const int tm = m0 + wm + MF * i + r;
        if (tm < T) Cs[(size_t)tm * E + n0 + wn + MF * j + fr] = acc[i][j][v];
      }
}

// out[i] = sum over s = 0..S-1 of part[s][i], in that order; four
// consecutive values per thread, the S partial loads issued together.
__global__ __launch_bounds__(THREADS) void sum_splits_kernel(const float *__restrict__ part,
                                                             int S, int64_t n4,
                                                             float *__restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * THREADS + threadIdx.x;
  if (i >= n4) return;
  const float4 *p = reinterpret_cast<const float4 *>(part) + i;
  float4 v[MAX_SPLITS];
#pragma unroll
  for (int s = 0; s < MAX_SPLITS; ++s)
    if (s < S) v[s] = p[(size_t)s * n4];
  float4 acc = v[0];
#pragma unroll
  for (int s = 1; s < MAX_SPLITS; ++s)
    if (s < S) {
      acc.x += v[s].x;
      acc.y += v[s].y;
      acc.z += v[s].z;
      acc.w += v[s].w;
    }
  reinterpret_cast<float4 *>(out)[i] = acc;
}

struct Plan {
  bool decode;
  int m_tiles, n_tiles, splits;
};

// Tile shape by token count; then the K split: the largest divisor of
// H / TK (at most MAX_SPLITS) that keeps the grid at or below about 256
// blocks, one per compute unit.
static Plan make_plan(int T, int E, int H) {
  Plan pl;
  pl.decode = T <= DECODE_MAX_T;
  const int tm = pl.decode ? DecodeTile::TM : PrefillTile::TM;
  const int tn = pl.decode ? DecodeTile::TN : PrefillTile::TN;
  pl.m_tiles = (T + tm - 1) / tm;
  pl.n_tiles = E / tn;
  const int tiles = pl.m_tiles * pl.n_tiles;
  int want = 256 / (tiles > 0 ? tiles : 1);
  if (want > MAX_SPLITS) want = MAX_SPLITS;
  const int kb = H / TK;
  pl.splits = 1;
  for (int d = 1; d <= want; ++d)
    if (kb % d == 0) pl.splits = d;
  return pl;
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

static size_t partial_bytes(int T, int E, int H) {
  const int S = make_plan(T, E, H).splits;
  return S > 1 ? align256((size_t)S * T * E * sizeof(float)) : 0;
}

}  // namespace moe_gemm

extern "C" {

size_t moe_router_gemm_route_workspace_bytes(int32_t num_tokens, int32_t hidden,
                                             int32_t num_experts, int32_t num_experts_out,
                                             int32_t top_k) {
  if (num_tokens < 0 || hidden <= 0 || num_experts <= 0 || num_experts_out <= 0 || top_k <= 0)
    return 0;
  const size_t r = (moe_route_workspace_bytes(num_tokens, num_experts_out, top_k) + 255) &
                   ~(size_t)255;
  if (hidden % moe_gemm::TK != 0 || num_experts % moe_gemm::PrefillTile::TN != 0) return r;
  return r + moe_gemm::partial_bytes(num_tokens, num_experts, hidden);
}

int moe_router_gemm_route(const uint16_t *hidden_bf16, const uint16_t *weight_bf16,
                          int32_t num_tokens, int32_t hidden, const float *bias,
                          float *logits_out, const moe_route_params *params,
                          int32_t local_expert_offset, int32_t num_local_experts,
                          const moe_route_outputs *out, void *workspace, size_t workspace_bytes,
                          void *stream) {
  using namespace moe_gemm;
  if (!params || !out) return MOE_ERR_NULL;
  const int T = num_tokens, H = hidden, E = params->num_experts;
  if (T < 0 || H <= 0 || E <= 0 || params->top_k <= 0) return MOE_ERR_SHAPE;
  if (H % TK != 0 || E % PrefillTile::TN != 0) return MOE_ERR_UNSUPPORTED;
  if (T > 0 && (!hidden_bf16 || !weight_bf16 || !logits_out)) return MOE_ERR_NULL;
  if (((uintptr_t)hidden_bf16 | (uintptr_t)weight_bf16 | (uintptr_t)logits_out) % 16 != 0)
    return MOE_ERR_SHAPE;
  if ((uintptr_t)workspace % 16 != 0) return MOE_ERR_WORKSPACE;
  const int32_t e_local =
      moe_route_local_num_experts(E, params->top_k, local_expert_offset, num_local_experts);
  if (e_local < 0) return e_local;
  const int e_out = e_local > 0 ? e_local : E;
  const size_t need = moe_router_gemm_route_workspace_bytes(T, H, E, e_out, params->top_k);
  if (!workspace) return MOE_ERR_WORKSPACE;
  if (workspace_bytes < need) return MOE_ERR_WORKSPACE;
  // the routing arguments are checked before anything is launched
  const int vst = moe::validate_route_call(logits_out, bias, T, params, local_expert_offset,
                                           num_local_experts, out, workspace, workspace_bytes,
                                           nullptr);
  if (vst != MOE_OK) return vst;
  const size_t route_bytes = (moe_route_workspace_bytes(T, e_out, params->top_k) + 255) &
                             ~(size_t)255;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (T > 0) {
    const Plan pl = make_plan(T, E, H);
    const int S = pl.splits;
    float *dst = S > 1 ? reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) +
                                                   route_bytes)
                       : logits_out;
    const int blocks = pl.m_tiles * pl.n_tiles * S;
    if (pl.decode)
      router_gemm_kernel<DecodeTile><<<blocks, DecodeTile::NTHREADS, 0, st>>>(
          hidden_bf16, weight_bf16, dst, T, E, H, H / S, pl.m_tiles, pl.n_tiles);
    else
      router_gemm_kernel<PrefillTile><<<blocks, PrefillTile::NTHREADS, 0, st>>>(
          hidden_bf16, weight_bf16, dst, T, E, H, H / S, pl.m_tiles, pl.n_tiles);
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
    if (S > 1) {
      const int64_t n4 = (int64_t)T * E / 4;
      const int64_t g = (n4 + THREADS - 1) / THREADS;
      sum_splits_kernel<<<(int)g, THREADS, 0, st>>>(dst, S, n4, logits_out);
      if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
    }
  }
  return moe_route_local(logits_out, bias, T, params, local_expert_offset, num_local_experts,
                         out, workspace, route_bytes, stream);
}

}  // extern "C"
