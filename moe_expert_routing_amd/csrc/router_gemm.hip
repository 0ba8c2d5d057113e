// router_gemm.hip - router GEMM (logits = hidden . W^T) on the gfx950 matrix
// cores, then routing through moe_route_local.
//
// The router is a [num_experts, hidden] bf16 matrix replicated on every rank
// ("feat(kimi): tensor- and expert-parallel sharding for the K3.1 decoder",
// memory table: router 0.59 B parameters = 896 x 7168 x 92 layers). Both
// operands keep the hidden dimension contiguous, so each lane's MFMA operand
// is one 16-byte run of 8 bf16 along K.
//
// Tiling: a block of 4 waves computes a 64 (tokens) x 64 (experts) tile;
// each wave owns 32 x 32 = 2 x 2 tiles of v_mfma_f32_16x16x32_bf16. K is
// staged through LDS in steps of 64. When there are too few tiles to fill the
// chip (decode), K is split into S equal ranges; each writes its own fp32
// partial and a second kernel sums the S partials in a fixed order, so the
// result does not depend on timing. Logits are written, never accumulated
// into existing memory.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_route.h"
#include "internal.hpp"

namespace moe_gemm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 64, BN = 64, BK = 64;
constexpr int THREADS = 256;
constexpr int LDS_STRIDE = BK + 8;  // bf16 elements per LDS row (16-byte pad)
constexpr int MAX_SPLITS = 16;

// Pick the K split: the largest divisor of H/BK not above the count that
// brings the grid to about 512 blocks (at most MAX_SPLITS).
static int pick_splits(int T, int E, int H) {
  const int mt = (T + BM - 1) / BM, nt = E / BN;
  const int tiles = mt * nt;
  int want = (512 + tiles - 1) / tiles;
  if (want > MAX_SPLITS) want = MAX_SPLITS;
  const int kb = H / BK;
  int s = 1;
  for (int d = 1; d <= want; ++d)
    if (kb % d == 0) s = d;
  return s;
}

__global__ __launch_bounds__(THREADS) void router_gemm_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, float *__restrict__ C,
    int T, int E, int H, int k_per_split) {
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDS_STRIDE];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * BN;
  const int m0 = blockIdx.y * BM;
  const int split = blockIdx.z;
  const int kbeg = split * k_per_split;
  float *Cs = C + (size_t)split * T * E;

  // global -> LDS: 64 rows x 128 bytes per operand = 512 16-byte pieces,
  // two per thread.
  const int lr = tid >> 3;         // 0..31
  const int lc = (tid & 7) * 8;    // bf16 column of the 16-byte piece
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
  const int fr = lane & 15, fk = (lane >> 4) * 8;

  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 ra[2], rb[2];
  auto gload = [&](int k0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = lr + 32 * h;
      const int tm = m0 + r;
      ra[h] = tm < T ? *reinterpret_cast<const uint4 *>(A + (size_t)tm * H + k0 + lc)
                     : make_uint4(0u, 0u, 0u, 0u);
      rb[h] = *reinterpret_cast<const uint4 *>(B + (size_t)(n0 + r) * H + k0 + lc);
    }
  };
  gload(kbeg);
  for (int k0 = kbeg; k0 < kbeg + k_per_split; k0 += BK) {
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = lr + 32 * h;
      *reinterpret_cast<uint4 *>(&As[r * LDS_STRIDE + lc]) = ra[h];
      *reinterpret_cast<uint4 *>(&Bs[r * LDS_STRIDE + lc]) = rb[h];
    }
    __syncthreads();
    if (k0 + BK < kbeg + k_per_split) gload(k0 + BK);  // overlap with the MFMAs
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8 *>(&As[(wm + 16 * i + fr) * LDS_STRIDE + kk + fk]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const bf16x8 *>(&Bs[(wn + 16 * j + fr) * LDS_STRIDE + kk + fk]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
  // D[m = 4*(lane/16) + v][n = lane % 16] of each 16x16 tile
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int tm = m0 + wm + 16 * i + 4 * (lane >> 4) + v;
        const int en = n0 + wn + 16 * j + (lane & 15);
        if (tm < T) Cs[(size_t)tm * E + en] = acc[i][j][v];
      }
}

// out[i] = sum over s = 0..S-1 of part[s][i], in that order.
__global__ __launch_bounds__(THREADS) void sum_splits_kernel(const float *__restrict__ part,
                                                             int S, int64_t n,
                                                             float *__restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * THREADS + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * THREADS) {
    float acc = part[i];
    for (int s = 1; s < S; ++s) acc += part[(size_t)s * n + i];
    out[i] = acc;
  }
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

static size_t partial_bytes(int T, int E, int H) {
  const int S = pick_splits(T, E, H);
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
  if (hidden % moe_gemm::BK != 0 || num_experts % moe_gemm::BN != 0) return r;
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
  if (H % BK != 0 || E % BN != 0) return MOE_ERR_UNSUPPORTED;
  if (T > 0 && (!hidden_bf16 || !weight_bf16 || !logits_out)) return MOE_ERR_NULL;
  if (((uintptr_t)hidden_bf16 | (uintptr_t)weight_bf16) % 16 != 0) return MOE_ERR_SHAPE;
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
    const int S = pick_splits(T, E, H);
    float *dst = S > 1 ? reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) +
                                                   route_bytes)
                       : logits_out;
    dim3 grid(E / BN, (T + BM - 1) / BM, S);
    router_gemm_kernel<<<grid, THREADS, 0, st>>>(hidden_bf16, weight_bf16, dst, T, E, H, H / S);
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
    if (S > 1) {
      const int64_t n = (int64_t)T * E;
      int64_t g = (n + THREADS * 4 - 1) / (THREADS * 4);
      if (g > 4096) g = 4096;
      sum_splits_kernel<<<(int)g, THREADS, 0, st>>>(dst, S, n, logits_out);
      if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
    }
  }
  return moe_route_local(logits_out, bias, T, params, local_expert_offset, num_local_experts,
                         out, workspace, route_bytes, stream);
}

}  // extern "C"
