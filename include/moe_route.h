/*
 * moe_route.h - C ABI of the MI355X (gfx950) routed-MoE routing library.
 *
 * The library computes, per token, the routing step of a large-expert routed
 * MoE: a sigmoid router with a correction bias and a grouped top-k ("[ROCm]
 * [Perf] Kimi-K3: token-sharded residual stream for long prefills", author's
 * reply on shard-routed test coverage), the renormalised weights, the packed
 * routed entries (expert id in bits 31..16, bf16 weight in bits 15..0) with
 * the optional rank-local relabel of the pack epilogue, and the per-expert
 * counts, exclusive offsets and expert-major permutation that the expert
 * GEMMs consume ("[kimi-k3] Rank-local expert ids for the EP routed MoE
 * (upstream #45544)", commit message, passages on the fused route+quant
 * launch and its plumbing).
 *
 * Conventions shared by every entry point:
 *  - Tensor pointers are DEVICE pointers owned by the caller; buffers are
 *    row-major and contiguous. The library allocates nothing.
 *  - `stream` is a hipStream_t (NULL = the null stream). Calls are
 *    asynchronous on it: no host synchronisation, no device-to-host reads.
 *  - Arguments are validated on the host before anything is launched. On a
 *    negative return nothing has been written.
 *  - Logits must be finite; NaN or infinity is outside the contract and is
 *    not detected.
 *  - Results are deterministic: the same inputs give the same bits on every
 *    call, and no atomic operation decides an order.
 */
#ifndef MOE_ROUTE_H
#define MOE_ROUTE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Largest token count routed by the single-launch decode path (the fused
 * launch's token cap on the pages is 64 tokens, and that cap is public).
 * Larger calls run the tiled prefill path; both give identical results. */
#define MOE_ROUTE_MAX_FUSED_TOKENS 64

/* Envelope of the kernels (outside it calls return MOE_ERR_UNSUPPORTED):
 * num_experts a multiple of 128 and at most 1024; n_groups a power of two
 * with 1 <= n_groups <= 64; 1 <= topk_group <= n_groups;
 * 1 <= top_k <= min(32, topk_group * num_experts / n_groups);
 * group_topn 1 or 2. */
#define MOE_ROUTE_MAX_EXPERTS 1024
#define MOE_ROUTE_MAX_TOPK 32

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,        /* a required pointer is NULL                    */
  MOE_ERR_SHAPE = -2,       /* negative size, or shape inconsistent          */
  MOE_ERR_RANGE = -3,       /* expert range outside [0, num_experts)         */
  MOE_ERR_UNSUPPORTED = -4, /* parameters outside the kernels' envelope      */
  MOE_ERR_WORKSPACE = -5,   /* workspace missing or too small                */
  MOE_ERR_HIP = -6          /* a HIP launch failed                           */
} moe_status;

/* Routing parameters. The workload on the pages: 896 experts, top_k 16;
 * grouping 8 groups of 112, keep 4, group score = sum of the group's top 2
 * biased scores. */
typedef struct moe_route_params {
  int32_t num_experts; /* E                                                 */
  int32_t n_groups;    /* G: groups of E/G consecutive experts              */
  int32_t topk_group;  /* groups kept per token                             */
  int32_t top_k;       /* K: experts selected per token                     */
  int32_t group_topn;  /* group score = fp32 sum of the group's top n sp    */
} moe_route_params;

/* Output buffers. E' is the output id space: num_experts for global ids,
 * or moe_route_local_num_experts(...) when a rank range applies. */
typedef struct moe_route_outputs {
  int32_t *topk_ids;     /* [T, K] global expert ids, slot k = k-th best     */
  float *topk_weights;   /* [T, K] s_k / sum_j s_j, s = unbiased sigmoid     */
  int32_t *packed;       /* [T, K] (id' << 16) | bf16_rne(weight)            */
  int32_t *counts;       /* [E'] entries per output id                       */
  int32_t *offsets;      /* [E' + 1] exclusive offsets, offsets[E'] = T*K    */
  int32_t *perm;         /* [T*K] expert-major position -> flat index t*K+k  */
  int32_t *inv_perm;     /* [T*K] flat index -> position (may be NULL)       */
} moe_route_outputs;

/*
 * Output id space of a rank range: round_up(num_local_experts + top_k, 4)
 * when the range [local_expert_offset, local_expert_offset +
 * num_local_experts) is a proper sub-range that shrinks the routing problem
 * (0 < count, and the rounded size is below num_experts); 0 when it does not
 * apply (global ids are kept). The rank-local relabel and the local problem
 * size are stated in "[kimi-k3] Rank-local expert ids for the EP routed MoE
 * (upstream #45544)", commit message (128 at EP8 for 896 experts, top_k 16).
 * Returns MOE_ERR_RANGE for a range outside [0, num_experts) and
 * MOE_ERR_SHAPE for num_experts <= 0 or top_k <= 0.
 */
int32_t moe_route_local_num_experts(int32_t num_experts, int32_t top_k,
                                    int32_t local_expert_offset,
                                    int32_t num_local_experts);

/*
 * Workspace bytes needed by moe_route / moe_route_local for `num_tokens`
 * tokens and `num_experts_out` output ids (E'): a 256-byte control block
 * and, above 64 tokens, the permutation's per-block id counts and in-block
 * ranks. The control block must be zero before the workspace is first used;
 * every call leaves it zero again. The rest needs no initial contents. One
 * workspace must not be used by two calls that can run at the same time.
 */
size_t moe_route_workspace_bytes(int32_t num_tokens, int32_t num_experts_out,
                                 int32_t top_k);

/*
 * Route T tokens with global ids (E' = num_experts): the routing of the
 * fused route launch with no rank range, which keeps the global ids in the
 * packed output ("[kimi-k3] Rank-local expert ids for the EP routed MoE
 * (upstream #45544)", commit message, the Plumbing passage: the range
 * arguments are optional and 0 keeps the global ids).
 *   logits   [T, E] fp32 router logits
 *   bias     [E]    fp32 correction bias (added for selection only)
 * Writes every buffer of `out`. T = 0 writes zero counts and offsets.
 * T * top_k above 2^31 - 1 -> MOE_ERR_SHAPE (entries and positions are int32).
 * Returns MOE_OK or a negative moe_status.
 */
int moe_route(const float *logits, const float *bias, int32_t num_tokens,
              const moe_route_params *params, const moe_route_outputs *out,
              void *workspace, size_t workspace_bytes, void *stream);

/*
 * Route T tokens for one expert-parallel rank range ("[kimi-k3] Rank-local
 * expert ids for the EP routed MoE (upstream #45544)", commit message: the
 * pack epilogue's relabel, and the Plumbing passage, where the optional
 * (local_expert_offset, num_local_experts) pair changes the packed output
 * only and 0 keeps the global ids). Identical to moe_route
 * except for the packed ids and the permutation space: when the range
 * applies (moe_route_local_num_experts > 0), experts of the range are
 * written as id - local_expert_offset, and any other expert chosen in top-k
 * slot k as num_local_experts + k (unique within a row); counts, offsets and
 * perm cover the E' = round_up(count + top_k, 4) output ids. topk_ids stay
 * global. num_local_experts = 0 keeps global ids.
 */
int moe_route_local(const float *logits, const float *bias,
                    int32_t num_tokens, const moe_route_params *params,
                    int32_t local_expert_offset, int32_t num_local_experts,
                    const moe_route_outputs *out, void *workspace,
                    size_t workspace_bytes, void *stream);

/*
 * Allocation-free moe_route_local, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same arguments, checks and results as moe_route_local,
 * without the workspace: the control block and the permutation's tile counts
 * and ranks live in a static device array of MOE_ROUTE_NOALLOC_SCRATCH_BYTES,
 * one copy per GPU, which the library holds until the process ends. Nothing
 * is allocated, by the library or by any routine it calls. The first call on
 * a device looks up that device's copy (the current device must be the
 * stream's) and clears its control block on `stream`; every call leaves the
 * control block zero again. All calls on one GPU share the array: calls that
 * can overlap on one GPU (other streams, other threads) race and give wrong
 * results; serialise them.
 * A call whose scratch need exceeds the array returns MOE_ERR_WORKSPACE
 * before any launch. The need is below moe_route_workspace_bytes(T, E', K);
 * for 896 experts in 8 groups, top_k <= 16 and 16-byte aligned logits it is
 * 256 + 4 E' * 16 ceil(T / 256) + T * top_k bytes (256-byte aligned parts),
 * which admits up to 69,888 tokens with global ids (E' = 896).
 */
#define MOE_ROUTE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int moe_route_local_noalloc(const float *logits, const float *bias, int32_t num_tokens,
                            const moe_route_params *params, int32_t local_expert_offset,
                            int32_t num_local_experts, const moe_route_outputs *out,
                            void *stream);

/*
 * Workspace bytes needed by moe_router_gemm_route: the routing workspace
 * first (moe_route_workspace_bytes, same control-block rule), then the
 * router GEMM's split-K partial sums.
 */
size_t moe_router_gemm_route_workspace_bytes(int32_t num_tokens, int32_t hidden,
                                             int32_t num_experts,
                                             int32_t num_experts_out,
                                             int32_t top_k);

/*
 * Router GEMM followed by routing: logits = hidden . W^T with bf16 operands
 * and fp32 accumulation on the matrix cores, then moe_route_local on them.
 * The router is a [num_experts, hidden] matrix replicated on every rank
 * ("feat(kimi): tensor- and expert-parallel sharding for the K3.1 decoder",
 * memory table: router 0.59 B parameters).
 *   hidden_bf16 [T, H] bf16 bit patterns, weight_bf16 [E, H] bf16 bit
 *   patterns, H a multiple of 64; logits_out [T, E] fp32 (required: the
 *   routing reads the logits from it). hidden_bf16, weight_bf16 and
 *   logits_out must be 16-byte aligned (else MOE_ERR_SHAPE), the workspace
 *   too (else MOE_ERR_WORKSPACE). The accumulation order along H depends on
 *   the token count (K is split when the tiles do not fill the device), not
 *   on timing: the same inputs give the same logits on every call.
 */
int moe_router_gemm_route(const uint16_t *hidden_bf16,
                          const uint16_t *weight_bf16, int32_t num_tokens,
                          int32_t hidden, const float *bias, float *logits_out,
                          const moe_route_params *params,
                          int32_t local_expert_offset,
                          int32_t num_local_experts,
                          const moe_route_outputs *out, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * Fused route + activation quantisation ("[kimi-k3] Rank-local expert ids
 * for the EP routed MoE (upstream #45544)", commit message: the fused
 * route+quant launch for decode batches up to MAX_TOKENS, whose routed MoE
 * runs MXFP4 expert weights). Routes exactly as moe_route_local and
 * quantises the activations to OCP MXFP8 (the pages do not name the
 * activation format; this is the reading taken):
 *   hidden_bf16 [T, H] bf16 bit patterns, H a multiple of 32;
 *   act_q [T, H] E4M3 codes: element v -> E4M3(v * 2^-shared), round to
 *       nearest even, saturating at +-448;
 *   act_scale [T, H/32] E8M0 codes: shared + 127 with shared =
 *       max(floor(log2(max |v| of the 32-element block)) - 8, -127), and
 *       -127 for a block of zeros.
 * For T <= MOE_ROUTE_MAX_FUSED_TOKENS everything runs in ONE launch (the
 * quantisation blocks run beside the routing blocks); above it the
 * quantisation is one more launch before the routing. hidden_bf16 and act_q
 * must be 16-byte aligned (else MOE_ERR_SHAPE); H not a positive multiple
 * of 32 -> MOE_ERR_SHAPE; NULL activation pointers with T > 0 ->
 * MOE_ERR_NULL; every routing argument is checked as by moe_route_local,
 * all before any launch.
 */
int moe_route_quant_local(const float *logits, const float *bias, int32_t num_tokens,
                          const moe_route_params *params, int32_t local_expert_offset,
                          int32_t num_local_experts, const uint16_t *hidden_bf16,
                          int32_t hidden, uint8_t *act_q, uint8_t *act_scale,
                          const moe_route_outputs *out, void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * Grouped-GEMM layout of a routing call's entries, the index arrays a
 * contiguous grouped GEMM over the experts consumes (an expert-parallel
 * backend builds them after routing: "Add MoonEP expert-parallel arm of the
 * Kimi-K3 B300 agentic sweep", review summary of the patch, its
 * prepare/finalize step). From counts [E'] and perm [n_entries] of one
 * routing call (same stream, so the call has finished writing them):
 *   padded_offsets [E'+1]: padded[0] = 0, padded[e+1] = padded[e] +
 *       round_up(counts[e], tile_m);
 *   m_indices [rows]: row padded[e] + j holds id e for j < counts[e] and -1
 *       on the padding rows after it; rows from padded[E'] on are -1;
 *   row_entry [rows] (nullable): the flat entry f = t*K + k of each real
 *       row, perm[offsets[e] + j] (ascending within an id), -1 elsewhere.
 * rows must be at least moe_grouped_layout_rows(n_entries, E', tile_m), the
 * padded total when every id wastes tile_m - 1 rows (the actual total,
 * padded[E'], is only known on the device). Device pointers owned by the
 * caller; asynchronous on stream; nothing is allocated. Checked on the host
 * before any launch: NULL pointers (perm may be NULL when n_entries == 0,
 * m_indices when rows == 0) -> MOE_ERR_NULL; 1 <= E' <= 1024,
 * 1 <= tile_m <= MOE_GROUPED_MAX_TILE, 0 <= n_entries <=
 * MOE_GROUPED_MAX_ENTRIES, rows too small -> MOE_ERR_SHAPE. counts must
 * sum to n_entries (as a routing call's do); if they do not, the rows are
 * wrong but every access stays inside the arrays.
 */
#define MOE_GROUPED_MAX_TILE 4096
#define MOE_GROUPED_MAX_ENTRIES (1 << 30)
int64_t moe_grouped_layout_rows(int64_t n_entries, int32_t num_experts_out, int32_t tile_m);
int moe_grouped_layout(const int32_t *counts, const int32_t *perm, int32_t num_experts_out,
                       int64_t n_entries, int32_t tile_m, int32_t *padded_offsets,
                       int32_t *m_indices, int32_t *row_entry, int64_t rows, void *stream);

/*
 * moe_route_local and the grouped-GEMM layout of its entries in one call:
 * every output of moe_route_local, and padded_offsets, m_indices and
 * row_entry exactly as moe_grouped_layout computes them from that call's
 * counts and perm (the layout the expert GEMM consumes, "[Kernel] Enable
 * Kimi-K3 SiTU on the CuteDSL MoE backend and the SM107 low-latency GEMM
 * plan", the m_indices of its grouped GEMM). Above MOE_ROUTE_MAX_FUSED_TOKENS
 * the routing's own permutation kernel writes the layout as it places the
 * entries, so the layout costs no launch of its own; at decode sizes the
 * layout kernel follows the single routing launch. Arguments, workspace and
 * checks are those of moe_route_local and moe_grouped_layout (with n_entries
 * = T * top_k and num_experts_out = E' of the call), all made on the host
 * before any launch.
 */
int moe_route_local_grouped(const float *logits, const float *bias, int32_t num_tokens,
                            const moe_route_params *params, int32_t local_expert_offset,
                            int32_t num_local_experts, const moe_route_outputs *out,
                            int32_t tile_m, int32_t *padded_offsets, int32_t *m_indices,
                            int32_t *row_entry, int64_t rows, void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * Static per-rank balancing plan for an expert-parallel dispatch that holds
 * every rank at the same number of routed entries by moving the surplus of
 * overloaded expert owners ("Add MoonEP expert-parallel arm of the Kimi-K3
 * B300 agentic sweep", PR description; the pages give the goal, this is the
 * plan taken). From counts [E] of one routing call with GLOBAL ids (n_entries
 * = T*K, counts summing to it) and n_ranks ranks owning the experts in
 * contiguous ranges of E / n_ranks:
 *   target[r] = n_entries / n_ranks, +1 for the first n_entries % n_ranks;
 *   rank r keeps the first min(load[r], target[r]) of its own entries in
 *   expert-major order (the order of perm); the remaining entries of every
 *   overloaded rank, in rank order, are handed out in consecutive runs to the
 *   ranks below target, in rank order, until each holds its target.
 *   dest [n_entries]: the rank that processes the p-th entry of perm;
 *   rank_counts [n_ranks][E]: entries of expert e processed on rank r.
 * Device pointers owned by the caller; asynchronous on stream; nothing
 * allocated. Checked on the host before any launch: 1 <= n_ranks <= 64,
 * 1 <= E <= 1024 with E % n_ranks == 0, 0 <= n_entries <=
 * MOE_GROUPED_MAX_ENTRIES (else MOE_ERR_SHAPE); NULL counts / rank_counts,
 * or NULL dest with n_entries > 0 -> MOE_ERR_NULL. Counts that do not sum
 * to n_entries give a wrong plan but no access outside the arrays.
 */
int moe_balance_plan(const int32_t *counts, int32_t num_experts, int32_t n_ranks,
                     int64_t n_entries, int32_t *dest, int32_t *rank_counts, void *stream);

/*
 * Diagnostic: y[i] = the binary32 nearest to 1 / (1 + e^-x[i]) for n
 * elements, with the routing kernels' own sigmoid. mode 0 = the production
 * evaluation; mode 1 = the double-double re-evaluation only (the path taken
 * near binary32 rounding boundaries), so that tests can reach it; mode 2 =
 * the fast hardware approximation the kernels use to pick candidates (NOT
 * correctly rounded: its error bound is what tests check).
 */
int moe_sigmoid_rn32(const float *x, float *y, int64_t n, int32_t mode,
                     void *stream);

/*
 * Benchmark hook. When `before` and `after` are hipEvent_t handles, every
 * later routing call records `before` on its stream just before its first
 * routing kernel (the per-token route kernel: the single kernel of the
 * decode path, the tile kernel of the prefill path) and `after` just after
 * it. NULL, NULL turns recording off. Process-wide and not thread-safe; it
 * exists so that a benchmark can time that kernel on its own stream.
 */
int moe_route_set_kernel_events(void *before, void *after);

/*
 * Diagnostic: number of tokens routed through the exact path (the fast path
 * could not prove its answer) since the last reset, summed over calls on the
 * current device. Synchronises with the device. reset != 0 zeroes the count.
 * Returns the count or MOE_ERR_HIP.
 */
int64_t moe_route_exact_path_tokens(int32_t reset);

/*
 * Diagnostic: tokens per kernel path since the last reset, summed over calls
 * on the current device. Synchronises with the device.
 *   path 0: the one-token-per-wave exact pipeline (as
 *           moe_route_exact_path_tokens);
 *   path 1: the exact refinement of the four-tokens-per-wave prefill path
 *           (896 experts, 8 groups, top_k <= 16, more than 64 tokens), taken
 *           when its fast certificate does not hold;
 *   path 2: tokens of that path routed again one token per wave because the
 *           refinement could not decide either;
 *   path 3: tokens of the one-token-per-wave fast path whose candidates were
 *           scored again exactly because the certificate on approximate
 *           candidate scores did not hold (near-ties among the candidates).
 * reset != 0 zeroes that path's count. Returns the count, MOE_ERR_UNSUPPORTED
 * for another path, or MOE_ERR_HIP.
 */
int64_t moe_route_path_tokens(int32_t path, int32_t reset);

/* Human-readable name of a moe_status value. */
const char *moe_route_status_string(int status);

/* ABI version of this header (major * 100 + minor). */
int32_t moe_route_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ROUTE_H */
