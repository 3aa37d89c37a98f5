/*
 * ep_get.h -- C ABI of the MI355X (gfx950) MoE expert-parallel dispatch /
 * combine library, single GPU, with the EP ranks as virtual partitions of one
 * GPU's memory.
 *
 * What the operations are (cited by page title and section):
 *   - DeepEP walkthrough (2kiu.com news 5702702), sec. 2.1: an MoE layer moves
 *     tokens in two steps, dispatch (token to the holders of its top-k
 *     experts) and combine (expert results back to the token's origin);
 *     sec. 2.3: the dispatched payload may be quantised to FP8 to halve its
 *     bytes; sec. 4.1: communication buffers are allocated once and reused.
 *   - Lesson 14 "DeepSeek DeepEP core architecture and MoE expert-parallel
 *     communication operators" (hsthanb4 hpclearning), sec. 3 and the practice
 *     task: dispatch fills per-expert queues in token order; combine sums
 *     weight * expert output over the token's top-k choices.
 *   - DeepEP book ch.1 "positioning and version boundaries" (bowenzhou.top),
 *     sec. 1.4: the V1 dispatch consumes a layout (num_tokens_per_rank,
 *     is_token_in_rank, num_tokens_per_expert) and an expert_alignment, and
 *     hands back per-expert receive counts and a handle that combine uses;
 *     sec. 1.1: the V2 dispatch takes num_experts, expert_alignment and can
 *     reuse a handle.
 *   - DeepEP EP all-to-all analysis (hotdry blog), section on buffer
 *     engineering: fixed buffers sized for the worst case are the simple,
 *     deadlock-free choice; the experts must divide evenly over the ranks.
 *
 * Conventions shared by every call:
 *   - All array arguments are DEVICE pointers unless noted; the caller owns
 *     every buffer.  The library never allocates, frees, memsets or waits on
 *     device memory (ep_layout_error is the one synchronous call).
 *   - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *     Calls only enqueue work on it and return, so they can be captured into a
 *     HIP graph.
 *   - Token t belongs to virtual source rank t / (N/R); expert e lives on rank
 *     e / (E/R).  Slots of one expert are contiguous, ordered by (source rank,
 *     token, k), and each expert region is padded to a multiple of
 *     expert_alignment.  The handle that combine needs is slot_of (plus the
 *     caller's topk_weights); it stays valid for any number of dispatch /
 *     combine calls with the same routing.
 *   - Return values: EP_OK, or an EP_ERR_* code.  Argument checks run on the
 *     host only and never synchronise.  No C++ exception crosses this ABI.
 *   - The library keeps no mutable global state besides per-device caches of
 *     the architecture check, the LDS size and the scratch address, and the
 *     static scratch array of ep_get_layout_noalloc; concurrent calls need
 *     distinct workspaces.
 *   - Set EP_GET_LOG=1 in the environment to print launch shapes to stderr.
 */
#ifndef EP_GET_H
#define EP_GET_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  EP_OK = 0,
  EP_ERR_INVALID_ARG = 1, /* a size, pointer or divisibility rule is violated      */
  EP_ERR_CAPACITY = 2,    /* recv_capacity below ep_recv_capacity()                */
  EP_ERR_HIP = 3,         /* a HIP launch or copy failed (logged with EP_GET_LOG)  */
  EP_ERR_UNSUPPORTED = 4, /* the current device is not gfx950                      */
  EP_ERR_SCRATCH = 5      /* ep_get_layout_noalloc: workspace above its scratch     */
};

/* Compile-time limits of the library. */
#define EP_MAX_EXPERTS 1024
#define EP_MAX_RANKS 256
#define EP_MAX_TOPK 32
#define EP_MAX_HIDDEN (1 << 24)

/* Bits of the device error word read by ep_layout_error, and of the
 * per-source flags of ep_ll_dispatch. */
#define EP_LAYOUT_ERR_INDEX 1    /* some topk_idx entry was outside [-1, E)        */
#define EP_LAYOUT_ERR_OVERFLOW 2 /* ep_ll_dispatch: a sub-block had more than M pairs */

/* Problem descriptor (host memory, read during the call only).
 *   num_tokens        N >= 0, all virtual source ranks together, N % R == 0
 *   hidden            H, 1..EP_MAX_HIDDEN, H % 8 == 0; H % 128 == 0 when
 *                     use_fp8 (the kernels index a row's bytes in 32 bits)
 *   num_topk          K, 1..EP_MAX_TOPK
 *   num_experts       E, 1..EP_MAX_EXPERTS, E % R == 0 (the experts divide
 *                     evenly over the ranks, as DeepEP asserts)
 *   num_ranks         R, 1..min(E, EP_MAX_RANKS)
 *   expert_alignment  A >= 1: each expert's receive region is rounded up to a
 *                     multiple of A slots (DeepEP's expert_alignment)
 *   use_fp8           0: bf16 payload; 1: OCP E4M3FN payload with one fp32
 *                     scale per token and 128-channel group
 *   topk_idx_bytes    width of topk_idx entries: 0 or 4 = int32, 8 = int64
 *                     (DeepEP passes int64 indices); an int64 value outside
 *                     the int32 range counts as an invalid expert id
 *   cu_budget         0: dispatch and combine use the whole GPU.  n > 0: they
 *                     run as persistent grids of at most n workgroups, one
 *                     per CU (each reserves over half of a CU's LDS), so they
 *                     occupy at most n CUs and leave the rest to concurrent
 *                     work -- the role of DeepEP's num_sms (hotdry analysis,
 *                     "two kernel families": a fixed SM share for
 *                     communication).  Results are identical for every n.
 *                     Layout and low-latency dispatch ignore it.
 * Only the fields a call uses are checked (layout ignores hidden/use_fp8). */
typedef struct ep_problem {
  int32_t num_tokens;
  int32_t hidden;
  int32_t num_topk;
  int32_t num_experts;
  int32_t num_ranks;
  int32_t expert_alignment;
  int32_t use_fp8;
  int32_t topk_idx_bytes;
  int32_t cu_budget;
} ep_problem_t;

/* Receive capacity (slots) that always suffices without learning the counts:
 * N*K + E*(A-1).  Host-only; returns -1 for an invalid descriptor or when the
 * bound exceeds INT32_MAX.  This is the worst-case sizing that lets DeepEP's
 * num_worst_tokens path run without a CPU sync. */
int64_t ep_recv_capacity(const ep_problem_t* p);

/* Bytes of device workspace ep_get_layout needs for this descriptor (host
 * only; -1 if invalid).  The workspace holds the error word and, for problems
 * laid out in two launches, per-block expert histograms, rank counts and
 * error flags.  It needs no initialisation, and its error word stays
 * meaningful for ep_layout_error until the next layout call. */
int64_t ep_workspace_bytes(const ep_problem_t* p);

/* Routing layout (DeepEP book ch.1 sec. 1.4 names the first three outputs).
 *   topk_idx               [N][K] int32 or int64 (topk_idx_bytes), global
 *                          expert ids; -1 = no expert;
 *                          any other value outside [0, E) is skipped and sets
 *                          EP_LAYOUT_ERR_INDEX in the workspace error word
 *   num_tokens_per_rank    [R][R] int32 out: [s][r] = tokens of source s with
 *                          at least one expert on rank r
 *   num_tokens_per_expert  [R][E] int32 out: [s][e] = pairs of source s
 *                          routed to expert e
 *   is_token_in_rank       [N][R] uint8 out: 1 iff token t has an expert on r
 *   num_recv_per_expert    [E] int32 out: pairs expert e receives
 *   expert_slot_offset     [E+1] int32 out: first slot of each expert region
 *                          (padded to A); [E] = slots in use
 *   slot_of                [N][K] int32 out: slot of pair (t,k), -1 if none
 *   workspace              ep_workspace_bytes(p) bytes, 256-byte aligned
 * N == 0 is valid: offsets and counts come out zero.  Output pointers for
 * arrays of zero size may be NULL. */
int ep_get_layout(const ep_problem_t* p, const void* topk_idx,
                  int32_t* num_tokens_per_rank, int32_t* num_tokens_per_expert,
                  uint8_t* is_token_in_rank, int32_t* num_recv_per_expert,
                  int32_t* expert_slot_offset, int32_t* slot_of, void* workspace,
                  void* stream);

/* ep_get_layout without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The workspace is a static device array
 * of EP_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until
 * the process ends (every valid descriptor's ep_workspace_bytes fits in it;
 * a larger one returns EP_ERR_SCRATCH without launching).  The call itself
 * allocates nothing.  All other arguments and outputs are those of
 * ep_get_layout, plus
 *   error_word  [1] int32 device pointer or NULL: receives the error bits
 *               (EP_LAYOUT_ERR_INDEX) that ep_layout_error would report.
 * The array needs no initialisation; every call on one GPU shares it, so
 * calls that overlap on one GPU (concurrent streams) race. */
#define EP_NOALLOC_SCRATCH_BYTES (2u << 20)
int ep_get_layout_noalloc(const ep_problem_t* p, const void* topk_idx,
                          int32_t* num_tokens_per_rank, int32_t* num_tokens_per_expert,
                          uint8_t* is_token_in_rank, int32_t* num_recv_per_expert,
                          int32_t* expert_slot_offset, int32_t* slot_of, int32_t* error_word,
                          void* stream);

/* Dispatch: copy (bf16) or quantise-and-copy (e4m3) every token row into the
 * slots slot_of names, and tag every slot with its source and weight.
 *   x                   [N][H] bf16 token rows
 *   topk_weights        [N][K] fp32 gate weights (may be NULL iff
 *                       recv_topk_weights is NULL)
 *   slot_of, expert_slot_offset, num_recv_per_expert: from ep_get_layout
 *                       (the last two are read only to tag padding slots,
 *                       i.e. when recv_src_idx or recv_topk_weights is given)
 *   recv_x              [recv_capacity][H] bf16 (use_fp8 == 0) or E4M3FN
 *                       bytes (use_fp8 == 1); only slots that hold a pair are
 *                       written, padding rows keep their previous bytes
 *   recv_scales         [recv_capacity][H/128] fp32 (use_fp8 == 1, else
 *                       ignored): scale = amax/448 of the 128-channel group;
 *                       dequantise as code * scale
 *   recv_src_idx        [recv_capacity] int32 out or NULL: source token of the
 *                       slot, -1 for padding and unused slots
 *   recv_topk_weights   [recv_capacity] fp32 out or NULL: the pair's weight,
 *                       0 for padding and unused slots
 *   recv_capacity       rows of the receive buffers; must be at least
 *                       ep_recv_capacity(p) (else EP_ERR_CAPACITY)
 * FP8: per token and group, amax = max |x|; scale = amax/448 and
 * inv = 448/amax (fp32 divisions); code = E4M3FN(x * inv), round to nearest
 * even, saturating; amax == 0 gives scale 1 and signed zero codes.  Where
 * 448/amax overflows fp32 (amax below about 1.3e-36) the group's values and
 * amax are first multiplied by 2^64 (exact), which changes no code of a
 * group whose inverse is finite either way; the scale is still amax/448. */
int ep_dispatch(const ep_problem_t* p, const void* x, const float* topk_weights,
                const int32_t* slot_of, const int32_t* expert_slot_offset,
                const int32_t* num_recv_per_expert, void* recv_x, float* recv_scales,
                int32_t* recv_src_idx, float* recv_topk_weights, int64_t recv_capacity,
                void* stream);

/* Dispatch with the options of DeepEP's V2 dispatch (DeepEP book ch.1
 * sec. 1.1: x may be a pair of FP8 data and scale factors; a running
 * cumulative_local_expert_recv_stats tensor; do_zero_padding; a handle reused
 * from an earlier call).  Every field not named below means what the
 * argument of the same name of ep_dispatch means.
 *   x_scales    NULL: x is bf16 and is quantised when use_fp8 (as ep_dispatch).
 *               Otherwise x holds pre-quantised E4M3FN codes [N][H] and
 *               x_scales their fp32 scales [N][H/128]; both are copied
 *               unchanged to every slot of the token (requires use_fp8).
 *   cumulative_recv_stats  [E] int64 or NULL: stats[e] += num_recv_per_expert[e]
 *               once per call (in stream order; calls that overlap race).
 *   flags       EP_DISPATCH_ZERO_PADDING: also set the padding rows of every
 *               expert region, slots [off[e] + count[e], off[e+1]), to zero
 *               bytes, and their scale rows to 0.0f when use_fp8.  Slots at or
 *               beyond off[E] are left alone.
 * A handle (slot_of, expert_slot_offset, num_recv_per_expert) from one
 * ep_get_layout serves any number of dispatches of new token rows with the
 * same routing; no call changes it. */
#define EP_DISPATCH_ZERO_PADDING 1u
typedef struct ep_dispatch_args {
  const void* x;
  const float* x_scales;
  const float* topk_weights;
  const int32_t* slot_of;
  const int32_t* expert_slot_offset;
  const int32_t* num_recv_per_expert;
  void* recv_x;
  float* recv_scales;
  int32_t* recv_src_idx;
  float* recv_topk_weights;
  int64_t recv_capacity;
  int64_t* cumulative_recv_stats;
  uint32_t flags;
} ep_dispatch_args_t;
int ep_dispatch_ex(const ep_problem_t* p, const ep_dispatch_args_t* args, void* stream);

/* Combine: y[t][c] = bf16( sum over k = 0..K-1 with slot_of[t][k] >= 0 of
 * topk_weights[t][k] * expert_out[slot_of[t][k]][c] ), accumulated in fp32 in
 * ascending k, each product and sum rounded separately, stored with
 * round-to-nearest-even (lesson 14's combine step, DeepEP walkthrough 2.1).
 *   expert_out     [recv_capacity][H] bf16; recv_capacity >= 1 when N > 0
 *                  (else EP_ERR_INVALID_ARG)
 *   slot_of        [N][K] int32 from ep_get_layout (entries outside
 *                  [0, recv_capacity) are treated as "no expert")
 *   topk_weights   [N][K] fp32
 *   y              [N][H] bf16 out
 * Does not read use_fp8: expert outputs are bf16 in both modes. */
int ep_combine(const ep_problem_t* p, const void* expert_out, const int32_t* slot_of,
               const float* topk_weights, void* y, int64_t recv_capacity, void* stream);

/* Low-latency dispatch: routing and payload in ONE launch, for decode-sized
 * batches (DeepEP's second kernel family: lesson 14 sec. 3 shows
 * low_latency_dispatch(x, topk_idx, topk_weights,
 * num_max_dispatch_tokens_per_rank) feeding a masked grouped GEMM; the
 * hotdry analysis, section "two kernel families", places it at decode batches
 * of at most a few hundred tokens per rank).
 * Layout: expert e owns R sub-blocks of M = max_tokens_per_rank rows, one per
 * source rank, [E][R][M][H].  Pair (t, k) of source s routed to expert e goes
 * to slot (e*R + s)*M + j, where j counts the earlier pairs of source s routed
 * to e in (token, k) order.  A slot thus depends only on its own source's
 * pairs: no device-wide scan, no workspace, deterministic.
 *   max_tokens_per_rank  M >= 1; E*R*M <= INT32_MAX; (N/R)*K <= 4096
 *   topk_idx, x, topk_weights  as for ep_get_layout / ep_dispatch
 *   recv_count  [E][R] int32 out: rows used in sub-block (e, s) (<= M); the
 *               mask of the masked GEMM
 *   slot_of     [N][K] int32 out: the handle for ep_combine (with
 *               recv_capacity = ep_ll_capacity), -1 = no slot
 *   flags       [R] int32 out: per-source EP_LAYOUT_ERR_* bits; a pair beyond
 *               M in its sub-block gets no slot and sets ..._OVERFLOW
 *   recv_x, recv_scales, recv_src_idx, recv_topk_weights: as for ep_dispatch,
 *               with ep_ll_capacity rows; only rows holding a pair are
 *               written (rows j >= recv_count of a sub-block keep old bytes)
 * Ignores expert_alignment. */
int64_t ep_ll_capacity(const ep_problem_t* p, int32_t max_tokens_per_rank);
int ep_ll_dispatch(const ep_problem_t* p, int32_t max_tokens_per_rank, const void* topk_idx,
                   const void* x, const float* topk_weights, int32_t* recv_count,
                   int32_t* slot_of, int32_t* flags, void* recv_x, float* recv_scales,
                   int32_t* recv_src_idx, float* recv_topk_weights, void* stream);

/* Low-latency dispatch with the options of DeepEP's V2 dispatch that apply to
 * fixed sub-blocks (DeepEP book ch.1 sec. 1.1): every field means what the
 * argument of the same name of ep_ll_dispatch means, plus
 *   x_scales    NULL: x is bf16 (quantised when use_fp8).  Otherwise x holds
 *               pre-quantised E4M3FN codes [N][H] and x_scales their fp32
 *               scales [N][H/128], copied unchanged (requires use_fp8).
 *   cumulative_recv_stats  [E] int64 or NULL: stats[e] += sum over sources s
 *               of recv_count[e][s] (rows actually placed), once per call.
 * Zero padding is not offered here: the unused rows of the sub-blocks are
 * E*R*M - placed rows, usually most of the buffer. */
typedef struct ep_ll_args {
  const void* topk_idx;
  const void* x;
  const float* x_scales;
  const float* topk_weights;
  int32_t* recv_count;
  int32_t* slot_of;
  int32_t* flags;
  void* recv_x;
  float* recv_scales;
  int32_t* recv_src_idx;
  float* recv_topk_weights;
  int64_t* cumulative_recv_stats;
} ep_ll_args_t;
int ep_ll_dispatch_ex(const ep_problem_t* p, int32_t max_tokens_per_rank, const ep_ll_args_t* args,
                      void* stream);

/* SYNCHRONOUS debug query: waits for `stream`, then stores the error word of
 * the last ep_get_layout that used `workspace` into *flags (host pointer).
 * Bits: EP_LAYOUT_ERR_INDEX. */
int ep_layout_error(const void* workspace, int32_t* flags, void* stream);

/* Static string for a status code. */
const char* ep_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* EP_GET_H */
