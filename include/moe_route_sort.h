/*
 * moe_route_sort.h -- C ABI of the MI355X (gfx950) MoE route-sort library.
 *
 * The operation (page "Kimi-K3 B1 route-sort + prepared-MoE handoff (stack)",
 * Summary section): router logits are converted to FP32, a per-expert
 * correction bias is added, a grouped top-k picks k experts per token, and the
 * two sort phases turn the picks into expert-sorted, block-padded dispatch
 * metadata that a grouped GEMM consumes directly, with no second top-k or sort.
 *
 * Definitions used by every entry point (t = token, j = pick, e = expert):
 *   s[t,e]    = sigmoid(FP32(logits[t,e])), correctly rounded to FP32
 *   key[t,e]  = FP32(s[t,e] + bias[e])              (choice uses the biased key)
 *   groups    = n_group contiguous blocks of E / n_group experts; a group's
 *               score is the FP32 sum of its two largest keys (its only key
 *               when a group holds one expert); the topk_group best groups are
 *               kept, ties to the lower group index
 *   out_ids   = the k best keys inside the kept groups, ties to the lower
 *               expert index, listed in ascending expert id
 *   out_w     = s[t,id] / sum of s over the k picks (unbiased scores); the
 *               sum is formed in float64 and the returned FP32 weight lies
 *               within 2^-22 (relative) of the exact quotient
 *   slot      = t*k + j; sentinel = M*k
 *   count[e]  = number of slots routed to e (phase 1: histogram)
 *   padded[e] = ceil(count[e] / block) * block
 *   off[e]    = sum of padded[e'] for e' < e (phase 2: exclusive prefix)
 *   sorted_ids[off[e] + r] = r-th slot routed to e in ascending slot order for
 *               r < count[e]; sentinel for count[e] <= r < padded[e]
 *   expert_of_block[b] = e for off[e] <= b*block < off[e] + padded[e]
 *   *num_post_pad = sum of padded[e]
 * The page "gfx1250 ordinary-TP route optimization" (Capacity and dispatch)
 * bounds the expert set at 4096 (a 16 KiB histogram of 256-bucket tiles);
 * this library keeps that bound.
 *
 * Memory: every pointer argument of moe_route_sort / moe_route_sort_ex is
 * device memory owned by the caller.  Inputs are never written.  Nothing
 * outside the defined ranges of the outputs is written.  Calls are
 * asynchronous on `stream` (a hipStream_t; NULL = the default stream), never
 * allocate, never wait on the host, and may be captured in a HIP graph.  BF16
 * logits are scored through a constant table (the correctly rounded sigmoid
 * of every BF16 value) that is part of the library's code object.
 *
 * Errors: a negative return code, detected before any launch; on error the
 * outputs are untouched.  moe_route_sort_strerror() names each code.
 */
#ifndef MOE_ROUTE_SORT_H
#define MOE_ROUTE_SORT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MRS_OK = 0,
  MRS_ERR_INVALID_ARG = -1,   /* a size or mode outside the contract below      */
  MRS_ERR_NULL_POINTER = -2,  /* a required pointer is NULL                     */
  MRS_ERR_MISALIGNED = -3,    /* logits not 16-byte aligned, or another array   */
                              /* not 4-byte aligned                             */
  MRS_ERR_WORKSPACE = -4,     /* workspace missing or smaller than required     */
  MRS_ERR_OVERFLOW = -5,      /* M*k or the row capacity does not fit int32     */
  MRS_ERR_LAUNCH = -6,        /* the HIP runtime rejected a kernel launch       */
  MRS_ERR_SCRATCH = -7        /* moe_route_sort_static: the call needs more     */
                              /* scratch than the library's static 8 MiB        */
};

enum { MRS_DTYPE_F32 = 0, MRS_DTYPE_BF16 = 1 };

/*
 * moe_route_sort -- the whole route-sort path in one call.
 *
 *   logits          [M, E] row-major, FP32 or BF16 (logits_dtype), 16-byte
 *                   aligned base address.
 *   bias            [E] FP32 correction bias.
 *   M               tokens, M >= 0.  M == 0 writes *num_post_pad = 0 only.
 *   E               experts, 1 <= E <= 4096.
 *   k               picks per token, 1 <= k <= 64 and k <= topk_group * E / n_group.
 *   n_group         groups, n_group >= 1 and E % n_group == 0.
 *   topk_group      kept groups, 1 <= topk_group <= n_group.
 *   block           padding granularity of each expert's segment, block >= 1.
 *   out_ids         [M, k] int32 (written).
 *   out_w           [M, k] FP32 (written).
 *   sorted_ids      int32 of at least moe_route_sort_max_rows(M, E, k, block)
 *                   entries; entries [0, *num_post_pad) are written.
 *   expert_of_block int32 of at least moe_route_sort_max_blocks(M, E, k, block)
 *                   entries; entries [0, *num_post_pad / block) are written.
 *   num_post_pad    one int32 (written).
 *   logits_dtype    MRS_DTYPE_F32 or MRS_DTYPE_BF16.
 *   workspace       device scratch of at least moe_route_sort_workspace_bytes()
 *                   bytes (may be NULL when that size is 0).  Zero it once when
 *                   it is allocated; every call leaves it reusable, with no
 *                   clearing between calls.  Calls that may overlap in time
 *                   need distinct workspaces.
 *   stream          hipStream_t cast to void* (NULL: default stream).
 * Returns MRS_OK or a negative MRS_ERR_* code.
 */
int moe_route_sort(const void* logits, const float* bias, int M, int E, int k, int n_group,
                   int topk_group, int block, int32_t* out_ids, float* out_w,
                   int32_t* sorted_ids, int32_t* expert_of_block, int32_t* num_post_pad,
                   int logits_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_route_sort_static -- moe_route_sort for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * device allocation) and so cannot provide a workspace.  The scratch is an
 * 8 MiB array in the library's own device memory, one per GPU, held until
 * the process ends; its address on the current device is looked up once per
 * device, and the call itself allocates nothing.
 *
 *   Arguments, results and errors as for moe_route_sort, without workspace
 *   and workspace_bytes.  Inputs whose moe_route_sort_workspace_bytes(M, E, k,
 *   block) exceeds 8 MiB return MRS_ERR_SCRATCH before any launch (every
 *   shape up to 16384 tokens x 4096 experts x top-16 fits; so does
 *   65536 x 896 x top-16).
 *   No call depends on what an earlier call left in the scratch.  All calls
 *   on one GPU share the array: calls that may overlap in time (other
 *   streams, other threads) race and give undefined results; serialise them
 *   or use moe_route_sort with distinct workspaces.
 */
int moe_route_sort_static(const void* logits, const float* bias, int M, int E, int k, int n_group,
                          int topk_group, int block, int32_t* out_ids, float* out_w, int32_t* sorted_ids,
                          int32_t* expert_of_block, int32_t* num_post_pad, int logits_dtype, void* stream);

/* Option bits for moe_route_sort_ex (path selection for tests and tuning;
 * every path computes the same result). */
enum {
  MRS_FLAG_FORCE_SINGLE_WG = 1u << 0, /* one workgroup does everything (M <= 64)           */
  MRS_FLAG_FORCE_MULTI_WG = 1u << 1,  /* many workgroups, even for small M                  */
  MRS_FLAG_FORCE_EXACT = 1u << 2      /* skip the one-wave selection; every token takes the */
                                      /* exact workgroup-wide selection                     */
};

/*
 * moe_route_sort_ex -- moe_route_sort with option bits and optional device
 * statistics.  `stats`, when not NULL, is device int32[3] that the call
 * increments: stats[0] += tokens decided by the workgroup-wide exact selection,
 * stats[1] += tokens decided by one wave, stats[2] += tokens whose group
 * scores one wave made exact (correctly rounded keys for the experts that can
 * be among their group's top two) because the fast (FP32) keys left the group
 * boundary uncertain (each also counts in stats[0] or stats[1], wherever it
 * was decided).  Unknown flag bits or a forced path that cannot take the shape
 * return MRS_ERR_INVALID_ARG.
 */
int moe_route_sort_ex(const void* logits, const float* bias, int M, int E, int k, int n_group,
                      int topk_group, int block, int32_t* out_ids, float* out_w,
                      int32_t* sorted_ids, int32_t* expert_of_block, int32_t* num_post_pad,
                      int logits_dtype, void* workspace, size_t workspace_bytes, void* stream,
                      unsigned flags, int32_t* stats);

/*
 * moe_route_sort_profiled -- moe_route_sort_ex that also stamps HIP events so
 * a caller can time the call's kernels one by one (diagnostics for benchmarks;
 * every kernel does all of its work).  `events` points to 6 hipEvent_t handles
 * (cast to void*) created by the caller; launch i (i = 0, 1, 2) is made with
 * hipExtLaunchKernel and stamps events[2i] and events[2i+1] with the start and
 * the end of that kernel's execution.  Pairs past the last launch are recorded
 * on `stream` after it (zero elapsed time).  *n_launches receives the number
 * of kernels launched (1 to 3).  Returns like moe_route_sort_ex;
 * MRS_ERR_NULL_POINTER when `events`, one of its handles or `n_launches` is
 * NULL.
 */
int moe_route_sort_profiled(const void* logits, const float* bias, int M, int E, int k, int n_group,
                            int topk_group, int block, int32_t* out_ids, float* out_w,
                            int32_t* sorted_ids, int32_t* expert_of_block, int32_t* num_post_pad,
                            int logits_dtype, void* workspace, size_t workspace_bytes, void* stream,
                            unsigned flags, int32_t* stats, void* const* events, int* n_launches);

/*
 * moe_route_sort_local -- moe_route_sort for a rank that owns only the experts
 * [local_begin, local_begin + local_count) (expert parallelism).  The pages
 * keep expert-parallel routing as its own dispatch path (page "gfx1250
 * ordinary-TP route optimization", Capacity and dispatch; Dispatch and
 * contracts) and treat a route that claims no slot as dropped; this entry
 * applies that to routes whose expert another rank owns.
 *
 *   The selection is the full one: out_ids / out_w hold the k global expert
 *   ids and weights of every token, exactly as moe_route_sort writes them.
 *   The metadata covers the local experts only, numbered from 0: sorted_ids
 *   holds the slots t*k + j whose expert lies in the range (ascending within
 *   an expert, sentinel M*k in the padding), expert_of_block holds
 *   expert - local_begin, num_post_pad the local padded total.  A slot routed
 *   to another rank's expert does not appear in sorted_ids.
 *   Capacities: sorted_ids >= moe_route_sort_max_rows(M, local_count, k, block),
 *   expert_of_block >= moe_route_sort_max_blocks(M, local_count, k, block).
 *   Workspace: moe_route_sort_workspace_bytes(M, E, k, block).
 *   0 <= local_begin, 1 <= local_count, local_begin + local_count <= E, else
 *   MRS_ERR_INVALID_ARG; everything else as for moe_route_sort.
 * With local_begin = 0 and local_count = E the result is moe_route_sort's.
 */
int moe_route_sort_local(const void* logits, const float* bias, int M, int E, int k, int n_group,
                         int topk_group, int block, int local_begin, int local_count, int32_t* out_ids,
                         float* out_w, int32_t* sorted_ids, int32_t* expert_of_block, int32_t* num_post_pad,
                         int logits_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_sort_from_ids -- the two sort phases alone, from expert ids chosen
 * elsewhere (page "gfx1250 ordinary-TP route optimization", Summary and
 * Dispatch and contracts: route rows built from selected ids with workgroup
 * histograms).
 *
 *   ids             [M, k] int32 device array, 4-byte aligned.  Slot t*k + j
 *                   routes to expert ids[t*k + j]; an id outside [0, E) is a
 *                   dropped route: it claims no row and its slot number does
 *                   not appear in sorted_ids.  A row may repeat an expert
 *                   (each slot then takes its own row; such workgroups are
 *                   ranked by a slower serial pass).
 *   M, E, k, block  as for moe_route_sort (k <= 64, E <= 4096).
 *   sorted_ids, expert_of_block, num_post_pad
 *                   the metadata of moe_route_sort with counts over the routed
 *                   slots only (same capacities, same sentinel M*k).
 *   workspace       as for moe_route_sort, same size
 *                   (moe_route_sort_workspace_bytes).
 * Asynchronous on `stream`; never allocates or waits.  Returns MRS_OK or a
 * negative MRS_ERR_* code, detected before any launch.
 */
int moe_sort_from_ids(const int32_t* ids, int M, int E, int k, int block, int32_t* sorted_ids,
                      int32_t* expert_of_block, int32_t* num_post_pad, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * moe_sort_from_ids_counters -- moe_sort_from_ids with caller-provided
 * per-expert counters (page "gfx1250 ordinary-TP route optimization",
 * Dispatch and contracts: counters the caller hands in start from the
 * values it gave them, and sizing the counters and rows is up to the caller).
 *
 *   counters        int32[E] device array, read and written.  On entry
 *                   counters[e] = c0[e] >= 0 is the number of rows the caller
 *                   already holds at the head of expert e's segment.  With
 *                   c[e] this call's routes to e (ids outside [0, E) dropped):
 *                     count[e]  = c0[e] + c[e]
 *                     padded[e] = ceil(count[e] / block) * block
 *                     off[e]    = sum of padded[e'] for e' < e
 *                     rows [off[e], off[e] + c0[e])  are not written (the
 *                                                    caller's rows)
 *                     sorted_ids[off[e] + c0[e] + r] = r-th slot routed to e in
 *                                                    ascending slot order
 *                     rows up to off[e] + padded[e]  = sentinel M*k
 *                     expert_of_block as for moe_route_sort (every block)
 *                     *num_post_pad = sum of padded[e]
 *                   and on return counters[e] = count[e].
 *   rows_capacity   entries of sorted_ids; expert_of_block must hold
 *                   rows_capacity / block entries.  0 <= rows_capacity <=
 *                   INT32_MAX - (block - 1), else MRS_ERR_INVALID_ARG.
 *   M == 0 is allowed (ids may then be NULL): the segments hold the caller's
 *   rows only.
 * Device-side failure: when some c0[e] < 0 or the padded total exceeds
 * rows_capacity, the call writes *num_post_pad = -1 and nothing else (the
 * counters, sorted_ids and expert_of_block keep their contents).
 * Counters are read before any of them is written, so the same array may be
 * passed to consecutive calls (and captured in a graph); calls that may
 * overlap in time need distinct counters and workspaces.  Everything else
 * as for moe_sort_from_ids; counters == NULL returns MRS_ERR_NULL_POINTER.
 */
int moe_sort_from_ids_counters(const int32_t* ids, int M, int E, int k, int block, int32_t* counters,
                               int64_t rows_capacity, int32_t* sorted_ids, int32_t* expert_of_block,
                               int32_t* num_post_pad, void* workspace, size_t workspace_bytes,
                               void* stream);

/* Capacity of sorted_ids: M*k + min(E, M*k)*(block-1), or -1 when the
 * arguments are invalid or the result does not fit int32. */
int64_t moe_route_sort_max_rows(int M, int E, int k, int block);

/* Capacity of expert_of_block: max_rows / block (rounded down), or -1. */
int64_t moe_route_sort_max_blocks(int M, int E, int k, int block);

/* Workspace bytes needed by any path for these sizes (0 when none is needed);
 * (size_t)-1 for invalid sizes. */
size_t moe_route_sort_workspace_bytes(int M, int E, int k, int block);

/* Static text for an MRS_* code; never NULL. */
const char* moe_route_sort_strerror(int code);

/*
 * Diagnostics: evaluate the two sigmoid forms the kernels use, elementwise on
 * device arrays of n FP32 values: fast_out = the approximate form used to rank
 * candidates, exact_out = the correctly rounded form used for weights and for
 * exact decisions.  Asynchronous on stream.  Returns MRS_OK or an error code.
 */
int moe_route_sort_sigmoid_probe(const float* x, int n, float* fast_out, float* exact_out,
                                 void* stream);

/*
 * Diagnostics: the correctly rounded sigmoid of BF16 logits as the kernels
 * read it from their LDS table, for n BF16 bit patterns (device uint16_t):
 * out_single[i] through the one-value address form, out_pair[i] through the
 * packed two-value form (element i paired with i ^ 1).  Asynchronous on
 * stream.
 * Returns MRS_OK or an error code.
 */
int moe_route_sort_sigmoid_table_probe(const uint16_t* bf16_bits, int n, float* out_single,
                                       float* out_pair, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ROUTE_SORT_H */
