/* Grouped GEMM over the route-sort metadata, for MI355X (gfx950).
 *
 * The page "Kimi-K3 B1 route-sort + prepared-MoE handoff (stack)", Summary:
 * the route-sort output is prepared for the first grouped GEMM of the MoE and
 * read by it directly, with no second top-k or sort.  This entry point is that
 * first GEMM (gate and up projections together): for every sorted row
 * r < *num_post_pad, with slot s = sorted_ids[r] and expert
 * e = expert_of_block[r / block],
 *
 *     y[r, :] = x[s / k, :] . W[e]^T     if 0 <= s < M*k   (a routed token)
 *     y[r, :] = 0                         otherwise        (padding row)
 *
 * Shapes of the page "gfx1250 ordinary-TP route optimization", Capacity and
 * dispatch (Kimi-K3 TP8: 896 experts, top-16, routed hidden size K = 3584,
 * intermediate size 384 per rank, so N = 2 * 384 = 768) are the target; any
 * K that is a multiple of 64 and any N that is a multiple of 128 work.
 *
 * Arguments (all pointers are caller-owned device memory):
 *   x                [M, K] BF16, row-major (hidden states of the tokens)
 *   w                [E, N, K] BF16, row-major (W[e] is [N, K]: output row n
 *                    of expert e is contiguous in K)
 *   sorted_ids, expert_of_block, num_post_pad
 *                    the metadata written by moe_route_sort or
 *                    moe_sort_from_ids with the same M, E, k and block; the
 *                    GEMM reads num_post_pad on the device (no host round trip)
 *   y                [moe_route_sort_max_rows(M, E, k, block), N] BF16,
 *                    row-major; rows below *num_post_pad are written (FP32
 *                    accumulation, rounded to nearest even), nothing else is
 *
 * Requirements: K > 0 and K % 64 == 0; N > 0 and N % 128 == 0; block >= 32 and
 * block % 32 == 0 (a tile of rows never spans two experts); x, w, y 16-byte
 * aligned.  Returns 0 or a negative MRS_ERR_* code (moe_route_sort.h) before
 * any launch.  Rows whose slot lies outside [0, M*k) are padding and are
 * written as zeros (their load reads row 0 of x and discards it).  A tile
 * whose block's expert id lies outside [0, E) reads no weights and writes
 * nothing (metadata from moe_route_sort never holds one).  Asynchronous on
 * `stream`; allocates nothing; one launch.
 */
#ifndef MOE_GEMM1_H_
#define MOE_GEMM1_H_

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int moe_grouped_gemm1(const void* x, const void* w, const int32_t* sorted_ids,
                      const int32_t* expert_of_block, const int32_t* num_post_pad, int M, int k,
                      int E, int K, int N, int block, void* y, hipStream_t stream);

/* Same computation; the launch is stamped with a start and an end HIP event
 * (hipExtLaunchKernel), for timing the kernel on its own stream. */
int moe_grouped_gemm1_profiled(const void* x, const void* w, const int32_t* sorted_ids,
                               const int32_t* expert_of_block, const int32_t* num_post_pad, int M,
                               int k, int E, int K, int N, int block, void* y, hipStream_t stream,
                               hipEvent_t start, hipEvent_t stop);

#ifdef __cplusplus
}
#endif

#endif  // MOE_GEMM1_H_
