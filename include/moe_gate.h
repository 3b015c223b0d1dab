/* Router gate projection followed by the route-sort path, for MI355X (gfx950).
 *
 * The page "Kimi-K3 B1 route-sort + prepared-MoE handoff (stack)", Summary,
 * places a specialised batch-1 gate projection directly in front of the
 * route-sort kernel (which starts from FP32 router logits).  This entry point
 * runs both on one stream:
 *
 *   out_logits[t, e] = RN32( sum_i hidden[t, i] * w_gate[e, i] )
 *
 * (the dot product accumulated in float64 from exact BF16 x BF16 products and
 * rounded once to FP32), then moe_route_sort on out_logits (FP32).
 *
 * Arguments (all pointers are caller-owned device memory):
 *   hidden          [M, H] BF16, row-major, 16-byte aligned
 *   w_gate          [E, H] BF16, row-major, 16-byte aligned
 *   bias            [E] FP32 correction bias
 *   M               tokens, 0 <= M <= 64 (decode batches; the weight matrix is
 *                   streamed once per four tokens)
 *   H               hidden size, H >= 8 and H % 8 == 0 (Kimi-K3: 7168)
 *   k, n_group, topk_group, block   as for moe_route_sort
 *   out_logits      [M, E] FP32, 16-byte aligned (written; also the logits the
 *                   route-sort reads)
 *   out_ids, out_w, sorted_ids, expert_of_block, num_post_pad
 *                   as for moe_route_sort (same capacities)
 *   stream          hipStream_t cast to void*
 * No workspace: at M <= 64 the route-sort runs in one workgroup.  Returns
 * MRS_OK or a negative MRS_ERR_* code (moe_route_sort.h), every argument error
 * detected before any launch.  Two launches; allocates nothing; never waits.
 */
#ifndef MOE_GATE_H_
#define MOE_GATE_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int moe_gate_route_sort(const void* hidden, const void* w_gate, const float* bias, int M, int E, int H, int k,
                        int n_group, int topk_group, int block, float* out_logits, int32_t* out_ids,
                        float* out_w, int32_t* sorted_ids, int32_t* expert_of_block, int32_t* num_post_pad,
                        void* stream);

#ifdef __cplusplus
}
#endif

#endif  /* MOE_GATE_H_ */
