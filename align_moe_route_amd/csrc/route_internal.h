// Internal interface between the library's translation units (not exported).
#ifndef MRS_ROUTE_INTERNAL_H_
#define MRS_ROUTE_INTERNAL_H_

#include <stdint.h>

// Every argument check of moe_route_sort that needs no workspace and no
// device: sizes, group shape, dtype, int32 capacity, null and misaligned
// pointers (the row-capacity overflow check is the caller's: it depends on
// how many experts get metadata).  Returns MRS_OK or the code moe_route_sort
// would return.
__attribute__((visibility("hidden"))) int mrs_check_route_args(const void* logits, const float* bias, int M, int E, int k, int n_group,
                         int topk_group, int block, const int32_t* out_ids, const float* out_w,
                         const int32_t* sorted_ids, const int32_t* expert_of_block,
                         const int32_t* num_post_pad, int logits_dtype);

#endif  // MRS_ROUTE_INTERNAL_H_
