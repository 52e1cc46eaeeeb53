// The pooled-score block selection split into its host checks and its
// launch, shared by the entry point that takes a caller's workspace and the
// one that uses the library's static scratch (noalloc.hip).
#pragma once

#include "host_common.h"

namespace sdattn {

struct SelectBlocksPlan {
    Problem pr;
    BlockPlan plan;
    int32_t block_q, block_k;
    size_t ws_bytes;  // workspace the launch needs (0 when L == 0)
};

// Host-side checks of sdattn_select_blocks' arguments (everything but the
// workspace) and the workspace size; enqueues nothing.
sdattn_status plan_select_blocks(const sdattn_problem* p, const void* q, const void* k, int32_t block_q,
                                 int32_t block_k, const sdattn_budget* budget, int32_t* row_ptr, int32_t* col_idx,
                                 int64_t col_capacity, SelectBlocksPlan* out);

// Enqueues the selection of a checked plan with `ws` (at least
// plan.ws_bytes bytes of device memory) on `stream`.
sdattn_status launch_planned_select_blocks(const SelectBlocksPlan& sp, const void* q, const void* k,
                                           const sdattn_budget* budget, int32_t* row_ptr, int32_t* col_idx,
                                           float* block_mass, void* ws, void* stream, const char* name);

}  // namespace sdattn
