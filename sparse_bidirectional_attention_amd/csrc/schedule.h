// Step-schedule driver internals.  The driver is plain C++ and reaches the
// GPU only through a Backend function table: the library installs the HIP
// backend (api.hip); CPU tests install a recording fake.
#pragma once

#include "host_common.h"

namespace sdattn {

struct Backend {
    void* ctx;
    sdattn_status (*dense)(void* ctx, const sdattn_problem*, const void* q, const void* k, const void* v,
                           void* o, float* lse, void* stream);
    sdattn_status (*select_blocks)(void* ctx, const sdattn_problem*, const void* q, const void* k, int32_t bq,
                                   int32_t bk, const sdattn_budget*, int32_t* row_ptr, int32_t* col_idx,
                                   int64_t cap, void* ws, size_t ws_bytes, void* stream);
    sdattn_status (*block_sparse)(void* ctx, const sdattn_problem*, const void* q, const void* k, const void* v,
                                  int32_t bq, int32_t bk, const int32_t* row_ptr, const int32_t* col_idx, void* o,
                                  float* lse, void* stream);
    sdattn_status (*select_columns)(void* ctx, const sdattn_problem*, const void* q, const void* k,
                                    const float* lse, int32_t kcol, int32_t* col_idx, void* ws, size_t ws_bytes,
                                    void* stream);
    sdattn_status (*column_sparse)(void* ctx, const sdattn_problem*, const void* q, const void* k, const void* v,
                                   const int32_t* col_idx, int32_t kcol, void* o, float* lse, void* stream);
    sdattn_status (*workspace_blocks)(void* ctx, const sdattn_problem*, int32_t bq, int32_t bk,
                                      const sdattn_budget*, size_t* ws, int64_t* max_nnz);
    sdattn_status (*workspace_columns)(void* ctx, const sdattn_problem*, int32_t kcol, size_t* ws);
    sdattn_status (*alloc)(void* ctx, size_t bytes, void** out);
    void (*release)(void* ctx, void* ptr);
};

// The backend used by sdattn_schedule_create (defined by the library build
// or by the test build).
const Backend& default_backend();

// Action of step t under the descriptor (validated elsewhere).
sdattn_action schedule_action_of(const sdattn_schedule_desc& d, int32_t t);

}  // namespace sdattn
