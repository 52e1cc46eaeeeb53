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
                                  int32_t bq, int32_t bk, const int32_t* row_ptr, const int32_t* col_idx,
                                  const int32_t* plan, void* o, float* lse, void* stream);
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
    // adaptive anchors: overlap counts of two CSR patterns (counts [3] on the
    // device), the probe's adoption decided and applied on the device, and
    // the device-resident probe record (4 int64: probes, adopted, last
    // |A n B|, last |A u B|)
    sdattn_status (*overlap)(void* ctx, int32_t rows, const int32_t* rpa, const int32_t* cia, const int32_t* rpb,
                             const int32_t* cib, int64_t* counts, void* stream);
    sdattn_status (*probe_adopt)(void* ctx, int32_t rows, int32_t* rp_dst, int32_t* ci_dst, const int32_t* rp_src,
                                 const int32_t* ci_src, const int64_t* counts, void* state, double min_overlap,
                                 int64_t max_copy, void* stream);
    sdattn_status (*probe_init)(void* ctx, void* state);                            // synchronous
    sdattn_status (*probe_read)(void* ctx, const void* state, int64_t out[4], void* stream);  // synchronous
    // exact block mass selection (uses the dense pass's lse)
    sdattn_status (*select_blocks_exact)(void* ctx, const sdattn_problem*, const void* q, const void* k,
                                         const float* lse, int32_t bq, int32_t bk, const sdattn_budget*,
                                         int32_t* row_ptr, int32_t* col_idx, int64_t cap, void* ws, size_t ws_bytes,
                                         void* stream);
    sdattn_status (*workspace_blocks_exact)(void* ctx, const sdattn_problem*, int32_t bq, int32_t bk,
                                            const sdattn_budget*, size_t* ws, int64_t* max_nnz);
    // column steps from rows gathered once per step
    sdattn_status (*gather_columns)(void* ctx, const sdattn_problem*, const void* k, const void* v,
                                    const int32_t* col_idx, int32_t kcol, void* kc, void* vc, void* stream);
    sdattn_status (*column_packed)(void* ctx, const sdattn_problem*, const void* q, const void* kc, const void* vc,
                                   int32_t kcol, void* o, float* lse, void* stream);
    // dispatch plan of the block-sparse forward for a pattern's row_ptr
    sdattn_status (*block_plan)(void* ctx, const sdattn_problem*, int32_t bq, int32_t bk, const int32_t* row_ptr,
                                int32_t* plan, void* stream);
    // split rows: workspace bytes, the split plan of a pattern, the forward over it
    sdattn_status (*block_split_ws)(void* ctx, const sdattn_problem*, int32_t bq, int32_t bk, size_t* ws_bytes);
    sdattn_status (*block_split_plan)(void* ctx, const sdattn_problem*, int32_t bq, int32_t bk,
                                      const int32_t* row_ptr, void* ws, size_t ws_bytes, void* stream);
    sdattn_status (*block_sparse_split)(void* ctx, const sdattn_problem*, const void* q, const void* k, const void* v,
                                        int32_t bq, int32_t bk, const int32_t* row_ptr, const int32_t* col_idx,
                                        void* ws, size_t ws_bytes, void* o, float* lse, void* stream);
};

// The backend used by sdattn_schedule_create (defined by the library build
// or by the test build).
const Backend& default_backend();

// Action of step t under the descriptor (validated elsewhere).
sdattn_action schedule_action_of(const sdattn_schedule_desc& d, int32_t t);

}  // namespace sdattn
