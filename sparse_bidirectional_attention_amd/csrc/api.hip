// C ABI of the library: argument checks on the host, then kernel launches on
// the caller's stream.  Also provides the HIP backend of the schedule driver.

#include <hip/hip_runtime.h>
#include <stdio.h>

#include <string>

#include "host_common.h"
#include "exact.h"
#include "select_api.h"
#include "launch.h"
#include "probe.h"
#include "schedule.h"

using namespace sdattn;

namespace {

sdattn_status hip_fail(hipError_t e, const char* what) {
    std::string m = what;
    m += ": ";
    m += hipGetErrorString(e);
    return fail(SDATTN_ERR_HIP, m);
}

AttnShape shape_of(const Problem& pr) { return AttnShape{pr.B, pr.Hq, pr.Hkv, pr.L, pr.D, pr.scale}; }

sdattn_status check_tensors(const Problem& pr, const void* q, const void* k, const void* v, const void* o) {
    if (pr.L == 0) return SDATTN_OK;
    if (q == nullptr || k == nullptr || v == nullptr || o == nullptr)
        return fail(SDATTN_ERR_NULL, "q, k, v and o must be non-NULL");
    return SDATTN_OK;
}

sdattn_status run_attention(AttnMode mode, const Problem& pr, const void* q, const void* k, const void* v,
                            void* o, float* lse, const SparseIndex& ix, void* stream, const char* name) {
    if (pr.L == 0) return SDATTN_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = pr.dtype == SDATTN_BF16 ? launch_flash_bf16(mode, shape_of(pr), q, k, v, o, lse, ix, st)
                                           : launch_flash_f32(mode, shape_of(pr), q, k, v, o, lse, ix, st);
    if (e != hipSuccess) return hip_fail(e, name);
    return SDATTN_OK;
}

}  // namespace

namespace sdattn {

sdattn_status plan_select_blocks(const sdattn_problem* p, const void* q, const void* k, int32_t block_q,
                                 int32_t block_k, const sdattn_budget* budget, int32_t* row_ptr, int32_t* col_idx,
                                 int64_t col_capacity, SelectBlocksPlan* out) {
    SelectBlocksPlan sp;
    sdattn_status s = check_problem(p, &sp.pr);
    if (s != SDATTN_OK) return s;
    s = check_blocks(sp.pr, block_q, block_k, budget, &sp.plan);
    if (s != SDATTN_OK) return s;
    sp.block_q = block_q;
    sp.block_k = block_k;
    sp.ws_bytes = 0;
    if (sp.pr.L > 0) {
        if (q == nullptr || k == nullptr || row_ptr == nullptr || col_idx == nullptr)
            return fail(SDATTN_ERR_NULL, "q, k, row_ptr and col_idx must be non-NULL");
        if (col_capacity < sp.plan.max_nnz) {
            char buf[160];
            snprintf(buf, sizeof buf, "col_capacity %lld < worst-case kept blocks %lld",
                     static_cast<long long>(col_capacity), static_cast<long long>(sp.plan.max_nnz));
            return fail(SDATTN_ERR_CAPACITY, buf);
        }
        sp.ws_bytes = select_blocks_ws_layout(shape_of(sp.pr), block_q, block_k, sp.plan.mass).total;
    }
    *out = sp;
    return SDATTN_OK;
}

sdattn_status launch_planned_select_blocks(const SelectBlocksPlan& sp, const void* q, const void* k,
                                           const sdattn_budget* budget, int32_t* row_ptr, int32_t* col_idx,
                                           float* block_mass, void* ws, void* stream, const char* name) {
    hipError_t e = launch_select_blocks(shape_of(sp.pr), sp.pr.dtype == SDATTN_BF16, q, k, sp.block_q, sp.block_k,
                                        sp.plan.mass, static_cast<int>(sp.plan.topk),
                                        static_cast<float>(budget->mass), sp.plan.cap_extra, row_ptr, col_idx,
                                        block_mass, ws, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, name);
    return SDATTN_OK;
}

}  // namespace sdattn

extern "C" {

sdattn_status sdattn_forward_dense(const sdattn_problem* p, const void* q, const void* k, const void* v,
                                   void* o, float* lse, void* stream) {
    Problem pr;
    sdattn_status s = check_problem(p, &pr);
    if (s != SDATTN_OK) return s;
    s = check_tensors(pr, q, k, v, o);
    if (s != SDATTN_OK) return s;
    return run_attention(MODE_DENSE, pr, q, k, v, o, lse, SparseIndex{}, stream, "sdattn_forward_dense");
}

sdattn_status sdattn_select_blocks_workspace(const sdattn_problem* p, int32_t block_q, int32_t block_k,
                                             const sdattn_budget* budget, size_t* ws_bytes, int64_t* max_nnz) {
    if (ws_bytes == nullptr || max_nnz == nullptr) return fail(SDATTN_ERR_NULL, "ws_bytes and max_nnz must be non-NULL");
    Problem pr;
    sdattn_status s = check_problem(p, &pr);
    if (s != SDATTN_OK) return s;
    BlockPlan plan;
    s = check_blocks(pr, block_q, block_k, budget, &plan);
    if (s != SDATTN_OK) return s;
    *ws_bytes = pr.L == 0 ? 0 : select_blocks_ws_layout(shape_of(pr), block_q, block_k, plan.mass).total;
    *max_nnz = plan.max_nnz;
    return SDATTN_OK;
}

sdattn_status sdattn_select_blocks(const sdattn_problem* p, const void* q, const void* k, int32_t block_q,
                                   int32_t block_k, const sdattn_budget* budget, int32_t* row_ptr,
                                   int32_t* col_idx, int64_t col_capacity, float* block_mass, void* ws,
                                   size_t ws_bytes, void* stream) {
    SelectBlocksPlan sp;
    sdattn_status s = plan_select_blocks(p, q, k, block_q, block_k, budget, row_ptr, col_idx, col_capacity, &sp);
    if (s != SDATTN_OK || sp.pr.L == 0) return s;
    if (ws_bytes < sp.ws_bytes || (sp.ws_bytes > 0 && ws == nullptr)) {
        char buf[160];
        snprintf(buf, sizeof buf, "workspace of %zu bytes < required %zu", ws_bytes, sp.ws_bytes);
        return fail(SDATTN_ERR_WORKSPACE, buf);
    }
    return launch_planned_select_blocks(sp, q, k, budget, row_ptr, col_idx, block_mass, ws, stream,
                                        "sdattn_select_blocks");
}

namespace {

// workspace of the exact selector: the selection stages' layout, then the
// mass matrix [rows][nKB] fp32
size_t exact_mass_offset(const Problem& pr, int32_t block_q, int32_t block_k, bool mass) {
    return (select_blocks_ws_layout(shape_of(pr), block_q, block_k, mass).total + 255) & ~static_cast<size_t>(255);
}
size_t exact_ws_bytes(const Problem& pr, int32_t block_q, int32_t block_k, const BlockPlan& plan) {
    return exact_mass_offset(pr, block_q, block_k, plan.mass) + static_cast<size_t>(plan.rows) * plan.nkb * 4;
}

}  // namespace

sdattn_status sdattn_select_blocks_exact_workspace(const sdattn_problem* p, int32_t block_q, int32_t block_k,
                                                   const sdattn_budget* budget, size_t* ws_bytes, int64_t* max_nnz) {
    if (ws_bytes == nullptr || max_nnz == nullptr) return fail(SDATTN_ERR_NULL, "ws_bytes and max_nnz must be non-NULL");
    Problem pr;
    sdattn_status s = check_problem(p, &pr);
    if (s != SDATTN_OK) return s;
    BlockPlan plan;
    s = check_blocks(pr, block_q, block_k, budget, &plan);
    if (s != SDATTN_OK) return s;
    *ws_bytes = pr.L == 0 ? 0 : exact_ws_bytes(pr, block_q, block_k, plan);
    *max_nnz = plan.max_nnz;
    return SDATTN_OK;
}

sdattn_status sdattn_select_blocks_exact(const sdattn_problem* p, const void* q, const void* k, const float* lse,
                                         int32_t block_q, int32_t block_k, const sdattn_budget* budget,
                                         int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity, float* block_mass,
                                         void* ws, size_t ws_bytes, void* stream) {
    Problem pr;
    sdattn_status s = check_problem(p, &pr);
    if (s != SDATTN_OK) return s;
    BlockPlan plan;
    s = check_blocks(pr, block_q, block_k, budget, &plan);
    if (s != SDATTN_OK) return s;
    if (pr.L == 0) return SDATTN_OK;
    if (q == nullptr || k == nullptr || lse == nullptr || row_ptr == nullptr || col_idx == nullptr)
        return fail(SDATTN_ERR_NULL, "q, k, lse, row_ptr and col_idx must be non-NULL");
    if (col_capacity < plan.max_nnz) {
        char buf[160];
        snprintf(buf, sizeof buf, "col_capacity %lld < worst-case kept blocks %lld", static_cast<long long>(col_capacity),
                 static_cast<long long>(plan.max_nnz));
        return fail(SDATTN_ERR_CAPACITY, buf);
    }
    const size_t need = exact_ws_bytes(pr, block_q, block_k, plan);
    if (ws_bytes < need || ws == nullptr) {
        char buf[160];
        snprintf(buf, sizeof buf, "workspace of %zu bytes < required %zu", ws_bytes, need);
        return fail(SDATTN_ERR_WORKSPACE, buf);
    }
    const hipStream_t st = static_cast<hipStream_t>(stream);
    float* mass = reinterpret_cast<float*>(static_cast<char*>(ws) + exact_mass_offset(pr, block_q, block_k, plan.mass));
    hipError_t e = launch_exact_block_mass(shape_of(pr), pr.dtype == SDATTN_BF16, q, k, lse, block_q, block_k, mass, st);
    if (e == hipSuccess)
        e = launch_select_blocks_from_mass(shape_of(pr), mass, block_q, block_k, plan.mass, static_cast<int>(plan.topk),
                                           static_cast<float>(budget->mass), plan.cap_extra, row_ptr, col_idx,
                                           block_mass, ws, st);
    if (e != hipSuccess) return hip_fail(e, "sdattn_select_blocks_exact");
    return SDATTN_OK;
}

sdattn_status sdattn_forward_block_sparse(const sdattn_problem* p, const void* q, const void* k, const void* v,
                                          int32_t block_q, int32_t block_k, const int32_t* row_ptr,
                                          const int32_t* col_idx, void* o, float* lse, void* stream) {
    return sdattn_forward_block_sparse_planned(p, q, k, v, block_q, block_k, row_ptr, col_idx, nullptr, o, lse,
                                               stream);
}

sdattn_status sdattn_block_plan(const sdattn_problem* p, int32_t block_q, int32_t block_k, const int32_t* row_ptr,
                                int32_t* plan, void* stream) {
    Problem pr;
    sdattn_status s = check_problem(p, &pr);
    if (s != SDATTN_OK) return s;
    if ((block_q != 64 && block_q != 128) || (block_k != 64 && block_k != 128))
        return fail(SDATTN_ERR_UNSUPPORTED, "block_q and block_k must be 64 or 128");
    if (pr.L == 0) return SDATTN_OK;
    if (row_ptr == nullptr || plan == nullptr) return fail(SDATTN_ERR_NULL, "row_ptr and plan must be non-NULL");
    const int nqt = (pr.L + block_q - 1) / block_q;
    const long long rows = static_cast<long long>(pr.B) * pr.Hq * nqt;
    if (rows > INT32_MAX) return fail(SDATTN_ERR_SHAPE, "B * Hq * nQB must fit in int32");
    hipError_t e = launch_block_plan(static_cast<int>(rows), nqt, block_q, row_ptr, plan,
                                     static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "sdattn_block_plan");
    return SDATTN_OK;
}

sdattn_status sdattn_forward_block_sparse_planned(const sdattn_problem* p, const void* q, const void* k,
                                                  const void* v, int32_t block_q, int32_t block_k,
                                                  const int32_t* row_ptr, const int32_t* col_idx,
                                                  const int32_t* plan, void* o, float* lse, void* stream) {
    const char* name = plan ? "sdattn_forward_block_sparse_planned" : "sdattn_forward_block_sparse";
    Problem pr;
    sdattn_status s = check_problem(p, &pr);
    if (s != SDATTN_OK) return s;
    if ((block_q != 64 && block_q != 128) || (block_k != 64 && block_k != 128))
        return fail(SDATTN_ERR_UNSUPPORTED, "block_q and block_k must be 64 or 128");
    s = check_tensors(pr, q, k, v, o);
    if (s != SDATTN_OK) return s;
    if (pr.L > 0 && (row_ptr == nullptr || col_idx == nullptr))
        return fail(SDATTN_ERR_NULL, "row_ptr and col_idx must be non-NULL");
    SparseIndex ix;
    ix.block_q = block_q;
    ix.block_k = block_k;
    ix.row_ptr = row_ptr;
    ix.col_idx = col_idx;
    ix.order = plan;
    return run_attention(MODE_BLOCK, pr, q, k, v, o, lse, ix, stream, name);
}

namespace {

// Shared checks of the split-plan calls; *rows_out = B * Hq * nQB.
sdattn_status check_split(const sdattn_problem* p, int32_t block_q, int32_t block_k, Problem* pr, int* rows_out) {
    sdattn_status s = check_problem(p, pr);
    if (s != SDATTN_OK) return s;
    if ((block_q != 64 && block_q != 128) || (block_k != 64 && block_k != 128))
        return fail(SDATTN_ERR_UNSUPPORTED, "block_q and block_k must be 64 or 128");
    const int nqt = (pr->L + block_q - 1) / block_q;
    const long long rows = static_cast<long long>(pr->B) * pr->Hq * nqt;
    if (rows >= (1LL << kSplitRowBits)) return fail(SDATTN_ERR_SHAPE, "B * Hq * nQB must be below 2^24 for a split plan");
    *rows_out = static_cast<int>(rows);
    return SDATTN_OK;
}

sdattn_status check_split_ws(const Problem& pr, int rows, int32_t block_q, const void* ws, size_t ws_bytes) {
    const size_t need = split_ws_bytes(rows, block_q, pr.D);
    if (ws == nullptr || ws_bytes < need) {
        char buf[160];
        snprintf(buf, sizeof buf, "workspace of %zu bytes < required %zu", ws == nullptr ? 0 : ws_bytes, need);
        return fail(SDATTN_ERR_WORKSPACE, buf);
    }
    return SDATTN_OK;
}

}  // namespace

sdattn_status sdattn_block_split_workspace(const sdattn_problem* p, int32_t block_q, int32_t block_k,
                                           size_t* ws_bytes) {
    if (ws_bytes == nullptr) return fail(SDATTN_ERR_NULL, "ws_bytes must be non-NULL");
    Problem pr;
    int rows = 0;
    sdattn_status s = check_split(p, block_q, block_k, &pr, &rows);
    if (s != SDATTN_OK) return s;
    *ws_bytes = pr.L == 0 ? 0 : split_ws_bytes(rows, block_q, pr.D);
    return SDATTN_OK;
}

sdattn_status sdattn_block_split_plan(const sdattn_problem* p, int32_t block_q, int32_t block_k,
                                      const int32_t* row_ptr, void* ws, size_t ws_bytes, void* stream) {
    Problem pr;
    int rows = 0;
    sdattn_status s = check_split(p, block_q, block_k, &pr, &rows);
    if (s != SDATTN_OK) return s;
    if (pr.L == 0) return SDATTN_OK;
    if (row_ptr == nullptr) return fail(SDATTN_ERR_NULL, "row_ptr must be non-NULL");
    s = check_split_ws(pr, rows, block_q, ws, ws_bytes);
    if (s != SDATTN_OK) return s;
    const int nqt = (pr.L + block_q - 1) / block_q;
    hipError_t e = launch_split_plan(rows, nqt, block_q, row_ptr, static_cast<int32_t*>(ws),
                                     static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "sdattn_block_split_plan");
    return SDATTN_OK;
}

sdattn_status sdattn_forward_block_sparse_split(const sdattn_problem* p, const void* q, const void* k,
                                                const void* v, int32_t block_q, int32_t block_k,
                                                const int32_t* row_ptr, const int32_t* col_idx, void* ws,
                                                size_t ws_bytes, void* o, float* lse, void* stream) {
    Problem pr;
    int rows = 0;
    sdattn_status s = check_split(p, block_q, block_k, &pr, &rows);
    if (s != SDATTN_OK) return s;
    s = check_tensors(pr, q, k, v, o);
    if (s != SDATTN_OK) return s;
    if (pr.L == 0) return SDATTN_OK;
    if (row_ptr == nullptr || col_idx == nullptr) return fail(SDATTN_ERR_NULL, "row_ptr and col_idx must be non-NULL");
    s = check_split_ws(pr, rows, block_q, ws, ws_bytes);
    if (s != SDATTN_OK) return s;
    SparseIndex ix;
    ix.block_q = block_q;
    ix.block_k = block_k;
    ix.row_ptr = row_ptr;
    ix.col_idx = col_idx;
    ix.split = static_cast<int32_t*>(ws);
    return run_attention(MODE_BLOCK, pr, q, k, v, o, lse, ix, stream, "sdattn_forward_block_sparse_split");
}

sdattn_status sdattn_select_columns_workspace(const sdattn_problem* p, int32_t kcol, size_t* ws_bytes) {
    if (ws_bytes == nullptr) return fail(SDATTN_ERR_NULL, "ws_bytes must be non-NULL");
    Problem pr;
    sdattn_status s = check_problem(p, &pr);
    if (s != SDATTN_OK) return s;
    if (pr.L > 0 && (kcol < 1 || kcol > pr.L)) return fail(SDATTN_ERR_BUDGET, "kcol must be in [1, seq_len]");
    *ws_bytes = pr.L == 0 ? 0 : select_columns_ws_bytes(shape_of(pr));
    return SDATTN_OK;
}

sdattn_status sdattn_select_columns(const sdattn_problem* p, const void* q, const void* k, const float* lse,
                                    int32_t kcol, int32_t* col_idx, double* col_scores, void* ws,
                                    size_t ws_bytes, void* stream) {
    Problem pr;
    sdattn_status s = check_problem(p, &pr);
    if (s != SDATTN_OK) return s;
    if (pr.L == 0) return SDATTN_OK;
    if (kcol < 1 || kcol > pr.L) return fail(SDATTN_ERR_BUDGET, "kcol must be in [1, seq_len]");
    if (q == nullptr || k == nullptr || lse == nullptr || col_idx == nullptr)
        return fail(SDATTN_ERR_NULL, "q, k, lse and col_idx must be non-NULL");
    const size_t need = select_columns_ws_bytes(shape_of(pr));
    if (ws_bytes < need || ws == nullptr) {
        char buf[160];
        snprintf(buf, sizeof buf, "workspace of %zu bytes < required %zu", ws_bytes, need);
        return fail(SDATTN_ERR_WORKSPACE, buf);
    }
    hipError_t e = launch_select_columns(shape_of(pr), pr.dtype == SDATTN_BF16, q, k, lse, kcol, col_idx, col_scores,
                                         ws, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "sdattn_select_columns");
    return SDATTN_OK;
}

sdattn_status sdattn_forward_column_sparse(const sdattn_problem* p, const void* q, const void* k, const void* v,
                                           const int32_t* col_idx, int32_t kcol, void* o, float* lse,
                                           void* stream) {
    Problem pr;
    sdattn_status s = check_problem(p, &pr);
    if (s != SDATTN_OK) return s;
    if (pr.L == 0) return SDATTN_OK;
    if (kcol < 1 || kcol > pr.L) return fail(SDATTN_ERR_BUDGET, "kcol must be in [1, seq_len]");
    s = check_tensors(pr, q, k, v, o);
    if (s != SDATTN_OK) return s;
    if (col_idx == nullptr) return fail(SDATTN_ERR_NULL, "col_idx must be non-NULL");
    SparseIndex ix;
    ix.col_idx = col_idx;
    ix.kcol = kcol;
    return run_attention(MODE_COLUMN, pr, q, k, v, o, lse, ix, stream, "sdattn_forward_column_sparse");
}

sdattn_status sdattn_gather_columns(const sdattn_problem* p, const void* k, const void* v, const int32_t* col_idx,
                                    int32_t kcol, void* kc, void* vc, void* stream) {
    Problem pr;
    sdattn_status s = check_problem(p, &pr);
    if (s != SDATTN_OK) return s;
    if (pr.L == 0) return SDATTN_OK;
    if (kcol < 1 || kcol > pr.L) return fail(SDATTN_ERR_BUDGET, "kcol must be in [1, seq_len]");
    if (k == nullptr || v == nullptr || col_idx == nullptr || kc == nullptr || vc == nullptr)
        return fail(SDATTN_ERR_NULL, "k, v, col_idx, kc and vc must be non-NULL");
    hipError_t e = launch_gather_columns(shape_of(pr), pr.dtype == SDATTN_BF16 ? 2 : 4, k, v, col_idx, kcol, kc, vc,
                                         static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "sdattn_gather_columns");
    return SDATTN_OK;
}

sdattn_status sdattn_forward_column_packed(const sdattn_problem* p, const void* q, const void* kc, const void* vc,
                                           int32_t kcol, void* o, float* lse, void* stream) {
    Problem pr;
    sdattn_status s = check_problem(p, &pr);
    if (s != SDATTN_OK) return s;
    if (pr.L == 0) return SDATTN_OK;
    if (kcol < 1 || kcol > pr.L) return fail(SDATTN_ERR_BUDGET, "kcol must be in [1, seq_len]");
    s = check_tensors(pr, q, kc, vc, o);
    if (s != SDATTN_OK) return s;
    SparseIndex ix;
    ix.kcol = kcol;
    return run_attention(MODE_COLUMN_PACKED, pr, q, kc, vc, o, lse, ix, stream, "sdattn_forward_column_packed");
}

sdattn_status sdattn_mask_overlap(int32_t rows, const int32_t* row_ptr_a, const int32_t* col_idx_a,
                                  const int32_t* row_ptr_b, const int32_t* col_idx_b, int64_t* counts,
                                  void* stream) {
    if (rows < 0) return fail(SDATTN_ERR_SHAPE, "rows must be >= 0");
    if (counts == nullptr) return fail(SDATTN_ERR_NULL, "counts must be non-NULL");
    if (rows > 0 && (row_ptr_a == nullptr || col_idx_a == nullptr || row_ptr_b == nullptr || col_idx_b == nullptr))
        return fail(SDATTN_ERR_NULL, "row_ptr and col_idx of both patterns must be non-NULL");
    hipError_t e = launch_mask_overlap(rows, row_ptr_a, col_idx_a, row_ptr_b, col_idx_b, counts,
                                       static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "sdattn_mask_overlap");
    return SDATTN_OK;
}

}  // extern "C"

// ---- HIP backend of the schedule driver ------------------------------------

namespace {

sdattn_status be_dense(void*, const sdattn_problem* p, const void* q, const void* k, const void* v, void* o,
                       float* lse, void* st) {
    return sdattn_forward_dense(p, q, k, v, o, lse, st);
}
sdattn_status be_select_blocks(void*, const sdattn_problem* p, const void* q, const void* k, int32_t bq, int32_t bk,
                               const sdattn_budget* b, int32_t* rp, int32_t* ci, int64_t cap, void* ws, size_t wsb,
                               void* st) {
    return sdattn_select_blocks(p, q, k, bq, bk, b, rp, ci, cap, nullptr, ws, wsb, st);
}
sdattn_status be_block_sparse(void*, const sdattn_problem* p, const void* q, const void* k, const void* v, int32_t bq,
                              int32_t bk, const int32_t* rp, const int32_t* ci, const int32_t* plan, void* o,
                              float* lse, void* st) {
    return sdattn_forward_block_sparse_planned(p, q, k, v, bq, bk, rp, ci, plan, o, lse, st);
}
sdattn_status be_block_plan(void*, const sdattn_problem* p, int32_t bq, int32_t bk, const int32_t* rp, int32_t* plan,
                            void* st) {
    return sdattn_block_plan(p, bq, bk, rp, plan, st);
}
sdattn_status be_block_split_ws(void*, const sdattn_problem* p, int32_t bq, int32_t bk, size_t* ws) {
    return sdattn_block_split_workspace(p, bq, bk, ws);
}
sdattn_status be_block_split_plan(void*, const sdattn_problem* p, int32_t bq, int32_t bk, const int32_t* rp, void* ws,
                                  size_t wsb, void* st) {
    return sdattn_block_split_plan(p, bq, bk, rp, ws, wsb, st);
}
sdattn_status be_block_sparse_split(void*, const sdattn_problem* p, const void* q, const void* k, const void* v,
                                    int32_t bq, int32_t bk, const int32_t* rp, const int32_t* ci, void* ws, size_t wsb,
                                    void* o, float* lse, void* st) {
    return sdattn_forward_block_sparse_split(p, q, k, v, bq, bk, rp, ci, ws, wsb, o, lse, st);
}
sdattn_status be_select_columns(void*, const sdattn_problem* p, const void* q, const void* k, const float* lse,
                                int32_t kcol, int32_t* ci, void* ws, size_t wsb, void* st) {
    return sdattn_select_columns(p, q, k, lse, kcol, ci, nullptr, ws, wsb, st);
}
sdattn_status be_column_sparse(void*, const sdattn_problem* p, const void* q, const void* k, const void* v,
                               const int32_t* ci, int32_t kcol, void* o, float* lse, void* st) {
    return sdattn_forward_column_sparse(p, q, k, v, ci, kcol, o, lse, st);
}
sdattn_status be_ws_blocks(void*, const sdattn_problem* p, int32_t bq, int32_t bk, const sdattn_budget* b, size_t* ws,
                           int64_t* nnz) {
    return sdattn_select_blocks_workspace(p, bq, bk, b, ws, nnz);
}
sdattn_status be_ws_columns(void*, const sdattn_problem* p, int32_t kcol, size_t* ws) {
    return sdattn_select_columns_workspace(p, kcol, ws);
}
sdattn_status be_alloc(void*, size_t bytes, void** out) {
    hipError_t e = hipMalloc(out, bytes ? bytes : 1);
    if (e != hipSuccess) {
        *out = nullptr;
        return hip_fail(e, "hipMalloc");
    }
    return SDATTN_OK;
}
void be_release(void*, void* ptr) { (void)hipFree(ptr); }
sdattn_status be_overlap(void*, int32_t rows, const int32_t* rpa, const int32_t* cia, const int32_t* rpb,
                         const int32_t* cib, int64_t* counts, void* st) {
    return sdattn_mask_overlap(rows, rpa, cia, rpb, cib, counts, st);
}
sdattn_status be_probe_adopt(void*, int32_t rows, int32_t* rp_dst, int32_t* ci_dst, const int32_t* rp_src,
                             const int32_t* ci_src, const int64_t* counts, void* state, double min_overlap,
                             int64_t max_copy, void* st) {
    hipError_t e = launch_probe_adopt(rows, rp_dst, ci_dst, rp_src, ci_src, counts, static_cast<ProbeState*>(state),
                                      min_overlap, max_copy, static_cast<hipStream_t>(st));
    if (e != hipSuccess) return hip_fail(e, "probe adoption");
    return SDATTN_OK;
}
sdattn_status be_probe_init(void*, void* state) {
    hipError_t e = launch_probe_init(static_cast<ProbeState*>(state), nullptr);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(e, "probe record initialisation");
    return SDATTN_OK;
}
sdattn_status be_probe_read(void*, const void* state, int64_t out[4], void* st) {
    hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(st));
    if (e == hipSuccess) e = hipMemcpy(out, state, sizeof(ProbeState), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "sdattn_schedule_probe_stats");
    return SDATTN_OK;
}

sdattn_status be_select_blocks_exact(void*, const sdattn_problem* p, const void* q, const void* k, const float* lse,
                                     int32_t bq, int32_t bk, const sdattn_budget* b, int32_t* rp, int32_t* ci,
                                     int64_t cap, void* ws, size_t wsb, void* st) {
    return sdattn_select_blocks_exact(p, q, k, lse, bq, bk, b, rp, ci, cap, nullptr, ws, wsb, st);
}
sdattn_status be_ws_blocks_exact(void*, const sdattn_problem* p, int32_t bq, int32_t bk, const sdattn_budget* b,
                                 size_t* ws, int64_t* nnz) {
    return sdattn_select_blocks_exact_workspace(p, bq, bk, b, ws, nnz);
}
sdattn_status be_gather_columns(void*, const sdattn_problem* p, const void* k, const void* v, const int32_t* ci,
                                int32_t kcol, void* kc, void* vc, void* st) {
    return sdattn_gather_columns(p, k, v, ci, kcol, kc, vc, st);
}
sdattn_status be_column_packed(void*, const sdattn_problem* p, const void* q, const void* kc, const void* vc,
                               int32_t kcol, void* o, float* lse, void* st) {
    return sdattn_forward_column_packed(p, q, kc, vc, kcol, o, lse, st);
}

const Backend kHipBackend = {nullptr,          be_dense,       be_select_blocks, be_block_sparse, be_select_columns,
                             be_column_sparse, be_ws_blocks,   be_ws_columns,    be_alloc,        be_release,
                             be_overlap,       be_probe_adopt, be_probe_init,    be_probe_read,   be_select_blocks_exact,
                             be_ws_blocks_exact, be_gather_columns, be_column_packed, be_block_plan,
                             be_block_split_ws, be_block_split_plan, be_block_sparse_split};

}  // namespace

namespace sdattn {
const Backend& default_backend() { return kHipBackend; }
}  // namespace sdattn
