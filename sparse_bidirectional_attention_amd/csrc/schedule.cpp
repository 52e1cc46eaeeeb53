// Host-side step-schedule driver (SparseD, abstract: full attention in the
// early steps, then a pattern computed once and reused; Step-dLLM, Abstract:
// refresh at anchor steps, reuse within each interval; PulseCol, Abstract:
// column pattern refreshed at a few intermediate steps).  Between anchors a
// block schedule can probe: rerun the pooled selector and adopt its pattern
// when it overlaps the cached one too little (Step-dLLM, Abstract: patterns
// hold only locally and change abruptly at some transitions).
//
// The handle owns two pattern buffers: a selection always writes the buffer
// not in use and the handle switches to it only when every call of the step
// was accepted, so a failed step leaves the cached pattern untouched.

#include <math.h>
#include <stdio.h>

#include <algorithm>
#include <new>
#include <vector>

#include "schedule.h"

struct sdattn_schedule {
    sdattn::Backend be;
    sdattn_problem prob;
    sdattn::Problem pr;
    sdattn_schedule_desc desc;
    std::vector<int32_t> refresh;  // owned copy of desc.refresh_steps
    // pattern buffers (device)
    int32_t* row_ptr[2] = {nullptr, nullptr};
    int32_t* col_idx[2] = {nullptr, nullptr};
    int32_t* plan[2] = {nullptr, nullptr};  // block patterns: dispatch plan (or split plan) of each buffer's forward
    size_t plan_bytes = 0;
    int64_t nnz_cap = 0;
    int32_t kcol = 0;
    int active = -1;  // -1: no pattern yet
    void* ws = nullptr;
    size_t ws_bytes = 0;
    float* lse = nullptr;  // own lse buffer (columns, exact blocks)
    void* kc = nullptr;    // columns: the kept K / V rows of the step, [B][Hkv][kcol][d]
    void* vc = nullptr;
    int64_t counts[4] = {0, 0, 0, 0};
    int32_t last_select = -1;
    // probes (blocks with probe_interval > 0): device counts [3] + ProbeState
    int64_t rows = 0;
    int64_t* probe_buf = nullptr;  // [0..2] overlap counts, [4..7] probe record
    int64_t n_probes = 0;          // probe steps enqueued (host count)
};

namespace sdattn {

namespace {

// The plan of pattern buffer i, and the block-sparse forward over it: the
// dispatch plan, or the split plan when the descriptor asks for split rows.
sdattn_status plan_pattern(sdattn_schedule* s, int i, void* stream) {
    const Backend& be = s->be;
    if (s->desc.split_rows)
        return be.block_split_plan(be.ctx, &s->prob, s->desc.block_q, s->desc.block_k, s->row_ptr[i], s->plan[i],
                                   s->plan_bytes, stream);
    return be.block_plan(be.ctx, &s->prob, s->desc.block_q, s->desc.block_k, s->row_ptr[i], s->plan[i], stream);
}

sdattn_status sparse_over(sdattn_schedule* s, int i, const void* q, const void* k, const void* v, void* o, float* lse,
                          void* stream) {
    const Backend& be = s->be;
    if (s->desc.split_rows)
        return be.block_sparse_split(be.ctx, &s->prob, q, k, v, s->desc.block_q, s->desc.block_k, s->row_ptr[i],
                                     s->col_idx[i], s->plan[i], s->plan_bytes, o, lse, stream);
    return be.block_sparse(be.ctx, &s->prob, q, k, v, s->desc.block_q, s->desc.block_k, s->row_ptr[i], s->col_idx[i],
                           s->plan[i], o, lse, stream);
}

}  // namespace

sdattn_action schedule_action_of(const sdattn_schedule_desc& d, int32_t t) {
    bool in_s = t == d.select_step;
    if (!in_s && d.refresh_interval > 0 && t > d.select_step)
        in_s = (t - d.select_step) % d.refresh_interval == 0;
    if (!in_s && d.refresh_steps != nullptr)
        for (int i = 0; i < d.n_refresh_steps; ++i) in_s = in_s || d.refresh_steps[i] == t;
    if (in_s) {
        const bool dense = t < d.dense_steps || (d.refresh_dense && t > d.select_step);
        return dense ? SDATTN_ACT_DENSE_SELECT : SDATTN_ACT_SELECT_SPARSE;
    }
    if (t < d.dense_steps) return SDATTN_ACT_DENSE;
    if (d.probe_interval > 0 && t > d.select_step && (t - d.select_step) % d.probe_interval == 0)
        return SDATTN_ACT_PROBE_SPARSE;
    return SDATTN_ACT_SPARSE;
}

namespace {

sdattn_status check_desc(const Problem& pr, const sdattn_schedule_desc* d) {
    if (d == nullptr) return fail(SDATTN_ERR_NULL, "schedule descriptor is NULL");
    if (d->total_steps < 1) return fail(SDATTN_ERR_SHAPE, "total_steps must be >= 1");
    if (d->dense_steps < 0 || d->dense_steps > d->total_steps)
        return fail(SDATTN_ERR_SHAPE, "dense_steps must be in [0, total_steps]");
    if (d->select_step < 0 || d->select_step >= d->total_steps)
        return fail(SDATTN_ERR_SHAPE, "select_step must be in [0, total_steps)");
    if (d->select_step > d->dense_steps)
        return fail(SDATTN_ERR_SHAPE, "select_step > dense_steps: a sparse step would run before any pattern exists");
    if (d->refresh_interval < 0) return fail(SDATTN_ERR_SHAPE, "refresh_interval must be >= 0");
    if (d->n_refresh_steps < 0 || (d->n_refresh_steps > 0 && d->refresh_steps == nullptr))
        return fail(SDATTN_ERR_NULL, "refresh_steps is NULL but n_refresh_steps > 0");
    if (d->sel != SDATTN_SEL_BLOCKS && d->sel != SDATTN_SEL_COLUMNS && d->sel != SDATTN_SEL_BLOCKS_EXACT)
        return fail(SDATTN_ERR_SHAPE, "unknown selector kind");
    if (d->sel == SDATTN_SEL_BLOCKS_EXACT) {
        // the exact block mass uses the lse of a dense pass of the same step
        if (!d->refresh_dense)
            return fail(SDATTN_ERR_SHAPE, "exact block selection needs refresh_dense = 1 (the mass uses the dense lse)");
        if (d->select_step >= d->dense_steps)
            return fail(SDATTN_ERR_SHAPE, "exact block selection step must be a dense step (select_step < dense_steps)");
        if (d->probe_interval != 0)
            return fail(SDATTN_ERR_UNSUPPORTED, "probes use the pooled selector (exact selection needs a dense pass)");
    }
    if (d->sel == SDATTN_SEL_COLUMNS) {
        if (!d->refresh_dense)
            return fail(SDATTN_ERR_SHAPE, "column selection needs refresh_dense = 1 (scores use the dense lse)");
        if (!(d->column_keep_frac > 0.0 && d->column_keep_frac <= 1.0))
            return fail(SDATTN_ERR_BUDGET, "column_keep_frac must be in (0, 1]");
        // the first column selection needs a dense pass for its lse
        if (d->select_step >= d->dense_steps)
            return fail(SDATTN_ERR_SHAPE, "column selection step must be a dense step (select_step < dense_steps)");
        if (d->probe_interval != 0)
            return fail(SDATTN_ERR_UNSUPPORTED, "probes are for block patterns (column selection needs a dense pass)");
    }
    if (d->probe_interval < 0) return fail(SDATTN_ERR_SHAPE, "probe_interval must be >= 0");
    if (d->split_rows != 0 && d->split_rows != 1) return fail(SDATTN_ERR_SHAPE, "split_rows must be 0 or 1");
    if (d->split_rows && d->sel == SDATTN_SEL_COLUMNS)
        return fail(SDATTN_ERR_UNSUPPORTED, "split_rows is for block patterns");
    if (d->probe_interval > 0 && !(d->min_overlap >= 0.0 && d->min_overlap <= 1.0))
        return fail(SDATTN_ERR_BUDGET, "min_overlap must be in [0, 1]");
    (void)pr;
    return SDATTN_OK;
}

}  // namespace
}  // namespace sdattn

using namespace sdattn;

extern "C" {

sdattn_status sdattn_schedule_create(const sdattn_problem* p, const sdattn_schedule_desc* desc,
                                     sdattn_schedule** out) {
    if (out == nullptr) return fail(SDATTN_ERR_NULL, "out is NULL");
    *out = nullptr;
    Problem pr;
    sdattn_status st = check_problem(p, &pr);
    if (st != SDATTN_OK) return st;
    st = check_desc(pr, desc);
    if (st != SDATTN_OK) return st;
    sdattn_schedule* s = new (std::nothrow) sdattn_schedule();
    if (s == nullptr) return fail(SDATTN_ERR_SHAPE, "out of host memory");
    s->be = default_backend();
    s->prob = *p;
    s->pr = pr;
    s->desc = *desc;
    if (desc->n_refresh_steps > 0) s->refresh.assign(desc->refresh_steps, desc->refresh_steps + desc->n_refresh_steps);
    s->desc.refresh_steps = s->refresh.empty() ? nullptr : s->refresh.data();
    s->desc.n_refresh_steps = static_cast<int32_t>(s->refresh.size());

    auto cleanup_fail = [&](sdattn_status e) {
        sdattn_schedule_destroy(s);
        return e;
    };
    size_t rp_bytes = 0, ci_bytes = 0;
    const size_t lse_bytes = static_cast<size_t>(pr.B) * pr.Hq * std::max(pr.L, 1) * sizeof(float);
    if (desc->sel == SDATTN_SEL_BLOCKS || desc->sel == SDATTN_SEL_BLOCKS_EXACT) {
        const bool exact = desc->sel == SDATTN_SEL_BLOCKS_EXACT;
        BlockPlan plan;
        st = check_blocks(pr, desc->block_q, desc->block_k, &desc->budget, &plan);
        if (st != SDATTN_OK) return cleanup_fail(st);
        int64_t max_nnz = 0;
        st = (exact ? s->be.workspace_blocks_exact : s->be.workspace_blocks)(s->be.ctx, p, desc->block_q, desc->block_k,
                                                                              &desc->budget, &s->ws_bytes, &max_nnz);
        if (st != SDATTN_OK) return cleanup_fail(st);
        if (exact) {  // own lse buffer for steps run with lse = NULL
            st = s->be.alloc(s->be.ctx, lse_bytes, reinterpret_cast<void**>(&s->lse));
            if (st != SDATTN_OK) return cleanup_fail(st);
        }
        s->nnz_cap = std::max<int64_t>(max_nnz, 1);
        s->rows = plan.rows;
        s->plan_bytes = static_cast<size_t>(std::max<int64_t>(s->rows, 1)) * sizeof(int32_t);
        if (desc->split_rows) {
            size_t split_bytes = 0;
            st = s->be.block_split_ws(s->be.ctx, p, desc->block_q, desc->block_k, &split_bytes);
            if (st != SDATTN_OK) return cleanup_fail(st);
            s->plan_bytes = std::max(split_bytes, s->plan_bytes);
        }
        rp_bytes = static_cast<size_t>(plan.rows + 1) * sizeof(int32_t);
        ci_bytes = static_cast<size_t>(s->nnz_cap) * sizeof(int32_t);
    } else {
        s->kcol = static_cast<int32_t>(count_from_fraction(desc->column_keep_frac, std::max(pr.L, 1)));
        st = s->be.workspace_columns(s->be.ctx, p, s->kcol, &s->ws_bytes);
        if (st != SDATTN_OK) return cleanup_fail(st);
        s->nnz_cap = static_cast<int64_t>(pr.B) * pr.Hkv * s->kcol;
        ci_bytes = static_cast<size_t>(std::max<int64_t>(s->nnz_cap, 1)) * sizeof(int32_t);
        st = s->be.alloc(s->be.ctx, lse_bytes, reinterpret_cast<void**>(&s->lse));
        if (st != SDATTN_OK) return cleanup_fail(st);
        const size_t packed = static_cast<size_t>(std::max<int64_t>(s->nnz_cap, 1)) * pr.D *
                              (pr.dtype == SDATTN_BF16 ? 2 : 4);
        st = s->be.alloc(s->be.ctx, packed, &s->kc);
        if (st != SDATTN_OK) return cleanup_fail(st);
        st = s->be.alloc(s->be.ctx, packed, &s->vc);
        if (st != SDATTN_OK) return cleanup_fail(st);
    }
    for (int i = 0; i < 2; ++i) {
        if (rp_bytes) {
            st = s->be.alloc(s->be.ctx, rp_bytes, reinterpret_cast<void**>(&s->row_ptr[i]));
            if (st != SDATTN_OK) return cleanup_fail(st);
            st = s->be.alloc(s->be.ctx, s->plan_bytes, reinterpret_cast<void**>(&s->plan[i]));
            if (st != SDATTN_OK) return cleanup_fail(st);
        }
        st = s->be.alloc(s->be.ctx, ci_bytes, reinterpret_cast<void**>(&s->col_idx[i]));
        if (st != SDATTN_OK) return cleanup_fail(st);
    }
    if (s->ws_bytes) {
        st = s->be.alloc(s->be.ctx, s->ws_bytes, &s->ws);
        if (st != SDATTN_OK) return cleanup_fail(st);
    }
    if (desc->probe_interval > 0) {
        st = s->be.alloc(s->be.ctx, 8 * sizeof(int64_t), reinterpret_cast<void**>(&s->probe_buf));
        if (st != SDATTN_OK) return cleanup_fail(st);
        st = s->be.probe_init(s->be.ctx, s->probe_buf + 4);
        if (st != SDATTN_OK) return cleanup_fail(st);
    }
    *out = s;
    return SDATTN_OK;
}

sdattn_status sdattn_schedule_action(const sdattn_schedule* s, int32_t step, sdattn_action* out) {
    if (s == nullptr || out == nullptr) return fail(SDATTN_ERR_NULL, "schedule or out is NULL");
    if (step < 0 || step >= s->desc.total_steps) return fail(SDATTN_ERR_SHAPE, "step outside [0, total_steps)");
    *out = schedule_action_of(s->desc, step);
    return SDATTN_OK;
}

sdattn_status sdattn_schedule_step(sdattn_schedule* s, int32_t step, const void* q, const void* k,
                                   const void* v, void* o, float* lse, void* stream) {
    if (s == nullptr) return fail(SDATTN_ERR_NULL, "schedule is NULL");
    if (step < 0 || step >= s->desc.total_steps) return fail(SDATTN_ERR_SHAPE, "step outside [0, total_steps)");
    const sdattn_action act = schedule_action_of(s->desc, step);
    const Backend& be = s->be;
    const sdattn_problem* p = &s->prob;
    const bool blocks = s->desc.sel != SDATTN_SEL_COLUMNS;  // pooled or exact block pattern
    const int next = s->active < 0 ? 0 : 1 - s->active;
    sdattn_status st = SDATTN_OK;
    switch (act) {
        case SDATTN_ACT_DENSE:
            st = be.dense(be.ctx, p, q, k, v, o, lse, stream);
            break;
        case SDATTN_ACT_DENSE_SELECT:
            if (s->desc.sel == SDATTN_SEL_BLOCKS_EXACT) {
                float* l = lse != nullptr ? lse : s->lse;
                st = be.dense(be.ctx, p, q, k, v, o, l, stream);
                if (st == SDATTN_OK)
                    st = be.select_blocks_exact(be.ctx, p, q, k, l, s->desc.block_q, s->desc.block_k, &s->desc.budget,
                                                s->row_ptr[next], s->col_idx[next], s->nnz_cap, s->ws, s->ws_bytes,
                                                stream);
                if (st == SDATTN_OK)
                    st = plan_pattern(s, next, stream);
            } else if (blocks) {
                st = be.dense(be.ctx, p, q, k, v, o, lse, stream);
                if (st == SDATTN_OK)
                    st = be.select_blocks(be.ctx, p, q, k, s->desc.block_q, s->desc.block_k, &s->desc.budget,
                                          s->row_ptr[next], s->col_idx[next], s->nnz_cap, s->ws, s->ws_bytes, stream);
                if (st == SDATTN_OK)
                    st = plan_pattern(s, next, stream);
            } else {
                float* l = lse != nullptr ? lse : s->lse;
                st = be.dense(be.ctx, p, q, k, v, o, l, stream);
                if (st == SDATTN_OK)
                    st = be.select_columns(be.ctx, p, q, k, l, s->kcol, s->col_idx[next], s->ws, s->ws_bytes, stream);
            }
            if (st == SDATTN_OK) {
                s->active = next;
                s->last_select = step;
            }
            break;
        case SDATTN_ACT_SELECT_SPARSE:
            if (s->desc.sel != SDATTN_SEL_BLOCKS)
                return fail(SDATTN_ERR_STATE, "this selection needs a dense step (it uses the dense lse)");
            st = be.select_blocks(be.ctx, p, q, k, s->desc.block_q, s->desc.block_k, &s->desc.budget,
                                  s->row_ptr[next], s->col_idx[next], s->nnz_cap, s->ws, s->ws_bytes, stream);
            if (st == SDATTN_OK)
                st = plan_pattern(s, next, stream);
            if (st == SDATTN_OK)
                st = sparse_over(s, next, q, k, v, o, lse, stream);
            if (st == SDATTN_OK) {
                s->active = next;
                s->last_select = step;
            }
            break;
        case SDATTN_ACT_PROBE_SPARSE: {
            // blocks only (checked at create).  The probe goes into the idle
            // buffer; the adoption kernel copies it over the cached pattern
            // when the overlap is below min_overlap, so the cached buffer
            // stays the active one either way.
            if (s->active < 0) return fail(SDATTN_ERR_STATE, "probe step before any pattern was selected");
            // the adoption changes the cached pattern before the attention
            // launch, so every argument that launch checks is checked first
            if (s->pr.L > 0 && (q == nullptr || k == nullptr || v == nullptr || o == nullptr))
                return fail(SDATTN_ERR_NULL, "q, k, v and o must be non-NULL");
            const int a = s->active;
            st = be.select_blocks(be.ctx, p, q, k, s->desc.block_q, s->desc.block_k, &s->desc.budget,
                                  s->row_ptr[next], s->col_idx[next], s->nnz_cap, s->ws, s->ws_bytes, stream);
            if (st == SDATTN_OK)
                st = be.overlap(be.ctx, static_cast<int32_t>(s->rows), s->row_ptr[a], s->col_idx[a], s->row_ptr[next],
                                s->col_idx[next], s->probe_buf, stream);
            if (st == SDATTN_OK)
                st = be.probe_adopt(be.ctx, static_cast<int32_t>(s->rows), s->row_ptr[a], s->col_idx[a],
                                    s->row_ptr[next], s->col_idx[next], s->probe_buf, s->probe_buf + 4,
                                    s->desc.min_overlap, s->nnz_cap, stream);
            // the cached pattern may have been replaced: plan it again
            if (st == SDATTN_OK)
                st = plan_pattern(s, a, stream);
            if (st == SDATTN_OK)
                st = sparse_over(s, a, q, k, v, o, lse, stream);
            if (st == SDATTN_OK) s->n_probes += 1;
            return st;
        }
        case SDATTN_ACT_SPARSE:
            if (s->active < 0) return fail(SDATTN_ERR_STATE, "sparse step before any pattern was selected");
            if (blocks)
                st = sparse_over(s, s->active, q, k, v, o, lse, stream);
            else {
                // the kept columns' K/V rows are gathered once, then streamed
                // by every query tile of the group
                if (s->pr.L > 0 && (q == nullptr || k == nullptr || v == nullptr || o == nullptr))
                    return fail(SDATTN_ERR_NULL, "q, k, v and o must be non-NULL");
                st = be.gather_columns(be.ctx, p, k, v, s->col_idx[s->active], s->kcol, s->kc, s->vc, stream);
                if (st == SDATTN_OK) st = be.column_packed(be.ctx, p, q, s->kc, s->vc, s->kcol, o, lse, stream);
            }
            break;
    }
    if (st == SDATTN_OK) s->counts[act] += 1;
    return st;
}

sdattn_status sdattn_schedule_mask(const sdattn_schedule* s, const int32_t** row_ptr, const int32_t** col_idx,
                                   int64_t* nnz_capacity) {
    if (s == nullptr || row_ptr == nullptr || col_idx == nullptr || nnz_capacity == nullptr)
        return fail(SDATTN_ERR_NULL, "schedule or an output pointer is NULL");
    if (s->active < 0) return fail(SDATTN_ERR_STATE, "no pattern has been selected yet");
    *row_ptr = s->row_ptr[s->active];
    *col_idx = s->col_idx[s->active];
    *nnz_capacity = s->nnz_cap;
    return SDATTN_OK;
}

sdattn_status sdattn_schedule_stats(const sdattn_schedule* s, int64_t counts[4], int32_t* last_select_step) {
    if (s == nullptr || counts == nullptr || last_select_step == nullptr)
        return fail(SDATTN_ERR_NULL, "schedule or an output pointer is NULL");
    for (int i = 0; i < 4; ++i) counts[i] = s->counts[i];
    *last_select_step = s->last_select;
    return SDATTN_OK;
}

sdattn_status sdattn_schedule_probe_stats(const sdattn_schedule* s, int64_t* n_probes, int64_t* n_adopted,
                                          double* last_overlap, void* stream) {
    if (s == nullptr || n_probes == nullptr || n_adopted == nullptr || last_overlap == nullptr)
        return fail(SDATTN_ERR_NULL, "schedule or an output pointer is NULL");
    *n_probes = 0;
    *n_adopted = 0;
    *last_overlap = 1.0;
    if (s->probe_buf == nullptr) return SDATTN_OK;
    int64_t rec[4] = {0, 0, 0, 0};
    const sdattn_status st = s->be.probe_read(s->be.ctx, s->probe_buf + 4, rec, stream);
    if (st != SDATTN_OK) return st;
    *n_probes = rec[0];
    *n_adopted = rec[1];
    if (rec[0] > 0) *last_overlap = rec[3] > 0 ? static_cast<double>(rec[2]) / static_cast<double>(rec[3]) : 1.0;
    return SDATTN_OK;
}

void sdattn_schedule_destroy(sdattn_schedule* s) {
    if (s == nullptr) return;
    const Backend& be = s->be;
    if (s->probe_buf) be.release(be.ctx, s->probe_buf);
    for (int i = 0; i < 2; ++i) {
        if (s->row_ptr[i]) be.release(be.ctx, s->row_ptr[i]);
        if (s->plan[i]) be.release(be.ctx, s->plan[i]);
        if (s->col_idx[i]) be.release(be.ctx, s->col_idx[i]);
    }
    if (s->ws) be.release(be.ctx, s->ws);
    if (s->lse) be.release(be.ctx, s->lse);
    if (s->kc) be.release(be.ctx, s->kc);
    if (s->vc) be.release(be.ctx, s->vc);
    delete s;
}

}  // extern "C"
