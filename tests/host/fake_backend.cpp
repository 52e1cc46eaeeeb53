// Recording fake backend for CPU tests of the schedule driver.
//
// Built (with the driver and the argument checks, no HIP) into
// libsdattn_fake.so.  Every backend call appends a line to a log; a call can
// be made to fail on purpose; "device" buffers are host allocations whose
// count is tracked so leaks show up.

#include <stdio.h>
#include <stdlib.h>

#include <string>
#include <vector>

#include "schedule.h"

namespace {

std::vector<std::string> g_log;
int g_calls = 0;
int g_fail_at = -1;  // 0-based index of the backend compute call that fails
sdattn_status g_fail_status = SDATTN_ERR_HIP;
int g_live = 0;

std::string ptr(const void* p) {
    char b[32];
    snprintf(b, sizeof b, "%p", p);
    return b;
}

sdattn_status record(const std::string& line) {
    const int idx = g_calls++;
    if (idx == g_fail_at) {
        g_log.push_back("FAIL " + line);
        return sdattn::fail(g_fail_status, "injected failure");
    }
    g_log.push_back(line);
    return SDATTN_OK;
}

sdattn_status f_dense(void*, const sdattn_problem*, const void*, const void*, const void*, void* o, float* lse,
                      void*) {
    return record("dense o=" + ptr(o) + " lse=" + ptr(lse));
}
sdattn_status f_select_blocks(void*, const sdattn_problem*, const void*, const void*, int32_t bq, int32_t bk,
                              const sdattn_budget*, int32_t* rp, int32_t* ci, int64_t cap, void* ws, size_t wsb,
                              void*) {
    return record("select_blocks rp=" + ptr(rp) + " ci=" + ptr(ci) + " cap=" + std::to_string(cap) +
                  " bq=" + std::to_string(bq) + " bk=" + std::to_string(bk));
}
sdattn_status f_block_sparse(void*, const sdattn_problem*, const void*, const void*, const void*, int32_t,
                             int32_t, const int32_t* rp, const int32_t* ci, const int32_t* plan, void* o, float*,
                             void*) {
    return record("block_sparse rp=" + ptr(rp) + " ci=" + ptr(ci) + " plan=" + ptr(plan) + " o=" + ptr(o));
}
sdattn_status f_block_plan(void*, const sdattn_problem*, int32_t bq, int32_t bk, const int32_t* rp, int32_t* plan,
                           void*) {
    return record("block_plan rp=" + ptr(rp) + " plan=" + ptr(plan) + " bq=" + std::to_string(bq) +
                  " bk=" + std::to_string(bk));
}
sdattn_status f_block_split_ws(void*, const sdattn_problem*, int32_t, int32_t, size_t* ws) {
    *ws = 1 << 20;
    return SDATTN_OK;
}
sdattn_status f_block_split_plan(void*, const sdattn_problem*, int32_t bq, int32_t bk, const int32_t* rp, void* ws,
                                 size_t wsb, void*) {
    return record("block_split_plan rp=" + ptr(rp) + " ws=" + ptr(ws) + " bytes=" + std::to_string(wsb) +
                  " bq=" + std::to_string(bq) + " bk=" + std::to_string(bk));
}
sdattn_status f_block_sparse_split(void*, const sdattn_problem*, const void*, const void*, const void*, int32_t,
                                   int32_t, const int32_t* rp, const int32_t* ci, void* ws, size_t wsb, void* o, float*,
                                   void*) {
    return record("block_sparse_split rp=" + ptr(rp) + " ci=" + ptr(ci) + " ws=" + ptr(ws) + " bytes=" +
                  std::to_string(wsb) + " o=" + ptr(o));
}
sdattn_status f_select_columns(void*, const sdattn_problem*, const void*, const void*, const float* lse, int32_t kcol,
                               int32_t* ci, void*, size_t, void*) {
    return record("select_columns lse=" + ptr(lse) + " ci=" + ptr(ci) + " kcol=" + std::to_string(kcol));
}
sdattn_status f_column_sparse(void*, const sdattn_problem*, const void*, const void*, const void*, const int32_t* ci,
                              int32_t kcol, void* o, float*, void*) {
    return record("column_sparse ci=" + ptr(ci) + " kcol=" + std::to_string(kcol) + " o=" + ptr(o));
}
sdattn_status f_ws_blocks(void*, const sdattn_problem* p, int32_t bq, int32_t bk, const sdattn_budget* b, size_t* ws,
                          int64_t* nnz) {
    sdattn::Problem pr;
    sdattn_status st = sdattn::check_problem(p, &pr);
    if (st != SDATTN_OK) return st;
    sdattn::BlockPlan plan;
    st = sdattn::check_blocks(pr, bq, bk, b, &plan);
    if (st != SDATTN_OK) return st;
    *ws = 4096;
    *nnz = plan.max_nnz;
    return SDATTN_OK;
}
sdattn_status f_ws_columns(void*, const sdattn_problem*, int32_t, size_t* ws) {
    *ws = 1024;
    return SDATTN_OK;
}
sdattn_status f_alloc(void*, size_t bytes, void** out) {
    *out = malloc(bytes ? bytes : 1);
    ++g_live;
    return SDATTN_OK;
}
void f_release(void*, void* p) {
    free(p);
    --g_live;
}

sdattn_status f_overlap(void*, int32_t rows, const int32_t* rpa, const int32_t* cia, const int32_t* rpb,
                        const int32_t* cib, int64_t* counts, void*) {
    return record("overlap rows=" + std::to_string(rows) + " a=" + ptr(rpa) + "," + ptr(cia) + " b=" + ptr(rpb) +
                  "," + ptr(cib) + " counts=" + ptr(counts));
}
sdattn_status f_probe_adopt(void*, int32_t rows, int32_t* rp_dst, int32_t* ci_dst, const int32_t* rp_src,
                            const int32_t* ci_src, const int64_t* counts, void* state, double min_overlap,
                            int64_t max_copy, void*) {
    char th[32];
    snprintf(th, sizeof th, "%g", min_overlap);
    const sdattn_status st = record("probe_adopt rows=" + std::to_string(rows) + " dst=" + ptr(rp_dst) + "," +
                                    ptr(ci_dst) + " src=" + ptr(rp_src) + "," + ptr(ci_src) + " counts=" +
                                    ptr(counts) + " state=" + ptr(state) + " min_overlap=" + th +
                                    " max_copy=" + std::to_string(max_copy));
    if (st == SDATTN_OK) static_cast<int64_t*>(state)[0] += 1;  // probes; the fake never adopts
    return st;
}
sdattn_status f_probe_init(void*, void* state) {
    for (int i = 0; i < 4; ++i) static_cast<int64_t*>(state)[i] = 0;
    g_log.push_back("probe_init state=" + ptr(state));
    return SDATTN_OK;
}
sdattn_status f_probe_read(void*, const void* state, int64_t out[4], void*) {
    for (int i = 0; i < 4; ++i) out[i] = static_cast<const int64_t*>(state)[i];
    return SDATTN_OK;
}

sdattn_status f_select_blocks_exact(void*, const sdattn_problem*, const void*, const void*, const float* lse,
                                    int32_t bq, int32_t bk, const sdattn_budget*, int32_t* rp, int32_t* ci,
                                    int64_t cap, void*, size_t, void*) {
    return record("select_blocks_exact lse=" + ptr(lse) + " rp=" + ptr(rp) + " ci=" + ptr(ci) +
                  " cap=" + std::to_string(cap) + " bq=" + std::to_string(bq) + " bk=" + std::to_string(bk));
}
sdattn_status f_ws_blocks_exact(void* ctx, const sdattn_problem* p, int32_t bq, int32_t bk, const sdattn_budget* b,
                                size_t* ws, int64_t* nnz) {
    const sdattn_status st = f_ws_blocks(ctx, p, bq, bk, b, ws, nnz);
    *ws += 8192;
    return st;
}

sdattn_status f_gather_columns(void*, const sdattn_problem*, const void*, const void*, const int32_t* ci, int32_t kcol,
                               void* kc, void* vc, void*) {
    return record("gather_columns ci=" + ptr(ci) + " kcol=" + std::to_string(kcol) + " kc=" + ptr(kc) +
                  " vc=" + ptr(vc));
}
sdattn_status f_column_packed(void*, const sdattn_problem*, const void*, const void* kc, const void* vc, int32_t kcol,
                              void* o, float*, void*) {
    return record("column_packed kc=" + ptr(kc) + " vc=" + ptr(vc) + " kcol=" + std::to_string(kcol) + " o=" + ptr(o));
}

const sdattn::Backend kFake = {nullptr,          f_dense,          f_select_blocks, f_block_sparse, f_select_columns,
                               f_column_sparse,  f_ws_blocks,      f_ws_columns,    f_alloc,        f_release,
                               f_overlap,        f_probe_adopt,    f_probe_init,    f_probe_read,   f_select_blocks_exact,
                               f_ws_blocks_exact, f_gather_columns, f_column_packed, f_block_plan,
                               f_block_split_ws, f_block_split_plan, f_block_sparse_split};

}  // namespace

namespace sdattn {
const Backend& default_backend() { return kFake; }
}  // namespace sdattn

#define FAKE_API __attribute__((visibility("default")))

extern "C" {
FAKE_API void sdattn_fake_reset(int fail_at_call, int fail_status) {
    g_log.clear();
    g_calls = 0;
    g_fail_at = fail_at_call;
    g_fail_status = static_cast<sdattn_status>(fail_status);
}
FAKE_API int sdattn_fake_log_size(void) { return static_cast<int>(g_log.size()); }
FAKE_API const char* sdattn_fake_log_entry(int i) { return g_log.at(static_cast<size_t>(i)).c_str(); }
FAKE_API int sdattn_fake_live_allocs(void) { return g_live; }
}
