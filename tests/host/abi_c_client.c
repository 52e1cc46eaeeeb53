/* A plain C99 client of the library: includes the public header, links
 * libsdattn.so and calls the entry points that run on the host only
 * (version, status strings, workspace queries, argument checks).  Exits
 * non-zero on the first mismatch, naming it. */
#include <stdio.h>
#include <string.h>

#include "sdattn.h"

#define CHECK(cond)                                                   \
    do {                                                              \
        if (!(cond)) {                                                \
            fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
            return 1;                                                 \
        }                                                             \
    } while (0)

int main(void) {
    CHECK(sdattn_abi_version() == SDATTN_ABI_VERSION);
    CHECK(strcmp(sdattn_status_string(SDATTN_ERR_SHAPE), "SDATTN_ERR_SHAPE") == 0);
    CHECK(strcmp(sdattn_status_string(SDATTN_OK), "SDATTN_OK") == 0);

    /* the 64K block workload: 32 heads, 128-token blocks, top 5% */
    sdattn_problem p = {1, 32, 32, 65536, 128, SDATTN_BF16, 0.0f};
    sdattn_budget topk = {SDATTN_BUDGET_TOPK, 0.05, 0.0, 1.0};
    size_t ws = 0, ws_exact = 0;
    int64_t nnz = 0, nnz_exact = 0;
    CHECK(sdattn_select_blocks_workspace(&p, 128, 128, &topk, &ws, &nnz) == SDATTN_OK);
    CHECK(nnz == 32 * 512 * 26);
    CHECK(sdattn_select_blocks_exact_workspace(&p, 128, 128, &topk, &ws_exact, &nnz_exact) == SDATTN_OK);
    CHECK(nnz_exact == nnz && ws_exact >= ws + (size_t)32 * 512 * 512 * 4);

    /* split plan of the 64K block workload: items, slot table and plan ints,
       then 2 * 512 partial slots of 128 * 129 floats */
    size_t wss = 0;
    CHECK(sdattn_block_split_workspace(&p, 128, 128, &wss) == SDATTN_OK);
    CHECK(wss >= (size_t)2 * 512 * 128 * 129 * 4 + (size_t)3 * 16384 * 4);
    CHECK(sdattn_block_split_workspace(&p, 128, 128, NULL) == SDATTN_ERR_NULL);

    /* the 16K GQA column workload: 492 columns per kv head */
    sdattn_problem pc = {1, 28, 4, 16384, 128, SDATTN_BF16, 0.0f};
    size_t wsc = 0;
    CHECK(sdattn_select_columns_workspace(&pc, 492, &wsc) == SDATTN_OK && wsc > 0);

    /* argument checks fail on the host, before anything is enqueued */
    CHECK(sdattn_forward_dense(NULL, NULL, NULL, NULL, NULL, NULL, NULL) == SDATTN_ERR_NULL);
    CHECK(strlen(sdattn_last_error()) > 0);
    sdattn_problem bad = p;
    bad.head_dim = 96;
    CHECK(sdattn_forward_dense(&bad, NULL, NULL, NULL, NULL, NULL, NULL) == SDATTN_ERR_UNSUPPORTED ||
          sdattn_forward_dense(&bad, NULL, NULL, NULL, NULL, NULL, NULL) == SDATTN_ERR_SHAPE);
    CHECK(sdattn_mask_overlap(-1, NULL, NULL, NULL, NULL, NULL, NULL) == SDATTN_ERR_SHAPE);

    /* a schedule whose first sparse step would have no pattern */
    sdattn_schedule_desc d;
    memset(&d, 0, sizeof d);
    d.total_steps = 10;
    d.dense_steps = 2;
    d.select_step = 5;
    d.sel = SDATTN_SEL_BLOCKS;
    d.block_q = d.block_k = 128;
    d.budget = topk;
    sdattn_schedule* s = NULL;
    CHECK(sdattn_schedule_create(&p, &d, &s) == SDATTN_ERR_SHAPE && s == NULL);
    sdattn_schedule_destroy(NULL); /* a no-op */

    printf("C client OK (ABI %d)\n", sdattn_abi_version());
    return 0;
}
