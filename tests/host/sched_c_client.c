/* A plain C99 client of the schedule driver, linked against the driver and
 * the argument checks with the recording fake backend (no GPU).  It builds
 * the schedules of the five workloads, checks their action counts against
 * hand-counted tables, runs every step, injects backend failures (the step
 * must fail and leave the handle usable), and destroys every handle; built
 * with AddressSanitizer and UndefinedBehaviorSanitizer by the CPU test
 * suite.  Exits non-zero on the first mismatch, naming it. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "sdattn.h"

void sdattn_fake_reset(int fail_at_call, int fail_status);
int sdattn_fake_live_allocs(void);
int sdattn_fake_log_size(void);

#define CHECK(cond)                                                                   \
    do {                                                                              \
        if (!(cond)) {                                                                \
            fprintf(stderr, "check failed: %s (line %d): %s\n", #cond, __LINE__, sdattn_last_error()); \
            return 1;                                                                 \
        }                                                                             \
    } while (0)

typedef struct {
    const char* name;
    sdattn_problem p;
    sdattn_schedule_desc d;
    int32_t counts[4]; /* DENSE, DENSE_SELECT, SELECT_SPARSE, SPARSE */
} Case;

static int run_case(Case* c, int32_t* refresh) {
    sdattn_schedule* s = NULL;
    CHECK(sdattn_schedule_create(&c->p, &c->d, &s) == SDATTN_OK && s != NULL);
    int32_t counts[5] = {0, 0, 0, 0, 0};
    /* dummy device pointers: the fake backend only records them */
    char* base = (char*)0x100000;
    for (int32_t t = 0; t < c->d.total_steps; ++t) {
        sdattn_action a;
        CHECK(sdattn_schedule_action(s, t, &a) == SDATTN_OK);
        CHECK((int)a >= 0 && (int)a < 5);
        counts[a]++;
        CHECK(sdattn_schedule_step(s, t, base, base + 64, base + 128, base + 192, (float*)(base + 256), NULL) ==
              SDATTN_OK);
    }
    for (int i = 0; i < 4; ++i) CHECK(counts[i] == c->counts[i]);
    int64_t stats[4] = {0, 0, 0, 0};
    int32_t last = -2;
    CHECK(sdattn_schedule_stats(s, stats, &last) == SDATTN_OK);
    for (int i = 0; i < 4; ++i) CHECK(stats[i] == c->counts[i]);
    const int32_t *rp = NULL, *ci = NULL;
    int64_t cap = 0;
    CHECK(sdattn_schedule_mask(s, &rp, &ci, &cap) == SDATTN_OK && ci != NULL && cap > 0);
    /* a failing backend call: the step reports it and the handle stays usable */
    sdattn_fake_reset(0, SDATTN_ERR_HIP);
    CHECK(sdattn_schedule_step(s, c->d.total_steps - 1, base, base + 64, base + 128, base + 192,
                               (float*)(base + 256), NULL) == SDATTN_ERR_HIP);
    CHECK(strlen(sdattn_last_error()) > 0);
    sdattn_fake_reset(-1, 0);
    CHECK(sdattn_schedule_step(s, c->d.total_steps - 1, base, base + 64, base + 128, base + 192,
                               (float*)(base + 256), NULL) == SDATTN_OK);
    /* out-of-range steps are rejected on the host */
    sdattn_action a;
    CHECK(sdattn_schedule_action(s, c->d.total_steps, &a) != SDATTN_OK);
    CHECK(sdattn_schedule_action(s, -1, &a) != SDATTN_OK);
    sdattn_schedule_destroy(s);
    CHECK(sdattn_fake_live_allocs() == 0);
    (void)refresh;
    printf("%s: %d dense, %d dense+select, %d select+sparse, %d sparse\n", c->name, counts[0], counts[1], counts[2],
           counts[3]);
    return 0;
}

int main(void) {
    sdattn_budget topk25 = {SDATTN_BUDGET_TOPK, 0.25, 0.0, 1.0};
    sdattn_budget topk10 = {SDATTN_BUDGET_TOPK, 0.10, 0.0, 1.0};
    sdattn_budget topk5 = {SDATTN_BUDGET_TOPK, 0.05, 0.0, 1.0};
    sdattn_budget mass = {SDATTN_BUDGET_MASS, 0.0, 0.95, 0.10};
    static int32_t refresh5[2] = {64, 128};
    Case cases[5];
    memset(cases, 0, sizeof cases);
    /* the tiny fp32 layer: step 0 dense + top-25%, three sparse steps */
    cases[0].name = "tiny_fp32_h4_l512";
    cases[0].p = (sdattn_problem){1, 4, 4, 512, 64, SDATTN_F32, 0.0f};
    cases[0].d.total_steps = 4, cases[0].d.dense_steps = 1, cases[0].d.select_step = 0;
    cases[0].d.sel = SDATTN_SEL_BLOCKS, cases[0].d.block_q = cases[0].d.block_k = 64, cases[0].d.budget = topk25;
    cases[0].counts[0] = 0, cases[0].counts[1] = 1, cases[0].counts[2] = 0, cases[0].counts[3] = 3;
    /* 8K, capped mass, refresh every 32 steps */
    cases[1].name = "llada8b_8k";
    cases[1].p = (sdattn_problem){1, 32, 32, 8192, 128, SDATTN_BF16, 0.0f};
    cases[1].d.total_steps = 256, cases[1].d.dense_steps = 1, cases[1].d.select_step = 0;
    cases[1].d.refresh_interval = 32;
    cases[1].d.sel = SDATTN_SEL_BLOCKS, cases[1].d.block_q = cases[1].d.block_k = 64, cases[1].d.budget = mass;
    cases[1].counts[0] = 0, cases[1].counts[1] = 1, cases[1].counts[2] = 7, cases[1].counts[3] = 248;
    /* 32K, 26 dense steps, top-10% from step 26 */
    cases[2].name = "sparsed_32k";
    cases[2].p = (sdattn_problem){1, 32, 32, 32768, 128, SDATTN_BF16, 0.0f};
    cases[2].d.total_steps = 128, cases[2].d.dense_steps = 26, cases[2].d.select_step = 26;
    cases[2].d.sel = SDATTN_SEL_BLOCKS, cases[2].d.block_q = cases[2].d.block_k = 128, cases[2].d.budget = topk10;
    cases[2].counts[0] = 26, cases[2].counts[1] = 0, cases[2].counts[2] = 1, cases[2].counts[3] = 101;
    /* 64K, 205 dense steps, top-5% from step 205 */
    cases[3].name = "sparsed_64k";
    cases[3].p = (sdattn_problem){1, 32, 32, 65536, 128, SDATTN_BF16, 0.0f};
    cases[3].d.total_steps = 1024, cases[3].d.dense_steps = 205, cases[3].d.select_step = 205;
    cases[3].d.sel = SDATTN_SEL_BLOCKS, cases[3].d.block_q = cases[3].d.block_k = 128, cases[3].d.budget = topk5;
    cases[3].counts[0] = 205, cases[3].counts[1] = 0, cases[3].counts[2] = 1, cases[3].counts[3] = 818;
    /* 16K GQA columns, dense selections at 0, 64, 128 */
    cases[4].name = "pulsecol_dream7b_16k";
    cases[4].p = (sdattn_problem){1, 28, 4, 16384, 128, SDATTN_BF16, 0.0f};
    cases[4].d.total_steps = 192, cases[4].d.dense_steps = 1, cases[4].d.select_step = 0;
    cases[4].d.refresh_steps = refresh5, cases[4].d.n_refresh_steps = 2, cases[4].d.refresh_dense = 1;
    cases[4].d.sel = SDATTN_SEL_COLUMNS, cases[4].d.block_q = cases[4].d.block_k = 64;
    cases[4].d.column_keep_frac = 0.03;
    cases[4].counts[0] = 0, cases[4].counts[1] = 3, cases[4].counts[2] = 0, cases[4].counts[3] = 189;
    for (int i = 0; i < 5; ++i) {
        sdattn_fake_reset(-1, 0);
        if (run_case(&cases[i], refresh5)) return 1;
    }
    /* invalid descriptors fail in create and return no handle */
    sdattn_schedule* s = (sdattn_schedule*)0x1;
    sdattn_schedule_desc bad = cases[3].d;
    bad.select_step = 2000;
    CHECK(sdattn_schedule_create(&cases[3].p, &bad, &s) != SDATTN_OK && s == NULL);
    CHECK(sdattn_schedule_create(NULL, &cases[3].d, &s) == SDATTN_ERR_NULL);
    sdattn_schedule_destroy(NULL);
    CHECK(sdattn_fake_live_allocs() == 0);
    printf("schedule C client OK (ABI %d)\n", sdattn_abi_version());
    return 0;
}
