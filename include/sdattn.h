/*
 * sdattn.h — sparse bidirectional attention for diffusion-LM denoising,
 * MI355X (gfx950) HIP library, C ABI.
 *
 * What the library computes (the pages' problem statement):
 *   - Diffusion LMs recompute full bidirectional attention at every denoising
 *     step because no KV cache applies (Step-dLLM, Abstract; PulseCol,
 *     Abstract).  sdattn_forward_dense is that non-causal attention.
 *   - Head-specific sparse patterns are computed once after full-attention
 *     warm-up steps and reused at the later steps (SparseD, abstract), or
 *     refreshed at anchor steps with a head-adaptive global budget
 *     (Step-dLLM, Abstract): sdattn_select_blocks builds per-head block lists
 *     from mean-pooled query/key block scores with a top-k or a cumulative
 *     pooled-mass budget, and sdattn_forward_block_sparse attends over them.
 *   - Column-sparse attention keeps individual key columns chosen from
 *     column-summed attention at an early step, refreshed at a few
 *     intermediate steps (PulseCol, Abstract): sdattn_select_columns and
 *     sdattn_forward_column_sparse.
 *   - The block pattern can also come from the exact attention mass of each
 *     block pair after a dense step (sdattn_select_blocks_exact).
 *   - A host-side schedule handle runs warm-up, reuse and refresh, and can
 *     probe the pattern between anchors and refresh it when it has moved
 *     (sdattn_mask_overlap).
 *
 * Conventions for every call
 *   Tensors.   Caller-owned device buffers, contiguous.  q and o are
 *              [B][Hq][L][d]; k and v are [B][Hkv][L][d]; lse is
 *              [B][Hq][L] float32 natural-log log-sum-exp.  Element type is
 *              the problem's dtype (float32 or bfloat16); o has the input
 *              dtype.  Query head h reads kv head h / (Hq / Hkv).
 *   Scale.     softmax_scale <= 0 selects 1/sqrt(d).
 *   Shapes.    B, Hq, Hkv >= 1; Hq % Hkv == 0; L >= 0 (L == 0 is a no-op that
 *              returns SDATTN_OK); d in {64, 128}.  Any L is accepted: a
 *              last, partial query or key block is handled (a partial block is
 *              pooled as the mean of the tokens it has).
 *   Blocks.    block_q, block_k in {64, 128}.  Block row r = (b*Hq + h)*nQB + I
 *              with nQB = ceil(L / block_q), nKB = ceil(L / block_k).
 *   CSR.       row_ptr[B*Hq*nQB + 1] int32, col_idx[nnz] int32; each row lists
 *              its kept key blocks in ascending order without duplicates.
 *   Streams.   `stream` is a hipStream_t (NULL = the null stream).  Compute
 *              calls enqueue kernels and return without synchronising; a
 *              fault inside a kernel surfaces at the caller's next sync.
 *   Errors.    Arguments are validated on the host before anything is
 *              enqueued, so a call that returns an error has written nothing.
 *              sdattn_last_error() returns a thread-local detail string for
 *              the last failing call on this thread.  No C++ exception
 *              crosses the ABI.
 *   Memory.    Stateless calls allocate nothing: workspace is passed in and
 *              sized by the *_workspace queries.  Only a schedule handle
 *              allocates (in create) and frees (in destroy).
 *   Threads.   Stateless calls are reentrant.  A schedule handle must not be
 *              used from two threads at once.
 */
#ifndef SDATTN_H
#define SDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SDATTN_ABI_VERSION 6

/* Exported entry points (the library is built with hidden visibility). */
#define SDATTN_API __attribute__((visibility("default")))

typedef enum {
    SDATTN_OK = 0,
    SDATTN_ERR_NULL = 1,        /* a required pointer is NULL                 */
    SDATTN_ERR_SHAPE = 2,       /* sizes out of range or inconsistent         */
    SDATTN_ERR_DTYPE = 3,       /* unsupported element type                   */
    SDATTN_ERR_BUDGET = 4,      /* budget parameters out of range             */
    SDATTN_ERR_WORKSPACE = 5,   /* workspace smaller than the query returned  */
    SDATTN_ERR_CAPACITY = 6,    /* output index buffer too small              */
    SDATTN_ERR_HIP = 7,         /* a HIP runtime call failed (see last_error) */
    SDATTN_ERR_UNSUPPORTED = 8, /* valid request this build does not support  */
    SDATTN_ERR_STATE = 9        /* schedule misuse (e.g. sparse step, no mask) */
} sdattn_status;

typedef enum { SDATTN_F32 = 0, SDATTN_BF16 = 1 } sdattn_dtype;

typedef struct {
    int32_t batch;       /* B   */
    int32_t q_heads;     /* Hq  */
    int32_t kv_heads;    /* Hkv */
    int32_t seq_len;     /* L   */
    int32_t head_dim;    /* d   */
    sdattn_dtype dtype;
    float softmax_scale; /* <= 0: 1/sqrt(d) */
} sdattn_problem;
/* Shape limits (SDATTN_ERR_SHAPE beyond): B * Hq * (L + 63) <= 2e9, and
 * (L + 128) * d * 4 < 2^32 - 2^16 (one head's K or V rows are addressed with
 * 32-bit byte offsets). */

typedef enum { SDATTN_BUDGET_TOPK = 0, SDATTN_BUDGET_MASS = 1 } sdattn_budget_kind;

/*
 * Block budget.
 *   TOPK: every row keeps k = max(1, ceil(keep_frac * nKB - 1e-9)) blocks
 *         (clamped to nKB), the blocks of largest pooled mass, ties toward
 *         the lower block index.  0 < keep_frac <= 1.
 *   MASS: every row keeps the shortest prefix of its blocks, ordered by
 *         (pooled mass desc, index asc), whose cumulative mass reaches tau*;
 *         tau* = mass unless that would make the mean kept fraction over all
 *         rows exceed max_mean_density, in which case tau* is the largest
 *         cumulative-mass value of any row, not above `mass`, that keeps the
 *         mean within the cap; every row keeps at least one block.
 *         0 < mass <= 1, 0 < max_mean_density <= 1 (1 = no cap).  The number
 *         of kept blocks is at most max(rows, floor(max_mean_density *
 *         rows * nKB + 1e-9)).
 * Pooled mass of row (b, h, I): softmax over J of scale * <Qp[I], Kp[J]>,
 * with Qp, Kp the means of the query / key tokens of each block.
 */
typedef struct {
    sdattn_budget_kind kind;
    double keep_frac;
    double mass;
    double max_mean_density;
} sdattn_budget;

/* ABI version of the loaded library (SDATTN_ABI_VERSION). */
SDATTN_API int sdattn_abi_version(void);

/* Static name of a status code ("SDATTN_OK", ...); never NULL. */
SDATTN_API const char* sdattn_status_string(sdattn_status s);

/* Thread-local detail of the last failing call on this thread ("" if none).
 * The pointer stays valid until the next failing call on the same thread. */
SDATTN_API const char* sdattn_last_error(void);

/*
 * Dense bidirectional attention (SparseD, abstract: full attention in the
 * early denoising steps; the FlashAttention baseline of all three methods).
 * For every query row i of head h over all L keys of kv head g(h):
 *   o_i = sum_j softmax_j(scale * q_i . k_j) v_j,  lse_i = ln sum_j exp(scale * q_i . k_j).
 * q, k, v, o: required device pointers (layout above).  lse: optional
 * (NULL = not written).  bf16 uses bf16 MFMA with fp32 accumulation and
 * bf16 probabilities; fp32 uses fp32 arithmetic throughout.
 */
SDATTN_API sdattn_status sdattn_forward_dense(const sdattn_problem* p, const void* q, const void* k,
                                   const void* v, void* o, float* lse, void* stream);

/*
 * Workspace bytes and the worst-case number of kept blocks (col_idx
 * capacity) for sdattn_select_blocks with this problem, block shape and
 * budget.  Host only; synchronous.
 */
SDATTN_API sdattn_status sdattn_select_blocks_workspace(const sdattn_problem* p, int32_t block_q,
                                             int32_t block_k, const sdattn_budget* budget,
                                             size_t* ws_bytes, int64_t* max_nnz);

/*
 * Head-specific block pattern from pooled scores (SparseD, abstract;
 * Step-dLLM, Abstract): mean-pool query and key blocks, score every (I, J)
 * pair, softmax over J, and keep blocks under the budget.  Writes row_ptr
 * [rows + 1] and col_idx [nnz] (CSR above, rows ascending).  col_capacity
 * is the number of int32 slots in col_idx; it must be >= max_nnz from the
 * workspace query.  block_mass (optional, [B][Hq][nQB][nKB] float32)
 * receives the pooled mass.  ws/ws_bytes: device workspace from
 * sdattn_select_blocks_workspace (ws may be NULL when ws_bytes is 0).
 * Selection is made in fp32: candidates whose mass lies within ~1e-6
 * relative of a row's cut may differ from an exact-arithmetic selection.
 * Limit: nKB <= 1024 (SDATTN_ERR_UNSUPPORTED beyond).
 */
SDATTN_API sdattn_status sdattn_select_blocks(const sdattn_problem* p, const void* q, const void* k,
                                   int32_t block_q, int32_t block_k, const sdattn_budget* budget,
                                   int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                                   float* block_mass, void* ws, size_t ws_bytes, void* stream);

/*
 * sdattn_select_blocks without any allocation, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, result and errors as
 * sdattn_select_blocks, without ws/ws_bytes: the workspace is a static
 * device array of SDATTN_NOALLOC_SCRATCH_BYTES inside the library, one copy
 * per GPU, held until the process ends (its address is looked up once per
 * device, at the first call on that device).  The call allocates nothing.
 * A selection whose workspace (sdattn_select_blocks_workspace) exceeds
 * SDATTN_NOALLOC_SCRATCH_BYTES fails with SDATTN_ERR_WORKSPACE before
 * anything is enqueued.  The work runs on the stream's device (the current
 * device for the NULL stream).  Every call on one GPU shares that GPU's
 * scratch: calls that overlap on one GPU (unordered streams or threads)
 * race and must be serialised by the caller.
 */
#define SDATTN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
SDATTN_API sdattn_status sdattn_select_blocks_noalloc(const sdattn_problem* p, const void* q, const void* k,
                                           int32_t block_q, int32_t block_k, const sdattn_budget* budget,
                                           int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                                           float* block_mass, void* stream);

/*
 * Exact block mass, the alternative to pooled scores (SparseD, abstract:
 * head-specific patterns of where attention goes; Step-dLLM, Abstract: heads
 * concentrate their attention mass to different extents).  The mass of key
 * block J for query block I of head h is the attention that block's queries
 * actually give to its keys:
 *   A[b][h][I][J] = (1/|I|) sum_{i in I} sum_{j in J} exp(scale q_i.k_j - lse_i),
 * with lse [B][Hq][L] the log-sum-exp of the full attention of the same q, k
 * (sdattn_forward_dense), so every row of A sums to 1.  The budget and the
 * output are those of sdattn_select_blocks, with A in place of the pooled
 * mass.  Workspace bytes and max_nnz from
 * sdattn_select_blocks_exact_workspace (host only); block_mass (optional)
 * receives A.  The scores are exact softmax probabilities (bf16 inputs: MFMA
 * with fp32 accumulation), summed in fp32; selection is made in fp32 as in
 * sdattn_select_blocks.  Cost: one pass of Q K^T over all (i, j).  Errors
 * as sdattn_select_blocks, and SDATTN_ERR_NULL when lse is NULL (L > 0);
 * the workspace must be non-NULL and at least the queried size.
 */
SDATTN_API sdattn_status sdattn_select_blocks_exact_workspace(const sdattn_problem* p, int32_t block_q,
                                                   int32_t block_k, const sdattn_budget* budget,
                                                   size_t* ws_bytes, int64_t* max_nnz);
SDATTN_API sdattn_status sdattn_select_blocks_exact(const sdattn_problem* p, const void* q, const void* k,
                                         const float* lse, int32_t block_q, int32_t block_k,
                                         const sdattn_budget* budget, int32_t* row_ptr,
                                         int32_t* col_idx, int64_t col_capacity, float* block_mass,
                                         void* ws, size_t ws_bytes, void* stream);

/*
 * Block-sparse attention (Step-dLLM, Abstract: block-sparse attention with a
 * reused mask).  Query block I of head h attends only the key tokens of the
 * key blocks listed in its CSR row; an empty row gives o = 0 and
 * lse = -inf.  row_ptr/col_idx: device CSR (above), not modified.
 */
SDATTN_API sdattn_status sdattn_forward_block_sparse(const sdattn_problem* p, const void* q, const void* k,
                                          const void* v, int32_t block_q, int32_t block_k,
                                          const int32_t* row_ptr, const int32_t* col_idx,
                                          void* o, float* lse, void* stream);

/*
 * Dispatch plan of the block-sparse forward for one pattern.  Under a
 * head-adaptive budget (Step-dLLM, Abstract) heads keep very different
 * numbers of key blocks, so the work of a block row depends on its head; the
 * plan spreads that work evenly over the GPU's XCDs while keeping each XCD on
 * consecutive rows of one head at a time (their K/V in its L2).  Computed on
 * the device from row_ptr alone (one small kernel, enqueued on `stream`);
 * worth computing once per pattern when the pattern is reused over many
 * steps.  plan: device int32 [B*Hq*nQB], written (a permutation of the block
 * rows: workgroup i of the planned forward computes row plan[i]).  Errors:
 * SDATTN_ERR_UNSUPPORTED for block sizes other than 64/128, SDATTN_ERR_NULL
 * for a NULL row_ptr or plan (L > 0), SDATTN_ERR_SHAPE when B*Hq*nQB does not
 * fit in int32.  row_ptr is trusted as for the forward.
 */
SDATTN_API sdattn_status sdattn_block_plan(const sdattn_problem* p, int32_t block_q, int32_t block_k,
                                const int32_t* row_ptr, int32_t* plan, void* stream);

/*
 * sdattn_forward_block_sparse over a dispatch plan from sdattn_block_plan for
 * the same row_ptr (same arguments, results and errors; plan NULL is the
 * unplanned call).  The result does not depend on the plan: every row is
 * computed by one workgroup either way.  Workgroups whose plan entry is not a
 * block row of the problem write nothing.  bfloat16 problems use the plan;
 * float32 problems accept it and compute rows in their natural order.
 */
SDATTN_API sdattn_status sdattn_forward_block_sparse_planned(const sdattn_problem* p, const void* q, const void* k,
                                                  const void* v, int32_t block_q, int32_t block_k,
                                                  const int32_t* row_ptr, const int32_t* col_idx,
                                                  const int32_t* plan, void* o, float* lse, void* stream);

/*
 * Split rows.  A dispatch plan cannot shorten a launch below its longest
 * block row: under a head-adaptive budget (Step-dLLM, Abstract) one head may
 * keep most key blocks while the others keep few.  A split plan cuts every
 * row with more kept blocks than T = max(4, ceil(nnz / slots)) (slots = the
 * workgroups the GPU holds at once: 1024 for 64-query blocks, 768 for 128)
 * into c = min(8, ceil(ne / T)) chunks of consecutive kept blocks.  Each
 * chunk is computed by its own workgroup, which writes its output
 * normalised over the chunk together with the chunk's log-sum-exp; a merge
 * then combines a row's chunks, O = sum_k exp(lse_k - LSE) O_k with
 * LSE = log sum_k exp(lse_k) (the online-softmax merge of partial rows, LoSA
 * section 3, step 5).  The chunks of the cut rows are dealt first, spread
 * over the XCDs; the rows that are not cut follow, computed whole, in the
 * dispatch plan's order.
 *
 * sdattn_block_split_workspace: bytes of the one workspace that holds the
 * plan and the partial results (host only; 0 when L == 0).  Errors as for
 * sdattn_block_plan, and SDATTN_ERR_SHAPE when B*Hq*nQB >= 2^24.
 *
 * sdattn_block_split_plan: computes the split plan of a pattern into ws
 * (device, enqueued on `stream`; worth doing once per pattern).  It depends on
 * row_ptr only.  SDATTN_ERR_NULL for a NULL row_ptr (L > 0),
 * SDATTN_ERR_WORKSPACE for a NULL or short ws.
 *
 * sdattn_forward_block_sparse_split: sdattn_forward_block_sparse over a split
 * plan computed for the same row_ptr and problem, in the same ws (which the
 * call also writes: the partial results).  The plan is trusted like row_ptr:
 * a ws that sdattn_block_split_plan did not fill for this pattern and
 * problem can make the kernels read and write outside it.  Results equal the unsplit
 * forward's within the bf16 rounding of O (rows that are not cut are
 * bit-identical to it).  Two kernels on `stream`: the forward over the plan's
 * items, then the merge.  Calls that share a ws must not overlap.  float32
 * problems compute every row whole.  Errors as for the forward, plus
 * SDATTN_ERR_WORKSPACE and SDATTN_ERR_SHAPE as above.
 */
SDATTN_API sdattn_status sdattn_block_split_workspace(const sdattn_problem* p, int32_t block_q, int32_t block_k,
                                           size_t* ws_bytes);
SDATTN_API sdattn_status sdattn_block_split_plan(const sdattn_problem* p, int32_t block_q, int32_t block_k,
                                      const int32_t* row_ptr, void* ws, size_t ws_bytes, void* stream);
SDATTN_API sdattn_status sdattn_forward_block_sparse_split(const sdattn_problem* p, const void* q, const void* k,
                                                const void* v, int32_t block_q, int32_t block_k,
                                                const int32_t* row_ptr, const int32_t* col_idx, void* ws,
                                                size_t ws_bytes, void* o, float* lse, void* stream);

/*
 * Overlap of two block patterns (the test of an adaptive anchor: Step-dLLM,
 * Abstract, patterns hold only locally across steps).  A and B are CSR
 * patterns over the same `rows` rows (row_ptr [rows + 1], rows ascending and
 * duplicate-free, as sdattn_select_blocks writes them).  Writes, to the
 * device array counts [3] (int64): |A n B| over (row, block) pairs, |A| =
 * row_ptr_a[rows] - row_ptr_a[0] and |B| likewise.  Enqueued on `stream`;
 * counts is overwritten (not accumulated).  rows >= 0 (rows == 0 gives
 * {0, 0, 0}); SDATTN_ERR_NULL if a pointer is NULL while rows > 0, or if
 * counts is NULL.  The patterns are trusted: a row_ptr that is not
 * non-decreasing, or that points past its col_idx, reads out of bounds.
 */
SDATTN_API sdattn_status sdattn_mask_overlap(int32_t rows, const int32_t* row_ptr_a, const int32_t* col_idx_a,
                                  const int32_t* row_ptr_b, const int32_t* col_idx_b, int64_t* counts,
                                  void* stream);

/* Workspace bytes for sdattn_select_columns.  Host only. */
SDATTN_API sdattn_status sdattn_select_columns_workspace(const sdattn_problem* p, int32_t kcol,
                                              size_t* ws_bytes);

/*
 * Column pattern from column-summed attention (PulseCol, Abstract).  For kv
 * head g: C[g, j] = sum over the query heads h of group g and all query rows
 * i of exp(scale * q_i . k_j - lse_i), lse from the full attention of the
 * same q, k (sdattn_forward_dense).  Keeps the kcol columns of largest C
 * (ties toward the lower index), 1 <= kcol <= L, written ascending to
 * col_idx [B][Hkv][kcol].  col_scores (optional, [B][Hkv][L] float64)
 * receives C.  Column sums are accumulated in fp64.
 */
SDATTN_API sdattn_status sdattn_select_columns(const sdattn_problem* p, const void* q, const void* k,
                                    const float* lse, int32_t kcol, int32_t* col_idx,
                                    double* col_scores, void* ws, size_t ws_bytes, void* stream);

/*
 * Column-sparse attention (PulseCol, Abstract): every query of every query
 * head of group g attends exactly the key tokens col_idx[b][g][0..kcol-1]
 * (ascending, distinct, each < L).  1 <= kcol <= L.
 */
SDATTN_API sdattn_status sdattn_forward_column_sparse(const sdattn_problem* p, const void* q, const void* k,
                                           const void* v, const int32_t* col_idx, int32_t kcol,
                                           void* o, float* lse, void* stream);

/*
 * The column-sparse forward in two calls, for steps that reuse one column
 * pattern (PulseCol, Abstract: the selected columns are shared by the query
 * heads of a group and reused across steps).  sdattn_gather_columns copies the
 * listed rows once: kc[b][g][j] = k[b][g][col_idx[b][g][j]] and likewise vc,
 * j < kcol (kc, vc caller-owned, [B][Hkv][kcol][d] in the problem's dtype;
 * indices outside [0, L) are clamped).  sdattn_forward_column_packed then
 * gives exactly the result of sdattn_forward_column_sparse with that col_idx,
 * reading the gathered rows as contiguous tiles instead of gathering in
 * every query tile.  Errors: SDATTN_ERR_NULL for a NULL q, kc, vc, o (or k,
 * v, col_idx, kc, vc for the gather); SDATTN_ERR_BUDGET unless
 * 1 <= kcol <= L; L == 0 is a no-op.
 */
SDATTN_API sdattn_status sdattn_gather_columns(const sdattn_problem* p, const void* k, const void* v,
                                    const int32_t* col_idx, int32_t kcol, void* kc, void* vc,
                                    void* stream);
SDATTN_API sdattn_status sdattn_forward_column_packed(const sdattn_problem* p, const void* q, const void* kc,
                                           const void* vc, int32_t kcol, void* o, float* lse,
                                           void* stream);

/* ------------------------------------------------------------------------ */
/* Host-side step-schedule driver.                                          */
/* ------------------------------------------------------------------------ */

typedef enum {
    SDATTN_SEL_BLOCKS = 0,        /* block pattern from pooled scores           */
    SDATTN_SEL_COLUMNS = 1,       /* column pattern from column sums (dense lse) */
    SDATTN_SEL_BLOCKS_EXACT = 2   /* block pattern from the exact block mass
                                     (dense lse; sdattn_select_blocks_exact)  */
} sdattn_sel_kind;

typedef enum {
    SDATTN_ACT_DENSE = 0,         /* dense attention                          */
    SDATTN_ACT_DENSE_SELECT = 1,  /* dense attention, then a new pattern      */
    SDATTN_ACT_SELECT_SPARSE = 2, /* new pattern from this step, then sparse  */
    SDATTN_ACT_SPARSE = 3,        /* sparse attention with the cached pattern */
    SDATTN_ACT_PROBE_SPARSE = 4   /* probe selection, adopt it if the pattern
                                     moved, then sparse attention            */
} sdattn_action;

/*
 * Schedule (SparseD, abstract: full attention early, pattern computed once
 * and reused; Step-dLLM, Abstract: refresh at anchor steps; PulseCol,
 * Abstract: refresh at a few intermediate steps).  Selection steps
 *   S = {select_step} u {select_step + m*refresh_interval, m >= 1}
 *       u refresh_steps[0..n_refresh_steps-1], all < total_steps.
 * Step t in S is DENSE_SELECT if t < dense_steps or (refresh_dense and
 * t > select_step), else SELECT_SPARSE.  Step t not in S is DENSE if
 * t < dense_steps, else SPARSE.  Requires select_step <= dense_steps.
 * Columns (sel = SDATTN_SEL_COLUMNS) and exact block mass
 * (SDATTN_SEL_BLOCKS_EXACT) need refresh_dense = 1 and select_step <
 * dense_steps, because their scores use the dense pass's lse; kcol = max(1,
 * ceil(column_keep_frac * L - 1e-9)).  A new pattern applies from the step that
 * builds it (SELECT_SPARSE) or from the next step (DENSE_SELECT).
 *
 * Adaptive anchors (blocks only; Step-dLLM, Abstract: attention patterns
 * hold only locally across steps and change abruptly at some transitions,
 * so the mask is refreshed at anchor steps).  With probe_interval = s > 0, a
 * step t not in S with t >= dense_steps, t > select_step and
 * (t - select_step) mod s == 0 is PROBE_SPARSE: the pooled selector runs on
 * the step's Q/K into the idle pattern buffer, the overlap
 * J = |A n B| / |A u B| of the cached pattern A and the probe B is taken
 * over (row, block) pairs (J = 1 when both are empty), and if
 * J < min_overlap the probe replaces the cached pattern before the sparse
 * attention of that step; otherwise the cached pattern stays.  The decision
 * is made on the GPU (no host synchronisation); see
 * sdattn_schedule_probe_stats.  0 <= min_overlap <= 1 (0: never adopt,
 * 1: adopt whenever the patterns differ).
 */
typedef struct {
    int32_t total_steps;
    int32_t dense_steps;
    int32_t select_step;
    int32_t refresh_interval;       /* 0 = none */
    const int32_t* refresh_steps;   /* host array, copied at create; may be NULL */
    int32_t n_refresh_steps;
    int32_t refresh_dense;
    sdattn_sel_kind sel;
    int32_t block_q, block_k;       /* blocks (pooled or exact) only */
    sdattn_budget budget;           /* blocks (pooled or exact) only */
    double column_keep_frac;        /* columns only */
    int32_t probe_interval;         /* 0 = no probes; blocks only (ABI 2) */
    double min_overlap;             /* adoption threshold of a probe (ABI 2) */
    int32_t split_rows;             /* blocks only: 1 = sparse steps run over a split plan
                                       (sdattn_forward_block_sparse_split: rows far longer
                                       than the rest are cut and merged), 0 = over the
                                       dispatch plan alone (ABI 6) */
} sdattn_schedule_desc;

typedef struct sdattn_schedule sdattn_schedule; /* opaque */

/* Validates, copies the descriptor and allocates the pattern buffers and
 * workspace on the current device.  *out = NULL on error. */
SDATTN_API sdattn_status sdattn_schedule_create(const sdattn_problem* p, const sdattn_schedule_desc* desc,
                                     sdattn_schedule** out);

/* Action of step `step` (0 <= step < total_steps).  Pure host. */
SDATTN_API sdattn_status sdattn_schedule_action(const sdattn_schedule* s, int32_t step, sdattn_action* out);

/*
 * Runs denoising step `step`: enqueues the step's kernels on `stream`.
 * o required; lse optional (the handle keeps its own buffer when NULL).
 * Steps may be run in any order, but a SPARSE or PROBE_SPARSE step fails
 * with SDATTN_ERR_STATE if no pattern has been built yet; a failed step
 * leaves the cached pattern and step counters unchanged (one exception: a
 * PROBE_SPARSE step whose last launch, the attention, fails after the
 * adoption kernel was enqueued may have replaced the pattern; all its
 * arguments are checked before anything is enqueued, so only a HIP launch
 * failure can do that).
 */
SDATTN_API sdattn_status sdattn_schedule_step(sdattn_schedule* s, int32_t step, const void* q,
                                   const void* k, const void* v, void* o, float* lse,
                                   void* stream);

/* Graph capture.  A step enqueues kernels only (no memset, copy, allocation
 * or host wait), so steps may be captured into a HIP graph and replayed with
 * new contents in the same buffers.  A captured step binds the pattern
 * buffer in use at capture time: capture again after a selection or refresh
 * step, which switches buffers.  A probe's adoption copies into the buffer in
 * use, so captured steps stay valid across probes. */

/* Borrowed device pointers of the cached pattern (valid until destroy):
 * blocks -> CSR row_ptr and col_idx; columns -> row_ptr = NULL and col_idx
 * [B][Hkv][kcol].  *nnz_capacity = int32 slots of col_idx.  Fails with
 * SDATTN_ERR_STATE before the first selection. */
SDATTN_API sdattn_status sdattn_schedule_mask(const sdattn_schedule* s, const int32_t** row_ptr,
                                   const int32_t** col_idx, int64_t* nnz_capacity);

/* Counters: number of steps run by action (4 entries, indexed by
 * sdattn_action; PROBE_SPARSE steps are counted by
 * sdattn_schedule_probe_stats) and the step of the last selection or
 * adopted probe known to the host (-1 if none; adoption is decided on the
 * GPU, so probes are not reflected here). */
SDATTN_API sdattn_status sdattn_schedule_stats(const sdattn_schedule* s, int64_t counts[4],
                                    int32_t* last_select_step);

/* Probe counters: probe steps run, probes adopted, and the overlap J of
 * the last probe (1.0 if none).  Waits for `stream` (the stream the steps
 * were enqueued on; NULL = default stream), then reads the counters from
 * device memory: a synchronous call. */
SDATTN_API sdattn_status sdattn_schedule_probe_stats(const sdattn_schedule* s, int64_t* n_probes,
                                          int64_t* n_adopted, double* last_overlap, void* stream);

/* Frees the handle and its device buffers (NULL is a no-op).  The caller
 * must make sure no enqueued step still uses them (synchronise first). */
SDATTN_API void sdattn_schedule_destroy(sdattn_schedule* s);

/* ===================================================================== */
/* Block-wise diffusion over a cached prefix: LoSA-style partial          */
/* attention (LoSA: Locality Aware Sparse Attention for block-wise        */
/* diffusion language models, section 3, core principles and workflow).   */
/* ===================================================================== */

/* A block of block_len tokens is denoised on top of a prefix of
 * prefix_len tokens whose keys and values are cached.  Layouts (contiguous,
 * bf16 unless stated):
 *   q, q_prev, o      [B][Hq][block_len][d]   (the block's queries, outputs)
 *   k_cache, v_cache  [B][Hkv][prefix_len][d] (the prefix cache)
 *   k_blk, v_blk      [B][Hkv][block_len][d]  (the block's own keys, values)
 *   lse               [B][Hq][block_len] fp32, natural log
 *   kp                [B][Hkv][prefix_len/page][d] fp32 page means of k_cache
 * Every query attends, without a causal mask, to the prefix and to all keys
 * of its block; query head h reads kv head h / (Hq/Hkv).
 * Constraints: dtype SDATTN_BF16 (SDATTN_F32 -> SDATTN_ERR_UNSUPPORTED),
 * head_dim 64 or 128, block_len <= 64, page divides prefix_len,
 * prefix_len/page <= 4096, 1 <= n_active <= block_len (else
 * SDATTN_ERR_BUDGET), 1 <= pages_per_query <= prefix_len/page (else
 * SDATTN_ERR_BUDGET).  softmax_scale <= 0 means 1/sqrt(head_dim).  Launch
 * grids bound batch <= 65535 and kv_heads <= 65535, and every launch of a
 * call must fit 2^32 work-items per grid dimension: the top-k launch takes
 * 256 work-items per (batch, query head, Active token) row, so
 * batch * q_heads * n_active < 2^24, and the merge takes 64 per (batch,
 * query head, block token) row (else SDATTN_ERR_SHAPE, before anything is
 * enqueued).
 * Calls that share a workspace must be ordered on one stream. */
typedef struct {
    int32_t batch, q_heads, kv_heads, prefix_len, block_len, head_dim;
    sdattn_dtype dtype;
    float softmax_scale;
    int32_t page;            /* prefix tokens per page (the selection unit) */
    int32_t n_active;        /* Active tokens per later iteration */
    int32_t pages_per_query; /* pages kept per Active query and head */
} sdattn_losa_problem;

/* Workspace bytes for sdattn_losa_dense and sdattn_losa_step (the larger of
 * the two) and the capacity of one kv head's page union,
 * min(prefix_len/page, (Hq/Hkv) * n_active * pages_per_query). */
SDATTN_API sdattn_status sdattn_losa_workspace(const sdattn_losa_problem* p, size_t* ws_bytes,
                                               int32_t* max_union_pages);

/* kp[b][g][P] = mean of k_cache[b][g][P*page .. P*page+page-1] (fp32).  The
 * selector's page keys (section 3, the sparse selector run for the Active
 * tokens; a per-page mean key stands in for the unnamed selector's page
 * summary).  Run once per prefix: it does not change while a block is
 * denoised. */
SDATTN_API sdattn_status sdattn_losa_pool_pages(const sdattn_losa_problem* p, const void* k_cache, float* kp,
                                                void* stream);

/* The first iteration of a block (section 3, workflow: initialisation):
 * every block query attends to the whole prefix and the whole block; writes
 * all of o and lse, which later iterations keep for Stable tokens. */
SDATTN_API sdattn_status sdattn_losa_dense(const sdattn_losa_problem* p, const void* q, const void* k_cache,
                                           const void* v_cache, const void* k_blk, const void* v_blk, void* o,
                                           float* lse, void* ws, size_t ws_bytes, void* stream);

/* A later iteration (section 2, locality of representation changes;
 * section 3, workflow steps 1-5):
 *   1. locality[b][i] = mean over heads and channels of (q - q_prev)^2 (fp64);
 *   2. active_idx[b][0..n_active) = the n_active largest, ties to the lower
 *      index, listed ascending;
 *   3. page_scores[b][h][a][P] = scale * <q[b][h][active_idx[b][a]], kp[b][g][P]>
 *      (fp32), and each (b, h, a) row keeps its pages_per_query best pages
 *      (score descending, page ascending);
 *   4. union_pages[b][g][0..union_count[b][g]) = the ascending union of the
 *      pages kept by the query heads of kv head g over all Active tokens
 *      (capacity max_union_pages per kv head);
 *   5. each Active query row attends to the prefix tokens of its kv head's
 *      union and to the block's keys; o and lse rows of Active tokens are
 *      overwritten, the rows of Stable tokens are left as they are
 *      (section 3, reuse for Stable tokens).
 * q_prev is the previous iteration's q.  locality and page_scores are
 * optional outputs (NULL: not written; page_scores otherwise lives in the
 * workspace).  All enqueued on `stream`; no host synchronisation.  Errors:
 * SDATTN_ERR_NULL for a missing required pointer, SDATTN_ERR_WORKSPACE for
 * a workspace below sdattn_losa_workspace, the problem errors above. */
SDATTN_API sdattn_status sdattn_losa_step(const sdattn_losa_problem* p, const void* q, const void* q_prev,
                                          const void* k_cache, const void* v_cache, const float* kp,
                                          const void* k_blk, const void* v_blk, void* o, float* lse,
                                          int32_t* active_idx, int32_t* union_pages, int32_t* union_count,
                                          double* locality, float* page_scores, void* ws, size_t ws_bytes,
                                          void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SDATTN_H */
