// Internal host launchers (C++ linkage).  The C ABI in api.hip validates all
// arguments before calling any of these; launchers assume valid input.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sdattn {

// MODE_COLUMN_PACKED: the kept columns' K/V rows are given gathered,
// [B][Hkv][kcol][d], and streamed like contiguous tiles.
enum AttnMode { MODE_DENSE = 0, MODE_BLOCK = 1, MODE_COLUMN = 2, MODE_COLUMN_PACKED = 3 };

struct AttnShape {
    int B, Hq, Hkv, L, D;
    float scale;  // softmax scale (already resolved, > 0)
};

struct SparseIndex {
    int block_q = 128, block_k = 128;     // MODE_BLOCK
    const int32_t* row_ptr = nullptr;     // MODE_BLOCK
    const int32_t* col_idx = nullptr;     // MODE_BLOCK (CSR) / MODE_COLUMN ([B][Hkv][kcol])
    int kcol = 0;                         // MODE_COLUMN, MODE_COLUMN_PACKED
    const int32_t* order = nullptr;       // MODE_BLOCK: dispatch plan (launch_block_plan), or computed in the kernel
};

// Flash-style forward; bf16 inputs (MFMA) or f32 inputs (VALU).
hipError_t launch_flash_bf16(AttnMode mode, const AttnShape& s, const void* q, const void* k,
                             const void* v, void* o, float* lse, const SparseIndex& ix,
                             hipStream_t st);
hipError_t launch_flash_f32(AttnMode mode, const AttnShape& s, const void* q, const void* k,
                            const void* v, void* o, float* lse, const SparseIndex& ix,
                            hipStream_t st);

// Workgroups of the bf16 block-sparse forward per CU for this block size.
int block_rows_per_cu(int block_q);
// Dispatch plan of the block-sparse forward: plan[id] = the block row that
// workgroup id computes, a permutation of [0, rows) that gives every XCD an
// equal share of the kept blocks (see block_plan.hip).  rows = B*Hq*nqt.
int block_plan_segment_rows(int block_q, int nqt);
hipError_t launch_block_plan(int rows, int nqt, int block_q, const int32_t* row_ptr, int32_t* plan, hipStream_t st);

// Block selection.  Workspace layout is defined by select_blocks_ws_layout.
struct BlockSelectWs {
    size_t qp_off, kp_off, cum_off, ord_off, cnt_off, hist_off, state_off, total;
};
BlockSelectWs select_blocks_ws_layout(const AttnShape& s, int block_q, int block_k, bool mass);

hipError_t launch_select_blocks(const AttnShape& s, bool bf16, const void* q, const void* k,
                                int block_q, int block_k, bool mass, int topk, float mass_target,
                                long long cap_extra, int32_t* row_ptr, int32_t* col_idx,
                                float* block_mass, void* ws, hipStream_t st);

// Column selection.
size_t select_columns_ws_bytes(const AttnShape& s);
hipError_t launch_select_columns(const AttnShape& s, bool bf16, const void* q, const void* k,
                                 const float* lse, int kcol, int32_t* col_idx, double* col_scores,
                                 void* ws, hipStream_t st);

// kc/vc [B][Hkv][kcol][d] = the rows of k/v listed in col_idx [B][Hkv][kcol]
// (indices clamped to [0, L)); elem_bytes is 2 (bf16) or 4 (fp32).
hipError_t launch_gather_columns(const AttnShape& s, int elem_bytes, const void* k, const void* v,
                                 const int32_t* col_idx, int kcol, void* kc, void* vc, hipStream_t st);

}  // namespace sdattn
