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
    int32_t* split = nullptr;             // MODE_BLOCK: a split plan's workspace (launch_split_plan) instead of `order`
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

// Split plan of the block-sparse forward.  Rows with more kept blocks than
// one workgroup slot's share of the launch (T = max(kSplitMinBlocks,
// ceil(nnz / slots)), slots = the workgroups the GPU holds at once) are cut
// into c = min(8, ceil(ne / T)) chunks of consecutive kept blocks; every
// chunk is a workgroup of the forward that writes a partial result (O
// normalised over its chunk, fp32, and its log-sum-exp), and a merge kernel
// combines a row's chunks by their log-sum-exps.  One workspace holds it
// all, in int32 units from its start:
//   items      [rows + 2 slots]  workgroup id -> item: -1 (idle) or
//                                row | chunk << 24 | (c - 1) << 27
//   slot_base  [rows]            first partial slot of a split row (-1: not cut)
//   counts     [2]               split rows S, chunk length T
//   split_rows [slots]           the S split rows (item encoding, chunk 0)
//   plan       [rows]            the dispatch plan the items are built from
// then, from the next 256-byte boundary, 2 slots partial slots of
// block_q * (D + 1) floats each (O in the MFMA accumulator layout, then the
// log-sum-exps).  Items: every chunk of the split rows first, chunk k of row
// r at its partial slot slot_base[r] + k (consecutive ids: the chunks of a
// row go to different XCDs), idle entries up to a multiple of 8, then the
// dispatch plan with the split rows idle (so each remaining entry keeps its
// XCD), then idle entries.  Needs rows < 2^24.
constexpr int kSplitCUs = 256;        // MI355X compute units
constexpr int kSplitMinBlocks = 4;    // rows of at most this many kept blocks stay whole
constexpr int kSplitRowBits = 24;
constexpr int kSplitChunkShift = 24;  // 3 bits
constexpr int kSplitCountShift = 27;  // 3 bits: chunks - 1
constexpr int kSplitMaxChunks = 8;
inline int split_slots(int block_q) { return kSplitCUs * block_rows_per_cu(block_q); }
__host__ __device__ inline size_t split_items(int rows, int slots) { return static_cast<size_t>(rows) + 2 * slots; }
__host__ __device__ inline size_t split_slot_base_offset(int rows, int slots) { return split_items(rows, slots); }
__host__ __device__ inline size_t split_counts_offset(int rows, int slots) { return split_items(rows, slots) + rows; }
__host__ __device__ inline size_t split_rows_offset(int rows, int slots) { return split_counts_offset(rows, slots) + 2; }
__host__ __device__ inline size_t split_plan_offset(int rows, int slots) { return split_rows_offset(rows, slots) + slots; }
__host__ __device__ inline size_t split_partial_offset(int rows, int slots) {
    return (split_plan_offset(rows, slots) + rows + 63) / 64 * 64;  // int32 units, 256-byte aligned
}
inline size_t split_ws_bytes(int rows, int block_q, int D) {
    const int slots = split_slots(block_q);
    return split_partial_offset(rows, slots) * 4 + 2 * static_cast<size_t>(slots) * block_q * (D + 1) * 4;
}
hipError_t launch_split_plan(int rows, int nqt, int block_q, const int32_t* row_ptr, int32_t* ws, hipStream_t st);

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
