// Internal host launchers of the exact block-mass selector.  The C ABI in
// api.hip validates the arguments first.
#pragma once

#include "launch.h"

namespace sdattn {

// A[b, h, I, J] = mean over the queries i of block I of the sum over the keys
// j of block J of exp(scale q_i.k_j - lse_i), fp32, [B][Hq][nQB][nKB].
hipError_t launch_exact_block_mass(const AttnShape& s, bool bf16, const void* q, const void* k, const float* lse,
                                   int block_q, int block_k, float* mass, hipStream_t st);

// Block selection (top-k, or mass with the global cap) from a given mass
// matrix [B][Hq][nQB][nKB] instead of the pooled scores; the workspace is
// laid out by select_blocks_ws_layout (its pooling buffers go unused).
hipError_t launch_select_blocks_from_mass(const AttnShape& s, const float* mass_in, int block_q, int block_k,
                                          bool mass, int topk, float mass_target, long long cap_extra,
                                          int32_t* row_ptr, int32_t* col_idx, float* block_mass, void* ws,
                                          hipStream_t st);

}  // namespace sdattn
