// Host-side helpers shared by the C ABI (api.hip) and the schedule driver
// (schedule.cpp).  Plain C++: no HIP headers, so the driver and the argument
// checks also build into a CPU-only test library.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>

#include "../../include/sdattn.h"

namespace sdattn {

// Records `msg` as this thread's last error and returns `st`.
sdattn_status fail(sdattn_status st, const std::string& msg);

// Resolved, validated problem.
struct Problem {
    int B, Hq, Hkv, L, D;
    sdattn_dtype dtype;
    float scale;
};

// Checks the problem descriptor (not the tensor pointers).
sdattn_status check_problem(const sdattn_problem* p, Problem* out);

// Top-k count max(1, ceil(frac * n - 1e-9)) clamped to n.
int64_t count_from_fraction(double frac, int64_t n);

// Checks a block budget and the block shape; fills nQB, nKB, rows, topk
// (0 for mass), the worst-case nnz and the mass cap's extra-block allowance
// floor(cap * rows * nKB + 1e-9) - rows.
struct BlockPlan {
    int nqb, nkb;
    int64_t rows, max_nnz, topk, cap_extra;
    bool mass;
};
sdattn_status check_blocks(const Problem& pr, int32_t block_q, int32_t block_k,
                           const sdattn_budget* b, BlockPlan* out);

constexpr int kMaxKeyBlocks = 1024;  // selector limit on nKB (LDS-resident rows)

}  // namespace sdattn
