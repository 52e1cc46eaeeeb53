// Dispatch plan of the block-sparse forward.
//
// Under a head-adaptive budget (Step-dLLM, Abstract) the heads keep very
// different numbers of key blocks, so the work of a block row depends on its
// head.  The hardware hands workgroup ids to the eight XCDs in turn (id mod
// 8), the same number to each, and every XCD has its own L2.  The plan maps
// workgroup ids to block rows so that each XCD gets an equal share of the
// kept blocks and, at any moment, works through rows of few heads:
//   * the rows of every (batch, head) pair are cut into segments of S
//     consecutive query blocks, S about the number of rows one XCD runs at
//     once (so an XCD works on one segment, one head's K/V, at a time);
//   * the segments are ranked by their kept blocks (row_ptr differences),
//     most first, and dealt to the XCDs in snake order (ranks 0..7 to XCDs
//     0..7, ranks 8..15 to XCDs 7..0, ...), which evens the XCDs' totals and
//     leaves the lightest segments for the end of the launch;
//   * equal totals keep the plain order (segment s on XCD s mod 8, in round
//     s / 8), so a top-k pattern gets the same dispatch as without the ranking.
// The k-th workgroup of XCD x (id 8k + x) then takes row k mod S of the
// segment dealt to x in round k / S.  Any order gives the same result: each
// row is computed by one workgroup.
//
// One workgroup of 1024 threads sorts the segment keys in LDS (bitonic, at
// most kMaxSegments); shapes whose segments do not fill whole rounds of eight
// get the identity plan.

#include <stdint.h>

#include "common.h"
#include "launch.h"

namespace sdattn {
namespace {

constexpr int kMaxSegments = 8192;
constexpr int kTieBits = 20;  // >= log2(kMaxSegments)

// position of segment s in the snake deal (an involution)
__device__ __forceinline__ int snake_pos(int s) {
    const int j = s >> 3, x = s & 7;
    return 8 * j + ((j & 1) ? 7 - x : x);
}

__global__ __launch_bounds__(1024) void block_plan_kernel(const int32_t* __restrict__ row_ptr, int rows, int nqt,
                                                          int seg_rows, int n_seg, int np2,
                                                          int32_t* __restrict__ plan) {
    __shared__ unsigned long long keys[kMaxSegments];
    const int tid = threadIdx.x;
    if (n_seg == 0) {  // identity plan
        for (int id = tid; id < rows; id += blockDim.x) plan[id] = id;
        return;
    }
    const int parts = nqt / seg_rows;
    // key: (kept blocks + 1) above the tie bits, larger first; ties in the
    // plain order (rank of segment s = its snake position)
    for (int s = tid; s < np2; s += blockDim.x) {
        unsigned long long key = 0;
        if (s < n_seg) {
            const int p = s / parts, j = s - (s / parts) * parts;
            const int r0 = p * nqt + j * seg_rows;
            const long long total = static_cast<long long>(row_ptr[r0 + seg_rows]) - row_ptr[r0];
            const unsigned long long t = static_cast<unsigned long long>(min(max(total, 0LL), (1LL << 40))) + 1;
            key = (t << kTieBits) | static_cast<unsigned long long>(n_seg - 1 - snake_pos(s));
        }
        keys[s] = key;
    }
    __syncthreads();
    // bitonic sort, descending
    for (int k = 2; k <= np2; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = tid; i < np2; i += blockDim.x) {
                const int l = i ^ j;
                if (l > i) {
                    const unsigned long long a = keys[i], b = keys[l];
                    const bool swap = (i & k) == 0 ? a < b : a > b;
                    if (swap) {
                        keys[i] = b;
                        keys[l] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
    // workgroup id -> block row
    constexpr unsigned long long kTieMask = (1ull << kTieBits) - 1;
    for (int id = tid; id < rows; id += blockDim.x) {
        const int x = id & 7, m = id >> 3;
        const int k = m / seg_rows, i = m - (m / seg_rows) * seg_rows;
        const int r = 8 * k + ((k & 1) ? 7 - x : x);  // rank dealt to XCD x in round k
        const int s = snake_pos(n_seg - 1 - static_cast<int>(keys[r] & kTieMask));
        const int p = s / parts, j = s - (s / parts) * parts;
        plan[id] = p * nqt + j * seg_rows + i;
    }
}

}  // namespace

int block_plan_segment_rows(int block_q, int nqt) {
    // block rows one XCD runs at once: 32 CUs, times the forward's workgroups
    // per CU for this block size
    const int in_flight = 32 * block_rows_per_cu(block_q);
    int s = nqt;
    if (nqt > in_flight) {
        s = in_flight;
        while (s > 1 && nqt % s != 0) s >>= 1;
    }
    return s;
}

hipError_t launch_block_plan(int rows, int nqt, int block_q, const int32_t* row_ptr, int32_t* plan, hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    const int seg_rows = block_plan_segment_rows(block_q, nqt);
    int n_seg = rows / seg_rows;
    if (nqt % seg_rows != 0 || n_seg % 8 != 0 || n_seg > kMaxSegments) n_seg = 0;  // identity plan
    int np2 = 1;
    while (np2 < n_seg) np2 <<= 1;
    hipLaunchKernelGGL(block_plan_kernel, dim3(1), dim3(1024), 0, st, row_ptr, rows, nqt, seg_rows, n_seg, np2, plan);
    return hipGetLastError();
}

}  // namespace sdattn
