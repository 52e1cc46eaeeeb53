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
//   * within a segment the rows go longest first, so the rows an XCD starts
//     last, as its slots drain at the end of the launch, are its shortest;
//   * equal totals keep the plain order (segment s on XCD s mod 8, in round
//     s / 8, its rows in order), so a top-k pattern gets the same dispatch as
//     without the ranking.
// The k-th workgroup of XCD x (id 8k + x) then takes position k mod S of the
// segment dealt to x in round k / S.  Any order gives the same result: each
// row is computed by one workgroup.
//
// One workgroup per segment: it ranks its segment against all the others
// (their totals read from row_ptr), sorts its rows in LDS and writes their
// plan entries.  Shapes whose segments do not fill whole rounds of eight get
// the identity plan.

#include <stdint.h>

#include "common.h"
#include "launch.h"

namespace sdattn {
namespace {

constexpr int kMaxSegments = 1 << 20;  // segment indices fit the tie bits
constexpr int kMaxSegRows = 1024;      // rows of one segment, sorted in LDS
constexpr int kTieBits = 20;
constexpr unsigned long long kTieMask = (1ull << kTieBits) - 1;

// position of segment s in the snake deal (an involution)
__device__ __forceinline__ int snake_pos(int s) {
    const int j = s >> 3, x = s & 7;
    return 8 * j + ((j & 1) ? 7 - x : x);
}

__global__ __launch_bounds__(256) void identity_plan_kernel(int rows, int32_t* __restrict__ plan) {
    const int id = blockIdx.x * blockDim.x + threadIdx.x;
    if (id < rows) plan[id] = id;
}

__global__ __launch_bounds__(256) void block_plan_kernel(const int32_t* __restrict__ row_ptr, int nqt, int seg_rows,
                                                         int n_seg, int np2, int32_t* __restrict__ plan) {
    __shared__ unsigned long long keys[kMaxSegRows];
    __shared__ int part[256 / 64];
    const int seg = blockIdx.x;
    const int tid = threadIdx.x;
    const int parts = nqt / seg_rows;
    auto first_row = [&](int t) { return (t / parts) * nqt + (t % parts) * seg_rows; };
    // key of segment t: (kept blocks + 1) above the tie bits, larger first;
    // ties in the plain order (rank of segment t = its snake position)
    auto seg_key = [&](int t) -> unsigned long long {
        const int r0 = first_row(t);
        const long long total = static_cast<long long>(row_ptr[r0 + seg_rows]) - row_ptr[r0];
        const unsigned long long v = static_cast<unsigned long long>(min(max(total, 0LL), (1LL << 40))) + 1;
        return (v << kTieBits) | static_cast<unsigned long long>(n_seg - 1 - snake_pos(t));
    };
    // rank of this segment: the number of segments with a larger key
    const unsigned long long mine = seg_key(seg);
    int c = 0;
    for (int t = tid; t < n_seg; t += blockDim.x) c += seg_key(t) > mine ? 1 : 0;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
    if ((tid & 63) == 0) part[tid >> 6] = c;
    // rows of this segment, most kept blocks first (ties: lower row first)
    const int r0 = first_row(seg);
    for (int i = tid; i < np2; i += blockDim.x) {
        unsigned long long key = 0;
        if (i < seg_rows) {
            const long long ne = static_cast<long long>(row_ptr[r0 + i + 1]) - row_ptr[r0 + i];
            const unsigned long long v = static_cast<unsigned long long>(min(max(ne, 0LL), (1LL << 40))) + 1;
            key = (v << kTieBits) | (kTieMask - static_cast<unsigned long long>(i));
        }
        keys[i] = key;
    }
    __syncthreads();
    const int rank = part[0] + part[1] + part[2] + part[3];
    for (int k = 2; k <= np2; k <<= 1) {  // bitonic sort, descending
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = tid; i < np2; i += blockDim.x) {
                const int l = i ^ j;
                if (l > i) {
                    const unsigned long long a = keys[i], b = keys[l];
                    if ((i & k) == 0 ? a < b : a > b) {
                        keys[i] = b;
                        keys[l] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
    // the segment of rank `rank` goes to XCD x in round rank / 8; position i
    // of it to workgroup 8 (round * S + i) + x
    const int round = rank >> 3, w = rank & 7;
    const int x = (round & 1) ? 7 - w : w;
    for (int i = tid; i < seg_rows; i += blockDim.x) {
        const int row = r0 + static_cast<int>(kTieMask - (keys[i] & kTieMask));
        plan[8 * (round * seg_rows + i) + x] = row;
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
    const int n_seg = rows / seg_rows;
    if (nqt % seg_rows != 0 || n_seg % 8 != 0 || n_seg > kMaxSegments || seg_rows > kMaxSegRows) {
        hipLaunchKernelGGL(identity_plan_kernel, dim3((rows + 255) / 256), dim3(256), 0, st, rows, plan);
        return hipGetLastError();
    }
    int np2 = 1;
    while (np2 < seg_rows) np2 <<= 1;
    hipLaunchKernelGGL(block_plan_kernel, dim3(n_seg), dim3(256), 0, st, row_ptr, nqt, seg_rows, n_seg, np2, plan);
    return hipGetLastError();
}

}  // namespace sdattn
