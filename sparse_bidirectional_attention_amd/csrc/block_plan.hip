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

// Split plan (layout in launch.h), one 1024-thread workgroup after the
// dispatch plan has been written into the workspace.  Each thread takes a
// contiguous range of rows; an exclusive scan over the threads of (split
// rows, partial slots) gives every split row its entry in the split-row list
// and its c consecutive partial slots, in row order; chunk k of the row is
// the workgroup at its slot, so the items' chunk section is the slot list.
constexpr int kSplitThreads = 1024;
constexpr int kPackBits = 24;  // per-field totals stay below 2 slots <= 2^12

__global__ __launch_bounds__(kSplitThreads) void split_plan_kernel(const int32_t* __restrict__ row_ptr, int rows,
                                                                 int slots, int32_t* __restrict__ ws) {
    __shared__ unsigned long long scan[kSplitThreads];
    const int tid = threadIdx.x;
    const long long nnz = static_cast<long long>(row_ptr[rows]) - row_ptr[0];
    const long long tl = max(static_cast<long long>(kSplitMinBlocks), (nnz + slots - 1) / slots);
    const int T = static_cast<int>(min(tl, static_cast<long long>(INT32_MAX)));
    auto chunks = [&](int r) -> int {
        const long long ne = static_cast<long long>(row_ptr[r + 1]) - row_ptr[r];
        if (ne <= T) return 1;
        return static_cast<int>(min(static_cast<long long>(kSplitMaxChunks), (ne + T - 1) / T));
    };
    constexpr unsigned long long kMask = (1ull << kPackBits) - 1;
    const int per = (rows + kSplitThreads - 1) / kSplitThreads;
    const int r0 = min(rows, tid * per), r1 = min(rows, r0 + per);
    unsigned long long n = 0, sl = 0;
    for (int r = r0; r < r1; ++r) {
        const int c = chunks(r);
        if (c > 1) {
            n += 1;
            sl += c;
        }
    }
    const unsigned long long mine = n | (sl << kPackBits);
    scan[tid] = mine;
    __syncthreads();
    for (int off = 1; off < kSplitThreads; off <<= 1) {  // inclusive scan (the packed fields never carry)
        const unsigned long long add = tid >= off ? scan[tid - off] : 0ull;
        __syncthreads();
        scan[tid] += add;
        __syncthreads();
    }
    const unsigned long long total = scan[kSplitThreads - 1];
    const unsigned long long ex = scan[tid] - mine;
    int pn = static_cast<int>(ex & kMask), ps = static_cast<int>((ex >> kPackBits) & kMask);
    int32_t* slot_base = ws + split_slot_base_offset(rows, slots);
    int32_t* split_rows = ws + split_rows_offset(rows, slots);
    for (int r = r0; r < r1; ++r) {
        const int c = chunks(r);
        if (c > 1) {
            const int head = r | ((c - 1) << kSplitCountShift);
            slot_base[r] = ps;
            split_rows[pn] = head;
            for (int k = 0; k < c; ++k) ws[ps + k] = head | (k << kSplitChunkShift);
            pn += 1;
            ps += c;
        } else {
            slot_base[r] = -1;
        }
    }
    const int CS = static_cast<int>((total >> kPackBits) & kMask);  // chunks of the split rows (< 2 slots)
    const int C8 = (CS + 7) & ~7;  // the plan part starts on a multiple of 8: each entry keeps its XCD
    for (int i = CS + tid; i < C8; i += kSplitThreads) ws[i] = -1;
    const int32_t* plan = ws + split_plan_offset(rows, slots);
    for (int i = tid; i < rows; i += kSplitThreads) {
        const int r = plan[i];
        ws[C8 + i] = chunks(r) > 1 ? -1 : r;
    }
    const int items = static_cast<int>(split_items(rows, slots));
    for (int i = C8 + rows + tid; i < items; i += kSplitThreads) ws[i] = -1;
    if (tid == 0) {
        int32_t* counts = ws + split_counts_offset(rows, slots);
        counts[0] = static_cast<int>(total & kMask);
        counts[1] = T;
    }
}

}  // namespace

int block_plan_segment_rows(int block_q, int nqt) {
    // block rows one XCD runs at once (32 CUs, times the forward's workgroups
    // per CU for this block size), lowered to the largest divisor of nqt
    const int in_flight = 32 * block_rows_per_cu(block_q);
    int s = nqt;
    if (nqt > in_flight) {
        s = in_flight;
        while (s > 1 && nqt % s != 0) --s;
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

hipError_t launch_split_plan(int rows, int nqt, int block_q, const int32_t* row_ptr, int32_t* ws, hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    const int slots = split_slots(block_q);
    hipError_t e = launch_block_plan(rows, nqt, block_q, row_ptr, ws + split_plan_offset(rows, slots), st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(split_plan_kernel, dim3(1), dim3(kSplitThreads), 0, st, row_ptr, rows, slots, ws);
    return hipGetLastError();
}

}  // namespace sdattn
