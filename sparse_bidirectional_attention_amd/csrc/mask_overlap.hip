// Overlap of two block patterns, and the adoption of a probed pattern.
//
// Step-dLLM (Abstract) refreshes the block mask at anchor steps because
// attention patterns hold only locally across denoising steps and change
// abruptly at some transitions.  An adaptive anchor needs to know whether the
// pattern has moved: the pooled selector is rerun on the current step (a
// probe), and its CSR pattern B is compared with the cached pattern A by the
// overlap J = |A n B| / |A u B| over (row, block) pairs.  The probe replaces
// the cached pattern when J falls below a threshold.
//
// Both kernels are tiny next to the attention step: the overlap reads the two
// CSR patterns once (one wave per row, each lane looking its entries of A up
// in B's ascending row by binary search; at most 256 workgroups, because the
// workgroups' 64-bit atomics on the one count serialise), and the adoption
// copies B over A only when the decision, taken on the GPU from the counts,
// says so.

#include "probe.h"

namespace sdattn {
namespace {

constexpr int kOvWaves = 16;     // waves per workgroup
constexpr int kOvMaxGroups = 256;  // at most one 64-bit atomic per workgroup on the shared count

__global__ void overlap_zero_kernel(int64_t* counts) {
    if (threadIdx.x < 3) counts[threadIdx.x] = 0;
}

// counts[0] += |A n B| over this workgroup's rows; workgroup 0 also writes
// |A| and |B| from the row pointers.
__global__ __launch_bounds__(kOvWaves * 64) void overlap_kernel(int rows, const int32_t* __restrict__ rpa,
                                                                const int32_t* __restrict__ cia,
                                                                const int32_t* __restrict__ rpb,
                                                                const int32_t* __restrict__ cib, int64_t* counts) {
    __shared__ int part[kOvWaves];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    int hits = 0;
    // one row per wave at a time (each row is a chain of dependent loads),
    // grid-stride over the rows
    for (int64_t r = static_cast<int64_t>(blockIdx.x) * kOvWaves + wave; r < rows;
         r += static_cast<int64_t>(gridDim.x) * kOvWaves) {
        const int a1 = rpa[r + 1], b0 = rpb[r], b1 = rpb[r + 1];
        for (int e = rpa[r] + lane; e < a1; e += 64) {
            const int32_t x = cia[e];
            // first position in [b0, b1) whose block is not below x
            int lo = b0, hi = b1;
            while (lo < hi) {
                const int mid = lo + ((hi - lo) >> 1);
                if (cib[mid] < x)
                    lo = mid + 1;
                else
                    hi = mid;
            }
            hits += (lo < b1 && cib[lo] == x) ? 1 : 0;
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) hits += __shfl_xor(hits, off, 64);
    if (lane == 0) part[wave] = hits;
    __syncthreads();
    if (threadIdx.x == 0) {
        int64_t s = 0;
#pragma unroll
        for (int w = 0; w < kOvWaves; ++w) s += part[w];
        if (s != 0) atomicAdd(reinterpret_cast<unsigned long long*>(counts), static_cast<unsigned long long>(s));
        if (blockIdx.x == 0) {
            counts[1] = static_cast<int64_t>(rpa[rows]) - rpa[0];
            counts[2] = static_cast<int64_t>(rpb[rows]) - rpb[0];
        }
    }
}

// Decision of a probe from the overlap counts: adopt the probe when
// J = |A n B| / |A u B| < min_overlap (J = 1 when both patterns are empty).
// Every thread takes the same decision from the same counts; workgroup 0
// records it in the probe state.  Adopting copies the probe's CSR over the
// cached one.
__global__ __launch_bounds__(256) void probe_adopt_kernel(int rows, int32_t* __restrict__ rp_dst,
                                                          int32_t* __restrict__ ci_dst,
                                                          const int32_t* __restrict__ rp_src,
                                                          const int32_t* __restrict__ ci_src,
                                                          const int64_t* __restrict__ counts, ProbeState* state,
                                                          double min_overlap) {
    const int64_t inter = counts[0], na = counts[1], nb = counts[2];
    const int64_t uni = na + nb - inter;
    const double j = uni > 0 ? static_cast<double>(inter) / static_cast<double>(uni) : 1.0;
    const bool adopt = j < min_overlap;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        state->probes += 1;
        state->adopted += adopt ? 1 : 0;
        state->last_inter = inter;
        state->last_union = uni;
    }
    if (!adopt) return;
    const int64_t n_rp = static_cast<int64_t>(rows) + 1;
    const int64_t c0 = rp_src[0];
    const int64_t n = n_rp > nb ? n_rp : nb;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
        if (i < n_rp) rp_dst[i] = rp_src[i];
        if (i < nb) ci_dst[c0 + i] = ci_src[c0 + i];
    }
}

__global__ void probe_init_kernel(ProbeState* state) {
    if (threadIdx.x == 0) *state = ProbeState{0, 0, 0, 0};
}

}  // namespace

hipError_t launch_mask_overlap(int rows, const int32_t* rpa, const int32_t* cia, const int32_t* rpb,
                               const int32_t* cib, int64_t* counts, hipStream_t st) {
    hipLaunchKernelGGL(overlap_zero_kernel, dim3(1), dim3(64), 0, st, counts);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || rows == 0) return e;
    int64_t grid = (static_cast<int64_t>(rows) + kOvWaves - 1) / kOvWaves;
    if (grid > kOvMaxGroups) grid = kOvMaxGroups;
    hipLaunchKernelGGL(overlap_kernel, dim3(static_cast<unsigned>(grid)), dim3(kOvWaves * 64), 0, st, rows, rpa,
                       cia, rpb, cib, counts);
    return hipGetLastError();
}

hipError_t launch_probe_adopt(int rows, int32_t* rp_dst, int32_t* ci_dst, const int32_t* rp_src,
                              const int32_t* ci_src, const int64_t* counts, ProbeState* state, double min_overlap,
                              int64_t max_copy, hipStream_t st) {
    // enough threads to copy the larger of the row pointers and the
    // largest possible pattern in a few grid-stride passes
    const int64_t n = (static_cast<int64_t>(rows) + 1 > max_copy) ? static_cast<int64_t>(rows) + 1 : max_copy;
    int64_t grid = (n + 255) / 256;
    if (grid > 1024) grid = 1024;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(probe_adopt_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, st, rows, rp_dst, ci_dst,
                       rp_src, ci_src, counts, state, min_overlap);
    return hipGetLastError();
}

hipError_t launch_probe_init(ProbeState* state, hipStream_t st) {
    hipLaunchKernelGGL(probe_init_kernel, dim3(1), dim3(64), 0, st, state);
    return hipGetLastError();
}

}  // namespace sdattn
