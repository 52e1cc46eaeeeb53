// Internal host launchers of the pattern overlap and of the probe adoption
// (adaptive anchors of the schedule driver).  The C ABI in api.hip validates
// the arguments first.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdattn {

// Pattern overlap: counts[0] = |A n B| over (row, block) pairs, counts[1] =
// |A|, counts[2] = |B| (overwritten).
hipError_t launch_mask_overlap(int rows, const int32_t* rpa, const int32_t* cia, const int32_t* rpb,
                               const int32_t* cib, int64_t* counts, hipStream_t st);

// Device-resident record of a schedule's probes.
struct ProbeState {
    int64_t probes, adopted, last_inter, last_union;
};

// Adopt the probe (src) over the cached pattern (dst) when the overlap in
// `counts` is below min_overlap, and record the probe in `state`.  max_copy:
// the largest possible number of pattern entries.
hipError_t launch_probe_adopt(int rows, int32_t* rp_dst, int32_t* ci_dst, const int32_t* rp_src,
                              const int32_t* ci_src, const int64_t* counts, ProbeState* state, double min_overlap,
                              int64_t max_copy, hipStream_t st);

// Zeroes a probe record.
hipError_t launch_probe_init(ProbeState* state, hipStream_t st);

}  // namespace sdattn
