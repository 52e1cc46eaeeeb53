// Pooled-score block selection without any allocation: the entry point for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).  It computes what
// sdattn_select_blocks computes, with the same kernels, but its workspace is
// a file-scope device array of SDATTN_NOALLOC_SCRATCH_BYTES instead of a
// caller's buffer.
//
// Each GPU the library runs on holds its own copy of the array until the
// process ends.  In host code the array's name is only a host-side stand-in
// for the symbol: the device address is resolved once per device with
// hipGetSymbolAddress (that device current) and kept, and only that address
// is passed to kernels.  Every call on one GPU uses the same array, which
// keeps the last call's contents; the selection kernels initialise every
// part of it they read, so nothing needs clearing between calls.  Calls that
// overlap on one GPU (different streams, or threads without ordering) race
// on the array.

#include <hip/hip_runtime.h>
#include <stdio.h>

#include <mutex>

#include "host_common.h"
#include "select_api.h"

using namespace sdattn;

namespace {

static __device__ __align__(256) char scratch[SDATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, resolved once

sdattn_status hip_error(hipError_t e, const char* what) {
    char buf[200];
    snprintf(buf, sizeof buf, "sdattn_select_blocks_noalloc: %s: %s", what, hipGetErrorString(e));
    return fail(SDATTN_ERR_HIP, buf);
}

// Device address of this device's copy of `scratch`.
sdattn_status scratch_on(int dev, void** out) {
    if (dev < 0 || dev >= kMaxDevices) return fail(SDATTN_ERR_UNSUPPORTED, "device ordinal beyond 64");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return hip_error(e, "hipGetDevice");
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_error(e, "hipSetDevice");
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess && r != hipSuccess) e = r;
        }
        if (e != hipSuccess) return hip_error(e, "hipGetSymbolAddress");
        if (ptr == nullptr) return fail(SDATTN_ERR_HIP, "sdattn_select_blocks_noalloc: scratch has no device address");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return SDATTN_OK;
}

}  // namespace

extern "C" {

sdattn_status sdattn_select_blocks_noalloc(const sdattn_problem* p, const void* q, const void* k, int32_t block_q,
                                           int32_t block_k, const sdattn_budget* budget, int32_t* row_ptr,
                                           int32_t* col_idx, int64_t col_capacity, float* block_mass, void* stream) {
    SelectBlocksPlan sp;
    sdattn_status s = plan_select_blocks(p, q, k, block_q, block_k, budget, row_ptr, col_idx, col_capacity, &sp);
    if (s != SDATTN_OK || sp.pr.L == 0) return s;
    if (sp.ws_bytes > SDATTN_NOALLOC_SCRATCH_BYTES) {
        char buf[200];
        snprintf(buf, sizeof buf,
                 "this selection needs %zu bytes of workspace; the static scratch holds %zu "
                 "(use sdattn_select_blocks with a caller workspace)",
                 sp.ws_bytes, static_cast<size_t>(SDATTN_NOALLOC_SCRATCH_BYTES));
        return fail(SDATTN_ERR_WORKSPACE, buf);
    }
    // the device the work runs on: the stream's, or the current one for the NULL stream
    int dev = 0;
    hipError_t e = stream != nullptr ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return hip_error(e, "device of the stream");
    void* ws = nullptr;
    s = scratch_on(dev, &ws);
    if (s != SDATTN_OK) return s;
    return launch_planned_select_blocks(sp, q, k, budget, row_ptr, col_idx, block_mass, ws, stream,
                                        "sdattn_select_blocks_noalloc");
}

}  // extern "C"
