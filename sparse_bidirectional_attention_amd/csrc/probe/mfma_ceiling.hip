// MFMA-only throughput probe for gfx950 (measurement aid, not part of the
// attention path).
//
// Every wave keeps eight bf16 A operands, eight B operands and eight 32x32
// fp32 accumulators in registers and issues v_mfma_f32_32x32x16_bf16 back to
// back, the A/B pair changing at every instruction as in the attention
// kernels' QK^T and PV products, with no memory traffic, no LDS and no VALU
// work in the loop.  Eight independent accumulators, in the accumulation
// registers the compiler picks by default (the build does not force arch
// VGPRs here: nothing but the MFMAs reads them), keep the matrix pipe free of
// dependent-accumulator stalls, so the probe measures the pipe itself.
//
// Under sustained load the chip runs at its package power limit, and what a
// bf16 MFMA costs depends on how many operand bits switch between
// instructions; the probe therefore reports the MFMA ceiling for the operand
// values it is given (random data against all zeros and all ones), at
// whatever clock the power limit allows.  The bench compares the attention
// kernels with it.
//
// Built as its own library (libsdattn_probe.so); one C entry point.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kSets = 8;     // operand pairs per wave
constexpr int kAcc = 8;      // independent accumulators (no back-to-back dependence)

// operands: [grid * 4 waves][kSets][2][64 lanes] of bf16x8 (16 bytes)
__global__ __launch_bounds__(256) void mfma_ceiling_kernel(const bf16x8* __restrict__ operands, int iters,
                                                           float* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
    const bf16x8* src = operands + static_cast<size_t>(wave) * kSets * 2 * 64;
    bf16x8 a[kSets], b[kSets];
#pragma unroll
    for (int s = 0; s < kSets; ++s) {
        a[s] = src[(2 * s) * 64 + lane];
        b[s] = src[(2 * s + 1) * 64 + lane];
    }
    f32x16 acc[kAcc];
#pragma unroll
    for (int c = 0; c < kAcc; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int s = 0; s < kSets; ++s)
            acc[s % kAcc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], b[(s + 3) % kSets], acc[s % kAcc], 0, 0, 0);
    }
    float t = 0.f;
#pragma unroll
    for (int c = 0; c < kAcc; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) t += acc[c][r];
    sink[static_cast<size_t>(wave) * 64 + lane] = t;
}

}  // namespace

extern "C" {

// MFMA instructions one launch issues: grid * 4 waves * iters * 8.
// operands: grid * 4 * 8 * 2 * 64 * 16 bytes of bf16 values (device);
// sink: grid * 4 * 64 floats (device).  Returns a hipError_t value.
__attribute__((visibility("default"))) int sdattn_probe_mfma_ceiling(const void* operands, int grid, int iters,
                                                                    void* sink, void* stream) {
    if (operands == nullptr || sink == nullptr || grid <= 0 || iters <= 0) return static_cast<int>(hipErrorInvalidValue);
    hipLaunchKernelGGL(mfma_ceiling_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const bf16x8*>(operands), iters, static_cast<float*>(sink));
    return static_cast<int>(hipGetLastError());
}

}  // extern "C"
