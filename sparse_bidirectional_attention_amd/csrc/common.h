// Device-side helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kInf = __builtin_huge_valf();
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even pack of two floats into two bf16 (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 v = {lo, hi};
    bf16x2 b = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// max(x, x of lane ^ 32) for every lane, through v_permlane32_swap (VALU,
// no LDS crossbar traffic).
__device__ __forceinline__ float max_with_half_swap(float x) {
    uint32_t u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_with_half_swap(float x) {
    uint32_t u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup order that keeps neighbouring work on one XCD.  The hardware
// hands consecutive workgroup ids to the 8 XCDs in turn; within each group
// of `group` ids (a multiple of 8) this remaps id -> logical work item so
// that XCD x receives a contiguous run of group/8 logical items.  Ids past
// the last full group keep their order.
__device__ __forceinline__ int xcd_remap(int id, int total, int group) {
    if (group <= 0 || (group & 7)) return id;
    int full = (total / group) * group;
    if (id >= full) return id;
    int g0 = id - id % group;
    int w = id - g0;
    return g0 + (w & 7) * (group >> 3) + (w >> 3);
}

// Wave-level inclusive prefix sum of an int (64 lanes).
__device__ __forceinline__ int wave_inclusive_scan(int x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// Exclusive prefix sum across a workgroup of NT threads (NT multiple of 64,
// at most 1024).  `scratch` must hold NT/64 + 1 ints.  Returns the
// exclusive prefix; *total receives the workgroup total.  Contains barriers:
// every thread must call it.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int x, int* scratch, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int inc = wave_inclusive_scan(x);
    if (lane == 63) scratch[wave] = inc;
    __syncthreads();
    if (threadIdx.x == 0) {
        int run = 0;
        for (int w = 0; w < NT / 64; ++w) {
            int t = scratch[w];
            scratch[w] = run;
            run += t;
        }
        scratch[NT / 64] = run;
    }
    __syncthreads();
    int res = scratch[wave] + inc - x;
    *total = scratch[NT / 64];
    __syncthreads();
    return res;
}

}  // namespace sdattn
