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


// ---- LDS and buffer-to-LDS DMA helpers ----------------------------------

// Raw buffer descriptor word 3 for gfx9-family parts: 32-bit data format,
// offsets checked against num_records (loads past it return zero).
constexpr int kRsrcWord3 = 0x00020000;

// A buffer offset at or beyond every valid one (tile past the end): the
// range check returns zeros.  Valid offsets stay below it while L * 2d bytes
// fit in kOOB.
constexpr uint32_t kOOB = 0xFFFF0000u;

typedef short s16x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

// 8-byte transposing LDS read: in each group of 16 lanes, lane 4s+e receives
// element e of the 8-byte chunks addressed by lanes s, s+4, s+8, s+12.
__device__ __forceinline__ s16x4 lds_read_tr(const char* base, int off) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (LDS_AS s16x4*)((LDS_AS char*)(base) + off));
}

// 32-bit LDS address of a shared-memory pointer, as a wave-uniform value
__device__ __forceinline__ uint32_t lds_addr(LDS_AS char* ptr) {
    return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ptr)));
}

// Raw buffer descriptor for `bytes` bytes at `base` (gfx9 layout: base
// address, stride 0, record count, kRsrcWord3).  The values are uniform; each
// dword is passed through readfirstlane so that the descriptor is an SGPR
// quad wherever the compiler keeps it, as the DMA below requires.
__device__ __forceinline__ u32x4 buffer_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    u32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
    r[1] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32) & 0xFFFFu);
    r[2] = __builtin_amdgcn_readfirstlane(bytes);
    r[3] = kRsrcWord3;
    return r;
}

// 16-byte buffer load of every lane into LDS at lds + 16 * lane (the
// buffer-to-LDS DMA; offsets at or past the range read as zero).  Issued
// through asm because the compiler, unable to tell which stage a DMA writes,
// would otherwise wait for it before every later LDS read; the kernel orders
// DMA and LDS reads itself (memory-count wait and barrier once per tile).
__device__ __forceinline__ void dma_load16(u32x4 rsrc, uint32_t lds, uint32_t voffset) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds), "v"(voffset), "s"(rsrc));
}

// s_waitcnt until at most N vector-memory operations of this wave are
// outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and
// lgkmcnt left at their maxima, i.e. not waited on).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | (((N >> 4) & 0x3) << 14));
}

}  // namespace sdattn
