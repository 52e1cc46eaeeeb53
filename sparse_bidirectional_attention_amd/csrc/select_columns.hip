// Column-pattern selection from column-summed attention on gfx950
// (PulseCol, Abstract: key columns selected from column-level attention at
// an early step, shared by the queries).
//
//   colsum kernels  partial[b, h, j] = sum_i exp(scale q_i.k_j - lse_i) over
//                   all query rows of one query head h: bf16 inputs use
//                   v_mfma_f32_32x32x16_bf16 for S^T = K Q^T with each
//                   wave's 32-key K operand kept in registers and Q tiles
//                   streamed through LDS for all waves of a workgroup;
//                   exponentials in fp32, accumulated per lane in fp32 over
//                   512 queries, then in fp64.  fp32 inputs use exact fp32
//                   FMAs and expf with fp64 accumulation.
//   reduce kernel   C[b, g, j] = sum over the heads of group g, fp64, in a
//                   fixed order (deterministic, no atomics).
//   topk kernel     per (b, g): the kcol-th largest C by an 8-pass radix
//                   select on the fp64 bit pattern, ties toward the lower
//                   index through an index-ordered scan, ascending output.

#include <algorithm>

#include "common.h"
#include "launch.h"

namespace sdattn {
namespace {

struct ColParams {
    const void* q;
    const void* k;
    const float* lse;
    double* partial;  // [B][Hq][L]
    int Hq, Hkv, L, group, n_ktiles;
    float c;          // scale * log2(e)
    float scale;
};

// bf16: 8 waves x 32 keys = 256 keys per workgroup, K in registers.  All L
// queries of the head stream through LDS in 64-query tiles (buffer-to-LDS
// DMA, CS_NST stages), shared by the 8 waves, together with the tile's 64
// log-sum-exp values (each wave fetches 8 of them), so that every load of the
// loop is a DMA under the loop's own wait; each wave takes S^T = K Q^T for
// its 32 keys and both 32-query halves of a tile.  exp2(s c - lse log2 e) in
// fp32, accumulated per lane in fp32 over 8 tiles (512 queries), then in
// fp64.  Queries past L are given lse = +inf and add zero.
constexpr int CS_NW = 8;
constexpr int CS_QT = 64;
constexpr int CS_NST = 3;

template <int D>
__global__ __launch_bounds__(CS_NW * 64) void colsum_bf16_kernel(ColParams p) {
    constexpr int DK = D / 16;
    constexpr int T = CS_NW * 64;
    constexpr int ROWB = D * 2;
    constexpr int TILEB = CS_QT * ROWB;
    constexpr int UNITS = D / 8;
    constexpr int NDMA = CS_QT * UNITS / T;      // 16-byte DMA chunks per thread per tile (Q)
    constexpr int ROWS_PER_DMA = T / UNITS;
    constexpr int STAGEB = TILEB + CS_QT * 4;     // Q tile, then its log-sum-exp values
    static_assert(NDMA * T == CS_QT * UNITS, "DMA tiling");
    static_assert(CS_QT * 4 == CS_NW * 32, "each wave fetches 8 lse values (two 16-byte lanes)");
    __shared__ __attribute__((aligned(16))) char smem[CS_NST * STAGEB];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hl = lane >> 5;
    const int kt = blockIdx.x % p.n_ktiles;
    const int bh = blockIdx.x / p.n_ktiles;
    const int h = bh % p.Hq, b = bh / p.Hq;
    const int g = h / p.group;
    const int L = p.L;
    const int key0 = kt * (CS_NW * 32) + wave * 32;
    const uint16_t* kh = static_cast<const uint16_t*>(p.k) + (static_cast<size_t>(b) * p.Hkv + g) * L * D;
    const uint16_t* qh = static_cast<const uint16_t*>(p.q) + static_cast<size_t>(bh) * L * D;
    const float* lh = p.lse + static_cast<size_t>(bh) * L;
    const u32x4 rq = buffer_rsrc(qh, static_cast<uint32_t>(L) * ROWB);
    const u32x4 rl = buffer_rsrc(lh, static_cast<uint32_t>(L) * 4);

    bf16x8 kreg[DK];
    {
        const int kr = min(key0 + l32, L - 1);
#pragma unroll
        for (int st = 0; st < DK; ++st)
            kreg[st] = *reinterpret_cast<const bf16x8*>(kh + static_cast<size_t>(kr) * D + 16 * st + 8 * hl);
    }
    // Q tile in LDS: row r, 16-byte unit u stored at unit u ^ (r mod UNITS);
    // each DMA lane fetches the chunk that belongs at its slot.
    const uint32_t smem_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((LDS_AS char*)smem));
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int dr0 = tid / UNITS, dpu = tid % UNITS;
    int qslot[NDMA];
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
        const int row = dr0 + i * ROWS_PER_DMA;
        qslot[i] = row * ROWB + ((dpu ^ (row & (UNITS - 1))) << 4);
    }
    const int n_qt = (L + CS_QT - 1) / CS_QT;
    auto dma_tile = [&](int qt, int stage) __attribute__((always_inline)) {
        const uint32_t base = qt < n_qt ? static_cast<uint32_t>(qt) * TILEB : kOOB;
#pragma unroll
        for (int i = 0; i < NDMA; ++i)
            dma_load16(rq, smem_lds + stage * STAGEB + (i * T + wave_u * 64) * 16, base + qslot[i]);
        // lse values 8 w .. 8 w + 7 of the tile (lanes 0 and 1 of wave w);
        // past L they read as zero and are replaced by +inf when read
        const uint32_t lbase = qt < n_qt ? static_cast<uint32_t>(qt) * (CS_QT * 4) : kOOB;
        if (lane < 2) dma_load16(rl, smem_lds + stage * STAGEB + TILEB + wave_u * 32, lbase + wave_u * 32 + lane * 16);
    };
    // B operand (query row l32 of half qb, unit 2 st + hl)
    int qoff[DK];
#pragma unroll
    for (int st = 0; st < DK; ++st) qoff[st] = l32 * ROWB + (((2 * st + hl) ^ (l32 & (UNITS - 1))) << 4);

    double dacc[16];
    float facc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        dacc[r] = 0.0;
        facc[r] = 0.f;
    }
    // lse (times log2 e) of query row j of the tile in `stage`
    auto lse_at = [&](int stage, int qt, int j) __attribute__((always_inline)) -> float {
        const float x = *reinterpret_cast<const float*>(smem + stage * STAGEB + TILEB + 4 * j);
        return qt * CS_QT + j < L ? x * kLog2e : kInf;
    };
#pragma unroll
    for (int s0 = 0; s0 < CS_NST - 1; ++s0) dma_tile(s0, s0);
    // Software pipeline: the exponentials of one 32-query half run beside
    // the MFMAs of the next half (the second half's across the barrier: they
    // touch no LDS).
    f32x16 a1;
#pragma unroll
    for (int r = 0; r < 16; ++r) a1[r] = 0.f;
    float lb = kInf;  // lse of the pending half (none yet: adds exp2(-inf) = 0)
    auto accumulate = [&](const f32x16& a, float l) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) facc[r] += exp2_fast(fmaf(a[r], p.c, -l));
    };
    auto tile = [&](int qt, int stage) __attribute__((always_inline)) {
        wait_vmcnt<(CS_NST - 2) * (NDMA + 1)>();
        __syncthreads();
        dma_tile(qt + CS_NST - 1, (stage + CS_NST - 1) % CS_NST);
        const float la = lse_at(stage, qt, l32), lnext = lse_at(stage, qt, 32 + l32);
        __builtin_amdgcn_sched_barrier(0);
        const char* stg = smem + stage * STAGEB;
        f32x16 a0;
#pragma unroll
        for (int r = 0; r < 16; ++r) a0[r] = 0.f;
#pragma unroll
        for (int st = 0; st < DK; ++st) {
            const bf16x8 q0 = *reinterpret_cast<const bf16x8*>(stg + qoff[st]);
            a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kreg[st], q0, a0, 0, 0, 0);
        }
        accumulate(a1, lb);  // the previous tile's second half
        if constexpr (DK == 8) {
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (i < 6) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < 16; ++r) a1[r] = 0.f;
#pragma unroll
        for (int st = 0; st < DK; ++st) {
            const bf16x8 q1 = *reinterpret_cast<const bf16x8*>(stg + qoff[st] + 32 * ROWB);
            a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kreg[st], q1, a1, 0, 0, 0);
        }
        accumulate(a0, la);
        lb = lnext;
        if constexpr (DK == 8) {
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (i < 6) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if ((qt & 7) == 7) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                dacc[r] += static_cast<double>(facc[r]);
                facc[r] = 0.f;
            }
        }
    };
    int qt = 0;
    for (; qt + CS_NST <= n_qt; qt += CS_NST) {
#pragma unroll
        for (int s = 0; s < CS_NST; ++s) tile(qt + s, s);
    }
    for (; qt < n_qt; ++qt) tile(qt, qt % CS_NST);
    accumulate(a1, lb);
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        double x = dacc[r] + static_cast<double>(facc[r]);
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) x += __shfl_xor(x, off, 64);
        dacc[r] = x;
    }
    if (l32 == 0) {
        double* out = p.partial + static_cast<size_t>(bh) * L;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = key0 + 8 * (r >> 2) + 4 * hl + (r & 3);
            if (key < L) out[key] = dacc[r];
        }
    }
}

// fp32: one key column per thread, 256 keys per workgroup.
template <int D>
__global__ __launch_bounds__(256) void colsum_f32_kernel(ColParams p) {
    constexpr int QT = 16;
    __shared__ float qs[QT][D];
    __shared__ float ls[QT];
    const int kt = blockIdx.x % p.n_ktiles;
    const int bh = blockIdx.x / p.n_ktiles;
    const int h = bh % p.Hq, b = bh / p.Hq;
    const int g = h / p.group;
    const int L = p.L;
    const int j = kt * 256 + threadIdx.x;
    const float* kh = static_cast<const float*>(p.k) + (static_cast<size_t>(b) * p.Hkv + g) * L * D;
    const float* qh = static_cast<const float*>(p.q) + static_cast<size_t>(bh) * L * D;
    const float* lh = p.lse + static_cast<size_t>(bh) * L;
    float kv[D];
#pragma unroll
    for (int d = 0; d < D; ++d) kv[d] = kh[static_cast<size_t>(min(j, L - 1)) * D + d];
    double acc = 0.0;
    for (int q0 = 0; q0 < L; q0 += QT) {
        __syncthreads();
        for (int e = threadIdx.x; e < QT * D; e += 256) {
            const int qi = q0 + e / D;
            qs[e / D][e % D] = qi < L ? qh[static_cast<size_t>(qi) * D + e % D] : 0.f;
        }
        if (threadIdx.x < QT) ls[threadIdx.x] = q0 + threadIdx.x < L ? lh[q0 + threadIdx.x] : kInf;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < QT; ++i) {
            float s = 0.f;
#pragma unroll
            for (int d = 0; d < D; ++d) s = fmaf(qs[i][d], kv[d], s);
            acc += static_cast<double>(expf(s * p.scale - ls[i]));
        }
    }
    if (j < L) p.partial[static_cast<size_t>(bh) * L + j] = acc;
}

__global__ __launch_bounds__(256) void colsum_reduce_kernel(const double* __restrict__ partial, int B, int Hq,
                                                            int Hkv, int L, double* __restrict__ C,
                                                            double* __restrict__ out) {
    const long long n = static_cast<long long>(B) * Hkv * L;
    const int G = Hq / Hkv;
    for (long long i = threadIdx.x + static_cast<long long>(blockIdx.x) * 256; i < n;
         i += static_cast<long long>(gridDim.x) * 256) {
        const long long j = i % L;
        const long long bg = i / L;
        double s = 0.0;
        for (int t = 0; t < G; ++t) s += partial[(bg * G + t) * L + j];
        C[i] = s;
        if (out) out[i] = s;
    }
}

// One workgroup of 1024 threads per (b, g).
__global__ __launch_bounds__(1024) void col_topk_kernel(const double* __restrict__ C, int L, int kcol,
                                                        int32_t* __restrict__ col_idx) {
    constexpr int NT = 1024;
    __shared__ unsigned hist[256];
    __shared__ unsigned long long s_prefix;
    __shared__ int s_rank;
    __shared__ int tmp[NT / 64 + 1];
    const double* c = C + static_cast<size_t>(blockIdx.x) * L;
    int32_t* out = col_idx + static_cast<size_t>(blockIdx.x) * kcol;
    if (threadIdx.x == 0) {
        s_prefix = 0;
        s_rank = kcol - 1;  // 0-based rank in descending order
    }
    for (int pass = 0; pass < 8; ++pass) {
        const int shift = 56 - 8 * pass;
        for (int i = threadIdx.x; i < 256; i += NT) hist[i] = 0;
        __syncthreads();
        const unsigned long long prefix = s_prefix;
        for (int j = threadIdx.x; j < L; j += NT) {
            const unsigned long long u = static_cast<unsigned long long>(__double_as_longlong(c[j]));
            const bool match = pass == 0 || (u >> (shift + 8)) == (prefix >> (shift + 8));
            if (match) atomicAdd(&hist[(u >> shift) & 255], 1u);
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            int rank = s_rank;
            for (int bin = 255; bin >= 0; --bin) {
                if (rank < static_cast<int>(hist[bin])) {
                    s_prefix = prefix | (static_cast<unsigned long long>(bin) << shift);
                    s_rank = rank;
                    break;
                }
                rank -= hist[bin];
            }
        }
        __syncthreads();
    }
    const unsigned long long vstar = s_prefix;
    const int take_eq = s_rank + 1;  // equal values to keep, lowest indices first
    int eq_base = 0, out_base = 0;
    for (int j0 = 0; j0 < L; j0 += NT) {
        const int j = j0 + threadIdx.x;
        unsigned long long u = 0;
        if (j < L) u = static_cast<unsigned long long>(__double_as_longlong(c[j]));
        const int eq = (j < L && u == vstar) ? 1 : 0;
        int eq_tot;
        const int eq_rank = block_exclusive_scan<NT>(eq, tmp, &eq_tot);
        const int keep = (j < L && (u > vstar || (eq && eq_base + eq_rank < take_eq))) ? 1 : 0;
        int k_tot;
        const int pos = block_exclusive_scan<NT>(keep, tmp, &k_tot);
        if (keep && out_base + pos < kcol) out[out_base + pos] = j;
        eq_base += eq_tot;
        out_base += k_tot;
    }
}

// Rows of k and v at the listed columns, packed [B][Hkv][kcol][d]: one
// 16-byte unit per thread and pass (grid-stride), K and V together.  The
// packed rows serve every query tile of the group, so the gather by index
// happens once per step instead of in every workgroup.
__global__ __launch_bounds__(256) void gather_columns_kernel(const char* __restrict__ k, const char* __restrict__ v,
                                                             const int32_t* __restrict__ col_idx, int L, int kcol,
                                                             int units, long long n_units, int row_bytes,
                                                             char* __restrict__ kc, char* __restrict__ vc) {
    for (long long i = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x; i < n_units;
         i += static_cast<long long>(gridDim.x) * 256) {
        const long long row = i / units;  // (b Hkv + g) kcol + j
        const int u = static_cast<int>(i - row * units);
        const long long bg = row / kcol;
        const int col = min(max(col_idx[row], 0), L - 1);
        const size_t src = static_cast<size_t>(bg * L + col) * row_bytes + u * 16;
        const size_t dst = static_cast<size_t>(row) * row_bytes + u * 16;
        *reinterpret_cast<u32x4*>(kc + dst) = *reinterpret_cast<const u32x4*>(k + src);
        *reinterpret_cast<u32x4*>(vc + dst) = *reinterpret_cast<const u32x4*>(v + src);
    }
}

}  // namespace

hipError_t launch_gather_columns(const AttnShape& s, int elem_bytes, const void* k, const void* v,
                                 const int32_t* col_idx, int kcol, void* kc, void* vc, hipStream_t st) {
    const int row_bytes = s.D * elem_bytes;
    const int units = row_bytes / 16;
    const long long n_units = static_cast<long long>(s.B) * s.Hkv * kcol * units;
    if (n_units == 0 || s.L == 0) return hipSuccess;
    const unsigned grid = static_cast<unsigned>(std::min<long long>(4096, (n_units + 255) / 256));
    hipLaunchKernelGGL(gather_columns_kernel, dim3(grid), dim3(256), 0, st, static_cast<const char*>(k),
                       static_cast<const char*>(v), col_idx, s.L, kcol, units, n_units, row_bytes,
                       static_cast<char*>(kc), static_cast<char*>(vc));
    return hipGetLastError();
}

size_t select_columns_ws_bytes(const AttnShape& s) {
    const size_t a = static_cast<size_t>(s.B) * s.Hq * s.L * 8;
    const size_t b = static_cast<size_t>(s.B) * s.Hkv * s.L * 8;
    return ((a + 255) & ~static_cast<size_t>(255)) + ((b + 255) & ~static_cast<size_t>(255));
}

hipError_t launch_select_columns(const AttnShape& s, bool bf16, const void* q, const void* k,
                                 const float* lse, int kcol, int32_t* col_idx, double* col_scores,
                                 void* ws, hipStream_t st) {
    if (s.B == 0 || s.L == 0) return hipSuccess;
    ColParams cp{};
    cp.q = q;
    cp.k = k;
    cp.lse = lse;
    cp.partial = static_cast<double*>(ws);
    cp.Hq = s.Hq;
    cp.Hkv = s.Hkv;
    cp.L = s.L;
    cp.group = s.Hq / s.Hkv;
    cp.scale = s.scale;
    cp.c = s.scale * kLog2e;
    const size_t a = static_cast<size_t>(s.B) * s.Hq * s.L * 8;
    double* Cbuf = reinterpret_cast<double*>(static_cast<char*>(ws) + ((a + 255) & ~static_cast<size_t>(255)));
    if (bf16) {
        cp.n_ktiles = (s.L + CS_NW * 32 - 1) / (CS_NW * 32);
        const dim3 grid(s.B * s.Hq * cp.n_ktiles);
        if (s.D == 128) hipLaunchKernelGGL(colsum_bf16_kernel<128>, grid, dim3(CS_NW * 64), 0, st, cp);
        else hipLaunchKernelGGL(colsum_bf16_kernel<64>, grid, dim3(CS_NW * 64), 0, st, cp);
    } else {
        cp.n_ktiles = (s.L + 255) / 256;
        const dim3 grid(s.B * s.Hq * cp.n_ktiles);
        if (s.D == 128) hipLaunchKernelGGL(colsum_f32_kernel<128>, grid, dim3(256), 0, st, cp);
        else hipLaunchKernelGGL(colsum_f32_kernel<64>, grid, dim3(256), 0, st, cp);
    }
    const long long n = static_cast<long long>(s.B) * s.Hkv * s.L;
    const unsigned rg = static_cast<unsigned>(std::min<long long>(4096, (n + 255) / 256));
    hipLaunchKernelGGL(colsum_reduce_kernel, dim3(rg), dim3(256), 0, st, cp.partial, s.B, s.Hq, s.Hkv, s.L, Cbuf, col_scores);
    hipLaunchKernelGGL(col_topk_kernel, dim3(s.B * s.Hkv), dim3(1024), 0, st, Cbuf, s.L, kcol, col_idx);
    return hipGetLastError();
}

}  // namespace sdattn
