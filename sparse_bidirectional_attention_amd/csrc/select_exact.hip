// Exact block attention mass from the dense pass's log-sum-exp.
//
// The pooled selector scores block pairs by the mean query against the mean
// key.  The other plain reading of a block's "attention mass" (SparseD,
// abstract: head-specific patterns of where the attention goes; Step-dLLM,
// Abstract: heads concentrate their attention mass to different extents) is
// the mass the attention itself puts there:
//
//   A[b, h, I, J] = (1 / |I|) sum_{i in I} sum_{j in J} exp(scale q_i.k_j - lse_i)
//
// i.e. the mean over the queries of block I of the probability they give to
// the keys of block J.  Each row of A sums to 1 over J.  It needs the lse of
// the full attention of the same q, k, so it follows a dense step.
//
// bf16: 8 waves x 32 keys = 256 keys per workgroup with K in registers; all
// queries of the head stream through LDS in 64-query tiles (buffer-to-LDS
// DMA, three stages) with their 64 lse values; S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16, exp2(s c - lse log2 e) in fp32 accumulated per
// lane over the query block's tiles.  At each query block's end a wave sums
// its lanes in registers (its 32 keys x the block's queries); after the next
// barrier wave 0 adds the waves of each key block in a fixed order and
// writes A.
// fp32: one workgroup per query block, one key per thread, exact fp32 FMAs
// and expf.

#include "common.h"
#include "exact.h"

namespace sdattn {
namespace {

struct MassParams {
    const void* q;
    const void* k;
    const float* lse;
    float* mass;  // [B][Hq][nQB][nKB]
    int Hq, Hkv, L, group, n_ktiles, bq, bk, nqb, nkb;
    float c;      // scale * log2(e)
    float scale;
};

constexpr int BM_NW = 8;
constexpr int BM_QT = 64;
constexpr int BM_NST = 3;

// Sum over the 64 lanes of a wave, in every lane, in registers: DPP
// quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror and row_mirror pair each
// lane with one in the other half of its 4, 8 and 16 lanes; v_permlane16_swap
// and v_permlane32_swap then add the other row and the other half-wave.  All
// VALU (no LDS crossbar round trips), and the same value in every lane
// (each step adds the same two values in every pair).
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum_regs(float x) {
    x += dpp_move<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp_move<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp_move<0x141>(x);  // row_half_mirror
    x += dpp_move<0x140>(x);  // row_mirror
    uint32_t u = __float_as_uint(x);
    const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
    u = __float_as_uint(x);
    const auto r32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

template <int D>
__global__ __launch_bounds__(BM_NW * 64) void block_mass_bf16_kernel(MassParams p) {
    constexpr int DK = D / 16;
    constexpr int T = BM_NW * 64;
    constexpr int ROWB = D * 2;
    constexpr int TILEB = BM_QT * ROWB;
    constexpr int UNITS = D / 8;
    constexpr int NDMA = BM_QT * UNITS / T;       // 16-byte DMA chunks per thread per tile (Q)
    constexpr int ROWS_PER_DMA = T / UNITS;
    constexpr int STAGEB = TILEB + BM_QT * 4;      // Q tile, then its log-sum-exp values
    static_assert(NDMA * T == BM_QT * UNITS, "DMA tiling");
    static_assert(BM_QT * 4 == BM_NW * 32, "each wave fetches 8 lse values (two 16-byte lanes)");
    __shared__ __attribute__((aligned(16))) char smem[BM_NST * STAGEB];
    __shared__ float red[2][BM_NW];  // per-wave sums of a query block (by block parity)

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hl = lane >> 5;
    const int kt = blockIdx.x % p.n_ktiles;
    const int bh = blockIdx.x / p.n_ktiles;
    const int h = bh % p.Hq, b = bh / p.Hq;
    const int g = h / p.group;
    const int L = p.L;
    const int key0 = kt * (BM_NW * 32) + wave * 32;
    const uint16_t* kh = static_cast<const uint16_t*>(p.k) + (static_cast<size_t>(b) * p.Hkv + g) * L * D;
    const uint16_t* qh = static_cast<const uint16_t*>(p.q) + static_cast<size_t>(bh) * L * D;
    const float* lh = p.lse + static_cast<size_t>(bh) * L;
    const u32x4 rq = buffer_rsrc(qh, static_cast<uint32_t>(L) * ROWB);
    const u32x4 rl = buffer_rsrc(lh, static_cast<uint32_t>(L) * 4);

    bf16x8 kreg[DK];
    {
        const int kr = min(key0 + l32, L - 1);  // keys past L are masked when summed
#pragma unroll
        for (int st = 0; st < DK; ++st)
            kreg[st] = *reinterpret_cast<const bf16x8*>(kh + static_cast<size_t>(kr) * D + 16 * st + 8 * hl);
    }
    // Q tile in LDS: row r, 16-byte unit u stored at unit u ^ (r mod UNITS)
    const uint32_t smem_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((LDS_AS char*)smem));
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int dr0 = tid / UNITS, dpu = tid % UNITS;
    int qslot[NDMA];
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
        const int row = dr0 + i * ROWS_PER_DMA;
        qslot[i] = row * ROWB + ((dpu ^ (row & (UNITS - 1))) << 4);
    }
    const int n_qt = (L + BM_QT - 1) / BM_QT;
    auto dma_tile = [&](int qt, int stage) __attribute__((always_inline)) {
        const uint32_t base = qt < n_qt ? static_cast<uint32_t>(qt) * TILEB : kOOB;
#pragma unroll
        for (int i = 0; i < NDMA; ++i)
            dma_load16(rq, smem_lds + stage * STAGEB + (i * T + wave_u * 64) * 16, base + qslot[i]);
        const uint32_t lbase = qt < n_qt ? static_cast<uint32_t>(qt) * (BM_QT * 4) : kOOB;
        if (lane < 2) dma_load16(rl, smem_lds + stage * STAGEB + TILEB + wave_u * 32, lbase + wave_u * 32 + lane * 16);
    };
    int qoff[DK];
#pragma unroll
    for (int st = 0; st < DK; ++st) qoff[st] = l32 * ROWB + (((2 * st + hl) ^ (l32 & (UNITS - 1))) << 4);
    // lse (times log2 e) of query row j of the tile in `stage`; +inf past L
    auto lse_at = [&](int stage, int qt, int j) __attribute__((always_inline)) -> float {
        const float x = *reinterpret_cast<const float*>(smem + stage * STAGEB + TILEB + 4 * j);
        return qt * BM_QT + j < L ? x * kLog2e : kInf;
    };

    float facc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) facc[r] = 0.f;
    const int tpb = p.bq / BM_QT;  // Q tiles per query block (1 or 2)
    const int wpb = p.bk / 32;     // waves per key block (2 or 4)
    // this wave's sum over its (real) keys and the finished block's queries;
    // only a wave of the last key tile can hold keys past L
    const bool partial_keys = key0 + 32 > L;
    auto finalize = [&](int I) __attribute__((always_inline)) {
        float x = 0.f;
        if (partial_keys) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = key0 + 8 * (r >> 2) + 4 * hl + (r & 3);
                x += key < L ? facc[r] : 0.f;
                facc[r] = 0.f;
            }
        } else {
            float y[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) y[j] = (facc[4 * j] + facc[4 * j + 1]) + (facc[4 * j + 2] + facc[4 * j + 3]);
            x = (y[0] + y[1]) + (y[2] + y[3]);
#pragma unroll
            for (int r = 0; r < 16; ++r) facc[r] = 0.f;
        }
        x = wave_sum_regs(x);
        if (lane == 0) red[I & 1][wave] = x;
    };
    // after a barrier that follows finalize(I) in every wave
    auto combine = [&](int I) __attribute__((always_inline)) {
        if (wave == 0 && lane < BM_NW / wpb) {
            float s = 0.f;
            for (int w = 0; w < wpb; ++w) s += red[I & 1][lane * wpb + w];
            const int J = kt * (BM_NW * 32) / p.bk + lane;
            const int nI = min(p.bq, L - I * p.bq);
            if (J < p.nkb) p.mass[(static_cast<size_t>(bh) * p.nqb + I) * p.nkb + J] = s / static_cast<float>(nI);
        }
    };
    auto accumulate = [&](const f32x16& a, float l) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) facc[r] += exp2_fast(fmaf(a[r], p.c, -l));
    };
#pragma unroll
    for (int s0 = 0; s0 < BM_NST - 1; ++s0) dma_tile(s0, s0);
    // The exponentials of one 32-query half run beside the MFMAs of the next
    // half; the second half of tile qt is accumulated during tile qt+1, so a
    // query block is finished there.
    // Q operand reads two ahead of the MFMAs, and five VALU instructions of the
    // other half's exponentials between consecutive MFMAs
    auto interleave = [&]() __attribute__((always_inline)) {
        if constexpr (DK == 8) {
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (i < 6) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
            }
        }
    };
    f32x16 a1;
#pragma unroll
    for (int r = 0; r < 16; ++r) a1[r] = 0.f;
    float lb = kInf;   // lse of the pending half (none yet: adds exp2(-inf) = 0)
    int pending = -1;  // finished query block whose waves' sums await combining
    auto tile = [&](int qt, int stage) __attribute__((always_inline)) {
        wait_vmcnt<(BM_NST - 2) * (NDMA + 1)>();
        __syncthreads();
        dma_tile(qt + BM_NST - 1, (stage + BM_NST - 1) % BM_NST);
        const float la = lse_at(stage, qt, l32), lnext = lse_at(stage, qt, 32 + l32);
        if (pending >= 0) {
            combine(pending);
            pending = -1;
        }
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
        interleave();
        __builtin_amdgcn_sched_barrier(0);
        if (qt > 0 && (qt & (tpb - 1)) == 0) {
            finalize(qt / tpb - 1);
            pending = qt / tpb - 1;
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
        interleave();
        __builtin_amdgcn_sched_barrier(0);
    };
    int qt = 0;
    for (; qt + BM_NST <= n_qt; qt += BM_NST) {
#pragma unroll
        for (int s = 0; s < BM_NST; ++s) tile(qt + s, s);
    }
    for (; qt < n_qt; ++qt) tile(qt, qt % BM_NST);
    accumulate(a1, lb);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (pending >= 0) combine(pending);
    finalize(p.nqb - 1);
    __syncthreads();
    combine(p.nqb - 1);
}

// fp32: one workgroup per (b, h, query block), one key per thread
template <int D>
__global__ __launch_bounds__(256) void block_mass_f32_kernel(MassParams p) {
    constexpr int QT = 16;
    __shared__ float qs[QT][D];
    __shared__ float ls[QT];
    __shared__ float part[256];
    const int I = blockIdx.x % p.nqb;
    const int bh = blockIdx.x / p.nqb;
    const int h = bh % p.Hq, b = bh / p.Hq;
    const int g = h / p.group;
    const int L = p.L;
    const int i0 = I * p.bq;
    const int nI = min(p.bq, L - i0);
    const float* kh = static_cast<const float*>(p.k) + (static_cast<size_t>(b) * p.Hkv + g) * L * D;
    const float* qh = static_cast<const float*>(p.q) + static_cast<size_t>(bh) * L * D;
    const float* lh = p.lse + static_cast<size_t>(bh) * L;
    for (int j0 = 0; j0 < L; j0 += 256) {
        const int j = j0 + threadIdx.x;
        float kv[D];
#pragma unroll
        for (int d = 0; d < D; ++d) kv[d] = kh[static_cast<size_t>(min(j, L - 1)) * D + d];
        float acc = 0.f;
        for (int q0 = 0; q0 < nI; q0 += QT) {
            __syncthreads();
            for (int e = threadIdx.x; e < QT * D; e += 256) {
                const int qi = q0 + e / D;
                qs[e / D][e % D] = qi < nI ? qh[static_cast<size_t>(i0 + qi) * D + e % D] : 0.f;
            }
            if (threadIdx.x < QT) ls[threadIdx.x] = q0 + threadIdx.x < nI ? lh[i0 + q0 + threadIdx.x] : kInf;
            __syncthreads();
#pragma unroll
            for (int i = 0; i < QT; ++i) {
                float s = 0.f;
#pragma unroll
                for (int d = 0; d < D; ++d) s = fmaf(qs[i][d], kv[d], s);
                acc += expf(s * p.scale - ls[i]);
            }
        }
        part[threadIdx.x] = j < L ? acc : 0.f;
        __syncthreads();
        if (threadIdx.x < 256 / p.bk) {
            const int J = j0 / p.bk + threadIdx.x;
            if (J < p.nkb) {
                float s = 0.f;
                for (int e = 0; e < p.bk; ++e) s += part[threadIdx.x * p.bk + e];
                p.mass[(static_cast<size_t>(bh) * p.nqb + I) * p.nkb + J] = s / static_cast<float>(nI);
            }
        }
    }
}

}  // namespace

hipError_t launch_exact_block_mass(const AttnShape& s, bool bf16, const void* q, const void* k, const float* lse,
                                   int block_q, int block_k, float* mass, hipStream_t st) {
    if (s.B == 0 || s.L == 0) return hipSuccess;
    MassParams mp{};
    mp.q = q;
    mp.k = k;
    mp.lse = lse;
    mp.mass = mass;
    mp.Hq = s.Hq;
    mp.Hkv = s.Hkv;
    mp.L = s.L;
    mp.group = s.Hq / s.Hkv;
    mp.bq = block_q;
    mp.bk = block_k;
    mp.nqb = (s.L + block_q - 1) / block_q;
    mp.nkb = (s.L + block_k - 1) / block_k;
    mp.scale = s.scale;
    mp.c = s.scale * kLog2e;
    if (bf16) {
        mp.n_ktiles = (s.L + BM_NW * 32 - 1) / (BM_NW * 32);
        const dim3 grid(static_cast<unsigned>(s.B * s.Hq * mp.n_ktiles));
        if (s.D == 128) hipLaunchKernelGGL(block_mass_bf16_kernel<128>, grid, dim3(BM_NW * 64), 0, st, mp);
        else hipLaunchKernelGGL(block_mass_bf16_kernel<64>, grid, dim3(BM_NW * 64), 0, st, mp);
    } else {
        const dim3 grid(static_cast<unsigned>(s.B * s.Hq * mp.nqb));
        if (s.D == 128) hipLaunchKernelGGL(block_mass_f32_kernel<128>, grid, dim3(256), 0, st, mp);
        else hipLaunchKernelGGL(block_mass_f32_kernel<64>, grid, dim3(256), 0, st, mp);
    }
    return hipGetLastError();
}

}  // namespace sdattn
