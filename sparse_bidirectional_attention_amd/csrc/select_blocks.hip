// Block-pattern selection from mean-pooled query/key blocks on gfx950
// (SparseD, abstract: head-specific patterns computed once; Step-dLLM,
// Abstract: uniform or head-adaptive global budget).
//
//   pool_kernel        Qp / Kp = mean of each block's tokens (fp32), one
//                      workgroup per block; reads Q and K once with 16-byte
//                      coalesced loads (HBM-bound).
//   scores_kernel      per group of 8 query blocks of one head: pooled
//                      scores against every key block (each Kp row is read
//                      once per group); then one wave per row: softmax over
//                      J, a bitonic sort on the key (mass desc, J asc) held
//                      in registers (shuffles across lanes), then
//                        top-k: kept flags -> ascending CSR row, or
//                        mass:  the row's cumulative mass array and order.
//   radix select       mass budget with a global cap: the (N+1)-th smallest
//                      cumulative-mass value over all rows (N = extra
//                      blocks the cap allows beyond one per row) in three
//                      digit passes (11/11/10 bits of the fp32 pattern);
//                      tau* = min(mass, that value).
//   count / scan / write  per-row counts 1 + #{c_m < tau*}, exclusive scan
//                      into row_ptr, ascending CSR rows.

#include <algorithm>

#include "common.h"
#include "exact.h"
#include "launch.h"

namespace sdattn {
namespace {

constexpr int kRowsPerGroup = 8;
constexpr int kSelThreads = 256;
constexpr int kMaxKeyBlocks = 1024;
constexpr int kHistBins = 2048;

// One workgroup per (b, head, block): mean over the block's tokens.
template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ x, float* __restrict__ out,
                                                   int L, int block, int nb) {
    constexpr int VEC = 16 / sizeof(T);
    constexpr int UNITS = D / VEC;
    constexpr int RG = 256 / UNITS;  // row groups
    __shared__ float part[RG][D];
    const int item = blockIdx.x;
    const int I = item % nb;
    const size_t bh = item / nb;
    const int r0 = I * block;
    const int n = min(block, L - r0);
    const int u = threadIdx.x % UNITS, rg = threadIdx.x / UNITS;
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
    const T* base = x + (bh * L + r0) * D;
    for (int r = rg; r < n; r += RG) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(base + static_cast<size_t>(r) * D + u * VEC);
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t w = raw[e >> 1];
                acc[e] += __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += __uint_as_float(raw[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) part[rg][u * VEC + e] = acc[e];
    __syncthreads();
    if (threadIdx.x < D) {
        float s = 0.f;
        for (int j = 0; j < RG; ++j) s += part[j][threadIdx.x];
        out[(bh * nb + I) * D + threadIdx.x] = s / static_cast<float>(n);
    }
}

struct ScoreParams {
    const float* qp;   // [B][Hq][nQB][D]
    const float* kp;   // [B][Hkv][nKB][D]
    int Hq, Hkv, group, nqb, nkb, n2;  // n2 = next power of two >= nkb
    float scale;
    int topk;          // > 0: top-k selection; 0: mass (write cum/ord)
    int32_t* row_ptr;
    int32_t* col_idx;
    float* block_mass;  // nullable
    float* cum;         // [rows][nkb] (mass)
    int32_t* ord;       // [rows][nkb] (mass)
    const float* mass_in;  // nullable: the rows' mass, given (no pooled scores, no softmax)
};

// 64-bit shuffle (two 32-bit halves)
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int m) {
    const uint32_t lo = __shfl_xor(static_cast<uint32_t>(x), m, 64);
    const uint32_t hi = __shfl_xor(static_cast<uint32_t>(x >> 32), m, 64);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ float wave_inclusive_scan_f(float x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    return x;
}

// R: sort keys per lane (the row's 64 R >= nKB sort slots; element i = 64 k + lane)
template <int D, int R>
__global__ __launch_bounds__(kSelThreads) void scores_kernel(ScoreParams p) {
    constexpr int NT = kSelThreads;
    constexpr int NS = 64 * R;  // sorted length (padding keys are 0, below every real key)
    __shared__ float qs[kRowsPerGroup][D];
    __shared__ float sc[kRowsPerGroup][kMaxKeyBlocks];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int groups_per_head = (p.nqb + kRowsPerGroup - 1) / kRowsPerGroup;
    const int bh = blockIdx.x / groups_per_head;
    const int I0 = (blockIdx.x % groups_per_head) * kRowsPerGroup;
    const int nrows = min(kRowsPerGroup, p.nqb - I0);
    const int h = bh % p.Hq, b = bh / p.Hq;
    const int g = h / p.group;
    const int nkb = p.nkb;

    if (p.mass_in != nullptr) {
        // the rows' mass is given
        for (int e = tid; e < nrows * nkb; e += NT)
            sc[e / nkb][e % nkb] = p.mass_in[(static_cast<size_t>(bh) * p.nqb + I0) * nkb + e];
        __syncthreads();
    } else {
    // pooled scores of the group's rows against every key block (each Kp row read once)
    for (int e = tid; e < nrows * D; e += NT) qs[e / D][e % D] = p.qp[(static_cast<size_t>(bh) * p.nqb + I0) * D + e];
    __syncthreads();
    const float* kp = p.kp + (static_cast<size_t>(b) * p.Hkv + g) * nkb * D;
    for (int J = tid; J < nkb; J += NT) {
        float acc[kRowsPerGroup];
#pragma unroll
        for (int r = 0; r < kRowsPerGroup; ++r) acc[r] = 0.f;
        const f32x4* kr = reinterpret_cast<const f32x4*>(kp + static_cast<size_t>(J) * D);
#pragma unroll 4
        for (int d4 = 0; d4 < D / 4; ++d4) {
            const f32x4 kv = kr[d4];
#pragma unroll
            for (int r = 0; r < kRowsPerGroup; ++r) {
                acc[r] = fmaf(qs[r][4 * d4 + 0], kv[0], acc[r]);
                acc[r] = fmaf(qs[r][4 * d4 + 1], kv[1], acc[r]);
                acc[r] = fmaf(qs[r][4 * d4 + 2], kv[2], acc[r]);
                acc[r] = fmaf(qs[r][4 * d4 + 3], kv[3], acc[r]);
            }
        }
#pragma unroll
        for (int r = 0; r < kRowsPerGroup; ++r) sc[r][J] = acc[r] * p.scale;
    }
    __syncthreads();
    }

    // one wave per row from here on: no workgroup barriers
    for (int rr = tid >> 6; rr < nrows; rr += NT / 64) {
        const int row = bh * p.nqb + I0 + rr;
        // softmax over J (pooled scores), or the given mass as it is
        float v[R];
        float inv = 1.f;
        if (p.mass_in != nullptr) {
#pragma unroll
            for (int k = 0; k < R; ++k) {
                const int J = 64 * k + lane;
                v[k] = J < nkb ? sc[rr][J] : 0.f;
            }
        } else {
            float mx = -kInf;
#pragma unroll
            for (int k = 0; k < R; ++k) {
                const int J = 64 * k + lane;
                v[k] = J < nkb ? sc[rr][J] : -kInf;
                mx = fmaxf(mx, v[k]);
            }
            mx = wave_max(mx);
            float sm = 0.f;
#pragma unroll
            for (int k = 0; k < R; ++k) {
                const int J = 64 * k + lane;
                v[k] = J < nkb ? expf(v[k] - mx) : 0.f;
                sm += v[k];
            }
            sm = wave_sum(sm);
            inv = 1.f / sm;
        }
        // key = mass bits << 32 | ~J: descending order is mass desc, then J asc
        uint64_t key[R];
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const int J = 64 * k + lane;
            key[k] = 0;
            if (J < nkb) {
                const float a = v[k] * inv;
                if (p.block_mass) p.block_mass[static_cast<size_t>(row) * nkb + J] = a;
                key[k] = (static_cast<uint64_t>(__float_as_uint(a)) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(J));
            }
        }
        // bitonic sort, descending: at each compare-exchange the lower index of
        // a pair keeps the larger key in descending segments, the smaller in
        // ascending ones
#pragma unroll
        for (int size = 2; size <= NS; size <<= 1) {
#pragma unroll
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                if (stride >= 64) {
                    const int ks = stride >> 6;
#pragma unroll
                    for (int k = 0; k < R; ++k) {
                        const int kq = k ^ ks;
                        if (kq > k) {
                            const bool desc = ((64 * k + lane) & size) == 0;
                            const uint64_t lo = key[k], hi = key[kq];
                            if ((lo < hi) == desc) {
                                key[k] = hi;
                                key[kq] = lo;
                            }
                        }
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < R; ++k) {
                        const uint64_t o = shfl_xor_u64(key[k], stride);
                        const bool lower = (lane & stride) == 0;
                        const bool desc = ((64 * k + lane) & size) == 0;
                        const uint64_t mxk = key[k] > o ? key[k] : o, mnk = key[k] > o ? o : key[k];
                        key[k] = (lower == desc) ? mxk : mnk;
                    }
                }
            }
        }
        if (p.topk > 0) {
            // kept flags in natural order (over the row's score storage), then an
            // ascending compaction by wave scans
            int* flag = reinterpret_cast<int*>(&sc[rr][0]);
#pragma unroll
            for (int k = 0; k < R; ++k) {
                const int J = 64 * k + lane;
                if (J < nkb) flag[J] = 0;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int k = 0; k < R; ++k)
                if (64 * k + lane < p.topk) flag[0xFFFFFFFFu - static_cast<uint32_t>(key[k])] = 1;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            int base = 0;
#pragma unroll
            for (int k = 0; k < R; ++k) {
                const int J = 64 * k + lane;
                const int f = J < nkb ? flag[J] : 0;
                const int inc = wave_inclusive_scan(f);
                if (f) p.col_idx[static_cast<size_t>(row) * p.topk + base + inc - 1] = J;
                base += __shfl(inc, 63, 64);
            }
            if (lane == 0) {
                p.row_ptr[row + 1] = (row + 1) * p.topk;
                if (row == 0) p.row_ptr[0] = 0;
            }
        } else {
            // cumulative mass of the sorted row and its block order
            float carry = 0.f;
#pragma unroll
            for (int k = 0; k < R; ++k) {
                const int m = 64 * k + lane;
                const float a = m < nkb ? __uint_as_float(static_cast<uint32_t>(key[k] >> 32)) : 0.f;
                const float x = wave_inclusive_scan_f(a);
                if (m < nkb) {
                    p.cum[static_cast<size_t>(row) * nkb + m] = carry + x;
                    p.ord[static_cast<size_t>(row) * nkb + m] = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(key[k]));
                }
                carry += __shfl(x, 63, 64);
            }
        }
    }
}

// ---- mass budget with a global cap: radix select of the threshold --------

struct SelState {
    uint32_t prefix;     // selected high bits so far
    uint32_t pad;
    long long rank;      // remaining 0-based rank inside the current prefix
};

__global__ void radix_init_kernel(uint32_t* hist, SelState* st, long long rank) {
    for (int i = threadIdx.x + blockIdx.x * blockDim.x; i < 3 * kHistBins; i += blockDim.x * gridDim.x) hist[i] = 0;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        st->prefix = 0;
        st->rank = rank;
    }
}

__device__ __forceinline__ void pass_bits(int pass, int& shift, int& width) {
    shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    width = pass == 2 ? 10 : 11;
}

__global__ __launch_bounds__(256) void radix_hist_kernel(const float* __restrict__ vals, long long n, int pass,
                                                         uint32_t* __restrict__ hist, const SelState* st) {
    __shared__ uint32_t lh[kHistBins];
    for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) lh[i] = 0;
    __syncthreads();
    int shift, width;
    pass_bits(pass, shift, width);
    const int hi_shift = shift + width;  // bits above this pass's digit are fixed
    const uint32_t prefix = st->prefix;
    const uint32_t bmask = (1u << width) - 1;
    for (long long i = threadIdx.x + static_cast<long long>(blockIdx.x) * blockDim.x; i < n;
         i += static_cast<long long>(blockDim.x) * gridDim.x) {
        const uint32_t u = __float_as_uint(vals[i]);
        if (hi_shift >= 32 || (u >> hi_shift) == (prefix >> hi_shift)) atomicAdd(&lh[(u >> shift) & bmask], 1u);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kHistBins; i += blockDim.x)
        if (lh[i]) atomicAdd(&hist[pass * kHistBins + i], lh[i]);
}

// The bin of this pass's digit that holds the remaining rank: a workgroup
// prefix sum over the histogram (two bins per thread, 64-bit counts); the one
// thread whose bins span the rank appends the digit and keeps the rank left
// inside the bin.  A rank past the total leaves the state unchanged.
__global__ __launch_bounds__(kHistBins / 2) void radix_find_kernel(const uint32_t* hist, int pass, SelState* st) {
    __shared__ long long wsum[kHistBins / 2 / 64];
    int shift, width;
    pass_bits(pass, shift, width);
    const int nb = 1 << width;
    const uint32_t* hh = hist + pass * kHistBins;
    const long long rank = st->rank;  // read by every thread before the one write below
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int b0 = 2 * t;
    const long long h0 = b0 < nb ? hh[b0] : 0;
    const long long h1 = b0 + 1 < nb ? hh[b0 + 1] : 0;
    long long x = h0 + h1;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const long long y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    long long base = 0;
    for (int i = 0; i < w; ++i) base += wsum[i];
    const long long incl = base + x;        // bins 0 .. b0+1
    const long long ex = incl - (h0 + h1);  // bins 0 .. b0-1
    if (rank >= ex && rank < incl) {
        const bool first = rank < ex + h0;
        st->prefix |= static_cast<uint32_t>(first ? b0 : b0 + 1) << shift;
        st->rank = rank - (first ? ex : ex + h0);
    }
}

__global__ __launch_bounds__(256) void mass_count_kernel(const float* __restrict__ cum, int rows, int nkb,
                                                         float mass, int tau_mode, const SelState* st,
                                                         int32_t* __restrict__ cnt) {
    // tau_mode: 0 = radix-selected value capped at mass, 1 = mass, 2 = one block per row
    const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int lane = threadIdx.x & 63;
    if (wave >= rows) return;
    float tau = mass;
    if (tau_mode == 0) tau = fminf(mass, __uint_as_float(st->prefix));
    int c = 0;
    if (tau_mode != 2) {
        for (int m = lane; m < nkb; m += 64) c += cum[static_cast<size_t>(wave) * nkb + m] < tau ? 1 : 0;
        c = wave_sum(c);
    }
    if (lane == 0) cnt[wave] = min(nkb, max(1, c + 1));
}

__global__ __launch_bounds__(1024) void rows_scan_kernel(const int32_t* __restrict__ cnt, int rows,
                                                         int32_t* __restrict__ row_ptr) {
    __shared__ int tmp[1024 / 64 + 1];
    int base = 0;
    for (int r0 = 0; r0 < rows; r0 += 1024) {
        const int r = r0 + threadIdx.x;
        const int x = r < rows ? cnt[r] : 0;
        int tot;
        const int ex = block_exclusive_scan<1024>(x, tmp, &tot);
        if (r < rows) row_ptr[r] = base + ex;
        base += tot;
    }
    if (threadIdx.x == 0) row_ptr[rows] = base;
}

__global__ __launch_bounds__(256) void mass_write_kernel(const int32_t* __restrict__ ord, const int32_t* __restrict__ cnt,
                                                         const int32_t* __restrict__ row_ptr, int nkb,
                                                         int32_t* __restrict__ col_idx) {
    __shared__ int flag[kMaxKeyBlocks];
    __shared__ int tmp[256 / 64 + 1];
    const int row = blockIdx.x;
    const int n = cnt[row];
    for (int J = threadIdx.x; J < nkb; J += 256) flag[J] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += 256) flag[ord[static_cast<size_t>(row) * nkb + i]] = 1;
    __syncthreads();
    int base = row_ptr[row];
    for (int J0 = 0; J0 < nkb; J0 += 256) {
        const int J = J0 + threadIdx.x;
        const int f = J < nkb ? flag[J] : 0;
        int tot;
        const int pos = block_exclusive_scan<256>(f, tmp, &tot);
        if (f) col_idx[base + pos] = J;
        base += tot;
    }
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

template <int R>
void launch_scores(int D, unsigned grid, const ScoreParams& sp, hipStream_t st) {
    if (D == 128) hipLaunchKernelGGL((scores_kernel<128, R>), dim3(grid), dim3(kSelThreads), 0, st, sp);
    else hipLaunchKernelGGL((scores_kernel<64, R>), dim3(grid), dim3(kSelThreads), 0, st, sp);
}

}  // namespace

BlockSelectWs select_blocks_ws_layout(const AttnShape& s, int block_q, int block_k, bool mass) {
    const size_t nqb = (s.L + block_q - 1) / block_q, nkb = (s.L + block_k - 1) / block_k;
    const size_t rows = static_cast<size_t>(s.B) * s.Hq * nqb;
    BlockSelectWs w{};
    size_t off = 0;
    w.qp_off = off; off += align256(rows * s.D * 4);
    w.kp_off = off; off += align256(static_cast<size_t>(s.B) * s.Hkv * nkb * s.D * 4);
    if (mass) {
        w.cum_off = off; off += align256(rows * nkb * 4);
        w.ord_off = off; off += align256(rows * nkb * 4);
        w.cnt_off = off; off += align256(rows * 4);
        w.hist_off = off; off += align256(3 * kHistBins * 4);
        w.state_off = off; off += 256;
    }
    w.total = off;
    return w;
}

namespace {

// Per row: the pooled scores and their softmax, or the given mass; the sort;
// the top-k CSR or the cumulative mass.  Then, for the capped mass budget, the
// global threshold and the CSR.
hipError_t select_stages(const AttnShape& s, const float* qp, const float* kp, const float* mass_in, int block_q,
                         int block_k, bool mass, int topk, float mass_target, long long cap_extra, int32_t* row_ptr,
                         int32_t* col_idx, float* block_mass, void* ws, hipStream_t st) {
    const int nqb = (s.L + block_q - 1) / block_q, nkb = (s.L + block_k - 1) / block_k;
    const long long rows = static_cast<long long>(s.B) * s.Hq * nqb;
    const BlockSelectWs w = select_blocks_ws_layout(s, block_q, block_k, mass);
    char* wsb = static_cast<char*>(ws);
    hipError_t e;
    ScoreParams sp{};
    sp.qp = qp;
    sp.kp = kp;
    sp.mass_in = mass_in;
    sp.Hq = s.Hq;
    sp.Hkv = s.Hkv;
    sp.group = s.Hq / s.Hkv;
    sp.nqb = nqb;
    sp.nkb = nkb;
    int n2 = 1;
    while (n2 < nkb) n2 <<= 1;
    sp.n2 = n2;
    sp.scale = s.scale;
    sp.topk = mass ? 0 : topk;
    sp.row_ptr = row_ptr;
    sp.col_idx = col_idx;
    sp.block_mass = block_mass;
    if (mass) {
        sp.cum = reinterpret_cast<float*>(wsb + w.cum_off);
        sp.ord = reinterpret_cast<int32_t*>(wsb + w.ord_off);
    }
    const int groups = (nqb + kRowsPerGroup - 1) / kRowsPerGroup;
    const unsigned gs = static_cast<unsigned>(s.B * s.Hq * groups);
    const int R = n2 <= 64 ? 1 : n2 / 64;
    switch (R) {
        case 1: launch_scores<1>(s.D, gs, sp, st); break;
        case 2: launch_scores<2>(s.D, gs, sp, st); break;
        case 4: launch_scores<4>(s.D, gs, sp, st); break;
        case 8: launch_scores<8>(s.D, gs, sp, st); break;
        default: launch_scores<16>(s.D, gs, sp, st); break;
    }
    e = hipGetLastError();
    if (e != hipSuccess || !mass) return e;

    // 3. global threshold for the capped mass budget
    uint32_t* hist = reinterpret_cast<uint32_t*>(wsb + w.hist_off);
    SelState* sst = reinterpret_cast<SelState*>(wsb + w.state_off);
    int32_t* cnt = reinterpret_cast<int32_t*>(wsb + w.cnt_off);
    const long long nvals = rows * nkb;
    int tau_mode;
    if (cap_extra < 0) tau_mode = 2;
    else if (cap_extra >= nvals) tau_mode = 1;
    else tau_mode = 0;
    if (tau_mode == 0) {
        hipLaunchKernelGGL(radix_init_kernel, dim3(8), dim3(256), 0, st, hist, sst, cap_extra);
        const unsigned hg = static_cast<unsigned>(std::min<long long>(1024, (nvals + 255) / 256));
        for (int pass = 0; pass < 3; ++pass) {
            hipLaunchKernelGGL(radix_hist_kernel, dim3(hg), dim3(256), 0, st, sp.cum, nvals, pass, hist, sst);
            hipLaunchKernelGGL(radix_find_kernel, dim3(1), dim3(kHistBins / 2), 0, st, hist, pass, sst);
        }
    }
    hipLaunchKernelGGL(mass_count_kernel, dim3(static_cast<unsigned>((rows * 64 + 255) / 256)), dim3(256), 0, st,
                       sp.cum, static_cast<int>(rows), nkb, mass_target, tau_mode, sst, cnt);
    hipLaunchKernelGGL(rows_scan_kernel, dim3(1), dim3(1024), 0, st, cnt, static_cast<int>(rows), row_ptr);
    hipLaunchKernelGGL(mass_write_kernel, dim3(static_cast<unsigned>(rows)), dim3(256), 0, st, sp.ord, cnt, row_ptr, nkb, col_idx);
    return hipGetLastError();
}


}  // namespace

hipError_t launch_select_blocks(const AttnShape& s, bool bf16, const void* q, const void* k,
                                int block_q, int block_k, bool mass, int topk, float mass_target,
                                long long cap_extra, int32_t* row_ptr, int32_t* col_idx,
                                float* block_mass, void* ws, hipStream_t st) {
    const int nqb = (s.L + block_q - 1) / block_q, nkb = (s.L + block_k - 1) / block_k;
    const long long rows = static_cast<long long>(s.B) * s.Hq * nqb;
    if (rows == 0) return hipSuccess;
    const BlockSelectWs w = select_blocks_ws_layout(s, block_q, block_k, mass);
    char* wsb = static_cast<char*>(ws);
    float* qp = reinterpret_cast<float*>(wsb + w.qp_off);
    float* kp = reinterpret_cast<float*>(wsb + w.kp_off);

    // 1. pooling
    const unsigned gq = static_cast<unsigned>(rows), gk = static_cast<unsigned>(s.B * s.Hkv * nkb);
    if (bf16) {
        if (s.D == 128) {
            hipLaunchKernelGGL((pool_kernel<uint16_t, 128>), dim3(gq), dim3(256), 0, st, static_cast<const uint16_t*>(q), qp, s.L, block_q, nqb);
            hipLaunchKernelGGL((pool_kernel<uint16_t, 128>), dim3(gk), dim3(256), 0, st, static_cast<const uint16_t*>(k), kp, s.L, block_k, nkb);
        } else {
            hipLaunchKernelGGL((pool_kernel<uint16_t, 64>), dim3(gq), dim3(256), 0, st, static_cast<const uint16_t*>(q), qp, s.L, block_q, nqb);
            hipLaunchKernelGGL((pool_kernel<uint16_t, 64>), dim3(gk), dim3(256), 0, st, static_cast<const uint16_t*>(k), kp, s.L, block_k, nkb);
        }
    } else {
        if (s.D == 128) {
            hipLaunchKernelGGL((pool_kernel<float, 128>), dim3(gq), dim3(256), 0, st, static_cast<const float*>(q), qp, s.L, block_q, nqb);
            hipLaunchKernelGGL((pool_kernel<float, 128>), dim3(gk), dim3(256), 0, st, static_cast<const float*>(k), kp, s.L, block_k, nkb);
        } else {
            hipLaunchKernelGGL((pool_kernel<float, 64>), dim3(gq), dim3(256), 0, st, static_cast<const float*>(q), qp, s.L, block_q, nqb);
            hipLaunchKernelGGL((pool_kernel<float, 64>), dim3(gk), dim3(256), 0, st, static_cast<const float*>(k), kp, s.L, block_k, nkb);
        }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return select_stages(s, qp, kp, nullptr, block_q, block_k, mass, topk, mass_target, cap_extra, row_ptr, col_idx,
                         block_mass, ws, st);
}

hipError_t launch_select_blocks_from_mass(const AttnShape& s, const float* mass_in, int block_q, int block_k,
                                          bool mass, int topk, float mass_target, long long cap_extra,
                                          int32_t* row_ptr, int32_t* col_idx, float* block_mass, void* ws,
                                          hipStream_t st) {
    const int nqb = (s.L + block_q - 1) / block_q;
    if (static_cast<long long>(s.B) * s.Hq * nqb == 0) return hipSuccess;
    return select_stages(s, nullptr, nullptr, mass_in, block_q, block_k, mass, topk, mass_target, cap_extra, row_ptr,
                         col_idx, block_mass, ws, st);
}

}  // namespace sdattn
