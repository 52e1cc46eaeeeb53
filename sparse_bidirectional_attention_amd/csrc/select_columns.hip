// Column-pattern selection from column-summed attention on gfx950
// (PulseCol, Abstract: key columns selected from column-level attention at
// an early step, shared by the queries).
//
//   colsum kernels  partial[b, h, j] = sum_i exp(scale q_i.k_j - lse_i) over
//                   all query rows of one query head h: bf16 inputs use
//                   v_mfma_f32_32x32x16_bf16 for S^T = K Q^T with the 32-key
//                   K operand kept in registers and Q streamed through
//                   registers; exponentials in fp32, accumulated per lane
//                   in fp32 over 16 query tiles, then in fp64.  fp32 inputs
//                   use exact fp32 FMAs and expf with fp64 accumulation.
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

// bf16: 4 waves x 32 keys = 128 keys per workgroup; all L queries of one head.
template <int D>
__global__ __launch_bounds__(256) void colsum_bf16_kernel(ColParams p) {
    constexpr int DK = D / 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l32 = lane & 31, hl = lane >> 5;
    const int kt = blockIdx.x % p.n_ktiles;
    const int bh = blockIdx.x / p.n_ktiles;
    const int h = bh % p.Hq, b = bh / p.Hq;
    const int g = h / p.group;
    const int L = p.L;
    const int key0 = kt * 128 + wave * 32;
    const uint16_t* kh = static_cast<const uint16_t*>(p.k) + (static_cast<size_t>(b) * p.Hkv + g) * L * D;
    const uint16_t* qh = static_cast<const uint16_t*>(p.q) + static_cast<size_t>(bh) * L * D;
    const float* lh = p.lse + static_cast<size_t>(bh) * L;

    bf16x8 kreg[DK];
    {
        const int kr = min(key0 + l32, L - 1);
#pragma unroll
        for (int st = 0; st < DK; ++st)
            kreg[st] = *reinterpret_cast<const bf16x8*>(kh + static_cast<size_t>(kr) * D + 16 * st + 8 * hl);
    }
    double dacc[16];
    float facc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        dacc[r] = 0.0;
        facc[r] = 0.f;
    }
    const int n_qt = (L + 31) / 32;
    for (int qt = 0; qt < n_qt; ++qt) {
        const int qi = qt * 32 + l32;
        const int qr = min(qi, L - 1);
        bf16x8 qb[DK];
#pragma unroll
        for (int st = 0; st < DK; ++st)
            qb[st] = *reinterpret_cast<const bf16x8*>(qh + static_cast<size_t>(qr) * D + 16 * st + 8 * hl);
        const float lsel = qi < L ? lh[qi] * kLog2e : kInf;
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int st = 0; st < DK; ++st) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kreg[st], qb[st], acc, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) facc[r] += exp2_fast(fmaf(acc[r], p.c, -lsel));
        if ((qt & 15) == 15) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                dacc[r] += static_cast<double>(facc[r]);
                facc[r] = 0.f;
            }
        }
    }
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

}  // namespace

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
        cp.n_ktiles = (s.L + 127) / 128;
        const dim3 grid(s.B * s.Hq * cp.n_ktiles);
        if (s.D == 128) hipLaunchKernelGGL(colsum_bf16_kernel<128>, grid, dim3(256), 0, st, cp);
        else hipLaunchKernelGGL(colsum_bf16_kernel<64>, grid, dim3(256), 0, st, cp);
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
