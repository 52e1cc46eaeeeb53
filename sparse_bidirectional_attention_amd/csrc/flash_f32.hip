// Bidirectional attention forward for fp32 inputs (VALU, fp32 throughout).
//
// Same forms as the bf16 kernel (dense / block-sparse / column-sparse, the
// latter also from gathered column rows);
// this path exists for fp32 problems, whose results must agree with fp64 to
// ~1e-5, so it uses exact fp32 FMAs and the accurate expf instead of MFMA.
// One query row per thread, BQ queries per workgroup; 32-key K/V tiles are
// staged in LDS and read as broadcasts.  Exact (non-lazy) online softmax.

#include "common.h"
#include "launch.h"

namespace sdattn {
namespace {

struct F32Params {
    const float* q;
    const float* k;
    const float* v;
    float* o;
    float* lse;
    const int32_t* row_ptr;
    const int32_t* col_idx;
    int Hq, Hkv, L, group, n_qtiles, n_items, block_k, kcol;
    float scale;
};

template <int D, int BQ, int MODE>
__global__ __launch_bounds__(BQ) void flash_fwd_f32(F32Params p) {
    constexpr int KT = 32;
    __shared__ float Ks[KT][D];
    __shared__ float Vs[KT][D];

    const int tid = threadIdx.x;
    const int item = blockIdx.x;
    const int qt = item % p.n_qtiles;
    const int bh = item / p.n_qtiles;
    const int h = bh % p.Hq;
    const int b = bh / p.Hq;
    const int g = h / p.group;
    const int L = p.L;
    const size_t kvoff = (static_cast<size_t>(b) * p.Hkv + g) * (MODE == MODE_COLUMN_PACKED ? p.kcol : L) * D;
    const float* kh = p.k + kvoff;
    const float* vh = p.v + kvoff;
    const int qi = qt * BQ + tid;
    const size_t obase = (static_cast<size_t>(b) * p.Hq + h) * L;

    int n_tiles = 0, e0 = 0, sub = 1;
    const int32_t* cb = nullptr;
    if constexpr (MODE == MODE_DENSE) {
        n_tiles = (L + KT - 1) / KT;
    } else if constexpr (MODE == MODE_BLOCK) {
        const int r = bh * p.n_qtiles + qt;
        e0 = p.row_ptr[r];
        sub = p.block_k / KT;
        n_tiles = (p.row_ptr[r + 1] - e0) * sub;
    } else {
        if constexpr (MODE == MODE_COLUMN) cb = p.col_idx + (static_cast<size_t>(b) * p.Hkv + g) * p.kcol;
        n_tiles = (p.kcol + KT - 1) / KT;
    }

    float qv[D], ov[D];
    {
        const float* qp = p.q + (obase + min(qi, L - 1)) * D;
#pragma unroll
        for (int d = 0; d < D; ++d) {
            qv[d] = qp[d];
            ov[d] = 0.f;
        }
    }
    float m = -kInf, l = 0.f;

    for (int t = 0; t < n_tiles; ++t) {
        int base, nvalid;
        if constexpr (MODE == MODE_COLUMN || MODE == MODE_COLUMN_PACKED) {
            base = t * KT;
            nvalid = min(KT, p.kcol - base);
        } else {
            if constexpr (MODE == MODE_DENSE) {
                base = t * KT;
            } else {
                base = p.col_idx[e0 + t / sub] * p.block_k + (t % sub) * KT;
            }
            nvalid = max(0, min(KT, L - base));
        }
        __syncthreads();
        for (int e = tid; e < KT * D; e += BQ) {
            const int r = e / D, d = e % D;
            int row;
            if constexpr (MODE == MODE_COLUMN) row = min(max(cb[base + min(r, nvalid - 1)], 0), L - 1);
            else if constexpr (MODE == MODE_COLUMN_PACKED) row = base + min(r, nvalid - 1);
            else row = min(max(base + r, 0), L - 1);
            Ks[r][d] = kh[static_cast<size_t>(row) * D + d];
            Vs[r][d] = vh[static_cast<size_t>(row) * D + d];
        }
        __syncthreads();
        float s[KT];
        float mt = -kInf;
#pragma unroll
        for (int j = 0; j < KT; ++j) {
            float acc = 0.f;
#pragma unroll
            for (int d = 0; d < D; ++d) acc = fmaf(qv[d], Ks[j][d], acc);
            s[j] = j < nvalid ? acc * p.scale : -kInf;
            mt = fmaxf(mt, s[j]);
        }
        const float mn = fmaxf(m, mt);
        if (mn == -kInf) continue;
        const float alpha = expf(m - mn);
        l *= alpha;
#pragma unroll
        for (int d = 0; d < D; ++d) ov[d] *= alpha;
#pragma unroll
        for (int j = 0; j < KT; ++j) {
            const float pj = expf(s[j] - mn);
            l += pj;
#pragma unroll
            for (int d = 0; d < D; ++d) ov[d] = fmaf(pj, Vs[j][d], ov[d]);
        }
        m = mn;
    }
    if (qi < L) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        float* op = p.o + (obase + qi) * D;
#pragma unroll
        for (int d = 0; d < D; ++d) op[d] = ov[d] * inv;
        if (p.lse != nullptr) p.lse[obase + qi] = l > 0.f ? m + logf(l) : -kInf;
    }
}

template <int D, int BQ>
hipError_t launch_mode(AttnMode mode, const F32Params& fp, hipStream_t st) {
    dim3 grid(fp.n_items), block(BQ);
    switch (mode) {
        case MODE_DENSE: hipLaunchKernelGGL((flash_fwd_f32<D, BQ, MODE_DENSE>), grid, block, 0, st, fp); break;
        case MODE_BLOCK: hipLaunchKernelGGL((flash_fwd_f32<D, BQ, MODE_BLOCK>), grid, block, 0, st, fp); break;
        case MODE_COLUMN: hipLaunchKernelGGL((flash_fwd_f32<D, BQ, MODE_COLUMN>), grid, block, 0, st, fp); break;
        case MODE_COLUMN_PACKED:
            hipLaunchKernelGGL((flash_fwd_f32<D, BQ, MODE_COLUMN_PACKED>), grid, block, 0, st, fp);
            break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_flash_f32(AttnMode mode, const AttnShape& s, const void* q, const void* k,
                            const void* v, void* o, float* lse, const SparseIndex& ix,
                            hipStream_t st) {
    const int bq = mode == MODE_BLOCK ? ix.block_q : 64;
    F32Params fp{};
    fp.q = static_cast<const float*>(q);
    fp.k = static_cast<const float*>(k);
    fp.v = static_cast<const float*>(v);
    fp.o = static_cast<float*>(o);
    fp.lse = lse;
    fp.row_ptr = ix.row_ptr;
    fp.col_idx = ix.col_idx;
    fp.Hq = s.Hq;
    fp.Hkv = s.Hkv;
    fp.L = s.L;
    fp.group = s.Hq / s.Hkv;
    fp.n_qtiles = (s.L + bq - 1) / bq;
    fp.n_items = s.B * s.Hq * fp.n_qtiles;
    fp.block_k = ix.block_k;
    fp.kcol = ix.kcol;
    fp.scale = s.scale;
    if (fp.n_items == 0) return hipSuccess;
    if (s.D == 128) return bq == 128 ? launch_mode<128, 128>(mode, fp, st) : launch_mode<128, 64>(mode, fp, st);
    return bq == 128 ? launch_mode<64, 128>(mode, fp, st) : launch_mode<64, 64>(mode, fp, st);
}

}  // namespace sdattn
