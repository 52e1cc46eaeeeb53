// LoSA-style partial attention for block-wise diffusion LMs (LoSA: Locality
// Aware Sparse Attention for block-wise diffusion language models, section 3,
// core principles and workflow).  A block of Bs tokens is denoised on top of a
// prefix of Lp tokens whose keys and values are cached.  The first iteration
// of a block attends densely; each later iteration
//   1. scores the change of every block token's query since the previous
//      iteration (mean squared difference over all query heads),
//   2. keeps the n_active most-changed tokens Active,
//   3. for each Active query picks its top pages of the prefix by the score of
//      the page's mean key,
//   4. forms, per kv head, the union of those pages (the only prefix K/V read),
//   5. attends Active queries to the union's tokens and to the block's own
//      keys, chunk by chunk, and merges the chunks' partial softmaxes,
//   6. leaves the outputs of Stable tokens as they are.
//
// Kernels, in stream order for one later iteration:
//   losa_locality_kernel     one workgroup per batch row: fp64 locality score
//                            of each block token, the Active list (ascending),
//                            and zeroes that row's page bitmaps;
//   losa_scores_kernel       page scores of every Active query row (fp32 FMA);
//   losa_topk_kernel         one wave per Active query row: top-k pages by
//                            (score desc, page asc), OR-ed into the bitmap;
//   losa_union_kernel        one workgroup per (b, kv head): the ascending page
//                            list of the bitmap and its length;
//   losa_attend_kernel       one workgroup per (key chunk, kv head, 64-row
//                            tile): partial softmax over the chunk's keys;
//                            the last chunk index is the block's own keys;
//   losa_merge_kernel        one wave per query row: log-sum-exp merge of the
//                            partials, bf16 output and fp32 LSE.
// The dense first iteration runs the last two over every prefix token and
// every block query.

#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>

#include <algorithm>
#include <string>

#include "common.h"
#include "host_common.h"

using namespace sdattn;

namespace {

constexpr int kMaxBlockLen = 64;     // block tokens (one per lane of the locality wave)
constexpr int kMaxPages = 4096;      // prefix pages (rows of scores held in registers)
constexpr int kRowTile = 64;         // query rows per attention workgroup
constexpr int kKeyTile = 64;         // keys per LDS tile
constexpr int kChunkSparse = 128;    // keys per attention workgroup, later iterations
constexpr int kChunkDense = 512;     // keys per attention workgroup, first iteration

struct Dims {
    int B, Hq, Hkv, G, Lp, Bs, D, page, n_pages, n_a, kpq;
    float scale;
};

// ---- 0. page means of the cached keys --------------------------------------

template <int D>
__global__ __launch_bounds__(D) void losa_pool_kernel(const uint16_t* __restrict__ kc, float* __restrict__ kp,
                                                      int Lp, int page, int n_pages) {
    const int P = blockIdx.x, g = blockIdx.y, b = blockIdx.z, c = threadIdx.x;
    const int64_t head = static_cast<int64_t>(b) * gridDim.y + g;
    const uint16_t* src = kc + (head * Lp + static_cast<int64_t>(P) * page) * D + c;
    float acc = 0.f;
    for (int r = 0; r < page; ++r) acc += bf16_to_f32(src[static_cast<int64_t>(r) * D]);
    kp[(head * n_pages + P) * D + c] = acc / static_cast<float>(page);
}

// ---- 1. locality scores and the Active list --------------------------------

__global__ __launch_bounds__(256) void losa_locality_kernel(Dims dm, const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ qp,
                                                            int32_t* __restrict__ active, double* locality,
                                                            uint32_t* __restrict__ bitmap, int n_words) {
    __shared__ double delta[kMaxBlockLen];
    const int b = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t* bm = bitmap + static_cast<int64_t>(b) * dm.Hkv * n_words;
    for (int w = threadIdx.x; w < dm.Hkv * n_words; w += 256) bm[w] = 0u;
    const int n = dm.Hq * dm.D;
    for (int i = wave; i < dm.Bs; i += 4) {
        double acc = 0.0;
        for (int e = lane; e < n; e += 64) {
            const int h = e / dm.D, c = e - h * dm.D;
            const int64_t off = ((static_cast<int64_t>(b) * dm.Hq + h) * dm.Bs + i) * dm.D + c;
            const double d = static_cast<double>(bf16_to_f32(q[off])) - static_cast<double>(bf16_to_f32(qp[off]));
            acc = fma(d, d, acc);
        }
        acc = wave_sum(acc);
        if (lane == 0) delta[i] = acc / static_cast<double>(n);
    }
    __syncthreads();
    if (wave != 0) return;
    const bool valid = lane < dm.Bs;
    const double di = valid ? delta[lane] : 0.0;
    int rank = 0;
    for (int j = 0; j < dm.Bs; ++j) {
        const double dj = delta[j];
        rank += (dj > di || (dj == di && j < lane)) ? 1 : 0;
    }
    const bool act = valid && rank < dm.n_a;
    const unsigned long long mask = __ballot(act);
    if (act) active[static_cast<int64_t>(b) * dm.n_a + __popcll(mask & ((1ull << lane) - 1ull))] = lane;
    if (valid && locality != nullptr) locality[static_cast<int64_t>(b) * dm.Bs + lane] = di;
}

// ---- 2. page scores of the Active query rows --------------------------------
// Workgroup (64-page chunk, kv head g, b).  Group row r = (query head
// g*G + r / n_a, Active slot r % n_a).  Each wave scores 4 rows at a time,
// one page per lane.

template <int D>
__global__ __launch_bounds__(256) void losa_scores_kernel(Dims dm, const uint16_t* __restrict__ q,
                                                          const int32_t* __restrict__ active,
                                                          const float* __restrict__ kp, float* __restrict__ scores) {
    __shared__ float ks[64][D + 1];
    __shared__ float qs[16][D];
    const int P0 = blockIdx.x * 64, g = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t kvh = static_cast<int64_t>(b) * dm.Hkv + g;
    for (int idx = threadIdx.x; idx < 64 * D; idx += 256) {
        const int p = idx / D, c = idx - p * D;
        ks[p][c] = P0 + p < dm.n_pages ? kp[(kvh * dm.n_pages + P0 + p) * D + c] : 0.f;
    }
    const int R = dm.G * dm.n_a;
    for (int r0 = 0; r0 < R; r0 += 16) {
        __syncthreads();
        for (int idx = threadIdx.x; idx < 16 * D; idx += 256) {
            const int rr = idx / D, c = idx - rr * D, r = r0 + rr;
            float v = 0.f;
            if (r < R) {
                const int h = g * dm.G + r / dm.n_a, i = active[static_cast<int64_t>(b) * dm.n_a + r % dm.n_a];
                v = bf16_to_f32(q[((static_cast<int64_t>(b) * dm.Hq + h) * dm.Bs + i) * D + c]);
            }
            qs[rr][c] = v;
        }
        __syncthreads();
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
        for (int c = 0; c < D; ++c) {
            const float kv = ks[lane][c];
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = fmaf(qs[wave * 4 + j][c], kv, acc[j]);
        }
        const int P = P0 + lane;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = r0 + wave * 4 + j;
            if (r < R && P < dm.n_pages) {
                const int h = g * dm.G + r / dm.n_a, a = r % dm.n_a;
                scores[((static_cast<int64_t>(b) * dm.Hq + h) * dm.n_a + a) * dm.n_pages + P] = dm.scale * acc[j];
            }
        }
    }
}

// ---- 3. per-row top-k pages into the kv head's bitmap -----------------------
// One wave per (b, h, a) row, NPL scores per lane in registers (page
// lane + 64 j).  Round k takes the best entry ordered after round k-1's pick
// under (score desc, page asc), so nothing is marked or moved.

template <int NPL>
__global__ __launch_bounds__(256) void losa_topk_kernel(Dims dm, const float* __restrict__ scores,
                                                        uint32_t* __restrict__ bitmap, int n_words, int64_t n_rows) {
    const int lane = threadIdx.x & 63;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (row >= n_rows) return;
    const int64_t bh = row / dm.n_a;  // b * Hq + h
    const int b = static_cast<int>(bh / dm.Hq), h = static_cast<int>(bh % dm.Hq);
    const float* sr = scores + row * dm.n_pages;
    float vals[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
        const int P = lane + 64 * j;
        vals[j] = P < dm.n_pages ? sr[P] : 0.f;
    }
    uint32_t* bm = bitmap + (static_cast<int64_t>(b) * dm.Hkv + h / dm.G) * n_words;
    float pv = INFINITY;
    int pp = -1;
    for (int k = 0; k < dm.kpq; ++k) {
        float bv = -INFINITY;
        int bp = INT_MAX;
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
            const int P = lane + 64 * j;
            const float v = vals[j];
            const bool after = v < pv || (v == pv && P > pp);
            const bool better = v > bv || (v == bv && P < bp);
            if (P < dm.n_pages && after && better) {
                bv = v;
                bp = P;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off, 64);
            const int op = __shfl_xor(bp, off, 64);
            if (ov > bv || (ov == bv && op < bp)) {
                bv = ov;
                bp = op;
            }
        }
        if (bp >= dm.n_pages) break;  // no orderable entry left (non-finite scores)
        pv = bv;
        pp = bp;
        if (lane == 0) atomicOr(&bm[bp >> 5], 1u << (bp & 31));
    }
}

// ---- 4. bitmap -> ascending page list ----------------------------------------

__global__ __launch_bounds__(256) void losa_union_kernel(int Hkv, const uint32_t* __restrict__ bitmap, int n_words,
                                                         int32_t* __restrict__ union_pages,
                                                         int32_t* __restrict__ union_count, int cap) {
    __shared__ int scratch[256 / 64 + 1];
    const int g = blockIdx.x, b = blockIdx.y;
    const int64_t kvh = static_cast<int64_t>(b) * Hkv + g;
    const int w = threadIdx.x;  // n_words <= 256
    uint32_t word = w < n_words ? bitmap[kvh * n_words + w] : 0u;
    int total = 0;
    int off = block_exclusive_scan<256>(__popc(word), scratch, &total);
    int32_t* out = union_pages + kvh * cap;
    while (word != 0u) {
        const int bit = __ffs(word) - 1;
        word &= word - 1u;
        out[off++] = w * 32 + bit;
    }
    if (threadIdx.x == 0) union_count[kvh] = total;
}

// ---- 5. partial softmax of a 64-row tile over one key chunk -------------------

struct AttendArgs {
    Dims dm;
    const uint16_t* q;
    const uint16_t* kc;
    const uint16_t* vc;
    const uint16_t* kb;
    const uint16_t* vb;
    const int32_t* active;       // Active list [B][n_a]; unused when dense
    const int32_t* upages;       // union pages [B][Hkv][cap]; unused when dense
    const int32_t* ucount;       // union lengths [B][Hkv]; unused when dense
    float* part;                 // partials [B][Hkv][row_tiles*64][n_chunks+1][D+2]
    int cap, R, row_tiles, chunk, n_chunks, dense;
    float scale_log2;            // scale * log2(e)
};

template <int D>
__global__ __launch_bounds__(256) void losa_attend_kernel(AttendArgs a) {
    constexpr int QW = D / 2 + 4;  // LDS row stride of Q and K tiles in 32-bit words (16-byte aligned, odd bank step)
    constexpr int VU = D / 8;      // 16-byte units per row
    constexpr int DT = D / 16;     // output dims per thread
    __shared__ __align__(16) uint32_t qs[kRowTile * QW];
    __shared__ __align__(16) uint32_t ks[kKeyTile * QW];
    __shared__ __align__(16) uint4 vs[kKeyTile * VU];
    __shared__ float ss[kRowTile][kKeyTile + 1];
    __shared__ float m_s[kRowTile], l_s[kRowTile], al_s[kRowTile];

    const Dims& dm = a.dm;
    const int c = blockIdx.x;
    const int g = blockIdx.y / a.row_tiles, rt = blockIdx.y - g * a.row_tiles, b = blockIdx.z;
    const int64_t kvh = static_cast<int64_t>(b) * dm.Hkv + g;
    const bool suffix = c == a.n_chunks;
    int n_keys;
    if (suffix) {
        n_keys = dm.Bs;
    } else {
        const int total = a.dense ? dm.Lp : a.ucount[kvh] * dm.page;
        n_keys = min(a.chunk, total - c * a.chunk);
        if (n_keys <= 0) return;  // past the union: the merge reads only chunks below its length
    }
    const int r0 = rt * kRowTile;
    const int nrows = min(kRowTile, a.R - r0);
    const int n_a = a.dense ? dm.Bs : dm.n_a;
    const int t = threadIdx.x;

    for (int idx = t; idx < kRowTile * VU; idx += 256) {
        const int rr = idx / VU, u = idx - rr * VU;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (rr < nrows) {
            const int r = r0 + rr;
            const int h = g * dm.G + r / n_a, s = r % n_a;
            const int i = a.dense ? s : a.active[static_cast<int64_t>(b) * dm.n_a + s];
            v = *reinterpret_cast<const uint4*>(a.q + ((static_cast<int64_t>(b) * dm.Hq + h) * dm.Bs + i) * D + u * 8);
        }
        *reinterpret_cast<uint4*>(&qs[rr * QW + u * 4]) = v;
    }
    if (t < kRowTile) {
        m_s[t] = -INFINITY;
        l_s[t] = 0.f;
    }

    const int rb = t >> 4, kb = t & 15;  // scores: rows 4rb..4rb+3, keys kb + 16j; PV: dims kb*DT..
    float o[4][DT];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < DT; ++e) o[i][e] = 0.f;

    for (int k0 = 0; k0 < n_keys; k0 += kKeyTile) {
        const int nk = min(kKeyTile, n_keys - k0);
        for (int idx = t; idx < kKeyTile * VU; idx += 256) {
            const int kk = idx / VU, u = idx - kk * VU;
            uint4 kv = make_uint4(0u, 0u, 0u, 0u), vv = kv;
            if (kk < nk) {
                int64_t row;
                const uint16_t *kbase, *vbase;
                if (suffix) {
                    row = kvh * dm.Bs + k0 + kk;
                    kbase = a.kb;
                    vbase = a.vb;
                } else {
                    const int j = c * a.chunk + k0 + kk;
                    const int pos = a.dense ? j : a.upages[kvh * a.cap + j / dm.page] * dm.page + j % dm.page;
                    row = kvh * dm.Lp + pos;
                    kbase = a.kc;
                    vbase = a.vc;
                }
                kv = *reinterpret_cast<const uint4*>(kbase + row * D + u * 8);
                vv = *reinterpret_cast<const uint4*>(vbase + row * D + u * 8);
            }
            *reinterpret_cast<uint4*>(&ks[kk * QW + u * 4]) = kv;
            vs[kk * VU + u] = vv;
        }
        __syncthreads();

        float acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
        for (int w2 = 0; w2 < D / 2; ++w2) {
            float qlo[4], qhi[4], klo[4], khi[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t x = qs[(rb * 4 + i) * QW + w2];
                qlo[i] = __uint_as_float(x << 16);
                qhi[i] = __uint_as_float(x & 0xFFFF0000u);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t x = ks[(kb + 16 * j) * QW + w2];
                klo[j] = __uint_as_float(x << 16);
                khi[j] = __uint_as_float(x & 0xFFFF0000u);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(qhi[i], khi[j], fmaf(qlo[i], klo[j], acc[i][j]));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                ss[rb * 4 + i][kb + 16 * j] = kb + 16 * j < nk ? acc[i][j] * a.scale_log2 : -INFINITY;
        __syncthreads();

        {  // online softmax: 4 lanes per row, keys part + 4j
            const int row = t >> 2, pt = t & 3;
            float mx = -INFINITY;
#pragma unroll
            for (int j = 0; j < 16; ++j) mx = fmaxf(mx, ss[row][pt + 4 * j]);
            mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
            const float m_old = m_s[row];
            const float m_new = fmaxf(m_old, mx);
            float sum = 0.f;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float p = exp2f(ss[row][pt + 4 * j] - m_new);
                ss[row][pt + 4 * j] = p;
                sum += p;
            }
            sum += __shfl_xor(sum, 1, 64);
            sum += __shfl_xor(sum, 2, 64);
            if (pt == 0) {
                const float alpha = exp2f(m_old - m_new);
                l_s[row] = l_s[row] * alpha + sum;
                m_s[row] = m_new;
                al_s[row] = alpha;
            }
        }
        __syncthreads();

#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float al = al_s[rb * 4 + i];
#pragma unroll
            for (int e = 0; e < DT; ++e) o[i][e] *= al;
        }
        for (int kk = 0; kk < nk; ++kk) {
            float v[DT];
            if constexpr (DT == 8) {
                const uint4 x = vs[kk * VU + kb];
                const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[2 * e] = __uint_as_float(w[e] << 16);
                    v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
                }
            } else {
                const uint2 x = reinterpret_cast<const uint2*>(vs)[kk * (D / 4) + kb];
                const uint32_t w[2] = {x.x, x.y};
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    v[2 * e] = __uint_as_float(w[e] << 16);
                    v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = ss[rb * 4 + i][kk];
#pragma unroll
                for (int e = 0; e < DT; ++e) o[i][e] = fmaf(p, v[e], o[i][e]);
            }
        }
        __syncthreads();
    }

    const int parts = a.n_chunks + 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rr = rb * 4 + i;
        if (rr >= nrows) continue;
        float* dst = a.part + ((kvh * a.row_tiles * kRowTile + r0 + rr) * parts + c) * (D + 2);
#pragma unroll
        for (int e = 0; e < DT; ++e) dst[kb * DT + e] = o[i][e];
        if (kb == 0) {
            dst[D] = m_s[rr];
            dst[D + 1] = l_s[rr];
        }
    }
}

// ---- 6. merge of the partials -------------------------------------------------

struct MergeArgs {
    Dims dm;
    const float* part;
    const int32_t* active;
    const int32_t* ucount;
    uint16_t* o;
    float* lse;
    int R, row_tiles, chunk, n_chunks, dense;
};

template <int D>
__global__ __launch_bounds__(256) void losa_merge_kernel(MergeArgs a) {
    const Dims& dm = a.dm;
    const int lane = threadIdx.x & 63;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const int64_t n_rows = static_cast<int64_t>(dm.B) * dm.Hkv * a.R;
    if (row >= n_rows) return;
    const int64_t kvh = row / a.R;
    const int r = static_cast<int>(row - kvh * a.R);
    const int b = static_cast<int>(kvh / dm.Hkv), g = static_cast<int>(kvh % dm.Hkv);
    const int n_a = a.dense ? dm.Bs : dm.n_a;
    const int h = g * dm.G + r / n_a, s = r % n_a;
    const int i = a.dense ? s : a.active[static_cast<int64_t>(b) * dm.n_a + s];
    const int parts = a.n_chunks + 1;
    const int n_valid = a.dense ? a.n_chunks : (a.ucount[kvh] * dm.page + a.chunk - 1) / a.chunk;
    const float* base = a.part + (kvh * a.row_tiles * kRowTile + r) * static_cast<int64_t>(parts) * (D + 2);

    float M = base[static_cast<int64_t>(a.n_chunks) * (D + 2) + D];  // the block's keys: always present
    for (int c = 0; c < n_valid; ++c) M = fmaxf(M, base[static_cast<int64_t>(c) * (D + 2) + D]);
    constexpr int E = D / 64;
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    float L = 0.f;
    for (int k = 0; k <= n_valid; ++k) {
        const int c = k == n_valid ? a.n_chunks : k;
        const float* p = base + static_cast<int64_t>(c) * (D + 2);
        const float w = exp2f(p[D] - M);
        L = fmaf(p[D + 1], w, L);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = fmaf(p[lane + 64 * e], w, acc[e]);
    }
    const float inv = 1.f / L;
    uint16_t* dst = a.o + ((static_cast<int64_t>(b) * dm.Hq + h) * dm.Bs + i) * D;
#pragma unroll
    for (int e = 0; e < E; ++e) dst[lane + 64 * e] = static_cast<uint16_t>(pack_bf16x2(acc[e] * inv, 0.f) & 0xFFFFu);
    if (lane == 0) a.lse[(static_cast<int64_t>(b) * dm.Hq + h) * dm.Bs + i] = (M + log2f(L)) * 0.6931471805599453f;
}

// ---- host side ------------------------------------------------------------------

struct Plan {
    Dims dm;
    int n_words, cap, npl;
    int R_s, rt_s, nch_s;      // later iterations
    int R_d, rt_d, nch_d;      // first iteration
    size_t off_scores, off_bits, off_part, ws_step, ws_dense;
};

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

sdattn_status check_losa(const sdattn_losa_problem* p, Plan* out) {
    if (p == nullptr) return fail(SDATTN_ERR_NULL, "problem must be non-NULL");
    if (p->batch < 1 || p->q_heads < 1 || p->kv_heads < 1 || p->prefix_len < 1 || p->block_len < 1)
        return fail(SDATTN_ERR_SHAPE, "batch, q_heads, kv_heads, prefix_len and block_len must be >= 1");
    if (p->q_heads % p->kv_heads != 0) return fail(SDATTN_ERR_SHAPE, "q_heads must be a multiple of kv_heads");
    if (p->head_dim != 64 && p->head_dim != 128) return fail(SDATTN_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    if (p->dtype == SDATTN_F32) return fail(SDATTN_ERR_UNSUPPORTED, "the block-wise path takes bf16 tensors only");
    if (p->dtype != SDATTN_BF16) return fail(SDATTN_ERR_DTYPE, "dtype must be SDATTN_BF16");
    if (p->block_len > kMaxBlockLen) return fail(SDATTN_ERR_SHAPE, "block_len must be <= 64");
    if (p->page < 1 || p->prefix_len % p->page != 0)
        return fail(SDATTN_ERR_SHAPE, "page must be >= 1 and divide prefix_len");
    const int n_pages = p->prefix_len / p->page;
    if (n_pages > kMaxPages) return fail(SDATTN_ERR_SHAPE, "prefix_len / page must be <= 4096");
    if (p->n_active < 1 || p->n_active > p->block_len)
        return fail(SDATTN_ERR_BUDGET, "n_active must be in [1, block_len]");
    if (p->pages_per_query < 1 || p->pages_per_query > n_pages)
        return fail(SDATTN_ERR_BUDGET, "pages_per_query must be in [1, prefix_len / page]");
    float scale = p->softmax_scale;
    if (!(scale > 0.f)) scale = 1.f / sqrtf(static_cast<float>(p->head_dim));
    if (!isfinite(scale)) return fail(SDATTN_ERR_SHAPE, "softmax_scale must be finite");
    const int64_t G = p->q_heads / p->kv_heads;
    if (p->batch > 65535 || static_cast<int64_t>(p->kv_heads) * ((G * p->block_len + kRowTile - 1) / kRowTile) > 65535)
        return fail(SDATTN_ERR_SHAPE, "batch and kv_heads * ceil(q_heads/kv_heads * block_len / 64) must be <= 65535");

    Plan pl;
    Dims& dm = pl.dm;
    dm.B = p->batch;
    dm.Hq = p->q_heads;
    dm.Hkv = p->kv_heads;
    dm.G = p->q_heads / p->kv_heads;
    dm.Lp = p->prefix_len;
    dm.Bs = p->block_len;
    dm.D = p->head_dim;
    dm.page = p->page;
    dm.n_pages = n_pages;
    dm.n_a = p->n_active;
    dm.kpq = p->pages_per_query;
    dm.scale = scale;
    pl.n_words = (n_pages + 31) / 32;
    pl.npl = 8;
    while (pl.npl * 64 < n_pages) pl.npl *= 2;
    pl.R_s = dm.G * dm.n_a;
    pl.rt_s = (pl.R_s + kRowTile - 1) / kRowTile;
    pl.cap = static_cast<int>(std::min<int64_t>(n_pages, static_cast<int64_t>(pl.R_s) * dm.kpq));
    pl.nch_s = static_cast<int>((static_cast<int64_t>(pl.cap) * dm.page + kChunkSparse - 1) / kChunkSparse);
    pl.R_d = dm.G * dm.Bs;
    pl.rt_d = (pl.R_d + kRowTile - 1) / kRowTile;
    pl.nch_d = (dm.Lp + kChunkDense - 1) / kChunkDense;
    const size_t part_row = static_cast<size_t>(dm.D + 2) * sizeof(float);
    pl.off_scores = 0;
    pl.off_bits = align256(static_cast<size_t>(dm.B) * dm.Hq * dm.n_a * n_pages * sizeof(float));
    pl.off_part = pl.off_bits + align256(static_cast<size_t>(dm.B) * dm.Hkv * pl.n_words * sizeof(uint32_t));
    pl.ws_step = pl.off_part + static_cast<size_t>(dm.B) * dm.Hkv * pl.rt_s * kRowTile * (pl.nch_s + 1) * part_row;
    pl.ws_dense = static_cast<size_t>(dm.B) * dm.Hkv * pl.rt_d * kRowTile * (pl.nch_d + 1) * part_row;
    *out = pl;
    return SDATTN_OK;
}

sdattn_status hip_status(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e == hipSuccess) return SDATTN_OK;
    return fail(SDATTN_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

template <int D>
void launch_attend_merge(const Plan& pl, bool dense, const void* q, const void* kc, const void* vc, const void* kb,
                         const void* vb, const int32_t* active, const int32_t* upages, const int32_t* ucount,
                         float* part, void* o, float* lse, hipStream_t st) {
    const Dims& dm = pl.dm;
    AttendArgs a;
    a.dm = dm;
    a.q = static_cast<const uint16_t*>(q);
    a.kc = static_cast<const uint16_t*>(kc);
    a.vc = static_cast<const uint16_t*>(vc);
    a.kb = static_cast<const uint16_t*>(kb);
    a.vb = static_cast<const uint16_t*>(vb);
    a.active = active;
    a.upages = upages;
    a.ucount = ucount;
    a.part = part;
    a.cap = pl.cap;
    a.R = dense ? pl.R_d : pl.R_s;
    a.row_tiles = dense ? pl.rt_d : pl.rt_s;
    a.chunk = dense ? kChunkDense : kChunkSparse;
    a.n_chunks = dense ? pl.nch_d : pl.nch_s;
    a.dense = dense ? 1 : 0;
    a.scale_log2 = dm.scale * kLog2e;
    hipLaunchKernelGGL(losa_attend_kernel<D>, dim3(a.n_chunks + 1, dm.Hkv * a.row_tiles, dm.B), dim3(256), 0, st, a);
    MergeArgs m;
    m.dm = dm;
    m.part = part;
    m.active = active;
    m.ucount = ucount;
    m.o = static_cast<uint16_t*>(o);
    m.lse = lse;
    m.R = a.R;
    m.row_tiles = a.row_tiles;
    m.chunk = a.chunk;
    m.n_chunks = a.n_chunks;
    m.dense = a.dense;
    const int64_t rows = static_cast<int64_t>(dm.B) * dm.Hkv * a.R;
    hipLaunchKernelGGL(losa_merge_kernel<D>, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0, st, m);
}

template <int NPL>
void launch_topk(const Plan& pl, const float* scores, uint32_t* bits, hipStream_t st) {
    const int64_t rows = static_cast<int64_t>(pl.dm.B) * pl.dm.Hq * pl.dm.n_a;
    hipLaunchKernelGGL(losa_topk_kernel<NPL>, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0, st, pl.dm,
                       scores, bits, pl.n_words, rows);
}

}  // namespace

extern "C" {

sdattn_status sdattn_losa_workspace(const sdattn_losa_problem* p, size_t* ws_bytes, int32_t* max_union_pages) {
    if (ws_bytes == nullptr || max_union_pages == nullptr)
        return fail(SDATTN_ERR_NULL, "ws_bytes and max_union_pages must be non-NULL");
    Plan pl;
    sdattn_status s = check_losa(p, &pl);
    if (s != SDATTN_OK) return s;
    *ws_bytes = std::max(pl.ws_step, pl.ws_dense);
    *max_union_pages = pl.cap;
    return SDATTN_OK;
}

sdattn_status sdattn_losa_pool_pages(const sdattn_losa_problem* p, const void* k_cache, float* kp, void* stream) {
    Plan pl;
    sdattn_status s = check_losa(p, &pl);
    if (s != SDATTN_OK) return s;
    if (k_cache == nullptr || kp == nullptr) return fail(SDATTN_ERR_NULL, "k_cache and kp must be non-NULL");
    const Dims& dm = pl.dm;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 grid(dm.n_pages, dm.Hkv, dm.B);
    if (dm.D == 128)
        hipLaunchKernelGGL(losa_pool_kernel<128>, grid, dim3(128), 0, st, static_cast<const uint16_t*>(k_cache), kp,
                           dm.Lp, dm.page, dm.n_pages);
    else
        hipLaunchKernelGGL(losa_pool_kernel<64>, grid, dim3(64), 0, st, static_cast<const uint16_t*>(k_cache), kp,
                           dm.Lp, dm.page, dm.n_pages);
    return hip_status("sdattn_losa_pool_pages");
}

sdattn_status sdattn_losa_dense(const sdattn_losa_problem* p, const void* q, const void* k_cache, const void* v_cache,
                                const void* k_blk, const void* v_blk, void* o, float* lse, void* ws, size_t ws_bytes,
                                void* stream) {
    Plan pl;
    sdattn_status s = check_losa(p, &pl);
    if (s != SDATTN_OK) return s;
    if (q == nullptr || k_cache == nullptr || v_cache == nullptr || k_blk == nullptr || v_blk == nullptr ||
        o == nullptr || lse == nullptr)
        return fail(SDATTN_ERR_NULL, "q, k_cache, v_cache, k_blk, v_blk, o and lse must be non-NULL");
    if (ws == nullptr || ws_bytes < pl.ws_dense)
        return fail(SDATTN_ERR_WORKSPACE, "workspace smaller than sdattn_losa_workspace reports");
    hipStream_t st = static_cast<hipStream_t>(stream);
    float* part = static_cast<float*>(ws);
    if (pl.dm.D == 128)
        launch_attend_merge<128>(pl, true, q, k_cache, v_cache, k_blk, v_blk, nullptr, nullptr, nullptr, part, o, lse,
                                 st);
    else
        launch_attend_merge<64>(pl, true, q, k_cache, v_cache, k_blk, v_blk, nullptr, nullptr, nullptr, part, o, lse,
                                st);
    return hip_status("sdattn_losa_dense");
}

sdattn_status sdattn_losa_step(const sdattn_losa_problem* p, const void* q, const void* q_prev, const void* k_cache,
                               const void* v_cache, const float* kp, const void* k_blk, const void* v_blk, void* o,
                               float* lse, int32_t* active_idx, int32_t* union_pages, int32_t* union_count,
                               double* locality, float* page_scores, void* ws, size_t ws_bytes, void* stream) {
    Plan pl;
    sdattn_status s = check_losa(p, &pl);
    if (s != SDATTN_OK) return s;
    if (q == nullptr || q_prev == nullptr || k_cache == nullptr || v_cache == nullptr || kp == nullptr ||
        k_blk == nullptr || v_blk == nullptr || o == nullptr || lse == nullptr || active_idx == nullptr ||
        union_pages == nullptr || union_count == nullptr)
        return fail(SDATTN_ERR_NULL,
                    "q, q_prev, k_cache, v_cache, kp, k_blk, v_blk, o, lse, active_idx, union_pages and union_count "
                    "must be non-NULL");
    if (ws == nullptr || ws_bytes < pl.ws_step)
        return fail(SDATTN_ERR_WORKSPACE, "workspace smaller than sdattn_losa_workspace reports");
    const Dims& dm = pl.dm;
    hipStream_t st = static_cast<hipStream_t>(stream);
    char* w = static_cast<char*>(ws);
    float* scores = page_scores != nullptr ? page_scores : reinterpret_cast<float*>(w + pl.off_scores);
    uint32_t* bits = reinterpret_cast<uint32_t*>(w + pl.off_bits);
    float* part = reinterpret_cast<float*>(w + pl.off_part);
    const uint16_t* q16 = static_cast<const uint16_t*>(q);

    hipLaunchKernelGGL(losa_locality_kernel, dim3(dm.B), dim3(256), 0, st, dm, q16,
                       static_cast<const uint16_t*>(q_prev), active_idx, locality, bits, pl.n_words);
    const dim3 sgrid((dm.n_pages + 63) / 64, dm.Hkv, dm.B);
    if (dm.D == 128)
        hipLaunchKernelGGL(losa_scores_kernel<128>, sgrid, dim3(256), 0, st, dm, q16, active_idx, kp, scores);
    else
        hipLaunchKernelGGL(losa_scores_kernel<64>, sgrid, dim3(256), 0, st, dm, q16, active_idx, kp, scores);
    switch (pl.npl) {
        case 8: launch_topk<8>(pl, scores, bits, st); break;
        case 16: launch_topk<16>(pl, scores, bits, st); break;
        case 32: launch_topk<32>(pl, scores, bits, st); break;
        default: launch_topk<64>(pl, scores, bits, st); break;
    }
    hipLaunchKernelGGL(losa_union_kernel, dim3(dm.Hkv, dm.B), dim3(256), 0, st, dm.Hkv, bits, pl.n_words, union_pages,
                       union_count, pl.cap);
    if (dm.D == 128)
        launch_attend_merge<128>(pl, false, q, k_cache, v_cache, k_blk, v_blk, active_idx, union_pages, union_count,
                                 part, o, lse, st);
    else
        launch_attend_merge<64>(pl, false, q, k_cache, v_cache, k_blk, v_blk, active_idx, union_pages, union_count,
                                part, o, lse, st);
    return hip_status("sdattn_losa_step");
}

}  // extern "C"
