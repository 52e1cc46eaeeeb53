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
//   losa_delta_kernel        one workgroup per block token: its fp64
//                            locality score;
//   losa_scores_kernel       the Active list (ascending; every workgroup ranks
//                            the block's tokens), page scores of every Active
//                            query row (fp32 FMA), and clears the page bitmaps;
//   losa_topk4_kernel        one workgroup per Active query row (budgets up to
//                            64 pages; losa_topk_kernel, one wave per row,
//                            above): top-k pages by (score desc, page asc),
//                            OR-ed into the bitmap;
//   losa_union_kernel        one workgroup per (b, kv head): the ascending page
//                            list of the bitmap and its length;
//   losa_attend_kernel       one workgroup per (key chunk, kv head, 32- or
//                            64-row tile): partial softmax over the chunk's keys;
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
constexpr int kKeyTile = 64;         // keys per LDS tile
constexpr int kChunkSparse = 128;    // keys per attention workgroup, later iterations
constexpr int kChunkDense = 1024;    // keys per attention workgroup, first iteration

struct Dims {
    int B, Hq, Hkv, G, Lp, Bs, D, page, n_pages, n_a, kpq;
    float scale;
};

// ---- 0. page means of the cached keys --------------------------------------

// Thread = (page, 8-channel unit): a 16-byte load per page row; a workgroup
// covers 256 / (D/8) pages.
template <int D>
__global__ __launch_bounds__(256) void losa_pool_kernel(const uint16_t* __restrict__ kc, float* __restrict__ kp,
                                                        int Lp, int page, int n_pages) {
    constexpr int U = D / 8;
    const int P = blockIdx.x * (256 / U) + threadIdx.x / U, u = threadIdx.x % U;
    const int g = blockIdx.y, b = blockIdx.z;
    if (P >= n_pages) return;
    const int64_t head = static_cast<int64_t>(b) * gridDim.y + g;
    const uint16_t* src = kc + (head * Lp + static_cast<int64_t>(P) * page) * D + u * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int r = 0; r < page; ++r) {
        const uint4 x = *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(r) * D);
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += __uint_as_float(w[e] << 16);
            acc[2 * e + 1] += __uint_as_float(w[e] & 0xFFFF0000u);
        }
    }
    float* dst = kp + (head * n_pages + P) * D + u * 8;
    const float inv = static_cast<float>(page);
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[e] = acc[e] / inv;
}

// ---- 1. locality scores and the Active list --------------------------------

// Workgroup (token i, b): delta over the Hq * D channels of the token, 16-byte
// loads, fp64 squares and sums.
__global__ __launch_bounds__(256) void losa_delta_kernel(Dims dm, const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ qp, double* __restrict__ delta,
                                                         double* locality) {
    __shared__ double part[4];
    const int i = blockIdx.x, b = blockIdx.y, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int U = dm.D / 8, n_units = dm.Hq * U;
    double acc = 0.0;
    for (int k = threadIdx.x; k < n_units; k += 256) {
        const int h = k / U, u = k - h * U;
        const int64_t off = ((static_cast<int64_t>(b) * dm.Hq + h) * dm.Bs + i) * dm.D + u * 8;
        const uint4 x = *reinterpret_cast<const uint4*>(q + off);
        const uint4 y = *reinterpret_cast<const uint4*>(qp + off);
        const uint32_t xa[4] = {x.x, x.y, x.z, x.w}, ya[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const double dl = static_cast<double>(__uint_as_float(xa[e] << 16)) -
                              static_cast<double>(__uint_as_float(ya[e] << 16));
            const double dh = static_cast<double>(__uint_as_float(xa[e] & 0xFFFF0000u)) -
                              static_cast<double>(__uint_as_float(ya[e] & 0xFFFF0000u));
            acc = fma(dl, dl, acc);
            acc = fma(dh, dh, acc);
        }
    }
    acc = wave_sum(acc);
    if (lane == 0) part[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        const double dv = (part[0] + part[1] + part[2] + part[3]) / static_cast<double>(dm.Hq * dm.D);
        delta[static_cast<int64_t>(b) * dm.Bs + i] = dv;
        if (locality != nullptr) locality[static_cast<int64_t>(b) * dm.Bs + i] = dv;
    }
}

// ---- 2. the Active set and the page scores of its query rows ----------------
// Workgroup (32-page chunk, kv head g, b).  Wave 0 ranks the block's tokens by
// (delta desc, index asc) into the Active list (ascending); the workgroups of
// chunk 0 also write that list out (kv head 0) and clear the kv head's page
// bitmap for the top-k kernel.  Group row r = (query head g*G + r / n_a,
// Active slot r % n_a).  Thread = (page t % 32, row slot t / 32); 32 rows per
// pass, 4 per thread.

template <int D>
__global__ __launch_bounds__(256) void losa_scores_kernel(Dims dm, const uint16_t* __restrict__ q,
                                                          const double* __restrict__ delta,
                                                          int32_t* __restrict__ active_out,
                                                          uint32_t* __restrict__ bitmap, int n_words,
                                                          const float* __restrict__ kp, float* __restrict__ scores) {
    constexpr int KW = D + 4;  // page-mean row stride in floats (16-byte aligned; lanes 0-15 hit distinct banks)
    __shared__ __align__(16) float ks[32 * KW];
    __shared__ __align__(16) float qs[32 * D];
    __shared__ int act[kMaxBlockLen];
    __shared__ double dsh[kMaxBlockLen];
    const int P0 = blockIdx.x * 32, g = blockIdx.y, b = blockIdx.z;
    const int t = threadIdx.x, pg = t & 31, slot = t >> 5;
    const int64_t kvh = static_cast<int64_t>(b) * dm.Hkv + g;
    // the page means first: their loads overlap the ranking below
    for (int idx = t; idx < 32 * (D / 4); idx += 256) {
        const int p = idx / (D / 4), c4 = idx - p * (D / 4);
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (P0 + p < dm.n_pages) v = *reinterpret_cast<const float4*>(kp + (kvh * dm.n_pages + P0 + p) * D + 4 * c4);
        *reinterpret_cast<float4*>(&ks[p * KW + 4 * c4]) = v;
    }
    if (t < dm.Bs) dsh[t] = delta[static_cast<int64_t>(b) * dm.Bs + t];
    __syncthreads();
    if (t < 64) {
        const int lane = t;
        const bool valid = lane < dm.Bs;
        const double di = valid ? dsh[lane] : 0.0;
        int rank = 0;
        for (int j = 0; j < dm.Bs; ++j) {
            const double dj = dsh[j];
            rank += (dj > di || (dj == di && j < lane)) ? 1 : 0;
        }
        const bool is_act = valid && rank < dm.n_a;
        const unsigned long long mask = __ballot(is_act);
        if (is_act) {
            const int pos = __popcll(mask & ((1ull << lane) - 1ull));
            act[pos] = lane;
            if (blockIdx.x == 0 && g == 0) active_out[static_cast<int64_t>(b) * dm.n_a + pos] = lane;
        }
    }
    if (blockIdx.x == 0)
        for (int w = t; w < n_words; w += 256) bitmap[kvh * n_words + w] = 0u;
    const int R = dm.G * dm.n_a;
    for (int r0 = 0; r0 < R; r0 += 32) {
        __syncthreads();
        for (int idx = t; idx < 32 * (D / 8); idx += 256) {
            const int rr = idx / (D / 8), u = idx - rr * (D / 8), r = r0 + rr;
            uint4 x = make_uint4(0u, 0u, 0u, 0u);
            if (r < R) {
                const int h = g * dm.G + r / dm.n_a, i = act[r % dm.n_a];
                x = *reinterpret_cast<const uint4*>(q + ((static_cast<int64_t>(b) * dm.Hq + h) * dm.Bs + i) * D + 8 * u);
            }
            float4* dst = reinterpret_cast<float4*>(&qs[rr * D + 8 * u]);
            dst[0] = make_float4(__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xFFFF0000u),
                                 __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xFFFF0000u));
            dst[1] = make_float4(__uint_as_float(x.z << 16), __uint_as_float(x.z & 0xFFFF0000u),
                                 __uint_as_float(x.w << 16), __uint_as_float(x.w & 0xFFFF0000u));
        }
        __syncthreads();
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int c4 = 0; c4 < D / 4; ++c4) {
            const float4 kv = *reinterpret_cast<const float4*>(&ks[pg * KW + 4 * c4]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 qv = *reinterpret_cast<const float4*>(&qs[(slot + 8 * j) * D + 4 * c4]);
                acc[j] = fmaf(qv.x, kv.x, acc[j]);
                acc[j] = fmaf(qv.y, kv.y, acc[j]);
                acc[j] = fmaf(qv.z, kv.z, acc[j]);
                acc[j] = fmaf(qv.w, kv.w, acc[j]);
            }
        }
        const int P = P0 + pg;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = r0 + slot + 8 * j;
            if (r < R && P < dm.n_pages) {
                const int h = g * dm.G + r / dm.n_a, a = r % dm.n_a;
                scores[((static_cast<int64_t>(b) * dm.Hq + h) * dm.n_a + a) * dm.n_pages + P] = dm.scale * acc[j];
            }
        }
    }
}

// ---- 3. per-row top-k pages into the kv head's bitmap -----------------------
// One wave per (b, h, a) row, NPL entries per lane in registers (page
// lane + 64 j) as 64-bit keys: the order-preserving image of the score in the
// high word, ~page in the low word, so a larger key is a better entry under
// (score desc, page asc).  Round k takes the largest key below round k-1's
// pick, so nothing is marked or moved.  Key 0 is "no entry".

__device__ __forceinline__ uint64_t score_key(float v, int P) {
    const uint32_t u = __float_as_uint(v);
    const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return (static_cast<uint64_t>(ord) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(P));
}

// Wave-wide max of a 64-bit key in registers: DPP moves pair every lane with
// one in the other half of its 2, 4, 8 and 16 lanes, then v_permlane16_swap
// and v_permlane32_swap bring in the other row and the other half-wave.
template <int CTRL>
__device__ __forceinline__ uint64_t max_with_dpp(uint64_t x) {
    const uint32_t hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(x >> 32), CTRL, 0xF, 0xF, false);
    const uint32_t lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, 0xF, 0xF, false);
    const uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
    return o > x ? o : x;
}

__device__ __forceinline__ uint64_t max_of_pair(uint32_t h0, uint32_t l0, uint32_t h1, uint32_t l1) {
    const uint64_t a = (static_cast<uint64_t>(h0) << 32) | l0, b = (static_cast<uint64_t>(h1) << 32) | l1;
    return a > b ? a : b;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
    x = max_with_dpp<0xB1>(x);   // quad_perm [1,0,3,2]
    x = max_with_dpp<0x4E>(x);   // quad_perm [2,3,0,1]
    x = max_with_dpp<0x141>(x);  // row_half_mirror
    x = max_with_dpp<0x140>(x);  // row_mirror
    uint32_t hi = static_cast<uint32_t>(x >> 32), lo = static_cast<uint32_t>(x);
    const auto h16 = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    const auto l16 = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    x = max_of_pair(h16[0], l16[0], h16[1], l16[1]);
    hi = static_cast<uint32_t>(x >> 32);
    lo = static_cast<uint32_t>(x);
    const auto h32 = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    const auto l32 = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    return max_of_pair(h32[0], l32[0], h32[1], l32[1]);
}

template <int NPL>
__global__ __launch_bounds__(256) void losa_topk_kernel(Dims dm, const float* __restrict__ scores,
                                                        uint32_t* __restrict__ bitmap, int n_words, int64_t n_rows) {
    const int lane = threadIdx.x & 63;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (row >= n_rows) return;
    const int64_t bh = row / dm.n_a;  // b * Hq + h
    const int b = static_cast<int>(bh / dm.Hq), h = static_cast<int>(bh % dm.Hq);
    const float* sr = scores + row * dm.n_pages;
    uint64_t keys[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
        const int P = lane + 64 * j;
        keys[j] = P < dm.n_pages ? score_key(sr[P], P) : 0ull;
    }
    uint32_t* bm = bitmap + (static_cast<int64_t>(b) * dm.Hkv + h / dm.G) * n_words;
    uint64_t prev = ~0ull;
    for (int k = 0; k < dm.kpq; ++k) {
        uint64_t bq[4] = {0ull, 0ull, 0ull, 0ull};  // four independent chains over j mod 4
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
            const uint64_t x = keys[j];
            bq[j & 3] = (x < prev && x > bq[j & 3]) ? x : bq[j & 3];
        }
        uint64_t best = bq[0] > bq[1] ? bq[0] : bq[1];
        const uint64_t b23 = bq[2] > bq[3] ? bq[2] : bq[3];
        best = best > b23 ? best : b23;
        best = wave_max_u64(best);
        if (best == 0ull) break;  // fewer orderable entries than kpq
        prev = best;
        const int P = static_cast<int>(~static_cast<uint32_t>(best));
        if (lane == 0) atomicOr(&bm[P >> 5], 1u << (P & 31));
    }
}

// One workgroup per row for budgets of at most 64 pages: wave w takes the
// top-k keys of pages w*64 + lane + 256 j (NPL4 per lane) into LDS; wave 0
// then takes the top-k of those 4k candidates, which hold the row's top-k.
template <int NPL4>
__global__ __launch_bounds__(256) void losa_topk4_kernel(Dims dm, const float* __restrict__ scores,
                                                         uint32_t* __restrict__ bitmap, int n_words) {
    __shared__ uint64_t cand[4][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t row = blockIdx.x;
    const int64_t bh = row / dm.n_a;  // b * Hq + h
    const int b = static_cast<int>(bh / dm.Hq), h = static_cast<int>(bh % dm.Hq);
    const float* sr = scores + row * dm.n_pages;
    uint64_t keys[NPL4];
#pragma unroll
    for (int j = 0; j < NPL4; ++j) {
        const int P = wave * 64 + lane + 256 * j;
        keys[j] = P < dm.n_pages ? score_key(sr[P], P) : 0ull;
    }
    uint64_t prev = ~0ull;
    for (int k = 0; k < dm.kpq; ++k) {
        uint64_t best = 0ull;
#pragma unroll
        for (int j = 0; j < NPL4; ++j) best = (keys[j] < prev && keys[j] > best) ? keys[j] : best;
        best = wave_max_u64(best);
        if (lane == 0) cand[wave][k] = best;  // 0 once this quarter has no entry left
        prev = best;
    }
    __syncthreads();
    if (wave != 0) return;
    uint64_t c4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) c4[q] = lane < dm.kpq ? cand[q][lane] : 0ull;
    uint32_t* bm = bitmap + (static_cast<int64_t>(b) * dm.Hkv + h / dm.G) * n_words;
    prev = ~0ull;
    for (int k = 0; k < dm.kpq; ++k) {
        uint64_t best = 0ull;
#pragma unroll
        for (int q = 0; q < 4; ++q) best = (c4[q] < prev && c4[q] > best) ? c4[q] : best;
        best = wave_max_u64(best);
        if (best == 0ull) break;  // fewer orderable entries than kpq
        prev = best;
        const int P = static_cast<int>(~static_cast<uint32_t>(best));
        if (lane == 0) atomicOr(&bm[P >> 5], 1u << (P & 31));
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

// ---- 5. partial softmax of a row tile over one key chunk ---------------------
// A tile of RT = 16 * RPT query rows (32 or 64) against 64-key tiles of the
// chunk.  Scores: 32x32 blocks S^T = K Q^T with v_mfma_f32_32x32x16_bf16, one
// block per wave (RT/32 row blocks x 2 key blocks), scaled into LDS.
// Softmax: 256 / RT lanes per row, P packed to bf16 key pairs.  Output:
// 32-channel x 32-row blocks O^T += V^T P^T on MFMA, the V^T operand read
// from V stored as key-pair words, the P^T operand as four pair words.

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
    float* part;                 // partials [B][Hkv][row_tiles*RT][n_chunks+1][D+4]: o, m, l, 2 pad
    int cap, R, row_tiles, chunk, n_chunks, dense;
    float scale_log2;            // scale * log2(e)
};

template <int D, int RPT>
__global__ __launch_bounds__(256) void losa_attend_kernel(AttendArgs a) {
    constexpr int RT = 16 * RPT;      // rows per tile (32 or 64)
    constexpr int QW = D / 2 + 4;     // LDS row stride of Q and K tiles in 32-bit words (16-byte aligned)
    constexpr int VU = D / 8;         // 16-byte units per row
    constexpr int TPR = 256 / RT;     // softmax lanes per row
    constexpr int KPL = kKeyTile / TPR;
    constexpr int PW = kKeyTile / 2 + 4;     // P pair row stride in words (16-byte aligned)
    constexpr int NSB = (RT / 32) * 2;       // 32x32 score blocks per tile (row block x key block)
    constexpr int NOB = (RT / 32) * (D / 32);  // 32-row x 32-channel output blocks
    constexpr int OPW = (NOB + 3) / 4;       // output blocks per wave
    constexpr int DK = D / 16;               // MFMA k-steps of q.k
    __shared__ __align__(16) uint32_t qs[RT * QW];
    __shared__ __align__(16) uint32_t ks[kKeyTile * QW];
    __shared__ __align__(16) uint4 vp[(kKeyTile / 2) * (D / 4)];  // V as key pairs: word (m, c) = {v[2m][c], v[2m+1][c]}
    __shared__ float ss[RT][kKeyTile + 1];
    __shared__ __align__(16) uint32_t ps[RT * PW];                 // P as bf16 key pairs
    __shared__ float m_s[RT], l_s[RT], al_s[RT];

    const Dims& dm = a.dm;
    // workgroup id -> (chunk, row tile): ids x and x + 8 share the chunk and take
    // consecutive row tiles, so the tiles of one chunk run together on one XCD
    // (ids go to the 8 XCDs in turn) and read its K/V through the same L2
    const int x = blockIdx.x;
    const int rt = (x >> 3) % a.row_tiles;
    const int c = (x & 7) + 8 * (x / (8 * a.row_tiles));
    if (c > a.n_chunks) return;
    const int g = blockIdx.y, b = blockIdx.z;
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
    const int r0 = rt * RT;
    const int nrows = min(RT, a.R - r0);
    const int n_a = a.dense ? dm.Bs : dm.n_a;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, l32 = lane & 31, hl = lane >> 5;

    for (int idx = t; idx < RT * VU; idx += 256) {
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
    if (t < RT) {
        m_s[t] = -INFINITY;
        l_s[t] = 0.f;
    }

    // row of key kk of the current tile in its K/V tensor (the block's own, or the cache)
    auto key_row = [&](int k0, int kk) -> int64_t {
        if (suffix) return kvh * dm.Bs + k0 + kk;
        const int j = c * a.chunk + k0 + kk;
        const int pos = a.dense ? j : a.upages[kvh * a.cap + j / dm.page] * dm.page + j % dm.page;
        return kvh * dm.Lp + pos;
    };
    const uint16_t* kbase = suffix ? a.kb : a.kc;
    const uint16_t* vbase = suffix ? a.vb : a.vc;

    // output blocks of this wave: block ob = wave + 4 j -> rows 32 (ob / (D/32)), channels 32 (ob % (D/32))
    f32x16 oacc[OPW];
#pragma unroll
    for (int j = 0; j < OPW; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[j][r] = 0.f;

    // K/V of a tile pass through registers: the next tile's loads are issued
    // before the current tile is computed, so their latency overlaps it
    constexpr int KIT = kKeyTile * VU / 256;         // K units per thread
    constexpr int VIT = (kKeyTile / 2) * VU / 256;   // V key-pair units per thread
    uint4 kr[KIT], va[VIT], vb[VIT];
    auto load_tile = [&](int k0) {
        const int nk = min(kKeyTile, n_keys - k0);
#pragma unroll
        for (int it = 0; it < KIT; ++it) {
            const int idx = t + 256 * it, kk = idx / VU, u = idx - kk * VU;
            kr[it] = kk < nk ? *reinterpret_cast<const uint4*>(kbase + key_row(k0, kk) * D + u * 8)
                             : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int it = 0; it < VIT; ++it) {
            const int idx = t + 256 * it, m = idx / VU, u = idx - m * VU;
            va[it] = 2 * m < nk ? *reinterpret_cast<const uint4*>(vbase + key_row(k0, 2 * m) * D + u * 8)
                                : make_uint4(0u, 0u, 0u, 0u);
            vb[it] = 2 * m + 1 < nk ? *reinterpret_cast<const uint4*>(vbase + key_row(k0, 2 * m + 1) * D + u * 8)
                                    : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int it = 0; it < KIT; ++it) {
            const int idx = t + 256 * it, kk = idx / VU, u = idx - kk * VU;
            *reinterpret_cast<uint4*>(&ks[kk * QW + u * 4]) = kr[it];
        }
#pragma unroll
        for (int it = 0; it < VIT; ++it) {
            const int idx = t + 256 * it, m = idx / VU, u = idx - m * VU;
            const uint32_t a0[4] = {va[it].x, va[it].y, va[it].z, va[it].w};
            const uint32_t a1[4] = {vb[it].x, vb[it].y, vb[it].z, vb[it].w};
            uint32_t w[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                w[2 * e] = (a0[e] & 0xFFFFu) | (a1[e] << 16);               // channel 2e of keys 2m, 2m+1
                w[2 * e + 1] = (a0[e] >> 16) | (a1[e] & 0xFFFF0000u);      // channel 2e+1
            }
            vp[m * (D / 4) + 2 * u] = make_uint4(w[0], w[1], w[2], w[3]);
            vp[m * (D / 4) + 2 * u + 1] = make_uint4(w[4], w[5], w[6], w[7]);
        }
    };

    load_tile(0);
    for (int k0 = 0; k0 < n_keys; k0 += kKeyTile) {
        const int nk = min(kKeyTile, n_keys - k0);
        store_tile();
        __syncthreads();
        if (k0 + kKeyTile < n_keys) load_tile(k0 + kKeyTile);

        // S^T block (32 keys x 32 rows) = K Q^T: lane holds row l32 of the tile's row block,
        // keys 8 (r / 4) + 4 hl + r % 4 of its key block
        if (wave < NSB) {
            const int rw = wave >> 1, kw = wave & 1;
            f32x16 sacc;
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
            for (int st = 0; st < DK; ++st) {
                const bf16x8 kop = *reinterpret_cast<const bf16x8*>(&ks[(kw * 32 + l32) * QW + 8 * st + 4 * hl]);
                const bf16x8 qop = *reinterpret_cast<const bf16x8*>(&qs[(rw * 32 + l32) * QW + 8 * st + 4 * hl]);
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop, sacc, 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kw * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
                ss[rw * 32 + l32][key] = key < nk ? sacc[r] * a.scale_log2 : -INFINITY;
            }
        }
        __syncthreads();

        {  // online softmax: TPR lanes per row, key pairs pt + TPR j; P stored as bf16 pairs
            const int row = t / TPR, pt = t % TPR;
            float mx = -INFINITY;
#pragma unroll
            for (int j = 0; j < KPL / 2; ++j) {
                const int m = pt + TPR * j;
                mx = fmaxf(mx, fmaxf(ss[row][2 * m], ss[row][2 * m + 1]));
            }
#pragma unroll
            for (int off = 1; off < TPR; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
            const float m_old = m_s[row];
            const float m_new = fmaxf(m_old, mx);
            float sum = 0.f;
#pragma unroll
            for (int j = 0; j < KPL / 2; ++j) {
                const int m = pt + TPR * j;
                const float p0 = exp2f(ss[row][2 * m] - m_new), p1 = exp2f(ss[row][2 * m + 1] - m_new);
                ps[row * PW + m] = pack_bf16x2(p0, p1);
                sum += p0 + p1;
            }
#pragma unroll
            for (int off = 1; off < TPR; off <<= 1) sum += __shfl_xor(sum, off, 64);
            if (pt == 0) {
                const float alpha = exp2f(m_old - m_new);
                l_s[row] = l_s[row] * alpha + sum;
                m_s[row] = m_new;
                al_s[row] = alpha;
            }
        }
        __syncthreads();

        // O^T block (32 channels x 32 rows) += V^T P^T over the tile's 64 keys (4 k-steps of 16)
#pragma unroll
        for (int j = 0; j < OPW; ++j) {
            const int ob = wave + 4 * j;
            if (ob < NOB) {
                const int rw = ob / (D / 32), dw = ob % (D / 32);
                const int row = rw * 32 + l32;
                const float al = al_s[row];
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[j][r] *= al;
                const uint32_t* vw = reinterpret_cast<const uint32_t*>(vp);
#pragma unroll
                for (int kst = 0; kst < kKeyTile / 16; ++kst) {
                    const int m0 = 8 * kst + 4 * hl;  // first key pair of this lane's 8 keys
                    const uint32_t vv[4] = {vw[(m0 + 0) * D + dw * 32 + l32], vw[(m0 + 1) * D + dw * 32 + l32],
                                            vw[(m0 + 2) * D + dw * 32 + l32], vw[(m0 + 3) * D + dw * 32 + l32]};
                    const uint4 pp = *reinterpret_cast<const uint4*>(&ps[row * PW + m0]);
                    oacc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv),
                                                                     __builtin_bit_cast(bf16x8, pp), oacc[j], 0, 0, 0);
                }
            }
        }
        __syncthreads();
    }

    // partial (unnormalised o, m, l) of every row: lane holds row l32, channels 8 (r / 4) + 4 hl + r % 4
    const int parts = a.n_chunks + 1;
#pragma unroll
    for (int j = 0; j < OPW; ++j) {
        const int ob = wave + 4 * j;
        if (ob >= NOB) continue;
        const int rw = ob / (D / 32), dw = ob % (D / 32);
        const int rr = rw * 32 + l32;
        if (rr >= nrows) continue;
        float* dst = a.part + ((kvh * a.row_tiles * RT + r0 + rr) * parts + c) * (D + 4) + dw * 32 + 4 * hl;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            *reinterpret_cast<float4*>(dst + 8 * q4) =
                make_float4(oacc[j][4 * q4], oacc[j][4 * q4 + 1], oacc[j][4 * q4 + 2], oacc[j][4 * q4 + 3]);
    }
    if (t < nrows) {
        float* dst = a.part + ((kvh * a.row_tiles * RT + r0 + t) * parts + c) * (D + 4);
        dst[D] = m_s[t];
        dst[D + 1] = l_s[t];
    }
}

// ---- 6. merge of the partials -------------------------------------------------
// One wave per query row.  The maximum M of the partials' m comes first
// (lanes over partials); then lane (group cg = lane / 16, column cl =
// lane % 16) accumulates channels cl*D/16 .. of partials cg, cg + 4, ... with
// weight 2^(m - M), so four partials' loads are in flight per step; the four
// groups are summed with shuffles.

struct MergeArgs {
    Dims dm;
    const float* part;
    const int32_t* active;
    const int32_t* ucount;
    uint16_t* o;
    float* lse;
    int R, RT, row_tiles, chunk, n_chunks, dense;
};

template <int D>
__global__ __launch_bounds__(256) void losa_merge_kernel(MergeArgs a) {
    constexpr int DC = D / 16;  // channels per lane
    const Dims& dm = a.dm;
    const int lane = threadIdx.x & 63, cg = lane >> 4, cl = lane & 15;
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
    // entries k = 0 .. n_valid - 1 are prefix chunks, entry n_valid is the block's keys (chunk n_chunks)
    const int n_valid = a.dense ? a.n_chunks : (a.ucount[kvh] * dm.page + a.chunk - 1) / a.chunk;
    const float* base = a.part + (kvh * a.row_tiles * a.RT + r) * static_cast<int64_t>(parts) * (D + 4);
    auto entry = [&](int k) { return base + static_cast<int64_t>(k == n_valid ? a.n_chunks : k) * (D + 4); };

    float M = -INFINITY;
    for (int k = lane; k <= n_valid; k += 64) M = fmaxf(M, entry(k)[D]);
    M = wave_max(M);
    float acc[DC];
#pragma unroll
    for (int e = 0; e < DC; ++e) acc[e] = 0.f;
    float L = 0.f;
    for (int k0 = 0; k0 <= n_valid; k0 += 64) {
        // weight of entry k0 + lane, and its share of the denominator
        float wl = 0.f;
        if (k0 + lane <= n_valid) {
            const float* p = entry(k0 + lane);
            wl = exp2f(p[D] - M);
            L = fmaf(p[D + 1], wl, L);
        }
        const int nb = min(n_valid, k0 + 63) - k0 + 1;  // entries in this batch of 64
        // uniform trip count: every lane takes part in the shuffle, lanes past the batch skip the sum
#pragma unroll 4
    for (int i = 0; i < nb; i += 4) {
        const float w = __shfl(wl, (i + cg) & 63, 64);
        if (i + cg >= nb) continue;
        const float* p = entry(k0 + i + cg);
        const float4* x = reinterpret_cast<const float4*>(p + cl * DC);
#pragma unroll
        for (int e = 0; e < DC / 4; ++e) {
            const float4 v = x[e];
            acc[4 * e] = fmaf(v.x, w, acc[4 * e]);
            acc[4 * e + 1] = fmaf(v.y, w, acc[4 * e + 1]);
            acc[4 * e + 2] = fmaf(v.z, w, acc[4 * e + 2]);
            acc[4 * e + 3] = fmaf(v.w, w, acc[4 * e + 3]);
        }
    }
    }
#pragma unroll
    for (int e = 0; e < DC; ++e) {
        acc[e] += __shfl_xor(acc[e], 16, 64);
        acc[e] += __shfl_xor(acc[e], 32, 64);
    }
    L = wave_sum(L);
    if (cg != 0) return;
    const float inv = 1.f / L;
    uint32_t packed[DC / 2];
#pragma unroll
    for (int e = 0; e < DC / 2; ++e) packed[e] = pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
    uint16_t* dst = a.o + ((static_cast<int64_t>(b) * dm.Hq + h) * dm.Bs + i) * D + cl * DC;
    if constexpr (DC == 8)
        *reinterpret_cast<uint4*>(dst) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    else
        *reinterpret_cast<uint2*>(dst) = make_uint2(packed[0], packed[1]);
    if (lane == 0) a.lse[(static_cast<int64_t>(b) * dm.Hq + h) * dm.Bs + i] = (M + log2f(L)) * 0.6931471805599453f;
}

// ---- host side ------------------------------------------------------------------

struct Plan {
    Dims dm;
    int n_words, cap, npl;
    int R_s, RT_s, rt_s, nch_s;    // later iterations: rows per kv head, tile rows, tiles, prefix chunks
    int R_d, RT_d, rt_d, nch_d;    // first iteration
    size_t off_scores, off_bits, off_delta, off_part, ws_step, ws_dense;
};

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

int tile_rows(int R) { return R <= 32 ? 32 : 64; }

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
    if (p->batch > 65535 || p->kv_heads > 65535) return fail(SDATTN_ERR_SHAPE, "batch and kv_heads must be <= 65535");

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
    pl.RT_s = tile_rows(pl.R_s);
    pl.rt_s = (pl.R_s + pl.RT_s - 1) / pl.RT_s;
    pl.cap = static_cast<int>(std::min<int64_t>(n_pages, static_cast<int64_t>(pl.R_s) * dm.kpq));
    pl.nch_s = static_cast<int>((static_cast<int64_t>(pl.cap) * dm.page + kChunkSparse - 1) / kChunkSparse);
    pl.R_d = dm.G * dm.Bs;
    pl.RT_d = tile_rows(pl.R_d);
    pl.rt_d = (pl.R_d + pl.RT_d - 1) / pl.RT_d;
    pl.nch_d = (dm.Lp + kChunkDense - 1) / kChunkDense;
    const size_t part_row = static_cast<size_t>(dm.D + 4) * sizeof(float);  // 16-byte multiple
    pl.off_scores = 0;
    pl.off_bits = align256(static_cast<size_t>(dm.B) * dm.Hq * dm.n_a * n_pages * sizeof(float));
    pl.off_delta = pl.off_bits + align256(static_cast<size_t>(dm.B) * dm.Hkv * pl.n_words * sizeof(uint32_t));
    pl.off_part = pl.off_delta + align256(static_cast<size_t>(dm.B) * dm.Bs * sizeof(double));
    pl.ws_step = pl.off_part +
                 static_cast<size_t>(dm.B) * dm.Hkv * pl.rt_s * pl.RT_s * (pl.nch_s + 1) * part_row;
    pl.ws_dense = static_cast<size_t>(dm.B) * dm.Hkv * pl.rt_d * pl.RT_d * (pl.nch_d + 1) * part_row;
    // Every launch of a call must fit HIP's limit of 2^32 work-items per grid
    // dimension; checked here, before anything is enqueued, so that a call
    // that fails writes nothing.
    constexpr int64_t kMaxItems = int64_t{1} << 32;
    const int64_t topk_rows = static_cast<int64_t>(dm.B) * dm.Hq * dm.n_a;
    const int64_t topk_items = dm.kpq <= 64 ? topk_rows * 256 : (topk_rows + 3) / 4 * 256;
    const int64_t merge_items = (static_cast<int64_t>(dm.B) * dm.Hkv * std::max(pl.R_s, pl.R_d) + 3) / 4 * 256;
    const int64_t attend_s = static_cast<int64_t>((pl.nch_s + 1 + 7) / 8) * 8 * pl.rt_s * 256;
    const int64_t attend_d = static_cast<int64_t>((pl.nch_d + 1 + 7) / 8) * 8 * pl.rt_d * 256;
    if (topk_items >= kMaxItems || merge_items >= kMaxItems || attend_s >= kMaxItems || attend_d >= kMaxItems)
        return fail(SDATTN_ERR_SHAPE, "problem too large for one launch: batch * q_heads * n_active (and "
                                      "batch * q_heads * block_len / 4) must stay below 2^24");
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
    const int RT = dense ? pl.RT_d : pl.RT_s;
    a.row_tiles = dense ? pl.rt_d : pl.rt_s;
    a.chunk = dense ? kChunkDense : kChunkSparse;
    a.n_chunks = dense ? pl.nch_d : pl.nch_s;
    a.dense = dense ? 1 : 0;
    a.scale_log2 = dm.scale * kLog2e;
    const dim3 grid(((a.n_chunks + 1 + 7) / 8) * 8 * a.row_tiles, dm.Hkv, dm.B);
    if (RT == 32)
        hipLaunchKernelGGL((losa_attend_kernel<D, 2>), grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((losa_attend_kernel<D, 4>), grid, dim3(256), 0, st, a);
    MergeArgs m;
    m.dm = dm;
    m.part = part;
    m.active = active;
    m.ucount = ucount;
    m.o = static_cast<uint16_t*>(o);
    m.lse = lse;
    m.R = a.R;
    m.RT = RT;
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
    const int ppw = 256 / (dm.D / 8);  // pages per workgroup
    const dim3 grid((dm.n_pages + ppw - 1) / ppw, dm.Hkv, dm.B);
    if (dm.D == 128)
        hipLaunchKernelGGL(losa_pool_kernel<128>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(k_cache), kp,
                           dm.Lp, dm.page, dm.n_pages);
    else
        hipLaunchKernelGGL(losa_pool_kernel<64>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(k_cache), kp,
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

    double* delta = reinterpret_cast<double*>(w + pl.off_delta);
    hipLaunchKernelGGL(losa_delta_kernel, dim3(dm.Bs, dm.B), dim3(256), 0, st, dm, q16,
                       static_cast<const uint16_t*>(q_prev), delta, locality);
    const dim3 sgrid((dm.n_pages + 31) / 32, dm.Hkv, dm.B);
    if (dm.D == 128)
        hipLaunchKernelGGL(losa_scores_kernel<128>, sgrid, dim3(256), 0, st, dm, q16, delta, active_idx, bits,
                           pl.n_words, kp, scores);
    else
        hipLaunchKernelGGL(losa_scores_kernel<64>, sgrid, dim3(256), 0, st, dm, q16, delta, active_idx, bits,
                           pl.n_words, kp, scores);
    if (dm.kpq <= 64) {
        const dim3 tgrid(static_cast<unsigned>(static_cast<int64_t>(dm.B) * dm.Hq * dm.n_a));
        switch (pl.npl) {  // pages per lane over a quarter row: npl / 4
            case 8: hipLaunchKernelGGL(losa_topk4_kernel<2>, tgrid, dim3(256), 0, st, dm, scores, bits, pl.n_words); break;
            case 16: hipLaunchKernelGGL(losa_topk4_kernel<4>, tgrid, dim3(256), 0, st, dm, scores, bits, pl.n_words); break;
            case 32: hipLaunchKernelGGL(losa_topk4_kernel<8>, tgrid, dim3(256), 0, st, dm, scores, bits, pl.n_words); break;
            default: hipLaunchKernelGGL(losa_topk4_kernel<16>, tgrid, dim3(256), 0, st, dm, scores, bits, pl.n_words); break;
        }
    } else {
        switch (pl.npl) {
            case 8: launch_topk<8>(pl, scores, bits, st); break;
            case 16: launch_topk<16>(pl, scores, bits, st); break;
            case 32: launch_topk<32>(pl, scores, bits, st); break;
            default: launch_topk<64>(pl, scores, bits, st); break;
        }
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
