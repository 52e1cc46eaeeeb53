// Bidirectional flash-style attention forward for bf16 inputs on gfx950.
//
// One kernel template serves the three attention forms of the library:
//   dense         every query attends all L keys (SparseD, abstract: full
//                 attention in the early steps);
//   block-sparse  query block I of head h attends the key tokens of the key
//                 blocks in its CSR row (Step-dLLM, Abstract);
//   column-sparse every query of group g attends a shared list of key
//                 tokens (PulseCol, Abstract), either gathered by index in
//                 every workgroup or read from rows gathered once per step
//                 (packed, [B][Hkv][kcol][d], streamed like dense tiles).
// Each form streams key tiles; only where the tile's rows come from differs.
//
// Work decomposition: one workgroup per (batch, head, tile of 32 NW queries),
// each of the NW waves owning 32 query rows.  Per KT-key tile (KT = 64, or 32
// for 64-query blocks):
//   * the K and V rows of the tile go from HBM straight into LDS with the
//     buffer-to-LDS DMA, NST stages deep (one barrier per tile); each lane
//     fetches the 16-byte chunk that belongs at its LDS slot, so the tile
//     lands XOR-swizzled and every MFMA operand read is conflict-free;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16, Q held in registers;
//     computing the transpose puts one query per lane, so row sums stay
//     in-lane;
//   * P^T is packed to bf16 straight from the MFMA accumulator layout and is
//     the B operand of O^T += V^T P^T, whose A operand comes from the
//     row-major V tile through the transposing LDS read;
//   * the softmax reference is the maximum of the first tile, not a running
//     maximum: the other tiles exponentiate against it without a per-tile
//     maximum or branch, and a row whose sum leaves a safe range is redone
//     in a second pass that raises the reference whenever a block's
//     probabilities grow too large (exact either way: numerator and
//     denominator share the reference).
// The log-sum-exp (natural log) is written per query row.

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace sdattn {
namespace {

struct FlashParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    const int32_t* row_ptr;
    const int32_t* col_idx;
    int Hq, Hkv, L, group, n_qtiles, n_items, block_k, kcol, xcd_group;
    float c;      // scale * log2(e)
    float scale;  // softmax scale
};

// Bound on one lane's sum of 16 probabilities before the reference is raised
// (checked tiles), and on a lane's whole row sum after an unchecked pass.
constexpr float kBigSum = 0x1p64f;
constexpr float kBigRow = 0x1p32f;

// instruction classes for __builtin_amdgcn_sched_group_barrier
constexpr int SG_VALU = 0x002;
constexpr int SG_MFMA = 0x008;
constexpr int SG_DSR = 0x100;

template <int D, int NW, int KT, int NST, int MODE>
__global__ __launch_bounds__(NW * 64) void flash_fwd_bf16(FlashParams p) {
    // KT keys per tile (32 or 64), NST LDS stages (tiles in flight: NST - 1)
    constexpr int KB = KT / 32;             // 32-key MFMA blocks per tile
    constexpr int T = NW * 64;
    constexpr int DK = D / 16;
    constexpr int ND = D / 32;
    constexpr int ROWB = D * 2;             // bytes of one K / V row (HBM and LDS)
    constexpr int TILEB = KT * ROWB;        // one K or V tile
    constexpr int UNITS = D / 8;            // 16-byte units per row
    constexpr int SLOTS = KT * UNITS;       // 16-byte slots per tile
    constexpr int NDMA = SLOTS / T;         // DMA instructions per thread per tile (K; same for V)
    constexpr int ROWS_PER_DMA = T / UNITS;
    constexpr int OPITCH = D * 2;           // epilogue staging row (units XOR-swizzled by row)
    constexpr int STAGEB = 2 * TILEB;       // K tile then V tile
    static_assert(NDMA * T == SLOTS && T % UNITS == 0 && ROWS_PER_DMA % 4 == 0, "DMA tiling");
    static_assert(NW * 32 * OPITCH <= NST * STAGEB, "epilogue staging fits in the stages");

    __shared__ __attribute__((aligned(16))) char smem[NST * STAGEB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hl = lane >> 5;

    const int item = xcd_remap(blockIdx.x, p.n_items, p.xcd_group);
    const int qt = item % p.n_qtiles;
    const int bh = item / p.n_qtiles;
    const int h = bh % p.Hq;
    const int b = bh / p.Hq;
    const int g = h / p.group;
    const int L = p.L;
    const int kv_len = MODE == MODE_COLUMN_PACKED ? p.kcol : L;  // K/V rows per kv head
    const size_t kvoff = (static_cast<size_t>(b) * p.Hkv + g) * kv_len * D;
    const uint32_t head_bytes = static_cast<uint32_t>(kv_len) * ROWB;
    const u32x4 rk = buffer_rsrc(p.k + kvoff, head_bytes);
    const u32x4 rv = buffer_rsrc(p.v + kvoff, head_bytes);
    const int q0 = qt * (NW * 32);

    // ---- tile source ------------------------------------------------------
    // n_tiles tiles, of which the first n_full hold KT in-range keys; only
    // the end of the sequence (dense), the last kept block of a row (block:
    // rows are ascending) or the end of the column list can be partial.
    int n_tiles = 0, n_full = 0, e0 = 0, ne = 0, sub_shift = 0;
    int j_first = 0;  // block form: the row's first kept block
    const int32_t* cb = nullptr;
    if constexpr (MODE == MODE_DENSE) {
        n_tiles = (L + KT - 1) / KT;
        n_full = L / KT;
    } else if constexpr (MODE == MODE_BLOCK) {
        const int r = bh * p.n_qtiles + qt;
        e0 = p.row_ptr[r];
        ne = p.row_ptr[r + 1] - e0;
        // block_k / KT tiles per kept key block (block_k in {64, 128}, KT in {32, 64})
        sub_shift = (p.block_k == 128 ? 1 : 0) + (KT == 32 ? 1 : 0);
        if (ne > 0) {
            // the first and the last kept block, loaded together
            j_first = p.col_idx[e0];
            const int rem = L - p.col_idx[e0 + ne - 1] * p.block_k;  // keys of the last block in range
            const int per = 1 << sub_shift;
            n_tiles = ((ne - 1) << sub_shift) + min(per, (rem + KT - 1) / KT);
            n_full = ((ne - 1) << sub_shift) + min(per, rem / KT);
        }
    } else {
        if constexpr (MODE == MODE_COLUMN) cb = p.col_idx + (static_cast<size_t>(b) * p.Hkv + g) * p.kcol;
        n_tiles = (p.kcol + KT - 1) / KT;
        n_full = p.kcol / KT;
    }
    // first key of tile u (dense / block: a token index; column: an entry of
    // the column list; packed: a row of the gathered rows); J is the tile's
    // kept block (block form)
    auto tile_key0 = [&](int u, int J) __attribute__((always_inline)) -> int {
        if constexpr (MODE == MODE_BLOCK)
            return J * p.block_k + (u & ((1 << sub_shift) - 1)) * KT;
        else
            return u * KT;
    };
    // number of real keys in the tile that starts at key0
    auto tile_valid = [&](int key0) __attribute__((always_inline)) -> int {
        if constexpr (MODE == MODE_COLUMN || MODE == MODE_COLUMN_PACKED)
            return min(KT, p.kcol - key0);
        else
            return max(0, min(KT, L - key0));
    };
    auto block_of = [&](int u) __attribute__((always_inline)) -> int {
        return p.col_idx[e0 + min(u >> sub_shift, ne - 1)];
    };

    // LDS layouts (16-byte units, XOR-swizzled so that reads hit distinct banks):
    //   K tile: row r (key), unit u stored at unit u ^ (r & (UNITS-1));
    //   V tile: row r (key), unit u stored at unit u ^ (4 (r & 3)) mod UNITS.
    // The DMA writes 16 bytes per lane at consecutive LDS slots; each lane
    // fetches the HBM chunk that belongs at its slot.  All of a chunk's
    // offset is in the VGPR offset, which the buffer range check covers:
    // rows past L, and tiles past the last one (offset kOOB), read as zero.
    const int dr0 = tid / UNITS, dpu = tid % UNITS;  // row / physical unit of slot `tid`
    int kslot[NDMA], vslot[NDMA];  // byte offset of this lane's chunks within a tile (column: within a row)
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
        const int row = dr0 + i * ROWS_PER_DMA;
        const int uk = dpu ^ (row & (UNITS - 1));
        const int uv = dpu ^ ((4 * (row & 3)) & (UNITS - 1));
        const int rowb = MODE == MODE_COLUMN ? 0 : row * ROWB;
        kslot[i] = rowb + uk * 16;
        vslot[i] = rowb + uv * 16;
    }
    // Source of a tile to fetch, loaded one step before its DMA so that no
    // index load sits between a barrier and the DMA it feeds: the kept block
    // (block form) or this lane's key per DMA row (column form).
    struct Src {
        int j;
        int kn[NDMA];
    };
    constexpr int NPF = MODE == MODE_BLOCK ? 1 : (MODE == MODE_COLUMN ? NDMA : 0);  // loads per source
    auto load_src = [&](Src& sr, int u) __attribute__((always_inline)) {
        if constexpr (MODE == MODE_BLOCK) {
            sr.j = block_of(u);
        } else if constexpr (MODE == MODE_COLUMN) {
#pragma unroll
            for (int i = 0; i < NDMA; ++i) sr.kn[i] = cb[min(u * KT + dr0 + i * ROWS_PER_DMA, p.kcol - 1)];
        }
    };
    auto init_src = [&](Src& sr) __attribute__((always_inline)) {
        sr.j = 0;
#pragma unroll
        for (int i = 0; i < NDMA; ++i) sr.kn[i] = 0;
    };
    // DMA of the K rows (V = false) or V rows (V = true) of tile u into
    // `stage`, from its source
    auto dma_rows = [&](char* stage, int u, const Src& sr, auto is_v) __attribute__((always_inline)) {
        const bool live = u < n_tiles;
        const int key0 = tile_key0(u, sr.j);
        const int nv = tile_valid(key0);
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            LDS_AS char* dst = (LDS_AS char*)(stage) + (is_v.value ? TILEB : 0) + (i * T + wave * 64) * 16;
            uint32_t base;
            if constexpr (MODE == MODE_COLUMN)
                base = (live && dr0 + i * ROWS_PER_DMA < nv) ? static_cast<uint32_t>(sr.kn[i]) * ROWB : kOOB;
            else
                base = live ? static_cast<uint32_t>(key0) * ROWB : kOOB;
            if constexpr (is_v.value)
                dma_load16(rv, lds_addr(dst), base + vslot[i]);
            else
                dma_load16(rk, lds_addr(dst), base + kslot[i]);
        }
    };
    Src sn;  // source of the next tile (one-stage-ring passes)
    init_src(sn);
    auto prefetch_src = [&](int u) __attribute__((always_inline)) { load_src(sn, u); };
    auto dma_tile = [&](char* stage, int u) __attribute__((always_inline)) {
        dma_rows(stage, u, sn, std::false_type{});
        dma_rows(stage, u, sn, std::true_type{});
    };

    // ---- Q operand (registers, whole kernel) -------------------------------
    bf16x8 qreg[DK];
    {
        const int qrow = min(q0 + wave * 32 + l32, L - 1);
        const uint16_t* qp = p.q + (static_cast<size_t>(b) * p.Hq + h) * L * D + static_cast<size_t>(qrow) * D;
#pragma unroll
        for (int st = 0; st < DK; ++st)
            qreg[st] = *reinterpret_cast<const bf16x8*>(qp + 16 * st + 8 * hl);
    }

    // per-lane LDS read offsets inside a stage
    //   K operand (row l32 + 32 kb, unit 2 st + hl)
    int koff[DK];
#pragma unroll
    for (int st = 0; st < DK; ++st) koff[st] = l32 * ROWB + (((2 * st + hl) ^ (l32 & (UNITS - 1))) << 4);
    //   V^T operand by transposing reads: source lane q of 16-lane group g names
    //   key row 4 (g/2) + q/4 (+ 16 m + 8 rd + 32 kb) and the 4 columns
    //   32 db + 16 (g & 1) + 4 (q & 3) ...
    const int gq = lane & 15, gg = lane >> 4;
    int voff[ND];
#pragma unroll
    for (int db = 0; db < ND; ++db) {
        const int u = 2 * (gg & 1) + ((gq & 3) >> 1) + 4 * db;
        const int x = (4 * ((gq >> 2) & 3)) & (UNITS - 1);
        voff[db] = TILEB + (4 * (gg >> 1) + (gq >> 2)) * ROWB + ((u ^ x) << 4) + (gq & 1) * 8;
    }

    f32x16 oacc[ND];
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    // Softmax reference: probabilities are exp2(s c - mc) with mc = m_ref c.
    // m_ref is not the running maximum; it is only raised when a half tile's
    // probabilities sum past kBig in some lane (or when no reference exists
    // yet, mc = -inf, which makes every sum inf or NaN).  Any reference gives
    // the same normalised result; kBig only keeps O and l finite.
    float m_ref = -kInf;
    float mc = -kInf;
    float l_acc = 0.f;
    const float c = p.c;

    auto qk = [&](const char* stg, int kb, f32x16& acc) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int st = 0; st < DK; ++st) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(stg + koff[st] + kb * 32 * ROWB);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[st], acc, 0, 0, 0);
        }
    };
    auto mask = [&](int kb, int nvalid, f32x16& acc) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
            if (key >= nvalid) acc[r] = -kInf;
        }
    };
    // P^T of one 32-key block in bf16 and its fp32 sum in this lane
    auto exps = [&](const f32x16& s, float mcu, uint32_t (&pk)[8]) __attribute__((always_inline)) -> float {
        float pair[8];
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const float p0 = exp2_fast(fmaf(s[r], c, -mcu));
            const float p1 = exp2_fast(fmaf(s[r + 1], c, -mcu));
            pk[r >> 1] = pack_bf16x2(p0, p1);
            pair[r >> 1] = p0 + p1;
        }
        return ((pair[0] + pair[1]) + (pair[2] + pair[3])) + ((pair[4] + pair[5]) + (pair[6] + pair[7]));
    };
    // half H of a 32-key block (accumulator rows 8H .. 8H+7, pk[4H .. 4H+3]);
    // returns their fp32 sum in this lane
    auto exps_half = [&](const f32x16& s, auto H, float mcu, uint32_t (&pk)[8]) __attribute__((always_inline)) -> float {
        float pair[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 8 * H.value + 2 * j;
            const float p0 = exp2_fast(fmaf(s[r], c, -mcu));
            const float p1 = exp2_fast(fmaf(s[r + 1], c, -mcu));
            pk[4 * H.value + j] = pack_bf16x2(p0, p1);
            pair[j] = p0 + p1;
        }
        return (pair[0] + pair[1]) + (pair[2] + pair[3]);
    };
    // raise the reference to this block's maximum, rescale O and l, redo P
    auto rebase = [&](const f32x16& s, uint32_t (&pk)[8]) __attribute__((always_inline)) -> float {
        float mt = -kInf;
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[r]);
        mt = max_with_half_swap(mt);
        if (mt > m_ref) {
            const float alpha = (m_ref > -kInf) ? exp2_fast((m_ref - mt) * c) : 0.f;
            m_ref = mt;
            mc = mt * c;
            l_acc *= alpha;
#pragma unroll
            for (int db = 0; db < ND; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        }
        return exps(s, (m_ref > -kInf) ? mc : 0.f, pk);
    };
    auto softmax = [&](const f32x16& s, uint32_t (&pk)[8]) __attribute__((always_inline)) {
        float ts = exps(s, mc, pk);
        if (__any(!(ts <= kBigSum))) ts = rebase(s, pk);
        l_acc += ts;
    };
    // O^T += V^T P^T; the V^T operand of MFMA (kb, m) over keys
    // 32 kb + 16 m + [0, 16) is two transposing reads (slots 0-3, 4-7)
    auto pv = [&](const char* stg, int kb, const uint32_t (&pk)[8]) __attribute__((always_inline)) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            u32x4 bb = {pk[4 * m], pk[4 * m + 1], pk[4 * m + 2], pk[4 * m + 3]};
#pragma unroll
            for (int db = 0; db < ND; ++db) {
                const int roff = (32 * kb + 16 * m) * ROWB;
                const s16x4 lo = lds_read_tr(stg, voff[db] + roff);
                const s16x4 hi = lds_read_tr(stg, voff[db] + roff + 8 * ROWB);
                const s16x4 a4[2] = {lo, hi};
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a4),
                                                                  __builtin_bit_cast(bf16x8, bb), oacc[db], 0, 0, 0);
            }
        }
    };
    // One tile.  Program order puts independent MFMA and VALU work side by
    // side (QK of block 1 with the softmax of block 0, PV of block 0 with the
    // softmax of block 1) so the scheduler can interleave them.
    auto compute_tile = [&](const char* stg, int nvalid, auto masked, auto checked) __attribute__((always_inline)) {
        f32x16 s0, s1;
        uint32_t pk0[8], pk1[8];
        qk(stg, 0, s0);
        if constexpr (masked.value) mask(0, nvalid, s0);
        if constexpr (KB == 2) {
            qk(stg, 1, s1);
            if constexpr (masked.value) mask(1, nvalid, s1);
        }
        float ts0 = exps(s0, mc, pk0);
        if constexpr (KB == 2 && !masked.value) {
            // K reads four ahead of the QK MFMAs; the softmax of block 0
            // fills the gaps between the MFMAs of block 1
            __builtin_amdgcn_sched_group_barrier(SG_DSR, 4, 0);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                __builtin_amdgcn_sched_group_barrier(SG_DSR, 1, 0);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                if (i < 4) __builtin_amdgcn_sched_group_barrier(SG_DSR, 1, 0);
                __builtin_amdgcn_sched_group_barrier(SG_VALU, 6, 0);
            }
        }
        if constexpr (checked.value)
            if (__any(!(ts0 <= kBigSum))) ts0 = rebase(s0, pk0);
        l_acc += ts0;
        pv(stg, 0, pk0);
        if constexpr (KB == 2) {
            float ts1 = exps(s1, mc, pk1);
            if constexpr (!masked.value) {
                // V^T reads four ahead of the PV MFMAs of block 0, with the
                // softmax of block 1 between them
                __builtin_amdgcn_sched_group_barrier(SG_DSR, 4, 0);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                    if (i < 6) __builtin_amdgcn_sched_group_barrier(SG_DSR, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(SG_VALU, 7, 0);
                }
            }
            if constexpr (checked.value)
                if (__any(!(ts1 <= kBigSum))) ts1 = rebase(s1, pk1);
            l_acc += ts1;
            pv(stg, 1, pk1);
            if constexpr (!masked.value) {
                __builtin_amdgcn_sched_group_barrier(SG_DSR, 4, 0);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                    if (i < 6) __builtin_amdgcn_sched_group_barrier(SG_DSR, 2, 0);
                }
            }
        }
    };
    // One barrier per tile: after it, tile t is in LDS for every wave and every
    // wave has finished tile t-1, whose stage then receives tile t+NST-1 (a
    // DMA is issued every step; past the last tile it reads zeros).
    auto step = [&](int t, int s, auto masked, auto checked) __attribute__((always_inline)) {
        // the DMA (and source prefetch) of tiles t+1 .. t+NST-2 may still be in flight
        wait_vmcnt<(NST - 2) * (2 * NDMA + NPF)>();
        __syncthreads();
        dma_tile(smem + ((s + NST - 1) % NST) * STAGEB, t + NST - 1);
        prefetch_src(t + NST);
        // keep the DMA issue first: it has one tile of compute to land
        __builtin_amdgcn_sched_barrier(0);
        int nvalid = KT;
        if constexpr (masked.value) {
            int J = 0;
            if constexpr (MODE == MODE_BLOCK) J = block_of(t);
            nvalid = tile_valid(tile_key0(t, J));
        }
        compute_tile(smem + s * STAGEB, nvalid, masked, checked);
        __builtin_amdgcn_sched_barrier(0);
    };
    // One pass over the tiles.  Tile 0 is always checked, which sets the
    // reference to its maximum; the other tiles are checked only in a
    // checked pass.
    auto run_pass = [&](auto checked) __attribute__((always_inline)) {
        if (n_tiles == 0) return;
#pragma unroll
        for (int s0 = 0; s0 < NST - 1; ++s0) {
            prefetch_src(s0);
            dma_tile(smem + s0 * STAGEB, s0);
        }
        prefetch_src(NST - 1);
        if (n_full > 0)
            step(0, 0, std::false_type{}, std::true_type{});
        else
            step(0, 0, std::true_type{}, std::true_type{});
        // full tiles, unrolled over the stages so every LDS offset is a
        // constant (t = 1 mod NST throughout)
        int t = 1;
        for (; t + NST <= n_full; t += NST) {
#pragma unroll
            for (int s = 0; s < NST; ++s) step(t + s, (1 + s) % NST, std::false_type{}, checked);
        }
        // the rest (at most NST - 1 full tiles and the partial ones), masked
        for (; t < n_tiles; ++t) step(t, t % NST, std::true_type{}, checked);
        // DMA past the last tile (zeros) and the last prefetch
        __builtin_amdgcn_s_waitcnt(0);
    };
    // Unchecked pass over 64-key tiles, software-pipelined in units: unit t is
    // PV of block 0 of tile t, QK of both blocks of tile t+1, PV of block 1 of
    // tile t, with the softmax of block 1 of tile t and of block 0 of tile
    // t+1 spread over those four MFMA groups.  K and V each use two stages:
    // at unit t's barrier every wave is done with K(t) and V(t-1), so V(t+1)
    // and K(t+2) are fetched into their places.  Tile 0 is computed before
    // the first unit and sets the reference to its maximum; the last tile
    // gets a half unit (its PV and the softmax of its block 1) without the QK
    // of a tile past the end.
    auto run_pass_piped = [&]() __attribute__((always_inline)) {
        const int n = n_tiles;
        Src sv, sk;  // sources of the next V and K fetches
        init_src(sv);
        init_src(sk);
        if constexpr (MODE == MODE_COLUMN) {
            // the column lists of tiles 0 and 1 first, then all three gathers:
            // no gather waits behind another's index load
            Src s1c;
            init_src(s1c);
            load_src(sk, 0);
            load_src(s1c, 1);
            dma_rows(smem, 0, sk, std::false_type{});
            dma_rows(smem + STAGEB, 1, s1c, std::false_type{});
            dma_rows(smem, 0, sk, std::true_type{});
            sv = s1c;
            load_src(sk, 2);
        } else {
            // block form: tile 0 is in the first kept block, and so is tile 1
            // with two tiles per block, so neither DMA waits for an index load
            if constexpr (MODE == MODE_BLOCK)
                sk.j = j_first;
            else
                load_src(sk, 0);
            dma_rows(smem, 0, sk, std::false_type{});
            dma_rows(smem, 0, sk, std::true_type{});
            if constexpr (MODE == MODE_BLOCK) {
                if (sub_shift == 0) load_src(sk, 1);
            } else {
                load_src(sk, 1);
            }
            dma_rows(smem + STAGEB, 1, sk, std::false_type{});
            load_src(sv, 1);
            load_src(sk, 2);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        f32x16 s0, s1;
        uint32_t pk0[8], pk1[8];
        qk(smem, 0, s0);
        qk(smem, 1, s1);
        if (n_full == 0) {
            int J = 0;
            if constexpr (MODE == MODE_BLOCK) J = block_of(0);
            const int nv0 = tile_valid(tile_key0(0, J));
            mask(0, nv0, s0);
            mask(1, nv0, s1);
        }
        {
            float mt = -kInf;
#pragma unroll
            for (int r = 0; r < 16; ++r) mt = fmaxf(mt, fmaxf(s0[r], s1[r]));
            m_ref = max_with_half_swap(mt);
            mc = m_ref * c;
        }
        l_acc += exps_half(s0, std::integral_constant<int, 0>{}, mc, pk0) +
                 exps_half(s0, std::integral_constant<int, 1>{}, mc, pk0);
        // kind: 0 = tile t+1 full; 1 = any (tile t+1 masked to its real keys,
        // none past the last tile, where its K rows are zeros)
        auto unit = [&](int t, auto par, auto kind) __attribute__((always_inline)) {
            wait_vmcnt<0>();
            __syncthreads();
            char* st_t = smem + par * STAGEB;
            char* st_n = smem + (1 - par) * STAGEB;
            int nvn = KT;
            if constexpr (kind.value == 1) nvn = t + 1 < n ? tile_valid(tile_key0(t + 1, sv.j)) : 0;
            dma_rows(st_n, t + 1, sv, std::true_type{});   // V(t+1)
            dma_rows(st_t, t + 2, sk, std::false_type{});  // K(t+2)
            load_src(sv, t + 2);
            load_src(sk, t + 3);
            __builtin_amdgcn_sched_barrier(0);
            constexpr std::integral_constant<int, 0> lo{};
            constexpr std::integral_constant<int, 1> hi{};
            // Each MFMA group is scheduled with a quarter of the softmax work
            // in a region of its own (sched_barrier), which keeps the live
            // ranges in program order.
            auto fence = [&](auto is_pv) __attribute__((always_inline)) {
                if constexpr (kind.value == 0) {
                    __builtin_amdgcn_sched_group_barrier(SG_DSR, 4, 0);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                        if (is_pv.value && i < 6) __builtin_amdgcn_sched_group_barrier(SG_DSR, 2, 0);
                        if (!is_pv.value && i < 4) __builtin_amdgcn_sched_group_barrier(SG_DSR, 1, 0);
                        if (i & 1)
                            __builtin_amdgcn_sched_group_barrier(SG_VALU, 3, 0);
                        else
                            __builtin_amdgcn_sched_group_barrier(SG_VALU, 4, 0);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            };
            pv(st_t, 0, pk0);                                // P0(t)
            const float ta = exps_half(s1, lo, mc, pk1);     // S1a(t)
            fence(std::true_type{});
            {
                f32x16 n0, n1;
                uint32_t q0[8];
                qk(st_n, 0, n0);                             // Q0(t+1)
                const float tb = exps_half(s1, hi, mc, pk1); // S1b(t)
                fence(std::false_type{});
                if constexpr (kind.value == 1) mask(0, nvn, n0);
                qk(st_n, 1, n1);                             // Q1(t+1)
                if constexpr (kind.value == 1) mask(1, nvn, n1);
                const float ua = exps_half(n0, lo, mc, q0);  // S0a(t+1)
                fence(std::false_type{});
                pv(st_t, 1, pk1);                            // P1(t)
                const float ub = exps_half(n0, hi, mc, q0);  // S0b(t+1)
                fence(std::true_type{});
                l_acc += (ta + tb) + (ua + ub);
                s1 = n1;
#pragma unroll
                for (int i = 0; i < 8; ++i) pk0[i] = q0[i];
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        // The last tile: PV of both blocks and the softmax of block 1; there is
        // no next tile to score.
        auto last = [&](auto par) __attribute__((always_inline)) {
            wait_vmcnt<0>();
            __syncthreads();
            char* st_t = smem + par * STAGEB;
            constexpr std::integral_constant<int, 0> lo{};
            constexpr std::integral_constant<int, 1> hi{};
            pv(st_t, 0, pk0);
            const float ta = exps_half(s1, lo, mc, pk1);
            const float tb = exps_half(s1, hi, mc, pk1);
            __builtin_amdgcn_sched_group_barrier(SG_DSR, 4, 0);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                if (i < 6) __builtin_amdgcn_sched_group_barrier(SG_DSR, 2, 0);
                __builtin_amdgcn_sched_group_barrier(SG_VALU, 7, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            pv(st_t, 1, pk1);
            l_acc += ta + tb;
        };
        constexpr std::integral_constant<int, 0> P0{};
        constexpr std::integral_constant<int, 1> P1{};
        constexpr std::integral_constant<int, 0> FULL{};
        constexpr std::integral_constant<int, 1> ANY{};
        int t = 0;
        // units whose next tile is full, in pairs so the stage parity is a constant
        for (; t + 3 <= n_full; t += 2) {
            unit(t, P0, FULL);
            unit(t + 1, P1, FULL);
        }
        if constexpr (MODE == MODE_DENSE) {
            // the rest (at most four units, t even on entry); the last one scores
            // a tile of zeros past the end, masked (one unit in a thousand)
            for (; t < n; t += 2) {
                unit(t, P0, ANY);
                if (t + 1 < n) unit(t + 1, P1, ANY);
            }
        } else {
            // the rest of units 0 .. n-2 (only the last tile can be partial), then
            // the last tile's half unit: short sparse rows feel a wasted unit
            for (; t < n - 1; t += 2) {
                unit(t, P0, ANY);
                if (t + 1 < n - 1) unit(t + 1, P1, ANY);
            }
            if ((n - 1) & 1)
                last(P1);
            else
                last(P0);
        }
        __builtin_amdgcn_s_waitcnt(0);
    };
    // Unchecked pass: probabilities relative to tile 0's maximum are not
    // bounded, so a lane whose row sum leaves [0, 2^32] (including inf and
    // NaN) sends the whole workgroup through a second, checked pass.
    if constexpr (KB == 2) {
        if (n_tiles > 0) run_pass_piped();
    } else {
        run_pass(std::false_type{});
    }
    // one flag per wave and one barrier; the barrier also ends every wave's
    // reads of the stages, which the epilogue reuses
    __shared__ int redo_flag[NW];
    const bool wave_redo = __any(!(l_acc <= kBigRow));
    if (lane == 0) redo_flag[wave] = wave_redo ? 1 : 0;
    __syncthreads();
    int redo = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) redo |= redo_flag[w];
    if (redo) {
        m_ref = -kInf;
        mc = -kInf;
        l_acc = 0.f;
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
        run_pass(std::true_type{});
        __syncthreads();
    }

    // ---- epilogue: normalise, stage through LDS, coalesced stores ----------
    const float lt = sum_with_half_swap(l_acc);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    // Each wave stages its own 32 rows; 16-byte unit u of row r sits at unit
    // u ^ (r mod UNITS), so the column-wise writes spread over the banks and
    // the row-wise reads stay conflict-free.
    char* ob = smem + wave * 32 * OPITCH;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
            // d = 32 db + 8 rq + 4 hl: unit 4 db + rq, half hl
            const int pu = (4 * db + rq) ^ (l32 & (UNITS - 1));
            u32x2 w = {pack_bf16x2(oacc[db][4 * rq] * inv, oacc[db][4 * rq + 1] * inv),
                       pack_bf16x2(oacc[db][4 * rq + 2] * inv, oacc[db][4 * rq + 3] * inv)};
            *reinterpret_cast<u32x2*>(ob + l32 * OPITCH + pu * 16 + hl * 8) = w;
        }
    // only this wave reads these rows back
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const size_t obase = (static_cast<size_t>(b) * p.Hq + h) * L;
    constexpr int CHUNKS = 32 * D * 2 / 16;
#pragma unroll
    for (int i = 0; i < CHUNKS / 64; ++i) {
        const int cid = lane + 64 * i;
        const int row = cid / UNITS, u = cid % UNITS;
        const int qi = q0 + wave * 32 + row;
        if (qi < L) {
            const u32x4 val = *reinterpret_cast<const u32x4*>(ob + row * OPITCH + ((u ^ (row & (UNITS - 1))) << 4));
            *reinterpret_cast<u32x4*>(p.o + (obase + qi) * D + u * 8) = val;
        }
    }
    if (p.lse != nullptr && hl == 0) {
        const int qi = q0 + wave * 32 + l32;
        if (qi < L) p.lse[obase + qi] = lt > 0.f ? m_ref * p.scale + __logf(lt) : -kInf;
    }
}

template <int D, int NW, int KT, int NST, int MODE>
hipError_t launch_one(const FlashParams& fp, hipStream_t st) {
    hipLaunchKernelGGL((flash_fwd_bf16<D, NW, KT, NST, MODE>), dim3(fp.n_items), dim3(NW * 64), 0, st, fp);
    return hipGetLastError();
}

// Query tile of a launch: 64- or 128-query blocks for the block-sparse form,
// 256 queries otherwise.
inline int query_tile(AttnMode mode, const SparseIndex& ix) { return mode == MODE_BLOCK ? ix.block_q : 256; }

// Tile shapes (waves, keys per tile, LDS stages):
//   256-query tiles (dense, column): 8 waves, 64-key tiles, two stages (64 KiB);
//   128-query blocks: 4 waves, 64-key tiles, two stages (64 KiB, two
//   workgroups per CU);
//   64-query blocks: 2 waves, 32-key tiles, two stages (32 KiB).
template <int D>
hipError_t launch_d(AttnMode mode, const FlashParams& fp, int bq, hipStream_t st) {
    switch (mode) {
        case MODE_DENSE: return launch_one<D, 8, 64, 2, MODE_DENSE>(fp, st);
        case MODE_COLUMN: return launch_one<D, 8, 64, 2, MODE_COLUMN>(fp, st);
        case MODE_COLUMN_PACKED: return launch_one<D, 8, 64, 2, MODE_COLUMN_PACKED>(fp, st);
        case MODE_BLOCK:
            if (bq == 64) return launch_one<D, 2, 32, 2, MODE_BLOCK>(fp, st);
            return launch_one<D, 4, 64, 2, MODE_BLOCK>(fp, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_flash_bf16(AttnMode mode, const AttnShape& s, const void* q, const void* k,
                             const void* v, void* o, float* lse, const SparseIndex& ix,
                             hipStream_t st) {
    const int bq = query_tile(mode, ix);
    FlashParams fp{};
    fp.q = static_cast<const uint16_t*>(q);
    fp.k = static_cast<const uint16_t*>(k);
    fp.v = static_cast<const uint16_t*>(v);
    fp.o = static_cast<uint16_t*>(o);
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
    fp.xcd_group = (fp.n_qtiles % 8 == 0) ? fp.n_qtiles : 0;
    fp.scale = s.scale;
    fp.c = s.scale * kLog2e;
    if (fp.n_items == 0) return hipSuccess;
    return s.D == 128 ? launch_d<128>(mode, fp, bq, st) : launch_d<64>(mode, fp, bq, st);
}

}  // namespace sdattn
