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
// each of the NW waves owning 32 query rows.  Per KT-key tile (KT = 64 for
// 256-query tiles and 128-query blocks at d = 64; 32 for 64-query blocks, and
// for 128-query tiles at d = 128, which run three workgroups per CU):
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
    const int32_t* order;  // block form: block row of each workgroup id (a dispatch plan), a split
                           // plan's workspace (split instantiations), or nullptr
    int Hq, Hkv, L, group, n_qtiles, n_items, block_k;
    union {
        int kcol;         // column forms: kept columns per kv head
        int n_pairs;      // block form without a plan: (batch, head) pairs of the balanced order (0: the xcd_group order)
        int split_slots;  // block form over a split plan: its slot count
    };
    int xcd_group;
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

constexpr int gcd_c(int a, int b) { return b ? gcd_c(b, a % b) : a; }
constexpr int lcm_c(int a, int b) { return a / gcd_c(a, b) * b; }

// f(integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time
template <int I, int N, class F>
__device__ __forceinline__ void static_for_from(F& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for_from<I + 1, N>(f);
    }
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_from<0, N>(f);
}

// Block indices and row pointers are read through the constant address
// space: they are uniform and read-only for the kernel's lifetime, so the
// loads become scalar loads (an SGPR result, counted apart from the tile
// DMAs' vector-memory counter).
typedef const __attribute__((address_space(4))) int32_t cint32;

// Balanced grid order of the block form.  Rows of one (batch, head) pair keep
// the same number of kept blocks to within a few, but pairs differ (heads
// concentrate their mass to different extents), and the grid's ids reach the
// eight XCDs round robin (id mod 8).  Ids come in rounds of 8 * n_qtiles: in
// round j, XCD x runs the n_qtiles query blocks of one pair, so each XCD works
// through whole heads and keeps their K/V in its L2.  The pairs are ranked by
// their kept-block totals (the row_ptr difference over their rows) and dealt
// to the XCDs in snake order, largest first: ranks 0..7 to XCDs 0..7 in round
// 0, ranks 8..15 to XCDs 7..0 in round 1, and so on, which evens the XCDs'
// totals and leaves the shortest rows for the last round.  Equal totals are
// ranked so that pair 8j + x still lands on XCD x in round j: with every
// total equal (a top-k budget) the order is the plain one.  n_pairs <= 64
// and a multiple of 8 (one key per lane); returns the same value in every
// lane of the wave.
__device__ __forceinline__ int snake_rank(int pair) {
    const int j = pair >> 3, x = pair & 7;
    return 8 * j + ((j & 1) ? 7 - x : x);
}
__device__ __forceinline__ int balanced_block_item(int id, int n_qtiles, int n_pairs,
                                                   const int32_t* __restrict__ row_ptr, int lane) {
    const int per_round = 8 * n_qtiles;
    const int round = id / per_round;
    const int w = id - round * per_round;
    const int qt = w >> 3;
    const int rank = snake_rank(8 * round + (w & 7));  // this id's rank in the snake
    // key: total << 6 | (63 - snake_rank(pair)): unique, larger total first
    constexpr int kTotalBits = 20;
    const bool valid = lane < n_pairs;
    uint32_t total = 0;
    if (valid) {
        const int lo = row_ptr[lane * n_qtiles];
        const int hi = row_ptr[(lane + 1) * n_qtiles];
        total = static_cast<uint32_t>(min(max(hi - lo, 0), (1 << kTotalBits) - 1));
    }
    uint64_t cand = __ballot(valid);
    // every total equal: the plain order
    const uint32_t t0 = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(total)));
    if ((__ballot(total == t0) & cand) == cand) return (8 * round + (w & 7)) * n_qtiles + qt;
    const uint32_t key = valid ? (total << 6) | static_cast<uint32_t>(63 - snake_rank(lane)) : 0u;
    // the key of rank `rank` (0 = largest), bit by bit from the top over the
    // candidates that share the bits found so far (ballots, no shuffles)
    int k = rank;
#pragma unroll
    for (int b = kTotalBits + 5; b >= 0; --b) {
        const uint64_t ones = __ballot((key >> b) & 1u) & cand;
        const int c = __popcll(ones);
        if (k < c) {
            cand = ones;
        } else {
            k -= c;
            cand &= ~ones;
        }
    }
    const int pair = __ffsll(static_cast<unsigned long long>(cand)) - 1;  // the one lane left
    return pair * n_qtiles + qt;
}

template <int D, int NW, int KT, int NST, int MODE, int NK = NST, int NV = NST, bool SPLIT = false, int WPE = 1>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE))) void flash_fwd_bf16(FlashParams p) {
    // KT keys per tile (32 or 64), NST LDS stages (tiles in flight: NST - 1);
    // the pipelined pass over 32-key tiles uses a ring of NK K slots and NV V
    // slots instead (K fetched NK - 1 units ahead, V NV - 1).  SPLIT: block
    // form over a split plan (p.order is its workspace, launch.h): a
    // workgroup may compute one chunk of a row's kept blocks and write a
    // partial result that split_merge_kernel combines.  WPE: waves per SIMD
    // the register allocation must leave room for (at most 512 / WPE
    // registers per lane).  At three the 32-key block form runs the plain
    // tile loop: the ring pass keeps two tiles' scores and probabilities
    // live and would spill, while the third wave on the SIMD overlaps one
    // wave's softmax with another's MFMAs instead.
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
    // 32-key piped pass: K ring slots 0..NK-1, then V ring slots 0..NV-1
    constexpr bool RING = KT == 32 && MODE == MODE_BLOCK && WPE < 3;
    constexpr int RINGB = (NK + NV) * TILEB;
    constexpr int SMEMB = RING && RINGB > NST * STAGEB ? RINGB : NST * STAGEB;
    static_assert(!RING || (NK >= 2 && NV >= 2 && RINGB >= NST * STAGEB), "ring holds the checked pass's stages");
    // with a K ring of three or more slots the redo flags sit in it, past the
    // epilogue's staging rows, so the shared memory is exactly the ring (see
    // the flag exchange below)
    constexpr int FLAGOFF = NW * 32 * OPITCH;
    constexpr bool FLAGS_IN_RING = RING && FLAGOFF + NW * 4 <= NK * TILEB;

    __shared__ __attribute__((aligned(16))) char smem[SMEMB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // the same value, as a scalar
    const int l32 = lane & 31;
    const int hl = lane >> 5;

    int item;
    int chunk = 0, n_chunks = 1;  // split plan: this workgroup's chunk of its row
    if constexpr (SPLIT) {
        const int raw = ((const cint32*)(p.order))[blockIdx.x];
        if (raw < 0) return;  // idle entry
        item = raw & ((1 << kSplitRowBits) - 1);
        chunk = (raw >> kSplitChunkShift) & (kSplitMaxChunks - 1);
        n_chunks = ((raw >> kSplitCountShift) & (kSplitMaxChunks - 1)) + 1;
        if (item >= p.n_items) return;
    } else if (MODE == MODE_BLOCK && p.order != nullptr) {
        item = ((const cint32*)(p.order))[blockIdx.x];
        if (static_cast<unsigned>(item) >= static_cast<unsigned>(p.n_items)) return;  // not a plan: nothing read
    }
    else if (MODE == MODE_BLOCK && p.n_pairs > 0)
        item = balanced_block_item(blockIdx.x, p.n_qtiles, p.n_pairs, p.row_ptr, lane);
    else
        item = xcd_remap(blockIdx.x, p.n_items, p.xcd_group);
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
    // contiguous tile sources: the descriptor of tile bytes [tb, head_bytes)
    // of the head, so the lanes' offsets within a tile stay fixed and rows
    // past the head's end (all of a tile past the last, tb = head_bytes)
    // read as zero
    // a uniform 64-bit value as two scalar dwords (readfirstlane returns a
    // signed int: each half is taken back to uint32 before widening, so the
    // low half does not sign-extend into the high one)
    auto uniform64 = [](uint64_t x) __attribute__((always_inline)) -> uint64_t {
        const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x >> 32)));
        const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x)));
        return (static_cast<uint64_t>(hi) << 32) | lo;
    };
    const uint64_t kaddr = uniform64(reinterpret_cast<uint64_t>(p.k + kvoff));
    const uint64_t vaddr = uniform64(reinterpret_cast<uint64_t>(p.v + kvoff));
    auto tile_rsrc = [&](uint64_t base, uint32_t tb) __attribute__((always_inline)) -> u32x4 {
        return buffer_rsrc(reinterpret_cast<const void*>(base + tb), head_bytes - tb);
    };
    // LDS address (M0) of this wave's first DMA slot in the shared array
    const uint32_t lds_wave = lds_addr((LDS_AS char*)smem) + static_cast<uint32_t>(wave_u) * 64 * 16;
    const int q0 = qt * (NW * 32);

    // ---- tile source ------------------------------------------------------
    // n_tiles tiles, of which the first n_full hold KT in-range keys; only
    // the end of the sequence (dense), the last kept block of a row (block:
    // rows are ascending) or the end of the column list can be partial.
    int n_tiles = 0, n_full = 0, e0 = 0, ne = 0, sub_shift = 0;
    int j_first = 0;  // block form: the row's first kept block
    int jwin = 0;     // ring pass: lane i holds the row's i-th kept block (rows of at most 64 blocks)
    const int32_t* cb = nullptr;
    if constexpr (MODE == MODE_DENSE) {
        n_tiles = (L + KT - 1) / KT;
        n_full = L / KT;
    } else if constexpr (MODE == MODE_BLOCK) {
        const int r = bh * p.n_qtiles + qt;
        const cint32* rp = (const cint32*)(p.row_ptr);
        e0 = rp[r];
        ne = rp[r + 1] - e0;
        if constexpr (SPLIT) {
            // chunk k of c: kept blocks [floor(k ne / c), floor((k + 1) ne / c)) of the row
            if (n_chunks > 1) {
                const int a = static_cast<int>(static_cast<long long>(ne) * chunk / n_chunks);
                const int z = static_cast<int>(static_cast<long long>(ne) * (chunk + 1) / n_chunks);
                e0 += a;
                ne = z - a;
            }
        }
        // block_k / KT tiles per kept key block (block_k in {64, 128}, KT in {32, 64})
        sub_shift = (p.block_k == 128 ? 1 : 0) + (KT == 32 ? 1 : 0);
        if constexpr (RING) {
            if (ne > 0 && ne <= 64) jwin = p.col_idx[e0 + min(lane, ne - 1)];
        }
        if (ne > 0) {
            // the first and the last kept block, loaded together
            const cint32* cx = (const cint32*)(p.col_idx);
            j_first = cx[e0];
            const int rem = L - cx[e0 + ne - 1] * p.block_k;  // keys of the last block in range
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
        return ((const cint32*)(p.col_idx))[e0 + min(u >> sub_shift, ne - 1)];
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
        if constexpr (MODE == MODE_COLUMN) {
            // gathered rows: each lane's row has its own offset
            const int nv = tile_valid(key0);
#pragma unroll
            for (int i = 0; i < NDMA; ++i) {
                LDS_AS char* dst = (LDS_AS char*)(stage) + (is_v.value ? TILEB : 0) + (i * T + wave * 64) * 16;
                const uint32_t base =
                    (live && dr0 + i * ROWS_PER_DMA < nv) ? static_cast<uint32_t>(sr.kn[i]) * ROWB : kOOB;
                dma_load16(is_v.value ? rv : rk, lds_addr(dst), base + (is_v.value ? vslot[i] : kslot[i]));
            }
        } else {
            const uint32_t m0 = lds_wave + static_cast<uint32_t>((stage - smem) + (is_v.value ? TILEB : 0));
            // a contiguous tile: its start goes into the descriptor, the lanes keep their offsets
            const uint32_t tb = live ? static_cast<uint32_t>(key0) * ROWB : head_bytes;
            const u32x4 r = tile_rsrc(is_v.value ? vaddr : kaddr, tb);
#pragma unroll
            for (int i = 0; i < NDMA; ++i)
                dma_load16(r, m0 + i * T * 16, is_v.value ? vslot[i] : kslot[i]);
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
    // With three waves per SIMD in the plain loop over 32-key tiles, a wave
    // raises its priority while it issues its MFMAs, so the SIMD's arbiter
    // prefers it to the waves in their softmax and the matrix pipe stays fed
    // (results unchanged).
    constexpr bool PRIO = WPE >= 3 && KB == 1;
    auto compute_tile = [&](const char* stg, int nvalid, auto masked, auto checked) __attribute__((always_inline)) {
        f32x16 s0, s1;
        uint32_t pk0[8], pk1[8];
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
        qk(stg, 0, s0);
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
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
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
        pv(stg, 0, pk0);
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
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
    // Unchecked pass over 32-key tiles (64-query blocks), software-pipelined
    // in units through a ring of NK K slots and NV V slots.  Unit t computes
    // QK of tile t+1 beside the second half of tile t's softmax, then PV of
    // tile t beside the first half of tile t+1's.  At unit t's barrier every
    // wave is done with K(t) and V(t-1), so K(t+NK) is fetched into K(t)'s
    // slot and V(t+NV-1) into V(t-1)'s: K arrives NK-1 units ahead of its
    // use, V NV-1.  Tile 0 is scored before the first unit and sets the
    // reference to its maximum; the last tile gets a half unit (the rest of
    // its softmax and its PV).  Block indices come from the row's register
    // window by v_readlane, so the loop issues no memory operation besides
    // the tile DMAs, and each unit waits for exactly the DMAs it needs.
    auto run_pass_ring = [&]() __attribute__((always_inline)) {
        constexpr int U = lcm_c(lcm_c(NK, NV), 2);  // units per unrolled group: every slot offset constant
        // DMAs that may stay in flight at a unit's start: those issued after
        // the later of V(t) (issued NV-1 units earlier, before that unit's K)
        // and K(t+1) (issued NK-1 units earlier)
        constexpr int WAIT = NK > NV ? NDMA * (1 + 2 * (NV - 2)) : 2 * NDMA * (NK - 2);
        static_assert(WAIT < 64, "vmcnt range");
        const int n = n_tiles;
        constexpr std::integral_constant<int, 0> lo{};
        constexpr std::integral_constant<int, 1> hi{};
        auto J = [&](int u) __attribute__((always_inline)) -> int {
            return __builtin_amdgcn_readlane(jwin, min(u >> sub_shift, ne - 1));
        };
        // K (is_v false) or V rows of tile u into the ring slot at byte offset `off`
        // (tiles past the last read as zeros)
        auto dma_ring = [&](int u, int off, auto is_v) __attribute__((always_inline)) {
            const uint32_t tb = u < n ? static_cast<uint32_t>(tile_key0(u, J(u))) * ROWB : head_bytes;
            const u32x4 r = tile_rsrc(is_v.value ? vaddr : kaddr, tb);
            const uint32_t m0 = lds_wave + static_cast<uint32_t>(off);
#pragma unroll
            for (int i = 0; i < NDMA; ++i) dma_load16(r, m0 + i * T * 16, is_v.value ? vslot[i] : kslot[i]);
        };
        auto fence = [&](auto is_pv) __attribute__((always_inline)) {
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
            __builtin_amdgcn_sched_barrier(0);
        };
        // unit t at phase PH = t mod U: (s, pk, ta) hold tile t's scores, the
        // first half of its P and that half's sum; (sn, pkn, tn) receive tile
        // t+1's.  Only the last unit (LASTU) scores the last tile, the one tile
        // that can be partial.
        auto unit = [&](int t, auto PH, auto LASTU, f32x16& s, uint32_t (&pk)[8], float& ta, f32x16& sn,
                        uint32_t (&pkn)[8], float& tn) __attribute__((always_inline)) {
            constexpr int ph = decltype(PH)::value;
            wait_vmcnt<WAIT>();
            __syncthreads();
            dma_ring(t + NV - 1, (NK + (ph + NV - 1) % NV) * TILEB, std::true_type{});  // V(t+NV-1)
            dma_ring(t + NK, (ph % NK) * TILEB, std::false_type{});                    // K(t+NK)
            __builtin_amdgcn_sched_barrier(0);
            qk(smem + ((ph + 1) % NK) * TILEB, 0, sn);  // S(t+1)
            const float tb = exps_half(s, hi, mc, pk);  // P(t), second half
            fence(std::false_type{});
            if constexpr (decltype(LASTU)::value) {
                if (n_full < n) mask(0, tile_valid(tile_key0(t + 1, J(t + 1))), sn);
            }
            pv(smem + (NK + ph % NV) * TILEB - TILEB, 0, pk);  // O += V(t)^T P(t)^T (voff holds the V offset)
            tn = exps_half(sn, lo, mc, pkn);                    // P(t+1), first half
            fence(std::true_type{});
            l_acc += ta + tb;
        };
        auto last = [&](auto PH, f32x16& s, uint32_t (&pk)[8], float& ta) __attribute__((always_inline)) {
            constexpr int ph = decltype(PH)::value;
            wait_vmcnt<WAIT>();
            __syncthreads();
            const float tb = exps_half(s, hi, mc, pk);
            pv(smem + (NK + ph % NV) * TILEB - TILEB, 0, pk);
            l_acc += ta + tb;
        };

        // tile 0's K, then the pseudo-units -(NK-1) .. -1 with the unit's
        // order (V(u+NV-1), K(u+NK)); a V tile before the first goes to its
        // slot as zeros, ahead of the real tile that later fills that slot
        dma_ring(0, 0, std::false_type{});
#pragma unroll
        for (int u = -(NK - 1); u < 0; ++u) {
            const int vt = u + NV - 1;
            dma_ring(vt >= 0 ? vt : n, (NK + ((vt % NV) + NV) % NV) * TILEB, std::true_type{});
            dma_ring(u + NK, ((u + NK) % NK) * TILEB, std::false_type{});
        }
        wait_vmcnt<2 * NDMA * (NK - 1)>();  // K(0) is in; the rest may still be in flight
        __syncthreads();
        f32x16 sa, sb;
        uint32_t pka[8], pkb[8];
        float taa = 0.f, tab = 0.f;
        qk(smem, 0, sa);
        if (n_full == 0) mask(0, tile_valid(tile_key0(0, J(0))), sa);
        {
            float mt = -kInf;
#pragma unroll
            for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sa[r]);
            m_ref = max_with_half_swap(mt);
            mc = m_ref * c;
        }
        taa = exps_half(sa, lo, mc, pka);
        // units 0 .. n-2 in groups of U, the state alternating between a and b
        constexpr std::false_type MID{};
        constexpr std::true_type LASTU{};
        auto unit_at = [&](int t0, auto PH, auto is_last) __attribute__((always_inline)) {
            constexpr int ph = decltype(PH)::value;
            if constexpr (ph % 2 == 0)
                unit(t0 + ph, PH, is_last, sa, pka, taa, sb, pkb, tab);
            else
                unit(t0 + ph, PH, is_last, sb, pkb, tab, sa, pka, taa);
        };
        const int nu = n - 1;
        int t = 0;
        // groups of U units that hold neither the last unit nor the last tile
        for (; t + U < nu; t += U)
            static_for<U>([&](auto PH) __attribute__((always_inline)) { unit_at(t, PH, MID); });
        // the remaining r units (1 <= r <= U, or none for a one-tile row): phases
        // 0 .. r-2, the last unit at phase r-1, then the last tile's half unit
        auto tail = [&](auto R) __attribute__((always_inline)) {
            constexpr int rr = decltype(R)::value;
            if constexpr (rr >= 1) {
                static_for<rr - 1>([&](auto PH) __attribute__((always_inline)) { unit_at(t, PH, MID); });
                unit_at(t, std::integral_constant<int, rr - 1>{}, LASTU);
            }
            constexpr std::integral_constant<int, rr % U> PL{};
            if constexpr (rr % 2 == 0)
                last(PL, sa, pka, taa);
            else
                last(PL, sb, pkb, tab);
        };
        const int r = nu - t;
        static_for<U + 1>([&](auto R) __attribute__((always_inline)) {
            if (r == decltype(R)::value) tail(R);
        });
        __builtin_amdgcn_s_waitcnt(0);  // K fetches past the last tile
    };
    // Unchecked pass: probabilities relative to tile 0's maximum are not
    // bounded, so a lane whose row sum leaves [0, 2^32] (including inf and
    // NaN) sends the whole workgroup through a second, checked pass.
    if constexpr (KB == 2) {
        if (n_tiles > 0) run_pass_piped();
    } else if constexpr (RING) {
        if (n_tiles > 0) {
            if (ne <= 64) {
                run_pass_ring();
            } else {
                run_pass(std::false_type{});
                // the flags below may sit in a stage another wave still reads
                if constexpr (FLAGS_IN_RING) __syncthreads();
            }
        }
    } else {
        run_pass(std::false_type{});
    }
    // one flag per wave and one barrier; the barrier also ends every wave's
    // reads of the stages, which the epilogue reuses.  With a deep enough K
    // ring the flags live in it, past the epilogue's staging rows: every read
    // of the K slots and every DMA has ended before a flag is written, and
    // the epilogue's staging does not reach them.
    int* redo_flag;
    if constexpr (FLAGS_IN_RING) {
        redo_flag = reinterpret_cast<int*>(smem + FLAGOFF);
    } else {
        __shared__ int flags[NW];
        redo_flag = flags;
    }
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
        if constexpr (FLAGS_IN_RING) __syncthreads();  // every wave has read the flags before the DMAs
        run_pass(std::true_type{});
        __syncthreads();
    }

    // ---- epilogue: normalise, stage through LDS, coalesced stores ----------
    const float lt = sum_with_half_swap(l_acc);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if constexpr (SPLIT) {
        if (n_chunks > 1) {
            // one chunk of a split row: O over the chunk, normalised, in the
            // accumulator layout (16-byte unit (wave, db, rq) of lane `lane`),
            // and the chunk's log-sum-exp per query, into its partial slot
            const int rows = p.n_items, slots = p.split_slots;
            const cint32* ws = (const cint32*)(p.order);
            const int slot = ws[split_slot_base_offset(rows, slots) + item] + chunk;
            constexpr int BQ = NW * 32;
            float* part = reinterpret_cast<float*>(const_cast<int32_t*>(p.order) + split_partial_offset(rows, slots)) +
                          static_cast<size_t>(slot) * BQ * (D + 1);
#pragma unroll
            for (int db = 0; db < ND; ++db)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    const f32x4 val = {oacc[db][4 * rq] * inv, oacc[db][4 * rq + 1] * inv, oacc[db][4 * rq + 2] * inv,
                                       oacc[db][4 * rq + 3] * inv};
                    reinterpret_cast<f32x4*>(part)[((wave * ND + db) * 4 + rq) * 64 + lane] = val;
                }
            if (hl == 0) part[BQ * D + wave * 32 + l32] = lt > 0.f ? m_ref * p.scale + __logf(lt) : -kInf;
            return;
        }
    }
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
    // the wave's 32 output rows through one buffer descriptor: chunk cid sits
    // at byte 16 cid of them, and rows past the sequence's end fall outside
    // the descriptor's range, so the hardware drops those stores
    const int qw0 = q0 + wave_u * 32;
    const uint64_t obytes = uniform64(reinterpret_cast<uint64_t>(p.o + (obase + qw0) * D));
    const int orange = __builtin_amdgcn_readfirstlane(max(0, min(32, L - qw0)) * ROWB);
    const __amdgpu_buffer_rsrc_t rso = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>(obytes), static_cast<short>(0), orange, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < CHUNKS / 64; ++i) {
        const int cid = lane + 64 * i;
        const int row = cid / UNITS, u = cid % UNITS;
        const u32x4 val = *reinterpret_cast<const u32x4*>(ob + row * OPITCH + ((u ^ (row & (UNITS - 1))) << 4));
        __builtin_amdgcn_raw_buffer_store_b128(val, rso, cid * 16, 0, 0);
    }
    if (p.lse != nullptr && hl == 0) {
        const int qi = q0 + wave * 32 + l32;
        if (qi < L) p.lse[obase + qi] = lt > 0.f ? m_ref * p.scale + __logf(lt) : -kInf;
    }
}

// Merge of split rows (split plan, launch.h): workgroup s combines the c
// chunks of the s-th split row, with NW * 64 threads per 32 channels (one
// group of waves per db).  Each thread takes the 16-byte units of the
// accumulator layout that the forward's lane of the same wave and lane wrote
// (query 32 wave + lane mod 32, channels 32 db + 8 rq + 4 (lane / 32) +
// [0, 4)), weights chunk k by exp(lse_k - LSE), LSE = log sum_k exp(lse_k)
// (the online-softmax merge of partial rows), and writes O in bf16; the
// db = 0 threads write LSE.  For each unit the c chunks' loads are issued
// before any is used, so they are in flight together.
struct MergeParams {
    const int32_t* ws;
    uint16_t* o;
    float* lse;
    int Hq, L, n_qtiles, rows, slots;
};

template <int D, int NW>
__global__ __launch_bounds__(NW * 64 * (D / 32)) void split_merge_kernel(MergeParams m) {
    constexpr int ND = D / 32;
    constexpr int BQ = NW * 32;
    constexpr size_t SLOT = static_cast<size_t>(BQ) * (D + 1);  // floats per partial slot
    const int s = blockIdx.x;
    const int db = threadIdx.x / (NW * 64);
    const int32_t* ws = m.ws;
    if (s >= ws[split_counts_offset(m.rows, m.slots)]) return;
    const int raw = ws[split_rows_offset(m.rows, m.slots) + s];
    const int row = raw & ((1 << kSplitRowBits) - 1);
    const int c = ((raw >> kSplitCountShift) & (kSplitMaxChunks - 1)) + 1;
    const int slot0 = ws[split_slot_base_offset(m.rows, m.slots) + row];
    const float* part = reinterpret_cast<const float*>(ws + split_partial_offset(m.rows, m.slots)) + slot0 * SLOT;
    const int lane = threadIdx.x & 63, wave = (threadIdx.x >> 6) % NW;
    const int l32 = lane & 31, hl = lane >> 5;
    const int qq = wave * 32 + l32;
    const int bh = row / m.n_qtiles, qt = row - bh * m.n_qtiles;
    const int qi = qt * BQ + qq;
    if (qi >= m.L) return;
    float lk[kSplitMaxChunks];
#pragma unroll
    for (int k = 0; k < kSplitMaxChunks; ++k) lk[k] = k < c ? part[k * SLOT + BQ * D + qq] : -kInf;
    float mx = -kInf;
#pragma unroll
    for (int k = 0; k < kSplitMaxChunks; ++k) mx = fmaxf(mx, lk[k]);
    float w[kSplitMaxChunks];
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < kSplitMaxChunks; ++k) {
        w[k] = (k < c && lk[k] > -kInf) ? __expf(lk[k] - mx) : 0.f;
        sum += w[k];
    }
    const float inv = sum > 0.f ? 1.f / sum : 0.f;
    uint16_t* orow = m.o + (static_cast<size_t>(bh) * m.L + qi) * D;
#pragma unroll 1
    for (int rq = 0; rq < 4; ++rq) {
        f32x4 v[kSplitMaxChunks];
#pragma unroll
        for (int k = 0; k < kSplitMaxChunks; ++k)
            if (k < c) v[k] = reinterpret_cast<const f32x4*>(part + k * SLOT)[((wave * ND + db) * 4 + rq) * 64 + lane];
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < kSplitMaxChunks; ++k)
            if (k < c) acc += v[k] * (w[k] * inv);
        const u32x2 out = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
        *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * rq + 4 * hl) = out;
    }
    if (db == 0 && m.lse != nullptr && hl == 0)
        m.lse[static_cast<size_t>(bh) * m.L + qi] = sum > 0.f ? mx + __logf(sum) : -kInf;
}

template <int D, int NW, int KT, int NST, int MODE, int NK = NST, int NV = NST, bool SPLIT = false, int WPE = 1>
hipError_t launch_one(const FlashParams& fp, hipStream_t st, int grid) {
    hipLaunchKernelGGL((flash_fwd_bf16<D, NW, KT, NST, MODE, NK, NV, SPLIT, WPE>), dim3(grid), dim3(NW * 64), 0, st, fp);
    return hipGetLastError();
}

// K and V ring slots of the 64-query block form's pipelined pass: K fetched
// two units ahead, V one; five 8 KiB slots (d = 128) fill the 160 KiB of LDS
// with four workgroups per CU.
constexpr int kRingK = 3, kRingV = 2;

// Column lists of at most this many keys take the 128-query column form at
// d = 128 (three workgroups per CU): a short list leaves each workgroup few
// tiles, and a third workgroup hides one's Q load and O stores behind the
// others' tiles.  Longer lists keep the 256-query form, whose K/V tiles feed
// twice the queries (measured on the 16K GQA shape: 64 and 492 columns 20%
// and 13% faster in the 128-query form, 2048 columns within 1%).
constexpr int kColumnShortList = 1024;

// Query tile of a launch: 64- or 128-query blocks for the block-sparse form;
// 128 queries for short column lists at d = 128; 256 queries otherwise.
inline int query_tile(AttnMode mode, const AttnShape& s, const SparseIndex& ix) {
    if (mode == MODE_BLOCK) return ix.block_q;
    if ((mode == MODE_COLUMN || mode == MODE_COLUMN_PACKED) && s.D == 128 && ix.kcol <= kColumnShortList) return 128;
    return 256;
}

}  // namespace

// Workgroups of the block-sparse form that share one CU (LDS and registers):
// four of the 40 KiB 64-query form; three of the 128-query form (d = 128:
// 32 KiB and at most 168 registers, three waves per SIMD; d = 64: 32 KiB
// and 164 registers).
int block_rows_per_cu(int block_q) { return block_q == 64 ? 4 : 3; }

namespace {

// Tile shapes (waves, keys per tile, LDS stages):
//   256-query tiles (dense, long column lists): 8 waves, 64-key tiles, two
//   stages (64 KiB);
//   128-query tiles of short column lists at d = 128: as the 128-query
//   blocks below;
//   128-query blocks, d = 128: 4 waves, 32-key tiles, two stages (32 KiB),
//   the plain tile loop in at most 168 registers, so three workgroups share
//   a CU with three waves per SIMD (faster than 64-key tiles pipelined in
//   253 registers with two workgroups per CU);
//   128-query blocks, d = 64: 4 waves, 64-key tiles, two stages (32 KiB, 164
//   registers: three workgroups per CU);
//   64-query blocks: 2 waves, 32-key tiles through a ring of kRingK K and
//   kRingV V slots (40 KiB at d = 128, four workgroups per CU).
template <int D>
hipError_t launch_d(AttnMode mode, const FlashParams& fp, int bq, hipStream_t st) {
    const int g = fp.n_items;
    switch (mode) {
        case MODE_DENSE: return launch_one<D, 8, 64, 2, MODE_DENSE>(fp, st, g);
        case MODE_COLUMN:
            if constexpr (D == 128)
                if (bq == 128) return launch_one<D, 4, 32, 2, MODE_COLUMN, 2, 2, false, 3>(fp, st, g);
            return launch_one<D, 8, 64, 2, MODE_COLUMN>(fp, st, g);
        case MODE_COLUMN_PACKED:
            if constexpr (D == 128)
                if (bq == 128) return launch_one<D, 4, 32, 2, MODE_COLUMN_PACKED, 2, 2, false, 3>(fp, st, g);
            return launch_one<D, 8, 64, 2, MODE_COLUMN_PACKED>(fp, st, g);
        case MODE_BLOCK:
            if (bq == 64) return launch_one<D, 2, 32, 2, MODE_BLOCK, kRingK, kRingV>(fp, st, g);
            if constexpr (D == 128)
                return launch_one<D, 4, 32, 2, MODE_BLOCK, 2, 2, false, 3>(fp, st, g);
            else
                return launch_one<D, 4, 64, 2, MODE_BLOCK>(fp, st, g);
    }
    return hipErrorInvalidValue;
}

// Block form over a split plan: the forward over its items (rows + 2 slots
// workgroups), then the merge of the split rows (slots workgroups, the idle
// ones return at once).
template <int D>
hipError_t launch_split_d(const FlashParams& fp, int bq, hipStream_t st) {
    const int slots = fp.split_slots;
    const int grid = static_cast<int>(split_items(fp.n_items, slots));
    MergeParams m{fp.order, fp.o, fp.lse, fp.Hq, fp.L, fp.n_qtiles, fp.n_items, slots};
    hipError_t e;
    if (bq == 64) {
        e = launch_one<D, 2, 32, 2, MODE_BLOCK, kRingK, kRingV, true>(fp, st, grid);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((split_merge_kernel<D, 2>), dim3(slots), dim3(128 * (D / 32)), 0, st, m);
    } else {
        // the same tile shape as the unsplit forward, so a row that is not cut
        // gets the same arithmetic
        if constexpr (D == 128)
            e = launch_one<D, 4, 32, 2, MODE_BLOCK, 2, 2, true, 3>(fp, st, grid);
        else
            e = launch_one<D, 4, 64, 2, MODE_BLOCK, 2, 2, true>(fp, st, grid);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((split_merge_kernel<D, 4>), dim3(slots), dim3(256 * (D / 32)), 0, st, m);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_flash_bf16(AttnMode mode, const AttnShape& s, const void* q, const void* k,
                             const void* v, void* o, float* lse, const SparseIndex& ix,
                             hipStream_t st) {
    const int bq = query_tile(mode, s, ix);
    FlashParams fp{};
    fp.q = static_cast<const uint16_t*>(q);
    fp.k = static_cast<const uint16_t*>(k);
    fp.v = static_cast<const uint16_t*>(v);
    fp.o = static_cast<uint16_t*>(o);
    fp.lse = lse;
    fp.row_ptr = ix.row_ptr;
    fp.col_idx = ix.col_idx;
    fp.order = mode == MODE_BLOCK ? (ix.split != nullptr ? ix.split : ix.order) : nullptr;
    fp.Hq = s.Hq;
    fp.Hkv = s.Hkv;
    fp.L = s.L;
    fp.group = s.Hq / s.Hkv;
    fp.n_qtiles = (s.L + bq - 1) / bq;
    fp.n_items = s.B * s.Hq * fp.n_qtiles;
    fp.block_k = ix.block_k;
    // XCD-aware order: the block form gives each XCD whole heads (eight heads
    // per group of 8 * n_qtiles ids), so the rows in flight on an XCD share one
    // head's K/V in its L2; the other forms give each XCD a contiguous run of
    // every head's query tiles
    if (mode == MODE_BLOCK && static_cast<long long>(fp.n_items) % (8LL * fp.n_qtiles) == 0)
        fp.xcd_group = 8 * fp.n_qtiles;
    else
        fp.xcd_group = (fp.n_qtiles % 8 == 0) ? fp.n_qtiles : 0;
    // block form: up to 64 (batch, head) pairs in whole rounds of eight are
    // ranked by their kept blocks and dealt to the XCDs evenly
    // (balanced_block_item).  The pair count shares kcol's slot: with one
    // more field in the parameters the dense launch's L2-to-fabric reads
    // tripled (same instructions, same time)
    if (mode == MODE_BLOCK) {
        const int n_pairs = s.B * s.Hq;
        fp.n_pairs = (n_pairs % 8 == 0 && n_pairs <= 64) ? n_pairs : 0;
    } else {
        fp.kcol = ix.kcol;
    }
    fp.scale = s.scale;
    fp.c = s.scale * kLog2e;
    if (fp.n_items == 0) return hipSuccess;
    if (mode == MODE_BLOCK && ix.split != nullptr) {
        fp.split_slots = split_slots(bq);
        return s.D == 128 ? launch_split_d<128>(fp, bq, st) : launch_split_d<64>(fp, bq, st);
    }
    return s.D == 128 ? launch_d<128>(mode, fp, bq, st) : launch_d<64>(mode, fp, bq, st);
}

}  // namespace sdattn
