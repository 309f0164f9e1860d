// Routing layout on gfx950: top-k expert indices -> per-expert and per-group
// counts, prefix offsets and stable receive slots, with no global atomics.
//
// What it computes follows "perf(ep): optimize IntraNode dispatch kernel for
// MI350X" (ROCm/mori pull request 586): the count / reserve phases of its
// dispatch (Motivation; per-destination dedup with destination = expert /
// experts-per-rank) and the cached per-pair destination that dispatch and
// combine reuse (Technical Details 1). That page measured a single-pass
// variant with per-token atomics as slower, found no wave64 match intrinsic
// for token-level dedup on gfx950, and proposed computing the routing in a
// launch of its own ("Approaches tested"). This file is that launch, built
// for wave64 without atomics on global memory:
//
// The tokens are cut into tiles of 256 (one per thread of a 256-thread
// workgroup = 4 waves). For each tile, LDS holds one 64-bit word per
// (expert, wave): bit `lane` is set when that lane's token lists the expert.
// The words are built with LDS atomic ORs, whose result does not depend on
// their order, so
//   rank of (t, k) inside the tile = popcount of the expert's words of earlier
//   waves + popcount(word of its own wave & lanes below it),
// which is the stable token-ascending order, and a token repeats an expert
// iff one of its earlier entries names it. Groups use one ballot per group per
// wave, which gives the same kind of word per (group, wave).
//
// Kernel 1 (count): per tile, expert and group counts + error bits -> one row
// of a tile-major table in the workspace; for top-k <= 8 also the tile's
// expert and group words.
// Kernel 2 (place, moe_layout): every tile reads the table column-wise (tiny:
// (E+G+1) x tiles ints, coalesced), forms global offsets = exclusive prefix
// over experts of the totals + prefix over earlier tiles, takes its words
// (loaded, or rebuilt for top-k > 8) and writes the slots and receive-source
// lists. Tile 0 also writes the counts, offsets and status.
// Kernel 2' (finalize, the fused layout + dispatch): one workgroup computes the
// counts, offsets and status once and a base per (tile, column), from which
// each dispatch workgroup places its own token (place.hpp).
// One launch instead: up to 128 tiles exchange their counts through a table in
// library memory (layout_exchange.hip, top-k <= 8); where no table can be used
// (graph capture, more streams than tables), with top-k <= 8 and T * K <=
// 16384, each tile's workgroup counts all tokens itself (see
// layout_onepass_kernel).
// Global loads are issued ahead of their first use, so each kernel
// costs about one memory round trip plus its LDS work; the stores are shaped
// so that a wave's store touches few cache lines (a token's slot row as one
// or two 16-byte stores, the tile's expert receive list as per-expert runs
// staged in LDS), since scattered 4-byte stores cost one line each.
#include "moe_ep.h"

#include "layout_tile.hpp"

namespace moe {

namespace {

// Count kernel: one tile per workgroup. Writes row `tile` of the tile-major
// count table: E expert counts, G group counts, then the tile's error bits;
// for top-k <= 8 also the tile's E x 4 expert words and G x 4 group words
// (as 32-bit halves), which the place kernel, or a dispatch kernel placing
// its own token, loads instead of rebuilding them.
template <int KMAX, bool EXACT>
__global__ __launch_bounds__(kLayoutTile) void layout_count_kernel(
    const int32_t *__restrict__ idx, int T, int Krt, int E, int G, uint32_t gmagic,
    uint32_t *__restrict__ tok_group_mask, int32_t *__restrict__ table, uint32_t *__restrict__ words,
    uint32_t *__restrict__ gwords, int32_t *__restrict__ clear_bases, int32_t *__restrict__ clear_status)
{
    extern __shared__ unsigned long long emask[];   // [E][kWaves]
    __shared__ int gcnt[kMaxG][kWaves];
    __shared__ unsigned long long gball[kMaxG][kWaves];
    __shared__ int s_err;
    const int K = EXACT ? KMAX : Krt;   // a compile-time constant for the common top-k
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int tile = blockIdx.x;
    const int t = tile * kLayoutTile + tid;
    int e[KMAX];
    load_row<KMAX>(idx, t, T, K, e);
    for (int i = tid; i < E * kWaves; i += kLayoutTile) emask[i] = 0ull;
    if (tid == 0) s_err = 0;
    __syncthreads();
    mask_row<KMAX>(t, T, K, e);

    const Inserted ins = insert_token<KMAX>(e, t < T, K, E, gmagic, emask, wave, lane);
    const uint32_t gm = ins.gm;
    const int err = ins.err();
    if (t < T) tok_group_mask[t] = gm;
    for (int g = 0; g < G; ++g) {
        const uint64_t b = __ballot((gm >> g) & 1u);
        if (lane == 0) {
            gcnt[g][wave] = __popcll(b);
            gball[g][wave] = b;
        }
    }
    if (err) atomicOr(&s_err, err);
    __syncthreads();

    int32_t *row = table + (size_t)tile * (E + G + 1);
    for (int x = tid; x < E; x += kLayoutTile) {
        const unsigned long long *m = emask + x * kWaves;
        row[x] = __popcll(m[0]) + __popcll(m[1]) + __popcll(m[2]) + __popcll(m[3]);
    }
    if (tid < G) row[E + tid] = gcnt[tid][0] + gcnt[tid][1] + gcnt[tid][2] + gcnt[tid][3];
    if (tid == 0) row[E + G] = s_err;
    if (clear_bases) {   // fused path: the tile's bases are not yet known
        for (int x = tid; x < E + G; x += kLayoutTile) clear_bases[(size_t)tile * (E + G) + x] = -1;
        if (tile == 0 && tid == 0) *clear_status = 0;
    }
    if constexpr (KMAX <= 8) {
        uint32_t *wt = words + (size_t)tile * E * kWaves * 2;
        for (int i = tid; i < E * kWaves; i += kLayoutTile) {
            const unsigned long long w = emask[i];
            wt[2 * i] = (uint32_t)w;
            wt[2 * i + 1] = (uint32_t)(w >> 32);
        }
        if (tid < G * kWaves) {
            const unsigned long long w = gball[tid / kWaves][tid % kWaves];
            uint32_t *gt = gwords + (size_t)tile * G * kWaves * 2;
            gt[2 * tid] = (uint32_t)w;
            gt[2 * tid + 1] = (uint32_t)(w >> 32);
        }
    }
}

// A token's slot_tg row (four groups per store where the array allows) and
// its group receive-list entries.
__device__ __forceinline__ void token_group_entries(int t, int T, int K, int G, int wave, uint64_t below,
                                                    uint32_t gm, const int (*off_g)[kWaves],
                                                    const uint64_t (*gball)[kWaves], const LayoutPtrs &L,
                                                    int vec)
{
    int32_t *tg = L.slot_tg + (size_t)t * G;
    for (int g0 = 0; g0 < G; g0 += 4) {
        int s4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int g = g0 + u;
            s4[u] = -1;
            if (g < G && ((gm >> g) & 1u)) {
                s4[u] = off_g[g][wave] + __popcll(gball[g][wave] & below);
                L.recv_src_g[s4[u]] = t;
            }
        }
        if (vec & 2) {   // G % 4 == 0 and slot_tg 16-byte aligned
            *reinterpret_cast<u32x4 *>(tg + g0) = u32x4{(uint32_t)s4[0], (uint32_t)s4[1], (uint32_t)s4[2], (uint32_t)s4[3]};
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (g0 + u < G) tg[g0 + u] = s4[u];
        }
    }
}

// A token's layout entries from its tile's words and per-(column, wave)
// offsets (top-k <= 8; lane `lane` of wave `wave` holds token t < T with
// entries e, groups gm and non-counting entries bad): its slot_e / slot_g row,
// its slot_tg row and its group receive-list entries; its expert
// receive-list entries are staged in slot order (s_src, s_dst) for the caller
// to write as runs.
template <int KMAX, bool EXACT>
__device__ __forceinline__ void tile_token_entries(
    int t, int T, int K, int G, uint32_t gmagic, int wave, int lane, const int (&e)[KMAX], uint32_t gm,
    uint32_t bad, const unsigned long long *emask, const int *off_e, const int *ldelta,
    const int (*off_g)[kWaves], const uint64_t (*gball)[kWaves], int32_t *s_src, int32_t *s_dst,
    const LayoutPtrs &L, int vec)
{
    const uint64_t below = lanemask_lt(lane);
    const size_t p0 = (size_t)t * K;
    int se[KMAX], sg[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        se[k] = sg[k] = -1;
        if (k < K && !((bad >> k) & 1u)) {
            const int x = e[k];
            se[k] = off_e[x * kWaves + wave] + __popcll(emask[x * kWaves + wave] & below);
            const int g = group_of(x, gmagic);
            sg[k] = off_g[g][wave] + __popcll(gball[g][wave] & below);
            const int li = se[k] + ldelta[x];
            s_src[li] = (int32_t)(p0 + k);
            s_dst[li] = se[k];
        }
    }
    if (EXACT && (vec & 1)) {   // 16-byte aligned slot arrays, K in {2, 4, 8}
        if constexpr (KMAX == 2) {
            *reinterpret_cast<u32x2 *>(L.slot_e + p0) = u32x2{(uint32_t)se[0], (uint32_t)se[1]};
            *reinterpret_cast<u32x2 *>(L.slot_g + p0) = u32x2{(uint32_t)sg[0], (uint32_t)sg[1]};
        } else {
#pragma unroll
            for (int k = 0; k < KMAX; k += 4) {
                *reinterpret_cast<u32x4 *>(L.slot_e + p0 + k) =
                    u32x4{(uint32_t)se[k], (uint32_t)se[k + 1], (uint32_t)se[k + 2], (uint32_t)se[k + 3]};
                *reinterpret_cast<u32x4 *>(L.slot_g + p0 + k) =
                    u32x4{(uint32_t)sg[k], (uint32_t)sg[k + 1], (uint32_t)sg[k + 2], (uint32_t)sg[k + 3]};
            }
        }
    } else {
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (k < K) {
                L.slot_e[p0 + k] = se[k];
                L.slot_g[p0 + k] = sg[k];
            }
        }
    }
    token_group_entries(t, T, K, G, wave, below, gm, off_g, gball, L, vec);
}

// Sum of table column `col` over tiles, and over the tiles before `tile`.
// The first kBatch tiles' entries are loaded by the caller (together with its
// other loads, so they share one memory round trip); later tiles are loaded
// kBatch at a time here.
constexpr int kBatch = 16;

// Loads of a column's first kBatch entries, unconditional and from clamped
// in-range addresses (`col` < rows, ntiles >= 1); the caller masks the sums,
// not the loads, so that the compiler keeps them out of lane-dependent
// branches (a predicated load costs a branch and a wait of its own).
__device__ __forceinline__ void column_first(const int32_t *__restrict__ table, int rows, int col,
                                             int ntiles, int (&c)[kBatch])
{
    const int32_t *colp = table + col;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) c[u] = colp[(size_t)(u < ntiles ? u : ntiles - 1) * rows];
}

__device__ __forceinline__ void column_sums(const int32_t *__restrict__ table, int rows, int col,
                                            int ntiles, int tile, const int (&first)[kBatch],
                                            int &tot, int &pre)
{
    tot = 0;
    pre = 0;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
        tot += u < ntiles ? first[u] : 0;
        pre += u < tile ? first[u] : 0;
    }
    for (int b0 = kBatch; b0 < ntiles; b0 += 16) {
        int c[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) c[u] = (b0 + u < ntiles) ? table[(size_t)(b0 + u) * rows + col] : 0;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            tot += c[u];
            pre += (b0 + u < tile) ? c[u] : 0;
        }
    }
}

// Place kernel: one tile per workgroup. Global offsets of the tile = exclusive
// prefix over experts of the totals + prefix over earlier tiles (read from
// the table, coalesced: thread x reads column x); then the tile's LDS words
// are rebuilt exactly as the count kernel built them, and each pair's slot is
// its expert's offset for this (tile, wave) plus its rank among the wave's
// lanes. Experts are owned in NCH chunks of 256 (x = chunk * 256 + tid):
// NCH = 1 for E <= 256 keeps the code and its registers to one chunk.
template <int KMAX, bool EXACT, int NCH>
__global__ __launch_bounds__(kLayoutTile) void layout_place_kernel(
    const int32_t *__restrict__ idx, int T, int Krt, int E, int G, uint32_t gmagic,
    int ntiles, const int32_t *__restrict__ table, const uint32_t *__restrict__ words, LayoutPtrs L,
    int vec)
{
    // For top-k <= 8 the tile's receive-list entries are staged in LDS in slot
    // order and written out as contiguous runs (one run per expert) instead of
    // one scattered 4-byte store per pair.
    constexpr bool kStage = KMAX <= 8;
    extern __shared__ unsigned long long emask[];   // [E][kWaves], int off_e[E][kWaves], int ldelta[E]
    int *off_e = reinterpret_cast<int *>(emask + E * kWaves);
    int *ldelta = off_e + E * kWaves;   // tile-local position of expert x's pairs minus their global base
    __shared__ int32_t s_src[kStage ? kLayoutTile * KMAX : 1];   // staged pair ids, slot order
    __shared__ int32_t s_dst[kStage ? kLayoutTile * KMAX : 1];   // and their receive slots
    __shared__ int s_wave_tot[kWaves];
    __shared__ int base_g[kMaxG];
    __shared__ int tot_g[kMaxG];
    __shared__ int off_g[kMaxG][kWaves];
    __shared__ uint64_t gball[kMaxG][kWaves];
    __shared__ int s_err;
    const int K = EXACT ? KMAX : Krt;   // a compile-time constant for the common top-k
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int tile = blockIdx.x;
    const int t = tile * kLayoutTile + tid;
    const int rows = E + G + 1;

    // All global loads first (table columns, the tile's tokens, its words), so
    // that they share one memory round trip: nothing below consumes them
    // before the scheduling barrier.
    int c0[NCH][kBatch], cg0[kBatch];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const int x = j * kLayoutTile + tid;
        if (j * kLayoutTile < E)   // uniform
            column_first(table, rows, x < E ? x : E - 1, ntiles, c0[j]);
    }
    column_first(table, rows, E + (tid < G ? tid : G - 1), ntiles, cg0);
    const int er_v = table[(size_t)(tid < ntiles ? tid : ntiles - 1) * rows + E + G];
    int e[KMAX];
    load_row<KMAX>(idx, t, T, K, e);
    // the tile's words from the count kernel (top-k <= 8)
    constexpr int kWordsPerThread = NCH * kWaves;
    uint32_t wlo[kStage ? kWordsPerThread : 1], whi[kStage ? kWordsPerThread : 1];
    if constexpr (kStage) {
        const uint32_t *wt = words + (size_t)tile * E * kWaves * 2;
#pragma unroll
        for (int u = 0; u < kWordsPerThread; ++u) {
            wlo[u] = whi[u] = 0;
            if (u * kLayoutTile < E * kWaves) {   // uniform
                const int i = u * kLayoutTile + tid;
                const int ic = i < E * kWaves ? i : E * kWaves - 1;
                wlo[u] = wt[2 * ic];
                whi[u] = wt[2 * ic + 1];
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    mask_row<KMAX>(t, T, K, e);
    if constexpr (!kStage)
        for (int i = tid; i < E * kWaves; i += kLayoutTile) emask[i] = 0ull;
    if (tid == 0) s_err = 0;

    // expert offsets: experts are owned in chunks of 256 (x = chunk * 256 + tid)
    int tot[NCH], pre[NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        tot[j] = pre[j] = 0;
        const int x = j * kLayoutTile + tid;
        if (j * kLayoutTile < E) {   // uniform; lanes past E sum column E - 1 and drop it
            column_sums(table, rows, x < E ? x : E - 1, ntiles, tile, c0[j], tot[j], pre[j]);
            tot[j] = x < E ? tot[j] : 0;
            pre[j] = x < E ? pre[j] : 0;
        }
    }
    {
        int tg, pg;
        column_sums(table, rows, E + (tid < G ? tid : G - 1), ntiles, tile, cg0, tg, pg);
        if (tid < G) {
            tot_g[tid] = tg;
            base_g[tid] = pg;
        }
    }
    __syncthreads();   // s_err cleared
    if (tile == 0) {
        int er = tid < ntiles ? er_v : 0;
        for (int b = tid + kLayoutTile; b < ntiles; b += kLayoutTile) er |= table[(size_t)b * rows + E + G];
        if (er) atomicOr(&s_err, er);
    }
    if constexpr (kStage) {
#pragma unroll
        for (int u = 0; u < kWordsPerThread; ++u) {
            const int i = u * kLayoutTile + tid;
            if (i < E * kWaves) emask[i] = (unsigned long long)wlo[u] | ((unsigned long long)whi[u] << 32);
        }
    }
    int carry = 0;
    int base[NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        base[j] = 0;
        if (j * kLayoutTile < E) {   // uniform
            int all;
            const int excl = block_exclusive_scan(tot[j], s_wave_tot, &all);
            const int x = j * kLayoutTile + tid;
            if (x < E) {
                base[j] = carry + excl + pre[j];
                if (tile == 0) {
                    L.expert_count[x] = tot[j];
                    L.expert_offset[x] = carry + excl;
                }
            }
            carry += all;
        }
    }
    if (tile == 0 && tid == 0) L.expert_offset[E] = carry;
    // Group offsets: an exclusive scan over the G <= 32 groups in wave 0.
    if (wave == 0) {
        const int gt = lane < G ? tot_g[lane] : 0;
        const int incl = wave_incl_scan(gt);
        if (lane < G) {
            const int goff = incl - gt;
            if (tile == 0) {
                L.group_count[lane] = gt;
                L.group_offset[lane] = goff;
            }
            base_g[lane] += goff;
        }
        if (tile == 0 && lane == G - 1) L.group_offset[G] = incl;
        if (tile == 0 && lane == 0) *L.status = s_err;
    }

    // The tile's LDS words: loaded above (top-k <= 8), else rebuilt.
    Inserted ins;
    if constexpr (kStage) ins = classify_token<KMAX>(e, t < T, K, E, gmagic);
    else ins = insert_token<KMAX>(e, t < T, K, E, gmagic, emask, wave, lane);
    const uint32_t gm = ins.gm, bad = ins.bad();
    for (int g = 0; g < G; ++g) {
        const uint64_t b = __ballot((gm >> g) & 1u);
        if (lane == 0) gball[g][wave] = b;
    }
    __syncthreads();

    // Offsets per (expert, wave) and (group, wave): base + lanes of earlier
    // waves. With staging, also each expert's first position in the tile's
    // slot-ordered pair list (an exclusive scan over experts of the tile's counts).
    int npairs = 0;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        if (j * kLayoutTile < E) {   // uniform
            const int x = j * kLayoutTile + tid;
            int cnt = 0;
            if (x < E) {
                const unsigned long long *m = emask + x * kWaves;
                int r = base[j];
#pragma unroll
                for (int w = 0; w < kWaves; ++w) {
                    off_e[x * kWaves + w] = r;
                    r += __popcll(m[w]);
                }
                cnt = r - base[j];
            }
            if constexpr (kStage) {
                int all;
                const int lex = block_exclusive_scan(cnt, s_wave_tot, &all);
                if (x < E) ldelta[x] = npairs + lex - base[j];
                npairs += all;
            }
        }
    }
    if (tid < G) {
        int r = base_g[tid];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            off_g[tid][w] = r;
            r += __popcll(gball[tid][w]);
        }
    }
    __syncthreads();

    if (t < T) {
        if constexpr (kStage) {
            tile_token_entries<KMAX, EXACT>(t, T, K, G, gmagic, wave, lane, e, gm, bad, emask, off_e, ldelta,
                                            off_g, gball, s_src, s_dst, L, vec);
        } else {
            const uint64_t below = lanemask_lt(lane);
            const size_t p0 = (size_t)t * K;
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                if (k < K) {
                    int se = -1, sg = -1;
                    if (!((bad >> k) & 1u)) {
                        const int x = e[k];
                        se = off_e[x * kWaves + wave] + __popcll(emask[x * kWaves + wave] & below);
                        L.recv_src_e[se] = (int32_t)(p0 + k);
                        const int g = group_of(x, gmagic);
                        sg = off_g[g][wave] + __popcll(gball[g][wave] & below);
                    }
                    L.slot_e[p0 + k] = se;
                    L.slot_g[p0 + k] = sg;
                }
            }
            token_group_entries(t, T, K, G, wave, below, gm, off_g, gball, L, vec);
        }
    }
    if constexpr (kStage) {
        __syncthreads();
        tile_write_recv_src_e(npairs, s_src, s_dst, L.recv_src_e, tid, kLayoutTile);
    }
}

constexpr int kFinBS = 1024;                  // finalize: one workgroup, a thread per expert
constexpr int kFinSerialTiles = 8;            // tiles past the first batch loaded one by one
constexpr int kFinWaves = kFinBS / kWave;

// Exclusive prefix sum over the 1024 threads of the finalize (or one-pass)
// workgroup, with no barrier before it: the caller orders it after any earlier
// reader of s_wave_tot.
__device__ __forceinline__ int fin_scan(int v, int *s_wave_tot, int &total)
{
    return block_exclusive_scan<kFinWaves>(v, s_wave_tot, &total, true);
}

// Finalize (fused layout + dispatch): one workgroup. A column's total over the
// tiles is an expert's (group's) count, the exclusive prefix of the totals its
// offset, and a tile's base in the column the offset plus the counts of the
// tiles before it. Writes the counts, offsets and status of the layout and the
// bases [tiles][E + G] into the workspace.
__global__ __launch_bounds__(kFinBS) void layout_finalize_kernel(
    int ntiles, int E, int G, const int32_t *__restrict__ table, int32_t *__restrict__ bases, LayoutPtrs L)
{
    __shared__ int s_wave_tot[kFinWaves];
    __shared__ int s_err;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int rows = E + G + 1, cols = E + G;
    const int xe = tid < E ? tid : E - 1;   // this thread's expert column (clamped)
    const int xg = tid < G ? tid : G - 1;   // and group column
    // every first load before any use (one round trip; see column_first)
    int ce[kBatch], cg[kBatch];
    column_first(table, rows, xe, ntiles, ce);
    column_first(table, rows, E + xg, ntiles, cg);
    const int er_v = table[(size_t)(tid < ntiles ? tid : ntiles - 1) * rows + E + G];
    __builtin_amdgcn_sched_barrier(0);
    if (tid == 0) s_err = 0;

    int te = 0, tg = 0;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
        te += u < ntiles ? ce[u] : 0;
        tg += u < ntiles ? cg[u] : 0;
    }
    // Tiles past the first batch: one load at a time for a few (a batch costs
    // more than a handful of L2 round trips), else kBatch loads at a time from
    // clamped rows (measured: 17 tiles 4.7 / 7.1 us, 24: 7.0 / 7.5, 32: 10.6 /
    // 7.8, 64: 24.2 / 13.9 us, one by one / batched).
    const bool batched = ntiles > kBatch + kFinSerialTiles;
    for (int b = kBatch; !batched && b < ntiles; ++b) {
        te += table[(size_t)b * rows + xe];
        tg += table[(size_t)b * rows + E + xg];
    }
    for (int b0 = kBatch; batched && b0 < ntiles; b0 += kBatch) {
        int ve[kBatch], vg[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const size_t b = (size_t)(b0 + u < ntiles ? b0 + u : ntiles - 1);
            ve[u] = table[b * rows + xe];
            vg[u] = table[b * rows + E + xg];
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            te += b0 + u < ntiles ? ve[u] : 0;
            tg += b0 + u < ntiles ? vg[u] : 0;
        }
    }
    te = tid < E ? te : 0;
    __syncthreads();   // s_err cleared
    int er = tid < ntiles ? er_v : 0;
    for (int b = tid + kFinBS; b < ntiles; b += kFinBS) er |= table[(size_t)b * rows + E + G];
    if (er) atomicOr(&s_err, er);

    int etot;
    const int eoff = fin_scan(te, s_wave_tot, etot);
    if (tid < E) {
        L.expert_count[tid] = te;
        L.expert_offset[tid] = eoff;
        int r = eoff;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (u < ntiles) {
                bases[(size_t)u * cols + tid] = r;
                r += ce[u];
            }
        }
        for (int b = kBatch; !batched && b < ntiles; ++b) {
            bases[(size_t)b * cols + tid] = r;
            r += table[(size_t)b * rows + tid];
        }
        for (int b0 = kBatch; batched && b0 < ntiles; b0 += kBatch) {
            int v[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) v[u] = table[(size_t)(b0 + u < ntiles ? b0 + u : ntiles - 1) * rows + tid];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                if (b0 + u < ntiles) {
                    bases[(size_t)(b0 + u) * cols + tid] = r;
                    r += v[u];
                }
            }
        }
    }
    if (tid == 0) L.expert_offset[E] = etot;
    if (wave == 0) {   // groups: an exclusive scan over the G <= 32 totals in wave 0
        const int gt = lane < G ? tg : 0;
        const int incl = wave_incl_scan(gt);
        if (lane < G) {
            const int goff = incl - gt;
            L.group_count[lane] = gt;
            L.group_offset[lane] = goff;
            int r = goff;
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                if (u < ntiles) {
                    bases[(size_t)u * cols + E + lane] = r;
                    r += cg[u];
                }
            }
            for (int b = kBatch; !batched && b < ntiles; ++b) {
                bases[(size_t)b * cols + E + lane] = r;
                r += table[(size_t)b * rows + E + lane];
            }
            for (int b0 = kBatch; batched && b0 < ntiles; b0 += kBatch) {
                int v[kBatch];
#pragma unroll
                for (int u = 0; u < kBatch; ++u)
                    v[u] = table[(size_t)(b0 + u < ntiles ? b0 + u : ntiles - 1) * rows + E + lane];
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    if (b0 + u < ntiles) {
                        bases[(size_t)(b0 + u) * cols + E + lane] = r;
                        r += v[u];
                    }
                }
            }
        }
        if (lane == G - 1) L.group_offset[G] = incl;
    }
    __syncthreads();   // s_err complete
    if (tid == 0) *L.status = s_err;
}

// One-launch layout (top-k <= 8, batches up to a few thousand tokens): a
// 1024-thread workgroup per tile of 256 tokens. Every workgroup counts the
// valid entries of all T tokens itself, into LDS histograms split into the
// tokens before its tile and the others, so it has each expert's and group's
// total (hence the offsets) and its tile's base in every column with no
// second launch and no exchange between workgroups. The split is uniform per
// wave: a wave's 64 consecutive tokens lie on one side of the tile boundary (a
// multiple of 64). Waves 0-3 then rank the tile's own tokens with the
// per-(expert, wave) words and write its entries as the place kernel does.
// Each workgroup reads the T*K indices once (from L2 after the first).
constexpr int kOpBS = kFinBS;          // 1024 threads: one expert per thread (E <= 1024)
constexpr int kOpTok = 4;              // tokens per thread per round of the count
static_assert(kOpBS >= 1024, "one expert per thread");

// Count one token's valid entries into the histogram h (expert bins) and
// return the groups it reaches. Branch-free (this code runs once per CU from a
// cold instruction cache, so its length is its cost): an entry that does not
// count adds 0 to a bin chosen by the lane, so no exec-mask regions and no
// same-address pile-up. Error bits go to er.
template <int KMAX>
__device__ __forceinline__ uint32_t onepass_token(const int (&e)[KMAX], bool live, int K, int E,
                                                  uint32_t gmagic, int *h, int lane, int &er)
{
    uint32_t gm = 0;
    const int spare = lane < E ? lane : 0;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        const int x = e[k];
        const bool in = live && k < K && (unsigned)x < (unsigned)E;
        bool rep = false;
#pragma unroll
        for (int q = 0; q < k; ++q) rep = rep || e[q] == x;
        const bool v = in && !rep;
        er |= (live && k < K && !in) ? 1 : 0;
        er |= (in && rep) ? 2 : 0;
        atomicAdd(&h[v ? x : spare], v ? 1 : 0);
        gm |= v ? 1u << group_of(x, gmagic) : 0u;
    }
    return gm;
}

template <int KMAX, bool EXACT>
__global__ __launch_bounds__(kOpBS) void layout_onepass_kernel(
    const int32_t *__restrict__ idx, int T, int Krt, int E, int G, uint32_t gmagic, LayoutPtrs L, int vec)
{
    static_assert(KMAX <= 8, "the tile's entries are staged for at most 8 per token");
    // dynamic LDS: emask [E][kWaves] u64, then int hb[E], ha[E], off_e[E][kWaves], ldelta[E]
    extern __shared__ unsigned long long emask[];
    int *hb = reinterpret_cast<int *>(emask + E * kWaves);
    int *ha = hb + E;
    int *off_e = ha + E;
    int *ldelta = off_e + E * kWaves;
    __shared__ int32_t s_src[kLayoutTile * KMAX];   // the tile's pair ids in slot order
    __shared__ int32_t s_dst[kLayoutTile * KMAX];   // and their receive slots
    __shared__ int s_wave_tot[kFinWaves];
    __shared__ int gb[kMaxG], ga[kMaxG], base_g[kMaxG];
    __shared__ int off_g[kMaxG][kWaves];
    __shared__ uint64_t gball[kMaxG][kWaves];
    __shared__ int s_err;
    const int K = EXACT ? KMAX : Krt;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int tile = blockIdx.x;
    const int t0 = tile * kLayoutTile;
    const bool mine = tid < kLayoutTile;   // waves 0-3 hold the tile's tokens
    const int t = t0 + tid;

    // the first round of the count and the tile's own tokens: one round trip
    int e0[KMAX], e1[KMAX], e2[KMAX], e3[KMAX];
    load_row<KMAX>(idx, tid, T, K, e0);
    load_row<KMAX>(idx, kOpBS + tid, T, K, e1);
    load_row<KMAX>(idx, 2 * kOpBS + tid, T, K, e2);
    load_row<KMAX>(idx, 3 * kOpBS + tid, T, K, e3);
    int eo[KMAX];
    load_row<KMAX>(idx, t, T, K, eo);
    __builtin_amdgcn_sched_barrier(0);
    for (int i = tid; i < E * kWaves; i += kOpBS) emask[i] = 0ull;
    for (int x = tid; x < E; x += kOpBS) hb[x] = ha[x] = 0;
    if (tid < kMaxG) gb[tid] = ga[tid] = 0;
    if (tid == 0) s_err = 0;
    __syncthreads();

    // Tokens r0 + j * kOpBS + tid, j < kOpTok, per round; rows rotate through
    // e0 (the loop is not unrolled, to keep the code short). Lane g < G keeps
    // the wave's count of group g, split before / not before the tile.
    int er = 0, accb = 0, acca = 0;
    for (int r0 = 0;;) {
#pragma unroll 1
        for (int j = 0; j < kOpTok; ++j) {
            const int ub = r0 + j * kOpBS + wave * kWave;   // the wave's first token
            if (ub < T) {                                     // uniform
                const int u = ub + lane;
                const bool before = ub < t0;                  // uniform
                const uint32_t gm = onepass_token<KMAX>(e0, u < T, K, E, gmagic, before ? hb : ha, lane, er);
                for (int g = 0; g < G; ++g) {
                    const int c = __popcll(__ballot((gm >> g) & 1u));
                    const int add = lane == g ? c : 0;
                    accb += before ? add : 0;
                    acca += before ? 0 : add;
                }
            }
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                e0[k] = e1[k];
                e1[k] = e2[k];
                e2[k] = e3[k];
            }
        }
        r0 += kOpBS * kOpTok;
        if (r0 >= T) break;
        load_row<KMAX>(idx, r0 + tid, T, K, e0);
        load_row<KMAX>(idx, r0 + kOpBS + tid, T, K, e1);
        load_row<KMAX>(idx, r0 + 2 * kOpBS + tid, T, K, e2);
        load_row<KMAX>(idx, r0 + 3 * kOpBS + tid, T, K, e3);
    }
    if (lane < G) {
        atomicAdd(&gb[lane], accb);
        atomicAdd(&ga[lane], acca);
    }
    if (er) atomicOr(&s_err, er);
    // the tile's words (waves 0-3), built while the counts settle
    // the tile's words (waves 0-3): the same classification, OR-ing 0 for an
    // entry that does not count
    uint32_t gm_t = 0, bad_t = 0;
    if (mine) {   // uniform per wave
        const bool live = t < T;
        const unsigned long long bit = 1ull << lane;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const int x = eo[k];
            const bool in = live && k < K && (unsigned)x < (unsigned)E;
            bool rep = false;
#pragma unroll
            for (int q = 0; q < k; ++q) rep = rep || eo[q] == x;
            const bool v = in && !rep;
            bad_t |= (k < K && !v) ? 1u << k : 0u;
            atomicOr(&emask[(v ? x : 0) * kWaves + wave], v ? bit : 0ull);
            gm_t |= v ? 1u << group_of(x, gmagic) : 0u;
        }
        uint64_t mine_b = 0;
        for (int g = 0; g < G; ++g) {
            const uint64_t b = __ballot((gm_t >> g) & 1u);
            mine_b = lane == g ? b : mine_b;
        }
        if (lane < G) gball[lane][wave] = mine_b;
    }
    __syncthreads();

    // offsets: an exclusive scan over the experts (one per thread) of the totals;
    // the tile's base in column x is x's offset plus the count before the tile
    const int x = tid;
    const int cb = x < E ? hb[x] : 0, ca = x < E ? ha[x] : 0;
    int etot;
    const int eoff = fin_scan(cb + ca, s_wave_tot, etot);
    const int base_x = eoff + cb;
    if (tile == 0) {
        if (x < E) {
            L.expert_count[x] = cb + ca;
            L.expert_offset[x] = eoff;
        }
        if (x == 0) L.expert_offset[E] = etot;
    }
    if (wave == 0) {   // groups: an exclusive scan over the G <= 32 totals
        const int gbv = lane < G ? gb[lane] : 0;
        const int gt = lane < G ? gbv + ga[lane] : 0;
        const int incl = wave_incl_scan(gt);
        if (lane < G) {
            const int goff = incl - gt;
            if (tile == 0) {
                L.group_count[lane] = gt;
                L.group_offset[lane] = goff;
            }
            base_g[lane] = goff + gbv;
        }
        if (tile == 0 && lane == G - 1) L.group_offset[G] = incl;
        if (tile == 0 && lane == 0) *L.status = s_err;
    }
    // per (expert, wave) offsets of the tile, and each expert's first position
    // in the tile's slot-ordered pair list
    int cnt = 0;
    if (x < E) {
        const unsigned long long *m = emask + x * kWaves;
        int r = base_x;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            off_e[x * kWaves + w] = r;
            r += __popcll(m[w]);
        }
        cnt = r - base_x;
    }
    __syncthreads();   // s_wave_tot and base_g
    int npairs;
    const int lex = fin_scan(cnt, s_wave_tot, npairs);
    if (x < E) ldelta[x] = lex - base_x;
    if (tid < G) {
        int r = base_g[tid];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            off_g[tid][w] = r;
            r += __popcll(gball[tid][w]);
        }
    }
    __syncthreads();

    if (mine && t < T)
        tile_token_entries<KMAX, EXACT>(t, T, K, G, gmagic, wave, lane, eo, gm_t, bad_t, emask, off_e, ldelta,
                                        off_g, gball, s_src, s_dst, L, vec);
    if (mine && t < T) L.tok_group_mask[t] = gm_t;
    __syncthreads();
    tile_write_recv_src_e(npairs, s_src, s_dst, L.recv_src_e, tid, kOpBS);
}

// No tokens: every count and offset is 0 and the status is clear.
__global__ __launch_bounds__(kLayoutTile) void layout_empty_kernel(int E, int G, LayoutPtrs L)
{
    for (int e = threadIdx.x; e <= E; e += kLayoutTile) {
        if (e < E) L.expert_count[e] = 0;
        L.expert_offset[e] = 0;
    }
    for (int g = threadIdx.x; g <= G; g += kLayoutTile) {
        if (g < G) L.group_count[g] = 0;
        L.group_offset[g] = 0;
    }
    if (threadIdx.x == 0) *L.status = 0;
}

}  // namespace

namespace {

using CountFn = void (*)(const int32_t *, int, int, int, int, uint32_t, uint32_t *, int32_t *, uint32_t *,
                         uint32_t *, int32_t *, int32_t *);
using PlaceFn = void (*)(const int32_t *, int, int, int, int, uint32_t, int, const int32_t *,
                         const uint32_t *, LayoutPtrs, int);
using OnepassFn = void (*)(const int32_t *, int, int, int, int, uint32_t, LayoutPtrs, int);

template <int NCH>
void pick_layout_n(int K, CountFn &count, PlaceFn &place)
{
    switch (K) {
    case 2: count = layout_count_kernel<2, true>; place = layout_place_kernel<2, true, NCH>; break;
    case 4: count = layout_count_kernel<4, true>; place = layout_place_kernel<4, true, NCH>; break;
    case 8: count = layout_count_kernel<8, true>; place = layout_place_kernel<8, true, NCH>; break;
    default:
        if (K <= 8) { count = layout_count_kernel<8, false>; place = layout_place_kernel<8, false, NCH>; }
        else { count = layout_count_kernel<32, false>; place = layout_place_kernel<32, false, NCH>; }
    }
}

void pick_layout(int K, int E, CountFn &count, PlaceFn &place)
{
    if (E <= kLayoutTile) pick_layout_n<1>(K, count, place);
    else pick_layout_n<kMaxEChunks>(K, count, place);
}

}  // namespace

hipError_t launch_layout(const int32_t *idx, int T, int K, int E, int G, const LayoutPtrs &L,
                         int32_t *ws, hipStream_t stream)
{
    if (T == 0) {
        hipLaunchKernelGGL(layout_empty_kernel, dim3(1), dim3(kLayoutTile), 0, stream, E, G, L);
        return hipGetLastError();
    }
    const int ntiles = layout_tiles(T);
    const LayoutWs w = layout_ws(ws, T, E, G);
    const uint32_t gmagic = group_magic(E, G);
    const size_t lds1 = (size_t)E * kWaves * sizeof(unsigned long long);
    const size_t lds2 = lds1 + (size_t)E * (kWaves + 1) * sizeof(int);
    // vector stores of the slot rows when the arrays allow them
    const auto a16 = [](const void *q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
    const int vec = (a16(L.slot_e) && a16(L.slot_g) ? 1 : 0) | (G % 4 == 0 && a16(L.slot_tg) ? 2 : 0);
    bool launched = false;
    const hipError_t xe = launch_layout_exchange(idx, T, K, E, G, L, vec | (a16(idx) ? 4 : 0), stream, launched);
    if (xe != hipSuccess || launched) return xe;
    if (K <= 8 && (int64_t)T * K <= tuning().layout_onepass_max_pairs) {
        OnepassFn onepass = K == 2 ? layout_onepass_kernel<2, true>
                          : K == 4 ? layout_onepass_kernel<4, true>
                          : K == 8 ? layout_onepass_kernel<8, true>
                                   : layout_onepass_kernel<8, false>;
        const size_t lds = (size_t)E * kWaves * sizeof(unsigned long long) + (size_t)E * (kWaves + 3) * sizeof(int);
        hipLaunchKernelGGL(onepass, dim3(ntiles), dim3(kOpBS), lds, stream, idx, T, K, E, G, gmagic, L, vec);
        return hipGetLastError();
    }
    CountFn count;
    PlaceFn place;
    pick_layout(K, E, count, place);
    hipLaunchKernelGGL(count, dim3(ntiles), dim3(kLayoutTile), lds1, stream, idx, T, K, E, G, gmagic,
                       L.tok_group_mask, w.table, w.words, w.gwords, nullptr, nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(place, dim3(ntiles), dim3(kLayoutTile), lds2, stream, idx, T, K, E, G, gmagic,
                       ntiles, w.table, w.words, L, vec);
    return hipGetLastError();
}

hipError_t launch_layout_count_finalize(const int32_t *idx, int T, int K, int E, int G,
                                        const LayoutPtrs &L, int32_t *ws, bool finalize_in_dispatch,
                                        hipStream_t stream)
{
    const int ntiles = layout_tiles(T);
    const LayoutWs w = layout_ws(ws, T, E, G);
    CountFn count;
    PlaceFn place;
    pick_layout(K, E, count, place);
    const size_t lds1 = (size_t)E * kWaves * sizeof(unsigned long long);
    hipLaunchKernelGGL(count, dim3(ntiles), dim3(kLayoutTile), lds1, stream, idx, T, K, E, G,
                       group_magic(E, G), L.tok_group_mask, w.table, w.words, w.gwords, w.bases, L.status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || finalize_in_dispatch) return e;
    hipLaunchKernelGGL(layout_finalize_kernel, dim3(1), dim3(kFinBS), 0, stream, ntiles, E, G, w.table,
                       w.bases, L);
    return hipGetLastError();
}

}  // namespace moe
