// Placement of one token inside a dispatch kernel (the fused layout +
// dispatch for large batches): the token's receive slots from the count
// kernel's per-tile token masks and the per-tile bases.
//
// For expert x of token t (tile b = t / 256, wave w and lane l of t in b):
//   slot = bases[b][x] + popcount of x's words of waves before w
//          + popcount(x's word of wave w & lanes below l),
// the number of earlier tokens that listed x, after x's offset: the same
// stable order moe_layout() gives. Groups likewise with the group words and
// group bases. Wave 0 of the workgroup does the work (lane k holds entry k,
// lane g group g), writes the token's layout entries, and leaves the rows to
// copy to (slot_e for the per-expert layout, slot_tg for the per-group one)
// in dst[]; the call ends with a workgroup barrier.
//
// The bases come either from the finalize kernel, launched before, or from
// workgroup 0 of the dispatch itself (finalize_role), which computes them
// while the other workgroups load their rows. The count kernel sets every
// base to -1 first (a valid base is >= 0), so a token's wave polls exactly the
// base words it needs until they are valid: agent-scope atomic stores and
// loads of those words, no flag and no state that outlives the call. Workgroup
// 0 waits for nothing, and is the first workgroup dispatched; a wait is still
// bounded (P.wait_ticks of the constant 100 MHz clock, 0.2 s by default,
// against the few µs it takes). A wave that waited that long computes its
// token's bases itself from the count table (self_bases: a few hundred loads,
// exact) and sets the diagnostic bit MOE_STATUS_SYNC_FALLBACK, so no wave waits
// forever and a late workgroup 0 costs time, never results.
#pragma once

#include "moe_ep.h"

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// The rank of token lane `l` of wave `w` among a tile's tokens whose masks
// are words q[0..3] (32-bit halves): tokens of earlier waves, then of earlier
// lanes of its own wave.
__device__ __forceinline__ int place_rank(const uint32_t *__restrict__ q, int w, int l)
{
    int r = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint64_t word = (uint64_t)q[2 * j] | ((uint64_t)q[2 * j + 1] << 32);
        r += j < w ? __popcll(word) : (j == w ? __popcll(word & lanemask_lt(l)) : 0);
    }
    return r;
}

constexpr int kFinBatch = kFinTiles;

__device__ __forceinline__ int base_load(int32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The count table as a buffer resource: loads past its nt rows return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t fin_table_rsrc(const int32_t *tab, int nt, int rows)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t *>(tab), (short)0, nt * rows * 4, 0x00020000);
}

// Column `col` of the count table over the (at most kFinBatch) tiles: the
// counts in v (0 past the last tile) and their total. One buffer load per
// tile, all in flight together, from one running offset.
__device__ __forceinline__ int fin_column_sum(__amdgpu_buffer_rsrc_t tab, int rows, int col,
                                              int (&v)[kFinBatch])
{
    int off = col * 4;
#pragma unroll
    for (int u = 0; u < kFinBatch; ++u) {
        v[u] = __builtin_amdgcn_raw_buffer_load_b32(tab, off, 0, 0);
        off += rows * 4;
    }
    int s = 0;
#pragma unroll
    for (int u = 0; u < kFinBatch; ++u) s += v[u];
    return s;
}

// Bases of column `col` in the nt tiles: the column's offset plus the counts
// of the tiles before. `bases` is a buffer resource over the nt rows, so the
// stores of rows past the last tile are dropped by the hardware; the stores
// carry sc1 (kCpolSc1), the agent-scope coherent form, so the polling loads of
// other workgroups see them.
__device__ __forceinline__ void fin_column_bases(int col, const int (&v)[kFinBatch], int offset,
                                                 __amdgpu_buffer_rsrc_t bases, int cols)
{
    int r = offset, off = col * 4;
#pragma unroll
    for (int u = 0; u < kFinBatch; ++u) {
        __builtin_amdgcn_raw_buffer_store_b32(r, bases, off, 0, kCpolSc1);
        r += v[u];
        off += cols * 4;
    }
}

// Exclusive prefix sum over the workgroup (at most 16 waves); `total` gets
// the sum of all. Ends with a barrier, so s_tot can be reused.
__device__ __forceinline__ int fin_block_scan(int v, int *s_tot, int &total)
{
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave, nw = blockDim.x / kWave;
    const int x = wave_incl_scan(v);
    if (lane == kWave - 1) s_tot[wave] = x;
    __syncthreads();
    int base = 0, all = 0;
    for (int w = 0; w < nw; ++w) {
        const int c = s_tot[w];
        base += w < wave ? c : 0;
        all += c;
    }
    __syncthreads();
    total = all;
    return base + x - v;
}

// Workgroup 0 of a placing dispatch (P.finalize; at most kFinBatch tiles):
// what the finalize kernel computes, with the workgroup's threads (a whole
// number of waves) taking the expert columns in rounds. A column's total over
// the tiles is an expert's (group's) count, the exclusive prefix of the
// totals its offset, and a tile's base in the column the offset plus the
// counts of the tiles before it. The status was set to 0 by the count kernel;
// the tiles' error bits are ORed into it.
__device__ void finalize_role(const PlaceArgs &P)
{
    __shared__ int s_tot[16];
    const int tid = threadIdx.x, lane = tid % kWave, nth = blockDim.x;
    const int E = P.E, G = P.G, nt = P.ntiles, rows = E + G + 1, cols = E + G;
    const __amdgpu_buffer_rsrc_t tab = fin_table_rsrc(P.table, nt, rows);
    const __amdgpu_buffer_rsrc_t bases = __builtin_amdgcn_make_buffer_rsrc(P.bases, (short)0, nt * cols * 4, 0x00020000);
    int carry = 0;
    for (int c0 = 0; c0 < E; c0 += nth) {
        const int e = c0 + tid;
        const bool live = e < E;
        int v[kFinBatch];
        int tot = fin_column_sum(tab, rows, live ? e : E - 1, v);
        tot = live ? tot : 0;
        int all;
        const int off = carry + fin_block_scan(tot, s_tot, all);
        carry += all;
        if (live) {
            P.L.expert_count[e] = tot;
            P.L.expert_offset[e] = off;
            fin_column_bases(e, v, off, bases, cols);
        }
    }
    if (tid == 0) P.L.expert_offset[E] = carry;
    if (tid < kWave) {   // groups (G <= 32) and the error bits (column E + G): wave 0
        const bool live = lane < G;
        int v[kFinBatch];
        int tot = fin_column_sum(tab, rows, live ? E + lane : E + G, v);
        const int incl = wave_incl_scan(live ? tot : 0);
        if (live) {
            const int goff = incl - tot;
            P.L.group_count[lane] = tot;
            P.L.group_offset[lane] = goff;
            fin_column_bases(E + lane, v, goff, bases, cols);
        }
        if (lane == G - 1) P.L.group_offset[G] = incl;
        if (lane == G) {   // G <= 32 < 64: this lane summed the error column; OR it instead
            int er = 0;
#pragma unroll
            for (int u = 0; u < kFinBatch; ++u) er |= v[u];
            if (er) atomicOr(P.L.status, er);
        }
    }
}

// The bases of this wave's token from the count table alone (what workgroup 0
// or the finalize kernel writes): lane k with a valid expert e gets be = the
// expert's offset (the totals of every column before e, over all tiles) plus
// the counts of e in the tiles before `tile`; lane g < G gets bg likewise for
// group g. Lane j of the wave first totals the expert columns of its chunk
// [j * cpl, (j + 1) * cpl); a scan over the lanes gives each chunk's offset;
// lane k then adds the columns of e's chunk before e. Every lane of the wave
// calls this together (shuffles).
__device__ __forceinline__ void self_bases(const PlaceArgs &P, int tile, bool valid, int e, bool hg, int &be,
                                        int &bg)
{
    const int lane = threadIdx.x % kWave;
    const int E = P.E, G = P.G, nt = P.ntiles, rows = E + G + 1;
    const int32_t *tab = P.table;
    const int cpl = (E + kWave - 1) / kWave;
    const int c0 = lane * cpl, c1 = min(c0 + cpl, E);
    int tot = 0;
    for (int c = c0; c < c1; ++c)
        for (int b = 0; b < nt; ++b) tot += tab[(size_t)b * rows + c];
    const int incl = wave_incl_scan(tot);
    const int owner = valid ? e / cpl : 0;
    int x = __shfl(incl - tot, owner);
    if (valid) {
        for (int c = owner * cpl; c < e; ++c)
            for (int b = 0; b < nt; ++b) x += tab[(size_t)b * rows + c];
        for (int b = 0; b < tile; ++b) x += tab[(size_t)b * rows + e];
        be = x;
    }
    int gt = 0;
    if (lane < G)
        for (int b = 0; b < nt; ++b) gt += tab[(size_t)b * rows + E + lane];
    const int gincl = wave_incl_scan(gt);
    if (hg) {
        int y = gincl - gt;
        for (int b = 0; b < tile; ++b) y += tab[(size_t)b * rows + E + lane];
        bg = y;
    }
}

__device__ __forceinline__ void place_token(const PlaceArgs &P, int t, int K, int32_t *dst)
{
    if (threadIdx.x < kWave) {
        const int lane = threadIdx.x;
        const int E = P.E, G = P.G;
        const int tile = t / kLayoutTile, w = (t % kLayoutTile) / kWave, l = t % kWave;
        const bool mine = lane < K;
        const int e = P.idx[(size_t)t * K + (mine ? lane : K - 1)];
        // an entry repeats iff an earlier entry of the token names the same expert
        bool rep = false;
        for (int j = 0; j < K; ++j) {
            const int ej = __shfl(e, j);
            rep = rep || (j < lane && ej == e);
        }
        const bool valid = mine && (unsigned)e < (unsigned)E && !rep;
        const int g = valid ? group_of(e, P.gmagic) : 0;
        // the groups the token reaches, on every lane
        uint32_t gm = valid ? 1u << g : 0u;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) gm |= __shfl_xor(gm, o);
        const bool hg = lane < G && ((gm >> lane) & 1u);
        // ranks from the count kernel's words, then the tile's bases
        const int re = valid ? place_rank(P.words + ((size_t)tile * E + e) * 8, w, l) : 0;
        const int rg = hg ? place_rank(P.gwords + ((size_t)tile * G + lane) * 8, w, l) : 0;
        int32_t *tb = P.bases + (size_t)tile * (E + G);
        int be = 0, bg = 0;
        // (wall_clock64 is a scalar read, so the time test and `ok` are wave-uniform)
        bool ok = !P.self_bases;
        const uint64_t t0 = wall_clock64();
        while (ok) {
            if (valid) be = base_load(tb + e);
            if (hg) bg = base_load(tb + E + lane);
            if (__all(be >= 0 && bg >= 0)) break;
            if (wall_clock64() - t0 > P.wait_ticks) ok = false;
            else __builtin_amdgcn_s_sleep(2);
        }
        if (!ok) {
            self_bases(P, tile, valid, e, hg, be, bg);
            if (lane == 0) atomicOr(P.L.status, MOE_STATUS_SYNC_FALLBACK);
        }
        const int se = valid ? be + re : -1;
        const int sgl = hg ? bg + rg : -1;   // lane g < G: the token's row in group g, or -1
        const int sg = __shfl(sgl, g);
        // (the receive lists hold T*K and T*min(K, G) entries; T = the grid)
        const int64_t T = gridDim.x;
        if (mine) {
            const size_t p = (size_t)t * K + lane;
            P.L.slot_e[p] = se;
            P.L.slot_g[p] = valid ? sg : -1;
            if (valid && se >= 0 && se < T * K) P.L.recv_src_e[se] = (int32_t)p;
        }
        if (lane < G) {
            P.L.slot_tg[(size_t)t * G + lane] = sgl;
            if (sgl >= 0 && sgl < T * (K < G ? K : G)) P.L.recv_src_g[sgl] = t;
        }
        if (P.mode == 0) {
            if (mine) dst[lane] = se;
        } else if (lane < G) {
            dst[lane] = sgl;
        }
    }
    __syncthreads();
}

}  // namespace moe
