// One-launch layout with an exchange between tiles (moe_layout, top-k <= 8, up
// to 128 tiles): the count and place kernels of layout.hip as one workgroup
// per tile, which learns what it needs of the other tiles from a
// table in library memory instead of from a second launch. The workgroup
// counts its tile with per-(expert, wave) words in LDS as the count kernel
// does (with two lanes per token, below) and takes the tile's own exclusive
// prefix of its counts over the experts, and over the groups. It writes, per column (E experts, G groups,
// two summary columns: the tile's numbers of expert and group pairs, and its
// error bits; one padding column to an even count), one 64-bit entry
// tag << 32 | value with one atomic store, the value packing the tile's count
// and its prefix. Each thread then reads two adjacent columns of every tile
// (one 16-byte read per tile). Summed over
// the tiles, the prefixes give each expert's offset, and the counts of the
// tiles before this one its first receive row in this tile, so no scan is
// left after the exchange. The tag is this call's number on its stream, which
// the host never repeats while the table can hold entries of earlier calls;
// an entry of an earlier call, or one that a concurrent call overwrote, never
// carries it, so every value taken is this call's and nothing needs to be set
// before the call. The reads are bounded (wait_ticks of the constant 100 MHz
// clock); a workgroup whose wait runs out, or every workgroup when `recount`
// is set, counts all T tokens itself instead (exact, O(T * K) per workgroup),
// scans the totals, and reports MOE_STATUS_SYNC_FALLBACK if it is tile 0.
// With one tile there is nothing to exchange and xt is NULL.
//
// This file is compiled with kernel-argument preloading (the first arguments
// arrive in SGPRs when a wave starts, instead of by a scalar load at its
// entry), which took about 0.6 µs off this kernel at 4096 tokens x top-8
// (10.8 -> 10.2 µs per call); the other kernels stay without it, as the
// placing dispatch measured slower with it. Two lanes per token (each with
// half the entries to insert, rank and place) then took it to 9.8 µs; one
// lane per token with 4 waves had half as many threads for the same work.
#include "moe_ep.h"

#include "layout_tile.hpp"

#include <algorithm>
#include <mutex>

namespace moe {

namespace {

__device__ __forceinline__ void xch_put(uint64_t *p, uint32_t tag, uint32_t v)
{
    __hip_atomic_store(p, ((uint64_t)tag << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Packed values of a table entry, two 16-bit fields, so that a column is
// summed over up to 16 tiles with one 32-bit add per entry and no carry
// between the fields (a field is at most 256 * 8 per tile): count | prefix
// << 16 for an expert or group column; expert pairs | group pairs << 16 for
// the first summary column; for the second, the tile's error bits as counts,
// bit 0 in the low byte and bit 1 in the next, so the sum tells whether any
// tile had each bit.
__device__ __forceinline__ uint32_t xch_pack(int lo, int hi) { return (uint32_t)lo | (uint32_t)hi << 16; }
__device__ __forceinline__ uint32_t xch_err_pack(int err) { return (uint32_t)(err & 1) | (uint32_t)(err & 2) << 7; }
__device__ __forceinline__ int xch_err_unpack(uint32_t s) { return ((s & 0xFFu) ? 1 : 0) | ((s & 0xFF00u) ? 2 : 0); }

// The workgroup: two lanes per token of the 256-token tile, kXT = 512
// threads in 8 waves of 32 tokens. Lane l of a wave takes token l % 32 of the
// wave and half l / 32 of its entries (k in [h * KMAX / 2, (h + 1) * KMAX / 2)),
// so each lane inserts, ranks and places half of a token's entries; both lanes
// of a token hold its whole index row, so the repeats of an entry are still
// found in registers. The LDS words are 32-bit, one per (expert, wave), bit j
// for token j of the wave; the group words come from ballots over the lanes of
// the first half. Rank of an entry inside the tile = popcounts of its expert's
// words of earlier waves + popcount of its own wave's word below bit j: the
// token-ascending order, as with one lane per token.
constexpr int kXT = 2 * kLayoutTile;
constexpr int kXW = kXT / kWave;   // 8
// Pair sums left by the reader groups after the first: (groups - 1) x pairs,
// at most (8 - waves per pair set) x 64 with groups = 8 / waves per pair set.
constexpr int kXPartMax = (kXW - 1) * kWave;

// Every token's valid entries counted into s_tot (all tiles) and s_pre (tiles
// before `tile`), groups likewise in columns E.., error bits ORed into column
// E + G: the counts the exchange would have given, from the indices alone.
template <int KMAX, bool EXACT>
__device__ void xch_recount(const int32_t *__restrict__ idx, int T, int Krt, int E, int G, uint32_t gmagic,
                            int tile, int *s_tot, int *s_pre)
{
    const int K = EXACT ? KMAX : Krt;
    const int tid = threadIdx.x, rows = E + G + 1;
    for (int c = tid; c < rows; c += kXT) s_tot[c] = s_pre[c] = 0;
    __syncthreads();
#pragma unroll 1
    for (int u0 = 0; u0 < T; u0 += kXT) {
        const int u = u0 + tid;
        const bool before = u < tile * kLayoutTile;
        int e[KMAX];
        load_row<KMAX>(idx, u, T, K, e);
        mask_row<KMAX>(u, T, K, e);
        const Inserted ins = classify_token<KMAX>(e, u < T, K, E, gmagic);
        const uint32_t bad = ins.bad();
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (k < K && u < T && !((bad >> k) & 1u)) {
                atomicAdd(&s_tot[e[k]], 1);
                if (before) atomicAdd(&s_pre[e[k]], 1);
            }
        }
        for (int g = 0; g < G; ++g) {
            if ((ins.gm >> g) & 1u) {
                atomicAdd(&s_tot[E + g], 1);
                if (before) atomicAdd(&s_pre[E + g], 1);
            }
        }
        if (ins.err()) atomicOr(&s_tot[E + G], ins.err());
    }
    __syncthreads();
}

// The fallback's offsets: from the recounted totals and prefixes, scans over
// the experts and groups give each column's offset; base = offset + the count
// of earlier tiles; tile 0 writes the counts, offsets and status.
template <int NX>
__device__ void xch_fallback_offsets(int E, int G, int tile, const int *s_tot, const int *s_pre, int *base_e,
                                     int *base_g, int *s_wave_tot, const LayoutPtrs &L)
{
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    int carry = 0;
#pragma unroll
    for (int j = 0; j < NX; ++j) {
        if (j * kXT < E) {   // uniform
            const int x = j * kXT + tid;
            const int tx = x < E ? s_tot[x] : 0;
            int all;
            const int excl = block_exclusive_scan<kXW>(tx, s_wave_tot, &all);
            if (x < E) {
                base_e[x] = carry + excl + s_pre[x];
                if (tile == 0) {
                    L.expert_count[x] = tx;
                    L.expert_offset[x] = carry + excl;
                }
            }
            carry += all;
        }
    }
    if (tile == 0 && tid == 0) L.expert_offset[E] = carry;
    if (wave == 0) {
        const int gt = lane < G ? s_tot[E + lane] : 0;
        const int incl = wave_incl_scan(gt);
        if (lane < G) {
            const int goff = incl - gt;
            if (tile == 0) {
                L.group_count[lane] = gt;
                L.group_offset[lane] = goff;
            }
            base_g[lane] = goff + s_pre[E + lane];
        }
        if (tile == 0 && lane == G - 1) L.group_offset[G] = incl;
        if (tile == 0 && lane == 0) *L.status = s_tot[E + G] | MOE_STATUS_SYNC_FALLBACK;
    }
}

// NX: experts in chunks of kXT (E <= NX * 512). MR: more than one round of
// tiles, read by several groups of waves (E <= 512 only).
template <int KMAX, bool EXACT, int NX, bool MR>
__global__ __launch_bounds__(kXT) void layout_exchange_kernel(
    const int32_t *__restrict__ idx, int T, int vec, int Krt, int E, int G, uint32_t gmagic, int ntiles,
    uint64_t *__restrict__ xt, uint32_t tag, uint64_t wait_ticks, int recount, LayoutPtrs L)
{
    static_assert(KMAX == 2 || KMAX == 4 || KMAX == 8, "two lanes take KMAX / 2 entries of a token each");
    constexpr int KH = KMAX / 2;                   // entries per lane
    constexpr int NCOL = NX + 1;                   // columns a thread publishes (E + G + 3 <= NCOL * 512)
    constexpr int kXB = 16;                        // tiles per round of reads
    // dynamic LDS: uint32 ew [E][kXW]; int loff_e [E][kXW], lstart [E], base_e [E],
    // s_tot [E+G+1], s_pre [E+G+1] (the fallback's)
    extern __shared__ uint32_t ew[];
    int *loff_e = reinterpret_cast<int *>(ew + E * kXW);   // rank base of (expert, wave) in the tile
    int *lstart = loff_e + E * kXW;                        // expert's first place in the tile's pair list
    int *base_e = lstart + E;                              // expert's first receive row of the tile
    int *s_tot = base_e + E;
    int *s_pre = s_tot + E + G + 1;
    __shared__ int32_t s_src[kLayoutTile * KMAX];   // the tile's pair ids in slot order
    __shared__ int32_t s_dst[kLayoutTile * KMAX];   // and their receive slots
    __shared__ int s_wave_tot[kXW];
    __shared__ int lgstart[kMaxG];
    __shared__ int gtot[kMaxG];   // the tile's count of each group
    __shared__ int base_g[kMaxG];
    __shared__ int loff_g[kMaxG][kXW];
    __shared__ uint32_t gball[kMaxG][kXW];
    __shared__ int s_err, s_late, s_gpairs;
    constexpr bool kMR = MR && NX == 1;
    __shared__ int s_part[kMR ? kXPartMax : 1][6];   // the other reader groups' column sums (below)
    const int K = EXACT ? KMAX : Krt;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int j = lane & 31, h = lane >> 5;   // token j of the wave, half h of its entries
    const int tile = blockIdx.x;
    const int t = tile * kLayoutTile + wave * 32 + j;
    const int rows = (E + G + 3) & ~1;   // table columns: experts, groups, pairs, error bits (+1: even)
    const uint32_t below = (1u << j) - 1u;

    // Count the tile. Lane h loads its own entries k = h * KH + q and the other
    // lane's (k = (1 - h) * KH + q), choosing them by address: selecting
    // between registers by h would make the compiler index a private array.
    int own[KH], oth[KH];
    {
        const int tc = t < T ? t : T - 1;
        if constexpr (EXACT && KMAX == 8) {
            if (vec & 4) {   // 16-byte aligned index rows: two vector loads
                const u32x4 *row = reinterpret_cast<const u32x4 *>(idx + (size_t)tc * KMAX);
                const u32x4 a = row[h], b = row[h ^ 1];
                own[0] = (int)a.x; own[1] = (int)a.y; own[2] = (int)a.z; own[3] = (int)a.w;
                oth[0] = (int)b.x; oth[1] = (int)b.y; oth[2] = (int)b.z; oth[3] = (int)b.w;
            } else {
                const int32_t *row = idx + (size_t)tc * KMAX;
#pragma unroll
                for (int q = 0; q < KH; ++q) {
                    own[q] = row[h * KH + q];
                    oth[q] = row[(h ^ 1) * KH + q];
                }
            }
        } else {
            // clamped in-range addresses; entries k >= K are masked below
            const int32_t *row = idx + (size_t)tc * K;
#pragma unroll
            for (int q = 0; q < KH; ++q) {
                const int ko = h * KH + q, kt = (h ^ 1) * KH + q;
                own[q] = row[ko < K ? ko : K - 1];
                oth[q] = row[kt < K ? kt : K - 1];
            }
        }
    }
    for (int i = tid; i < E * kXW; i += kXT) ew[i] = 0u;
    if (tid == 0) {
        s_err = 0;
        s_late = recount;
    }
    __syncthreads();
    // Classify (as the count kernel: an entry repeats iff its expert equals an
    // earlier in-range entry of the token; the groups are those of its in-range
    // entries) and insert this lane's valid entries. Each lane reports the
    // errors of its own entries; both lanes find the token's groups.
    const bool live = t < T;
    uint32_t gm = 0, ok_q = 0;   // ok_q bit q: entry h * KH + q counts
    int err = 0;
#pragma unroll
    for (int q = 0; q < KH; ++q) {
        const int ko = h * KH + q, kt = (h ^ 1) * KH + q;
        if (!(live && ko < K)) own[q] = -1;
        if (!(live && kt < K)) oth[q] = -1;
    }
#pragma unroll
    for (int q = 0; q < KH; ++q) {
        const bool ino = (unsigned)own[q] < (unsigned)E, int_ = (unsigned)oth[q] < (unsigned)E;
        gm |= ino ? 1u << group_of(own[q], gmagic) : 0u;
        gm |= int_ ? 1u << group_of(oth[q], gmagic) : 0u;
        err |= (live && h * KH + q < K && !ino) ? 1 : 0;   // an entry of the token, out of range
        bool rep = false;
#pragma unroll
        for (int p = 0; p < q; ++p) rep = rep || own[p] == own[q];
#pragma unroll
        for (int p = 0; p < KH; ++p) rep = rep || (h != 0 && oth[p] == own[q]);   // the first half comes first
        err |= (ino && rep) ? 2 : 0;
        const bool v = ino && !rep;
        ok_q |= v ? 1u << q : 0u;
        if (v) atomicOr(&ew[own[q] * kXW + wave], 1u << j);
    }
    if (t < T && h == 0) L.tok_group_mask[t] = gm;
    for (int g = 0; g < G; ++g) {
        const uint64_t b = __ballot(h == 0 && ((gm >> g) & 1u));   // bits 0-31: the wave's tokens
        if (lane == 0) gball[g][wave] = (uint32_t)b;
    }
    if (err) atomicOr(&s_err, err);
    __syncthreads();

    // The tile's own layout: per (expert, wave) the rank base inside the tile
    // and the expert's count; an exclusive scan of the counts over the experts
    // (each expert's first place in the tile's slot-ordered pair list); per
    // (group, wave) the rank base and over the groups the same scan.
    // The groups first, in the last wave (lane g < G), which has no experts of
    // the first chunk for E <= 448: it runs beside the experts' popcounts.
    if (wave == kXW - 1) {
        const int gl = lane < G ? lane : 0;
        int r = 0;
#pragma unroll
        for (int w = 0; w < kXW; ++w) {
            if (lane < G) loff_g[gl][w] = r;
            r += lane < G ? __popc(gball[gl][w]) : 0;
        }
        const int incl = wave_incl_scan(r);
        if (lane < G) {
            lgstart[lane] = incl - r;
            gtot[lane] = r;
        }
        if (lane == kMaxG - 1) s_gpairs = incl;
    }
    int npairs = 0, cnt_x[NX] = {};   // cnt_x[c]: the count of expert c * 512 + tid in the tile
#pragma unroll
    for (int c = 0; c < NX; ++c) {
        if (c * kXT < E) {   // uniform
            const int x = c * kXT + tid;
            int cnt = 0;
            if (x < E) {
#pragma unroll
                for (int w = 0; w < kXW; ++w) {
                    loff_e[x * kXW + w] = cnt;
                    cnt += __popc(ew[x * kXW + w]);
                }
            }
            cnt_x[c] = cnt;
            int all;
            const int lex = block_exclusive_scan<kXW>(cnt, s_wave_tot, &all, c == 0);   // (s_wave_tot unused before)
            if (x < E) lstart[x] = npairs + lex;
            npairs += all;
        }
    }
    __syncthreads();

    // The tile's value of column c (see xch_pack); n: an expert's count, when
    // the caller has it.
    auto own_value = [&](int c, int n) -> uint32_t {
        if (c < E) return xch_pack(n, lstart[c]);
        if (c < E + G) return xch_pack(gtot[c - E], lgstart[c - E]);
        if (c == E + G) return xch_pack(npairs, s_gpairs);
        if (c == E + G + 1) return xch_err_pack(s_err);
        return 0u;   // the padding column
    };
    auto expert_count = [&](int c) -> int {
        int n = 0;
#pragma unroll
        for (int w = 0; w < kXW; ++w) n += __popc(ew[c * kXW + w]);
        return n;
    };
    // Publish it, for the columns c = tid + jj * 512 (an expert's count is this
    // thread's cnt_x[jj]).
    const bool xch = xt != nullptr && !recount;   // uniform
    if (xch) {
#pragma unroll
        for (int jj = 0; jj < NCOL; ++jj) {
            const int c = tid + jj * kXT;
            if (c < rows) xch_put(xt + (size_t)tile * rows + c, tag, own_value(c, jj < NX ? cnt_x[jj] : 0));
        }
    }

    // Each of this lane's entries' rank inside the tile (lr among the tile's
    // pairs of its expert, lg of its group) and its place li in the tile's pair
    // list, where its pair id is staged. (LDS reads from clamped indices,
    // masked afterwards: a read under a lane-dependent branch gets a branch and
    // a wait of its own.)
    const size_t p0 = (size_t)t * K;
    int lr[KH], lg[KH], li[KH];
#pragma unroll
    for (int q = 0; q < KH; ++q) {
        const bool v = (ok_q >> q) & 1u;
        const int x = v ? own[q] : 0, g = group_of(x, gmagic);
        lr[q] = loff_e[x * kXW + wave] + __popc(ew[x * kXW + wave] & below);
        lg[q] = loff_g[g][wave] + __popc(gball[g][wave] & below);
        li[q] = lstart[x] + lr[q];
    }
#pragma unroll
    for (int q = 0; q < KH; ++q)
        if ((ok_q >> q) & 1u) s_src[li[q]] = (int32_t)(p0 + h * KH + q);

    // Every tile's values of the column pairs this thread owns (columns 2p and
    // 2p + 1, p = tid + jj * 512), summed: a column's total, its offset (the
    // tiles' prefixes summed) and its count in the tiles before this one. A
    // pair is one 16-byte read per tile, and a wave reads consecutive pairs of
    // one tile row; kXB tiles per round, their reads in flight together; a
    // round is read again until each of its entries carries the tag or the
    // wait runs out (both uniform per wave). Within a round the packed values
    // are summed whole (no carry crosses a 16-bit field in 16 tiles). (A
    // 16-byte read racing with the 8-byte atomic stores of its two entries can
    // see one old and one new, never half of an entry, both being single
    // requests within one cache line.) With one tile the values are this
    // tile's own.
    // With more than one round of tiles (and E <= 512) the waves without pairs
    // read too: reader group r (waves r * wpp .. r * wpp + wpp - 1) takes the
    // rounds r, r + nrg, ...; the groups after the first leave their sums in
    // LDS for the first, whose threads own the columns.
    const int npair = rows / 2;
    const int wpp = (npair + kWave - 1) / kWave;   // waves per set of pairs
    const int nrg = kMR ? max(1, min(kXW / wpp, (ntiles + kXB - 1) / kXB)) : 1;
    const int rg = kMR ? wave / wpp : 0;           // this wave's reader group (idle if >= nrg)
    int ctot[2 * NX], coff[2 * NX], cpre[2 * NX];
#pragma unroll
    for (int q = 0; q < 2 * NX; ++q) ctot[q] = coff[q] = cpre[q] = 0;
    if (xch) {
        const __amdgpu_buffer_rsrc_t tab =
            __builtin_amdgcn_make_buffer_rsrc(xt, (short)0, ntiles * rows * 8, 0x00020000);
        const uint64_t t0 = wall_clock64();
        bool late = false;
#pragma unroll
        for (int jj = 0; jj < NX; ++jj) {
            // uniform per wave: in a reader group (one pair set: some lane has a pair)
            if (kMR ? rg < nrg : jj * kXT + wave * kWave < npair) {
                const int p = kMR ? (wave - rg * wpp) * kWave + lane : tid + jj * kXT;
                const int pc = p < npair ? p : npair - 1;
                for (int b0 = rg * kXB; b0 < ntiles && !late; b0 += nrg * kXB) {
                    u32x4 v[kXB];
                    while (true) {
                        // The offset passes through an empty asm on each pass, so
                        // the compiler cannot take the reads as loop-invariant and
                        // hoist them out of the wait (the buffer-load builtin counts
                        // as a plain read of its buffer).
                        int off = pc * 16;
                        __asm__ volatile("" : "+v"(off));
#pragma unroll
                        for (int u = 0; u < kXB; ++u) {
                            const int b = b0 + u < ntiles ? b0 + u : ntiles - 1;
                            v[u] = __builtin_amdgcn_raw_buffer_load_b128(tab, off, b * rows * 8, kCpolSc1);
                        }
                        uint32_t miss = 0;
#pragma unroll
                        for (int u = 0; u < kXB; ++u)
                            miss |= b0 + u < ntiles ? (v[u].y ^ tag) | (v[u].w ^ tag) : 0u;
                        if (__all(miss == 0)) break;
                        if (wall_clock64() - t0 > wait_ticks) {
                            late = true;
                            break;
                        }
                        __builtin_amdgcn_s_sleep(2);
                    }
                    uint32_t s0 = 0, s1 = 0, p0s = 0, p1s = 0;
#pragma unroll
                    for (int u = 0; u < kXB; ++u) {
                        s0 += b0 + u < ntiles ? v[u].x : 0u;
                        s1 += b0 + u < ntiles ? v[u].z : 0u;
                        p0s += b0 + u < tile ? v[u].x : 0u;
                        p1s += b0 + u < tile ? v[u].z : 0u;
                    }
                    ctot[2 * jj] += (int)(s0 & 0xFFFFu);
                    coff[2 * jj] += (int)(s0 >> 16);
                    cpre[2 * jj] += (int)(p0s & 0xFFFFu);
                    ctot[2 * jj + 1] += (int)(s1 & 0xFFFFu);
                    coff[2 * jj + 1] += (int)(s1 >> 16);
                    cpre[2 * jj + 1] += (int)(p1s & 0xFFFFu);
                }
            }
        }
        if (kMR && rg > 0 && rg < nrg) {
            const int p = (wave - rg * wpp) * kWave + lane;
            if (p < npair) {
                int *sp = s_part[(rg - 1) * npair + p];
                sp[0] = ctot[0];
                sp[1] = coff[0];
                sp[2] = cpre[0];
                sp[3] = ctot[1];
                sp[4] = coff[1];
                sp[5] = cpre[1];
            }
        }
        if (late) s_late = 1;
    } else if (!recount) {
#pragma unroll
        for (int jj = 0; jj < NX; ++jj) {
            const int pc = tid + jj * kXT;
            if (pc < npair) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int c = 2 * pc + hh;
                    const uint32_t w = own_value(c, c < E ? expert_count(c) : 0);
                    ctot[2 * jj + hh] = (int)(w & 0xFFFFu);
                    coff[2 * jj + hh] = (int)(w >> 16);
                }
            }
        }
    }
    __syncthreads();
    const bool fell_back = s_late != 0;   // uniform
    if (kMR && xch && !fell_back && tid < npair) {
        for (int r = 1; r < nrg; ++r) {
            const int *sp = s_part[(r - 1) * npair + tid];
            ctot[0] += sp[0];
            coff[0] += sp[1];
            cpre[0] += sp[2];
            ctot[1] += sp[3];
            coff[1] += sp[4];
            cpre[1] += sp[5];
        }
    }
    if (!fell_back) {
        // Each owned column's results: an expert's (group's) first receive row
        // in this tile is its offset + its count in earlier tiles; tile 0
        // writes the counts, offsets and status.
#pragma unroll
        for (int jj = 0; jj < NX; ++jj) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int c = 2 * (tid + jj * kXT) + hh;
                const int tot = ctot[2 * jj + hh], off = coff[2 * jj + hh], pre = cpre[2 * jj + hh];
                if (c < E) {
                    base_e[c] = off + pre;
                    if (tile == 0) {
                        L.expert_count[c] = tot;
                        L.expert_offset[c] = off;
                    }
                } else if (c < E + G) {
                    base_g[c - E] = off + pre;
                    if (tile == 0) {
                        L.group_count[c - E] = tot;
                        L.group_offset[c - E] = off;
                    }
                } else if (c == E + G && tile == 0) {
                    L.expert_offset[E] = tot;
                    L.group_offset[G] = off;
                } else if (c == E + G + 1 && tile == 0) {
                    *L.status = xch_err_unpack((uint32_t)tot);
                }
            }
        }
    } else {
        xch_recount<KMAX, EXACT>(idx, T, K, E, G, gmagic, tile, s_tot, s_pre);
        xch_fallback_offsets<NX>(E, G, tile, s_tot, s_pre, base_e, base_g, s_wave_tot, L);
    }
    __syncthreads();   // base_e, base_g

    // Slots: base + rank inside the tile, this lane's KH entries.
    if (t < T) {
        int se[KH], sg[KH];
#pragma unroll
        for (int q = 0; q < KH; ++q) {
            const bool v = (ok_q >> q) & 1u;
            const int x = v ? own[q] : 0;
            const int be = base_e[x], bg = base_g[group_of(x, gmagic)];
            se[q] = v ? be + lr[q] : -1;
            sg[q] = v ? bg + lg[q] : -1;
        }
        const size_t pk = p0 + h * KH;   // this lane's first entry
        if (EXACT && (vec & 1)) {        // 16-byte aligned slot arrays, K in {2, 4, 8}
            if constexpr (KH == 4) {
                *reinterpret_cast<u32x4 *>(L.slot_e + pk) =
                    u32x4{(uint32_t)se[0], (uint32_t)se[1], (uint32_t)se[2], (uint32_t)se[3]};
                *reinterpret_cast<u32x4 *>(L.slot_g + pk) =
                    u32x4{(uint32_t)sg[0], (uint32_t)sg[1], (uint32_t)sg[2], (uint32_t)sg[3]};
            } else if constexpr (KH == 2) {
                *reinterpret_cast<u32x2 *>(L.slot_e + pk) = u32x2{(uint32_t)se[0], (uint32_t)se[1]};
                *reinterpret_cast<u32x2 *>(L.slot_g + pk) = u32x2{(uint32_t)sg[0], (uint32_t)sg[1]};
            } else {
                L.slot_e[pk] = se[0];
                L.slot_g[pk] = sg[0];
            }
        } else {
#pragma unroll
            for (int q = 0; q < KH; ++q) {
                if (h * KH + q < K) {
                    L.slot_e[pk + q] = se[q];
                    L.slot_g[pk + q] = sg[q];
                }
            }
        }
#pragma unroll
        for (int q = 0; q < KH; ++q)
            if ((ok_q >> q) & 1u) s_dst[li[q]] = se[q];
        // the token's groups, in blocks of 4: lane h takes the blocks 4 * (2 i + h)
        int32_t *tg = L.slot_tg + (size_t)t * G;
        for (int g0 = 4 * h; g0 < G; g0 += 8) {
            int r4[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int g = g0 + u < kMaxG ? g0 + u : kMaxG - 1;
                const int r = base_g[g] + loff_g[g][wave] + __popc(gball[g][wave] & below);
                r4[u] = g0 + u < G && ((gm >> (g0 + u)) & 1u) ? r : -1;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (r4[u] >= 0) L.recv_src_g[r4[u]] = t;
            if (vec & 2) {   // G % 4 == 0 and slot_tg 16-byte aligned
                *reinterpret_cast<u32x4 *>(tg + g0) = u32x4{(uint32_t)r4[0], (uint32_t)r4[1], (uint32_t)r4[2], (uint32_t)r4[3]};
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (g0 + u < G) tg[g0 + u] = r4[u];
            }
        }
    }
    __syncthreads();
    tile_write_recv_src_e(npairs, s_src, s_dst, L.recv_src_e, tid, kXT);
}

using ExchangeFn = void (*)(const int32_t *, int, int, int, int, int, uint32_t, int, uint64_t *, uint32_t, uint64_t,
                            int, LayoutPtrs);

template <int NX, bool MR>
ExchangeFn pick_exchange_n(int K)
{
    switch (K) {
    case 2: return layout_exchange_kernel<2, true, NX, MR>;
    case 4: return layout_exchange_kernel<4, true, NX, MR>;
    case 8: return layout_exchange_kernel<8, true, NX, MR>;
    default: return layout_exchange_kernel<8, false, NX, MR>;
    }
}

// The reader groups only where there are at least two (more than one round
// of tiles, and idle waves for a second set of pairs): the other instance stays
// as compact as it was (the groups' code cost it registers and 0.5 µs at 16
// tiles, 0.8 µs at 32 tiles of E = 512 with one group).
ExchangeFn pick_exchange(int K, int E, int G, int ntiles)
{
    static_assert(2 * kXT >= 1024, "E <= 1024 in two chunks");
    constexpr int kRound = 16;   // tiles per round of reads
    if (E > kXT) return pick_exchange_n<2, false>(K);
    const int npair = ((E + G + 3) & ~1) / 2, wpp = (npair + kWave - 1) / kWave;
    const int groups = std::min(kXW / wpp, (ntiles + kRound - 1) / kRound);
    return groups >= 2 ? pick_exchange_n<1, true>(K) : pick_exchange_n<1, false>(K);
}

// Exchange tables of the one-launch layout, in library memory (zero when the
// library is loaded): one table of kXchEntries 64-bit entries for each of up to
// kXchSlots streams per GPU. In host code `xch_tables` only names the symbol;
// its address on each GPU comes from hipGetSymbolAddress (xch_slot).
constexpr int kXchSlots = 8;
constexpr size_t kXchEntries = (size_t)64 * (1024 + 32 + 4);   // 64 tiles of the widest row (E = 1024, G = 32): 530 KiB per table
// Most tiles of one exchange. Every tile's workgroup waits for all the others,
// so all of them must be able to run at once: 128 workgroups take at most half
// of the chip's 256 CUs, leaving room for other work on the GPU. (A workgroup
// whose wait runs out still finishes exactly, by recounting.)
constexpr int kXchMaxTiles = 128;
__device__ __align__(256) uint64_t xch_tables[kXchSlots * kXchEntries];

constexpr int kXchMaxDevices = 64;
struct XchDevice {
    uint64_t *tables = nullptr;        // address of xch_tables on this GPU
    hipStream_t stream[kXchSlots] = {};
    uint32_t seq[kXchSlots] = {};      // the last tag given out on each stream's table
    int used = 0;
};
std::mutex g_xch_mu;
XchDevice g_xch[kXchMaxDevices];

// The exchange table of `stream` and this call's tag on it: the stream's
// previous tag + 1. Calls on one stream run in order, so a table is never
// used by two calls at once unless the caller reuses a stream handle across
// threads or devices in ways HIP does not order; even then an entry is only
// taken when it carries the reader's own tag, so a clash costs a timed-out
// wait, never a wrong count. *xt stays NULL (the caller takes the two-launch
// layout) for a stream under graph capture (a replay would repeat the tag),
// for the per-thread default stream (its calls from different threads are not
// ordered) and for streams beyond kXchSlots on one GPU.
hipError_t xch_slot(hipStream_t stream, uint64_t **xt, uint32_t *tag)
{
    *xt = nullptr;
    if (stream == hipStreamPerThread) return hipSuccess;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
        (void)hipGetLastError();   // not ours to report; take the two-launch form
        return hipSuccess;
    }
    if (cs != hipStreamCaptureStatusNone) return hipSuccess;
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    int dev = cur;
    if (stream) {
        hipDevice_t sd = -1;
        if ((e = hipStreamGetDevice(stream, &sd)) != hipSuccess) return e;
        dev = sd;
    }
    if (dev < 0 || dev >= kXchMaxDevices) return hipSuccess;
    std::lock_guard<std::mutex> lock(g_xch_mu);
    XchDevice &d = g_xch[dev];
    if (!d.tables) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(xch_tables));
        if (dev != cur) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        d.tables = static_cast<uint64_t *>(p);
    }
    int s = 0;
    while (s < d.used && d.stream[s] != stream) ++s;
    if (s == d.used) {
        if (d.used == kXchSlots) return hipSuccess;
        d.stream[s] = stream;
        d.seq[s] = 0;
        ++d.used;
    }
    uint64_t *tab = d.tables + (size_t)s * kXchEntries;
    if (d.seq[s] == 0xFFFFFFFFu) {   // every tag used: clear the table in stream order and start again
        if ((e = hipMemsetAsync(tab, 0, sizeof(uint64_t) * kXchEntries, stream)) != hipSuccess) return e;
        d.seq[s] = 0;
    }
    *tag = ++d.seq[s];
    *xt = tab;
    return hipSuccess;
}

}  // namespace

hipError_t launch_layout_exchange(const int32_t *idx, int T, int K, int E, int G, const LayoutPtrs &L, int vec,
                                  hipStream_t stream, bool &launched)
{
    launched = false;
    const int ntiles = layout_tiles(T);
    const int rows = (E + G + 3) & ~1;   // exchange table columns (even)
    if (T == 0 || K > 8 || ntiles > tuning().layout_exchange_max_tiles || ntiles > kXchMaxTiles ||
        (size_t)ntiles * rows > kXchEntries)
        return hipSuccess;
    uint64_t *xt = nullptr;
    uint32_t tag = 0;
    if (ntiles > 1) {
        const hipError_t e = xch_slot(stream, &xt, &tag);
        if (e != hipSuccess || !xt) return e;
    }
    const long long wt = tuning().base_wait_ticks;
    const size_t lds = (size_t)E * kXW * sizeof(uint32_t) +
                       ((size_t)E * (kXW + 2) + 2 * (size_t)(E + G + 1)) * sizeof(int);
    hipLaunchKernelGGL(pick_exchange(K, E, G, ntiles), dim3(ntiles), dim3(kXT), lds, stream, idx, T, vec, K, E, G,
                       group_magic(E, G), ntiles, xt, tag, (uint64_t)(wt < 0 ? 0 : wt), wt < 0 ? 1 : 0, L);
    launched = true;
    return hipGetLastError();
}

}  // namespace moe
