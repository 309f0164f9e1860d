// Device pieces shared by the routing-layout kernels of layout.hip and
// layout_exchange.hip: a token's index row in registers, its insertion into
// the tile's per-(expert, wave) LDS words (bit `lane` of the word of (expert,
// wave) is set when that lane's token lists the expert; the rank of an entry
// inside the tile is the popcount of its expert's words of earlier waves plus
// that of its own wave's word below its lane), the classification of a row
// without LDS, the staged receive-list write and a workgroup scan.
#pragma once

#include "moe_ep.h"

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kWaves = kLayoutTile / kWave;   // 4
constexpr int kMaxG = 32;
constexpr int kMaxEChunks = (1024 + kLayoutTile - 1) / kLayoutTile;   // E <= 1024

// A token's K expert indices, loaded into registers at kernel entry so the
// loads overlap other work. The loads are unconditional, from clamped in-range
// addresses (T >= 1), so they issue back to back with no branches; mask_row
// then sets entries k >= K, and every entry of a lane past the last token, to
// -1. (Masking next to the load lets the compiler turn each load into a
// branch with a wait of its own.)
template <int KMAX>
__device__ __forceinline__ void load_row(const int32_t *__restrict__ idx, int t, int T, int K,
                                         int (&e)[KMAX])
{
    const int32_t *row = idx + (size_t)(t < T ? t : T - 1) * K;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) e[k] = row[k < K ? k : K - 1];
}

template <int KMAX>
__device__ __forceinline__ void mask_row(int t, int T, int K, int (&e)[KMAX])
{
#pragma unroll
    for (int k = 0; k < KMAX; ++k) e[k] = (t < T && k < K) ? e[k] : -1;
}

// What inserting one token found: k positions out of range, k positions that
// repeat an earlier k, and the groups the token reaches.
struct Inserted {
    uint32_t oor, dup, gm;
    __device__ int err() const { return (oor ? 1 : 0) | (dup ? 2 : 0); }
    __device__ uint32_t bad() const { return oor | dup; }
};

// Insert a token's valid experts into the LDS words. A token is handled by one
// lane, in k order, so "earlier k" is well defined: an entry repeats iff its
// expert equals an earlier in-range entry of the same token (that entry, or
// the first of its repeats, set the lane's bit). For top-k <= 8 the repeats
// are found by comparing registers, so the LDS ORs return nothing and do not
// wait; for larger k the returned old word tells (the lane's own bit already
// set). (Results are returned by value: with reference out-parameters the
// compiler merged the updates into a dynamically indexed private array, i.e.
// scratch memory.)
template <int KMAX>
__device__ __forceinline__ Inserted insert_token(const int (&e)[KMAX], bool live, int K, int E,
                                                 uint32_t gmagic,
                                                 unsigned long long *emask, int wave, int lane)
{
    const unsigned long long bit = 1ull << lane;
    uint32_t oor = 0, dup = 0, gm = 0;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        const int x = e[k];
        const bool in = live && k < K && (unsigned)x < (unsigned)E;
        oor |= (live && k < K && !in) ? 1u << k : 0u;
        if constexpr (KMAX <= 8) {
            bool rep = false;
#pragma unroll
            for (int j = 0; j < k; ++j) rep = rep || e[j] == x;
            if (in) {
                dup |= rep ? 1u << k : 0u;
                if (!rep) {
                    atomicOr(&emask[x * kWaves + wave], bit);
                    gm |= 1u << group_of(x, gmagic);
                }
            }
        } else {
            if (in) {
                const unsigned long long old = atomicOr(&emask[x * kWaves + wave], bit);
                const bool rep = (old & bit) != 0;
                dup |= rep ? 1u << k : 0u;
                gm |= rep ? 0u : 1u << group_of(x, gmagic);
            }
        }
    }
    return Inserted{oor, dup, gm};
}

// The same classification as insert_token without touching LDS (top-k <= 8),
// for a tile whose words were already built.
template <int KMAX>
__device__ __forceinline__ Inserted classify_token(const int (&e)[KMAX], bool live, int K, int E,
                                                   uint32_t gmagic)
{
    uint32_t oor = 0, dup = 0, gm = 0;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        const int x = e[k];
        const bool in = live && k < K && (unsigned)x < (unsigned)E;
        oor |= (live && k < K && !in) ? 1u << k : 0u;
        bool rep = false;
#pragma unroll
        for (int j = 0; j < k; ++j) rep = rep || e[j] == x;
        if (in) {
            dup |= rep ? 1u << k : 0u;
            gm |= rep ? 0u : 1u << group_of(x, gmagic);
        }
    }
    return Inserted{oor, dup, gm};
}

// The staged expert receive-list entries of a tile, written as runs by
// threads tid, tid + nthreads, ...
__device__ __forceinline__ void tile_write_recv_src_e(int npairs, const int32_t *s_src, const int32_t *s_dst,
                                                      int32_t *recv_src_e, int tid, int nthreads)
{
    for (int i = tid; i < npairs; i += nthreads) recv_src_e[s_dst[i]] = s_src[i];
}

// Exclusive prefix sum over the NW waves of the workgroup; *total gets the sum.
// `first`: no earlier scan may still be reading s_wave_tot (its first barrier
// is then left out).
template <int NW = kWaves>
__device__ __forceinline__ int block_exclusive_scan(int v, int *s_wave_tot, int *total, bool first = false)
{
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int x = wave_incl_scan(v);
    if (!first) __syncthreads();   // s_wave_tot free (a previous scan may still be reading it)
    if (lane == kWave - 1) s_wave_tot[wave] = x;
    __syncthreads();
    int base = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int c = s_wave_tot[w];
        base += w < wave ? c : 0;
        all += c;
    }
    *total = all;
    return base + x - v;
}


}  // namespace

}  // namespace moe
