// Placement of one token inside a dispatch kernel (the fused layout +
// dispatch for large batches): the token's receive slots from the count
// kernel's per-tile token masks and the finalize kernel's per-tile bases.
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
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

__device__ __forceinline__ int place_group_of(int x, uint32_t magic)
{
    return magic == 0 ? x : (int)__umulhi((uint32_t)x, magic);
}

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
        const int g = valid ? place_group_of(e, P.gmagic) : 0;
        const int32_t *tb = P.bases + (size_t)tile * (E + G);
        int se = -1;
        if (valid) se = tb[e] + place_rank(P.words + ((size_t)tile * E + e) * 8, w, l);
        // the groups the token reaches, on every lane
        uint32_t gm = valid ? 1u << g : 0u;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) gm |= __shfl_xor(gm, o);
        int sgl = -1;   // lane g < G: the token's row in group g, or -1
        if (lane < G && ((gm >> lane) & 1u))
            sgl = tb[E + lane] + place_rank(P.gwords + ((size_t)tile * G + lane) * 8, w, l);
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
