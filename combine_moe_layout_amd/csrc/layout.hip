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
// which is the stable token-ascending order, and a token's repeated expert is
// seen as its own bit already set. Groups use one ballot per group per wave.
//
// Kernel 1 (count): per tile, expert and group counts + error bits -> workspace.
// Kernel 2 (place): every tile re-reads the [E][tiles] count table it needs
// (tiny: E * tiles ints), forms global offsets = exclusive prefix over experts
// of the totals + prefix over earlier tiles, rebuilds its LDS words and
// writes the slots and receive-source lists. Tile 0 also writes the counts,
// offsets and status.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kWaves = kLayoutTile / kWave;   // 4
constexpr int kMaxG = 32;

// Insert token t's valid experts into the LDS words; returns the bitmask of
// k positions that are invalid (out of range, or a repeat of an earlier k),
// and ORs error bits into err and the token's groups into gm.
__device__ __forceinline__ uint32_t insert_token(const int32_t *__restrict__ row, int K, int E,
                                                 int epg, unsigned long long *emask, int wave,
                                                 int lane, int &err, uint32_t &gm)
{
    const unsigned long long bit = 1ull << lane;
    uint32_t bad = 0;
    for (int k = 0; k < K; ++k) {
        const int e = row[k];
        if ((unsigned)e >= (unsigned)E) { err |= 1; bad |= 1u << k; continue; }
        const unsigned long long old = atomicOr(&emask[e * kWaves + wave], bit);
        if (old & bit) { err |= 2; bad |= 1u << k; continue; }
        gm |= 1u << (e / epg);
    }
    return bad;
}

__global__ __launch_bounds__(kLayoutTile) void layout_count_kernel(
    const int32_t *__restrict__ idx, int T, int K, int E, int G, int epg, int ntiles,
    uint32_t *__restrict__ tok_group_mask, int32_t *__restrict__ tile_cnt_e,
    int32_t *__restrict__ tile_cnt_g, int32_t *__restrict__ tile_err)
{
    extern __shared__ unsigned long long emask[];   // [E][kWaves]
    __shared__ int gcnt[kMaxG][kWaves];
    __shared__ int s_err;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int tile = blockIdx.x;
    for (int i = tid; i < E * kWaves; i += kLayoutTile) emask[i] = 0ull;
    if (tid == 0) s_err = 0;
    __syncthreads();

    const int t = tile * kLayoutTile + tid;
    int err = 0;
    uint32_t gm = 0;
    if (t < T) {
        insert_token(idx + (size_t)t * K, K, E, epg, emask, wave, lane, err, gm);
        tok_group_mask[t] = gm;
    }
    for (int g = 0; g < G; ++g) {
        const uint64_t b = __ballot((gm >> g) & 1u);
        if (lane == 0) gcnt[g][wave] = __popcll(b);
    }
    if (err) atomicOr(&s_err, err);
    __syncthreads();

    for (int e = tid; e < E; e += kLayoutTile) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) c += __popcll(emask[e * kWaves + w]);
        tile_cnt_e[(size_t)e * ntiles + tile] = c;
    }
    if (tid < G) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) c += gcnt[tid][w];
        tile_cnt_g[(size_t)tid * ntiles + tile] = c;
    }
    if (tid == 0) tile_err[tile] = s_err;
}

// Exclusive prefix sum over the 256 threads of the workgroup.
__device__ __forceinline__ int block_exclusive_scan(int v, int *s_wave_tot)
{
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    int x = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == kWave - 1) s_wave_tot[wave] = x;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += s_wave_tot[w];
    return base + x - v;
}

__global__ __launch_bounds__(kLayoutTile) void layout_place_kernel(
    const int32_t *__restrict__ idx, int T, int K, int E, int G, int epg, int ntiles,
    const int32_t *__restrict__ tile_cnt_e, const int32_t *__restrict__ tile_cnt_g,
    const int32_t *__restrict__ tile_err, LayoutPtrs L)
{
    extern __shared__ unsigned long long emask[];   // [E][kWaves], then int base_e[E]
    int *base_e = reinterpret_cast<int *>(emask + E * kWaves);
    __shared__ int s_wave_tot[kWaves];
    __shared__ int base_g[kMaxG];
    __shared__ int tot_g[kMaxG];
    __shared__ uint64_t gball[kMaxG][kWaves];
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int tile = blockIdx.x;

    for (int i = tid; i < E * kWaves; i += kLayoutTile) emask[i] = 0ull;

    // Global offsets of this tile: experts e = tid*ept .. tid*ept+ept-1 per thread.
    const int ept = (E + kLayoutTile - 1) / kLayoutTile;   // <= 4
    int tot[4] = {0, 0, 0, 0}, pre[4] = {0, 0, 0, 0};
    int local = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = tid * ept + j;
        if (j < ept && e < E) {
            const int32_t *row = tile_cnt_e + (size_t)e * ntiles;
            for (int b = 0; b < ntiles; ++b) {
                const int c = row[b];
                tot[j] += c;
                if (b < tile) pre[j] += c;
            }
            local += tot[j];
        }
    }
    const int excl = block_exclusive_scan(local, s_wave_tot);
    int run = excl;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = tid * ept + j;
        if (j < ept && e < E) {
            base_e[e] = run + pre[j];
            if (tile == 0) {
                L.expert_count[e] = tot[j];
                L.expert_offset[e] = run;
            }
            run += tot[j];
        }
    }
    if (tile == 0 && tid == kLayoutTile - 1) L.expert_offset[E] = excl + local;

    if (tid < G) {
        int tg = 0, pg = 0;
        for (int b = 0; b < ntiles; ++b) {
            const int c = tile_cnt_g[(size_t)tid * ntiles + b];
            tg += c;
            if (b < tile) pg += c;
        }
        tot_g[tid] = tg;
        base_g[tid] = pg;
    }
    __syncthreads();
    if (tid == 0) {
        int off = 0;
        for (int g = 0; g < G; ++g) {
            if (tile == 0) {
                L.group_count[g] = tot_g[g];
                L.group_offset[g] = off;
            }
            base_g[g] += off;
            off += tot_g[g];
        }
        if (tile == 0) {
            L.group_offset[G] = off;
            int st = 0;
            for (int b = 0; b < ntiles; ++b) st |= tile_err[b];
            *L.status = st;
        }
    }

    // Rebuild the tile's LDS words exactly as the count kernel did.
    const int t = tile * kLayoutTile + tid;
    const int32_t *row = idx + (size_t)t * K;
    int err = 0;
    uint32_t gm = 0, bad = 0;
    if (t < T) bad = insert_token(row, K, E, epg, emask, wave, lane, err, gm);
    for (int g = 0; g < G; ++g) {
        const uint64_t b = __ballot((gm >> g) & 1u);
        if (lane == 0) gball[g][wave] = b;
    }
    __syncthreads();
    if (t >= T) return;

    const uint64_t below = lanemask_lt(lane);
    auto group_slot = [&](int g) {
        int r = base_g[g];
        for (int w = 0; w < wave; ++w) r += __popcll(gball[g][w]);
        return r + __popcll(gball[g][wave] & below);
    };
    for (int k = 0; k < K; ++k) {
        const size_t p = (size_t)t * K + k;
        if ((bad >> k) & 1u) {
            L.slot_e[p] = -1;
            L.slot_g[p] = -1;
            continue;
        }
        const int e = row[k];
        int r = base_e[e];
        for (int w = 0; w < wave; ++w) r += __popcll(emask[e * kWaves + w]);
        r += __popcll(emask[e * kWaves + wave] & below);
        L.slot_e[p] = r;
        L.recv_src_e[r] = (int32_t)p;
        L.slot_g[p] = group_slot(e / epg);
    }
    for (int g = 0; g < G; ++g) {
        int s = -1;
        if ((gm >> g) & 1u) {
            s = group_slot(g);
            L.recv_src_g[s] = t;
        }
        L.slot_tg[(size_t)t * G + g] = s;
    }
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

hipError_t launch_layout(const int32_t *idx, int T, int K, int E, int G, const LayoutPtrs &L,
                         int32_t *ws, hipStream_t stream)
{
    if (T == 0) {
        hipLaunchKernelGGL(layout_empty_kernel, dim3(1), dim3(kLayoutTile), 0, stream, E, G, L);
        return hipGetLastError();
    }
    const int ntiles = layout_tiles(T);
    const int epg = E / G;
    int32_t *tile_cnt_e = ws;
    int32_t *tile_cnt_g = tile_cnt_e + (size_t)E * ntiles;
    int32_t *tile_err = tile_cnt_g + (size_t)G * ntiles;
    const size_t lds1 = (size_t)E * kWaves * sizeof(unsigned long long);
    const size_t lds2 = lds1 + (size_t)E * sizeof(int);
    hipLaunchKernelGGL(layout_count_kernel, dim3(ntiles), dim3(kLayoutTile), lds1, stream, idx, T, K,
                       E, G, epg, ntiles, L.tok_group_mask, tile_cnt_e, tile_cnt_g, tile_err);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(layout_place_kernel, dim3(ntiles), dim3(kLayoutTile), lds2, stream, idx, T, K,
                       E, G, epg, ntiles, tile_cnt_e, tile_cnt_g, tile_err, L);
    return hipGetLastError();
}

}  // namespace moe
