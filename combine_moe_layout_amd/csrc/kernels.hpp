// Host-side launchers of the gfx950 kernels. Arguments are already validated
// by the C ABI (api.hip); each launcher only picks a kernel instance and
// launches it on `stream`, returning the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Tokens per layout tile (= threads per layout workgroup).
constexpr int kLayoutTile = 256;

inline int layout_tiles(int T) { return (T + kLayoutTile - 1) / kLayoutTile; }

// Layout workspace, in 32-bit words:
//   table  [tiles][E + G + 1]   per-tile expert counts, group counts, error bits
//                               (padded to a multiple of 64 words)
//   words  [tiles][E][4][2]     per-(expert, wave) token masks of each tile, as
//                               32-bit halves (top-k <= 8)
//   gwords [tiles][G][4][2]     per-(group, wave) token masks (top-k <= 8)
//   bases  [tiles][E + G]       first receive row of each tile in each expert
//                               (group) segment: the segment's offset plus the
//                               counts of the tiles before (fused path only)
struct LayoutWs {
    int32_t *table;
    uint32_t *words, *gwords;
    int32_t *bases;
};
inline size_t layout_table_words(int tiles, int E, int G)
{
    return ((size_t)tiles * (E + G + 1) + 63) & ~(size_t)63;
}
inline size_t layout_ws_words(int T, int E, int G)
{
    const size_t tiles = (size_t)layout_tiles(T);
    return layout_table_words((int)tiles, E, G) + tiles * E * 8 + tiles * G * 8 + tiles * (E + G);
}
inline size_t layout_ws_bytes_for(int T, int E, int G) { return 4 * layout_ws_words(T, E, G); }
inline LayoutWs layout_ws(void *ws, int T, int E, int G)
{
    const size_t tiles = (size_t)layout_tiles(T);
    int32_t *base = static_cast<int32_t *>(ws);
    LayoutWs w;
    w.table = base;
    w.words = reinterpret_cast<uint32_t *>(base + layout_table_words((int)tiles, E, G));
    w.gwords = w.words + tiles * E * 8;
    w.bases = reinterpret_cast<int32_t *>(w.gwords + tiles * G * 8);
    return w;
}

struct LayoutPtrs {
    int32_t *expert_count, *expert_offset, *group_count, *group_offset;
    uint32_t *tok_group_mask;
    int32_t *slot_e, *slot_g, *slot_tg, *recv_src_e, *recv_src_g, *status;
};

// moe_layout: count + place kernels (ws: the layout workspace above).
hipError_t launch_layout(const int32_t *idx, int T, int K, int E, int G, const LayoutPtrs &L,
                         int32_t *ws, hipStream_t stream);

// The one-launch exchange layout (layout_exchange.hip) when it applies (top-k
// <= 8, T >= 1, at most the tuned number of tiles, an exchange table free for
// the stream); `launched` tells whether it ran. vec: bit 0 slot_e and slot_g,
// bit 1 slot_tg (with G % 4 == 0), bit 2 the index rows, 16-byte aligned.
hipError_t launch_layout_exchange(const int32_t *idx, int T, int K, int E, int G, const LayoutPtrs &L, int vec,
                                  hipStream_t stream, bool &launched);

// First half of the fused layout + dispatch for T > the small-batch limit
// and top-k <= 8: the count kernel, which also sets every tile's bases in
// the workspace to -1 and the status to 0; then, unless `finalize_in_dispatch`,
// one workgroup that writes the counts, offsets and status and each tile's
// bases. The dispatch kernels then place each token themselves (PlaceArgs);
// with `finalize_in_dispatch` their workgroup 0 computes the bases first.
hipError_t launch_layout_count_finalize(const int32_t *idx, int T, int K, int E, int G,
                                        const LayoutPtrs &L, int32_t *ws, bool finalize_in_dispatch,
                                        hipStream_t stream);

// Tiles per batch of the count-table loads of an in-dispatch finalize.
constexpr int kFinTiles = 16;

// What a dispatch kernel needs to compute its token's slots and write the
// token's layout entries (see place_token in place.hpp).
struct PlaceArgs {
    const int32_t *idx;
    int E, G;
    uint32_t gmagic;
    const uint32_t *words, *gwords;
    int32_t *bases;            // [tiles][E + G]; -1 until written
    const int32_t *table;      // the count kernel's per-tile counts and error bits
    int ntiles;
    int finalize;              // 1: workgroup 0 computes the bases, counts, offsets and status
    uint64_t wait_ticks;       // longest wait for a tile's bases (constant 100 MHz clock)
    int self_bases;            // 1: every token computes its bases from the table (no wait; tests)
    LayoutPtrs L;
    int mode;   // destinations: slot_e (0) or slot_tg (1)
};
inline uint32_t group_magic(int E, int G)
{
    const int epg = E / G;
    return epg == 1 ? 0u : (uint32_t)((1ull << 32) / (unsigned)epg) + 1u;
}

// Cache policy of the dispatch row loads and stores, the FP8 dispatch's form
// and the largest batch of the one-launch layout. Defaults are the measured
// best on MI355X; MOE_EP_DISPATCH_NT_{LOAD,STORE}=0/1, MOE_EP_FP8_FORM=0/1/2,
// MOE_EP_FP8_GROUP_W4=0/1, MOE_EP_FUSED_FP8_PLACE_MAX_T=<T>, MOE_EP_{LAYOUT,FUSED}_ONEPASS_MAX_PAIRS=<T*K>,
// MOE_EP_FUSED_SMALL_MAX_WORK=<T*K*E>, MOE_EP_LAYOUT_EXCHANGE_MAX_TILES=<tiles>,
// MOE_EP_FUSED_FINALIZE=0/1/2, MOE_EP_FUSED_FINALIZE_ROUNDS=<n>, MOE_EP_DISPATCH_SPLIT_MAX_WGS=<n> and
// MOE_EP_BASE_WAIT_TICKS=<ticks> in the environment override them (read once per
// process) for A/B runs and tests.
struct Tuning {
    bool dispatch_nt_load = true;    // x rows are read once
    bool dispatch_nt_store = false;  // receive rows
    int fp8_form = 1;                // FP8 dispatch: 0 row-sized workgroups, 1 one wave
                                     // per token, 2 two waves per token (H <= 16 * BS * 8)
    bool fp8_group_w4 = true;        // plain per-group FP8 dispatch at 4 waves per SIMD
    int fused_fp8_place_max_t = 3072;  // moe_layout_dispatch with FP8: a placing dispatch up
                                       // to this T, moe_layout + the plain dispatch above
    int layout_exchange_max_tiles = 128;    // moe_layout in one launch exchanging per-tile counts, up to
                                            // this many tiles of 256 tokens (top-k <= 8; at most 128;
                                            // 0: never)
    int layout_onepass_max_pairs = 16384;   // else in one launch counting every token per tile, up to
                                            // T * K pairs (top-k <= 8)
    int fused_onepass_max_pairs = 0;        // moe_layout_dispatch as that layout + a plain dispatch
    int fused_small_max_work = 4096;        // moe_layout_dispatch in one launch up to T * K * E
    long long base_wait_ticks = 20000000;   // placing dispatch: longest wait for a tile's bases
                                            // (0.2 s at 100 MHz) before a token computes them
                                            // itself; 0 makes most tokens do so, -1 every token
                                            // (tests of that path)
    int fused_finalize = 2;                 // placing dispatch: 0 the finalize kernel, 1 its
                                            // workgroup 0 (bf16), 2 workgroup 0 (bf16 and FP8)
    int fused_finalize_rounds = 4;          // ... for E up to this many columns per thread
    bool regroup_xcd_order = true;          // regroup: each XCD takes a contiguous run of group rows
    int dispatch_split_max_wgs = 4096;      // plain bf16 dispatch: a workgroup per (token, row slice)
                                            // while T * slices stays within this (0: never)
};
const Tuning &tuning();
// Whether the FP8 dispatch of rows of H elements runs in a small-workgroup form.
bool fp8_wave_form(int H);
// Threads per workgroup of the placing dispatch (FP8: of its small-workgroup form).
int placing_dispatch_threads(bool fp8, int H);

// BF16 dispatch. slots: [T, nslot] (slot_e with nslot = K, or slot_tg with nslot = G).
// place: NULL to read the destinations from `slots`, else the token's slots
// are computed in the kernel (fused layout + dispatch; `slots` unused).
hipError_t launch_dispatch_bf16(const void *x, int T, int H, int K, int nslot, const int32_t *slots,
                                const float *topk_w, const int32_t *topk_idx, void *recv_x,
                                float *recv_w, int32_t *recv_idx, const PlaceArgs *place,
                                hipStream_t stream);

// group_rows: the destinations are per-group rows (chooses the instance).
hipError_t launch_dispatch_fp8(const void *x, int T, int H, int K, int nslot, const int32_t *slots,
                               const float *topk_w, const int32_t *topk_idx, void *recv_q,
                               float *recv_scale, float *recv_w, int32_t *recv_idx,
                               const PlaceArgs *place, bool group_rows, hipStream_t stream);

// Combine. slot: [T, K] (slot_e, or slot_g whose entries may repeat within a token).
hipError_t launch_combine(const void *y, int64_t y_rows, int T, int H, int K, const int32_t *slot,
                          bool rows_repeat, const float *topk_w, void *out, int32_t *status,
                          hipStream_t stream);

// FP8 identity expert; rows to convert = *nrows (device), grid covers `capacity` rows.
hipError_t launch_fp8_dequant(const void *q, const float *scale, void *y, int64_t capacity, int H,
                              const int32_t *nrows, hipStream_t stream);

hipError_t launch_ref_copy(void *dst, const void *src, int64_t bytes, hipStream_t stream);
// (nr, nw): (1, 1), (2|4|8, 1) or (1, 2|4|8), checked by the caller.
hipError_t launch_ref_mix(void *dst, const void *src, int64_t row_bytes, int64_t units, int nr, int nw,
                          hipStream_t stream);

// Receive-side regroup: per-group rows -> per-expert rows (row_bytes % 16 == 0).
hipError_t launch_regroup(const void *in_rows, int row_bytes, const float *in_scale, int nscale,
                          const float *in_w, const int32_t *in_idx, int T, int K, int G,
                          const int32_t *group_offset, const int32_t *recv_src_g,
                          const int32_t *slot_g, const int32_t *slot_e, void *out_rows,
                          float *out_scale, float *out_w, int32_t *out_idx, hipStream_t stream);

// Per-expert FP8 cast + padded transpose.
int64_t cast_transpose_t_bound(int64_t rows, int E, int H);
hipError_t launch_cast_transpose(const void *x, int64_t rows_bound, int H, int E,
                                 const int32_t *expert_offset, const float *scale, void *c_out,
                                 void *t_out, float *amax, int32_t *pad_offset, hipStream_t stream);

// Fused layout + dispatch for small batches (one workgroup per token).
constexpr int kFusedMaxT = 512;
constexpr int kFusedMaxPairs = 16384;   // T * K
size_t fused_lds_bytes(int T, int K, int E, int G);
hipError_t launch_layout_dispatch(const int32_t *idx, int T, int K, int E, int G, const LayoutPtrs &L,
                                  int mode, int fp8, int H, const void *x, const float *topk_w,
                                  void *recv_x, float *recv_scale, float *recv_w, int32_t *recv_idx,
                                  hipStream_t stream);

}  // namespace moe
