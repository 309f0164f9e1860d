// Receive-side regroup: rows in the per-group receive layout (one row per
// token and destination group) -> rows in the per-expert layout (one row per
// token and expert, contiguous per expert), the form a grouped expert GEMM
// consumes. In an expert-parallel deployment this is the receiving rank's
// step after a deduplicated exchange: "Optimizing Distributed Inference
// Kernels for AMD DEVELOPER CHALLENGE 2025", section 3.1, the dispatch-recv
// kernel that copies received tokens into per-local-expert buffers.
//
// Design: one workgroup per group row (the grid covers the row bound; rows
// past the layout's count exit at once), so the group rows are read in order.
// The row is read once into registers (ITER 16-byte vectors per lane) and
// stored to the per-expert rows of its token's pairs in that group (found
// through the cached slots: recv_src_g names the row's token, slot_g the group
// row of each of its pairs, slot_e their expert rows). The K weights and K
// indices of the row, and for e4m3 rows the per-128-block scales, travel with
// it unchanged. Reads each group row once, writes each expert row once: bound
// by HBM like dispatch.
//
// XCD-aware order: workgroups are handed to the 8 XCDs round-robin by
// blockIdx, and each XCD has its own L2. Neighbouring group rows share the
// 128-byte lines of their 32-byte metadata (weights, indices, and the slots of
// neighbouring tokens), so with row = blockIdx each such line is fetched by up
// to four XCDs. The rows are dealt to the XCDs in runs of kRun consecutive rows
// instead (block-cyclic), so a line is fetched by one XCD while all XCDs still
// work on neighbouring runs (one contiguous eighth per XCD measured slower: the
// eight XCDs' stores then go to eight distant regions at once).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kRegroupBS = 128;
constexpr int kMaxIter = 8;
constexpr int kXcds = 8;   // MI355X: 8 XCDs, workgroups assigned round-robin
constexpr int kRun = 16;   // consecutive group rows per XCD
// Smallest row bound given the XCD order: at t4096 (32768) it moves 316 MB
// instead of 323 MB in equal time (+-1-2% across t4096, skew, fp8); with the
// 2048 rows of a 256-token batch it measured 1.6 us slower (13.3 -> 14.9 us).
constexpr int64_t kXcdOrderMinRows = 8192;

template <int ITER, bool FULL>
__global__ __launch_bounds__(kRegroupBS) void regroup_kernel(
    const u32x4 *__restrict__ in_rows, int nvec, const float *__restrict__ in_scale, int nscale,
    const float *__restrict__ in_w, const int32_t *__restrict__ in_idx, int T, int K, int G,
    const int32_t *__restrict__ group_offset, const int32_t *__restrict__ recv_src_g,
    const int32_t *__restrict__ slot_g, const int32_t *__restrict__ slot_e,
    u32x4 *__restrict__ out_rows, float *__restrict__ out_scale, float *__restrict__ out_w,
    int32_t *__restrict__ out_idx, bool nt_store, bool xcd_order)
{
    // the grid covers the row bound rounded up to a multiple of kXcds * kRun (a
    // bijection of [0, grid) either way); rows used: group_offset[G]
    const int P = group_offset[G];
    int s = blockIdx.x;   // group row
    if (xcd_order) {
        const int b = blockIdx.x, j = b / kXcds;
        s = (j / kRun) * (kXcds * kRun) + (b % kXcds) * kRun + j % kRun;
    }
    if (s >= P) return;
    const int tid = threadIdx.x;
    const int t = recv_src_g[s];
    // a valid layout names a token in [0, T) and expert rows in [0, T * K);
    // anything else (a layout not written for these sizes) is skipped
    if (t < 0 || t >= T) return;
    const int64_t erows = (int64_t)T * K;
    const int32_t *sg = slot_g + (size_t)t * K;
    const int32_t *se = slot_e + (size_t)t * K;

    const u32x4 *src = in_rows + (size_t)s * nvec;
    for (int base = 0; base < nvec; base += kRegroupBS * ITER) {
        u32x4 v[ITER];
#pragma unroll
        for (int i = 0; i < ITER; ++i) {
            const int j = base + i * kRegroupBS + tid;
            if (FULL || j < nvec) v[i] = __builtin_nontemporal_load(src + j);
        }
        for (int k = 0; k < K; ++k) {
            if (sg[k] != s || se[k] < 0 || se[k] >= erows) continue;
            u32x4 *dst = out_rows + (size_t)se[k] * nvec;
#pragma unroll
            for (int i = 0; i < ITER; ++i) {
                const int j = base + i * kRegroupBS + tid;
                if (FULL || j < nvec) {
                    if (nt_store) store16<true>(dst + j, v[i]);
                    else store16<false>(dst + j, v[i]);
                }
            }
        }
    }
    // metadata (lanes [0, K) weights, [K, 2K) indices) and scales
    const bool wl = tid < K, il = tid >= K && tid < 2 * K;
    float wv = 0.f;
    int iv = 0;
    if (wl) wv = in_w[(size_t)s * K + tid];
    if (il) iv = in_idx[(size_t)s * K + tid - K];
    for (int k = 0; k < K; ++k) {
        if (sg[k] != s || se[k] < 0 || se[k] >= erows) continue;
        const int r = se[k];
        if (wl) out_w[(size_t)r * K + tid] = wv;
        if (il) out_idx[(size_t)r * K + tid - K] = iv;
        for (int c = tid; c < nscale; c += kRegroupBS)
            out_scale[(size_t)r * nscale + c] = in_scale[(size_t)s * nscale + c];
    }
}

template <int ITER>
auto pick_full(bool full)
{
    return full ? regroup_kernel<ITER, true> : regroup_kernel<ITER, false>;
}

}  // namespace

hipError_t launch_regroup(const void *in_rows, int row_bytes, const float *in_scale, int nscale,
                          const float *in_w, const int32_t *in_idx, int T, int K, int G,
                          const int32_t *group_offset, const int32_t *recv_src_g,
                          const int32_t *slot_g, const int32_t *slot_e, void *out_rows,
                          float *out_scale, float *out_w, int32_t *out_idx, hipStream_t stream)
{
    const int nvec = row_bytes / 16;
    int iter = (nvec + kRegroupBS - 1) / kRegroupBS;
    iter = iter < 1 ? 1 : (iter > kMaxIter ? kMaxIter : iter);
    const bool full = nvec % (kRegroupBS * iter) == 0;
    void (*fn)(const u32x4 *, int, const float *, int, const float *, const int32_t *, int, int, int,
               const int32_t *, const int32_t *, const int32_t *, const int32_t *, u32x4 *, float *,
               float *, int32_t *, bool, bool);
    switch (iter) {
    case 1: fn = pick_full<1>(full); break;
    case 2: fn = pick_full<2>(full); break;
    case 3: fn = pick_full<3>(full); break;
    case 4: fn = pick_full<4>(full); break;
    case 5: fn = pick_full<5>(full); break;
    case 6: fn = pick_full<6>(full); break;
    case 7: fn = pick_full<7>(full); break;
    default: fn = pick_full<8>(full); break;
    }
    const int64_t bound = (int64_t)T * (K < G ? K : G);   // group rows used <= bound
    const int64_t grid = (bound + kXcds * kRun - 1) / (kXcds * kRun) * (kXcds * kRun);
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(kRegroupBS), 0, stream, (const u32x4 *)in_rows,
                       nvec, in_scale, nscale, in_w, in_idx, T, K, G, group_offset, recv_src_g, slot_g,
                       slot_e, (u32x4 *)out_rows, out_scale, out_w, out_idx,
                       tuning().dispatch_nt_store, tuning().regroup_xcd_order && bound >= kXcdOrderMinRows);
    return hipGetLastError();
}

}  // namespace moe
