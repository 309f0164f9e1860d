// The C ABI of the MoE token path (declared in include/moe_ep.h): argument
// checks on the host, then kernel launches on the caller's stream. Every
// check happens before the first HIP call, so a rejected call touches neither
// the device nor the HIP runtime.
#include "moe_ep.h"

#include "kernels.hpp"

#include <mutex>
#include <stdio.h>
#include <string.h>

namespace {

// Library-owned layout workspace of moe_layout_dispatch_noalloc(), for callers
// that cannot allocate. Each GPU the library runs on holds its own copy until
// the process ends. In host code `scratch` only names the symbol; its device
// address on the current GPU comes from hipGetSymbolAddress (scratch_ptr).
constexpr size_t kScratchBytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the GPU the call's kernels run on (the
// stream's device; the current device for the null stream), looked up once per
// device with that device current and kept; NULL with *err set if the lookup
// fails. The caller's current device is restored after a lookup.
void *scratch_ptr(hipStream_t stream, hipError_t *err)
{
    int dev = -1, cur = -1;
    *err = hipGetDevice(&cur);
    if (*err != hipSuccess) return nullptr;
    dev = cur;
    if (stream) {
        hipDevice_t sd = -1;
        *err = hipStreamGetDevice(stream, &sd);
        if (*err != hipSuccess) return nullptr;
        dev = sd;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        if (dev != cur && (*err = hipSetDevice(dev)) != hipSuccess) return nullptr;
        void *p = nullptr;
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t e2 = hipSetDevice(cur);
            if (*err == hipSuccess) *err = e2;
        }
        if (*err != hipSuccess) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

thread_local char g_hip_msg[160] = "";

int hip_fail(hipError_t e)
{
    snprintf(g_hip_msg, sizeof g_hip_msg, "%s (%d)", hipGetErrorString(e), (int)e);
    return MOE_ERR_HIP;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

int check_dims(int T, int K, int E, int G)
{
    if (T < 0 || K < 1 || K > MOE_MAX_TOPK || E < K || E > MOE_MAX_EXPERTS || G < 1 ||
        G > MOE_MAX_GROUPS || E % G != 0)
        return MOE_ERR_BAD_SHAPE;
    const int64_t m = K > G ? K : G;
    if ((int64_t)T * m >= (int64_t)1 << 30) return MOE_ERR_BAD_SHAPE;
    return MOE_OK;
}

// The count / offset / status arrays are always required; the per-token
// arrays only when there are tokens (T = 0 callers may pass NULL for them).
int check_layout_ptrs(const moe_layout_t *L)
{
    if (!L) return MOE_ERR_NULL_PTR;
    if (!L->expert_count || !L->expert_offset || !L->group_count || !L->group_offset || !L->status)
        return MOE_ERR_NULL_PTR;
    if (L->T > 0 && (!L->tok_group_mask || !L->slot_e || !L->slot_g || !L->slot_tg ||
                     !L->recv_src_e || !L->recv_src_g))
        return MOE_ERR_NULL_PTR;
    return MOE_OK;
}

size_t layout_ws_bytes(int T, int E, int G)
{
    return (moe::layout_ws_bytes_for(T, E, G) + 255) & ~(size_t)255;
}

int64_t rows_bound(int T, int K, int G, int mode)
{
    return mode == MOE_MODE_EXPERT ? (int64_t)T * K : (int64_t)T * (K < G ? K : G);
}

moe::LayoutPtrs ptrs_of(const moe_layout_t *L)
{
    return moe::LayoutPtrs{L->expert_count, L->expert_offset, L->group_count, L->group_offset,
                           L->tok_group_mask, L->slot_e, L->slot_g, L->slot_tg,
                           L->recv_src_e, L->recv_src_g, L->status};
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_EP_ABI_VERSION; }

int moe_layout_workspace_bytes(int T, int K, int E, int G, size_t *bytes)
{
    if (!bytes) return MOE_ERR_NULL_PTR;
    if (int rc = check_dims(T, K, E, G)) return rc;
    *bytes = layout_ws_bytes(T, E, G);
    return MOE_OK;
}

int64_t moe_recv_rows_bound(int T, int K, int G, int mode)
{
    if (mode != MOE_MODE_EXPERT && mode != MOE_MODE_GROUP) return MOE_ERR_BAD_MODE;
    if (T < 0 || K < 1 || G < 1) return MOE_ERR_BAD_SHAPE;
    return rows_bound(T, K, G, mode);
}

int moe_layout(const int32_t *topk_idx, const moe_layout_t *L, void *ws, size_t ws_bytes,
               void *stream)
{
    if (int rc = check_layout_ptrs(L)) return rc;
    if (int rc = check_dims(L->T, L->K, L->E, L->G)) return rc;
    if (L->T > 0) {
        if (!topk_idx) return MOE_ERR_NULL_PTR;
        if (!ws || ws_bytes < layout_ws_bytes(L->T, L->E, L->G)) return MOE_ERR_WORKSPACE;
        if (!aligned4(topk_idx) || !aligned4(ws)) return MOE_ERR_MISALIGNED;
    }
    hipError_t e = moe::launch_layout(topk_idx, L->T, L->K, L->E, L->G, ptrs_of(L),
                                      static_cast<int32_t *>(ws), (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e);
}

int moe_dispatch(const moe_layout_t *L, int mode, int dtype, int H, const void *x,
                 const float *topk_w, const int32_t *topk_idx, void *recv_x, float *recv_scale,
                 float *recv_topk_w, int32_t *recv_topk_idx, int64_t recv_capacity, void *stream)
{
    if (int rc = check_layout_ptrs(L)) return rc;
    if (int rc = check_dims(L->T, L->K, L->E, L->G)) return rc;
    if (mode != MOE_MODE_EXPERT && mode != MOE_MODE_GROUP) return MOE_ERR_BAD_MODE;
    if (dtype != MOE_DTYPE_BF16 && dtype != MOE_DTYPE_FP8_E4M3_B128) return MOE_ERR_BAD_MODE;
    if (H <= 0 || H % 8 != 0) return MOE_ERR_BAD_SHAPE;
    if (dtype == MOE_DTYPE_FP8_E4M3_B128 && H % 128 != 0) return MOE_ERR_BAD_SHAPE;
    if (L->T == 0) return MOE_OK;
    if (!x || !topk_w || !topk_idx || !recv_x || !recv_topk_w || !recv_topk_idx)
        return MOE_ERR_NULL_PTR;
    if (dtype == MOE_DTYPE_FP8_E4M3_B128 && !recv_scale) return MOE_ERR_NULL_PTR;
    if (recv_capacity < rows_bound(L->T, L->K, L->G, mode)) return MOE_ERR_CAPACITY;
    if (!aligned16(x) || !aligned16(recv_x) || !aligned4(topk_w) || !aligned4(topk_idx) ||
        !aligned4(recv_topk_w) || !aligned4(recv_topk_idx) ||
        (recv_scale && !aligned4(recv_scale)))
        return MOE_ERR_MISALIGNED;
    const int nslot = mode == MOE_MODE_EXPERT ? L->K : L->G;
    const int32_t *slots = mode == MOE_MODE_EXPERT ? L->slot_e : L->slot_tg;
    hipError_t e;
    if (dtype == MOE_DTYPE_BF16)
        e = moe::launch_dispatch_bf16(x, L->T, H, L->K, nslot, slots, topk_w, topk_idx, recv_x,
                                      recv_topk_w, recv_topk_idx, nullptr, (hipStream_t)stream);
    else
        e = moe::launch_dispatch_fp8(x, L->T, H, L->K, nslot, slots, topk_w, topk_idx, recv_x,
                                     recv_scale, recv_topk_w, recv_topk_idx, nullptr,
                                     mode == MOE_MODE_GROUP, (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e);
}

}  // extern "C"

namespace {

// The argument checks of moe_layout_dispatch() that do not concern the workspace.
int check_layout_dispatch(const int32_t *topk_idx, const moe_layout_t *L, int mode, int dtype, int H,
                          const void *x, const float *topk_w, const void *recv_x, const float *recv_scale,
                          const float *recv_topk_w, const int32_t *recv_topk_idx, int64_t recv_capacity)
{
    if (int rc = check_layout_ptrs(L)) return rc;
    if (int rc = check_dims(L->T, L->K, L->E, L->G)) return rc;
    if (mode != MOE_MODE_EXPERT && mode != MOE_MODE_GROUP) return MOE_ERR_BAD_MODE;
    if (dtype != MOE_DTYPE_BF16 && dtype != MOE_DTYPE_FP8_E4M3_B128) return MOE_ERR_BAD_MODE;
    if (H <= 0 || H % 8 != 0) return MOE_ERR_BAD_SHAPE;
    if (dtype == MOE_DTYPE_FP8_E4M3_B128 && H % 128 != 0) return MOE_ERR_BAD_SHAPE;
    if (L->T == 0) return MOE_OK;
    if (!topk_idx || !x || !topk_w || !recv_x || !recv_topk_w || !recv_topk_idx)
        return MOE_ERR_NULL_PTR;
    if (dtype == MOE_DTYPE_FP8_E4M3_B128 && !recv_scale) return MOE_ERR_NULL_PTR;
    if (recv_capacity < rows_bound(L->T, L->K, L->G, mode)) return MOE_ERR_CAPACITY;
    if (!aligned4(topk_idx) || !aligned16(x) || !aligned16(recv_x) || !aligned4(topk_w) ||
        !aligned4(recv_topk_w) || !aligned4(recv_topk_idx) || (recv_scale && !aligned4(recv_scale)))
        return MOE_ERR_MISALIGNED;
    return MOE_OK;
}

int layout_dispatch_impl(const int32_t *topk_idx, const moe_layout_t *L, void *ws, size_t ws_bytes,
                         int mode, int dtype, int H, const void *x, const float *topk_w, void *recv_x,
                         float *recv_scale, float *recv_topk_w, int32_t *recv_topk_idx,
                         int64_t recv_capacity, void *stream)
{
    if (int rc = check_layout_ptrs(L)) return rc;
    if (int rc = check_dims(L->T, L->K, L->E, L->G)) return rc;
    if (mode != MOE_MODE_EXPERT && mode != MOE_MODE_GROUP) return MOE_ERR_BAD_MODE;
    if (dtype != MOE_DTYPE_BF16 && dtype != MOE_DTYPE_FP8_E4M3_B128) return MOE_ERR_BAD_MODE;
    if (H <= 0 || H % 8 != 0) return MOE_ERR_BAD_SHAPE;
    if (dtype == MOE_DTYPE_FP8_E4M3_B128 && H % 128 != 0) return MOE_ERR_BAD_SHAPE;
    if (L->T == 0) return moe_layout(topk_idx, L, ws, ws_bytes, stream);
    if (!topk_idx || !x || !topk_w || !recv_x || !recv_topk_w || !recv_topk_idx)
        return MOE_ERR_NULL_PTR;
    if (dtype == MOE_DTYPE_FP8_E4M3_B128 && !recv_scale) return MOE_ERR_NULL_PTR;
    if (recv_capacity < rows_bound(L->T, L->K, L->G, mode)) return MOE_ERR_CAPACITY;
    if (!aligned4(topk_idx) || !aligned16(x) || !aligned16(recv_x) || !aligned4(topk_w) ||
        !aligned4(recv_topk_w) || !aligned4(recv_topk_idx) || (recv_scale && !aligned4(recv_scale)))
        return MOE_ERR_MISALIGNED;
    const bool fp8 = dtype == MOE_DTYPE_FP8_E4M3_B128;
    hipError_t e;
    // One launch for the smallest batches, where its per-token recomputation of
    // the routing (work growing with T * K and E per workgroup) is cheaper than
    // the two launches of the placing form below (measured: at E = 8, K = 2
    // 0.3-1 us faster up to T = 256, slower at T = 512; at E = 64 and 256 slower
    // by 6-9 us from the smallest T), and whenever no workspace is given.
    const bool one_launch_fits = L->T <= MOE_FUSED_MAX_TOKENS && (int64_t)L->T * L->K <= MOE_FUSED_MAX_PAIRS;
    const bool small = (int64_t)L->T * L->K * L->E <= moe::tuning().fused_small_max_work;
    if (one_launch_fits && (small || !ws)) {
        e = moe::launch_layout_dispatch(topk_idx, L->T, L->K, L->E, L->G, ptrs_of(L), mode, fp8, H, x,
                                        topk_w, recv_x, recv_scale, recv_topk_w, recv_topk_idx,
                                        (hipStream_t)stream);
        return e == hipSuccess ? MOE_OK : hip_fail(e);
    }
    if (!ws || ws_bytes < layout_ws_bytes(L->T, L->E, L->G)) return MOE_ERR_WORKSPACE;
    if (!aligned4(ws)) return MOE_ERR_MISALIGNED;
    const moe::LayoutPtrs P = ptrs_of(L);
    const int nslot = mode == MOE_MODE_EXPERT ? L->K : L->G;
    const int32_t *slots = mode == MOE_MODE_EXPERT ? L->slot_e : L->slot_tg;
    // The placing dispatch needs the per-tile masks (K <= 8) and pays its
    // placement latency once per round of resident workgroups. For bf16 (few
    // rounds of 128-thread workgroups) it beats moe_layout + the plain dispatch
    // at every size tried. The one-wave FP8 workgroups (3 per SIMD, so 3072 at
    // once) measured 1-4 us faster up to T = 3072 and even to 1.2 us slower at
    // T = 4096, where a second round pays the placement again: placing up to
    // 3072 tokens, moe_layout + the plain FP8 dispatch above. The row-sized FP8
    // workgroups (H > 8192) are slower placing. (The one-launch layout + a
    // plain dispatch, once used up to T * K = 8192, measured 1-2.5 us slower
    // than the bf16 placing form at every size tried; it stays selectable for
    // A/B runs.)
    const int64_t pairs = (int64_t)L->T * L->K;
    const bool via_onepass = L->K <= 8 && pairs <= moe::tuning().fused_onepass_max_pairs &&
                             pairs <= moe::tuning().layout_onepass_max_pairs;
    if (L->K > 8 || (fp8 && (!moe::fp8_wave_form(H) || L->T > moe::tuning().fused_fp8_place_max_t)) ||
        via_onepass) {
        e = moe::launch_layout(topk_idx, L->T, L->K, L->E, L->G, P, static_cast<int32_t *>(ws),
                               (hipStream_t)stream);
        if (e == hipSuccess)
            e = fp8 ? moe::launch_dispatch_fp8(x, L->T, H, L->K, nslot, slots, topk_w, topk_idx, recv_x,
                                               recv_scale, recv_topk_w, recv_topk_idx, nullptr,
                                               mode == MOE_MODE_GROUP, (hipStream_t)stream)
                    : moe::launch_dispatch_bf16(x, L->T, H, L->K, nslot, slots, topk_w, topk_idx, recv_x,
                                                recv_topk_w, recv_topk_idx, nullptr, (hipStream_t)stream);
        return e == hipSuccess ? MOE_OK : hip_fail(e);
    }
    // The count kernel, then each dispatch workgroup places its own token. The
    // counts, offsets and per-tile bases come from a one-workgroup finalize
    // kernel in between, or from workgroup 0 of the dispatch while the others
    // load their rows: there for batches whose table it reads in one round of
    // loads per column (at most 16 tiles), with at most four expert columns per
    // thread (at E = 256: bf16 ≈ 2.8 µs and FP8 ≈ 2.2 µs faster per call).
    const int fin_threads = moe::placing_dispatch_threads(fp8, H);
    const bool fin_in_dispatch = moe::tuning().fused_finalize >= (fp8 ? 2 : 1) &&
                                 L->E <= moe::tuning().fused_finalize_rounds * fin_threads &&
                                 moe::layout_tiles(L->T) <= moe::kFinTiles;
    e = moe::launch_layout_count_finalize(topk_idx, L->T, L->K, L->E, L->G, P, static_cast<int32_t *>(ws),
                                          fin_in_dispatch, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e);
    const moe::LayoutWs w = moe::layout_ws(ws, L->T, L->E, L->G);
    moe::PlaceArgs pa;
    pa.idx = topk_idx;
    pa.E = L->E;
    pa.G = L->G;
    pa.gmagic = moe::group_magic(L->E, L->G);
    pa.words = w.words;
    pa.gwords = w.gwords;
    pa.bases = w.bases;
    pa.table = w.table;
    pa.ntiles = moe::layout_tiles(L->T);
    pa.finalize = fin_in_dispatch ? 1 : 0;
    pa.wait_ticks = moe::tuning().base_wait_ticks < 0 ? 0 : (uint64_t)moe::tuning().base_wait_ticks;
    pa.self_bases = moe::tuning().base_wait_ticks < 0 ? 1 : 0;
    pa.L = P;
    pa.mode = mode == MOE_MODE_EXPERT ? 0 : 1;
    e = fp8 ? moe::launch_dispatch_fp8(x, L->T, H, L->K, nslot, nullptr, topk_w, topk_idx, recv_x, recv_scale,
                                       recv_topk_w, recv_topk_idx, &pa, mode == MOE_MODE_GROUP, (hipStream_t)stream)
            : moe::launch_dispatch_bf16(x, L->T, H, L->K, nslot, nullptr, topk_w, topk_idx, recv_x,
                                        recv_topk_w, recv_topk_idx, &pa, (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e);
}

}  // namespace

extern "C" {

int moe_layout_dispatch(const int32_t *topk_idx, const moe_layout_t *L, void *ws, size_t ws_bytes,
                        int mode, int dtype, int H, const void *x, const float *topk_w, void *recv_x,
                        float *recv_scale, float *recv_topk_w, int32_t *recv_topk_idx,
                        int64_t recv_capacity, void *stream)
{
    return layout_dispatch_impl(topk_idx, L, ws, ws_bytes, mode, dtype, H, x, topk_w, recv_x, recv_scale,
                                recv_topk_w, recv_topk_idx, recv_capacity, stream);
}

int moe_layout_dispatch_noalloc(const int32_t *topk_idx, const moe_layout_t *L, int mode, int dtype, int H,
                                const void *x, const float *topk_w, void *recv_x, float *recv_scale,
                                float *recv_topk_w, int32_t *recv_topk_idx, int64_t recv_capacity,
                                void *stream)
{
    if (int rc = check_layout_dispatch(topk_idx, L, mode, dtype, H, x, topk_w, recv_x, recv_scale, recv_topk_w,
                                       recv_topk_idx, recv_capacity))
        return rc;
    if (L->T > 0 && layout_ws_bytes(L->T, L->E, L->G) > kScratchBytes) return MOE_ERR_SCRATCH_LIMIT;
    hipError_t err;
    void *ws = scratch_ptr((hipStream_t)stream, &err);
    if (!ws) return hip_fail(err);
    return layout_dispatch_impl(topk_idx, L, ws, kScratchBytes, mode, dtype, H, x, topk_w, recv_x, recv_scale,
                                recv_topk_w, recv_topk_idx, recv_capacity, stream);
}

int moe_regroup(const moe_layout_t *L, int dtype, int H, const void *recv_g, const float *recv_scale_g,
                const float *recv_topk_w_g, const int32_t *recv_topk_idx_g, int64_t g_capacity,
                void *recv_e, float *recv_scale_e, float *recv_topk_w_e, int32_t *recv_topk_idx_e,
                int64_t e_capacity, void *stream)
{
    if (int rc = check_layout_ptrs(L)) return rc;
    if (int rc = check_dims(L->T, L->K, L->E, L->G)) return rc;
    if (dtype != MOE_DTYPE_BF16 && dtype != MOE_DTYPE_FP8_E4M3_B128) return MOE_ERR_BAD_MODE;
    const bool fp8 = dtype == MOE_DTYPE_FP8_E4M3_B128;
    if (H <= 0 || H % 8 != 0 || (fp8 && H % 128 != 0)) return MOE_ERR_BAD_SHAPE;
    if (L->T == 0) return MOE_OK;
    if (!recv_g || !recv_topk_w_g || !recv_topk_idx_g || !recv_e || !recv_topk_w_e ||
        !recv_topk_idx_e)
        return MOE_ERR_NULL_PTR;
    if (fp8 && (!recv_scale_g || !recv_scale_e)) return MOE_ERR_NULL_PTR;
    if (g_capacity < rows_bound(L->T, L->K, L->G, MOE_MODE_GROUP) ||
        e_capacity < rows_bound(L->T, L->K, L->G, MOE_MODE_EXPERT))
        return MOE_ERR_CAPACITY;
    if (!aligned16(recv_g) || !aligned16(recv_e) || !aligned4(recv_topk_w_g) ||
        !aligned4(recv_topk_idx_g) || !aligned4(recv_topk_w_e) || !aligned4(recv_topk_idx_e) ||
        (fp8 && (!aligned4(recv_scale_g) || !aligned4(recv_scale_e))))
        return MOE_ERR_MISALIGNED;
    hipError_t e = moe::launch_regroup(recv_g, fp8 ? H : 2 * H, fp8 ? recv_scale_g : nullptr,
                                       fp8 ? H / 128 : 0, recv_topk_w_g, recv_topk_idx_g, L->T, L->K,
                                       L->G, L->group_offset, L->recv_src_g, L->slot_g, L->slot_e, recv_e,
                                       fp8 ? recv_scale_e : nullptr, recv_topk_w_e, recv_topk_idx_e,
                                       (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e);
}

int64_t moe_cast_transpose_t_bytes(int T, int K, int E, int H)
{
    if (T < 0 || K < 1 || E < 1 || E > MOE_MAX_EXPERTS || H <= 0 || H % 64 != 0) return MOE_ERR_BAD_SHAPE;
    return moe::cast_transpose_t_bound((int64_t)T * K, E, H);
}

int moe_cast_transpose_fp8(const moe_layout_t *L, int H, const void *x, int64_t x_rows,
                           const float *scale, void *c_out, void *t_out, int64_t t_bytes, float *amax,
                           int32_t *pad_offset, void *stream)
{
    if (int rc = check_layout_ptrs(L)) return rc;
    if (int rc = check_dims(L->T, L->K, L->E, L->G)) return rc;
    if (H <= 0 || H % 64 != 0) return MOE_ERR_BAD_SHAPE;
    if (!x || !scale || !c_out || !t_out || !amax || !pad_offset) return MOE_ERR_NULL_PTR;
    const int64_t bound = (int64_t)L->T * L->K;
    if (x_rows < bound || t_bytes < moe::cast_transpose_t_bound(bound, L->E, H)) return MOE_ERR_CAPACITY;
    if (!aligned16(x) || !aligned16(c_out) || !aligned16(t_out) || !aligned4(scale) || !aligned4(amax) ||
        !aligned4(pad_offset))
        return MOE_ERR_MISALIGNED;
    hipError_t e = moe::launch_cast_transpose(x, bound, H, L->E, L->expert_offset, scale, c_out, t_out,
                                              amax, pad_offset, (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e);
}

int moe_combine(const moe_layout_t *L, int mode, int H, const void *y, int64_t y_rows,
                const float *topk_w, void *out, void *stream)
{
    if (int rc = check_layout_ptrs(L)) return rc;
    if (int rc = check_dims(L->T, L->K, L->E, L->G)) return rc;
    if (mode != MOE_MODE_EXPERT && mode != MOE_MODE_GROUP) return MOE_ERR_BAD_MODE;
    if (H <= 0 || H % 8 != 0 || y_rows < 0) return MOE_ERR_BAD_SHAPE;
    if (L->T == 0) return MOE_OK;
    if (!y || !topk_w || !out) return MOE_ERR_NULL_PTR;
    if (!aligned16(y) || !aligned16(out) || !aligned4(topk_w)) return MOE_ERR_MISALIGNED;
    const int32_t *slot = mode == MOE_MODE_EXPERT ? L->slot_e : L->slot_g;
    hipError_t e = moe::launch_combine(y, y_rows, L->T, H, L->K, slot, mode == MOE_MODE_GROUP,
                                       topk_w, out, L->status, (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e);
}

int moe_fp8_dequant(const moe_layout_t *L, int mode, int H, const void *q, const float *scale,
                    void *y, int64_t capacity, void *stream)
{
    if (int rc = check_layout_ptrs(L)) return rc;
    if (int rc = check_dims(L->T, L->K, L->E, L->G)) return rc;
    if (mode != MOE_MODE_EXPERT && mode != MOE_MODE_GROUP) return MOE_ERR_BAD_MODE;
    if (H <= 0 || H % 128 != 0 || capacity < 0 || capacity >= ((int64_t)1 << 31))
        return MOE_ERR_BAD_SHAPE;
    if (L->T == 0 || capacity == 0) return MOE_OK;
    if (!q || !scale || !y) return MOE_ERR_NULL_PTR;
    if (!aligned16(q) || !aligned16(y) || !aligned4(scale)) return MOE_ERR_MISALIGNED;
    const int32_t *nrows = mode == MOE_MODE_EXPERT ? L->expert_offset + L->E : L->group_offset + L->G;
    hipError_t e = moe::launch_fp8_dequant(q, scale, y, capacity, H, nrows, (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e);
}

int moe_ref_copy(void *dst, const void *src, int64_t bytes, void *stream)
{
    if (bytes < 0 || bytes % 16 != 0) return MOE_ERR_BAD_SHAPE;
    if (bytes == 0) return MOE_OK;
    if (!dst || !src) return MOE_ERR_NULL_PTR;
    if (!aligned16(dst) || !aligned16(src)) return MOE_ERR_MISALIGNED;
    hipError_t e = moe::launch_ref_copy(dst, src, bytes, (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e);
}

int moe_ref_mix(void *dst, const void *src, int64_t row_bytes, int64_t units, int nr, int nw,
                void *stream)
{
    auto pow2_le8 = [](int v) { return v == 1 || v == 2 || v == 4 || v == 8; };
    if (!pow2_le8(nr) || !pow2_le8(nw) || (nr > 1 && nw > 1)) return MOE_ERR_BAD_MODE;
    if (row_bytes <= 0 || row_bytes % 16 != 0 || row_bytes / 16 > (1 << 24) || units < 0 ||
        units >= ((int64_t)1 << 31))
        return MOE_ERR_BAD_SHAPE;
    if (units == 0) return MOE_OK;
    if (!dst || !src) return MOE_ERR_NULL_PTR;
    if (!aligned16(dst) || !aligned16(src)) return MOE_ERR_MISALIGNED;
    hipError_t e = moe::launch_ref_mix(dst, src, row_bytes, units, nr, nw, (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e);
}

const char *moe_status_string(int code)
{
    static thread_local char buf[256];
    switch (code) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL_PTR: return "a required pointer is NULL";
    case MOE_ERR_BAD_SHAPE: return "shape outside the supported range";
    case MOE_ERR_MISALIGNED: return "buffer not aligned (rows need 16 bytes, others 4)";
    case MOE_ERR_CAPACITY: return "receive buffer smaller than moe_recv_rows_bound()";
    case MOE_ERR_WORKSPACE: return "layout workspace missing or smaller than moe_layout_workspace_bytes()";
    case MOE_ERR_BAD_MODE: return "unknown mode or dtype";
    case MOE_ERR_SCRATCH_LIMIT:
        return "sizes need more layout workspace than moe_layout_dispatch_noalloc() holds "
               "(MOE_NOALLOC_SCRATCH_BYTES); use moe_layout_dispatch() with a workspace";
    case MOE_ERR_HIP:
        snprintf(buf, sizeof buf, "HIP error: %s", g_hip_msg);
        return buf;
    default: return "unknown error code";
    }
}

}  // extern "C"
