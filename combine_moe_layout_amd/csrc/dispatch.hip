// Dispatch on gfx950: scatter each source token's hidden row (bf16, or FP8
// e4m3 with one fp32 scale per 1x128 block) plus its K weights and K indices
// to every receive row the routing layout gave it.
//
// Design. One workgroup per source token. The workgroup reads the token's row
// once into registers with 16-byte loads (each lane holds ITER vectors, so
// the row is read exactly once from HBM), then writes those registers to each
// destination row with 16-byte stores: the traffic is one read of x and R
// row writes, the minimum. This is the single-GPU form of the row
// copy of "perf(ep): optimize IntraNode dispatch kernel for MI350X" (ROCm/mori
// pull request 586): Technical Details 3 (a wave-wide vector copy whose
// unroll must fit the hidden size — here ITER is chosen from H so the row is
// covered in whole passes with no remainder loop) and 4 (the K weights and K
// indices travel with each row, written by K lanes each). Destination slots
// come from the layout's cached slots (Technical Details 1): a token reads K
// (or G) integers instead of re-deriving its routing. The cache policy of the
// row accesses is chosen by measurement on MI355X, not copied from the
// non-temporal stores of "Optimized rocm specific multicast transpose kernel"
// (ROCm/TransformerEngine pull request 586, Change Summary): there, CDNA4's
// write-allocate L2 made NT stores pay; here a plain streaming store sustains
// more write bandwidth than an NT one, while NT loads read markedly faster.
//
// FP8: each lane holds chunks of 16 consecutive elements (two 16-byte loads
// each): one wave per token with H/1024 chunks per lane for H <= 8192 (so the
// 4096 token workgroups of a large batch are mostly resident at once), else a
// workgroup sized to the row with one chunk per lane per pass. The 8 lanes of
// one 128-block (8 consecutive lanes in either form) reduce amax with three
// xor-shuffles (NaNs are passed over: see amax_step); every lane then forms
// scale = amax / 448 and inv = 448 / amax (correctly rounded fp32 divisions:
// the library is built with -fhip-fp32-correctly-rounded-divide-sqrt),
// multiplies, saturates to +-448 (sat448: equal to saturating
// round-to-nearest-even for every value; a NaN stays a NaN) and converts pairs
// with the packed e4m3 conversion (its NaN byte mapped to the code 0x7F),
// giving one 16-byte store per lane per destination. The quantisation runs
// once per source token, not once per destination.
#include "common.hpp"
#include "kernels.hpp"
#include "place.hpp"

#include <stdlib.h>

namespace moe {

namespace {

constexpr int kDispatchBS = 128;   // threads per workgroup, bf16
constexpr int kFp8MaxBS = 1024;    // threads per workgroup, fp8: up to one per 16-element chunk
constexpr int kMaxIter = 8;
constexpr int kMaxSlots = 32;      // K or G destinations per token

// PLACE: the token's slots are not read from the layout but computed here
// (place_token; the fused layout + dispatch), after the row's first loads
// are issued.
template <int ITER, bool NT, bool NTL, bool FULL, bool PLACE>
__global__ __launch_bounds__(kDispatchBS) void dispatch_bf16_kernel(
    const u32x4 *__restrict__ x, int nvec, int K, int nslot, const int32_t *__restrict__ slots,
    const float *__restrict__ topk_w, const int32_t *__restrict__ topk_idx,
    u32x4 *__restrict__ recv_x, float *__restrict__ recv_w, int32_t *__restrict__ recv_idx,
    PlaceArgs P)
{
    __shared__ int32_t s_dst[PLACE ? kMaxSlots : 1];
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const u32x4 *src = x + (size_t)t * nvec;
    const int32_t *ts = PLACE ? s_dst : slots + (size_t)t * nslot;
    // receive rows of a valid layout are < T * min(K, nslot) (T = the grid),
    // which the caller's buffers hold; anything else is skipped
    const int64_t rows = (int64_t)gridDim.x * (K < nslot ? K : nslot);

    u32x4 v[ITER];
    auto load_pass = [&](int base) {
#pragma unroll
        for (int i = 0; i < ITER; ++i) {
            const int j = base + i * kDispatchBS + tid;
            if (FULL || j < nvec) v[i] = load16<NTL>(src + j);
        }
    };
    if constexpr (PLACE) {
        if (P.finalize && t == 0) finalize_role(P);
    }
    load_pass(0);
    if constexpr (PLACE) place_token(P, t, K, s_dst);
    for (int base = 0; base < nvec; base += kDispatchBS * ITER) {
        if (base > 0) load_pass(base);
        for (int d = 0; d < nslot; ++d) {
            const int s = ts[d];
            if (s < 0 || s >= rows) continue;
            u32x4 *dst = recv_x + (size_t)s * nvec;
#pragma unroll
            for (int i = 0; i < ITER; ++i) {
                const int j = base + i * kDispatchBS + tid;
                if (FULL || j < nvec) store16<NT>(dst + j, v[i]);
            }
        }
    }

    // Metadata: lanes [0, K) carry the weights, lanes [K, 2K) the indices.
    const bool wl = tid < K, il = tid >= K && tid < 2 * K;
    float wv = 0.f;
    int iv = 0;
    if (wl) wv = topk_w[(size_t)t * K + tid];
    if (il) iv = topk_idx[(size_t)t * K + tid - K];
    for (int d = 0; d < nslot; ++d) {
        const int s = ts[d];
        if (s < 0 || s >= rows) continue;
        if (wl) recv_w[(size_t)s * K + tid] = wv;
        if (il) recv_idx[(size_t)s * K + tid - K] = iv;
    }
}

// Small batches: one workgroup per (token, slice of kDispatchBS vectors of its
// row), grid T x slices. A lane loads its one vector and stores it to each
// destination row, so a workgroup's chain is one load and nslot stores instead
// of ITER loads and ITER * nslot stores: with few tokens the grid is then large
// enough to fill the chip and each workgroup short. Slice 0 also writes the
// metadata. Same rows, same bytes as dispatch_bf16_kernel.
template <bool NT, bool NTL>
__global__ __launch_bounds__(kDispatchBS) void dispatch_bf16_split_kernel(
    const u32x4 *__restrict__ x, int nvec, int K, int nslot, const int32_t *__restrict__ slots,
    const float *__restrict__ topk_w, const int32_t *__restrict__ topk_idx,
    u32x4 *__restrict__ recv_x, float *__restrict__ recv_w, int32_t *__restrict__ recv_idx)
{
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const int j = blockIdx.y * kDispatchBS + tid;
    const int32_t *ts = slots + (size_t)t * nslot;
    const int64_t rows = (int64_t)gridDim.x * (K < nslot ? K : nslot);
    u32x4 v = {};
    if (j < nvec) v = load16<NTL>(x + (size_t)t * nvec + j);
    for (int d = 0; d < nslot; ++d) {
        const int s = ts[d];
        if (s < 0 || s >= rows) continue;
        if (j < nvec) store16<NT>(recv_x + (size_t)s * nvec + j, v);
    }
    if (blockIdx.y != 0) return;
    const bool wl = tid < K, il = tid >= K && tid < 2 * K;
    float wv = 0.f;
    int iv = 0;
    if (wl) wv = topk_w[(size_t)t * K + tid];
    if (il) iv = topk_idx[(size_t)t * K + tid - K];
    for (int d = 0; d < nslot; ++d) {
        const int s = ts[d];
        if (s < 0 || s >= rows) continue;
        if (wl) recv_w[(size_t)s * K + tid] = wv;
        if (il) recv_idx[(size_t)s * K + tid - K] = iv;
    }
}

// One 16-element chunk per lane per pass; the workgroup has as many lanes as
// the row has chunks (rounded up to whole waves, at most kFp8MaxBS), so a
// lane holds one chunk's state and occupancy stays high.
template <bool NT, bool NTL, bool FULL, bool PLACE>
__global__ __launch_bounds__(kFp8MaxBS) void dispatch_fp8_kernel(
    const u32x4 *__restrict__ x, int nch, int K, int nslot, const int32_t *__restrict__ slots,
    const float *__restrict__ topk_w, const int32_t *__restrict__ topk_idx,
    u32x4 *__restrict__ recv_q, float *__restrict__ recv_scale, float *__restrict__ recv_w,
    int32_t *__restrict__ recv_idx, PlaceArgs P)
{
    __shared__ int32_t s_dst[PLACE ? kMaxSlots : 1];
    // nch = H / 16 chunks of 16 elements; a row of x is 2 * nch vectors, a
    // receive row nch vectors of 16 e4m3 bytes, and nch / 8 scales.
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const int bs = blockDim.x;
    const u32x4 *src = x + (size_t)t * nch * 2;
    const int32_t *ts = PLACE ? s_dst : slots + (size_t)t * nslot;
    const int nblk = nch / 8;
    const int64_t rows = (int64_t)gridDim.x * (K < nslot ? K : nslot);   // as in the bf16 kernel

    // The first pass is loaded and quantised before the token is placed
    // (PLACE), so the placement overlaps it.
    if constexpr (PLACE) {
        if (P.finalize && t == 0) finalize_role(P);
    }
    u32x4 q0;
    float scale0;
    {
        u32x4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
        if (FULL || tid < nch) {
            a = load16<NTL>(src + 2 * tid);
            b = load16<NTL>(src + 2 * tid + 1);
        }
        quantize16(a, b, q0, scale0);
    }
    if constexpr (PLACE) place_token(P, t, K, s_dst);
    for (int j = tid; FULL ? j < nch : j - tid < nch; j += bs) {
        const bool in = FULL || j < nch;
        u32x4 q = q0;
        float scale = scale0;
        if (j != tid) {   // later passes (rows longer than the workgroup)
            u32x4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
            if (in) {
                a = load16<NTL>(src + 2 * j);
                b = load16<NTL>(src + 2 * j + 1);
            }
            quantize16(a, b, q, scale);
        }
        if (in) {
            for (int d = 0; d < nslot; ++d) {
                const int s = ts[d];
                if (s < 0 || s >= rows) continue;
                store16<NT>(recv_q + (size_t)s * nch + j, q);
                if ((tid & 7) == 0) recv_scale[(size_t)s * nblk + (j >> 3)] = scale;
            }
        }
    }

    const bool wl = tid < K, il = tid >= K && tid < 2 * K;
    float wv = 0.f;
    int iv = 0;
    if (wl) wv = topk_w[(size_t)t * K + tid];
    if (il) iv = topk_idx[(size_t)t * K + tid - K];
    for (int d = 0; d < nslot; ++d) {
        const int s = ts[d];
        if (s < 0 || s >= rows) continue;
        if (wl) recv_w[(size_t)s * K + tid] = wv;
        if (il) recv_idx[(size_t)s * K + tid - K] = iv;
    }
}

// Small workgroups (BS = 64 or 128 lanes per token, H <= 16 * BS * 8): lane
// l holds chunks l, l + BS, ..., l + BS (ITER - 1), so a 128-block is still
// 8 consecutive lanes in every pass, and more workgroups are resident at once
// than with the row-sized workgroups above. WPE: the fewest waves per SIMD the
// register allocation must allow (1: no bound; 4: 128 VGPRs, which spills a
// few bytes and pays off only for the plain per-group dispatch, measured).
template <int BS, int ITER, bool NT, bool NTL, bool PLACE, int WPE>
__global__ __launch_bounds__(BS) __attribute__((amdgpu_waves_per_eu(WPE))) void dispatch_fp8_wave_kernel(
    const u32x4 *__restrict__ x, int nch, int K, int nslot, const int32_t *__restrict__ slots,
    const float *__restrict__ topk_w, const int32_t *__restrict__ topk_idx,
    u32x4 *__restrict__ recv_q, float *__restrict__ recv_scale, float *__restrict__ recv_w,
    int32_t *__restrict__ recv_idx, PlaceArgs P)
{
    __shared__ int32_t s_dst[PLACE ? kMaxSlots : 1];
    const int t = blockIdx.x;
    const int lane = threadIdx.x;   // lane of the workgroup
    const u32x4 *src = x + (size_t)t * nch * 2;
    const int32_t *ts = PLACE ? s_dst : slots + (size_t)t * nslot;
    const int nblk = nch / 8;
    const int64_t rows = (int64_t)gridDim.x * (K < nslot ? K : nslot);   // as in the bf16 kernel

    if constexpr (PLACE) {
        if (P.finalize && t == 0) finalize_role(P);
    }
    u32x4 q[ITER];
    float sc[ITER];
    {
        u32x4 a[ITER], b[ITER];
#pragma unroll
        for (int i = 0; i < ITER; ++i) {
            const int j = lane + i * BS;
            a[i] = b[i] = u32x4{0, 0, 0, 0};
            if (j < nch) {
                a[i] = load16<NTL>(src + 2 * j);
                b[i] = load16<NTL>(src + 2 * j + 1);
            }
        }
#pragma unroll
        for (int i = 0; i < ITER; ++i) quantize16(a[i], b[i], q[i], sc[i]);
    }
    if constexpr (PLACE) place_token(P, t, K, s_dst);
    for (int d = 0; d < nslot; ++d) {
        const int s = ts[d];
        if (s < 0 || s >= rows) continue;
#pragma unroll
        for (int i = 0; i < ITER; ++i) {
            const int j = lane + i * BS;
            if (j < nch) {
                store16<NT>(recv_q + (size_t)s * nch + j, q[i]);
                if ((lane & 7) == 0) recv_scale[(size_t)s * nblk + (j >> 3)] = sc[i];
            }
        }
    }
    const bool wl = lane < K, il = lane >= K && lane < 2 * K;
    float wv = 0.f;
    int iv = 0;
    if (wl) wv = topk_w[(size_t)t * K + lane];
    if (il) iv = topk_idx[(size_t)t * K + lane - K];
    for (int d = 0; d < nslot; ++d) {
        const int s = ts[d];
        if (s < 0 || s >= rows) continue;
        if (wl) recv_w[(size_t)s * K + lane] = wv;
        if (il) recv_idx[(size_t)s * K + lane - K] = iv;
    }
}

// Kernel instances by (ITER, NT store, NT load, FULL).
template <int ITER, bool NT, bool NTL, bool FULL>
struct Bf16Inst {
    static constexpr auto fn = dispatch_bf16_kernel<ITER, NT, NTL, FULL, false>;
};
template <int ITER, bool NT, bool NTL, bool FULL>
struct Bf16PlaceInst {
    static constexpr auto fn = dispatch_bf16_kernel<ITER, NT, NTL, FULL, true>;
};

template <template <int, bool, bool, bool> class Inst, int ITER>
auto pick_flags(bool nt, bool ntl, bool full)
{
    if (nt) {
        if (ntl) return full ? Inst<ITER, true, true, true>::fn : Inst<ITER, true, true, false>::fn;
        return full ? Inst<ITER, true, false, true>::fn : Inst<ITER, true, false, false>::fn;
    }
    if (ntl) return full ? Inst<ITER, false, true, true>::fn : Inst<ITER, false, true, false>::fn;
    return full ? Inst<ITER, false, false, true>::fn : Inst<ITER, false, false, false>::fn;
}

template <template <int, bool, bool, bool> class Inst>
auto pick(int iter, bool nt, bool ntl, bool full)
{
    switch (iter) {
    case 1: return pick_flags<Inst, 1>(nt, ntl, full);
    case 2: return pick_flags<Inst, 2>(nt, ntl, full);
    case 3: return pick_flags<Inst, 3>(nt, ntl, full);
    case 4: return pick_flags<Inst, 4>(nt, ntl, full);
    case 5: return pick_flags<Inst, 5>(nt, ntl, full);
    case 6: return pick_flags<Inst, 6>(nt, ntl, full);
    case 7: return pick_flags<Inst, 7>(nt, ntl, full);
    default: return pick_flags<Inst, 8>(nt, ntl, full);
    }
}

// Vectors per lane: the fewest whole passes of BS lanes that cover n vectors,
// at most kMaxIter per pass (larger rows loop over passes).
inline int iters_for(int n, int bs)
{
    const int it = (n + bs - 1) / bs;
    return it < 1 ? 1 : (it > kMaxIter ? kMaxIter : it);
}

}  // namespace

const Tuning &tuning()
{
    static const Tuning t = [] {
        Tuning r;
        auto env = [](const char *name, bool &v) {
            if (const char *s = getenv(name)) v = atoi(s) != 0;
        };
        env("MOE_EP_DISPATCH_NT_LOAD", r.dispatch_nt_load);
        env("MOE_EP_DISPATCH_NT_STORE", r.dispatch_nt_store);
        if (const char *f = getenv("MOE_EP_FP8_FORM")) r.fp8_form = atoi(f);
        if (const char *f = getenv("MOE_EP_LAYOUT_ONEPASS_MAX_PAIRS")) r.layout_onepass_max_pairs = atoi(f);
        if (const char *f = getenv("MOE_EP_LAYOUT_EXCHANGE_MAX_TILES")) r.layout_exchange_max_tiles = atoi(f);
        if (const char *f = getenv("MOE_EP_FUSED_ONEPASS_MAX_PAIRS")) r.fused_onepass_max_pairs = atoi(f);
        if (const char *f = getenv("MOE_EP_FUSED_FINALIZE")) r.fused_finalize = atoi(f);
        if (const char *f = getenv("MOE_EP_FUSED_FINALIZE_ROUNDS")) r.fused_finalize_rounds = atoi(f);
        if (const char *f = getenv("MOE_EP_FUSED_SMALL_MAX_WORK")) r.fused_small_max_work = atoi(f);
        if (const char *f = getenv("MOE_EP_BASE_WAIT_TICKS")) r.base_wait_ticks = atoll(f);
        env("MOE_EP_FP8_GROUP_W4", r.fp8_group_w4);
        if (const char *f = getenv("MOE_EP_FUSED_FP8_PLACE_MAX_T")) r.fused_fp8_place_max_t = atoi(f);
        env("MOE_EP_REGROUP_XCD_ORDER", r.regroup_xcd_order);
        if (const char *f = getenv("MOE_EP_DISPATCH_SPLIT_MAX_WGS")) r.dispatch_split_max_wgs = atoi(f);
        return r;
    }();
    return t;
}

hipError_t launch_dispatch_bf16(const void *x, int T, int H, int K, int nslot, const int32_t *slots,
                                const float *topk_w, const int32_t *topk_idx, void *recv_x,
                                float *recv_w, int32_t *recv_idx, const PlaceArgs *place,
                                hipStream_t stream)
{
    const int nvec = H / 8;
    const int iter = iters_for(nvec, kDispatchBS);
    const bool full = nvec % (kDispatchBS * iter) == 0;
    const bool nt = tuning().dispatch_nt_store, ntl = tuning().dispatch_nt_load;
    const int slices = (nvec + kDispatchBS - 1) / kDispatchBS;
    if (!place && slices > 1 && slices <= 65535 && (int64_t)T * slices <= tuning().dispatch_split_max_wgs) {
        auto sfn = nt ? (ntl ? dispatch_bf16_split_kernel<true, true> : dispatch_bf16_split_kernel<true, false>)
                      : (ntl ? dispatch_bf16_split_kernel<false, true> : dispatch_bf16_split_kernel<false, false>);
        hipLaunchKernelGGL(sfn, dim3(T, slices), dim3(kDispatchBS), 0, stream, (const u32x4 *)x, nvec, K, nslot,
                           slots, topk_w, topk_idx, (u32x4 *)recv_x, recv_w, recv_idx);
        return hipGetLastError();
    }
    auto fn = place ? pick<Bf16PlaceInst>(iter, nt, ntl, full) : pick<Bf16Inst>(iter, nt, ntl, full);
    hipLaunchKernelGGL(fn, dim3(T), dim3(kDispatchBS), 0, stream, (const u32x4 *)x, nvec, K, nslot,
                       slots, topk_w, topk_idx, (u32x4 *)recv_x, recv_w, recv_idx,
                       place ? *place : PlaceArgs{});
    return hipGetLastError();
}

namespace {

template <bool PLACE>
auto pick_fp8(bool nt, bool ntl, bool full)
{
    if (nt) {
        if (ntl) return full ? dispatch_fp8_kernel<true, true, true, PLACE> : dispatch_fp8_kernel<true, true, false, PLACE>;
        return full ? dispatch_fp8_kernel<true, false, true, PLACE> : dispatch_fp8_kernel<true, false, false, PLACE>;
    }
    if (ntl) return full ? dispatch_fp8_kernel<false, true, true, PLACE> : dispatch_fp8_kernel<false, true, false, PLACE>;
    return full ? dispatch_fp8_kernel<false, false, true, PLACE> : dispatch_fp8_kernel<false, false, false, PLACE>;
}

}  // namespace

namespace {

template <int BS, bool NT, bool NTL, bool PLACE, int WPE>
auto pick_fp8_wave(int iter)
{
    switch (iter) {
    case 1: return dispatch_fp8_wave_kernel<BS, 1, NT, NTL, PLACE, WPE>;
    case 2: return dispatch_fp8_wave_kernel<BS, 2, NT, NTL, PLACE, WPE>;
    case 3: return dispatch_fp8_wave_kernel<BS, 3, NT, NTL, PLACE, WPE>;
    case 4: return dispatch_fp8_wave_kernel<BS, 4, NT, NTL, PLACE, WPE>;
    case 5: return dispatch_fp8_wave_kernel<BS, 5, NT, NTL, PLACE, WPE>;
    case 6: return dispatch_fp8_wave_kernel<BS, 6, NT, NTL, PLACE, WPE>;
    case 7: return dispatch_fp8_wave_kernel<BS, 7, NT, NTL, PLACE, WPE>;
    default: return dispatch_fp8_wave_kernel<BS, 8, NT, NTL, PLACE, WPE>;
    }
}

template <int BS, bool PLACE, int WPE = 1>
auto pick_fp8_wave_flags(int iter, bool nt, bool ntl)
{
    if (nt) return ntl ? pick_fp8_wave<BS, true, true, PLACE, WPE>(iter) : pick_fp8_wave<BS, true, false, PLACE, WPE>(iter);
    return ntl ? pick_fp8_wave<BS, false, true, PLACE, WPE>(iter) : pick_fp8_wave<BS, false, false, PLACE, WPE>(iter);
}

// lanes per token of the small-workgroup FP8 form (0: the row-sized form)
int fp8_small_bs(int H)
{
    const int bs = tuning().fp8_form == 1 ? kWave : (tuning().fp8_form == 2 ? 2 * kWave : 0);
    return bs && H / 16 <= 8 * bs ? bs : 0;
}

}  // namespace

bool fp8_wave_form(int H) { return fp8_small_bs(H) != 0; }

int placing_dispatch_threads(bool fp8, int H) { return fp8 ? fp8_small_bs(H) : kDispatchBS; }

hipError_t launch_dispatch_fp8(const void *x, int T, int H, int K, int nslot, const int32_t *slots,
                               const float *topk_w, const int32_t *topk_idx, void *recv_q,
                               float *recv_scale, float *recv_w, int32_t *recv_idx,
                               const PlaceArgs *place, bool group_rows, hipStream_t stream)
{
    const int nch = H / 16;
    const bool nt = tuning().dispatch_nt_store, ntl = tuning().dispatch_nt_load;
    if (const int sbs = fp8_small_bs(H)) {
        const int iter = (nch + sbs - 1) / sbs;
        // the plain per-group dispatch: 4 waves per SIMD (38.5 against 40.6 us at
        // t4096; the per-expert one and the placing forms are slower so)
        const bool w4 = !place && group_rows && sbs == kWave && tuning().fp8_group_w4;
        auto fn = sbs == kWave
                      ? (place ? pick_fp8_wave_flags<kWave, true>(iter, nt, ntl)
                               : (w4 ? pick_fp8_wave_flags<kWave, false, 4>(iter, nt, ntl)
                                     : pick_fp8_wave_flags<kWave, false>(iter, nt, ntl)))
                      : (place ? pick_fp8_wave_flags<2 * kWave, true>(iter, nt, ntl)
                               : pick_fp8_wave_flags<2 * kWave, false>(iter, nt, ntl));
        hipLaunchKernelGGL(fn, dim3(T), dim3(sbs), 0, stream, (const u32x4 *)x, nch, K, nslot, slots,
                           topk_w, topk_idx, (u32x4 *)recv_q, recv_scale, recv_w, recv_idx,
                           place ? *place : PlaceArgs{});
        return hipGetLastError();
    }
    int bs = (nch + kWave - 1) / kWave * kWave;
    if (bs > kFp8MaxBS) bs = kFp8MaxBS;
    const bool full = nch % bs == 0;
    auto fn = place ? pick_fp8<true>(nt, ntl, full) : pick_fp8<false>(nt, ntl, full);
    hipLaunchKernelGGL(fn, dim3(T), dim3(bs), 0, stream, (const u32x4 *)x, nch, K, nslot, slots,
                       topk_w, topk_idx, (u32x4 *)recv_q, recv_scale, recv_w, recv_idx,
                       place ? *place : PlaceArgs{});
    return hipGetLastError();
}

}  // namespace moe
