// Combine on gfx950: gather each token's expert outputs and reduce them as a
// weighted top-k sum, accumulated in fp32 in fixed k order and rounded once
// to bf16. Also the FP8 identity expert (dequantisation glue) and a plain
// copy kernel used as a measurement reference.
//
// Combine is what "perf(ep): optimize IntraNode dispatch kernel for MI350X"
// (ROCm/mori pull request 586) describes as reads of the expert rows plus FMA
// accumulation with no routing phase ("Remaining gap — profiled root cause"):
// the rows are found through the layout's cached slots. The single rounding
// of an fp32 accumulator follows ROCm/vllm pull request 1297, Accuracy.
//
// Design. One workgroup per token; each lane owns ITER 16-byte vectors (8
// elements each) of the output row per pass and keeps their fp32
// accumulators in registers (ITER = 1 with the workgroup sized to the row
// where it divides evenly into waves, which measured best). For a token whose
// K slots are all valid (the normal case) the rows are read either row by row
// in contiguous bursts (per-expert layout) or column by column with the next
// column prefetched (per-group layout, where rows repeat), and folded with one
// fmaf per element and k, in k order, starting from -0. Tokens with skipped
// entries take a general loop with the same arithmetic. The sums are rounded
// to bf16 by the packed hardware conversion (round to nearest even; see
// pack_bf16x2). Nothing here is a dense contraction (K <= 32 weights per
// row), so there is no MFMA: the kernel is bound by the HBM reads of the
// expert rows.
#include "common.hpp"
#include "kernels.hpp"
#include "moe_ep.h"

namespace moe {

namespace {

constexpr int kCombineBS = 128;      // workgroup size of the general shape
constexpr int kCombineMaxBS = 1024;
constexpr int kMaxIter = 8;

__device__ __forceinline__ void fma8(float (&acc)[8], float w, u32x4 v)
{
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        acc[2 * m] = fmaf(w, bf16_lo(v[m]), acc[2 * m]);
        acc[2 * m + 1] = fmaf(w, bf16_hi(v[m]), acc[2 * m + 1]);
    }
}

__device__ __forceinline__ u32x4 pack8(const float (&acc)[8])
{
    return u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                 pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
}

// KT > 0: fast path compiled for exactly KT valid entries; KT == 0: general only.
// ROWWISE: traversal of the fast path (see below). Rows are read with
// non-temporal loads (each byte of y is read once in the per-expert layout)
// and the output is written with plain stores, the faster pair measured on
// MI355X.
template <int ITER, int KT, bool ROWWISE, bool FULL>
__global__ __launch_bounds__(kCombineMaxBS) void combine_kernel(
    const u32x4 *__restrict__ y, int64_t y_rows, int nvec, int K,
    const int32_t *__restrict__ slot, const float *__restrict__ topk_w, u32x4 *__restrict__ out,
    int32_t *__restrict__ status)
{
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const int bs = blockDim.x;   // a multiple of 64; bs * ITER vectors per pass
    const int32_t *ts = slot + (size_t)t * K;
    const float *tw = topk_w + (size_t)t * K;
    u32x4 *orow = out + (size_t)t * nvec;

    bool fast = KT > 0 && KT == K;
    if constexpr (KT > 0) {
#pragma unroll
        for (int k = 0; k < KT; ++k) {
            const int s = ts[k];
            fast = fast && s >= 0 && s < y_rows;
        }
    }

    if constexpr (KT > 0) {
        if (fast) {
            const u32x4 *rows[KT];
            float w[KT];
#pragma unroll
            for (int k = 0; k < KT; ++k) {
                rows[k] = y + (size_t)ts[k] * nvec;
                w[k] = tw[k];
            }
            if constexpr (ROWWISE && FULL) {
                // Row-wise: wave w owns the contiguous span of ITER * 64 vectors
                // starting at w * ITER * 64 of every pass; it reads that span of
                // row k (ITER loads of 1 KiB, back to back in memory), folds it
                // into ITER x 8 fp32 accumulators, then moves to row k + 1. Each
                // row is thus visited in long contiguous bursts, and the fma
                // chain of every element still runs in k order.
                const int wave = tid / kWave, lane = tid % kWave;
                for (int base = 0; base < nvec; base += bs * ITER) {
                    const int j0 = base + wave * (kWave * ITER) + lane;
                    float acc[ITER][8];
#pragma unroll
                    for (int i = 0; i < ITER; ++i)
#pragma unroll
                        for (int m = 0; m < 8; ++m) acc[i][m] = -0.f;
#pragma unroll
                    for (int k = 0; k < KT; ++k) {
                        u32x4 v[ITER];
#pragma unroll
                        for (int i = 0; i < ITER; ++i) v[i] = load16<true>(rows[k] + j0 + i * kWave);
#pragma unroll
                        for (int i = 0; i < ITER; ++i) fma8(acc[i], w[k], v[i]);
                    }
#pragma unroll
                    for (int i = 0; i < ITER; ++i) store16<false>(orow + j0 + i * kWave, pack8(acc[i]));
                }
            } else if constexpr (FULL) {
                // Column-wise, double-buffered: pass i reads one vector of each
                // of the K rows; the K loads of pass i + 1 are issued before the
                // FMAs of pass i, so 2K row loads per lane stay in flight. Used
                // for the per-group layout, where one token's K slots repeat
                // rows: the repeats are loaded back to back, while still cached.
                for (int base = 0; base < nvec; base += bs * ITER) {
                    u32x4 cur[KT], nxt[KT];
#pragma unroll
                    for (int k = 0; k < KT; ++k) cur[k] = load16<true>(rows[k] + base + tid);
#pragma unroll
                    for (int i = 0; i < ITER; ++i) {
                        const int j = base + i * bs + tid;
                        if (i + 1 < ITER) {
#pragma unroll
                            for (int k = 0; k < KT; ++k) nxt[k] = load16<true>(rows[k] + j + bs);
                        }
                        float acc[8];
#pragma unroll
                        for (int m = 0; m < 8; ++m) acc[m] = -0.f;
#pragma unroll
                        for (int k = 0; k < KT; ++k) fma8(acc, w[k], cur[k]);
                        store16<false>(orow + j, pack8(acc));
                        if (i + 1 < ITER) {
#pragma unroll
                            for (int k = 0; k < KT; ++k) cur[k] = nxt[k];
                        }
                    }
                }
            } else {
                for (int base = 0; base < nvec; base += bs * ITER) {
#pragma unroll
                    for (int i = 0; i < ITER; ++i) {
                        const int j = base + i * bs + tid;
                        if (FULL || j < nvec) {
                            u32x4 v[KT];
#pragma unroll
                            for (int k = 0; k < KT; ++k) v[k] = load16<true>(rows[k] + j);
                            float acc[8];
#pragma unroll
                            for (int m = 0; m < 8; ++m) acc[m] = -0.f;
#pragma unroll
                            for (int k = 0; k < KT; ++k) fma8(acc, w[k], v[k]);
                            store16<false>(orow + j, pack8(acc));
                        }
                    }
                }
            }
            return;
        }
    }

    // General path: any K, entries with slot < 0 skipped, slots >= y_rows
    // skipped and reported.
    if (tid == 0) {
        for (int k = 0; k < K; ++k)
            if (ts[k] >= y_rows) { atomicOr(status, MOE_STATUS_Y_ROWS); break; }
    }
    for (int j = tid; j < nvec; j += bs) {
        float acc[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) acc[m] = -0.f;
        for (int k = 0; k < K; ++k) {
            const int s = ts[k];
            if (s < 0 || s >= y_rows) continue;
            fma8(acc, tw[k], load16<true>(y + (size_t)s * nvec + j));
        }
        store16<false>(orow + j, pack8(acc));
    }
}

template <int ITER, int KT>
auto pick_variant(bool rowwise, bool full)
{
    if (rowwise) return full ? combine_kernel<ITER, KT, true, true> : combine_kernel<ITER, KT, true, false>;
    return full ? combine_kernel<ITER, KT, false, true> : combine_kernel<ITER, KT, false, false>;
}

template <int KT>
auto pick_iter(int iter, bool rowwise, bool full)
{
    switch (iter) {
    case 1: return pick_variant<1, KT>(rowwise, full);
    case 2: return pick_variant<2, KT>(rowwise, full);
    case 3: return pick_variant<3, KT>(rowwise, full);
    case 4: return pick_variant<4, KT>(rowwise, full);
    case 5: return pick_variant<5, KT>(rowwise, full);
    case 6: return pick_variant<6, KT>(rowwise, full);
    case 7: return pick_variant<7, KT>(rowwise, full);
    default: return pick_variant<8, KT>(rowwise, full);
    }
}

__global__ __launch_bounds__(256) void fp8_dequant_kernel(
    const u32x4 *__restrict__ q, const float *__restrict__ scale, u32x4 *__restrict__ y, int nch,
    const int32_t *__restrict__ nrows)
{
    const int r = blockIdx.x;
    if (r >= *nrows) return;
    const int nblk = nch / 8;
    for (int j = threadIdx.x; j < nch; j += blockDim.x) {
        const u32x4 v = q[(size_t)r * nch + j];
        const float s = scale[(size_t)r * nblk + (j >> 3)];
        uint32_t o[8];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int word = (int)v[m];
            const float f0 = __builtin_amdgcn_cvt_f32_fp8(word, 0) * s;
            const float f1 = __builtin_amdgcn_cvt_f32_fp8(word, 1) * s;
            const float f2 = __builtin_amdgcn_cvt_f32_fp8(word, 2) * s;
            const float f3 = __builtin_amdgcn_cvt_f32_fp8(word, 3) * s;
            o[2 * m] = pack_bf16x2(f0, f1);
            o[2 * m + 1] = pack_bf16x2(f2, f3);
        }
        y[(size_t)r * nch * 2 + 2 * j] = u32x4{o[0], o[1], o[2], o[3]};
        y[(size_t)r * nch * 2 + 2 * j + 1] = u32x4{o[4], o[5], o[6], o[7]};
    }
}

__global__ __launch_bounds__(256) void ref_copy_kernel(const u32x4 *__restrict__ src,
                                                       u32x4 *__restrict__ dst, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src[i];
}

// Measurement aid: the read/write mix of a combine (NR rows read per row
// written) or of a dispatch (one row read, NW written) over contiguous rows,
// with the same cache policy (non-temporal loads, plain stores) and shape (one
// workgroup per unit, one 16-byte vector per lane and pass). Unit u reads rows
// u * NR .. u * NR + NR - 1 of src, all NR loads in flight, and writes their
// XOR to rows u * NW .. u * NW + NW - 1 of dst.
template <int NR, int NW>
__global__ __launch_bounds__(kCombineMaxBS) void ref_mix_kernel(const u32x4 *__restrict__ src,
                                                                u32x4 *__restrict__ dst, int nvec)
{
    const size_t u = blockIdx.x;
    for (int j = threadIdx.x; j < nvec; j += blockDim.x) {
        u32x4 v[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) v[r] = load16<true>(src + (u * NR + r) * nvec + j);
        u32x4 acc = v[0];
#pragma unroll
        for (int r = 1; r < NR; ++r) acc ^= v[r];
#pragma unroll
        for (int w = 0; w < NW; ++w) store16<false>(dst + (u * NW + w) * nvec + j, acc);
    }
}

inline int iters_for(int n, int bs)
{
    const int it = (n + bs - 1) / bs;
    return it < 1 ? 1 : (it > kMaxIter ? kMaxIter : it);
}

}  // namespace

hipError_t launch_ref_mix(void *dst, const void *src, int64_t row_bytes, int64_t units, int nr, int nw,
                          hipStream_t stream)
{
    const int nvec = (int)(row_bytes / 16);
    int bs = (nvec + kWave - 1) / kWave * kWave;
    if (bs > kCombineMaxBS) bs = kCombineMaxBS;
    void (*fn)(const u32x4 *, u32x4 *, int) = nullptr;
    if (nr == 1 && nw == 1) fn = ref_mix_kernel<1, 1>;
    else if (nw == 1) fn = nr == 2 ? ref_mix_kernel<2, 1> : (nr == 4 ? ref_mix_kernel<4, 1> : ref_mix_kernel<8, 1>);
    else fn = nw == 2 ? ref_mix_kernel<1, 2> : (nw == 4 ? ref_mix_kernel<1, 4> : ref_mix_kernel<1, 8>);
    hipLaunchKernelGGL(fn, dim3((unsigned)units), dim3(bs), 0, stream, (const u32x4 *)src, (u32x4 *)dst, nvec);
    return hipGetLastError();
}

hipError_t launch_combine(const void *y, int64_t y_rows, int T, int H, int K, const int32_t *slot,
                          bool rows_repeat, const float *topk_w, void *out, int32_t *status,
                          hipStream_t stream)
{
    // Shape: one vector per lane and one workgroup lane per vector when the
    // row is whole waves of at most 1024 vectors (896 threads at H = 7168);
    // else two per lane when that fits; else 128 threads with up to kMaxIter
    // vectors per lane. (One per lane measured equal to two per lane for the
    // per-expert layout and about 10% faster for the per-group layout.)
    const int nvec = H / 8;
    int bs, iter;
    if (nvec % kWave == 0 && nvec <= kCombineMaxBS) {
        bs = nvec;
        iter = 1;
    } else if (nvec % (2 * kWave) == 0 && nvec / 2 <= kCombineMaxBS) {
        bs = nvec / 2;
        iter = 2;
    } else {
        bs = kCombineBS;
        iter = iters_for(nvec, kCombineBS);
    }
    const bool full = nvec % (bs * iter) == 0;
    const bool rowwise = !rows_repeat;
    void (*fn)(const u32x4 *, int64_t, int, int, const int32_t *, const float *, u32x4 *, int32_t *);
    switch (K) {
    case 2: fn = pick_iter<2>(iter, rowwise, full); break;
    case 4: fn = pick_iter<4>(iter, rowwise, full); break;
    case 6: fn = pick_iter<6>(iter, rowwise, full); break;
    case 8: fn = pick_iter<8>(iter, rowwise, full); break;
    default: fn = pick_iter<0>(iter, rowwise, full); break;
    }
    hipLaunchKernelGGL(fn, dim3(T), dim3(bs), 0, stream, (const u32x4 *)y, y_rows, nvec, K,
                       slot, topk_w, (u32x4 *)out, status);
    return hipGetLastError();
}

hipError_t launch_fp8_dequant(const void *q, const float *scale, void *y, int64_t capacity, int H,
                              const int32_t *nrows, hipStream_t stream)
{
    hipLaunchKernelGGL(fp8_dequant_kernel, dim3((unsigned)capacity), dim3(256), 0, stream,
                       (const u32x4 *)q, scale, (u32x4 *)y, H / 16, nrows);
    return hipGetLastError();
}

hipError_t launch_ref_copy(void *dst, const void *src, int64_t bytes, hipStream_t stream)
{
    const int64_t n = bytes / 16;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 256 * 64) blocks = 256 * 64;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(ref_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const u32x4 *)src, (u32x4 *)dst, n);
    return hipGetLastError();
}

}  // namespace moe
