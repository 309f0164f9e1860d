// Low-latency form of layout + dispatch for small batches: one launch.
//
// "perf(ep): optimize IntraNode dispatch kernel for MI350X" (ROCm/mori pull
// request 586) contrasts its three-phase dispatch with the IntraNodeLL kernel,
// which routes each token in a single pass, one block per token, with the copy
// fused in (the "IntraNodeLL" reply in its review thread); at small token
// counts its tables show latency, not bandwidth, dominating. This is that
// shape on one GPU: one workgroup per token. Every workgroup reads the whole
// (small) index array into LDS and recomputes what it needs of the routing
// layout — the expert and group histograms with their exclusive prefixes, and
// how many earlier tokens chose each of its own experts and groups — writes its
// token's entries of the layout (workgroup 0 also the counts, offsets and
// status), and then copies its row to its destinations exactly as the
// dispatch kernels do. The results are those of moe_layout followed by
// moe_dispatch, bit for bit. The redundant routing work is O(T * K) per
// workgroup, which is why the form is limited to T <= 512.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kFusedBS = 256;
constexpr int kFusedWaves = kFusedBS / kWave;
constexpr int kMaxG = 32;
constexpr int kMaxK = 32;


// LDS layout (ints): idx[T*K] | vmask[T] | gmask[T] | cnt[E] | off[E+1] | gcnt[G] | goff[G+1]
//                    | rank[K] | grank[G] | dst[max(K, G)] | misc
__global__ __launch_bounds__(kFusedBS) void fused_layout_dispatch_kernel(
    const int32_t *__restrict__ idx, int T, int K, int E, int G, uint32_t gmagic, LayoutPtrs L,
    int mode, int fp8, int H, const u32x4 *__restrict__ x, const float *__restrict__ topk_w,
    u32x4 *__restrict__ recv_x, float *__restrict__ recv_scale, float *__restrict__ recv_w,
    int32_t *__restrict__ recv_idx, int nt_store)
{
    extern __shared__ int sm[];
    int *s_idx = sm;
    uint32_t *s_vmask = reinterpret_cast<uint32_t *>(s_idx + T * K);
    uint32_t *s_gmask = s_vmask + T;
    int *s_cnt = reinterpret_cast<int *>(s_gmask + T);
    int *s_off = s_cnt + E;
    int *s_gcnt = s_off + E + 1;
    int *s_goff = s_gcnt + G;
    __shared__ int s_rank[kMaxK];
    __shared__ int s_grank[kMaxG];
    __shared__ int s_dst[kMaxK > kMaxG ? kMaxK : kMaxG];
    __shared__ int s_red[kFusedWaves];
    __shared__ int s_err;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int t = blockIdx.x;

    // 1. The index array into LDS (all loads of a batch issued before the
    //    first is stored); counters cleared.
    constexpr int kLoadBatch = 16;
    for (int b0 = 0; b0 < T * K; b0 += kFusedBS * kLoadBatch) {
        int v[kLoadBatch];
#pragma unroll
        for (int u = 0; u < kLoadBatch; ++u) {
            const int i = b0 + u * kFusedBS + tid;
            v[u] = i < T * K ? idx[i] : 0;
        }
#pragma unroll
        for (int u = 0; u < kLoadBatch; ++u) {
            const int i = b0 + u * kFusedBS + tid;
            if (i < T * K) s_idx[i] = v[u];
        }
    }
    for (int i = tid; i < E; i += kFusedBS) s_cnt[i] = 0;
    if (tid < G) s_gcnt[tid] = 0;
    if (tid < kMaxK) s_rank[tid] = 0;
    if (tid < kMaxG) s_grank[tid] = 0;
    if (tid == 0) s_err = 0;
    __syncthreads();

    // 2. Validity and group masks of every token (one thread per token), the
    //    expert histogram, and the group histogram by one ballot per group.
    int err = 0;
    for (int tb = 0; tb < T; tb += kFusedBS) {
        const int u = tb + tid;
        uint32_t vm = 0, gm = 0;
        if (u < T) {
            for (int k = 0; k < K; ++k) {
                const int e = s_idx[u * K + k];
                if ((unsigned)e >= (unsigned)E) { err |= 1; continue; }
                bool rep = false;
                for (int k2 = 0; k2 < k; ++k2) rep = rep || s_idx[u * K + k2] == e;
                if (rep) { err |= 2; continue; }
                vm |= 1u << k;
                gm |= 1u << group_of(e, gmagic);
                atomicAdd(&s_cnt[e], 1);
            }
            s_vmask[u] = vm;
            s_gmask[u] = gm;
        }
        for (int g = 0; g < G; ++g) {
            const uint64_t b = __ballot((gm >> g) & 1u);
            if (lane == 0 && b) atomicAdd(&s_gcnt[g], __popcll(b));
        }
    }
    if (err) atomicOr(&s_err, err);
    __syncthreads();

    // 3. Exclusive prefixes: experts by a workgroup scan (E <= 1024, up to
    //    four consecutive experts per thread), groups in wave 0.
    {
        const int ept = (E + kFusedBS - 1) / kFusedBS;
        int c[4], local = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = tid * ept + j;
            c[j] = (j < ept && e < E) ? s_cnt[e] : 0;
            local += c[j];
        }
        const int incl = wave_incl_scan(local);
        if (lane == kWave - 1) s_red[wave] = incl;
        __syncthreads();
        int base = 0;
        for (int w = 0; w < wave; ++w) base += s_red[w];
        int run = base + incl - local;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = tid * ept + j;
            if (j < ept && e < E) s_off[e] = run;
            run += c[j];
        }
        if (tid == kFusedBS - 1) s_off[E] = run;
    }
    if (wave == 0) {
        const int gt = lane < G ? s_gcnt[lane] : 0;
        const int incl = wave_incl_scan(gt);
        if (lane < G) s_goff[lane] = incl - gt;
        if (lane == G - 1) s_goff[G] = incl;
    }

    // 4. Ranks of this token: for each of its valid experts, the earlier
    //    tokens that chose it; for each of its groups, the earlier tokens that
    //    reach it. Lanes take the earlier tokens in turn; each wave counts its
    //    matches with a ballot and adds them with one LDS atomic.
    const uint32_t my_vm = s_vmask[t], my_gm = s_gmask[t];
    for (int ub = 0; ub < t; ub += kFusedBS) {
        const int u = ub + tid;
        const bool in = u < t;
        const uint32_t vm = in ? s_vmask[u] : 0u, gm = in ? s_gmask[u] : 0u;
        for (int k = 0; k < K; ++k) {
            if (!((my_vm >> k) & 1u)) continue;   // uniform
            const int x0 = s_idx[t * K + k];
            bool hit = false;
            for (int k2 = 0; k2 < K; ++k2) hit = hit || (((vm >> k2) & 1u) && s_idx[u * K + k2] == x0);
            const uint64_t b = __ballot(hit);
            if (lane == 0 && b) atomicAdd(&s_rank[k], __popcll(b));
        }
        for (int g = 0; g < G; ++g) {
            if (!((my_gm >> g) & 1u)) continue;   // uniform
            const uint64_t b = __ballot((gm >> g) & 1u);
            if (lane == 0 && b) atomicAdd(&s_grank[g], __popcll(b));
        }
    }
    __syncthreads();

    // 5. This token's layout entries; workgroup 0 also the counts, offsets, status.
    if (tid < K) {
        const int k = tid;
        const bool ok = (my_vm >> k) & 1u;
        const int e = s_idx[t * K + k];
        const int se = ok ? s_off[e] + s_rank[k] : -1;
        int sg = -1;
        if (ok) {
            const int g = group_of(e, gmagic);
            sg = s_goff[g] + s_grank[g];
            L.recv_src_e[se] = t * K + k;
        }
        L.slot_e[(size_t)t * K + k] = se;
        L.slot_g[(size_t)t * K + k] = sg;
        if (mode == 0) s_dst[k] = se;
    }
    if (tid >= kWave && tid < kWave + G) {
        const int g = tid - kWave;
        const bool hit = (my_gm >> g) & 1u;
        const int s = hit ? s_goff[g] + s_grank[g] : -1;
        if (hit) L.recv_src_g[s] = t;
        L.slot_tg[(size_t)t * G + g] = s;
        if (mode == 1) s_dst[g] = s;
    }
    if (tid == 2 * kWave) L.tok_group_mask[t] = my_gm;
    if (t == 0) {
        for (int e = tid; e < E; e += kFusedBS) {
            L.expert_count[e] = s_cnt[e];
            L.expert_offset[e] = s_off[e];
        }
        if (tid == 0) L.expert_offset[E] = s_off[E];
        if (tid < G) {
            L.group_count[tid] = s_gcnt[tid];
            L.group_offset[tid] = s_goff[tid];
        }
        if (tid == 0) {
            L.group_offset[G] = s_goff[G];
            *L.status = s_err;
        }
    }
    __syncthreads();

    // 6. The copy (as the dispatch kernels): bf16 rows, or e4m3 bytes + scales.
    const int nslot = mode == 0 ? K : G;
    if (!fp8) {
        // the row in registers (up to kRowBatch vectors per lane per pass),
        // then written to each destination
        constexpr int kRowBatch = 8;
        const int nvec = H / 8;
        const u32x4 *src = x + (size_t)t * nvec;
        for (int b0 = 0; b0 < nvec; b0 += kFusedBS * kRowBatch) {
            u32x4 v[kRowBatch];
#pragma unroll
            for (int u = 0; u < kRowBatch; ++u) {
                const int j = b0 + u * kFusedBS + tid;
                if (j < nvec) v[u] = __builtin_nontemporal_load(src + j);
            }
            for (int d = 0; d < nslot; ++d) {
                const int s = s_dst[d];
                if (s < 0) continue;
                u32x4 *dst = recv_x + (size_t)s * nvec;
#pragma unroll
                for (int u = 0; u < kRowBatch; ++u) {
                    const int j = b0 + u * kFusedBS + tid;
                    if (j < nvec) {
                        if (nt_store) store16<true>(dst + j, v[u]);
                        else store16<false>(dst + j, v[u]);
                    }
                }
            }
        }
    } else {
        const int nch = H / 16, nblk = nch / 8;
        const u32x4 *src = x + (size_t)t * nch * 2;
        for (int j = tid; j - tid < nch; j += kFusedBS) {   // whole passes: the shuffles need all lanes
            const bool in = j < nch;
            u32x4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
            if (in) {
                a = __builtin_nontemporal_load(src + 2 * j);
                b = __builtin_nontemporal_load(src + 2 * j + 1);
            }
            u32x4 q;
            float scale;
            quantize16(a, b, q, scale);
            if (in) {
                for (int d = 0; d < nslot; ++d) {
                    const int s = s_dst[d];
                    if (s < 0) continue;
                    if (nt_store) store16<true>(recv_x + (size_t)s * nch + j, q);
                    else store16<false>(recv_x + (size_t)s * nch + j, q);
                    if ((tid & 7) == 0) recv_scale[(size_t)s * nblk + (j >> 3)] = scale;
                }
            }
        }
    }
    // metadata: lanes [0, K) weights, [K, 2K) indices
    const bool wl = tid < K, il = tid >= K && tid < 2 * K;
    float wv = 0.f;
    int iv = 0;
    if (wl) wv = topk_w[(size_t)t * K + tid];
    if (il) iv = idx[(size_t)t * K + tid - K];
    for (int d = 0; d < nslot; ++d) {
        const int s = s_dst[d];
        if (s < 0) continue;
        if (wl) recv_w[(size_t)s * K + tid] = wv;
        if (il) recv_idx[(size_t)s * K + tid - K] = iv;
    }
}

}  // namespace

size_t fused_lds_bytes(int T, int K, int E, int G)
{
    return sizeof(int) * ((size_t)T * K + 2 * (size_t)T + E + (E + 1) + G + (G + 1));
}

hipError_t launch_layout_dispatch(const int32_t *idx, int T, int K, int E, int G, const LayoutPtrs &L,
                                  int mode, int fp8, int H, const void *x, const float *topk_w,
                                  void *recv_x, float *recv_scale, float *recv_w, int32_t *recv_idx,
                                  hipStream_t stream)
{
    const uint32_t gmagic = group_magic(E, G);
    static const hipError_t lds_ok = hipFuncSetAttribute(
        reinterpret_cast<const void *>(fused_layout_dispatch_kernel),
        hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024);
    if (lds_ok != hipSuccess) return lds_ok;
    hipLaunchKernelGGL(fused_layout_dispatch_kernel, dim3(T), dim3(kFusedBS), fused_lds_bytes(T, K, E, G),
                       stream, idx, T, K, E, G, gmagic, L, mode, fp8, H, (const u32x4 *)x, topk_w,
                       (u32x4 *)recv_x, recv_scale, recv_w, recv_idx,
                       (int)tuning().dispatch_nt_store);
    return hipGetLastError();
}

}  // namespace moe
