/*
 * A plain-C caller of the library, through include/moe_ep.h and libmoe_ep.so
 * only (the HIP runtime's C API for device memory): routing layout, dispatch
 * and combine in both receive layouts on a small deterministic batch, checked
 * on the host by definitions that need no reference implementation:
 *   - the counts sum to T*K, the offsets are their exclusive prefix, and the
 *     group counts are the tokens reaching each group; the status is 0;
 *   - every receive row is a bitwise copy of the source row its receive list
 *     names, with that token's indices;
 *   - combine with identity experts and weights 1/K (exact, summing to 1)
 *     returns every input row bit for bit;
 *   - documented argument errors come back as their codes, with nothing run.
 * Prints "ok" and exits 0 on success; prints the first failure and exits 1.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_ep.h"

enum { T = 300, H = 1024, E = 32, G = 4, K = 4 };

#define CHECK_HIP(x)                                                               \
    do {                                                                           \
        hipError_t e_ = (x);                                                       \
        if (e_ != hipSuccess) {                                                    \
            printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);  \
            return 1;                                                              \
        }                                                                          \
    } while (0)
#define EXPECT(c, ...)                                                             \
    do {                                                                           \
        if (!(c)) {                                                                \
            printf("FAILED line %d: ", __LINE__);                                  \
            printf(__VA_ARGS__);                                                   \
            printf("\n");                                                          \
            return 1;                                                              \
        }                                                                          \
    } while (0)

static uint32_t lcg(uint32_t *s) { return *s = *s * 1664525u + 1013904223u; }

static void *dmalloc(size_t n)
{
    void *p = NULL;
    return hipMalloc(&p, n ? n : 16) == hipSuccess ? p : NULL;
}

static int run_mode(const moe_layout_t *L, int mode, const uint16_t *x, const int32_t *idx,
                    const void *x_d, const float *w_d, const int32_t *idx_d, const int32_t *recv_src,
                    int rows)
{
    const int64_t cap = moe_recv_rows_bound(T, K, G, mode);
    EXPECT(cap >= rows, "row bound %lld below %d", (long long)cap, rows);
    void *recv = dmalloc((size_t)cap * H * 2);
    float *rw = (float *)dmalloc((size_t)cap * K * 4);
    int32_t *ri = (int32_t *)dmalloc((size_t)cap * K * 4);
    void *out = dmalloc((size_t)T * H * 2);
    EXPECT(recv && rw && ri && out, "hipMalloc");
    EXPECT(moe_dispatch(L, mode, MOE_DTYPE_BF16, H, x_d, w_d, idx_d, recv, NULL, rw, ri, cap - 1, NULL) ==
               MOE_ERR_CAPACITY, "capacity below the bound accepted");
    EXPECT(moe_dispatch(L, mode, MOE_DTYPE_BF16, H, x_d, w_d, idx_d, recv, NULL, rw, ri, cap, NULL) == MOE_OK,
           "moe_dispatch");
    EXPECT(moe_combine(L, mode, H, recv, cap, w_d, out, NULL) == MOE_OK, "moe_combine");
    CHECK_HIP(hipDeviceSynchronize());

    uint16_t *hrecv = (uint16_t *)malloc((size_t)rows * H * 2);
    int32_t *hri = (int32_t *)malloc((size_t)rows * K * 4);
    uint16_t *hout = (uint16_t *)malloc((size_t)T * H * 2);
    CHECK_HIP(hipMemcpy(hrecv, recv, (size_t)rows * H * 2, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(hri, ri, (size_t)rows * K * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(hout, out, (size_t)T * H * 2, hipMemcpyDeviceToHost));
    for (int r = 0; r < rows; ++r) {
        const int t = mode == MOE_MODE_EXPERT ? recv_src[r] / K : recv_src[r];
        EXPECT(t >= 0 && t < T, "mode %d row %d names token %d", mode, r, t);
        EXPECT(memcmp(hrecv + (size_t)r * H, x + (size_t)t * H, H * 2) == 0, "mode %d row %d differs", mode, r);
        EXPECT(memcmp(hri + (size_t)r * K, idx + (size_t)t * K, K * 4) == 0, "mode %d row %d indices", mode, r);
    }
    EXPECT(memcmp(hout, x, (size_t)T * H * 2) == 0, "mode %d: combine of identity experts is not x", mode);
    free(hrecv);
    free(hri);
    free(hout);
    hipFree(recv);
    hipFree(rw);
    hipFree(ri);
    hipFree(out);
    return 0;
}

/* moe_layout_dispatch_noalloc (the library's own workspace): rows equal to their
 * source tokens in the per-expert layout, counts equal to moe_layout's. */
static int run_noalloc(moe_layout_t *L, const uint16_t *x, const int32_t *idx, const void *x_d,
                       const float *w_d, const int32_t *idx_d, const int32_t *want_off)
{
    const int64_t cap = moe_recv_rows_bound(T, K, G, MOE_MODE_EXPERT);
    void *recv = dmalloc((size_t)cap * H * 2);
    float *rw = (float *)dmalloc((size_t)cap * K * 4);
    int32_t *ri = (int32_t *)dmalloc((size_t)cap * K * 4);
    EXPECT(recv && rw && ri, "hipMalloc");
    EXPECT(moe_layout_dispatch_noalloc(idx_d, L, MOE_MODE_EXPERT, MOE_DTYPE_BF16, H, x_d, w_d, recv, NULL, rw, ri,
                                       cap, NULL) == MOE_OK,
           "moe_layout_dispatch_noalloc");
    CHECK_HIP(hipDeviceSynchronize());
    int32_t off[E + 1], status = -1;
    static int32_t src[T * K];
    uint16_t *hrecv = (uint16_t *)malloc((size_t)T * K * H * 2);
    CHECK_HIP(hipMemcpy(off, L->expert_offset, sizeof off, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(&status, L->status, 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(src, L->recv_src_e, T * K * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(hrecv, recv, (size_t)T * K * H * 2, hipMemcpyDeviceToHost));
    EXPECT(status == 0, "noalloc status %d", status);
    for (int e = 0; e <= E; ++e) EXPECT(off[e] == want_off[e], "noalloc expert offset %d", e);
    for (int r = 0; r < T * K; ++r) {
        const int t = src[r] / K;
        EXPECT(t >= 0 && t < T && memcmp(hrecv + (size_t)r * H, x + (size_t)t * H, H * 2) == 0,
               "noalloc row %d", r);
    }
    (void)idx;
    free(hrecv);
    hipFree(recv);
    hipFree(rw);
    hipFree(ri);
    return 0;
}

int main(void)
{
    EXPECT(moe_abi_version() == MOE_EP_ABI_VERSION, "ABI version %d", moe_abi_version());
    EXPECT(moe_status_string(MOE_ERR_CAPACITY) != NULL, "status string");

    /* K distinct experts per token (9k mod 32 differs for k < 4), finite bf16
     * values, weights 1/K */
    static int32_t idx[T * K];
    static uint16_t x[T * H];
    static float w[T * K];
    uint32_t s = 12345u;
    for (int t = 0; t < T; ++t)
        for (int k = 0; k < K; ++k) {
            idx[t * K + k] = (int32_t)((7 * t + 9 * k) % E);
            w[t * K + k] = 1.0f / K;
        }
    for (int i = 0; i < T * H; ++i) {
        const uint32_t u = lcg(&s);
        x[i] = (uint16_t)(((u >> 31) << 15) | ((120u + ((u >> 24) & 7u)) << 7) | (u & 0x7Fu));
    }

    int32_t *idx_d = (int32_t *)dmalloc(sizeof idx);
    void *x_d = dmalloc(sizeof x);
    float *w_d = (float *)dmalloc(sizeof w);
    EXPECT(idx_d && x_d && w_d, "hipMalloc");
    CHECK_HIP(hipMemcpy(idx_d, idx, sizeof idx, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(x_d, x, sizeof x, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(w_d, w, sizeof w, hipMemcpyHostToDevice));

    moe_layout_t L;
    memset(&L, 0, sizeof L);
    L.T = T; L.K = K; L.E = E; L.G = G;
    L.expert_count = (int32_t *)dmalloc(E * 4);
    L.expert_offset = (int32_t *)dmalloc((E + 1) * 4);
    L.group_count = (int32_t *)dmalloc(G * 4);
    L.group_offset = (int32_t *)dmalloc((G + 1) * 4);
    L.tok_group_mask = (uint32_t *)dmalloc(T * 4);
    L.slot_e = (int32_t *)dmalloc(T * K * 4);
    L.slot_g = (int32_t *)dmalloc(T * K * 4);
    L.slot_tg = (int32_t *)dmalloc(T * G * 4);
    L.recv_src_e = (int32_t *)dmalloc(T * K * 4);
    L.recv_src_g = (int32_t *)dmalloc(T * (K < G ? K : G) * 4);
    L.status = (int32_t *)dmalloc(4);
    size_t wsb = 0;
    EXPECT(moe_layout_workspace_bytes(T, K, E, G, &wsb) == MOE_OK, "workspace bytes");
    void *ws = dmalloc(wsb);
    EXPECT(L.status && ws, "hipMalloc");

    EXPECT(moe_layout(idx_d, NULL, ws, wsb, NULL) == MOE_ERR_NULL_PTR, "NULL layout accepted");
    EXPECT(moe_layout_workspace_bytes(T, K, 33, G, &wsb) == MOE_ERR_BAD_SHAPE, "E %% G != 0 accepted");
    EXPECT(moe_layout_workspace_bytes(T, K, E, G, &wsb) == MOE_OK, "workspace bytes");
    EXPECT(moe_layout(idx_d, &L, ws, wsb, NULL) == MOE_OK, "moe_layout");
    CHECK_HIP(hipDeviceSynchronize());

    int32_t cnt[E], off[E + 1], gcnt[G], goff[G + 1], status = -1;
    static int32_t src_e[T * K], src_g[T * K];
    CHECK_HIP(hipMemcpy(cnt, L.expert_count, sizeof cnt, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(off, L.expert_offset, sizeof off, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(gcnt, L.group_count, sizeof gcnt, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(goff, L.group_offset, sizeof goff, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(&status, L.status, 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(src_e, L.recv_src_e, T * K * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(src_g, L.recv_src_g, T * (K < G ? K : G) * 4, hipMemcpyDeviceToHost));
    EXPECT(status == 0, "status %d", status);
    int want_cnt[E] = {0}, want_g[G] = {0};
    for (int t = 0; t < T; ++t) {
        uint32_t m = 0;
        for (int k = 0; k < K; ++k) {
            ++want_cnt[idx[t * K + k]];
            m |= 1u << (idx[t * K + k] / (E / G));
        }
        for (int g = 0; g < G; ++g) want_g[g] += (m >> g) & 1u;
    }
    EXPECT(off[0] == 0 && goff[0] == 0, "offsets start at %d, %d", off[0], goff[0]);
    for (int e = 0; e < E; ++e) {
        EXPECT(cnt[e] == want_cnt[e], "expert %d count %d, want %d", e, cnt[e], want_cnt[e]);
        EXPECT(off[e + 1] == off[e] + cnt[e], "expert offset %d", e);
        for (int r = off[e]; r + 1 < off[e + 1]; ++r)
            EXPECT(src_e[r] < src_e[r + 1], "expert %d rows out of token order at %d", e, r);
    }
    for (int g = 0; g < G; ++g) {
        EXPECT(gcnt[g] == want_g[g], "group %d count %d, want %d", g, gcnt[g], want_g[g]);
        EXPECT(goff[g + 1] == goff[g] + gcnt[g], "group offset %d", g);
    }
    EXPECT(off[E] == T * K, "pairs %d", off[E]);

    if (run_mode(&L, MOE_MODE_EXPERT, x, idx, x_d, w_d, idx_d, src_e, off[E])) return 1;
    if (run_mode(&L, MOE_MODE_GROUP, x, idx, x_d, w_d, idx_d, src_g, goff[G])) return 1;
    if (run_noalloc(&L, x, idx, x_d, w_d, idx_d, off)) return 1;
    printf("ok\n");
    return 0;
}
