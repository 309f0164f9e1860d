/*
 * Test infrastructure: drives every function of oracle.c over edge shapes and
 * special values with exactly sized heap buffers, so that a build with
 * -fsanitize=address,undefined reports any out-of-bounds access or undefined
 * behaviour in the oracle. A few consistency checks ride along (counts sum to
 * the valid pairs, each receive list is a permutation, identity round trips).
 * Prints "ok" and exits 0; a sanitizer report or a failed check exits non-zero.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float oracle_bf16_to_f32(uint16_t h);
uint16_t oracle_f32_to_bf16(float f);
float oracle_e4m3_to_f32(uint8_t c);
uint8_t oracle_f32_to_e4m3(float f);
int oracle_layout(int T, int K, int E, int G, const int32_t *idx, int32_t *expert_count,
                  int32_t *expert_offset, int32_t *group_count, int32_t *group_offset,
                  uint32_t *tok_group_mask, int32_t *slot_e, int32_t *slot_g, int32_t *slot_tg,
                  int32_t *recv_src_e, int32_t *recv_src_g);
void oracle_dispatch_bf16(int mode, int K, int H, int64_t R, const int32_t *recv_src, const uint16_t *x,
                          const float *topk_w, const int32_t *topk_idx, uint16_t *recv_x, float *recv_w,
                          int32_t *recv_idx);
void oracle_dispatch_fp8(int mode, int T, int K, int H, int64_t R, const int32_t *recv_src,
                         const uint16_t *x, const float *topk_w, const int32_t *topk_idx, uint8_t *recv_q,
                         float *recv_scale, float *recv_w, int32_t *recv_idx);
void oracle_quantize_row_fp8(int H, const uint16_t *xrow, uint8_t *q, float *scale);
void oracle_dequant_fp8(int64_t R, int H, const uint8_t *q, const float *scale, uint16_t *y);
void oracle_combine(int T, int K, int H, const int32_t *slot, const uint16_t *y, const float *topk_w,
                    uint16_t *out);
void oracle_f32_to_bf16_n(int64_t n, const float *in, uint16_t *out);
void oracle_f32_to_e4m3_n(int64_t n, const float *in, uint8_t *out);
void oracle_regroup_rows(int64_t R, int64_t row_bytes, const int32_t *recv_src_e, const int32_t *slot_g,
                         const void *rows_g, void *rows_e);
void oracle_cast_transpose_fp8(int E, int H, const int32_t *expert_offset, const uint16_t *x,
                               const float *scale, uint8_t *c_out, uint8_t *t_out, float *amax,
                               int32_t *pad_offset);

#define CHECK(c)                                                            \
    do {                                                                    \
        if (!(c)) {                                                         \
            printf("check failed: %s (line %d)\n", #c, __LINE__);           \
            exit(2);                                                        \
        }                                                                   \
    } while (0)

static uint32_t st = 2024u;
static uint32_t rnd(void) { return st = st * 1664525u + 1013904223u; }
static void *alloc(size_t n) { void *p = malloc(n ? n : 1); CHECK(p != NULL); return p; }

static void one_case(int T, int K, int E, int G, int H, int invalid)
{
    const size_t TK = (size_t)T * K, KG = (size_t)T * (K < G ? K : G);
    int32_t *idx = alloc(TK * 4);
    for (int t = 0; t < T; ++t)
        for (int k = 0; k < K; ++k) {
            int e = (int)(rnd() % (uint32_t)E);
            if (invalid && rnd() % 16 == 0) e = (rnd() & 1) ? -1 - (int)(rnd() % 5) : E + (int)(rnd() % 5);
            idx[(size_t)t * K + k] = e;   /* repeats are likely: invalid entries too */
        }
    if (!invalid)   /* distinct experts per token: a shuffled prefix of 0..E-1 */
        for (int t = 0; t < T; ++t) {
            int *perm = alloc((size_t)E * sizeof(int));
            for (int e = 0; e < E; ++e) perm[e] = e;
            for (int e = E - 1; e > 0; --e) { int j = (int)(rnd() % (uint32_t)(e + 1)); int s = perm[e]; perm[e] = perm[j]; perm[j] = s; }
            for (int k = 0; k < K; ++k) idx[(size_t)t * K + k] = perm[k];
            free(perm);
        }
    int32_t *ec = alloc((size_t)E * 4), *eo = alloc(((size_t)E + 1) * 4);
    int32_t *gc = alloc((size_t)G * 4), *go = alloc(((size_t)G + 1) * 4);
    uint32_t *tgm = alloc((size_t)T * 4);
    int32_t *se = alloc(TK * 4), *sg = alloc(TK * 4), *stg = alloc((size_t)T * G * 4);
    int32_t *rse = alloc(TK * 4), *rsg = alloc(KG * 4);
    const int status = oracle_layout(T, K, E, G, idx, ec, eo, gc, go, tgm, se, sg, stg, rse, rsg);
    size_t nvalid = 0;
    for (size_t p = 0; p < TK; ++p) nvalid += se[p] >= 0;
    CHECK((size_t)eo[E] == nvalid && (invalid || nvalid == TK) && (invalid || status == 0));
    const int64_t RE = eo[E], RG = go[G];
    CHECK(RG <= (int64_t)KG);

    uint16_t *x = alloc((size_t)T * H * 2);
    float *w = alloc(TK * 4);
    for (size_t i = 0; i < (size_t)T * H; ++i) {
        uint32_t u = rnd();
        uint16_t b = (uint16_t)(u >> 16);
        if ((b & 0x7F80) == 0x7F80) b ^= 0x4000;    /* finite */
        x[i] = b;
    }
    for (size_t i = 0; i < TK; ++i) w[i] = 1.0f / (float)K;
    for (int mode = 0; mode < 2; ++mode) {
        const int64_t R = mode == 0 ? RE : RG;
        const int32_t *src = mode == 0 ? rse : rsg;
        uint16_t *rx = alloc((size_t)R * H * 2);
        float *rw = alloc((size_t)R * K * 4);
        int32_t *ri = alloc((size_t)R * K * 4);
        oracle_dispatch_bf16(mode, K, H, R, src, x, w, idx, rx, rw, ri);
        uint16_t *out = alloc((size_t)T * H * 2);
        oracle_combine(T, K, H, mode == 0 ? se : sg, rx, w, out);
        if (H % 128 == 0) {
            uint8_t *q = alloc((size_t)R * H);
            float *sc = alloc((size_t)R * (H / 128) * 4);
            oracle_dispatch_fp8(mode, T, K, H, R, src, x, w, idx, q, sc, rw, ri);
            uint16_t *y = alloc((size_t)R * H * 2);
            oracle_dequant_fp8(R, H, q, sc, y);
            free(q); free(sc); free(y);
        }
        if (mode == 1) {   /* regroup the per-group rows: equal to the per-expert dispatch */
            uint16_t *re = alloc((size_t)RE * H * 2), *rx_e = alloc((size_t)RE * H * 2);
            float *rw_e = alloc((size_t)RE * K * 4);
            int32_t *ri_e = alloc((size_t)RE * K * 4);
            oracle_regroup_rows(RE, (int64_t)H * 2, rse, sg, rx, re);
            oracle_dispatch_bf16(0, K, H, RE, rse, x, w, idx, rx_e, rw_e, ri_e);
            CHECK(memcmp(re, rx_e, (size_t)RE * H * 2) == 0);
            free(re); free(rx_e); free(rw_e); free(ri_e);
        }
        free(rx); free(rw); free(ri); free(out);
    }
    /* cast-transpose of the per-expert rows (experts may be empty) */
    {
        uint16_t *rx = alloc((size_t)RE * H * 2);
        float *rw = alloc((size_t)RE * K * 4);
        int32_t *ri = alloc((size_t)RE * K * 4);
        oracle_dispatch_bf16(0, K, H, RE, rse, x, w, idx, rx, rw, ri);
        size_t tot = 0;
        for (int e = 0; e < E; ++e) tot += (size_t)(ec[e] + 15) / 16 * 16;
        float *scale = alloc((size_t)E * 4), *amax = alloc((size_t)E * 4);
        for (int e = 0; e < E; ++e) { scale[e] = 0.5f + (float)(rnd() % 100); amax[e] = 0.0f; }
        uint8_t *c = alloc((size_t)RE * H), *tt = alloc(tot * (size_t)H);
        int32_t *po = alloc(((size_t)E + 1) * 4);
        oracle_cast_transpose_fp8(E, H, eo, rx, scale, c, tt, amax, po);
        CHECK((size_t)po[E] == tot);
        free(rx); free(rw); free(ri); free(scale); free(amax); free(c); free(tt); free(po);
    }
    free(idx); free(ec); free(eo); free(gc); free(go); free(tgm); free(se); free(sg); free(stg);
    free(rse); free(rsg); free(x); free(w);
}

int main(void)
{
    /* T, K, E, G, H, invalid entries */
    one_case(0, 8, 256, 8, 128, 0);
    one_case(1, 1, 1, 1, 8, 0);
    one_case(37, 4, 16, 4, 256, 0);
    one_case(37, 4, 16, 4, 264, 1);
    one_case(64, 32, 32, 32, 128, 0);    /* K = E = G */
    one_case(100, 8, 8, 1, 128, 0);      /* K = E, one group */
    one_case(300, 8, 256, 8, 512, 1);
    one_case(129, 6, 1024, 32, 128, 1);
    /* codecs on special values */
    const uint32_t specials[] = {0x00000000u, 0x80000000u, 0x00000001u, 0x807FFFFFu, 0x7F7FFFFFu, 0xFF7FFFFFu,
                                 0x7F800000u, 0xFF800000u, 0x7FC00000u, 0xFFFFFFFFu, 0x7F800001u, 0x43E00000u,
                                 0x43E80000u, 0x3A800000u, 0x3A000000u};
    const int ns = (int)(sizeof specials / sizeof specials[0]);
    float *f = alloc((size_t)ns * 4);
    uint16_t *h = alloc((size_t)ns * 2);
    uint8_t *c = alloc((size_t)ns);
    for (int i = 0; i < ns; ++i) memcpy(&f[i], &specials[i], 4);
    oracle_f32_to_bf16_n(ns, f, h);
    oracle_f32_to_e4m3_n(ns, f, c);
    for (int i = 0; i < ns; ++i) {
        (void)oracle_bf16_to_f32(h[i]);
        (void)oracle_e4m3_to_f32(c[i]);
        (void)oracle_f32_to_bf16(f[i]);
        (void)oracle_f32_to_e4m3(f[i]);
    }
    for (int code = 0; code < 256; ++code) CHECK(oracle_f32_to_e4m3(oracle_e4m3_to_f32((uint8_t)code)) == (uint8_t)code || (code & 0x7F) == 0x7F || code == 0x80 || code == 0xFF);
    uint16_t row[256];
    uint8_t q[256];
    float sc[2];
    for (int i = 0; i < 256; ++i) row[i] = (uint16_t)(i < 128 ? 0x7FC0 : (i == 128 ? 0x7F80 : 0x3F80));
    oracle_quantize_row_fp8(256, row, q, sc);
    free(f); free(h); free(c);
    printf("ok\n");
    return 0;
}
