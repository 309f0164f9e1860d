/*
 * CPU oracle for the MoE token path: routing layout, dispatch (bf16 and FP8 e4m3
 * with one fp32 scale per 1x128 block), identity-expert dequantisation and the
 * weighted top-k combine.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, plain, obviously correct
 * statement of what the path computes. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the product path never does. It
 * shares no code, header, table or helper with the HIP library.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared (no fast-math), so every float
 * operation below is one IEEE binary32 operation in the order written. The
 * canonical build has no OpenMP: the `omp` pragmas below are ignored and it runs
 * on one thread. A second build of this same file with -fopenmp (used only to
 * time the oracle on every host core) runs the loops marked `omp parallel for`
 * on several threads: each marks a loop over tokens or receive rows whose
 * iterations write disjoint outputs from inputs no iteration writes, with the
 * same arithmetic per element, so both builds give the same bits (a test
 * checks it). The cursor walks that assign slots stay serial in both.
 *
 * Sources (pages of the method):
 *  - "perf(ep): optimize IntraNode dispatch kernel for MI350X" (ROCm/mori pull
 *    request 586): Motivation (per-destination deduplication, destination =
 *    expert / experts-per-rank), Technical Details 1 "Cached routing" (the
 *    per-pair cached destination that dispatch and combine reuse), Technical
 *    Details 4 "Vectorized metadata copies" (the K weights and K indices that
 *    travel with each row).
 *  - "Optimizing Distributed Inference Kernels for AMD DEVELOPER CHALLENGE
 *    2025", section 3.1 (per-local-expert contiguous receive buffers; combine
 *    gathers expert outputs back to their source tokens).
 *  - ROCm/vllm pull request 1297, "Accuracy" (accumulate in fp32, round once on
 *    the store).
 *  - "Optimized rocm specific multicast transpose kernel" (ROCm/TransformerEngine
 *    pull request 586), "Change Summary" (fused amax, packed FP8 conversion).
 *
 * Readings where the pages leave a step open (each is also listed in the
 * design notes):
 *  - receive order inside a buffer is stable: expert (or group) ascending, then
 *    token ascending, then k ascending;
 *  - experts map to groups in contiguous blocks, g = e / (E/G);
 *  - an entry idx[t,k] is valid iff 0 <= idx < E and it does not repeat an
 *    earlier idx[t,k'] (k' < k); invalid entries get slot -1, are not counted,
 *    and set status bit 1 (out of range) or bit 2 (repeat);
 *  - FP8: scale = amax/448, inv = 448/amax (0 when amax = 0), q = e4m3fn(x*inv)
 *    with round-to-nearest-even and saturation to +-448;
 *  - combine: acc = -0; for k ascending: acc = fma(w[t,k], y[slot(t,k)], acc);
 *    out = bf16 round-to-nearest-even(acc); entries with slot -1 are skipped.
 *    The chain starts from -0, the additive identity of IEEE arithmetic
 *    (-0 + v = v for every v, +0 included), so a single term comes back as its
 *    rounded product exactly and identity experts return x bit for bit, signed
 *    zeros included.
 */
#include <math.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- codecs */

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bf16 is the top half of a binary32. */
float oracle_bf16_to_f32(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/* Round a finite binary32 to bf16, nearest even: add half an ulp of the kept
 * part (0x7FFF plus the kept lsb, which breaks ties toward even) and truncate. */
uint16_t oracle_f32_to_bf16(float f)
{
    /* a NaN stays a NaN: the canonical quiet NaN (the carry of the rounding
       below would turn some NaNs into an infinity or wrap others to zero) */
    if (isnan(f)) return 0x7FC0;
    uint32_t u = bits_from_f32(f);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/* OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities;
 * S.1111.111 is NaN, so the largest finite magnitude is 1.75 * 2^8 = 448.
 * Normal codes: (-1)^s * 2^(e-7) * (1 + m/8); subnormals (e = 0): 2^-6 * m/8. */
float oracle_e4m3_to_f32(uint8_t c)
{
    int s = (c >> 7) & 1, e = (c >> 3) & 0xF, m = c & 7;
    double v;
    if (e == 0xF && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp(1.0 + m / 8.0, e - 7);
    return (float)(s ? -v : v);
}

/* binary32 -> E4M3FN, round to nearest even, saturating finite values to 448.
 * Every step is exact except the one rounding done by nearbyint (current mode:
 * nearest, ties to even). */
uint8_t oracle_f32_to_e4m3(float f)
{
    uint8_t sign = (bits_from_f32(f) >> 31) ? 0x80 : 0x00;
    double a = fabs((double)f);
    if (isnan(f)) return 0x7F;
    if (isinf(f)) return (uint8_t)(sign | 0x7E);   /* satfinite */
    if (a == 0.0) return sign;
    if (a < ldexp(1.0, -6)) {                /* subnormal range: step 2^-9 */
        double m = nearbyint(a * 512.0);     /* may round up to 8 = min normal */
        return (uint8_t)(sign | (uint8_t)m);
    }
    int e2;
    double fr = frexp(a, &e2);               /* a = fr * 2^e2, fr in [0.5, 1) */
    int ex = e2 - 1;                         /* a = (2 fr) * 2^ex, 2 fr in [1, 2) */
    double m = nearbyint((2.0 * fr - 1.0) * 8.0);
    if (m == 8.0) { m = 0.0; ex += 1; }
    int be = ex + 7;
    if (be > 15 || (be == 15 && m > 6.0)) return (uint8_t)(sign | 0x7E);  /* satfinite */
    return (uint8_t)(sign | (uint8_t)(be << 3) | (uint8_t)m);
}

/* ---------------------------------------------------------------- layout */

/* Status bits written by the layout. */
#define ORC_BAD_INDEX 1
#define ORC_DUPLICATE 2

/* Routing layout. Arrays follow the library's layout contract:
 *  expert_count[E], expert_offset[E+1], group_count[G], group_offset[G+1],
 *  tok_group_mask[T], slot_e[T*K], slot_g[T*K], slot_tg[T*G],
 *  recv_src_e[T*K] (flat pair id t*K+k, first expert_offset[E] entries written),
 *  recv_src_g[T*min(K,G)] (token id, first group_offset[G] entries written).
 * Returns the status bits. */
int oracle_layout(int T, int K, int E, int G, const int32_t *idx,
                  int32_t *expert_count, int32_t *expert_offset,
                  int32_t *group_count, int32_t *group_offset,
                  uint32_t *tok_group_mask, int32_t *slot_e, int32_t *slot_g,
                  int32_t *slot_tg, int32_t *recv_src_e, int32_t *recv_src_g)
{
    int status = 0;
    int epg = E / G;
    unsigned char *valid = (unsigned char *)calloc((size_t)T * K + 1, 1);
    int32_t *cur = (int32_t *)calloc((size_t)E + 1, sizeof(int32_t));
    int32_t *gcur = (int32_t *)calloc((size_t)G + 1, sizeof(int32_t));

    /* validity: in range, and not a repeat of an earlier k of the same token */
#pragma omp parallel for reduction(| : status)
    for (int t = 0; t < T; ++t)
        for (int k = 0; k < K; ++k) {
            int e = idx[(size_t)t * K + k];
            int ok = 1;
            if (e < 0 || e >= E) { ok = 0; status |= ORC_BAD_INDEX; }
            else
                for (int k2 = 0; k2 < k; ++k2)
                    if (idx[(size_t)t * K + k2] == e) { ok = 0; status |= ORC_DUPLICATE; break; }
            valid[(size_t)t * K + k] = (unsigned char)ok;
        }

    /* expert histogram and exclusive prefix */
    for (int e = 0; e < E; ++e) expert_count[e] = 0;
    for (int t = 0; t < T; ++t)
        for (int k = 0; k < K; ++k)
            if (valid[(size_t)t * K + k]) expert_count[idx[(size_t)t * K + k]] += 1;
    expert_offset[0] = 0;
    for (int e = 0; e < E; ++e) expert_offset[e + 1] = expert_offset[e] + expert_count[e];

    /* stable slots: pairs visited in flat (t, k) order, one cursor per expert */
    for (int e = 0; e < E; ++e) cur[e] = expert_offset[e];
    for (int t = 0; t < T; ++t)
        for (int k = 0; k < K; ++k) {
            size_t p = (size_t)t * K + k;
            if (!valid[p]) { slot_e[p] = -1; continue; }
            int e = idx[p];
            int s = cur[e]++;
            slot_e[p] = s;
            recv_src_e[s] = (int32_t)p;
        }

    /* groups: which groups each token reaches (each group once per token) */
#pragma omp parallel for
    for (int t = 0; t < T; ++t) {
        uint32_t m = 0;
        for (int k = 0; k < K; ++k)
            if (valid[(size_t)t * K + k]) m |= 1u << (idx[(size_t)t * K + k] / epg);
        tok_group_mask[t] = m;
    }
    for (int g = 0; g < G; ++g) group_count[g] = 0;
    for (int t = 0; t < T; ++t)
        for (int g = 0; g < G; ++g)
            if ((tok_group_mask[t] >> g) & 1u) group_count[g] += 1;
    group_offset[0] = 0;
    for (int g = 0; g < G; ++g) group_offset[g + 1] = group_offset[g] + group_count[g];
    for (int g = 0; g < G; ++g) gcur[g] = group_offset[g];
    for (int t = 0; t < T; ++t)
        for (int g = 0; g < G; ++g) {
            size_t q = (size_t)t * G + g;
            if ((tok_group_mask[t] >> g) & 1u) {
                int s = gcur[g]++;
                slot_tg[q] = s;
                recv_src_g[s] = t;
            } else {
                slot_tg[q] = -1;
            }
        }
#pragma omp parallel for
    for (int t = 0; t < T; ++t)
        for (int k = 0; k < K; ++k) {
            size_t p = (size_t)t * K + k;
            slot_g[p] = valid[p] ? slot_tg[(size_t)t * G + idx[p] / epg] : -1;
        }

    free(valid); free(cur); free(gcur);
    return status;
}

/* ---------------------------------------------------------------- dispatch */

/* Source token of receive row r. EXPERT rows come from recv_src_e (a pair id,
 * token = pair / K); GROUP rows from recv_src_g (a token id). */
static int src_token(int mode, int K, const int32_t *recv_src, int64_t r)
{
    return mode == 0 ? recv_src[r] / K : recv_src[r];
}

/* bf16 dispatch: receive row r is a bitwise copy of its source token's hidden
 * row, with that token's K weights and K indices beside it. Rows r >= R (R =
 * number of receive rows) are not touched. */
void oracle_dispatch_bf16(int mode, int K, int H, int64_t R, const int32_t *recv_src,
                          const uint16_t *x, const float *topk_w, const int32_t *topk_idx,
                          uint16_t *recv_x, float *recv_w, int32_t *recv_idx)
{
#pragma omp parallel for
    for (int64_t r = 0; r < R; ++r) {
        int t = src_token(mode, K, recv_src, r);
        for (int i = 0; i < H; ++i) recv_x[r * H + i] = x[(int64_t)t * H + i];
        for (int k = 0; k < K; ++k) {
            recv_w[r * K + k] = topk_w[(int64_t)t * K + k];
            recv_idx[r * K + k] = topk_idx[(int64_t)t * K + k];
        }
    }
}

/* Quantise one source row: for each 128-element block b,
 *   amax = max |x|, scale = amax / 448, inv = 448 / amax (0 if amax == 0),
 *   q[i] = e4m3fn_rne_satfinite(x[i] * inv).  */
void oracle_quantize_row_fp8(int H, const uint16_t *xrow, uint8_t *q, float *scale)
{
    for (int b = 0; b < H / 128; ++b) {
        float amax = 0.0f;
        for (int i = 0; i < 128; ++i) {
            float v = fabsf(oracle_bf16_to_f32(xrow[b * 128 + i]));
            if (v > amax) amax = v;
        }
        float s = amax / 448.0f;
        float inv = amax > 0.0f ? 448.0f / amax : 0.0f;
        scale[b] = s;
        for (int i = 0; i < 128; ++i) {
            float v = oracle_bf16_to_f32(xrow[b * 128 + i]) * inv;
            q[b * 128 + i] = oracle_f32_to_e4m3(v);
        }
    }
}

/* FP8 dispatch: every token is quantised once; receive row r holds the bytes
 * and scales of its source token, with its K weights and indices. */
void oracle_dispatch_fp8(int mode, int T, int K, int H, int64_t R, const int32_t *recv_src,
                         const uint16_t *x, const float *topk_w, const int32_t *topk_idx,
                         uint8_t *recv_q, float *recv_scale, float *recv_w, int32_t *recv_idx)
{
    int nb = H / 128;
    uint8_t *qt = (uint8_t *)malloc((size_t)T * H + 1);
    float *st = (float *)malloc(((size_t)T * nb + 1) * sizeof(float));
#pragma omp parallel for
    for (int t = 0; t < T; ++t)
        oracle_quantize_row_fp8(H, x + (int64_t)t * H, qt + (int64_t)t * H, st + (int64_t)t * nb);
#pragma omp parallel for
    for (int64_t r = 0; r < R; ++r) {
        int t = src_token(mode, K, recv_src, r);
        memcpy(recv_q + r * H, qt + (int64_t)t * H, (size_t)H);
        for (int b = 0; b < nb; ++b) recv_scale[r * nb + b] = st[(int64_t)t * nb + b];
        for (int k = 0; k < K; ++k) {
            recv_w[r * K + k] = topk_w[(int64_t)t * K + k];
            recv_idx[r * K + k] = topk_idx[(int64_t)t * K + k];
        }
    }
    free(qt); free(st);
}

/* Identity expert on FP8 rows: y = bf16_rne(decode(q) * scale of its block). */
void oracle_dequant_fp8(int64_t R, int H, const uint8_t *q, const float *scale, uint16_t *y)
{
    int nb = H / 128;
#pragma omp parallel for
    for (int64_t r = 0; r < R; ++r)
        for (int i = 0; i < H; ++i) {
            float v = oracle_e4m3_to_f32(q[r * H + i]) * scale[r * nb + i / 128];
            y[r * H + i] = oracle_f32_to_bf16(v);
        }
}

/* ---------------------------------------------------------------- combine */

/* out[t,i] = bf16_rne( fma chain over k = 0..K-1 of w[t,k] * y[slot[t,k], i] ),
 * accumulated in fp32 from -0, one rounding at the end. slot is slot_e (one row
 * per pair) or slot_g (one row per token and group; a row shared by several k
 * is weighted once per k). Entries with slot < 0 are skipped. */
void oracle_combine(int T, int K, int H, const int32_t *slot, const uint16_t *y,
                    const float *topk_w, uint16_t *out)
{
#pragma omp parallel for
    for (int t = 0; t < T; ++t)
        for (int i = 0; i < H; ++i) {
            float acc = -0.0f;
            for (int k = 0; k < K; ++k) {
                int s = slot[(int64_t)t * K + k];
                if (s < 0) continue;
                acc = fmaf(topk_w[(int64_t)t * K + k], oracle_bf16_to_f32(y[(int64_t)s * H + i]), acc);
            }
            out[(int64_t)t * H + i] = oracle_f32_to_bf16(acc);
        }
}

/* ---------------------------------------------------------------- array codecs
 * Element-wise forms of the codecs above, for exhaustive tests. */
void oracle_f32_to_bf16_n(int64_t n, const float *in, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_bf16(in[i]);
}

void oracle_f32_to_e4m3_n(int64_t n, const float *in, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_e4m3(in[i]);
}

/* ---------------------------------------------------------------- regroup */

/* Receive-side regroup: rows in the per-group layout -> rows in the per-expert
 * layout. EXPERT row r holds pair p = recv_src_e[r]; its content is the GROUP
 * row of that pair, slot_g[p]. Rows are opaque byte strings of row_bytes bytes
 * (a bf16 hidden row, an e4m3 row, a row of scales or of metadata), so one
 * function serves every per-row array. Rows r >= R are not touched. */
void oracle_regroup_rows(int64_t R, int64_t row_bytes, const int32_t *recv_src_e,
                         const int32_t *slot_g, const void *in_rows, void *out_rows)
{
    const unsigned char *in = (const unsigned char *)in_rows;
    unsigned char *out = (unsigned char *)out_rows;
#pragma omp parallel for
    for (int64_t r = 0; r < R; ++r) {
        int32_t p = recv_src_e[r];
        int32_t s = slot_g[p];
        memcpy(out + r * row_bytes, in + (int64_t)s * row_bytes, (size_t)row_bytes);
    }
}

/* ---------------------------------------------------------------- per-expert FP8 cast + transpose */

/* For each expert e with rows [o, o + n) of the per-expert layout (o =
 * expert_offset[e], n = expert_offset[e+1] - o) and its scale s = scale[e]:
 *   C[r, i]           = e4m3fn_rne_satfinite(x[r, i] * s)        (fp32 multiply)
 *   T_e[i, j]         = C[o + j, i] for j < n, 0 for n <= j < np, np = n rounded up to 16
 *   amax[e]           = max(amax[e], max |x[r, i]| over the expert's rows)
 * T_e is a row-major [H, np] byte matrix stored at t_out + H * po[e], with
 * po[e] = sum over e' < e of np(e'); pad_offset[e] = po[e], pad_offset[E] = total. */
void oracle_cast_transpose_fp8(int E, int H, const int32_t *expert_offset, const uint16_t *x,
                               const float *scale, uint8_t *c_out, uint8_t *t_out, float *amax,
                               int32_t *pad_offset)
{
    int64_t po = 0;
    for (int e = 0; e < E; ++e) {
        int64_t o = expert_offset[e], n = expert_offset[e + 1] - o;
        int64_t np = (n + 15) / 16 * 16;
        pad_offset[e] = (int32_t)po;
        float a = amax[e];
        for (int64_t r = o; r < o + n; ++r)
            for (int i = 0; i < H; ++i) {
                float v = oracle_bf16_to_f32(x[r * H + i]);
                if (fabsf(v) > a) a = fabsf(v);
                uint8_t q = oracle_f32_to_e4m3(v * scale[e]);
                c_out[r * H + i] = q;
                t_out[(int64_t)H * po + (int64_t)i * np + (r - o)] = q;
            }
        for (int i = 0; i < H; ++i)
            for (int64_t j = n; j < np; ++j) t_out[(int64_t)H * po + (int64_t)i * np + j] = 0;
        amax[e] = a;
        po += np;
    }
    pad_offset[E] = (int32_t)po;
}

/* ---------------------------------------------------------------- threads
 * Threads the parallel loops may use: 1 in the canonical build. */
int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
