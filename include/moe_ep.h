/*
 * moe_ep.h — C ABI of the MoE token path on one MI355X (gfx950):
 * routing layout -> dispatch -> combine.
 *
 * The expert-parallel "ranks" of an EP group are expert groups inside one
 * GPU's HBM: expert e belongs to group g = e / (E / G). Every call is
 * asynchronous on the caller's HIP stream and is ordered only by that stream.
 * The library allocates no device memory: every array is owned by the caller
 * (device memory unless stated), and the receive buffers are sized at the
 * bounds given by moe_recv_rows_bound(), so no device-to-host synchronisation
 * is needed anywhere on the path. What it keeps between calls is fixed in
 * size: on each GPU, the workspace of moe_layout_dispatch_noalloc() and the
 * exchange tables of moe_layout() (arrays in its own code object, zero when
 * it is loaded), and on the host a call counter per stream for those tables.
 * No result depends on what they hold when a call starts.
 *
 * Errors. Every entry point returns 0 (MOE_OK) or a negative moe_error code.
 * All argument checks happen on the host before anything is launched; a call
 * that returns an error has launched nothing. Problems found in the data
 * itself (an expert index out of range, an expert repeated within a token, a
 * combine slot beyond the rows supplied) set bits in the device word
 * layout->status; entries found invalid are skipped, never read or written
 * out of bounds. Read the status after synchronising the stream.
 *
 * T = 0 is valid: moe_layout() then only zeroes the counts, offsets and
 * status (the per-token arrays may be NULL), and the other calls do nothing.
 */
#ifndef MOE_EP_H
#define MOE_EP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_EP_ABI_VERSION 3

/* Limits checked at the boundary. */
#define MOE_MAX_EXPERTS 1024 /* E */
#define MOE_MAX_GROUPS 32    /* G: a token's groups form one 32-bit mask */
#define MOE_MAX_TOPK 32      /* K */
#define MOE_FUSED_MAX_TOKENS 512   /* T of moe_layout_dispatch()'s one-launch form */
#define MOE_FUSED_MAX_PAIRS 16384  /* T * K of moe_layout_dispatch()'s one-launch form */
#define MOE_NOALLOC_SCRATCH_BYTES 8388608 /* layout workspace held by moe_layout_dispatch_noalloc() */

enum moe_error {
    MOE_OK = 0,
    MOE_ERR_NULL_PTR = -1,   /* a required pointer is NULL */
    MOE_ERR_BAD_SHAPE = -2,  /* T, K, E, G or H outside the supported range */
    MOE_ERR_MISALIGNED = -3, /* a row buffer is not 16-byte aligned */
    MOE_ERR_CAPACITY = -4,   /* a receive buffer is smaller than its bound */
    MOE_ERR_WORKSPACE = -5,  /* workspace missing or too small */
    MOE_ERR_HIP = -6,        /* a HIP runtime call or launch failed */
    MOE_ERR_BAD_MODE = -7,   /* unknown mode or dtype */
    MOE_ERR_SCRATCH_LIMIT = -8 /* sizes need more than MOE_NOALLOC_SCRATCH_BYTES of layout workspace */
};

/* Bits of layout->status (device int32). */
#define MOE_STATUS_BAD_INDEX 1 /* some topk_idx entry outside [0, E) */
#define MOE_STATUS_DUPLICATE 2 /* some token lists one expert twice */
#define MOE_STATUS_Y_ROWS 4    /* combine met a slot >= the rows of y */
#define MOE_STATUS_SYNC_FALLBACK 8 /* diagnostic, not an error: a workgroup waited longer
                                      than its limit (0.2 s) for values other workgroups of
                                      its launch write and computed them itself (in
                                      moe_layout_dispatch a token's bases, from the count
                                      table; in moe_layout the first tile's counts, from the
                                      indices); every result is still exact */
/* The bits that mark bad input or output that cannot be trusted. */
#define MOE_STATUS_ERRORS (MOE_STATUS_BAD_INDEX | MOE_STATUS_DUPLICATE | MOE_STATUS_Y_ROWS)

/* Receive-buffer layouts.
 * EXPERT: one row per valid (token, k) pair, rows ordered by expert, then
 *         token, then k; expert e owns rows [expert_offset[e], expert_offset[e+1]).
 * GROUP:  one row per (token, group) the token reaches — a token routed to
 *         several experts of one group is sent to it once — ordered by group,
 *         then token; group g owns rows [group_offset[g], group_offset[g+1]).
 * Source: "perf(ep): optimize IntraNode dispatch kernel for MI350X" (ROCm/mori
 * pull request 586), Motivation (per-destination deduplication, destination =
 * expert / experts-per-rank); "Optimizing Distributed Inference Kernels for AMD
 * DEVELOPER CHALLENGE 2025", section 3.1 (per-local-expert receive buffers). */
enum moe_mode { MOE_MODE_EXPERT = 0, MOE_MODE_GROUP = 1 };

/* Element type of the dispatched rows.
 * BF16: rows are bitwise copies of x.
 * FP8_E4M3_B128: rows are OCP e4m3fn bytes with one fp32 scale per 1x128
 * block: amax = max |x| over the block, scale = amax / 448,
 * q = e4m3fn_rne_satfinite(x * (448 / amax)) (q = 0 when amax = 0).
 * Non-finite values (here and in every call that computes on values): the
 * amax skips NaNs (quiet or signalling); an infinity makes amax infinite, so
 * the block's scale is +inf and its codes are +-0 (finite x) or the NaN code
 * (x infinite or NaN: inf * 0). A NaN encodes as 0x7F in e4m3; infinities
 * saturate to +-448 in e4m3 (satfinite). Rows copied as bf16 keep every bit.
 * A bf16 result computed from a NaN (combine, dequant) is a quiet NaN whose
 * sign and payload are not specified (IEEE 754 leaves open which input's
 * payload a NaN result carries); infinities there follow IEEE fp32
 * arithmetic.
 * Source: "Optimized rocm specific multicast transpose kernel"
 * (ROCm/TransformerEngine pull request 586), Change Summary (fused amax,
 * packed FP8 conversion). */
enum moe_dtype { MOE_DTYPE_BF16 = 0, MOE_DTYPE_FP8_E4M3_B128 = 1 };

/* The routing layout: a plain struct of dimensions and caller-owned device
 * pointers. moe_layout() fills the arrays; moe_dispatch() and moe_combine()
 * read them (the cached destination slots of "Cached routing", mori pull
 * request 586, Technical Details 1). The struct itself is read on the host at
 * each call and may live on the stack.
 *
 * Array                 elements               meaning
 * expert_count          E                      valid pairs routed to expert e
 * expert_offset         E + 1                  exclusive prefix; [E] = rows in EXPERT mode
 * group_count           G                      tokens that reach group g
 * group_offset          G + 1                  exclusive prefix; [G] = rows in GROUP mode
 * tok_group_mask        T   (uint32)           bit g set iff token t reaches group g
 * slot_e                T*K                    EXPERT row of pair (t, k), -1 if invalid
 * slot_g                T*K                    GROUP row of pair (t, k), -1 if invalid
 * slot_tg               T*G                    GROUP row of (t, g), -1 if t misses g
 * recv_src_e            T*K                    pair id t*K + k of EXPERT row r
 * recv_src_g            T*min(K, G)            token id of GROUP row r
 * status                1                      MOE_STATUS_* bits of the last layout/combine
 *
 * recv_src_e / recv_src_g hold valid data in their first expert_offset[E] /
 * group_offset[G] entries; the rest is left untouched. */
typedef struct moe_layout_t {
    int32_t T, K, E, G;
    int32_t *expert_count, *expert_offset;
    int32_t *group_count, *group_offset;
    uint32_t *tok_group_mask;
    int32_t *slot_e, *slot_g, *slot_tg;
    int32_t *recv_src_e, *recv_src_g;
    int32_t *status;
} moe_layout_t;

/* Bytes of device workspace moe_layout() needs for these sizes (written to
 * *bytes). The workspace holds per-tile expert and group counts, per-tile
 * error bits and, for K <= 8, each tile's token-by-expert bit masks (about
 * T * E / 8 bytes); its contents need no initialisation and are dead after
 * the call.
 * Returns MOE_ERR_BAD_SHAPE for sizes outside the limits.
 * Source: the per-destination counts of mori pull request 586 (the per-block
 * count, reserved base and running index its launch-geometry table sizes),
 * here one row per tile of tokens; the caller allocates it once at the size
 * this query gives, as DeepEP pull request 347 ("Feature/sm free normal
 * kernel", Design, RDMA buffer management) has callers size their buffer with
 * a size-hint function, and as the challenge write-up, section 3.1
 * ("Persistent Buffer Reuse"), preallocates for the largest problem. */
int moe_layout_workspace_bytes(int T, int K, int E, int G, size_t *bytes);

/* Rows a receive buffer must hold for moe_dispatch() in `mode`: T*K for
 * EXPERT (exact when all entries are valid), T*min(K, G) for GROUP (an upper
 * bound on the deduplicated pairs). Returns a negative moe_error on bad input.
 * Source: mori pull request 586, Technical Details 1 (receive rows are bounded
 * by a fixed per-destination capacity, MaxNumTokensToSend, so no count needs
 * to come back to the host before the copy); DeepEP pull request 347, Design
 * (a size-hint function for the buffer that receives every token of a batch);
 * the challenge write-up, section 3.1 (buffers sized for the maximum problem). */
int64_t moe_recv_rows_bound(int T, int K, int G, int mode);

/* Routing layout of topk_idx (device int32 [T, K], row-major) into L's arrays.
 * Stable order: inside every expert (group) segment rows are in ascending
 * token order, and ascending k within a token. An entry is valid iff it is in
 * [0, E) and does not repeat an earlier entry of the same token; invalid
 * entries get slot -1, are not counted, and set status bits.
 * Requires 1 <= K <= MOE_MAX_TOPK, K <= E <= MOE_MAX_EXPERTS,
 * 1 <= G <= MOE_MAX_GROUPS, E % G == 0, T >= 0, T * max(K, G) < 2^30.
 * ws: device workspace of at least moe_layout_workspace_bytes() bytes,
 * required in every case (the one-launch forms below do not touch it).
 * stream: a hipStream_t (NULL = the null stream).
 * Forms. For K <= 8 the layout is one launch with a workgroup per tile of 256
 * tokens. For up to 128 tiles (T <= 32768) whose rows of E + G + 2 columns,
 * rounded up to even, fit the table's 67840 entries (so 64 tiles at E = 1024,
 * G = 32; the workgroups must be able to run at once) the workgroups learn one
 * another's per-tile counts through a table in library memory, one per
 * stream on each GPU (8
 * streams per GPU get one; later streams, streams under graph capture and
 * hipStreamPerThread take the forms below): each entry carries the call's
 * number on its stream, so an entry of an earlier call or of a concurrent
 * call is never taken, and a workgroup that has waited 0.2 s for the others
 * counts every token itself (exact; MOE_STATUS_SYNC_FALLBACK is set when the
 * first tile's workgroup does so). Otherwise, for T * K <= 16384, each
 * workgroup counts every token itself; otherwise two launches (per-tile
 * counts into ws, then the placement).
 * Source: mori pull request 586, Motivation and Technical Details 1; the
 * separate routing launch is the one its profiling section proposes. */
int moe_layout(const int32_t *topk_idx, const moe_layout_t *L, void *ws, size_t ws_bytes,
               void *stream);

/* Dispatch: for every source token t and each of its destination rows r
 * (slot_e[t, k] for valid k in EXPERT mode; slot_tg[t, g] >= 0 in GROUP mode):
 *   recv_x[r, :]        = x[t, :]               (BF16: bitwise copy)
 *                         or e4m3 bytes of x[t, :] with recv_scale[r, :] (FP8)
 *   recv_topk_w[r, :]   = topk_w[t, :]          (all K weights)
 *   recv_topk_idx[r, :] = topk_idx[t, :]        (all K indices, as given)
 * Rows beyond the layout's row count are not written.
 * x:          device bf16 [T, H] (raw 16-bit), 16-byte aligned, H % 8 == 0.
 * topk_w:     device fp32 [T, K]; topk_idx: the int32 [T, K] given to moe_layout.
 * recv_x:     device [recv_capacity, H] bf16 (BF16) or uint8 (FP8), 16-byte aligned.
 * recv_scale: device fp32 [recv_capacity, H / 128] (FP8 only; NULL for BF16).
 * recv_topk_w / recv_topk_idx: device [recv_capacity, K].
 * recv_capacity >= moe_recv_rows_bound(T, K, G, mode), else MOE_ERR_CAPACITY.
 * FP8 needs H % 128 == 0. L must hold the layout of topk_idx. As a guard
 * against a layout not written by moe_layout() for these sizes, slots outside
 * [0, moe_recv_rows_bound()) are skipped, so no write leaves the buffers.
 * Source: mori pull request 586, Technical Details 3 (wave-wide row copy) and
 * 4 (vectorised metadata copies); the challenge write-up, section 3.1. */
int moe_dispatch(const moe_layout_t *L, int mode, int dtype, int H, const void *x,
                 const float *topk_w, const int32_t *topk_idx, void *recv_x, float *recv_scale,
                 float *recv_topk_w, int32_t *recv_topk_idx, int64_t recv_capacity,
                 void *stream);

/* moe_layout() and moe_dispatch() as one call. The layout arrays and the
 * receive buffers it writes are, bit for bit, those the two calls write, and
 * so is layout->status apart from the diagnostic bit MOE_STATUS_SYNC_FALLBACK.
 * Arguments as for moe_layout() and moe_dispatch().
 * The smallest batches (T * K * E <= 4096), and any batch within
 * T <= MOE_FUSED_MAX_TOKENS and T * K <= MOE_FUSED_MAX_PAIRS when ws is NULL,
 * take one launch and need no workspace: one workgroup per token recomputes
 * the routing it needs from the whole index array, a cost that grows with
 * T * K and E. Other batches need ws (moe_layout_workspace_bytes()). With
 * K <= 8 (BF16, or FP8 with H <= 8192 and T <= 3072) they run the layout's
 * count kernel and then a dispatch in which each workgroup computes its own
 * token's slots from the per-tile token masks while its row loads are in
 * flight, so the separate placement launch of moe_layout() disappears. The
 * offsets and per-tile bases come from workgroup 0 of that dispatch
 * (T <= 4096 and at most four experts per dispatch thread: E <= 512 for
 * BF16, E <= 256 for FP8), which the other workgroups wait for within a
 * bounded time (past it a workgroup computes its bases itself from the count
 * table and sets MOE_STATUS_SYNC_FALLBACK), or else from one workgroup launched
 * in between. Otherwise (K > 8, or FP8 with H > 8192 or T > 3072) the call
 * runs moe_layout() and moe_dispatch(). The workspace holds no state from one
 * call to the next.
 * Source: mori pull request 586, the IntraNodeLL reply in its review thread
 * (single-pass per-token routing, one block per token, copy fused in; latency
 * dominates at small token counts) and its profiling section (routing
 * overhead is what separates dispatch from combine). */
int moe_layout_dispatch(const int32_t *topk_idx, const moe_layout_t *L, void *ws, size_t ws_bytes,
                        int mode, int dtype, int H, const void *x, const float *topk_w, void *recv_x,
                        float *recv_scale, float *recv_topk_w, int32_t *recv_topk_idx,
                        int64_t recv_capacity, void *stream);

/* moe_layout_dispatch() for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation. Same arguments, results and forms as moe_layout_dispatch()
 * without ws / ws_bytes: the layout workspace is a fixed array of
 * MOE_NOALLOC_SCRATCH_BYTES (8 MiB) inside the library, one per GPU, held until
 * the process ends. Sizes whose workspace (moe_layout_workspace_bytes()) exceeds
 * it return MOE_ERR_SCRATCH_LIMIT before anything is launched (E = 256, G = 8:
 * up to about 200,000 tokens; E = 1024, G = 32: about 50,000). The call
 * allocates nothing: it looks up the array's device address once per GPU (the
 * GPU of `stream`, or the current one for the null stream), on its first call
 * there. The workspace needs no initialisation (each call
 * writes what it reads before reading it), so nothing carries over between
 * calls; but every call on one GPU uses the same array, so calls that overlap
 * on one GPU (other streams, other threads, concurrently replayed graphs)
 * race and must be serialised by the caller. */
int moe_layout_dispatch_noalloc(const int32_t *topk_idx, const moe_layout_t *L, int mode, int dtype, int H,
                                const void *x, const float *topk_w, void *recv_x, float *recv_scale,
                                float *recv_topk_w, int32_t *recv_topk_idx, int64_t recv_capacity,
                                void *stream);

/* Receive-side regroup: the arrays of a per-group (GROUP) dispatch result ->
 * the per-expert (EXPERT) layout, i.e. for every EXPERT row r with pair
 * p = recv_src_e[r]:  out[r, :] = in[slot_g[p], :]  for the row data, the K
 * weights, the K indices and (FP8) the H/128 scales. The result equals, bit for
 * bit, moe_dispatch() in EXPERT mode of the same tokens. Each group row is read
 * once. recv_g: [g_capacity, H] bf16 or e4m3 as `dtype`; recv_scale_*: fp32
 * [*, H/128] (FP8 only, else NULL); recv_topk_*: [*, K]. g_capacity and
 * e_capacity must reach the GROUP and EXPERT bounds of moe_recv_rows_bound().
 * Group rows naming a token outside [0, T), or pairs whose expert row is
 * outside [0, T*K) (possible only for a layout not written by moe_layout()
 * for these sizes), are skipped.
 * Source: "Optimizing Distributed Inference Kernels for AMD DEVELOPER CHALLENGE
 * 2025", section 3.1 (the receive kernel copies tokens into per-local-expert
 * buffers). */
int moe_regroup(const moe_layout_t *L, int dtype, int H, const void *recv_g, const float *recv_scale_g,
                const float *recv_topk_w_g, const int32_t *recv_topk_idx_g, int64_t g_capacity,
                void *recv_e, float *recv_scale_e, float *recv_topk_w_e, int32_t *recv_topk_idx_e,
                int64_t e_capacity, void *stream);

/* Per-expert FP8 cast + transpose of per-expert (EXPERT layout) bf16 rows x,
 * the inputs of an FP8 expert GEMM and of its transposed (weight-gradient)
 * GEMM. For each expert e, rows [o, o + n) with o = expert_offset[e],
 * n = expert_count[e], and its scale s = scale[e]:
 *   c_out[r, i]   = e4m3fn_rne_satfinite(x[r, i] * s)            (fp32 multiply)
 *   T_e[i, j]     = c_out[o + j, i] for j < n, 0 for n <= j < np, np = n rounded up to 16
 *   amax[e]       = max(amax[e], max |x[r, i]| over the expert's rows)
 * T_e is a row-major [H, np] byte matrix at t_out + H * pad_offset[e], where the
 * call writes pad_offset[e] = sum of np over experts before e (pad_offset[E] =
 * total). amax is max-accumulated: it must hold non-negative values (zero it
 * for a fresh maximum). x: bf16 [x_rows, H], x_rows >= T*K; c_out: uint8
 * [x_rows, H]; t_out: at least moe_cast_transpose_t_bytes() bytes; H % 64 == 0.
 * Rows of c_out beyond expert_offset[E] are not written. If the layout's
 * offsets do not satisfy 0 <= expert_offset[e] <= expert_offset[e+1] <= T*K
 * (a layout not written by moe_layout() for these sizes), the call writes
 * nothing.
 * Source: "Optimized rocm specific multicast transpose kernel"
 * (ROCm/TransformerEngine pull request 586), Change Summary: both outputs from
 * one read with amax fused in, packed FP8 conversion, all experts in one launch,
 * row counts padded to 16. */
int64_t moe_cast_transpose_t_bytes(int T, int K, int E, int H);
int moe_cast_transpose_fp8(const moe_layout_t *L, int H, const void *x, int64_t x_rows,
                           const float *scale, void *c_out, void *t_out, int64_t t_bytes, float *amax,
                           int32_t *pad_offset, void *stream);

/* Combine: out[t, i] = bf16_rne( acc ), where acc starts at -0 and, for
 * k = 0 .. K-1 in order with slot(t, k) >= 0,
 *   acc = fmaf(topk_w[t, k], y[slot(t, k), i], acc)        (fp32)
 * slot = slot_e (EXPERT) or slot_g (GROUP; a row shared by several k is
 * weighted once per k). Slots >= y_rows are skipped and set MOE_STATUS_Y_ROWS.
 * y:   device bf16 [y_rows, H], 16-byte aligned (the expert outputs, in the
 *      receive layout of `mode`).
 * out: device bf16 [T, H], 16-byte aligned; must not overlap y.
 * Source: mori pull request 586, "Remaining gap — profiled root cause" (combine
 * gathers the expert rows and accumulates with FMAs); ROCm/vllm pull request
 * 1297, Accuracy (fp32 accumulation, one rounding on the store). */
int moe_combine(const moe_layout_t *L, int mode, int H, const void *y, int64_t y_rows,
                const float *topk_w, void *out, void *stream);

/* Identity expert for FP8 rows (glue between dispatch and combine, not part
 * of the timed path): y[r, i] = bf16_rne(e4m3_decode(q[r, i]) * scale[r, i / 128])
 * for r < the layout's row count in `mode` (read on the device); rows beyond
 * it are not written. q: device uint8 [capacity, H]; scale: fp32
 * [capacity, H / 128]; y: bf16 [capacity, H]. H % 128 == 0.
 * Source: mori pull request 586 measures dispatch and combine with zero-copy
 * combine (Motivation: combine reads the experts' outputs where they are) and
 * regression-tests FP8 dispatch with a bf16 combine (Test Plan); the challenge
 * write-up, section 3.1, stands a simple per-rank function in for the expert
 * computation. Here the stand-in is the identity on the dequantised rows, so
 * the FP8 round trip can be checked against its error bound. */
int moe_fp8_dequant(const moe_layout_t *L, int mode, int H, const void *q, const float *scale,
                    void *y, int64_t capacity, void *stream);

/* Measurement aid, not part of the method: a plain 16-byte-vector streaming
 * copy of `bytes` bytes (bytes % 16 == 0, both pointers 16-byte aligned). It
 * calibrates hardware traffic counters and gives a measured copy ceiling. */
int moe_ref_copy(void *dst, const void *src, int64_t bytes, void *stream);

/* Measurement aid, not part of the method: the read/write mix of a combine or
 * a dispatch over contiguous rows, the ceiling of each call's own mix. For
 * each of `units` units u, rows u*nr .. u*nr + nr - 1 of src (rows of
 * row_bytes bytes) are read and their bitwise XOR is written to rows
 * u*nw .. u*nw + nw - 1 of dst; src holds units*nr rows, dst units*nw rows.
 * (nr, nw) is (1, 1), (2, 4 or 8, 1) — a combine's K reads per written row —
 * or (1, 2, 4 or 8) — a dispatch's K writes per read row; else
 * MOE_ERR_BAD_MODE. row_bytes % 16 == 0; pointers 16-byte aligned. */
int moe_ref_mix(void *dst, const void *src, int64_t row_bytes, int64_t units, int nr, int nw,
                void *stream);

/* Text for a moe_error code (static storage). For MOE_ERR_HIP the text of the
 * last HIP error seen by this library on the calling thread is appended.
 * Not a step of the method: the pages define no error codes. It reports this
 * ABI's host-side argument checks (the stress test and FP8 regression command of
 * mori pull request 586's Test Plan are where such failures would surface). */
const char *moe_status_string(int code);

/* MOE_EP_ABI_VERSION of the built library. */
int moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_EP_H */
