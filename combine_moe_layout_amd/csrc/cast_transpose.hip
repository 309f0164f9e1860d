// Per-expert FP8 cast + transpose of the per-expert receive rows: for each
// expert e with scale s_e, C = e4m3(x * s_e) in the receive layout, T_e =
// C_e^T as a row-major [H, n_e rounded up to 16] matrix (zero padded), and
// amax_e = max |x| folded into the caller's amax. This is the multi-tensor
// cast-transpose of "Optimized rocm specific multicast transpose kernel"
// (ROCm/TransformerEngine pull request 586): both outputs from one read, amax
// fused into the conversion, packed e4m3 conversions, 128-bit loads, all
// experts in one launch, edge tiles predicated per row with rows padded to 16.
//
// Design. Two forms, picked by the rows per expert on average (the host knows
// the row bound and E, not the counts): for at most 32, row tiles of 128 rows
// x 512 columns (cast_transpose_kernel), whose pass shape follows a tile's few
// rows; for more, column blocks (cast_transpose_cols_kernel), where a
// workgroup owns up to 256 rows of one expert and 128 columns, stores C as it
// goes and writes its part of T_e from LDS at the end in consecutive 16-byte
// runs, so no T_e line is split between workgroups. C goes out with
// non-temporal stores and T with plain ones, the pair measured fastest on
// MI355X. A workgroup finds its expert and tile (segment) from a scan of
// per-expert tile counts over all experts (E <= 1024). Bound by HBM: 2 bytes
// read and 2 written per element.
// Measured (µs; 4096 tokens x 7168, 256 experts / 4096 x 4096, 128 experts,
// Zipf routing / 256 tokens x 7168, 256 experts): row tiles 185.0 / 112.2 /
// 28.8, column blocks 180.6 / 100.7 / 86.9. At 4096 x 7168 the row tiles wrote
// 514.4 MB to HBM for 483.9 MB of C and T (x1.063: an expert of more than 128
// rows has its T_e rows split at the tile boundary, inside cache lines that
// two workgroups, in general on two XCDs, write back in parts), the column
// blocks 484.3 MB (x1.001).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kCtBS = 256;
constexpr int kCtWaves = kCtBS / kWave;
constexpr int kMaxE = 1024;                          // the library's expert limit
constexpr int kCtEpt = (kMaxE + kCtBS - 1) / kCtBS;   // experts per thread in the scan


// Exclusive scan of two values over the 256 threads, with both totals, and
// the OR of a flag over the threads (returned).
__device__ __forceinline__ bool ct_scan2(int va, int vb, bool flag, int *s, int &ea, int &eb, int &ta,
                                         int &tb)
{
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const bool wflag = __any(flag);
    const int xa = wave_incl_scan(va), xb = wave_incl_scan(vb);
    if (lane == kWave - 1) {
        s[wave] = xa;
        s[kCtWaves + wave] = xb;
        s[2 * kCtWaves + wave] = wflag ? 1 : 0;
    }
    __syncthreads();
    int ba = 0, bb = 0, any = 0;
    ta = 0;
    tb = 0;
#pragma unroll
    for (int w = 0; w < kCtWaves; ++w) {
        ba += w < wave ? s[w] : 0;
        bb += w < wave ? s[kCtWaves + w] : 0;
        ta += s[w];
        tb += s[kCtWaves + w];
        any |= s[2 * kCtWaves + w];
    }
    ea = ba + xa - va;
    eb = bb + xb - vb;
    return any != 0;
}

// Row-tile form, for experts of a few dozen rows: a workgroup owns a tile of
// up to 128 rows of one expert (tiles never straddle experts) and the 512
// columns of one column group, the 1-D grid running column groups fastest.
// Threads work on items of 4 consecutive rows x 8 columns (four 16-byte
// loads); the tile's padded row count picks the shape of a pass: Q row quads
// (4..32, the power of two that covers the rows) by 256/Q column chunks, so a
// tile of 16 rows covers its 512 columns in one pass and a full tile takes
// eight passes of 64 columns. Each thread converts its item, stores four
// 8-byte runs of C, and packs each column's 4 bytes into one 32-bit word of an
// LDS tile [columns][Q + 1 words] (column c also shifted by c/8 words). After
// a barrier each thread reads 16 rows of a column (4 words) and stores them as
// one 16-byte run of T_e; padding rows come from zero inputs. The loads of
// pass k+1 are issued before pass k is converted, and the LDS tile is
// double-buffered, so one barrier per pass suffices. A T_e row is written by
// one workgroup while its expert fits one tile; for more rows it is split
// between two, which write the line at the split back in parts (the form
// below is used then).
constexpr int kCtRows = 128;        // rows per tile
constexpr int kCtGroupCols = 512;   // columns per workgroup
// LDS words of one tile buffer: max over Q in {4, 8, 16, 32} of
// (2048 / Q) columns x (Q + 1) words, plus the c/8 shift
constexpr int kCtLdsWords = 512 * 5 + 64;

__global__ __launch_bounds__(kCtBS) void cast_transpose_kernel(
    const u32x4 *__restrict__ x, int H, int E, int rows_bound, const int32_t *__restrict__ expert_offset,
    const float *__restrict__ scale, uint8_t *__restrict__ c_out, uint8_t *__restrict__ t_out,
    float *__restrict__ amax, int32_t *__restrict__ pad_offset)
{
    __shared__ int s_red[3 * kCtWaves];
    __shared__ int s_info[5];   // expert, its first tile, its padded-row prefix, row offset, rows
    __shared__ uint32_t s_t[2][kCtLdsWords];
    __shared__ float s_amax[kCtWaves];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    // 1-D grid, column group fastest: the workgroups in flight read whole rows
    // of a compact window of tiles rather than one column slice of every row
    const int ncg = (H + kCtGroupCols - 1) / kCtGroupCols;
    const int tile = blockIdx.x / ncg, cg = blockIdx.x % ncg;

    // Per-expert tile counts and padded row counts; thread owns experts
    // tid*ept .. tid*ept+ept-1 (contiguous, so one scan gives the prefixes).
    const int ept = (E + kCtBS - 1) / kCtBS;
    int lo[kCtEpt], nn[kCtEpt], lt = 0, lp = 0;
    bool bad = false;
#pragma unroll
    for (int j = 0; j < kCtEpt; ++j) {
        const int e = tid * ept + j;
        lo[j] = 0;
        nn[j] = 0;
        if (j < ept && e < E) {
            // a layout's offsets rise from 0 to at most rows_bound, the rows x
            // and C hold; any others (a layout not written for these sizes)
            // stop the whole grid below, before any write
            const int a = expert_offset[e], b = expert_offset[e + 1];
            bad = bad || a < 0 || b < a || b > rows_bound;
            lo[j] = a;
            nn[j] = bad ? 0 : b - a;
        }
        lt += (nn[j] + kCtRows - 1) / kCtRows;
        lp += (nn[j] + 15) / 16 * 16;
    }
    int rt, rp, tot_t, tot_p;
    if (ct_scan2(lt, lp, bad, s_red, rt, rp, tot_t, tot_p)) return;   // uniform
    const bool first = blockIdx.x == 0;
#pragma unroll
    for (int j = 0; j < kCtEpt; ++j) {
        const int e = tid * ept + j;
        const int nt = (nn[j] + kCtRows - 1) / kCtRows;
        if (j < ept && e < E) {
            if (first) pad_offset[e] = rp;
            if (rt <= tile && tile < rt + nt) {   // exactly one thread owns the tile
                s_info[0] = e;
                s_info[1] = rt;
                s_info[2] = rp;
                s_info[3] = lo[j];
                s_info[4] = nn[j];
            }
        }
        rt += nt;
        rp += (nn[j] + 15) / 16 * 16;
    }
    if (first && tid == 0) pad_offset[E] = tot_p;
    if (tile >= tot_t) return;   // uniform: the grid covers the tile bound
    __syncthreads();

    const int e = s_info[0], o = s_info[3], n = s_info[4];
    const int npad = (n + 15) / 16 * 16;
    const int r0 = (tile - s_info[1]) * kCtRows;                   // first row of the tile
    const int nrows = n - r0 < kCtRows ? n - r0 : kCtRows;         // valid rows
    const int prows = npad - r0 < kCtRows ? npad - r0 : kCtRows;   // rows of T to write (x16)
    const float s = scale[e];
    const int hv = H / 8;   // 16-byte chunks per row
    uint8_t *te = t_out + (size_t)H * s_info[2];
    const u32x4 *xt = x + (size_t)(o + r0) * hv;
    uint8_t *ct_rows = c_out + (size_t)(o + r0) * H;

    // pass shape: Q = 2^lq row quads, C = 2^lc column chunks, W = 8C columns
    const int nq = prows / 4;
    const int lq = nq <= 4 ? 2 : nq <= 8 ? 3 : nq <= 16 ? 4 : 5;
    const int lc = 8 - lq, lr = lq - 2;   // run blocks of 16 rows per column: 2^lr
    const int Q = 1 << lq, W = 8 << lc;
    const int q = tid >> lc, cc = tid & ((1 << lc) - 1);
    const int gcol = cg * kCtGroupCols;
    const int ncols = H - gcol < kCtGroupCols ? H - gcol : kCtGroupCols;
    const int passes = (ncols + W - 1) / W;

    auto load = [&](u32x4(&v)[4], int k) {
        const int ch = ((gcol + k * W) >> 3) + cc;   // chunk index within the row
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 4 * q + i;
            v[i] = u32x4{0, 0, 0, 0};
            if (ch < hv && row < nrows) v[i] = __builtin_nontemporal_load(xt + (size_t)row * hv + ch);
        }
    };

    float a = 0.f;
    u32x4 cur[4], nxt[4];
    load(cur, 0);
    for (int k = 0; k < passes; ++k) {
        if (k + 1 < passes) load(nxt, k + 1);
        uint32_t *buf = s_t[k & 1];
        const int c0 = gcol + k * W;
        const int ch = (c0 >> 3) + cc;
        uint32_t b[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float f[8];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                f[2 * m] = bf16_lo(cur[i][m]);
                f[2 * m + 1] = bf16_hi(cur[i][m]);
            }
#pragma unroll
            for (int m = 0; m < 8; ++m) a = amax_step(a, f[m]);
            const int p0 = (int)e4m3x4(f[0], f[1], f[2], f[3], s);
            const int p1 = (int)e4m3x4(f[4], f[5], f[6], f[7], s);
            b[i][0] = (uint32_t)p0;
            b[i][1] = (uint32_t)p1;
            const int row = 4 * q + i;
            if (ch < hv && row < nrows)
                __builtin_nontemporal_store(u32x2{(uint32_t)p0, (uint32_t)p1},
                                            reinterpret_cast<u32x2 *>(ct_rows + (size_t)row * H + 8 * ch));
        }
        // column 8cc + m holds byte m of each row's 8; 4 rows -> one word
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int w = m >> 2, sh = (m & 3) * 8;
            const uint32_t word = ((b[0][w] >> sh) & 0xFFu) | (((b[1][w] >> sh) & 0xFFu) << 8) |
                                  (((b[2][w] >> sh) & 0xFFu) << 16) | (((b[3][w] >> sh) & 0xFFu) << 24);
            buf[(8 * cc + m) * (Q + 1) + cc + q] = word;
        }
        __syncthreads();
        // T: W columns x 2^lr runs of 16 rows = 512 runs, two per thread
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int p = u * kCtBS + tid;
            const int col = p >> lr, rb = p & ((1 << lr) - 1);
            if (c0 + col < H && rb * 16 < prows) {
                const uint32_t *src = buf + col * (Q + 1) + (col >> 3) + rb * 4;
                const u32x4 run = u32x4{src[0], src[1], src[2], src[3]};
                store16<false>(reinterpret_cast<u32x4 *>(te + (size_t)(c0 + col) * npad + r0 + rb * 16), run);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) cur[i] = nxt[i];
    }
    // amax: workgroup max, one atomic per workgroup (max of non-negative
    // floats = max of their bit patterns as unsigned integers)
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
    if (lane == 0) s_amax[wave] = a;
    __syncthreads();
    if (tid == 0) {
        float m = s_amax[0];
#pragma unroll
        for (int w = 1; w < kCtWaves; ++w) m = fmaxf(m, s_amax[w]);
        atomicMax(reinterpret_cast<unsigned int *>(amax + e), __float_as_uint(m));
    }
}

// Column-block form, for experts of more rows. A workgroup owns a segment of up to 256 rows of one expert (all of its rows
// for nearly every expert at uniform routing) and 128 columns. It walks the
// segment 64 rows at a time, storing C as it goes (whole 128-byte segments of
// a row), and builds the segment's part of T_e (128 columns x up to 256 rows)
// in LDS; at the end it writes that part out as consecutive 16-byte runs,
// which for a one-segment expert is one contiguous region of T_e, so every
// cache line of it is written whole by one workgroup at one time (but the two
// at its ends, shared with the neighbouring column blocks). With row tiles of
// 128 rows a T_e row of an expert with more rows is split between workgroups,
// in general on different XCDs, each writing back part of the line at every
// split; writing each 64-row chunk's runs as it was converted (measured)
// left lines half-written between chunks, and so did one workgroup per expert
// and column block without segments, which was also slow where one expert
// holds nearly every token (171 against 112 us at the skewed routing). An item
// is 4 consecutive rows x 8 columns (four 16-byte loads; 16 row quads x 16
// column chunks = one per thread per chunk); the next chunk's loads are in
// flight while the current one is converted. Each column's 4 bytes of the 4
// rows are packed into one 32-bit word; LDS holds the T part column-major, 65
// words per column (64 + 1), column c shifted by c / 8 words, spreading a
// wave's writes over the banks.
constexpr int kCbCols = 128;
constexpr int kCbRows = 64;
constexpr int kCbSeg = 256;                  // rows per segment (a multiple of kCbRows)
constexpr int kCbStride = kCbSeg / 4 + 1;    // words per column in LDS
constexpr int kCbLdsWords = kCbCols * kCbStride + kCbCols / 8;

__global__ __launch_bounds__(kCtBS) void cast_transpose_cols_kernel(
    const u32x4 *__restrict__ x, int H, int E, int rows_bound, const int32_t *__restrict__ expert_offset,
    const float *__restrict__ scale, uint8_t *__restrict__ c_out, uint8_t *__restrict__ t_out,
    float *__restrict__ amax, int32_t *__restrict__ pad_offset)
{
    __shared__ int s_red[3 * kCtWaves];
    __shared__ int s_info[5];   // expert, its first segment, its padded-row prefix, row offset, rows
    __shared__ uint32_t s_t[kCbLdsWords];
    __shared__ float s_amax[kCtWaves];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int ncb = (H + kCbCols - 1) / kCbCols;
    const int seg = blockIdx.x / ncb, cb = blockIdx.x % ncb;   // column block fastest

    // Per-expert segment counts and padded row counts (as the row-tile form
    // finds its tile): thread owns experts tid*ept .. tid*ept+ept-1. Offsets
    // that do not rise from 0 to at most rows_bound (a layout not written for
    // these sizes) stop the whole grid, before any write.
    const int ept = (E + kCtBS - 1) / kCtBS;
    int lo[kCtEpt], nn[kCtEpt], lt = 0, lp = 0;
    bool bad = false;
#pragma unroll
    for (int j = 0; j < kCtEpt; ++j) {
        const int ex = tid * ept + j;
        lo[j] = 0;
        nn[j] = 0;
        if (j < ept && ex < E) {
            const int a = expert_offset[ex], b = expert_offset[ex + 1];
            bad = bad || a < 0 || b < a || b > rows_bound;
            lo[j] = a;
            nn[j] = bad ? 0 : b - a;
        }
        lt += (nn[j] + kCbSeg - 1) / kCbSeg;
        lp += (nn[j] + 15) / 16 * 16;
    }
    int rt, rp, tot_t, tot_p;
    if (ct_scan2(lt, lp, bad, s_red, rt, rp, tot_t, tot_p)) return;   // uniform
    const bool first = blockIdx.x == 0;
#pragma unroll
    for (int j = 0; j < kCtEpt; ++j) {
        const int ex = tid * ept + j;
        const int nt = (nn[j] + kCbSeg - 1) / kCbSeg;
        if (j < ept && ex < E) {
            if (first) pad_offset[ex] = rp;
            if (rt <= seg && seg < rt + nt) {   // exactly one thread owns the segment
                s_info[0] = ex;
                s_info[1] = rt;
                s_info[2] = rp;
                s_info[3] = lo[j];
                s_info[4] = nn[j];
            }
        }
        rt += nt;
        rp += (nn[j] + 15) / 16 * 16;
    }
    if (first && tid == 0) pad_offset[E] = tot_p;
    if (seg >= tot_t) return;   // uniform: the grid covers the segment bound
    __syncthreads();

    const int e = s_info[0], n = s_info[4];
    const int npad = (n + 15) / 16 * 16;
    const int s0 = (seg - s_info[1]) * kCbSeg;                 // first row of the segment
    const int send = npad - s0 < kCbSeg ? npad : s0 + kCbSeg;   // end of its T rows (x16)
    const float s = scale[e];
    const int hv = H / 8;   // 16-byte chunks per row
    const int c0 = cb * kCbCols;
    const int q = tid >> 4, cc = tid & 15;   // row quad, column chunk of 8
    const int ch = (c0 >> 3) + cc;
    const bool colok = ch < hv;              // the last block may be 64 columns wide
    const u32x4 *xe = x + (size_t)s_info[3] * hv;
    uint8_t *ce = c_out + (size_t)s_info[3] * H;
    uint8_t *te = t_out + (size_t)H * s_info[2];
    const int nchunks = (send - s0 + kCbRows - 1) / kCbRows;

    auto load = [&](u32x4(&v)[4], int r0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = r0 + 4 * q + i;
            v[i] = u32x4{0, 0, 0, 0};
            if (colok && row < n) v[i] = __builtin_nontemporal_load(xe + (size_t)row * hv + ch);
        }
    };

    float a = 0.f;
    u32x4 cur[4], nxt[4];
    load(cur, s0);
    for (int k = 0; k < nchunks; ++k) {
        const int r0 = s0 + k * kCbRows;
        if (k + 1 < nchunks) load(nxt, r0 + kCbRows);
        uint32_t b[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float f[8];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                f[2 * m] = bf16_lo(cur[i][m]);
                f[2 * m + 1] = bf16_hi(cur[i][m]);
            }
#pragma unroll
            for (int m = 0; m < 8; ++m) a = amax_step(a, f[m]);
            b[i][0] = e4m3x4(f[0], f[1], f[2], f[3], s);
            b[i][1] = e4m3x4(f[4], f[5], f[6], f[7], s);
            const int row = r0 + 4 * q + i;
            if (colok && row < n)
                __builtin_nontemporal_store(u32x2{b[i][0], b[i][1]},
                                            reinterpret_cast<u32x2 *>(ce + (size_t)row * H + 8 * ch));
        }
        // column 8cc + m holds byte m of each row's 8; 4 rows -> one word, at
        // word (r0 - s0) / 4 + q of the column
        const int wq = (r0 - s0) / 4 + q;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int w = m >> 2, sh = (m & 3) * 8;
            const uint32_t word = ((b[0][w] >> sh) & 0xFFu) | (((b[1][w] >> sh) & 0xFFu) << 8) |
                                  (((b[2][w] >> sh) & 0xFFu) << 16) | (((b[3][w] >> sh) & 0xFFu) << 24);
            s_t[(8 * cc + m) * kCbStride + cc + wq] = word;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) cur[i] = nxt[i];
    }
    __syncthreads();
    // The T part: run j (16 bytes) is bytes s0 + 16 * (j % m) .. of T row
    // c0 + j / m, m = runs per row in the segment; for a one-segment expert the
    // runs are consecutive in memory. (j / m by a multiply-high for m >= 2,
    // exact for j < 2^16; floor(2^32 / m) + 1 does not fit 32 bits for m = 1.)
    {
        const int m = (send - s0) / 16;
        const int ncols = H - c0 < kCbCols ? H - c0 : kCbCols;
        const uint32_t mmag = m > 1 ? (uint32_t)((1ull << 32) / (unsigned)m) + 1u : 0u;
        for (int j = tid; j < ncols * m; j += kCtBS) {
            const int col = m > 1 ? (int)__umulhi((uint32_t)j, mmag) : j, rr = j - col * m;
            const uint32_t *src = s_t + col * kCbStride + (col >> 3) + rr * 4;
            const u32x4 run = u32x4{src[0], src[1], src[2], src[3]};
            store16<false>(reinterpret_cast<u32x4 *>(te + (size_t)(c0 + col) * npad + s0 + rr * 16), run);
        }
    }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
    if (lane == 0) s_amax[wave] = a;
    __syncthreads();
    if (tid == 0) {
        float m = s_amax[0];
#pragma unroll
        for (int w = 1; w < kCtWaves; ++w) m = fmaxf(m, s_amax[w]);
        atomicMax(reinterpret_cast<unsigned int *>(amax + e), __float_as_uint(m));
    }
}

}  // namespace

int64_t cast_transpose_t_bound(int64_t rows, int E, int H)
{
    return (int64_t)H * (rows + 15 * (int64_t)E);
}

hipError_t launch_cast_transpose(const void *x, int64_t rows_bound, int H, int E,
                                 const int32_t *expert_offset, const float *scale, void *c_out,
                                 void *t_out, float *amax, int32_t *pad_offset, hipStream_t stream)
{
    if (rows_bound <= (int64_t)32 * E) {   // a few dozen rows per expert: row tiles
        const int64_t tiles = (rows_bound + kCtRows - 1) / kCtRows + E;   // >= sum of ceil(n_e / 128)
        const int64_t blocks = tiles * ((H + kCtGroupCols - 1) / kCtGroupCols);
        if (blocks > INT32_MAX) return hipErrorInvalidValue;   // the 1-D grid's limit
        hipLaunchKernelGGL(cast_transpose_kernel, dim3((unsigned)blocks), dim3(kCtBS), 0, stream,
                           (const u32x4 *)x, H, E, (int)rows_bound, expert_offset, scale, (uint8_t *)c_out,
                           (uint8_t *)t_out, amax, pad_offset);
        return hipGetLastError();
    }
    const int64_t segs = (rows_bound + kCbSeg - 1) / kCbSeg + E;   // >= sum of ceil(n_e / 256)
    const int64_t blocks = segs * ((H + kCbCols - 1) / kCbCols);
    if (blocks > INT32_MAX) return hipErrorInvalidValue;   // the 1-D grid's limit
    hipLaunchKernelGGL(cast_transpose_cols_kernel, dim3((unsigned)blocks), dim3(kCtBS), 0, stream,
                       (const u32x4 *)x, H, E, (int)rows_bound, expert_offset, scale, (uint8_t *)c_out,
                       (uint8_t *)t_out, amax, pad_offset);
    return hipGetLastError();
}

}  // namespace moe
