// Device helpers shared by the gfx950 kernels of the MoE token path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// 16-byte vector: the unit of every row load and store (one global_load_dwordx4 /
// global_store_dwordx4 per lane).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Cache-policy operand of the buffer load / store builtins for the
// agent-scope coherent form (sc1: what an agent-scope atomic load or store
// compiles to), for data exchanged between workgroups of one launch.
constexpr int kCpolSc1 = 16;

// Non-temporal 16-byte store: the destination rows are written once and not
// re-read by this kernel, so they should not displace useful lines in the
// write-allocate L2.
template <bool NT>
__device__ __forceinline__ void store16(u32x4 *p, u32x4 v)
{
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4 *p)
{
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// One step of an amax: max(m, |v|), passing over a NaN v. fmaxf alone does
// not: for a signalling NaN (a bf16 such as 0x7F81 widened by a shift stays
// signalling) the hardware max returns a quiet NaN and m is lost. The
// canonicalisation quietens it first, and a max with a quiet NaN returns the
// other operand.
__device__ __forceinline__ float amax_step(float m, float v)
{
    return fmaxf(m, __builtin_canonicalizef(fabsf(v)));
}

// Saturation of a scaled value to the finite e4m3 range before the packed
// conversion (satfinite: infinities too); a NaN stays a NaN.
__device__ __forceinline__ float sat448(float v)
{
    return v != v ? __builtin_nanf("") : fminf(fmaxf(v, -448.f), 448.f);
}

// The packed conversion writes a NaN as the byte 0xFF; the library's e4m3 NaN
// code is 0x7F (S.1111.111 with the sign clear, as a cast of a positive NaN
// gives). Clears bit 7 of every byte of w that is 0xFF and leaves the rest:
// in t = ~w those bytes are zero, and z below has 0x80 in exactly the zero
// bytes of t (no carry crosses a byte: each addend is at most 0x7F + 0x7F).
__device__ __forceinline__ uint32_t e4m3_nan_canon(uint32_t w)
{
    const uint32_t t = ~w;
    const uint32_t z = ~(((t & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | t | 0x7F7F7F7Fu);
    return w ^ z;
}

// Two floats -> two bf16 (lo in the low half), round to nearest even, with
// gfx950's packed conversion: one instruction per pair. On every input that
// is not a NaN it equals the integer rounding (bits + 0x7FFF + kept lsb,
// truncated): infinities, overflow to infinity and subnormals included. A NaN
// gives a quiet NaN with its sign and leading payload bits.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane)
{
    return (lane == 0) ? 0ull : (~0ull >> (64 - lane));
}

// Inclusive prefix sum over the 64 lanes of a wave, in registers by DPP moves:
// shifts by 1, 2, 4 and 8 lanes inside each row of 16 (a Hillis-Steele scan of
// the row; lanes shifted in from outside the row read 0), then the last lane of
// row 0 added into rows 1 and 3 (row_bcast:15) and the last lane of row 1, by
// then the total of rows 0-1, into rows 2 and 3 (row_bcast:31). Each step is a
// VALU operation, not an LDS round trip as a lane shuffle is. Every lane of the
// wave must be active.
__device__ __forceinline__ int wave_incl_scan(int x)
{
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);    // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);    // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);    // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);    // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15, rows 1 and 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31, rows 2 and 3
    return x;
}

// Group of expert x, floor(x / epg), without a division: a multiply-high by
// magic = floor(2^32 / epg) + 1 (for x < 2^16 the product's error is below
// 2^-16 and cannot cross an integer), or x itself when epg = 1 (magic = 0;
// the host computes magic with group_magic()).
__device__ __forceinline__ int group_of(int x, uint32_t magic)
{
    return magic == 0 ? x : (int)__umulhi((uint32_t)x, magic);
}

// Four values times s -> four e4m3fn codes in one word (value 0 in the low
// byte): saturated to +-448 (sat448), converted in pairs by gfx950's packed
// conversion (round to nearest even), the NaN byte mapped to 0x7F.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d, float s)
{
    int p = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a * s), sat448(b * s), 0, false);
    p = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(c * s), sat448(d * s), p, true);
    return e4m3_nan_canon((uint32_t)p);
}

// One lane's 16-element chunk of a bf16 row (a, b: 16 bf16, in order) quantised
// with one fp32 scale per 1x128 block, the block being 8 consecutive lanes of
// the wave (every lane of the wave must call this together): the block's amax
// (NaNs passed over, see amax_step) by three xor-shuffles, scale = amax / 448
// and inv = 448 / amax (0 when amax = 0; correctly rounded divisions, the
// library is built with -fhip-fp32-correctly-rounded-divide-sqrt), and the 16
// codes of x * inv.
__device__ __forceinline__ void quantize16(u32x4 a, u32x4 b, u32x4 &q, float &scale)
{
    float f[16];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        f[2 * m] = bf16_lo(a[m]);
        f[2 * m + 1] = bf16_hi(a[m]);
        f[8 + 2 * m] = bf16_lo(b[m]);
        f[8 + 2 * m + 1] = bf16_hi(b[m]);
    }
    float amax = 0.f;
#pragma unroll
    for (int m = 0; m < 16; ++m) amax = amax_step(amax, f[m]);
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    amax = fmaxf(amax, __shfl_xor(amax, 4));
    scale = amax / 448.f;
    const float inv = amax > 0.f ? 448.f / amax : 0.f;
    q = u32x4{e4m3x4(f[0], f[1], f[2], f[3], inv), e4m3x4(f[4], f[5], f[6], f[7], inv),
              e4m3x4(f[8], f[9], f[10], f[11], inv), e4m3x4(f[12], f[13], f[14], f[15], inv)};
}

}  // namespace moe
