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

// Round a finite float to bf16, nearest even, by adding 0x7FFF plus the kept
// lsb and truncating.
__device__ __forceinline__ uint32_t bf16_rne_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return bf16_rne_bits(lo) | (bf16_rne_bits(hi) << 16);
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane)
{
    return (lane == 0) ? 0ull : (~0ull >> (64 - lane));
}

}  // namespace moe
