// Device-side helpers shared by the libpkv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Exact widening of the low / high bf16 of a packed pair.
__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// 16-byte load with the non-temporal (streaming) cache policy: for data
// read once per launch, like cached K/V rows.
__device__ __forceinline__ uint4 load_stream16(const void *p)
{
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(w.x, w.y, w.z, w.w);
}

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_round(float f)
{
    uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// c + a.lo*b.lo + a.hi*b.hi on packed bf16 pairs, fp32 accumulate
// (v_dot2_f32_bf16; bf16 products are exact in fp32).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// DPP lane moves inside a 16-lane row.
enum : int {
    DPP_QUAD_XOR1 = 0xB1,   // quad_perm [1,0,3,2]
    DPP_QUAD_XOR2 = 0x4E,   // quad_perm [2,3,0,1]
    DPP_ROW_HALF_MIRROR = 0x141,
    DPP_ROW_MIRROR = 0x140,
};

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of LANES (2..16) consecutive lanes; every lane of
// a group ends with the same (bit-identical) sum.
template <int LANES>
__device__ __forceinline__ float group_sum(float v)
{
    static_assert(LANES == 2 || LANES == 4 || LANES == 8 || LANES == 16, "group size");
    v += dpp_mov<DPP_QUAD_XOR1>(v);
    if constexpr (LANES >= 4) v += dpp_mov<DPP_QUAD_XOR2>(v);
    if constexpr (LANES >= 8) v += dpp_mov<DPP_ROW_HALF_MIRROR>(v);
    if constexpr (LANES >= 16) v += dpp_mov<DPP_ROW_MIRROR>(v);
    return v;
}

// Lane `lane`'s value, as a scalar.
__device__ __forceinline__ float read_lane(float v, int lane)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Max and sum over the whole wave: the four 16-lane rows reduce by DPP, then
// the row results are read as scalars and combined in a fixed order.  Every
// lane of the wave must be active; every lane gets the result.
__device__ __forceinline__ float wave_max(float v)
{
    v = fmaxf(v, dpp_mov<DPP_QUAD_XOR1>(v));
    v = fmaxf(v, dpp_mov<DPP_QUAD_XOR2>(v));
    v = fmaxf(v, dpp_mov<DPP_ROW_HALF_MIRROR>(v));
    v = fmaxf(v, dpp_mov<DPP_ROW_MIRROR>(v));
    return fmaxf(fmaxf(read_lane(v, 0), read_lane(v, 16)), fmaxf(read_lane(v, 32), read_lane(v, 48)));
}

__device__ __forceinline__ float wave_sum(float v)
{
    v = group_sum<16>(v);
    return (read_lane(v, 0) + read_lane(v, 16)) + (read_lane(v, 32) + read_lane(v, 48));
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Records contract violations (PKV_DEVERR_* bits) in the caller's device
// error word, if one is set.  A vector-memory atomic OR; callers keep it off
// their hot paths (it runs only when a bad value was actually seen).
__device__ __forceinline__ void report_error(uint32_t *err, uint32_t bits)
{
    if (err) __hip_atomic_fetch_or(err, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Block id j of a block table, as a scalar load.  The table is read-only in
// every kernel, but where the same kernel also stores to the KV pools the
// compiler cannot tell that the stores leave it alone and would fetch it
// through the vector path (a full memory round trip before each chunk's
// addresses are known); reading it through the constant address space
// states that it is not written.
__device__ __forceinline__ int load_block_id(const int32_t *table, int j)
{
    typedef const int32_t __attribute__((address_space(4))) *const_i32_ptr;
    return ((const_i32_ptr)table)[j];
}

// Order-preserving map of fp32 onto uint32 (larger float -> larger key);
// -0 is folded onto +0 first so equal floats get equal keys.
__device__ __forceinline__ uint32_t float_key(float f)
{
    f = f + 0.0f;
    const uint32_t u = __float_as_uint(f);
    // negative: all bits flipped; otherwise the sign bit set
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

__device__ __forceinline__ float key_float(uint32_t k)
{
    uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}

}  // namespace pkv
