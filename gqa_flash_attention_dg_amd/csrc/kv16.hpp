// kv16.hpp -- f32 -> 16-bit rounding shared by the pack pass (dg_pack_kv16) and the norm launch
// that writes 16-bit twins of its outputs (dg_qkv_headnorm_rope_kv16), so both round alike.
// IEEE binary16 or bfloat16, round to nearest with ties to even.
#pragma once

#include "dg_common.hpp"

namespace dg {

__device__ inline uint32_t to_f16(float f) {
    const _Float16 h = static_cast<_Float16>(f);   // v_cvt_f16_f32: IEEE round to nearest even
    return __builtin_bit_cast(uint16_t, h);
}

__device__ inline uint32_t to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x7fffffu)) return (u >> 16) | 0x40u;  // NaN
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;                                    // RNE
}

// fmt: DG_KV_F16 or DG_KV_BF16 (wave-uniform).
__device__ inline uint16_t to_kv16(float f, int fmt) {
    return (uint16_t)(fmt == DG_KV_F16 ? to_f16(f) : to_bf16(f));
}

}  // namespace dg
