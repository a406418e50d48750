// Device helpers shared by the score and top-k kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace idx {

// Order-preserving map of a logit onto uint32: larger logit -> larger key.
// -0.0 and +0.0 map to one key (they are equal values); -inf and NaN map to
// 0, the "never selectable" key (masked columns are -inf).
__device__ __forceinline__ uint32_t order_key(float v) {
    if (!(v > -__builtin_inff())) return 0u;        // -inf or NaN
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t key) {
    uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
    return __uint_as_float(u);
}

}  // namespace idx
