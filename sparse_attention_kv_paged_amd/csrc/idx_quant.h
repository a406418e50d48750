// e4m3 quantisation of bf16 values by the index-plane writer's rule (the
// scale s = amax / 448 per key, each byte the nearest e4m3 value of v / s,
// ties to the even code), shared by the writer kernel and by the score
// kernel when it quantises the query itself.  Sixteen lanes of one DPP row
// hold one 128-value key (or query head), eight values each.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace idx {
namespace {

// Quotients q[i] = v[i] / s, rounded to binary32 as an IEEE division would
// round them, as far as the e4m3 code can tell: r = 1/s is divided once per
// key, then each quotient is q0 = v*r corrected once with the exact residual
// v - q0*s (Markstein's correction step, two FMAs).  Checked against the IEEE
// quotient over every bf16 pair |v| <= amax: the e4m3 codes agree for every
// amax >= 2^-104 once the sign is taken from v (the correction turns -0 into
// +0); below that the residual underflows, so keys with amax < 2^-100 divide
// each element instead.
__device__ __forceinline__ void quotients(const float *v, float scale, float r, bool tiny, float *q) {
#pragma clang fp contract(off)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float q0 = v[i] * r;
        const float rho = __builtin_fmaf(-q0, scale, v[i]);
        q[i] = __builtin_fmaf(rho, r, q0);
    }
    if (tiny) {
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = v[i] / scale;
    }
}

// Codes of four elements, byte i for element i: the magnitude from the
// hardware's packed binary32 -> e4m3fn conversion of |q| (nearest, ties to
// even; |q| never exceeds 448 by more than a few ulps, which still rounds to
// 448), the sign bit from the bf16 value itself.  raw_lo / raw_hi hold the
// four bf16 values (sign bits at 15 and 31 of each).
__device__ __forceinline__ uint32_t codes4(const float *q, uint32_t raw_lo, uint32_t raw_hi) {
    uint32_t c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_fabsf(q[0]), __builtin_fabsf(q[1]), 0, false);
    c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_fabsf(q[2]), __builtin_fabsf(q[3]), (int)c, true);
    const uint32_t sign = ((raw_lo >> 8) & 0x80u) | ((raw_lo >> 16) & 0x8000u) |
                          ((raw_hi << 8) & 0x800000u) | (raw_hi & 0x80000000u);
    return (c & 0x7F7F7F7Fu) | sign;
}

// The value of the lane N places further along this lane's 16-lane DPP row,
// wrapping within the row (row_ror:N).
template <int N>
__device__ __forceinline__ float row_ror(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + N, 0xF, 0xF, false));
}

// Quantise the eight bf16 values of a lane (raw: four dwords, two values
// each) whose key has absolute maximum amax: the eight codes as two dwords
// (byte i = value i) and the key's scale amax / 448.  A key of zeros gives
// zero codes and scale 0.
__device__ __forceinline__ void quantize8(const uint32_t (&raw)[4], float amax, uint32_t &lo, uint32_t &hi,
                                          float &scale) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(raw[i] << 16);
        v[2 * i + 1] = __uint_as_float(raw[i] & 0xFFFF0000u);
    }
    scale = amax / 448.0f;
    float q[8];
    quotients(v, scale, 1.0f / scale, amax < 0x1p-100f, q);
    const bool zero = amax == 0.0f;
    lo = zero ? 0u : codes4(q, raw[0], raw[1]);
    hi = zero ? 0u : codes4(q + 4, raw[2], raw[3]);
}

// Quantise 32 bf16 values of a head (raw: sixteen dwords, two values each)
// whose absolute maximum is amax: byte i of codes = value i; the scale once.
__device__ __forceinline__ void quantize32(const uint32_t (&raw)[16], float amax, uint32_t (&codes)[8],
                                           float &scale) {
    scale = amax / 448.0f;
    const float r = 1.0f / scale;
    const bool tiny = amax < 0x1p-100f, zero = amax == 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float v[8], q[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(raw[4 * j + i] << 16);
            v[2 * i + 1] = __uint_as_float(raw[4 * j + i] & 0xFFFF0000u);
        }
        quotients(v, scale, r, tiny, q);
        codes[2 * j] = zero ? 0u : codes4(q, raw[4 * j], raw[4 * j + 1]);
        codes[2 * j + 1] = zero ? 0u : codes4(q + 4, raw[4 * j + 2], raw[4 * j + 3]);
    }
}

// Absolute maximum of the eight bf16 values of a lane.
__device__ __forceinline__ float amax8(const uint32_t (&raw)[4]) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        m = fmaxf(m, __builtin_fabsf(__uint_as_float(raw[i] << 16)));
        m = fmaxf(m, __builtin_fabsf(__uint_as_float(raw[i] & 0xFFFF0000u)));
    }
    return m;
}

// Absolute maximum over the 16 lanes of this lane's DPP row (one key).
__device__ __forceinline__ float row_amax(float m) {
    m = fmaxf(m, row_ror<8>(m));
    m = fmaxf(m, row_ror<4>(m));
    m = fmaxf(m, row_ror<2>(m));
    m = fmaxf(m, row_ror<1>(m));
    return m;
}

}  // namespace
}  // namespace idx
