// Index-plane writer for gfx950: new compressed keys (bf16) become pool rows
// of D float8_e4m3fn bytes followed by the fp32 scale, the row layout the
// score kernel reads ("FlashMemory-DeepSeek-V4" README, section
// "compressed_k format"; the batchgen pull request's fp8 indexer-pool insert
// writes rows of that layout).  The pages leave the scale rule open; the
// reading taken is the per-row absolute maximum over e4m3's largest finite
// value, s = amax / 448, and byte d = e4m3(k[d] / s), both divisions in
// binary32 rounded to nearest, the e4m3 rounding to nearest with ties to the
// even code and saturating at +-448.  An all-zero key is stored as zero bytes
// and scale 0.
//
// The writer is a stream: 256 bytes of bf16 in, 132 bytes out per key.  Sixteen
// lanes share one key: each loads 16 consecutive bytes (8 values), the key's
// absolute maximum comes from four DPP max steps inside the 16-lane group (a
// DPP row), and each lane stores its 8 codes as one 8-byte store, so the 16 lanes
// of a key write its 128 code bytes as one contiguous run.  A wave takes 8
// consecutive keys per step (two 1 KB loads) and walks the keys with a grid
// stride, issuing the loads of its next step before it converts the current
// one, so loads stay in flight while the conversion runs.
#include <algorithm>

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "../../include/idx.h"
#include "idx_internal.h"
#include "idx_write.h"

namespace idx {
namespace {

constexpr int kWriteThreads = 256;
constexpr int kLanesPerKey = kHeadDim / 8;                    // 16
constexpr int kKeysPerLoad = 64 / kLanesPerKey;               // 4 keys per wave-wide load
constexpr int kKeysPerWaveStep = 2 * kKeysPerLoad;            // 8
constexpr int kKeysPerGroupStep = (kWriteThreads / 64) * kKeysPerWaveStep;  // 32
constexpr int kMaxWriteGroups = 2048;                         // 8 workgroups per CU

// Quotients q[i] = v[i] / s, rounded to binary32 as an IEEE division would
// round them, as far as the e4m3 code can tell: r = 1/s is divided once per
// key, then each quotient is q0 = v*r corrected once with the exact residual
// v - q0*s (Markstein's correction step, two FMAs).  Checked against the IEEE
// quotient over every bf16 pair |v| <= amax: the e4m3 codes agree for every
// amax >= 2^-104 once the sign is taken from v (the correction turns -0 into
// +0); below that the residual underflows, so keys with amax < 2^-100 divide
// each element instead.
__device__ __forceinline__ void quotients(const float *v, float scale, bool tiny, float *q) {
#pragma clang fp contract(off)
    const float r = 1.0f / scale;
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

// A pair of dwords stored with one 8-byte store at a 4-byte aligned address
// (pool rows are 132 bytes apart).
struct __attribute__((aligned(4))) Dword2 {
    uint32_t lo, hi;
};

// The loads of one key for one lane: its 16-byte slice and the key's slot.
struct KeyLoad {
    uint4 raw;
    int64_t slot;
};

__device__ __forceinline__ KeyLoad load_key(const WriteArgs &a, int64_t key, int part) {
    KeyLoad l{make_uint4(0u, 0u, 0u, 0u), -1};
    if (key < a.n) {
        l.slot = a.slots[key];
        l.raw = *reinterpret_cast<const uint4 *>(a.k + key * kHeadDim + part * 8);
    }
    return l;
}

// Quantise one key slice and store it; returns whether the slot was bad.
__device__ __forceinline__ bool store_key(const WriteArgs &a, const KeyLoad &l, int64_t key, int part) {
    // bf16 -> binary32 is exact: the 16 bits are the high half of the float
    float v[8];
    const uint32_t w4[4] = {l.raw.x, l.raw.y, l.raw.z, l.raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w4[i] << 16);
        v[2 * i + 1] = __uint_as_float(w4[i] & 0xFFFF0000u);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, __builtin_fabsf(v[i]));
    // maximum over the 16 lanes of this key: a DPP row is 16 lanes, so row
    // rotations by 8, 4, 2, 1 leave every lane of the row with the maximum
    amax = fmaxf(amax, row_ror<8>(amax));
    amax = fmaxf(amax, row_ror<4>(amax));
    amax = fmaxf(amax, row_ror<2>(amax));
    amax = fmaxf(amax, row_ror<1>(amax));

    const float scale = amax / 448.0f;
    float q[8];
    quotients(v, scale, amax < 0x1p-100f, q);
    // a key of zeros: zero bytes (its quotients are 0/0)
    const bool zero = amax == 0.0f;
    Dword2 codes;
    codes.lo = zero ? 0u : codes4(q, l.raw.x, l.raw.y);
    codes.hi = zero ? 0u : codes4(q + 4, l.raw.z, l.raw.w);

    const bool in_pool = l.slot >= 0 && l.slot < a.n_pool_rows;
    if (in_pool) {
        uint8_t *row = a.pool + l.slot * kRowBytes;
        *reinterpret_cast<Dword2 *>(row + part * 8) = codes;
        if (part == 0) *reinterpret_cast<float *>(row + kHeadDim) = scale;
    }
    return key < a.n && l.slot != -1 && !in_pool;
}

__global__ __launch_bounds__(kWriteThreads) void write_keys_kernel(WriteArgs a) {
    const int lane = threadIdx.x % 64;
    const int part = lane % kLanesPerKey;
    const int64_t wave = (int64_t)blockIdx.x * (kWriteThreads / 64) + threadIdx.x / 64;
    const int64_t stride = (int64_t)gridDim.x * (kWriteThreads / 64) * kKeysPerWaveStep;
    // this lane's two keys of a step: base + lane/16 and base + 4 + lane/16
    int64_t key = wave * kKeysPerWaveStep + lane / kLanesPerKey;
    KeyLoad c0 = load_key(a, key, part);
    KeyLoad c1 = load_key(a, key + kKeysPerLoad, part);
    bool bad = false;
    // every lane of a wave runs the same number of steps (the loop bound is
    // the wave's base), so the cross-lane max always sees all 64 lanes
    for (int64_t base = wave * kKeysPerWaveStep; base < a.n; base += stride, key += stride) {
        const KeyLoad n0 = load_key(a, key + stride, part);
        const KeyLoad n1 = load_key(a, key + stride + kKeysPerLoad, part);
        bad |= store_key(a, c0, key, part);
        bad |= store_key(a, c1, key + kKeysPerLoad, part);
        c0 = n0;
        c1 = n1;
    }
    if (a.status && __ballot(bad) != 0 && lane == 0) atomicOr(a.status, IDX_STATUS_BAD_SLOT);
}

}  // namespace

hipError_t launch_write_keys(const WriteArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    const int64_t groups = std::min<int64_t>(kMaxWriteGroups, (a.n + kKeysPerGroupStep - 1) / kKeysPerGroupStep);
    hipExtLaunchKernelGGL(write_keys_kernel, dim3((uint32_t)groups), dim3(kWriteThreads), 0, s, e0, e1, 0, a);
    return hipGetLastError();
}

}  // namespace idx
