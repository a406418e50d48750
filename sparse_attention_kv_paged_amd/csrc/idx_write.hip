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
#include "idx_quant.h"
#include "idx_write.h"

namespace idx {
namespace {

constexpr int kWriteThreads = 256;
constexpr int kLanesPerKey = kHeadDim / 8;                    // 16
constexpr int kKeysPerLoad = 64 / kLanesPerKey;               // 4 keys per wave-wide load
constexpr int kKeysPerWaveStep = 2 * kKeysPerLoad;            // 8
constexpr int kKeysPerGroupStep = (kWriteThreads / 64) * kKeysPerWaveStep;  // 32
constexpr int kMaxWriteGroups = 2048;                         // 8 workgroups per CU

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
    // bf16 -> binary32 is exact: the 16 bits are the high half of the float;
    // the key's maximum over the 16 lanes of its DPP row
    const uint32_t w4[4] = {l.raw.x, l.raw.y, l.raw.z, l.raw.w};
    const float amax = row_amax(amax8(w4));
    Dword2 codes;
    float scale;
    quantize8(w4, amax, codes.lo, codes.hi, scale);

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
