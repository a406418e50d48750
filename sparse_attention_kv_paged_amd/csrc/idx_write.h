// Internal launch interface of the index-plane writer (idx_write.hip), used
// by the C-ABI layer (idx_api.cpp).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace idx {

// One launch of the writer: key i goes to pool row slots[i].
struct WriteArgs {
    const uint16_t *k;          // [n, 128] bf16 keys, 16-byte aligned
    int64_t n;
    const int64_t *slots;       // [n] pool row of each key; -1 = none
    uint8_t *pool;              // [n_pool_rows, 132]
    int64_t n_pool_rows;
    uint32_t *status;           // optional
};

// ev_start / ev_stop (optional): events the dispatch itself stamps with the
// kernel's start and end time (hipExtLaunchKernelGGL).
hipError_t launch_write_keys(const WriteArgs &a, hipStream_t s, hipEvent_t ev_start = nullptr,
                             hipEvent_t ev_stop = nullptr);

}  // namespace idx
