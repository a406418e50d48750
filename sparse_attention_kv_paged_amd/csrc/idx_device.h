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

// DPP controls (GFX9): row_shr:n = 0x110 + n, row_bcast:15, row_bcast:31.
// Lanes the control leaves without a source keep `old`.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp(uint32_t v, uint32_t old = 0u) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xF, false);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts and
// row broadcasts (no LDS round trips).
__device__ __forceinline__ uint32_t wave_scan(uint32_t v) {
    v += dpp<0x111, 0xF>(v);
    v += dpp<0x112, 0xF>(v);
    v += dpp<0x114, 0xF>(v);
    v += dpp<0x118, 0xF>(v);
    v += dpp<0x142, 0xA>(v);
    v += dpp<0x143, 0xC>(v);
    return v;
}

// A workgroup barrier for LDS traffic only: each wave's LDS operations have
// completed (lgkmcnt 0) when it arrives, but its vector-memory loads still in
// flight are not waited for, as __syncthreads would (it waits for vmcnt 0).
// For barriers that only order LDS data between the waves.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Raw buffer descriptor over [base, base + bytes): loads outside the range
// return 0 and stores outside it are dropped, so bounds need no branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Cache-policy operand of buffer loads/stores: sc1 (device scope), i.e. the
// access is coherent across the per-XCD L2 caches.
constexpr int kDeviceCoherent = 16;
// Cache-policy operand: nt (non-temporal), a streaming access the caches
// need not keep.
constexpr int kNonTemporal = 2;

}  // namespace idx
