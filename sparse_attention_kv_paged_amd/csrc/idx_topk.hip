// Per-row top-k selection for gfx950: the k largest logits of each query row
// ("FlashMemory-DeepSeek-V4" README, "Two-level recall algorithm": Level 2
// keeps the top-512 of the resident logits, the rest being -inf).
//
// One workgroup selects the top-k of one segment of a row.  Each thread holds
// a contiguous run of the segment's order-preserving keys (idx_device.h) in
// registers for the whole kernel, so after the single global read the passes
// below are register work plus a few LDS histograms and block scans; nothing
// needs a global atomic or a zeroed workspace:
//   1. load the keys and reduce the count, min and max of the selectable
//      values;
//   2. histogram the values into 2048 bins LINEAR in value between min and
//      max (few LDS atomic collisions, unlike bins of the float's top bits,
//      which put most logits of a row into a handful of bins), and find the
//      bin t holding the k-th largest value;
//   3. copy bin t's members to LDS (positions from a block scan) and find the
//      exact k-th largest key among them: one wave ranks up to 64 members
//      against each other; larger bins take radix passes over their keys
//      (bits 31:21, 20:10, 9:0);
//   4. write the winners (keys above the k-th, plus as many copies of it as
//      needed, lowest columns first) in column order: one block scan of the
//      threads' winner and tie counts gives every thread its output offset.
// A row longer than one segment is split into parts; each part keeps its own
// top-k (key, column) list and a second launch merges the lists of a row the
// same way (lists are concatenated in part order, so column order holds).
// The result is deterministic and ordered by column.
#include "idx_device.h"
#include "idx_internal.h"

namespace idx {
namespace {

constexpr int kBins = 2048;

// DPP controls (GFX9): row_shr:n = 0x110 + n, row_bcast:15, row_bcast:31.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
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

// Inclusive scan over the NT threads of the workgroup; `sh` has NT/64 words.
template <int NT>
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t *sh) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_scan(v);
    if (lane == 63) sh[wave] = v;
    __syncthreads();
    uint32_t add = 0;
    for (int i = 0; i < wave; ++i) add += sh[i];
    __syncthreads();
    return v + add;
}

// Bin t of an LDS histogram `h` (nbins a multiple of NT) with
// count(bins > t) < need <= count(bins >= t).  res[0] = t (-1 if the total is
// below need), res[1] = count(bins > t).  All NT threads call it.
template <int NT>
__device__ void find_from_top(const uint32_t *h, int nbins, uint32_t need, int32_t *res,
                              uint32_t *scan_sh) {
    const int tid = threadIdx.x;
    const int bpt = nbins / NT;
    const int g = NT - 1 - tid;
    uint32_t local = 0;
    for (int i = 0; i < bpt; ++i) local += h[g * bpt + i];
    if (tid == 0) {
        res[0] = -1;
        res[1] = 0;
    }
    const uint32_t incl = block_scan<NT>(local, scan_sh);
    const uint32_t excl = incl - local;
    if (tid == NT - 1 && incl < need) res[1] = incl;
    if (excl < need && need <= incl) {
        uint32_t c = excl;
        for (int i = bpt - 1; i >= 0; --i) {
            const uint32_t n = h[g * bpt + i];
            if (c + n >= need) {
                res[0] = g * bpt + i;
                res[1] = c;
                break;
            }
            c += n;
        }
    }
    __syncthreads();
}

// Value-linear bin of a selectable key (monotone non-decreasing in value).
__device__ __forceinline__ int value_bin(uint32_t key, float vmin, float scale) {
    if (scale == 0.f) return 0;
    const float x = (key_value(key) - vmin) * scale;
    return (int)fminf(floorf(x), (float)(kBins - 1));
}

template <int CAP, bool LIST, int NT>
__global__ __launch_bounds__(NT) void topk_segment_kernel(SegArgs a) {
    constexpr int kW = NT / 64;                       // waves per workgroup
    constexpr int kPer = CAP / NT;                    // items per thread
    __shared__ uint32_t sh_cand[CAP];                 // keys of the cut bin's members
    __shared__ uint32_t sh_hist[kBins];
    __shared__ uint32_t sh_scan[kW];
    __shared__ float sh_fmin[kW], sh_fmax[kW];
    __shared__ uint32_t sh_cnt[kW];
    __shared__ int32_t sh_res[2];
    __shared__ uint32_t sh_cut[2];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.x / a.parts;
    const int part = blockIdx.x - b * a.parts;
    const int k = a.k;
    const int i0 = tid * kPer;                        // this thread's first item

    // ---- 1. this thread's keys (key 0 = not selectable), loads all issued
    // before any is used
    uint32_t key[kPer];
    uint32_t colv[LIST ? kPer : 1];
    int64_t col0 = 0;
    if (!LIST) {
        col0 = (int64_t)part * CAP;
        const int ncols = a.row_cols ? min((int)a.row_cols[b], a.n_cols) : a.n_cols;
        const int n = (int)max<int64_t>(0, min<int64_t>(CAP, ncols - col0));
        const float *src = a.logits + (int64_t)b * a.ld + col0 + i0;
        float v[kPer];
        if ((a.ld & 3) == 0 && (reinterpret_cast<uintptr_t>(a.logits) & 15) == 0 && i0 + kPer <= n) {
#pragma unroll
            for (int j = 0; j < kPer; j += 4) {
                const float4 f = *reinterpret_cast<const float4 *>(src + j);
                v[j] = f.x;
                v[j + 1] = f.y;
                v[j + 2] = f.z;
                v[j + 3] = f.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < kPer; ++j) v[j] = i0 + j < n ? src[j] : -__builtin_inff();
        }
#pragma unroll
        for (int j = 0; j < kPer; ++j) key[j] = order_key(v[j]);
    } else {
        // lists [part*G, part*G + G) of row b, each at a fixed stride
        const int G = CAP / a.in_cap;
        const int l0 = part * G;
        const int n = max(0, min(G, a.in_parts - l0)) * a.in_cap;
        uint2 it[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int i = i0 + j;
            const int g = i / a.in_cap, jj = i - g * a.in_cap;
            const int64_t li = (int64_t)b * a.in_parts + l0 + g;
            it[j] = make_uint2(0u, 0u);
            if (i < n && (uint32_t)jj < a.in_cnt[li]) it[j] = a.in_list[li * a.in_cap + jj];
        }
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            key[j] = it[j].x;
            colv[j] = it[j].y;
        }
    }
    uint32_t n_valid = 0;
    float fmn = __builtin_inff(), fmx = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        if (key[j]) {
            const float v = key_value(key[j]);
            ++n_valid;
            fmn = fminf(fmn, v);
            fmx = fmaxf(fmx, v);
        }
    }
    // wave reductions via DPP scans (the last lane holds the total)
    n_valid = wave_scan(n_valid);
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) {
        fmn = fminf(fmn, __shfl_xor(fmn, d, 64));
        fmx = fmaxf(fmx, __shfl_xor(fmx, d, 64));
    }
    if (lane == 63) sh_cnt[wave] = n_valid;
    if (lane == 0) {
        sh_fmin[wave] = fmn;
        sh_fmax[wave] = fmx;
    }
    __syncthreads();
    uint32_t total = 0;
    float vmin = __builtin_inff(), vmax = -__builtin_inff();
    for (int w = 0; w < kW; ++w) {
        total += sh_cnt[w];
        vmin = fminf(vmin, sh_fmin[w]);
        vmax = fmaxf(vmax, sh_fmax[w]);
    }

    // ---- 2./3. the exact k-th largest key kstar and how many of its
    // copies win (lowest columns first); kstar = 0 when all selectable win
    uint32_t kstar = 0u, need_ties = 0u;
    if (total > (uint32_t)k) {
        float scale = 0.f;
        const float range = vmax - vmin;
        if (range > 0.f && range < __builtin_inff()) scale = (float)kBins / range;
        if (!(scale < __builtin_inff())) scale = 0.f;
        for (int i = tid; i < kBins; i += NT) sh_hist[i] = 0u;
        __syncthreads();
        int bins[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            bins[j] = key[j] ? value_bin(key[j], vmin, scale) : -1;
            if (key[j]) atomicAdd(&sh_hist[bins[j]], 1u);
        }
        __syncthreads();
        find_from_top<NT>(sh_hist, kBins, (uint32_t)k, sh_res, sh_scan);
        const int cbin = sh_res[0];
        uint32_t rem = (uint32_t)k - (uint32_t)sh_res[1];
        const uint32_t n_in_bin = sh_hist[cbin];
        // members of the cut bin go to LDS, in column order
        uint32_t mine = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) mine += bins[j] == cbin;
        uint32_t at = block_scan<NT>(mine, sh_scan) - mine;
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            if (bins[j] == cbin) sh_cand[at++] = key[j];
        __syncthreads();
        if (n_in_bin <= 64u) {
            // few members: wave 0 ranks them against each other directly
            if (wave == 0) {
                const uint32_t my = lane < (int)n_in_bin ? sh_cand[lane] : 0u;
                uint32_t greater = 0, equal = 0;
                for (uint32_t j = 0; j < n_in_bin; ++j) {
                    const uint32_t other = (uint32_t)__builtin_amdgcn_readlane((int)my, (int)j);
                    greater += other > my;
                    equal += other == my;
                }
                if (lane < (int)n_in_bin && greater < rem && rem <= greater + equal) {
                    sh_cut[0] = my;              // every such lane holds the same key
                    sh_cut[1] = rem - greater;
                }
            }
            __syncthreads();
            kstar = sh_cut[0];
            need_ties = sh_cut[1];
        } else {
            // radix passes over the members' keys: bits 31:21, 20:10, 9:0
            uint32_t prefix = 0u;
            for (int stage = 0; stage < 3; ++stage) {
                const int hi = stage == 0 ? 32 : (stage == 1 ? 21 : 10);
                const int lo = stage == 0 ? 21 : (stage == 1 ? 10 : 0);
                __syncthreads();
                for (int i = tid; i < kBins; i += NT) sh_hist[i] = 0u;
                __syncthreads();
                const uint32_t mask = (1u << (hi - lo)) - 1u;
                for (uint32_t c = tid; c < n_in_bin; c += NT) {
                    const uint32_t kk = sh_cand[c];
                    if (hi == 32 || (kk >> hi) == prefix) atomicAdd(&sh_hist[(kk >> lo) & mask], 1u);
                }
                __syncthreads();
                find_from_top<NT>(sh_hist, kBins, rem, sh_res, sh_scan);
                rem -= (uint32_t)sh_res[1];
                prefix = (hi == 32 ? 0u : (prefix << (hi - lo))) | (uint32_t)sh_res[0];
            }
            kstar = prefix;
            need_ties = rem;
        }
    }

    // ---- 4. winners (key > kstar, plus the first need_ties keys == kstar)
    // in column order; one scan of packed (winners | ties << 16) per thread
    uint32_t n_win = 0, n_tie = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        n_win += key[j] > kstar;
        n_tie += kstar != 0u && key[j] == kstar;
    }
    const uint32_t packed = n_win | (n_tie << 16);
    const uint32_t excl = block_scan<NT>(packed, sh_scan) - packed;
    if (tid == NT - 1) {
        sh_cut[0] = (excl + packed) & 0xFFFFu;                  // all certain winners
        sh_cut[1] = (excl + packed) >> 16;                      // all ties
    }
    uint32_t tie_ord = excl >> 16;
    uint32_t pos = (excl & 0xFFFFu) + min(tie_ord, need_ties);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        bool win = key[j] > kstar;
        if (kstar != 0u && key[j] == kstar) win = tie_ord++ < need_ties;
        if (win) {
            const uint32_t col = LIST ? colv[j] : (uint32_t)(col0 + i0 + j);
            const uint32_t o = pos++;
            if (a.out_list) {
                a.out_list[((int64_t)b * a.parts + part) * k + o] = make_uint2(key[j], col);
            } else {
                int32_t e = (int32_t)col;
                if (a.chunk_ids) {
                    const int32_t beta = a.chunk_ids[(int64_t)b * a.max_chunks + (int32_t)col / kBlock];
                    e = beta * kBlock + (int32_t)col % kBlock;
                }
                a.out_idx[(int64_t)b * k + o] = e;
                if (a.out_val) a.out_val[(int64_t)b * k + o] = key_value(key[j]);
            }
        }
    }
    __syncthreads();
    const uint32_t count = min(sh_cut[0] + min(sh_cut[1], need_ties), (uint32_t)k);
    if (a.out_list) {
        if (tid == 0) a.out_cnt[(int64_t)b * a.parts + part] = count;
    } else {
        for (int i = (int)count + tid; i < k; i += NT) {
            a.out_idx[(int64_t)b * k + i] = -1;
            if (a.out_val) a.out_val[(int64_t)b * k + i] = -__builtin_inff();
        }
    }
}

template <int CAP, bool LIST, int NT>
hipError_t launch_seg(const SegArgs &a, hipStream_t s) {
    const int64_t grid = (int64_t)a.B * a.parts;
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL((topk_segment_kernel<CAP, LIST, NT>), dim3((unsigned)grid), dim3(NT), 0, s, a);
    return hipGetLastError();
}

}  // namespace

// Capacities (items per workgroup / threads): logits 4096/256, 8192/512,
// 16384/1024, 32768/1024; lists 4096/256, 16384/1024.
hipError_t launch_topk_segment(const SegArgs &a, bool list, int cap, hipStream_t s) {
    if (list) return cap <= 4096 ? launch_seg<4096, true, 256>(a, s) : launch_seg<kSegListCap, true, 1024>(a, s);
    switch (cap) {
    case 4096: return launch_seg<4096, false, 256>(a, s);
    case 8192: return launch_seg<8192, false, 512>(a, s);
    case 16384: return launch_seg<16384, false, 1024>(a, s);
    default: return launch_seg<kSegLogitCap, false, 1024>(a, s);
    }
}

}  // namespace idx
