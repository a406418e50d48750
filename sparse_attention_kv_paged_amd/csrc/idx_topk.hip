// Per-row top-k selection for gfx950: the k largest logits of each query row
// ("FlashMemory-DeepSeek-V4" README, "Two-level recall algorithm": Level 2
// keeps the top-512 of the resident logits, the rest being -inf).
//
// One workgroup of 1024 threads selects the top-k of one segment of a row
// with the whole segment resident in LDS, so every pass after the first
// global read is an LDS pass and nothing needs a global atomic or a zeroed
// workspace:
//   1. load the segment's order-preserving keys (idx_device.h) into LDS and
//      reduce the count, min and max of its selectable values;
//   2. histogram the values into 2048 bins LINEAR in value between min and
//      max (few LDS atomic collisions, unlike bins of the float's top bits,
//      which put most logits of a row into a handful of bins), and find the
//      bin t holding the k-th largest value;
//   3. resolve the exact cut inside bin t with radix passes over the keys of
//      the bin's members (bits 31:21, 20:10, 9:0), stopping as soon as a
//      sub-bin is taken whole;
//   4. write the winners in column order: every wave owns a contiguous range
//      of the segment, counts its winners with ballots, and a 16-entry scan
//      gives each wave its output offset.  Equal values at the cut are taken
//      from the lowest columns, via the same ordered scan.
// A row longer than one segment is split into parts; each part keeps its own
// top-k (key, column) list and a second launch merges the lists of a row the
// same way (lists are concatenated in part order, so column order holds).
// The result is deterministic and ordered by column.
#include "idx_device.h"
#include "idx_internal.h"

namespace idx {
namespace {

constexpr int kThreads = 1024;
constexpr int kWavesPerWg = kThreads / 64;
constexpr int kBins = 2048;

// Inclusive scan over the 1024 threads (16 waves); `sh` has 16 words.
__device__ __forceinline__ uint32_t block_scan1024(uint32_t v, uint32_t *sh) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        uint32_t o = __shfl_up(v, d, 64);
        if (lane >= d) v += o;
    }
    if (lane == 63) sh[wave] = v;
    __syncthreads();
    uint32_t add = 0;
    for (int i = 0; i < wave; ++i) add += sh[i];
    __syncthreads();
    return v + add;
}

// Bin t of an LDS histogram `h` (nbins a multiple of 1024) with
// count(bins > t) < need <= count(bins >= t).  res[0] = t (-1 if the total is
// below need), res[1] = count(bins > t).  All 1024 threads call it.
__device__ void find_from_top(const uint32_t *h, int nbins, uint32_t need, int32_t *res,
                              uint32_t *scan_sh) {
    const int tid = threadIdx.x;
    const int bpt = nbins / kThreads;
    const int g = kThreads - 1 - tid;
    uint32_t local = 0;
    for (int i = 0; i < bpt; ++i) local += h[g * bpt + i];
    if (tid == 0) {
        res[0] = -1;
        res[1] = 0;
    }
    const uint32_t incl = block_scan1024(local, scan_sh);
    const uint32_t excl = incl - local;
    if (tid == kThreads - 1 && incl < need) res[1] = incl;
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

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) v = fminf(v, __shfl_xor(v, d, 64));
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
    return v;
}
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) v += __shfl_xor(v, d, 64);
    return v;
}

// Value-linear bin of a selectable key (monotone non-decreasing in value).
__device__ __forceinline__ int value_bin(uint32_t key, float vmin, float scale) {
    if (scale == 0.f) return 0;
    const float x = (key_value(key) - vmin) * scale;
    return (int)fminf(floorf(x), (float)(kBins - 1));
}

struct Cut {
    int32_t bin;        // value bin of the cut (-1: every selectable item wins)
    int32_t lo;         // key bits below `lo` are unresolved
    uint32_t prefix;    // key >> lo of the cut
    uint32_t need_ties; // how many items of (bin, prefix) win, lowest columns first
};

template <int CAP, bool LIST>
__global__ __launch_bounds__(kThreads) void topk_segment_kernel(SegArgs a) {
    __shared__ uint32_t sh_key[CAP];
    __shared__ uint32_t sh_col[LIST ? CAP : 1];
    __shared__ uint32_t sh_hist[kBins];
    __shared__ uint32_t sh_scan[kWavesPerWg];
    __shared__ float sh_fmin[kWavesPerWg], sh_fmax[kWavesPerWg];
    __shared__ uint32_t sh_cnt[kWavesPerWg];
    __shared__ int32_t sh_res[2];
    __shared__ uint32_t sh_win_base[kWavesPerWg], sh_tie_base[kWavesPerWg];
    __shared__ uint32_t sh_total;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.x / a.parts;
    const int part = blockIdx.x - b * a.parts;
    const int k = a.k;

    // ---- 1. load the segment into LDS (key 0 = not selectable)
    int64_t col0 = 0;
    uint32_t n_valid = 0;
    float fmn = __builtin_inff(), fmx = -__builtin_inff();
    if (!LIST) {
        col0 = (int64_t)part * CAP;
        const int ncols = a.row_cols ? min((int)a.row_cols[b], a.n_cols) : a.n_cols;
        const int n = (int)max<int64_t>(0, min<int64_t>(CAP, ncols - col0));
        const float *src = a.logits + (int64_t)b * a.ld + col0;
#pragma unroll 8
        for (int i = tid; i < CAP; i += kThreads) {
            uint32_t key = 0;
            if (i < n) key = order_key(src[i]);
            sh_key[i] = key;
            if (key) {
                const float v = key_value(key);
                ++n_valid;
                fmn = fminf(fmn, v);
                fmx = fmaxf(fmx, v);
            }
        }
    } else {
        // lists [part*G, part*G + G) of row b, each at a fixed stride
        const int G = CAP / a.in_cap;
        const int l0 = part * G;
        for (int i = tid; i < CAP; i += kThreads) {
            const int g = i / a.in_cap, j = i - g * a.in_cap;
            const int l = l0 + g;
            uint32_t key = 0, col = 0;
            if (g < G && l < a.in_parts) {
                const int64_t li = (int64_t)b * a.in_parts + l;
                if ((uint32_t)j < a.in_cnt[li]) {
                    const uint2 it = a.in_list[li * a.in_cap + j];
                    key = it.x;
                    col = it.y;
                }
            }
            sh_key[i] = key;
            sh_col[i] = col;
            if (key) {
                const float v = key_value(key);
                ++n_valid;
                fmn = fminf(fmn, v);
                fmx = fmaxf(fmx, v);
            }
        }
    }
    n_valid = wave_sum(n_valid);
    fmn = wave_min(fmn);
    fmx = wave_max(fmx);
    if (lane == 0) {
        sh_cnt[wave] = n_valid;
        sh_fmin[wave] = fmn;
        sh_fmax[wave] = fmx;
    }
    __syncthreads();
    uint32_t total = 0;
    float vmin = __builtin_inff(), vmax = -__builtin_inff();
    for (int w = 0; w < kWavesPerWg; ++w) {
        total += sh_cnt[w];
        vmin = fminf(vmin, sh_fmin[w]);
        vmax = fmaxf(vmax, sh_fmax[w]);
    }

    // ---- 2./3. find the cut
    Cut cut{-1, 0, 0u, 0u};
    float scale = 0.f;
    if (total > (uint32_t)k) {
        const float range = vmax - vmin;
        if (range > 0.f && range < __builtin_inff()) scale = (float)kBins / range;
        if (!(scale < __builtin_inff())) scale = 0.f;
        for (int i = tid; i < kBins; i += kThreads) sh_hist[i] = 0u;
        __syncthreads();
        for (int i = tid; i < CAP; i += kThreads) {
            const uint32_t key = sh_key[i];
            if (key) atomicAdd(&sh_hist[value_bin(key, vmin, scale)], 1u);
        }
        __syncthreads();
        find_from_top(sh_hist, kBins, (uint32_t)k, sh_res, sh_scan);
        cut.bin = sh_res[0];
        uint32_t rem = (uint32_t)k - (uint32_t)sh_res[1];
        cut.lo = 32;
        cut.prefix = 0;
        bool whole = sh_hist[cut.bin] == rem;
        // radix passes over the keys of the cut bin's members
        for (int stage = 0; stage < 3 && !whole; ++stage) {
            const int nb = stage == 2 ? 10 : 11;
            const int nlo = cut.lo - nb;
            const int nbins = 1 << nb;
            __syncthreads();
            for (int i = tid; i < kBins; i += kThreads) sh_hist[i] = 0u;
            __syncthreads();
            for (int i = tid; i < CAP; i += kThreads) {
                const uint32_t key = sh_key[i];
                if (key && value_bin(key, vmin, scale) == cut.bin &&
                    (cut.lo == 32 || (key >> cut.lo) == cut.prefix))
                    atomicAdd(&sh_hist[(key >> nlo) & (nbins - 1)], 1u);
            }
            __syncthreads();
            find_from_top(sh_hist, kBins, rem, sh_res, sh_scan);
            const int t = sh_res[0];
            rem -= (uint32_t)sh_res[1];
            cut.prefix = (cut.lo == 32 ? 0u : (cut.prefix << nb)) | (uint32_t)t;
            cut.lo = nlo;
            whole = sh_hist[t] == rem;
        }
        cut.need_ties = rem;
    }

    // ---- 4. winners in column order
    // per item: 2 = certain winner, 1 = tie at the cut, 0 = loser
    auto klass = [&](uint32_t key) -> int {
        if (!key) return 0;
        if (cut.bin < 0) return 2;
        const int bn = value_bin(key, vmin, scale);
        if (bn != cut.bin) return bn > cut.bin ? 2 : 0;
        if (cut.lo == 32) return 1;
        const uint32_t p = key >> cut.lo;
        return p > cut.prefix ? 2 : (p == cut.prefix ? 1 : 0);
    };
    constexpr int per_wave = CAP / kWavesPerWg;
    const int w0 = wave * per_wave;
    uint32_t n_win = 0, n_tie = 0;
    for (int i = lane; i < per_wave; i += 64) {
        const int c = klass(sh_key[w0 + i]);
        n_win += __popcll(__ballot(c == 2));
        n_tie += __popcll(__ballot(c == 1));
    }
    __syncthreads();
    if (lane == 0) {
        sh_cnt[wave] = n_win;
        sh_scan[wave] = n_tie;
    }
    __syncthreads();
    if (tid == 0) {
        uint32_t wb = 0, tb = 0;
        for (int w = 0; w < kWavesPerWg; ++w) {
            sh_win_base[w] = wb;
            sh_tie_base[w] = tb;
            const uint32_t ties = sh_scan[w];
            const uint32_t taken = tb >= cut.need_ties ? 0u : min(ties, cut.need_ties - tb);
            wb += sh_cnt[w] + taken;
            tb += ties;
        }
        sh_total = wb;
    }
    __syncthreads();
    uint32_t pos = sh_win_base[wave], tie_ord = sh_tie_base[wave];
    const uint64_t below = (1ull << lane) - 1ull;
    for (int i = lane; i < per_wave; i += 64) {
        const int idx = w0 + i;
        const uint32_t key = sh_key[idx];
        const int c = klass(key);
        const uint64_t tm = __ballot(c == 1);
        const bool win = c == 2 || (c == 1 && tie_ord + (uint32_t)__popcll(tm & below) < cut.need_ties);
        const uint64_t wm = __ballot(win);
        if (win) {
            const uint32_t o = pos + (uint32_t)__popcll(wm & below);
            const uint32_t col = LIST ? sh_col[idx] : (uint32_t)(col0 + idx);
            if (a.out_list) {
                a.out_list[((int64_t)b * a.parts + part) * k + o] = make_uint2(key, col);
            } else {
                int32_t e = (int32_t)col;
                if (a.chunk_ids) {
                    const int32_t beta = a.chunk_ids[(int64_t)b * a.max_chunks + (int32_t)col / kBlock];
                    e = beta * kBlock + (int32_t)col % kBlock;
                }
                a.out_idx[(int64_t)b * k + o] = e;
                if (a.out_val) a.out_val[(int64_t)b * k + o] = key_value(key);
            }
        }
        pos += (uint32_t)__popcll(wm);
        tie_ord += (uint32_t)__popcll(tm);
    }
    const uint32_t count = min(sh_total, (uint32_t)k);
    if (a.out_list) {
        if (tid == 0) a.out_cnt[(int64_t)b * a.parts + part] = count;
    } else {
        for (int i = (int)count + tid; i < k; i += kThreads) {
            a.out_idx[(int64_t)b * k + i] = -1;
            if (a.out_val) a.out_val[(int64_t)b * k + i] = -__builtin_inff();
        }
    }
}

template <int CAP, bool LIST>
hipError_t launch_seg(const SegArgs &a, hipStream_t s) {
    const int64_t grid = (int64_t)a.B * a.parts;
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL((topk_segment_kernel<CAP, LIST>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

int topk_segment_capacity(bool list) { return list ? kSegListCap : kSegLogitCap; }

hipError_t launch_topk_segment(const SegArgs &a, bool list, int cap, hipStream_t s) {
    if (list) return launch_seg<kSegListCap, true>(a, s);
    switch (cap) {
    case 4096: return launch_seg<4096, false>(a, s);
    case 8192: return launch_seg<8192, false>(a, s);
    case 16384: return launch_seg<16384, false>(a, s);
    default: return launch_seg<kSegLogitCap, false>(a, s);
    }
}

}  // namespace idx
