// Per-row top-k selection for gfx950: the k largest logits of each query row
// ("FlashMemory-DeepSeek-V4" README, "Two-level recall algorithm": Level 2
// keeps the top-512 of the resident logits, the rest being -inf).
//
// Radix select on order-preserving uint32 keys (idx_device.h), three launches
// after the histogram pass:
//   1. histogram of the key's top 11 bits per row (fused into the score
//      kernel's epilogue for idx_score_topk, or topk_hist_kernel here);
//   2. select: each workgroup finds the row's threshold bin T (the bin that
//      holds the k-th largest key) from the histogram, then streams its
//      columns once: keys above T are certain members ("sure"), keys in T are
//      candidates; both are appended with one atomic per wave (ballot +
//      popcount);
//   3. final: one workgroup per row finishes the selection among the
//      candidates by radix passes over the low 21 key bits and, only when
//      equal keys straddle the cut, over the column (lower column wins), then
//      bitonic-sorts the k winners (value descending, column ascending) in
//      LDS and writes them.
// The result is deterministic: the chosen set and its order depend only on
// the values, never on atomic arrival order.
#include "idx_device.h"
#include "idx_internal.h"

namespace idx {
namespace {

__global__ __launch_bounds__(256) void topk_init_kernel(TopkArgs a) {
    const int64_t n_hist = (int64_t)a.B * kHistBins;
    const int64_t n_cnt = (int64_t)a.B * kCounters;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_hist + n_cnt; i += stride) {
        if (i < n_hist) {
            a.hist[i] = 0u;
        } else {
            const int64_t j = i - n_hist;
            a.counters[j] = (a.set_cols && (j % kCounters) == kCntCols) ? (uint32_t)a.n_cols : 0u;
        }
    }
}

__global__ __launch_bounds__(256) void topk_hist_kernel(TopkArgs a) {
    __shared__ uint32_t sh_hist[kHistBins];
    const int b = blockIdx.x / a.parts;
    const int part = blockIdx.x - b * a.parts;
    for (int i = threadIdx.x; i < kHistBins; i += 256) sh_hist[i] = 0u;
    __syncthreads();
    const int c0 = part * a.cols_per_wg;
    const int c1 = min(c0 + a.cols_per_wg, a.n_cols);
    const float *row = a.logits + (int64_t)b * a.ld;
    for (int c = c0 + threadIdx.x; c < c1; c += 256) {
        const uint32_t key = order_key(row[c]);
        if (key) atomicAdd(&sh_hist[key >> kHistShift], 1u);
    }
    __syncthreads();
    uint32_t *gh = a.hist + (int64_t)b * kHistBins;
    for (int i = threadIdx.x; i < kHistBins; i += 256) {
        const uint32_t c = sh_hist[i];
        if (c) atomicAdd(gh + i, c);
    }
}

// Threshold bin of row b: the bin holding the k-th largest key, or -1 when
// the row has at most k selectable entries (then all of them are members).
__device__ void row_threshold(const TopkArgs &a, int b, uint32_t *sh_hist, int32_t *res,
                              uint32_t *scan_sh) {
    const uint32_t *gh = a.hist + (int64_t)b * kHistBins;
    for (int i = threadIdx.x; i < kHistBins; i += 256) sh_hist[i] = gh[i];
    __syncthreads();
    // need k + 1 from the top: if fewer than k+1 exist, every entry is a member
    find_rank_bin<true>(sh_hist, kHistBins, (uint32_t)a.k + 1u, res, scan_sh);
    if (res[0] >= 0) {
        __syncthreads();
        find_rank_bin<true>(sh_hist, kHistBins, (uint32_t)a.k, res, scan_sh);
    }
}

// Appends the predicate-true lanes' items to list[*counter ...]; writes past
// `cap` are dropped (the counter still counts them).
__device__ __forceinline__ void wave_append(bool pred, uint2 item, uint2 *list, uint32_t *counter,
                                            uint32_t cap) {
    const uint64_t m = __ballot(pred);
    if (m == 0) return;
    const int lane = threadIdx.x & 63;
    const int leader = __ffsll((long long)m) - 1;
    uint32_t base = 0;
    if (lane == leader) base = atomicAdd(counter, (uint32_t)__popcll(m));
    base = __shfl(base, leader, 64);
    if (pred) {
        const uint32_t off = (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
        if (base + off < cap) list[base + off] = item;
    }
}

__global__ __launch_bounds__(256) void topk_select_kernel(TopkArgs a) {
    __shared__ uint32_t sh_hist[kHistBins];
    __shared__ int32_t sh_res[2];
    __shared__ uint32_t sh_scan[4];
    const int b = blockIdx.x / a.parts;
    const int part = blockIdx.x - b * a.parts;
    const uint32_t *cnt = a.counters + (int64_t)b * kCounters;
    const int ncols = min((int)cnt[kCntCols], a.n_cols);
    const int c0 = part * a.cols_per_wg;
    if (c0 >= ncols) return;                          // uniform per workgroup
    row_threshold(a, b, sh_hist, sh_res, sh_scan);
    const int32_t T = sh_res[0];
    const int c1 = min(c0 + a.cols_per_wg, ncols);
    const float *row = a.logits + (int64_t)b * a.ld;
    uint2 *sure = a.sure + (int64_t)b * a.k;
    uint2 *cand = a.cand + (int64_t)b * a.ldc;
    uint32_t *cnt_w = a.counters + (int64_t)b * kCounters;
    // every thread runs the same trip count so the wave-wide ballots line up
    for (int base = c0; base < c1; base += 256) {
        const int c = base + threadIdx.x;
        uint32_t key = 0;
        if (c < c1) key = order_key(row[c]);
        const int32_t bin = (int32_t)(key >> kHistShift);
        const bool is_sure = key != 0u && bin > T;
        const bool is_cand = key != 0u && T >= 0 && bin == T;
        wave_append(is_sure, make_uint2(key, (uint32_t)c), sure, cnt_w + kCntSure, (uint32_t)a.k);
        wave_append(is_cand, make_uint2(key, (uint32_t)c), cand, cnt_w + kCntCand, (uint32_t)a.ldc);
    }
}

__global__ __launch_bounds__(256) void topk_final_kernel(TopkArgs a) {
    __shared__ uint32_t sh_hist[kHistBins];
    __shared__ unsigned long long sh_out[kMaxK];
    __shared__ int32_t sh_res[2];
    __shared__ uint32_t sh_scan[4];
    __shared__ uint32_t sh_count;
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int k = a.k;

    row_threshold(a, b, sh_hist, sh_res, sh_scan);
    const int32_t T = sh_res[0];
    const uint32_t *cnt = a.counters + (int64_t)b * kCounters;
    const uint32_t n_sure = min(cnt[kCntSure], (uint32_t)k);
    const uint32_t n_cand = (uint32_t)min((int64_t)cnt[kCntCand], a.ldc);
    const uint2 *sure = a.sure + (int64_t)b * k;
    const uint2 *cand = a.cand + (int64_t)b * a.ldc;

    // Selection rule for a candidate (key, col):
    //   (key >> lo) > P, or (key >> lo) == P and col <= cstar.
    int lo = 32 - kHistBits;
    uint32_t P = (uint32_t)max(T, 0);
    uint32_t cstar = 0xFFFFFFFFu;
    if (T >= 0 && n_cand > 0) {
        uint32_t rem = (uint32_t)k - n_sure;          // 1 <= rem <= n_cand
        bool done = false;
        // radix passes over the low key bits: [20:10], then [9:0]
        for (int stage = 0; stage < 2 && !done; ++stage) {
            const int nlo = stage == 0 ? 10 : 0;
            const int nb = stage == 0 ? 11 : 10;
            const int nbins = 1 << nb;
            __syncthreads();
            for (int i = tid; i < nbins; i += 256) sh_hist[i] = 0u;
            __syncthreads();
            for (uint32_t i = tid; i < n_cand; i += 256) {
                const uint32_t key = cand[i].x;
                if ((key >> (nlo + nb)) == P) atomicAdd(&sh_hist[(key >> nlo) & (nbins - 1)], 1u);
            }
            __syncthreads();
            find_rank_bin<true>(sh_hist, nbins, rem, sh_res, sh_scan);
            const int t = sh_res[0];
            rem -= sh_res[1];
            P = (P << nb) | (uint32_t)t;
            lo = nlo;
            done = sh_hist[t] == rem;
        }
        if (!done) {
            // equal keys straddle the cut: keep the `rem` lowest columns of key P
            uint32_t cp = 0;
            for (int stage = 0; stage < 3; ++stage) {
                const int clo = stage == 0 ? 20 : (stage == 1 ? 10 : 0);
                const int nb = stage == 0 ? 11 : 10;
                const int nbins = 1 << nb;
                __syncthreads();
                for (int i = tid; i < nbins; i += 256) sh_hist[i] = 0u;
                __syncthreads();
                for (uint32_t i = tid; i < n_cand; i += 256) {
                    const uint2 it = cand[i];
                    if (it.x == P && (it.y >> (clo + nb)) == cp)
                        atomicAdd(&sh_hist[(it.y >> clo) & (nbins - 1)], 1u);
                }
                __syncthreads();
                find_rank_bin<false>(sh_hist, nbins, rem, sh_res, sh_scan);
                const int t = sh_res[0];
                rem -= sh_res[1];
                cp = (cp << nb) | (uint32_t)t;
                if (sh_hist[t] == rem) {
                    cstar = ((cp + 1u) << clo) - 1u;
                    break;
                }
            }
        }
    }

    // gather the winners: all sure entries plus the selected candidates
    if (tid == 0) sh_count = 0u;
    __syncthreads();
    for (uint32_t i = tid; i < n_sure; i += 256) {
        const uint2 it = sure[i];
        const uint32_t pos = atomicAdd(&sh_count, 1u);
        if (pos < (uint32_t)kMaxK)
            sh_out[pos] = ((unsigned long long)it.x << 32) | (unsigned long long)(~it.y);
    }
    if (T >= 0) {
        for (uint32_t i = tid; i < n_cand; i += 256) {
            const uint2 it = cand[i];
            const uint32_t hi = it.x >> lo;
            if (hi > P || (hi == P && it.y <= cstar)) {
                const uint32_t pos = atomicAdd(&sh_count, 1u);
                if (pos < (uint32_t)kMaxK)
                    sh_out[pos] = ((unsigned long long)it.x << 32) | (unsigned long long)(~it.y);
            }
        }
    }
    __syncthreads();
    const uint32_t count = min(sh_count, (uint32_t)k);
    int kp = 1;
    while (kp < (int)count) kp <<= 1;
    for (int i = (int)count + tid; i < kp; i += 256) sh_out[i] = 0ull;   // sorts last
    __syncthreads();

    // bitonic sort, descending composite (key desc, column asc)
    for (int size = 2; size <= kp; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < (kp >> 1); i += 256) {
                const int pos = 2 * i - (i & (stride - 1));
                const int par = pos + stride;
                const unsigned long long x = sh_out[pos], y = sh_out[par];
                const bool desc = (pos & size) == 0;
                if (desc ? (x < y) : (x > y)) {
                    sh_out[pos] = y;
                    sh_out[par] = x;
                }
            }
            __syncthreads();
        }
    }

    int32_t *oc = a.out_col + (int64_t)b * k;
    float *ov = a.out_val ? a.out_val + (int64_t)b * k : nullptr;
    for (int i = tid; i < k; i += 256) {
        int32_t c = -1;
        float v = -__builtin_inff();
        if (i < (int)count) {
            const unsigned long long x = sh_out[i];
            const uint32_t col = ~(uint32_t)(x & 0xFFFFFFFFull);
            v = key_value((uint32_t)(x >> 32));
            c = (int32_t)col;
            if (a.map_entries && a.chunk_ids) {
                const int32_t beta = a.chunk_ids[(int64_t)b * a.max_chunks + c / kBlock];
                c = beta * kBlock + c % kBlock;
            }
        }
        oc[i] = c;
        if (ov) ov[i] = v;
    }
}

unsigned grid_1d(int64_t n, int per) {
    int64_t g = (n + per - 1) / per;
    if (g < 1) g = 1;
    if (g > 65535) g = 65535;
    return (unsigned)g;
}

}  // namespace

hipError_t launch_topk_init(const TopkArgs &a, hipStream_t s) {
    const int64_t n = (int64_t)a.B * (kHistBins + kCounters);
    hipLaunchKernelGGL(topk_init_kernel, dim3(grid_1d(n, 256 * 4)), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_topk_hist(const TopkArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(topk_hist_kernel, dim3((unsigned)((int64_t)a.B * a.parts)), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_topk_select(const TopkArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(topk_select_kernel, dim3((unsigned)((int64_t)a.B * a.parts)), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_topk_final(const TopkArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(topk_final_kernel, dim3((unsigned)a.B), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace idx
