// Level-1 resident-set selection for gfx950: the page pass between the
// per-layer scoring (score kernel, sigmoid output) and the top-KMAX page
// selection (segment top-k kernel) ("FlashMemory-DeepSeek-V4" README,
// sections "Two-level recall algorithm" and "Joint checkpoint + ensemble";
// KMAX pages of 64 entries per request, section "Quick start").
//
// A wave takes four consecutive 64-entry pages: lane l reads entries
// 4l .. 4l + 3 of the 256 (one 16-byte load per layer), ensembles them (max,
// or the binary32 sum in layer order divided by L) and counts those at or
// above the threshold; a DPP row (16 lanes) covers one page, so four row
// rotations sum the page's density.  The page's key for the selection orders
// pages by (forced, density, lower page first) and is exact in binary32:
//     forced (sink or recent page)       (kMaxDensity + 1) * 2^17 + (2^17 - 1 - p)
//     density d > 0                      d * 2^17 + (2^17 - 1 - p)
//     otherwise (or past the history)    -inf
// so that every key of a row is distinct and the top-k's value-linear
// histogram separates them (a +inf or integer-only key would put whole tie
// groups in one bin).  Rows of more than 2^17 pages use keys d and +inf
// instead, which select the same pages through the top-k's own tie rule.
#include <hip/hip_runtime.h>

#include "../../include/idx.h"
#include "idx_device.h"
#include "idx_internal.h"
#include "idx_level1.h"

namespace idx {
namespace {

constexpr int kPageWaves = 4;
constexpr int kPagesPerWave = 4;
constexpr int kPageBits = 17;

// The value of the lane N places further along this lane's 16-lane DPP row.
template <int N>
__device__ __forceinline__ int row_ror(int x) {
    return __builtin_amdgcn_update_dpp(0, x, 0x120 + N, 0xF, 0xF, false);
}

__global__ __launch_bounds__(64 * kPageWaves) void page_kernel(PageArgs a) {
    const int b = blockIdx.y;
    const int lane = threadIdx.x % 64;
    const int p0 = (blockIdx.x * kPageWaves + threadIdx.x / 64) * kPagesPerWave;
    if (p0 >= a.n_pages) return;                      // uniform per wave
    const int hist = max(0, min(a.limits[b], a.n_cols));
    const int P = (hist + kBlock - 1) / kBlock;
    const int p = p0 + lane / 16;                      // this lane's page
    const int e0 = p0 * kBlock + 4 * lane;             // its first entry
    int count = 0;
    if (e0 < hist) {
        const float *row = a.scores + (int64_t)b * a.ld + e0;
        float s[4];
        // the four entries are in bounds of the row stride (ld is a multiple
        // of 64); entries past hist are not counted
        float4 x = *reinterpret_cast<const float4 *>(row);
        s[0] = x.x; s[1] = x.y; s[2] = x.z; s[3] = x.w;
        for (int l = 1; l < a.L; ++l) {
            x = *reinterpret_cast<const float4 *>(row + (int64_t)l * a.layer_stride);
            const float y[4] = {x.x, x.y, x.z, x.w};
            if (a.ensemble == IDX_ENSEMBLE_MAX) {
#pragma unroll
                for (int i = 0; i < 4; ++i) s[i] = y[i] > s[i] ? y[i] : s[i];
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) s[i] += y[i];
            }
        }
        if (a.ensemble == IDX_ENSEMBLE_MEAN) {
#pragma unroll
            for (int i = 0; i < 4; ++i) s[i] = s[i] / (float)a.L;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) count += (e0 + i < hist && s[i] >= a.threshold) ? 1 : 0;
    }
    count += row_ror<8>(count);
    count += row_ror<4>(count);
    count += row_ror<2>(count);
    count += row_ror<1>(count);
    if (lane % 16 == 0 && p < a.n_pages) {
        const bool forced = p < P && (p < a.n_sink || p >= P - a.n_recent);
        float key = -__builtin_inff();
        if (a.n_pages <= (1 << kPageBits)) {
            const int tie = (1 << kPageBits) - 1 - p;
            if (forced) key = (float)((kBlock + 1) * (1 << kPageBits) + tie);
            else if (p < P && count > 0) key = (float)(count * (1 << kPageBits) + tie);
        } else {
            if (forced) key = __builtin_inff();
            else if (p < P && count > 0) key = (float)count;
        }
        a.page_keys[(int64_t)b * a.ldp + p] = key;
    }
}

// One 1024-thread workgroup per row, four pages per thread and chunk: the
// selection is latency-bound on a few workgroups, so short per-thread chains
// beat more loads in flight per thread (16 pages on 256 threads took 40% longer).
constexpr int kSelThreads = 1024;
constexpr int kSelPer = 4;                            // consecutive pages per thread and chunk
constexpr int kForcedRank = kBlock + 1;               // above every density

// Rank of page p of row b for the selection: kForcedRank for a sink or
// recent page, else its density (entries below the history selected in some
// layer), 0 past the history.
__device__ __forceinline__ int page_rank(const PageArgs &a, int b, int p, int hist, int P) {
    if (p >= P) return 0;
    if (p < a.n_sink || p >= P - a.n_recent) return kForcedRank;
    uint64_t m = 0;
    for (int l = 0; l < a.L; ++l) {
        const uint32_t *row = a.bits + ((int64_t)l * a.B + b) * a.bits_ld;
        m |= (uint64_t)row[2 * p] | ((uint64_t)row[2 * p + 1] << 32);
    }
    const int valid = min(hist - p * kBlock, kBlock);
    if (valid < kBlock) m &= (1ull << valid) - 1;
    return __popcll(m);
}

// Exclusive prefix of v over the workgroup (kSelThreads threads); *total gets
// the sum.
__device__ __forceinline__ uint32_t block_excl(uint32_t v, uint32_t *sh, uint32_t *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t incl = wave_scan(v);
    if (lane == 63) sh[wave] = incl;
    __syncthreads();
    uint32_t add = 0, all = 0;
    for (int i = 0; i < kSelThreads / 64; ++i) {
        add += i < wave ? sh[i] : 0u;
        all += sh[i];
    }
    __syncthreads();
    *total = all;
    return incl - v + add;
}

// The Level-1 selection of one row from the selection bits: forced pages,
// then the densest, equal densities to the lower page, at most kmax, written
// in ascending page order with -1 after the last (the order and padding of
// the page top-k over the page keys).  Densities are integers 0..64, so a
// histogram of the ranks finds the cut: every page above the cut rank is
// kept, and at the cut rank the lowest `need` pages.  The first pass reads
// the bits in coalesced order (thread t: pages t, t + kSelThreads, ...) and keeps
// each page's rank in LDS for rows of up to kSelCap pages; longer rows
// recompute the ranks in the second pass.
constexpr int kSelCap = 16384;

__global__ __launch_bounds__(kSelThreads) void select_bits_kernel(PageArgs a) {
    __shared__ uint32_t sh_hist[kForcedRank + 1];
    __shared__ uint32_t sh_scan[kSelThreads / 64];
    __shared__ uint8_t sh_rank[kSelCap];
    __shared__ int32_t sh_cut, sh_need;
    const int b = blockIdx.x;
    const int hist = max(0, min(a.limits[b], a.n_cols));
    const int P = min((hist + kBlock - 1) / kBlock, a.n_pages);
    const bool cached = P <= kSelCap;
    for (int i = threadIdx.x; i <= kForcedRank; i += kSelThreads) sh_hist[i] = 0u;
    __syncthreads();
    // pages t + kSelThreads k (k < kSelPer) of each chunk: the chunk's loads of
    // one layer all in flight at once
    for (int base = 0; base < P; base += kSelThreads * kSelPer) {
        uint64_t m[kSelPer];
#pragma unroll
        for (int k = 0; k < kSelPer; ++k) m[k] = 0;
        // four layers' loads at a time (a layer past L reads layer L - 1 again)
        for (int l0 = 0; l0 < a.L; l0 += 4) {
            uint2 x[4][kSelPer];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int l = min(l0 + j, a.L - 1);
                const uint2 *row = reinterpret_cast<const uint2 *>(a.bits + ((int64_t)l * a.B + b) * a.bits_ld);
#pragma unroll
                for (int k = 0; k < kSelPer; ++k) {
                    const int p = min(base + (int)threadIdx.x + kSelThreads * k, P - 1);
                    x[j][k] = row[p];
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int k = 0; k < kSelPer; ++k) m[k] |= (uint64_t)x[j][k].x | ((uint64_t)x[j][k].y << 32);
        }
#pragma unroll
        for (int k = 0; k < kSelPer; ++k) {
            const int p = base + (int)threadIdx.x + kSelThreads * k;
            if (p < P) {
                int r;
                if (p < a.n_sink || p >= P - a.n_recent) {
                    r = kForcedRank;
                } else {
                    const int valid = min(hist - p * kBlock, kBlock);
                    r = __popcll(valid < kBlock ? m[k] & ((1ull << valid) - 1) : m[k]);
                }
                if (cached) sh_rank[p] = (uint8_t)r;
                atomicAdd(&sh_hist[r], 1u);
            }
        }
    }
    if (threadIdx.x == 0) {
        sh_cut = 0;                                    // no cut: every page of rank >= 1 fits
        sh_need = 0;
    }
    __syncthreads();
    // the cut: the rank r >= 1 at which the pages of higher rank number fewer
    // than kmax and those of rank >= r at least kmax, from a scan of the
    // histogram in descending rank over the first two waves (thread i: rank
    // kForcedRank - i)
    if (threadIdx.x < 128) {
        const int r = kForcedRank - (int)threadIdx.x;
        const uint32_t v = r >= 1 ? sh_hist[r] : 0u;
        uint32_t incl = wave_scan(v);
        if ((threadIdx.x & 63) == 63) sh_scan[threadIdx.x >> 6] = incl;
        __syncthreads();
        if (threadIdx.x >= 64) incl += sh_scan[0];
        const uint32_t before = incl - v;
        if (r >= 1 && before < (uint32_t)a.kmax && incl >= (uint32_t)a.kmax) {
            sh_cut = r;
            sh_need = a.kmax - (int)before;
        }
    } else {
        __syncthreads();                               // the other waves' half of the barrier above
    }
    __syncthreads();
    const int cut = sh_cut, need = sh_need;
    int32_t *out = a.out_pages + (int64_t)b * a.kmax;
    uint32_t kept = 0, seen_at_cut = 0;
    for (int base = 0; base < P; base += kSelThreads * kSelPer) {
        int rank[kSelPer];
        uint32_t n_at = 0;
#pragma unroll
        for (int i = 0; i < kSelPer; ++i) {
            const int p = base + (int)threadIdx.x * kSelPer + i;
            rank[i] = p >= P ? 0 : cached ? (int)sh_rank[p] : page_rank(a, b, p, hist, P);
            n_at += (cut > 0 && rank[i] == cut) ? 1u : 0u;
        }
        uint32_t at_total;
        uint32_t at = seen_at_cut + block_excl(n_at, sh_scan, &at_total);
        uint32_t take = 0;                             // bit i: page i of this thread is kept
        uint32_t n_keep = 0;
#pragma unroll
        for (int i = 0; i < kSelPer; ++i) {
            bool k = rank[i] > cut;
            if (cut > 0 && rank[i] == cut) k = at++ < (uint32_t)need;
            take |= k ? 1u << i : 0u;
            n_keep += k ? 1u : 0u;
        }
        uint32_t keep_total;
        uint32_t pos = kept + block_excl(n_keep, sh_scan, &keep_total);
#pragma unroll
        for (int i = 0; i < kSelPer; ++i)
            if (take & (1u << i)) {
                if (pos < (uint32_t)a.kmax) out[pos] = base + (int)threadIdx.x * kSelPer + i;
                ++pos;
            }
        kept += keep_total;
        seen_at_cut += at_total;
    }
    for (int i = (int)kept + (int)threadIdx.x; i < a.kmax; i += kSelThreads) out[i] = -1;
    if (threadIdx.x == 0 && a.out_count) a.out_count[b] = (int32_t)min(kept, (uint32_t)a.kmax);
}

}  // namespace

hipError_t launch_select_bits(const PageArgs &a, hipStream_t s) {
    if (a.B <= 0) return hipSuccess;
    if (!a.bits || a.ensemble != IDX_ENSEMBLE_MAX || a.bits_ld < 2 * (int64_t)a.n_pages || a.kmax < 1 ||
        !a.out_pages)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(select_bits_kernel, dim3((unsigned)a.B), dim3(kSelThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_pages(const PageArgs &a, hipStream_t s) {
    if (a.B <= 0 || a.n_pages <= 0) return hipSuccess;
    const int per_group = kPageWaves * kPagesPerWave;
    const dim3 grid((unsigned)((a.n_pages + per_group - 1) / per_group), (unsigned)a.B);
    hipLaunchKernelGGL(page_kernel, grid, dim3(64 * kPageWaves), 0, s, a);
    return hipGetLastError();
}

}  // namespace idx
