// Per-row top-k selection for gfx950: the k largest logits of each query row
// ("FlashMemory-DeepSeek-V4" README, "Two-level recall algorithm": Level 2
// keeps the top-512 of the resident logits, the rest being -inf).
//
// One workgroup selects the top-k of one segment of a row.  Each thread holds
// a contiguous run of the segment's order-preserving keys (idx_device.h) in
// registers for the whole kernel, so after the single global read the passes
// below are register work plus a few LDS histograms and block scans; nothing
// needs a global atomic or a zeroed workspace:
//   1. load the keys and reduce the min and max of the selectable values;
//   2. histogram the values into 2048 bins LINEAR in value between min and
//      max (few LDS atomic collisions, unlike bins of the float's top bits,
//      which put most logits of a row into a handful of bins), and find the
//      bin t holding the k-th largest value and the selectable count;
//   3. copy bin t's members to LDS (positions from a block scan) and find the
//      exact k-th largest key among them: one wave ranks up to 64 members
//      against each other; larger bins take radix passes over their keys
//      (bits 31:21, 20:10, 9:0);
//   4. write the winners (keys above the k-th, plus as many copies of it as
//      needed, lowest columns first) in column order: one block scan of the
//      threads' winner and tie counts gives every thread its output offset.
// A row longer than one segment is split into parts; each part keeps its own
// top-k (key, column) list and the lists of a row are merged the same way
// (concatenated in part order, so column order holds): by the row's last part
// in the same launch when the lists fit, else by further launches.
// Long segments (at least 16 items per thread) with k <= 640 first try a
// threshold sampled from one value per thread: the items at or above it are
// counted, and when they number between k and 2048 they are compacted into
// LDS and steps 2-4 run on them alone (select_sampled); the parts it leaves
// unsettled are re-run by a second launch of the path above.
// The result is deterministic and ordered by column.
#include <algorithm>

#include "idx_device.h"
#include "idx_internal.h"

namespace idx {
namespace {

constexpr int kBins = 2048;

// Same pattern for max and min: lane 63 ends with the wave's result.
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
    v = max(v, dpp<0x111, 0xF>(v));
    v = max(v, dpp<0x112, 0xF>(v));
    v = max(v, dpp<0x114, 0xF>(v));
    v = max(v, dpp<0x118, 0xF>(v));
    v = max(v, dpp<0x142, 0xA>(v));
    v = max(v, dpp<0x143, 0xC>(v));
    return v;
}
__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
    v = min(v, dpp<0x111, 0xF>(v, ~0u));
    v = min(v, dpp<0x112, 0xF>(v, ~0u));
    v = min(v, dpp<0x114, 0xF>(v, ~0u));
    v = min(v, dpp<0x118, 0xF>(v, ~0u));
    v = min(v, dpp<0x142, 0xA>(v, ~0u));
    v = min(v, dpp<0x143, 0xC>(v, ~0u));
    return v;
}

// Inclusive scan over the NT threads of the workgroup; `sh` has NT/64 words
// and must not be written again before every thread has passed another
// barrier.
template <int NT>
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t *sh) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_scan(v);
    if (NT == 64) return v;
    if (lane == 63) sh[wave] = v;
    lds_barrier();
    uint32_t add = 0;
    for (int i = 0; i < wave; ++i) add += sh[i];
    return v + add;
}

// block_scan that also gives every thread the workgroup's total.
template <int NT>
__device__ __forceinline__ uint32_t block_scan_total(uint32_t v, uint32_t *sh, uint32_t &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_scan(v);
    if (lane == 63) sh[wave] = v;
    lds_barrier();
    uint32_t add = 0, all = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
        const uint32_t t = sh[i];
        add += i < wave ? t : 0u;
        all += t;
    }
    total = all;
    return v + add;
}

// Bin t of an LDS histogram `h` (nbins a multiple of NT) with
// count(bins > t) < need <= count(bins >= t).  res[0] = t (-1 if the total is
// below need), res[1] = count(bins > t), res[2] = the total.  All NT threads
// call it.
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
    if (tid == NT - 1) {
        res[2] = (int32_t)incl;                       // the histogram's total
        if (incl < need) res[1] = incl;
    }
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
    lds_barrier();
}

// The next binary32 value above a finite x.
__device__ __forceinline__ float next_up(float x) {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) == 0u) return __uint_as_float(1u);          // +-0 -> smallest positive
    return __uint_as_float(x > 0.f ? u + 1u : u - 1u);
}

// LDS scratch of one selection by NT threads.  The histogram has 32 extra
// bins past kBins that absorb non-selectable items, so the histogram's
// atomics need no branch.
template <int NT, int CAND>
struct SelScratch {
    uint32_t cand[CAND];          // keys of the cut bin's members, when <= 64
    uint32_t hist[kBins + 32];
    uint32_t scan_a[NT / 64], scan_b[NT / 64];
    uint32_t kmin[NT / 64], kmax[NT / 64];
    int32_t res[3];
    uint32_t cut[2];
    uint32_t ncand;
    uint32_t flag;
};

// What find_cut expects zeroed (the histogram and the member count); it sees
// these stores through its first barrier.
template <int NT, int CAND>
__device__ __forceinline__ void sel_reset(SelScratch<NT, CAND> &sh) {
    for (int i = threadIdx.x; i < kBins + 32; i += NT) sh.hist[i] = 0u;
    if (threadIdx.x == 0) sh.ncand = 0u;
}

// Bins of a thread's PER slots, kept from the histogram pass for the passes
// after it: one per register up to 16 slots, else two 16-bit bins per
// register (bins < 2080).
template <int PER>
struct SlotBins {
    static constexpr bool kWide = PER <= 16;
    uint32_t r[kWide ? PER : (PER + 1) / 2];
    __device__ __forceinline__ uint32_t get(int j) const {
        if (kWide) return r[j];
        return (j & 1) ? r[j >> 1] >> 16 : r[j >> 1] & 0xFFFFu;
    }
    __device__ __forceinline__ void set(int j, uint32_t bn) {
        if (kWide)
            r[j] = bn;
        else if (j & 1)
            r[j >> 1] |= bn << 16;
        else
            r[j >> 1] = bn;
    }
};

// The map v -> fma(v, scale, off) that spreads the values between the keys
// kmn and kmax over kBins bins, linear in value (scale 0 when the range is
// empty or not finite: every value in bin 0).
__device__ __forceinline__ void linear_bins(uint32_t kmn, uint32_t kmx, float &scale, float &off) {
    const float vmin = key_value(kmn), vmax = key_value(kmx);
    scale = 0.f;
    const float range = vmax - vmin;
    if (range > 0.f && range < __builtin_inff()) scale = (float)kBins / range;
    if (!(scale < __builtin_inff())) scale = 0.f;
    off = -vmin * scale;
    // off is -vmin*scale rounded, so fma(vmin, scale, off) is that rounding's
    // error (exact, at most half an ulp of off); when it is negative, off
    // moves up one ulp so that no item's bin is negative -- with values far
    // from 0 in a narrow range the error exceeds 1, and a negative bin would
    // wrap past the top bin below
    if (fmaf(vmin, scale, off) < 0.f) off = next_up(off);
}

// Where the k-th largest selectable item lies after the value histogram:
// bin cbin, with `above` selectable items in higher bins and n_in_bin in it;
// total = the selectable count.  every: every selectable item wins (total
// <= k, none selectable included), and cbin, above and n_in_bin mean
// nothing.
struct CutBin {
    uint32_t cbin, above, n_in_bin, total;
    bool every;
};

// Steps 1-3 of find_cut over the items the workgroup holds in registers;
// bins gets each slot's bin (selectable items below kBins, the others at or
// above it), set whenever total > 0.  All threads call it, after sel_reset.
template <int NT, int PER, int CAND, bool HAVE_V>
__device__ __forceinline__ CutBin hist_cut(const uint32_t (&key)[PER], uint32_t k, SelScratch<NT, CAND> &sh,
                                           SlotBins<PER> &bins, const float *val) {
    constexpr int kW = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // 1. integer min/max of the order-preserving keys
    uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        kmn = min(kmn, key[j] ? key[j] : 0xFFFFFFFFu);
        kmx = max(kmx, key[j]);
    }
    kmn = wave_min(kmn);
    kmx = wave_max(kmx);
    if (lane == 63) {
        sh.kmin[wave] = kmn;
        sh.kmax[wave] = kmx;
    }
    lds_barrier();
    kmn = 0xFFFFFFFFu;
    kmx = 0u;
    for (int w = 0; w < kW; ++w) {
        kmn = min(kmn, sh.kmin[w]);
        kmx = max(kmx, sh.kmax[w]);
    }
    CutBin c{0u, 0u, 0u, 0u, true};
    if (kmx == 0u) return c;                          // uniform: nothing selectable

    // 2. value-linear bins (monotone in value); other items go to the extra
    // bins, 32 of them so that a wave's lanes hit distinct LDS banks
    float scale, off;
    linear_bins(kmn, kmx, scale, off);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const uint32_t kj = key[j];
        // fma(v, scale, off) is monotone in v like (v - vmin)*scale and at
        // least fma(vmin, scale, off) >= 0; it only has to be the same
        // function in every pass
        const float v = HAVE_V ? val[j] : key_value(kj);
        const int x = __float2int_rz(fmaf(v, scale, off));                // >= 0 (NaN -> 0)
        const uint32_t bn = kj ? min((uint32_t)x, (uint32_t)(kBins - 1)) : (uint32_t)(kBins + (lane & 31));
        bins.set(j, bn);
        atomicAdd(&sh.hist[bn], 1u);
    }
    lds_barrier();
    // 3.
    find_from_top<NT>(sh.hist, kBins, k, sh.res, sh.scan_a);
    c.total = (uint32_t)sh.res[2];
    if (c.total <= k) return c;                       // uniform: every selectable item wins
    c.every = false;
    c.cbin = (uint32_t)sh.res[0];
    c.above = (uint32_t)sh.res[1];
    c.n_in_bin = sh.hist[c.cbin];
    return c;
}

// Step 4 of find_cut: the exact k-th largest key among the members of bin
// c.cbin (the slots j with bins.get(j) == c.cbin) and how many of its copies
// win.  All threads call it, with c.every false.
template <int NT, int PER, int CAND>
__device__ __forceinline__ void resolve_cut(const uint32_t (&key)[PER], const SlotBins<PER> &bins, const CutBin &c,
                                            uint32_t k, SelScratch<NT, CAND> &sh, uint32_t &kstar,
                                            uint32_t &need_ties) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t rem = k - c.above;
    const uint32_t n_in_bin = c.n_in_bin;
    const auto in_cut_bin = [&](int j) { return bins.get(j) == c.cbin; };
    // few members: their keys go to LDS (in any order) and one wave ranks
    // them against each other
    if (n_in_bin <= 64u) {
#pragma unroll
        for (int j = 0; j < PER; ++j)
            if (in_cut_bin(j)) sh.cand[atomicAdd(&sh.ncand, 1u)] = key[j];
        lds_barrier();
        if (wave == 0) {
            const uint32_t my = lane < (int)n_in_bin ? sh.cand[lane] : 0u;
            uint32_t greater = 0, equal = 0;
            for (uint32_t j = 0; j < n_in_bin; ++j) {
                const uint32_t other = (uint32_t)__builtin_amdgcn_readlane((int)my, (int)j);
                greater += other > my;
                equal += other == my;
            }
            if (lane < (int)n_in_bin && greater < rem && rem <= greater + equal) {
                sh.cut[0] = my;                      // every such lane holds the same key
                sh.cut[1] = rem - greater;
            }
        }
        lds_barrier();
        kstar = sh.cut[0];
        need_ties = sh.cut[1];
        return;
    }
    // many members: radix passes over the keys of the cut bin, straight from
    // registers (bits 31:21, 20:10, 9:0)
    uint32_t prefix = 0u;
    for (int stage = 0; stage < 3; ++stage) {
        const int hi = stage == 0 ? 32 : (stage == 1 ? 21 : 10);
        const int lo = stage == 0 ? 21 : (stage == 1 ? 10 : 0);
        lds_barrier();
        for (int i = tid; i < kBins; i += NT) sh.hist[i] = 0u;
        lds_barrier();
        const uint32_t mask = (1u << (hi - lo)) - 1u;
        // the cut bin as a value the compiler cannot carry across stages, so
        // the slots' membership is tested again in each stage rather than
        // held in scalar registers (one 64-bit mask per slot)
        uint32_t cb = c.cbin;
        asm volatile("" : "+v"(cb));
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const uint32_t kk = key[j];
            if (bins.get(j) == cb && (hi == 32 || (kk >> hi) == prefix)) atomicAdd(&sh.hist[(kk >> lo) & mask], 1u);
        }
        lds_barrier();
        find_from_top<NT>(sh.hist, kBins, rem, sh.res, sh.scan_a);
        rem -= (uint32_t)sh.res[1];
        prefix = (hi == 32 ? 0u : (prefix << (hi - lo))) | (uint32_t)sh.res[0];
    }
    kstar = prefix;
    need_ties = rem;
}

// The exact k-th largest key (kstar) among the items the workgroup holds in
// registers (thread t: key[0..PER) of a column-ordered sequence; key 0 = not
// selectable), how many of its copies win (need_ties, lowest columns first)
// and the number of selectable items (total).  kstar = 0 when every
// selectable item wins.  All threads call it, after sel_reset.  With
// HAVE_V, val[j] is the float whose order key is key[j] (saves decoding it).
//   1. key range of the selectable items;
//   2. histogram of 2048 bins linear in value between min and max;
//   3. the bin t holding the k-th largest value (and the selectable count);
//   4. t's members go to LDS; one wave ranks up to 64 of them against each
//      other, larger bins take radix passes over their keys (bits 31:21,
//      20:10, 9:0).
template <int NT, int PER, int CAND, bool HAVE_V = false>
__device__ __forceinline__ void find_cut(const uint32_t (&key)[PER], uint32_t k, SelScratch<NT, CAND> &sh,
                                         uint32_t &kstar, uint32_t &need_ties, uint32_t &total,
                                         const float *val = nullptr) {
    SlotBins<PER> bins;
    const CutBin c = hist_cut<NT, PER, CAND, HAVE_V>(key, k, sh, bins, val);
    total = c.total;
    kstar = 0u;
    need_ties = 0u;
    if (!c.every) resolve_cut<NT, PER, CAND>(key, bins, c, k, sh, kstar, need_ties);
}

// Thresholds for the items of a long segment, from one sample per thread:
// the samples' histogram linear in value between their min and max, and
// for a rank r the lower edge of the bin holding the r-th largest
// selectable sample.  The items at or above such a threshold number about
// r times the items per sample; the caller counts them exactly and only
// uses a threshold whose count lies between k and its capacity.
struct SampleMap {
    float scale, off;     // linear_bins of the samples (scale 0: no selectable sample, or one value)
    float vmin;           // the smallest selectable sample
    bool any;             // a selectable sample exists
};

// The samples' histogram (s: this thread's sample).  All threads call it,
// with the histogram zeroed; they all get the same map, and the histogram
// holds the samples' counts afterwards.
template <int NT, int CAND>
__device__ SampleMap sample_hist(float s, SelScratch<NT, CAND> &sh) {
    constexpr int kW = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t sk = order_key(s);
    uint32_t kmn = wave_min(sk ? sk : 0xFFFFFFFFu), kmx = wave_max(sk);
    if (lane == 63) {
        sh.kmin[wave] = kmn;
        sh.kmax[wave] = kmx;
    }
    lds_barrier();
    kmn = 0xFFFFFFFFu;
    kmx = 0u;
    for (int w = 0; w < kW; ++w) {
        kmn = min(kmn, sh.kmin[w]);
        kmx = max(kmx, sh.kmax[w]);
    }
    SampleMap m{0.f, 0.f, 0.f, kmx != 0u};
    if (!m.any) return m;                             // uniform: no selectable sample
    linear_bins(kmn, kmx, m.scale, m.off);
    m.vmin = key_value(kmn);
    const int x = __float2int_rz(fmaf(s, m.scale, m.off));
    const uint32_t bn = sk ? min((uint32_t)x, (uint32_t)(kBins - 1)) : (uint32_t)(kBins + (lane & 31));
    atomicAdd(&sh.hist[bn], 1u);
    lds_barrier();
    return m;
}

// The threshold for rank r on the samples' histogram: -FLT_MAX (every
// selectable item) when fewer than r samples are selectable.  All threads
// call it and get the same value.
template <int NT, int CAND>
__device__ float sample_cut(uint32_t r, const SampleMap &m, SelScratch<NT, CAND> &sh) {
    if (!m.any) return -__FLT_MAX__;
    find_from_top<NT>(sh.hist, kBins, r, sh.res, sh.scan_a);
    if (sh.res[0] < 0) return -__FLT_MAX__;           // uniform: fewer than r selectable samples
    // fma(v, scale, off) >= cbin from about here on; any value serves, the
    // caller's count is exact
    return m.scale > 0.f ? ((float)sh.res[0] - m.off) / m.scale : m.vmin;
}

constexpr uint32_t kLoses = 0xFFFFFFFFu;              // position of a slot that does not win
constexpr uint32_t kDrop = 0x7FFFFFF0u;               // a byte offset every descriptor here rejects

__device__ __forceinline__ uint32_t byte_off(uint32_t pos, uint32_t size) {
    return pos == kLoses ? kDrop : pos * size;
}

// Output positions of a thread's register slots, visited in slot order:
// the keys above kstar plus the first need_ties keys equal to it win.
struct WinCursor {
    uint32_t p, tie_ord, kstar, need_ties;
    __device__ __forceinline__ uint32_t next(uint32_t key) {     // kLoses if it does not win
        bool win = key > kstar;
        if (kstar != 0u && key == kstar) win = tie_ord++ < need_ties;
        const uint32_t r = win ? p : kLoses;
        p += win;
        return r;
    }
};

// Winners numbered in column order from one block scan of packed
// (winners | ties << 16) per thread: sets the thread's cursor.  All threads
// call it; it leaves sh.scan_b in use until the next barrier.
template <int NT, int PER, int CAND>
__device__ __forceinline__ void scan_winners(const uint32_t (&key)[PER], uint32_t kstar, uint32_t need_ties,
                                             SelScratch<NT, CAND> &sh, WinCursor &cur) {
    uint32_t n_win = 0, n_tie = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        n_win += key[j] > kstar;
        n_tie += kstar != 0u && key[j] == kstar;
    }
    const uint32_t packed = n_win | (n_tie << 16);
    const uint32_t excl = block_scan<NT>(packed, sh.scan_b) - packed;
    cur.tie_ord = excl >> 16;
    cur.p = (excl & 0xFFFFu) + min(cur.tie_ord, need_ties);
    cur.kstar = kstar;
    cur.need_ties = need_ties;
}

// Final output of row b: the winners' logical entry ids (a column's chunk
// resolved through chunk_ids) and values at their positions, -1 / -inf in
// [count, k), and count itself when out_count is given.  The chunk loads and
// the id and value stores go through buffer descriptors, none behind a
// branch.
template <int NT, int PER, class ColOf>
__device__ __forceinline__ void write_final(const SegArgs &a, int b, WinCursor cur, const uint32_t (&key)[PER],
                                            ColOf col, uint32_t count) {
    const uint32_t k = (uint32_t)a.k;
    int32_t *oi = a.out_idx + (int64_t)b * k;
    float *ov = a.out_val ? a.out_val + (int64_t)b * k : nullptr;
    const __amdgpu_buffer_rsrc_t ir = make_rsrc(oi, k * 4u);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(ov ? (void *)ov : (void *)oi, ov ? k * 4u : 0u);
    // groups of up to 8 slots (a divisor of PER): their chunk lookups are in
    // flight together
    constexpr int kG = PER % 8 == 0 ? 8 : (PER % 4 == 0 ? 4 : (PER % 2 == 0 ? 2 : 1));
    static_assert(PER % kG == 0, "slot groups must tile the thread's slots");
#pragma unroll
    for (int g = 0; g < PER; g += kG) {
        uint32_t e[kG], pos[kG];
#pragma unroll
        for (int j = 0; j < kG; ++j) pos[j] = cur.next(key[g + j]);
        if (a.chunk_ids) {
            const __amdgpu_buffer_rsrc_t cr =
                make_rsrc(a.chunk_ids + (int64_t)b * a.max_chunks, (uint32_t)a.max_chunks * 4u);
#pragma unroll
            for (int j = 0; j < kG; ++j) {
                const uint32_t c = col(g + j);
                const uint32_t off = pos[j] == kLoses ? kDrop : (c >> a.chunk_shift) * 4u;
                e[j] = (__builtin_amdgcn_raw_buffer_load_b32(cr, off, 0, 0) << a.chunk_shift) |
                       (c & ((1u << a.chunk_shift) - 1u));
            }
#pragma unroll
            for (int j = 0; j < kG; ++j) {
                const uint32_t off = byte_off(pos[j], 4u);
                __builtin_amdgcn_raw_buffer_store_b32(e[j], ir, off, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(key_value(key[g + j])), vr, off, 0, 0);
            }
        } else {
            // few slots hold a winner: a slot no lane of the wave wins
            // issues no stores
#pragma unroll
            for (int j = 0; j < kG; ++j) {
                if (__any(pos[j] != kLoses)) {
                    const uint32_t off = byte_off(pos[j], 4u);
                    __builtin_amdgcn_raw_buffer_store_b32(col(g + j), ir, off, 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(key_value(key[g + j])), vr, off, 0, 0);
                }
            }
        }
    }
    for (uint32_t i = count + threadIdx.x; i < k; i += NT) {
        __builtin_amdgcn_raw_buffer_store_b32(0xFFFFFFFFu, ir, i * 4u, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(-__builtin_inff()), vr, i * 4u, 0, 0);
    }
    if (a.out_count && threadIdx.x == 0) a.out_count[b] = (int32_t)count;
}

// Merge lists: every list holds exactly lcap = k rounded up to even items,
// (key, column) pairs, the winners in column order followed by key 0 (never
// selectable), so the lists of a row form one contiguous run of memory, a
// reader needs no counts, and 16-byte accesses never straddle a list's end.
__host__ __device__ __forceinline__ uint32_t list_cap(uint32_t k) { return (k + 1u) & ~1u; }

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// COHERENT: the list is read by another workgroup of the same launch, so it
// is stored device-coherent (sc1) past the per-XCD L2s; the reader loads it
// the same way, and no L2 write-back or invalidate is needed.
template <int NT, int PER, bool COHERENT, class ColOf>
__device__ __forceinline__ void write_list(uint2 *dst, uint32_t lcap, WinCursor cur, const uint32_t (&key)[PER],
                                           ColOf col, uint32_t count) {
    constexpr int aux = COHERENT ? kDeviceCoherent : 0;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(dst, lcap * 8u);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const uint32_t pos = cur.next(key[j]);
        if (__any(pos != kLoses)) {                   // a slot no lane wins issues no store
            u32x2 v;
            v.x = key[j];
            v.y = col(j);
            __builtin_amdgcn_raw_buffer_store_b64(v, r, byte_off(pos, 8u), 0, aux);
        }
    }
    const u32x2 zero = {0u, 0u};
    for (uint32_t i = count + threadIdx.x; i < lcap; i += NT) __builtin_amdgcn_raw_buffer_store_b64(zero, r, i * 8u, 0, aux);
}

// Items [i0, i0 + PER) of the n items at `src` as (key, column); items past
// n read as key 0.  Loads through a buffer descriptor, none behind a branch.
template <int PER, bool COHERENT>
__device__ __forceinline__ void load_items(const uint2 *src, int n, int i0, uint32_t (&key)[PER],
                                           uint32_t (&col)[PER]) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(src, (uint32_t)max(n, 0) * 8u);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (uint32_t)(i0 + j) * 8u, 0,
                                                             COHERENT ? kDeviceCoherent : 0);
        key[j] = v.x;
        col[j] = v.y;
    }
}

// One workgroup per (row, part).  LIST: the part merges lists of a previous
// launch.  MMUL > 0 (logits input only): after writing its own list, the
// last part of a row to finish (per-row arrival counter, zeroed by the score
// kernel) merges all of the row's lists, up to MMUL x CAP items, in the same
// launch.
// 512-thread workgroups over long segments are held to 128 VGPRs (four waves
// per SIMD) so that two share a CU: many rows then keep the CU busy while one
// workgroup sits in its barrier-separated, latency-bound phases.  The
// sampled-threshold kernels need fewer: at most 85 (three workgroups of 512
// threads per CU; 64, four per CU, spilled around the retried threshold and
// ran 15 % slower); 1024 threads: 128.
// Launch modes of the segment kernel (see topk_segment_kernel).
constexpr int kSegPlain = 0, kSegSampled = 1, kSegRerun = 2;

template <int CAP, bool LIST, int NT, int MMUL, int MODE>
constexpr int seg_waves_per_eu() {
    if (MODE == kSegSampled) return NT == 1024 ? 4 : 6;
    return !LIST && MMUL == 0 && NT == 512 && CAP / NT >= 16 ? 4 : 1;
}

// Compacted items after a sampled threshold (see select_sampled).
constexpr int kPreCap = kTopkPreCap;

// Logits of workgroup g's segment (row g / parts, part g % parts) as the
// bits of the values: thread t's slot j is segment column t * CAP / NT + j,
// -inf past the row's columns.
template <int CAP, int NT>
__device__ __forceinline__ void load_segment(const SegArgs &a, int g, uint32_t (&x)[CAP / NT],
                                             int tid = threadIdx.x) {
    constexpr int kPer = CAP / NT;
    const int b = g / a.parts;
    const int part = g - b * a.parts;
    const int i0 = tid * kPer;
    const int64_t col0 = (int64_t)part * CAP;
    const int ncols = a.row_cols ? min((int)a.row_cols[b], a.n_cols) : a.n_cols;
    const int n = (int)max<int64_t>(0, min<int64_t>(CAP, ncols - col0));
    const float *src = a.logits + (int64_t)b * a.ld + col0 + i0;
    if ((a.ld & 3) == 0 && (reinterpret_cast<uintptr_t>(a.logits) & 15) == 0 && i0 + kPer <= n) {
#pragma unroll
        for (int j = 0; j < kPer; j += 4) {
            const float4 f = *reinterpret_cast<const float4 *>(src + j);
            x[j] = __float_as_uint(f.x);
            x[j + 1] = __float_as_uint(f.y);
            x[j + 2] = __float_as_uint(f.z);
            x[j + 3] = __float_as_uint(f.w);
        }
    } else {
        // ragged or unaligned: dword loads at offsets clamped into the
        // segment, the slots past its end masked
        const __amdgpu_buffer_rsrc_t r = make_rsrc(src - i0, (uint32_t)n * 4u);
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const uint32_t y = __builtin_amdgcn_raw_buffer_load_b32(r, (uint32_t)max(0, min(i0 + j, n - 1)) * 4u, 0, 0);
            x[j] = i0 + j < n ? y : 0xFF800000u;
        }
    }
}

// Workgroup g's selection through a sampled threshold, over the values'
// bits in key[] (load_segment): the items at or above a threshold T from
// the samples (thread t's first slot) are counted exactly, and when there
// are at least k and at most kPreCap of them, every winner is among them (at
// least k items reach T, so the k-th largest does) -- as when T admits every
// selectable item and there are fewer than k (all of them win) -- so they are compacted
// into LDS in column order -- a count pass, a block scan and a writing
// pass, a few VALU operations per item -- and the exact selection runs on
// those few items (kPreCap / NT per thread).  The threshold aims at about
// 2 k items (at least 320, at most 60 % of the capacity): each sample
// stands for CAP / NT items; a count outside the bounds takes another rank
// on the same samples, up to three in all.  Other counts (values the samples misrepresent, many ties
// at T) leave the workgroup's redo flag set, and the re-run launched next
// over the same segments (kSegRerun) runs those parts alone.  Every barrier
// is an LDS-only one, so loads issued before the call stay in flight.
template <int CAP, int NT>
__device__ __forceinline__ void select_sampled(const SegArgs &a, int g, const uint32_t (&key)[CAP / NT],
                                               SelScratch<NT, 64> &sh, uint2 *sh_items) {
    constexpr int kPer = CAP / NT;
    constexpr int kPreCI = kPreCap / NT;
    const int tid = threadIdx.x;
    const int b = g / a.parts;
    const int part = g - b * a.parts;
    const uint32_t k = (uint32_t)a.k;
    const uint32_t lcap = list_cap(k);
    const int i0 = tid * kPer;
    const int64_t col0 = (int64_t)part * CAP;
    uint32_t kstar = 0u, need_ties = 0u, total;
    WinCursor cur;
    sel_reset(sh);
    const uint32_t target = min(max(2u * k, 320u), (uint32_t)(kPreCap * 3 / 5));
    const SampleMap smap = sample_hist<NT, 64>(__uint_as_float(key[0]), sh);
    // up to three thresholds: a rank whose count is too small or too large
    // bounds the next one (bisection once both bounds are known)
    uint32_t r = max(1u, (target + kPer - 1) / kPer), r_lo = 0, r_hi = 0;
    float T;
    uint32_t tot, pos;
    bool settled;
    for (int attempt = 0;; ++attempt) {               // uniform
        T = sample_cut<NT, 64>(r, smap, sh);
        uint32_t m = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) m += __uint_as_float(key[j]) >= T;
        pos = block_scan_total<NT>(m, sh.scan_b, tot) - m;
        // settled: k to kPreCap items, or every selectable item when there
        // are fewer than k (they all win)
        settled = tot <= (uint32_t)kPreCap && (tot >= k || T == -__FLT_MAX__);
        if (settled || attempt == 2) break;
        if (tot < k) r_lo = r; else r_hi = r;
        uint32_t r2;
        if (r_lo && r_hi)
            r2 = (r_lo + r_hi) / 2u;
        else if (tot > (uint32_t)kPreCap)
            r2 = max(1u, (uint32_t)((uint64_t)r * target / tot));
        else
            r2 = min((uint32_t)NT, (uint32_t)((uint64_t)r * target / max(tot, 1u)) + 1u);
        if (r2 == r) break;
        r = r2;
        lds_barrier();                                // the scan's words were read
    }
    if (settled) {                                    // uniform
        // the selection below starts from a zeroed histogram; the
        // samples' counts were last read before the scan's barrier
        sel_reset(sh);
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            if (__uint_as_float(key[j]) >= T) sh_items[pos++] = make_uint2(key[j], (uint32_t)(i0 + j));
        lds_barrier();
        // items tid * kPreCI ..: (value bits, segment column); none: key 0.
        // Their bins come from the samples' map (monotone in value; values
        // past the samples' range clamp to the end bins), so no second
        // min / max pass: the value histogram, the cut bin, then its exact
        // cut as in find_cut.
        uint32_t key1[kPreCI], cl[kPreCI];
        SlotBins<kPreCI> bin1;
#pragma unroll
        for (int i = 0; i < kPreCI; ++i) {
            const int x = tid * kPreCI + i;
            const uint2 it = x < (int)tot ? sh_items[x] : make_uint2(0xFF800000u, 0u);
            const float val = __uint_as_float(it.x);
            key1[i] = order_key(val);
            cl[i] = it.y;
            const int y = max(__float2int_rz(fmaf(val, smap.scale, smap.off)), 0);       // NaN (inf * 0) -> 0
            const uint32_t bn = key1[i] ? min((uint32_t)y, (uint32_t)(kBins - 1)) : (uint32_t)(kBins + (tid & 31));
            bin1.set(i, bn);
            atomicAdd(&sh.hist[bn], 1u);
        }
        lds_barrier();
        find_from_top<NT>(sh.hist, kBins, k, sh.res, sh.scan_a);
        total = tot;                                  // every compacted item is selectable
        if (tot > k) {                                // uniform
            CutBin c;
            c.cbin = (uint32_t)sh.res[0];
            c.above = (uint32_t)sh.res[1];
            c.n_in_bin = sh.hist[c.cbin];
            c.total = tot;
            c.every = false;
            resolve_cut<NT, kPreCI, 64>(key1, bin1, c, k, sh, kstar, need_ties);
        }
        scan_winners<NT, kPreCI>(key1, kstar, need_ties, sh, cur);
        const uint32_t count = min(total, k);
        const auto col1 = [&](int i) { return (uint32_t)(col0 + cl[i]); };
        if (a.out_list)
            write_list<NT, kPreCI, false>(a.out_list + ((int64_t)b * a.parts + part) * lcap, lcap, cur, key1,
                                          col1, count);
        else
            write_final<NT, kPreCI>(a, b, cur, key1, col1, count);
    }
    if (tid == 0) a.redo[g] = settled ? 0u : 1u;
}

// LDS items of seg_body's compaction.
template <int CAP, bool LIST, int NT, bool PRE>
constexpr int seg_items() { return PRE ? kPreCap : (!LIST && CAP / NT >= 16 ? 1024 : 1); }

// Workgroup g (row g / parts, part g % parts) of a top-k launch.  OPAQUE
// (a loop over parts): the thread index is hidden from the optimiser, which
// would otherwise hoist every slot's column out of the loop (registers).
template <int CAP, bool LIST, int NT, int MMUL, bool OPAQUE = false>
__device__ __forceinline__ void seg_body(const SegArgs &a, int g, SelScratch<NT, 64> &sh, uint2 *sh_items) {
    constexpr bool kFused = MMUL > 0;
    constexpr int kPer = CAP / NT;                    // items per thread
    constexpr int kMPer = kFused ? MMUL * kPer : kPer;    // merge items per thread
    // long segments of logits: the items that can still win are compacted
    // into LDS, a few per thread (see below)
    constexpr bool kCompact = !LIST && kPer >= 16;
    constexpr int kCI = 1024 / NT;                    // after the histogram: up to 1024 items in all
    static_assert(seg_items<CAP, LIST, NT, false>() >= (kCompact ? kCI * NT : 1), "LDS items");

    int tid = threadIdx.x;
    if constexpr (OPAQUE) asm volatile("" : "+v"(tid));
    const int b = g / a.parts;
    const int part = g - b * a.parts;
    const uint32_t k = (uint32_t)a.k;
    const uint32_t lcap = list_cap(k);
    const int i0 = tid * kPer;
    sel_reset(sh);                                    // while the loads are in flight

    // logits input: slot j holds column col0 + i0 + j; list input: col[j]
    uint32_t key[kPer];
    uint32_t col[LIST ? kPer : 1];
    float v[LIST ? 1 : kPer];                         // logits input: the loaded values
    const int64_t col0 = (int64_t)part * CAP;
    if constexpr (!LIST) {
        load_segment<CAP, NT>(a, g, key, tid);
#pragma unroll
        for (int j = 0; j < kPer; ++j) v[j] = __uint_as_float(key[j]);
#pragma unroll
        for (int j = 0; j < kPer; ++j) key[j] = order_key(v[j]);
    } else {
        // lists [G * part, G * part + G) of the row, G = CAP / in_cap
        const int G = CAP / a.in_cap;
        const int l0 = part * G;
        const int n = max(0, min(G, a.in_parts - l0)) * a.in_cap;
        load_items<kPer, false>(a.in_list + ((int64_t)b * a.in_parts + l0) * a.in_cap, n, i0, key, col);
    }
    const auto col_of = [&](int j) { return LIST ? col[LIST ? j : 0] : (uint32_t)(col0 + i0 + j); };

    uint32_t kstar = 0u, need_ties = 0u, total;
    WinCursor cur;
    if constexpr (kCompact) {
        // After the histogram only the items in the cut bin or above can
        // win (every selectable item when none is cut): at most k plus the
        // cut bin's members.  When they number at most 1024, one counting
        // pass, a block scan and one writing pass put them into LDS in
        // column order (thread t's slots are columns i0 .. i0 + kPer - 1),
        // and the exact cut, the winner scan and the output run on those
        // few items (kCI per thread) instead of on every slot again.  The
        // bins come from the keys (the loaded floats are not kept: registers
        // decide how many workgroups share a CU).
        SlotBins<kPer> bins;
        const CutBin c = hist_cut<NT, kPer, 64, false>(key, k, sh, bins, nullptr);
        total = c.total;
        const uint32_t count = min(total, k);
        const uint32_t cands = c.every ? c.total : c.above + c.n_in_bin;    // uniform
        if (cands <= (uint32_t)(kCI * NT)) {
            // can win: lo <= bin < kBins (the other bins hold non-selectable items)
            const uint32_t lo = c.every ? 0u : c.cbin;
            uint32_t m = 0;
            if (c.total > 0u) {                       // uniform; bins are set
#pragma unroll
                for (int j = 0; j < kPer; ++j) m += bins.get(j) - lo < (uint32_t)kBins - lo;
            }
            uint32_t pos = block_scan<NT>(m, sh.scan_b) - m;
            if (c.total > 0u) {
#pragma unroll
                for (int j = 0; j < kPer; ++j) {
                    const uint32_t bn = bins.get(j);
                    if (bn - lo < (uint32_t)kBins - lo) sh_items[pos++] = make_uint2(key[j], (uint32_t)(i0 + j) << 16 | bn);
                }
            }
            lds_barrier();
            // items tid * kCI ..: (key, segment column << 16 | bin); none:
            // key 0 and a bin that is no member
            uint32_t key1[kCI], cl[kCI];
            SlotBins<kCI> bin1;
#pragma unroll
            for (int i = 0; i < kCI; ++i) {
                const int x = tid * kCI + i;
                const uint2 it = x < (int)cands ? sh_items[x] : make_uint2(0u, (uint32_t)kBins);
                key1[i] = it.x;
                cl[i] = it.y >> 16;
                bin1.set(i, it.y & 0xFFFFu);
            }
            if (!c.every) resolve_cut<NT, kCI, 64>(key1, bin1, c, k, sh, kstar, need_ties);
            scan_winners<NT, kCI>(key1, kstar, need_ties, sh, cur);
            const auto col1 = [&](int i) { return (uint32_t)(col0 + cl[i]); };
            if (a.out_list)
                write_list<NT, kCI, kFused>(a.out_list + ((int64_t)b * a.parts + part) * lcap, lcap, cur, key1, col1, count);
            else
                write_final<NT, kCI>(a, b, cur, key1, col1, count);
        } else {
            if (!c.every) resolve_cut<NT, kPer, 64>(key, bins, c, k, sh, kstar, need_ties);
            scan_winners<NT, kPer>(key, kstar, need_ties, sh, cur);
            if (a.out_list)
                write_list<NT, kPer, kFused>(a.out_list + ((int64_t)b * a.parts + part) * lcap, lcap, cur, key, col_of, count);
            else
                write_final<NT, kPer>(a, b, cur, key, col_of, count);
        }
    } else {
        find_cut<NT, kPer, 64, !LIST>(key, k, sh, kstar, need_ties, total, v);
        scan_winners<NT, kPer>(key, kstar, need_ties, sh, cur);
        const uint32_t count = min(total, k);
        if (a.out_list)
            write_list<NT, kPer, kFused>(a.out_list + ((int64_t)b * a.parts + part) * lcap, lcap, cur, key, col_of, count);
        else
            write_final<NT, kPer>(a, b, cur, key, col_of, count);
    }
    if constexpr (kFused) {
        // ---- fused merge: the row's last part to arrive merges its lists.
        // Once every list store of the workgroup has completed (vmcnt 0 in
        // each wave, then the barrier) the arrival is counted; the counter's
        // atomic and the list accesses are all device-coherent.
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) sh.flag = atomicAdd(a.row_done + b, 1u) == (uint32_t)(a.parts - 1);
        __syncthreads();
        if (!sh.flag) return;                         // uniform
        sel_reset(sh);
        uint32_t mkey[kMPer], mcol[kMPer];
        load_items<kMPer, true>(a.out_list + (int64_t)b * a.parts * lcap, a.parts * (int)lcap, tid * kMPer, mkey,
                                mcol);
        find_cut<NT, kMPer>(mkey, k, sh, kstar, need_ties, total);
        scan_winners<NT, kMPer>(mkey, kstar, need_ties, sh, cur);
        write_final<NT, kMPer>(a, b, cur, mkey, [&](int j) { return mcol[j]; }, min(total, k));
        if (tid == 0) a.row_done[b] = 0u;             // ready for the next call
    }
}

// kSegPlain and kSegSampled: one workgroup per (row, part).  kSegRerun
// (after kSegSampled): each workgroup takes the parts blockIdx.x,
// blockIdx.x + gridDim.x, ..., reads their flags NT at a time (ballots into
// LDS) and runs only the flagged ones, so that a re-run with nothing to do
// costs one short wave of workgroups.
template <int CAP, bool LIST, int NT, int MMUL, int MODE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(seg_waves_per_eu<CAP, LIST, NT, MMUL, MODE>())))
void topk_segment_kernel(SegArgs a) {
    constexpr bool PRE = MODE == kSegSampled;
    constexpr int kPer = CAP / NT;
    __shared__ SelScratch<NT, 64> sh;
    __shared__ uint2 sh_items[seg_items<CAP, LIST, NT, PRE>()];
    if constexpr (MODE == kSegPlain) {
        seg_body<CAP, LIST, NT, MMUL>(a, (int)blockIdx.x, sh, sh_items);
    } else if constexpr (MODE == kSegSampled) {
        static_assert(!LIST && MMUL == 0 && kPer >= 16, "the sampled threshold serves long segments of logits");
        uint32_t x[kPer];
        load_segment<CAP, NT>(a, (int)blockIdx.x, x);
        select_sampled<CAP, NT>(a, (int)blockIdx.x, x, sh, sh_items);
    } else {
        __shared__ uint64_t sh_redo[NT / 64];
        const int tid = threadIdx.x;
        const int ng = a.B * a.parts;
        const int mine = ng > (int)blockIdx.x ? (ng - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
        int loaded = -1;                              // chunk of flags in sh_redo
        // the first flagged one of this workgroup's parts from index `from`
        // on, or -1 (uniform: every thread reads the same masks)
        const auto next_flagged = [&](int from) -> int {
            for (int c = from - from % NT; c < mine; c += NT) {
                if (c != loaded) {
                    const int t = c + tid;
                    const bool f = t < mine && a.redo[(int64_t)blockIdx.x + (int64_t)t * gridDim.x] != 0u;
                    const uint64_t m = __ballot(f);
                    lds_barrier();                    // the previous chunk's masks have been read
                    if ((tid & 63) == 0) sh_redo[tid >> 6] = m;
                    lds_barrier();
                    loaded = c;
                }
                for (int w = 0; w < NT / 64; ++w) {
                    const int lo = from - c - 64 * w;  // positions below `from` are done
                    if (lo >= 64) continue;
                    uint64_t mm = sh_redo[w];
                    if (lo > 0) mm &= ~0ull << lo;
                    if (mm) return c + 64 * w + __builtin_ctzll(mm);
                }
            }
            return -1;
        };
        for (int t = next_flagged(0); t >= 0; t = next_flagged(t + 1)) {     // uniform
            seg_body<CAP, LIST, NT, MMUL, true>(a, (int)blockIdx.x + t * (int)gridDim.x, sh, sh_items);
            lds_barrier();                            // LDS is free for the next part
        }
    }
}

template <int CAP, bool LIST, int NT, int MMUL = 0>
hipError_t launch_seg(const SegArgs &a, hipStream_t s) {
    const int64_t grid = (int64_t)a.B * a.parts;
    if (grid <= 0) return hipSuccess;
    SegArgs r = a;
    if constexpr (!LIST && MMUL == 0 && CAP / NT >= 16) {
        // the sampled threshold, then the workgroups it left unsettled
        if (a.redo) {
            hipLaunchKernelGGL((topk_segment_kernel<CAP, LIST, NT, MMUL, kSegSampled>), dim3((unsigned)grid), dim3(NT),
                               0, s, a);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            // the re-run: about as many workgroups as are resident at once
            // (two per CU of 512 threads, one of 1024), each over its share;
            // a prime count, so that flagged parts recurring with a period
            // (every 4th row, say) still spread over all of them
            const int64_t g2 = std::min<int64_t>(grid, NT == 512 ? 509 : 251);
            hipLaunchKernelGGL((topk_segment_kernel<CAP, LIST, NT, MMUL, kSegRerun>), dim3((unsigned)g2), dim3(NT), 0,
                               s, a);
            return hipGetLastError();
        }
    }
    r.redo = nullptr;
    hipLaunchKernelGGL((topk_segment_kernel<CAP, LIST, NT, MMUL, kSegPlain>), dim3((unsigned)grid), dim3(NT), 0, s, r);
    return hipGetLastError();
}

}  // namespace

// Capacities (items per workgroup / threads): logits 4096/512 (4096/1024 when
// the row's last part merges: the latency-bound phases run faster on more
// waves), 8192/512, 16384/512, 20480/512, 24576/512 (two workgroups per CU:
// many long rows, one part each), 32768/1024 (the smallest that holds a
// part: every slot costs work whether it holds a column or not); lists
// 4096/512, 16384/1024.  `fused` (logits with
// several parts per row whose lists, parts * (k rounded up to even) items,
// fit in 2 * cap for caps up to 8192 or in cap for 16384; row_done zeroed)
// merges in the same launch.
hipError_t launch_topk_segment(const SegArgs &a, bool list, int cap, bool fused, hipStream_t s) {
    if (list) return cap <= 4096 ? launch_seg<4096, true, 512>(a, s) : launch_seg<kSegListCap, true, 1024>(a, s);
    if (fused) {
        const bool one = (int64_t)a.parts * list_cap((uint32_t)a.k) <= cap;
        switch (cap) {
        case 4096: return one ? launch_seg<4096, false, 1024, 1>(a, s) : launch_seg<4096, false, 1024, 2>(a, s);
        case 8192: return one ? launch_seg<8192, false, 1024, 1>(a, s) : launch_seg<8192, false, 1024, 2>(a, s);
        case 16384: return one ? launch_seg<16384, false, 1024, 1>(a, s) : hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
        }
    }
    switch (cap) {
    case 4096: return launch_seg<4096, false, 512>(a, s);
    case 8192: return launch_seg<8192, false, 512>(a, s);
    case 16384: return launch_seg<16384, false, 512>(a, s);
    case 20480: return launch_seg<20480, false, 512>(a, s);
    case 24576: return launch_seg<24576, false, 512>(a, s);
    default: return launch_seg<kSegLogitCap, false, 1024>(a, s);
    }
}

}  // namespace idx
