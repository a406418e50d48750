// Internal launch interface between the C-ABI layer (idx_api.cpp) and the
// gfx950 kernels (idx_score.hip, idx_topk.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace idx {

constexpr int kHeads = 64;
constexpr int kHeadDim = 128;
constexpr int kBlock = 64;                   // entries per paged block
constexpr int kRowBytes = kHeadDim + 4;      // 128 e4m3 bytes + fp32 scale
constexpr int kWaves = 4;                    // waves per score workgroup
constexpr int kHistBits = 11;                // first-level top-k histogram
constexpr int kHistBins = 1 << kHistBits;
constexpr int kHistShift = 32 - kHistBits;
constexpr int kMaxK = 2048;
constexpr int kCounters = 4;                 // per row: sure, cand, cols, spare

// Per-row counters in the top-k workspace.
enum { kCntSure = 0, kCntCand = 1, kCntCols = 2 };

struct ScoreArgs {
    const uint16_t *q;          // [B, 64, 128] bf16
    const float *w;             // [B, 64]
    int32_t B;
    const uint8_t *pool;        // [n_pool_rows, 132]
    int64_t n_pool_rows;
    const int32_t *block_table; // [n_req, max_blocks] or null
    int32_t n_req;
    int32_t max_blocks;
    const int32_t *q_req;       // [B] or null
    const int32_t *chunk_ids;   // [B, max_chunks] or null
    const int32_t *n_chunks;    // [B] (with chunk_ids)
    int32_t max_chunks;
    const int32_t *limits;      // [B]
    uint32_t *status;           // optional
    int32_t n_cols;             // columns per output row
    int64_t ld;                 // output row stride (floats)
    float *logits;              // [B, ld]
    float *scores;              // [B, ld] or null
    // top-k mode (hist != null): histogram + per-row counters, and only the
    // row's own columns are written
    uint32_t *hist;             // [B, kHistBins]
    uint32_t *counters;         // [B, kCounters]
    int32_t slots_per_wave;
    int32_t splits;             // workgroups per row
};

struct TopkArgs {
    const float *logits;        // [B, ld]
    int64_t ld;
    int32_t B;
    int32_t n_cols;
    int32_t k;
    uint32_t *hist;             // [B, kHistBins]
    uint32_t *counters;         // [B, kCounters]
    uint2 *sure;                // [B, k]      (key, column)
    uint2 *cand;                // [B, ldc]    (key, column)
    int64_t ldc;
    int32_t cols_per_wg;        // select/hist kernels: columns per workgroup
    int32_t parts;              // workgroups per row
    int32_t *out_col;           // [B, k]
    float *out_val;             // [B, k] or null
    const int32_t *chunk_ids;   // map columns to entries (score_topk), or null
    int32_t max_chunks;
    int32_t map_entries;        // 1: write logical entry ids
    int32_t set_cols;           // init kernel: counters[b][kCntCols] = n_cols
};

hipError_t launch_score(const ScoreArgs &a, hipStream_t s);
hipError_t launch_topk_init(const TopkArgs &a, hipStream_t s);
hipError_t launch_topk_hist(const TopkArgs &a, hipStream_t s);
hipError_t launch_topk_select(const TopkArgs &a, hipStream_t s);
hipError_t launch_topk_final(const TopkArgs &a, hipStream_t s);

}  // namespace idx
