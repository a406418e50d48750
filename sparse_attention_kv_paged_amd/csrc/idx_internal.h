// Internal launch interface between the C-ABI layer (idx_api.cpp) and the
// gfx950 kernels (idx_score.hip, idx_topk.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace idx {

constexpr int kHeads = 64;
constexpr int kHeadDim = 128;
constexpr int kBlock = 64;                   // entries per slot (and per paged block by default)
constexpr int kSmallBlock = 16;              // the other supported pool block size
constexpr int kRowBytes = kHeadDim + 4;      // 128 e4m3 bytes + fp32 scale
constexpr int kWaves = 4;                    // waves per score workgroup
constexpr int kFlatRows = 512;               // rows up to which the score launch shares work evenly over waves
constexpr int kMaxK = 2048;
constexpr int kSegLogitCap = 32768;          // logits per top-k workgroup
constexpr int kSegListCap = 16384;           // (key, column) items per merge workgroup

constexpr int kMaxLayers = 8;                // layers one score launch can take (IDX_MAX_LAYERS)

// The keys of one layer when a launch scores several layers' rows.
struct LayerKeys {
    const uint8_t *pool;
    int64_t n_pool_rows;
    const int32_t *block_table;
    int32_t n_req;
    int32_t max_blocks;
    const int32_t *q_req;
    const int32_t *limits;
};

struct ScoreArgs {
    const uint16_t *q;          // [B, 64, 128] bf16 (unused when q8 is set)
    const uint8_t *q8;          // [B, 64, 132] quantised q rows (e4m3 bytes, then the head's scale), or null
    int64_t q_row;              // elements from one q row to the next (64 * 128, or 128 * 128 for a head half)
    int32_t w_row;              // floats from one w row to the next (64, or 128)
    bool accum;                 // add to the logits already in the output (the second head half)
    bool quant_q;               // q is bf16 and is quantised here by the writer's rule (q8 null)
    bool mxfp4;                 // q (bf16) and the keys are rounded to MXFP4 blocks of 32 here (q8 null)
    const float *w;             // [B, 64]
    int32_t B;
    const uint8_t *pool;        // [n_pool_rows, 132]
    int64_t n_pool_rows;
    int32_t block_size;         // rows per pool block: 64, or 16 (four blocks per 64-column slot)
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
    float *logits;              // [B, ld], or null when only scores are wanted (not with accum)
    float *scores;              // [B, ld] or null
    // top-k feed (row_cols != null): only each row's own columns are written
    // (those below 64 x its tile-list length) and that count goes to row_cols
    uint32_t *row_cols;         // [B]
    uint32_t *row_done;         // [B] zeroed here for the top-k's fused merge (or null)
    int32_t slots_per_wave;
    int32_t splits;             // workgroups per row
    // Several layers in one launch (rows_per_layer > 0, the flattened split
    // only): row v of the launch is row v % rows_per_layer of layer
    // v / rows_per_layer; q, w and the outputs are indexed by v (the layers'
    // rows stacked), the keys come from layer[v / rows_per_layer].
    int32_t rows_per_layer;
    LayerKeys layer[kMaxLayers];
    // Selection bits (or null): word j of row v holds, for columns
    // 32*j .. 32*j + 31, the bits (sigmoid(logit) >= threshold), binary32.
    uint32_t *page_bits;
    int64_t bits_ld;            // words per row
    float threshold;
    // MXFP4 keys rounded ahead of the score launch (mxfp4, the per-row path,
    // one request, 64-row blocks, no chunk lists): logical block j of
    // request 0 at mx_keys + j * kMxKeyBlockBytes for j < mx_blocks, laid out
    // as mx_keys_kernel writes it.  Null: the score kernel rounds each tile.
    const uint8_t *mx_keys;
    int32_t mx_blocks;
};

// One 64-row block of pre-rounded MXFP4 keys: per row 64 code bytes (the
// four 32-value blocks, two e2m1 values a byte), then per row the four E8M0
// block scales (one word), then per row the fp32 row scale.
constexpr int kMxKeyBlockBytes = 64 * 64 + 64 * 4 + 64 * 4;

// One launch of the segment top-k (idx_topk.hip).  Input is either a logits
// matrix cut into `parts` segments of the kernel's capacity per row, or the
// per-part (key, column) lists of a previous launch; output is either lists
// (out_list != null) or the final ids.
struct SegArgs {
    int32_t B;
    int32_t k;
    int32_t parts;              // workgroups per row
    // logits input
    const float *logits;        // [B, ld]
    int64_t ld;
    int32_t n_cols;
    const uint32_t *row_cols;   // [B] columns per row, or null (= n_cols)
    // list input: in_parts lists of in_cap (= k) items per row, each padded
    // with key 0 after its winners
    const uint2 *in_list;       // [B, in_parts, in_cap]
    int32_t in_parts;
    int32_t in_cap;
    // intermediate output (same layout)
    uint2 *out_list;            // [B, parts, k] or null
    uint32_t *row_done;         // [B] arrival counters of the fused merge (zeroed)
    // final output
    int32_t *out_idx;           // [B, k]
    float *out_val;             // [B, k] or null
    int32_t *out_count;         // [B] number of winners per row, or null
    const int32_t *chunk_ids;   // columns -> logical entries, or null
    int32_t max_chunks;
    int32_t chunk_shift;        // log2 of the entries one chunk id names (6, or 4 for 16-row blocks)
    // [B * parts] or null: the sampled-threshold launch's flag per
    // workgroup (1 = not settled there); with it, the other launch over the
    // same segments only runs the flagged workgroups
    uint32_t *redo;
};

// Level-0 launches over segments of logits with at least 16 per thread
// (caps >= 8192), not merged in the same launch, and k <= kTopkPreMaxK
// first select through a threshold sampled from the segment (up to
// kTopkPreCap items compacted), then re-run the workgroups it could not
// settle: they need the redo flags.
constexpr int kTopkPreCap = 2048;
constexpr int32_t kTopkPreMaxK = kTopkPreCap * 5 / 16;
inline bool topk_sampled(int cap, bool fused, int32_t k) { return !fused && cap >= 8192 && k <= kTopkPreMaxK; }

// ev_start / ev_stop (optional): events the dispatch itself stamps with the
// kernel's start and end time (hipExtLaunchKernelGGL).
hipError_t launch_score(const ScoreArgs &a, hipStream_t s, hipEvent_t ev_start = nullptr,
                        hipEvent_t ev_stop = nullptr);
// Round logical blocks 0 .. nblocks - 1 of request 0's keys (a's pool and
// block table) to MXFP4 into dst (nblocks * kMxKeyBlockBytes bytes).
hipError_t launch_mx_keys(const ScoreArgs &a, uint8_t *dst, int32_t nblocks, hipStream_t s);
hipError_t launch_topk_segment(const SegArgs &a, bool list, int cap, bool fused, hipStream_t s);

}  // namespace idx
