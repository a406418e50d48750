/*
 * idx.h -- C ABI of the MI355X (gfx950) compressed-sparse-attention indexer:
 * paged fp8 key scoring and per-query top-k selection.
 *
 * What it computes ("FlashMemory-DeepSeek-V4" README, section "Retriever
 * architecture"): for query row b, head h and a compressed key entry with
 * fp8 bytes k8[0..D) and fp32 scale s ("compressed_k format": a row is
 * D float8_e4m3 bytes followed by the fp32 scale, 132 bytes at D = 128),
 *
 *     k[d]      = e4m3(k8[d]) * s
 *     logit     = sum_h relu( sum_d k[d] * q[b,h,d] ) * w[b,h]
 *     score     = sigmoid(logit)
 *
 * with relu applied to each head before the weighted head sum ("feat:
 * DeepSeek-V4-Flash integration + Blackwell (sm120) bring-up", Phase 3
 * summary).  Level 2 of the pages' "Two-level recall algorithm" keeps the
 * top-512 logits of each query, with non-resident entries at -inf.
 *
 * Tile lists ("DeepSeek-V4.1 native paged runtime", section "Current
 * execution scope"): every query row carries its own bound (limits[b], the
 * compressed length seq_len // 4 per the c4 fix in the batchgen pull request)
 * and its own list of blocks read in place from the paged pool; a
 * prefill token, a decode token and a ragged batch are all the same shape.
 *
 * Conventions for every entry point:
 *  - Every array pointer is a DEVICE pointer owned by the caller; the library
 *    never allocates, frees, synchronises, or reads device memory on the
 *    host.  Work is enqueued on `stream` (a hipStream_t; NULL = the null
 *    stream) and returns before it finishes.  Bounds, block ids and chunk
 *    lists stay on the device, so calls can be captured in a HIP graph.
 *  - Supported shapes: H = 64 or 128 heads, D = 128, block_size = 64 or 16,
 *    1 <= k <= 2048, 1 <= n_cols <= IDX_MAX_COLS.  Every per-row array
 *    (limits, q_req, n_chunks, and chunk_ids' rows) holds B entries: the
 *    kernels read that many.
 *  - The return value is IDX_OK (0) or an IDX_E_* code; nothing is launched
 *    when a host-side check fails.  idx_last_error() gives a message for the
 *    calling thread's last failure.
 *  - Data that only the device can see is never trusted: a bound above the
 *    tile list's capacity is clamped, a block id of -1 means "absent", and an
 *    out-of-range block id, chunk id or request id is treated as absent; the
 *    corresponding columns are -inf and, when keys->status is given, a bit is
 *    OR-ed into it (IDX_STATUS_*).  No kernel reads outside the pool.
 *  - Key rows at scored positions must hold finite values; NaN/inf there give
 *    an unspecified logit.
 */
#ifndef IDX_H
#define IDX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum idx_status_code {
    IDX_OK = 0,
    IDX_E_ARG = 1,        /* a required pointer is NULL or a count is negative */
    IDX_E_SHAPE = 2,      /* unsupported H, D, block_size, k, or inconsistent sizes */
    IDX_E_ALIGN = 3,      /* q, pool, logits or workspace not 16-byte aligned */
    IDX_E_WORKSPACE = 4,  /* ws_bytes below idx_workspace_bytes(...) */
    IDX_E_HIP = 5         /* a HIP launch failed; idx_last_error() has the text */
};

/* op argument of idx_workspace_bytes */
enum idx_op { IDX_OP_SCORE = 0, IDX_OP_TOPK = 1, IDX_OP_SCORE_TOPK = 2 };

/* bits OR-ed into *keys->status by the device */
#define IDX_STATUS_LIMIT_CLAMPED 0x1u  /* limits[b] exceeded the tile list's capacity */
#define IDX_STATUS_BAD_BLOCK 0x2u      /* a block-table entry < -1 or past the pool's end */
#define IDX_STATUS_BAD_REQUEST 0x4u    /* q_req[b] >= n_req (row treated as padding) */
#define IDX_STATUS_BAD_CHUNK 0x8u      /* chunk id < 0 or >= max_blocks, or n_chunks[b] > max_chunks */
#define IDX_STATUS_BAD_SLOT 0x10u      /* idx_write_keys: a slot < -1 or >= n_pool_rows (nothing written) */

#define IDX_HEADS 64
#define IDX_HEAD_DIM 128
#define IDX_BLOCK 64
#define IDX_ROW_BYTES (IDX_HEAD_DIM + 4)
#define IDX_MAX_K 2048
/* Largest n_cols any call takes (2^27 columns = 2^29 tokens at C4): column
 * byte offsets and the work index stay within 32 bits.  Larger values are
 * rejected with IDX_E_SHAPE. */
#define IDX_MAX_COLS (1 << 27)

/*
 * The paged index plane and each query row's tile list.  Host struct holding
 * device pointers; read by the call, not retained.
 *
 * pool         uint8 [n_pool_rows, D + 4]: row r = D e4m3fn bytes, then the
 *              fp32 scale (little-endian).  16-byte aligned.  Rows of one
 *              block are contiguous (8448 bytes for 64 rows).
 * n_pool_rows  rows in the pool (with a block table: a multiple of
 *              block_size).
 * block_size   entries (rows) per block: 64, or 16 ("DeepSeek-V4.1 native
 *              paged runtime": one block id names 16 index rows).  Block
 *              table entries and chunk ids count blocks of this size.
 * block_table  int32 [n_req, max_blocks]: logical block -> pool block, -1 =
 *              absent.  NULL = contiguous: logical entry e is pool row e for
 *              every request.
 * q_req        int32 [B]: request (block-table row) of each query row;
 *              -1 = padding row (all columns -inf, top-k all -1).
 *              NULL = identity (row b uses table row b).
 * chunk_ids    int32 [B, max_chunks]: the logical blocks row b scores (the
 *              resident subset); NULL = blocks 0, 1, 2, ... of the request.
 * n_chunks     int32 [B]: listed chunks per row; required iff chunk_ids.
 * limits       int32 [B]: row b scores logical entries e < limits[b].
 * status       optional uint32 device word; see IDX_STATUS_*.  Not cleared
 *              by the library.
 *
 * Column c of row b (the logits' second index):
 *   without chunk_ids: c is the logical entry id;
 *   with chunk_ids:    c = block_size*j + s is entry s of block
 *                      chunk_ids[b][j], i.e. logical entry
 *                      chunk_ids[b][j]*block_size + s.
 * A column is scored iff it maps to an entry below limits[b] whose block is
 * present; every other column is -inf.
 */
typedef struct idx_keys {
    const uint8_t *pool;
    int64_t n_pool_rows;
    int32_t block_size;
    int32_t n_req;
    const int32_t *block_table;
    int32_t max_blocks;
    int32_t max_chunks;
    const int32_t *q_req;
    const int32_t *chunk_ids;
    const int32_t *n_chunks;
    const int32_t *limits;
    uint32_t *status;
} idx_keys;

/*
 * idx_score: logits (and optionally sigmoid scores) of every column.
 *
 * q        bf16 bit patterns [B, H, D], 16-byte aligned.
 * w        fp32 [B, H]: fused head weights (weights_proj output already
 *          multiplied by D^-0.5 * H^-0.5, "Retriever architecture").
 * n_cols   columns per row of the outputs (>= 1).
 * logits   fp32 [B, n_cols] out, 16-byte aligned: the logit, or -inf for an
 *          unscored column.
 * scores   fp32 [B, n_cols] out, or NULL: sigmoid(logit), 0 where unscored.
 */
int idx_score(const uint16_t *q, const float *w, int32_t B, int32_t H,
              int32_t D, const idx_keys *keys, int32_t n_cols, float *logits,
              float *scores, void *stream);

/*
 * idx_topk: the k largest values of each row of a logits matrix.
 *
 * logits   fp32 [B, ld] in (row stride ld >= n_cols); -inf and NaN entries
 *          are never selected.
 * out_col  int32 [B, k] out: the selected columns in ascending column
 *          order; among equal values at the cut the lower columns win; rows
 *          with fewer than k selectable entries end in -1.
 * out_val  fp32 [B, k] out or NULL: the selected values (-inf for -1).
 * workspace / ws_bytes: device scratch of at least
 *          idx_workspace_bytes(IDX_OP_TOPK, B, n_cols, k) bytes, 256-byte
 *          aligned; contents on entry do not matter (the library keeps no
 *          state in it between calls).
 */
int idx_topk(const float *logits, int32_t B, int32_t n_cols, int64_t ld,
             int32_t k, int32_t *out_col, float *out_val, void *workspace,
             size_t ws_bytes, void *stream);

/*
 * idx_score_topk: the whole path: score every column as idx_score would,
 * then select the top-k of each row as idx_topk would.
 *
 * out_idx  int32 [B, k] out: LOGICAL entry ids (chunk lists resolved) of
 *          the selected columns, in ascending column order; among equal
 *          logits at the cut the lower columns win; -1 pads.
 * out_val  fp32 [B, k] out or NULL: their logits.
 * workspace / ws_bytes: at least
 *          idx_workspace_bytes(IDX_OP_SCORE_TOPK, B, n_cols, k) bytes,
 *          256-byte aligned; contents on entry do not matter (the score
 *          kernel clears the per-row counters the top-k's in-launch merge
 *          uses).  Calls that share one workspace must not overlap.
 */
int idx_score_topk(const uint16_t *q, const float *w, int32_t B, int32_t H,
                   int32_t D, const idx_keys *keys, int32_t n_cols, int32_t k,
                   int32_t *out_idx, float *out_val, void *workspace,
                   size_t ws_bytes, void *stream);

/*
 * idx_score_topk_noalloc: idx_score_topk for callers that cannot allocate
 * device memory -- code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments, rules and results as
 * idx_score_topk, without the workspace: the library's own static device
 * scratch of IDX_STATIC_SCRATCH_BYTES (16 MiB) takes its place.  Each GPU the
 * library runs on holds one such scratch from the first call on it until the
 * process ends.  Calls whose workspace would exceed it
 * (idx_workspace_bytes(IDX_OP_SCORE_TOPK, B, n_cols, k) > 16 MiB: every
 * decode shape up to 8 rows x 262,144 columns fits, a 4096-row prefill does
 * not) return IDX_E_WORKSPACE before anything is launched.  The call itself
 * allocates nothing; its first call on a device looks up that device's
 * scratch address.  Every call on one GPU shares that GPU's scratch, which
 * keeps the last call's contents: calls that overlap on one GPU (other
 * streams, other threads) race and must not be issued.
 */
#define IDX_STATIC_SCRATCH_BYTES (16u << 20)

int idx_score_topk_noalloc(const uint16_t *q, const float *w, int32_t B,
                           int32_t H, int32_t D, const idx_keys *keys,
                           int32_t n_cols, int32_t k, int32_t *out_idx,
                           float *out_val, void *stream);

/*
 * idx_score_q8 / idx_score_topk_q8: the same path with the query quantised
 * to e4m3 as well, so that the contraction runs on fp8 MFMA with both
 * operands taken as stored.  The pages' deployed indexers quantise the
 * query too (the batchgen pull request: fp4 where the hardware has it, an
 * e4m3 fallback with one scale per 32 values elsewhere; the ATOM runtime
 * page: the published model rounds query and key to fp4); this variant
 * gives the query the index plane's own row format instead, one e4m3 scale
 * per head, which is what lets the scale fold exactly into the head weight
 * below.  q8 holds, for each
 * row b and head h, one 132-byte row in the index-plane layout: 128 e4m3
 * bytes then the head's fp32 scale s_q[b,h] -- exactly what idx_write_keys
 * writes from q viewed as B*H keys of D values (slot b*H + h), i.e. the
 * amax/448 rule per head.  The logit is the definition above with q replaced
 * by its dequantised values:
 *
 *     logit = sum_h relu( sum_d k[d] * e4m3(q8[b,h,d]) * s_q[b,h] ) * w[b,h]
 *
 * (s_q >= 0, so relu(s_q x) = s_q relu(x) and the kernel folds s_q into w).
 * q8 is [B, H, D + 4] bytes, 4-byte aligned, with H = 64 (128 heads are
 * taken by the bf16 entry points only: IDX_E_SHAPE here); every other
 * argument, output and rule, 16-row blocks included, is as for idx_score /
 * idx_score_topk.
 */
int idx_score_q8(const uint8_t *q8, const float *w, int32_t B, int32_t H,
                 int32_t D, const idx_keys *keys, int32_t n_cols, float *logits,
                 float *scores, void *stream);
int idx_score_topk_q8(const uint8_t *q8, const float *w, int32_t B, int32_t H,
                      int32_t D, const idx_keys *keys, int32_t n_cols,
                      int32_t k, int32_t *out_idx, float *out_val,
                      void *workspace, size_t ws_bytes, void *stream);

/*
 * idx_score_fp8q / idx_score_topk_fp8q: the quantised-query path with the
 * query quantised inside the score kernel, as the pages' deployed paged
 * scorer does ("DeepSeek-V4.1 native paged runtime", section "Current
 * execution scope": the paged scorer quantises the query itself), so no
 * separate quantising launch precedes the scoring.  Arguments as for
 * idx_score / idx_score_topk (q bf16 [B, H, D], 16-byte aligned), H = 64.
 * Each query head is quantised exactly as idx_write_keys would quantise it
 * (the amax/448 rule, nearest-even e4m3 codes), so the results are bit for bit
 * those of idx_write_keys on q viewed as B*H keys followed by idx_score_q8 /
 * idx_score_topk_q8 on the written rows.
 */
int idx_score_fp8q(const uint16_t *q, const float *w, int32_t B, int32_t H,
                   int32_t D, const idx_keys *keys, int32_t n_cols,
                   float *logits, float *scores, void *stream);
int idx_score_topk_fp8q(const uint16_t *q, const float *w, int32_t B,
                        int32_t H, int32_t D, const idx_keys *keys,
                        int32_t n_cols, int32_t k, int32_t *out_idx,
                        float *out_val, void *workspace, size_t ws_bytes,
                        void *stream);

/*
 * idx_score_mxfp4 / idx_score_topk_mxfp4: the MXFP4 variant.  The published
 * model rounds the index query and key alike to FP4 before the index score,
 * whatever the index plane holds ("DeepSeek-V4.1 native paged runtime",
 * section "Current execution scope"); the batchgen pull request names the
 * format MXFP4 (its fp8-fallback commit: selector auto | mxfp4 | fp8, with an
 * e4m3 fallback at one scale per 32 values).  Here both are rounded inside
 * the score kernel to OCP MXFP4 blocks of 32 consecutive dims (one query
 * head's, or one key row's): the block scale is 2^e with
 * e = floor(log2(amax)) - 2 (clamped to >= -127), each value the nearest E2M1
 * value (0, 0.5, 1, 1.5, 2, 3, 4, 6) of v / 2^e, ties to the even code,
 * saturating at 6.  A key's e4m3 values are the block's values and its fp32
 * row scale stays a factor outside the rounding:
 *
 *     logit = sum_h relu( s * sum_d mx(e4m3(key))[d] * mx(q[b,h])[d] ) * w[b,h]
 *
 * The contraction runs on v_mfma_scale_f32_32x32x64_f8f6f4 with e2m1
 * operands and the blocks' E8M0 scales.  Arguments, outputs, rules and
 * errors as for idx_score / idx_score_topk (q bf16 [B, H, D], 16-byte
 * aligned), with H = 64 (IDX_E_SHAPE otherwise).  idx_score_topk_mxfp4 with
 * more than 512 rows of one request (n_req = 1, a block table, 64-row
 * blocks, no chunk lists) rounds that request's key blocks once into its
 * workspace before the score launch, by the same rule, so its result equals
 * idx_score_mxfp4's bit for bit; the workspace size already includes the
 * room (idx_workspace_bytes(IDX_OP_SCORE_TOPK, ...)).
 */
int idx_score_mxfp4(const uint16_t *q, const float *w, int32_t B, int32_t H,
                    int32_t D, const idx_keys *keys, int32_t n_cols,
                    float *logits, float *scores, void *stream);
int idx_score_topk_mxfp4(const uint16_t *q, const float *w, int32_t B,
                         int32_t H, int32_t D, const idx_keys *keys,
                         int32_t n_cols, int32_t k, int32_t *out_idx,
                         float *out_val, void *workspace, size_t ws_bytes,
                         void *stream);

/*
 * idx_write_keys: the index-plane writer -- quantise new compressed keys and
 * store them as pool rows in the layout idx_score reads ("FlashMemory-
 * DeepSeek-V4" README, section "compressed_k format": D float8_e4m3 bytes
 * then the fp32 scale; the batchgen pull request's fp8 indexer-pool insert
 * fills rows of that layout).  The pages do not state the scale rule; this
 * library takes the per-key absolute maximum over e4m3's largest finite
 * value:
 *
 *     s       = amax_d |k[d]| / 448          (binary32 division, nearest)
 *     byte d  = e4m3fn( k[d] / s )           (binary32 division, nearest;
 *                                             then the nearest e4m3 value,
 *                                             ties to the even code,
 *                                             saturating at +-448)
 *
 * so the largest element is stored as +-448 and every element is recovered
 * as e4m3(byte) * s within half an e4m3 step.  A key of zeros (either sign)
 * is stored as zero bytes and scale 0.
 *
 * k        bf16 bit patterns [n, D], 16-byte aligned; values must be finite.
 * n        number of keys (0 = nothing to do).
 * D        head dimension; must be 128.
 * slots    int64 [n]: pool row that receives key i.  -1 writes nothing (the
 *          padding id of "DeepSeek-V4.1 native paged runtime"); any other
 *          value outside [0, n_pool_rows) writes nothing and, when status is
 *          given, ORs IDX_STATUS_BAD_SLOT into *status.  Two keys naming the
 *          same slot leave that row unspecified.
 * pool     uint8 [n_pool_rows, D + 4] in/out, 4-byte aligned; only the named
 *          rows are written (each whole: D bytes and the scale).
 * status   optional uint32 device word (bits OR-ed in, never cleared).
 * The write is ordered on `stream` like every call: a later idx_score on the
 * same stream sees the new rows.
 */
int idx_write_keys(const uint16_t *k, int64_t n, int32_t D,
                   const int64_t *slots, uint8_t *pool, int64_t n_pool_rows,
                   uint32_t *status, void *stream);

/*
 * idx_select_resident: Level 1 of the two-level recall ("FlashMemory-
 * DeepSeek-V4" README, sections "Two-level recall algorithm" and "Joint
 * checkpoint + ensemble"; KMAX in section "Quick start"): score each row's
 * whole history at n_layers retriever layers, each with its own q, w and
 * index plane, ensemble the layers' sigmoid scores per entry, threshold them,
 * and choose the pages (64-entry blocks) to keep resident.  The pages give
 * the steps but not their details; this library takes:
 *   - entry e of row b (e < keys[0].limits[b], clamped to n_cols) is
 *     selected iff its ensemble score s >= cfg->threshold, where s is the
 *     maximum of the layers' binary32 sigmoid scores (IDX_ENSEMBLE_MAX, the
 *     pages' default) or their binary32 sum in layer order divided by
 *     n_layers (IDX_ENSEMBLE_MEAN);
 *   - a page's density is its number of selected entries; the row's history
 *     has P = ceil(limit / 64) pages;
 *   - pages p < n_sink (the attention sink) and p >= P - n_recent (the
 *     recency tail) are always resident; the others with density > 0 follow,
 *     densest first, equal densities to the lower page, up to kmax pages.
 *
 * n_layers  1 .. IDX_MAX_LAYERS (the pages' checkpoint has 3).
 * q, w      host arrays of n_layers device pointers: layer l's q [B, H, D]
 *           (bf16, 16-byte aligned) and fused weights [B, H].
 * keys      host array of n_layers structs: layer l's index plane and tile
 *           lists, as for idx_score, without chunk lists (the whole history
 *           is scored).  keys[0].limits also bounds the selection.
 * n_cols    columns per row (logical entries), >= 1.
 * cfg       ensemble, threshold, n_sink, n_recent >= 0, 1 <= kmax <= 2048,
 *           n_sink + n_recent <= kmax.
 * out_pages int32 [B, kmax] out: resident pages in ascending order, -1 after
 *           the last.  Pages are 64 entries whatever keys' block_size.
 *           Usable as chunk_ids (max_chunks = kmax) of a later idx_score /
 *           idx_score_topk on the same rows over 64-row blocks; over 16-row
 *           blocks page p is the chunks 4p .. 4p + 3.
 * out_count int32 [B] out, or NULL: resident pages per row (usable as
 *           n_chunks).
 * workspace / ws_bytes: at least idx_resident_workspace_bytes(n_layers, B,
 *           n_cols, kmax) bytes, 256-byte aligned; contents on entry do not
 *           matter.  Calls that share one workspace must not overlap.
 *
 * Layout that runs in one score launch: when q[l] == q[0] + l*B*H*D and
 * w[l] == w[0] + l*B*H for every layer (the layers stacked in one tensor),
 * H = 64, the ensemble is IDX_ENSEMBLE_MAX, every layer has the same status
 * word and block size, and n_layers * B <= 512, all layers are scored by one
 * launch that records only which entries reach the threshold.  The result
 * is the same either way.
 */
#define IDX_ENSEMBLE_MAX 0
#define IDX_ENSEMBLE_MEAN 1
#define IDX_MAX_LAYERS 8

typedef struct idx_resident_cfg {
    int32_t ensemble;
    float threshold;
    int32_t n_sink;
    int32_t n_recent;
    int32_t kmax;
} idx_resident_cfg;

int idx_select_resident(int32_t n_layers, const uint16_t *const *q,
                        const float *const *w, int32_t B, int32_t H, int32_t D,
                        const idx_keys *keys, int32_t n_cols,
                        const idx_resident_cfg *cfg, int32_t *out_pages,
                        int32_t *out_count, void *workspace, size_t ws_bytes,
                        void *stream);

/* Workspace bytes idx_select_resident needs; (size_t)-1 for invalid
 * arguments. */
size_t idx_resident_workspace_bytes(int32_t n_layers, int32_t B, int32_t n_cols,
                                    int32_t kmax);

/* Workspace bytes an op needs for B rows of n_cols columns and top-k
 * (0 for IDX_OP_SCORE); (size_t)-1 for invalid arguments. */
size_t idx_workspace_bytes(int32_t op, int32_t B, int32_t n_cols, int32_t k);

/* Static text of an IDX_* code. */
const char *idx_error_string(int32_t code);

/* Message of the calling thread's last failed call ("" if none). */
const char *idx_last_error(void);

/*
 * idx_profile_events: measurement hook for benchmark harnesses.  When both
 * are non-NULL (hipEvent_t handles created by the caller, with timing), every
 * later idx_score / idx_score_topk call on this thread launches its score
 * kernel, and every idx_write_keys call its writer kernel, so that the
 * dispatch itself stamps `before` with the kernel's start and `after` with
 * its end (hipExtLaunchKernelGGL), so hipEventElapsedTime(before, after) is
 * that kernel's execution time.  Pass NULL, NULL to stop.  Returns IDX_OK.
 */
int idx_profile_events(void *before, void *after);

/* ABI version of this header (increments on incompatible change). */
int32_t idx_abi_version(void);

#define IDX_ABI_VERSION 1

#ifdef __cplusplus
}
#endif

#endif /* IDX_H */
