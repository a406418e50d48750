// C-ABI layer of libidx.so: host-side validation, workspace layout and launch
// configuration.  Never allocates, synchronises or reads device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/idx.h"
#include "idx_internal.h"
#include "idx_level1.h"
#include "idx_write.h"

namespace {

thread_local char g_last_error[512] = "";
thread_local hipEvent_t g_ev_before = nullptr, g_ev_after = nullptr;

hipError_t launch_score_timed(const idx::ScoreArgs &a, hipStream_t s) {
    // with the profiling hook set, the dispatch stamps the events with the
    // kernel's own start and end
    return idx::launch_score(a, s, g_ev_before, g_ev_after);
}

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return code;
}

bool aligned(const void *p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Top-k launch plan and workspace, each workspace piece 256-byte aligned.
//   level 0: segments of `cap0` logits per workgroup, `parts0` per row;
//   level >= 1: merge up to kSegListCap / list_cap(k) lists per workgroup until one
//   workgroup per row remains.  Lists ping-pong between two buffers.
struct TopkPlan {
    int cap0 = 0, parts0 = 0;
    bool fused = false;         // one launch: the row's last part merges the lists
    size_t logits = 0, row_cols = 0, row_done = 0, list[2] = {0, 0}, total = 0;
    int64_t ld = 0;
    // the per-row split (B > kFlatRows): room for one request's key blocks
    // rounded to MXFP4 ahead of the score launch (idx_score_topk_mxfp4)
    size_t mx = 0;
    int32_t mx_blocks = 0;
    // level 0 through a sampled threshold first: one flag per workgroup
    size_t redo = 0;
    bool sampled = false;
};

// Items per merge list: k rounded up to even (the kernels pad every list
// with never-selectable items to this length).
int list_cap(int32_t k) { return (k + 1) & ~1; }

int seg_cap_for(int64_t cols) {
    for (int c : {4096, 8192, 16384, 20480, 24576})
        if (cols <= c) return c;
    return idx::kSegLogitCap;
}

// Level-0 split: enough parts per row that the whole launch covers the GPU's
// 256 CUs (few long rows), each part holding 4096..32768 columns.
TopkPlan topk_plan(bool with_logits, int32_t B, int32_t n_cols, int32_t k) {
    TopkPlan P;
    P.ld = round_up(std::max<int64_t>(n_cols, 1), 64);
    const int64_t want = std::max<int64_t>(1, (256 + std::max(B, 1) - 1) / std::max(B, 1));
    const int64_t most = std::max<int64_t>(1, ((int64_t)n_cols + 4095) / 4096);
    int64_t parts = std::min(want, most);
    // few long rows: at most 16 parts of up to 16384 columns, merged in the
    // same launch -- the merge of 16 short lists beats a part-selection of
    // 8192 columns followed by a merge of 32 lists
    if (B <= 16 && parts > 16 && ((int64_t)n_cols + 15) / 16 <= 16384) parts = 16;
    P.cap0 = seg_cap_for(((int64_t)n_cols + parts - 1) / parts);
    P.parts0 = (int)std::max<int64_t>(1, ((int64_t)n_cols + P.cap0 - 1) / P.cap0);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off += (size_t)round_up((int64_t)std::max<size_t>(bytes, 1), 256);
        return at;
    };
    if (with_logits) {
        P.logits = take((size_t)B * P.ld * sizeof(float));
        P.row_cols = take((size_t)B * sizeof(uint32_t));
        P.row_done = take((size_t)B * sizeof(uint32_t));
        // the score kernel zeroes row_done, so score_topk can merge in place
        P.fused = P.parts0 > 1 && P.cap0 <= 16384 &&
                  (int64_t)P.parts0 * list_cap(k) <= (P.cap0 <= 8192 ? 2 : 1) * (int64_t)P.cap0;
        if (B > idx::kFlatRows) {
            P.mx_blocks = (int32_t)(((int64_t)n_cols + idx::kBlock - 1) / idx::kBlock);
            P.mx = take((size_t)P.mx_blocks * idx::kMxKeyBlockBytes);
        }
    }
    P.sampled = idx::topk_sampled(P.cap0, P.fused, k);
    if (P.sampled) P.redo = take((size_t)std::max(B, 1) * P.parts0 * sizeof(uint32_t));
    if (P.parts0 > 1) {
        const int per = idx::kSegListCap / list_cap(k);
        const int parts1 = (P.parts0 + per - 1) / per;
        P.list[0] = take((size_t)B * P.parts0 * list_cap(k) * sizeof(uint2));
        P.list[1] = take((size_t)B * parts1 * list_cap(k) * sizeof(uint2));
    }
    P.total = off;
    return P;
}

// Enqueue the top-k launches for logits [B, ld] (row_cols optional).
hipError_t enqueue_topk(const TopkPlan &P, char *ws, const float *logits, int64_t ld,
                        const uint32_t *row_cols, int32_t B, int32_t n_cols, int32_t k,
                        int32_t *out_idx, float *out_val, const int32_t *chunk_ids,
                        int32_t max_chunks, int32_t chunk_shift, hipStream_t s,
                        int32_t *out_count = nullptr) {
    idx::SegArgs a{};
    a.out_count = out_count;
    a.B = B;
    a.k = k;
    a.logits = logits;
    a.ld = ld;
    a.n_cols = n_cols;
    a.row_cols = row_cols;
    a.parts = P.parts0;
    a.out_idx = out_idx;
    a.out_val = out_val;
    a.chunk_ids = chunk_ids;
    a.max_chunks = max_chunks;
    a.chunk_shift = chunk_shift;
    a.redo = P.sampled ? reinterpret_cast<uint32_t *>(ws + P.redo) : nullptr;
    if (P.parts0 == 1) return idx::launch_topk_segment(a, false, P.cap0, false, s);
    a.out_list = reinterpret_cast<uint2 *>(ws + P.list[0]);
    if (P.fused) {
        a.row_done = reinterpret_cast<uint32_t *>(ws + P.row_done);
        return idx::launch_topk_segment(a, false, P.cap0, true, s);
    }
    hipError_t e = idx::launch_topk_segment(a, false, P.cap0, false, s);
    if (e != hipSuccess) return e;
    const int lcap = list_cap(k);
    const int per = idx::kSegListCap / lcap;
    int in_parts = P.parts0, cur = 0;
    while (true) {
        idx::SegArgs m = a;
        m.redo = nullptr;
        m.logits = nullptr;
        m.row_cols = nullptr;
        m.in_list = reinterpret_cast<const uint2 *>(ws + P.list[cur]);
        m.in_parts = in_parts;
        m.in_cap = lcap;
        m.parts = (in_parts + per - 1) / per;
        // the small merge variant when a row's lists fit in 4096 items
        const int cap = (int64_t)in_parts * lcap <= 4096 ? 4096 : idx::kSegListCap;
        if (m.parts == 1) {
            m.out_list = nullptr;
            return idx::launch_topk_segment(m, true, cap, false, s);
        }
        m.out_list = reinterpret_cast<uint2 *>(ws + P.list[cur ^ 1]);
        if ((e = idx::launch_topk_segment(m, true, idx::kSegListCap, false, s)) != hipSuccess) return e;
        in_parts = m.parts;
        cur ^= 1;
    }
}

// Level-1 workspace: one logits scratch row block (written by every layer's
// score launch, never read), the layers' scores, the page keys, then the
// page top-k's own pieces; each piece 256-byte aligned.
struct ResidentPlan {
    int64_t ld = 0, ldp = 0;
    int32_t n_pages = 0;
    size_t logits = 0, scores = 0, page_keys = 0, topk = 0, total = 0;
    TopkPlan top;
};

ResidentPlan resident_plan(int32_t L, int32_t B, int32_t n_cols, int32_t kmax) {
    ResidentPlan R;
    R.ld = round_up(std::max<int64_t>(n_cols, 1), 64);
    R.n_pages = (int32_t)(R.ld / 64);
    R.ldp = round_up(R.n_pages, 64);
    R.top = topk_plan(false, B, R.n_pages, kmax);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off += (size_t)round_up((int64_t)std::max<size_t>(bytes, 1), 256);
        return at;
    };
    R.logits = take((size_t)B * R.ld * sizeof(float));
    R.scores = take((size_t)L * B * R.ld * sizeof(float));
    R.page_keys = take((size_t)B * R.ldp * sizeof(float));
    R.topk = take(R.top.total);
    R.total = off;
    return R;
}

int check_qw(const uint16_t *q, const float *w, int32_t B, int32_t H, int32_t D) {
    if (B < 0) return fail(IDX_E_ARG, "B must be >= 0 (got %d)", B);
    if ((H != idx::kHeads && H != 2 * idx::kHeads) || D != idx::kHeadDim)
        return fail(IDX_E_SHAPE, "only H=64 or 128 and D=128 are supported (got H=%d, D=%d)", H, D);
    if (B > 0 && (!q || !w)) return fail(IDX_E_ARG, "q and w must be non-null");
    if (!aligned(q, 16) || !aligned(w, 16)) return fail(IDX_E_ALIGN, "q and w must be 16-byte aligned");
    return IDX_OK;
}

int check_keys(const idx_keys *keys, int32_t B) {
    if (!keys) return fail(IDX_E_ARG, "keys must be non-null");
    const int32_t bs = keys->block_size;
    if (bs != idx::kBlock && bs != idx::kSmallBlock)
        return fail(IDX_E_SHAPE, "block_size must be 64 or 16 (got %d)", bs);
    if (keys->n_pool_rows < 0) return fail(IDX_E_ARG, "n_pool_rows must be >= 0");
    if (keys->n_pool_rows > 0 && !keys->pool) return fail(IDX_E_ARG, "pool is null");
    if (!aligned(keys->pool, 16)) return fail(IDX_E_ALIGN, "pool must be 16-byte aligned");
    if (B > 0 && !keys->limits) return fail(IDX_E_ARG, "limits must be non-null");
    if (keys->block_table) {
        if (keys->n_req <= 0 || keys->max_blocks <= 0)
            return fail(IDX_E_SHAPE, "a block table needs n_req >= 1 and max_blocks >= 1");
        if (keys->n_pool_rows % bs)
            return fail(IDX_E_SHAPE, "with a block table, n_pool_rows must be a multiple of block_size");
        if ((int64_t)keys->max_blocks * bs > INT32_MAX)
            return fail(IDX_E_SHAPE, "max_blocks too large");
    } else if (!keys->q_req && B > 0) {
        // contiguous pool: every row reads the same rows; nothing else to check
    }
    if (keys->chunk_ids) {
        if (!keys->n_chunks) return fail(IDX_E_ARG, "n_chunks is required with chunk_ids");
        if (keys->max_chunks <= 0) return fail(IDX_E_SHAPE, "max_chunks must be >= 1");
    }
    if (keys->n_pool_rows > ((int64_t)1 << 40)) return fail(IDX_E_SHAPE, "pool too large");
    return IDX_OK;
}

idx::ScoreArgs score_args(const uint16_t *q, const float *w, int32_t B, const idx_keys *keys,
                          int32_t n_cols) {
    idx::ScoreArgs a{};
    a.q = q;
    a.w = w;
    a.B = B;
    a.pool = keys->pool;
    a.n_pool_rows = keys->n_pool_rows;
    a.block_size = keys->block_size;
    a.block_table = keys->block_table;
    a.n_req = keys->n_req;
    a.max_blocks = keys->max_blocks;
    a.q_req = keys->q_req;
    a.chunk_ids = keys->chunk_ids;
    a.n_chunks = keys->n_chunks;
    a.max_chunks = keys->max_chunks;
    a.limits = keys->limits;
    a.status = keys->status;
    a.n_cols = n_cols;
    a.q_row = (int64_t)idx::kHeads * idx::kHeadDim;
    a.w_row = idx::kHeads;
    a.accum = false;
    // Launch shape: about one resident round of waves (256 CUs x 8 waves)
    // over the whole problem, at most one workgroup per row, so each wave
    // pays its start-up latency (bound, table, q) once and then streams
    // `slots_per_wave` blocks with its ring of loads in flight.
    const int64_t slots = (n_cols + idx::kBlock - 1) / idx::kBlock;
    const int64_t total = (int64_t)B * slots;
    int64_t spw = std::max<int64_t>(1, (total + 2047) / 2048);
    spw = std::min<int64_t>(spw, std::max<int64_t>(1, (slots + idx::kWaves - 1) / idx::kWaves));
    a.slots_per_wave = (int32_t)spw;
    a.splits = (int32_t)std::max<int64_t>(1, (slots + idx::kWaves * spw - 1) / (idx::kWaves * spw));
    return a;
}

int check_cols(int32_t n_cols) {
    if (n_cols < 1 || n_cols > IDX_MAX_COLS)
        return fail(IDX_E_SHAPE, "n_cols must be in [1, %d] (got %d)", IDX_MAX_COLS, n_cols);
    return IDX_OK;
}

int hip_fail(hipError_t e, const char *what) {
    return fail(IDX_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// The score kernel for H = 64 heads, or for H = 128 as two launches over the
// two halves of the heads: relu is per head, so the logit is the sum of the
// halves' weighted sums -- the first launch writes its logits (no scores),
// the second adds its own to them and writes the scores when asked.
hipError_t launch_heads(idx::ScoreArgs a, int32_t H, hipStream_t s) {
    if (H == idx::kHeads) return launch_score_timed(a, s);
    float *scores = a.scores;
    a.q_row = (int64_t)H * idx::kHeadDim;
    a.w_row = H;
    a.scores = nullptr;
    hipError_t e = launch_score_timed(a, s);
    if (e != hipSuccess) return e;
    a.q += (int64_t)idx::kHeads * idx::kHeadDim;
    a.w += idx::kHeads;
    a.accum = true;
    a.scores = scores;
    return launch_score_timed(a, s);
}

// q (bf16 [B, H, D], 16-byte aligned) or q8 (quantised rows [B, H, D + 4],
// 4-byte aligned): exactly one is used.
int check_qw8(const uint16_t *q, const uint8_t *q8, const float *w, int32_t B, int32_t H, int32_t D) {
    if (!q8) return check_qw(q, w, B, H, D);
    if (B < 0) return fail(IDX_E_ARG, "B must be >= 0 (got %d)", B);
    if (H != idx::kHeads || D != idx::kHeadDim)
        return fail(IDX_E_SHAPE, "only H=64, D=128 are supported (got H=%d, D=%d)", H, D);
    if (B > 0 && !w) return fail(IDX_E_ARG, "w must be non-null");
    if (!aligned(q8, 4) || !aligned(w, 16)) return fail(IDX_E_ALIGN, "q8 must be 4-byte and w 16-byte aligned");
    return IDX_OK;
}

// A bf16 query quantised inside the score kernel: bf16 q as for idx_score,
// 64 heads (the quantised path's operand holds one head block pair).
int check_qw_quant(const uint16_t *q, const float *w, int32_t B, int32_t H, int32_t D) {
    const int rc = check_qw(q, w, B, H, D);
    if (rc) return rc;
    if (H != idx::kHeads) return fail(IDX_E_SHAPE, "the in-kernel quantised query takes H=64 (got H=%d)", H);
    return IDX_OK;
}

int score_impl(const uint16_t *q, const uint8_t *q8, const float *w, int32_t B, int32_t H, int32_t D,
               const idx_keys *keys, int32_t n_cols, float *logits, float *scores, void *stream,
               bool quant_q = false, bool mx = false) {
    g_last_error[0] = 0;
    int rc = quant_q || mx ? check_qw_quant(q, w, B, H, D) : check_qw8(q, q8, w, B, H, D);
    if (rc) return rc;
    if ((rc = check_keys(keys, B))) return rc;
    if ((rc = check_cols(n_cols))) return rc;
    if (B == 0) return IDX_OK;
    if (q8 == nullptr && q == nullptr) return fail(IDX_E_ARG, "q must be non-null");
    if (!logits) return fail(IDX_E_ARG, "logits must be non-null");
    if (!aligned(logits, 16) || !aligned(scores, 4)) return fail(IDX_E_ALIGN, "logits must be 16-byte aligned");
    idx::ScoreArgs a = score_args(q, w, B, keys, n_cols);
    a.q8 = q8;
    a.quant_q = quant_q;
    a.mxfp4 = mx;
    a.ld = n_cols;
    a.logits = logits;
    a.scores = scores;
    hipError_t e = launch_heads(a, H, (hipStream_t)stream);
    return e == hipSuccess ? IDX_OK : hip_fail(e, "score kernel");
}

// Host-side checks of a score + top-k call; on success P is its plan.  A
// call with B == 0 passes with an empty plan (nothing to launch).
int score_topk_check(const uint16_t *q, const uint8_t *q8, const float *w, int32_t B, int32_t H, int32_t D,
                     const idx_keys *keys, int32_t n_cols, int32_t k, int32_t *out_idx, float *out_val,
                     TopkPlan &P, bool quant_q = false, bool mx = false) {
    int rc = quant_q || mx ? check_qw_quant(q, w, B, H, D) : check_qw8(q, q8, w, B, H, D);
    if (rc) return rc;
    if ((rc = check_keys(keys, B))) return rc;
    if ((rc = check_cols(n_cols))) return rc;
    if (k < 1 || k > idx::kMaxK) return fail(IDX_E_SHAPE, "k must be in [1, 2048] (got %d)", k);
    if (B == 0) return IDX_OK;
    if (q8 == nullptr && q == nullptr) return fail(IDX_E_ARG, "q must be non-null");
    if (!out_idx) return fail(IDX_E_ARG, "out_idx must be non-null");
    if (!aligned(out_idx, 4) || !aligned(out_val, 4)) return fail(IDX_E_ALIGN, "outputs must be 4-byte aligned");
    P = topk_plan(true, B, n_cols, k);
    return IDX_OK;
}

// Enqueue a checked score + top-k call (B > 0) on a workspace of P.total bytes.
int score_topk_launch(const uint16_t *q, const uint8_t *q8, const float *w, int32_t B, int32_t H,
                      const idx_keys *keys, int32_t n_cols, int32_t k, int32_t *out_idx, float *out_val,
                      const TopkPlan &P, char *ws, void *stream, bool quant_q = false, bool mx = false) {
    idx::ScoreArgs a = score_args(q, w, B, keys, n_cols);
    a.q8 = q8;
    a.quant_q = quant_q;
    a.mxfp4 = mx;
    a.ld = P.ld;
    a.logits = reinterpret_cast<float *>(ws + P.logits);
    a.scores = nullptr;
    a.row_cols = reinterpret_cast<uint32_t *>(ws + P.row_cols);
    a.row_done = reinterpret_cast<uint32_t *>(ws + P.row_done);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    // MXFP4 over many rows of one request: its key blocks are rounded once,
    // ahead of the score launch, instead of once per row in the tile loop
    if (mx && P.mx_blocks > 0 && keys->block_table && !keys->chunk_ids && keys->block_size == idx::kBlock &&
        keys->n_req == 1) {
        const int32_t nblk = std::min<int32_t>(keys->max_blocks, P.mx_blocks);
        uint8_t *mxk = reinterpret_cast<uint8_t *>(ws + P.mx);
        if ((e = idx::launch_mx_keys(a, mxk, nblk, s)) != hipSuccess) return hip_fail(e, "MXFP4 key rounding");
        a.mx_keys = mxk;
        a.mx_blocks = nblk;
    }
    if ((e = launch_heads(a, H, s)) != hipSuccess) return hip_fail(e, "score kernel");
    e = enqueue_topk(P, ws, a.logits, P.ld, a.row_cols, B, n_cols, k, out_idx, out_val,
                     keys->chunk_ids, keys->max_chunks, keys->block_size == idx::kSmallBlock ? 4 : 6, s);
    return e == hipSuccess ? IDX_OK : hip_fail(e, "top-k");
}

int score_topk_impl(const uint16_t *q, const uint8_t *q8, const float *w, int32_t B, int32_t H, int32_t D,
                    const idx_keys *keys, int32_t n_cols, int32_t k, int32_t *out_idx, float *out_val,
                    void *workspace, size_t ws_bytes, void *stream, bool quant_q = false, bool mx = false) {
    g_last_error[0] = 0;
    TopkPlan P;
    int rc = score_topk_check(q, q8, w, B, H, D, keys, n_cols, k, out_idx, out_val, P, quant_q, mx);
    if (rc || B == 0) return rc;
    if (P.total > 0 && (!workspace || ws_bytes < P.total))
        return fail(IDX_E_WORKSPACE, "workspace needs %zu bytes (got %zu)", P.total, ws_bytes);
    if (!aligned(workspace, 256)) return fail(IDX_E_ALIGN, "workspace must be 256-byte aligned");
    return score_topk_launch(q, q8, w, B, H, keys, n_cols, k, out_idx, out_val, P, static_cast<char *>(workspace),
                             stream, quant_q, mx);
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free entry point: a file-scope device array that
// holds idx_score_topk's workspace.  Every GPU the library runs on holds its
// own copy until the process ends.  In host code `scratch` is a host-side
// stand-in, not a device address: the address kernels may use comes from
// hipGetSymbolAddress, taken once per device with that device current and
// kept in g_scratch_ptr.  Nothing in it must start at zero (the score kernel
// clears the per-row counters the top-k's in-launch merge uses), and every
// call on a GPU overwrites what the last one left there.
static __device__ __align__(256) uint8_t scratch[IDX_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

int static_scratch(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(IDX_E_ARG, "device %d is beyond the %d this library tracks", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress of the static scratch");
        if (!p || !aligned(p, 256)) return fail(IDX_E_HIP, "the static scratch has no 256-byte aligned device address");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return IDX_OK;
}

}  // namespace

extern "C" {

int32_t idx_abi_version(void) { return IDX_ABI_VERSION; }

const char *idx_error_string(int32_t code) {
    switch (code) {
    case IDX_OK: return "ok";
    case IDX_E_ARG: return "invalid argument";
    case IDX_E_SHAPE: return "unsupported or inconsistent shape";
    case IDX_E_ALIGN: return "misaligned pointer";
    case IDX_E_WORKSPACE: return "workspace too small";
    case IDX_E_HIP: return "HIP launch failure";
    default: return "unknown error";
    }
}

const char *idx_last_error(void) { return g_last_error; }

int idx_profile_events(void *before, void *after) {
    g_ev_before = (before && after) ? static_cast<hipEvent_t>(before) : nullptr;
    g_ev_after = (before && after) ? static_cast<hipEvent_t>(after) : nullptr;
    return IDX_OK;
}

size_t idx_workspace_bytes(int32_t op, int32_t B, int32_t n_cols, int32_t k) {
    if (B < 0 || n_cols < 0 || n_cols > IDX_MAX_COLS || (op != IDX_OP_SCORE && (k < 1 || k > idx::kMaxK)))
        return (size_t)-1;
    switch (op) {
    case IDX_OP_SCORE: return 0;
    case IDX_OP_TOPK: return topk_plan(false, B, n_cols, k).total;
    case IDX_OP_SCORE_TOPK: return topk_plan(true, B, n_cols, k).total;
    default: return (size_t)-1;
    }
}

int idx_score(const uint16_t *q, const float *w, int32_t B, int32_t H, int32_t D,
              const idx_keys *keys, int32_t n_cols, float *logits, float *scores, void *stream) {
    return score_impl(q, nullptr, w, B, H, D, keys, n_cols, logits, scores, stream);
}

int idx_score_q8(const uint8_t *q8, const float *w, int32_t B, int32_t H, int32_t D, const idx_keys *keys,
                 int32_t n_cols, float *logits, float *scores, void *stream) {
    return score_impl(nullptr, q8, w, B, H, D, keys, n_cols, logits, scores, stream);
}

int idx_topk(const float *logits, int32_t B, int32_t n_cols, int64_t ld, int32_t k, int32_t *out_col,
             float *out_val, void *workspace, size_t ws_bytes, void *stream) {
    g_last_error[0] = 0;
    if (B < 0 || n_cols < 1 || ld < n_cols) return fail(IDX_E_SHAPE, "need B >= 0, n_cols >= 1, ld >= n_cols");
    if (check_cols(n_cols)) return IDX_E_SHAPE;
    if (k < 1 || k > idx::kMaxK) return fail(IDX_E_SHAPE, "k must be in [1, 2048] (got %d)", k);
    if (B == 0) return IDX_OK;
    if (!logits || !out_col) return fail(IDX_E_ARG, "logits and out_col must be non-null");
    if (!aligned(logits, 4) || !aligned(out_col, 4) || !aligned(out_val, 4))
        return fail(IDX_E_ALIGN, "logits/out_col/out_val must be 4-byte aligned");
    const TopkPlan P = topk_plan(false, B, n_cols, k);
    if (P.total > 0 && (!workspace || ws_bytes < P.total))
        return fail(IDX_E_WORKSPACE, "workspace needs %zu bytes (got %zu)", P.total, ws_bytes);
    if (!aligned(workspace, 256)) return fail(IDX_E_ALIGN, "workspace must be 256-byte aligned");
    hipError_t e = enqueue_topk(P, static_cast<char *>(workspace), logits, ld, nullptr, B, n_cols, k,
                                out_col, out_val, nullptr, 0, 6, (hipStream_t)stream);
    return e == hipSuccess ? IDX_OK : hip_fail(e, "top-k");
}

size_t idx_resident_workspace_bytes(int32_t n_layers, int32_t B, int32_t n_cols, int32_t kmax) {
    if (n_layers < 1 || n_layers > IDX_MAX_LAYERS || B < 0 || n_cols < 1 || n_cols > IDX_MAX_COLS || kmax < 1 ||
        kmax > idx::kMaxK)
        return (size_t)-1;
    return resident_plan(n_layers, B, n_cols, kmax).total;
}

int idx_select_resident(int32_t n_layers, const uint16_t *const *q, const float *const *w, int32_t B, int32_t H,
                        int32_t D, const idx_keys *keys, int32_t n_cols, const idx_resident_cfg *cfg,
                        int32_t *out_pages, int32_t *out_count, void *workspace, size_t ws_bytes, void *stream) {
    g_last_error[0] = 0;
    if (n_layers < 1 || n_layers > IDX_MAX_LAYERS)
        return fail(IDX_E_SHAPE, "n_layers must be in [1, %d] (got %d)", IDX_MAX_LAYERS, n_layers);
    if (!q || !w || !keys || !cfg) return fail(IDX_E_ARG, "q, w, keys and cfg must be non-null");
    if (check_cols(n_cols)) return IDX_E_SHAPE;
    if (cfg->ensemble != IDX_ENSEMBLE_MAX && cfg->ensemble != IDX_ENSEMBLE_MEAN)
        return fail(IDX_E_ARG, "ensemble must be IDX_ENSEMBLE_MAX or IDX_ENSEMBLE_MEAN");
    if (!(cfg->threshold == cfg->threshold)) return fail(IDX_E_ARG, "threshold is NaN");
    if (cfg->kmax < 1 || cfg->kmax > idx::kMaxK) return fail(IDX_E_SHAPE, "kmax must be in [1, 2048]");
    if (cfg->n_sink < 0 || cfg->n_recent < 0 || (int64_t)cfg->n_sink + cfg->n_recent > cfg->kmax)
        return fail(IDX_E_SHAPE, "need n_sink, n_recent >= 0 and n_sink + n_recent <= kmax");
    int rc;
    for (int l = 0; l < n_layers; ++l) {
        if ((rc = check_qw(q[l], w[l], B, H, D))) return rc;
        if ((rc = check_keys(&keys[l], B))) return rc;
        if (keys[l].chunk_ids) return fail(IDX_E_ARG, "Level-1 scoring takes no chunk lists (layer %d)", l);
    }
    if (B == 0) return IDX_OK;
    if (!out_pages) return fail(IDX_E_ARG, "out_pages must be non-null");
    if (!aligned(out_pages, 4) || !aligned(out_count, 4)) return fail(IDX_E_ALIGN, "outputs must be 4-byte aligned");
    const ResidentPlan R = resident_plan(n_layers, B, n_cols, cfg->kmax);
    if (!workspace || ws_bytes < R.total)
        return fail(IDX_E_WORKSPACE, "workspace needs %zu bytes (got %zu)", R.total, ws_bytes);
    if (!aligned(workspace, 256)) return fail(IDX_E_ALIGN, "workspace must be 256-byte aligned");
    char *ws = static_cast<char *>(workspace);
    float *scores = reinterpret_cast<float *>(ws + R.scores);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    idx::PageArgs pa{};
    // One score launch over every (layer, row) when the layers' queries and
    // weights are stacked ([L][B][H][D], [L][B][H]), they share one status
    // word, 64 heads and the max ensemble (an entry is selected iff some
    // layer's score reaches the threshold, so the launch only needs to
    // write each layer's selection bits); otherwise one launch per layer
    // writing scores.
    bool fused = n_layers > 1 && H == idx::kHeads && cfg->ensemble == IDX_ENSEMBLE_MAX &&
                 (int64_t)n_layers * B <= 512;
    for (int l = 1; fused && l < n_layers; ++l)
        fused = q[l] == q[0] + (int64_t)l * B * H * D && w[l] == w[0] + (int64_t)l * B * H &&
                keys[l].status == keys[0].status && keys[l].block_size == keys[0].block_size;
    if (fused) {
        idx::ScoreArgs a = score_args(q[0], w[0], n_layers * B, &keys[0], n_cols);
        a.rows_per_layer = B;
        for (int l = 0; l < n_layers; ++l) {
            idx::LayerKeys &k = a.layer[l];
            k.pool = keys[l].pool;
            k.n_pool_rows = keys[l].n_pool_rows;
            k.block_table = keys[l].block_table;
            k.n_req = keys[l].n_req;
            k.max_blocks = keys[l].max_blocks;
            k.q_req = keys[l].q_req;
            k.limits = keys[l].limits;
        }
        a.ld = R.ld;
        a.logits = nullptr;
        a.scores = nullptr;
        a.page_bits = reinterpret_cast<uint32_t *>(ws + R.scores);
        a.bits_ld = R.ld / 32;
        a.threshold = cfg->threshold;
        if ((e = launch_score_timed(a, s)) != hipSuccess) return hip_fail(e, "score kernel");
        pa.bits = a.page_bits;
        pa.bits_ld = a.bits_ld;
    }
    for (int l = 0; !fused && l < n_layers; ++l) {
        idx::ScoreArgs a = score_args(q[l], w[l], B, &keys[l], n_cols);
        a.ld = R.ld;
        // 64 heads: only the sigmoid scores are read later, so no logits
        // are stored; 128 heads keep them for the second head half
        a.logits = H == idx::kHeads ? nullptr : reinterpret_cast<float *>(ws + R.logits);
        a.scores = scores + (int64_t)l * B * R.ld;
        if ((e = launch_heads(a, H, s)) != hipSuccess) return hip_fail(e, "score kernel");
    }
    pa.scores = scores;
    pa.L = n_layers;
    pa.B = B;
    pa.ld = R.ld;
    pa.layer_stride = (int64_t)B * R.ld;
    pa.n_cols = n_cols;
    pa.limits = keys[0].limits;
    pa.ensemble = cfg->ensemble;
    pa.threshold = cfg->threshold;
    pa.n_sink = cfg->n_sink;
    pa.n_recent = cfg->n_recent;
    pa.page_keys = reinterpret_cast<float *>(ws + R.page_keys);
    pa.ldp = R.ldp;
    pa.n_pages = R.n_pages;
    if (fused) {
        // densities are small integers: one counting selection per row
        pa.kmax = cfg->kmax;
        pa.out_pages = out_pages;
        pa.out_count = out_count;
        e = idx::launch_select_bits(pa, s);
        return e == hipSuccess ? IDX_OK : hip_fail(e, "page selection");
    }
    if ((e = idx::launch_pages(pa, s)) != hipSuccess) return hip_fail(e, "page kernel");
    e = enqueue_topk(R.top, ws + R.topk, pa.page_keys, R.ldp, nullptr, B, R.n_pages, cfg->kmax, out_pages,
                     nullptr, nullptr, 0, 6, s, out_count);
    return e == hipSuccess ? IDX_OK : hip_fail(e, "page top-k");
}

int idx_write_keys(const uint16_t *k, int64_t n, int32_t D, const int64_t *slots, uint8_t *pool,
                   int64_t n_pool_rows, uint32_t *status, void *stream) {
    g_last_error[0] = 0;
    if (n < 0 || n_pool_rows < 0) return fail(IDX_E_ARG, "n and n_pool_rows must be >= 0");
    if (D != idx::kHeadDim) return fail(IDX_E_SHAPE, "only D=128 is supported (got D=%d)", D);
    // one workgroup per 16 keys: the grid's x extent bounds n
    if (n > (int64_t)INT32_MAX * 16) return fail(IDX_E_SHAPE, "too many keys in one call (%lld)", (long long)n);
    if (n == 0) return IDX_OK;
    if (!k || !slots) return fail(IDX_E_ARG, "k and slots must be non-null");
    if (n_pool_rows > 0 && !pool) return fail(IDX_E_ARG, "pool is null");
    if (!aligned(k, 16)) return fail(IDX_E_ALIGN, "k must be 16-byte aligned");
    if (!aligned(slots, 8) || !aligned(pool, 4) || !aligned(status, 4))
        return fail(IDX_E_ALIGN, "slots must be 8-byte aligned, pool and status 4-byte aligned");
    idx::WriteArgs a{};
    a.k = k;
    a.n = n;
    a.slots = slots;
    a.pool = pool;
    a.n_pool_rows = n_pool_rows;
    a.status = status;
    hipError_t e = idx::launch_write_keys(a, (hipStream_t)stream, g_ev_before, g_ev_after);
    return e == hipSuccess ? IDX_OK : hip_fail(e, "writer kernel");
}

int idx_score_topk(const uint16_t *q, const float *w, int32_t B, int32_t H, int32_t D,
                   const idx_keys *keys, int32_t n_cols, int32_t k, int32_t *out_idx, float *out_val,
                   void *workspace, size_t ws_bytes, void *stream) {
    return score_topk_impl(q, nullptr, w, B, H, D, keys, n_cols, k, out_idx, out_val, workspace, ws_bytes,
                           stream);
}

int idx_score_topk_noalloc(const uint16_t *q, const float *w, int32_t B, int32_t H, int32_t D,
                           const idx_keys *keys, int32_t n_cols, int32_t k, int32_t *out_idx, float *out_val,
                           void *stream) {
    g_last_error[0] = 0;
    TopkPlan P;
    int rc = score_topk_check(q, nullptr, w, B, H, D, keys, n_cols, k, out_idx, out_val, P);
    if (rc || B == 0) return rc;
    if (P.total > (size_t)IDX_STATIC_SCRATCH_BYTES)
        return fail(IDX_E_WORKSPACE,
                    "this call needs %zu bytes of scratch; the static scratch holds %zu "
                    "(call idx_score_topk with a workspace instead)",
                    P.total, (size_t)IDX_STATIC_SCRATCH_BYTES);
    void *ws = nullptr;
    if ((rc = static_scratch(&ws))) return rc;
    return score_topk_launch(q, nullptr, w, B, H, keys, n_cols, k, out_idx, out_val, P, static_cast<char *>(ws),
                             stream);
}

int idx_score_fp8q(const uint16_t *q, const float *w, int32_t B, int32_t H, int32_t D, const idx_keys *keys,
                   int32_t n_cols, float *logits, float *scores, void *stream) {
    return score_impl(q, nullptr, w, B, H, D, keys, n_cols, logits, scores, stream, true);
}

int idx_score_topk_fp8q(const uint16_t *q, const float *w, int32_t B, int32_t H, int32_t D, const idx_keys *keys,
                        int32_t n_cols, int32_t k, int32_t *out_idx, float *out_val, void *workspace,
                        size_t ws_bytes, void *stream) {
    return score_topk_impl(q, nullptr, w, B, H, D, keys, n_cols, k, out_idx, out_val, workspace, ws_bytes, stream,
                           true);
}

int idx_score_mxfp4(const uint16_t *q, const float *w, int32_t B, int32_t H, int32_t D, const idx_keys *keys,
                    int32_t n_cols, float *logits, float *scores, void *stream) {
    return score_impl(q, nullptr, w, B, H, D, keys, n_cols, logits, scores, stream, false, true);
}

int idx_score_topk_mxfp4(const uint16_t *q, const float *w, int32_t B, int32_t H, int32_t D, const idx_keys *keys,
                         int32_t n_cols, int32_t k, int32_t *out_idx, float *out_val, void *workspace,
                         size_t ws_bytes, void *stream) {
    return score_topk_impl(q, nullptr, w, B, H, D, keys, n_cols, k, out_idx, out_val, workspace, ws_bytes, stream,
                           false, true);
}

int idx_score_topk_q8(const uint8_t *q8, const float *w, int32_t B, int32_t H, int32_t D, const idx_keys *keys,
                      int32_t n_cols, int32_t k, int32_t *out_idx, float *out_val, void *workspace,
                      size_t ws_bytes, void *stream) {
    return score_topk_impl(nullptr, q8, w, B, H, D, keys, n_cols, k, out_idx, out_val, workspace, ws_bytes,
                           stream);
}

}  // extern "C"
