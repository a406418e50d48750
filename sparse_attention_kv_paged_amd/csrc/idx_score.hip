// Score kernel of the CSA indexer for gfx950 (MI355X).
//
// logit(b, e) = sum_h relu( sum_d k[e,d] * q[b,h,d] ) * w[b,h],
// k[e,d] = e4m3(byte) * scale      ("FlashMemory-DeepSeek-V4" README,
// "Retriever architecture" and "compressed_k format"; relu per head before
// the weighted head sum per the batchgen pull request's Phase 3 summary).
//
// Work decomposition: a workgroup is 4 independent waves on ONE query row;
// wave w of split s owns `slots_per_wave` consecutive 64-entry slots of that
// row's tile list ("DeepSeek-V4.1 native paged runtime", "Current execution
// scope": per-row bound + per-row tile list read in place).  A slot is one
// paged block, scored as two 32-entry tiles.
//
// Per tile, on MFMA v_mfma_f32_32x32x16_bf16 with heads as the 32 rows and
// entries as the 32 columns:
//   A (resident, registers) = q[b] as 2 head blocks x 8 k-steps of 16 dims
//   B (streamed)            = 32 key rows, each lane holding 64 contiguous
//                             fp8 bytes of one row, converted exactly to
//                             bf16 in registers (v_cvt_scalef32_pk_bf16_fp8,
//                             scale 1.0)
// The reduction index d is permuted identically in A and B: k-step kk, lane
// half hf covers d = 64*hf + 8*kk + 0..7, so each lane streams one contiguous
// 64-byte half row with four 16-byte loads and never re-reads it.
// The accumulator gives each lane 16 heads x 1 entry per head block, so the
// relu / head-weight / head-sum epilogue is 32 in-register FMAs plus one
// cross-half add.  The row scale s is applied after the head sum as
// |s| * sum_h relu(x_h) w_h, which equals the definition because
// relu(s x) = |s| relu(sign(s) x); for s < 0 the fp8 sign bits are flipped
// before conversion (exact).
#include "idx_device.h"
#include "idx_internal.h"

namespace idx {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

struct RowCtx {
    int32_t req;      // request row, -1 = padding
    int32_t nslots;   // slots of the tile list that may hold scored entries
    int32_t limit;    // bound on logical entry ids, clamped to capacity
};

__device__ __forceinline__ RowCtx row_context(const ScoreArgs &a, int b, uint32_t &st) {
    RowCtx r;
    r.req = a.q_req ? a.q_req[b] : b;
    r.limit = a.limits[b];
    r.nslots = 0;
    if (r.req >= 0 && a.block_table && r.req >= a.n_req) {
        st |= 0x4u;                                   // IDX_STATUS_BAD_REQUEST
        r.req = -1;
    }
    if (r.req < 0) return r;
    const int64_t cap = a.block_table ? (int64_t)a.max_blocks * kBlock : a.n_pool_rows;
    if ((int64_t)r.limit > cap) {
        st |= 0x1u;                                   // IDX_STATUS_LIMIT_CLAMPED
        r.limit = (int32_t)cap;
    }
    if (r.limit < 0) r.limit = 0;
    if (a.chunk_ids) {
        int32_t nc = a.n_chunks[b];
        if (nc > a.max_chunks) {
            st |= 0x8u;                               // IDX_STATUS_BAD_CHUNK
            nc = a.max_chunks;
        }
        r.nslots = nc < 0 ? 0 : nc;
    } else {
        r.nslots = (r.limit + kBlock - 1) / kBlock;
    }
    return r;
}

// First pool row of slot j of row b, or -1 when the slot's block is absent.
// *ebase receives the logical entry id of the slot's first entry.
__device__ __forceinline__ int64_t resolve_slot(const ScoreArgs &a, const RowCtx &r, int b,
                                                int j, int32_t &ebase, uint32_t &st) {
    int64_t beta = j;
    ebase = 0;
    if (r.req < 0 || j >= r.nslots) return -1;
    if (a.chunk_ids) {
        beta = a.chunk_ids[(int64_t)b * a.max_chunks + j];
        if (beta < 0) {
            if (beta != -1) st |= 0x8u;
            return -1;
        }
        if (a.block_table ? beta >= a.max_blocks : beta * kBlock >= a.n_pool_rows) {
            st |= 0x8u;
            return -1;
        }
    }
    ebase = (int32_t)(beta * kBlock);
    if (ebase >= r.limit) return -1;
    if (!a.block_table) return beta * kBlock;
    const int64_t pblk = a.block_table[(int64_t)r.req * a.max_blocks + beta];
    if (pblk < 0) {
        if (pblk != -1) st |= 0x2u;                   // IDX_STATUS_BAD_BLOCK
        return -1;
    }
    if ((pblk + 1) * kBlock > a.n_pool_rows) {
        st |= 0x2u;
        return -1;
    }
    return pblk * kBlock;
}

struct KeyHalf {
    u32x4 v[4];   // 64 fp8 bytes: d = 64*hf .. 64*hf + 63 of one key row
    float s;      // the row's scale
};

__device__ __forceinline__ KeyHalf load_key_half(const uint8_t *pool, int64_t prow, int hf) {
    const uint8_t *rp = pool + prow * kRowBytes;
    const u32x4_a4 *p = reinterpret_cast<const u32x4_a4 *>(rp + 64 * hf);
    KeyHalf k;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        u32x4_a4 t = p[i];
        k.v[i] = u32x4{t.x, t.y, t.z, t.w};
    }
    k.s = *reinterpret_cast<const float *>(rp + kHeadDim);
    return k;
}

// fp8 bytes [2*HI, 2*HI+1] of x -> two bf16 in one dword, exact (scale 1).
template <bool HI>
__device__ __forceinline__ uint32_t cvt_fp8x2_bf16x2(uint32_t x) {
    auto r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, HI);
    return __builtin_bit_cast(uint32_t, r);
}

// 8 fp8 bytes (two dwords) -> 8 bf16 (one MFMA operand), exact.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t d0, uint32_t d1) {
    u32x4 o{cvt_fp8x2_bf16x2<false>(d0), cvt_fp8x2_bf16x2<true>(d0),
            cvt_fp8x2_bf16x2<false>(d1), cvt_fp8x2_bf16x2<true>(d1)};
    return __builtin_bit_cast(bf16x8, o);
}

__device__ __forceinline__ int64_t readlane64(int64_t v, int lane) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), lane);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// One 32-entry tile: MFMA contraction, relu / head-weight / head-sum epilogue,
// scale and bound.  Returns the logit of entry (lane & 31) on every lane.
__device__ __forceinline__ float score_tile(KeyHalf k, const bf16x8 (&qa)[2][8],
                                            const float (&wr)[2][16], int e, int limit) {
    // relu(s x) = |s| relu(sign(s) x): flip the fp8 signs of rows with s < 0
    if (__any(k.s < 0.f)) {
        const uint32_t m = (k.s < 0.f) ? 0x80808080u : 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) k.v[i] ^= u32x4{m, m, m, m};
    }
    f32x16 acc0 = {}, acc1 = {};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        const u32x4 &v = k.v[kk >> 1];
        const bf16x8 kb = (kk & 1) ? fp8x8_to_bf16x8(v.z, v.w) : fp8x8_to_bf16x8(v.x, v.y);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][kk], kb, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][kk], kb, acc1, 0, 0, 0);
    }
    float T = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) T = fmaf(fmaxf(acc0[i], 0.f), wr[0][i], T);
#pragma unroll
    for (int i = 0; i < 16; ++i) T = fmaf(fmaxf(acc1[i], 0.f), wr[1][i], T);
    T += __shfl_xor(T, 32, 64);
    return e < limit ? fabsf(k.s) * T : -__builtin_inff();
}

constexpr int kRing = 3;   // key tiles in flight per wave

template <bool OWN_COLS>
__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a) {
    const int b = blockIdx.x / a.splits;
    const int split = blockIdx.x - b * a.splits;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int hf = lane >> 5;
    const int n32 = lane & 31;

    uint32_t st = 0;
    const RowCtx r = row_context(a, b, st);
    const int slot_cols = (a.n_cols + kBlock - 1) / kBlock;
    // OWN_COLS: write only the columns the row's tile list can reach (the
    // top-k reads exactly those); otherwise every column up to n_cols.
    const int col_end = OWN_COLS ? max(0, min(r.nslots * kBlock, a.n_cols)) : a.n_cols;
    const int slot_stop = OWN_COLS ? min(r.nslots, slot_cols) : slot_cols;
    if (OWN_COLS && split == 0 && threadIdx.x == 0) a.row_cols[b] = (uint32_t)col_end;

    const int slot0 = (split * kWaves + wave) * a.slots_per_wave;
    const int slot_end = min(slot0 + a.slots_per_wave, slot_stop);
    if (slot0 >= slot_end) {
        if (st && a.status && lane == 0) atomicOr(a.status, st);
        return;
    }
    float *out_row = a.logits + (int64_t)b * a.ld;
    float *score_row = a.scores ? a.scores + (int64_t)b * a.ld : nullptr;
    const bool live = r.req >= 0 && slot0 < r.nslots;
    const int64_t last_row = a.n_pool_rows - 1;

    // Block-table resolution, 64 slots at a time: lane j resolves slot j of
    // the current group with vector loads; tiles read it back with readlane.
    int cached_group = -1;
    int64_t lane_prow0 = -1;
    int32_t lane_ebase = 0;
    auto slot_info = [&](int j, int64_t &prow0, int32_t &ebase) {
        const int grp = (j - slot0) >> 6;
        if (grp != cached_group) {
            cached_group = grp;
            const int js = slot0 + (grp << 6) + lane;
            lane_prow0 = -1;
            lane_ebase = 0;
            if (live && js < slot_end) lane_prow0 = resolve_slot(a, r, b, js, lane_ebase, st);
        }
        const int src = (j - slot0) & 63;
        prow0 = readlane64(lane_prow0, src);
        ebase = __builtin_amdgcn_readlane(lane_ebase, src);
    };

    // Resident operands: q[b] (A fragments) and the head weights matching
    // this lane's accumulator rows.
    bf16x8 qa[2][8];
    float wr[2][16];
    if (live) {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            const u32x4 *qp = reinterpret_cast<const u32x4 *>(
                a.q + ((int64_t)b * kHeads + 32 * hb + n32) * kHeadDim + 64 * hf);
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) qa[hb][kk] = __builtin_bit_cast(bf16x8, qp[kk]);
            // accumulator register i holds head 32*hb + 8*(i/4) + 4*hf + i%4
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 wv = *reinterpret_cast<const float4 *>(
                    a.w + (int64_t)b * kHeads + 32 * hb + 8 * g + 4 * hf);
                wr[hb][4 * g + 0] = wv.x;
                wr[hb][4 * g + 1] = wv.y;
                wr[hb][4 * g + 2] = wv.z;
                wr[hb][4 * g + 3] = wv.w;
            }
        }
    }

    const int ntiles = 2 * (slot_end - slot0);
    // ring of kRing tiles in flight: tile tau lives in ring slot tau % kRing
    KeyHalf kv[kRing];
    int64_t prow_t[kRing];
    int32_t ebase_t[kRing];
    auto issue = [&](int tau, KeyHalf &dst, int64_t &prow0, int32_t &ebase) {
        prow0 = -1;
        ebase = 0;
        if (tau >= ntiles) return;
        slot_info(slot0 + (tau >> 1), prow0, ebase);
        if (prow0 >= 0) dst = load_key_half(a.pool, min(prow0 + 32 * (tau & 1) + n32, last_row), hf);
    };
    auto consume = [&](int tau, const KeyHalf &src, int64_t prow0, int32_t ebase) {
        if (tau >= ntiles) return;
        const int t = tau & 1;
        const int col = (slot0 + (tau >> 1)) * kBlock + 32 * t + n32;
        float logit = -__builtin_inff();
        if (prow0 >= 0) logit = score_tile(src, qa, wr, ebase + 32 * t + n32, r.limit);
        if (hf == 0 && col < col_end) {
            out_row[col] = logit;
            if (score_row) score_row[col] = 1.0f / (1.0f + expf(-logit));
        }
    };
#pragma unroll
    for (int i = 0; i < kRing; ++i) issue(i, kv[i], prow_t[i], ebase_t[i]);
    for (int base = 0; base < ntiles; base += kRing) {
#pragma unroll
        for (int i = 0; i < kRing; ++i) {
            consume(base + i, kv[i], prow_t[i], ebase_t[i]);
            issue(base + i + kRing, kv[i], prow_t[i], ebase_t[i]);
        }
    }
    if (st && a.status) atomicOr(a.status, st);
}

}  // namespace

hipError_t launch_score(const ScoreArgs &a, hipStream_t s) {
    const int64_t grid = (int64_t)a.B * a.splits;
    if (grid <= 0) return hipSuccess;
    if (a.row_cols)
        hipLaunchKernelGGL(score_kernel<true>, dim3((unsigned)grid), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(score_kernel<false>, dim3((unsigned)grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace idx
