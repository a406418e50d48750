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
// scope": per-row bound + per-row tile list read in place).  A slot is 64
// entries -- one 64-row pool block, or four 16-row blocks (the same page's
// index rows under 16-row block ids) -- scored as two 32-entry tiles.
//
// Per tile, on MFMA v_mfma_f32_32x32x16_bf16 with heads as the 32 rows and
// entries as the 32 columns:
//   A (resident, registers) = q[b] as 2 head blocks x 8 k-steps of 16 dims
//   B (streamed)            = 32 key rows, each lane holding 64 contiguous
//                             fp8 bytes of one row, converted exactly to
//                             bf16 in registers (v_cvt_scalef32_pk_bf16_fp8,
//                             scale 1.0)
// The reduction index d is permuted identically in A and B: k-step kk, lane
// half hf covers d = 64*hf + 8*kk + 0..7.  Key tiles reach LDS by
// buffer-to-LDS loads that each read eight whole consecutive rows (a per-wave
// two-slot ring), and each lane then reads its 64-byte half row from LDS.
// The accumulator gives each lane 16 heads x 1 entry per head block, so the
// relu / head-weight / head-sum epilogue is 32 in-register FMAs plus one
// cross-half add.  The row scale s is applied after the head sum as
// |s| * sum_h relu(x_h) w_h, which equals the definition because
// relu(s x) = |s| relu(sign(s) x); for s < 0 the fp8 sign bits are flipped
// before conversion (exact).  The tile loop is a two-stage pipeline: tile
// t's MFMAs are interleaved with tile t-1's epilogue, because the VALU work
// per tile (conversion + epilogue) is close to the MFMA time and the two
// only overlap when they sit in one straight-line stretch of code.
#include <algorithm>
#include <type_traits>

#include <hip/hip_ext.h>

#include "idx_device.h"
#include "idx_internal.h"
#include "idx_quant.h"

namespace idx {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
// 16 bytes at a 4-byte aligned address (q8 rows are 132 bytes apart)
typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));

// q[b] as the MFMA's A operand.  bf16 path: 2 head blocks x 8 k-steps of 8
// bf16 (v_mfma_f32_32x32x16_bf16).  fp8 path (quantised q): 2 head blocks x
// 2 k-steps of 32 e4m3 bytes (v_mfma_scale_f32_32x32x64_f8f6f4, scales 1).
struct QBf16 {
    bf16x8 v[2][8];
};
struct QFp8 {
    v8i v[2][2];
    float qs;       // the quantisation scale of head `lane` (the head whose weight the lane holds)
};
// MXFP4 path (query and key rounded to MXFP4 blocks of 32 in the kernel):
// 2 head blocks x 2 k-steps of 32 e2m1 codes (16 bytes, value j in nibble
// j % 8 of dword j / 8, low nibble first), and per head block the E8M0
// scales of the lane's two 32-value blocks (byte kk for k-step kk), for
// v_mfma_scale_f32_32x32x64_f8f6f4 with both operands e2m1.
struct QFp4 {
    u32x4 v[2][2];
    uint32_t sc[2];
};
template <bool Q8, bool MX = false> struct QSel {
    using Op = QBf16;
};
template <> struct QSel<true, false> {
    using Op = QFp8;
};
template <bool Q8> struct QSel<Q8, true> {
    using Op = QFp4;
};

struct RowCtx {
    int32_t req;      // request row, -1 = padding
    int32_t nslots;   // 64-column slots of the tile list that may hold scored entries
    int32_t nunits;   // pool blocks of the tile list (= nslots for 64-row blocks)
    int32_t limit;    // bound on logical entry ids, clamped to capacity
};

// A row's inputs (request, bound, chunk count), read without branches so
// that they are in flight together: absent arrays get empty descriptors,
// which read 0, and so do rows >= B.
struct RowRaw {
    int32_t qreq, limit, nchunks;
};

// The arguments row v of a launch sees: the launch's own, or, when it scores
// several layers, the same with the keys of row v's layer (bl: the row's
// index within its layer, for that layer's per-row arrays).
__device__ __forceinline__ ScoreArgs key_view(const ScoreArgs &a, int v, int &bl) {
    bl = v;
    if (a.rows_per_layer <= 0) return a;
    const int l = v / a.rows_per_layer;
    bl = v - l * a.rows_per_layer;
    ScoreArgs k = a;
    const LayerKeys &L = a.layer[l];
    k.pool = L.pool;
    k.n_pool_rows = L.n_pool_rows;
    k.block_table = L.block_table;
    k.n_req = L.n_req;
    k.max_blocks = L.max_blocks;
    k.q_req = L.q_req;
    k.limits = L.limits;
    k.B = a.rows_per_layer;
    return k;
}

__device__ __forceinline__ RowRaw row_raw(const ScoreArgs &a, int b) {
    const uint32_t nb = (uint32_t)a.B * 4u, off = (uint32_t)b * 4u;
    RowRaw r;
    r.qreq = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.q_req, a.q_req ? nb : 0u), off, 0, 0);
    r.limit = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.limits, nb), off, 0, 0);
    r.nchunks = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.n_chunks, a.chunk_ids ? nb : 0u), off, 0, 0);
    if (!a.q_req) r.qreq = b;
    return r;
}

// BS: rows per pool block (64, or 16: four blocks make one 64-column slot).
template <int BS>
__device__ __forceinline__ RowCtx row_context(const ScoreArgs &a, const RowRaw &raw, uint32_t &st) {
    constexpr int U = kBlock / BS;
    RowCtx r;
    r.req = raw.qreq;
    r.limit = raw.limit;
    r.nslots = 0;
    r.nunits = 0;
    if (r.req >= 0 && a.block_table && r.req >= a.n_req) {
        st |= 0x4u;                                   // IDX_STATUS_BAD_REQUEST
        r.req = -1;
    }
    if (r.req < 0) return r;
    const int64_t cap = a.block_table ? (int64_t)a.max_blocks * BS : a.n_pool_rows;
    if ((int64_t)r.limit > cap) {
        st |= 0x1u;                                   // IDX_STATUS_LIMIT_CLAMPED
        r.limit = (int32_t)cap;
    }
    if (r.limit < 0) r.limit = 0;
    if (a.chunk_ids) {
        int32_t nc = raw.nchunks;
        if (nc > a.max_chunks) {
            st |= 0x8u;                               // IDX_STATUS_BAD_CHUNK
            nc = a.max_chunks;
        }
        r.nunits = nc < 0 ? 0 : nc;
    } else {
        r.nunits = (int32_t)(((int64_t)r.limit + BS - 1) / BS);
    }
    r.nslots = (r.nunits + U - 1) / U;
    return r;
}

constexpr uint32_t kDrop = 0x7FFFFFF0u;               // a byte offset every descriptor rejects

// The table reads of slot j (lane_ok: the lane holds a slot), issued under
// bounds the host guarantees (j < max_chunks, beta < max_blocks,
// req < n_req) through buffer descriptors, without branches, so that later
// loads go out before these are waited on.  CHUNKED: the slot's logical
// block comes from the row's chunk list, a read the table read depends on.
struct SlotRaw {
    int32_t beta;   // logical block (chunk id), -1 if none
    int32_t p;      // the table's entry, valid when tok
    bool tok;       // the table was read (else: no pool block)
};

template <bool CHUNKED>
__device__ __forceinline__ SlotRaw slot_raw(const ScoreArgs &a, int req, int b, int j, bool lane_ok) {
    SlotRaw s{j, -1, false};
    if (CHUNKED) {
        const bool ok = lane_ok && j < a.max_chunks;
        const __amdgpu_buffer_rsrc_t cr =
            make_rsrc(a.chunk_ids + (int64_t)b * a.max_chunks, (uint32_t)a.max_chunks * 4u);
        const int32_t c = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(cr, ok ? (uint32_t)j * 4u : kDrop, 0, 0);
        s.beta = ok ? c : -1;
    }
    s.tok = lane_ok && a.block_table && req >= 0 && req < a.n_req && s.beta >= 0 && s.beta < a.max_blocks;
    const __amdgpu_buffer_rsrc_t tr =
        make_rsrc(a.block_table + (int64_t)max(req, 0) * a.max_blocks, a.block_table ? (uint32_t)a.max_blocks * 4u : 0u);
    // the value is only looked at in resolve_slot, so this read stays in
    // flight across whatever the caller issues in between
    s.p = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(tr, s.tok ? (uint32_t)s.beta * 4u : kDrop, 0, 0);
    return s;
}

// First pool row of pool block j (of BS rows) of row b's tile list, or -1
// when the block is absent (or !ok: the lane holds no block).  *ebase
// receives the logical entry id of the block's first entry.  Straight-line
// selects, no branches, so the wait for the table read is the only one the
// compiler needs here.
template <int BS>
__device__ __forceinline__ int64_t resolve_slot(const ScoreArgs &a, const RowCtx &r, const SlotRaw &raw,
                                                int j, bool ok, int32_t &ebase, uint32_t &st) {
    const int64_t beta = raw.beta;
    ok = ok && r.req >= 0 && j < r.nunits;
    uint32_t bad = 0;
    if (a.chunk_ids) {
        const bool beyond = a.block_table ? beta >= a.max_blocks : beta * BS >= a.n_pool_rows;
        bad |= (ok && (beta < -1 || (beta >= 0 && beyond))) ? 0x8u : 0u;        // IDX_STATUS_BAD_CHUNK
        ok = ok && beta >= 0 && !beyond;
    }
    ebase = (int32_t)(beta * BS);
    ok = ok && ebase < r.limit;
    int64_t prow = beta * BS;
    if (a.block_table) {
        const int64_t pblk = raw.tok ? raw.p : -1;
        const bool past = (pblk + 1) * BS > a.n_pool_rows;
        bad |= (ok && (pblk < -1 || (pblk >= 0 && past))) ? 0x2u : 0u;         // IDX_STATUS_BAD_BLOCK
        ok = ok && pblk >= 0 && !past;
        prow = pblk * BS;
    }
    st |= bad;
    return ok ? prow : -1;
}

struct KeyHalf {
    u32x4 v[4];   // 64 fp8 bytes: d = 64*hf .. 64*hf + 63 of one key row
    float s;      // the row's scale
};

// Key tiles travel from memory straight into a per-wave LDS ring
// (buffer_load ... lds: lane l of a load lands at byte 16*l -- or 4*l for a
// 4-byte load -- of the destination, no registers involved).  Load i of a
// 32-row tile brings rows 8*i .. 8*i + 7 whole, so every load instruction
// reads ~1 KB of consecutive bytes; lane l takes 16-byte chunk
// c = (l & 7) ^ (l >> 3) of row 8*i + (l >> 3).  In LDS, chunk c of tile
// row n is granule 8*n + (c ^ (n & 7)): the eight rows that eight
// consecutive lanes read back sit in eight different bank groups.  A fifth
// load puts the 32 row scales (twice: lanes 32-63 repeat lanes 0-31) after
// the fp8 bytes.  With 16-row pool blocks a tile spans two blocks, each
// with a descriptor of its own: loads 0-1 read the first, loads 2-3 the
// second, and each block's 16 scales come with a load of their own (64
// lanes, rows repeated four times), the second block's 256 bytes further on.
constexpr int kTileFp8 = 32 * kHeadDim;                // one tile's fp8 bytes in LDS
template <int BS> constexpr int tile_bytes() {         // + the scales
    return kTileFp8 + (BS == kBlock ? 64 : 128) * 4;
}
template <int BS> constexpr int loads_per_tile() { return BS == kBlock ? 5 : 6; }

// The lane's byte offset (within a tile) of the chunk it loads with load 0.
__device__ __forceinline__ uint32_t tile_load_offset(int lane) {
    return (uint32_t)(lane >> 3) * kRowBytes + 16u * (uint32_t)((lane & 7) ^ (lane >> 3));
}

// Issue the five loads of the tile whose first row is at byte t0 of the
// block described by r into the LDS slot dst.
__device__ __forceinline__ void load_tile(__amdgpu_buffer_rsrc_t r, uint32_t t0, uint32_t lo, uint8_t *dst) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)(dst + 1024 * i), 16,
                                                 t0 + lo + 8u * kRowBytes * i, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)(dst + kTileFp8), 4,
                                             t0 + (uint32_t)(threadIdx.x & 31) * kRowBytes + kHeadDim, 0, 0, 0);
}

// The six loads of a tile made of two 16-row pool blocks (ra: tile rows
// 0-15, rb: rows 16-31); lo as for load_tile.
__device__ __forceinline__ void load_tile16(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, uint32_t lo,
                                            uint8_t *dst) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (__attribute__((address_space(3))) void *)(dst + 1024 * i), 16,
                                                 lo + 8u * kRowBytes * i, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 2; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (__attribute__((address_space(3))) void *)(dst + 1024 * (i + 2)),
                                                 16, lo + 8u * kRowBytes * i, 0, 0, 0);
    const uint32_t so = (uint32_t)(threadIdx.x & 15) * kRowBytes + kHeadDim;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (__attribute__((address_space(3))) void *)(dst + kTileFp8), 4, so, 0,
                                             0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (__attribute__((address_space(3))) void *)(dst + kTileFp8 + 256), 4,
                                             so, 0, 0, 0);
}

// The lane's half row (lane >> 5) of tile row (lane & 31), and that row's
// scale, from an LDS slot.
template <int BS>
__device__ __forceinline__ void read_tile(const uint8_t *slot, KeyHalf &k) {
    const int lane = threadIdx.x & 63, n = lane & 31, hf = lane >> 5;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        k.v[j] = *reinterpret_cast<const u32x4 *>(slot + 128 * n + 16 * ((4 * hf + j) ^ (n & 7)));
    const int si = BS == kBlock ? lane : (n & 15) + 64 * (n >> 4);
    k.s = *reinterpret_cast<const float *>(slot + kTileFp8 + 4 * si);
}

// The compiler does not see that an LDS read depends on a buffer-to-LDS
// load, so the ring's waits are explicit, and each is also a compiler
// barrier for memory operations.  The barriers around q's staging and
// quantisation only order LDS data between the waves (lds_barrier: the
// first key tiles of the ring stay in flight).

template <int N>
__device__ __forceinline__ void wait_vmem() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

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

// A tile's contraction result: for head block hb, accumulator register i
// of lane (hf, n) is head 32*hb + 8*(i/4) + 4*hf + i%4 against entry n.
struct TileAcc {
    f32x16 h0, h1;
};

// MFMA half of one 32-entry tile: exact fp8 -> bf16 widening and the
// contraction over the 128 dims, for both head blocks.
__device__ __forceinline__ void tile_mma(KeyHalf &k, const QBf16 &qa, TileAcc &acc) {
    // relu(s x) = |s| relu(sign(s) x): flip the fp8 signs of rows with s < 0
    if (__any(k.s < 0.f)) {
        const uint32_t m = (k.s < 0.f) ? 0x80808080u : 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) k.v[i] ^= u32x4{m, m, m, m};
    }
    acc.h0 = f32x16{};
    acc.h1 = f32x16{};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        const u32x4 &v = k.v[kk >> 1];
        const bf16x8 kb = (kk & 1) ? fp8x8_to_bf16x8(v.z, v.w) : fp8x8_to_bf16x8(v.x, v.y);
        acc.h0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa.v[0][kk], kb, acc.h0, 0, 0, 0);
        acc.h1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa.v[1][kk], kb, acc.h1, 0, 0, 0);
    }
}

// The same with quantised q: both operands e4m3, so the key bytes feed the
// MFMA as they are (no widening); k-step kk covers d = 64*hf + 32*kk + 0..31
// in q and keys alike.  Products of two e4m3 values are exact in fp32.
__device__ __forceinline__ void tile_mma(KeyHalf &k, const QFp8 &qa, TileAcc &acc) {
    if (__any(k.s < 0.f)) {
        const uint32_t m = (k.s < 0.f) ? 0x80808080u : 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) k.v[i] ^= u32x4{m, m, m, m};
    }
    const v8i b0 = {(int)k.v[0].x, (int)k.v[0].y, (int)k.v[0].z, (int)k.v[0].w,
                    (int)k.v[1].x, (int)k.v[1].y, (int)k.v[1].z, (int)k.v[1].w};
    const v8i b1 = {(int)k.v[2].x, (int)k.v[2].y, (int)k.v[2].z, (int)k.v[2].w,
                    (int)k.v[3].x, (int)k.v[3].y, (int)k.v[3].z, (int)k.v[3].w};
    const f32x16 z = {};
    // format 0 = e4m3 for both operands; E8M0 scales 127 = 1.0
    acc.h0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa.v[0][0], b0, z, 0, 0, 0, 127, 0, 127);
    acc.h1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa.v[1][0], b0, z, 0, 0, 0, 127, 0, 127);
    acc.h0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa.v[0][1], b1, acc.h0, 0, 0, 0, 127, 0, 127);
    acc.h1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa.v[1][1], b1, acc.h1, 0, 0, 0, 127, 0, 127);
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// One MXFP4 block ("DeepSeek-V4.1 native paged runtime", "Current execution
// scope": the published model rounds index query and key to FP4; the format
// is OCP MXFP4): 32 bf16 values (raw: 16 dwords of two values, the lower
// half first) -> 32 e2m1 codes and the block's E8M0 scale byte e + 127, with
// e = floor(log2(amax)) - 2 clamped to >= -127.  Each code is the nearest
// e2m1 value of v / 2^e, ties to even, saturating at 6: the packed
// conversion divides by its scale operand and rounds so.  Blocks with
// e = -127 (amax < 2^-124, zero blocks included) are converted from binary32
// values scaled by 2^64 against 2^-63, so the scale operand stays normal
// (both products exact).
template <int SEL>
__device__ __forceinline__ uint32_t fp4_pair(uint32_t d, uint32_t raw, float scale) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(d, __builtin_bit_cast(bf16x2, raw), scale, SEL);
}
template <int SEL>
__device__ __forceinline__ uint32_t fp4_pair_f32(uint32_t d, float lo, float hi, float scale) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, lo, hi, scale, SEL);
}
__device__ __forceinline__ uint32_t mx_block_bf16(const uint32_t (&raw)[16], u32x4 &codes) {
    // bf16 magnitudes order like their bit patterns: a packed 16-bit max
    u16x2 m2 = {0, 0};
#pragma unroll
    for (int i = 0; i < 16; ++i)
        m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, raw[i] & 0x7FFF7FFFu));
    const uint32_t amax = m2.x > m2.y ? m2.x : m2.y;
    const int ex = (int)(amax >> 7);                 // biased exponent of the block's amax
    const int e = max(ex - 129, -127);
    uint32_t d[4];
    if (e > -127) {
        const float scale = __uint_as_float((uint32_t)(e + 127) << 23);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t x = fp4_pair<0>(0u, raw[4 * w], scale);
            x = fp4_pair<1>(x, raw[4 * w + 1], scale);
            x = fp4_pair<2>(x, raw[4 * w + 2], scale);
            d[w] = fp4_pair<3>(x, raw[4 * w + 3], scale);
        }
    } else {
        const float scale = 0x1p-63f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t x = 0u;
            const float l0 = __uint_as_float(raw[4 * w] << 16) * 0x1p64f;
            const float h0 = __uint_as_float(raw[4 * w] & 0xFFFF0000u) * 0x1p64f;
            const float l1 = __uint_as_float(raw[4 * w + 1] << 16) * 0x1p64f;
            const float h1 = __uint_as_float(raw[4 * w + 1] & 0xFFFF0000u) * 0x1p64f;
            const float l2 = __uint_as_float(raw[4 * w + 2] << 16) * 0x1p64f;
            const float h2 = __uint_as_float(raw[4 * w + 2] & 0xFFFF0000u) * 0x1p64f;
            const float l3 = __uint_as_float(raw[4 * w + 3] << 16) * 0x1p64f;
            const float h3 = __uint_as_float(raw[4 * w + 3] & 0xFFFF0000u) * 0x1p64f;
            x = fp4_pair_f32<0>(x, l0, h0, scale);
            x = fp4_pair_f32<1>(x, l1, h1, scale);
            x = fp4_pair_f32<2>(x, l2, h2, scale);
            d[w] = fp4_pair_f32<3>(x, l3, h3, scale);
        }
    }
    codes = u32x4{d[0], d[1], d[2], d[3]};
    return (uint32_t)(e + 127);
}

__device__ __forceinline__ v8i fp4_operand(const u32x4 &x) {
    return v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
}

// The MXFP4 path: the lane's 64 key bytes are its two 32-value blocks
// (d = 64*hf + 32*kk + 0..31 for k-step kk, as in q); each is widened
// exactly to bf16, rounded to an MXFP4 block, and the contraction runs on
// e2m1 operands with the blocks' E8M0 scales.  The row scale stays outside
// (its sign flipped into the fp8 bytes first, as in tile_mma above).
__device__ __forceinline__ void tile_mma(KeyHalf &k, const QFp4 &qa, TileAcc &acc) {
    if (__any(k.s < 0.f)) {
        const uint32_t m = (k.s < 0.f) ? 0x80808080u : 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) k.v[i] ^= u32x4{m, m, m, m};
    }
    u32x4 kc[2];
    uint32_t ksc = 0;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        uint32_t raw[16];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const u32x4 &x = k.v[2 * blk + j];
            const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                raw[8 * j + 2 * i] = cvt_fp8x2_bf16x2<false>(w4[i]);
                raw[8 * j + 2 * i + 1] = cvt_fp8x2_bf16x2<true>(w4[i]);
            }
        }
        ksc |= mx_block_bf16(raw, kc[blk]) << (8 * blk);
    }
    const f32x16 z = {};
    // format 4 = e2m1 for both operands; op_sel picks scale byte kk
    acc.h0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp4_operand(qa.v[0][0]), fp4_operand(kc[0]), z, 4, 4, 0,
                                                            (int)qa.sc[0], 0, (int)ksc);
    acc.h1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp4_operand(qa.v[1][0]), fp4_operand(kc[0]), z, 4, 4, 0,
                                                            (int)qa.sc[1], 0, (int)ksc);
    acc.h0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp4_operand(qa.v[0][1]), fp4_operand(kc[1]), acc.h0, 4,
                                                            4, 1, (int)qa.sc[0], 1, (int)ksc);
    acc.h1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp4_operand(qa.v[1][1]), fp4_operand(kc[1]), acc.h1, 4,
                                                            4, 1, (int)qa.sc[1], 1, (int)ksc);
}

// Pre-rounded MXFP4 keys (ScoreArgs::mx_keys, written by mx_keys_kernel): a
// 32-row tile in LDS holds the rows' code bytes -- 16-byte chunk c of row n
// at granule 4n + (c ^ ((n >> 2) & 3)), so that the 16 lanes of a read pass
// reach 16 different bank groups -- then the rows' E8M0 scale words, then
// their row scales: 2304 bytes, brought by three loads.
constexpr int kMxTileBytes = 32 * 64 + 32 * 4 + 32 * 4;

struct KeyMx {
    u32x4 kc[2];    // the codes of the lane's two 32-value blocks (d = 64*hf + 32*kk ..)
    uint32_t ksc;   // their E8M0 scales in bytes 0 and 1
    float s;        // the row's scale (a negative one's sign is in the codes)
};

// Issue the three loads of tile half `half` (rows 32*half .. 32*half + 31)
// of the pre-rounded block described by r into the LDS slot dst.
__device__ __forceinline__ void load_tile_mx(__amdgpu_buffer_rsrc_t r, int half, uint8_t *dst) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int p = 64 * i + lane;                  // the LDS granule this lane fills
        const int n = p >> 2, c = (p & 3) ^ ((n >> 2) & 3);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)(dst + 1024 * i), 16,
                                                 (uint32_t)(2048 * half + 64 * n + 16 * c), 0, 0, 0);
    }
    // lanes 0-31: the rows' scale words; lanes 32-63: their row scales
    const uint32_t so = lane < 32 ? (uint32_t)(4096 + 128 * half + 4 * lane)
                                  : (uint32_t)(4352 + 128 * half + 4 * (lane - 32));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)(dst + 2048), 4, so, 0, 0, 0);
}

__device__ __forceinline__ void read_tile(const uint8_t *slot, KeyMx &k) {
    const int lane = threadIdx.x & 63, n = lane & 31, hf = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
        k.kc[kk] = *reinterpret_cast<const u32x4 *>(slot + 16 * (4 * n + ((2 * hf + kk) ^ ((n >> 2) & 3))));
    k.ksc = *reinterpret_cast<const uint32_t *>(slot + 2048 + 4 * n) >> (16 * hf);
    k.s = *reinterpret_cast<const float *>(slot + 2176 + 4 * n);
}

// The MXFP4 contraction on codes rounded ahead: the same four MFMAs as
// tile_mma(KeyHalf &, const QFp4 &, ...) on the same operands.
__device__ __forceinline__ void tile_mma(const KeyMx &k, const QFp4 &qa, TileAcc &acc) {
    const f32x16 z = {};
    acc.h0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp4_operand(qa.v[0][0]), fp4_operand(k.kc[0]), z, 4, 4, 0,
                                                            (int)qa.sc[0], 0, (int)k.ksc);
    acc.h1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp4_operand(qa.v[1][0]), fp4_operand(k.kc[0]), z, 4, 4, 0,
                                                            (int)qa.sc[1], 0, (int)k.ksc);
    acc.h0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp4_operand(qa.v[0][1]), fp4_operand(k.kc[1]), acc.h0, 4,
                                                            4, 1, (int)qa.sc[0], 1, (int)k.ksc);
    acc.h1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp4_operand(qa.v[1][1]), fp4_operand(k.kc[1]), acc.h1, 4,
                                                            4, 1, (int)qa.sc[1], 1, (int)k.ksc);
}

// MXFP4 rounding of one request's key blocks ahead of the score launch, for
// many query rows sharing them: logical block j (64 rows) of request 0
// becomes, in the kMxKeyBlockBytes layout, each row's four 32-value blocks
// rounded exactly as tile_mma(KeyHalf &, const QFp4 &, ...) rounds them
// (fp8 sign bits flipped first for a negative row scale), their E8M0 scales
// and the row scale.  Absent and out-of-range blocks read as zeros.  One
// wave per block, lane = row.
__global__ __launch_bounds__(64) void mx_keys_kernel(ScoreArgs a, uint8_t *dst) {
    const int j = blockIdx.x, lane = threadIdx.x;
    const int64_t nb = a.n_pool_rows / kBlock;
    const int32_t pb = j < a.max_blocks ? a.block_table[j] : -1;      // request 0's table row
    const bool ok = pb >= 0 && pb < nb;
    const __amdgpu_buffer_rsrc_t r =
        make_rsrc(a.pool + (ok ? (int64_t)pb : 0) * kBlock * kRowBytes, ok ? (uint32_t)(kBlock * kRowBytes) : 0u);
    const uint32_t ro = (uint32_t)lane * kRowBytes;
    u32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(r, ro + 16u * i, 0, 0);
    const float s = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, ro + kHeadDim, 0, 0));
    const uint32_t m = s < 0.f ? 0x80808080u : 0u;
    uint32_t esc = 0;
    u32x4 codes[4];
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
        uint32_t raw[16];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const u32x4 x = v[2 * blk + jj] ^ u32x4{m, m, m, m};
            const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                raw[8 * jj + 2 * i] = cvt_fp8x2_bf16x2<false>(w4[i]);
                raw[8 * jj + 2 * i + 1] = cvt_fp8x2_bf16x2<true>(w4[i]);
            }
        }
        esc |= mx_block_bf16(raw, codes[blk]) << (8 * blk);
    }
    const __amdgpu_buffer_rsrc_t o = make_rsrc(dst + (int64_t)j * kMxKeyBlockBytes, (uint32_t)kMxKeyBlockBytes);
#pragma unroll
    for (int blk = 0; blk < 4; ++blk)
        __builtin_amdgcn_raw_buffer_store_b128(codes[blk], o, (uint32_t)(64 * lane + 16 * blk), 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(esc, o, (uint32_t)(4096 + 4 * lane), 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s), o, (uint32_t)(4352 + 4 * lane), 0, 0);
}

// Epilogue half: relu, head weights and head sum, then the row scale.
// wr[hb][g][i%4] holds the weight w[b] of the head that accumulator
// register i = 4*g + i%4 of head block hb carries on this lane.  Returns the
// logit of entry (lane & 31) on every lane, or -inf when !keep.
__device__ __forceinline__ float tile_logit(const TileAcc &acc, const float (&wr)[2][4][4], float s, bool keep) {
    // relu as a signed-integer max on the float's bits (negative floats,
    // -0.0 included, have the sign bit set and become +0.0): one VALU op with
    // no NaN canonicalisation; four partial sums break the FMA chain
    float Tp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
        const f32x16 &h = hb ? acc.h1 : acc.h0;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x = __int_as_float(max(__float_as_int(h[4 * g + e]), 0));
                Tp[e] = fmaf(x, wr[hb][g][e], Tp[e]);
            }
        }
    }
    const float T = (Tp[0] + Tp[1]) + (Tp[2] + Tp[3]);
    // the two lane halves hold the two halves of the head sum: swapping
    // them across lanes 0-31 / 32-63 gives both halves the same total
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(T), __float_as_uint(T), false, false);
    const float tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    return keep ? fabsf(s) * tot : -__builtin_inff();
}

// Key tiles in flight per wave: two (the LDS ring's slots).  Two per wave
// over the whole grid already keep more bytes in flight than HBM needs at
// its loaded latency; deeper rings (three slots measured on every workload)
// only lengthen the memory queues, which delays the dependent block-table
// reads of the waves that start last.

template <int BS>
__device__ __forceinline__ RowCtx uniform_row(const ScoreArgs &a, int b, uint32_t &st) {
    RowCtx r = row_context<BS>(a, row_raw(a, b), st);
    // wave-uniform values stay in scalar registers, so the tile loop is
    // uniform control flow and its loads stay in flight across iterations
    r.req = __builtin_amdgcn_readfirstlane(r.req);
    r.nslots = __builtin_amdgcn_readfirstlane(r.nslots);
    r.nunits = __builtin_amdgcn_readfirstlane(r.nunits);
    r.limit = __builtin_amdgcn_readfirstlane(r.limit);
    return r;
}

// q[b] staged in LDS for the waves of a workgroup: 64 heads of 128 bf16,
// rows padded to 136 elements so that the 32 heads a half-wave reads sit in
// different banks.
constexpr int kQPad = kHeadDim + 8;
constexpr int kQStage = kHeads * kQPad;                 // elements per staged row

// The lane's MFMA A operands of q[b]: head 32*hb + (lane & 31), dims
// 64*(lane >> 5) + 8*kk .. +7, from global memory or from a staged row.
__device__ __forceinline__ void load_q_global(const ScoreArgs &a, int b, QBf16 &qa) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
        const u32x4 *qp = reinterpret_cast<const u32x4 *>(
            a.q + (int64_t)b * a.q_row + (int64_t)(32 * hb + (lane & 31)) * kHeadDim + 64 * (lane >> 5));
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) qa.v[hb][kk] = __builtin_bit_cast(bf16x8, qp[kk]);
    }
}

// Quantised q: rows of 132 bytes (128 e4m3 bytes, then the head's scale).
constexpr int kQ8Row = kHeadDim + 4;

// The scale of head `lane` of quantised q[b].
__device__ __forceinline__ float q8_scale(const ScoreArgs &a, int b, int lane) {
    return *reinterpret_cast<const float *>(a.q8 + ((int64_t)b * kHeads + lane) * kQ8Row + kHeadDim);
}

// Quantised q from global memory: the caller's bytes (a.q8), or bf16 q
// quantised here by the index-plane writer's rule (a.q8 null): the lane holds
// 64 values of each of its two heads, its partner lane ^ 32 the other 64, so
// each head's absolute maximum is the larger of the two lanes'.
__device__ __forceinline__ void load_q_global(const ScoreArgs &a, int b, QFp8 &qa) {
    const int lane = threadIdx.x & 63;
    if (a.q8) {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            const u32x4a4 *qp = reinterpret_cast<const u32x4a4 *>(
                a.q8 + ((int64_t)b * kHeads + 32 * hb + (lane & 31)) * kQ8Row + 64 * (lane >> 5));
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const u32x4a4 x = qp[2 * kk], y = qp[2 * kk + 1];
                qa.v[hb][kk] = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
            }
        }
        qa.qs = q8_scale(a, b, lane);
        return;
    }
    // two passes over the (cached) row: the heads' maxima, then the codes,
    // so that only one 16-byte chunk is held at a time
    float scale[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
        const u32x4 *qp = reinterpret_cast<const u32x4 *>(
            a.q + (int64_t)b * a.q_row + (int64_t)(32 * hb + (lane & 31)) * kHeadDim + 64 * (lane >> 5));
        float m = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const u32x4 x = qp[j];
            const uint32_t raw[4] = {x.x, x.y, x.z, x.w};
            m = fmaxf(m, amax8(raw));
        }
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
        const float amax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            uint32_t c[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const u32x4 x = qp[4 * kk + j];
                const uint32_t raw[4] = {x.x, x.y, x.z, x.w};
                quantize8(raw, amax, c[2 * j], c[2 * j + 1], scale[hb]);
            }
            qa.v[hb][kk] = v8i{(int)c[0], (int)c[1], (int)c[2], (int)c[3], (int)c[4], (int)c[5], (int)c[6], (int)c[7]};
        }
    }
    // lane l holds the weight of head l: head block 0 for l < 32, else 1
    qa.qs = lane < 32 ? scale[0] : scale[1];
}

// q[b] rounded to MXFP4 from global memory: the lane's four 32-value blocks
// (head 32*hb + (lane & 31), d = 64*(lane >> 5) + 32*kk + 0..31), each held
// whole by the lane.
__device__ __forceinline__ void load_q_global(const ScoreArgs &a, int b, QFp4 &qa) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
        uint32_t sc = 0;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const u32x4 *qp = reinterpret_cast<const u32x4 *>(
                a.q + (int64_t)b * a.q_row + (int64_t)(32 * hb + (lane & 31)) * kHeadDim + 64 * (lane >> 5) + 32 * kk);
            uint32_t raw[16];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const u32x4 x = qp[j];
                raw[4 * j] = x.x;
                raw[4 * j + 1] = x.y;
                raw[4 * j + 2] = x.z;
                raw[4 * j + 3] = x.w;
            }
            sc |= mx_block_bf16(raw, qa.v[hb][kk]) << (8 * kk);
        }
        qa.sc[hb] = sc;
    }
}


// q of rows rb .. rb + NR - 1 (those below B) for padded LDS rows, read by
// all 256 threads of the workgroup: fetch_q_rows issues the reads,
// put_q_rows (after other loads have been issued) stores them to LDS; the
// caller synchronises before the rows are read.  bf16 rows: 64 heads of 128
// elements padded to 136; quantised rows (132 bytes a head) go to 144-byte
// LDS rows, so each lane's 64-byte half row starts 16-byte aligned.
template <bool Q8, int NR> struct QRows {
    u32x4 v[NR][4];
};
template <int NR> struct QRows<true, NR> {
    uint32_t v[NR][9];                                   // 2112 dwords per row over 256 threads
};
constexpr int kQ8Dwords = kHeads * kQ8Row / 4;           // 2112
constexpr int kQ8Stage = 144;                            // LDS bytes per staged head row

template <int NR>
__device__ __forceinline__ void fetch_q_rows(const ScoreArgs &a, int rb, QRows<false, NR> &qv) {
    // rows past B read row B - 1 instead (not stored): the reads are
    // unconditional so the compiler can count them when waiting for
    // earlier ones
#pragma unroll
    for (int rr = 0; rr < NR; ++rr) {
        const int row = min(rb + rr, a.B - 1);
        const u32x4 *src = reinterpret_cast<const u32x4 *>(a.q + (int64_t)row * a.q_row);
#pragma unroll
        for (int i = 0; i < 4; ++i) qv.v[rr][i] = src[threadIdx.x + 256 * i];
    }
}

template <int NR>
__device__ __forceinline__ void fetch_q_rows(const ScoreArgs &a, int rb, QRows<true, NR> &qv) {
#pragma unroll
    for (int rr = 0; rr < NR; ++rr) {
        const int row = min(rb + rr, a.B - 1);
        const uint32_t *src = reinterpret_cast<const uint32_t *>(a.q8 + (int64_t)row * kHeads * kQ8Row);
#pragma unroll
        for (int i = 0; i < 9; ++i) {
            const int j = min((int)threadIdx.x + 256 * i, kQ8Dwords - 1);
            qv.v[rr][i] = src[j];
        }
    }
}

template <int NR>
__device__ __forceinline__ void put_q_rows(const ScoreArgs &a, int rb, const QRows<false, NR> &qv,
                                           uint16_t (*sq)[kQStage]) {
#pragma unroll
    for (int rr = 0; rr < NR; ++rr) {
        if (rb + rr < a.B) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = threadIdx.x + 256 * i;             // 16-byte chunk: head c / 16, dims 8 (c % 16)
                *reinterpret_cast<u32x4 *>(&sq[rr][(c >> 4) * kQPad + 8 * (c & 15)]) = qv.v[rr][i];
            }
        }
    }
}

template <int NR>
__device__ __forceinline__ void put_q_rows(const ScoreArgs &a, int rb, const QRows<true, NR> &qv,
                                           uint16_t (*sq)[kQStage]) {
#pragma unroll
    for (int rr = 0; rr < NR; ++rr) {
        if (rb + rr < a.B) {
            uint8_t *dst = reinterpret_cast<uint8_t *>(sq[rr]);
#pragma unroll
            for (int i = 0; i < 9; ++i) {
                const int j = (int)threadIdx.x + 256 * i;        // dword j: head j / 33, dword j % 33
                if (j < kQ8Dwords)
                    *reinterpret_cast<uint32_t *>(dst + (j / 33) * kQ8Stage + 4 * (j % 33)) = qv.v[rr][i];
            }
        }
    }
}

// A staged bf16 row (LDS, padded rows) quantised in place into the quantised
// rows' layout, by the writer's rule.  Four threads share a head: thread t
// takes dims 32 (t % 4) .. + 31 of head t / 4, so the head's amax is a
// reduction over one DPP quad and each thread divides for one scale.  Every
// thread reads its values before any writes (the quantised row is shorter and
// overwrites the front of the bf16 one); the caller synchronises before (the
// bf16 row written) and after.
__device__ __forceinline__ void quantize_staged_row(uint16_t *slot) {
    const int h = threadIdx.x >> 2, qt = threadIdx.x & 3;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(slot + h * kQPad + 32 * qt);
    uint32_t raw[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const u32x4 x = src[j];
        raw[4 * j] = x.x;
        raw[4 * j + 1] = x.y;
        raw[4 * j + 2] = x.z;
        raw[4 * j + 3] = x.w;
    }
    lds_barrier();
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        m = fmaxf(m, __builtin_fabsf(__uint_as_float(raw[i] << 16)));
        m = fmaxf(m, __builtin_fabsf(__uint_as_float(raw[i] & 0xFFFF0000u)));
    }
    // quad_perm [1,0,3,2] then [2,3,0,1]: the max over the quad's four lanes
    m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0xB1, 0xF, 0xF, false)));
    m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x4E, 0xF, 0xF, false)));
    uint32_t codes[8];
    float scale;
    quantize32(raw, m, codes, scale);
    uint8_t *row = reinterpret_cast<uint8_t *>(slot) + h * kQ8Stage;
    u32x4 *dst = reinterpret_cast<u32x4 *>(row + 32 * qt);
    dst[0] = u32x4{codes[0], codes[1], codes[2], codes[3]};
    dst[1] = u32x4{codes[4], codes[5], codes[6], codes[7]};
    if (qt == 0) *reinterpret_cast<float *>(row + kHeadDim) = scale;
}

__device__ __forceinline__ void load_q_staged(const uint16_t *row, QBf16 &qa) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
        const u32x4 *qp = reinterpret_cast<const u32x4 *>(row + (32 * hb + (lane & 31)) * kQPad + 64 * (lane >> 5));
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) qa.v[hb][kk] = __builtin_bit_cast(bf16x8, qp[kk]);
    }
}

__device__ __forceinline__ void load_q_staged(const uint16_t *row, QFp8 &qa) {
    const int lane = threadIdx.x & 63;
    const uint8_t *base = reinterpret_cast<const uint8_t *>(row);
    qa.qs = *reinterpret_cast<const float *>(base + lane * kQ8Stage + kHeadDim);
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
        const u32x4 *qp = reinterpret_cast<const u32x4 *>(base + (32 * hb + (lane & 31)) * kQ8Stage + 64 * (lane >> 5));
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const u32x4 x = qp[2 * kk], y = qp[2 * kk + 1];
            qa.v[hb][kk] = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
        }
    }
}

// MXFP4 staged rows: per head 64 code bytes (blocks 0..3 of 16 bytes), its
// four scale bytes, padding to 80 bytes (the 16 heads a quarter-wave reads
// then sit in different bank groups).
constexpr int kMxStage = 80;

// A staged bf16 row (LDS, padded rows) rounded in place to MXFP4: thread t
// takes block t % 4 of head t / 4.  Every thread reads its values before any
// writes (the rounded row is shorter and overwrites the front of the bf16
// one); the caller synchronises before (the bf16 row written) and after.
__device__ __forceinline__ void quantize_staged_row_mx(uint16_t *slot) {
    const int h = threadIdx.x >> 2, blk = threadIdx.x & 3;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(slot + h * kQPad + 32 * blk);
    uint32_t raw[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const u32x4 x = src[j];
        raw[4 * j] = x.x;
        raw[4 * j + 1] = x.y;
        raw[4 * j + 2] = x.z;
        raw[4 * j + 3] = x.w;
    }
    lds_barrier();
    u32x4 codes;
    const uint32_t sb = mx_block_bf16(raw, codes);
    uint8_t *row = reinterpret_cast<uint8_t *>(slot) + h * kMxStage;
    *reinterpret_cast<u32x4 *>(row + 16 * blk) = codes;
    row[64 + blk] = (uint8_t)sb;
}

__device__ __forceinline__ void load_q_staged(const uint16_t *row, QFp4 &qa) {
    const int lane = threadIdx.x & 63, hf = lane >> 5;
    const uint8_t *base = reinterpret_cast<const uint8_t *>(row);
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
        const uint8_t *hr = base + (32 * hb + (lane & 31)) * kMxStage;
        qa.v[hb][0] = *reinterpret_cast<const u32x4 *>(hr + 32 * hf);
        qa.v[hb][1] = *reinterpret_cast<const u32x4 *>(hr + 32 * hf + 16);
        const uint32_t s4 = *reinterpret_cast<const uint32_t *>(hr + 64);
        qa.sc[hb] = hf ? s4 >> 16 : s4;                 // byte kk: block 2*hf + kk
    }
}

struct NoQ {
    template <class Op>
    __device__ void operator()(Op &) const {}
};

// Score slots [j0, j1) of row b with the calling wave.  sh_w is the wave's
// own 64-float LDS slot for w[b].  Columns >= col_end are not written.
// BS: rows per pool block; a 64-column slot is 64 / BS pool blocks.
// USE_PRE: pre holds the first group's table reads, already issued by the
// caller, and qfin(qa) -- called once, right after the first ring of key
// loads has been issued, by every wave of the workgroup (it synchronises
// the workgroup) -- delivers the MFMA operands of q[b].  Otherwise q[b] is
// read from q_lds when the workgroup has staged it there, else from memory.
// MXP (with MX, 64-row blocks, no chunk lists): the key tiles come already
// rounded from a.mx_keys instead of from the pool.
template <bool OWN_COLS, bool SCORES, bool CHUNKED, bool LEAN, bool Q8, bool ACCUM, int BS, bool MX, bool MXP,
          bool USE_PRE = false, class QFin = NoQ>
__device__ __forceinline__ void score_span(const ScoreArgs &a, int b, int j0, int j1, const RowCtx &r,
                                           int col_end, float *sh_w, uint8_t *ring, uint32_t &st,
                                           const SlotRaw &pre = SlotRaw{-1, -1, false}, QFin qfin = QFin{},
                                           const uint16_t *q_lds = nullptr) {
    const int lane = threadIdx.x & 63;
    const int hf = lane >> 5;
    const int n32 = lane & 31;
    constexpr int U = kBlock / BS;                    // pool blocks per slot
    constexpr int GS = 64 / U;                        // slots per group: one block per lane
    static_assert(!MXP || (MX && BS == kBlock && !CHUNKED), "pre-rounded keys: MXFP4, 64-row blocks, no chunk lists");
    constexpr int TB = MXP ? kMxTileBytes : tile_bytes<BS>();
    constexpr int LPT = MXP ? 3 : loads_per_tile<BS>();   // loads per tile
    using Key = typename std::conditional<MXP, KeyMx, KeyHalf>::type;
    const bool live = r.req >= 0 && j0 < r.nslots;
    // no logits buffer (scores only): the logit stores get an empty
    // descriptor and are dropped
    float *out_row = a.logits ? a.logits + (int64_t)b * a.ld : a.scores + (int64_t)b * a.ld;
    float *score_row = SCORES ? a.scores + (int64_t)b * a.ld : nullptr;

    // Start-up reads, issued back to back in the order they are needed (the
    // vector memory counter retires in order) and none behind a branch:
    // w[b], the first group's block-table entries, then q[b] -- resolving
    // the table then leaves q in flight, and the first ring of key loads goes
    // out before q is waited on.
    float w_lane = 0.f;
    SlotRaw raw0{-1, -1, false};
    typename QSel<Q8, MX>::Op qa;
    if (live) {
        w_lane = a.w[(int64_t)b * a.w_row + lane];
        raw0 = USE_PRE ? pre : slot_raw<CHUNKED>(a, r.req, b, U * j0 + lane, lane < min(64, U * (j1 - j0)));
        if (!USE_PRE) {
            if (q_lds) load_q_staged(q_lds, qa); else load_q_global(a, b, qa);
        }
    }

    // Slots go in groups of up to GS (64 pool blocks): lane j resolves block
    // j of the group (one vector load per table level), then its tiles stream
    // through the wave's two-slot LDS ring.  Tiles of absent blocks and
    // ring slots past the group's end get an empty descriptor (no traffic).
    const __amdgpu_buffer_rsrc_t out_r = make_rsrc(out_row, a.logits ? (uint32_t)col_end * 4u : 0u);
    const __amdgpu_buffer_rsrc_t sc_r =
        make_rsrc(score_row ? score_row : out_row, score_row ? (uint32_t)col_end * 4u : 0u);
    // selection bits of the row: one word per 32 columns below col_end
    const __amdgpu_buffer_rsrc_t bits_r =
        make_rsrc(a.page_bits ? (const void *)(a.page_bits + (int64_t)b * a.bits_ld) : (const void *)a.pool,
                  a.page_bits ? (uint32_t)((col_end + 31) / 32) * 4u : 0u);
    const uint32_t lane_lo = tile_load_offset(lane);
    // the lane's logit store offset within a tile (the upper half's lanes
    // hold the same entries and store nothing: kDrop plus any column stays
    // past every descriptor's end)
    const uint32_t lane_off = LEAN && hf == 0 ? (uint32_t)n32 * 4u : kDrop;
    SlotRaw graw = raw0;
    float wr[2][4][4];                                // the lane's 32 head weights
    for (int g0 = j0; g0 < j1; g0 += GS) {
        const int gn = min(GS, j1 - g0);
        int32_t lane_ebase = 0;
        int64_t lane_prow0 = -1;
        lane_prow0 = resolve_slot<BS>(a, r, graw, U * g0 + lane, live && lane < U * gn, lane_ebase, st);
        // the next group's table reads, in flight during this group's ring
        // (no traffic when there is no next group)
        graw = slot_raw<CHUNKED>(a, r.req, b, U * (g0 + GS) + lane, live && lane < min(64, U * (j1 - g0 - GS)));
        const int ntiles = 2 * gn;
        // tile tau of the group: rows 32*(tau & 1) .. +31 of slot tau >> 1,
        // into ring slot tau & 1; tiles past the group's end and tiles of
        // absent blocks get an empty descriptor (no traffic).  lim_t: how
        // many of the tile's entries lie below the bound (<= 0 when absent).
        // LEAN works out a slot's descriptor and bound at its first tile and
        // reuses them for its second (tiles are issued in order).  It runs
        // before a tile's MFMAs, so the scalar descriptor arithmetic never
        // splits the stretch where MFMAs and the epilogue interleave.
        // With 16-row blocks each tile has two blocks of its own: the lane's
        // bound is its block's, shifted by 16 for rows 16-31.
        int32_t lim_t[2];
        __amdgpu_buffer_rsrc_t slot_r = make_rsrc(a.pool, 0u);
        int32_t slot_lim = 0;
        auto issue = [&](int tau) {
            if constexpr (BS != kBlock) {
                const int u0 = U * min(tau >> 1, gn - 1) + 2 * (tau & 1);
                __amdgpu_buffer_rsrc_t rq[2];
                int32_t lq[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int64_t pr = readlane64(lane_prow0, u0 + h);
                    const int64_t p = tau < ntiles ? pr : -1;
                    const bool ok = p >= 0;
                    const int64_t p0 = ok ? p : 0;
                    const uint32_t bytes = ok ? (uint32_t)min<int64_t>(BS, a.n_pool_rows - p0) * kRowBytes : 0u;
                    rq[h] = make_rsrc(a.pool + p0 * kRowBytes, bytes);
                    lq[h] = ok ? min(r.limit - __builtin_amdgcn_readlane(lane_ebase, u0 + h), BS) : 0;
                }
                lim_t[tau & 1] = n32 < BS ? lq[0] : lq[1] + BS;
                load_tile16(rq[0], rq[1], lane_lo, ring + (tau & 1) * TB);
            } else {
                if (!LEAN || (tau & 1) == 0) {
                    const int j = min(tau >> 1, gn - 1);
                    const int64_t pr = readlane64(lane_prow0, j);
                    const int64_t prow0 = tau < ntiles ? pr : -1;
                    const bool ok = prow0 >= 0;
                    const int64_t p0 = ok ? prow0 : 0;
                    const uint32_t bytes = ok ? (uint32_t)min<int64_t>(kBlock, a.n_pool_rows - p0) * kRowBytes : 0u;
                    const int eb = __builtin_amdgcn_readlane(lane_ebase, j);   // the slot's first logical entry
                    if constexpr (MXP) {
                        // logical block eb / 64 of request 0, rounded ahead
                        const bool okm = ok && (eb >> 6) < a.mx_blocks;
                        slot_r = make_rsrc(a.mx_keys + (int64_t)(okm ? eb >> 6 : 0) * kMxKeyBlockBytes,
                                           okm ? (uint32_t)kMxKeyBlockBytes : 0u);
                    } else {
                        slot_r = make_rsrc(a.pool + p0 * kRowBytes, bytes);
                    }
                    slot_lim = ok ? r.limit - eb : 0;
                }
                lim_t[tau & 1] = slot_lim - 32 * (tau & 1);
                if constexpr (MXP)
                    load_tile_mx(slot_r, tau & 1, ring + (tau & 1) * TB);
                else
                    load_tile(slot_r, (uint32_t)(32 * (tau & 1)) * kRowBytes, lane_lo, ring + (tau & 1) * TB);
            }
        };
        // a tile's epilogue inputs, kept with its accumulators because the
        // ring slot is reloaded before the epilogue runs
        struct Stage {
            TileAcc acc;
            float s;
            bool keep;
            float prev;     // ACCUM: the logit already in the output
        };
        // the lane's logit offset of tile tau (kDrop for lanes that store nothing)
        const auto out_off = [&](int tau) {
            const uint32_t col0 = (uint32_t)((g0 + (tau >> 1)) * kBlock + 32 * (tau & 1));
            return LEAN ? lane_off + col0 * 4u : (hf == 0 ? (col0 + (uint32_t)n32) * 4u : kDrop);
        };
        // tile tau's contraction.  Its ring slot is free for tile tau + 2 as
        // soon as the lane has read it, and that reload goes out before the
        // MFMAs, so the contraction and the caller's next epilogue form one
        // straight-line stretch for the scheduler to interleave.  The wait
        // for the tile's loads counts only the loads of tile tau + 1 (five,
        // six with 16-row blocks) as later: vector memory loads complete in
        // order, so this holds whatever order stores take.
        auto mma = [&](int tau, Stage &st_) {
            const int k = tau & 1;
            wait_vmem<LPT>();
            Key kh;
            if constexpr (MXP)
                read_tile(ring + k * TB, kh);
            else
                read_tile<BS>(ring + k * TB, kh);
            wait_lds();
            st_.keep = n32 < lim_t[k];
            // ACCUM: the earlier logit is read before the next tile's loads
            // go out, so the ring's in-order wait still counts only those
            if (ACCUM) st_.prev = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(out_r, out_off(tau), 0, 0));
            issue(tau + 2);
            tile_mma(kh, qa, st_.acc);
            st_.s = kh.s;
        };
        auto finish = [&](int tau, const Stage &st_) {
            float logit = tile_logit(st_.acc, wr, st_.s, st_.keep);
            if (ACCUM) logit += st_.prev;             // -inf stays -inf: both halves mask alike
            const uint32_t off = out_off(tau);
            // per-row path (many rows over one key set): the logits stream
            // past the caches (non-temporal) so the keys stay resident in L2
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(logit), out_r, off, 0, LEAN ? kNonTemporal : 0);
            if (SCORES) {
                const float score = 1.0f / (1.0f + expf(-logit));
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(score), sc_r, off, 0, LEAN ? kNonTemporal : 0);
            }
            if (!SCORES && !OWN_COLS && a.page_bits) {
                // lanes 0-31 hold the tile's 32 entries (lanes 32-63 repeat them)
                const float score = 1.0f / (1.0f + expf(-logit));
                const uint32_t word = (uint32_t)__ballot(score >= a.threshold);
                const uint32_t woff = lane == 0 ? (uint32_t)((g0 + (tau >> 1)) * 2 + (tau & 1)) * 4u : kDrop;
                __builtin_amdgcn_raw_buffer_store_b32(word, bits_r, woff, 0, 0);
            }
        };
        issue(0);
        issue(1);
        if (USE_PRE && g0 == j0) qfin(qa);            // q arrives while the ring is in flight
        if (g0 == j0) {
            // w[b] into the wave's LDS slot; a quantised query's per-head scale
            // joins its weight: relu(s_q x) = s_q relu(x) for s_q >= 0
            if constexpr (Q8) sh_w[lane] = w_lane * qa.qs; else sh_w[lane] = w_lane;
            __builtin_amdgcn_wave_barrier();
            const float4 *w4 = reinterpret_cast<const float4 *>(sh_w);
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const float4 wv = w4[8 * hb + 2 * g + hf];
                    wr[hb][g][0] = wv.x;
                    wr[hb][g][1] = wv.y;
                    wr[hb][g][2] = wv.z;
                    wr[hb][g][3] = wv.w;
                }
        }
        // Two-stage pipeline over the ring: the contraction of tile tau is
        // issued before the epilogue of tile tau - 1, so the MFMA chain of
        // one tile runs under the other's VALU work.  ntiles is even.
        Stage sa, sb;
        mma(0, sa);
        for (int tau = 1;; tau += 2) {
            mma(tau, sb);
            finish(tau - 1, sa);
            if (tau + 1 >= ntiles) {
                finish(tau, sb);
                break;
            }
            mma(tau + 1, sa);
            finish(tau, sb);
        }
    }
}

// OWN_COLS: write only the columns each row's tile list can reach (what the
// top-k reads; the count goes to row_cols), else every column up to n_cols.
// FLAT: the (row, slot) work of all rows is flattened and split evenly over
// every wave of the grid (rows of very different lengths); otherwise each
// workgroup owns `slots_per_wave` x 4 consecutive slots of one row.
// QQ (with Q8): q arrives as bf16 and is quantised here, while it is staged.
// MX (with QQ): q and keys rounded to MXFP4 blocks here instead.
// MXP (with MX, the per-row split): the keys come rounded from a.mx_keys.
template <bool OWN_COLS, bool SCORES, bool FLAT, bool CHUNKED, bool Q8, bool ACCUM, int BS, bool QQ, bool MX,
          bool MXP = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void score_kernel(ScoreArgs a) {
    constexpr int U = kBlock / BS;                    // pool blocks per slot
    __shared__ __attribute__((aligned(16))) float sh_w[kWaves][kHeads];
    __shared__ int32_t sh_pre[FLAT ? kFlatRows + 1 : 1];
    // sh_runits: each row's pool blocks (its slots follow from them)
    __shared__ int32_t sh_rreq[FLAT ? kFlatRows : 1], sh_rlim[FLAT ? kFlatRows : 1], sh_runits[FLAT ? kFlatRows : 1];
    __shared__ uint32_t sh_scan[kWaves];
    __shared__ __attribute__((aligned(16))) uint16_t sh_q[FLAT ? 2 : 1][kQStage];
    __shared__ __attribute__((aligned(16))) uint8_t sh_ring[kWaves][2 * tile_bytes<BS>()];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int lane = threadIdx.x & 63;
    const int slot_cols = (a.n_cols + kBlock - 1) / kBlock;
    uint32_t st = 0;

    static_assert(!MXP || (!FLAT && MX && !CHUNKED && BS == kBlock), "pre-rounded keys on the per-row split only");
    if (!FLAT) {
        const int b = blockIdx.x / a.splits;
        const int split = blockIdx.x - b * a.splits;
        const RowCtx r = uniform_row<BS>(a, b, st);
        const int col_end = OWN_COLS ? max(0, min(r.nslots * kBlock, a.n_cols)) : a.n_cols;
        const int slot_stop = OWN_COLS ? min(r.nslots, slot_cols) : slot_cols;
        if (OWN_COLS && split == 0 && threadIdx.x == 0) {
            a.row_cols[b] = (uint32_t)col_end;
            if (a.row_done) a.row_done[b] = 0u;
        }
        // a row that one workgroup covers is split evenly over its four
        // waves by the row's own length (rows of one launch differ in length)
        const int spw = a.splits == 1 ? (slot_stop + kWaves - 1) / kWaves : a.slots_per_wave;
        const int j0 = (split * kWaves + wave) * spw;
        const int j1 = min(j0 + spw, slot_stop);
        // the first group's table reads, then q[b] staged in LDS once for
        // the four waves
        const SlotRaw raw0 = slot_raw<CHUNKED>(a, r.req, b, U * j0 + lane, lane < min(64, U * (j1 - j0)));
        QRows<Q8 && !QQ, 1> qv;
        fetch_q_rows<1>(a, b, qv);
        const auto put = [&] {
            put_q_rows<1>(a, b, qv, sh_q);
            if constexpr (QQ) {
                lds_barrier();
                if constexpr (MX) quantize_staged_row_mx(sh_q[0]); else quantize_staged_row(sh_q[0]);
            }
        };
        const auto qfin = [&](typename QSel<Q8, MX>::Op &qa) {
            put();
            lds_barrier();
            load_q_staged(sh_q[0], qa);
        };
        if (j0 < j1) {
            score_span<OWN_COLS, SCORES, CHUNKED, !FLAT, Q8, ACCUM, BS, MX, MXP, true>(a, b, j0, j1, r, col_end, sh_w[wave], sh_ring[wave], st, raw0, qfin);
        } else {
            put();                                    // the workgroup's one barrier
            lds_barrier();
        }
    } else {
        // per-row work (slots) and its prefix over rows, in LDS
        uint32_t st_rows = 0;
        int32_t cnt[2] = {0, 0};
        RowRaw raw[2];
        for (int k2 = 0; k2 < 2; ++k2) {                                       // all in flight
            int bl;
            const int row = min(2 * (int)threadIdx.x + k2, max(a.B - 1, 0));
            raw[k2] = row_raw(key_view(a, row, bl), bl);
        }
        for (int k2 = 0; k2 < 2; ++k2) {
            const int row = 2 * threadIdx.x + k2;
            if (row < a.B) {
                int bl;
                const RowCtx rr = row_context<BS>(key_view(a, row, bl), raw[k2], st_rows);
                sh_rreq[row] = rr.req;
                sh_rlim[row] = rr.limit;
                sh_runits[row] = rr.nunits;
                cnt[k2] = OWN_COLS ? max(0, min(rr.nslots, slot_cols)) : slot_cols;
                if (OWN_COLS && blockIdx.x == 0) {
                    a.row_cols[row] = (uint32_t)max(0, min(rr.nslots * kBlock, a.n_cols));
                    if (a.row_done) a.row_done[row] = 0u;
                }
            }
        }
        if (blockIdx.x == 0) st |= st_rows;
        // block exclusive scan of the pairs
        const uint32_t v = (uint32_t)(cnt[0] + cnt[1]);
        const uint32_t incl = wave_scan(v);
        if (lane == 63) sh_scan[wave] = incl;
        __syncthreads();
        uint32_t add = 0;
        for (int i = 0; i < wave; ++i) add += sh_scan[i];
        const uint32_t excl = incl - v + add;
        if (2 * (int)threadIdx.x < a.B) sh_pre[2 * threadIdx.x] = (int32_t)excl;
        if (2 * (int)threadIdx.x + 1 < a.B) sh_pre[2 * threadIdx.x + 1] = (int32_t)(excl + cnt[0]);
        if (threadIdx.x == 255) sh_pre[a.B] = (int32_t)(incl + add);
        __syncthreads();

        const int total = __builtin_amdgcn_readfirstlane(sh_pre[a.B]);
        const int nw = (int)gridDim.x * kWaves;
        const int chunk = (total + nw - 1) / nw;
        // the row whose work range holds flattened item x (x < total)
        const auto row_of = [&](int x) {
            int lo = 0, hi = a.B - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (sh_pre[mid] <= x) lo = mid; else hi = mid - 1;
            }
            return __builtin_amdgcn_readfirstlane(lo);
        };
        int f = ((int)blockIdx.x * kWaves + wave) * chunk;
        const int fend = min(f + chunk, total);

        // The wave's first span, and its table reads issued before the q
        // staging reads below.
        int b = row_of(min(f, max(total - 1, 0)));
        int pb = __builtin_amdgcn_readfirstlane(sh_pre[b]);
        int pe = __builtin_amdgcn_readfirstlane(sh_pre[b + 1]);
        RowCtx r0;
        r0.req = __builtin_amdgcn_readfirstlane(sh_rreq[b]);
        r0.limit = __builtin_amdgcn_readfirstlane(sh_rlim[b]);
        r0.nunits = __builtin_amdgcn_readfirstlane(sh_runits[b]);
        r0.nslots = (r0.nunits + U - 1) / U;
        int bl0;
        const ScoreArgs a0 = key_view(a, b, bl0);
        const SlotRaw raw0 =
            slot_raw<CHUNKED>(a0, r0.req, b, U * (f - pb) + lane, lane < min(64, U * (min(fend, pe) - f)));
        // q of the workgroup's first two rows, staged in LDS once for its
        // four waves (most workgroups lie within one or two rows)
        const int fw = (int)blockIdx.x * kWaves * chunk;
        const int rb = fw < total ? row_of(fw) : a.B;
        QRows<Q8 && !QQ, 2> qv;
        fetch_q_rows<2>(a, rb, qv);
        // QQ: the staged bf16 rows that the workgroup scores are quantised
        // in place (row rb + 1 only when the workgroup reaches it)
        const int wend = min(fw + kWaves * chunk, total);
        const int nquant = __builtin_amdgcn_readfirstlane(rb >= a.B ? 0 : rb + 1 < a.B && sh_pre[rb + 1] < wend ? 2 : 1);
        const auto put = [&] {
            put_q_rows<2>(a, rb, qv, sh_q);
            if constexpr (QQ) {
#pragma unroll 1
                for (int rr = 0; rr < nquant; ++rr) {
                    lds_barrier();
                    if constexpr (MX) quantize_staged_row_mx(sh_q[rr]); else quantize_staged_row(sh_q[rr]);
                }
            }
        };
        const auto qfin = [&](typename QSel<Q8, MX>::Op &qa) {
            put();
            lds_barrier();
            if (b == rb || b == rb + 1)
                load_q_staged(sh_q[b - rb], qa);
            else
                load_q_global(a, b, qa);
        };

        if (!(f < fend)) {
            put();                                    // the workgroup's one barrier
            lds_barrier();
        } else {
            const int col_end = OWN_COLS ? max(0, min(r0.nslots * kBlock, a.n_cols)) : a.n_cols;
            score_span<OWN_COLS, SCORES, CHUNKED, !FLAT, Q8, ACCUM, BS, MX, false, true>(a0, b, f - pb, min(fend, pe) - pb, r0, col_end, sh_w[wave], sh_ring[wave], st, raw0,
                                                    qfin);
            f = min(fend, pe);
            for (++b; f < fend; ++b) {
                pb = __builtin_amdgcn_readfirstlane(sh_pre[b]);
                pe = __builtin_amdgcn_readfirstlane(sh_pre[b + 1]);
                if (pe <= f) continue;
                RowCtx r;
                r.req = __builtin_amdgcn_readfirstlane(sh_rreq[b]);
                r.limit = __builtin_amdgcn_readfirstlane(sh_rlim[b]);
                r.nunits = __builtin_amdgcn_readfirstlane(sh_runits[b]);
                r.nslots = (r.nunits + U - 1) / U;
                const int ce = OWN_COLS ? max(0, min(r.nslots * kBlock, a.n_cols)) : a.n_cols;
                int bl;
                score_span<OWN_COLS, SCORES, CHUNKED, !FLAT, Q8, ACCUM, BS, MX, false>(key_view(a, b, bl), b, f - pb, min(fend, pe) - pb, r, ce, sh_w[wave], sh_ring[wave], st,
                                                                      SlotRaw{-1, -1, false}, NoQ{},
                                                                      b == rb + 1 ? sh_q[1] : nullptr);
                f = min(fend, pe);
            }
        }
    }
    wait_vmem<0>();     // no buffer-to-LDS load outlives the workgroup
    if (st && a.status) atomicOr(a.status, st);
}

}  // namespace

template <bool OWN_COLS, bool SCORES, bool FLAT, bool Q8, bool ACCUM, bool QQ, bool MX = false>
void launch_score_qa(const ScoreArgs &a, int64_t grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    const dim3 g((unsigned)grid), blk(256);
    const bool small = a.block_size == kSmallBlock;
    if constexpr (MX && !FLAT) {
        if (a.mx_keys) {                              // the keys rounded ahead (launch_score checked the shape)
            hipExtLaunchKernelGGL((score_kernel<OWN_COLS, SCORES, FLAT, false, Q8, ACCUM, kBlock, QQ, MX, true>), g, blk,
                                  0, s, e0, e1, 0, a);
            return;
        }
    }
    if (a.chunk_ids) {
        if (small)
            hipExtLaunchKernelGGL((score_kernel<OWN_COLS, SCORES, FLAT, true, Q8, ACCUM, kSmallBlock, QQ, MX>), g, blk, 0, s,
                                  e0, e1, 0, a);
        else
            hipExtLaunchKernelGGL((score_kernel<OWN_COLS, SCORES, FLAT, true, Q8, ACCUM, kBlock, QQ, MX>), g, blk, 0, s, e0,
                                  e1, 0, a);
    } else {
        if (small)
            hipExtLaunchKernelGGL((score_kernel<OWN_COLS, SCORES, FLAT, false, Q8, ACCUM, kSmallBlock, QQ, MX>), g, blk, 0,
                                  s, e0, e1, 0, a);
        else
            hipExtLaunchKernelGGL((score_kernel<OWN_COLS, SCORES, FLAT, false, Q8, ACCUM, kBlock, QQ, MX>), g, blk, 0, s,
                                  e0, e1, 0, a);
    }
}

// The accumulating second head half exists for bf16 queries only; a bf16
// query quantised in the kernel (a.quant_q) takes the quantised path.
template <bool OWN_COLS, bool SCORES, bool FLAT, bool Q8>
void launch_score_q(const ScoreArgs &a, int64_t grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    if constexpr (!Q8) {
        if (a.accum) return launch_score_qa<OWN_COLS, SCORES, FLAT, false, true, false>(a, grid, s, e0, e1);
        launch_score_qa<OWN_COLS, SCORES, FLAT, false, false, false>(a, grid, s, e0, e1);
    } else {
        if (a.quant_q) return launch_score_qa<OWN_COLS, SCORES, FLAT, true, false, true>(a, grid, s, e0, e1);
        launch_score_qa<OWN_COLS, SCORES, FLAT, true, false, false>(a, grid, s, e0, e1);
    }
}

template <bool OWN_COLS, bool SCORES, bool FLAT>
void launch_score_as(const ScoreArgs &a, int64_t grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    if (a.mxfp4) return launch_score_qa<OWN_COLS, SCORES, FLAT, false, false, true, true>(a, grid, s, e0, e1);
    if (a.q8 || a.quant_q)
        launch_score_q<OWN_COLS, SCORES, FLAT, true>(a, grid, s, e0, e1);
    else
        launch_score_q<OWN_COLS, SCORES, FLAT, false>(a, grid, s, e0, e1);
}

hipError_t launch_mx_keys(const ScoreArgs &a, uint8_t *dst, int32_t nblocks, hipStream_t s) {
    if (nblocks <= 0) return hipSuccess;
    if (!a.block_table || !a.pool || !dst || a.max_blocks < 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mx_keys_kernel, dim3((unsigned)nblocks), dim3(64), 0, s, a, dst);
    return hipGetLastError();
}

hipError_t launch_score(const ScoreArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    if (a.B <= 0) return hipSuccess;
    if (a.accum && (a.q8 || a.quant_q || a.mxfp4)) return hipErrorInvalidValue;
    if (a.quant_q && (a.q8 || !a.q)) return hipErrorInvalidValue;
    if (a.mxfp4 && (a.q8 || a.quant_q || !a.q)) return hipErrorInvalidValue;
    // keys rounded ahead: MXFP4 on the per-row split, 64-row blocks, a block
    // table and no chunk lists
    if (a.mx_keys && (!a.mxfp4 || a.B <= kFlatRows || a.block_size != kBlock || !a.block_table || a.chunk_ids ||
                      a.mx_blocks < 0))
        return hipErrorInvalidValue;
    if (a.block_size != kBlock && a.block_size != kSmallBlock) return hipErrorInvalidValue;
    if (!a.logits && (a.accum || (!a.scores && !a.page_bits) || a.row_cols)) return hipErrorInvalidValue;
    // several layers in one launch: the flattened split, selection bits, no
    // quantised query
    if (a.rows_per_layer > 0 &&
        (a.B > kFlatRows || a.row_cols || a.scores || a.logits || !a.page_bits || a.q8 || a.quant_q || a.mxfp4 ||
         a.accum || a.chunk_ids || a.B % a.rows_per_layer || a.B / a.rows_per_layer > kMaxLayers))
        return hipErrorInvalidValue;
    // the top-k feed (row_cols) never asks for scores
    const bool own = a.row_cols != nullptr;
    const bool scores = !own && a.scores != nullptr;
    const bool flat = a.B <= kFlatRows;
    int64_t grid;
    if (flat) {
        // one resident round: up to 2 workgroups per CU, never more waves
        // than (row, slot) pairs
        const int64_t slots = (a.n_cols + kBlock - 1) / kBlock;
        grid = std::max<int64_t>(1, std::min<int64_t>(512, ((int64_t)a.B * slots + kWaves - 1) / kWaves));
    } else {
        grid = (int64_t)a.B * a.splits;
    }
    if (own) {
        if (flat) launch_score_as<true, false, true>(a, grid, s, e0, e1);
        else launch_score_as<true, false, false>(a, grid, s, e0, e1);
    } else if (scores) {
        if (flat) launch_score_as<false, true, true>(a, grid, s, e0, e1);
        else launch_score_as<false, true, false>(a, grid, s, e0, e1);
    } else {
        if (flat) launch_score_as<false, false, true>(a, grid, s, e0, e1);
        else launch_score_as<false, false, false>(a, grid, s, e0, e1);
    }
    return hipGetLastError();
}

}  // namespace idx
