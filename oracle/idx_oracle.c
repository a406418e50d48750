/*
 * CPU oracle for the compressed-sparse-attention (CSA) indexer: score + top-k.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  The GPU product
 * path never calls, links or falls back to it.  It shares no code, header,
 * table or helper with the HIP implementation.
 *
 * It is the plain definition written out, slowly and in double precision:
 * no blocking, no fusion, no reordering of the sums, no SIMD intrinsics and
 * no fast-math.  OpenMP is used only to run independent query rows at once.
 *
 * Sources (page titles as published; section names are the pages' own):
 *  [FM]   "FlashMemory-DeepSeek-V4" README,
 *         section "Retriever architecture" (the score formula, the fused head
 *         weight and the compressed_k dequant) and section "compressed_k
 *         format" (132-byte rows: 128 fp8 bytes, then an fp32 scale),
 *         section "Two-level recall algorithm" (Level 2 keeps the top-512,
 *         with non-resident logits set to -inf).
 *  [BG]   "feat: DeepSeek-V4-Flash integration + Blackwell (sm120) bring-up"
 *         (batchgen pull request 153): the c4 fix (the scorer's bound is the
 *         compressed length seq_len // 4) and the Phase 3 summary (relu is
 *         applied to each head's score before the gate-weighted sum), and the
 *         indexer pool row layout [128 B fp8 | 4 B fp32 scale].
 *  [AT]   "DeepSeek-V4.1 native paged runtime" (ATOM docs), section "Current
 *         execution scope": one scorer for every shape; each query row has
 *         its own bound and its own tile list into the paged index plane; a
 *         padding row carries the id -1 and reads nothing.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - fp8 flavour: OCP E4M3 ("e4m3fn"): bias 7, no infinities, S.1111.111 is
 *    NaN, largest finite 448.
 *  - the scale is a little-endian IEEE binary32 at bytes HEAD_DIM..HEAD_DIM+3.
 *  - the product (fp8 value) x (scale) is taken exactly (the pages' fp32
 *    product differs by at most one fp32 rounding).
 *  - relu(x) = x if x > 0 else 0.
 *  - top-k keeps the k largest logits; equal logits go to the lower column;
 *    -inf (masked) and NaN entries are never selected; rows with fewer than k
 *    selectable entries are padded with column -1.
 *  - index-plane writer: scale = amax / 448 per row, values rounded to the
 *    nearest e4m3 value (ties to even, saturating), zero rows stored as
 *    zeros with scale 0 (see the writer section below).
 *  - Level-1 resident-set selection: per-entry ensemble (max or mean) of the
 *    layers' sigmoid scores, threshold, page density, sink and recent pages,
 *    the densest pages up to KMAX (see the Level-1 section below).
 *  - MXFP4 variant: query and key rounded to MXFP4 blocks of 32 before the
 *    score (see the MXFP4 section below).
 *
 * Build: plain C99, `gcc -O2 -fopenmp -shared -fPIC` (no -ffast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* [FM] "compressed_k format": the first HEAD_DIM bytes of a key row are
 * float8_e4m3 values.  OCP E4M3: sign bit, 4 exponent bits (bias 7), 3
 * mantissa bits; exponent 0 is subnormal (M * 2^-9); exponent 15 with
 * mantissa 7 is NaN; there is no infinity. */
double oracle_e4m3_value(uint8_t u)
{
    int sign = u >> 7;
    int e = (u >> 3) & 15;
    int m = u & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* bfloat16 is the top half of an IEEE binary32; widening is exact. */
static double bf16_value(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* [FM] "compressed_k format": bytes[HEAD_DIM:] viewed as float32
 * (little-endian, assembled byte by byte so the host's order never matters). */
static double le_f32_value(const uint8_t *p)
{
    uint32_t bits = (uint32_t)p[0] | ((uint32_t)p[1] << 8) |
                    ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

double oracle_scale_value(const uint8_t *row, int32_t head_dim)
{
    return le_f32_value(row + head_dim);
}

/* [AT] "Current execution scope": each query row has its own bound and its
 * own tile list.  Resolves column `col` of query row `b` to a physical pool
 * row, or returns -1 when the column scores nothing.
 *
 * Columns: without a chunk list, column c is logical entry c.  With a chunk
 * list, column c = block_size * j + s names entry s of the row's j-th listed
 * logical block ([FM] "Two-level recall algorithm": only the resident chunks
 * are scored).  *entry_out receives the logical entry id.
 *
 * An entry is scored iff it lies below the row's bound ([BG] c4 fix: the
 * bound is the compressed length), its logical block is present in the
 * request's block table (id >= 0 and inside the pool), and the query row is
 * not padding (request id -1, [AT] "Current execution scope"). */
int64_t oracle_resolve(int32_t b, int32_t col, int64_t n_pool_rows,
                       int32_t block_size, const int32_t *block_table,
                       int32_t n_req, int32_t max_blocks, const int32_t *q_req,
                       const int32_t *chunk_ids, const int32_t *n_chunks,
                       int32_t max_chunks, const int32_t *limits,
                       int64_t *entry_out)
{
    int32_t req = q_req ? q_req[b] : b;
    int32_t j = col / block_size;
    int32_t s = col % block_size;
    int64_t beta, entry, prow;
    *entry_out = -1;
    if (req < 0)
        return -1;
    if (chunk_ids) {
        int32_t nc = n_chunks[b];
        if (nc > max_chunks)
            nc = max_chunks;
        if (j >= nc)
            return -1;
        beta = chunk_ids[(int64_t)b * max_chunks + j];
        if (beta < 0)
            return -1;
    } else {
        beta = j;
    }
    entry = beta * block_size + s;
    *entry_out = entry;
    if (entry >= limits[b])
        return -1;
    if (block_table) {
        int64_t pblk;
        if (req >= n_req || beta >= max_blocks)
            return -1;
        pblk = block_table[(int64_t)req * max_blocks + beta];
        if (pblk < 0 || (pblk + 1) * block_size > n_pool_rows)
            return -1;
        prow = pblk * block_size + s;
    } else {
        prow = entry;
        if (prow >= n_pool_rows)
            return -1;
    }
    return prow;
}

/* ---------------------------------------------------------------------------
 * MXFP4 rounding of query and key.  [AT] "Current execution scope": the
 * published model rounds the index query and key alike to FP4 before the
 * index score, whatever the index plane holds.  [BG] the fp8-fallback commit
 * names that quantisation MXFP4 (selector auto | mxfp4 | fp8) with an e4m3
 * fallback at one scale per block of 32 values, and the Phase 3 summary
 * lists fp4 quantisation of the indexer's q and k.  MXFP4 is the OCP
 * Microscaling format: a block of 32 values shares one power-of-two scale
 * X = 2^e (an E8M0 byte), each value is an E2M1 number (1 sign, 2 exponent,
 * 1 mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6).
 * Readings where the pages are silent:
 *  - a block is 32 consecutive dims of one query head or one key row;
 *  - e = floor(log2(amax)) - 2 (2 is E2M1's largest exponent), clamped to
 *    the E8M0 range [-127, 127]; a block of zeros stays zero;
 *  - each value becomes the E2M1 value nearest v / X (ties to the even
 *    code), magnitudes above 6 saturate to 6, the sign is kept;
 *  - the key is rounded as the index plane holds it: its e4m3 values are
 *    the block's values, and its fp32 row scale stays a factor outside the
 *    rounding (the row scale is not a power of two, so rounding e4m3 * scale
 *    instead would move the block's grid).
 * Inputs are finite.
 */
static const double e2m1_magnitudes[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* The E2M1 value nearest x (search over the eight magnitudes; on a tie the
 * even code -- the one whose mantissa bit is 0 -- wins), saturating at 6. */
double oracle_e2m1_round(double x)
{
    double a = fabs(x), best = 0.0, best_d = INFINITY;
    int c, best_c = 0;
    if (a > 6.0)
        a = 6.0;
    for (c = 0; c < 8; ++c) {
        double d = fabs(a - e2m1_magnitudes[c]);
        if (d < best_d || (d == best_d && (c & 1) == 0 && (best_c & 1) == 1)) {
            best_d = d;
            best = e2m1_magnitudes[c];
            best_c = c;
        }
    }
    return x < 0.0 ? -best : best;
}

/* The block exponent e for a block whose largest magnitude is amax > 0. */
int oracle_mxfp4_exponent(double amax)
{
    int ex, e;
    frexp(amax, &ex);                    /* amax = m * 2^ex, 0.5 <= m < 1 */
    e = (ex - 1) - 2;                    /* floor(log2(amax)) - 2 */
    if (e < -127)
        e = -127;
    if (e > 127)
        e = 127;
    return e;
}

/* Round v[0 .. n) block by block (n a multiple of 32) into out (which may
 * be v itself). */
void oracle_mxfp4_round(const double *v, int32_t n, double *out)
{
    int32_t b, i;
    for (b = 0; b + 32 <= n; b += 32) {
        double amax = 0.0, x;
        for (i = 0; i < 32; ++i)
            if (fabs(v[b + i]) > amax)
                amax = fabs(v[b + i]);
        if (amax == 0.0) {
            for (i = 0; i < 32; ++i)
                out[b + i] = 0.0;
            continue;
        }
        x = ldexp(1.0, oracle_mxfp4_exponent(amax));
        for (i = 0; i < 32; ++i)
            out[b + i] = oracle_e2m1_round(v[b + i] / x) * x;
    }
}

/* One logit, straight from the definition in [FM] "Retriever architecture":
 *   k_d     = e4m3(byte_d) * scale                       (dequant)
 *   dot_h   = sum_d k_d * q[h,d]                          (k @ q^T)
 *   logit   = sum_h relu(dot_h) * w[h]                    (relu per head
 *             before the weighted sum, [BG] Phase 3)
 * q_row holds the query row already widened to double (exact for bf16).
 * Sums run in index order in double. */
static double logit_of_row(const double *q_row, const float *w_row, int32_t H,
                           int32_t D, const uint8_t *key_row, double *k, int mx)
{
    double scale = le_f32_value(key_row + D);
    double logit = 0.0;
    int32_t h, d;
    if (mx) {
        /* MXFP4 variant: the key's e4m3 values rounded block by block, then
         * the row scale */
        for (d = 0; d < D; ++d)
            k[d] = oracle_e4m3_value(key_row[d]);
        oracle_mxfp4_round(k, D, k);
        for (d = 0; d < D; ++d)
            k[d] = k[d] * scale;
    } else {
        for (d = 0; d < D; ++d)
            k[d] = oracle_e4m3_value(key_row[d]) * scale;
    }
    for (h = 0; h < H; ++h) {
        double dot = 0.0;
        for (d = 0; d < D; ++d)
            dot += k[d] * q_row[(int64_t)h * D + d];
        logit += (dot > 0.0 ? dot : 0.0) * (double)w_row[h];
    }
    return logit;
}

/* The same logit for a bf16 query row given as raw bits [H, D]. */
double oracle_logit(const uint16_t *q_row, const float *w_row, int32_t H,
                    int32_t D, const uint8_t *key_row)
{
    double *qd = (double *)malloc(sizeof(double) * (size_t)H * (size_t)D);
    double *k = (double *)malloc(sizeof(double) * (size_t)D);
    double v = NAN;
    int64_t i;
    if (qd && k) {
        for (i = 0; i < (int64_t)H * D; ++i)
            qd[i] = bf16_value(q_row[i]);
        v = logit_of_row(qd, w_row, H, D, key_row, k, 0);
    }
    free(qd);
    free(k);
    return v;
}

/* Logits of every (row, column); unscored columns hold -inf ([FM] "Two-level
 * recall algorithm": masked logits are -inf).  The query is q (bf16 bits
 * [B, H, D], widened exactly) or, when q8 is given instead, quantised rows
 * [B, H, D + 4] in the index-plane layout (e4m3 bytes, then the head's fp32
 * scale), dequantised exactly as e4m3(byte) * scale -- the quantised-query
 * variant.  With mx set, query heads and keys are rounded to MXFP4 first
 * (the MXFP4 variant; D a multiple of 32).  Returns 0, or -1 on bad sizes or
 * allocation failure. */
static int score_rows(const uint16_t *q, const uint8_t *q8, const float *w,
                      int32_t B, int32_t H, int32_t D, const uint8_t *pool,
                      int64_t n_pool_rows, int32_t block_size,
                      const int32_t *block_table, int32_t n_req,
                      int32_t max_blocks, const int32_t *q_req,
                      const int32_t *chunk_ids, const int32_t *n_chunks,
                      int32_t max_chunks, const int32_t *limits, int32_t n_cols,
                      double *logits, int32_t n_threads, int mx)
{
    int64_t row_bytes = (int64_t)D + 4;
    int32_t b;
    int failed = 0;
    if (B < 0 || H <= 0 || D <= 0 || block_size <= 0 || n_cols < 0)
        return -1;
    if (mx && D % 32 != 0)
        return -1;
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (b = 0; b < B; ++b) {
        double *qd = (double *)malloc(sizeof(double) * (size_t)H * (size_t)D);
        double *k = (double *)malloc(sizeof(double) * (size_t)D);
        int64_t i;
        int32_t c;
        if (!qd || !k) {
            free(qd);
            free(k);
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
            continue;
        }
        if (q8) {
            int32_t h, d;
            for (h = 0; h < H; ++h) {
                const uint8_t *qrow = q8 + ((int64_t)b * H + h) * row_bytes;
                double qs = le_f32_value(qrow + D);
                for (d = 0; d < D; ++d)
                    qd[(int64_t)h * D + d] = oracle_e4m3_value(qrow[d]) * qs;
            }
        } else {
            for (i = 0; i < (int64_t)H * D; ++i)
                qd[i] = bf16_value(q[(int64_t)b * H * D + i]);
            if (mx) {
                int32_t h;
                for (h = 0; h < H; ++h)
                    oracle_mxfp4_round(qd + (int64_t)h * D, D, qd + (int64_t)h * D);
            }
        }
        for (c = 0; c < n_cols; ++c) {
            int64_t entry;
            int64_t prow = oracle_resolve(b, c, n_pool_rows, block_size,
                                          block_table, n_req, max_blocks, q_req,
                                          chunk_ids, n_chunks, max_chunks,
                                          limits, &entry);
            double v = -INFINITY;
            if (prow >= 0)
                v = logit_of_row(qd, w + (int64_t)b * H, H, D,
                                 pool + prow * row_bytes, k, mx);
            logits[(int64_t)b * n_cols + c] = v;
        }
        free(qd);
        free(k);
    }
    return failed ? -1 : 0;
}

int oracle_score(const uint16_t *q, const float *w, int32_t B, int32_t H,
                 int32_t D, const uint8_t *pool, int64_t n_pool_rows,
                 int32_t block_size, const int32_t *block_table, int32_t n_req,
                 int32_t max_blocks, const int32_t *q_req,
                 const int32_t *chunk_ids, const int32_t *n_chunks,
                 int32_t max_chunks, const int32_t *limits, int32_t n_cols,
                 double *logits, int32_t n_threads)
{
    return score_rows(q, NULL, w, B, H, D, pool, n_pool_rows, block_size,
                      block_table, n_req, max_blocks, q_req, chunk_ids,
                      n_chunks, max_chunks, limits, n_cols, logits, n_threads, 0);
}

/* The MXFP4 variant: q (bf16 bits) and the keys rounded to MXFP4 blocks of
 * 32 (section above), then the same definition. */
int oracle_score_mxfp4(const uint16_t *q, const float *w, int32_t B, int32_t H,
                       int32_t D, const uint8_t *pool, int64_t n_pool_rows,
                       int32_t block_size, const int32_t *block_table,
                       int32_t n_req, int32_t max_blocks, const int32_t *q_req,
                       const int32_t *chunk_ids, const int32_t *n_chunks,
                       int32_t max_chunks, const int32_t *limits, int32_t n_cols,
                       double *logits, int32_t n_threads)
{
    return score_rows(q, NULL, w, B, H, D, pool, n_pool_rows, block_size,
                      block_table, n_req, max_blocks, q_req, chunk_ids,
                      n_chunks, max_chunks, limits, n_cols, logits, n_threads, 1);
}

int oracle_score_q8(const uint8_t *q8, const float *w, int32_t B, int32_t H,
                    int32_t D, const uint8_t *pool, int64_t n_pool_rows,
                    int32_t block_size, const int32_t *block_table,
                    int32_t n_req, int32_t max_blocks, const int32_t *q_req,
                    const int32_t *chunk_ids, const int32_t *n_chunks,
                    int32_t max_chunks, const int32_t *limits, int32_t n_cols,
                    double *logits, int32_t n_threads)
{
    if (!q8)
        return -1;
    return score_rows(NULL, q8, w, B, H, D, pool, n_pool_rows, block_size,
                      block_table, n_req, max_blocks, q_req, chunk_ids,
                      n_chunks, max_chunks, limits, n_cols, logits, n_threads, 0);
}

double oracle_sigmoid(double x)
{
    return 1.0 / (1.0 + exp(-x));
}

/* [FM] "Retriever architecture": score = sigmoid(logit), for a whole array
 * of logits (an unscored column's -inf gives exp(+inf) = inf, so score 0). */
void oracle_sigmoid_array(const double *x, int64_t n, double *out)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i)
        out[i] = oracle_sigmoid(x[i]);
}

typedef struct {
    double v;
    int32_t c;
} vc_pair;

/* Larger value first; equal values: lower column first. */
static int cmp_desc(const void *pa, const void *pb)
{
    const vc_pair *a = (const vc_pair *)pa, *b = (const vc_pair *)pb;
    if (a->v > b->v)
        return -1;
    if (a->v < b->v)
        return 1;
    return (a->c > b->c) - (a->c < b->c);
}

/* [FM] "Two-level recall algorithm": keep the top-k (k = 512 there) of a
 * row's logits.  Brute force: sort every selectable entry and take the head
 * of the list.  out_col/out_val are [B, k]; missing places get column -1 and
 * value -inf.  Returns 0, or -1 on bad sizes / allocation failure. */
int oracle_topk(const double *vals, int32_t B, int32_t n_cols, int64_t ld,
                int32_t k, int32_t *out_col, double *out_val, int32_t n_threads)
{
    int32_t b;
    int failed = 0;
    if (B < 0 || n_cols < 0 || k <= 0 || ld < n_cols)
        return -1;
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (b = 0; b < B; ++b) {
        vc_pair *buf = (vc_pair *)malloc(sizeof(vc_pair) * (size_t)(n_cols + 1));
        int32_t n = 0, c, i;
        if (!buf) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
            continue;
        }
        for (c = 0; c < n_cols; ++c) {
            double v = vals[(int64_t)b * ld + c];
            if (isnan(v) || v == -INFINITY)
                continue;
            buf[n].v = v;
            buf[n].c = c;
            ++n;
        }
        qsort(buf, (size_t)n, sizeof(vc_pair), cmp_desc);
        for (i = 0; i < k; ++i) {
            int64_t o = (int64_t)b * k + i;
            if (i < n) {
                out_col[o] = buf[i].c;
                if (out_val)
                    out_val[o] = buf[i].v;
            } else {
                out_col[o] = -1;
                if (out_val)
                    out_val[o] = -INFINITY;
            }
        }
        free(buf);
    }
    return failed ? -1 : 0;
}

/* Column -> logical entry id (the id the attention step consumes); -1 stays
 * -1.  With a chunk list, column 64*j+s is entry chunk_ids[b][j]*64+s. */
int oracle_cols_to_entries(const int32_t *cols, int32_t B, int32_t k,
                           int32_t block_size, const int32_t *chunk_ids,
                           int32_t max_chunks, int32_t *entries)
{
    int32_t b, i;
    for (b = 0; b < B; ++b) {
        for (i = 0; i < k; ++i) {
            int32_t c = cols[(int64_t)b * k + i];
            int32_t e = -1;
            if (c >= 0) {
                if (chunk_ids) {
                    int32_t j = c / block_size, s = c % block_size;
                    e = chunk_ids[(int64_t)b * max_chunks + j] * block_size + s;
                } else {
                    e = c;
                }
            }
            entries[(int64_t)b * k + i] = e;
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Index-plane writer: a new compressed key (HEAD_DIM values) becomes one pool
 * row in the [FM] "compressed_k format" layout, the inverse of the dequant
 * above ([BG]: the fp8 indexer-pool insert kernel writes rows of that same
 * layout).  The pages do not state the scale rule; the reading taken here is
 * the per-row absolute maximum over the largest finite e4m3 value:
 *     s = amax / 448,  byte d = e4m3(k[d] / s)
 * with s and each quotient rounded to binary32 (IEEE division) and e4m3
 * rounding to the nearest value, ties to the even code, saturating at
 * +-448.  A row of zeros gets bytes 0 and scale 0.  Keys arrive as bf16.
 * ------------------------------------------------------------------------- */

/* Nearest finite e4m3fn value to y, by search over every finite magnitude
 * code (0x00 .. 0x7E, increasing in value); on an exact tie the even code
 * wins, which is round-half-to-even on the 3-bit mantissa.  Magnitudes past
 * 448 give 448.  The sign bit is y's own (so -0.0 and small negatives give
 * 0x80).  NaN input is not defined. */
uint8_t oracle_e4m3_encode(float y)
{
    double a = fabs((double)y);
    double best_d = INFINITY;
    int best = 0, c;
    for (c = 0; c <= 0x7E; ++c) {
        double d = fabs(oracle_e4m3_value((uint8_t)c) - a);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best_d = d;
            best = c;
        }
    }
    return (uint8_t)(best | (signbit(y) ? 0x80 : 0));
}

/* One key row: k bf16 [head_dim] -> row [head_dim + 4]. */
void oracle_quantize_row(const uint16_t *k, int32_t head_dim, uint8_t *row)
{
    float amax = 0.0f, scale;
    uint32_t bits;
    int32_t d;
    for (d = 0; d < head_dim; ++d) {
        float v = (float)bf16_value(k[d]);
        if (fabsf(v) > amax)
            amax = fabsf(v);
    }
    scale = amax / 448.0f;
    for (d = 0; d < head_dim; ++d) {
        float v = (float)bf16_value(k[d]);
        row[d] = amax == 0.0f ? 0 : oracle_e4m3_encode(v / scale);
    }
    memcpy(&bits, &scale, sizeof bits);
    row[head_dim + 0] = (uint8_t)(bits & 0xFF);
    row[head_dim + 1] = (uint8_t)((bits >> 8) & 0xFF);
    row[head_dim + 2] = (uint8_t)((bits >> 16) & 0xFF);
    row[head_dim + 3] = (uint8_t)(bits >> 24);
}

/* Write n keys k [n, head_dim] into pool rows slots[i] ([AT]: -1 is the
 * padding id and writes nothing).  A slot outside [0, n_pool_rows) writes
 * nothing either and is counted.  Returns the count of such slots. */
int64_t oracle_write_keys(const uint16_t *k, int64_t n, int32_t head_dim,
                          const int64_t *slots, uint8_t *pool,
                          int64_t n_pool_rows)
{
    int64_t i, bad = 0;
    for (i = 0; i < n; ++i) {
        int64_t r = slots[i];
        if (r == -1)
            continue;
        if (r < 0 || r >= n_pool_rows) {
            ++bad;
            continue;
        }
        oracle_quantize_row(k + i * head_dim, head_dim,
                            pool + r * (int64_t)(head_dim + 4));
    }
    return bad;
}

/* ---------------------------------------------------------------------------
 * Level 1 of [FM] "Two-level recall algorithm" (the Memory Indexer): the
 * retriever scores a row's whole history at several layers ([FM] "Joint
 * checkpoint + ensemble": three layers, each with its own weights), the
 * per-layer sigmoid scores of each compressed entry are ensembled (max, the
 * default, or mean), a threshold picks the query-critical entries, and the
 * recency tail and the attention sink are kept; pages are recalled whole,
 * the densest KMAX per request ([FM] "Quick start": KMAX pages of 64
 * entries).  Readings taken where the pages give no detail:
 *  - entry e of row b (e < limits[b], clamped to n_cols) is selected iff its
 *    ensemble score s >= threshold;
 *  - page p holds entries 64p .. 64p+63; its density is its count of
 *    selected entries; the row's history has P = ceil(limit / 64) pages;
 *  - pages p < n_sink and p >= P - n_recent are always resident ("forced");
 *  - the other pages with density > 0 follow in order of density (higher
 *    first), equal densities to the lower page; the first kmax pages of
 *    (forced pages, then that order) are the resident set, listed in
 *    ascending page order and padded with -1; out_count[b] is their number;
 *  - the scores given are the binary32 sigmoid values the scorer reports;
 *    the ensemble is taken in binary32 too, so that the threshold decision
 *    (an integer outcome) is made in the scorer's precision: max is exact,
 *    mean is the binary32 sum in layer order divided by L in binary32.
 * scores is [L][B][ld].  Returns 0, or -1 on bad sizes / allocation failure.
 * ------------------------------------------------------------------------- */
enum { ORACLE_ENSEMBLE_MAX = 0, ORACLE_ENSEMBLE_MEAN = 1 };

typedef struct {
    int32_t rank;   /* 2: forced, 1: density > 0, 0: not resident */
    int32_t density;
    int32_t page;
} page_rank;

/* Forced pages first, then higher density, then the lower page. */
static int cmp_page(const void *pa, const void *pb)
{
    const page_rank *a = (const page_rank *)pa, *b = (const page_rank *)pb;
    if (a->rank != b->rank)
        return a->rank > b->rank ? -1 : 1;
    if (a->density != b->density)
        return a->density > b->density ? -1 : 1;
    return (a->page > b->page) - (a->page < b->page);
}

static int cmp_int(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

int oracle_level1_select(const float *scores, int32_t L, int32_t B,
                         int32_t n_cols, int64_t ld, const int32_t *limits,
                         int32_t ensemble, float threshold, int32_t n_sink,
                         int32_t n_recent, int32_t kmax, int32_t *out_pages,
                         int32_t *out_count)
{
    int32_t b;
    if (L < 1 || B < 0 || n_cols < 0 || ld < n_cols || kmax < 1 ||
        n_sink < 0 || n_recent < 0 ||
        (ensemble != ORACLE_ENSEMBLE_MAX && ensemble != ORACLE_ENSEMBLE_MEAN))
        return -1;
    for (b = 0; b < B; ++b) {
        int32_t hist = limits[b] < 0 ? 0 : (limits[b] > n_cols ? n_cols : limits[b]);
        int32_t P = (hist + 63) / 64, p, e, l, n = 0, i;
        page_rank *pr = (page_rank *)calloc((size_t)P + 1, sizeof(page_rank));
        int32_t *chosen = (int32_t *)malloc(sizeof(int32_t) * ((size_t)P + 1));
        if (!pr || !chosen) {
            free(pr);
            free(chosen);
            return -1;
        }
        for (p = 0; p < P; ++p)
            pr[p].page = p;
        for (e = 0; e < hist; ++e) {
            float s;
            if (ensemble == ORACLE_ENSEMBLE_MAX) {
                s = scores[(int64_t)b * ld + e];
                for (l = 1; l < L; ++l) {
                    float x = scores[((int64_t)l * B + b) * ld + e];
                    if (x > s)
                        s = x;
                }
            } else {
                float sum = 0.0f;
                for (l = 0; l < L; ++l)
                    sum += scores[((int64_t)l * B + b) * ld + e];
                s = sum / (float)L;
            }
            if (s >= threshold)
                pr[e / 64].density += 1;
        }
        for (p = 0; p < P; ++p) {
            if (p < n_sink || p >= P - n_recent)
                pr[p].rank = 2;
            else
                pr[p].rank = pr[p].density > 0 ? 1 : 0;
        }
        qsort(pr, (size_t)P, sizeof(page_rank), cmp_page);
        for (i = 0; i < P && n < kmax; ++i)
            if (pr[i].rank > 0)
                chosen[n++] = pr[i].page;
        qsort(chosen, (size_t)n, sizeof(int32_t), cmp_int);
        for (i = 0; i < kmax; ++i)
            out_pages[(int64_t)b * kmax + i] = i < n ? chosen[i] : -1;
        if (out_count)
            out_count[b] = n;
        free(pr);
        free(chosen);
    }
    return 0;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
