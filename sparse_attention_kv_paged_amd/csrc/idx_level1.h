// Internal launch interface of the Level-1 page pass (idx_level1.hip), used
// by the C-ABI layer (idx_api.cpp).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace idx {

struct PageArgs {
    const float *scores;        // [L][B][ld] binary32 sigmoid scores
    int32_t L;
    int32_t B;
    int64_t ld;                 // row stride of one layer's scores
    int64_t layer_stride;       // B * ld
    int32_t n_cols;             // scored columns (logical entries) per row
    const int32_t *limits;      // [B] history length of each row
    int32_t ensemble;           // IDX_ENSEMBLE_MAX or IDX_ENSEMBLE_MEAN
    float threshold;
    int32_t n_sink;
    int32_t n_recent;
    float *page_keys;           // [B, ldp] out
    int64_t ldp;
    int32_t n_pages;            // ceil(n_cols / 64)
    // selection bits instead of scores (max ensemble, launch_select_bits):
    // [L][B][bits_ld] words, bit i of word j of a row = (score of column
    // 32*j + i >= threshold)
    const uint32_t *bits;
    int64_t bits_ld;
    // the selection itself (launch_select_bits): kmax pages per row
    int32_t kmax;
    int32_t *out_pages;         // [B, kmax]
    int32_t *out_count;         // [B] or null
};

hipError_t launch_pages(const PageArgs &a, hipStream_t s);
// Pages straight from the selection bits (max ensemble), without page keys
// and a separate top-k: one workgroup per row.
hipError_t launch_select_bits(const PageArgs &a, hipStream_t s);

}  // namespace idx
