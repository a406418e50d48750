// Level-1 resident-set selection for gfx950: the page pass between the
// per-layer scoring (score kernel, sigmoid output) and the top-KMAX page
// selection (segment top-k kernel) ("FlashMemory-DeepSeek-V4" README,
// sections "Two-level recall algorithm" and "Joint checkpoint + ensemble";
// KMAX pages of 64 entries per request, section "Quick start").
//
// One wave per 64-entry page: lane e reads entry 64p + e of every layer's
// score row (one 256-byte coalesced load per layer), ensembles them (max, or
// the binary32 sum in layer order divided by L), compares with the threshold,
// and the ballot's popcount is the page's density.  The page's key for the
// selection is +inf for a sink or recent page (always resident), the density
// for another page with at least one selected entry, and -inf otherwise (past
// the row's history too); the top-k over these keys then keeps the forced
// pages, then the densest, equal densities to the lower page, in ascending
// page order.
#include <hip/hip_runtime.h>

#include "../../include/idx.h"
#include "idx_internal.h"
#include "idx_level1.h"

namespace idx {
namespace {

constexpr int kPageWaves = 4;

__global__ __launch_bounds__(64 * kPageWaves) void page_kernel(PageArgs a) {
    const int b = blockIdx.y;
    const int p = blockIdx.x * kPageWaves + threadIdx.x / 64;
    const int lane = threadIdx.x % 64;
    if (p >= a.n_pages) return;                       // uniform per wave
    const int hist = max(0, min(a.limits[b], a.n_cols));
    const int P = (hist + kBlock - 1) / kBlock;
    const int e = p * kBlock + lane;
    const bool valid = e < hist;
    float s = 0.0f;
    if (valid) {
        const float *row = a.scores + (int64_t)b * a.ld + e;
        if (a.ensemble == IDX_ENSEMBLE_MAX) {
            s = row[0];
            for (int l = 1; l < a.L; ++l) {
                const float x = row[(int64_t)l * a.layer_stride];
                s = x > s ? x : s;
            }
        } else {
            float sum = 0.0f;
            for (int l = 0; l < a.L; ++l) sum += row[(int64_t)l * a.layer_stride];
            s = sum / (float)a.L;
        }
    }
    const int density = __popcll(__ballot(valid && s >= a.threshold));
    if (lane == 0) {
        float key = -__builtin_inff();
        if (p < P) {
            if (p < a.n_sink || p >= P - a.n_recent) key = __builtin_inff();
            else if (density > 0) key = (float)density;
        }
        a.page_keys[(int64_t)b * a.ldp + p] = key;
    }
}

}  // namespace

hipError_t launch_pages(const PageArgs &a, hipStream_t s) {
    if (a.B <= 0 || a.n_pages <= 0) return hipSuccess;
    const dim3 grid((unsigned)((a.n_pages + kPageWaves - 1) / kPageWaves), (unsigned)a.B);
    hipLaunchKernelGGL(page_kernel, grid, dim3(64 * kPageWaves), 0, s, a);
    return hipGetLastError();
}

}  // namespace idx
