// Internal interface of the q8 update, used by the full optimizer step.
#pragma once
#include <hip/hip_runtime.h>

#include "plan_layout.h"
#include "qmuon.h"

namespace qm {

struct UpdateWorkspace {
    double *block_sums;  // [n_blocks]
    double *partials;    // [n_chunks]
    double *group_sums;  // [n_groups]
    float *inv;          // [n_groups]
    size_t bytes;
};

UpdateWorkspace update_workspace(const PlanHeader *h, void *ws);

qm_status validate_update(const void *host_plan, const void *dev_plan, float beta,
                          const PlanHeader **out);

// A tall tensor whose MXFP8 carrier goes to Newton-Schulz transposed (the
// row-wise carrier of m^T: data (cols, rows), one scale per 32 rows of a
// column).  rows % 32 == 0, cols % 256 == 0, tensor < 64.
struct TallCarrier {
    int32_t tensor;
    int64_t rows, cols;
};

// Update + per-group inverse norms (+ the in-place scale pass if asked).
// inv_out / sums_out may be null: the workspace sections are used.  ro:
// requantisation rounding (null: nearest).  carrier_data / carrier_scale
// non-null: m goes to the MXFP8 carrier (bytes [n_blocks * 256], scales
// [n_blocks * 8]) instead of the grad buffers; nearest rounding; every
// tensor's numel a multiple of 32 (checked by the caller).
qm_status run_update_normalize(const PlanHeader *h, const void *dev_plan, float beta, float eps,
                               bool write_normalized, float *inv_out, double *sums_out, void *ws,
                               const qm_round_opts *ro, hipStream_t stream, uint8_t *carrier_data = nullptr,
                               uint8_t *carrier_scale = nullptr, const void *host_plan = nullptr,
                               const TallCarrier *tall = nullptr, int n_tall = 0);

// QM_OK if every tensor of the plan can carry an MXFP8 carrier (numel a
// multiple of 32) and the two arrays are usable; else the error, recorded.
qm_status check_carrier(const PlanHeader *h, const void *host_plan, const void *data, const void *scale);

}  // namespace qm
