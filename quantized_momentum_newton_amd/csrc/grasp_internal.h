// Internal hook from the GRASP step into the Newton-Schulz driver.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmuon.h"

namespace qm {

size_t ns_f32_workspace_bytes(int64_t rows, int64_t cols);

// NS (fp32 operands: precision QM_NS_F32 or QM_NS_BF16X3; norm computed
// from M) of the fp32 rows x cols matrix M into `out` (same shape,
// contiguous, out_dtype), with W <- W - lr_s O - lr_wd W when w is not null.
qm_status run_ns_f32_into(const float *M, int64_t rows, int64_t cols, void *out, int32_t out_dtype, float *w,
                          float lr_s, float lr_wd, int steps, float a, float b, float c, float eps, int32_t precision,
                          void *ws, hipStream_t stream);

}  // namespace qm
