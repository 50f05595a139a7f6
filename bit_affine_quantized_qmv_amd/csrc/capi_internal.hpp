// Helpers the C ABI entry points in different source files share (host only).
#pragma once

#include <hip/hip_runtime.h>

#include <string>

#include "../../include/qmm.h"
#include "kernels.hpp"

namespace qmm {

// Set the calling thread's error message (cleared for QMM_OK) and return rc.
int32_t report(int32_t rc, const std::string& msg);
// QMM_OK for hipSuccess, else QMM_ERR_HIP with the runtime's message.
int32_t report_launch(hipError_t e);

// Validate a decode call with a fused argmax (everything but its workspace) and fill `out`
// with the kernel arguments (workspace pointers unset) and *rows with the collapsed
// activation rows (0: nothing to launch).  Returns QMM_OK or the error, message set.
int32_t prepare_qmv_argmax(const void* x, const qmm_tensor_desc_t* x_desc, const qmm_weight_desc_t* w, void* y,
                           const qmm_tensor_desc_t* y_desc, int32_t* out_index, float* out_value, MatArgs* out,
                           int64_t* rows);

}  // namespace qmm
