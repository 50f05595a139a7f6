// Host-side validation and planning shared by the C ABI entry points (no GPU calls).
#pragma once

#include <string>

#include "../../include/qmm.h"

namespace qmm {

// bits / group_size / dtype support check.
int check_codec(int32_t group_size, int32_t bits, int32_t dtype, std::string* err);

// Validate a qmv (entry 0) or qmm_t (entry 1) call and fold x's batch dims into a plan.
// With require_pointers == false, NULL data pointers are allowed (layout-only queries).
int plan_matmul(const void* x, const qmm_tensor_desc_t* xd, const qmm_weight_desc_t* w,
                const void* y, const qmm_tensor_desc_t* yd, uint32_t flags, int entry,
                bool require_pointers, qmm_plan_t* out, std::string* err);

}  // namespace qmm
