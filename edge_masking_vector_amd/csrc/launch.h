// launch.h -- internal launchers of libtilemap's kernels.  Each takes a plan that plan.cpp has
// already validated and enqueues the kernel(s) on `stream` with hipLaunchKernel, returning the
// launch status of exactly these launches.
#pragma once

#include <hip/hip_runtime_api.h>

#include "plan.h"

namespace tmk {

hipError_t launch_map(const tmp::MapPlan &plan, hipStream_t stream);
hipError_t launch_map_flat(const tmp::MapPlan &plan, hipStream_t stream);  // plan.flat
hipError_t launch_rows(const tmp::RowPlan &plan, hipStream_t stream);
hipError_t launch_cols(const tmp::ColPlan &plan, hipStream_t stream);
hipError_t launch_transpose(const tmp::TransposePlan &plan, hipStream_t stream);

}  // namespace tmk
