// Planner: turns cu_seqlens into the sorted work-unit list of a pass (see
// Plan in va_kernels.h).  One workgroup per plan, run right before the pass
// on the same stream; it also zeroes the pass's queue cursor, so a call
// needs no memset and no host read of device memory.
//
// Steps: (1) count the units of every tile (tiles spread over the threads)
// and histogram them by step count; if the split units would not
// fit the workspace's partial slots, count again without splitting (all or
// nothing, so the split rule stays per tile); (2) scan the histogram from
// the largest step count down; (3) place every unit at its bin's cursor.
// Within a bin the order is whatever the atomics give: the units of a bin
// are independent, and a unit's results do not depend on its position.
#include "va_plan.h"

namespace va {

namespace {

__global__ __launch_bounds__(plan::PT) void plan_kernel(PlanSet set) {
  __shared__ plan::PlanShared sh;
  plan::plan_body(set.p[blockIdx.x], sh);
}

}  // namespace

hipError_t launch_plan(const PlanSet& s, int nplans, hipStream_t st) {
  timing_before(st, "plan");
  hipLaunchKernelGGL(plan_kernel, dim3(nplans), dim3(plan::PT), 0, st, s);
  timing_after(st);
  return hipGetLastError();
}

}  // namespace va
