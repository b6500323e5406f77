// Planner: turns cu_seqlens into the sorted work-unit list of a pass (see
// Plan in va_kernels.h).  One workgroup per plan, run right before the pass
// on the same stream; it rewrites the whole plan, so a call needs no memset
// and no host read of device memory.
//
// Steps: (1) count, for the fixed chunk and for 2x, 4x, ... 32x it, the units,
// partial slots and split tiles every tile needs, and take the smallest
// chunk whose partials fit the workspace (normally the fixed one, so the
// split of a tile depends on its own sequence only; a batch too large for
// the workspace gets coarser chunks, or none, rather than failing);
// (2) histogram the units by step count and scan it from the largest count
// down; (3) place every unit at its bin's cursor.
// Within a bin the order is whatever the LDS atomics give: the units of a
// bin cost the same, and a unit's results depend neither on its position
// nor on the workgroup that runs it.
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
