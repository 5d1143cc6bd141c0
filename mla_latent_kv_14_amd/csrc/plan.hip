// Device-side work planner for split-KV decode, in a launch of its own (the
// planner itself is plan_body in plan_body.h).
#include "common.h"
#include "internal.h"
#include "plan_body.h"

namespace mla {
namespace {

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs pa) {
  __shared__ PlanShared sh;
  plan_body(pa, sh);
}

}  // namespace

hipError_t launch_plan(const mla_dims& d, const int32_t* seq_lens, int splits, int grid, int min_chunk, int ov,
                       int32_t* ws, hipStream_t stream, int hg_log2) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream,
                     make_plan_args(d, seq_lens, splits, grid, min_chunk, ov, ws, hg_log2));
  return hipGetLastError();
}

}  // namespace mla
