// accept.hip -- the staged accept scan: one wave64 per sequence (the scan
// itself is in accept_scan.h).  (Early exit's scan over the leading
// positions runs inside the first round, lead_pass.h.)
#include "accept_scan.h"

namespace sv {
namespace {

// One wave per workgroup: the scans spread over B compute units (256
// sequences of k = 8: 9.7 -> 8.6 us against four waves per workgroup).
__global__ __launch_bounds__(64) void accept_kernel(Problem p, Plan plan) {
    plan.epoch = call_epoch(plan);
    const int32_t b = blockIdx.x;
    if (plan.lead > 0 && plan.done[b]) return;     // decided by its leading positions
    accept_sequence<false>(p, plan, b);
}

}  // namespace

hipError_t launch_accept(const Problem& p, const Plan& plan, hipStream_t s) {
    accept_kernel<<<dim3(static_cast<uint32_t>(p.B)), dim3(64), 0, s>>>(p, plan);
    return hipGetLastError();
}

}  // namespace sv
