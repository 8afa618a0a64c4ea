// accept.hip -- the staged accept scan: one wave64 per sequence (the scan
// itself is in accept_scan.h); with early exit also the scan over the
// leading positions, which settles every sequence they decide.
#include "accept_scan.h"

namespace sv {
namespace {

__global__ __launch_bounds__(kThreads) void accept_kernel(Problem p, Plan plan) {
    const int32_t b = blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (b >= p.B) return;                          // whole wave leaves together
    if (plan.lead > 0 && plan.done[b]) return;     // decided by its leading positions
    accept_sequence<false>(p, plan, b);
}

// Early exit: the accept scan over the leading positions only.
__global__ __launch_bounds__(kThreads) void accept_lead_kernel(Problem p, Plan plan) {
    const int32_t b = blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (b >= p.B) return;
    accept_sequence<false>(p, plan, b, plan.lead, plan.done + b);
}

}  // namespace

hipError_t launch_accept(const Problem& p, const Plan& plan, hipStream_t s) {
    const int64_t blocks = (static_cast<int64_t>(p.B) + kWaves - 1) / kWaves;
    accept_kernel<<<dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s>>>(p, plan);
    return hipGetLastError();
}

hipError_t launch_accept_lead(const Problem& p, const Plan& plan, hipStream_t s) {
    const int64_t blocks = (static_cast<int64_t>(p.B) + kWaves - 1) / kWaves;
    accept_lead_kernel<<<dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s>>>(p, plan);
    return hipGetLastError();
}

}  // namespace sv
