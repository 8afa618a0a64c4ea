// accept.hip -- the staged accept scan: one wave64 per sequence (the scan
// itself is in accept_scan.h).
#include "accept_scan.h"

namespace sv {
namespace {

__global__ __launch_bounds__(kThreads) void accept_kernel(Problem p, Plan plan) {
    const int32_t b = blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (b >= p.B) return;                          // whole wave leaves together
    accept_sequence<false>(p, plan, b);
}

}  // namespace

hipError_t launch_accept(const Problem& p, const Plan& plan, hipStream_t s) {
    const int64_t blocks = (static_cast<int64_t>(p.B) + kWaves - 1) / kWaves;
    accept_kernel<<<dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s>>>(p, plan);
    return hipGetLastError();
}

}  // namespace sv
