// stream_probe.hip -- a bare read-reduce kernel: the practical HBM read
// ceiling the row pass is measured against.  It reads like the row pass
// (256-thread workgroups, one contiguous segment each, 16-byte raw buffer
// loads with 8 in flight per lane, non-temporal) and does the least work
// that keeps every load live: an XOR of the loaded dwords, one word per
// workgroup written out.
#include "sv_internal.h"

namespace sv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kWindow = 8;
constexpr int kBufferDword3 = 0x00020000;   // raw buffer descriptor word 3 (gfx9 family)
constexpr int kLoadNonTemporal = 2;

__global__ __launch_bounds__(kThreads) void stream_probe_kernel(const uint8_t* data, int64_t bytes,
                                                                int64_t seg_bytes, uint32_t* out) {
    const int64_t s0 = static_cast<int64_t>(blockIdx.x) * seg_bytes;
    const int64_t s1 = min(bytes, s0 + seg_bytes);
    const int32_t nvec = static_cast<int32_t>((s1 - s0) / 16);
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(data + s0), 0, nvec * 16, kBufferDword3);
    const int32_t voff = threadIdx.x * 16;
    constexpr int32_t kTile = kThreads * 16;
    const int32_t nt = (nvec + kThreads - 1) / kThreads;
    auto load = [&](int32_t t) {
        return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, t * kTile,
                                                                               kLoadNonTemporal));
    };
    u32x4 buf[kWindow];
#pragma unroll
    for (int u = 0; u < kWindow; ++u) buf[u] = load(u);
    uint32_t acc = 0;
    for (int32_t i = 0; i < nt; i += kWindow) {
#pragma unroll
        for (int u = 0; u < kWindow; ++u) {
            acc ^= buf[u][0] ^ buf[u][1] ^ buf[u][2] ^ buf[u][3];   // loads past the end read zeros
            buf[u] = load(i + kWindow + u);
        }
    }
    for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
    __shared__ uint32_t w[kWaves];
    if ((threadIdx.x & 63) == 0) w[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int i = 0; i < kWaves; ++i) r ^= w[i];
        out[blockIdx.x] = r;
    }
}

}  // namespace

hipError_t launch_stream_probe(const void* data, int64_t bytes, int64_t seg_bytes, uint32_t* out,
                               hipStream_t s) {
    const int64_t blocks = (bytes + seg_bytes - 1) / seg_bytes;
    if (blocks == 0) return hipSuccess;
    stream_probe_kernel<<<dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s>>>(
        static_cast<const uint8_t*>(data), bytes, seg_bytes, out);
    return hipGetLastError();
}

}  // namespace sv
