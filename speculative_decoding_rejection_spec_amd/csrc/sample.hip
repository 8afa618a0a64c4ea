// sample.hip -- the drafter's sampling step (spec_draft_sample): per row, a
// token drawn from softmax(z / T) by the inverse CDF with the row's uniform
// (page "投机解码", section 动手实践: the draft model samples each token from
// its tempered softmax), or the argmax at T = 0.  Two launches, one read of
// each row:
//
//   sample_sums (grid rows x chunks, 256 threads): wave w of a chunk's
//     workgroup covers sub-chunk w.  Sampling rows: its largest logit, a
//     reference Y_s that is a whole number of octaves (256 per octave in the
//     draw's Y = 256 z log2(e) / T units; rescaling between such references
//     is exact) at most 32 octaves below the largest Y, and the fp64 sum of
//     2^((Y - Y_s) / 256) over the sub-chunk, in one read.  Greedy rows: its
//     largest logit and the lowest id holding it.
//   sample_pick (one workgroup per row): the row's maximum over the
//     sub-chunks (a non-finite one is a data error, as in the verify), the
//     common reference Y_0 = max Y_s, the sub-chunk masses rescaled to it,
//     the sub-chunk that crosses u Z, and the scan of that sub-chunk shared
//     with the verify's pick.
//
// No row pass is needed: the weights are taken relative to the sub-chunks'
// own references instead of the row maximum, which changes every weight by
// the same factor and so neither the distribution nor the draw.
#include "draw_pass.h"

namespace sv {
namespace {

template <int DT>
__global__ __launch_bounds__(kThreads) void sample_sums_kernel(Problem p, Plan plan) {
    using namespace drawpass;
    using E = typename Vec<DT>::E;
    const int64_t w = blockIdx.x;
    const int32_t b = static_cast<int32_t>(w / plan.nchunk);
    const int32_t c = static_cast<int32_t>(w - static_cast<int64_t>(b) * plan.nchunk);
    const float T = p.temperature[b];
    if (!temperature_ok(T)) return;                      // the pick reports it
    __shared__ TabEntry tbl[256];
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int64_t s0, s1;
    sub_range<DT>(p, plan, c, wave, &s0, &s1);
    ChunkSums* out = plan.csum + (static_cast<int64_t>(b) * plan.nchunk + c) * kWaves + wave;
    const E* row = static_cast<const E*>(p.target) + static_cast<int64_t>(b) * p.V;

    if (T == 0.f) {
        // lowest id holding the maximum: each lane visits its ids in increasing order
        float m = -INFINITY;
        int32_t a = INT32_MAX;
        for (int64_t v = s0 + lane; v < s1; v += 64) {
            const float z = load_logit(row, DT, v);
            if (z > m) { m = z; a = static_cast<int32_t>(v); }
        }
        for (int off = 32; off > 0; off >>= 1) {
            const float m2 = __shfl_xor(m, off, 64);
            const int32_t a2 = __shfl_xor(a, off, 64);
            if (m2 > m || (m2 == m && a2 < a)) { m = m2; a = a2; }
        }
        if (lane == 0) {
            out->a = m;
            out->b = a;
        }
        return;
    }
    load_exp2_table(tbl, kThreads);
    __syncthreads();
    const double C = 256.0 * kLog2e / static_cast<double>(T);
    const Rows<DT> rows{row, row, C, 0.0, 0.0, tbl};
    double sum, R;
    float mx;
    self_ref_sum<DT>(rows, s0, s1, &sum, &R, &mx);
    if (lane == 0) {
        out->sp = sum;
        out->sq = R;
        out->a = mx;
    }
}

// Block-wide (NT threads) reductions through L's scratch.
template <int NT>
__device__ __forceinline__ void block_argmax(float& m, int32_t& a, double (*red)[2], int32_t* ldsi) {
    for (int off = 32; off > 0; off >>= 1) {
        const float m2 = __shfl_xor(m, off, 64);
        const int32_t a2 = __shfl_xor(a, off, 64);
        if (m2 > m || (m2 == m && a2 < a)) { m = m2; a = a2; }
    }
    __syncthreads();
    if ((threadIdx.x & 63) == 0) { red[threadIdx.x >> 6][0] = m; ldsi[threadIdx.x >> 6] = a; }
    __syncthreads();
    m = static_cast<float>(red[0][0]);
    a = ldsi[0];
    for (int w = 1; w < NT / 64; ++w) {
        const float m2 = static_cast<float>(red[w][0]);
        if (m2 > m || (m2 == m && ldsi[w] < a)) { m = m2; a = ldsi[w]; }
    }
}

template <int DT, int NT>
__global__ __launch_bounds__(NT, 4) void sample_pick_kernel(Problem p, Plan plan) {
    using namespace drawpass;
    using E = typename Vec<DT>::E;
    const int32_t b = blockIdx.x;
    const int tid = threadIdx.x;
    const float T = p.temperature[b];
    __shared__ TabEntry tbl[256];
    __shared__ PickLds<NT> L;
    auto data_error = [&]() {
        if (tid == 0) {
            p.out_tokens[b] = -1;
            if (p.out_emit_prob) p.out_emit_prob[b] = NAN;
        }
    };
    if (!temperature_ok(T)) { data_error(); return; }
    const int32_t nsub = plan.nchunk * kWaves;
    const ChunkSums* cs = plan.csum + static_cast<int64_t>(b) * nsub;

    if (T == 0.f) {
        float m = -INFINITY;
        int32_t a = INT32_MAX;
        for (int32_t j = tid; j < nsub; j += NT) {
            const float m2 = static_cast<float>(cs[j].a);
            const int32_t a2 = static_cast<int32_t>(cs[j].b);
            if (m2 > m || (m2 == m && a2 < a)) { m = m2; a = a2; }
        }
        block_argmax<NT>(m, a, L.red2, L.ldsi);
        if (!(fabsf(m) <= 3.4e38f)) { data_error(); return; }
        if (tid == 0) {
            p.out_tokens[b] = a;
            if (p.out_emit_prob) p.out_emit_prob[b] = 1.f;   // the T -> 0 limit: a point mass
        }
        return;
    }
    load_exp2_table(tbl, NT);
    // Every sub-chunk's record is loaded before anything depends on it.
    float mx = -INFINITY;
    double Y0 = -INFINITY;
    for (int32_t j = tid; j < nsub; j += NT) {
        const double y = cs[j].sq;
        L.spc[j] = cs[j].sp;
        L.mass[j] = y;                                    // (the reference, until rescaled)
        mx = fmaxf(mx, static_cast<float>(cs[j].a));
        Y0 = fmax(Y0, y);
    }
    pick_max2<NT>(mx, Y0, L.red2);                       // (its barriers also publish spc, mass)
    if (!(fabsf(mx) <= 3.4e38f)) { data_error(); return; }
    for (int32_t j = tid; j < nsub; j += NT) {
        const double y = L.mass[j];
        // exact rescale by a whole number of octaves (no sub-chunk: -inf)
        L.spc[j] = y == -INFINITY ? 0.0 : ldexp(L.spc[j], static_cast<int>(fmax((y - Y0) / 256.0, -2048.0)));
    }
    __syncthreads();
    if (tid < 64) {
        double Z = 0.0, base = 0.0;
        int32_t chunk = 0;
        find_chunk(L.spc, nsub, static_cast<double>(p.uniforms[b]), &Z, &chunk, &base);
        if (tid == 0) {
            L.base = base;
            L.Z = Z;
            L.target = static_cast<double>(p.uniforms[b]) * Z;
            L.chunk = chunk;
        }
    }
    __syncthreads();
    const double C = 256.0 * kLog2e / static_cast<double>(T);
    const E* row = static_cast<const E*>(p.target) + static_cast<int64_t>(b) * p.V;
    const Rows<DT> rows{row, row, C, -Y0, 0.0, tbl};
    pick_scan<DT, NT, kMaxPickSubs>(p, plan, rows, false, 1.0, 0.0, b, b, L);
}

}  // namespace

hipError_t launch_sample_sums(const Problem& p, const Plan& plan, hipStream_t s) {
    const int64_t blocks = static_cast<int64_t>(p.B) * plan.nchunk;
    if (p.dtype == SV_BF16)
        sample_sums_kernel<SV_BF16><<<dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s>>>(p, plan);
    else
        sample_sums_kernel<SV_F32><<<dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s>>>(p, plan);
    return hipGetLastError();
}

// One 512-thread workgroup per row (as the verify's pick).
hipError_t launch_sample_pick(const Problem& p, const Plan& plan, hipStream_t s) {
    const dim3 grid(static_cast<uint32_t>(p.B));
    if (p.dtype == SV_BF16)
        sample_pick_kernel<SV_BF16, 512><<<grid, dim3(512), 0, s>>>(p, plan);
    else
        sample_pick_kernel<SV_F32, 512><<<grid, dim3(512), 0, s>>>(p, plan);
    return hipGetLastError();
}

}  // namespace sv
