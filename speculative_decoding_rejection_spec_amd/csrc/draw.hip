// draw.hip -- the emitted token of every sampling sequence, in fp64.
//
// After the first rejection at position n the token is drawn from
// max(0, p_n - q_n) / Z, Z = sum_v max(0, p_n(v) - q_n(v)) (page "投机解码",
// section 无损保证：数学推导, reject-path equation; page
// "大模型推理无损加速:投机采样...", section 二.2); if all k drafts were accepted
// it is drawn from p_k (the bonus token, section 投机解码的三步流程).  The draw
// is an inverse CDF over ascending token ids with the supplied uniform u:
// t* = min{t : C_t > u Z}, C_t = sum_{v <= t} r_v.
//
// Tokens in the tail of a 10^5-entry distribution carry masses near 1e-10 and
// sit closer together than fp32 rounding, so a CDF built in fp32 picks a
// different token in a measurable fraction of draws.  Every quantity here is
// fp64: w = exp((z - m) / T) from the exact logits and row maxima, and fp64
// sums.  Three kernels, all on the caller's stream:
//   draw_sums     (grid B x nchunk): per chunk, sum of w over the target row
//                 and (residual) the draft row -> fp64 normalisers S_p, S_q;
//   draw_residual (grid B x nchunk, residual sequences only): per chunk
//                 residual mass R_c = sum max(0, w_t/S_p - w_d/S_q);
//   draw_pick     (grid B): prefix over chunk masses locates the chunk that
//                 holds u Z, then a workgroup-wide fp64 prefix scan over that
//                 one chunk locates t*.
// A bonus draw uses the unnormalised masses w_t (chunk masses are draw_sums'
// target sums); the comparison C_t > u Z is unchanged by the common factor.
#include "sv_internal.h"

namespace sv {
namespace {

constexpr double kDegenerateZ = 1e-9;   // residual mass treated as empty

__device__ __forceinline__ double wexp(const void* rows, int32_t dtype, int64_t idx, double m, double T) {
    return exp((static_cast<double>(load_logit(rows, dtype, idx)) - m) / T);
}

__global__ __launch_bounds__(kThreads) void draw_sums_kernel(Problem p, Plan plan) {
    const int64_t w = blockIdx.x;
    const int32_t b = static_cast<int32_t>(w / plan.nchunk);
    const int64_t c = w - static_cast<int64_t>(b) * plan.nchunk;
    const DrawTask t = plan.task[b];
    if (t.kind == kNone) return;
    const int64_t v0 = c * plan.chunk_len, v1 = min(p.V, v0 + plan.chunk_len);
    const double T = t.T, mt = t.m_t, md = t.m_d;
    const int64_t tb = t.trow * p.V, db = t.drow * p.V;
    double st = 0.0, sd = 0.0;
    for (int64_t v = v0 + threadIdx.x; v < v1; v += kThreads) {
        st += wexp(p.target, p.dtype, tb + v, mt, T);
        if (t.kind == kResidual) sd += wexp(p.draft, p.dtype, db + v, md, T);
    }
    __shared__ double lds[kWaves];
    st = block_sum(st, lds);
    sd = block_sum(sd, lds);
    if (threadIdx.x == 0) {
        plan.csum[2 * w] = st;
        plan.csum[2 * w + 1] = sd;
    }
}

// Residual mass of token v given the fp64 normalisers.
__device__ __forceinline__ double residual_mass(const Problem& p, const DrawTask& t, int64_t v,
                                                double Sp, double Sq) {
    const double pv = wexp(p.target, p.dtype, t.trow * p.V + v, t.m_t, t.T) / Sp;
    const double qv = wexp(p.draft, p.dtype, t.drow * p.V + v, t.m_d, t.T) / Sq;
    return fmax(0.0, pv - qv);
}

__device__ __forceinline__ void normalisers(const Plan& plan, int32_t b, double& Sp, double& Sq) {
    Sp = 0.0;
    Sq = 0.0;
    const double* cs = plan.csum + 2 * static_cast<int64_t>(b) * plan.nchunk;
    for (int32_t c = 0; c < plan.nchunk; ++c) { Sp += cs[2 * c]; Sq += cs[2 * c + 1]; }
}

__global__ __launch_bounds__(kThreads) void draw_residual_kernel(Problem p, Plan plan) {
    const int64_t w = blockIdx.x;
    const int32_t b = static_cast<int32_t>(w / plan.nchunk);
    const int64_t c = w - static_cast<int64_t>(b) * plan.nchunk;
    const DrawTask t = plan.task[b];
    if (t.kind != kResidual) return;
    double Sp, Sq;
    normalisers(plan, b, Sp, Sq);
    const int64_t v0 = c * plan.chunk_len, v1 = min(p.V, v0 + plan.chunk_len);
    double r = 0.0;
    for (int64_t v = v0 + threadIdx.x; v < v1; v += kThreads) r += residual_mass(p, t, v, Sp, Sq);
    __shared__ double lds[kWaves];
    r = block_sum(r, lds);
    if (threadIdx.x == 0) plan.cres[w] = r;
}

__global__ __launch_bounds__(kThreads) void draw_pick_kernel(Problem p, Plan plan) {
    const int32_t b = blockIdx.x;
    const DrawTask t = plan.task[b];
    if (t.kind == kNone) return;

    __shared__ double sh_base, sh_target, sh_Sp, sh_Sq;
    __shared__ int32_t sh_chunk, sh_resid;
    __shared__ double lds[kWaves];
    __shared__ int32_t lds_i[kWaves];

    if (threadIdx.x == 0) {
        double Sp, Sq;
        normalisers(plan, b, Sp, Sq);
        const int64_t cb = static_cast<int64_t>(b) * plan.nchunk;
        bool resid = (t.kind == kResidual);
        double Z = 0.0;
        if (resid) {
            for (int32_t c = 0; c < plan.nchunk; ++c) Z += plan.cres[cb + c];
            if (Z < kDegenerateZ) resid = false;       // fall back to p_n
        }
        if (!resid) {
            Z = 0.0;
            for (int32_t c = 0; c < plan.nchunk; ++c) Z += plan.csum[2 * (cb + c)];
        }
        const double target = static_cast<double>(t.u) * Z;
        double base = 0.0, last_base = 0.0;
        int32_t chunk = -1, last = 0;
        for (int32_t c = 0; c < plan.nchunk; ++c) {
            const double m = resid ? plan.cres[cb + c] : plan.csum[2 * (cb + c)];
            if (m > 0.0) { last = c; last_base = base; }
            if (base + m > target) { chunk = c; break; }
            base += m;
        }
        if (chunk < 0) { chunk = last; base = last_base; }   // rounding: u Z at the very end
        sh_base = base;
        sh_target = target;
        sh_chunk = chunk;
        sh_resid = resid;
        sh_Sp = Sp;
        sh_Sq = Sq;
    }
    __syncthreads();
    const bool resid = sh_resid;
    const double target = sh_target, Sp = sh_Sp, Sq = sh_Sq;
    const int64_t v0 = sh_chunk * plan.chunk_len, v1 = min(p.V, v0 + plan.chunk_len);

    // Each thread owns a contiguous run of the chunk, in token order.
    const int64_t per = (plan.chunk_len + kThreads - 1) / kThreads;
    const int64_t r0 = min(v1, v0 + threadIdx.x * per), r1 = min(v1, r0 + per);
    auto mass = [&](int64_t v) -> double {
        return resid ? residual_mass(p, t, v, Sp, Sq)
                     : wexp(p.target, p.dtype, t.trow * p.V + v, t.m_t, t.T);
    };
    double local = 0.0;
    int32_t last_pos = -1;
    for (int64_t v = r0; v < r1; ++v) {
        const double m = mass(v);
        local += m;
        if (m > 0.0) last_pos = static_cast<int32_t>(v);
    }
    // Exclusive prefix of the per-thread sums (wave scan + wave totals).
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    double inc = local;
    for (int off = 1; off < 64; off <<= 1) {
        const double y = __shfl_up(inc, off, 64);
        if (lane >= off) inc += y;
    }
    double excl = __shfl_up(inc, 1, 64);
    if (lane == 0) excl = 0.0;
    if (lane == 63) lds[wave] = inc;
    __syncthreads();
    double run = sh_base;
    for (int w = 0; w < wave; ++w) run += lds[w];
    run += excl;
    int32_t pick = INT32_MAX;
    for (int64_t v = r0; v < r1; ++v) {
        run += mass(v);
        if (run > target) { pick = static_cast<int32_t>(v); break; }
    }
    // Lowest crossing token over the workgroup; if rounding left none inside
    // the chunk, the last token of the chunk with positive mass.
    int32_t lp = last_pos;
    for (int off = 32; off > 0; off >>= 1) {
        pick = min(pick, __shfl_xor(pick, off, 64));
        lp = max(lp, __shfl_xor(lp, off, 64));
    }
    __syncthreads();
    if (lane == 0) { lds_i[wave] = pick; lds[wave] = static_cast<double>(lp); }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kWaves; ++w) {
            pick = min(pick, lds_i[w]);
            lp = max(lp, static_cast<int32_t>(lds[w]));
        }
        if (pick == INT32_MAX) pick = lp >= 0 ? lp : static_cast<int32_t>(v0);
        p.out_tokens[t.out_slot] = pick;
    }
}

}  // namespace

hipError_t launch_draw_sums(const Problem& p, const Plan& plan, hipStream_t s) {
    const int64_t blocks = static_cast<int64_t>(p.B) * plan.nchunk;
    draw_sums_kernel<<<dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s>>>(p, plan);
    return hipGetLastError();
}

hipError_t launch_draw_residual(const Problem& p, const Plan& plan, hipStream_t s) {
    const int64_t blocks = static_cast<int64_t>(p.B) * plan.nchunk;
    draw_residual_kernel<<<dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s>>>(p, plan);
    return hipGetLastError();
}

hipError_t launch_draw_pick(const Problem& p, const Plan& plan, hipStream_t s) {
    draw_pick_kernel<<<dim3(static_cast<uint32_t>(p.B)), dim3(kThreads), 0, s>>>(p, plan);
    return hipGetLastError();
}

}  // namespace sv
