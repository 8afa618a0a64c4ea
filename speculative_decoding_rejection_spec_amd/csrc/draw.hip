// draw.hip -- the emitted token of every sampling sequence, in fp64.
//
// After the first rejection at position n the token is drawn from
// r = max(0, p_n - q_n) / Z, Z = sum_v max(0, p_n(v) - q_n(v)) (page "投机解码",
// section 无损保证：数学推导, reject-path equation; page
// "大模型推理无损加速:投机采样...", section 二.2); if all k drafts were accepted
// it is drawn from p_k (the bonus token, section 投机解码的三步流程).  The draw
// is an inverse CDF over ascending token ids with the supplied uniform u:
// t* = min{t : C_t > u Z}, C_t = sum_{v <= t} r_v.
//
// Tail tokens of a 10^5-entry distribution carry masses near 1e-10 and sit
// closer together than fp32 rounding, so the CDF is built in fp64 from
// w = exp((z - m) / T) of the exact logits and row maxima.
//
// draw_sums (grid sequence x chunk) reads the draw rows once:
//   * bonus draw: per chunk, W_c = sum of w_t;
//   * residual draw: per chunk, S_p,c = sum w_t and S_q,c = sum w_d (the fp64
//     normalisers), and A_c, B_c = sums of w_t, w_d over the tokens with
//     p_v > q_v.  p_v > q_v iff d_v = (z_t - m_t)/T - (z_d - m_d)/T exceeds
//     theta = ln(S_p / S_q); the accept scan supplies theta from the row
//     pass's normalisers (within about 5e-6), so tokens with
//     |d_v - theta| > kBand are classified exactly, and the few inside the
//     band are listed (per wave, up to kWaveCap each) and get their exact mass
//     once S_p and S_q are known.  The residual mass of chunk c is
//     R_c = A_c / S_p - B_c / S_q + sum over its band tokens of
//     max(0, w_t/S_p - w_d/S_q); a chunk whose lists overflowed is rescanned.
// draw_pick (one workgroup per sequence) forms Z = sum_c R_c, finds the chunk
// whose cumulative mass crosses u Z, and scans that one chunk with a
// workgroup-wide fp64 prefix sum over masses held in registers.  The kernel
// boundary publishes the chunk sums; no device-wide fences are needed.
//
// exp in fp64 follows Tang's table-driven method (ACM TOMS 15(2), 1989):
// y = (64 k + j) ln2/64 + r with |r| <= ln2/128, exp(y) = 2^k 2^(j/64) e^r,
// e^r - 1 by its degree-5 Taylor polynomial (truncation < 4e-17 relative).
#include "sv_internal.h"

namespace sv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr double kDegenerateZ = 1e-9;   // residual mass treated as empty
constexpr double kBand = 2e-5;          // classification band around theta
constexpr int kMaxPickChunks = 1024;    // chunk masses held in LDS by the pick

// 2^(j/64), j = 0..63, correctly rounded.
__constant__ double kExp2Frac[64] = {
    0x1.0000000000000p+0, 0x1.02c9a3e778061p+0, 0x1.059b0d3158574p+0, 0x1.0874518759bc8p+0,
    0x1.0b5586cf9890fp+0, 0x1.0e3ec32d3d1a2p+0, 0x1.11301d0125b51p+0, 0x1.1429aaea92de0p+0,
    0x1.172b83c7d517bp+0, 0x1.1a35beb6fcb75p+0, 0x1.1d4873168b9aap+0, 0x1.2063b88628cd6p+0,
    0x1.2387a6e756238p+0, 0x1.26b4565e27cddp+0, 0x1.29e9df51fdee1p+0, 0x1.2d285a6e4030bp+0,
    0x1.306fe0a31b715p+0, 0x1.33c08b26416ffp+0, 0x1.371a7373aa9cbp+0, 0x1.3a7db34e59ff7p+0,
    0x1.3dea64c123422p+0, 0x1.4160a21f72e2ap+0, 0x1.44e086061892dp+0, 0x1.486a2b5c13cd0p+0,
    0x1.4bfdad5362a27p+0, 0x1.4f9b2769d2ca7p+0, 0x1.5342b569d4f82p+0, 0x1.56f4736b527dap+0,
    0x1.5ab07dd485429p+0, 0x1.5e76f15ad2148p+0, 0x1.6247eb03a5585p+0, 0x1.6623882552225p+0,
    0x1.6a09e667f3bcdp+0, 0x1.6dfb23c651a2fp+0, 0x1.71f75e8ec5f74p+0, 0x1.75feb564267c9p+0,
    0x1.7a11473eb0187p+0, 0x1.7e2f336cf4e62p+0, 0x1.82589994cce13p+0, 0x1.868d99b4492edp+0,
    0x1.8ace5422aa0dbp+0, 0x1.8f1ae99157736p+0, 0x1.93737b0cdc5e5p+0, 0x1.97d829fde4e50p+0,
    0x1.9c49182a3f090p+0, 0x1.a0c667b5de565p+0, 0x1.a5503b23e255dp+0, 0x1.a9e6b5579fdbfp+0,
    0x1.ae89f995ad3adp+0, 0x1.b33a2b84f15fbp+0, 0x1.b7f76f2fb5e47p+0, 0x1.bcc1e904bc1d2p+0,
    0x1.c199bdd85529cp+0, 0x1.c67f12e57d14bp+0, 0x1.cb720dcef9069p+0, 0x1.d072d4a07897cp+0,
    0x1.d5818dcfba487p+0, 0x1.da9e603db3285p+0, 0x1.dfc97337b9b5fp+0, 0x1.e502ee78b3ff6p+0,
    0x1.ea4afa2a490dap+0, 0x1.efa1bee615a27p+0, 0x1.f50765b6e4540p+0, 0x1.fa7c1819e90d8p+0,
};

// exp(y) in fp64 for y <= ~700 (arguments here are <= 0); tbl = kExp2Frac in LDS.
// Rounding y * 64/ln2 to an integer n uses the 1.5 * 2^52 shifter: after the
// add, the low 32 bits of the double hold n in two's complement.
__device__ __forceinline__ double exp_f64(double y, const double* tbl) {
    constexpr double kShift = 0x1.8p52;
    y = fmax(y, -1000.0);                          // exp(-1000) underflows to 0 anyway
    const double kd = fma(y, 0x1.71547652b82fep+6, kShift);    // y * 64 / ln2 + shifter
    const int n = static_cast<int>(static_cast<uint32_t>(__double_as_longlong(kd)));
    const double nd = kd - kShift;
    const double r = fma(-nd, 0x1.a39ef35793c76p-39, fma(-nd, 0x1.62e42fee00000p-7, y));
    double q = fma(r, 1.0 / 120.0, 1.0 / 24.0);
    q = fma(q, r, 1.0 / 6.0);
    q = fma(q, r, 0.5);
    q = fma(q, r, 1.0);
    const double t = tbl[n & 63];
    return ldexp(fma(t, q * r, t), n >> 6);
}

template <int DT> struct Vec;
template <> struct Vec<SV_BF16> {
    using E = uint16_t;
    static constexpr int N = 8;
    __device__ static __forceinline__ void unpack(const u32x4 v, float* x) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = __uint_as_float(v[j] << 16);
            x[2 * j + 1] = __uint_as_float(v[j] & 0xffff0000u);
        }
    }
};
template <> struct Vec<SV_F32> {
    using E = float;
    static constexpr int N = 4;
    __device__ static __forceinline__ void unpack(const u32x4 v, float* x) {
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = __uint_as_float(v[j]);
    }
};

// The one or two rows a draw reads.
template <int DT>
struct Rows {
    using E = typename Vec<DT>::E;
    const E* t;          // target row at position n
    const E* d;          // draft row at position n (residual only)
    double mt, md, invT;
    const double* tbl;

    __device__ __forceinline__ double zt(int64_t v) const { return load_logit(t, DT, v); }
    __device__ __forceinline__ double zd(int64_t v) const { return load_logit(d, DT, v); }
    __device__ __forceinline__ double wt(double z) const { return exp_f64((z - mt) * invT, tbl); }
    __device__ __forceinline__ double wd(double z) const { return exp_f64((z - md) * invT, tbl); }
    // residual mass max(0, w_t/S_p - w_d/S_q) of token v (iSp = 1/S_p, iSq = 1/S_q)
    __device__ __forceinline__ double residual(int64_t v, double iSp, double iSq) const {
        return residual_z(zt(v), zd(v), iSp, iSq);
    }
    __device__ __forceinline__ double residual_z(double z_t, double z_d, double iSp, double iSq) const {
        return fmax(0.0, wt(z_t) * iSp - wd(z_d) * iSq);
    }
};

// Calls f(v, z_t, z_d) for this thread's tokens of [v0, v1): 16-byte vector
// loads (lane-strided vectors) when both rows allow them, scalar otherwise.
template <int DT, bool kResid, class F>
__device__ __forceinline__ void for_chunk(const Rows<DT>& rows, int64_t v0, int64_t v1, F&& f) {
    using E = typename Vec<DT>::E;
    constexpr int N = Vec<DT>::N;
    const bool vec = (reinterpret_cast<uintptr_t>(rows.t + v0) & 15u) == 0 &&
                     (!kResid || (reinterpret_cast<uintptr_t>(rows.d + v0) & 15u) == 0);
    int64_t vs = v0;
    if (vec) {
        const int64_t nvec = (v1 - v0) / N;
        const u32x4* tp = reinterpret_cast<const u32x4*>(rows.t + v0);
        const u32x4* dp = reinterpret_cast<const u32x4*>(rows.d + v0);
        for (int64_t j = threadIdx.x; j < nvec; j += kThreads) {
            const u32x4 a0 = tp[j];
            const u32x4 b0 = kResid ? dp[j] : a0;
            float xt[N], xd[N];
            Vec<DT>::unpack(a0, xt);
            if (kResid) Vec<DT>::unpack(b0, xd);
#pragma unroll 2   // two tokens' fp64 work interleaved: occupancy 6 without spills
            for (int e = 0; e < N; ++e) f(v0 + j * N + e, xt[e], kResid ? xd[e] : 0.f);
        }
        vs = v0 + nvec * N;
    }
    for (int64_t v = vs + threadIdx.x; v < v1; v += kThreads)
        f(v, static_cast<float>(rows.zt(v)), kResid ? static_cast<float>(rows.zd(v)) : 0.f);
}

constexpr int kRun = 16;                      // tokens per lane in the pick's scan
constexpr int64_t kPiece = kThreads * kRun;   // tokens per scan step of the pick

// Sums of four doubles over the workgroup (valid in every thread).
__device__ __forceinline__ void block_sum4(double& a, double& b, double& c, double& d,
                                           double (*lds)[4]) {
    for (int off = 32; off > 0; off >>= 1) {
        a += __shfl_xor(a, off, 64);
        b += __shfl_xor(b, off, 64);
        c += __shfl_xor(c, off, 64);
        d += __shfl_xor(d, off, 64);
    }
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) { lds[wave][0] = a; lds[wave][1] = b; lds[wave][2] = c; lds[wave][3] = d; }
    __syncthreads();
    a = b = c = d = 0.0;
    for (int w = 0; w < kWaves; ++w) { a += lds[w][0]; b += lds[w][1]; c += lds[w][2]; d += lds[w][3]; }
}

// Exclusive prefix sum over the workgroup in thread order; *total = sum.
__device__ __forceinline__ double block_scan_excl(double x, double* total, double* lds) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    double inc = x;
    for (int off = 1; off < 64; off <<= 1) {
        const double y = __shfl_up(inc, off, 64);
        if (lane >= off) inc += y;
    }
    double excl = __shfl_up(inc, 1, 64);
    if (lane == 0) excl = 0.0;
    __syncthreads();
    if (lane == 63) lds[wave] = inc;
    __syncthreads();
    double before = 0.0, all = 0.0;
    for (int w = 0; w < kWaves; ++w) {
        if (w < wave) before += lds[w];
        all += lds[w];
    }
    *total = all;
    return before + excl;
}

__device__ __forceinline__ int32_t block_min_max(int32_t x, bool want_min, int32_t* lds) {
    for (int off = 32; off > 0; off >>= 1) {
        const int32_t y = __shfl_xor(x, off, 64);
        x = want_min ? min(x, y) : max(x, y);
    }
    __syncthreads();
    if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = x;
    __syncthreads();
    int32_t r = lds[0];
    for (int w = 1; w < kWaves; ++w) r = want_min ? min(r, lds[w]) : max(r, lds[w]);
    return r;
}

template <int DT>
__device__ __forceinline__ Rows<DT> rows_of(const Problem& p, const DrawTask& task, const double* tbl) {
    using E = typename Vec<DT>::E;
    return Rows<DT>{static_cast<const E*>(p.target) + task.trow * p.V,
                    static_cast<const E*>(p.draft) + task.drow * p.V,
                    task.m_t, task.m_d, 1.0 / static_cast<double>(task.T), tbl};
}

// Chunk pass: grid (sequence x chunk).
template <int DT>
__global__ __launch_bounds__(kThreads) void draw_sums_kernel(Problem p, Plan plan) {
    const int64_t w = blockIdx.x;
    const int32_t b = static_cast<int32_t>(w / plan.nchunk);
    const int32_t c = static_cast<int32_t>(w - static_cast<int64_t>(b) * plan.nchunk);
    const DrawTask task = plan.task[b];
    if (task.kind == kNone) return;
    const bool resid_task = (task.kind == kResidual);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

    __shared__ double tbl[64];
    __shared__ double lds4[kWaves][4];
    __shared__ int32_t wlist[kWaves][kWaveCap];
    __shared__ int32_t wcount[kWaves];
    if (threadIdx.x < 64) tbl[threadIdx.x] = kExp2Frac[threadIdx.x];
    __syncthreads();
    const Rows<DT> rows = rows_of<DT>(p, task, tbl);

    const int64_t v0 = static_cast<int64_t>(c) * plan.chunk_len;
    const int64_t v1 = min(p.V, v0 + plan.chunk_len);
    double sp = 0.0, sq = 0.0, a = 0.0, bq = 0.0;
    int32_t nband = 0;                         // uniform over the lanes still active
    if (resid_task) {
        const double th_hi = task.theta + kBand, th_lo = task.theta - kBand;
        for_chunk<DT, true>(rows, v0, v1, [&](int64_t v, float zt, float zd) {
            const double yt = (static_cast<double>(zt) - rows.mt) * rows.invT;
            const double yd = (static_cast<double>(zd) - rows.md) * rows.invT;
            const double wt = exp_f64(yt, tbl), wd = exp_f64(yd, tbl);
            sp += wt;
            sq += wd;
            const double dv = yt - yd;
            const bool hi = dv > th_hi;
            a += hi ? wt : 0.0;
            bq += hi ? wd : 0.0;
            const bool in_band = !hi && dv >= th_lo;
            const uint64_t m = __ballot(in_band);
            if (m) {
                const int pos = nband + __popcll(m & ((1ull << lane) - 1ull));
                if (in_band && pos < kWaveCap) wlist[wave][pos] = static_cast<int32_t>(v);
                nband += __popcll(m);
            }
        });
    } else {
        for_chunk<DT, false>(rows, v0, v1, [&](int64_t, float zt, float) { sp += rows.wt(zt); });
    }
    if (lane == 0) wcount[wave] = nband;      // lane 0 was active whenever any lane was
    block_sum4(sp, sq, a, bq, lds4);
    if (threadIdx.x == 0) {
        ChunkSums cs;
        cs.sp = sp; cs.sq = sq; cs.a = a; cs.b = bq;
        plan.csum[w] = cs;
    }
    if (resid_task) {
        int32_t* band = plan.band + w * kBandSlots;
        if (threadIdx.x < kWaves) band[threadIdx.x] = wcount[threadIdx.x];
        if (threadIdx.x < kWaves * kWaveCap) {
            const int wv = threadIdx.x / kWaveCap, e = threadIdx.x % kWaveCap;
            if (e < wcount[wv]) band[kWaves + threadIdx.x] = wlist[wv][e];
        }
    }
}

// Pick: one workgroup per sequence.
template <int DT>
__global__ __launch_bounds__(kThreads) void draw_pick_kernel(Problem p, Plan plan) {
    constexpr int N = Vec<DT>::N;
    const int32_t b = blockIdx.x;
    const DrawTask task = plan.task[b];
    if (task.kind == kNone) return;
    const bool resid_task = (task.kind == kResidual);

    __shared__ double tbl[64];
    __shared__ double lds4[kWaves][4];
    __shared__ double lds[kWaves];
    __shared__ int32_t ldsi[kWaves];
    __shared__ double mass[kMaxPickChunks];
    __shared__ double sh_base, sh_target;
    __shared__ int32_t sh_chunk, sh_resid, sh_rescan;
    if (threadIdx.x < 64) tbl[threadIdx.x] = kExp2Frac[threadIdx.x];
    if (threadIdx.x == 0) sh_rescan = 0;
    __syncthreads();
    const Rows<DT> rows = rows_of<DT>(p, task, tbl);
    const ChunkSums* cs = plan.csum + static_cast<int64_t>(b) * plan.nchunk;
    const int32_t* bands = plan.band + static_cast<int64_t>(b) * plan.nchunk * kBandSlots;
    const int32_t nchunk = plan.nchunk;

    double Sp = 0.0, Sq = 0.0, unused0 = 0.0, unused1 = 0.0;
    for (int32_t j = threadIdx.x; j < nchunk; j += kThreads) {
        Sp += cs[j].sp;
        Sq += cs[j].sq;
    }
    block_sum4(Sp, Sq, unused0, unused1, lds4);
    const double iSp = 1.0 / Sp, iSq = resid_task ? 1.0 / Sq : 0.0;

    if (resid_task) {
        // per-chunk residual mass: robust part plus band tokens (list order)
        for (int32_t j = threadIdx.x; j < nchunk; j += kThreads) {
            const int32_t* bj = bands + static_cast<int64_t>(j) * kBandSlots;
            double m = cs[j].a * iSp - cs[j].b * iSq;
            bool over = false;
            for (int wv = 0; wv < kWaves; ++wv) {
                const int32_t cnt = bj[wv];
                over |= cnt > kWaveCap;
                for (int32_t e = 0; e < cnt && e < kWaveCap; ++e)
                    m += rows.residual(bj[kWaves + wv * kWaveCap + e], iSp, iSq);
            }
            mass[j] = over ? NAN : m;
            if (over) atomicOr(&sh_rescan, 1);
        }
        __syncthreads();
        if (sh_rescan) {
            // chunks whose band lists overflowed: exact rescan (rare)
            for (int32_t j = 0; j < nchunk; ++j) {
                if (!isnan(mass[j])) continue;
                const int64_t u0 = static_cast<int64_t>(j) * plan.chunk_len;
                const int64_t u1 = min(p.V, u0 + plan.chunk_len);
                double m = 0.0;
                for (int64_t v = u0 + threadIdx.x; v < u1; v += kThreads) m += rows.residual(v, iSp, iSq);
                m = block_sum(m, lds);
                if (threadIdx.x == 0) mass[j] = m;
                __syncthreads();
            }
        }
    }
    if (threadIdx.x == 0) {
        bool resid = resid_task;
        double Z = 0.0;
        if (resid) {
            for (int32_t j = 0; j < nchunk; ++j) Z += mass[j];
            if (Z < kDegenerateZ) resid = false;       // draw from p_n instead
        }
        if (!resid) {
            Z = 0.0;
            for (int32_t j = 0; j < nchunk; ++j) { mass[j] = cs[j].sp; Z += mass[j]; }
        }
        const double target = static_cast<double>(task.u) * Z;
        double base = 0.0, last_base = 0.0;
        int32_t chunk = -1, last = 0;
        for (int32_t j = 0; j < nchunk; ++j) {
            if (mass[j] > 0.0) { last = j; last_base = base; }
            if (base + mass[j] > target) { chunk = j; break; }
            base += mass[j];
        }
        if (chunk < 0) { chunk = last; base = last_base; }   // rounding: u Z at the very end
        sh_base = base;
        sh_target = target;
        sh_chunk = chunk;
        sh_resid = resid;
    }
    __syncthreads();
    const bool resid = sh_resid;
    const double target = sh_target;
    double base = sh_base;
    const int64_t c0 = static_cast<int64_t>(sh_chunk) * plan.chunk_len;
    const int64_t c1 = min(p.V, c0 + plan.chunk_len);

    // Scan the chunk in pieces of kPiece tokens: lane tid owns kRun consecutive
    // tokens of the piece, loaded together, masses kept in registers.
    int32_t pick = INT32_MAX, last_pos = -1;
    for (int64_t q0 = c0; q0 < c1 && pick == INT32_MAX; q0 += kPiece) {
        const int64_t q1 = min(c1, q0 + kPiece);
        const int64_t r0 = q0 + static_cast<int64_t>(threadIdx.x) * kRun;
        float zt[kRun], zd[kRun];
        const bool vec = r0 + kRun <= q1 &&
                         (reinterpret_cast<uintptr_t>(rows.t + r0) & 15u) == 0 &&
                         (!resid || (reinterpret_cast<uintptr_t>(rows.d + r0) & 15u) == 0);
        if (vec) {
#pragma unroll
            for (int i = 0; i < kRun / N; ++i) {
                Vec<DT>::unpack(reinterpret_cast<const u32x4*>(rows.t + r0)[i], zt + i * N);
                if (resid) Vec<DT>::unpack(reinterpret_cast<const u32x4*>(rows.d + r0)[i], zd + i * N);
            }
        } else {
#pragma unroll
            for (int i = 0; i < kRun; ++i) {
                const bool in = r0 + i < q1;
                zt[i] = in ? static_cast<float>(rows.zt(r0 + i)) : 0.f;
                zd[i] = (in && resid) ? static_cast<float>(rows.zd(r0 + i)) : 0.f;
            }
        }
        double m[kRun];
        double local = 0.0;
        int32_t lp = -1;
#pragma unroll
        for (int i = 0; i < kRun; ++i) {
            const bool in = r0 + i < q1;
            m[i] = !in ? 0.0 : (resid ? rows.residual_z(zt[i], zd[i], iSp, iSq) : rows.wt(zt[i]));
            local += m[i];
            if (m[i] > 0.0) lp = static_cast<int32_t>(r0 + i);
        }
        double total;
        double run = base + block_scan_excl(local, &total, lds);
        int32_t mine = INT32_MAX;
#pragma unroll
        for (int i = 0; i < kRun; ++i) {
            run += m[i];
            if (mine == INT32_MAX && run > target) mine = static_cast<int32_t>(r0 + i);
        }
        pick = block_min_max(mine, true, ldsi);
        last_pos = max(last_pos, block_min_max(lp, false, ldsi));
        base += total;
    }
    // If rounding left no crossing inside the chunk: its last token with mass.
    if (threadIdx.x == 0) {
        if (pick == INT32_MAX) pick = last_pos >= 0 ? last_pos : static_cast<int32_t>(c0);
        p.out_tokens[task.out_slot] = pick;
    }
}

}  // namespace

hipError_t launch_draw_sums(const Problem& p, const Plan& plan, hipStream_t s) {
    const int64_t blocks = static_cast<int64_t>(p.B) * plan.nchunk;
    if (p.dtype == SV_BF16)
        draw_sums_kernel<SV_BF16><<<dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s>>>(p, plan);
    else
        draw_sums_kernel<SV_F32><<<dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s>>>(p, plan);
    return hipGetLastError();
}

hipError_t launch_draw_pick(const Problem& p, const Plan& plan, hipStream_t s) {
    if (p.dtype == SV_BF16)
        draw_pick_kernel<SV_BF16><<<dim3(static_cast<uint32_t>(p.B)), dim3(kThreads), 0, s>>>(p, plan);
    else
        draw_pick_kernel<SV_F32><<<dim3(static_cast<uint32_t>(p.B)), dim3(kThreads), 0, s>>>(p, plan);
    return hipGetLastError();
}

}  // namespace sv
