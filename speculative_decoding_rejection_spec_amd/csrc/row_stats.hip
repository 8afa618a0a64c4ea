// row_stats.hip -- pass 1 of the verify step: one streaming read of every
// needed logit row.
//
// Both acceptance tests and the bonus draw need the tempered softmax
// p = softmax(z / T) of each target row and q of each draft row (page
// "投机解码", section 动手实践; page "大模型推理无损加速:投机采样...", section 三,
// which softmaxes all gamma target positions at once).  Only two scalars per
// row are needed for that: the maximum m and S = sum_v exp((z_v - m) / T);
// p(x) = exp((z_x - m) / T) / S is then formed for the one drafted token in
// the accept scan.  Greedy rows (T = 0) need only the argmax (lowest token id
// on ties, the greedy branch of the same 动手实践 section).
//
// Work decomposition: the grid is (rows x segments); each 256-thread
// workgroup streams one contiguous segment of one row with 16-byte
// non-temporal loads (8 bf16 or 4 fp32 logits per lane, kUnroll loads in
// flight per lane), keeps an online (max, sum) per lane, and reduces across
// the workgroup in fp64 at the end.  Per element: one unpack, one max, one
// subtract, one multiply, one v_exp_f32, one add.  Splitting rows into
// segments keeps the grid far above the 256 CUs x 8 workgroups the chip can
// hold, so the last wave of workgroups is short.
#include "sv_internal.h"

namespace sv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kUnroll = 4;   // 16-byte loads per lane per batch

__device__ __forceinline__ u32x4 stream_load(const u32x4* p) {
    return __builtin_nontemporal_load(p);
}

// Hardware 2^x (v_exp_f32): 2^-inf = 0.
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int DT> struct Elem;
template <> struct Elem<SV_BF16> {
    using T = uint16_t;
    static constexpr int N = 8;   // logits per 16-byte vector
    __device__ static __forceinline__ void unpack(const u32x4 v, float* x) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = __uint_as_float(v[j] << 16);
            x[2 * j + 1] = __uint_as_float(v[j] & 0xffff0000u);
        }
    }
};
template <> struct Elem<SV_F32> {
    using T = float;
    static constexpr int N = 4;
    __device__ static __forceinline__ void unpack(const u32x4 v, float* x) {
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = __uint_as_float(v[j]);
    }
};

// Online max / sum of exp2((z - m) * c) with c = log2(e) / T, four partial
// sums to shorten the add dependency chains.
struct SoftmaxAcc {
    float m = -INFINITY;
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
    float c;

    template <int N>
    __device__ __forceinline__ void add(const float* x, const int32_t*) {
        float tm = x[0];
#pragma unroll
        for (int j = 1; j < N; ++j) tm = fmaxf(tm, x[j]);
        if (tm > m) {
            const float sc = hw_exp2((m - tm) * c);
            s0 *= sc; s1 *= sc; s2 *= sc; s3 *= sc;
            m = tm;
        }
#pragma unroll
        for (int j = 0; j < N; j += 4) {
            s0 += hw_exp2((x[j] - m) * c);
            if (j + 1 < N) s1 += hw_exp2((x[j + 1] - m) * c);
            if (j + 2 < N) s2 += hw_exp2((x[j + 2] - m) * c);
            if (j + 3 < N) s3 += hw_exp2((x[j + 3] - m) * c);
        }
    }
    __device__ __forceinline__ void add1(float x, int32_t) {
        if (x > m) {
            const float sc = hw_exp2((m - x) * c);
            s0 *= sc; s1 *= sc; s2 *= sc; s3 *= sc;
            m = x;
        }
        s0 += hw_exp2((x - m) * c);
    }
};

// First occurrence of the maximum.  Each lane visits its token ids in
// increasing order, so a strict '>' keeps the lowest id.
struct ArgmaxAcc {
    float m = -INFINITY;
    int32_t a = INT32_MAX;

    template <int N>
    __device__ __forceinline__ void add(const float* x, const int32_t* idx) {
#pragma unroll
        for (int j = 0; j < N; ++j)
            if (x[j] > m) { m = x[j]; a = idx[j]; }
    }
    __device__ __forceinline__ void add1(float x, int32_t i) {
        if (x > m) { m = x; a = i; }
    }
};

// Streams logits [s0, s1) of one row into acc.  Order per lane: the
// unaligned head element, full batches of kUnroll vectors, the remaining
// vectors, the tail element -- increasing token ids throughout.
template <int DT, class Acc>
__device__ __forceinline__ void stream_segment(const void* row_v, int64_t s0, int64_t s1, Acc& acc) {
    using E = typename Elem<DT>::T;
    constexpr int N = Elem<DT>::N;
    const E* row = static_cast<const E*>(row_v);
    const int tid = threadIdx.x;
    const uintptr_t addr = reinterpret_cast<uintptr_t>(row + s0);
    int64_t head = static_cast<int64_t>(((16u - (addr & 15u)) & 15u) / sizeof(E));
    if (head > s1 - s0) head = s1 - s0;
    const int64_t a0 = s0 + head;
    const int64_t nvec = (s1 - a0) / N;
    const int64_t a1 = a0 + nvec * N;

    if (tid < head) acc.add1(load_logit(row_v, DT, s0 + tid), static_cast<int32_t>(s0 + tid));

    const u32x4* vp = reinterpret_cast<const u32x4*>(row + a0);
    constexpr int64_t kPerBatch = static_cast<int64_t>(kThreads) * kUnroll;
    const int64_t nbatch = nvec / kPerBatch;
    for (int64_t bt = 0; bt < nbatch; ++bt) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = stream_load(vp + bt * kPerBatch + u * kThreads + tid);
        float x[kUnroll * N];
        int32_t idx[kUnroll * N];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            Elem<DT>::unpack(v[u], x + u * N);
            const int32_t base = static_cast<int32_t>(a0 + (bt * kPerBatch + u * kThreads + tid) * N);
#pragma unroll
            for (int e = 0; e < N; ++e) idx[u * N + e] = base + e;
        }
        acc.template add<kUnroll * N>(x, idx);
    }
    for (int64_t j = nbatch * kPerBatch + tid; j < nvec; j += kThreads) {
        float x[N];
        int32_t idx[N];
        Elem<DT>::unpack(stream_load(vp + j), x);
        const int32_t base = static_cast<int32_t>(a0 + j * N);
#pragma unroll
        for (int e = 0; e < N; ++e) idx[e] = base + e;
        acc.template add<N>(x, idx);
    }
    if (tid < s1 - a1) acc.add1(load_logit(row_v, DT, a1 + tid), static_cast<int32_t>(a1 + tid));
}

// (m, s) of two partial softmax sums over the same row, in fp64; cd = log2(e)/T.
__device__ __forceinline__ void merge_softmax(float& m, double& s, float m2, double s2, double cd) {
    const float mn = fmaxf(m, m2);
    const double a = (m == -INFINITY) ? 0.0 : s * exp2((static_cast<double>(m) - mn) * cd);
    const double b = (m2 == -INFINITY) ? 0.0 : s2 * exp2((static_cast<double>(m2) - mn) * cd);
    m = mn;
    s = a + b;
}

__device__ __forceinline__ void merge_argmax(float& m, int32_t& a, float m2, int32_t a2) {
    if (m2 > m || (m2 == m && a2 < a)) { m = m2; a = a2; }
}

template <int DT>
__global__ __launch_bounds__(kThreads) void row_stats_kernel(Problem p, Plan plan) {
    const int64_t w = blockIdx.x;
    const int64_t row_all = w / plan.nseg;
    const int64_t seg = w - row_all * plan.nseg;
    const int64_t ntarget = p.total + p.B;
    const bool is_target = row_all < ntarget;
    const int64_t r = is_target ? row_all : row_all - ntarget;
    const int32_t b = is_target ? seq_of_target_row(p, r) : seq_of_draft_row(p, r);
    const float T = p.temperature[b];
    if (!temperature_ok(T)) return;               // reported by the accept scan
    const bool greedy = (T == 0.f);
    if (greedy && !is_target) return;             // greedy never reads draft rows

    using E = typename Elem<DT>::T;
    const E* row = static_cast<const E*>(is_target ? p.target : p.draft) + r * p.V;
    const int64_t s0 = seg * plan.seg_len;
    const int64_t s1 = min(p.V, s0 + plan.seg_len);

    __shared__ float lds_m[kWaves];
    __shared__ double lds_s[kWaves];
    __shared__ int32_t lds_a[kWaves];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    SegStat out;

    if (greedy) {
        ArgmaxAcc acc;
        stream_segment<DT>(row, s0, s1, acc);
        float m = acc.m;
        int32_t a = acc.a;
        for (int off = 32; off > 0; off >>= 1)
            merge_argmax(m, a, __shfl_xor(m, off, 64), __shfl_xor(a, off, 64));
        if (lane == 0) { lds_m[wave] = m; lds_a[wave] = a; }
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int i = 1; i < kWaves; ++i) merge_argmax(m, a, lds_m[i], lds_a[i]);
            out.m = m; out.arg = a; out.s = 0.0;
        }
    } else {
        const double cd = 1.4426950408889634 / static_cast<double>(T);
        SoftmaxAcc acc;
        acc.c = static_cast<float>(fmin(cd, 3.0e38));
        stream_segment<DT>(row, s0, s1, acc);
        float m = acc.m;
        double s = (static_cast<double>(acc.s0) + acc.s1) + (static_cast<double>(acc.s2) + acc.s3);
        for (int off = 32; off > 0; off >>= 1)
            merge_softmax(m, s, __shfl_xor(m, off, 64), __shfl_xor(s, off, 64), cd);
        if (lane == 0) { lds_m[wave] = m; lds_s[wave] = s; }
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int i = 1; i < kWaves; ++i) merge_softmax(m, s, lds_m[i], lds_s[i], cd);
            out.m = m; out.arg = 0; out.s = s;
        }
    }
    if (threadIdx.x == 0) plan.seg[w] = out;
}

}  // namespace

hipError_t launch_row_stats(const Problem& p, const Plan& plan, hipStream_t s) {
    const int64_t blocks = (2 * p.total + p.B) * static_cast<int64_t>(plan.nseg);
    if (blocks == 0) return hipSuccess;
    if (p.dtype == SV_BF16)
        row_stats_kernel<SV_BF16><<<dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s>>>(p, plan);
    else
        row_stats_kernel<SV_F32><<<dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s>>>(p, plan);
    return hipGetLastError();
}

}  // namespace sv
