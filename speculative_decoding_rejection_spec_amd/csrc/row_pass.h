// row_pass.h -- the streaming read of one segment of one logit row (pass 1 of
// the verify step), shared by the row-pass kernels and the second round.
//
// The accept tests and the bonus draw need the tempered softmax
// p = softmax(z / T) of each target row and q of each draft row (page
// "投机解码", section 动手实践; page "大模型推理无损加速:投机采样...", section 三,
// which softmaxes all gamma target positions at once).  Two scalars per row
// suffice: the maximum m and S = sum_v exp((z_v - m) / T); p(x) for the one
// drafted token is formed later in the accept scan.  Greedy rows (T = 0)
// need only the argmax, lowest token id on ties (greedy branch of the same
// 动手实践 section).
//
// A 256-thread workgroup streams one contiguous segment.  Each lane owns
// every 256th 16-byte vector of the segment (8 bf16 or 4 fp32 logits) and
// keeps a rolling window of non-temporal loads in flight (8 for bf16, 4 for
// fp32): the load that replaces a vector is issued before that vector is
// processed, so memory requests stay outstanding while the lane computes.
//
// Per logit: one unpack (shift or mask), half a v_max3, one v_fma
// (z * c - R), one v_exp_f32, one add.  The running sum is kept relative to
// an integer-valued reference R (c = log2(e) / T), so rescaling when the
// maximum grows is an exact v_ldexp; the workgroup-wide merge is in fp64,
// also by exact powers of two.  R starts at ceil(m0 * c) for the largest
// logit m0 of the wave's first tile and is raised to ceil(m * c) only when
// a logit m exceeds it by more than kSlack (in log2 units): with every lane
// raising at its own new maxima, some lane of a wave raised on nearly every
// tile; seeded from the wave and given that slack, a raise is rare, and the
// exponent argument z * c - R stays below kSlack + 1, where its fp32
// rounding (at most 2^-23) adds under 1e-7 relative to a term.
#pragma once

#include "sv_internal.h"

namespace sv {
namespace rowpass {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Word 3 of a raw buffer descriptor on gfx9-family GPUs (32-bit data format,
// no swizzle, range checked against num_records).
constexpr int kBufferDword3 = 0x00020000;
// Cache policy of the streaming loads: non-temporal.
constexpr int kLoadNonTemporal = 2;

// Hardware 2^x (v_exp_f32): 2^-inf = 0.
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int DT> struct Elem;
template <> struct Elem<SV_BF16> {
    using T = uint16_t;
    static constexpr int N = 8;        // logits per 16-byte vector
    static constexpr int kWindow = 8;  // 16-byte loads in flight per lane
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
    static constexpr int kWindow = 4;  // (8 more than doubles the register footprint here)
    __device__ static __forceinline__ void unpack(const u32x4 v, float* x) {
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = __uint_as_float(v[j]);
    }
};

template <int N>
__device__ __forceinline__ float max_of(const float* x) {
    float t = x[0];
#pragma unroll
    for (int j = 1; j < N; ++j) t = fmaxf(t, x[j]);
    return t;
}

// Online sum of 2^(z*c - R) with an integer-valued reference R >= m*c - kSlack
// for the running maximum m, in 4 fp32 partial sums: sum j takes logit j of
// each vector (fp32, 4 per vector) or the pair j, j + 4 added first (bf16, 8
// per vector), and a head or tail element goes to sum 3.  With at most
// max_seg_elems(dtype) logits per segment a sum is built from at most 40
// vectors' terms and 2 single ones, so its rounding stays below 42 * 2^-24
// relative.
constexpr int kSums = 4;
struct SoftmaxAcc {
    static constexpr float kSlack = 2.f;
    float m = -INFINITY;    // running maximum logit
    float R = -INFINITY;    // reference exponent (integer valued)
    float nR = 0.f;         // -R, or 0 while R = -inf (every logit so far -inf: its terms are then 0)
    float thr = -INFINITY;  // R + kSlack: a logit z with z * c above it raises R
    float s[kSums] = {};
    float c;

    __device__ __forceinline__ void set_ref(float Rn) {
        R = Rn;
        nR = -Rn;
        thr = Rn + kSlack;
    }
    // The first reference, from the largest logit of the wave's first tile
    // (-inf: none; the first finite logit seen sets it).  Called before any add.
    __device__ __forceinline__ void prime(float wm) {
        if (wm > -INFINITY) set_ref(ceilf(wm * c));
    }
    __device__ __forceinline__ void raise(float tm) {
        const float Rn = ceilf(tm * c);
        // exact rescale by 2^(R - Rn); R = -inf only while the sums are 0
        const int d = static_cast<int>(fmaxf(R - Rn, -512.f));
#pragma unroll
        for (int j = 0; j < kSums; ++j) s[j] = ldexpf(s[j], d);
        set_ref(Rn);
    }
    // The vector's logits are folded into the running maximum one by one
    // (v_max3, with no canonicalising moves: the chain starts from a
    // maximum), and since m * c <= thr holds after every add, testing the
    // new maximum tests the vector's.
    template <int N>
    __device__ __forceinline__ void add(const float* x, int32_t) {
        static_assert(N == kSums || N == 2 * kSums, "partial sums per vector");
        float mm = m;
#pragma unroll
        for (int j = 0; j < N; ++j) mm = fmaxf(mm, x[j]);
        m = mm;
        if (mm * c > thr) raise(mm);
#pragma unroll
        for (int j = 0; j < kSums; ++j) {
            if constexpr (N == 2 * kSums)
                s[j] += hw_exp2(fmaf(x[j], c, nR)) + hw_exp2(fmaf(x[j + kSums], c, nR));
            else
                s[j] += hw_exp2(fmaf(x[j], c, nR));
        }
    }
    // A single logit (a segment's unaligned head or tail): its own sum.
    __device__ __forceinline__ void add1(float x, int32_t) {
        m = fmaxf(m, x);
        if (m * c > thr) raise(m);
        s[kSums - 1] += hw_exp2(fmaf(x, c, nR));
    }
    __device__ __forceinline__ double total() const {
        double t = 0.0;
#pragma unroll
        for (int j = 0; j < kSums; ++j) t += static_cast<double>(s[j]);
        return t;
    }
};

// First occurrence of the maximum.  Each lane visits its token ids in
// increasing order, so a strict '>' keeps the lowest id.
struct ArgmaxAcc {
    float m = -INFINITY;
    int32_t a = INT32_MAX;

    __device__ __forceinline__ void prime(float) {}

    template <int N>
    __device__ __forceinline__ void add(const float* x, int32_t base) {
        const float tm = max_of<N>(x);
        if (tm > m) {
            int32_t j = 0;
#pragma unroll
            for (int e = N - 1; e >= 0; --e)
                if (x[e] == tm) j = e;
            m = tm;
            a = base + j;
        }
    }
    __device__ __forceinline__ void add1(float x, int32_t i) {
        if (x > m) { m = x; a = i; }
    }
};

// Streams logits [s0, s1) of one row into acc.  Order per lane: the
// unaligned head element, its vectors in increasing order, the tail element
// -- increasing token ids throughout.
//
// The aligned body is read with raw buffer loads against a descriptor that
// spans exactly its nvec vectors: a load past the end returns zeros and
// touches no memory.  Every load is therefore issued on every path, with no
// branch around it and no clamped re-read, and since the hardware counts
// outstanding loads in issue order the compiler can wait for exactly the
// oldest one instead of draining the window.
template <int DT, int kWindow, class Acc>
__device__ __forceinline__ void stream_segment(const void* row_v, int64_t s0, int64_t s1, Acc& acc) {
    using E = typename Elem<DT>::T;
    constexpr int N = Elem<DT>::N;
    constexpr int32_t kTileBytes = kThreads * 16;
    const E* row = static_cast<const E*>(row_v);
    const int tid = threadIdx.x;
    const uintptr_t addr = reinterpret_cast<uintptr_t>(row + s0);
    int64_t head = static_cast<int64_t>(((16u - (addr & 15u)) & 15u) / sizeof(E));
    if (head > s1 - s0) head = s1 - s0;
    const int64_t a0 = s0 + head;
    const int32_t nvec = static_cast<int32_t>((s1 - a0) / N);
    const int64_t a1 = a0 + static_cast<int64_t>(nvec) * N;
    const int64_t ntail = s1 - a1;

    const int32_t nfull = nvec / kThreads;                       // full tiles
    const int32_t nt = (nvec + kThreads - 1) / kThreads;         // plus the partial one
    const int32_t rem = nvec - nfull * kThreads;                 // its lanes: tid < rem
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<E*>(row + a0), 0, nvec * 16, kBufferDword3);
    const int32_t voff = tid * 16;
    auto load_tile = [&](int32_t t) {
        return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, t * kTileBytes,
                                                                               kLoadNonTemporal));
    };
    const int32_t base0 = static_cast<int32_t>(a0) + tid * N;
    auto process = [&](const u32x4 v, int32_t t) {
        float x[N];
        Elem<DT>::unpack(v, x);
        acc.template add<N>(x, base0 + t * kThreads * N);
    };
    auto process_last = [&](const u32x4 v, int32_t t) {
        if (t < nfull || tid < rem) process(v, t);
    };

    // Head and tail elements (clamped into the segment; used only by the
    // lanes that own one), then the first window of tiles.  The scheduling
    // barriers keep this issue order: the loop waits on slot 0 being oldest.
    const int64_t hi = s0 + min(static_cast<int64_t>(tid), s1 - s0 - 1);
    const int64_t ti = ntail > 0 ? a1 + min(static_cast<int64_t>(tid), ntail - 1) : hi;
    const float hv = load_logit(row_v, DT, hi);
    const float tv = load_logit(row_v, DT, ti);
    __builtin_amdgcn_sched_barrier(0);
    u32x4 buf[kWindow];
#pragma unroll
    for (int u = 0; u < kWindow; ++u) {
        buf[u] = load_tile(u);
        __builtin_amdgcn_sched_barrier(0);
    }
    {
        // The wave's largest logit in its first tile (and head elements)
        // seeds the accumulator's reference.
        float x[N];
        Elem<DT>::unpack(buf[0], x);
        float lm = (0 < nfull || tid < rem) ? max_of<N>(x) : -INFINITY;
        if (tid < head) lm = fmaxf(lm, hv);
        for (int off = 32; off > 0; off >>= 1) lm = fmaxf(lm, __shfl_xor(lm, off, 64));
        acc.prime(lm);
    }
    if (tid < head) acc.add1(hv, static_cast<int32_t>(hi));

    // Steady state: tiles i .. i+W-1 are full (i + 2W <= nt <= nfull + 1).
    int32_t i = 0;
    for (; i + 2 * kWindow <= nt; i += kWindow) {
#pragma unroll
        for (int u = 0; u < kWindow; ++u) {
            process(buf[u], i + u);
            buf[u] = load_tile(i + kWindow + u);
        }
    }
    // Drain: fewer than 2W tiles remain; loads past the end are free.
#pragma unroll
    for (int u = 0; u < kWindow; ++u) {
        if (i + u < nt) process_last(buf[u], i + u);
        buf[u] = load_tile(i + kWindow + u);
    }
#pragma unroll
    for (int u = 0; u < kWindow; ++u)
        if (i + kWindow + u < nt) process_last(buf[u], i + kWindow + u);
    if (tid < ntail) acc.add1(tv, static_cast<int32_t>(ti));
}

// Two partial sums s * 2^R of the same row, merged exactly in fp64.
__device__ __forceinline__ void merge_softmax(float& m, float& R, double& s, float m2, float R2, double s2) {
    m = fmaxf(m, m2);
    if (R2 == -INFINITY) return;
    if (R == -INFINITY) { R = R2; s = s2; return; }
    const float Rn = fmaxf(R, R2);
    s = ldexp(s, static_cast<int>(fmaxf(R - Rn, -2048.f))) +
        ldexp(s2, static_cast<int>(fmaxf(R2 - Rn, -2048.f)));
    R = Rn;
}

__device__ __forceinline__ void merge_argmax(float& m, int32_t& a, float m2, int32_t a2) {
    if (m2 > m || (m2 == m && a2 < a)) { m = m2; a = a2; }
}

}  // namespace rowpass

// Workgroup scratch of one row segment.
struct RowLds {
    float m[kWaves], R[kWaves];
    double s[kWaves];
    int32_t a[kWaves];
};

// Pass 1 over segment `seg` of one logit row of sequence b: target row r
// (is_target) or draft row r.  Writes the segment's SegStat and, from the
// workgroup whose segment holds the row's drafted token, that token's logit.
// The row index must lie inside its array.  Rows that are never needed
// (sequences with an unusable temperature, draft rows of greedy sequences)
// are skipped.  kCo selects stores that other workgroups of the same launch
// may read (see st_co).  kWindow: 16-byte loads in flight per lane (0: the
// dtype's default, sized for full occupancy).  x_hint: the drafted token of
// this row (-1: none), when the caller knows it, else kXFromOffsets.  rec
// (first round, see LeadRec): also written, whether or not the row is read.
constexpr int32_t kXFromOffsets = -2;   // row_segment's x_hint: look the drafted token up

template <int DT, bool kCo, int kWindowArg = 0>
__device__ __forceinline__ void row_segment(const Problem& p, const Plan& plan, int32_t b, bool is_target,
                                            int64_t r, int64_t seg, RowLds& lds,
                                            int32_t x_hint = kXFromOffsets, LeadRec* rec = nullptr) {
    using namespace rowpass;
    constexpr int kWindow = kWindowArg > 0 ? kWindowArg : Elem<DT>::kWindow;
    const float T = p.temperature[b];
    const bool greedy = (T == 0.f);
    // (a bad temperature is reported by the accept scan; greedy never reads
    // draft rows)
    if (!temperature_ok(T) || (greedy && !is_target)) {
        if (rec && threadIdx.x == 0) store_lead_rec(rec, plan.epoch, 0, 0.0, 0.f);
        return;
    }

    using E = typename Elem<DT>::T;
    const int64_t ntarget = p.total + p.B;
    const int64_t w = (is_target ? r : ntarget + r) * plan.nseg + seg;
    const E* row = static_cast<const E*>(is_target ? p.target : p.draft) + r * p.V;
    const int64_t s0 = seg * plan.seg_len;
    const int64_t s1 = min(p.V, s0 + plan.seg_len);

    // The workgroup whose segment holds this row's drafted token records that
    // token's logit for the accept scan.  Every workgroup issues the (uniform)
    // load, at s0 when it captures nothing, so no load sits under a branch.
    bool capture = false;
    int64_t xc = s0;
    if (!greedy && x_hint != kXFromOffsets) {
        capture = x_hint >= s0 && x_hint < s1;
        if (capture) xc = x_hint;
    } else if (!greedy) {
        const int64_t o = p.offsets ? static_cast<int64_t>(p.offsets[b]) : static_cast<int64_t>(b) * p.k_uniform;
        const int64_t k = p.offsets ? static_cast<int64_t>(p.offsets[b + 1]) - o : p.k_uniform;
        const int64_t i = is_target ? r - o - b : r - o;
        if (i >= 0 && i < k && o >= 0 && o + i < p.total) {
            const int32_t x = p.tokens[o + i];
            capture = x >= s0 && x < s1;
            if (capture) xc = x;
        }
    }
    const float zx = load_logit(row, DT, xc);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (greedy) {
        ArgmaxAcc acc;
        stream_segment<DT, kWindow>(row, s0, s1, acc);
        float m = acc.m;
        int32_t a = acc.a;
        for (int off = 32; off > 0; off >>= 1)
            merge_argmax(m, a, __shfl_xor(m, off, 64), __shfl_xor(a, off, 64));
        if (lane == 0) { lds.m[wave] = m; lds.a[wave] = a; }
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int i = 1; i < kWaves; ++i) merge_argmax(m, a, lds.m[i], lds.a[i]);
            st_co<kCo>(&plan.seg[w].head, seg_head(m, static_cast<uint32_t>(a)));
            st_co<kCo>(&plan.seg[w].s, 0.0);
            if (rec) store_lead_rec(rec, plan.epoch, seg_head(m, static_cast<uint32_t>(a)), 0.0, 0.f);
        }
    } else {
        SoftmaxAcc acc;
        acc.c = row_scale(T);
        stream_segment<DT, kWindow>(row, s0, s1, acc);
        float m = acc.m, R = acc.R;
        double s = acc.total();
        for (int off = 32; off > 0; off >>= 1)
            merge_softmax(m, R, s, __shfl_xor(m, off, 64), __shfl_xor(R, off, 64),
                          __shfl_xor(s, off, 64));
        if (lane == 0) { lds.m[wave] = m; lds.R[wave] = R; lds.s[wave] = s; }
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int i = 1; i < kWaves; ++i) merge_softmax(m, R, s, lds.m[i], lds.R[i], lds.s[i]);
            st_co<kCo>(&plan.seg[w].head, seg_head(m, __float_as_uint(R)));
            st_co<kCo>(&plan.seg[w].s, s);
            if (capture) st_co<kCo>(&plan.xlogit[is_target ? r : ntarget + r], zx);
            if (rec) store_lead_rec(rec, plan.epoch, seg_head(m, __float_as_uint(R)), s, capture ? zx : 0.f);
        }
    }
}

}  // namespace sv
