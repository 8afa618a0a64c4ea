// draw_pass.h -- the emitted token of every sampling sequence, in fp64;
// shared by the staged draw kernels, the second round and the one-launch draw.
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
// w = 2^((z - m) log2(e) / T) of the exact logits and row maxima.
//
// draw_chunk (one workgroup per (sequence, chunk)) reads the draw rows once;
// wave w of it covers sub-chunk w, a contiguous quarter of the chunk, and
// keeps its sums on its own:
//   * bonus draw: per sub-chunk, W_s = sum of w_t;
//   * residual draw: per sub-chunk, S_p,s = sum w_t and S_q,s = sum w_d (the
//     fp64 normalisers), and A_s, B_s = sums of w_t, w_d over the tokens with
//     p_v > q_v.  p_v > q_v iff d_v = log2(w_t / w_d) exceeds
//     theta = log2(S_p / S_q); the accept scan supplies theta from the row
//     pass's normalisers (within about 1e-5 in log2 units), so tokens with
//     |d_v - theta| > kBand are classified exactly, and the few inside the
//     band are listed per sub-chunk (up to kWaveCap) with their (w_t, w_d),
//     to get their exact mass once S_p and S_q are known.  The residual mass
//     of sub-chunk s is R_s = A_s / S_p - B_s / S_q + sum over its band
//     tokens of max(0, w_t/S_p - w_d/S_q); a sub-chunk whose list overflowed
//     is rescanned.
// pick_sequence (one workgroup per sequence) forms Z = sum_s R_s, finds the
// sub-chunk whose cumulative mass crosses u Z with a wave-wide scan, and
// scans that one sub-chunk with a workgroup-wide fp64 prefix sum over masses
// held in registers.
//
// 2^y in fp64 follows Tang's table-driven method (ACM TOMS 15(2), 1989) in
// base 2 with a 256-entry table: y = k + j/256 + r with |r| <= 1/512,
// 2^y = 2^k 2^(j/256) e^(r ln2), e^(r ln2) - 1 by its degree-4 Taylor
// polynomial (truncation < 4e-17 relative).  The kernels carry Y = 256 y.
// The scaling by 2^k is folded into the table: each entry keeps the high
// word of 2^(j/256) minus j << 12, so adding round(Y) << 12 to it adds k to
// the exponent field in one integer add.
#pragma once

#include "accept_scan.h"

namespace sv {
namespace drawpass {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr double kLog2e = 0x1.71547652b82fep+0;
constexpr double kDegenerateZ = 1e-9;            // residual mass treated as empty
constexpr double kBand = 3e-5;                   // classification band (log2 units)
// Lower clamp of Y.  At exactly -1023 * 256 the table trick below yields +0.0
// (high word 0x3ff00000 - (1023 << 20) = 0, low word 0, r = 0), so a masked
// logit (z = -inf, Y = -inf) and any weight below 2^-1023 get exactly zero
// mass; Y in (-1023, -1022) * 256 gives a value below 2^-1022 (no weight
// that small can move a fp64 sum that holds the reference's weight 1).
constexpr double kMinY = -1023.0 * 256.0;
constexpr int kSlots = kWaves * kWaveCap;        // band entries per chunk (32)
constexpr int kBufferDword3 = 0x00020000;        // raw buffer descriptor word 3 (gfx9 family)

// 2^(j/256), j = 0..255, correctly rounded.
static __constant__ double kExp2Frac[256] = {
    0x1.0000000000000p+0, 0x1.00b1afa5abcbfp+0, 0x1.0163da9fb3335p+0, 0x1.02168143b0281p+0,
    0x1.02c9a3e778061p+0, 0x1.037d42e11bbccp+0, 0x1.04315e86e7f85p+0, 0x1.04e5f72f654b1p+0,
    0x1.059b0d3158574p+0, 0x1.0650a0e3c1f89p+0, 0x1.0706b29ddf6dep+0, 0x1.07bd42b72a836p+0,
    0x1.0874518759bc8p+0, 0x1.092bdf66607e0p+0, 0x1.09e3ecac6f383p+0, 0x1.0a9c79b1f3919p+0,
    0x1.0b5586cf9890fp+0, 0x1.0c0f145e46c85p+0, 0x1.0cc922b7247f7p+0, 0x1.0d83b23395decp+0,
    0x1.0e3ec32d3d1a2p+0, 0x1.0efa55fdfa9c5p+0, 0x1.0fb66affed31bp+0, 0x1.1073028d7233ep+0,
    0x1.11301d0125b51p+0, 0x1.11edbab5e2ab6p+0, 0x1.12abdc06c31ccp+0, 0x1.136a814f204abp+0,
    0x1.1429aaea92de0p+0, 0x1.14e95934f312ep+0, 0x1.15a98c8a58e51p+0, 0x1.166a45471c3c2p+0,
    0x1.172b83c7d517bp+0, 0x1.17ed48695bbc0p+0, 0x1.18af9388c8deap+0, 0x1.1972658375d2fp+0,
    0x1.1a35beb6fcb75p+0, 0x1.1af99f8138a1cp+0, 0x1.1bbe084045cd4p+0, 0x1.1c82f95281c6bp+0,
    0x1.1d4873168b9aap+0, 0x1.1e0e75eb44027p+0, 0x1.1ed5022fcd91dp+0, 0x1.1f9c18438ce4dp+0,
    0x1.2063b88628cd6p+0, 0x1.212be3578a819p+0, 0x1.21f49917ddc96p+0, 0x1.22bdda27912d1p+0,
    0x1.2387a6e756238p+0, 0x1.2451ffb82140ap+0, 0x1.251ce4fb2a63fp+0, 0x1.25e85711ece75p+0,
    0x1.26b4565e27cddp+0, 0x1.2780e341ddf29p+0, 0x1.284dfe1f56381p+0, 0x1.291ba7591bb70p+0,
    0x1.29e9df51fdee1p+0, 0x1.2ab8a66d10f13p+0, 0x1.2b87fd0dad990p+0, 0x1.2c57e39771b2fp+0,
    0x1.2d285a6e4030bp+0, 0x1.2df961f641589p+0, 0x1.2ecafa93e2f56p+0, 0x1.2f9d24abd886bp+0,
    0x1.306fe0a31b715p+0, 0x1.31432edeeb2fdp+0, 0x1.32170fc4cd831p+0, 0x1.32eb83ba8ea32p+0,
    0x1.33c08b26416ffp+0, 0x1.3496266e3fa2dp+0, 0x1.356c55f929ff1p+0, 0x1.36431a2de883bp+0,
    0x1.371a7373aa9cbp+0, 0x1.37f26231e754ap+0, 0x1.38cae6d05d866p+0, 0x1.39a401b7140efp+0,
    0x1.3a7db34e59ff7p+0, 0x1.3b57fbfec6cf4p+0, 0x1.3c32dc313a8e5p+0, 0x1.3d0e544ede173p+0,
    0x1.3dea64c123422p+0, 0x1.3ec70df1c5175p+0, 0x1.3fa4504ac801cp+0, 0x1.40822c367a024p+0,
    0x1.4160a21f72e2ap+0, 0x1.423fb2709468ap+0, 0x1.431f5d950a897p+0, 0x1.43ffa3f84b9d4p+0,
    0x1.44e086061892dp+0, 0x1.45c2042a7d232p+0, 0x1.46a41ed1d0057p+0, 0x1.4786d668b3237p+0,
    0x1.486a2b5c13cd0p+0, 0x1.494e1e192aed2p+0, 0x1.4a32af0d7d3dep+0, 0x1.4b17dea6db7d7p+0,
    0x1.4bfdad5362a27p+0, 0x1.4ce41b817c114p+0, 0x1.4dcb299fddd0dp+0, 0x1.4eb2d81d8abffp+0,
    0x1.4f9b2769d2ca7p+0, 0x1.508417f4531eep+0, 0x1.516daa2cf6642p+0, 0x1.5257de83f4eefp+0,
    0x1.5342b569d4f82p+0, 0x1.542e2f4f6ad27p+0, 0x1.551a4ca5d920fp+0, 0x1.56070dde910d2p+0,
    0x1.56f4736b527dap+0, 0x1.57e27dbe2c4cfp+0, 0x1.58d12d497c7fdp+0, 0x1.59c0827ff07ccp+0,
    0x1.5ab07dd485429p+0, 0x1.5ba11fba87a03p+0, 0x1.5c9268a5946b7p+0, 0x1.5d84590998b93p+0,
    0x1.5e76f15ad2148p+0, 0x1.5f6a320dceb71p+0, 0x1.605e1b976dc09p+0, 0x1.6152ae6cdf6f4p+0,
    0x1.6247eb03a5585p+0, 0x1.633dd1d1929fdp+0, 0x1.6434634ccc320p+0, 0x1.652b9febc8fb7p+0,
    0x1.6623882552225p+0, 0x1.671c1c70833f6p+0, 0x1.68155d44ca973p+0, 0x1.690f4b19e9538p+0,
    0x1.6a09e667f3bcdp+0, 0x1.6b052fa75173ep+0, 0x1.6c012750bdabfp+0, 0x1.6cfdcddd47645p+0,
    0x1.6dfb23c651a2fp+0, 0x1.6ef9298593ae5p+0, 0x1.6ff7df9519484p+0, 0x1.70f7466f42e87p+0,
    0x1.71f75e8ec5f74p+0, 0x1.72f8286ead08ap+0, 0x1.73f9a48a58174p+0, 0x1.74fbd35d7cbfdp+0,
    0x1.75feb564267c9p+0, 0x1.77024b1ab6e09p+0, 0x1.780694fde5d3fp+0, 0x1.790b938ac1cf6p+0,
    0x1.7a11473eb0187p+0, 0x1.7b17b0976cfdbp+0, 0x1.7c1ed0130c132p+0, 0x1.7d26a62ff86f0p+0,
    0x1.7e2f336cf4e62p+0, 0x1.7f3878491c491p+0, 0x1.80427543e1a12p+0, 0x1.814d2add106d9p+0,
    0x1.82589994cce13p+0, 0x1.8364c1eb941f7p+0, 0x1.8471a4623c7adp+0, 0x1.857f4179f5b21p+0,
    0x1.868d99b4492edp+0, 0x1.879cad931a436p+0, 0x1.88ac7d98a6699p+0, 0x1.89bd0a478580fp+0,
    0x1.8ace5422aa0dbp+0, 0x1.8be05bad61778p+0, 0x1.8cf3216b5448cp+0, 0x1.8e06a5e0866d9p+0,
    0x1.8f1ae99157736p+0, 0x1.902fed0282c8ap+0, 0x1.9145b0b91ffc6p+0, 0x1.925c353aa2fe2p+0,
    0x1.93737b0cdc5e5p+0, 0x1.948b82b5f98e5p+0, 0x1.95a44cbc8520fp+0, 0x1.96bdd9a7670b3p+0,
    0x1.97d829fde4e50p+0, 0x1.98f33e47a22a2p+0, 0x1.9a0f170ca07bap+0, 0x1.9b2bb4d53fe0dp+0,
    0x1.9c49182a3f090p+0, 0x1.9d674194bb8d5p+0, 0x1.9e86319e32323p+0, 0x1.9fa5e8d07f29ep+0,
    0x1.a0c667b5de565p+0, 0x1.a1e7aed8eb8bbp+0, 0x1.a309bec4a2d33p+0, 0x1.a42c980460ad8p+0,
    0x1.a5503b23e255dp+0, 0x1.a674a8af46052p+0, 0x1.a799e1330b358p+0, 0x1.a8bfe53c12e59p+0,
    0x1.a9e6b5579fdbfp+0, 0x1.ab0e521356ebap+0, 0x1.ac36bbfd3f37ap+0, 0x1.ad5ff3a3c2774p+0,
    0x1.ae89f995ad3adp+0, 0x1.afb4ce622f2ffp+0, 0x1.b0e07298db666p+0, 0x1.b20ce6c9a8952p+0,
    0x1.b33a2b84f15fbp+0, 0x1.b468415b749b1p+0, 0x1.b59728de5593ap+0, 0x1.b6c6e29f1c52ap+0,
    0x1.b7f76f2fb5e47p+0, 0x1.b928cf22749e4p+0, 0x1.ba5b030a1064ap+0, 0x1.bb8e0b79a6f1fp+0,
    0x1.bcc1e904bc1d2p+0, 0x1.bdf69c3f3a207p+0, 0x1.bf2c25bd71e09p+0, 0x1.c06286141b33dp+0,
    0x1.c199bdd85529cp+0, 0x1.c2d1cd9fa652cp+0, 0x1.c40ab5fffd07ap+0, 0x1.c544778fafb22p+0,
    0x1.c67f12e57d14bp+0, 0x1.c7ba88988c933p+0, 0x1.c8f6d9406e7b5p+0, 0x1.ca3405751c4dbp+0,
    0x1.cb720dcef9069p+0, 0x1.ccb0f2e6d1675p+0, 0x1.cdf0b555dc3fap+0, 0x1.cf3155b5bab74p+0,
    0x1.d072d4a07897cp+0, 0x1.d1b532b08c968p+0, 0x1.d2f87080d89f2p+0, 0x1.d43c8eacaa1d6p+0,
    0x1.d5818dcfba487p+0, 0x1.d6c76e862e6d3p+0, 0x1.d80e316c98398p+0, 0x1.d955d71ff6075p+0,
    0x1.da9e603db3285p+0, 0x1.dbe7cd63a8315p+0, 0x1.dd321f301b460p+0, 0x1.de7d5641c0658p+0,
    0x1.dfc97337b9b5fp+0, 0x1.e11676b197d17p+0, 0x1.e264614f5a129p+0, 0x1.e3b333b16ee12p+0,
    0x1.e502ee78b3ff6p+0, 0x1.e653924676d76p+0, 0x1.e7a51fbc74c83p+0, 0x1.e8f7977cdb740p+0,
    0x1.ea4afa2a490dap+0, 0x1.eb9f4867cca6ep+0, 0x1.ecf482d8e67f1p+0, 0x1.ee4aaa2188510p+0,
    0x1.efa1bee615a27p+0, 0x1.f0f9c1cb6412ap+0, 0x1.f252b376bba97p+0, 0x1.f3ac948dd7274p+0,
    0x1.f50765b6e4540p+0, 0x1.f6632798844f8p+0, 0x1.f7bfdad9cbe14p+0, 0x1.f91d802243c89p+0,
    0x1.fa7c1819e90d8p+0, 0x1.fbdba3692d514p+0, 0x1.fd3c22b8f71f1p+0, 0x1.fe9d96b2a23d9p+0,
};

// One table entry: the low word of 2^(j/256) and its high word minus j << 12.
struct alignas(8) TabEntry {
    uint32_t lo, hi;
};

// Fills the LDS table; call with every thread of the workgroup, then barrier.
__device__ __forceinline__ void load_table(TabEntry* tbl, int nthreads) {
    for (int i = threadIdx.x; i < 256; i += nthreads) {
        const uint64_t bits = static_cast<uint64_t>(__double_as_longlong(kExp2Frac[i]));
        tbl[i].lo = static_cast<uint32_t>(bits);
        tbl[i].hi = static_cast<uint32_t>(bits >> 32) - (static_cast<uint32_t>(i) << 12);
    }
}

// 2^(Y/256) in fp64 for Y <= 0 (Y is clamped at kMinY, where it is 0).  Y = n + r with
// n = round(Y) (the 1.5 * 2^52 shifter: after the add the low 32 bits of the
// double hold n in two's complement) and |r| <= 1/2, so
// 2^(Y/256) = 2^(n>>8) 2^((n&255)/256) e^x with x = r ln2/256, |x| <= ln2/512;
// e^x - 1 by its degree-4 Taylor polynomial (truncation < 4e-17 relative).
__device__ __forceinline__ double exp2_256(double Y, const TabEntry* tbl) {
    constexpr double kShift = 0x1.8p52;
    Y = fmax(Y, kMinY);
    const double kd = Y + kShift;
    const uint32_t n = static_cast<uint32_t>(__double_as_longlong(kd));
    const double r = Y - (kd - kShift);            // exact
    double q = fma(r, 0x1.3b2ab6fba4e77p-39, 0x1.c6b08d704a0c0p-29);
    q = fma(q, r, 0x1.ebfbdff82c58fp-19);
    q = fma(q, r, 0x1.62e42fefa39efp-9);
    const TabEntry e = tbl[n & 255u];
    const double t = __hiloint2double(static_cast<int>(e.hi + (n << 12)), static_cast<int>(e.lo));
    return fma(t, q * r, t);
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

// kR consecutive logits of one row, loaded by one lane in as few loads as
// their alignment allows (aligned(): to their size, at most 16 bytes).
template <int DT, int kR>
struct Run {
    using E = typename Vec<DT>::E;
    static constexpr int kBytes = kR * static_cast<int>(sizeof(E));
    static constexpr int kWords = kBytes / 4;
    static constexpr uintptr_t kAlign = kBytes < 16 ? kBytes : 16;
    __device__ static __forceinline__ bool aligned(const E* ptr) {
        return (reinterpret_cast<uintptr_t>(ptr) & (kAlign - 1)) == 0;
    }
    __device__ static __forceinline__ void load(const E* ptr, float* z) {
        uint32_t w[kWords];
        if constexpr (kBytes >= 16) {
#pragma unroll
            for (int i = 0; i < kBytes / 16; ++i) {
                const u32x4 v = reinterpret_cast<const u32x4*>(ptr)[i];
#pragma unroll
                for (int j = 0; j < 4; ++j) w[4 * i + j] = v[j];
            }
        } else if constexpr (kBytes == 8) {
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            const u32x2 v = *reinterpret_cast<const u32x2*>(ptr);
            w[0] = v[0];
            w[1] = v[1];
        } else {
            static_assert(kBytes == 4, "run size");
            w[0] = *reinterpret_cast<const uint32_t*>(ptr);
        }
#pragma unroll
        for (int i = 0; i < kWords; ++i) {
            if constexpr (DT == SV_BF16) {
                z[2 * i] = __uint_as_float(w[i] << 16);
                z[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
            } else {
                z[i] = __uint_as_float(w[i]);
            }
        }
    }
};

// The one or two rows a draw reads, and Y = 256 (z - m) log2(e) / T as one fma.
template <int DT>
struct Rows {
    using E = typename Vec<DT>::E;
    const E* t;          // target row at position n
    const E* d;          // draft row at position n (residual only)
    double c;            // 256 log2(e) / T
    double ot, od;       // -m_t * c, -m_d * c
    const TabEntry* tbl;

    __device__ __forceinline__ double Yt(float z) const { return fma(static_cast<double>(z), c, ot); }
    __device__ __forceinline__ double Yd(float z) const { return fma(static_cast<double>(z), c, od); }
    __device__ __forceinline__ double wt(float z) const { return exp2_256(Yt(z), tbl); }
    __device__ __forceinline__ double wd(float z) const { return exp2_256(Yd(z), tbl); }
    __device__ __forceinline__ float zt(int64_t v) const { return load_logit(t, DT, v); }
    __device__ __forceinline__ float zd(int64_t v) const { return load_logit(d, DT, v); }
};

template <int DT>
__device__ __forceinline__ Rows<DT> rows_of(const Problem& p, const DrawTask& task, const TabEntry* tbl) {
    using E = typename Vec<DT>::E;
    const double c = 256.0 * kLog2e / static_cast<double>(task.T);
    return Rows<DT>{static_cast<const E*>(p.target) + task.trow * p.V,
                    static_cast<const E*>(p.draft) + task.drow * p.V,
                    c, -static_cast<double>(task.m_t) * c, -static_cast<double>(task.m_d) * c, tbl};
}

// Cache policy of the draw's row loads: non-temporal.  Each draw chunk reads
// its piece of a row once; letting those lines allocate in the caches only
// evicts others (512 ragged sequences of V = 128256: the two-round launch
// 162.7-163.0 against 166.3-166.5 us; 256 of V = 152064: 157.2-157.6
// against 157.6-158.5).
constexpr int kDrawLoadPolicy = 2;

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, int32_t byte_off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kDrawLoadPolicy));
}

// Calls f(z_t, z_d) for this lane's tokens of [v0, v1), run by one whole
// wave: lane-strided 16-byte vectors, then single tokens for a ragged tail.
// When both rows are 16-byte aligned at v0 the vectors come from raw buffer
// loads against descriptors that span exactly the range's vectors, one
// iteration ahead of use (a load past the end returns zeros and touches no
// memory); otherwise every token is loaded on its own.
template <int DT, bool kResid, class F>
__device__ __forceinline__ void for_range(const Rows<DT>& rows, int64_t v0, int64_t v1, F&& f) {
    using E = typename Vec<DT>::E;
    constexpr int N = Vec<DT>::N;
    const int lane = threadIdx.x & 63;
    const bool vec = (reinterpret_cast<uintptr_t>(rows.t + v0) & 15u) == 0 &&
                     (!kResid || (reinterpret_cast<uintptr_t>(rows.d + v0) & 15u) == 0);
    int64_t vs = v0;
    if (vec) {
        const int32_t nvec = static_cast<int32_t>((v1 - v0) / N);
        const __amdgpu_buffer_rsrc_t rt =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<E*>(rows.t + v0), 0, nvec * 16, kBufferDword3);
        const __amdgpu_buffer_rsrc_t rd = kResid
            ? __builtin_amdgcn_make_buffer_rsrc(const_cast<E*>(rows.d + v0), 0, nvec * 16, kBufferDword3)
            : rt;
        int32_t j = lane;
        u32x4 a = buffer_load16(rt, j * 16);
        u32x4 bb = kResid ? buffer_load16(rd, j * 16) : a;
        for (; j < nvec; j += 64) {
            const u32x4 an = buffer_load16(rt, (j + 64) * 16);
            const u32x4 bn = kResid ? buffer_load16(rd, (j + 64) * 16) : an;
            float xt[N], xd[N];
            Vec<DT>::unpack(a, xt);
            if (kResid) Vec<DT>::unpack(bb, xd);
#pragma unroll
            for (int e = 0; e < N; ++e) {
                f(xt[e], kResid ? xd[e] : 0.f);
                // interleave at most two tokens' fp64 work: bounds the register count
                if (e % 2 == 1) __builtin_amdgcn_sched_barrier(0);
            }
            a = an;
            bb = bn;
        }
        vs = v0 + static_cast<int64_t>(nvec) * N;
    }
    for (int64_t v = vs + lane; v < v1; v += 64)
        f(rows.zt(v), kResid ? rows.zd(v) : 0.f);
}

// Sums of four doubles over one wave (valid in every lane; a fixed
// butterfly, so every lane holds the same bits).
__device__ __forceinline__ void wave_sum4(double& a, double& b, double& c, double& d) {
    for (int off = 32; off > 0; off >>= 1) {
        a += __shfl_xor(a, off, 64);
        b += __shfl_xor(b, off, 64);
        c += __shfl_xor(c, off, 64);
        d += __shfl_xor(d, off, 64);
    }
}

}  // namespace drawpass

// Sub-chunk w (0 <= w < kWaves) of chunk c: the chunk cut into kWaves
// contiguous pieces of a whole number of 16-byte vectors (the last one
// shorter, possibly empty), one per wave of the chunk's workgroup.  The
// pick keeps the masses of sub-chunks, so its final scan covers a quarter
// of a chunk.  [*s0, *s1) in token ids.
template <int DT>
__device__ __forceinline__ void sub_range(const Problem& p, const Plan& plan, int64_t c, int w, int64_t* s0,
                                          int64_t* s1) {
    constexpr int64_t N = drawpass::Vec<DT>::N;
    const int64_t q = ((plan.chunk_len + kWaves - 1) / kWaves + N - 1) / N * N;
    const int64_t c0 = c * plan.chunk_len, c1 = min(p.V, c0 + plan.chunk_len);
    *s0 = min(c1, c0 + w * q);
    *s1 = min(c1, c0 + (w + 1) * q);
}

// Sum over [v0, v1) (one whole wave) of w = 2^((Y - R) / 256),
// Y = fma(z, rows.c, 0) = 256 z log2(e) / T, relative to a reference R of
// the range's own: a whole number of octaves (a multiple of 256) at most
// kSlackOct octaves below the largest Y.  Each lane raises its reference,
// with an exact power-of-two rescale of its sum, only when a logit passes
// it by that much; the lanes' sums are then rescaled to the wave's largest
// reference.  Weights relative to any common reference give the same
// distribution.  In every lane: *s, *R (-inf: no finite logit) and the
// range's largest logit *mx (a non-finite one: *s = 0, *R = -inf).
template <int DT>
__device__ __forceinline__ void self_ref_sum(const drawpass::Rows<DT>& rows, int64_t v0, int64_t v1, double* s_out,
                                             double* R_out, float* mx_out) {
    using namespace drawpass;
    constexpr double kSlackY = 256.0 * 32.0;     // kSlackOct = 32 octaves
    const double C = rows.c;
    float mx = -INFINITY;
    double R = -INFINITY, s = 0.0;
    for_range<DT, false>(rows, v0, v1, [&](float z, float) {
        mx = fmaxf(mx, z);
        double Y = fma(static_cast<double>(z), C, -R);
        if (Y > kSlackY) {                        // (the first finite logit: Y = +inf)
            const double Rn = 256.0 * ceil(static_cast<double>(z) * (C / 256.0));
            s = ldexp(s, static_cast<int>(fmax((R - Rn) / 256.0, -2048.0)));
            R = Rn;
            Y = fma(static_cast<double>(z), C, -R);
        }
        s += exp2_256(Y, rows.tbl);
    });
    double Rw = R;
    for (int off = 32; off > 0; off >>= 1) {
        mx = fmaxf(mx, __shfl_xor(mx, off, 64));
        Rw = fmax(Rw, __shfl_xor(Rw, off, 64));
    }
    const bool finite = fabsf(mx) <= 3.4e38f;
    s = (R == -INFINITY || !finite) ? 0.0 : ldexp(s, static_cast<int>(fmax((R - Rw) / 256.0, -2048.0)));
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    *s_out = finite ? s : 0.0;
    *R_out = finite ? Rw : -INFINITY;
    *mx_out = mx;
}

// Workgroup scratch of one draw chunk (256 threads): each wave's band list.
struct DrawLds {
    double wlist[kWaves][kWaveCap][2];
    int32_t wcount[kWaves];
};

// The exp2 table in LDS: every thread of the workgroup calls this, then the
// workgroup synchronises before first use.
__device__ __forceinline__ void load_exp2_table(drawpass::TabEntry* tbl, int nthreads) {
    drawpass::load_table(tbl, nthreads);
}

// Chunk c of the draw of sequence b (256 threads): wave w accumulates the
// fp64 sums and band list of sub-chunk w (see the file comment).  `task` is
// the sequence's DrawTask (kind != kNone).  kCo: the results go to the pick
// in another workgroup of the same launch.  NT: the workgroup size; threads
// past the first 256 do no work but take part in the barrier, so the
// results are those of a 256-thread workgroup, bit for bit.
template <int DT, bool kCo, int NT = kThreads>
__device__ __forceinline__ void draw_chunk(const Problem& p, const Plan& plan, const DrawTask& task,
                                           int32_t b, int32_t c, const drawpass::TabEntry* tbl,
                                           DrawLds& lds) {
    using namespace drawpass;
    // (the wave index through readfirstlane: the compiler then keeps the
    // sub-chunk's bounds and buffer descriptors in scalar registers)
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t sub = (static_cast<int64_t>(b) * plan.nchunk + c) * kWaves;   // sub-chunk 0 of the chunk
    const bool resid_task = (task.kind == kResidual);
    const Rows<DT> rows = rows_of<DT>(p, task, tbl);
    const bool active = NT == kThreads || threadIdx.x < kThreads;
    int64_t v0 = 0, v1 = 0;
    if (active) sub_range<DT>(p, plan, c, wave, &v0, &v1);

    double sp = 0.0, sq = 0.0, a = 0.0, bq = 0.0;
    int32_t nband = 0;                         // uniform over the lanes still active
    if (!active) {
    } else if (resid_task) {
        const double th_hi = 256.0 * (task.theta + kBand), th_lo = 256.0 * (task.theta - kBand);
        for_range<DT, true>(rows, v0, v1, [&](float zt, float zd) {
            const double yt = rows.Yt(zt), yd = rows.Yd(zd);
            const double wt = exp2_256(yt, tbl), wd = exp2_256(yd, tbl);
            sp += wt;
            sq += wd;
            const double dv = yt - yd;
            const bool hi = dv > th_hi;
            const double h = hi ? 1.0 : 0.0;
            a = fma(h, wt, a);
            bq = fma(h, wd, bq);
            // band = lanes with th_lo <= d_v <= th_hi (wave-uniform mask)
            const uint64_t band = __ballot(dv >= th_lo) & ~__ballot(hi);
            if (band) {
                const int pos = nband + __popcll(band & ((1ull << lane) - 1ull));
                if (((band >> lane) & 1ull) && pos < kWaveCap) {
                    lds.wlist[wave][pos][0] = wt;
                    lds.wlist[wave][pos][1] = wd;
                }
                nband += __popcll(band);
            }
        });
    } else if (task.kind == kBonusSelf) {
        float mx;
        self_ref_sum<DT>(rows, v0, v1, &sp, &sq, &mx);   // (already summed over the wave)
        a = mx;
    } else {
        for_range<DT, false>(rows, v0, v1, [&](float zt, float) { sp += rows.wt(zt); });
    }
    if (active) {
        if (task.kind != kBonusSelf) wave_sum4(sp, sq, a, bq);
        if (lane == 0) {                       // lane 0 was active whenever any lane was
            lds.wcount[wave] = nband;
            ChunkSums* cs = plan.csum + sub + wave;
            st_co<kCo>(&cs->sp, sp);
            st_co<kCo>(&cs->sq, sq);
            st_co<kCo>(&cs->a, a);
            st_co<kCo>(&cs->b, bq);
            if (resid_task) st_co<kCo>(&plan.band_n[sub + wave], nband);
        }
    }
    if (resid_task) {
        __syncthreads();
        if (threadIdx.x < kSlots) {
            const int wv = threadIdx.x / kWaveCap, e = threadIdx.x % kWaveCap;
            if (e < lds.wcount[wv]) {
                double* dst = plan.band_w + (sub * kWaveCap + threadIdx.x) * 2;
                st_co<kCo>(&dst[0], lds.wlist[wv][e][0]);
                st_co<kCo>(&dst[1], lds.wlist[wv][e][1]);
            }
        }
        // A caller that sums another chunk next would otherwise let waves
        // 1-3 refill their lists while wave 0 still copies them out.
        __syncthreads();
    }
}

// ---- the pick: one NT-thread workgroup per sequence -----------------------

constexpr int kMaxPickSubs = kMaxChunks * kWaves;   // sub-chunk masses held in LDS by the pick
constexpr int64_t kPiece = 2048;                     // tokens per step of the pick's final scan

template <int NT, int MAXS = kMaxPickSubs>
struct PickLds {
    static constexpr int kW = NT / 64;
    double red2[kW][2];
    double scan[kW];
    int32_t ldsi[2 * kW];
    double mass[MAXS];
    double spc[MAXS];
    double base, target, Z;
    int32_t chunk, resid, rescan;
};

namespace drawpass {

// Sum of two doubles over an NT-thread workgroup (valid in every thread).
template <int NT>
__device__ __forceinline__ void pick_sum2(double& a, double& b, double (*lds)[2]) {
    for (int off = 32; off > 0; off >>= 1) {
        a += __shfl_xor(a, off, 64);
        b += __shfl_xor(b, off, 64);
    }
    __syncthreads();
    if ((threadIdx.x & 63) == 0) { lds[threadIdx.x >> 6][0] = a; lds[threadIdx.x >> 6][1] = b; }
    __syncthreads();
    a = b = 0.0;
    for (int w = 0; w < NT / 64; ++w) { a += lds[w][0]; b += lds[w][1]; }
}

// The maxima of a float and a double over an NT-thread workgroup (valid in
// every thread).
template <int NT>
__device__ __forceinline__ void pick_max2(float& x, double& y, double (*lds)[2]) {
    for (int off = 32; off > 0; off >>= 1) {
        x = fmaxf(x, __shfl_xor(x, off, 64));
        y = fmax(y, __shfl_xor(y, off, 64));
    }
    __syncthreads();
    if ((threadIdx.x & 63) == 0) { lds[threadIdx.x >> 6][0] = x; lds[threadIdx.x >> 6][1] = y; }
    __syncthreads();
    x = static_cast<float>(lds[0][0]);
    y = lds[0][1];
    for (int w = 1; w < NT / 64; ++w) { x = fmaxf(x, static_cast<float>(lds[w][0])); y = fmax(y, lds[w][1]); }
}

// Exclusive prefix sum over an NT-thread workgroup in thread order; *total = sum.
template <int NT>
__device__ __forceinline__ double pick_scan_excl(double x, double* total, double* lds) {
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
    for (int w = 0; w < NT / 64; ++w) {
        if (w < wave) before += lds[w];
        all += lds[w];
    }
    *total = all;
    return before + excl;
}

// The minimum of x and the maximum of y over an NT-thread workgroup, in one
// exchange through LDS (lds: 2 * NT / 64 ints).
template <int NT>
__device__ __forceinline__ void pick_min_and_max(int32_t& x, int32_t& y, int32_t* lds) {
    for (int off = 32; off > 0; off >>= 1) {
        x = min(x, __shfl_xor(x, off, 64));
        y = max(y, __shfl_xor(y, off, 64));
    }
    __syncthreads();
    if ((threadIdx.x & 63) == 0) { lds[2 * (threadIdx.x >> 6)] = x; lds[2 * (threadIdx.x >> 6) + 1] = y; }
    __syncthreads();
    x = lds[0];
    y = lds[1];
    for (int w = 1; w < NT / 64; ++w) { x = min(x, lds[2 * w]); y = max(y, lds[2 * w + 1]); }
}

// Wave-wide search over chunk masses m[0..n) (run by one whole wave): the
// first chunk whose cumulative mass exceeds target, with the mass before it;
// when rounding leaves target at or past the total, the last chunk with
// positive mass.  Returns the total in *Z.
__device__ __forceinline__ void find_chunk(const double* m, int32_t n, double u, double* Z,
                                           int32_t* chunk, double* base) {
    const int lane = threadIdx.x & 63;
    const int32_t per = (n + 63) / 64;        // chunks per lane, in order
    const int32_t j0 = min(n, lane * per), j1 = min(n, j0 + per);
    double mine = 0.0;
    for (int32_t j = j0; j < j1; ++j) mine += m[j];
    double inc = mine;
    for (int off = 1; off < 64; off <<= 1) {
        const double y = __shfl_up(inc, off, 64);
        if (lane >= off) inc += y;
    }
    const double total = __shfl(inc, 63, 64);
    const double target = u * total;
    const double excl = inc - mine;
    // the lane whose range holds the crossing: excl <= target < inc
    int32_t found = -1;
    double fb = 0.0;
    if (excl <= target && target < inc) {
        double run = excl;
        for (int32_t j = j0; j < j1; ++j) {
            if (run + m[j] > target) { found = j; fb = run; break; }
            run += m[j];
        }
    }
    // fallback: the last chunk with positive mass
    int32_t lastj = -1;
    double lastb = 0.0;
    {
        double run = excl;
        for (int32_t j = j0; j < j1; ++j) {
            if (m[j] > 0.0) { lastj = j; lastb = run; }
            run += m[j];
        }
    }
    const uint64_t fm = __ballot(found >= 0);
    if (fm) {
        const int src = __ffsll(static_cast<unsigned long long>(fm)) - 1;
        *chunk = __shfl(found, src, 64);
        *base = __shfl(fb, src, 64);
    } else {
        const uint64_t lm = __ballot(lastj >= 0);
        const int src = lm ? 63 - __clzll(static_cast<long long>(lm)) : 0;
        *chunk = lm ? __shfl(lastj, src, 64) : 0;
        *base = lm ? __shfl(lastb, src, 64) : 0.0;
    }
    *Z = total;
}

}  // namespace drawpass

// The final step of a pick (every thread of the NT-thread workgroup): scans
// sub-chunk L.chunk from the cumulative mass L.base for the first token whose
// cumulative mass exceeds L.target, and writes it to out_tokens[out_slot]
// (and its probability, mass / L.Z, to out_emit_prob[b]).  Masses are
// max(0, w_t iSp - w_d iSq) for a residual draw, w_t otherwise.
template <int DT, int NT, int MAXS>
__device__ __forceinline__ void pick_scan(const Problem& p, const Plan& plan, const drawpass::Rows<DT>& rows,
                                          bool resid, double iSp, double iSq, int64_t out_slot, int32_t b,
                                          PickLds<NT, MAXS>& L) {
    using namespace drawpass;
    constexpr int kRun = kPiece / NT;        // tokens per lane per scan step
    const int tid = threadIdx.x;
    const double target = L.target;
    double base = L.base;
    int64_t c0, c1;
    sub_range<DT>(p, plan, L.chunk / kWaves, L.chunk % kWaves, &c0, &c1);

    // Scan the sub-chunk in pieces of kPiece tokens: lane tid owns kRun
    // consecutive tokens of the piece, loaded together, masses kept in
    // registers.  The next piece's loads are issued before this piece's
    // arithmetic.
    auto load_piece = [&](int64_t q0, float (&zt)[kRun], float (&zd)[kRun]) {
        const int64_t q1 = min(c1, q0 + kPiece);
        const int64_t r0 = q0 + static_cast<int64_t>(tid) * kRun;
        // (fp32 runs shorter than 16 bytes take the per-token path: two
        // dword loads cost no more, and the two-path form put zt/zd in
        // scratch memory)
        constexpr bool kVec = DT == SV_BF16 || kRun * 4 >= 16;
        if (kVec && r0 + kRun <= q1 && Run<DT, kRun>::aligned(rows.t + r0) &&
            (!resid || Run<DT, kRun>::aligned(rows.d + r0))) {
            Run<DT, kRun>::load(rows.t + r0, zt);
            if (resid) Run<DT, kRun>::load(rows.d + r0, zd);
        } else {
#pragma unroll
            for (int i = 0; i < kRun; ++i) {
                const bool in = r0 + i < q1;
                zt[i] = in ? rows.zt(r0 + i) : 0.f;
                zd[i] = (in && resid) ? rows.zd(r0 + i) : 0.f;
            }
        }
    };
    int32_t pick = INT32_MAX, last_pos = -1, mine = INT32_MAX;
    double mine_mass = 0.0;
    float zt[kRun], zd[kRun];
#pragma unroll
    for (int i = 0; i < kRun; ++i) zd[i] = 0.f;
    load_piece(c0, zt, zd);
    for (int64_t q0 = c0; q0 < c1 && pick == INT32_MAX; q0 += kPiece) {
        const int64_t q1 = min(c1, q0 + kPiece);
        const int64_t r0 = q0 + static_cast<int64_t>(tid) * kRun;
        float nzt[kRun], nzd[kRun];
#pragma unroll
        for (int i = 0; i < kRun; ++i) { nzt[i] = 0.f; nzd[i] = 0.f; }
        if (q1 < c1) load_piece(q1, nzt, nzd);
        double m[kRun];
        double local = 0.0;
        int32_t lp = -1;
#pragma unroll
        for (int i = 0; i < kRun; ++i) {
            const bool in = r0 + i < q1;
            m[i] = !in ? 0.0
                       : (resid ? fmax(0.0, rows.wt(zt[i]) * iSp - rows.wd(zd[i]) * iSq) : rows.wt(zt[i]));
            local += m[i];
            if (m[i] > 0.0) lp = static_cast<int32_t>(r0 + i);
        }
        double total;
        double run = base + pick_scan_excl<NT>(local, &total, L.scan);
        mine = INT32_MAX;
#pragma unroll
        for (int i = 0; i < kRun; ++i) {
            run += m[i];
            if (mine == INT32_MAX && run > target) { mine = static_cast<int32_t>(r0 + i); mine_mass = m[i]; }
        }
        int32_t first = mine;
        pick_min_and_max<NT>(first, lp, L.ldsi);
        pick = first;
        last_pos = max(last_pos, lp);
        base += total;
#pragma unroll
        for (int i = 0; i < kRun; ++i) { zt[i] = nzt[i]; zd[i] = nzd[i]; }
    }
    if (pick != INT32_MAX) {
        // the thread that found the crossing holds the token's mass
        if (mine == pick) {
            p.out_tokens[out_slot] = pick;
            if (p.out_emit_prob) p.out_emit_prob[b] = static_cast<float>(mine_mass / L.Z);
        }
    } else if (tid == 0) {
        // rounding left no crossing inside the chunk: its last token with mass
        pick = last_pos >= 0 ? last_pos : static_cast<int32_t>(c0);
        p.out_tokens[out_slot] = pick;
        if (p.out_emit_prob) {
            // its probability under the distribution it was drawn from
            const double wt = rows.wt(rows.zt(pick));
            const double mass = resid ? fmax(0.0, wt * iSp - rows.wd(rows.zd(pick)) * iSq) : wt;
            p.out_emit_prob[b] = static_cast<float>(mass / L.Z);
        }
    }
}

// The loads of a pick that need only the sequence, for sub-chunk
// threadIdx.x: its sums and band count (so they can be issued before the
// task is known; for a bonus draw all but sp are unused).
struct PickPrefetch {
    double sp = 0.0, sq = 0.0, a = 0.0, b = 0.0;
    int32_t cnt = 0;
};
template <bool kCo>
__device__ __forceinline__ PickPrefetch pick_prefetch(const Plan& plan, int32_t b) {
    PickPrefetch f;
    const int32_t j = threadIdx.x;
    if (j < plan.nchunk * kWaves) {
        const int64_t sj = static_cast<int64_t>(b) * plan.nchunk * kWaves + j;
        const ChunkSums* c = plan.csum + sj;
        f.sp = ld_co<kCo>(&c->sp);
        f.sq = ld_co<kCo>(&c->sq);
        f.a = ld_co<kCo>(&c->a);
        f.b = ld_co<kCo>(&c->b);
        f.cnt = ld_co<kCo>(&plan.band_n[sj]);
    }
    return f;
}

// The pick of sequence b (NT threads, NT a multiple of 256): from the sums
// of every sub-chunk of its draw, the emitted token.  `task` is the
// sequence's DrawTask (kind != kNone); plan.nchunk * kWaves <= MAXS; pf is
// pick_prefetch<kCo>(plan, b).  kCo: the sums come from other workgroups of
// the same launch.
template <int DT, int NT, bool kCo, int MAXS = kMaxPickSubs>
__device__ __forceinline__ void pick_sequence(const Problem& p, const Plan& plan, const DrawTask& task,
                                              int32_t b, const drawpass::TabEntry* tbl,
                                              PickLds<NT, MAXS>& L, const PickPrefetch& pf) {
    using namespace drawpass;
    static_assert(NT % 256 == 0 && NT <= 1024, "pick workgroup size");
    const int tid = threadIdx.x, wave = tid >> 6;
    const bool resid_task = (task.kind == kResidual);
    Rows<DT> rows = rows_of<DT>(p, task, tbl);
    const int32_t nsub = plan.nchunk * kWaves;
    const int64_t sb = static_cast<int64_t>(b) * nsub;
    const ChunkSums* cs = plan.csum + sb;
    if (tid == 0) L.rescan = 0;

    // A bonus draw of a row the row pass did not read: a non-finite maximum
    // of the row makes the sequence a data error; otherwise the sub-chunk
    // sums are rescaled exactly to their largest reference Y0 (by wave 0,
    // which then searches them), and the scan's weights are taken relative
    // to Y0.  A bonus draw needs no S_p: the search forms Z itself.
    const bool self_ref = task.kind == kBonusSelf;
    double Sp = 1.0, Sq = 1.0;
    if (self_ref) {
        float mx = -INFINITY;
        double Ym = -INFINITY;
        for (int32_t j = tid; j < nsub; j += NT) {
            const double y = j == tid ? pf.sq : ld_co<kCo>(&cs[j].sq);
            L.spc[j] = j == tid ? pf.sp : ld_co<kCo>(&cs[j].sp);
            L.mass[j] = y;
            Ym = fmax(Ym, y);
            mx = fmaxf(mx, static_cast<float>(j == tid ? pf.a : ld_co<kCo>(&cs[j].a)));
        }
        pick_max2<NT>(mx, Ym, L.red2);          // (its barriers also publish spc and mass)
        if (!(fabsf(mx) <= 3.4e38f)) {
            const int64_t o = p.offsets ? static_cast<int64_t>(p.offsets[b]) : static_cast<int64_t>(b) * p.k_uniform;
            const int64_t k = p.offsets ? static_cast<int64_t>(p.offsets[b + 1]) - o : p.k_uniform;
            for (int64_t i = tid; i <= k; i += NT) p.out_tokens[o + b + i] = -1;
            if (tid == 0) {
                p.out_n[b] = -1;
                if (p.out_emit_prob) p.out_emit_prob[b] = NAN;
            }
            return;
        }
        rows.ot = -Ym;
        if (wave == 0) {
            for (int32_t j = tid; j < nsub; j += 64) {
                const double y = L.mass[j];
                L.spc[j] = y == -INFINITY ? 0.0 : ldexp(L.spc[j], static_cast<int>(fmax((y - Ym) / 256.0, -2048.0)));
            }
            __builtin_amdgcn_wave_barrier();    // (LDS accesses of one wave complete in order)
        }
    } else {
        // Sub-chunk tid's sums and band count come prefetched (a row with
        // more sub-chunks than the workgroup has threads loads the others'
        // here and in the loop below).
        Sp = 0.0;
        Sq = 0.0;
        for (int32_t j = tid; j < nsub; j += NT) {
            const double xsp = j == tid ? pf.sp : ld_co<kCo>(&cs[j].sp);
            Sq += j == tid ? pf.sq : ld_co<kCo>(&cs[j].sq);
            Sp += xsp;
            L.spc[j] = xsp;
        }
        pick_sum2<NT>(Sp, Sq, L.red2);          // (its barriers also publish spc)
    }
    const double iSp = 1.0 / Sp, iSq = resid_task ? 1.0 / Sq : 0.0;

    if (resid_task) {
        // Sub-chunk j's residual mass, by thread j: A_j / S_p - B_j / S_q plus
        // max(0, w_t / S_p - w_d / S_q) of its listed band tokens in list
        // order; NaN marks a sub-chunk whose list overflowed (rescanned below).
        for (int32_t j = tid; j < nsub; j += NT) {
            double a = pf.a, bq = pf.b;
            int32_t cnt = pf.cnt;
            if (j != tid) {
                a = ld_co<kCo>(&cs[j].a);
                bq = ld_co<kCo>(&cs[j].b);
                cnt = ld_co<kCo>(&plan.band_n[sb + j]);
            }
            double m = a * iSp - bq * iSq;
            const int32_t nw = min(cnt, kWaveCap);
            if (nw > 0) {
                const double* pw = plan.band_w + (sb + j) * kWaveCap * 2;
                double wt[kWaveCap], wd[kWaveCap];
#pragma unroll
                for (int e = 0; e < kWaveCap; ++e) {
                    wt[e] = e < nw ? ld_co<kCo>(&pw[2 * e]) : 0.0;
                    wd[e] = e < nw ? ld_co<kCo>(&pw[2 * e + 1]) : 0.0;
                }
#pragma unroll
                for (int e = 0; e < kWaveCap; ++e)
                    if (e < nw) m += fmax(0.0, wt[e] * iSp - wd[e] * iSq);
            }
            L.mass[j] = cnt > kWaveCap ? NAN : m;
            if (cnt > kWaveCap) L.rescan = 1;  // benign race: every writer stores 1
        }
        __syncthreads();
        if (L.rescan) {
            // sub-chunks whose band list overflowed: exact rescan (rare)
            for (int32_t j = 0; j < nsub; ++j) {
                if (!isnan(L.mass[j])) continue;
                int64_t u0, u1;
                sub_range<DT>(p, plan, j / kWaves, j % kWaves, &u0, &u1);
                double m = 0.0, unused = 0.0;
                for (int64_t v = u0 + tid; v < u1; v += NT)
                    m += fmax(0.0, rows.wt(rows.zt(v)) * iSp - rows.wd(rows.zd(v)) * iSq);
                pick_sum2<NT>(m, unused, L.red2);
                if (tid == 0) L.mass[j] = m;
                __syncthreads();
            }
        }
    }
    if (wave == 0) {
        bool resid = resid_task;
        double Z = 0.0, base = 0.0;
        int32_t chunk = 0;
        if (resid) {
            find_chunk(L.mass, nsub, static_cast<double>(task.u), &Z, &chunk, &base);
            if (Z < kDegenerateZ) resid = false;   // draw from p_n instead
        }
        if (!resid) find_chunk(L.spc, nsub, static_cast<double>(task.u), &Z, &chunk, &base);
        if (tid == 0) {
            L.base = base;
            L.Z = Z;
            L.target = static_cast<double>(task.u) * Z;
            L.chunk = chunk;
            L.resid = resid;
        }
    }
    __syncthreads();
    pick_scan<DT, NT, MAXS>(p, plan, rows, L.resid, iSp, iSq, task.out_slot, b, L);
}

}  // namespace sv
