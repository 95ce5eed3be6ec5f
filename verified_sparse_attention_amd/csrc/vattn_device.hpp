// Device building blocks for the gfx950 decode step: Philox, the pinned fp32
// dot product and exp, exact fixed-point weights, wavefront/block scans and a
// block-wide multi-problem radix select.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vattn_plan.hpp"

namespace vattn {

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
// as 1, 2, 3", SC'11).  One call yields the sample keys of four consecutive
// tokens: counter (i >> 2, g, b, 0), key = seed, token i takes word i & 3.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                               uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        if (round) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint32_t hi0 = __umulhi(0xD2511F53u, c0), lo0 = 0xD2511F53u * c0;
        const uint32_t hi1 = __umulhi(0xCD9E8D57u, c2), lo1 = 0xCD9E8D57u * c2;
        const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
    }
    return make_uint4(c0, c1, c2, c3);
}

__device__ __forceinline__ uint32_t word_of(const uint4& w, int e) {
    return e == 0 ? w.x : e == 1 ? w.y : e == 2 ? w.z : w.w;
}

// Sample order: ascending (Philox word u, token index i).  Stored complemented
// so that "first n of the order" == "n largest keys".
__device__ __forceinline__ uint64_t sample_key(uint32_t u, uint32_t i) {
    return ~((static_cast<uint64_t>(u) << 32) | i);
}

// Top-k order: descending score, then ascending index; also "n largest keys".
__device__ __forceinline__ uint32_t okey(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint64_t topk_key(uint32_t ok, uint32_t i) {
    return (static_cast<uint64_t>(ok) << 32) | static_cast<uint32_t>(~i);
}

// ---------------------------------------------------------------------------
// Pinned arithmetic.  Every score that decides a discrete outcome is the same
// sequence of IEEE fp32 operations: for each block of 8 elements an fma chain
// from +0 in element order, then the block partials added pairwise (adjacent
// pairs first).  On the GPU a block is one lane's 16-byte slice and the tree is
// an xor butterfly across the lanes of a row; IEEE addition is commutative, so
// both lanes of a pair hold the identical sum.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float chain8(const float (&a)[8], const float (&b)[8]) {
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(a[e], b[e], acc);
    return acc;
}

template <int LPT>
__device__ __forceinline__ float tree_across_lanes(float v) {
#pragma unroll
    for (int m = 1; m < LPT; m <<= 1) v = v + __shfl_xor(v, m, 64);
    return v;
}

// Sequential form of the same blocked dot (one thread), N a multiple of 8 with
// N / 8 a power of two.
template <int N>
__device__ __forceinline__ float pdot_serial(const float* a, int sa, const float* b, int sb) {
    constexpr int NB = N / 8;
    float part[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        float acc = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(a[(8 * j + e) * sa], b[(8 * j + e) * sb], acc);
        part[j] = acc;
    }
#pragma unroll
    for (int w = NB; w > 1; w >>= 1) {
#pragma unroll
        for (int j = 0; j < w / 2; ++j) part[j] = part[2 * j] + part[2 * j + 1];
    }
    return part[0];
}

// exp(x) for x in [-28, 0]: Cody-Waite reduction with ln 2 split into a 15-bit
// head (n * LN2_HI exact for |n| < 2^9) and an fp32 tail, then the degree-7
// Taylor polynomial with coefficients fl32(1/k!) in Horner form, scaled by 2^n.
__device__ __forceinline__ float pinned_exp(float x) {
    const float kLog2e = 0x1.715476p+0f;   // fl32(1 / ln 2)
    const float kLn2Hi = 0x1.62e4p-1f;     // 22713 / 32768
    const float kLn2Lo = 0x1.7f7d1cp-20f;  // fl32(ln 2 - kLn2Hi)
    const float t = x * kLog2e;
    const float n = __builtin_rintf(t);
    float r = __builtin_fmaf(-n, kLn2Hi, x);
    r = __builtin_fmaf(-n, kLn2Lo, r);
    float p = 0x1.a01a02p-13f;                 // 1/7!
    p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f);  // 1/6!
    p = __builtin_fmaf(p, r, 0x1.111112p-7f);   // 1/5!
    p = __builtin_fmaf(p, r, 0x1.555556p-5f);   // 1/4!
    p = __builtin_fmaf(p, r, 0x1.555556p-3f);   // 1/3!
    p = __builtin_fmaf(p, r, 0x1p-1f);          // 1/2!
    p = __builtin_fmaf(p, r, 1.0f);             // 1/1!
    p = __builtin_fmaf(p, r, 1.0f);             // 1/0!
    return __builtin_ldexpf(p, static_cast<int>(n));
}

// E = trunc(exp(x) * 2^40), 0 below x = -28, at most 2^40.  The fp32 product is
// exact (power-of-two scale); the truncation is done on the bits.
__device__ __forceinline__ uint64_t fixed_weight(float x) {
    if (!(x >= -28.0f)) return 0;
    const float v = pinned_exp(x) * 0x1p40f;
    const uint32_t bits = __float_as_uint(v);
    const int ex = static_cast<int>((bits >> 23) & 0xFFu);
    if (ex == 0) return 0;
    const uint64_t mant = (bits & 0x7FFFFFu) | 0x800000u;
    const int sh = ex - 150;
    uint64_t e = sh >= 0 ? (mant << sh) : (sh > -24 ? (mant >> -sh) : 0);
    return e > (1ull << 40) ? (1ull << 40) : e;
}

// Unsigned 128-bit integer to fp64, round to nearest even.
__device__ __forceinline__ double u128_to_f64(unsigned __int128 x) {
    if (x == 0) return 0.0;
    const uint64_t hi = static_cast<uint64_t>(x >> 64), lo = static_cast<uint64_t>(x);
    const int msb = hi ? 127 - __clzll(hi) : 63 - __clzll(lo);
    if (msb <= 52) return static_cast<double>(lo);  // exact
    int s = msb - 52;
    unsigned __int128 m = x >> s;
    const unsigned __int128 rem = x & ((static_cast<unsigned __int128>(1) << s) - 1);
    const unsigned __int128 half = static_cast<unsigned __int128>(1) << (s - 1);
    if (rem > half || (rem == half && (m & 1))) m += 1;
    if (m >> 53) {
        m >>= 1;
        s += 1;
    }
    return __builtin_ldexp(static_cast<double>(static_cast<uint64_t>(m)), s);
}

// ---------------------------------------------------------------------------
// Loads of 8 consecutive elements (one lane's block) as fp32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void load8(const uint16_t* p, float (&f)[8]) {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        f[2 * k] = __uint_as_float(ws[k] << 16);
        f[2 * k + 1] = __uint_as_float(ws[k] & 0xFFFF0000u);
    }
}
__device__ __forceinline__ void load8(const float* p, float (&f)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// ---------------------------------------------------------------------------
// Sequence regions (sinks, window, middle), k, tail size and base-sample size.
// ---------------------------------------------------------------------------
struct Regions {
    int sp, wp, lo, hi, k, NT, nb;
};

__device__ __forceinline__ Regions regions(const Plan& P, int L) {
    Regions R;
    R.sp = min(P.sinks, L);
    R.wp = min(P.window, L - R.sp);
    R.lo = R.sp;
    R.hi = L - R.wp;
    const int nM = R.hi - R.lo;
    const long long k64 = P.topk_abs >= 0 ? static_cast<long long>(P.topk_abs)
                                          : (static_cast<long long>(L) * P.topk_ppm + 999999) / 1000000;
    R.k = static_cast<int>(k64 < nM ? k64 : nM);
    R.NT = nM - R.k;
    if (R.NT > 0) {
        long long want = (static_cast<long long>(R.NT) * P.base_ppm + 999999) / 1000000;
        if (want < 2) want = 2;
        R.nb = static_cast<int>(want < R.NT ? want : R.NT);
    } else {
        R.nb = 0;
    }
    return R;
}

// ---------------------------------------------------------------------------
// Scans and reductions.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    return v;
}

// Exclusive prefix over the block in thread order; `total` gets the block sum.
// `wsum` is LDS scratch of >= blockDim.x / 64 words.  All threads must call.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const uint32_t inc = wave_incl_scan(v);
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    uint32_t before = 0, tot = 0;
    for (int w = 0; w < nw; ++w) {
        const uint32_t x = wsum[w];
        before += (w < wave) ? x : 0u;
        tot += x;
    }
    __syncthreads();
    total = tot;
    return before + inc - v;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
    const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), m, 64);
    const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), m, 64);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// ---------------------------------------------------------------------------
// Block-wide radix select for NH independent problems at once.
// For problem h it finds thr[h] such that exactly want[h] of its keys are
// >= thr[h] (keys are unique 64-bit values).  Digits of 8 bits from the top;
// a problem stops as soon as its whole bucket is inside the answer.  Keys are
// produced by `items(visit)`, which calls visit(h, key) for every key assigned
// to this thread; it is called once per pass, so keys may be recomputed.
// want[h] must not exceed the number of keys of problem h (if it does, thr[h]
// selects all keys seen).  want[h] == 0 leaves problem h inactive.
// ---------------------------------------------------------------------------
template <int NH>
struct SelShared {
    uint32_t hist[NH][256];
    uint64_t prefix[NH];
    uint64_t thr[NH];
    uint32_t rem[NH];
    uint32_t active;
};

template <int NH, class Items>
__device__ void block_select(SelShared<NH>& S, const uint32_t (&want)[NH], Items&& items) {
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int lane = tid & 63, wave = tid >> 6, nwaves = nthr >> 6;
    if (tid == 0) {
        uint32_t act = 0;
        for (int h = 0; h < NH; ++h) {
            S.prefix[h] = 0;
            S.thr[h] = 0;
            S.rem[h] = want[h];
            if (want[h] > 0) act |= 1u << h;
        }
        S.active = act;
    }
    __syncthreads();
    for (int pass = 0; pass < 8; ++pass) {
        const uint32_t act = S.active;
        if (act == 0) break;  // block-uniform: read after a barrier
        const int shift = 56 - 8 * pass;
        for (int x = tid; x < NH * 256; x += nthr) (&S.hist[0][0])[x] = 0;
        uint64_t pre[NH];
#pragma unroll
        for (int h = 0; h < NH; ++h) pre[h] = S.prefix[h];
        __syncthreads();
        items([&](int h, uint64_t key) {
            if (!((act >> h) & 1u)) return;
            if (pass > 0 && ((key ^ pre[h]) >> (shift + 8)) != 0) return;
            atomicAdd(&S.hist[h][static_cast<uint32_t>(key >> shift) & 255u], 1u);
        });
        __syncthreads();
        for (int h = wave; h < NH; h += nwaves) {
            if (!((act >> h) & 1u)) continue;
            const uint32_t rem = S.rem[h];
            const int top = 255 - 4 * lane;  // this lane's bins: top, top-1, top-2, top-3
            const uint32_t c0 = S.hist[h][top], c1 = S.hist[h][top - 1];
            const uint32_t c2 = S.hist[h][top - 2], c3 = S.hist[h][top - 3];
            const uint32_t cnt = c0 + c1 + c2 + c3;
            const uint32_t inc = wave_incl_scan(cnt);
            const unsigned long long ball = __ballot(inc >= rem);
            if (ball == 0ull) {
                if (lane == 0) {  // fewer keys than wanted: take all of this prefix
                    S.thr[h] = S.prefix[h];
                    atomicAnd(&S.active, ~(1u << h));
                }
                continue;
            }
            const int owner = __ffsll(static_cast<long long>(ball)) - 1;
            if (lane == owner) {
                const uint32_t cs[4] = {c0, c1, c2, c3};
                uint32_t above = inc - cnt;
                int dg = top - 3;
                for (int e = 0; e < 4; ++e) {
                    if (above + cs[e] >= rem) {
                        dg = top - e;
                        break;
                    }
                    above += cs[e];
                }
                const uint32_t r2 = rem - above;
                const uint64_t p = S.prefix[h] | (static_cast<uint64_t>(dg) << shift);
                S.prefix[h] = p;
                S.rem[h] = r2;
                if (S.hist[h][dg] == r2 || shift == 0) {
                    S.thr[h] = p;
                    atomicAnd(&S.active, ~(1u << h));
                }
            }
        }
        __syncthreads();
    }
}

}  // namespace vattn
